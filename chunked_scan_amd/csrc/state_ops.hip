// state_ops.hip -- the segment-level kernels of the decomposition: the segmented state scan
// (All-Scan on one GPU), the cumulative-decay helper, the generic output correction, and the
// final states of empty segments.  All of them are HBM-bound streaming kernels.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

// ---------------------------------------------------------------------------------------------
// Segmented state scan.  Thread = one state element of one (b,h); it walks the P segments in
// order:  y = lam[p] * y + x[p];  out[p] = y.  The state chain is serial but its loads are not:
// a batch of BATCH segments is loaded before any of them is combined (loads past P repeat the
// last segment, so the batch is branch-free), and each thread keeps that many HBM reads in
// flight.  out may alias x: every element is read before the same thread overwrites it.
template <int BATCH>
__global__ __launch_bounds__(256) void state_scan_kernel(const float* x, const float* __restrict__ lam,
                                                         float* out, int P, int dk, int dv, int64_t per_state,
                                                         int vblocks) {
    const int64_t n = blockIdx.x / vblocks;  // state index: (b,h) or (b,h,segment)
    const int64_t e = (int64_t)(blockIdx.x % vblocks) * blockDim.x + threadIdx.x;
    if (e >= per_state) return;
    const int d = (int)(e / dv);
    const float* xs = x + n * (int64_t)P * per_state + e;
    float* ys = out + n * (int64_t)P * per_state + e;
    const float* ls = lam ? lam + n * (int64_t)P * dk + d : nullptr;  // null: no decay
    float y = 0.f;
    for (int p0 = 0; p0 < P; p0 += BATCH) {
        float xb[BATCH], lb[BATCH];
        const int nb = min(BATCH, P - p0);
#pragma unroll
        for (int j = 0; j < BATCH; j++) {
            const int pp = p0 + min(j, nb - 1);
            xb[j] = xs[(int64_t)pp * per_state];
            lb[j] = ls ? ls[(int64_t)pp * dk] : 1.f;
        }
#pragma unroll
        for (int j = 0; j < BATCH; j++) {
            if (j < nb) {
                y = (p0 + j == 0) ? xb[j] : lb[j] * y + xb[j];  // out[-1] = 0: segment 0's decay is never applied
                ys[(int64_t)(p0 + j) * per_state] = y;
            }
        }
    }
}

// Long scans (16 < P <= 4 PER): four threads share an element's chain, each owning PER consecutive
// segments.  Each computes its part as an affine map of the incoming value (local inclusive scan
// from zero, and the product of its decays), the four maps are composed in order through LDS, and
// each thread applies its carry to its outputs: one memory round trip per thread, every element
// read and written once.  Threads of a workgroup: 64 consecutive elements x 4 parts.
template <int PER>
__global__ __launch_bounds__(256) void state_scan4_kernel(const float* x, const float* __restrict__ lam, float* out,
                                                          int P, int dk, int dv, int64_t per_state, int vblocks) {
    __shared__ float loc_last[4][64], dec_last[4][64];
    const int el = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int64_t n = blockIdx.x / vblocks;
    const int64_t e = (int64_t)(blockIdx.x % vblocks) * 64 + el;
    const bool active = e < per_state;
    const int64_t ec = active ? e : per_state - 1;  // inactive lanes read a valid element, write nothing
    const int d = (int)(ec / dv);
    const float* xs = x + n * (int64_t)P * per_state + ec;
    float* ys = out + n * (int64_t)P * per_state + ec;
    const float* ls = lam ? lam + n * (int64_t)P * dk + d : nullptr;  // null: no decay
    const int p0 = part * PER, nb = max(0, min(PER, P - p0));
    float xb[PER], lb[PER];
    const int plast = max(0, min(p0 + PER, P) - 1);  // loads past the part's end repeat its last segment
#pragma unroll
    for (int j = 0; j < PER; j++) {
        const int pp = min(p0 + j, plast);
        xb[j] = xs[(int64_t)pp * per_state];
        lb[j] = (ls && pp > 0) ? ls[(int64_t)pp * dk] : 1.f;  // segment 0's decay only meets out[-1] = 0
    }
    // local inclusive scan from zero and the running product of the decays
    float loc[PER], dec[PER];
    float y = 0.f, dd = 1.f;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        if (j < nb) {
            y = lb[j] * y + xb[j];
            dd *= lb[j];
        }
        loc[j] = y;
        dec[j] = dd;
    }
    loc_last[part][el] = y;
    dec_last[part][el] = dd;
    __syncthreads();
    float c = 0.f;  // out[p0 - 1]
    for (int q = 0; q < part; q++) c = dec_last[q][el] * c + loc_last[q][el];
    if (!active) return;
#pragma unroll
    for (int j = 0; j < PER; j++)
        if (j < nb) ys[(int64_t)(p0 + j) * per_state] = loc[j] + dec[j] * c;
}

// Vector form of the same scan for 16-byte aligned states with dv % 4 == 0: a thread owns four
// consecutive elements of one row d (so one decay serves all four) and moves them as one 16-byte
// load or store per segment.  The P segments are cut into PARTS parts of ceil(P / PARTS) <= PER
// segments; each part scans its own segments from zero, keeps the running product of its decays,
// and the parts' affine maps are composed in order through LDS (as in the kernel above).  More
// parts means more short chains in flight per element, fewer means fewer threads per element.
template <int PER, int PARTS>
__global__ __launch_bounds__(256) void state_scan_vec_kernel(const float* x, const float* __restrict__ lam,
                                                             float* out, int P, int dk, int dv, int64_t per4,
                                                             int vblocks) {
    constexpr int EL = 256 / PARTS;  // float4 columns per workgroup
    __shared__ float4 loc_last[PARTS][EL];
    __shared__ float dec_last[PARTS][EL];
    const int el = threadIdx.x % EL, part = threadIdx.x / EL;
    const int64_t n = blockIdx.x / vblocks;
    const int64_t e = (int64_t)(blockIdx.x % vblocks) * EL + el;
    const bool active = e < per4;
    const int64_t ec = active ? e : per4 - 1;  // inactive lanes read a valid column, write nothing
    const int d = (int)(ec * 4 / dv);
    const float4* xs = reinterpret_cast<const float4*>(x) + n * (int64_t)P * per4 + ec;
    float4* ys = reinterpret_cast<float4*>(out) + n * (int64_t)P * per4 + ec;
    const float* ls = lam ? lam + n * (int64_t)P * dk + d : nullptr;  // null: no decay
    const int per = (P + PARTS - 1) / PARTS;
    const int p0 = part * per, nb = max(0, min(per, P - p0));
    float4 xb[PER];
    float lb[PER];
#pragma unroll
    for (int j = 0; j < PER; j++) {
        if (j < nb) {
            const int pp = p0 + j;
            xb[j] = xs[(int64_t)pp * per4];
            lb[j] = (ls && pp > 0) ? ls[(int64_t)pp * dk] : 1.f;  // segment 0's decay only meets out[-1] = 0
        }
    }
    // local inclusive scan from zero (kept in xb) and the running product of the decays (in lb)
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    float dd = 1.f;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        if (j < nb) {
            y.x = lb[j] * y.x + xb[j].x;
            y.y = lb[j] * y.y + xb[j].y;
            y.z = lb[j] * y.z + xb[j].z;
            y.w = lb[j] * y.w + xb[j].w;
            dd *= lb[j];
            xb[j] = y;
            lb[j] = dd;
        }
    }
    float4 c = make_float4(0.f, 0.f, 0.f, 0.f);  // out[p0 - 1]
    if (PARTS > 1) {
        loc_last[part][el] = y;
        dec_last[part][el] = dd;
        __syncthreads();
        for (int q = 0; q < part; q++) {
            const float4 l = loc_last[q][el];
            const float dq = dec_last[q][el];
            c.x = dq * c.x + l.x;
            c.y = dq * c.y + l.y;
            c.z = dq * c.z + l.z;
            c.w = dq * c.w + l.w;
        }
    }
    if (!active) return;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        if (j < nb) {
            float4 o = xb[j];
            o.x += lb[j] * c.x;
            o.y += lb[j] * c.y;
            o.z += lb[j] * c.z;
            o.w += lb[j] * c.w;
            ys[(int64_t)(p0 + j) * per4] = o;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Cumulative decay.  HEAD and NONE have closed forms; GATE needs a running sum of log a over the
// segment (below).
constexpr int CUM_TB = 64;

__global__ __launch_bounds__(256) void cumdecay_closed_kernel(const float* __restrict__ lamh, float* __restrict__ cum,
                                                              float* __restrict__ total, int64_t total_stride,
                                                              int64_t H, int64_t L, int dk, int nseg, int64_t n_cum,
                                                              int64_t n_tot, int mode) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t Ls = L / nseg;
    if (cum && i < n_cum) {
        const int64_t row = i / dk;  // (b,h,t)
        const int64_t t = row % L;
        const int64_t h = (row / L) % H;
        const int64_t tau = t % Ls + 1;
        cum[i] = (mode == DECAY_HEAD) ? expf(lamh[h] * (float)tau) : 1.f;
    }
    if (total && i < n_tot) {
        const int64_t bh = i / ((int64_t)dk * nseg);
        const int64_t h = bh % H;
        total[bh * total_stride + i % ((int64_t)dk * nseg)] =
            (mode == DECAY_HEAD) ? (Ls == 0 ? 1.f : expf(lamh[h] * (float)Ls)) : 1.f;
    }
}

// Gate mode, three passes over blocks of CUM_TB tokens of a segment:
//   1. partial[(bh*nseg + p)*nblk + blk][d] = sum of log a over the block's tokens;
//   2. the partials of each (b,h,segment) replaced in place by their exclusive prefix;
//   3. cum = exp(prefix + running sum inside the block) for every token, and the segment total.
// A thread owns one key dim of one block; consecutive threads take consecutive key dims, so every
// load and store of a token row is contiguous.  Each thread issues its loads GBATCH at a time
// before using any of them, so a block costs CUM_TB / GBATCH memory round trips.
constexpr int GBATCH = 16;

struct GateBlock {
    int64_t bh, bhp;
    int p, blk, d;
    int64_t t0, t1;
};
__device__ __forceinline__ GateBlock gate_block(int64_t i, int64_t L, int dk, int nseg, int nblk) {
    GateBlock x;
    x.d = (int)(i % dk);
    const int64_t r = i / dk;  // (bh*nseg + p)*nblk + blk
    x.blk = (int)(r % nblk);
    x.bhp = r / nblk;
    x.p = (int)(x.bhp % nseg);
    x.bh = x.bhp / nseg;
    const int64_t Ls = L / nseg;
    x.t0 = (int64_t)x.p * Ls + (int64_t)x.blk * CUM_TB;
    x.t1 = min(x.t0 + CUM_TB, (int64_t)(x.p + 1) * Ls);
    return x;
}

__global__ __launch_bounds__(256) void cumdecay_gate_blocksum_kernel(const float* __restrict__ g, float* __restrict__ partial,
                                                                     int64_t L, int dk, int nseg, int nblk,
                                                                     int64_t nthreads, float inv_norm) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nthreads) return;
    const GateBlock x = gate_block(i, L, dk, nseg, nblk);
    const float* gp = g + (x.bh * L) * dk + x.d;
    float s = 0.f;
    for (int64_t t = x.t0; t < x.t1; t += GBATCH) {
        float gv[GBATCH];
#pragma unroll
        for (int j = 0; j < GBATCH; j++) gv[j] = gp[min(t + j, x.t1 - 1) * dk];
#pragma unroll
        for (int j = 0; j < GBATCH; j++)
            if (t + j < x.t1) s += gate_logdecay(gv[j], inv_norm);
    }
    partial[i] = s;
}

// One workgroup per (b,h,segment) and 32 key dims: eight parts of the block list each sum their
// share, exchange the part sums through LDS, and write their blocks' exclusive prefixes.
__global__ __launch_bounds__(256) void cumdecay_gate_prefix_kernel(float* __restrict__ partial, int dk, int nblk) {
    __shared__ float part_sum[8][32];
    const int dl = threadIdx.x & 31, part = threadIdx.x >> 5;
    const int dgroups = (dk + 31) / 32;
    const int64_t bhp = blockIdx.x / dgroups;
    const int d = (int)(blockIdx.x % dgroups) * 32 + dl;
    const int per = (nblk + 7) / 8;
    const int b0 = min(nblk, part * per), b1 = min(nblk, b0 + per);
    float* base = partial + bhp * (int64_t)nblk * dk + min(d, dk - 1);
    float s = 0.f;
    for (int b = b0; b < b1; b += GBATCH) {
        float v[GBATCH];
#pragma unroll
        for (int j = 0; j < GBATCH; j++) v[j] = base[(int64_t)min(b + j, b1 - 1) * dk];
#pragma unroll
        for (int j = 0; j < GBATCH; j++)
            if (b + j < b1) s += v[j];
    }
    part_sum[part][dl] = s;
    __syncthreads();
    float run = 0.f;
    for (int j = 0; j < part; j++) run += part_sum[j][dl];
    if (d >= dk) return;
    for (int b = b0; b < b1; b += GBATCH) {
        float v[GBATCH];
#pragma unroll
        for (int j = 0; j < GBATCH; j++) v[j] = base[(int64_t)min(b + j, b1 - 1) * dk];
#pragma unroll
        for (int j = 0; j < GBATCH; j++)
            if (b + j < b1) {
                base[(int64_t)(b + j) * dk] = run;
                run += v[j];
            }
    }
}

__global__ __launch_bounds__(256) void cumdecay_gate_scan_kernel(const float* __restrict__ g, const float* __restrict__ partial,
                                                                 float* __restrict__ cum, float* __restrict__ total,
                                                                 int64_t total_stride, int64_t L, int dk, int nseg, int nblk,
                                                                 int64_t nthreads, float inv_norm) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nthreads) return;
    const GateBlock x = gate_block(i, L, dk, nseg, nblk);
    float run = partial[i];  // exclusive prefix of this block
    const float* gp = g + (x.bh * L) * dk + x.d;
    float* cp = cum ? cum + (x.bh * L) * dk + x.d : nullptr;
    const bool last = x.blk == nblk - 1;
    if (cp || last) {
        for (int64_t t = x.t0; t < x.t1; t += GBATCH) {
            float gv[GBATCH];
#pragma unroll
            for (int j = 0; j < GBATCH; j++) gv[j] = gp[min(t + j, x.t1 - 1) * dk];
#pragma unroll
            for (int j = 0; j < GBATCH; j++)
                if (t + j < x.t1) {
                    run += gate_logdecay(gv[j], inv_norm);
                    if (cp) cp[(t + j) * dk] = __builtin_amdgcn_exp2f(run * LOG2E);
                }
        }
    }
    if (total && last) total[x.bh * total_stride + (int64_t)x.p * dk + x.d] = __builtin_amdgcn_exp2f(run * LOG2E);
}

// The third gate pass writing q times the cumulative decay instead of the decay itself, the
// segment totals, and the tile flags: a block is one 64-token tile, live when the decay at its
// start is nonzero for some key dim (the flags were zeroed first; live dims all write the same
// word).
template <typename T>
__global__ __launch_bounds__(256) void decayed_q_gate_scan_kernel(
    const T* __restrict__ q, const float* __restrict__ g, const float* __restrict__ partial, T* __restrict__ q_dec,
    float* __restrict__ total, int64_t total_stride, uint32_t* __restrict__ live, int64_t L, int dk, int nseg,
    int nblk, int64_t nthreads, float inv_norm) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nthreads) return;
    const GateBlock x = gate_block(i, L, dk, nseg, nblk);
    float run = partial[i];  // exclusive prefix of this block
    if (live && __builtin_amdgcn_exp2f(run * LOG2E) != 0.f) live[x.bhp * nblk + x.blk] = 0x01010101u;
    const float* gp = g + (x.bh * L) * dk + x.d;
    const T* qp = q + (x.bh * L) * dk + x.d;
    T* dp = q_dec ? q_dec + (x.bh * L) * dk + x.d : nullptr;
    const bool last = x.blk == nblk - 1;
    if (dp || last) {
        for (int64_t t = x.t0; t < x.t1; t += GBATCH) {
            float gv[GBATCH], qv[GBATCH];
#pragma unroll
            for (int j = 0; j < GBATCH; j++) {
                const int64_t tt = min(t + j, x.t1 - 1) * dk;
                gv[j] = gp[tt];
                qv[j] = dp ? (float)qp[tt] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < GBATCH; j++)
                if (t + j < x.t1) {
                    run += gate_logdecay(gv[j], inv_norm);
                    if (dp) dp[(t + j) * dk] = (T)(qv[j] * __builtin_amdgcn_exp2f(run * LOG2E));
                }
        }
    }
    if (total && last) total[x.bh * total_stride + (int64_t)x.p * dk + x.d] = __builtin_amdgcn_exp2f(run * LOG2E);
}

// ---------------------------------------------------------------------------------------------
// Generic output correction (fp32 arithmetic): block = (b,h,segment, 64-token tile, 32-wide
// dv slice).  o_t[c] += sum_d q_t[d] cum_t[d] S[d][c].
constexpr int CT = 64;
constexpr int CDVT = 32;

template <typename T, int MODE>
__global__ __launch_bounds__(256) void state_correct_generic_kernel(
    const T* __restrict__ q, const float* __restrict__ cum, const float* __restrict__ s_recv, T* __restrict__ o,
    int64_t H, int64_t L, int dk, int dv, int nseg, int seg_begin, int64_t state_stride, int ntiles) {
    __shared__ float Ss[128 * CDVT];
    __shared__ float Qs[CT * 128];
    const int tid = threadIdx.x;
    int64_t r = blockIdx.x;
    const int tile = (int)(r % ntiles);
    r /= ntiles;
    const int np = nseg - seg_begin;
    const int p = seg_begin + (int)(r % np);
    const int64_t bh = r / np;
    const int64_t h = bh % H;
    const int c0 = blockIdx.y * CDVT;
    const int nc = min(CDVT, dv - c0);
    const int64_t Ls = L / nseg;
    const int64_t tt0 = (int64_t)tile * CT;  // offset inside the segment
    const int n = (int)min((int64_t)CT, Ls - tt0);
    if (n <= 0) return;
    const int64_t row0 = bh * L + (int64_t)p * Ls + tt0;
    const float* S = s_recv + bh * state_stride + (int64_t)(p - seg_begin) * dk * dv;
    for (int e = tid; e < dk * nc; e += 256) {
        int d = e / nc, c = e % nc;
        Ss[d * CDVT + c] = S[d * dv + c0 + c];
    }
    const float lam = (MODE == DECAY_HEAD) ? cum[h] : 0.f;
    for (int e = tid; e < n * dk; e += 256) {
        int i = e / dk, d = e % dk;
        float w = io<T>::ld(q + (row0 + i) * dk + d);
        if (MODE == DECAY_HEAD) w *= expf(lam * (float)(tt0 + i + 1));
        if (MODE == DECAY_GATE) w *= cum[(row0 + i) * dk + d];
        Qs[i * 128 + d] = w;
    }
    __syncthreads();
    for (int e = tid; e < n * nc; e += 256) {
        int i = e / nc, c = e % nc;
        float acc = 0.f;
        for (int d = 0; d < dk; d++) acc += Qs[i * 128 + d] * Ss[d * CDVT + c];
        T* po = o + (row0 + i) * dv + c0 + c;
        io<T>::st(po, io<T>::ld(po) + acc);
    }
}

template <typename T>
hipError_t correct_typed(const CorrectArgs& a) {
    const int64_t Ls = a.L / a.nseg;
    const int ntiles = (int)((Ls + CT - 1) / CT);
    const int64_t nblk = a.B * a.H * (int64_t)(a.nseg - a.seg_begin) * ntiles;
    if (nblk == 0) return hipSuccess;
    dim3 grid((unsigned)nblk, (unsigned)((a.dv + CDVT - 1) / CDVT));
    const T* q = (const T*)a.q;
    T* o = (T*)a.o;
    const int64_t ss = a.state_stride;
    switch (a.mode) {
        case DECAY_HEAD:
            LA_TRACED(a.tr, "state_correct_generic", state_correct_generic_kernel<T, DECAY_HEAD><<<grid, 256, 0, a.stream>>>(
                q, a.cum, a.s_recv, o, a.H, a.L, a.dk, a.dv, a.nseg, a.seg_begin, ss, ntiles));
            break;
        case DECAY_GATE:
            LA_TRACED(a.tr, "state_correct_generic", state_correct_generic_kernel<T, DECAY_GATE><<<grid, 256, 0, a.stream>>>(
                q, a.cum, a.s_recv, o, a.H, a.L, a.dk, a.dv, a.nseg, a.seg_begin, ss, ntiles));
            break;
        default:
            LA_TRACED(a.tr, "state_correct_generic", state_correct_generic_kernel<T, DECAY_NONE><<<grid, 256, 0, a.stream>>>(
                q, a.cum, a.s_recv, o, a.H, a.L, a.dk, a.dv, a.nseg, a.seg_begin, ss, ntiles));
            break;
    }
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void empty_states_kernel(const float* __restrict__ s_in, float* __restrict__ s_out,
                                                           int64_t s_out_stride, int nseg, int64_t SZ, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t e = i % SZ;
    const int64_t bhp = i / SZ;
    const int p = (int)(bhp % nseg);
    const int64_t bh = bhp / nseg;
    s_out[bh * s_out_stride + (int64_t)p * SZ + e] = (p == 0 && s_in) ? s_in[bh * SZ + e] : 0.f;
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// q times its cumulative decay from the segment start, where the forward does not emit it itself.
// Head and no-decay modes: one thread per element, the closed form exp(lambda_h * tau).
template <typename T>
__global__ __launch_bounds__(256) void decayed_q_closed_kernel(const T* __restrict__ q, const float* __restrict__ lamh,
                                                               T* __restrict__ q_dec, int64_t n, int64_t H, int64_t L,
                                                               int dk, int nseg, int mode) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t row = i / dk;  // (b,h,t)
    const int64_t tau = row % L % (L / nseg) + 1;
    const float c = mode == DECAY_HEAD ? expf(lamh[(row / L) % H] * (float)tau) : 1.f;
    q_dec[i] = (T)((float)q[i] * c);
}

// Head and no-decay modes: tile flags from the decay at each 64-token tile's first token.
__global__ __launch_bounds__(256) void tile_live_closed_kernel(const float* __restrict__ lamh,
                                                               uint32_t* __restrict__ live, int64_t n, int64_t H,
                                                               int nseg, int64_t tps, int mode) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t tile = i % tps, h = (i / tps / nseg) % H;
    live[i] = (mode != DECAY_HEAD || expf(lamh[h] * (float)(tile * 64 + 1)) != 0.f) ? 0x01010101u : 0u;
}

}  // namespace

hipError_t launch_state_scan(const float* x, const float* lam, float* out, int64_t nstates, int P, int dk, int dv,
                             hipStream_t stream, Tracer* tr) {
    if (nstates == 0 || P == 0) return hipSuccess;
    const int64_t per_state = (int64_t)dk * dv;
    const int vblocks = (int)((per_state + 255) / 256);
    const unsigned grid = (unsigned)(nstates * vblocks);
    const bool vec = dv % 4 == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)out % 16) == 0;
    // Segment counts up to 40 take the vector scan (one, four or eight parts); 41..64 the four-part
    // scalar scan, which measured faster there; longer scans the batched chain.
    if (vec && P <= 40) {
        const int64_t per4 = per_state / 4;
        auto vec_launch = [&](auto kern, int parts) {
            const int vb = (int)((per4 + 256 / parts - 1) / (256 / parts));
            kern<<<(unsigned)(nstates * vb), 256, 0, stream>>>(x, lam, out, P, dk, dv, per4, vb);
        };
        if (P <= 8)
            LA_TRACED(tr, "state_scan", vec_launch(state_scan_vec_kernel<8, 1>, 1));
        else if (P <= 20)
            LA_TRACED(tr, "state_scan", vec_launch(state_scan_vec_kernel<5, 4>, 4));
        else
            LA_TRACED(tr, "state_scan", vec_launch(state_scan_vec_kernel<5, 8>, 8));
    } else if (P <= 4)
        LA_TRACED(tr, "state_scan", state_scan_kernel<4><<<grid, 256, 0, stream>>>(x, lam, out, P, dk, dv, per_state, vblocks));
    else if (P <= 8)
        LA_TRACED(tr, "state_scan", state_scan_kernel<8><<<grid, 256, 0, stream>>>(x, lam, out, P, dk, dv, per_state, vblocks));
    else if (P <= 16)
        LA_TRACED(tr, "state_scan", state_scan_kernel<16><<<grid, 256, 0, stream>>>(x, lam, out, P, dk, dv, per_state, vblocks));
    else if (P <= 32) {
        const int vb64 = (int)((per_state + 63) / 64);
        LA_TRACED(tr, "state_scan", state_scan4_kernel<8><<<(unsigned)(nstates * vb64), 256, 0, stream>>>(
                                        x, lam, out, P, dk, dv, per_state, vb64));
    } else if (P <= 64) {
        const int vb64 = (int)((per_state + 63) / 64);
        LA_TRACED(tr, "state_scan", state_scan4_kernel<16><<<(unsigned)(nstates * vb64), 256, 0, stream>>>(
                                        x, lam, out, P, dk, dv, per_state, vb64));
    } else
        LA_TRACED(tr, "state_scan", state_scan_kernel<16><<<grid, 256, 0, stream>>>(x, lam, out, P, dk, dv, per_state, vblocks));
    return hipGetLastError();
}

namespace {

template <typename T>
hipError_t decayed_q_typed(const FwdArgs& a) {
    const int64_t BH = a.B * a.H;
    const int64_t Ls = a.L / a.nseg;
    const int64_t tps = (Ls + 63) / 64;
    const int64_t ntile = BH * a.nseg * tps;
    hipError_t e = hipSuccess;
    if (a.mode != DECAY_GATE || Ls == 0) {
        const int64_t n = BH * a.L * a.dk;
        if (a.q_dec && n > 0) {
            LA_TRACED(a.tr, "decayed_q_closed",
                      decayed_q_closed_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, a.stream>>>(
                          (const T*)a.q, a.decay, (T*)a.q_dec, n, a.H, a.L, a.dk, a.nseg, a.mode));
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (a.tile_live && ntile > 0) {
            LA_TRACED(a.tr, "tile_live_closed",
                      tile_live_closed_kernel<<<(unsigned)((ntile + 255) / 256), 256, 0, a.stream>>>(
                          a.decay, a.tile_live, ntile, a.H, a.nseg, tps, a.mode == DECAY_HEAD ? DECAY_HEAD : DECAY_NONE));
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (a.total)  // closed forms (gate with empty segments: the empty product)
            e = launch_cumdecay(a.decay, nullptr, a.total, a.total_stride, a.B, a.H, a.L, a.dk, a.nseg,
                                a.mode == DECAY_GATE ? DECAY_NONE : a.mode, a.inv_norm, a.stream, a.tr);
        return e;
    }
    // gate: block sums of log a, their exclusive prefix, then the pass over q
    const int nblk = (int)tps;
    const int64_t nthreads = BH * a.nseg * nblk * a.dk;
    float* partial = nullptr;
    e = workspace_alloc((void**)&partial, sizeof(float) * (size_t)nthreads, a.stream);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((nthreads + 255) / 256);
    if (a.tile_live)
        LA_TRACED(a.tr, "tile_live_fill",
                  fill_u32_kernel<<<(unsigned)((ntile + 255) / 256), 256, 0, a.stream>>>(a.tile_live, ntile, 0u));
    e = hipGetLastError();
    if (e == hipSuccess) {
        LA_TRACED(a.tr, "cumdecay_gate_blocksum",
                  cumdecay_gate_blocksum_kernel<<<grid, 256, 0, a.stream>>>(a.decay, partial, a.L, a.dk, a.nseg, nblk,
                                                                          nthreads, a.inv_norm));
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        LA_TRACED(a.tr, "cumdecay_gate_prefix",
                  cumdecay_gate_prefix_kernel<<<(unsigned)(BH * a.nseg * ((a.dk + 31) / 32)), 256, 0, a.stream>>>(
                      partial, a.dk, nblk));
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        LA_TRACED(a.tr, "decayed_q_gate_scan",
                  decayed_q_gate_scan_kernel<T><<<grid, 256, 0, a.stream>>>(
                      (const T*)a.q, a.decay, partial, (T*)a.q_dec, a.total, a.total_stride, a.tile_live, a.L, a.dk,
                      a.nseg, nblk, nthreads, a.inv_norm));
        e = hipGetLastError();
    }
    const hipError_t f = hipFreeAsync(partial, a.stream);
    return e != hipSuccess ? e : f;
}

}  // namespace

hipError_t launch_decayed_q(const FwdArgs& a) {
    if (a.B * a.H * (int64_t)a.nseg * a.dk == 0 || (!a.q_dec && !a.total && !a.tile_live)) return hipSuccess;
    return a.bf16 ? decayed_q_typed<__bf16>(a) : decayed_q_typed<float>(a);
}

hipError_t launch_cumdecay(const float* decay, float* cum, float* total, int64_t total_stride, int64_t B, int64_t H,
                           int64_t L, int dk, int nseg, int mode, float inv_norm, hipStream_t stream, Tracer* tr) {
    const int64_t n_cum = B * H * L * dk;
    const int64_t n_tot = B * H * (int64_t)nseg * dk;
    if (mode != DECAY_GATE) {
        const int64_t n = max(cum ? n_cum : 0, total ? n_tot : 0);
        if (n == 0) return hipSuccess;
        LA_TRACED(tr, "cumdecay_closed",
                  cumdecay_closed_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
                      decay, cum, total, total_stride, H, L, dk, nseg, n_cum, n_tot, mode));
        return hipGetLastError();
    }
    const int64_t Ls = L / nseg;
    if (Ls == 0) {  // empty segments: cumulative decay is the empty product
        if (!total || n_tot == 0) return hipSuccess;
        LA_TRACED(tr, "cumdecay_closed",
                  cumdecay_closed_kernel<<<(unsigned)((n_tot + 255) / 256), 256, 0, stream>>>(
                      decay, nullptr, total, total_stride, H, L, dk, nseg, 0, n_tot, DECAY_NONE));
        return hipGetLastError();
    }
    const int nblk = (int)((Ls + CUM_TB - 1) / CUM_TB);
    const int64_t nthreads = B * H * (int64_t)nseg * nblk * dk;
    if (nthreads == 0) return hipSuccess;
    float* partial = nullptr;
    hipError_t e = workspace_alloc((void**)&partial, sizeof(float) * (size_t)nthreads, stream);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((nthreads + 255) / 256);
    LA_TRACED(tr, "cumdecay_gate_blocksum",
              cumdecay_gate_blocksum_kernel<<<grid, 256, 0, stream>>>(decay, partial, L, dk, nseg, nblk, nthreads,
                                                                      inv_norm));
    e = hipGetLastError();
    if (e == hipSuccess) {
        const int64_t nbhp = B * H * (int64_t)nseg;
        LA_TRACED(tr, "cumdecay_gate_prefix",
                  cumdecay_gate_prefix_kernel<<<(unsigned)(nbhp * ((dk + 31) / 32)), 256, 0, stream>>>(partial, dk,
                                                                                                       nblk));
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        LA_TRACED(tr, "cumdecay_gate_scan",
                  cumdecay_gate_scan_kernel<<<grid, 256, 0, stream>>>(decay, partial, cum, total, total_stride, L, dk,
                                                                      nseg, nblk, nthreads, inv_norm));
        e = hipGetLastError();
    }
    hipError_t f = hipFreeAsync(partial, stream);
    return e != hipSuccess ? e : f;
}

hipError_t launch_state_correct_generic(const CorrectArgs& a) {
    return a.bf16 ? correct_typed<__bf16>(a) : correct_typed<float>(a);
}

hipError_t launch_empty_states(const float* s_in, float* s_out, int64_t s_out_stride, int64_t BH, int nseg, int dk,
                               int dv, hipStream_t stream, Tracer* tr) {
    const int64_t SZ = (int64_t)dk * dv;
    const int64_t n = BH * nseg * SZ;
    if (n == 0) return hipSuccess;
    LA_TRACED(tr, "empty_states",
              empty_states_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(s_in, s_out, s_out_stride, nseg,
                                                                                   SZ, n));
    return hipGetLastError();
}

}  // namespace la
