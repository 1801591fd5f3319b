// chunk_fwd_mfma.hip -- bf16 matrix-core (MFMA) chunked forward for dk = dv = 128, chunk = 64
// on gfx950.
//
// Work unit.  One workgroup (4 waves, 256 lanes) owns one sub-segment of one (b, h, segment) and
// walks its 64-token chunks in order.  The fp32 state S (128 x 128) lives in accumulator
// registers for the whole walk: wave w holds value columns 32w..32w+31 as four 32 x 32 MFMA
// accumulator tiles (one per 32 key rows).  Nothing per chunk goes back to HBM except O.
//
// Parallelism across the sequence.  A (b,h) sequence alone offers one serial chain of chunks,
// far too few workgroups for 256 compute units, so each segment is cut into G sub-segments and
// the linear-decomposition identity of the ZeCO review page (pith_extraction.key_machinery)
// is applied inside the GPU:
//   pass 1 (state-only): every sub-segment but the last computes its local end state from zero
//          (sub-segment 0 of segment 0 from s_in) and its total decay;
//   scan:  an inclusive state scan over the sub-segments turns those into exact incoming states;
//   pass 2 (outputs):  every sub-segment re-runs its chunks from its exact incoming state and
//          writes O; the last one writes s_out.
// Pass 2 therefore needs no output correction.  The cost is one extra read of K and V.
//
// Per chunk of n <= 64 tokens, with B_i the inclusive in-chunk cumulative log-decay (per key dim
// in gate mode, lambda*(i+1) in head mode):
//   P[i][j] = sum_d qbar_i[d] kbar_j[d]     masked to j <= i            (intra-chunk "diagonal")
//   O       = diag-scaled (Qbar S) + P V                                 (inter + intra)
//   S      <- diag(exp(B_{n-1})) S + Ktilde^T V,   Ktilde_j = k_j * exp(B_{n-1} - B_j)
// Head/none modes compute P from raw q, k and apply exp(lambda (i-j)) elementwise, and scale the
// rows of Q S by exp(lambda (i+1)) after the product, so every factor is <= 1.  Gate mode must put
// the per-key-dim decay inside the contraction: qbar = q*exp(B_i) (<= 1), kbar = k*exp(-B_j)
// (>= 1, bounded by the chunk's decay span), as in the K-bar / Lambda / Gamma vectors that the
// ZeCO review page discusses (referee_report.minor_comments[3]).
#include "la_device.h"
#include "la_internal.h"

#include <mutex>

namespace la {
namespace {

constexpr int C = 64;        // chunk length
constexpr int D = 128;       // dk = dv
constexpr int PITCH = 136;   // bf16 row pitch of the staged tiles (272 B: conflict-free 16 B row reads)
constexpr int PPITCH = 72;   // bf16 row pitch of P
constexpr int TILE = C * PITCH;
constexpr int NT = 256;      // lanes per workgroup

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x4 lds_tr16(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((__attribute__((address_space(3))) __bf16*)p));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 bf16 (one 16-byte word) scaled by 8 fp32 factors, rounded to nearest even.
__device__ __forceinline__ u32x4 scale8(u32x4 w, const float* f) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 4; h++) {
        float lo = bits_lo_bf16(w[h]) * f[2 * h];
        float hi = bits_hi_bf16(w[h]) * f[2 * h + 1];
        __bf16 blo = (__bf16)lo, bhi = (__bf16)hi;
        r[h] = (uint32_t)__builtin_bit_cast(uint16_t, blo) | ((uint32_t)__builtin_bit_cast(uint16_t, bhi) << 16);
    }
    return r;
}

__device__ __forceinline__ u32x4 scale8s(u32x4 w, float f) {
    float ff[8] = {f, f, f, f, f, f, f, f};
    return scale8(w, ff);
}

struct Smem {
    __bf16 q[TILE];    // qbar (gate) or q
    __bf16 kp[TILE];   // kbar (gate) or k: the K side of P
    __bf16 kt[TILE];   // ktilde: keys scaled by the decay to the chunk end
    __bf16 v[TILE];
    __bf16 p[C * PPITCH];
};
struct SmemGate {
    float b[C * D];    // in-chunk inclusive cumulative log-decay
    float el[D];       // exp(B_{n-1}): the chunk's total decay per key dim
    float tot[D];      // scratch for the two-half scan
};

template <int MODE, bool STATE_ONLY>
__global__ __launch_bounds__(NT) void mfma_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ decay, const float* __restrict__ s_in, __bf16* __restrict__ o,
    float* __restrict__ s_out, int64_t s_out_stride,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // pass 1 outputs
    const float* __restrict__ init_state,                            // pass 2 inputs (scanned)
    int64_t H, int64_t L, int nseg, int G, int cps, float inv_norm) {
    __shared__ __attribute__((aligned(16))) Smem sm;
    __shared__ __attribute__((aligned(16))) SmemGate sg_[1];  // dropped by the compiler outside gate mode
    SmemGate& sg = sg_[0];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int n32 = lane & 31;
    const int kg = lane >> 5;

    const int64_t u = blockIdx.x;
    const int g = (int)(u % (STATE_ONLY ? (G - 1) : G));
    const int64_t ub = u / (STATE_ONLY ? (G - 1) : G);  // (bh, seg)
    const int seg = (int)(ub % nseg);
    const int64_t bh = ub / nseg;
    const int64_t h = bh % H;
    const int64_t Lseg = L / nseg;
    const int64_t t_begin = (int64_t)seg * Lseg + (int64_t)g * cps * C;
    const int64_t t_end = min(t_begin + (int64_t)cps * C, (int64_t)(seg + 1) * Lseg);
    const int64_t row_base = bh * L;  // token rows of this (b,h)
    const float lam = (MODE == DECAY_HEAD) ? decay[h] : 0.f;

    // ---- initial state into the accumulator tiles
    f32x16 S[4];
    {
        const float* src = nullptr;
        if (g == 0) {
            if (seg == 0 && s_in) src = s_in + bh * (int64_t)D * D;
        } else if (!STATE_ONLY) {
            src = init_state + (ub * (G - 1) + (g - 1)) * (int64_t)D * D;
        }
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                S[m][i] = src ? src[r * D + 32 * w + n32] : 0.f;
            }
    }

    // ---- register prefetch of one chunk: 4 x 16 B of q, k, v per lane (+ 8 x 16 B of g)
    u32x4 rq[4], rk[4], rv[4];
    f32x4 rg[MODE == DECAY_GATE ? 8 : 1];
    auto load_chunk = [&](int64_t t0, int n) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int p = tid + NT * r;
            const int row = p >> 4, c8 = (p & 15) * 8;
            const int64_t off = (row_base + t0 + row) * D + c8;
            const bool ok = row < n;
            if (!STATE_ONLY) rq[r] = ok ? *(const u32x4*)(q + off) : u32x4{0, 0, 0, 0};
            rk[r] = ok ? *(const u32x4*)(k + off) : u32x4{0, 0, 0, 0};
            rv[r] = ok ? *(const u32x4*)(v + off) : u32x4{0, 0, 0, 0};
        }
        if (MODE == DECAY_GATE) {
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const int p = tid + NT * r;
                const int row = p >> 5, c4 = (p & 31) * 4;
                rg[r] = row < n ? *(const f32x4*)(decay + (row_base + t0 + row) * D + c4) : f32x4{0, 0, 0, 0};
            }
        }
    };

    float gate_total = 0.f;  // pass 1, gate mode: running sum of log-decay of key dim tid (tid < 128)

    const int nchunks = (int)((t_end - t_begin + C - 1) / C);
    if (nchunks > 0) load_chunk(t_begin, (int)min((int64_t)C, t_end - t_begin));

    for (int c = 0; c < nchunks; c++) {
        const int64_t t0 = t_begin + (int64_t)c * C;
        const int n = (int)min((int64_t)C, t_end - t0);
        __syncthreads();  // previous chunk is done with every LDS tile

        // ---- stage the prefetched chunk into LDS, folding in the decay factors
        if (MODE == DECAY_GATE) {
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const int p = tid + NT * r;
                const int row = p >> 5, c4 = (p & 31) * 4;
                f32x4 lg;
#pragma unroll
                for (int e = 0; e < 4; e++) lg[e] = row < n ? gate_logdecay(rg[r][e], inv_norm) : 0.f;
                *(f32x4*)(&sg.b[row * D + c4]) = lg;
            }
            __syncthreads();
            {   // inclusive cumsum over the 64 rows, per key dim; two halves of 32 rows
                const int d = tid & 127, half = tid >> 7;
                float vals[32];
#pragma unroll
                for (int i = 0; i < 32; i++) vals[i] = sg.b[(half * 32 + i) * D + d];
#pragma unroll
                for (int i = 1; i < 32; i++) vals[i] += vals[i - 1];
                if (half == 0) {
#pragma unroll
                    for (int i = 0; i < 32; i++) sg.b[i * D + d] = vals[i];
                    sg.tot[d] = vals[31];
                }
                __syncthreads();
                if (half == 1) {
                    const float off = sg.tot[d];
#pragma unroll
                    for (int i = 0; i < 32; i++) sg.b[(32 + i) * D + d] = vals[i] + off;
                }
                __syncthreads();
                if (tid < D) {
                    const float bl = sg.b[(n - 1) * D + tid];
                    sg.el[tid] = expf(bl);
                    gate_total += bl;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int p = tid + NT * r;
                const int row = p >> 4, c8 = (p & 15) * 8;
                float eb[8], einv[8], et[8];
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float bi = sg.b[row * D + c8 + e];
                    const float bl = sg.b[(n - 1) * D + c8 + e];
                    eb[e] = expf(bi);
                    einv[e] = expf(-bi);
                    et[e] = expf(bl - bi);
                }
                if (!STATE_ONLY) {
                    *(u32x4*)(&sm.q[row * PITCH + c8]) = scale8(rq[r], eb);
                    *(u32x4*)(&sm.kp[row * PITCH + c8]) = scale8(rk[r], einv);
                }
                *(u32x4*)(&sm.kt[row * PITCH + c8]) = scale8(rk[r], et);
                *(u32x4*)(&sm.v[row * PITCH + c8]) = rv[r];
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int p = tid + NT * r;
                const int row = p >> 4, c8 = (p & 15) * 8;
                if (!STATE_ONLY) {
                    *(u32x4*)(&sm.q[row * PITCH + c8]) = rq[r];
                    *(u32x4*)(&sm.kp[row * PITCH + c8]) = rk[r];
                }
                if (MODE == DECAY_HEAD)
                    *(u32x4*)(&sm.kt[row * PITCH + c8]) = scale8s(rk[r], decay_pow(lam, max(n - 1 - row, 0)));
                else
                    *(u32x4*)(&sm.kt[row * PITCH + c8]) = rk[r];
                *(u32x4*)(&sm.v[row * PITCH + c8]) = rv[r];
            }
        }
        __syncthreads();

        // ---- prefetch the next chunk while this one is computed
        if (c + 1 < nchunks) load_chunk(t0 + C, (int)min((int64_t)C, t_end - (t0 + C)));

        // ---- V operand of this wave's 32 value columns, for the 4 token slabs (shared by P V and K^T V)
        bf16x8 vb[4];
        {
            const int G16 = lane >> 4, i16 = lane & 15;
            const int col = 32 * w + (G16 & 1) * 16 + (i16 & 3) * 4;
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const int tb = 16 * ks + (G16 >> 1) * 8 + (i16 >> 2);
                vb[ks] = cat(lds_tr16(&sm.v[tb * PITCH + col]), lds_tr16(&sm.v[(tb + 4) * PITCH + col]));
            }
        }

        if (!STATE_ONLY) {
            // ---- intra-chunk scores: causal 32x32 blocks (0,0), (1,0), (1,1) on waves 0, 2, 3
            if (w != 1) {
                const int rb = w >> 1, cb = (w == 3) ? 1 : 0;
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < 8; ks++) {
                    const bf16x8 a = *(const bf16x8*)(&sm.q[(rb * 32 + n32) * PITCH + ks * 16 + kg * 8]);
                    const bf16x8 b = *(const bf16x8*)(&sm.kp[(cb * 32 + n32) * PITCH + ks * 16 + kg * 8]);
                    acc = mfma(a, b, acc);
                }
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = rb * 32 + (i >> 2) * 8 + kg * 4 + (i & 3);
                    const int col = cb * 32 + n32;
                    float val = acc[i];
                    if (MODE == DECAY_HEAD) val *= decay_pow(lam, max(row - col, 0));
                    if (col > row) val = 0.f;
                    sm.p[row * PPITCH + col] = (__bf16)val;
                }
            }
            // state as bf16 B operands: slab (m, h) covers key rows 32m + 16h + {kg*4 + 0..3, 8 + kg*4 + 0..3}
            bf16x8 sb[8];
#pragma unroll
            for (int m = 0; m < 4; m++)
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    bf16x8 x;
#pragma unroll
                    for (int j = 0; j < 8; j++) x[j] = (__bf16)S[m][8 * hh + j];
                    sb[2 * m + hh] = x;
                }
            __syncthreads();  // P complete

            // ---- outputs of this wave's 32 columns, two 32-row blocks
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                f32x16 acc = {};
                const __bf16* qrow = &sm.q[(rb * 32 + n32) * PITCH + kg * 4];
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
                        const int d0 = 32 * m + 16 * hh;
                        const bf16x4 lo = *(const bf16x4*)(qrow + d0);
                        const bf16x4 hi = *(const bf16x4*)(qrow + d0 + 8);
                        acc = mfma(cat(lo, hi), sb[2 * m + hh], acc);
                    }
                if (MODE == DECAY_HEAD) {
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        const int row = rb * 32 + (i >> 2) * 8 + kg * 4 + (i & 3);
                        acc[i] *= decay_pow(lam, row + 1);
                    }
                }
#pragma unroll
                for (int ks = 0; ks < 2 * (rb + 1); ks++) {
                    const bf16x8 a = *(const bf16x8*)(&sm.p[(rb * 32 + n32) * PPITCH + ks * 16 + kg * 8]);
                    acc = mfma(a, vb[ks], acc);
                }
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = rb * 32 + (i >> 2) * 8 + kg * 4 + (i & 3);
                    if (row < n) o[(row_base + t0 + row) * D + 32 * w + n32] = (__bf16)acc[i];
                }
            }
        }

        // ---- state update: S <- diag(decay over the chunk) S + Ktilde^T V
        {
            float srow[4][16];
            if (MODE == DECAY_GATE) {
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int i = 0; i < 16; i++) srow[m][i] = sg.el[32 * m + (i >> 2) * 8 + kg * 4 + (i & 3)];
            }
            const float fh = (MODE == DECAY_HEAD) ? decay_pow(lam, n) : 1.f;
            const int G16 = lane >> 4, i16 = lane & 15;
#pragma unroll
            for (int m = 0; m < 4; m++) {
                if (MODE == DECAY_GATE) {
#pragma unroll
                    for (int i = 0; i < 16; i++) S[m][i] *= srow[m][i];
                } else if (MODE == DECAY_HEAD) {
#pragma unroll
                    for (int i = 0; i < 16; i++) S[m][i] *= fh;
                }
                const int col = 32 * m + (G16 & 1) * 16 + (i16 & 3) * 4;
#pragma unroll
                for (int ks = 0; ks < 4; ks++) {
                    const int tb = 16 * ks + (G16 >> 1) * 8 + (i16 >> 2);
                    const bf16x8 a = cat(lds_tr16(&sm.kt[tb * PITCH + col]), lds_tr16(&sm.kt[(tb + 4) * PITCH + col]));
                    S[m] = mfma(a, vb[ks], S[m]);
                }
            }
        }
    }

    // ---- write the final state
    float* dst = nullptr;
    if (STATE_ONLY) {
        dst = part_state + (ub * (G - 1) + g) * (int64_t)D * D;
    } else if (g == G - 1 && s_out) {
        dst = s_out + bh * s_out_stride + (int64_t)seg * D * D;
    }
    if (dst) {
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                dst[r * D + 32 * w + n32] = S[m][i];
            }
    }
    if (STATE_ONLY && tid < D) {
        float tot;
        if (MODE == DECAY_GATE) tot = expf(gate_total);
        else if (MODE == DECAY_HEAD) tot = decay_pow(lam, (int)(t_end - t_begin));
        else tot = 1.f;
        part_decay[(ub * (G - 1) + g) * D + tid] = tot;
    }
}

// ---- workspace: a stream-ordered pool per device that keeps its memory between calls
hipMemPool_t workspace_pool(int dev) {
    static std::mutex mu;
    static hipMemPool_t pools[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 0 || dev >= 64) return nullptr;
    if (!pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        if (hipMemPoolCreate(&p, &props) != hipSuccess) return nullptr;
        uint64_t keep = ~0ull;
        (void)hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
        pools[dev] = p;
    }
    return pools[dev];
}

template <int MODE>
hipError_t launch_mode(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay) {
    const int64_t ub = a.B * a.H * a.nseg;
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    __bf16* o = (__bf16*)a.o;
    if (G > 1) {
        LA_TRACED(a.tr, "chunk_fwd_mfma_state_pass",
                  mfma_fwd_kernel<MODE, true><<<(unsigned)(ub * (G - 1)), NT, 0, a.stream>>>(
                      q, k, v, a.decay, a.s_in, o, a.s_out, a.s_out_stride, part_state, part_decay, nullptr, a.H,
                      a.L, a.nseg, G, cps, a.inv_norm));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_state_scan(part_state, part_decay, part_state, ub, G - 1, D, D, a.stream, a.tr);
        if (e != hipSuccess) return e;
    }
    LA_TRACED(a.tr, "chunk_fwd_mfma_output_pass",
              mfma_fwd_kernel<MODE, false><<<(unsigned)(ub * G), NT, 0, a.stream>>>(
                  q, k, v, a.decay, a.s_in, o, a.s_out, a.s_out_stride, nullptr, nullptr, part_state, a.H, a.L,
                  a.nseg, G, cps, a.inv_norm));
    return hipGetLastError();
}

}  // namespace

// Sub-segment length in chunks: about one workgroup per compute unit (256 on MI355X) in one
// round -- a second round costs a full extra sub-segment walk, and more sub-segments lengthen the
// state scan -- but at least four chunks each so that the state traffic stays small next to the
// token traffic.
void mfma_split(const FwdArgs& a, int* G_out, int* cps_out) {
    const int64_t units = a.B * a.H * a.nseg;
    const int64_t Lseg = a.L / a.nseg;
    const int64_t nch = (Lseg + C - 1) / C;
    int64_t cps;
    if (a.subseg_chunks > 0) {
        cps = a.subseg_chunks;
    } else {
        const int64_t target = 256;
        const int64_t g_want = (target + units - 1) / units;
        cps = (nch + g_want - 1) / g_want;
        if (cps < 4) cps = 4;
    }
    if (cps > nch) cps = nch > 0 ? nch : 1;
    *G_out = (int)((nch + cps - 1) / cps);
    if (*G_out < 1) *G_out = 1;
    *cps_out = (int)cps;
}

hipError_t launch_chunk_fwd_mfma(const FwdArgs& a) {
    int G, cps;
    mfma_split(a, &G, &cps);
    float* part_state = nullptr;
    float* part_decay = nullptr;
    hipMemPool_t pool = nullptr;
    if (G > 1) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        pool = workspace_pool(dev);
        if (!pool) return hipErrorOutOfMemory;
        const size_t n = (size_t)(a.B * a.H * a.nseg) * (G - 1);
        e = hipMallocFromPoolAsync((void**)&part_state, n * D * D * sizeof(float) + n * D * sizeof(float), pool,
                                   a.stream);
        if (e != hipSuccess) return e;
        part_decay = part_state + n * D * D;
    }
    hipError_t e;
    switch (a.mode) {
        case DECAY_HEAD: e = launch_chunk_fwd_pipe(a, G, cps, part_state, part_decay); break;
        case DECAY_GATE: e = launch_mode<DECAY_GATE>(a, G, cps, part_state, part_decay); break;
        default: e = launch_chunk_fwd_pipe(a, G, cps, part_state, part_decay); break;
    }
    if (part_state) {
        hipError_t f = hipFreeAsync(part_state, a.stream);
        if (e == hipSuccess) e = f;
    }
    return e;
}

}  // namespace la
