// chunk_bwd_mfma_impl.h -- bf16 matrix-core (MFMA) backward pass for dk = dv = 32, 64 or 128, chunk 64,
// with no decay or one decay per head (the backward pass the ZeCO review page lists as a consequence of the
// forward design, pith_extraction.forward_implications).  With a scalar decay per head the weight
// of token j in output t is a^{t-j} whatever the key dim.
//
// dq runs forwards in time with the forward state S (dq_t = S_t d_o_t); dk and dv run backwards
// with the state derivative D (G_t of the recurrence).  Each segment is split into G sub-segments
// so that about 256 workgroups share the work; the decomposition identity of the same page
// (pith_extraction.key_machinery) joins them: a state pass leaves each sub-segment's local state
// (forwards: from zero, sub-segment 0 from s_in) or local derivative (backwards: from zero, the last
// sub-segment from ds_out), a scan over them with each sub-segment's total decay (in reverse order
// for D) gives every sub-segment its exact incoming state or derivative, and the output pass walks
// each sub-segment from it.  Per chunk of n tokens:
//   forwards (S = the state before the chunk):
//     P'[i][j] = d_o_i . v_j a^{i-j}  (j <= i),      dq_i = sum_j P'[i][j] k_j + a^{i+1} S d_o_i
//     S <- a^n S + sum_j a^{n-1-j} k_j v_j^T
//   backwards (D = the derivative at the chunk's end):
//     P'[i][j] as above, P[i][j] = q_i . k_j a^{i-j}  (j <= i)
//     dk_j = sum_{i>=j} P'[i][j] q_i + a^{n-1-j} D v_j,   dv_j = sum_{i>=j} P[i][j] d_o_i + a^{n-1-j} D^T k_j
//     D <- a^n D + sum_i a^{i+1} q_i d_o_i^T
// The head-decay derivative is not taken from q . dq - k . dk (whose terms cancel by a factor that
// grows with the sequence length over the decay length, beyond what the bf16 operands of these
// products carry) but summed pair by pair with dS/dlambda carried beside S (bwd_dlam_kernel).
//
// Wave roles (both directions): wave w keeps value-column block cb = w % (D / 32) of S or D (all key
// rows) in MFMA accumulators and computes the 32-wide column block cb of dq / dk / dv for its share of
// the chunk's row blocks; the causal 32x32 score blocks are shared out; the state's transpose reaches
// the products that need it through a bf16 copy in LDS.
#pragma once
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int C = 64;          // chunk length
constexpr int NT = 256;        // lanes per workgroup
constexpr int PPITCH = C + 8;  // bf16 row pitch of the transposed score tiles

// Sizes per head dim D (= dk = dv: 32, 64 or 128).  The D / 32 value-column blocks of every state
// are spread over the four waves: wave w keeps block cb = w % NCB, and when blocks are fewer than
// waves (D = 32, 64) the waves of a block keep identical copies of its state columns (more
// matrix-core work, no state traffic through LDS); they split that block's output row blocks by
// rank = w / NCB, and only rank 0 writes shared copies, final states and partial sums.
template <int D>
struct Geo {
    static constexpr int PITCH = D + 8;          // bf16 row pitch of the tiles: 16-byte aligned, conflict-free rows
    static constexpr int TILE = C * PITCH;
    static constexpr int PR = C * D / 8 / NT;    // 16-byte pieces of a bf16 chunk tile per lane
    static constexpr int PIECES_ROW = D / 8;
    static constexpr int NCB = D / 32;           // value-column blocks
    static constexpr int WPC = 4 / NCB;          // waves per column block
    static_assert(TILE % 8 == 0 && (D * PITCH) % 8 == 0 && (C * PPITCH) % 8 == 0, "16-byte tiles");
    static_assert(PR >= 1 && NCB >= 1, "head dim");
    // output row block rb of a chunk (two of 32 rows) is computed by the waves of rank rb % WPC
    __device__ __forceinline__ static bool owns_rows(int rb, int rank) { return rb % WPC == rank % WPC && !(WPC > 2 && rank >= 2); }
};

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
__device__ __forceinline__ u32x4 scale8s(u32x4 w, float f) {
    const float ff[8] = {f, f, f, f, f, f, f, f};
    return scale8(w, ff);
}
// Operand of 16 consecutive tile rows (the contraction index) and 32 columns starting at col0,
// read transposed: element e of lane (G16, i16) is tile[16 ks + (G16 >> 1) 8 + (i16 >> 2) + 4 (e >> 2)]
// [col0 + (G16 & 1) 16 + (i16 & 3) 4 + (e & 3)].
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* tile, int pitch, int ks, int col0, int lane) {
    const int G16 = lane >> 4, i16 = lane & 15;
    const int col = col0 + (G16 & 1) * 16 + (i16 & 3) * 4;
    const int tb = 16 * ks + (G16 >> 1) * 8 + (i16 >> 2);
    return cat(lds_tr16(&tile[tb * pitch + col]), lds_tr16(&tile[(tb + 4) * pitch + col]));
}

// Gate mode: a chunk's raw gate rows [C][D] (fp32) in registers, PG 16-byte pieces per lane, rows
// past the chunk's end as zero.  The loads are issued together and converted only later (inside
// the conversion each piece's use would follow its own load and wait).
template <int D>
struct GateTile {
    static constexpr int PG = C * D / 4 / NT;
};

template <int D>
__device__ __forceinline__ void gate_load(const float* __restrict__ g, int64_t row0, int n, f32x4* rg, int tid) {
#pragma unroll
    for (int r = 0; r < GateTile<D>::PG; r++) {
        const int p = tid + NT * r;
        const int row = p / (D / 4), c4 = (p % (D / 4)) * 4;
        rg[r] = row < n ? *(const f32x4*)(g + (row0 + row) * D + c4) : f32x4{0, 0, 0, 0};
    }
}

// The per-token log2-decay, log2 a = -softplus(-g) / gate_norm * log2(e), of the chunk's rows s0 ..
// s1 - 1 from its gate tile rg (rows past the chunk's end read as zero), into gb rows 0 .. s1 - s0 - 1
// (chunk row r at row (r - s0) mod C; every other row 0), then replaced by its inclusive running sum
// B (per key dim), in NT / D parts of C * D / NT rows; gel[d] = 2^{B_last[d]} is the decay over the
// rows.  A whole chunk is s0 = 0, s1 = n.  Every factor built from B later on is 2^{B} <= 1, 2^{-B}
// or 2^{B_last - B} <= 1; 2^{-B} stays within 2^GATE_SPAN_LOG2 when the rows' decay does, which
// the callers ensure by cutting a chunk into windows where it does not (chunk_gate_windows).
template <int D>
__device__ __forceinline__ void gate_chunk_logdecay(const f32x4* rg, int s0, int s1, float inv_norm, float* gb,
                                                    float* gtot, float* gel, int tid) {
#pragma unroll
    for (int r = 0; r < GateTile<D>::PG; r++) {
        const int p = tid + NT * r;
        const int row = p / (D / 4), c4 = (p % (D / 4)) * 4;
        const f32x4 x = rg[r];
        const bool in = row >= s0 && row < s1;
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; e++) y[e] = in ? gate_logdecay(x[e], inv_norm) * LOG2E : 0.f;
        *(f32x4*)(&gb[((row - s0) & (C - 1)) * D + c4]) = y;
    }
    __syncthreads();
    constexpr int NPART = NT / D, R = C / NPART;
    const int d = tid % D, part = tid / D;
    float vals[R];
#pragma unroll
    for (int i = 0; i < R; i++) vals[i] = gb[(part * R + i) * D + d];
#pragma unroll
    for (int i = 1; i < R; i++) vals[i] += vals[i - 1];
    gtot[part * D + d] = vals[R - 1];
    __syncthreads();
    float off = 0.f;
    for (int pp = 0; pp < part; pp++) off += gtot[pp * D + d];
#pragma unroll
    for (int i = 0; i < R; i++) gb[(part * R + i) * D + d] = vals[i] + off;
    __syncthreads();
    if (tid < D) gel[tid] = __builtin_amdgcn_exp2f(gb[(C - 1) * D + tid]);
}

// The window length (tokens) at which a gate chunk of n tokens is taken, from its whole-chunk running
// sums gb (gate_chunk_logdecay over rows 0 .. n - 1): the chunk itself when its decay stays within
// 2^GATE_SPAN_LOG2 on every key dim (the common case), else the longest C >> lv whose windows' decays,
// their first token included, each stay within it (two tokens always do, given the floor on log a).
// The result is read from *lvl after the caller's next barrier; *lvl must be 0 before this call.
template <int D>
__device__ __forceinline__ void chunk_gate_windows(const float* gb, int n, int* lvl, int tid) {
    if (tid >= D || gb[(C - 1) * D + tid] >= -GATE_SPAN_LOG2) return;
    int lv = 1;
    for (; (C >> lv) > 1; lv++) {
        const int wl = C >> lv;
        bool fits = true;
        for (int s0 = 0; s0 < n && fits; s0 += wl) {
            const float base = s0 ? gb[(s0 - 1) * D + tid] : 0.f;
            fits = gb[(min(s0 + wl, n) - 1) * D + tid] - base >= -GATE_SPAN_LOG2;
        }
        if (fits) break;
    }
    atomicMax(lvl, lv);
}

// LDS of the backward-direction kernel; the state pass keeps only the tiles of the D update.
template <int D, int MODE, bool SO>
struct BwdSmem {
    static constexpr int TILE = Geo<D>::TILE, PITCH = Geo<D>::PITCH;
    static constexpr bool GATE = MODE == DECAY_GATE;
    // unused tiles shrink to 8 elements, which keeps every tile 16-byte aligned
    __bf16 q[(SO || GATE) ? 8 : TILE];
    // q_i a^{i+1} (head mode), q 2^{B} (gate), q (state pass): the D update (and gate's P)
    __bf16 qs[(MODE != DECAY_NONE || SO) ? TILE : 8];
    __bf16 k[SO ? 8 : TILE];
    __bf16 v[SO ? 8 : TILE];
    __bf16 o[TILE];                  // d_o
    __bf16 dm[SO ? 8 : D * PITCH];   // D^T as bf16, [value column][key row]
    __bf16 pt[SO ? 8 : C * PPITCH];  // (P' w)^T: [j][i]
    __bf16 pv[SO ? 8 : C * PPITCH];  // (P w)^T:  [j][i]
    float gb[GATE ? C * D : 4];      // gate: in-chunk cumulative log2-decay B, then 2^{-B}
    float gtot[GATE ? NT : 4];
    float gel[GATE ? D : 4];         // gate: 2^{B_last}
    float apow[C + 1];               // a^m, m = 0..C (head mode)
    double red[NT / 64];
    int lvl;                         // gate: the chunk is taken in windows of C >> lvl tokens
};

// The chunk walk prefetches the next chunk (in walk order) into registers while the current one is
// computed (PF; off, each chunk is loaded at its top).
// WIN (gate mode): the instance that cuts chunks into windows; it redoes only the units (workgroups)
// whose wide[] flag the plain instance set when it met a chunk too wide for one piece, and the plain
// instance stops such a unit there (the redo overwrites everything the unit writes).
// FACT (head decay, output pass, no d lambda_h): the factorised walk, for the heads whose a^-C is
// finite (lambda C log2(e) >= -100); the instance without it takes the other heads (and all of them
// when d lambda_h is wanted), every workgroup leaving at once when its head is the other instance's.
// With q~_i = q_i a^{i+1} (already staged for the D update) and D first decayed, D' = a^n D:
//   dk_j = a^{-(j+1)} (D' v_j + sum_{i>=j} p'_ij q~_i),  dv_j = a^{-(j+1)} (D'^T k_j + sum_{i>=j} (q~_i . k_j) d_o_i),
//   D <- D' + q~^T d_o,
// so the scores take only the causal mask, and q itself need not be staged.
template <int D, int MODE, bool STATE_ONLY, bool WIN, bool FACT>
__device__ __forceinline__ void bwd_dkdv_body(
    BwdSmem<D, MODE, STATE_ONLY>& sm,
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ decay, const float* __restrict__ ds_out,
    int64_t sstride, __bf16* __restrict__ dk_out, __bf16* __restrict__ dv_out, float* __restrict__ ds_in,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // state pass outputs
    const float* __restrict__ init_state,                            // output pass: scanned D^(g)
    double* __restrict__ intra_part,  // head mode, output pass: the intra-chunk part of d lambda_h, or null
    __bf16* __restrict__ d_start,     // output pass, gate derivative: D^T at every chunk's start (bf16 [D][D]), or null
    int64_t H, int64_t L, int nseg, int G, int cps, float inv_norm, int* __restrict__ wide) {
    if constexpr (MODE == DECAY_GATE) {
        if constexpr (WIN) {
            if (wide[blockIdx.x] == 0) return;
        } else if (threadIdx.x == 0) {
            wide[blockIdx.x] = 0;
        }
    }
    using Gm = Geo<D>;
    constexpr int PITCH = Gm::PITCH, PR = Gm::PR, PIECES_ROW = Gm::PIECES_ROW, NCB = Gm::NCB;
    constexpr bool PF = true;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int cb = (Gm::WPC == 1) ? w : w % NCB, rank = (Gm::WPC == 1) ? 0 : w / NCB;
    const int lane = tid & 63;
    const int n32 = lane & 31;
    const int kg = lane >> 5;
    const int64_t u = blockIdx.x;
    const int gper = STATE_ONLY ? (G - 1) : G;
    const int g = STATE_ONLY ? (int)(u % gper) + 1 : (int)(u % gper);  // the state pass covers 1..G-1
    const int64_t ub = u / gper;  // (bh, seg)
    const int seg = (int)(ub % nseg);
    const int64_t bh = ub / nseg;
    const int64_t h = bh % H;
    const int64_t Lseg = L / nseg;
    const int64_t tseg = (int64_t)seg * Lseg;
    const int64_t t_begin = tseg + (int64_t)g * cps * C;
    const int64_t t_end = min(t_begin + (int64_t)cps * C, tseg + Lseg);
    const int64_t row_base = bh * L;
    const float lam = (MODE == DECAY_HEAD) ? decay[h] : 0.f;
    const int64_t nch_seg = (Lseg + C - 1) / C;
    static_assert(!FACT || (MODE == DECAY_HEAD && !STATE_ONLY && !WIN), "the factorised walk: head output pass");
    if constexpr (MODE == DECAY_HEAD && !STATE_ONLY) {
        if ((!intra_part && lam * LOG2E * (float)C >= -100.f) != FACT) return;  // the other instance's head
    }

    // ---- D at the sub-segment's end: key rows 32 m + (i / 4) 8 + kg 4 + i % 4, value column 32 w + n32
    f32x16 Dm[NCB];
    {
        const float* src = nullptr;
        if (g == G - 1) {
            if (ds_out) src = ds_out + bh * sstride + (int64_t)seg * D * D;
        } else if (!STATE_ONLY) {
            src = init_state + (ub * (G - 1) + (G - 2 - g)) * (int64_t)D * D;
        }
#pragma unroll
        for (int m = 0; m < NCB; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                Dm[m][i] = src ? src[r * D + 32 * cb + n32] : 0.f;
            }
    }

    if (MODE == DECAY_HEAD && tid <= C) sm.apow[tid] = decay_pow(lam, tid);  // read after the loop's first barrier
    double hacc = 0.0;
    float gate_total = 0.f;  // gate: log2 of the sub-segment's decay so far, key dim tid (tid < D)
    const int nchunks = (int)((t_end - t_begin + C - 1) / C);
    // one chunk's tiles in registers (rows past the end read as zero); gate mode: the gate tile too,
    // prefetched with the others except in the d = 128 output pass, which has no registers left for
    // it (it would spill) and loads it at the chunk's start
    constexpr bool GPF = MODE == DECAY_GATE && !(D == 128 && !STATE_ONLY);
    u32x4 rq[PR], ro[PR], rk[STATE_ONLY ? 1 : PR], rv[STATE_ONLY ? 1 : PR];
    f32x4 rg[MODE == DECAY_GATE ? GateTile<D>::PG : 1];
    auto load_chunk = [&](int cc) {
        const int64_t t0c = t_begin + (int64_t)cc * C;
        const int nc = (int)min((int64_t)C, t_end - t0c);
        const u32x4 z = {0, 0, 0, 0};
        if (GPF) gate_load<D>(decay, row_base + t0c, nc, rg, tid);
#pragma unroll
        for (int r = 0; r < PR; r++) {
            const int p = tid + NT * r;
            const int row = p / PIECES_ROW, c8 = (p % PIECES_ROW) * 8;
            const int64_t off = (row_base + t0c + row) * D + c8;
            const bool ok = row < nc;
            rq[r] = ok ? *(const u32x4*)(q + off) : z;
            ro[r] = ok ? *(const u32x4*)(d_o + off) : z;
            if (!STATE_ONLY) {
                rk[r] = ok ? *(const u32x4*)(k + off) : z;
                rv[r] = ok ? *(const u32x4*)(v + off) : z;
            }
        }
    };
    if (PF && nchunks > 0) load_chunk(nchunks - 1);
    for (int c = nchunks - 1; c >= 0; c--) {
        const int64_t t0c = t_begin + (int64_t)c * C;
        const int nc = (int)min((int64_t)C, t_end - t0c);
        __syncthreads();  // the previous chunk is done with every LDS tile
        if (!PF) load_chunk(c);
        // gate mode: the chunk's running log2-decay, and the windows it is taken in (one, unless its
        // decay is too wide for the factorised pair weights; chunk_gate_windows)
        int ws = C;
        if (MODE == DECAY_GATE) {
            if (WIN && tid == 0) sm.lvl = 0;
            if (!GPF) gate_load<D>(decay, row_base + t0c, nc, rg, tid);
            gate_chunk_logdecay<D>(rg, 0, nc, inv_norm, sm.gb, sm.gtot, sm.gel, tid);
            if (tid < D) gate_total += sm.gb[(C - 1) * D + tid];
            if constexpr (WIN) {
                chunk_gate_windows<D>(sm.gb, nc, &sm.lvl, tid);
                __syncthreads();  // gel, lvl
                ws = C >> sm.lvl;
            } else {
                // a chunk too wide for one piece sends the unit to the windowed instance, which
                // overwrites all it writes (this instance finishes the unit all the same: its register
                // allocation is left exactly as without the check)
                if (tid < D && sm.gb[(C - 1) * D + tid] < -GATE_SPAN_LOG2) wide[blockIdx.x] = 1;
                __syncthreads();  // gel
            }
        }
        // The windows run backwards in time, each staged as a ragged chunk of its own (chunk row r at
        // tile row (r - s0) mod C, the rest zero) with its first token as the decay reference, from the
        // registers, which keep the chunk until its last window is staged (the next chunk's prefetch
        // waits until then).
        const int nwin = (MODE == DECAY_GATE && WIN) ? (nc + ws - 1) / ws : 1;
        for (int wi = 0; wi < nwin; wi++) {
        const int s0 = (MODE == DECAY_GATE && WIN) ? (nwin - 1 - wi) * ws : 0;
        const int n = (MODE == DECAY_GATE && WIN) ? min(s0 + ws, nc) - s0 : nc;
        const int64_t t0 = t0c + s0;
        if (MODE == DECAY_GATE && WIN && nwin > 1) {
            if (wi > 0) __syncthreads();  // the previous window is done with every LDS tile
            f32x4 xg[GateTile<D>::PG];  // the gate rows again (cached), not held across the windows
            gate_load<D>(decay, row_base + t0c, nc, xg, tid);
            gate_chunk_logdecay<D>(xg, s0, s0 + n, inv_norm, sm.gb, sm.gtot, sm.gel, tid);
            __syncthreads();  // gel
        }

        // ---- stage the chunk (window) and D as bf16
        auto stage = [&](auto fetch) {
#pragma unroll
            for (int r = 0; r < PR; r++) {
                const int p = tid + NT * r;
                const int row = p / PIECES_ROW, c8 = (p % PIECES_ROW) * 8;
                const int tr = (MODE == DECAY_GATE && WIN) ? (row - s0) & (C - 1) : row;
                const bool in = !(MODE == DECAY_GATE && WIN) || (row >= s0 && row < s0 + n);
                u32x4 xq, xo, xk, xv;
                fetch(r, row, c8, xq, xo, xk, xv);
                const u32x4 z = {0, 0, 0, 0};
                if (MODE == DECAY_GATE) {  // q 2^{B}; k 2^{-B}
                    float fq[8], fk[8];
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const float b = sm.gb[tr * D + c8 + e];
                        fq[e] = __builtin_amdgcn_exp2f(b);
                        fk[e] = __builtin_amdgcn_exp2f(-b);
                    }
                    *(u32x4*)(&sm.qs[tr * PITCH + c8]) = in ? scale8(xq, fq) : z;
                    if (!STATE_ONLY) *(u32x4*)(&sm.k[tr * PITCH + c8]) = in ? scale8(xk, fk) : z;
                } else if (MODE == DECAY_HEAD) {
                    *(u32x4*)(&sm.qs[row * PITCH + c8]) = scale8s(xq, sm.apow[row + 1]);
                } else if (STATE_ONLY) {
                    *(u32x4*)(&sm.qs[row * PITCH + c8]) = xq;
                }
                *(u32x4*)(&sm.o[tr * PITCH + c8]) = in ? xo : z;
                if (!STATE_ONLY) {
                    if (MODE != DECAY_GATE) {
                        if (!FACT) *(u32x4*)(&sm.q[row * PITCH + c8]) = xq;
                        *(u32x4*)(&sm.k[row * PITCH + c8]) = xk;
                    }
                    *(u32x4*)(&sm.v[tr * PITCH + c8]) = in ? xv : z;
                }
            }
        };
        stage([&](int r, int, int, u32x4& xq, u32x4& xo, u32x4& xk, u32x4& xv) {
            xq = rq[r];
            xo = ro[r];
            if (!STATE_ONLY) {
                xk = rk[r];
                xv = rv[r];
            }
        });
        if constexpr (FACT) {  // D' = a^n D: the chunk's outputs and the update start from it
            const float fh = sm.apow[n];
#pragma unroll
            for (int m = 0; m < NCB; m++)
#pragma unroll
                for (int i = 0; i < 16; i++) Dm[m][i] *= fh;
        }
        if (!STATE_ONLY && rank == 0) {  // D^T as bf16: this lane's value column, key rows in runs of four
#pragma unroll
            for (int m = 0; m < NCB; m++)
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++)
                    *(bf16x4*)(&sm.dm[(32 * cb + n32) * PITCH + 32 * m + g4 * 8 + kg * 4]) =
                        bf16x4{(__bf16)Dm[m][4 * g4], (__bf16)Dm[m][4 * g4 + 1], (__bf16)Dm[m][4 * g4 + 2],
                               (__bf16)Dm[m][4 * g4 + 3]};
        }
        __syncthreads();
        if (PF && c > 0 && wi == nwin - 1) load_chunk(c - 1);  // the previous chunk, while this one is computed
        if (!STATE_ONLY && d_start && c + 1 < nchunks && wi == 0) {  // D^T here = D^T at the start of chunk c + 1
            __bf16* dst = d_start + (ub * nch_seg + (int64_t)g * cps + c + 1) * D * D;
#pragma unroll
            for (int r = 0; r < (D * D / 8 + NT - 1) / NT; r++) {
                const int p = tid + NT * r;
                if (p < D * D / 8) {
                    const int row = p / (D / 8), c8 = (p % (D / 8)) * 8;
                    *(u32x4*)(dst + row * D + c8) = *(const u32x4*)(&sm.dm[row * PITCH + c8]);
                }
            }
        }
        if (MODE == DECAY_GATE && !STATE_ONLY) {  // B -> 2^{-B} (dk's per-key-dim factor); read after the next barrier
#pragma unroll
            for (int r = 0; r < C * D / NT; r++) sm.gb[tid + NT * r] = __builtin_amdgcn_exp2f(-sm.gb[tid + NT * r]);
        }
        // the q side of the D update: q a^{i+1} (head mode), else q itself
        const __bf16* qsd = (MODE != DECAY_NONE || STATE_ONLY) ? sm.qs : sm.q;

        // d_o operands of this wave's value columns for the four 16-token slabs
        bf16x8 ob[4];
#pragma unroll
        for (int ks = 0; ks < 4; ks++) ob[ks] = tr_operand(sm.o, PITCH, ks, 32 * cb, lane);

        if (!STATE_ONLY) {
            // ---- causal score blocks (row block = i, column block = j) (0,0), (1,0), (1,1) on waves 0, 1, 2,
            // P' and P of a block on the same wave: written transposed with the weight a^{i-j} and the
            // mask j <= i; head mode with intra_part also sums (i - j) a^{i-j} P[i][j] P'[i][j], the
            // intra-chunk token pairs' share of d lambda_h, from the unrounded scores
            if (w < 3) {
                const int ib = (w == 0) ? 0 : 1, jb = (w == 2) ? 1 : 0;
                f32x16 po = {}, pq = {};
#pragma unroll
                for (int ks = 0; ks < D / 16; ks++) {
                    const int ka = ks * 16 + kg * 8;
                    po = mfma(*(const bf16x8*)(&sm.o[(ib * 32 + n32) * PITCH + ka]),
                              *(const bf16x8*)(&sm.v[(jb * 32 + n32) * PITCH + ka]), po);
                    pq = mfma(*(const bf16x8*)(&(MODE == DECAY_GATE || FACT ? sm.qs : sm.q)[(ib * 32 + n32) * PITCH + ka]),
                              *(const bf16x8*)(&sm.k[(jb * 32 + n32) * PITCH + ka]), pq);
                }
                // a lane holds column j = jb 32 + n32 and rows i in four runs of four: one 8-byte
                // store per run into the transposed tiles
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    bf16x4 xo, xq;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int i = 4 * g4 + e;
                        const int row = ib * 32 + g4 * 8 + kg * 4 + e;  // i index
                        const int col = jb * 32 + n32;                   // j index
                        float wgt = (col > row) ? 0.f : 1.f;
                        if (MODE == DECAY_HEAD && !FACT) {
                            wgt *= sm.apow[max(row - col, 0)];
                            if (intra_part && col < row) hacc += (double)((float)(row - col) * wgt) * ((double)po[i] * (double)pq[i]);
                        }
                        xo[e] = (__bf16)(po[i] * wgt);
                        xq[e] = (__bf16)(pq[i] * wgt);
                    }
                    const int off = (jb * 32 + n32) * PPITCH + ib * 32 + g4 * 8 + kg * 4;
                    *(bf16x4*)(&sm.pt[off]) = xo;
                    *(bf16x4*)(&sm.pv[off]) = xq;
                }
            }
            __syncthreads();  // score tiles complete

            // ---- dk, column block w (key dims 32 w ..), and dv, column block w (value columns 32 w ..)
            bf16x8 qb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ks++) qb[ks] = tr_operand(MODE == DECAY_GATE || FACT ? sm.qs : sm.q, PITCH, ks, 32 * cb, lane);
            // D's own columns as B operands (key-row order permuted as the A reads below)
            bf16x8 db[2 * NCB];
#pragma unroll
            for (int m = 0; m < NCB; m++)
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    bf16x8 x;
#pragma unroll
                    for (int j = 0; j < 8; j++) {
                        float dv_ = Dm[m][8 * hh + j];
                        if (MODE == DECAY_GATE)  // gate: D's rows times 2^{B_last}, so that K-hat D = K-tilde D
                            dv_ *= sm.gel[32 * m + ((8 * hh + j) >> 2) * 8 + kg * 4 + (j & 3)];
                        x[j] = (__bf16)dv_;
                    }
                    db[2 * m + hh] = x;
                }
            // dk and dv are formed transposed (feature dims x tokens), with the operands of each
            // product swapped: a lane then holds token j = jb 32 + n32 and 16 feature dims in four
            // runs of four, stored 8 bytes at a time
#pragma unroll
            for (int jb = 0; jb < 2; jb++) {
                if (!Gm::owns_rows(jb, rank)) continue;
                const int jt = jb * 32 + n32;  // this lane's token
                const float wj = (MODE == DECAY_HEAD) ? sm.apow[max(n - 1 - jt, 0)] : 1.f;
                // FACT: a^-(j+1), at most 2^100 by the bound on lambda
                const float ainv = FACT ? __builtin_amdgcn_exp2f(-lam * LOG2E * (float)(jt + 1)) : 1.f;
                // dk^T: a^{n-1-j} (D V^T) + Q^T (P' w)
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < D / 16; ks++) {
                    const bf16x8 a = tr_operand(sm.dm, PITCH, ks, 32 * cb, lane);  // D rows, from D^T
                    const bf16x8 b = *(const bf16x8*)(&sm.v[jt * PITCH + ks * 16 + kg * 8]);
                    acc = mfma(a, b, acc);
                }
                if (MODE == DECAY_HEAD && !FACT) {
#pragma unroll
                    for (int i = 0; i < 16; i++) acc[i] *= wj;
                }
                if (MODE == DECAY_GATE) {
#pragma unroll
                    for (int i = 0; i < 16; i++) acc[i] *= sm.gel[32 * cb + (i >> 2) * 8 + kg * 4 + (i & 3)];
                }
#pragma unroll
                for (int ks = 2 * jb; ks < 4; ks++) {
                    const bf16x8 b = *(const bf16x8*)(&sm.pt[jt * PPITCH + ks * 16 + kg * 8]);
                    acc = mfma(qb[ks], b, acc);
                }
                if (MODE == DECAY_GATE) {  // dk_j = 2^{-B_j} (2^{B_last} D V^T + Q-bar^T P')_j, per key dim
#pragma unroll
                    for (int i = 0; i < 16; i++) acc[i] *= sm.gb[jt * D + 32 * cb + (i >> 2) * 8 + kg * 4 + (i & 3)];
                }
                if constexpr (FACT) {
#pragma unroll
                    for (int i = 0; i < 16; i++) acc[i] *= ainv;
                }
                if (jt < n) {
                    __bf16* drow = dk_out + (row_base + t0 + jt) * D + 32 * cb + kg * 4;
#pragma unroll
                    for (int g4 = 0; g4 < 4; g4++)
                        *(bf16x4*)(drow + g4 * 8) = bf16x4{(__bf16)acc[4 * g4], (__bf16)acc[4 * g4 + 1],
                                                           (__bf16)acc[4 * g4 + 2], (__bf16)acc[4 * g4 + 3]};
                }
                // dv^T: a^{n-1-j} (D^T K^T) + d_o^T (P w)
                acc = f32x16{};
                const __bf16* krow = &sm.k[jt * PITCH + kg * 4];
#pragma unroll
                for (int m = 0; m < NCB; m++)
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
                        const int d0 = 32 * m + 16 * hh;
                        acc = mfma(db[2 * m + hh], cat(*(const bf16x4*)(krow + d0), *(const bf16x4*)(krow + d0 + 8)),
                                   acc);
                    }
                if (MODE == DECAY_HEAD && !FACT) {
#pragma unroll
                    for (int i = 0; i < 16; i++) acc[i] *= wj;
                }
#pragma unroll
                for (int ks = 2 * jb; ks < 4; ks++) {
                    const bf16x8 b = *(const bf16x8*)(&sm.pv[jt * PPITCH + ks * 16 + kg * 8]);
                    acc = mfma(ob[ks], b, acc);
                }
                if constexpr (FACT) {
#pragma unroll
                    for (int i = 0; i < 16; i++) acc[i] *= ainv;
                }
                if (jt < n) {
                    __bf16* vrow = dv_out + (row_base + t0 + jt) * D + 32 * cb + kg * 4;
#pragma unroll
                    for (int g4 = 0; g4 < 4; g4++)
                        *(bf16x4*)(vrow + g4 * 8) = bf16x4{(__bf16)acc[4 * g4], (__bf16)acc[4 * g4 + 1],
                                                           (__bf16)acc[4 * g4 + 2], (__bf16)acc[4 * g4 + 3]};
                }
            }
        }

        // ---- D <- a^n D + (q a^{i+1})^T d_o (FACT: D is a^n D already)
        {
            const float fh = (MODE == DECAY_HEAD) ? sm.apow[n] : 1.f;
#pragma unroll
            for (int m = 0; m < NCB; m++) {
                if (MODE == DECAY_HEAD && !FACT) {
#pragma unroll
                    for (int i = 0; i < 16; i++) Dm[m][i] *= fh;
                }
                if (MODE == DECAY_GATE) {
#pragma unroll
                    for (int i = 0; i < 16; i++) Dm[m][i] *= sm.gel[32 * m + (i >> 2) * 8 + kg * 4 + (i & 3)];
                }
#pragma unroll
                for (int ks = 0; ks < 4; ks++) Dm[m] = mfma(tr_operand(qsd, PITCH, ks, 32 * m, lane), ob[ks], Dm[m]);
            }
        }
        }  // windows
    }

    // ---- the derivative at the sub-segment's start
    float* dst = nullptr;
    if (STATE_ONLY) dst = part_state + (ub * (G - 1) + (G - 1 - g)) * (int64_t)D * D;
    else if (g == 0 && ds_in) dst = ds_in + bh * sstride + (int64_t)seg * D * D;
    if (dst && rank == 0) {
#pragma unroll
        for (int m = 0; m < NCB; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                dst[r * D + 32 * cb + n32] = Dm[m][i];
            }
    }
    if (!STATE_ONLY && d_start && nchunks > 0 && rank == 0) {  // ... which is D at its first chunk's start (D^T)
        __bf16* dsd = d_start + (ub * nch_seg + (int64_t)g * cps) * D * D;
#pragma unroll
        for (int m = 0; m < NCB; m++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++)
                *(bf16x4*)(dsd + (32 * cb + n32) * D + 32 * m + g4 * 8 + kg * 4) =
                    bf16x4{(__bf16)Dm[m][4 * g4], (__bf16)Dm[m][4 * g4 + 1], (__bf16)Dm[m][4 * g4 + 2],
                           (__bf16)Dm[m][4 * g4 + 3]};
    }
    if (STATE_ONLY && tid < D) {  // the total decay over this sub-segment, per key dim
        float tot = 1.f;
        if (MODE == DECAY_HEAD) tot = decay_pow(lam, (int)(t_end - t_begin));
        if (MODE == DECAY_GATE) tot = __builtin_amdgcn_exp2f(gate_total);
        part_decay[(ub * (G - 1) + (G - 1 - g)) * D + tid] = tot;
    }
    if (MODE == DECAY_HEAD && !STATE_ONLY && intra_part) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) hacc += __shfl_xor(hacc, off);
        __syncthreads();
        if (lane == 0) sm.red[w] = hacc;
        __syncthreads();
        if (tid == 0) intra_part[ub * G + g] = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
    }
}

template <int D, int MODE, bool STATE_ONLY, bool WIN = false, bool FACT = false>
__global__ __launch_bounds__(NT) void bwd_dkdv_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ decay, const float* __restrict__ ds_out,
    int64_t sstride, __bf16* __restrict__ dk_out, __bf16* __restrict__ dv_out, float* __restrict__ ds_in,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // state pass outputs
    const float* __restrict__ init_state,                            // output pass: scanned D^(g)
    double* __restrict__ intra_part,  // head mode, output pass: the intra-chunk part of d lambda_h, or null
    __bf16* __restrict__ d_start,     // output pass, gate derivative: D^T at every chunk's start (bf16 [D][D]), or null
    int64_t H, int64_t L, int nseg, int G, int cps, float inv_norm, int* __restrict__ wide) {
    __shared__ __attribute__((aligned(16))) BwdSmem<D, MODE, STATE_ONLY> sm;
    bwd_dkdv_body<D, MODE, STATE_ONLY, WIN, FACT>(sm, q, k, v, d_o, decay, ds_out, sstride, dk_out, dv_out, ds_in, part_state, part_decay, init_state, intra_part,
        d_start, H, L, nseg, G, cps, inv_norm, wide);
}

// Gate mode: the plain walk, then the windowed one for a unit the plain walk flagged (as for
// bwd_dq_gate_kernel).
template <int D, bool STATE_ONLY>
__global__ __launch_bounds__(NT) void bwd_dkdv_gate_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ decay, const float* __restrict__ ds_out,
    int64_t sstride, __bf16* __restrict__ dk_out, __bf16* __restrict__ dv_out, float* __restrict__ ds_in,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // state pass outputs
    const float* __restrict__ init_state,                            // output pass: scanned D^(g)
    double* __restrict__ intra_part,  // head mode, output pass: the intra-chunk part of d lambda_h, or null
    __bf16* __restrict__ d_start,     // output pass, gate derivative: D^T at every chunk's start (bf16 [D][D]), or null
    int64_t H, int64_t L, int nseg, int G, int cps, float inv_norm, int* __restrict__ wide) {
    __shared__ __attribute__((aligned(16))) BwdSmem<D, DECAY_GATE, STATE_ONLY> sm;
    bwd_dkdv_body<D, DECAY_GATE, STATE_ONLY, false, false>(sm, q, k, v, d_o, decay, ds_out, sstride, dk_out, dv_out, ds_in, part_state, part_decay, init_state, intra_part,
        d_start, H, L, nseg, G, cps, inv_norm, wide);
    __syncthreads();
    if (__hip_atomic_load(wide + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
        bwd_dkdv_body<D, DECAY_GATE, STATE_ONLY, true, false>(sm, q, k, v, d_o, decay, ds_out, sstride, dk_out, dv_out, ds_in, part_state, part_decay, init_state, intra_part,
        d_start, H, L, nseg, G, cps, inv_norm, wide);
}

// Head decay, output pass, d lambda_h not wanted: both walks in one launch, every workgroup taking
// the one its head's decay allows (the factorised walk when lambda C log2(e) >= -100, the test the
// body itself makes), so no launch is spent on workgroups that all leave.
template <int D>
__global__ __launch_bounds__(NT) void bwd_dkdv_head_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ decay, const float* __restrict__ ds_out,
    int64_t sstride, __bf16* __restrict__ dk_out, __bf16* __restrict__ dv_out, float* __restrict__ ds_in,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // state pass outputs
    const float* __restrict__ init_state,                            // output pass: scanned D^(g)
    double* __restrict__ intra_part,  // head mode, output pass: the intra-chunk part of d lambda_h, or null
    __bf16* __restrict__ d_start,     // output pass, gate derivative: D^T at every chunk's start (bf16 [D][D]), or null
    int64_t H, int64_t L, int nseg, int G, int cps, float inv_norm, int* __restrict__ wide) {
    __shared__ __attribute__((aligned(16))) BwdSmem<D, DECAY_HEAD, false> sm;
    const int64_t h = ((int64_t)blockIdx.x / G / nseg) % H;  // unit (bh, seg, g) of the output pass
    if (decay[h] * LOG2E * (float)C >= -100.f)
        bwd_dkdv_body<D, DECAY_HEAD, false, false, true>(sm, q, k, v, d_o, decay, ds_out, sstride, dk_out, dv_out, ds_in, part_state, part_decay, init_state, intra_part,
        d_start, H, L, nseg, G, cps, inv_norm, wide);
    else
        bwd_dkdv_body<D, DECAY_HEAD, false, false, false>(sm, q, k, v, d_o, decay, ds_out, sstride, dk_out, dv_out, ds_in, part_state, part_decay, init_state, intra_part,
        d_start, H, L, nseg, G, cps, inv_norm, wide);
}


// LDS of the forward-direction kernel; the state pass keeps only the tiles of the state update.
template <int D, int MODE, bool SO>
struct DqSmem {
    static constexpr int TILE = Geo<D>::TILE, PITCH = Geo<D>::PITCH;
    static constexpr bool GATE = MODE == DECAY_GATE;
    // unused tiles shrink to 8 elements, which keeps every tile 16-byte aligned
    __bf16 o[SO ? 8 : TILE];  // d_o
    __bf16 v[TILE];
    __bf16 k[SO ? 8 : TILE];  // k (the P' K product); gate: k 2^{-B}
    // k_j a^{n-1-j} (the state update); gate: k 2^{B_last - B}; without decay the output pass
    // reads k itself
    __bf16 kt[(MODE == DECAY_NONE && !SO) ? 8 : TILE];
    __bf16 sm[SO ? 8 : D * PITCH];  // S^T as bf16, [value column][key row]
    __bf16 p[SO ? 8 : C * PPITCH];  // P' w, [i][j]
    float gb[GATE ? C * D : 4];     // gate: in-chunk cumulative log2-decay
    float gtot[GATE ? NT : 4];
    float gel[GATE ? D : 4];        // gate: 2^{B_last}
    float apow[C + 1];              // a^m, m = 0..C (head mode)
    int lvl;                        // gate: the chunk is taken in windows of C >> lvl tokens
};

// WIN: as for bwd_dkdv_kernel.
template <int D, int MODE, bool STATE_ONLY, bool WIN>
__device__ __forceinline__ void bwd_dq_body(
    DqSmem<D, MODE, STATE_ONLY>& sm,
    const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ decay, const float* __restrict__ s_in,
    const float* __restrict__ ds_out, int64_t sstride, __bf16* __restrict__ dq,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // state pass outputs
    // output pass: the state entering sub-segment g >= 1 of (bh, seg) at
    // init_state + bh * ist_bh + (seg * ist_g + g + ist_off) * D * D (the scan buffer, or states the caller gives)
    const float* __restrict__ init_state, int64_t ist_bh, int ist_g, int ist_off,
    const __bf16* __restrict__ d_start,  // gate derivative: D^T at every chunk's start (bf16 [D][D]), or null
    float* __restrict__ c0_out,          // gate derivative: rowsum(S (.) D) at every chunk's start ([D])
    int64_t H, int64_t L, int nseg, int G, int cps, float inv_norm, int* __restrict__ wide) {
    if constexpr (MODE == DECAY_GATE) {
        if constexpr (WIN) {
            if (wide[blockIdx.x] == 0) return;
        } else if (threadIdx.x == 0) {
            wide[blockIdx.x] = 0;
        }
    }
    using Gm = Geo<D>;
    constexpr int PITCH = Gm::PITCH, PR = Gm::PR, PIECES_ROW = Gm::PIECES_ROW, NCB = Gm::NCB;
    constexpr bool PF = true;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int cb = (Gm::WPC == 1) ? w : w % NCB, rank = (Gm::WPC == 1) ? 0 : w / NCB;
    const int lane = tid & 63;
    const int n32 = lane & 31;
    const int kg = lane >> 5;
    const int64_t u = blockIdx.x;
    const int gper = STATE_ONLY ? (G - 1) : G;
    const int g = (int)(u % gper);  // the state pass covers 0..G-2
    const int64_t ub = u / gper;
    const int seg = (int)(ub % nseg);
    const int64_t bh = ub / nseg;
    const int64_t h = bh % H;
    const int64_t Lseg = L / nseg;
    const int64_t tseg = (int64_t)seg * Lseg;
    const int64_t t_begin = tseg + (int64_t)g * cps * C;
    const int64_t t_end = min(t_begin + (int64_t)cps * C, tseg + Lseg);
    const int64_t row_base = bh * L;
    const int64_t nch_seg = (Lseg + C - 1) / C;
    const float lam = (MODE == DECAY_HEAD) ? decay[h] : 0.f;
    float gate_total = 0.f;  // gate: log2 of the sub-segment's decay so far, key dim tid (tid < D)

    // ---- the state entering the sub-segment: key rows 32 m + (i / 4) 8 + kg 4 + i % 4, column 32 w + n32
    f32x16 Sm[NCB];
    {
        const float* src = nullptr;
        if (g == 0) {
            if (seg == 0 && s_in) src = s_in + bh * (int64_t)D * D;
        } else if (!STATE_ONLY) {
            src = init_state + bh * ist_bh + ((int64_t)seg * ist_g + g + ist_off) * D * D;
        }
#pragma unroll
        for (int m = 0; m < NCB; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                Sm[m][i] = src ? src[r * D + 32 * cb + n32] : 0.f;
            }
    }

    if (MODE == DECAY_HEAD && tid <= C) sm.apow[tid] = decay_pow(lam, tid);  // read after the loop's first barrier
    const int nchunks = (int)((t_end - t_begin + C - 1) / C);
    // one chunk's tiles in registers (rows past the end read as zero); gate mode: the gate tile too,
    // prefetched with the others
    u32x4 rk[PR], rv[PR], ro[STATE_ONLY ? 1 : PR];
    f32x4 rg[MODE == DECAY_GATE ? GateTile<D>::PG : 1];
    auto load_chunk = [&](int cc) {
        const int64_t t0c = t_begin + (int64_t)cc * C;
        const int nc = (int)min((int64_t)C, t_end - t0c);
        const u32x4 z = {0, 0, 0, 0};
        if (MODE == DECAY_GATE) gate_load<D>(decay, row_base + t0c, nc, rg, tid);
#pragma unroll
        for (int r = 0; r < PR; r++) {
            const int p = tid + NT * r;
            const int row = p / PIECES_ROW, c8 = (p % PIECES_ROW) * 8;
            const int64_t off = (row_base + t0c + row) * D + c8;
            const bool ok = row < nc;
            rk[r] = ok ? *(const u32x4*)(k + off) : z;
            rv[r] = ok ? *(const u32x4*)(v + off) : z;
            if (!STATE_ONLY) ro[r] = ok ? *(const u32x4*)(d_o + off) : z;
        }
    };
    if (PF && nchunks > 0) load_chunk(0);
    for (int c = 0; c < nchunks; c++) {
        const int64_t t0c = t_begin + (int64_t)c * C;
        const int nc = (int)min((int64_t)C, t_end - t0c);
        __syncthreads();  // the previous chunk is done with every LDS tile
        if (!PF) load_chunk(c);
        // gate derivative: this thread's part of D^T at the chunk's start (key dims 4 (tid % (D / 4))
        // .. + 3, value rows of part tid / (D / 4)), loaded here so that it arrives while the chunk
        // is staged
        constexpr int NPART = NT / (D / 4), RPP = D / NPART;  // parts of the value rows, rows per part
        bf16x4 dst4[STATE_ONLY ? 1 : RPP];
        const int64_t ci = ub * nch_seg + (int64_t)g * cps + c;
        if (!STATE_ONLY && c0_out) {
            const __bf16* src = d_start + (ci * D + (tid / (D / 4)) * RPP) * D + (tid % (D / 4)) * 4;
#pragma unroll
            for (int j = 0; j < RPP; j++) dst4[j] = *(const bf16x4*)(src + j * D);
        }
        // gate mode: the chunk's running log2-decay, and the windows it is taken in (one, unless its
        // decay is too wide for the factorised pair weights; chunk_gate_windows)
        int ws = C;
        if (MODE == DECAY_GATE) {
            if (WIN && tid == 0) sm.lvl = 0;
            gate_chunk_logdecay<D>(rg, 0, nc, inv_norm, sm.gb, sm.gtot, sm.gel, tid);
            if (tid < D) gate_total += sm.gb[(C - 1) * D + tid];
            if constexpr (WIN) {
                chunk_gate_windows<D>(sm.gb, nc, &sm.lvl, tid);
                __syncthreads();  // gel, lvl
                ws = C >> sm.lvl;
            } else {
                // a chunk too wide for one piece sends the unit to the windowed instance, which
                // overwrites all it writes (this instance finishes the unit all the same: its register
                // allocation is left exactly as without the check)
                if (tid < D && sm.gb[(C - 1) * D + tid] < -GATE_SPAN_LOG2) wide[blockIdx.x] = 1;
                __syncthreads();  // gel
            }
        }
        // The windows run forwards, each staged as a ragged chunk of its own (chunk row r at tile row
        // (r - s0) mod C, the rest zero) with its first token as the decay reference, from the
        // registers, which keep the chunk until its last window is staged.
        const int nwin = (MODE == DECAY_GATE && WIN) ? (nc + ws - 1) / ws : 1;
        for (int wi = 0; wi < nwin; wi++) {
        const int s0 = (MODE == DECAY_GATE && WIN) ? wi * ws : 0;
        const int n = (MODE == DECAY_GATE && WIN) ? min(s0 + ws, nc) - s0 : nc;
        const int64_t t0 = t0c + s0;
        if (MODE == DECAY_GATE && WIN && nwin > 1) {
            if (wi > 0) __syncthreads();  // the previous window is done with every LDS tile
            f32x4 xg[GateTile<D>::PG];  // the gate rows again (cached), not held across the windows
            gate_load<D>(decay, row_base + t0c, nc, xg, tid);
            gate_chunk_logdecay<D>(xg, s0, s0 + n, inv_norm, sm.gb, sm.gtot, sm.gel, tid);
            __syncthreads();  // gel
        }
        auto stage = [&](auto fetch) {
#pragma unroll
            for (int r = 0; r < PR; r++) {
                const int p = tid + NT * r;
                const int row = p / PIECES_ROW, c8 = (p % PIECES_ROW) * 8;
                const int tr = (MODE == DECAY_GATE && WIN) ? (row - s0) & (C - 1) : row;
                const bool in = !(MODE == DECAY_GATE && WIN) || (row >= s0 && row < s0 + n);
                u32x4 xk, xv, xo;
                fetch(r, row, c8, xk, xv, xo);
                const u32x4 z = {0, 0, 0, 0};
                *(u32x4*)(&sm.v[tr * PITCH + c8]) = in ? xv : z;
                if (MODE == DECAY_GATE) {
                    float ft[8], fh[8];
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const float b = sm.gb[tr * D + c8 + e];
                        ft[e] = __builtin_amdgcn_exp2f(sm.gb[(C - 1) * D + c8 + e] - b);
                        fh[e] = __builtin_amdgcn_exp2f(-b);
                    }
                    *(u32x4*)(&sm.kt[tr * PITCH + c8]) = in ? scale8(xk, ft) : z;
                    if (!STATE_ONLY) *(u32x4*)(&sm.k[tr * PITCH + c8]) = in ? scale8(xk, fh) : z;
                } else if (MODE == DECAY_HEAD) {
                    *(u32x4*)(&sm.kt[row * PITCH + c8]) = scale8s(xk, sm.apow[max(n - 1 - row, 0)]);
                } else if (STATE_ONLY) {
                    *(u32x4*)(&sm.kt[row * PITCH + c8]) = xk;
                }
                if (!STATE_ONLY) {
                    if (MODE != DECAY_GATE) *(u32x4*)(&sm.k[row * PITCH + c8]) = xk;
                    *(u32x4*)(&sm.o[tr * PITCH + c8]) = in ? xo : z;
                }
            }
        };
        stage([&](int r, int, int, u32x4& xk, u32x4& xv, u32x4& xo) {
            xk = rk[r];
            xv = rv[r];
            if (!STATE_ONLY) xo = ro[r];
        });
        if (!STATE_ONLY && rank == 0) {  // S^T as bf16: this lane's value column, key rows in runs of four
#pragma unroll
            for (int m = 0; m < NCB; m++)
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++)
                    *(bf16x4*)(&sm.sm[(32 * cb + n32) * PITCH + 32 * m + g4 * 8 + kg * 4]) =
                        bf16x4{(__bf16)Sm[m][4 * g4], (__bf16)Sm[m][4 * g4 + 1], (__bf16)Sm[m][4 * g4 + 2],
                               (__bf16)Sm[m][4 * g4 + 3]};
        }
        __syncthreads();
        if (PF && c + 1 < nchunks && wi == nwin - 1) load_chunk(c + 1);  // the next chunk, while this one is computed
        if (!STATE_ONLY && c0_out && wi == 0) {  // rowsum(S (.) D) at this chunk's start, per key dim, from S's bf16 copy
            // partial sums over this thread's value rows for its four key dims, then summed over the
            // parts through the score tile's LDS (free until the scores below are written)
            const int r4 = (tid % (D / 4)) * 4, part = tid / (D / 4);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < RPP; j++) {
                const bf16x4 ss = *(const bf16x4*)(&sm.sm[(part * RPP + j) * PITCH + r4]);
#pragma unroll
                for (int e = 0; e < 4; e++) acc[e] += (float)ss[e] * (float)dst4[j][e];
            }
            float* red = (float*)sm.p;  // [NPART][D]
            *(f32x4*)(&red[part * D + r4]) = acc;
            __syncthreads();
            if (tid < D) {
                float t = 0.f;
                for (int pp = 0; pp < NPART; pp++) t += red[pp * D + tid];
                c0_out[ci * D + tid] = t;
            }
            __syncthreads();  // the score tile is free again
        }

        bf16x8 vb[4];  // v operands of this wave's value columns, four 16-token slabs
#pragma unroll
        for (int ks = 0; ks < 4; ks++) vb[ks] = tr_operand(sm.v, PITCH, ks, 32 * cb, lane);

        if (!STATE_ONLY) {
            // ---- P' blocks (0,0), (1,0), (1,1) on waves 0, 2, 3: weight a^{i-j}, mask j <= i
            if (w != 1) {
                const int ib = w >> 1, jb = (w == 3) ? 1 : 0;
                // the block transposed (V d_o^T), so that a lane holds row i = ib 32 + n32 and columns
                // j in four runs of four: one 8-byte store per run
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < D / 16; ks++) {
                    const bf16x8 a = *(const bf16x8*)(&sm.v[(jb * 32 + n32) * PITCH + ks * 16 + kg * 8]);
                    const bf16x8 b = *(const bf16x8*)(&sm.o[(ib * 32 + n32) * PITCH + ks * 16 + kg * 8]);
                    acc = mfma(a, b, acc);
                }
                const int row = ib * 32 + n32;
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int col = jb * 32 + g4 * 8 + kg * 4 + e;
                        float val = acc[4 * g4 + e];
                        if (MODE == DECAY_HEAD) val *= sm.apow[max(row - col, 0)];
                        if (col > row) val = 0.f;
                        x[e] = (__bf16)val;
                    }
                    *(bf16x4*)(&sm.p[row * PPITCH + jb * 32 + g4 * 8 + kg * 4]) = x;
                }
            }
            __syncthreads();  // P' complete

            // ---- dq, column block w (key dims 32 w ..): a^{i+1} (d_o S^T) + P' K
            bf16x8 kb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ks++) kb[ks] = tr_operand(sm.k, PITCH, ks, 32 * cb, lane);
            // dq is formed transposed (key dims x tokens), the operands of each product swapped: a
            // lane holds token i = ib 32 + n32 and 16 key dims in four runs of four (8-byte stores)
#pragma unroll
            for (int ib = 0; ib < 2; ib++) {
                if (!Gm::owns_rows(ib, rank)) continue;
                const int it = ib * 32 + n32;  // this lane's token
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < D / 16; ks++) {
                    const bf16x8 a = tr_operand(sm.sm, PITCH, ks, 32 * cb, lane);  // S rows, from S^T
                    const bf16x8 b = *(const bf16x8*)(&sm.o[it * PITCH + ks * 16 + kg * 8]);
                    acc = mfma(a, b, acc);
                }
                if (MODE == DECAY_HEAD) {
                    const float f = sm.apow[it + 1];
#pragma unroll
                    for (int i = 0; i < 16; i++) acc[i] *= f;
                }
#pragma unroll
                for (int ks = 0; ks < 2 * (ib + 1); ks++) {
                    const bf16x8 b = *(const bf16x8*)(&sm.p[it * PPITCH + ks * 16 + kg * 8]);
                    acc = mfma(kb[ks], b, acc);
                }
                if (MODE == DECAY_GATE) {  // dq_i = 2^{B_i} (S d_o^T + Khat^T P'^T)_i, per key dim
#pragma unroll
                    for (int i = 0; i < 16; i++)
                        acc[i] *= __builtin_amdgcn_exp2f(sm.gb[it * D + 32 * cb + (i >> 2) * 8 + kg * 4 + (i & 3)]);
                }
                if (it < n) {
                    __bf16* qrow = dq + (row_base + t0 + it) * D + 32 * cb + kg * 4;
#pragma unroll
                    for (int g4 = 0; g4 < 4; g4++)
                        *(bf16x4*)(qrow + g4 * 8) = bf16x4{(__bf16)acc[4 * g4], (__bf16)acc[4 * g4 + 1],
                                                           (__bf16)acc[4 * g4 + 2], (__bf16)acc[4 * g4 + 3]};
                }
            }
        }

        // ---- S <- a^n S + (K a^{n-1-j})^T V  (gate: rows scaled by 2^{B_last})
        {
            const float fh = (MODE == DECAY_HEAD) ? sm.apow[n] : 1.f;
#pragma unroll
            for (int m = 0; m < NCB; m++) {
                if (MODE == DECAY_HEAD) {
#pragma unroll
                    for (int i = 0; i < 16; i++) Sm[m][i] *= fh;
                }
                if (MODE == DECAY_GATE) {
#pragma unroll
                    for (int i = 0; i < 16; i++) Sm[m][i] *= sm.gel[32 * m + (i >> 2) * 8 + kg * 4 + (i & 3)];
                }
#pragma unroll
                for (int ks = 0; ks < 4; ks++)
                    Sm[m] = mfma(tr_operand((MODE == DECAY_NONE && !STATE_ONLY) ? sm.k : sm.kt, PITCH, ks, 32 * m, lane),
                                 vb[ks], Sm[m]);
            }
        }
        }  // windows
    }

    if (STATE_ONLY && rank == 0) {
        float* dst = part_state + (ub * (G - 1) + g) * (int64_t)D * D;
#pragma unroll
        for (int m = 0; m < NCB; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                dst[r * D + 32 * cb + n32] = Sm[m][i];
            }
    }
    if (STATE_ONLY && tid < D) {
        float tot = 1.f;
        if (MODE == DECAY_HEAD) tot = decay_pow(lam, (int)(t_end - t_begin));
        if (MODE == DECAY_GATE) tot = __builtin_amdgcn_exp2f(gate_total);
        part_decay[(ub * (G - 1) + g) * D + tid] = tot;
    }
}

template <int D, int MODE, bool STATE_ONLY, bool WIN = false>
__global__ __launch_bounds__(NT) void bwd_dq_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ decay, const float* __restrict__ s_in,
    const float* __restrict__ ds_out, int64_t sstride, __bf16* __restrict__ dq,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // state pass outputs
    // output pass: the state entering sub-segment g >= 1 of (bh, seg) at
    // init_state + bh * ist_bh + (seg * ist_g + g + ist_off) * D * D (the scan buffer, or states the caller gives)
    const float* __restrict__ init_state, int64_t ist_bh, int ist_g, int ist_off,
    const __bf16* __restrict__ d_start,  // gate derivative: D^T at every chunk's start (bf16 [D][D]), or null
    float* __restrict__ c0_out,          // gate derivative: rowsum(S (.) D) at every chunk's start ([D])
    int64_t H, int64_t L, int nseg, int G, int cps, float inv_norm, int* __restrict__ wide) {
    __shared__ __attribute__((aligned(16))) DqSmem<D, MODE, STATE_ONLY> sm;
    bwd_dq_body<D, MODE, STATE_ONLY, WIN>(sm, k, v, d_o, decay, s_in, ds_out, sstride, dq, part_state, part_decay, init_state, ist_bh, ist_g,
        ist_off, d_start, c0_out, H, L, nseg, G, cps, inv_norm, wide);
}

// Gate mode: the plain walk and, for a unit it flagged as holding a chunk too wide for one piece,
// the windowed walk after it in the same workgroup (which overwrites all the plain walk wrote for
// the unit), instead of a second launch whose workgroups almost all leave.  The flag is read at
// device scope after the barrier that ends the plain walk.
template <int D, bool STATE_ONLY>
__global__ __launch_bounds__(NT) void bwd_dq_gate_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ decay, const float* __restrict__ s_in,
    const float* __restrict__ ds_out, int64_t sstride, __bf16* __restrict__ dq,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // state pass outputs
    // output pass: the state entering sub-segment g >= 1 of (bh, seg) at
    // init_state + bh * ist_bh + (seg * ist_g + g + ist_off) * D * D (the scan buffer, or states the caller gives)
    const float* __restrict__ init_state, int64_t ist_bh, int ist_g, int ist_off,
    const __bf16* __restrict__ d_start,  // gate derivative: D^T at every chunk's start (bf16 [D][D]), or null
    float* __restrict__ c0_out,          // gate derivative: rowsum(S (.) D) at every chunk's start ([D])
    int64_t H, int64_t L, int nseg, int G, int cps, float inv_norm, int* __restrict__ wide) {
    __shared__ __attribute__((aligned(16))) DqSmem<D, DECAY_GATE, STATE_ONLY> sm;
    bwd_dq_body<D, DECAY_GATE, STATE_ONLY, false>(sm, k, v, d_o, decay, s_in, ds_out, sstride, dq, part_state, part_decay, init_state, ist_bh, ist_g,
        ist_off, d_start, c0_out, H, L, nseg, G, cps, inv_norm, wide);
    __syncthreads();
    if (__hip_atomic_load(wide + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
        bwd_dq_body<D, DECAY_GATE, STATE_ONLY, true>(sm, k, v, d_o, decay, s_in, ds_out, sstride, dq, part_state, part_decay, init_state, ist_bh, ist_g,
        ist_off, d_start, c0_out, H, L, nseg, G, cps, inv_norm, wide);
}

// ---------------------------------------------------------------------------------------------
// The head-decay derivative, summed without cancellation.  Every pair of tokens j <= t contributes
// (t - j) a^{t-j} (q_t . k_j)(v_j . d_o_t) to d lambda_h (and s_in, seen as a token before the
// segment, and ds_out add their own terms).  Per chunk of n tokens, with S the state and
// St = dS/dlambda before it:
//   intra-chunk pairs  sum_{j<=i} (i - j) a^{i-j} P[i][j] P'[i][j]       (P = q k^T, P' = d_o v^T),
//                      summed by the dk/dv output pass, which forms both score matrices anyway
//   earlier tokens     <S, M'> + <St, M>,   M = sum_i a^{i+1} q_i d_o_i^T,   M' = sum_i (i+1) a^{i+1} q_i d_o_i^T
//   St <- a^n St + n a^n S + sum_j (n-1-j) a^{n-1-j} k_j v_j^T,   S <- a^n S + sum_j a^{n-1-j} k_j v_j^T
// and <ds_out, St> at the segment's end.  Sub-segments compose as S_out = A S_in + S_loc and
// St_out = A St_in + l A S_in + St_loc (A = a^l over l tokens): a state pass leaves (S_loc, St_loc),
// the S scan runs first, a fix-up adds l A S_in to each St_loc, and the St scan follows.
template <int D, bool SO>
struct DlamSmem {
    static constexpr int TILE = Geo<D>::TILE;
    // the state pass keeps only v and the scaled k tiles (the others shrink to 16-byte stubs)
    __bf16 v[TILE];
    __bf16 o[SO ? 8 : TILE];
    __bf16 qs[SO ? 8 : TILE];   // q_i a^{i+1}
    __bf16 qs2[SO ? 8 : TILE];  // q_i (i+1) a^{i+1}
    __bf16 kt[TILE];            // k_j a^{n-1-j}
    __bf16 kt2[TILE];           // k_j (n-1-j) a^{n-1-j}
    float apow[C + 1];
    double red[NT / 64];
};

template <int D, bool STATE_ONLY>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dlam_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ decay, const float* __restrict__ s_in,
    const float* __restrict__ ds_out, int64_t sstride,
    float* __restrict__ part_s, float* __restrict__ part_st, float* __restrict__ part_decay,  // state pass
    const float* __restrict__ init_s, const float* __restrict__ init_st,                     // output pass
    double* __restrict__ part, int64_t H, int64_t L, int nseg, int G, int cps) {
    __shared__ __attribute__((aligned(16))) DlamSmem<D, STATE_ONLY> sm;
    using Gm = Geo<D>;
    constexpr int PITCH = Gm::PITCH, PR = Gm::PR, PIECES_ROW = Gm::PIECES_ROW, NCB = Gm::NCB;
    constexpr bool PF = true;  // (at d = 128 the output pass then spills 2 registers and is still ~20 us faster)
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int cb = (Gm::WPC == 1) ? w : w % NCB, rank = (Gm::WPC == 1) ? 0 : w / NCB;
    const int lane = tid & 63;
    const int n32 = lane & 31;
    const int kg = lane >> 5;
    const int64_t u = blockIdx.x;
    const int gper = STATE_ONLY ? (G - 1) : G;
    const int g = (int)(u % gper);  // the state pass covers 0..G-2
    const int64_t ub = u / gper;
    const int seg = (int)(ub % nseg);
    const int64_t bh = ub / nseg;
    const int64_t h = bh % H;
    const int64_t Lseg = L / nseg;
    const int64_t tseg = (int64_t)seg * Lseg;
    const int64_t t_begin = tseg + (int64_t)g * cps * C;
    const int64_t t_end = min(t_begin + (int64_t)cps * C, tseg + Lseg);
    const int64_t row_base = bh * L;
    const float lam = decay[h];
    if (tid <= C) sm.apow[tid] = decay_pow(lam, tid);  // read after the loop's first barrier

    // S and St entering the sub-segment (value columns 32 w + n32, key rows as the accumulators)
    f32x16 Sm[NCB], St[NCB];
    {
        const float* src = nullptr;
        const float* srct = nullptr;
        if (g == 0) {
            if (seg == 0 && s_in) src = s_in + bh * (int64_t)D * D;
        } else if (!STATE_ONLY) {
            src = init_s + (ub * (G - 1) + (g - 1)) * (int64_t)D * D;
            srct = init_st + (ub * (G - 1) + (g - 1)) * (int64_t)D * D;
        }
#pragma unroll
        for (int m = 0; m < NCB; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                Sm[m][i] = src ? src[r * D + 32 * cb + n32] : 0.f;
                St[m][i] = srct ? srct[r * D + 32 * cb + n32] : 0.f;
            }
    }

    double acc = 0.0;
    const int nchunks = (int)((t_end - t_begin + C - 1) / C);
    // one chunk's tiles in registers (rows past the end read as zero)
    u32x4 rk[PR], rv[PR], rq[STATE_ONLY ? 1 : PR], ro[STATE_ONLY ? 1 : PR];
    auto load_chunk = [&](int cc) {
        const int64_t t0c = t_begin + (int64_t)cc * C;
        const int nc = (int)min((int64_t)C, t_end - t0c);
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < PR; r++) {
            const int p = tid + NT * r;
            const int row = p / PIECES_ROW, c8 = (p % PIECES_ROW) * 8;
            const int64_t off = (row_base + t0c + row) * D + c8;
            const bool ok = row < nc;
            rk[r] = ok ? *(const u32x4*)(k + off) : z;
            rv[r] = ok ? *(const u32x4*)(v + off) : z;
            if (!STATE_ONLY) {
                rq[r] = ok ? *(const u32x4*)(q + off) : z;
                ro[r] = ok ? *(const u32x4*)(d_o + off) : z;
            }
        }
    };
    if (PF && nchunks > 0) load_chunk(0);
    for (int c = 0; c < nchunks; c++) {
        const int64_t t0 = t_begin + (int64_t)c * C;
        const int n = (int)min((int64_t)C, t_end - t0);
        __syncthreads();  // the previous chunk is done with every LDS tile
        if (!PF) load_chunk(c);
#pragma unroll
        for (int r = 0; r < PR; r++) {
            const int p = tid + NT * r;
            const int row = p / PIECES_ROW, c8 = (p % PIECES_ROW) * 8;
            const int jr = max(n - 1 - row, 0);
            *(u32x4*)(&sm.v[row * PITCH + c8]) = rv[r];
            *(u32x4*)(&sm.kt[row * PITCH + c8]) = scale8s(rk[r], sm.apow[jr]);
            *(u32x4*)(&sm.kt2[row * PITCH + c8]) = scale8s(rk[r], (float)jr * sm.apow[jr]);
            if (!STATE_ONLY) {
                *(u32x4*)(&sm.o[row * PITCH + c8]) = ro[r];
                *(u32x4*)(&sm.qs[row * PITCH + c8]) = scale8s(rq[r], sm.apow[row + 1]);
                *(u32x4*)(&sm.qs2[row * PITCH + c8]) = scale8s(rq[r], (float)(row + 1) * sm.apow[row + 1]);
            }
        }
        __syncthreads();
        if (PF && c + 1 < nchunks) load_chunk(c + 1);  // the next chunk, while this one is computed

        if (!STATE_ONLY && rank == 0) {
            // ---- earlier tokens: <S, M'> + <St, M> over this wave's value columns (one wave per block)
            bf16x8 ob[4];
#pragma unroll
            for (int ks = 0; ks < 4; ks++) ob[ks] = tr_operand(sm.o, PITCH, ks, 32 * cb, lane);
#pragma unroll
            for (int m = 0; m < NCB; m++) {  // one 16-register product at a time: M' with S, then M with St
                f32x16 M = {};
#pragma unroll
                for (int ks = 0; ks < 4; ks++) M = mfma(tr_operand(sm.qs2, PITCH, ks, 32 * m, lane), ob[ks], M);
                double x = 0.0;
#pragma unroll
                for (int i = 0; i < 16; i++) x += (double)Sm[m][i] * (double)M[i];
                M = f32x16{};
#pragma unroll
                for (int ks = 0; ks < 4; ks++) M = mfma(tr_operand(sm.qs, PITCH, ks, 32 * m, lane), ob[ks], M);
#pragma unroll
                for (int i = 0; i < 16; i++) x += (double)St[m][i] * (double)M[i];
                acc += x;
            }
        }

        // ---- St <- a^n St + n a^n S + (k (n-1-j) a^{n-1-j})^T V, then S <- a^n S + (k a^{n-1-j})^T V
        {
            bf16x8 vb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ks++) vb[ks] = tr_operand(sm.v, PITCH, ks, 32 * cb, lane);
            const float an = sm.apow[n], nan_ = (float)n * sm.apow[n];
#pragma unroll
            for (int m = 0; m < NCB; m++) {
#pragma unroll
                for (int i = 0; i < 16; i++) St[m][i] = an * St[m][i] + nan_ * Sm[m][i];
#pragma unroll
                for (int ks = 0; ks < 4; ks++) St[m] = mfma(tr_operand(sm.kt2, PITCH, ks, 32 * m, lane), vb[ks], St[m]);
#pragma unroll
                for (int i = 0; i < 16; i++) Sm[m][i] *= an;
#pragma unroll
                for (int ks = 0; ks < 4; ks++) Sm[m] = mfma(tr_operand(sm.kt, PITCH, ks, 32 * m, lane), vb[ks], Sm[m]);
            }
        }
    }

    if (STATE_ONLY) {
        float* ds = part_s + (ub * (G - 1) + g) * (int64_t)D * D;
        float* dt = part_st + (ub * (G - 1) + g) * (int64_t)D * D;
        if (rank == 0) {
#pragma unroll
            for (int m = 0; m < NCB; m++)
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                    ds[r * D + 32 * cb + n32] = Sm[m][i];
                    dt[r * D + 32 * cb + n32] = St[m][i];
                }
        }
        if (tid < D) part_decay[(ub * (G - 1) + g) * D + tid] = decay_pow(lam, (int)(t_end - t_begin));
        return;
    }
    if (g == G - 1 && ds_out && rank == 0) {  // <ds_out, dS_out / dlambda>
        const float* dso = ds_out + bh * sstride + (int64_t)seg * D * D;
#pragma unroll
        for (int m = 0; m < NCB; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                acc += (double)St[m][i] * (double)dso[r * D + 32 * cb + n32];
            }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) sm.red[w] = acc;
    __syncthreads();
    if (tid == 0) part[ub * G + g] = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
}

// St_loc[g] += l A S_end[g-1] for the state pass's slots g = 1..G-2 (S already scanned in place).
template <int D>
__global__ __launch_bounds__(256) void dlam_fixup_kernel(float* __restrict__ part_st, const float* __restrict__ part_s,
                                                         const float* __restrict__ decay, int64_t H, int nseg, int G,
                                                         int ell) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // element of one state
    const int g = blockIdx.y + 1;
    const int64_t ub = blockIdx.z;
    if (e >= (int64_t)D * D) return;
    const int64_t h = (ub / nseg) % H;
    const float f = (float)ell * decay_pow(decay[h], ell);
    part_st[(ub * (G - 1) + g) * (int64_t)D * D + e] += f * part_s[(ub * (G - 1) + g - 1) * (int64_t)D * D + e];
}

// d lambda_h = sum over batch, segments and sub-segments of the inter-chunk and intra-chunk parts
// (part and intra: [units][G] each).
__global__ __launch_bounds__(256) void dlam_final_kernel(const double* __restrict__ part,
                                                         const double* __restrict__ intra,
                                                         float* __restrict__ d_decay, int64_t B, int64_t H, int nseg,
                                                         int G) {
    const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    double s = 0.0;
    for (int64_t b = 0; b < B; b++)
        for (int p = 0; p < nseg; p++) {
            const int64_t o = ((b * H + h) * nseg + p) * (int64_t)G;
            for (int y = 0; y < G; y++) s += part[o + y] + intra[o + y];
        }
    d_decay[h] = (float)s;
}

// d lambda_h, first part: the local S and dS/dlambda of every sub-segment but the last, and the
// scan of S, which leaves the state entering every sub-segment after the first in ps (the same
// values, in the same layout, as the dq passes' own scan, which it then replaces).
template <int D>
hipError_t launch_dlam_states(const BwdArgs& a, int G, int cps, float* ps, float* pst, float* pdec) {
    const int64_t units = a.B * a.H * a.nseg;
    hipError_t e;
    if (G > 1) {
        LA_TRACED(a.tr, "chunk_bwd_dlam_state_pass",
                  bwd_dlam_kernel<D, true><<<(unsigned)(units * (G - 1)), NT, 0, a.stream>>>(
                      (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.d_o, a.decay,
                      a.s_in, a.ds_out, a.state_stride, ps, pst, pdec, nullptr, nullptr, nullptr, a.H, a.L, a.nseg, G,
                      cps));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_state_scan(ps, pdec, ps, units, G - 1, D, D, a.stream, a.tr)) != hipSuccess) return e;
    }
    return hipSuccess;
}

// d lambda_h, second part: dS/dlambda across sub-segments (fix-up and scan), the output pass and the
// final sum.
template <int D>
hipError_t launch_dlam(const BwdArgs& a, int G, int cps, float* ps, float* pst, float* pdec, double* part,
                       const double* intra) {
    const int64_t units = a.B * a.H * a.nseg;
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    const __bf16* d_o = (const __bf16*)a.d_o;
    hipError_t e;
    if (G > 1) {
        if (G > 2) {
            LA_TRACED(a.tr, "chunk_bwd_dlam_fixup",
                      dlam_fixup_kernel<D><<<dim3(D * D / 256, (unsigned)(G - 2), (unsigned)units), 256, 0, a.stream>>>(
                          pst, ps, a.decay, a.H, a.nseg, G, cps * C));
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if ((e = launch_state_scan(pst, pdec, pst, units, G - 1, D, D, a.stream, a.tr)) != hipSuccess) return e;
    }
    LA_TRACED(a.tr, "chunk_bwd_dlam",
              bwd_dlam_kernel<D, false><<<(unsigned)(units * G), NT, 0, a.stream>>>(
                  q, k, v, d_o, a.decay, a.s_in, a.ds_out, a.state_stride, nullptr, nullptr, nullptr, ps, pst, part,
                  a.H, a.L, a.nseg, G, cps));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    LA_TRACED(a.tr, "chunk_bwd_dlam_final",
              dlam_final_kernel<<<(unsigned)((a.H + 255) / 256), 256, 0, a.stream>>>(part, intra, a.d_decay, a.B, a.H,
                                                                                     a.nseg, G));
    return hipGetLastError();
}

// Gate derivative, one chunk of one (b, h, segment) per workgroup.  With S the state entering the
// chunk and D the derivative with respect to it (both from the chunk's start: c0 = rowsum(S (.) D)),
// the derivative with respect to log a_s of a token s of the chunk is
//     dlog a_s = c0 + sum over the chunk's tokens t < s of (k_t (.) dk_t - q_t (.) dq_t)
// (every pair of tokens j < s <= i contributes q_i k_j e^{B_i - B_j} (v_j . d_o_i); the chunk's
// dq, dk hold the pairs with one end in it, c0 those that cross its start), and log a = -softplus(-g)
// / gate_norm gives dg = dlog a * sigmoid(-g) / gate_norm.  Lanes take column pairs, NT / (D / 2)
// groups of C / groups rows each, whose totals are combined through LDS.
template <int D>
__global__ __launch_bounds__(NT) void dg_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                const __bf16* __restrict__ dq, const __bf16* __restrict__ dk,
                                                const float* __restrict__ gate, const float* __restrict__ c0,
                                                float* __restrict__ dg, int64_t L, int nseg, float inv_norm) {
    constexpr int PAIRS = D / 2, GROUPS = NT / PAIRS, RPG = C / GROUPS;
    __shared__ float tot[GROUPS * D];
    const int tid = threadIdx.x;
    const int64_t Lseg = L / nseg;
    const int64_t nch_seg = (Lseg + C - 1) / C;
    const int64_t ci = blockIdx.x;  // (b, h, segment) * nch_seg + chunk
    const int64_t ub = ci / nch_seg, sc = ci % nch_seg;
    const int seg = (int)(ub % nseg);
    const int64_t bh = ub / nseg;
    const int64_t t0 = (int64_t)seg * Lseg + sc * C;
    const int n = (int)min((int64_t)C, (int64_t)seg * Lseg + Lseg - t0);
    const int d0 = 2 * (tid % PAIRS), grp = tid / PAIRS;
    float ex0[RPG], ex1[RPG];  // exclusive running sums inside the group
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < RPG; i++) {
        const int row = grp * RPG + i;
        ex0[i] = s0;
        ex1[i] = s1;
        if (row < n) {
            const int64_t off = (bh * L + t0 + row) * D + d0;
            const bf16x2 qq = *(const bf16x2*)(q + off), kk = *(const bf16x2*)(k + off);
            const bf16x2 gq = *(const bf16x2*)(dq + off), gk = *(const bf16x2*)(dk + off);
            s0 += (float)kk[0] * (float)gk[0] - (float)qq[0] * (float)gq[0];
            s1 += (float)kk[1] * (float)gk[1] - (float)qq[1] * (float)gq[1];
        }
    }
    tot[grp * D + d0] = s0;
    tot[grp * D + d0 + 1] = s1;
    __syncthreads();
    float b0 = c0[ci * D + d0], b1 = c0[ci * D + d0 + 1];
    for (int gg = 0; gg < grp; gg++) {
        b0 += tot[gg * D + d0];
        b1 += tot[gg * D + d0 + 1];
    }
#pragma unroll
    for (int i = 0; i < RPG; i++) {
        const int row = grp * RPG + i;
        if (row < n) {
            const int64_t off = (bh * L + t0 + row) * D + d0;
            const f32x2 gg = *(const f32x2*)(gate + off);
            f32x2 out;
            out[0] = (b0 + ex0[i]) * inv_norm / (1.f + __expf(gg[0]));
            out[1] = (b1 + ex1[i]) * inv_norm / (1.f + __expf(gg[1]));
            *(f32x2*)(dg + off) = out;
        }
    }
}

// wide: gate mode, one int per workgroup of the largest pass (B*H*nseg*G), the flags that send a unit
// of a pass to its windowed redo (each pass and its redo run before the next pass writes them).
template <int D, int MODE>
hipError_t launch_mode(const BwdArgs& a, int G, int cps, float* f_state, float* f_decay, float* b_state,
                       float* b_decay, double* intra_part, __bf16* d_start, float* c0, int* wide,
                       const float* s_scanned = nullptr) {
    const int64_t units = a.B * a.H * a.nseg;
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    const __bf16* d_o = (const __bf16*)a.d_o;
    // dq: forward state pass, scan, output pass (with the gate derivative also rowsum(S (.) D) per chunk)
    // (the states entering the sub-segments given by the caller: no state pass, no scan)
    auto dq_passes = [&]() -> hipError_t {
        const float* init = f_state;
        int64_t ist_bh = (int64_t)a.nseg * (G - 1) * D * D;
        int ist_g = G - 1, ist_off = -1;
        if (a.s_sub) {
            init = a.s_sub;
            ist_bh = a.sub_stride;
            ist_g = G;
            ist_off = 0;
        } else if (s_scanned) {  // the scanned states of the d lambda_h pipeline, same layout as f_state
            init = s_scanned;
        }
        if constexpr (D == 128 && MODE != DECAY_GATE) {  // on the forward's kernel (chunk_fwd_pipe.hip)
            return launch_pipe_dq(a, G, cps, f_state, f_decay, init == f_state ? nullptr : init, ist_bh, ist_g,
                                  ist_off);
        } else {
            hipError_t e;
            if (init == f_state && G > 1) {
                if constexpr (MODE == DECAY_GATE)  // the plain walk and the windowed one in one launch
                    LA_TRACED(a.tr, "chunk_bwd_dq_state_pass",
                              bwd_dq_gate_kernel<D, true><<<(unsigned)(units * (G - 1)), NT, 0, a.stream>>>(
                                  k, v, d_o, a.decay, a.s_in, a.ds_out, a.state_stride, nullptr, f_state, f_decay,
                                  nullptr, 0, 0, 0, nullptr, nullptr, a.H, a.L, a.nseg, G, cps, a.inv_norm, wide));
                else
                    LA_TRACED(a.tr, "chunk_bwd_dq_state_pass",
                              bwd_dq_kernel<D, MODE, true><<<(unsigned)(units * (G - 1)), NT, 0, a.stream>>>(
                                  k, v, d_o, a.decay, a.s_in, a.ds_out, a.state_stride, nullptr, f_state, f_decay,
                                  nullptr, 0, 0, 0, nullptr, nullptr, a.H, a.L, a.nseg, G, cps, a.inv_norm, wide));
                if ((e = hipGetLastError()) != hipSuccess) return e;
                e = launch_state_scan(f_state, f_decay, f_state, units, G - 1, D, D, a.stream, a.tr);
                if (e != hipSuccess) return e;
            }
            if constexpr (MODE == DECAY_GATE)
                LA_TRACED(a.tr, "chunk_bwd_dq",
                          bwd_dq_gate_kernel<D, false><<<(unsigned)(units * G), NT, 0, a.stream>>>(
                              k, v, d_o, a.decay, a.s_in, a.ds_out, a.state_stride, (__bf16*)a.dq, nullptr, nullptr,
                              init, ist_bh, ist_g, ist_off, d_start, c0, a.H, a.L, a.nseg, G, cps, a.inv_norm, wide));
            else
                LA_TRACED(a.tr, "chunk_bwd_dq",
                          bwd_dq_kernel<D, MODE, false><<<(unsigned)(units * G), NT, 0, a.stream>>>(
                              k, v, d_o, a.decay, a.s_in, a.ds_out, a.state_stride, (__bf16*)a.dq, nullptr, nullptr,
                              init, ist_bh, ist_g, ist_off, d_start, c0, a.H, a.L, a.nseg, G, cps, a.inv_norm, wide));
            return hipGetLastError();
        }
    };
    // dk, dv: backward state pass, reverse-order scan, output pass (with the gate derivative also D at
    // every chunk's start)
    auto dkdv_passes = [&]() -> hipError_t {
        hipError_t e;
        if (G > 1) {
            if constexpr (MODE == DECAY_GATE)  // the plain walk and the windowed one in one launch
                LA_TRACED(a.tr, "chunk_bwd_dkdv_state_pass",
                          bwd_dkdv_gate_kernel<D, true><<<(unsigned)(units * (G - 1)), NT, 0, a.stream>>>(
                              q, k, v, d_o, a.decay, a.ds_out, a.state_stride, nullptr, nullptr, nullptr, b_state,
                              b_decay, nullptr, nullptr, nullptr, a.H, a.L, a.nseg, G, cps, a.inv_norm, wide));
            else
                LA_TRACED(a.tr, "chunk_bwd_dkdv_state_pass",
                          bwd_dkdv_kernel<D, MODE, true><<<(unsigned)(units * (G - 1)), NT, 0, a.stream>>>(
                              q, k, v, d_o, a.decay, a.ds_out, a.state_stride, nullptr, nullptr, nullptr, b_state,
                              b_decay, nullptr, nullptr, nullptr, a.H, a.L, a.nseg, G, cps, a.inv_norm, wide));
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if ((e = launch_state_scan(b_state, b_decay, b_state, units, G - 1, D, D, a.stream, a.tr)) != hipSuccess)
                return e;
        }
        if constexpr (MODE == DECAY_HEAD) {
            if (!intra_part) {  // the factorised walk, or the per-pair one for heads with a stronger decay
                LA_TRACED(a.tr, "chunk_bwd_dkdv",
                          bwd_dkdv_head_kernel<D><<<(unsigned)(units * G), NT, 0, a.stream>>>(
                              q, k, v, d_o, a.decay, a.ds_out, a.state_stride, (__bf16*)a.dk_out, (__bf16*)a.dv_out,
                              a.ds_in, nullptr, nullptr, b_state, nullptr, nullptr, a.H, a.L, a.nseg, G, cps,
                              a.inv_norm, wide));
                return hipGetLastError();
            }
        }
        if constexpr (MODE == DECAY_GATE)
            LA_TRACED(a.tr, "chunk_bwd_dkdv",
                      bwd_dkdv_gate_kernel<D, false><<<(unsigned)(units * G), NT, 0, a.stream>>>(
                          q, k, v, d_o, a.decay, a.ds_out, a.state_stride, (__bf16*)a.dk_out, (__bf16*)a.dv_out,
                          a.ds_in, nullptr, nullptr, b_state, intra_part, d_start, a.H, a.L, a.nseg, G, cps,
                          a.inv_norm, wide));
        else
            LA_TRACED(a.tr, "chunk_bwd_dkdv",
                      bwd_dkdv_kernel<D, MODE, false><<<(unsigned)(units * G), NT, 0, a.stream>>>(
                          q, k, v, d_o, a.decay, a.ds_out, a.state_stride, (__bf16*)a.dk_out, (__bf16*)a.dv_out,
                          a.ds_in, nullptr, nullptr, b_state, intra_part, d_start, a.H, a.L, a.nseg, G, cps,
                          a.inv_norm, wide));
        return hipGetLastError();
    };
    hipError_t e;
    if (!d_start) {
        if ((e = dq_passes()) != hipSuccess) return e;
        return dkdv_passes();
    }
    // gate derivative: D per chunk first, then S with rowsum(S (.) D), then the in-chunk sums
    if ((e = dkdv_passes()) != hipSuccess) return e;
    if ((e = dq_passes()) != hipSuccess) return e;
    const int64_t nch_seg = (a.L / a.nseg + C - 1) / C;
    LA_TRACED(a.tr, "chunk_bwd_dg",
              dg_kernel<D><<<(unsigned)(units * nch_seg), NT, 0, a.stream>>>(
                  q, k, (const __bf16*)a.dq, (const __bf16*)a.dk_out, a.decay, c0, a.d_decay, a.L, a.nseg,
                  a.inv_norm));
    return hipGetLastError();
}

// The whole backward for head dim D.  Each D is compiled in a translation unit of its own
// (chunk_bwd_mfma_d<D>.hip): with all three in one unit the d = 128 d lambda output pass was
// allocated differently and spilled 33 registers instead of 2.
template <int D>
hipError_t launch_d(const BwdArgs& a) {
    FwdArgs sp;
    sp.B = a.B; sp.H = a.H; sp.L = a.L; sp.nseg = a.nseg; sp.subseg_chunks = a.subseg_chunks;
    int G, cps;
    if (a.s_sub) {
        sp.subseg_chunks = a.sub_len / C;  // the caller's sub-segments (validated: a multiple of 64)
    } else if (D == 32 && a.subseg_chunks == 0) {
        // d = 32: sub-segments for about 512 workgroups rather than the forward's 256 (several share
        // a compute unit; B1 H16 L16k: 120 -> 96 us without decay, 217 -> 205 us with d lambda_h);
        // d = 64 and 128 gain nothing from more
        const int64_t u32 = a.B * a.H * a.nseg;
        const int64_t g_want = (512 + u32 - 1) / u32;
        const int64_t nch = (a.L / a.nseg + C - 1) / C;
        sp.subseg_chunks = (int)max((int64_t)4, (nch + g_want - 1) / g_want);
    }
    mfma_split(sp, &G, &cps);
    const int64_t units = a.B * a.H * a.nseg;
    const bool dlam = a.mode == DECAY_HEAD && a.d_decay;
    const bool dgate = a.mode == DECAY_GATE && a.d_decay;
    // workspace: fp64 partials of d lambda_h, then the sub-segment states and decays of the dq and
    // dk/dv passes (and of S and dS/dlambda for d lambda_h), then for the gate derivative
    // rowsum(S (.) D) (fp32) and D (bf16) at every chunk's start
    const size_t n_dbl = dlam ? 2 * (size_t)units * G : 0;  // inter- and intra-chunk partials
    const size_t n_state = (size_t)units * (G - 1) * D * D, n_decay = (size_t)units * (G - 1) * D;
    const int nsets = dlam ? 4 : 2;  // state arrays: forward, backward (+ S, St)
    const size_t n_chunks = dgate ? (size_t)units * (size_t)((a.L / a.nseg + C - 1) / C) : 0;
    const size_t n_wide = a.mode == DECAY_GATE ? (size_t)units * G : 0;  // the gate passes' redo flags
    const size_t f_bytes =
        sizeof(double) * n_dbl + sizeof(float) * (nsets * n_state + 3 * n_decay + n_chunks * D) + sizeof(int) * n_wide;
    const size_t ds_off = (f_bytes + 255) / 256 * 256;
    const size_t bytes = n_chunks ? ds_off + sizeof(__bf16) * n_chunks * D * D : f_bytes;
    char* ws = nullptr;
    hipError_t e = hipSuccess;
    bool owned = false;
    if (bytes > 0 && (e = workspace_acquire(WS_BACKWARD, (void**)&ws, bytes, a.stream, &owned)) != hipSuccess)
        return e;
    double* part = n_dbl ? (double*)ws : nullptr;
    double* intra = n_dbl ? part + (size_t)units * G : nullptr;
    float* fp = (float*)(ws + sizeof(double) * n_dbl);
    float* f_state = n_state ? fp : nullptr;
    float* b_state = n_state ? fp + n_state : nullptr;
    float* l_state = (n_state && dlam) ? fp + 2 * n_state : nullptr;
    float* lt_state = (n_state && dlam) ? fp + 3 * n_state : nullptr;
    float* f_decay = n_decay ? fp + nsets * n_state : nullptr;
    float* b_decay = n_decay ? fp + nsets * n_state + n_decay : nullptr;
    float* l_decay = n_decay ? fp + nsets * n_state + 2 * n_decay : nullptr;
    float* c0 = n_chunks ? fp + nsets * n_state + 3 * n_decay : nullptr;
    int* wide = n_wide ? (int*)(fp + nsets * n_state + 3 * n_decay + n_chunks * D) : nullptr;
    __bf16* d_start = n_chunks ? (__bf16*)(ws + ds_off) : nullptr;
    if (dlam && !a.s_sub) {  // the S scan of the d lambda_h pipeline replaces the dq passes' own
        e = launch_dlam_states<D>(a, G, cps, l_state, lt_state, l_decay);
        if (e == hipSuccess)
            e = launch_mode<D, DECAY_HEAD>(a, G, cps, f_state, f_decay, b_state, b_decay, intra, nullptr, nullptr,
                                           nullptr, l_state);
    } else if (a.mode == DECAY_HEAD)
        e = launch_mode<D, DECAY_HEAD>(a, G, cps, f_state, f_decay, b_state, b_decay, intra, nullptr, nullptr,
                                       nullptr);
    else if (a.mode == DECAY_GATE)
        e = launch_mode<D, DECAY_GATE>(a, G, cps, f_state, f_decay, b_state, b_decay, nullptr, d_start, c0, wide);
    else
        e = launch_mode<D, DECAY_NONE>(a, G, cps, f_state, f_decay, b_state, b_decay, nullptr, nullptr, nullptr,
                                       nullptr);
    if (e == hipSuccess && dlam && a.s_sub) e = launch_dlam_states<D>(a, G, cps, l_state, lt_state, l_decay);
    if (e == hipSuccess && dlam) e = launch_dlam<D>(a, G, cps, l_state, lt_state, l_decay, part, intra);
    const hipError_t f = workspace_release(ws, a.stream, owned);
    return e == hipSuccess ? f : e;
}

}  // namespace
}  // namespace la
