// chunk_fwd_tiled.hip -- bf16 matrix-core (MFMA) chunked forward with the value dims tiled across
// workgroups, for the head-dim and chunk-length variants the other kernels do not cover:
//   dk = dv = 256, 64-token chunks, 64-column value tiles (four workgroups per sub-segment);
//   dk = dv = 128, 128-token chunks, one 128-column tile.
// No decay or one decay per head (the ZeCO review page's falsifier and the reviewers' ask for the
// chunk length and state size to move: pith_extraction.falsifier, referee_report.major_comments[2]).
//
// The chunk algebra is the small-head kernel's (chunk_fwd_small.hip).  Per chunk of n tokens:
//   P[i][j] = q_i . k_j a^{i-j}  (j <= i),   O = a^{i+1} (Q S) + P V,
//   S <- a^n S + sum_j a^{n-1-j} k_j v_j^T
// with every factor <= 1 applied in registers: the scores scaled after the product, the rows of
// Q S scaled, and the key-to-chunk-end weights applied to the V operand of the state update (so
// no scaled copy of the keys is staged).  A workgroup owns one (b, h, segment, sub-segment,
// value tile): it reads the chunk's whole q and k rows (all DK key dims: the scores and the
// state's rows need them) and only its tile's columns of v; the tiles of a sub-segment are
// launched on the same XCD (block index + 8 t), so q and k come from its L2 after the first.
// Four waves: value-column block cb = w % (DVT / 32) of the state and outputs, all DK key rows of
// the state in MFMA accumulators; waves sharing a block keep identical copies and split the
// chunk's 32-row output blocks.  The causal 32x32 score blocks are dealt to the waves in turn and
// pass through LDS.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int NT = 256;  // lanes per workgroup

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

template <int DK, int DVT, int CH>
struct TiledSmem {
    static constexpr int QPITCH = DK + 8;   // bf16: 16-byte aligned rows, conflict-free row reads
    static constexpr int VPITCH = DVT + 8;
    static constexpr int PP = CH + 8;
    __bf16 q[CH * QPITCH];
    __bf16 k[CH * QPITCH];
    __bf16 v[CH * VPITCH];
    __bf16 p[CH * PP];
};

// DK key dims, DVT value columns per workgroup (the full value dim is DK), chunks of CH tokens.
template <int DK, int DVT, int CH, int MODE, bool STATE_ONLY>
__global__ __launch_bounds__(NT) void tiled_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ decay, const float* __restrict__ s_in, __bf16* __restrict__ o,
    float* __restrict__ s_out, int64_t s_out_stride,
    float* __restrict__ part_state, float* __restrict__ part_decay,  // state pass outputs
    const float* __restrict__ init_state,                            // output pass inputs (scanned)
    int64_t H, int64_t L, int nseg, int G, int cps, int64_t nunits) {
    static_assert(MODE != DECAY_GATE, "no decay or head decay");
    constexpr int DV = DK;                 // full value dim
    constexpr int NTILE = DV / DVT;        // value tiles per sub-segment
    constexpr int NCB = DVT / 32;          // 32-wide value-column blocks of a tile
    constexpr int WPC = 4 / NCB;           // waves per column block
    constexpr int NKB = DK / 32;           // 32-row key blocks of the state
    constexpr int KS = DK / 16;            // 16-wide slabs of the key contraction
    constexpr int PRQ = CH * DK / 8 / NT;  // 16-byte pieces of a q (k) tile per lane
    constexpr int PRV = CH * DVT / 8 / NT; // 16-byte pieces of the v tile per lane
    constexpr int NSLAB = CH / 16;         // 16-token slabs of a chunk
    constexpr int NRB = CH / 32;           // 32-row blocks of a chunk
    static_assert(NCB >= 1 && NCB <= 4 && PRQ >= 1 && PRV >= 1, "tile shape");
    using Sm = TiledSmem<DK, DVT, CH>;
    constexpr int QP = Sm::QPITCH, VP = Sm::VPITCH, PP = Sm::PP;
    __shared__ __attribute__((aligned(16))) Sm sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int n32 = lane & 31;
    const int kg = lane >> 5;
    const int cb = w % NCB;
    const int rank = w / NCB;
    // block index -> (unit, value tile): the NTILE tiles of a unit are 8 blocks apart (one XCD)
    const int64_t bx = blockIdx.x;
    const int tile = (int)((bx / 8) % NTILE);
    const int64_t u = (bx / (8 * NTILE)) * 8 + bx % 8;
    if (u >= nunits) return;
    const int gper = STATE_ONLY ? (G - 1) : G;
    const int g = (int)(u % gper);
    const int64_t ub = u / gper;  // (bh, seg)
    const int seg = (int)(ub % nseg);
    const int64_t bh = ub / nseg;
    const int64_t h = bh % H;
    const int64_t Lseg = L / nseg;
    const int64_t t_begin = (int64_t)seg * Lseg + (int64_t)g * cps * CH;
    const int64_t t_end = min(t_begin + (int64_t)cps * CH, (int64_t)(seg + 1) * Lseg);
    const int64_t row_base = bh * L;
    const int c0 = tile * DVT;  // this workgroup's first value column
    const float lam = (MODE == DECAY_HEAD) ? decay[h] : 0.f;
    const float lam2 = lam * LOG2E;  // head factors through the hardware base-2 exponential

    // ---- initial state: key rows 32 m + (i / 4) 8 + kg 4 + i % 4, value column c0 + 32 cb + n32
    f32x16 S[NKB];
    {
        const float* src = nullptr;
        if (g == 0) {
            if (seg == 0 && s_in) src = s_in + bh * (int64_t)DK * DV;
        } else if (!STATE_ONLY) {
            src = init_state + (ub * (G - 1) + (g - 1)) * (int64_t)DK * DV;
        }
#pragma unroll
        for (int m = 0; m < NKB; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                S[m][i] = src ? src[r * DV + c0 + 32 * cb + n32] : 0.f;
            }
    }

    // ---- register prefetch of one chunk (rows past the end read as zero)
    u32x4 rq[STATE_ONLY ? 1 : PRQ], rk[PRQ], rv[PRV];
    auto load_chunk = [&](int64_t t0, int n) {
        const int64_t qbase = (row_base + t0) * DK, vbase = (row_base + t0) * DV + c0;
#pragma unroll
        for (int r = 0; r < PRQ; r++) {
            const int p = tid + NT * r;
            const int row = p / (DK / 8), c8 = (p % (DK / 8)) * 8;
            const bool ok = row < n;
            if (!STATE_ONLY) rq[r] = ok ? *(const u32x4*)(q + qbase + (row * DK + c8)) : u32x4{0, 0, 0, 0};
            rk[r] = ok ? *(const u32x4*)(k + qbase + (row * DK + c8)) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < PRV; r++) {
            const int p = tid + NT * r;
            const int row = p / (DVT / 8), c8 = (p % (DVT / 8)) * 8;
            rv[r] = row < n ? *(const u32x4*)(v + vbase + (row * DV + c8)) : u32x4{0, 0, 0, 0};
        }
    };

    const int nchunks = (int)((t_end - t_begin + CH - 1) / CH);
    if (nchunks > 0) load_chunk(t_begin, (int)min((int64_t)CH, t_end - t_begin));
    const int G16 = lane >> 4, i16 = lane & 15;

    for (int c = 0; c < nchunks; c++) {
        const int64_t t0 = t_begin + (int64_t)c * CH;
        const int n = (int)min((int64_t)CH, t_end - t0);
        // the head factors are recomputed every chunk: hiding lam2's value from the optimiser keeps
        // these loop invariants from being hoisted into registers for the whole walk (which spills)
        float lamc = lam2;
        if (MODE == DECAY_HEAD) asm volatile("" : "+v"(lamc));
        __syncthreads();  // the previous chunk is done with every LDS tile
#pragma unroll
        for (int r = 0; r < PRQ; r++) {
            const int p = tid + NT * r;
            const int row = p / (DK / 8), c8 = (p % (DK / 8)) * 8;
            if (!STATE_ONLY) *(u32x4*)(&sm.q[row * QP + c8]) = rq[r];
            *(u32x4*)(&sm.k[row * QP + c8]) = rk[r];
        }
#pragma unroll
        for (int r = 0; r < PRV; r++) {
            const int p = tid + NT * r;
            const int row = p / (DVT / 8), c8 = (p % (DVT / 8)) * 8;
            *(u32x4*)(&sm.v[row * VP + c8]) = rv[r];
        }
        __syncthreads();
        if (c + 1 < nchunks) load_chunk(t0 + CH, (int)min((int64_t)CH, t_end - (t0 + CH)));

        // ---- V operand of this wave's 32 value columns for the chunk's token slabs: element e of
        // lane (G16, i16) in slab ks is token 16 ks + (G16 / 2) 8 + i16 / 4 + 4 (e / 4)
        bf16x8 vb[NSLAB];
        {
            const int col = 32 * cb + (G16 & 1) * 16 + (i16 & 3) * 4;
#pragma unroll
            for (int ks = 0; ks < NSLAB; ks++) {
                const int tb = 16 * ks + (G16 >> 1) * 8 + (i16 >> 2);
                vb[ks] = cat(lds_tr16(&sm.v[tb * VP + col]), lds_tr16(&sm.v[(tb + 4) * VP + col]));
            }
        }

        if (!STATE_ONLY) {
            // ---- intra-chunk scores: the causal 32x32 blocks (rb, sb), sb <= rb, dealt to the waves
            auto score_block = [&](int rb, int sb_) {
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const bf16x8 a = *(const bf16x8*)(&sm.q[(rb * 32 + n32) * QP + ks * 16 + kg * 8]);
                    const bf16x8 b = *(const bf16x8*)(&sm.k[(sb_ * 32 + n32) * QP + ks * 16 + kg * 8]);
                    acc = mfma(a, b, acc);
                }
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = rb * 32 + (i >> 2) * 8 + kg * 4 + (i & 3);
                    const int col = sb_ * 32 + n32;
                    float val = acc[i];
                    if (MODE == DECAY_HEAD) val *= decay_pow2(lamc, max(row - col, 0));
                    if (col > row) val = 0.f;
                    sm.p[row * PP + col] = (__bf16)val;
                }
            };
            if constexpr (CH == 64) {
                if (w != 1) score_block(w >> 1, (w == 3) ? 1 : 0);
            } else {
                for (int blk = w; blk < NRB * (NRB + 1) / 2; blk += 4) {
                    int rb = 0;
                    while ((rb + 1) * (rb + 2) / 2 <= blk) rb++;
                    score_block(rb, blk - rb * (rb + 1) / 2);
                }
            }
            __syncthreads();  // P complete

            // ---- outputs: this wave's column block, its row blocks; the state as bf16 B operands
            // (slab (m, hh): key rows 32 m + 16 hh + {kg 4 + 0..3, 8 + kg 4 + 0..3})
            // (formed once per chunk when the wave has several row blocks, else at their use)
            constexpr bool SB_ONCE = NRB / WPC > 1;
            bf16x8 sb[SB_ONCE ? 2 * NKB : 1];
            if (SB_ONCE) {
#pragma unroll
                for (int m = 0; m < NKB; m++)
#pragma unroll
                    for (int hh = 0; hh < 2; hh++)
#pragma unroll
                        for (int j = 0; j < 8; j++) sb[2 * m + hh][j] = (__bf16)S[m][8 * hh + j];
            }
#pragma unroll
            for (int rb = 0; rb < NRB; rb++) {
                if (rb % WPC != rank % WPC) continue;
                f32x16 acc = {};
                const __bf16* qrow = &sm.q[(rb * 32 + n32) * QP + kg * 4];
#pragma unroll
                for (int m = 0; m < NKB; m++)
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
                        const int d0 = 32 * m + 16 * hh;
                        const bf16x4 lo = *(const bf16x4*)(qrow + d0);
                        const bf16x4 hi = *(const bf16x4*)(qrow + d0 + 8);
                        bf16x8 b;
                        if (SB_ONCE) {
                            b = sb[2 * m + hh];
                        } else {
#pragma unroll
                            for (int j = 0; j < 8; j++) b[j] = (__bf16)S[m][8 * hh + j];
                        }
                        acc = mfma(cat(lo, hi), b, acc);
                    }
                if (MODE == DECAY_HEAD) {
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        const int row = rb * 32 + (i >> 2) * 8 + kg * 4 + (i & 3);
                        acc[i] *= decay_pow2(lamc, row + 1);
                    }
                }
#pragma unroll
                for (int ks = 0; ks < 2 * (rb + 1); ks++) {
                    const bf16x8 a = *(const bf16x8*)(&sm.p[(rb * 32 + n32) * PP + ks * 16 + kg * 8]);
                    acc = mfma(a, vb[ks], acc);
                }
                // accumulator i: row rb 32 + (i / 4) 8 + kg 4 + i % 4, column c0 + 32 cb + n32
                __bf16* orow = o + (row_base + t0 + rb * 32) * DV + c0 + 32 * cb + n32;
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = (i >> 2) * 8 + kg * 4 + (i & 3);
                    if (rb * 32 + row < n) orow[row * DV] = (__bf16)acc[i];
                }
            }
        }

        // ---- state update: S <- a^n S + K^T diag(a^{n-1-j}) V (weights on the V operand; tokens past
        // the chunk's end have zero rows)
        {
            if (MODE == DECAY_HEAD) {
                const float fh = decay_pow2(lamc, n);
#pragma unroll
                for (int m = 0; m < NKB; m++)
#pragma unroll
                    for (int i = 0; i < 16; i++) S[m][i] *= fh;
                // element e of a lane's slab operand (the contraction index) is token 16 ks + 8 kg + e
#pragma unroll
                for (int ks = 0; ks < NSLAB; ks++)
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const int tok = 16 * ks + 8 * kg + e;
                        vb[ks][e] = tok < n ? (__bf16)((float)vb[ks][e] * decay_pow2(lamc, n - 1 - tok)) : (__bf16)0.f;
                    }
            }
#pragma unroll
            for (int m = 0; m < NKB; m++) {
                const int col = 32 * m + (G16 & 1) * 16 + (i16 & 3) * 4;
#pragma unroll
                for (int ks = 0; ks < NSLAB; ks++) {
                    const int tb = 16 * ks + (G16 >> 1) * 8 + (i16 >> 2);
                    const bf16x8 a = cat(lds_tr16(&sm.k[tb * QP + col]), lds_tr16(&sm.k[(tb + 4) * QP + col]));
                    S[m] = mfma(a, vb[ks], S[m]);
                }
            }
        }
    }

    // ---- the final state, from one wave per column block
    float* dst = nullptr;
    if (STATE_ONLY) dst = part_state + (ub * (G - 1) + g) * (int64_t)DK * DV;
    else if (g == G - 1 && s_out) dst = s_out + bh * s_out_stride + (int64_t)seg * DK * DV;
    if (dst && rank == 0) {
#pragma unroll
        for (int m = 0; m < NKB; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = 32 * m + (i >> 2) * 8 + kg * 4 + (i & 3);
                dst[r * DV + c0 + 32 * cb + n32] = S[m][i];
            }
    }
    if (STATE_ONLY && tile == 0 && tid < DK)
        part_decay[(ub * (G - 1) + g) * DK + tid] = (MODE == DECAY_HEAD) ? decay_pow(lam, (int)(t_end - t_begin)) : 1.f;
}

// Blocks for `units` units of NTILE tiles, grouped by eight (one per XCD): every unit index below
// a multiple of 8 is covered; blocks whose unit is past the end return at once.
template <int DK, int DVT, int CH, int MODE, bool SO>
hipError_t launch_tiled(const FwdArgs& a, int64_t units, int G, int cps, float* part_state, float* part_decay,
                        const char* name) {
    constexpr int NTILE = DK / DVT;
    const int64_t blocks = ((units + 7) / 8) * 8 * NTILE;
    LA_TRACED(a.tr, name,
              tiled_fwd_kernel<DK, DVT, CH, MODE, SO><<<(unsigned)blocks, NT, 0, a.stream>>>(
                  (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.decay, a.s_in, (__bf16*)a.o,
                  a.s_out, a.s_out_stride, part_state, part_decay, part_state, a.H, a.L, a.nseg, G, cps, units));
    return hipGetLastError();
}

template <int DK, int DVT, int CH, int MODE>
hipError_t launch_tiled_mode(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay) {
    const int64_t ub = a.B * a.H * a.nseg;
    if (G > 1) {
        hipError_t e = launch_tiled<DK, DVT, CH, MODE, true>(a, ub * (G - 1), G, cps, part_state, part_decay,
                                                            "chunk_fwd_tiled_state_pass");
        if (e != hipSuccess) return e;
        e = launch_state_scan(part_state, part_decay, part_state, ub, G - 1, DK, DK, a.stream, a.tr);
        if (e != hipSuccess) return e;
    }
    return launch_tiled<DK, DVT, CH, MODE, false>(a, ub * G, G, cps, part_state, part_decay,
                                                  "chunk_fwd_tiled_output_pass");
}

template <int DK, int DVT, int CH>
hipError_t launch_tiled_d(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay) {
    return a.mode == DECAY_HEAD ? launch_tiled_mode<DK, DVT, CH, DECAY_HEAD>(a, G, cps, part_state, part_decay)
                                : launch_tiled_mode<DK, DVT, CH, DECAY_NONE>(a, G, cps, part_state, part_decay);
}

}  // namespace

hipError_t launch_chunk_fwd_tiled(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay) {
    if (a.dk == 256) return launch_tiled_d<256, 64, 64>(a, G, cps, part_state, part_decay);
    return launch_tiled_d<128, 128, 128>(a, G, cps, part_state, part_decay);
}

}  // namespace la
