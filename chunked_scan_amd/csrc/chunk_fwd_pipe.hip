// chunk_fwd_pipe.hip -- bf16 MFMA chunked forward for dk = dv = 128, chunk = 64, all three
// decay modes, with the chunk tiles streamed HBM -> LDS ahead of the matrix cores.
//
// One workgroup owns one sub-segment of one (b, h, segment) (the split is in chunk_fwd_split.hip)
// and walks its 64-token chunks in order; the fp32 state S (128 x 128) lives in MFMA accumulator
// registers for the whole walk.  Per chunk of n <= 64 tokens, with B_i the inclusive in-chunk
// cumulative log-decay (per key dim in gate mode, lambda*(i+1) in head mode):
//   P[i][j] = sum_d qbar_i[d] kbar_j[d]     masked to j <= i            (intra-chunk "diagonal")
//   O       = diag-scaled (Qbar S) + P V                                 (inter + intra)
//   S      <- diag(exp(B_{n-1})) S + Ktilde^T V,   Ktilde_j = k_j * exp(B_{n-1} - B_j)
// Head/none modes compute P from raw q, k and apply exp(lambda (i-j)) elementwise, and scale the
// rows of Q S by exp(lambda (i+1)) after the product, so every factor is <= 1.  Gate mode must put
// the per-key-dim decay inside the contraction: qbar = q*exp(B_i) (<= 1), kbar = k*exp(-B_j)
// (>= 1, bounded by the chunk's decay span), as in the K-bar / Lambda / Gamma vectors that the
// ZeCO review page discusses (referee_report.minor_comments[3]); its state update is written
// S <- diag(exp(B_{n-1})) (S + Kbar^T V), which needs no third key tile.
//
// The data path is designed around the MFMA register layouts so that almost nothing but MFMA
// operands moves per chunk:
//
// * Loader and compute waves.  Without decay and with head decay the tiles are used exactly as
//   stored (all decay factors are applied to products in registers), so q, k, v go straight from
//   HBM into LDS with global_load_lds_dwordx4, issued by four loader waves.  The stage buffers
//   form a ring: three stages of q, k, v (two chunks in flight while one is computed) in the
//   output pass, five of k, v (four in flight) in the state pass, whose compute per chunk is
//   light.  The compute waves touch no global memory after their start: they write each chunk's
//   outputs into an LDS tile, which the loader waves store row-major (1 KiB contiguous per
//   instruction).  Per chunk one barrier hands a landed stage to the compute waves and frees the
//   stage they finished, and (in the output pass) a second one hands the output tile over.
// * Gate mode.  The loader waves load q, k, v and g into registers two chunks ahead and, while
//   the compute waves work on chunk c, prepare chunk c + 1 in its stage: the in-chunk cumulative
//   log-decay (a per-lane prefix plus a DPP scan across lanes), qbar, kbar, v and the chunk's
//   decay per key dim.  The compute waves then run the no-decay products and scale their state
//   rows by the chunk decay; they store their outputs themselves (the prepared stages leave no
//   room for an output tile).
// * Ragged chunks.  DMA rows past a chunk's end re-read its last row, which only reaches output
//   rows that are never stored; the state update zeroes those tokens' V operand in registers.
// * Swizzle.  Tiles are unpadded (one DMA instruction writes 1 KiB contiguous), so the 16-byte
//   slots of a row are XOR-swizzled with a row-dependent 4-bit pattern chosen to make both the
//   16-byte row reads (16 lanes, 16 consecutive rows) and the transposing 8-byte reads (16 lanes,
//   4 consecutive rows x 2 adjacent slots) free of bank conflicts.
// * Transposed outputs.  Each compute wave owns 32 value columns and computes O^T = S^T Qbar^T +
//   V^T P^T for them.  The score block P^T = K Q^T is computed by every wave with the key rows
//   read in an order sigma (bits 2 and 3 of the row index swapped); with that order the score
//   accumulator of each lane is exactly the B operand the V^T P^T product needs, so scores never
//   go through LDS.
// * Value column order.  Index r of the wave's 32 value columns is column 32 w + sigma(r) (the
//   V operand's transposing reads choose their 4-column groups accordingly); then each lane's
//   output accumulators are 2 runs of 8 consecutive columns, written to the output tile with two
//   16-byte stores.
// * State row order.  The state accumulator S (key rows x this wave's value columns) is built
//   from transposing reads of K whose column starts follow the same sigma; then every state slab
//   is directly the A operand of S^T Qbar^T and its Q operand is the same 16-byte row read the
//   score product uses.
// * Head decay: scores get exp(lambda (i-j)), the inter-chunk part of output column i gets the
//   per-lane scalar exp(lambda (i+1)), and K^T V becomes K^T diag(w) V with the key-to-chunk-end
//   weights w_j = exp(lambda (n-1-j)) on the V operand.  Every factor is <= 1.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int C = 64;
constexpr int D = 128;
constexpr int NT = 512;    // four compute waves, then four loader waves
constexpr int TE = C * D;  // elements of one unpadded tile
constexpr int LDS_TILES = 10;  // 160 KiB: 3 stages of q, k, v plus the output tile, or 5 stages of k, v

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bf16x4 lds_tr16(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((__attribute__((address_space(3))) __bf16*)p));
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// row swizzle: bit0 <- row bit2, bits1-2 <- row bits0-1, bit3 <- row bit3
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1) | (row & 8); }
// element offset of logical (row, col) in a swizzled tile
__device__ __forceinline__ int sw(int row, int col) { return row * D + ((((col >> 3) ^ swz(row))) << 3) + (col & 7); }
// sigma: swap bits 2 and 3 (an involution on 0..31)
__device__ __forceinline__ int sigma(int x) { return (x & 0x13) | ((x & 4) << 1) | ((x & 8) >> 1); }
// accumulator element i of a 32x32 MFMA tile -> its row, for lane group kg
__device__ __forceinline__ int acc_row(int i, int kg) { return (i >> 2) * 8 + kg * 4 + (i & 3); }

struct Ring {
    __bf16* q;
    __bf16* k;
    __bf16* v;
    float* el;  // gate mode: the chunk's decay per key dim, exp(B of its last token)
};

template <bool STATE_ONLY>
struct Dma {
    static constexpr int NDMA = (STATE_ONLY ? 2 : 3) * 4;  // DMA instructions per chunk per loader wave
    // Loader wave lw fills rows 16 lw .. 16 lw + 15 of each tile; rows past the chunk end re-read
    // the chunk's last valid row.
    // Cache policy: the output pass is the last reader of k and v, so their loads are marked
    // non-temporal (nt), which keeps them from displacing q and o in the last-level cache before
    // the output correction reads those two again (head-decay step, B2: 206 -> 186 us); q keeps the
    // default policy, and so does the state pass, whose k and v the output pass reads next.
    static constexpr int KV_CPOL = STATE_ONLY ? 0 : 2;
    __device__ static __forceinline__ void issue(const __bf16* q, const __bf16* k, const __bf16* v, Ring r,
                                                 int64_t row0, int n, int lw, int lane) {
        // a wave-uniform base plus a 32-bit lane offset per instruction
        const int64_t base = row0 * D;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int R = (4 * lw + j) * 4 + (lane >> 4);
            const int off = min(R, n - 1) * D + (((lane & 15) ^ swz(R)) << 3);
            const int dst = (4 * lw + j) * 512;
            if (!STATE_ONLY)
                __builtin_amdgcn_global_load_lds((const void*)(q + base + off), (lds_void*)(r.q + dst), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(k + base + off), (lds_void*)(r.k + dst), 16, 0, KV_CPOL);
            __builtin_amdgcn_global_load_lds((const void*)(v + base + off), (lds_void*)(r.v + dst), 16, 0, KV_CPOL);
        }
    }
};

template <int MODE, bool STATE_ONLY>
__global__ __launch_bounds__(NT, 1) void pipe_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ decay, const float* __restrict__ s_in, __bf16* __restrict__ o,
    float* __restrict__ s_out, int64_t s_out_stride, float* __restrict__ part_state,
    float* __restrict__ part_decay, const float* __restrict__ init_state, int64_t H, int64_t L, int nseg, int G,
    int cps, float inv_norm, __bf16* __restrict__ q_dec, float* __restrict__ total, int64_t total_stride,
    uint8_t* __restrict__ tile_live) {
    constexpr bool GATE = MODE == DECAY_GATE;
    constexpr bool OTILE = !STATE_ONLY && !GATE;  // outputs leave through an LDS tile stored by the loaders
    constexpr int SLOT = STATE_ONLY ? 2 : 3;      // tiles per stage
    constexpr int STAGE = SLOT * TE + (GATE ? 2 * D : 0);  // gate: D floats of chunk decay after the tiles
    // ring stages: NST - 1 chunks in flight (gate: the loaders prepare one stage ahead, so three)
    constexpr int NST = GATE ? 3 : (LDS_TILES - (OTILE ? 1 : 0)) / SLOT;
    __shared__ __attribute__((aligned(16))) __bf16 ring[NST * STAGE];
    // the chunk's outputs, rows unpadded with 16-byte slot s of row r at s ^ (r % 16)
    __shared__ __attribute__((aligned(16))) __bf16 otile[OTILE ? TE : 8];
    __shared__ int first_dead[4];  // gate loader wave lw: its first chunk with zero cumulative decay
    using DM = Dma<STATE_ONLY>;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t u = blockIdx.x;
    const int gper = STATE_ONLY ? (G - 1) : G;
    const int g = (int)(u % gper);
    const int64_t ub = u / gper;
    const int seg = (int)(ub % nseg);
    const int64_t bh = ub / nseg;
    const int64_t h = bh % H;
    const int64_t Lseg = L / nseg;
    const int64_t t_begin = (int64_t)seg * Lseg + (int64_t)g * cps * C;
    const int64_t t_end = min(t_begin + (int64_t)cps * C, (int64_t)(seg + 1) * Lseg);
    const int64_t row_base = bh * L;
    const int nch = (int)((t_end - t_begin + C - 1) / C);
    auto stage = [&](int c) {
        __bf16* b = ring + (c % NST) * STAGE;
        // q is unused in the state pass
        return Ring{b, b + (SLOT - 2) * TE, b + (SLOT - 1) * TE, (float*)(b + SLOT * TE)};
    };
    auto chunk_len = [&](int c) { return (int)min((int64_t)C, t_end - t_begin - (int64_t)c * C); };

    if (wave >= 4 && GATE) {
        // ---- gate-mode loader wave lw.  Its lanes load q, k, v and g two chunks ahead into
        // registers (plain loads: a wave that mixes LDS DMA with reads of what it loaded gets every
        // wait widened to the whole queue), and while the compute waves work on chunk c it prepares
        // chunk c + 1 in its stage: B = inclusive in-chunk sum of log2 a per key dim, q exp2(B),
        // k exp2(-B) and v written to the tiles, el = exp2(B of the last token).  Lane: key dims
        // 8 o8 .. +7 of tokens 4 tg .. +3; the 16 token groups of a dim octet are one 16-lane row,
        // so the scan over them is DPP.
        const int lw = wave - 4;
        const int o8 = 4 * lw + (lane >> 4);
        const int tg = lane & 15;
        struct Raw {
            u32x4 q[4], k[4], v[4];
            f32x4 g[8];
        };
        Raw rA, rB;
        // log2 of the decay from the segment's first token (state pass: the sub-segment's first
        // token) to the end of the last prepared chunk, per key dim of the lane; the output pass
        // starts it from the totals of the sub-segments before this one
        float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (!STATE_ONLY && (q_dec || total || tile_live))
            for (int gg = 0; gg < g; gg++) {
                const float* pd = part_decay + (ub * (G - 1) + gg) * D + 8 * o8;
#pragma unroll
                for (int e = 0; e < 8; e++) run[e] += __builtin_amdgcn_logf(pd[e]);
            }
        // Tile liveness: chunk c is dead for this wave when the exponential of run (the log2 decay from
        // the segment start to the chunk's start; the same instruction that scales q) is zero for all
        // of the wave's key dims, so q times the cumulative decay is exactly zero on them for every
        // token of the chunk.  run only decreases, so the dead chunks are a suffix: the wave keeps the
        // first one in LDS (an atomic min, no register held across the walk) and writes its byte of
        // every chunk's tile word after the walk.
        const bool flags = !STATE_ONLY && tile_live;
        if (flags && lane == 0) first_dead[lw] = nch;
        auto flag_chunk = [&](int c) {
            // exp2 is monotone: all of the lane's dims are zero exactly when the largest one is
            float m = run[0];
#pragma unroll
            for (int e = 1; e < 8; e++) m = fmaxf(m, run[e]);
            if (__ballot(__builtin_amdgcn_exp2f(m) != 0.f) == 0 && lane == 0) atomicMin(&first_dead[lw], c);
        };
        int issued = 0;
        // token row r of chunk `issued` into x (5 loads); the chunk counts as issued after row 3
        auto load_row = [&](Raw& x, int r) {
            const int n = chunk_len(issued);
            const int64_t base = (row_base + t_begin + (int64_t)issued * C) * D;
            const int off = min(4 * tg + r, n - 1) * D + 8 * o8;
            if (!STATE_ONLY) x.q[r] = *(const u32x4*)(q + base + off);
            x.k[r] = *(const u32x4*)(k + base + off);
            x.v[r] = *(const u32x4*)(v + base + off);
            x.g[2 * r] = *(const f32x4*)(decay + base + off);
            x.g[2 * r + 1] = *(const f32x4*)(decay + base + off + 4);
            if (r == 3) issued++;
        };
        auto load = [&](Raw& x) {
#pragma unroll
            for (int r = 0; r < 4; r++) load_row(x, r);
        };
        // Prepares chunk cc from x while (if more) the rows of the next chunk load into fill, one row
        // between the steps of the preparation: the wave keeps the memory pipeline fed instead of
        // stalling on a burst of loads.
        auto prep = [&](const Raw& x, int cc, bool more, Raw& fill) {
            if (flags) flag_chunk(cc);  // before the next chunk's loads take their registers
            const int n = chunk_len(cc);
            const Ring st = stage(cc);
            float b[4][8];
#pragma unroll
            for (int r = 0; r < 4; r++) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    // computed for every row (past the end, g is a copy of the last row), then selected
                    const float la = gate_logdecay(x.g[2 * r + (e >> 2)][e & 3], inv_norm) * LOG2E;
                    b[r][e] = (r ? b[r - 1][e] : 0.f) + (4 * tg + r < n ? la : 0.f);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (more && r < 3) load_row(fill, r);
                __builtin_amdgcn_sched_barrier(0);
            }
            // exclusive prefix of the lane totals over the 16 token groups: an inclusive scan along
            // the 16-lane row (row_shr by 1, 2, 4, 8; lanes shifted in from outside the row add 0)
#pragma unroll
            for (int e = 0; e < 8; e++) {
                float y = b[3][e];
                y += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), 0x111, 0xf, 0xf, true));
                y += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), 0x112, 0xf, 0xf, true));
                y += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), 0x114, 0xf, 0xf, true));
                y += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), 0x118, 0xf, 0xf, true));
                const float ex = y - b[3][e];
#pragma unroll
                for (int r = 0; r < 4; r++) b[r][e] += ex;
            }
            // the chunk's decay per key dim: B of its last token (lane 15 of the row for a full chunk)
            float bl[8];
            if (n == C) {
                const int row = lane >> 4;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const int r0v = __builtin_amdgcn_readlane(__float_as_int(b[3][e]), 15);
                    const int r1v = __builtin_amdgcn_readlane(__float_as_int(b[3][e]), 31);
                    const int r2v = __builtin_amdgcn_readlane(__float_as_int(b[3][e]), 47);
                    const int r3v = __builtin_amdgcn_readlane(__float_as_int(b[3][e]), 63);
                    bl[e] = __int_as_float(row == 0 ? r0v : row == 1 ? r1v : row == 2 ? r2v : r3v);
                }
            } else {
                const int tl = n - 1, src = (lane & 48) + (tl >> 2), rl = tl & 3;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float sel = rl == 0 ? b[0][e] : rl == 1 ? b[1][e] : rl == 2 ? b[2][e] : b[3][e];
                    bl[e] = __shfl(sel, src);
                }
            }
            if (tg == 0) {
                f32x4 e0, e1;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    e0[e] = __builtin_amdgcn_exp2f(bl[e]);
                    e1[e] = __builtin_amdgcn_exp2f(bl[4 + e]);
                }
                *(f32x4*)(st.el + 8 * o8) = e0;
                *(f32x4*)(st.el + 8 * o8 + 4) = e1;
            }
            // decay from the segment start to this chunk's start (for q times the cumulative decay)
            float cf[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                cf[e] = (!STATE_ONLY && q_dec) ? __builtin_amdgcn_exp2f(run[e]) : 0.f;
                run[e] += bl[e];
            }

            __builtin_amdgcn_sched_barrier(0);
            if (more) load_row(fill, 3);
            __builtin_amdgcn_sched_barrier(0);
            // the prepared rows; past the chunk's end every tile row is zero
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int t = 4 * tg + r;
                const int off = sw(t, 8 * o8);
                const bool in = t < n;
                float fk[8], fq[8];
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    fk[e] = in ? __builtin_amdgcn_exp2f(-b[r][e]) : 0.f;
                    fq[e] = in ? __builtin_amdgcn_exp2f(b[r][e]) : 0.f;
                }
                *(u32x4*)(st.k + off) = scale8(x.k[r], fk);
                *(u32x4*)(st.v + off) = in ? x.v[r] : u32x4{0, 0, 0, 0};
                if (!STATE_ONLY) *(u32x4*)(st.q + off) = scale8(x.q[r], fq);
                if (!STATE_ONLY && q_dec && in) {
                    // q times its cumulative decay from the segment start, rounded once
                    float fd[8];
#pragma unroll
                    for (int e = 0; e < 8; e++) fd[e] = fq[e] * cf[e];
                    // a wave-uniform row base plus a 32-bit lane offset (no 64-bit per-lane address)
                    __bf16* const qrow = q_dec + (row_base + t_begin + (int64_t)cc * C) * D;
                    *(u32x4*)(qrow + (t * D + 8 * o8)) = scale8(x.q[r], fd);
                }
            }
        };
        load(rA);
        prep(rA, 0, nch > 1, rB);  // chunk 1 loads meanwhile
        // chunk j's raw data lives in rA for even j, rB for odd j
        auto step = [&](int c, Raw& fill, const Raw& pre) {
            lds_barrier();  // chunk c (prepared) is handed to the compute waves; stage (c - 1) % NST is free
            if (c + 1 < nch) prep(pre, c + 1, issued < nch, fill);  // chunk c + 2 loads meanwhile
        };
        for (int c = 0; c < nch; c += 2) {
            step(c, rA, rB);
            if (c + 1 < nch) step(c + 1, rB, rA);
        }
        if (STATE_ONLY && tg == 0) {
            float* pd = part_decay + (ub * (G - 1) + g) * D + 8 * o8;
#pragma unroll
            for (int e = 0; e < 8; e++) pd[e] = __builtin_amdgcn_exp2f(run[e]);
        }
        if (flags) {
            const int fd = first_dead[lw];
            uint8_t* fl = tile_live + ((bh * nseg + seg) * ((Lseg + C - 1) / C) + (int64_t)g * cps) * 4 + lw;
            for (int c = lane; c < nch; c += 64) fl[4 * c] = c < fd;
        }
        if (!STATE_ONLY && total && g == G - 1 && tg == 0) {  // the segment's total decay
            float* tt = total + bh * total_stride + (int64_t)seg * D + 8 * o8;
#pragma unroll
            for (int e = 0; e < 8; e++) tt[e] = __builtin_amdgcn_exp2f(run[e]);
        }
        return;
    }
    if (wave >= 4) {
        // ---- loader wave: chunk c + 2 is requested as soon as every wave is done with chunk c - 1
        const int lw = wave - 4;
        int issued = 0;
        for (; issued < NST - 1 && issued < nch; issued++)
            DM::issue(q, k, v, stage(issued), row_base + t_begin + (int64_t)issued * C, chunk_len(issued), lw, lane);
        for (int c = 0; c < nch; c++) {
            // this wave's part of chunk c has landed.  Only the younger DMA batches are allowed to be
            // outstanding: loads complete in order, so while any load of chunk c is pending all
            // younger loads are too and the count cannot drop that low, whatever the stores do.
            wait_batches<DM::NDMA>(issued - c - 1);
            __builtin_amdgcn_s_barrier();  // chunk c is handed to the compute waves
            if (issued < nch) {
                DM::issue(q, k, v, stage(issued), row_base + t_begin + (int64_t)issued * C, chunk_len(issued), lw,
                          lane);
                issued++;
            }
            if (OTILE) {
                lds_barrier_keep_dma();  // the compute waves have written chunk c's outputs
                const int n = chunk_len(c);
                const int64_t r0 = row_base + t_begin + (int64_t)c * C;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int pc = (threadIdx.x - 256) + 256 * r;
                    const int row = pc >> 4, sl = pc & 15;
                    const u32x4 y = *(const u32x4*)(otile + row * D + ((sl ^ (row & 15)) << 3));
                    if (row < n) *(u32x4*)(o + (r0 + row) * D + sl * 8) = y;
                }
            }
        }
        return;
    }

    // ---- compute wave w: value columns 32 w + sigma(0..31)
    const int w = wave, n32 = lane & 31, kg = lane >> 5;
    const int G16 = lane >> 4, i16 = lane & 15;
    const float lam = (MODE == DECAY_HEAD) ? decay[h] : 0.f;
    const int vcol_lane = 32 * w + sigma(n32);

    // state tile m: accumulator element i <-> key row 32m + sigma(acc_row(i)), value column vcol_lane
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
            for (int i = 0; i < 16; i++) S[m][i] = src ? src[(32 * m + sigma(acc_row(i, kg))) * D + vcol_lane] : 0.f;
    }

    // per-lane LDS offsets of the transposing reads for the first 16-token slab (tokens kg*8 +
    // {0..3 | 4..7}); slab ks adds 16 ks rows, which leaves the swizzle (row bits 0-3) unchanged.
    // The 4-column group a = i16 % 4 that a read fetches is placed at 4 (bits of a swapped), the
    // sigma order.
    const int quad = 4 * (((i16 & 1) << 1) | ((i16 >> 1) & 1));
    const int tb = (G16 >> 1) * 8 + (i16 >> 2);
    int voff[2];      // V: value column vcol_lane
    int ktoff[4][2];  // K for the state: key column 32m + sigma(n32)
    {
        const int vcol = 32 * w + (G16 & 1) * 16 + quad;
        voff[0] = sw(tb, vcol);
        voff[1] = sw(tb + 4, vcol);
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const int kcol = 32 * m + (G16 & 1) * 16 + quad;
            ktoff[m][0] = sw(tb, kcol);
            ktoff[m][1] = sw(tb + 4, kcol);
        }
    }

    for (int c = 0; c < nch; c++) {
        const Ring cur = stage(c);
        const int n = chunk_len(c);
        // Head decay: the factors exp(lambda d) are recomputed every chunk from a few base-2
        // exponentials and chains of multiplications by exp(lambda) (every factor <= 1).  Hiding
        // lambda's value from the optimiser each chunk keeps these loop invariants from being
        // hoisted into registers for the whole loop.
        float lamc = lam;
        if (MODE == DECAY_HEAD) asm volatile("" : "+s"(lamc));
        lamc *= LOG2E;
        const float e1 = (MODE == DECAY_HEAD) ? decay_pow2(lamc, 1) : 1.f;
        lds_barrier();  // chunk c has landed; every wave is done with chunk c - 1

        // V operand: tokens 16ks + kg*8 + jj (plain order), value column vcol_lane
        bf16x8 vb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            vb[ks] = cat(lds_tr16(cur.v + 16 * ks * D + voff[0]), lds_tr16(cur.v + 16 * ks * D + voff[1]));

        if (!STATE_ONLY) {
            // the state as A operands of S^T Qbar^T: slab (m, hh) holds key dims 32m + 16hh + kg*8 + jj
            bf16x8 sa[4][2];
#pragma unroll
            for (int m = 0; m < 4; m++)
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    bf16x8 x;
#pragma unroll
                    for (int jj = 0; jj < 8; jj++) x[jj] = (__bf16)S[m][8 * hh + jj];
                    sa[m][hh] = x;
                }
#pragma unroll
            for (int ib = 0; ib < 2; ib++) {
                const int itok = ib * 32 + n32;
                // the diagonal block's decay factors are the same for both halves: recomputing them
                // is cheaper than keeping them live
                float lamb = lam;
                if (MODE == DECAY_HEAD) asm volatile("" : "+s"(lamb));
                lamb *= LOG2E;
                const float e1b = (MODE == DECAY_HEAD) ? decay_pow2(lamb, 1) : 1.f;
                const float einv = (MODE == DECAY_HEAD) ? __builtin_amdgcn_exp2f(-lamb) : 1.f;
                // the upward chain below needs exp(31 lambda) to stay a normal float
                const bool up = lamb >= -4.f;
                // Q operand (B of both products): token itok, key dims ks*16 + kg*8 .. +8
                bf16x8 qb[8];
#pragma unroll
                for (int ks = 0; ks < 8; ks++) qb[ks] = *(const bf16x8*)(cur.q + sw(itok, ks * 16 + kg * 8));
                // scores P^T = K Q^T on the causal blocks (jb <= ib); key rows in sigma order, so
                // element 8hh + jj of lane (itok, kg) is key jb*32 + 16hh + kg*8 + jj
                bf16x8 pt[4];  // 16-key slabs: B operand of V^T P^T
#pragma unroll
                for (int jb = 0; jb <= ib; jb++) {
                    f32x16 sc = {};
                    const int krow = jb * 32 + sigma(n32);
#pragma unroll
                    for (int ks = 0; ks < 8; ks++)
                        sc = mfma(*(const bf16x8*)(cur.k + sw(krow, ks * 16 + kg * 8)), qb[ks], sc);
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
                        // head decay: fac[jj] = exp(lambda (itok - jtok)) where itok >= jtok.  The distance
                        // shrinks by one per jj.  Off the diagonal it is always positive: a plain chain.
                        // On the diagonal, for moderate decay, the chain starts at jj = 0 (the largest
                        // distance, at most 31) and multiplies by exp(-lambda): every kept element is
                        // reached before any masked one (negative distance), whose factor may grow but is
                        // discarded by the causal mask below.  For stronger decay (exp(31 lambda) could
                        // underflow) the chain runs downward and restarts at 1 where the distance
                        // reaches 0.
                        float fac[8];
                        if (MODE == DECAY_HEAD) {
                            const int d0 = 32 * (ib - jb) + n32 - 16 * hh - 8 * kg;
                            if (jb < ib) {
                                float gch = decay_pow2(lamb, d0 - 7);
#pragma unroll
                                for (int jj = 7; jj >= 0; jj--) {
                                    fac[jj] = gch;
                                    gch *= e1b;
                                }
                            } else if (up) {
                                float gch = decay_pow2(lamb, max(d0, 0));
#pragma unroll
                                for (int jj = 0; jj < 8; jj++) {
                                    fac[jj] = gch;
                                    gch *= einv;
                                }
                            } else {
                                const int d7 = d0 - 7;
                                float gch = decay_pow2(lamb, max(d7, 0));
                                fac[7] = gch;
#pragma unroll
                                for (int jj = 6; jj >= 0; jj--) {
                                    gch = (d7 + 7 - jj > 0) ? gch * e1b : 1.f;
                                    fac[jj] = gch;
                                }
                            }
                        }
                        bf16x8 x;
#pragma unroll
                        for (int jj = 0; jj < 8; jj++) {
                            const int jtok = jb * 32 + 16 * hh + kg * 8 + jj;
                            float val = sc[8 * hh + jj];
                            if (MODE == DECAY_HEAD) val *= fac[jj];
                            if (jb == ib && jtok > itok) val = 0.f;
                            x[jj] = (__bf16)val;
                        }
                        pt[2 * jb + hh] = x;
                    }
                }
                // O^T for this wave's 32 value columns and the 32 tokens of block ib
                f32x16 acc = {};
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) acc = mfma(sa[m][hh], qb[2 * m + hh], acc);
                if (MODE == DECAY_HEAD) {
                    const float f = decay_pow2(lamb, itok + 1);
#pragma unroll
                    for (int i = 0; i < 16; i++) acc[i] *= f;
                }
#pragma unroll
                for (int s2 = 0; s2 < 2 * (ib + 1); s2++) acc = mfma(vb[s2], pt[s2], acc);
                // accumulators 0..7 are value columns 32w + 8kg + 0..7 (slot 4w + kg), 8..15 are
                // 32w + 16 + 8kg + 0..7 (slot 4w + 2 + kg)
                {
                    bf16x8 x0, x1;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        x0[e] = (__bf16)acc[e];
                        x1[e] = (__bf16)acc[8 + e];
                    }
                    if (OTILE) {
                        __bf16* orow = otile + itok * D;
                        *(bf16x8*)(orow + (((4 * w + kg) ^ (itok & 15)) << 3)) = x0;
                        *(bf16x8*)(orow + (((4 * w + 2 + kg) ^ (itok & 15)) << 3)) = x1;
                    } else if (itok < n) {  // gate mode: no room for the tile beside the prepared stages
                        __bf16* orow = o + (row_base + t_begin + (int64_t)c * C + itok) * D + 32 * w + 8 * kg;
                        *(bf16x8*)orow = x0;
                        *(bf16x8*)(orow + 16) = x1;
                    }
                }
            }
        }

        if (OTILE) lds_barrier();  // the output tile is complete; the loader waves store it

        // state: S <- decay(chunk) S + K^T diag(w) V over the chunk's n tokens
        if (MODE == DECAY_HEAD) {
            const float fh = decay_pow2(lamc, n);
#pragma unroll
            for (int m = 0; m < 4; m++)
#pragma unroll
                for (int i = 0; i < 16; i++) S[m][i] *= fh;
            // token t = 16 ks + kg*8 + jj gets exp(lambda (n - 1 - t)), or 0 past the chunk's end;
            // the exponent grows by one from jj = 7 down to jj = 0
            if (n == C) {  // every chunk but a ragged last one: no token past the end
#pragma unroll
                for (int ks = 0; ks < 4; ks++) {
                    float gch = decay_pow2(lamc, C - 1 - (16 * ks + kg * 8 + 7));
                    float f[8];
#pragma unroll
                    for (int jj = 7; jj >= 0; jj--) {
                        f[jj] = gch;
                        gch *= e1;
                    }
                    vb[ks] = __builtin_bit_cast(bf16x8, scale8(__builtin_bit_cast(u32x4, vb[ks]), f));
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < 4; ks++) {
                    const int e7 = n - 1 - (16 * ks + kg * 8 + 7);
                    float gch = decay_pow2(lamc, max(e7, 0));
#pragma unroll
                    for (int jj = 7; jj >= 0; jj--) {
                        const int e = e7 + 7 - jj;
                        if (jj < 7) gch = (e > 0) ? gch * e1 : 1.f;
                        vb[ks][jj] = (e >= 0) ? (__bf16)((float)vb[ks][jj] * gch) : (__bf16)0.f;
                    }
                }
            }
        } else if (n < C) {
#pragma unroll
            for (int ks = 0; ks < 4; ks++)
#pragma unroll
                for (int jj = 0; jj < 8; jj++)
                    if (16 * ks + kg * 8 + jj >= n) vb[ks][jj] = (__bf16)0.f;
        }
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const bf16x8 a = cat(lds_tr16(cur.k + 16 * ks * D + ktoff[m][0]), lds_tr16(cur.k + 16 * ks * D + ktoff[m][1]));
                S[m] = mfma(a, vb[ks], S[m]);
            }
        if (GATE) {
            // S <- diag(exp(B_end)) (S + Kbar^T V), Kbar = K exp(-B): the same as decaying S and adding
            // (K exp(B_end - B))^T V.  Rows 4 at a time: element 4 g4 + e of tile m is key row
            // 32m + sigma(8 g4 + 4 kg) + e.
#pragma unroll
            for (int m = 0; m < 4; m++)
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    const f32x4 f = *(const f32x4*)(cur.el + 32 * m + sigma(8 * g4 + 4 * kg));
#pragma unroll
                    for (int e = 0; e < 4; e++) S[m][4 * g4 + e] *= f[e];
                }
        }
    }

    float* dst = nullptr;
    if (STATE_ONLY) dst = part_state + (ub * (G - 1) + g) * (int64_t)D * D;
    else if (g == G - 1 && s_out) dst = s_out + bh * s_out_stride + (int64_t)seg * D * D;
    if (dst) {
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
            for (int i = 0; i < 16; i++) dst[(32 * m + sigma(acc_row(i, kg))) * D + vcol_lane] = S[m][i];
    }
    if (STATE_ONLY && !GATE && threadIdx.x < D)
        part_decay[(ub * (G - 1) + g) * D + threadIdx.x] =
            (MODE == DECAY_HEAD) ? decay_pow(lam, (int)(t_end - t_begin)) : 1.f;
}

template <int MODE>
hipError_t launch_mode(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay) {
    const int64_t ub = a.B * a.H * a.nseg;
    const bool fused = MODE == DECAY_GATE;  // q times cumulative decay and the segment totals come from the loaders
    const __bf16* q = (const __bf16*)a.q;
    const __bf16* k = (const __bf16*)a.k;
    const __bf16* v = (const __bf16*)a.v;
    __bf16* o = (__bf16*)a.o;
    if (G > 1) {
        LA_TRACED(a.tr, "chunk_fwd_pipe_state_pass",
                  pipe_fwd_kernel<MODE, true><<<(unsigned)(ub * (G - 1)), NT, 0, a.stream>>>(
                      q, k, v, a.decay, a.s_in, o, a.s_out, a.s_out_stride, part_state, part_decay, nullptr, a.H,
                      a.L, a.nseg, G, cps, a.inv_norm, nullptr, nullptr, 0, nullptr));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_state_scan(part_state, part_decay, part_state, ub, G - 1, D, D, a.stream, a.tr);
        if (e != hipSuccess) return e;
    }
    LA_TRACED(a.tr, "chunk_fwd_pipe_output_pass",
              pipe_fwd_kernel<MODE, false><<<(unsigned)(ub * G), NT, 0, a.stream>>>(
                  q, k, v, a.decay, a.s_in, o, a.s_out, a.s_out_stride, nullptr, part_decay, part_state, a.H, a.L,
                  a.nseg, G, cps, a.inv_norm, fused ? (__bf16*)a.q_dec : nullptr, fused ? a.total : nullptr,
                  a.total_stride, fused ? (uint8_t*)a.tile_live : nullptr));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd_pipe(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay) {
    switch (a.mode) {
        case DECAY_HEAD: return launch_mode<DECAY_HEAD>(a, G, cps, part_state, part_decay);
        case DECAY_GATE: return launch_mode<DECAY_GATE>(a, G, cps, part_state, part_decay);
        default: return launch_mode<DECAY_NONE>(a, G, cps, part_state, part_decay);
    }
}

}  // namespace la
