// state_correct_mfma.hip -- bf16 output correction o_t += (q_t * cum_t)^T S_recv for dk = dv = 128.
//
// The rank-dk term of the decomposition identity (ZeCO review page, pith_extraction.key_machinery)
// is a tall-skinny product per segment: [tokens x 128] queries, scaled by the cumulative decay
// from the segment start, times the fp32 incoming state [128 x 128], added to O in place.  It is
// HBM-bound (q read, o read and written).
//
// Layout.  Each wave owns 32 value columns and computes the correction transposed,
// Corr^T = S^T (Q * cum)^T, so every lane ends with 4 consecutive value columns of one token per
// accumulator group and updates O with 8-byte read-modify-writes straight from registers.  The
// query tile goes through LDS once (16-byte coalesced loads, double-buffered); the next tile's q and
// o loads are in flight while the current one is multiplied; S^T is loaded once per workgroup as bf16 A
// operands, split hi + lo so it enters with about 16 mantissa bits.
//
// Head mode applies exp(lambda * tau) to the product of each token (a per-lane scalar) and skips
// tiles whose factor is exactly zero in fp32: their correction is exactly zero, so O is
// bit-identical either way.  Gate mode multiplies q by the cumulative decay before the product
// (rounded to bf16 once).
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int TT = 64;        // tokens per tile
constexpr int QPITCH = 136;   // bf16 pitch of the staged query tile (conflict-free 16-byte row reads)
constexpr int NT = 256;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(NT) void state_correct_mfma_kernel(
    const __bf16* __restrict__ q, const float* __restrict__ cum, const float* __restrict__ s_recv,
    __bf16* __restrict__ o, int64_t H, int64_t L, int nseg, int seg_begin, int64_t state_stride,
    int64_t tiles_per_seg, int64_t total_tiles) {
    __shared__ __attribute__((aligned(16))) __bf16 sQ[2][TT * QPITCH];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n32 = lane & 31, kg = lane >> 5;
    // a contiguous, balanced range of the (b, h, segment, tile) list; the grid is sized to fill
    // the machine in one round
    const int64_t tile_begin = total_tiles * blockIdx.x / gridDim.x;
    const int64_t tile_end = total_tiles * (blockIdx.x + 1) / gridDim.x;
    const int np = nseg - seg_begin;
    const int64_t Ls = L / nseg;

    struct Tile {
        int64_t row;   // global row of the tile's first token
        int64_t tau0;  // position of that token inside its segment
        int n;         // tokens in the tile
        int64_t sid;   // (b, h, segment) index of the incoming state
        float lam;
    };
    auto tile_at = [&](int64_t t) {
        Tile x;
        const int64_t ti = t % tiles_per_seg;
        const int64_t sp = t / tiles_per_seg;  // (bh, p - seg_begin)
        const int p = seg_begin + (int)(sp % np);
        const int64_t bh = sp / np;
        x.tau0 = ti * TT;
        x.row = bh * L + (int64_t)p * Ls + x.tau0;
        x.n = (int)min((int64_t)TT, Ls - x.tau0);
        x.sid = sp;
        x.lam = (MODE == DECAY_HEAD) ? cum[bh % H] : 0.f;
        return x;
    };
    // head mode: tiles whose cumulative decay is exactly zero contribute exactly zero
    auto live = [&](const Tile& x) { return MODE != DECAY_HEAD || expf(x.lam * (float)(x.tau0 + 1)) != 0.f; };

    // tile loads, one tile ahead: 4 x 16 bytes of q (and 2 x 4 x 16 bytes of cum in gate mode) per
    // lane for the staging, and this lane's 2 x 4 x 8 bytes of o for the read-modify-write
    u32x4 rq[4];
    f32x4 rc[MODE == DECAY_GATE ? 8 : 1];
    bf16x4 ro[2][4];
    auto load_tile = [&](int64_t row0, int n) {
#pragma unroll
        for (int ib = 0; ib < 2; ib++) {
            const int itok = ib * 32 + n32;
            if (itok < n) {
                const __bf16* orow = o + (row0 + itok) * D + 32 * w + kg * 4;
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) ro[ib][g4] = *(const bf16x4*)(orow + g4 * 8);
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            const int pc = tid + NT * rr;
            const int row = pc >> 4, c8 = (pc & 15) * 8;
            rq[rr] = row < n ? *(const u32x4*)(q + (row0 + row) * D + c8) : u32x4{0, 0, 0, 0};
            if (MODE == DECAY_GATE) {
                const float* cp = cum + (row0 + row) * D + c8;
                rc[2 * rr] = row < n ? *(const f32x4*)cp : f32x4{0, 0, 0, 0};
                rc[2 * rr + 1] = row < n ? *(const f32x4*)(cp + 4) : f32x4{0, 0, 0, 0};
            }
        }
    };
    auto stage_tile = [&](__bf16* dst) {
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            const int pc = tid + NT * rr;
            const int row = pc >> 4, c8 = (pc & 15) * 8;
            u32x4 x = rq[rr];
            if (MODE == DECAY_GATE) {
                const float cf[8] = {rc[2 * rr][0], rc[2 * rr][1], rc[2 * rr][2], rc[2 * rr][3],
                                     rc[2 * rr + 1][0], rc[2 * rr + 1][1], rc[2 * rr + 1][2], rc[2 * rr + 1][3]};
#pragma unroll
                for (int hh = 0; hh < 4; hh++) {
                    const __bf16 lo = (__bf16)(bits_lo_bf16(x[hh]) * cf[2 * hh]);
                    const __bf16 hi = (__bf16)(bits_hi_bf16(x[hh]) * cf[2 * hh + 1]);
                    x[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
            }
            *(u32x4*)(dst + row * QPITCH + c8) = x;
        }
    };

    // S^T as hi/lo bf16 A operands: k-slab ks holds key dims ks*16 + kg*8 + jj, column 32w + n32
    bf16x8 shi[8], slo[8];
    int64_t loaded_sid = -1;
    auto load_state = [&](int64_t sid) {
        const int64_t bh = sid / np;
        const int pp = (int)(sid % np);
        const float* S = s_recv + bh * state_stride + (int64_t)pp * D * D;
#pragma unroll
        for (int ks = 0; ks < 8; ks++)
#pragma unroll
            for (int jj = 0; jj < 8; jj++) {
                const float x = S[(ks * 16 + kg * 8 + jj) * D + 32 * w + n32];
                const __bf16 hi = (__bf16)x;
                shi[ks][jj] = hi;
                slo[ks][jj] = (__bf16)(x - (float)hi);
            }
        loaded_sid = sid;
    };

    // find the first live tile, load it
    int64_t t = tile_begin;
    while (t < tile_end && !live(tile_at(t))) t++;
    if (t >= tile_end) return;
    Tile cur_t = tile_at(t);
    load_tile(cur_t.row, cur_t.n);
    int buf = 0;
    while (true) {
        // next live tile (its loads go out while this one is multiplied)
        int64_t tn = t + 1;
        while (tn < tile_end && !live(tile_at(tn))) tn++;
        const bool has_next = tn < tile_end;
        if (cur_t.sid != loaded_sid) load_state(cur_t.sid);
        __bf16* cur = sQ[buf];
        stage_tile(cur);
        __syncthreads();  // tile staged; the other buffer's readers finished a tile ago
        bf16x4 ov[2][4];
#pragma unroll
        for (int ib = 0; ib < 2; ib++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) ov[ib][g4] = ro[ib][g4];
        Tile nxt_t = cur_t;
        if (has_next) {
            nxt_t = tile_at(tn);
            load_tile(nxt_t.row, nxt_t.n);
        }
#pragma unroll
        for (int ib = 0; ib < 2; ib++) {
            const int itok = ib * 32 + n32;
            // this lane's outputs: token itok, value columns 32w + g4*8 + kg*4 + 0..3
            __bf16* orow = o + (cur_t.row + itok) * D + 32 * w + kg * 4;
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const bf16x8 b = *(const bf16x8*)(cur + itok * QPITCH + ks * 16 + kg * 8);
                acc = mfma(shi[ks], b, acc);
                acc = mfma(slo[ks], b, acc);
            }
            if (itok < cur_t.n) {
                const float f = (MODE == DECAY_HEAD) ? expf(cur_t.lam * (float)(cur_t.tau0 + itok + 1)) : 1.f;
#pragma unroll
                for (int g4 = 0; g4 < 4; g4++) {
                    bf16x4 x;
#pragma unroll
                    for (int e = 0; e < 4; e++) x[e] = (__bf16)((float)ov[ib][g4][e] + f * acc[4 * g4 + e]);
                    *(bf16x4*)(orow + g4 * 8) = x;
                }
            }
        }
        if (!has_next) break;
        t = tn;
        cur_t = nxt_t;
        buf ^= 1;
    }
}

// One round of resident workgroups: compute units x workgroups per unit for this kernel.
template <typename K>
int resident_grid(K kernel, int64_t total_tiles) {
    static int cached = 0;  // one per kernel instantiation
    if (cached == 0) {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, NT, 0) != hipSuccess || per <= 0) per = 1;
        cached = cus * per;
    }
    return (int)min((int64_t)cached, total_tiles);
}

template <int MODE>
hipError_t launch_correct(const CorrectArgs& a, int64_t tps, int64_t total) {
    auto kernel = state_correct_mfma_kernel<MODE>;
    const unsigned grid = (unsigned)resident_grid(kernel, total);
    LA_TRACED(a.tr, "state_correct_mfma",
              kernel<<<grid, NT, 0, a.stream>>>((const __bf16*)a.q, a.cum, a.s_recv, (__bf16*)a.o, a.H, a.L, a.nseg,
                                                a.seg_begin, a.state_stride, tps, total));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_correct(const CorrectArgs& a) {
    if (!(a.bf16 && a.dk == D && a.dv == D)) return launch_state_correct_generic(a);
    const int64_t Ls = a.L / a.nseg;
    const int64_t tps = (Ls + TT - 1) / TT;
    const int64_t total = a.B * a.H * (int64_t)(a.nseg - a.seg_begin) * tps;
    if (total == 0) return hipSuccess;
    switch (a.mode) {
        case DECAY_HEAD: return launch_correct<DECAY_HEAD>(a, tps, total);
        case DECAY_GATE: return launch_correct<DECAY_GATE>(a, tps, total);
        default: return launch_correct<DECAY_NONE>(a, tps, total);
    }
}

}  // namespace la
