// state_correct_mfma.hip -- bf16 output correction o_t += (q_t * cum_t)^T S_recv for dk = dv = 128.
//
// The rank-dk term of the decomposition identity (ZeCO review page, pith_extraction.key_machinery)
// is a tall-skinny product per segment: [tokens x 128] queries, scaled by the cumulative decay
// from the segment start, times the fp32 incoming state [128 x 128], added to O in place.  It is
// HBM-bound (q read, o read and written).
//
// Layout.  Each wave owns 32 value columns and computes the correction transposed,
// Corr^T = S^T (Q * cum)^T, from a query tile staged in LDS; S^T is loaded once per (b, h, segment)
// as bf16 A operands, split hi + lo so that it enters with about 16 mantissa bits.  The fp32
// correction goes back through LDS so that the read-modify-write of O is row-major: every global
// access is 16 bytes per lane and 1 KiB contiguous per wave instruction (a per-lane transposed
// update touches 32 rows per instruction and streams at about half the rate).  The next tile's q
// and o loads are in flight while the current tile is multiplied and written.
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
constexpr int CPITCH = 132;   // fp32 pitch of the staged correction (conflict-free 16-byte column writes)
constexpr int NT = 256;
constexpr int PIECES = TT * D / 8 / NT;  // 16-byte pieces of a tile per thread

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(NT) void state_correct_mfma_kernel(
    const __bf16* __restrict__ q, const float* __restrict__ cum, const float* __restrict__ s_recv,
    __bf16* __restrict__ o, int64_t H, int64_t L, int nseg, int seg_begin, int64_t state_stride,
    int64_t tiles_per_seg, int64_t total_tiles) {
    __shared__ __attribute__((aligned(16))) __bf16 sQ[TT * QPITCH];
    __shared__ __attribute__((aligned(16))) float sC[TT * CPITCH];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n32 = lane & 31, kg = lane >> 5;
    const int np = nseg - seg_begin;
    const int64_t Ls = L / nseg;

    // Tiles are taken in (b, h, segment, tile) order; each workgroup walks a contiguous, balanced
    // range of that list (the grid is sized to fill the machine in one round), advancing a cursor
    // instead of dividing per tile.
    struct Cursor {
        int64_t ti, pidx, bh, h;
    };
    auto advance = [&](Cursor& c) {
        if (++c.ti == tiles_per_seg) {
            c.ti = 0;
            if (++c.pidx == np) {
                c.pidx = 0;
                c.bh++;
                if (++c.h == H) c.h = 0;
            }
        }
    };
    struct Tile {
        int64_t row;   // global row of the tile's first token
        int64_t tau0;  // position of that token inside its segment
        int n;         // tokens in the tile (at least one)
        int64_t sid;   // (b, h, segment) index of the incoming state
        float lam;
    };
    auto tile_of = [&](const Cursor& c) {
        Tile x;
        x.tau0 = c.ti * TT;
        x.row = c.bh * L + (seg_begin + c.pidx) * Ls + x.tau0;
        x.n = (int)min((int64_t)TT, Ls - x.tau0);
        x.sid = c.bh * np + c.pidx;
        x.lam = (MODE == DECAY_HEAD) ? cum[c.h] : 0.f;
        return x;
    };
    // head mode: tiles whose cumulative decay is exactly zero contribute exactly zero
    auto live = [&](const Tile& x) { return MODE != DECAY_HEAD || expf(x.lam * (float)(x.tau0 + 1)) != 0.f; };

    // this thread's 16-byte pieces of a tile: piece r is row (tid + NT r) / 16, columns 8 ((tid + NT r) % 16) + 0..7
    auto piece_row = [&](int r) { return (tid + NT * r) >> 4; };
    auto piece_col = [&](int r) { return ((tid + NT * r) & 15) * 8; };

    // tile loads, one tile ahead: q (and the fp32 cumulative decay in gate mode) for the staging,
    // o for the read-modify-write.  Rows past the tile's end load its last row (no branch, so the
    // loads stay in flight); their q is zeroed at staging and their o is never written.
    u32x4 rq[PIECES], ro[PIECES];
    f32x4 rc[MODE == DECAY_GATE ? 2 * PIECES : 1];
    auto load_tile = [&](int64_t row0, int n) {
#pragma unroll
        for (int r = 0; r < PIECES; r++) {
            const int64_t off = (row0 + min(piece_row(r), n - 1)) * D + piece_col(r);
            rq[r] = *(const u32x4*)(q + off);
            ro[r] = *(const u32x4*)(o + off);
            if (MODE == DECAY_GATE) {
                rc[2 * r] = *(const f32x4*)(cum + off);
                rc[2 * r + 1] = *(const f32x4*)(cum + off + 4);
            }
        }
    };
    auto stage_tile = [&](int n) {
#pragma unroll
        for (int r = 0; r < PIECES; r++) {
            u32x4 x = rq[r];
            if (MODE == DECAY_GATE) {
                const float cf[8] = {rc[2 * r][0], rc[2 * r][1], rc[2 * r][2], rc[2 * r][3],
                                     rc[2 * r + 1][0], rc[2 * r + 1][1], rc[2 * r + 1][2], rc[2 * r + 1][3]};
#pragma unroll
                for (int hh = 0; hh < 4; hh++) {
                    const __bf16 lo = (__bf16)(bits_lo_bf16(x[hh]) * cf[2 * hh]);
                    const __bf16 hi = (__bf16)(bits_hi_bf16(x[hh]) * cf[2 * hh + 1]);
                    x[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
            }
            if (piece_row(r) >= n) x = u32x4{0, 0, 0, 0};
            *(u32x4*)(sQ + piece_row(r) * QPITCH + piece_col(r)) = x;
        }
    };

    // S^T as hi/lo bf16 A operands: k-slab ks holds key dims ks*16 + kg*8 + jj, column 32w + n32
    bf16x8 shi[8], slo[8];
    int64_t loaded_sid = -1;
    auto load_state = [&](const Cursor& c, int64_t sid) {
        const float* S = s_recv + c.bh * state_stride + c.pidx * D * D;
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

    // first live tile of the range
    const int64_t tile_begin = total_tiles * blockIdx.x / gridDim.x;
    const int64_t tile_end = total_tiles * (blockIdx.x + 1) / gridDim.x;
    Cursor cur_c;
    {
        const int64_t sp = tile_begin / tiles_per_seg;
        cur_c.ti = tile_begin % tiles_per_seg;
        cur_c.pidx = sp % np;
        cur_c.bh = sp / np;
        cur_c.h = cur_c.bh % H;
    }
    int64_t t = tile_begin;
    while (t < tile_end && !live(tile_of(cur_c))) {
        t++;
        advance(cur_c);
    }
    if (t >= tile_end) return;
    Tile cur_t = tile_of(cur_c);
    load_tile(cur_t.row, cur_t.n);
    while (true) {
        // next live tile (its loads go out while this one is multiplied)
        int64_t tn = t + 1;
        Cursor nxt_c = cur_c;
        advance(nxt_c);
        while (tn < tile_end && !live(tile_of(nxt_c))) {
            tn++;
            advance(nxt_c);
        }
        const bool has_next = tn < tile_end;
        if (cur_t.sid != loaded_sid) load_state(cur_c, cur_t.sid);
        stage_tile(cur_t.n);
        u32x4 ov[PIECES];
#pragma unroll
        for (int r = 0; r < PIECES; r++) ov[r] = ro[r];
        // the staged tile is complete and the previous tile's correction has been consumed
        lds_barrier();
        Tile nxt_t = cur_t;
        if (has_next) {
            nxt_t = tile_of(nxt_c);
            load_tile(nxt_t.row, nxt_t.n);
        }
#pragma unroll
        for (int ib = 0; ib < 2; ib++) {
            const int itok = ib * 32 + n32;
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const bf16x8 b = *(const bf16x8*)(sQ + itok * QPITCH + ks * 16 + kg * 8);
                acc = mfma(shi[ks], b, acc);
                acc = mfma(slo[ks], b, acc);
            }
            // accumulator 4 g4 + e is token itok, value column 32w + 8 g4 + 4 kg + e
            const float f = (MODE == DECAY_HEAD) ? expf(cur_t.lam * (float)(cur_t.tau0 + itok + 1)) : 1.f;
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++)
                *(f32x4*)(sC + itok * CPITCH + 32 * w + 8 * g4 + 4 * kg) =
                    f32x4{f * acc[4 * g4], f * acc[4 * g4 + 1], f * acc[4 * g4 + 2], f * acc[4 * g4 + 3]};
        }
        lds_barrier();  // correction tile complete; the query tile is no longer read
#pragma unroll
        for (int r = 0; r < PIECES; r++) {
            const int row = piece_row(r), c8 = piece_col(r);
            if (row < cur_t.n) {
                const f32x4 c0 = *(const f32x4*)(sC + row * CPITCH + c8);
                const f32x4 c1 = *(const f32x4*)(sC + row * CPITCH + c8 + 4);
                const float cf[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                u32x4 x;
#pragma unroll
                for (int hh = 0; hh < 4; hh++) {
                    const __bf16 lo = (__bf16)(bits_lo_bf16(ov[r][hh]) + cf[2 * hh]);
                    const __bf16 hi = (__bf16)(bits_hi_bf16(ov[r][hh]) + cf[2 * hh + 1]);
                    x[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *(u32x4*)(o + (cur_t.row + row) * D + c8) = x;
            }
        }
        if (!has_next) break;
        t = tn;
        cur_c = nxt_c;
        cur_t = nxt_t;
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
