// state_correct_mfma.hip -- bf16 output correction o_t += (q_t * cum_t)^T S_recv for dk = dv = 128.
//
// The rank-dk term of the decomposition identity (ZeCO review page, pith_extraction.key_machinery)
// is a tall-skinny product per segment: [tokens x 128] queries, scaled by the cumulative decay
// from the segment start, times the fp32 incoming state [128 x 128], added to O in place.  It is
// HBM-bound (q read, o read and written).
//
// Both kernels compute the correction transposed, Corr^T = S^T (Q * cum)^T: each compute wave
// owns 32 value columns, holds its slice of S^T as bf16 A operands split hi + lo (about 16
// mantissa bits), and takes 64-token tiles of q from LDS as B operands; every lane then holds 4
// consecutive value columns of one token per accumulator group.  Global accesses are row-major,
// 16 bytes per lane and 1 KiB contiguous per wave instruction (a per-lane transposed update
// touches 32 rows per instruction and streams at about half the rate).
//
// No decay / head decay: loader waves and compute waves.  Four loader waves only issue LDS-DMA
// loads of q and o tiles into a ring of NST stages, so their waits count exactly their own loads;
// four compute waves only read LDS and store O, so their stores never hold up a load.  The
// compute waves update the o tile in LDS in the transposed layout and then store it row-major.
// Head mode applies exp(lambda * tau) to each token's product (a per-lane scalar) and skips tiles
// whose factor is exactly zero in fp32: their correction is exactly zero, so O is bit-identical
// either way.  With per-tile liveness flags (from the forward that formed q * cum), tiles flagged
// zero are skipped in every mode, for the same reason.
//
// Gate decay: the per-token, per-key cumulative decay is an fp32 tensor twice the size of q, so
// q * cum is formed in registers on the way into LDS (rounded to bf16 once) and the fp32
// correction goes back through LDS for a row-major read-modify-write of O; the next tile's loads
// are in flight while the current one is multiplied.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int TT = 64;        // tokens per tile
constexpr int TE = TT * D;    // elements of one tile
constexpr int QPITCH = 136;   // bf16 pitch of the register-staged query tile (conflict-free 16-byte row reads)
constexpr int CPITCH = 132;   // fp32 pitch of the staged correction (conflict-free 16-byte column writes)
constexpr int NT = 256;       // gate kernel: four compute waves
constexpr int NT_WS = 512;    // loader / compute kernel: four of each
constexpr int NST = 5;        // ring stages of the loader / compute kernel (160 KiB of LDS)
constexpr int PIECES = TT * D / 8 / NT;  // 16-byte pieces of a tile per compute thread
constexpr int NDMA = 2 * TT * D / 8 / 64 / 4;  // DMA instructions per tile per loader wave (q and o)

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte slot of logical slot s in row r of an unpadded 256-byte LDS row (XOR swizzle: the 16
// rows read together by one half-wave land on 16 different bank groups)
__device__ __forceinline__ int pslot(int r, int s) { return s ^ (r & 15); }

// Tiles are taken in (b, h, segment, tile) order; each workgroup walks a contiguous, balanced
// range of that list (the grid is sized to fill the machine in one round), advancing a cursor
// instead of dividing per tile.  Head mode lists only the tiles whose cumulative decay at their
// first token is nonzero in fp32 (the others contribute exactly zero): a leading run of every
// segment, whose length depends on the head only, so the ranges balance the work that remains.
struct Tile {
    int64_t row;   // global row of the tile's first token
    int64_t tau0;  // position of that token inside its segment
    int n;         // tokens in the tile (at least one)
    int64_t sid;   // (b, h, segment) index of the incoming state
    float lam;     // head mode: the head's log-decay
};

// Head mode: tiles of a segment with a nonzero cumulative decay exp(lam (64 ti + 1)) at their first
// token -- the same test the kernels' factors use; it only falls as ti grows, so a binary search.
__device__ __forceinline__ int64_t head_live_tiles(float lam, int64_t tps) {
    int64_t lo = 0, hi = tps;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (expf(lam * (float)(mid * TT + 1)) != 0.f) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

template <int MODE>
struct TileWalk {
    int64_t H, L, Ls, tiles_per_seg;
    int nseg, np, seg_begin;
    const float* cum;
    int64_t t, end;        // position in the tile list and end of this workgroup's range
    int64_t ti, pidx, bh, h;
    int64_t nl;            // tiles of the current segment in the list (head mode: its live tiles)
    int64_t nl_lane = 0;   // head mode with H <= 64: live tiles of head `lane`, looked up by shuffle
    // optional liveness flags [(b,h), segment, tile] (0: the tile's q rows are exactly zero), read
    // 64 tiles of the list at a time into a wave-wide bit mask; head mode skips by its own test
    const uint32_t* flags;
    int64_t wbase = -1;
    uint64_t wmask = 0;

    __device__ int64_t seg_tiles(int64_t hh) const {
        if (MODE != DECAY_HEAD) return tiles_per_seg;
        if (H <= 64) return __shfl(nl_lane, (int)hh);
        return head_live_tiles(cum[hh], tiles_per_seg);
    }

    __device__ TileWalk(int64_t H_, int64_t L_, int nseg_, int seg_begin_, int64_t tps, int64_t total,
                        const float* cum_, const uint32_t* flags_)
        : H(H_), L(L_), Ls(L_ / nseg_), tiles_per_seg(tps), nseg(nseg_), np(nseg_ - seg_begin_),
          seg_begin(seg_begin_), cum(cum_), flags(MODE == DECAY_HEAD ? nullptr : flags_) {
        if (MODE == DECAY_HEAD) {
            // per batch entry the list holds np * sum_h live(h) tiles; lane j finds the live tiles of
            // heads j, j + 64, ...
            const int lane = threadIdx.x & 63;
            int64_t per_b = 0;
            for (int64_t h0 = 0; h0 < H; h0 += 64) {
                const int64_t v = (h0 + lane < H) ? head_live_tiles(cum[h0 + lane], tps) : 0;
                if (h0 == 0) nl_lane = v;
                int64_t sum = v;
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
                per_b += np * sum;
            }
            const int64_t nb = total / (np * tps * H);
            const int64_t live_total = nb * per_b;
            t = live_total * blockIdx.x / gridDim.x;
            end = live_total * (blockIdx.x + 1) / gridDim.x;
            if (t >= end) return;
            int64_t r = t - (t / per_b) * per_b;
            bh = (t / per_b) * H;
            h = 0;
            nl = seg_tiles(0);
            while (r >= np * nl) {  // the head holding list position t
                r -= np * nl;
                bh++;
                h++;
                nl = seg_tiles(h);
            }
            pidx = r / nl;
            ti = r - pidx * nl;
        } else {
            t = total * blockIdx.x / gridDim.x;
            end = total * (blockIdx.x + 1) / gridDim.x;
            const int64_t sp = t / tps;
            ti = t % tps;
            pidx = sp % np;
            bh = sp / np;
            h = bh % H;
            nl = tps;
            skip_dead();
        }
    }
    __device__ bool done() const { return t >= end; }
    __device__ Tile tile() const {
        Tile x;
        x.tau0 = ti * TT;
        x.row = bh * L + (seg_begin + pidx) * Ls + x.tau0;
        x.n = (int)min((int64_t)TT, Ls - x.tau0);
        x.sid = bh * np + pidx;
        x.lam = (MODE == DECAY_HEAD) ? cum[h] : 0.f;
        return x;
    }
    // tiles flagged zero contribute exactly zero.  Called by every lane of a wave with the same state.
    __device__ bool live() {
        if (!flags) return true;
        if (wbase < 0 || t >= wbase + 64) {  // the walk only moves forward
            wbase = t;
            const int64_t tl = t + (threadIdx.x & 63);
            bool f = false;
            if (tl < end) {
                const int64_t sp = tl / tiles_per_seg;
                f = flags[((sp / np) * nseg + seg_begin + sp % np) * tiles_per_seg + tl % tiles_per_seg] != 0;
            }
            wmask = __ballot(f);
        }
        return (wmask >> (t - wbase)) & 1;
    }
    __device__ void step() {
        t++;
        if (++ti == nl) {
            ti = 0;
            if (++pidx == np) {
                pidx = 0;
                // next (b, h); head mode passes over heads with no live tile
                do {
                    bh++;
                    if (++h == H) h = 0;
                    if (MODE == DECAY_HEAD) nl = seg_tiles(h);
                } while (MODE == DECAY_HEAD && nl == 0 && t < end);
            }
        }
    }
    __device__ void skip_dead() {
        while (!done() && !live()) step();
    }
    __device__ void next() {
        step();
        skip_dead();
    }
};

// S^T slice of compute wave cw as hi/lo bf16 A operands: k-slab ks holds key dims
// ks*16 + kg*8 + jj of value column 32 cw + n32
__device__ __forceinline__ void load_state_ops(const float* S, int cw, int n32, int kg, bf16x8 (&shi)[8],
                                               bf16x8 (&slo)[8]) {
    // the lane's offset, hidden from the optimiser: otherwise the 64 per-lane addresses are hoisted
    // out of the tile loop as loop invariants and spill
    int lo = kg * 8 * D + 32 * cw + n32;
    asm volatile("" : "+v"(lo));
#pragma unroll
    for (int ks = 0; ks < 8; ks++)
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
            const float x = S[lo + (ks * 16 + jj) * D];
            const __bf16 hi = (__bf16)x;
            shi[ks][jj] = hi;
            slo[ks][jj] = (__bf16)(x - (float)hi);
        }
}

// ---------------------------------------------------------------- no decay / head decay

template <int MODE>
__global__ __launch_bounds__(NT_WS, 1) void state_correct_ws_kernel(
    const __bf16* __restrict__ q, const float* __restrict__ cum, const float* __restrict__ s_recv,
    __bf16* __restrict__ o, int64_t H, int64_t L, int nseg, int seg_begin, int64_t state_stride,
    int64_t tiles_per_seg, int64_t total_tiles, const uint32_t* __restrict__ flags) {
    // stage b: q tile at ring + 2 b TE, o tile at ring + (2 b + 1) TE; rows unpadded, slots swizzled
    __shared__ __attribute__((aligned(16))) __bf16 ring[NST * 2 * TE];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    TileWalk<MODE> walk(H, L, nseg, seg_begin, tiles_per_seg, total_tiles, cum, flags);
    if (walk.done()) return;  // every wave of the workgroup sees the same (empty) range

    if (wave >= 4) {
        // ---- loader wave lw: rows 16 lw .. 16 lw + 15 of each tile's q and o
        const int lw = wave - 4;
        int issued = 0;
        auto issue = [&](const Tile& x, int b) {
            __bf16* qs = ring + 2 * b * TE;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                // one instruction fills 4 rows (1 KiB): lane l writes row R, physical slot l % 16
                const int R = 16 * lw + 4 * j + (lane >> 4);
                const int64_t off = (x.row + min(R, x.n - 1)) * D + pslot(R, lane & 15) * 8;
                const int dst = (16 * lw + 4 * j) * D;
                __builtin_amdgcn_global_load_lds((const void*)(q + off), (lds_void*)(qs + dst), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((const void*)(o + off), (lds_void*)(qs + TE + dst), 16, 0, 0);
            }
        };
        while (issued < NST - 1 && !walk.done()) {
            issue(walk.tile(), issued % NST);
            issued++;
            walk.next();
        }
        for (int k = 0; k < issued; k++) {
            // tile k has landed once at most (issued - k - 1) younger tiles are outstanding
            static_assert(NST <= 5, "at most three younger tiles in flight");
            wait_batches<NDMA>(issued - k - 1);
            __builtin_amdgcn_s_barrier();  // B1: tile k is in LDS; stage (k - 1) % NST is free
            if (!walk.done()) {
                issue(walk.tile(), issued % NST);
                issued++;
                walk.next();
            }
            __builtin_amdgcn_s_barrier();  // B2: the compute waves have updated tile k
        }
        return;
    }

    // ---- compute wave cw = wave: value columns 32 cw .. 32 cw + 31
    const int cw = wave, n32 = lane & 31, kg = lane >> 5;
    // the first state goes out before the first tile has landed, so both latencies overlap
    bf16x8 shi[8], slo[8];
    load_state_ops(s_recv + walk.bh * state_stride + walk.pidx * D * D, cw, n32, kg, shi, slo);
    int64_t loaded_sid = walk.tile().sid;
    for (int k = 0; !walk.done(); k++, walk.next()) {
        const Tile x = walk.tile();
        const __bf16* qs = ring + 2 * (k % NST) * TE;
        __bf16* os = ring + (2 * (k % NST) + 1) * TE;
        lds_barrier();  // B1
        if (x.sid != loaded_sid) {
            load_state_ops(s_recv + walk.bh * state_stride + walk.pidx * D * D, cw, n32, kg, shi, slo);
            loaded_sid = x.sid;
        }
#pragma unroll
        for (int ib = 0; ib < 2; ib++) {
            const int itok = ib * 32 + n32;
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const bf16x8 bq = *(const bf16x8*)(qs + itok * D + pslot(itok, 2 * ks + kg) * 8);
                acc = mfma(shi[ks], bq, acc);
                acc = mfma(slo[ks], bq, acc);
            }
            // accumulator 4 g4 + e is token itok, value column 32 cw + 8 g4 + 4 kg + e: logical
            // slot 4 cw + g4 of the row, half kg
            const float f = (MODE == DECAY_HEAD) ? expf(x.lam * (float)(x.tau0 + itok + 1)) : 1.f;
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
                bf16x4* p = (bf16x4*)(os + itok * D + pslot(itok, 4 * cw + g4) * 8 + 4 * kg);
                bf16x4 y = *p;
#pragma unroll
                for (int e = 0; e < 4; e++) y[e] = (__bf16)((float)y[e] + f * acc[4 * g4 + e]);
                *p = y;
            }
        }
        lds_barrier();  // B2: the o tile is updated
#pragma unroll
        for (int r = 0; r < PIECES; r++) {
            const int pc = threadIdx.x + NT * r;
            const int row = pc >> 4, s = pc & 15;
            const u32x4 y = *(const u32x4*)(os + row * D + pslot(row, s) * 8);
            if (row < x.n) *(u32x4*)(o + (x.row + row) * D + s * 8) = y;
        }
    }
}

// ---------------------------------------------------------------- gate decay

__global__ __launch_bounds__(NT) void state_correct_gate_kernel(
    const __bf16* __restrict__ q, const float* __restrict__ cum, const float* __restrict__ s_recv,
    __bf16* __restrict__ o, int64_t H, int64_t L, int nseg, int seg_begin, int64_t state_stride,
    int64_t tiles_per_seg, int64_t total_tiles, const uint32_t* __restrict__ flags) {
    __shared__ __attribute__((aligned(16))) __bf16 sQ[TT * QPITCH];
    __shared__ __attribute__((aligned(16))) float sC[TT * CPITCH];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n32 = lane & 31, kg = lane >> 5;
    TileWalk<DECAY_GATE> walk(H, L, nseg, seg_begin, tiles_per_seg, total_tiles, cum, flags);
    if (walk.done()) return;

    // this thread's 16-byte pieces of a tile: piece r is row (tid + NT r) / 16, columns 8 ((tid + NT r) % 16) + 0..7
    auto piece_row = [&](int r) { return (tid + NT * r) >> 4; };
    auto piece_col = [&](int r) { return ((tid + NT * r) & 15) * 8; };

    // tile loads, one tile ahead.  Rows past the tile's end load its last row (no branch, so the
    // loads stay in flight); their q is zeroed at staging and their o is never written.
    u32x4 rq[PIECES], ro[PIECES];
    f32x4 rc[2 * PIECES];
    auto load_tile = [&](int64_t row0, int n) {
#pragma unroll
        for (int r = 0; r < PIECES; r++) {
            const int64_t off = (row0 + min(piece_row(r), n - 1)) * D + piece_col(r);
            rq[r] = *(const u32x4*)(q + off);
            ro[r] = *(const u32x4*)(o + off);
            rc[2 * r] = *(const f32x4*)(cum + off);
            rc[2 * r + 1] = *(const f32x4*)(cum + off + 4);
        }
    };
    auto stage_tile = [&](int n) {
#pragma unroll
        for (int r = 0; r < PIECES; r++) {
            u32x4 x = rq[r];
            const float cf[8] = {rc[2 * r][0], rc[2 * r][1], rc[2 * r][2], rc[2 * r][3],
                                 rc[2 * r + 1][0], rc[2 * r + 1][1], rc[2 * r + 1][2], rc[2 * r + 1][3]};
#pragma unroll
            for (int hh = 0; hh < 4; hh++) {
                const __bf16 lo = (__bf16)(bits_lo_bf16(x[hh]) * cf[2 * hh]);
                const __bf16 hi = (__bf16)(bits_hi_bf16(x[hh]) * cf[2 * hh + 1]);
                x[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            if (piece_row(r) >= n) x = u32x4{0, 0, 0, 0};
            *(u32x4*)(sQ + piece_row(r) * QPITCH + piece_col(r)) = x;
        }
    };

    bf16x8 shi[8], slo[8];
    int64_t loaded_sid = -1;
    Tile cur_t = walk.tile();
    int64_t cur_bh = walk.bh, cur_pidx = walk.pidx;
    load_tile(cur_t.row, cur_t.n);
    while (true) {
        walk.next();  // the next tile's loads go out while this one is multiplied
        const bool has_next = !walk.done();
        if (cur_t.sid != loaded_sid) {
            load_state_ops(s_recv + cur_bh * state_stride + cur_pidx * D * D, w, n32, kg, shi, slo);
            loaded_sid = cur_t.sid;
        }
        stage_tile(cur_t.n);
        u32x4 ov[PIECES];
#pragma unroll
        for (int r = 0; r < PIECES; r++) ov[r] = ro[r];
        // the staged tile is complete and the previous tile's correction has been consumed
        lds_barrier();
        Tile nxt_t = cur_t;
        if (has_next) {
            nxt_t = walk.tile();
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
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++)
                *(f32x4*)(sC + itok * CPITCH + 32 * w + 8 * g4 + 4 * kg) =
                    f32x4{acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]};
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
                    x[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *(u32x4*)(o + (cur_t.row + row) * D + c8) = x;
            }
        }
        if (!has_next) break;
        cur_t = nxt_t;
        cur_bh = walk.bh;
        cur_pidx = walk.pidx;
    }
}

// ---------------------------------------------------------------- dk = dv = 32 or 64

// Four waves, register-prefetched tiles (one ahead), q (times cum in gate mode) staged into LDS,
// the fp32 correction back through LDS for a row-major read-modify-write of O.  Wave w computes
// the 32 x 32 block (value-column block w % (D / 32), token block w / (D / 32)) of Corr^T = S^T Qc^T
// (d = 32: waves 0 and 1 only); its slice of S^T is held as hi + lo bf16 A operands.
template <int D, int MODE>
__global__ __launch_bounds__(NT) void state_correct_small_kernel(
    const __bf16* __restrict__ q, const float* __restrict__ cum, const float* __restrict__ s_recv,
    __bf16* __restrict__ o, int64_t H, int64_t L, int nseg, int seg_begin, int64_t state_stride,
    int64_t tiles_per_seg, int64_t total_tiles, const uint32_t* __restrict__ flags) {
    constexpr int NCB = D / 32;
    constexpr int KS = D / 16;
    constexpr int QP = D + 8;             // bf16 pitch of the staged queries
    constexpr int CP = D + 4;             // fp32 pitch of the staged correction
    constexpr int PR = TT * D / 8 / NT;   // 16-byte bf16 pieces of a tile per lane
    constexpr int PIECES_ROW = D / 8;
    __shared__ __attribute__((aligned(16))) __bf16 sQ[TT * QP];
    __shared__ __attribute__((aligned(16))) float sC[TT * CP];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n32 = lane & 31, kg = lane >> 5;
    const int cb = w % NCB, ib = w / NCB;
    const bool active = ib < 2;  // d = 32: waves 2 and 3 compute nothing
    TileWalk<MODE> walk(H, L, nseg, seg_begin, tiles_per_seg, total_tiles, cum, flags);
    if (walk.done()) return;

    auto piece_row = [&](int r) { return (tid + NT * r) / PIECES_ROW; };
    auto piece_col = [&](int r) { return ((tid + NT * r) % PIECES_ROW) * 8; };
    // tile loads; rows past the tile's end load its last row (their q is zeroed at staging and
    // their o is never written)
    u32x4 rq[PR], ro[PR];
    f32x4 rc[MODE == DECAY_GATE ? 2 * PR : 1];
    auto load_tile = [&](int64_t row0, int n) {
#pragma unroll
        for (int r = 0; r < PR; r++) {
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
        for (int r = 0; r < PR; r++) {
            u32x4 x = rq[r];
            if (MODE == DECAY_GATE) {
                const float cf[8] = {rc[2 * r][0], rc[2 * r][1], rc[2 * r][2], rc[2 * r][3],
                                     rc[2 * r + 1][0], rc[2 * r + 1][1], rc[2 * r + 1][2], rc[2 * r + 1][3]};
                x = scale8(x, cf);
            }
            if (piece_row(r) >= n) x = u32x4{0, 0, 0, 0};
            *(u32x4*)(sQ + piece_row(r) * QP + piece_col(r)) = x;
        }
    };
    // S^T slice: k-slab ks holds key dims ks*16 + kg*8 + jj of value column 32 cb + n32
    bf16x8 shi[KS], slo[KS];
    auto load_state = [&](const float* S) {
        int lo = kg * 8 * D + 32 * cb + n32;  // hidden from the optimiser: no hoisted address array
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int jj = 0; jj < 8; jj++) {
                const float x = S[lo + (ks * 16 + jj) * D];
                const __bf16 hi = (__bf16)x;
                shi[ks][jj] = hi;
                slo[ks][jj] = (__bf16)(x - (float)hi);
            }
    };

    int64_t loaded_sid = -1;
    Tile cur_t = walk.tile();
    int64_t cur_bh = walk.bh, cur_pidx = walk.pidx;
    load_tile(cur_t.row, cur_t.n);
    while (true) {
        walk.next();  // the next tile's loads go out while this one is multiplied
        const bool has_next = !walk.done();
        if (cur_t.sid != loaded_sid) {
            load_state(s_recv + cur_bh * state_stride + cur_pidx * D * D);
            loaded_sid = cur_t.sid;
        }
        stage_tile(cur_t.n);
        u32x4 ov[PR];
#pragma unroll
        for (int r = 0; r < PR; r++) ov[r] = ro[r];
        lds_barrier();  // the staged tile is complete and the previous correction has been consumed
        Tile nxt_t = cur_t;
        if (has_next) {
            nxt_t = walk.tile();
            load_tile(nxt_t.row, nxt_t.n);
        }
        if (active) {
            const int itok = ib * 32 + n32;
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                const bf16x8 b = *(const bf16x8*)(sQ + itok * QP + ks * 16 + kg * 8);
                acc = mfma(shi[ks], b, acc);
                acc = mfma(slo[ks], b, acc);
            }
            const float f = (MODE == DECAY_HEAD) ? expf(cur_t.lam * (float)(cur_t.tau0 + itok + 1)) : 1.f;
            // accumulator 4 g4 + e is token itok, value column 32 cb + 8 g4 + 4 kg + e
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++)
                *(f32x4*)(sC + itok * CP + 32 * cb + 8 * g4 + 4 * kg) =
                    f32x4{f * acc[4 * g4], f * acc[4 * g4 + 1], f * acc[4 * g4 + 2], f * acc[4 * g4 + 3]};
        }
        lds_barrier();  // correction tile complete; the query tile is no longer read
#pragma unroll
        for (int r = 0; r < PR; r++) {
            const int row = piece_row(r), c8 = piece_col(r);
            if (row < cur_t.n) {
                const f32x4 c0 = *(const f32x4*)(sC + row * CP + c8);
                const f32x4 c1 = *(const f32x4*)(sC + row * CP + c8 + 4);
                const float cf[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                u32x4 x;
#pragma unroll
                for (int hh = 0; hh < 4; hh++) {
                    const __bf16 lo = (__bf16)(bits_lo_bf16(ov[r][hh]) + cf[2 * hh]);
                    const __bf16 hi = (__bf16)(bits_hi_bf16(ov[r][hh]) + cf[2 * hh + 1]);
                    x[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *(u32x4*)(o + (cur_t.row + row) * D + c8) = x;
            }
        }
        if (!has_next) break;
        cur_t = nxt_t;
        cur_bh = walk.bh;
        cur_pidx = walk.pidx;
    }
}

// One round of resident workgroups on the current device: compute units x workgroups per unit.
template <typename K>
int resident_grid(K kernel, int threads, int64_t total_tiles) {
    constexpr int MAXDEV = 64;
    static int cached[MAXDEV] = {};  // per kernel instantiation and device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV) dev = 0;
    if (cached[dev] == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess || per <= 0)
            per = 1;
        cached[dev] = cus * per;
    }
    return (int)min((int64_t)cached[dev], total_tiles);
}

template <typename K>
hipError_t launch_correct(K kernel, int threads, const CorrectArgs& a, int64_t tps, int64_t total) {
    const unsigned grid = (unsigned)resident_grid(kernel, threads, total);
    LA_TRACED(a.tr, "state_correct_mfma",
              kernel<<<grid, threads, 0, a.stream>>>((const __bf16*)a.q, a.cum, a.s_recv, (__bf16*)a.o, a.H, a.L,
                                                     a.nseg, a.seg_begin, a.state_stride, tps, total,
                                                     a.tile_live));
    return hipGetLastError();
}

template <int DS>
hipError_t launch_small(const CorrectArgs& a, int64_t tps, int64_t total) {
    switch (a.mode) {
        case DECAY_HEAD: return launch_correct(state_correct_small_kernel<DS, DECAY_HEAD>, NT, a, tps, total);
        case DECAY_GATE: return launch_correct(state_correct_small_kernel<DS, DECAY_GATE>, NT, a, tps, total);
        default: return launch_correct(state_correct_small_kernel<DS, DECAY_NONE>, NT, a, tps, total);
    }
}

}  // namespace

hipError_t launch_state_correct(const CorrectArgs& a) {
    const bool small = a.bf16 && a.dk == a.dv && (a.dk == 32 || a.dk == 64);
    if (!(a.bf16 && a.dk == D && a.dv == D) && !small) return launch_state_correct_generic(a);
    const int64_t Ls = a.L / a.nseg;
    const int64_t tps = (Ls + TT - 1) / TT;
    const int64_t total = a.B * a.H * (int64_t)(a.nseg - a.seg_begin) * tps;
    if (total == 0) return hipSuccess;
    if (small) return a.dk == 64 ? launch_small<64>(a, tps, total) : launch_small<32>(a, tps, total);
    switch (a.mode) {
        case DECAY_HEAD: return launch_correct(state_correct_ws_kernel<DECAY_HEAD>, NT_WS, a, tps, total);
        case DECAY_GATE: return launch_correct(state_correct_gate_kernel, NT, a, tps, total);
        default: return launch_correct(state_correct_ws_kernel<DECAY_NONE>, NT_WS, a, tps, total);
    }
}

}  // namespace la
