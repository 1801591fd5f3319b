// state_correct_mfma.hip -- bf16 output correction o_t += (q_t * cum_t)^T S_recv for dk = dv = 128.
//
// The rank-dk term of the decomposition identity (ZeCO review page, pith_extraction.key_machinery)
// is a tall-skinny product per segment: [tokens x 128] (queries, scaled by the cumulative decay
// from the segment start) times the fp32 incoming state [128 x 128], added to O in place.  It is
// HBM-bound (q read, o read and written), so the kernel streams 64-token tiles with 16-byte
// coalesced accesses and uses matrix cores only to keep the arithmetic off the critical path.
//
// Accuracy: S_recv is split into two bf16 parts (hi + lo), so it enters with ~16 mantissa bits;
// in head mode the decay is applied to the fp32 product rows, in gate mode q * cum is rounded to
// bf16 before the product.  Accumulation is fp32, O is rounded once.
//
// Head mode skips tiles whose cumulative decay exp(lambda * tau) is exactly zero in fp32: their
// correction is exactly zero, so O is bit-identical either way.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int TT = 64;        // tokens per tile
constexpr int QPITCH = 136;   // bf16 pitch of the staged query tile
constexpr int CPITCH = 132;   // fp32 pitch of the correction tile
constexpr int TILES_PER_BLOCK = 8;
constexpr int NT = 256;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(NT) void state_correct_mfma_kernel(
    const __bf16* __restrict__ q, const float* __restrict__ cum, const float* __restrict__ s_recv,
    __bf16* __restrict__ o, int64_t H, int64_t L, int nseg, int seg_begin, int64_t state_stride,
    int blocks_per_seg) {
    __shared__ __attribute__((aligned(16))) __bf16 sQ[TT * QPITCH];
    __shared__ __attribute__((aligned(16))) float sC[TT * CPITCH];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, n32 = lane & 31, kg = lane >> 5;
    int64_t r = blockIdx.x;
    const int blk = (int)(r % blocks_per_seg);
    r /= blocks_per_seg;
    const int np = nseg - seg_begin;
    const int p = seg_begin + (int)(r % np);
    const int64_t bh = r / np;
    const int64_t h = bh % H;
    const int64_t Ls = L / nseg;
    const int64_t tb0 = (int64_t)blk * TILES_PER_BLOCK * TT;  // first token of the block, inside the segment
    const int64_t tb1 = min(tb0 + (int64_t)TILES_PER_BLOCK * TT, Ls);
    if (tb0 >= tb1) return;
    const float lam = (MODE == DECAY_HEAD) ? cum[h] : 0.f;
    if (MODE == DECAY_HEAD && expf(lam * (float)(tb0 + 1)) == 0.f) return;  // whole block decayed to 0
    const int64_t row0 = bh * L + (int64_t)p * Ls;  // global row of the segment's first token

    // incoming state of this wave's 32 columns as hi/lo bf16 B operands, 8 k-slabs of 16 rows
    bf16x8 bhi[8], blo[8];
    {
        const float* S = s_recv + bh * state_stride + (int64_t)(p - seg_begin) * D * D;
#pragma unroll
        for (int ks = 0; ks < 8; ks++)
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float x = S[(16 * ks + kg * 8 + j) * D + 32 * w + n32];
                const __bf16 hi = (__bf16)x;
                bhi[ks][j] = hi;
                blo[ks][j] = (__bf16)(x - (float)hi);
            }
    }

    for (int64_t tt = tb0; tt < tb1; tt += TT) {
        const int n = (int)min((int64_t)TT, tb1 - tt);
        if (MODE == DECAY_HEAD && expf(lam * (float)(tt + 1)) == 0.f) break;  // later tiles decay further
        __syncthreads();  // previous tile done with sQ / sC
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            const int pc = tid + NT * rr;
            const int row = pc >> 4, c8 = (pc & 15) * 8;
            u32x4 x = {0, 0, 0, 0};
            if (row < n) {
                x = *(const u32x4*)(q + (row0 + tt + row) * D + c8);
                if (MODE == DECAY_GATE) {
                    const float* cp = cum + (row0 + tt + row) * D + c8;
                    const f32x4 c0 = *(const f32x4*)cp, c1 = *(const f32x4*)(cp + 4);
                    const float cf[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
#pragma unroll
                    for (int hh = 0; hh < 4; hh++) {
                        const __bf16 lo = (__bf16)(bits_lo_bf16(x[hh]) * cf[2 * hh]);
                        const __bf16 hi = (__bf16)(bits_hi_bf16(x[hh]) * cf[2 * hh + 1]);
                        x[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                    }
                }
            }
            *(u32x4*)(&sQ[row * QPITCH + c8]) = x;
        }
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const bf16x8 a = *(const bf16x8*)(&sQ[(rb * 32 + n32) * QPITCH + ks * 16 + kg * 8]);
                acc = mfma(a, bhi[ks], acc);
                acc = mfma(a, blo[ks], acc);
            }
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int row = rb * 32 + (i >> 2) * 8 + kg * 4 + (i & 3);
                float val = acc[i];
                if (MODE == DECAY_HEAD) val *= expf(lam * (float)(tt + row + 1));
                sC[row * CPITCH + 32 * w + n32] = val;
            }
        }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            const int pc = tid + NT * rr;
            const int row = pc >> 4, c8 = (pc & 15) * 8;
            if (row < n) {
                __bf16* po = o + (row0 + tt + row) * D + c8;
                u32x4 x = *(const u32x4*)po;
                const f32x4 a0 = *(const f32x4*)(&sC[row * CPITCH + c8]);
                const f32x4 a1 = *(const f32x4*)(&sC[row * CPITCH + c8 + 4]);
                const float add[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
                for (int hh = 0; hh < 4; hh++) {
                    const __bf16 lo = (__bf16)(bits_lo_bf16(x[hh]) + add[2 * hh]);
                    const __bf16 hi = (__bf16)(bits_hi_bf16(x[hh]) + add[2 * hh + 1]);
                    x[hh] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                *(u32x4*)po = x;
            }
        }
    }
}

}  // namespace

hipError_t launch_state_correct(const CorrectArgs& a) {
    if (!(a.bf16 && a.dk == D && a.dv == D)) return launch_state_correct_generic(a);
    const int64_t Ls = a.L / a.nseg;
    const int bps = (int)((Ls + TILES_PER_BLOCK * TT - 1) / (TILES_PER_BLOCK * TT));
    const int64_t nblk = a.B * a.H * (int64_t)(a.nseg - a.seg_begin) * bps;
    if (nblk == 0) return hipSuccess;
    const __bf16* q = (const __bf16*)a.q;
    __bf16* o = (__bf16*)a.o;
    switch (a.mode) {
        case DECAY_HEAD:
            LA_TRACED(a.tr, "state_correct_mfma",
                      state_correct_mfma_kernel<DECAY_HEAD><<<(unsigned)nblk, NT, 0, a.stream>>>(
                          q, a.cum, a.s_recv, o, a.H, a.L, a.nseg, a.seg_begin, a.state_stride, bps));
            break;
        case DECAY_GATE:
            LA_TRACED(a.tr, "state_correct_mfma",
                      state_correct_mfma_kernel<DECAY_GATE><<<(unsigned)nblk, NT, 0, a.stream>>>(
                          q, a.cum, a.s_recv, o, a.H, a.L, a.nseg, a.seg_begin, a.state_stride, bps));
            break;
        default:
            LA_TRACED(a.tr, "state_correct_mfma",
                      state_correct_mfma_kernel<DECAY_NONE><<<(unsigned)nblk, NT, 0, a.stream>>>(
                          q, a.cum, a.s_recv, o, a.H, a.L, a.nseg, a.seg_begin, a.state_stride, bps));
            break;
    }
    return hipGetLastError();
}

}  // namespace la
