// la_device.h -- device-side helpers shared by the HIP kernels of liblachunk (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { DECAY_NONE = 0, DECAY_HEAD = 1, DECAY_GATE = 2 };

constexpr float LOG2E = 1.44269504088896340736f;
constexpr float LN2 = 0.69314718055994530942f;

// bf16 <-> f32.  The widening is exact; the narrowing rounds to nearest even (gfx950 has a
// native packed instruction for it, which the compiler selects for this cast).
__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }
__device__ __forceinline__ __bf16 f2bf(float x) { return (__bf16)x; }

__device__ __forceinline__ float bits_lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bits_hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 bf16 (one 16-byte word) scaled by 8 fp32 factors, rounded to nearest even.
__device__ __forceinline__ u32x4 scale8(u32x4 w, const float* f) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 4; h++) {
        const __bf16 lo = (__bf16)(bits_lo_bf16(w[h]) * f[2 * h]);
        const __bf16 hi = (__bf16)(bits_hi_bf16(w[h]) * f[2 * h + 1]);
        r[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return r;
}

template <typename T> struct io;
template <> struct io<float> {
    __device__ static __forceinline__ float ld(const float* p) { return *p; }
    __device__ static __forceinline__ void st(float* p, float x) { *p = x; }
};
template <> struct io<__bf16> {
    __device__ static __forceinline__ float ld(const __bf16* p) { return (float)*p; }
    __device__ static __forceinline__ void st(__bf16* p, float x) { *p = (__bf16)x; }
};

// Floor on the per-token log-decay of the gate mode (natural log): a_t >= e^-33 ~ 4.7e-15.  A
// decay below it (down to a = 0, g = -inf) is raised to it, which moves every token-pair weight
// prod a_s by at most e^-33 in absolute terms -- far below fp32 resolution of any output -- and
// keeps every cumulative log-decay finite, so no difference of two of them is -inf - -inf.  With
// it, any two consecutive tokens decay by at least 2^-95.3, inside the 2^-96 span the
// matrix-core kernels' factorised pair weights accept (GATE_SPAN_LOG2).
constexpr float GATE_LOG_FLOOR = -33.f;
// Largest decay span, in log2, that one factorisation reference may cover: a key scaled by
// 2^{+96} and a query by 2^{-96} stay normal floats (and bf16) for |q|, |k| in [2^-30, 2^31].
constexpr float GATE_SPAN_LOG2 = 96.f;

// Per-token log-decay of the gate mode: log sigmoid(g) / norm = -softplus(-g) / norm, written
// so that neither branch overflows: softplus(x) = max(x, 0) + log(1 + exp(-|x|)).  The hardware
// base-2 exponential and logarithm (about 1 ulp each) evaluate it; 1 + exp(-|x|) lies in (1, 2],
// so rounding it costs at most 2^-24 in absolute terms, which is what the cumulative sums see.
// The result is floored at GATE_LOG_FLOOR (g = -inf gives the floor, not -inf).
__device__ __forceinline__ float gate_logdecay(float g, float inv_norm) {
    const float x = -g;
    const float y = __builtin_amdgcn_exp2f(-fabsf(x) * LOG2E);
    const float sp = fmaxf(x, 0.f) + LN2 * __builtin_amdgcn_logf(1.f + y);
    return fmaxf(-sp * inv_norm, GATE_LOG_FLOOR);
}

// The same in base 2, log2 a = log a * log2(e), folded into fewer instructions: with
// c1 = inv_norm * log2(e) (and ln 2 * log2(e) = 1), -softplus(-g) * inv_norm * log2(e) =
// min(g, 0) * c1 - inv_norm * log2(1 + 2^{-|g| log2(e)}); floored at GATE_LOG_FLOOR * log2(e).
__device__ __forceinline__ float gate_log2decay(float g, float inv_norm, float c1) {
    const float y = __builtin_amdgcn_exp2f(-fabsf(g) * LOG2E);
    return fmaxf(fmaf(__builtin_amdgcn_logf(1.f + y), -inv_norm, fminf(g, 0.f) * c1), GATE_LOG_FLOOR * LOG2E);
}

// 8 bf16 (one 16-byte word) times 8 fp32 factors, unrounded; and 8 fp32 values rounded to
// nearest even and packed as 8 bf16.
__device__ __forceinline__ void mul8(u32x4 w, const float* f, float* out) {
#pragma unroll
    for (int h = 0; h < 4; h++) {
        out[2 * h] = bits_lo_bf16(w[h]) * f[2 * h];
        out[2 * h + 1] = bits_hi_bf16(w[h]) * f[2 * h + 1];
    }
}
__device__ __forceinline__ u32x4 pack8(const float* x) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 4; h++) {
        const __bf16 lo = (__bf16)x[2 * h];
        const __bf16 hi = (__bf16)x[2 * h + 1];
        r[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return r;
}

// a^m for a per-token log-decay lam and a token distance m >= 0, with a^0 = 1 exactly even when
// lam = -inf (a = 0).
__device__ __forceinline__ float decay_pow(float lam, int m) { return m == 0 ? 1.f : expf(lam * (float)m); }

// The same power through the hardware base-2 exponential (one instruction, about 1 ulp):
// lam2 = lam * log2(e); a^0 = 1 exactly, also for lam2 = -inf.
__device__ __forceinline__ float decay_pow2(float lam2, int m) {
    return m == 0 ? 1.f : __builtin_amdgcn_exp2f(lam2 * (float)m);
}

// s_waitcnt with vmcnt = N (outstanding vector memory operations of this wave) and lgkmcnt = Lg
// (outstanding LDS operations), expcnt left alone.  Used with a bare s_barrier where a full
// __syncthreads would also drain this wave's global loads that are meant to stay in flight.
template <int N, int Lg>
__device__ __forceinline__ void waitcnt() {
    static_assert(N >= 0 && N < 64 && Lg >= 0 && Lg < 16, "counter range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (Lg << 8));
}

// Wait until at most `younger` batches of NPER vector memory operations issued after the batch
// of interest are outstanding (younger < 4).
template <int NPER>
__device__ __forceinline__ void wait_batches(int younger) {
    static_assert(3 * NPER < 64, "counter range");
    if (younger >= 3) waitcnt<3 * NPER, 15>();
    else if (younger == 2) waitcnt<2 * NPER, 15>();
    else if (younger == 1) waitcnt<NPER, 15>();
    else waitcnt<0, 15>();
}

// Workgroup barrier that orders LDS accesses only: LDS writes before it are visible to every wave
// after it, while this wave's global loads stay in flight (a full __syncthreads drains them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The same barrier for a wave that has LDS DMA (global loads into LDS) in flight: an LDS fence
// would wait for those too, because they write LDS.  This waits only for the wave's own LDS
// instructions; the empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier_keep_dma() {
    asm volatile("" ::: "memory");
    waitcnt<63, 0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace la
