// chunk_bwd_generic.hip -- chunked backward of the linear-attention recurrence with fp32
// arithmetic on the vector ALUs, for every shape the generic forward takes (f32 or bf16 inputs,
// dk, dv in {16,32,64,128}, chunk in {16,32,64}).  The backward pass is the consequence of the
// forward design that the ZeCO review page lists (pith_extraction.forward_implications): a
// reverse-direction chunk recurrence for the state derivative, next to the forward one.
//
// Per segment (an independent sequence: segment 0 starts from s_in, the others from zero) and per
// chunk of n tokens, with B_i the inclusive in-chunk sum of log a up to token i (per key dim),
// S_{c-1} the state entering the chunk and D_c the derivative of the loss with respect to the state
// leaving it (ds_out for the last chunk):
//   P'[i][j] = d_o_i . v_j                                                         (j <= i)
//   dq_i  = sum_{j<=i} P'[i][j] k_j e^{B_i - B_j} + e^{B_i} (S_{c-1} d_o_i)
//   dk_j  = sum_{i>=j} P'[i][j] q_i e^{B_i - B_j} + e^{B_{n-1} - B_j} (D_c v_j)
//   dv_j  = sum_{i>=j} P[i][j] d_o_i + D_c^T (k_j e^{B_{n-1} - B_j}),   P[i][j] = sum_d q_i k_j e^{B_i - B_j}
//   D_{c-1} = diag(e^{B_{n-1}}) D_c + sum_i (q_i e^{B_i}) d_o_i^T,          ds_in = D before chunk 0
// (the products are per key dim d; every exponent is <= 0).  The decay's derivative uses the
// identity for a loss written through q_t e^{B_t}, k_t e^{-B_t} and e^{B_last} s_out:
//   dL/dB_t = q_t * dq_t - k_t * dk_t  (+ rowsum(s_out * ds_out) at the segment's last token),
// and log a_s enters every B_t with t >= s, so d log a_s = the reverse running sum of dL/dB from s
// to the segment's end.  GATE turns that into dg = d log a * (1 - sigmoid(g)) / gate_norm; HEAD
// sums it over tokens, key dims, batch and segments: d lambda_h = sum (t - t0 + 1) dL/dB_t + Ls E.
//
// Gate mode factorises the pair weight, e^{B_i - B_j} = e^{B_i} e^{-B_j}, into q e^{B} and k e^{-B}
// staged once per chunk, so the inner loops are plain multiply-adds; a chunk whose decay sum is below
// -80 for one of the workgroup's key dims (where e^{-B} could leave fp32's range) keeps the
// per-pair exponentials, so this path has no range restriction.
//
// Three sweeps, each workgroup owning a 32-wide slice of the state:
//   bwd_dq_kernel  (forward in time, rows of dk): recomputes S, writes dq, q * dq (GATE) and
//                  E = rowsum(S_out * ds_out);
//   bwd_dk_kernel  (reverse, rows of dk): carries D rows, writes dk, ds_in and the decay derivative;
//   bwd_dv_kernel  (reverse, columns of dv): carries D columns, writes dv.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int BC = 64;   // largest chunk
constexpr int BD = 128;  // largest head dim
constexpr int BDP = BD + 1;  // row pitch of [row][BD] tiles: odd, so rows a wave steps over fall in different banks
constexpr int BS = 32;   // rows (dk) or columns (dv) of the state per workgroup
constexpr float FACT_MIN = -80.f;  // lowest in-chunk log-decay sum for which e^{-B} is formed

// Sum of x over the workgroup (256 threads), returned to thread 0.
__device__ double block_sum(double x, double* red) {
    __syncthreads();
    red[threadIdx.x] = x;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    return red[0];
}

template <typename T, int MODE>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ decay,
    const float* __restrict__ s_in, const T* __restrict__ d_o, const float* __restrict__ ds_out, int64_t sstride,
    T* __restrict__ dq, float* __restrict__ qdq, float* __restrict__ efin, double* __restrict__ hpart, int64_t H,
    int64_t L, int dk, int dv, int nseg, int C, float inv_norm) {
    __shared__ float Vs[BC * BDP], Os[BC * BDP], Ks[BC * BS], Ps[BC * BC], Ss[BS * BDP];
    __shared__ float Bs[MODE == DECAY_GATE ? BC * BS : 1];
    __shared__ float KH[MODE == DECAY_GATE ? BC * BS : 1], EB[MODE == DECAY_GATE ? BC * BS : 1];  // k e^{-B}, e^{B}
    __shared__ double red[256];
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const int seg = (int)(unit % nseg);
    const int64_t bh = unit / nseg, h = bh % H;
    const int r0 = blockIdx.y * BS, nr = min(BS, dk - r0);
    const int64_t Ls = L / nseg, t0 = (int64_t)seg * Ls;
    const float lam = MODE == DECAY_HEAD ? decay[h] : 0.f;
    bool fact = false;  // gate mode: this chunk uses the factorised weights

    for (int e = tid; e < nr * dv; e += 256) {
        const int r = e / dv, c = e % dv;
        Ss[r * BDP + c] = (seg == 0 && s_in) ? s_in[(bh * dk + r0 + r) * dv + c] : 0.f;
    }
    double hacc = 0.0;
    for (int64_t cs = 0; cs < Ls; cs += C) {
        const int n = (int)min((int64_t)C, Ls - cs);
        const int64_t tb = bh * L + t0 + cs;
        __syncthreads();
        for (int e = tid; e < n * dv; e += 256) {
            const int i = e / dv, c = e % dv;
            Vs[i * BDP + c] = io<T>::ld(v + (tb + i) * dv + c);
            Os[i * BDP + c] = io<T>::ld(d_o + (tb + i) * dv + c);
        }
        for (int e = tid; e < n * nr; e += 256) {
            const int i = e / nr, r = e % nr;
            const int64_t gi = (tb + i) * dk + r0 + r;
            Ks[i * BS + r] = io<T>::ld(k + gi);
            if (MODE == DECAY_GATE) Bs[i * BS + r] = gate_logdecay(decay[gi], inv_norm);
        }
        __syncthreads();
        if (MODE == DECAY_GATE) {
            bool low = false;
            if (tid < nr) {
                float run = 0.f;
                for (int i = 0; i < n; i++) {
                    run += Bs[i * BS + tid];
                    Bs[i * BS + tid] = run;
                }
                low = run < FACT_MIN;
            }
            fact = !__syncthreads_or(low);
            if (fact) {
                for (int e = tid; e < n * nr; e += 256) {
                    const int i = e / nr, r = e % nr;
                    const float b = Bs[i * BS + r];
                    EB[i * BS + r] = expf(b);
                    KH[i * BS + r] = Ks[i * BS + r] * expf(-b);
                }
                __syncthreads();
            }
        }
        for (int e = tid; e < n * n; e += 256) {
            const int i = e / n, j = e % n;
            float p = 0.f;
            if (j <= i)
                for (int c = 0; c < dv; c++) p += Os[i * BDP + c] * Vs[j * BDP + c];
            Ps[i * BC + j] = p;
        }
        __syncthreads();
        for (int e = tid; e < n * nr; e += 256) {
            const int i = e / nr, r = e % nr;
            float acc = 0.f;
            float inter = 0.f;
            for (int c = 0; c < dv; c++) inter += Ss[r * BDP + c] * Os[i * BDP + c];
            if (MODE == DECAY_GATE && fact) {
                for (int j = 0; j <= i; j++) acc += Ps[i * BC + j] * KH[j * BS + r];
                acc = EB[i * BS + r] * (acc + inter);
                inter = 0.f;
            } else {
                for (int j = 0; j <= i; j++) {
                    float w = Ps[i * BC + j] * Ks[j * BS + r];
                    if (MODE == DECAY_GATE) w *= expf(Bs[i * BS + r] - Bs[j * BS + r]);
                    if (MODE == DECAY_HEAD) w *= decay_pow(lam, i - j);
                    acc += w;
                }
                if (MODE == DECAY_GATE) inter *= expf(Bs[i * BS + r]);
                if (MODE == DECAY_HEAD) inter *= decay_pow(lam, i + 1);
            }
            const float g = acc + inter;
            const int64_t gi = (tb + i) * dk + r0 + r;
            io<T>::st(dq + gi, g);
            if (MODE == DECAY_GATE && qdq) qdq[gi] = io<T>::ld(q + gi) * g;
            if (MODE == DECAY_HEAD) hacc += (double)(cs + i + 1) * (double)(io<T>::ld(q + gi) * g);
        }
        __syncthreads();
        for (int e = tid; e < nr * dv; e += 256) {
            const int r = e / dv, c = e % dv;
            float s = Ss[r * BDP + c];
            if (MODE == DECAY_GATE && fact) {
                for (int j = 0; j < n; j++) s += KH[j * BS + r] * Vs[j * BDP + c];
                s *= EB[(n - 1) * BS + r];
            } else if (MODE == DECAY_GATE) {
                const float bl = Bs[(n - 1) * BS + r];
                s *= expf(bl);
                for (int j = 0; j < n; j++) s += Ks[j * BS + r] * expf(bl - Bs[j * BS + r]) * Vs[j * BDP + c];
            } else if (MODE == DECAY_HEAD) {
                s *= decay_pow(lam, n);
                for (int j = 0; j < n; j++) s += Ks[j * BS + r] * decay_pow(lam, n - 1 - j) * Vs[j * BDP + c];
            } else {
                for (int j = 0; j < n; j++) s += Ks[j * BS + r] * Vs[j * BDP + c];
            }
            Ss[r * BDP + c] = s;
        }
    }
    __syncthreads();
    if (MODE == DECAY_NONE) return;
    // E[r] = sum_c S_out[r][c] ds_out[r][c]: the loss's dependence on the segment's total decay
    if (tid < nr) {
        float e = 0.f;
        if (ds_out) {
            const float* dso = ds_out + bh * sstride + ((int64_t)seg * dk + r0 + tid) * dv;
            for (int c = 0; c < dv; c++) e += Ss[tid * BDP + c] * dso[c];
        }
        if (MODE == DECAY_GATE && efin) efin[(bh * nseg + seg) * dk + r0 + tid] = e;
        if (MODE == DECAY_HEAD) hacc += (double)Ls * (double)e;
    }
    if (MODE == DECAY_HEAD && hpart) {
        const double s = block_sum(hacc, red);
        if (tid == 0) hpart[(unit * gridDim.y + blockIdx.y) * 2 + 0] = s;
    }
}

template <typename T, int MODE>
__global__ __launch_bounds__(256) void bwd_dk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ decay,
    const T* __restrict__ d_o, const float* __restrict__ ds_out, int64_t sstride, T* __restrict__ dk_out,
    float* __restrict__ ds_in, const float* __restrict__ qdq, const float* __restrict__ efin,
    float* __restrict__ d_decay, double* __restrict__ hpart, int64_t H, int64_t L, int dk, int dv, int nseg, int C,
    float inv_norm) {
    __shared__ float Vs[BC * BDP], Os[BC * BDP], Qs[BC * BS], Ks[BC * BS], Ps[BC * BC], Ds[BS * BDP];
    __shared__ float Bs[MODE == DECAY_GATE ? BC * BS : 1], KD[MODE == DECAY_GATE ? BC * BS : 1];
    __shared__ float QB[MODE == DECAY_GATE ? BC * BS : 1], EI[MODE == DECAY_GATE ? BC * BS : 1];  // q e^{B}, e^{-B}
    __shared__ float ELs[MODE == DECAY_GATE ? BS : 1];  // e^{B_{n-1}}
    __shared__ double red[256];
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const int seg = (int)(unit % nseg);
    const int64_t bh = unit / nseg, h = bh % H;
    const int r0 = blockIdx.y * BS, nr = min(BS, dk - r0);
    const int64_t Ls = L / nseg, t0 = (int64_t)seg * Ls;
    const float lam = MODE == DECAY_HEAD ? decay[h] : 0.f;
    const bool want_gate = MODE == DECAY_GATE && d_decay && qdq && efin;
    bool fact = false;  // gate mode: this chunk uses the factorised weights

    for (int e = tid; e < nr * dv; e += 256) {
        const int r = e / dv, c = e % dv;
        Ds[r * BDP + c] = ds_out ? ds_out[bh * sstride + ((int64_t)seg * dk + r0 + r) * dv + c] : 0.f;
    }
    float carry = (want_gate && tid < nr) ? efin[(bh * nseg + seg) * dk + r0 + tid] : 0.f;
    double hacc = 0.0;
    const int64_t nch = (Ls + C - 1) / C;
    for (int64_t cc = nch - 1; cc >= 0; cc--) {
        const int64_t cs = cc * C;
        const int n = (int)min((int64_t)C, Ls - cs);
        const int64_t tb = bh * L + t0 + cs;
        __syncthreads();
        for (int e = tid; e < n * dv; e += 256) {
            const int i = e / dv, c = e % dv;
            Vs[i * BDP + c] = io<T>::ld(v + (tb + i) * dv + c);
            Os[i * BDP + c] = io<T>::ld(d_o + (tb + i) * dv + c);
        }
        for (int e = tid; e < n * nr; e += 256) {
            const int i = e / nr, r = e % nr;
            const int64_t gi = (tb + i) * dk + r0 + r;
            Qs[i * BS + r] = io<T>::ld(q + gi);
            Ks[i * BS + r] = io<T>::ld(k + gi);
            if (MODE == DECAY_GATE) Bs[i * BS + r] = gate_logdecay(decay[gi], inv_norm);
        }
        __syncthreads();
        if (MODE == DECAY_GATE) {
            bool low = false;
            if (tid < nr) {
                float run = 0.f;
                for (int i = 0; i < n; i++) {
                    run += Bs[i * BS + tid];
                    Bs[i * BS + tid] = run;
                }
                low = run < FACT_MIN;
                ELs[tid] = expf(run);
            }
            fact = !__syncthreads_or(low);
            if (fact) {
                for (int e = tid; e < n * nr; e += 256) {
                    const int i = e / nr, r = e % nr;
                    const float b = Bs[i * BS + r];
                    QB[i * BS + r] = Qs[i * BS + r] * expf(b);
                    EI[i * BS + r] = expf(-b);
                }
                __syncthreads();
            }
        }
        for (int e = tid; e < n * n; e += 256) {
            const int i = e / n, j = e % n;
            float p = 0.f;
            if (j <= i)
                for (int c = 0; c < dv; c++) p += Os[i * BDP + c] * Vs[j * BDP + c];
            Ps[i * BC + j] = p;
        }
        __syncthreads();
        for (int e = tid; e < n * nr; e += 256) {
            const int j = e / nr, r = e % nr;
            float acc = 0.f;
            float inter = 0.f;
            for (int c = 0; c < dv; c++) inter += Ds[r * BDP + c] * Vs[j * BDP + c];
            if (MODE == DECAY_GATE && fact) {
                for (int i = j; i < n; i++) acc += Ps[i * BC + j] * QB[i * BS + r];
                acc = EI[j * BS + r] * (acc + ELs[r] * inter);
                inter = 0.f;
            } else {
                for (int i = j; i < n; i++) {
                    float w = Ps[i * BC + j] * Qs[i * BS + r];
                    if (MODE == DECAY_GATE) w *= expf(Bs[i * BS + r] - Bs[j * BS + r]);
                    if (MODE == DECAY_HEAD) w *= decay_pow(lam, i - j);
                    acc += w;
                }
                if (MODE == DECAY_GATE) inter *= expf(Bs[(n - 1) * BS + r] - Bs[j * BS + r]);
                if (MODE == DECAY_HEAD) inter *= decay_pow(lam, n - 1 - j);
            }
            const float g = acc + inter;
            io<T>::st(dk_out + (tb + j) * dk + r0 + r, g);
            const float kg = Ks[j * BS + r] * g;
            if (MODE == DECAY_GATE) KD[j * BS + r] = kg;
            if (MODE == DECAY_HEAD) hacc -= (double)(cs + j + 1) * (double)kg;
        }
        __syncthreads();
        // decay derivative of the gate: reverse running sum of q dq - k dk, one thread per key dim
        if (want_gate && tid < nr) {
            for (int j = n - 1; j >= 0; j--) {
                const int64_t gi = (tb + j) * dk + r0 + tid;
                carry += qdq[gi] - KD[j * BS + tid];
                const float one_minus_sig = 1.f / (1.f + expf(decay[gi]));
                d_decay[gi] = carry * one_minus_sig * inv_norm;
            }
        }
        // D rows carried to the previous chunk
        for (int e = tid; e < nr * dv; e += 256) {
            const int r = e / dv, c = e % dv;
            float s = Ds[r * BDP + c];
            if (MODE == DECAY_GATE && fact) {
                s *= ELs[r];
                for (int i = 0; i < n; i++) s += QB[i * BS + r] * Os[i * BDP + c];
            } else if (MODE == DECAY_GATE) {
                s *= expf(Bs[(n - 1) * BS + r]);
                for (int i = 0; i < n; i++) s += Qs[i * BS + r] * expf(Bs[i * BS + r]) * Os[i * BDP + c];
            } else if (MODE == DECAY_HEAD) {
                s *= decay_pow(lam, n);
                for (int i = 0; i < n; i++) s += Qs[i * BS + r] * decay_pow(lam, i + 1) * Os[i * BDP + c];
            } else {
                for (int i = 0; i < n; i++) s += Qs[i * BS + r] * Os[i * BDP + c];
            }
            Ds[r * BDP + c] = s;
        }
    }
    __syncthreads();
    if (ds_in)
        for (int e = tid; e < nr * dv; e += 256) {
            const int r = e / dv, c = e % dv;
            ds_in[bh * sstride + ((int64_t)seg * dk + r0 + r) * dv + c] = Ds[r * BDP + c];
        }
    if (MODE == DECAY_HEAD && hpart) {
        const double s = block_sum(hacc, red);
        if (tid == 0) hpart[(unit * gridDim.y + blockIdx.y) * 2 + 1] = s;
    }
}

template <typename T, int MODE>
__global__ __launch_bounds__(256) void bwd_dv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ decay, const T* __restrict__ d_o,
    const float* __restrict__ ds_out, int64_t sstride, T* __restrict__ dv_out, int64_t H, int64_t L, int dk, int dv,
    int nseg, int C, float inv_norm) {
    __shared__ float Qs[BC * BDP], Ks[BC * BDP], Os[BC * BS], Ps[BC * BC], Ds[BD * BS];
    __shared__ float Bs[MODE == DECAY_GATE ? BC * BDP : 1];
    __shared__ float ELd[MODE == DECAY_GATE ? BD : 1];  // e^{B_{n-1}} per key dim
    bool fact = false;  // gate mode: this chunk's q, k tiles hold q e^{B} and k e^{-B}
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const int seg = (int)(unit % nseg);
    const int64_t bh = unit / nseg, h = bh % H;
    const int c0 = blockIdx.y * BS, nc = min(BS, dv - c0);
    const int64_t Ls = L / nseg, t0 = (int64_t)seg * Ls;
    const float lam = MODE == DECAY_HEAD ? decay[h] : 0.f;

    for (int e = tid; e < dk * nc; e += 256) {
        const int d = e / nc, c = e % nc;
        Ds[d * BS + c] = ds_out ? ds_out[bh * sstride + ((int64_t)seg * dk + d) * dv + c0 + c] : 0.f;
    }
    const int64_t nch = (Ls + C - 1) / C;
    for (int64_t cc = nch - 1; cc >= 0; cc--) {
        const int64_t cs = cc * C;
        const int n = (int)min((int64_t)C, Ls - cs);
        const int64_t tb = bh * L + t0 + cs;
        __syncthreads();
        for (int e = tid; e < n * dk; e += 256) {
            const int i = e / dk, d = e % dk;
            const int64_t gi = (tb + i) * dk + d;
            Qs[i * BDP + d] = io<T>::ld(q + gi);
            Ks[i * BDP + d] = io<T>::ld(k + gi);
            if (MODE == DECAY_GATE) Bs[i * BDP + d] = gate_logdecay(decay[gi], inv_norm);
        }
        for (int e = tid; e < n * nc; e += 256) {
            const int i = e / nc, c = e % nc;
            Os[i * BS + c] = io<T>::ld(d_o + (tb + i) * dv + c0 + c);
        }
        __syncthreads();
        if (MODE == DECAY_GATE) {
            bool low = false;
            for (int d = tid; d < dk; d += 256) {
                float run = 0.f;
                for (int i = 0; i < n; i++) {
                    run += Bs[i * BDP + d];
                    Bs[i * BDP + d] = run;
                }
                low = low || run < FACT_MIN;
                ELd[d] = expf(run);
            }
            fact = !__syncthreads_or(low);
            if (fact) {
                for (int e = tid; e < n * dk; e += 256) {
                    const int i = e / dk, d = e % dk;
                    const float b = Bs[i * BDP + d];
                    Qs[i * BDP + d] *= expf(b);
                    Ks[i * BDP + d] *= expf(-b);
                }
                __syncthreads();
            }
        }
        // P[i][j] = sum_d q_i[d] k_j[d] e^{B_i[d] - B_j[d]}   (j <= i)
        for (int e = tid; e < n * n; e += 256) {
            const int i = e / n, j = e % n;
            float p = 0.f;
            if (j <= i) {
                if (MODE == DECAY_GATE && !fact) {
                    for (int d = 0; d < dk; d++)
                        p += Qs[i * BDP + d] * Ks[j * BDP + d] * expf(Bs[i * BDP + d] - Bs[j * BDP + d]);
                } else {
                    for (int d = 0; d < dk; d++) p += Qs[i * BDP + d] * Ks[j * BDP + d];
                    if (MODE == DECAY_HEAD) p *= decay_pow(lam, i - j);
                }
            }
            Ps[i * BC + j] = p;
        }
        __syncthreads();
        for (int e = tid; e < n * nc; e += 256) {
            const int j = e / nc, c = e % nc;
            float acc = 0.f;
            for (int i = j; i < n; i++) acc += Ps[i * BC + j] * Os[i * BS + c];
            float inter = 0.f;
            if (MODE == DECAY_GATE && fact) {
                for (int d = 0; d < dk; d++) inter += Ks[j * BDP + d] * ELd[d] * Ds[d * BS + c];
            } else if (MODE == DECAY_GATE) {
                const float* bl = Bs + (n - 1) * BDP;
                for (int d = 0; d < dk; d++) inter += Ks[j * BDP + d] * expf(bl[d] - Bs[j * BDP + d]) * Ds[d * BS + c];
            } else {
                for (int d = 0; d < dk; d++) inter += Ks[j * BDP + d] * Ds[d * BS + c];
                if (MODE == DECAY_HEAD) inter *= decay_pow(lam, n - 1 - j);
            }
            io<T>::st(dv_out + (tb + j) * dv + c0 + c, acc + inter);
        }
        __syncthreads();
        for (int e = tid; e < dk * nc; e += 256) {
            const int d = e / nc, c = e % nc;
            float s = Ds[d * BS + c];
            if (MODE == DECAY_GATE && fact) {
                s *= ELd[d];
                for (int i = 0; i < n; i++) s += Qs[i * BDP + d] * Os[i * BS + c];
            } else if (MODE == DECAY_GATE) {
                s *= expf(Bs[(n - 1) * BDP + d]);
                for (int i = 0; i < n; i++) s += Qs[i * BDP + d] * expf(Bs[i * BDP + d]) * Os[i * BS + c];
            } else if (MODE == DECAY_HEAD) {
                s *= decay_pow(lam, n);
                for (int i = 0; i < n; i++) s += Qs[i * BDP + d] * decay_pow(lam, i + 1) * Os[i * BS + c];
            } else {
                for (int i = 0; i < n; i++) s += Qs[i * BDP + d] * Os[i * BS + c];
            }
            Ds[d * BS + c] = s;
        }
    }
}

// d lambda_h = sum over batch, segments and key-dim slices of the two sweeps' partial sums.
__global__ __launch_bounds__(256) void bwd_head_reduce_kernel(const double* __restrict__ hpart,
                                                              float* __restrict__ d_decay, int64_t B, int64_t H,
                                                              int nseg, int nsl) {
    const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    double s = 0.0;
    for (int64_t b = 0; b < B; b++)
        for (int p = 0; p < nseg; p++) {
            const double* x = hpart + (((b * H + h) * nseg + p) * nsl) * 2;
            for (int y = 0; y < 2 * nsl; y++) s += x[y];
        }
    d_decay[h] = (float)s;
}

template <typename T, int MODE>
hipError_t launch_mode(const BwdArgs& a, float* qdq, float* efin, double* hpart) {
    const int64_t units = a.B * a.H * a.nseg;
    const int nsl = (a.dk + BS - 1) / BS, nsv = (a.dv + BS - 1) / BS;
    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const T* d_o = (const T*)a.d_o;
    const int64_t ss = a.state_stride;
    if (units > 0) {
        const dim3 g1((unsigned)units, (unsigned)nsl), g3((unsigned)units, (unsigned)nsv);
        LA_TRACED(a.tr, "chunk_bwd_dq", bwd_dq_kernel<T, MODE><<<g1, 256, 0, a.stream>>>(
                                            q, k, v, a.decay, a.s_in, d_o, a.ds_out, ss, (T*)a.dq, qdq, efin, hpart,
                                            a.H, a.L, a.dk, a.dv, a.nseg, a.chunk, a.inv_norm));
        LA_TRACED(a.tr, "chunk_bwd_dk", bwd_dk_kernel<T, MODE><<<g1, 256, 0, a.stream>>>(
                                            q, k, v, a.decay, d_o, a.ds_out, ss, (T*)a.dk_out, a.ds_in, qdq, efin,
                                            MODE == DECAY_GATE ? a.d_decay : nullptr, hpart, a.H, a.L, a.dk, a.dv,
                                            a.nseg, a.chunk, a.inv_norm));
        LA_TRACED(a.tr, "chunk_bwd_dv", bwd_dv_kernel<T, MODE><<<g3, 256, 0, a.stream>>>(
                                            q, k, a.decay, d_o, a.ds_out, ss, (T*)a.dv_out, a.H, a.L, a.dk, a.dv,
                                            a.nseg, a.chunk, a.inv_norm));
    }
    if (MODE == DECAY_HEAD && a.d_decay && a.H > 0)
        LA_TRACED(a.tr, "chunk_bwd_head_reduce",
                  bwd_head_reduce_kernel<<<(unsigned)((a.H + 255) / 256), 256, 0, a.stream>>>(
                      hpart, a.d_decay, a.B, a.H, a.nseg, nsl));
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const BwdArgs& a, float* qdq, float* efin, double* hpart) {
    switch (a.mode) {
        case DECAY_HEAD: return launch_mode<T, DECAY_HEAD>(a, qdq, efin, hpart);
        case DECAY_GATE: return launch_mode<T, DECAY_GATE>(a, qdq, efin, hpart);
        default: return launch_mode<T, DECAY_NONE>(a, qdq, efin, hpart);
    }
}

}  // namespace

hipError_t launch_chunk_bwd_generic(const BwdArgs& a) {
    // workspace: GATE q * dq per token and E per segment row; HEAD two fp64 partial sums per workgroup
    const int64_t units = a.B * a.H * a.nseg;
    const int nsl = (a.dk + BS - 1) / BS;
    size_t nfloat = 0;
    if (a.d_decay && a.mode == DECAY_GATE) nfloat = (size_t)(a.B * a.H * a.L * a.dk + units * a.dk);
    if (a.d_decay && a.mode == DECAY_HEAD) nfloat = (size_t)(units * nsl * 4);  // two doubles per workgroup
    float* ws = nullptr;
    if (nfloat > 0) {
        hipError_t e = workspace_alloc((void**)&ws, nfloat * sizeof(float), a.stream);
        if (e != hipSuccess) return e;
    }
    float *qdq = nullptr, *efin = nullptr;
    double* hpart = nullptr;
    if (ws && a.mode == DECAY_GATE) {
        qdq = ws;
        efin = ws + a.B * a.H * a.L * a.dk;
    }
    if (ws && a.mode == DECAY_HEAD) hpart = reinterpret_cast<double*>(ws);
    hipError_t e = a.bf16 ? launch_typed<__bf16>(a, qdq, efin, hpart) : launch_typed<float>(a, qdq, efin, hpart);
    if (ws) {
        hipError_t f = hipFreeAsync(ws, a.stream);
        if (e == hipSuccess) e = f;
    }
    return e;
}

}  // namespace la
