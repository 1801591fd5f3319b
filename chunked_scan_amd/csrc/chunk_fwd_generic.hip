// chunk_fwd_generic.hip -- chunked linear-attention forward with fp32 arithmetic on the vector
// ALUs.  Serves fp32 inputs (where bf16 matrix cores could not meet fp32 accuracy) and every
// head-dim / chunk combination that the MFMA kernel does not cover.  Not the throughput path.
//
// One workgroup owns one (b, h, segment, 32-wide slice of dv) and walks the segment's chunks in
// order.  Per chunk of n <= C tokens, with B_i = sum_{s<=i} log a_s (inclusive, per key dim,
// from the chunk start):
//   P[i][j]  = sum_d q_i[d] k_j[d] exp(B_i[d] - B_j[d])          j <= i   (intra-chunk, diagonal kept)
//   o_i      = sum_{j<=i} P[i][j] v_j + sum_d q_i[d] exp(B_i[d]) S[d,:]      (intra + inter)
//   S[d,:]   = exp(B_{n-1}[d]) S[d,:] + sum_j k_j[d] exp(B_{n-1}[d] - B_j[d]) v_j
// Every exponent is <= 0, so no range restriction applies on this path.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int GMAXC = 64;    // largest chunk
constexpr int GMAXDK = 128;  // largest key dim
constexpr int GKP = GMAXDK + 1;  // row pitch of the q, k, log-decay tiles: odd, so the score loop's rows fall in different banks
constexpr int GDVT = 32;     // dv slice per workgroup

template <typename T, int MODE>
__global__ __launch_bounds__(256) void chunk_fwd_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ decay, const float* __restrict__ s_in, T* __restrict__ o,
    float* __restrict__ s_out, int64_t s_out_stride, int64_t H, int64_t L, int dk, int dv, int nseg, int C,
    float inv_norm) {
    __shared__ float Qs[GMAXC * GKP];
    __shared__ float Ks[GMAXC * GKP];
    __shared__ float Bs[MODE == DECAY_GATE ? GMAXC * GKP : 1];
    __shared__ float Vs[GMAXC * GDVT];
    __shared__ float Ps[GMAXC * GMAXC];
    __shared__ float Ss[GMAXDK * GDVT];

    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const int seg = (int)(unit % nseg);
    const int64_t bh = unit / nseg;
    const int64_t h = bh % H;
    const int c0 = blockIdx.y * GDVT;
    const int nc = min(GDVT, dv - c0);
    const int64_t Ls = L / nseg;
    const int64_t t0 = (int64_t)seg * Ls;
    const float lam = (MODE == DECAY_HEAD) ? decay[h] : 0.f;

    for (int e = tid; e < dk * nc; e += 256) {
        int d = e / nc, c = e % nc;
        Ss[d * GDVT + c] = (seg == 0 && s_in) ? s_in[(bh * dk + d) * dv + c0 + c] : 0.f;
    }

    for (int64_t cs = 0; cs < Ls; cs += C) {
        const int n = (int)min((int64_t)C, Ls - cs);
        const int64_t tb = bh * L + t0 + cs;  // global row of the chunk's first token
        __syncthreads();
        for (int e = tid; e < n * dk; e += 256) {
            int i = e / dk, d = e % dk;
            int64_t gi = (tb + i) * dk + d;
            Qs[i * GKP + d] = io<T>::ld(q + gi);
            Ks[i * GKP + d] = io<T>::ld(k + gi);
            if (MODE == DECAY_GATE) Bs[i * GKP + d] = gate_logdecay(decay[gi], inv_norm);
        }
        for (int e = tid; e < n * nc; e += 256) {
            int i = e / nc, c = e % nc;
            Vs[i * GDVT + c] = io<T>::ld(v + (tb + i) * dv + c0 + c);
        }
        __syncthreads();
        if (MODE == DECAY_GATE) {
            for (int d = tid; d < dk; d += 256) {
                float run = 0.f;
                for (int i = 0; i < n; i++) {
                    run += Bs[i * GKP + d];
                    Bs[i * GKP + d] = run;
                }
            }
            __syncthreads();
        }
        // intra-chunk scores
        for (int e = tid; e < n * n; e += 256) {
            int i = e / n, j = e % n;
            float p = 0.f;
            if (j <= i) {
                if (MODE == DECAY_GATE) {
                    for (int d = 0; d < dk; d++)
                        p += Qs[i * GKP + d] * Ks[j * GKP + d] *
                             expf(Bs[i * GKP + d] - Bs[j * GKP + d]);
                } else {
                    for (int d = 0; d < dk; d++) p += Qs[i * GKP + d] * Ks[j * GKP + d];
                    if (MODE == DECAY_HEAD) p *= decay_pow(lam, i - j);
                }
            }
            Ps[i * GMAXC + j] = p;
        }
        __syncthreads();
        // outputs: intra + inter
        for (int e = tid; e < n * nc; e += 256) {
            int i = e / nc, c = e % nc;
            float acc = 0.f;
            for (int j = 0; j <= i; j++) acc += Ps[i * GMAXC + j] * Vs[j * GDVT + c];
            float inter = 0.f;
            if (MODE == DECAY_GATE) {
                for (int d = 0; d < dk; d++)
                    inter += Qs[i * GKP + d] * expf(Bs[i * GKP + d]) * Ss[d * GDVT + c];
            } else {
                for (int d = 0; d < dk; d++) inter += Qs[i * GKP + d] * Ss[d * GDVT + c];
                if (MODE == DECAY_HEAD) inter *= decay_pow(lam, i + 1);
            }
            io<T>::st(o + (tb + i) * dv + c0 + c, acc + inter);
        }
        __syncthreads();
        // state carried to the next chunk
        for (int e = tid; e < dk * nc; e += 256) {
            int d = e / nc, c = e % nc;
            float s = Ss[d * GDVT + c];
            if (MODE == DECAY_GATE) {
                const float bl = Bs[(n - 1) * GKP + d];
                s *= expf(bl);
                for (int j = 0; j < n; j++)
                    s += Ks[j * GKP + d] * expf(bl - Bs[j * GKP + d]) * Vs[j * GDVT + c];
            } else if (MODE == DECAY_HEAD) {
                s *= decay_pow(lam, n);
                for (int j = 0; j < n; j++) s += Ks[j * GKP + d] * decay_pow(lam, n - 1 - j) * Vs[j * GDVT + c];
            } else {
                for (int j = 0; j < n; j++) s += Ks[j * GKP + d] * Vs[j * GDVT + c];
            }
            Ss[d * GDVT + c] = s;
        }
    }
    __syncthreads();
    if (s_out) {
        for (int e = tid; e < dk * nc; e += 256) {
            int d = e / nc, c = e % nc;
            s_out[bh * s_out_stride + ((int64_t)seg * dk + d) * dv + c0 + c] = Ss[d * GDVT + c];
        }
    }
}

template <typename T>
hipError_t launch_typed(const FwdArgs& a) {
    const int64_t units = a.B * a.H * a.nseg;
    dim3 grid((unsigned)units, (unsigned)((a.dv + GDVT - 1) / GDVT));
    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    T* o = (T*)a.o;
    switch (a.mode) {
        case DECAY_HEAD:
            LA_TRACED(a.tr, "chunk_fwd_generic", chunk_fwd_generic_kernel<T, DECAY_HEAD><<<grid, 256, 0, a.stream>>>(
                q, k, v, a.decay, a.s_in, o, a.s_out, a.s_out_stride, a.H, a.L, a.dk, a.dv, a.nseg, a.chunk, a.inv_norm));
            break;
        case DECAY_GATE:
            LA_TRACED(a.tr, "chunk_fwd_generic", chunk_fwd_generic_kernel<T, DECAY_GATE><<<grid, 256, 0, a.stream>>>(
                q, k, v, a.decay, a.s_in, o, a.s_out, a.s_out_stride, a.H, a.L, a.dk, a.dv, a.nseg, a.chunk, a.inv_norm));
            break;
        default:
            LA_TRACED(a.tr, "chunk_fwd_generic", chunk_fwd_generic_kernel<T, DECAY_NONE><<<grid, 256, 0, a.stream>>>(
                q, k, v, a.decay, a.s_in, o, a.s_out, a.s_out_stride, a.H, a.L, a.dk, a.dv, a.nseg, a.chunk, a.inv_norm));
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd_generic(const FwdArgs& a) {
    return a.bf16 ? launch_typed<__bf16>(a) : launch_typed<float>(a);
}

}  // namespace la
