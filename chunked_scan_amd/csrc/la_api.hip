// la_api.hip -- the C ABI of liblachunk.so (declared in include/la_chunk.h).
//
// Every entry point validates all of its arguments on the host before the first HIP call, so a
// rejected call enqueues nothing and touches no device state.  Validation order: shape pointer,
// sizes, dtypes, decay mode, required pointers, aliasing; the first failure is returned.
#include <math.h>
#include <stdint.h>

#include "la_chunk.h"
#include "la_internal.h"

namespace {

using la::CorrectArgs;
using la::FwdArgs;

constexpr int64_t kMaxElems = (int64_t)1 << 60;  // keeps every byte count below 2^63

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }
// The forward's further variants, on matrix-core kernels only (bf16, dk = dv): 128-token chunks
// for d = 32 and 64 (every decay mode) and d = 128 (no or head decay), and d = 256 with 64-token
// chunks (no or head decay).
bool fwd_wide(const la_shape* s) { return s->dk == 256 || s->dv == 256; }
bool fwd_chunk_ok(const la_shape* s, int c) {
    const bool bf = s->in_dtype == LA_BF16 && s->dk == s->dv;
    if (fwd_wide(s)) return bf && s->dk == 256 && c == 64 && s->decay_mode != LA_DECAY_GATE;
    return chunk_ok(c) ||
           (c == 128 && bf && (s->dk == 32 || s->dk == 64 || (s->dk == 128 && s->decay_mode != LA_DECAY_GATE)));
}
size_t esize(int dtype) { return dtype == LA_BF16 ? 2 : 4; }

// Overflow-safe product of non-negative sizes; -1 if it exceeds kMaxElems.
int64_t prod(int64_t a, int64_t b) {
    if (a == 0 || b == 0) return 0;
    if (a > kMaxElems / b) return -1;
    return a * b;
}
int64_t prod4(int64_t a, int64_t b, int64_t c, int64_t d) {
    int64_t x = prod(a, b);
    if (x < 0) return -1;
    x = prod(x, c);
    if (x < 0) return -1;
    return prod(x, d);
}

struct Span {
    const void* p;
    size_t bytes;
};
bool overlap(Span a, Span b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
    return x < y + b.bytes && y < x + a.bytes;
}

// wide_ok: the forward, which also takes dk = dv = 256 (checked with the chunk length)
la_status check_common(const la_shape* s, bool wide_ok = false) {
    if (!s) return LA_ERR_NULL;
    if (s->B < 0 || s->H < 0 || s->L < 0 || s->nseg < 1 || s->dk <= 0 || s->dv <= 0) return LA_ERR_SHAPE;
    if (s->L % s->nseg != 0) return LA_ERR_SHAPE;
    if (prod4(s->B, s->H, s->L, s->dk > s->dv ? s->dk : s->dv) < 0) return LA_ERR_SHAPE;
    if (prod4(s->B, s->H, s->nseg, (int64_t)s->dk * s->dv) < 0) return LA_ERR_SHAPE;
    if (wide_ok && fwd_wide(s)) return LA_OK;
    if (!head_dim_ok(s->dk) || !head_dim_ok(s->dv)) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

la_status check_dtype(const la_shape* s) {
    if (s->in_dtype != LA_F32 && s->in_dtype != LA_BF16) return LA_ERR_DTYPE;
    if (s->out_dtype != s->in_dtype) return LA_ERR_DTYPE;
    return LA_OK;
}

la_status check_decay_mode(const la_shape* s) {
    if (s->decay_mode != LA_DECAY_NONE && s->decay_mode != LA_DECAY_HEAD && s->decay_mode != LA_DECAY_GATE)
        return LA_ERR_DECAY;
    if (s->decay_mode == LA_DECAY_GATE && !(s->gate_norm > 0.f && isfinite(s->gate_norm))) return LA_ERR_DECAY;
    return LA_OK;
}

// Bytes of the decay argument for this shape and mode.
size_t decay_bytes(const la_shape* s) {
    if (s->decay_mode == LA_DECAY_HEAD) return sizeof(float) * (size_t)s->H;
    if (s->decay_mode == LA_DECAY_GATE) return sizeof(float) * (size_t)(s->B * s->H * s->L * s->dk);
    return 0;
}

// Bytes of a per-tile flag array (one uint32 per 64-token tile of every segment).
size_t tile_flag_bytes(const la_shape* s) {
    return sizeof(uint32_t) * (size_t)(s->B * s->H * s->nseg * ((s->L / s->nseg + 63) / 64));
}

// A caller's per-(b,h) stride (0: dense) over blocks of `min` elements: at least `min`, and
// B*H strides within the element bound, so that no byte count derived from it overflows.
bool stride_ok(int64_t stride, int64_t min, const la_shape* s) {
    if (stride == 0) return true;
    return stride >= min && prod(s->B * s->H, stride) >= 0;
}

// Everything la_chunk_fwd checks that does not depend on the pointers.
la_status check_fwd_shape(const la_shape* s, int chunk) {
    la_status st = check_common(s, true);
    if (st != LA_OK) return st;
    if (chunk <= 0 || s->subseg_chunks < 0 || s->state_stride < 0) return LA_ERR_SHAPE;
    if (s->fwd_schedule < 0 || s->fwd_schedule > 2) return LA_ERR_SHAPE;
    if (!stride_ok(s->state_stride, (int64_t)s->nseg * s->dk * s->dv, s)) return LA_ERR_SHAPE;
    if (!fwd_chunk_ok(s, chunk)) return LA_ERR_UNSUPPORTED;
    if ((st = check_dtype(s)) != LA_OK) return st;
    return check_decay_mode(s);
}

la_status validate_fwd(const void* q, const void* k, const void* v, const float* decay, const float* s_in,
                       const void* o, const float* s_out, const la_shape* s, int chunk,
                       const void* q_dec = nullptr, const float* total = nullptr,
                       const uint32_t* tile_live = nullptr) {
    la_status st = check_fwd_shape(s, chunk);
    if (st != LA_OK) return st;
    if (s->decay_mode == LA_DECAY_NONE && decay) return LA_ERR_DECAY;
    const int64_t nqk = s->B * s->H * s->L * s->dk;
    const int64_t nv = s->B * s->H * s->L * s->dv;
    if (nqk > 0 && (!q || !k || !v || !o)) return LA_ERR_NULL;
    if (s->decay_mode == LA_DECAY_HEAD && s->H > 0 && !decay) return LA_ERR_NULL;
    if (s->decay_mode == LA_DECAY_GATE && nqk > 0 && !decay) return LA_ERR_NULL;
    const size_t es = esize(s->in_dtype);
    const int64_t BH = s->B * s->H;
    const int64_t per_seg = (int64_t)s->dk * s->dv;
    const int64_t so_stride = s->state_stride ? s->state_stride : s->nseg * per_seg;
    const size_t st_bytes = sizeof(float) * (size_t)(BH * per_seg);
    const size_t so_bytes = BH > 0 ? sizeof(float) * (size_t)((BH - 1) * so_stride + s->nseg * per_seg) : 0;
    Span sq{q, es * nqk}, sk{k, es * nqk}, sv{v, es * nv}, sd{decay, decay_bytes(s)}, si{s_in, s_in ? st_bytes : 0};
    Span so{o, es * nv}, sso{s_out, s_out ? so_bytes : 0};
    for (Span in : {sq, sk, sv, sd, si})
        if (overlap(so, in) || overlap(sso, in)) return LA_ERR_ALIAS;
    if (overlap(so, sso)) return LA_ERR_ALIAS;
    // the optional outputs of la_chunk_fwd_decayed
    if (total && (s->total_stride < 0 || !stride_ok(s->total_stride, (int64_t)s->nseg * s->dk, s)))
        return LA_ERR_SHAPE;
    const int64_t tstride = s->total_stride ? s->total_stride : (int64_t)s->nseg * s->dk;
    Span sqd{q_dec, q_dec ? es * nqk : 0};
    Span stt{total, (total && BH > 0) ? sizeof(float) * (size_t)((BH - 1) * tstride + (int64_t)s->nseg * s->dk) : 0};
    Span stl{tile_live, tile_live ? tile_flag_bytes(s) : 0};
    for (Span x : {sq, sk, sv, sd, si, so, sso})
        if (overlap(sqd, x) || overlap(stt, x) || overlap(stl, x)) return LA_ERR_ALIAS;
    if (overlap(sqd, stt) || overlap(stl, sqd) || overlap(stl, stt)) return LA_ERR_ALIAS;
    return LA_OK;
}

la_status from_hip(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH; }

la_status check_trace(const la_shape* s) {
    la_trace* t = s->trace;
    if (!t) return LA_OK;
    if (t->capacity < 0 || t->capacity > LA_TRACE_MAX_KERNELS) return LA_ERR_SHAPE;
    for (int i = 0; i < t->capacity; i++)
        if (!t->start[i] || !t->stop[i]) return LA_ERR_NULL;
    return LA_OK;
}

// A tracer bound to the call's stream; resets the trace's count.
la::Tracer make_tracer(const la_shape* s) {
    la::Tracer tr;
    tr.t = s->trace;
    tr.s = (hipStream_t)s->stream;
    if (tr.t) tr.t->count = 0;
    return tr;
}

}  // namespace

extern "C" {

int32_t la_version(void) { return (1 << 16) | 2; }

la_status la_trim_workspace(void) { return from_hip(la::workspace_trim()); }

const char* la_status_str(int32_t status) {
    switch (status) {
        case LA_OK: return "ok";
        case LA_ERR_NULL: return "a required pointer is NULL";
        case LA_ERR_SHAPE: return "invalid or inconsistent sizes";
        case LA_ERR_DTYPE: return "unsupported dtype combination";
        case LA_ERR_ALIAS: return "an output overlaps an input";
        case LA_ERR_UNSUPPORTED: return "no kernel for this head dim / chunk / layout";
        case LA_ERR_LAUNCH: return "HIP launch or workspace allocation failed";
        case LA_ERR_DECAY: return "invalid decay mode or gate_norm";
        case LA_ERR_WORKSPACE: return "the call needs more workspace than the allocation-free entry point holds";
        case LA_ERR_TIMEOUT: return "a chained forward's bounded wait gave up; its outputs hold NaN";
    }
    return "unknown status";
}

int32_t la_supported(const la_shape* s, int32_t chunk) { return check_fwd_shape(s, chunk) == LA_OK ? 1 : 0; }

la_status la_chain_status(int32_t clear, int64_t* give_ups) {
    unsigned int n = 0;
    if (la::chain_status(&n, clear != 0) != hipSuccess) return LA_ERR_LAUNCH;
    if (give_ups) *give_ups = n;
    return n ? LA_ERR_TIMEOUT : LA_OK;
}

int32_t la_set_chain_spin_limit(int32_t limit) {
    const int32_t prev = la::chain_spin_limit;
    if (limit >= 0) la::chain_spin_limit = limit;
    return prev;
}

}  // extern "C"

namespace {

// The forward of la_chunk_fwd, plus the optional outputs of la_chunk_fwd_decayed (q_dec, total);
// noalloc: the workspace of the matrix-core split comes from the library's fixed device array
// (la_chunk_fwd_noalloc), and a call that needs more than it holds is rejected.
la_status chunk_fwd_impl(const void* q, const void* k, const void* v, const float* decay, const float* s_in, void* o,
                         float* s_out, void* q_dec, float* total, uint32_t* tile_live, const la_shape* s,
                         int32_t chunk, bool noalloc = false) {
    la_status st = validate_fwd(q, k, v, decay, s_in, o, s_out, s, chunk, q_dec, total, tile_live);
    if (st != LA_OK) return st;
    if (fwd_wide(s) && (q_dec || total || tile_live)) return LA_ERR_UNSUPPORTED;  // la_chunk_fwd only
    if ((st = check_trace(s)) != LA_OK) return st;
    la::Tracer tr = make_tracer(s);
    hipStream_t stream = (hipStream_t)s->stream;
    const int64_t so_stride = s->state_stride ? s->state_stride : (int64_t)s->nseg * s->dk * s->dv;
    if (s->B * s->H == 0) return LA_OK;
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.decay = decay; a.s_in = s_in; a.o = o; a.s_out = s_out;
    a.s_out_stride = so_stride;
    a.B = s->B; a.H = s->H; a.L = s->L;
    a.dk = s->dk; a.dv = s->dv; a.nseg = s->nseg; a.chunk = chunk;
    a.bf16 = s->in_dtype == LA_BF16;
    a.mode = s->decay_mode;
    a.inv_norm = s->decay_mode == LA_DECAY_GATE ? 1.f / s->gate_norm : 1.f;
    a.subseg_chunks = s->subseg_chunks;
    a.schedule = s->fwd_schedule;
    a.stream = stream;
    a.tr = &tr;
    a.q_dec = q_dec;
    a.total = total;
    a.total_stride = s->total_stride ? s->total_stride : (int64_t)s->nseg * s->dk;
    a.tile_live = tile_live;
    // matrix cores: bf16 with dk = dv in {32, 64, 128} and 64-token chunks, or 128-token chunks
    // (bf16, dk = dv in {32, 64}, validated)
    const bool mfma = s->L > 0 && ((a.bf16 && a.dk == a.dv && (a.dk == 32 || a.dk == 64 || a.dk == 128) && chunk == 64) ||
                                   chunk == 128 || a.dk == 256);
    if (noalloc && mfma && la::fwd_noalloc_bytes(a) > LA_NOALLOC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;
    hipError_t e = hipSuccess;
    bool fused = false;  // the forward itself wrote q_dec and total
    if (s->L == 0) {
        if (s_out) e = la::launch_empty_states(s_in, s_out, so_stride, s->B * s->H, s->nseg, s->dk, s->dv, stream, &tr);
    } else if (mfma) {
        e = noalloc ? la::launch_chunk_fwd_mfma_noalloc(a) : la::launch_chunk_fwd_mfma(a);
        fused = a.mode == LA_DECAY_GATE;  // the gate kernels emit q_dec, totals and tile flags themselves
    } else {
        e = la::launch_chunk_fwd_generic(a);
    }
    if (e == hipSuccess && !fused && (q_dec || total || tile_live)) e = la::launch_decayed_q(a);
    return from_hip(e);
}

}  // namespace

extern "C" {

la_status la_chunk_fwd(const void* q, const void* k, const void* v, const float* decay, const float* s_in, void* o,
                       float* s_out, const la_shape* s, int32_t chunk) {
    return chunk_fwd_impl(q, k, v, decay, s_in, o, s_out, nullptr, nullptr, nullptr, s, chunk);
}

la_status la_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* decay, const float* s_in,
                               void* o, float* s_out, const la_shape* s, int32_t chunk) {
    return chunk_fwd_impl(q, k, v, decay, s_in, o, s_out, nullptr, nullptr, nullptr, s, chunk, true);
}

la_status la_chunk_fwd_decayed(const void* q, const void* k, const void* v, const float* decay, const float* s_in,
                               void* o, float* s_out, void* q_decayed, float* total, uint32_t* tile_live,
                               const la_shape* s, int32_t chunk) {
    return chunk_fwd_impl(q, k, v, decay, s_in, o, s_out, q_decayed, total, tile_live, s, chunk);
}

la_status la_state_scan(const float* seg_states, const float* seg_decay, int32_t P, float* out_states,
                        const la_shape* s) {
    if (!s) return LA_ERR_NULL;
    if (s->B < 0 || s->H < 0 || P < 1 || s->dk <= 0 || s->dv <= 0) return LA_ERR_SHAPE;
    const int64_t nst = prod4(s->B, s->H, P, (int64_t)s->dk * s->dv);
    if (nst < 0) return LA_ERR_SHAPE;
    if (s->dv % 4 != 0) return LA_ERR_UNSUPPORTED;
    if (nst > 0 && (!seg_states || !out_states)) return LA_ERR_NULL;  // seg_decay NULL: no decay
    if (((uintptr_t)seg_states | (uintptr_t)out_states) % 16 != 0) return LA_ERR_UNSUPPORTED;
    Span sx{seg_states, sizeof(float) * (size_t)nst}, sy{out_states, sizeof(float) * (size_t)nst};
    Span sl{seg_decay, sizeof(float) * (size_t)(s->B * s->H * P * s->dk)};
    if (seg_states != out_states && overlap(sx, sy)) return LA_ERR_ALIAS;
    if (seg_decay && overlap(sl, sy)) return LA_ERR_ALIAS;
    la_status st = check_trace(s);
    if (st != LA_OK) return st;
    la::Tracer tr = make_tracer(s);
    if (nst == 0) return LA_OK;
    return from_hip(la::launch_state_scan(seg_states, seg_decay, out_states, s->B * s->H, P, s->dk, s->dv,
                                          (hipStream_t)s->stream, &tr));
}

}  // extern "C"

namespace {

la_status state_correct_impl(const void* q, const float* cumdecay, const float* s_recv, void* o,
                             const uint32_t* tile_live, const la_shape* s) {
    la_status st = check_common(s);
    if (st != LA_OK) return st;
    if (s->seg_begin < 0 || s->seg_begin > s->nseg || s->state_stride < 0) return LA_ERR_SHAPE;
    if ((st = check_dtype(s)) != LA_OK) return st;
    if ((st = check_decay_mode(s)) != LA_OK) return st;
    if (s->decay_mode == LA_DECAY_NONE && cumdecay) return LA_ERR_DECAY;
    const int64_t np = s->nseg - s->seg_begin;
    const int64_t per_state = (int64_t)s->dk * s->dv;
    const int64_t stride = s->state_stride ? s->state_stride : np * per_state;
    if (!stride_ok(s->state_stride, np * per_state, s)) return LA_ERR_SHAPE;
    const int64_t BH = s->B * s->H;
    const int64_t Ls = s->L / s->nseg;
    const int64_t nq = BH * s->L * s->dk;
    const int64_t ncorr = BH * np * Ls;  // tokens to correct
    if (ncorr > 0 && (!q || !s_recv || !o)) return LA_ERR_NULL;
    if (ncorr > 0 && s->decay_mode != LA_DECAY_NONE && !cumdecay) return LA_ERR_NULL;
    const size_t es = esize(s->in_dtype);
    size_t cum_bytes = s->decay_mode == LA_DECAY_HEAD ? sizeof(float) * (size_t)s->H
                       : s->decay_mode == LA_DECAY_GATE ? sizeof(float) * (size_t)nq : 0;
    size_t recv_bytes = BH > 0 ? sizeof(float) * (size_t)((BH - 1) * stride + np * per_state) : 0;
    Span so{o, es * (size_t)(BH * s->L * s->dv)};
    if (overlap(so, Span{q, es * (size_t)nq}) || overlap(so, Span{cumdecay, cum_bytes}) ||
        overlap(so, Span{s_recv, recv_bytes}) || overlap(so, Span{tile_live, tile_live ? tile_flag_bytes(s) : 0}))
        return LA_ERR_ALIAS;
    if ((st = check_trace(s)) != LA_OK) return st;
    la::Tracer tr = make_tracer(s);
    if (ncorr == 0) return LA_OK;
    CorrectArgs a;
    a.q = q; a.cum = cumdecay; a.s_recv = s_recv; a.o = o;
    a.B = s->B; a.H = s->H; a.L = s->L;
    a.dk = s->dk; a.dv = s->dv; a.nseg = s->nseg; a.seg_begin = s->seg_begin;
    a.state_stride = stride;
    a.bf16 = s->in_dtype == LA_BF16;
    a.mode = s->decay_mode;
    a.stream = (hipStream_t)s->stream;
    a.tr = &tr;
    a.tile_live = tile_live;
    return from_hip(la::launch_state_correct(a));
}

}  // namespace

extern "C" {

la_status la_state_correct(const void* q, const float* cumdecay, const float* s_recv, void* o, const la_shape* s) {
    return state_correct_impl(q, cumdecay, s_recv, o, nullptr, s);
}

la_status la_state_correct_live(const void* q, const float* cumdecay, const float* s_recv, void* o,
                                const uint32_t* tile_live, const la_shape* s) {
    return state_correct_impl(q, cumdecay, s_recv, o, tile_live, s);
}

la_status la_cumdecay(const float* decay, float* cumdecay, float* total, const la_shape* s) {
    la_status st = check_common(s);
    if (st != LA_OK) return st;
    if ((st = check_decay_mode(s)) != LA_OK) return st;
    if (s->decay_mode == LA_DECAY_NONE && decay) return LA_ERR_DECAY;
    const int64_t BH = s->B * s->H;
    const int64_t ncum = BH * s->L * s->dk;
    const int64_t ntot = BH * s->nseg * s->dk;
    if (s->total_stride < 0 || !stride_ok(s->total_stride, (int64_t)s->nseg * s->dk, s)) return LA_ERR_SHAPE;
    const int64_t tstride = s->total_stride ? s->total_stride : (int64_t)s->nseg * s->dk;
    const bool need = (cumdecay && ncum > 0) || (total && ntot > 0);
    if (need && s->decay_mode == LA_DECAY_HEAD && !decay) return LA_ERR_NULL;
    if (need && s->decay_mode == LA_DECAY_GATE && ncum > 0 && !decay) return LA_ERR_NULL;
    Span sd{decay, decay_bytes(s)}, sc{cumdecay, cumdecay ? sizeof(float) * (size_t)ncum : 0};
    Span stt{total, (total && BH > 0) ? sizeof(float) * (size_t)((BH - 1) * tstride + (int64_t)s->nseg * s->dk) : 0};
    if (overlap(sc, sd) || overlap(stt, sd) || overlap(sc, stt)) return LA_ERR_ALIAS;
    if ((st = check_trace(s)) != LA_OK) return st;
    la::Tracer tr = make_tracer(s);
    if (!need) return LA_OK;
    const float inv_norm = s->decay_mode == LA_DECAY_GATE ? 1.f / s->gate_norm : 1.f;
    return from_hip(la::launch_cumdecay(decay, cumdecay, total, tstride, s->B, s->H, s->L, s->dk, s->nseg,
                                        s->decay_mode, inv_norm, (hipStream_t)s->stream, &tr));
}

}  // extern "C"

namespace {

la_status chunk_bwd_impl(const void* q, const void* k, const void* v, const float* decay, const float* s_in,
                         const float* s_sub, int32_t sub_len, int64_t sub_stride, const void* d_o,
                         const float* ds_out, void* dq, void* dk, void* dv, float* d_decay, float* ds_in,
                         const la_shape* s, int32_t chunk) {
    la_status st = check_common(s);
    if (st != LA_OK) return st;
    if (chunk <= 0 || s->state_stride < 0 || s->subseg_chunks < 0) return LA_ERR_SHAPE;
    const int64_t per_seg = (int64_t)s->dk * s->dv;
    if (!stride_ok(s->state_stride, (int64_t)s->nseg * per_seg, s)) return LA_ERR_SHAPE;
    if (!chunk_ok(chunk)) return LA_ERR_UNSUPPORTED;
    if ((st = check_dtype(s)) != LA_OK) return st;
    if ((st = check_decay_mode(s)) != LA_OK) return st;
    if (s->decay_mode == LA_DECAY_NONE && (decay || d_decay)) return LA_ERR_DECAY;
    const int64_t BH = s->B * s->H;
    const int64_t nqk = BH * s->L * s->dk;
    const int64_t nv = BH * s->L * s->dv;
    if (nqk > 0 && (!q || !k || !v || !d_o || !dq || !dk || !dv)) return LA_ERR_NULL;
    if (s->decay_mode == LA_DECAY_HEAD && s->H > 0 && !decay) return LA_ERR_NULL;
    if (s->decay_mode == LA_DECAY_GATE && nqk > 0 && !decay) return LA_ERR_NULL;
    const size_t es = esize(s->in_dtype);
    const int64_t sstride = s->state_stride ? s->state_stride : (int64_t)s->nseg * per_seg;
    const size_t st_bytes = BH > 0 ? sizeof(float) * (size_t)((BH - 1) * sstride + s->nseg * per_seg) : 0;
    // states entering the sub-segments: sub_len a positive multiple of the chunk (64 on the
    // matrix-core path that uses them), (b,h) blocks of sub_stride floats (0 = dense)
    const int64_t Lseg = s->nseg > 0 ? s->L / s->nseg : 0;
    const int64_t nsub = s_sub && sub_len > 0 ? (Lseg + sub_len - 1) / sub_len : 0;
    if (s_sub && (sub_len <= 0 || sub_len % chunk != 0 || sub_stride < 0)) return LA_ERR_SHAPE;
    if (s_sub && !stride_ok(sub_stride, (int64_t)s->nseg * nsub * per_seg, s)) return LA_ERR_SHAPE;
    const int64_t substride = s_sub ? (sub_stride ? sub_stride : (int64_t)s->nseg * nsub * per_seg) : 0;
    const size_t sub_bytes =
        s_sub && BH > 0 ? sizeof(float) * (size_t)((BH - 1) * substride + s->nseg * nsub * per_seg) : 0;
    const Span ins[] = {{q, es * nqk},
                        {k, es * nqk},
                        {v, es * nv},
                        {decay, decay ? decay_bytes(s) : 0},
                        {s_in, s_in ? sizeof(float) * (size_t)(BH * per_seg) : 0},
                        {s_sub, sub_bytes},
                        {d_o, es * nv},
                        {ds_out, ds_out ? st_bytes : 0}};
    const Span outs[] = {{dq, es * nqk},
                         {dk, es * nqk},
                         {dv, es * nv},
                         {d_decay, d_decay ? decay_bytes(s) : 0},
                         {ds_in, ds_in ? st_bytes : 0}};
    for (const Span& o : outs) {
        for (const Span& i : ins)
            if (overlap(o, i)) return LA_ERR_ALIAS;
        for (const Span& p : outs)
            if (&p != &o && overlap(o, p)) return LA_ERR_ALIAS;
    }
    if ((st = check_trace(s)) != LA_OK) return st;
    la::Tracer tr = make_tracer(s);
    const bool head_grad = s->decay_mode == LA_DECAY_HEAD && d_decay && s->H > 0;
    if (BH * s->nseg == 0 && !head_grad) return LA_OK;
    la::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.decay = decay; a.s_in = s_in; a.d_o = d_o; a.ds_out = ds_out;
    a.dq = dq; a.dk_out = dk; a.dv_out = dv; a.d_decay = d_decay; a.ds_in = ds_in;
    a.state_stride = sstride;
    a.B = s->B; a.H = s->H; a.L = s->L;
    a.dk = s->dk; a.dv = s->dv; a.nseg = s->nseg; a.chunk = chunk;
    a.bf16 = s->in_dtype == LA_BF16;
    a.mode = s->decay_mode;
    a.inv_norm = s->decay_mode == LA_DECAY_GATE ? 1.f / s->gate_norm : 1.f;
    a.subseg_chunks = s->subseg_chunks;
    // the given sub-segment states serve the matrix-core path with 64-token chunks; elsewhere the
    // backward does not split segments and they are not needed
    const bool use_sub = s_sub && chunk == 64 && sub_len % 64 == 0 && nsub > 1;
    a.s_sub = use_sub ? s_sub : nullptr;
    a.sub_stride = substride;
    a.sub_len = sub_len;
    a.stream = (hipStream_t)s->stream;
    a.tr = &tr;
    return from_hip(la::chunk_bwd_mfma_supported(a) ? la::launch_chunk_bwd_mfma(a) : la::launch_chunk_bwd_generic(a));
}

}  // namespace

extern "C" {

la_status la_chunk_bwd(const void* q, const void* k, const void* v, const float* decay, const float* s_in,
                       const void* d_o, const float* ds_out, void* dq, void* dk, void* dv, float* d_decay,
                       float* ds_in, const la_shape* s, int32_t chunk) {
    return chunk_bwd_impl(q, k, v, decay, s_in, nullptr, 0, 0, d_o, ds_out, dq, dk, dv, d_decay, ds_in, s, chunk);
}

la_status la_chunk_bwd_states(const void* q, const void* k, const void* v, const float* decay, const float* s_in,
                              const float* s_sub, int32_t sub_len, int64_t sub_stride, const void* d_o,
                              const float* ds_out, void* dq, void* dk, void* dv, float* d_decay, float* ds_in,
                              const la_shape* s, int32_t chunk) {
    if (!s_sub) return LA_ERR_NULL;
    return chunk_bwd_impl(q, k, v, decay, s_in, s_sub, sub_len, sub_stride, d_o, ds_out, dq, dk, dv, d_decay, ds_in,
                          s, chunk);
}

}  // extern "C"
