/*
 * la_chunk.h -- C ABI of liblachunk.so: chunked causal linear attention with a segmented state
 * scan, hand-written for AMD MI355X (gfx950).
 *
 * What is computed.  Per (batch b, head h) sequence of L tokens with queries q_t, keys k_t in
 * R^dk, values v_t in R^dv and per-token decay a_t in (0,1]^dk, the linear-attention state
 * recurrence
 *        S_t = diag(a_t) S_{t-1} + k_t v_t^T,     o_t = S_t^T q_t,          S in R^{dk x dv}
 * (review page "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear Attention":
 * linear attention as a fixed-size state recurrence, pith_extraction.supporting_citations[0];
 * the gated, GLA-style chunkwise form, supporting_citations[1]; S is the only object that
 * crosses a device boundary, pith_extraction.core_discovery).  The library evaluates it chunk
 * by chunk, and splits it over sequence segments with the linear-decomposition identity of the
 * same page (pith_extraction.key_machinery): the state at the end of a segment is the segment's
 * cumulative decay applied to the incoming state plus the segment's locally computed state, and
 * the outputs take the matching rank-dk correction.
 *
 * Memory.  Every pointer is a device pointer (HBM) owned by the caller; the library never
 * frees or keeps one past the call.  Tensors are dense, row-major, in the layouts stated per
 * argument.  Temporary device workspace comes from a stream-ordered memory pool the library keeps
 * per device.  The matrix-core forward and backward (la_chunk_fwd, la_chunk_fwd_decayed,
 * la_chunk_bwd, la_chunk_bwd_states: per sub-segment states when a segment is split across
 * compute units, in gate mode a few flags per workgroup, the decay derivative's partials) keep
 * theirs between calls: one buffer per device, stream and call, taken from the pool on the
 * stream's first call and replaced by a larger one when a call needs more, so repeated calls on a
 * stream allocate nothing; calls on different streams use different buffers.  On a stream under
 * graph capture they take it per call and free it (stream-ordered) before returning, so a graph
 * holds no kept buffer.  Per call, freed the same way: la_cumdecay in gate mode and
 * la_chunk_fwd_decayed on the shapes whose forward does not emit its outputs (one float per 64
 * tokens and key dim in gate mode), and the fp32 backward's decay-derivative partials.  The pool
 * keeps the memory it has obtained (so repeated calls never reach the driver); la_trim_workspace
 * releases the kept buffers and that memory.  la_chunk_fwd_noalloc, la_state_scan,
 * la_state_correct and la_state_correct_live allocate nothing.
 *
 * Execution.  Calls validate every argument on the host first, then enqueue kernels on
 * shape->stream (a hipStream_t; NULL = the default stream) and return without waiting.  A
 * fault inside a kernel is reported by the caller's next synchronisation, not by the call.
 * Calls touching the same buffers must be ordered by the caller (same stream or events).
 * Apart from the workspace pools (and the fixed array of la_chunk_fwd_noalloc) the library holds
 * no mutable global state; concurrent calls from several host threads are safe.
 *
 * Errors.  A call returns LA_OK or a negative la_status and, on error, enqueues nothing.
 */
#ifndef LA_CHUNK_H
#define LA_CHUNK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
    LA_OK = 0,
    LA_ERR_NULL = -1,        /* a required pointer is NULL (or shape is NULL) */
    LA_ERR_SHAPE = -2,       /* a size is negative / zero where it must not be, or does not divide */
    LA_ERR_DTYPE = -3,       /* unknown dtype, or a dtype combination that is not supported */
    LA_ERR_ALIAS = -4,       /* an output overlaps an input it may not overlap */
    LA_ERR_UNSUPPORTED = -5, /* valid request that the library has no kernel for (e.g. dk > 128) */
    LA_ERR_LAUNCH = -6,      /* the HIP runtime refused a launch or a workspace allocation */
    LA_ERR_DECAY = -7,       /* unknown decay mode, or gate_norm <= 0 in gate mode */
    LA_ERR_WORKSPACE = -8,   /* la_chunk_fwd_noalloc: the call needs more than LA_NOALLOC_SCRATCH_BYTES */
    LA_ERR_TIMEOUT = -9      /* la_chain_status: a chained forward's bounded wait gave up */
} la_status;

typedef enum la_dtype { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* How the per-token decay a_t in R^dk is given (argument `decay`):
 *   LA_DECAY_NONE : a_t = 1; decay must be NULL.
 *   LA_DECAY_HEAD : one log-decay per head, decay = float[H] holding lambda_h <= 0, a_t = exp(lambda_h)
 *                   for every token and key dimension (per-head scalar decay, RetNet/Lightning style).
 *   LA_DECAY_GATE : per token and key dimension, decay = float[B,H,L,dk] holding the raw gate g,
 *                   a_t[d] = sigmoid(g_t[d])^(1/gate_norm) (GLA style).  Evaluated in log space:
 *                   log a = -softplus(-g) / gate_norm, summed within each chunk. */
typedef enum la_decay_mode { LA_DECAY_NONE = 0, LA_DECAY_HEAD = 1, LA_DECAY_GATE = 2 } la_decay_mode;

/* Optional per-kernel timing.  Each call that is handed an la_trace sets count = 0, then for
 * every kernel it enqueues (up to capacity) records start[i] just before and stop[i] just after
 * the launch on the call's stream and stores a static kernel name in name[i].  The events are
 * caller-created hipEvent_t handles; the caller reads them after synchronising. */
#define LA_TRACE_MAX_KERNELS 16
typedef struct la_trace {
    void* start[LA_TRACE_MAX_KERNELS];
    void* stop[LA_TRACE_MAX_KERNELS];
    int32_t capacity;                       /* usable entries, 0..LA_TRACE_MAX_KERNELS */
    int32_t count;                          /* out: kernels bracketed by the last call */
    const char* name[LA_TRACE_MAX_KERNELS]; /* out */
} la_trace;

typedef struct la_shape {
    int64_t B;            /* batch size, >= 0 */
    int64_t H;            /* heads, >= 0 */
    int64_t L;            /* tokens per (b,h) sequence, >= 0; L % nseg == 0 */
    int32_t dk;           /* key/query head dim: 16, 32, 64 or 128 (la_chunk_fwd also 256) */
    int32_t dv;           /* value head dim: 16, 32, 64 or 128 (la_chunk_fwd also 256) */
    int32_t nseg;         /* independent segments per sequence, >= 1, each L/nseg tokens */
    int32_t in_dtype;     /* la_dtype of q, k, v */
    int32_t out_dtype;    /* la_dtype of o (must equal in_dtype in this version) */
    int32_t decay_mode;   /* la_decay_mode */
    float gate_norm;      /* LA_DECAY_GATE only: exponent 1/gate_norm on the sigmoid, > 0 */
    int32_t seg_begin;    /* la_state_correct only: first segment to correct, 0 <= seg_begin <= nseg */
    int64_t state_stride; /* elements between consecutive (b,h) blocks of a per-segment state
                             array: s_out of la_chunk_fwd (0 = dense, nseg*dk*dv) and s_recv of
                             la_state_correct (0 = dense, (nseg - seg_begin)*dk*dv).  Lets the
                             local state land directly in a slot of a larger scan buffer. */
    int64_t total_stride; /* la_cumdecay and la_chunk_fwd_decayed: elements between consecutive
                             (b,h) blocks of total; 0 = dense, nseg*dk */
    int32_t subseg_chunks;/* la_chunk_fwd and la_chunk_bwd (matrix-core kernels): chunks per internal
                             sub-segment when one segment is split across compute units (the
                             decomposition identity applied inside the GPU); 0 = choose
                             automatically, >= 1 forces that length.  Changes the rounding order
                             only, never the mathematical result. */
    int32_t fwd_schedule; /* la_chunk_fwd / la_chunk_fwd_noalloc, matrix-core kernels, when a
                             segment is split into sub-segments: 0 = the library's choice (on this
                             build: 1), 1 = separate passes (local states, a scan over them, then
                             the outputs from the exact incoming states), 2 = one launch whose
                             workgroups hand the sub-segment states on through flags (bf16,
                             dk = dv = 128, chunk 64, no or per-head decay, and only when every
                             workgroup fits on the device at once; otherwise 1).  Changes the
                             rounding order only. */
    void* stream;         /* hipStream_t the work is enqueued on; NULL = default stream */
    la_trace* trace;      /* optional per-kernel event recording (NULL = off); see la_trace */
} la_shape;
/* A zero-initialised la_shape plus B, H, L, dk, dv, nseg = 1 and the dtypes is a valid
 * description for every call; the other fields only matter to the calls that name them. */

/*
 * Chunkwise forward of the recurrence over every segment of every (b,h) sequence.
 *
 * Per chunk of `chunk` tokens it computes the intra-chunk "diagonal" term -- the causal
 * (j <= i, diagonal included), decay-weighted Q K^T of the chunk times V -- plus the inter-chunk
 * term Q-bar S_{c-1}, and carries the state S_c = diag(Lambda_c) S_{c-1} + K-tilde^T V across
 * chunks, where Lambda_c is the chunk's cumulative decay and K-tilde scales each key by the decay
 * from its token to the chunk end (page "ZeCO ...": the diagonal P computation,
 * skeptic_critique.concrete_test and pith_extraction.core_discovery; the decay vectors Lambda,
 * Gamma and K-bar of referee_report.minor_comments[3]).  The result equals the token-by-token
 * recurrence up to floating-point rounding.
 *
 *   q, k   : [B,H,L,dk] in_dtype        v : [B,H,L,dv] in_dtype        (read only)
 *   decay  : see la_decay_mode                                          (read only)
 *   s_in   : float[B,H,dk,dv] initial state of segment 0 of each sequence, or NULL for zero.
 *            Segments 1..nseg-1 always start from zero (each is a device's local share).
 *   o      : [B,H,L,dv] out_dtype, written (every element); must not overlap q, k, v, decay, s_in.
 *   s_out  : float, final local state of every segment, or NULL to skip it: segment p of (b,h)
 *            at s_out + (b*H + h) * state_stride + p * dk * dv (dense [B,H,nseg,dk,dv] when
 *            state_stride = 0); must not overlap any other argument.
 *   chunk  : chunk length in tokens: 16, 32 or 64 (64 is the production size), or 128 for bf16
 *            with dk = dv in {32, 64}, and with dk = dv = 128 without gate decay (the chunk-length
 *            variants, on the matrix-core kernels).
 * Head dims: dk, dv in {16, 32, 64, 128}, and dk = dv = 256 for bf16 with 64-token chunks and no
 * or per-head decay (the state-size variant: the value dims are tiled across workgroups; only
 * la_chunk_fwd, la_chunk_fwd_noalloc and la_state_scan take it).
 * A partial last chunk (L/nseg not a multiple of chunk) is allowed.  Gate mode takes any gate
 * value, g = -inf (a = 0) included: each token's log-decay is floored at -33 (a >= e^-33, which
 * moves every token-pair weight by at most e^-33), and a chunk whose decay is too wide for the
 * matrix-core kernels' factorised pair weights (beyond 2^-96 on some key dim) is taken in shorter
 * windows (down to two tokens) by a windowed variant of the same kernels.
 * Returns LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_DECAY, LA_ERR_ALIAS,
 * LA_ERR_UNSUPPORTED or LA_ERR_LAUNCH.
 */
la_status la_chunk_fwd(const void* q, const void* k, const void* v, const float* decay,
                       const float* s_in, void* o, float* s_out, const la_shape* shape,
                       int32_t chunk);

/*
 * la_chunk_fwd for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments, results and rounding as
 * la_chunk_fwd (the same kernels with the same split into sub-segments); the only difference is
 * where the workspace of that split lives.  It is a fixed device array of
 * LA_NOALLOC_SCRATCH_BYTES in the library, one per device the library runs on, held from its first
 * use until the process ends; the call itself allocates nothing (no hipMalloc, no pool).  Every
 * call on a device shares that device's array, so calls that may overlap in time on one device
 * (other streams, other host threads) race on it and must be ordered by the caller.  Nothing in it
 * needs to be cleared between calls.  The automatic split (subseg_chunks = 0) always fits; a call
 * whose caller-chosen subseg_chunks would need more workspace returns LA_ERR_WORKSPACE and
 * enqueues nothing.
 * Returns the codes of la_chunk_fwd, or LA_ERR_WORKSPACE.
 */
#define LA_NOALLOC_SCRATCH_BYTES ((uint64_t)32 << 20)
la_status la_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* decay,
                               const float* s_in, void* o, float* s_out, const la_shape* shape,
                               int32_t chunk);

/*
 * la_chunk_fwd plus the two decay quantities that the rest of a device's step needs, emitted by
 * the same pass, so that no separate cumulative-decay pass is needed.  In the decomposition
 * identity of the ZeCO review page (pith_extraction.key_machinery) the incoming state reaches
 * the outputs through q_t scaled by the decay accumulated since the segment start, and reaches
 * the outgoing state through the segment's total decay:
 *   q_decayed[b,h,t,:] = q_t (*) cum_t, cum_t[d] = prod of a_s[d] from the first token of t's
 *                        segment to t inclusive; [B,H,L,dk] in_dtype, rounded once from fp32;
 *                        or NULL.  Then la_state_correct(q_decayed, NULL, ...) with decay_mode
 *                        NONE adds exactly the correction la_state_correct(q, cumdecay, ...)
 *                        adds in the shape's own mode.
 *   total              = Lambda of every segment, as la_cumdecay writes it (segment p of (b,h)
 *                        at total + (b*H + h) * total_stride + p * dk; dense [B,H,nseg,dk] when
 *                        shape->total_stride = 0); or NULL.
 *   tile_live          = uint32[B,H,nseg,ceil(L/nseg/64)] or NULL: entry i of segment p covers the
 *                        segment's tokens 64i .. 64i+63.  Zero promises that q_t (*) cum_t is exactly
 *                        zero on every one of them (the cumulative decay has underflowed for every
 *                        key dim); nonzero promises nothing.  For la_state_correct_live.  When
 *                        tile_live is given, q_decayed may be left unwritten on the tiles whose
 *                        entry is zero (the values there would be zero, and la_state_correct_live
 *                        does not read them); without tile_live every q_decayed row is written.
 * Every other argument, and every result la_chunk_fwd writes, is as for la_chunk_fwd.  In gate
 * mode with bf16, dk = dv = 128 and chunk 64 all three come out of the forward's own decay
 * preparation (cum = exp2 of an fp32 running sum of log2 a); otherwise one extra streaming pass
 * forms them (gate: exp of an fp32 running sum of log a; head: exp(lambda_h * tau); none: cum = 1,
 * q_decayed = q; every tile_live entry nonzero).  No output may overlap any other argument.
 * Returns LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_DECAY, LA_ERR_ALIAS,
 * LA_ERR_UNSUPPORTED or LA_ERR_LAUNCH.
 */
la_status la_chunk_fwd_decayed(const void* q, const void* k, const void* v, const float* decay,
                               const float* s_in, void* o, float* s_out, void* q_decayed,
                               float* total, uint32_t* tile_live, const la_shape* shape,
                               int32_t chunk);

/*
 * Backward pass of la_chunk_fwd: the derivatives of a loss with respect to q, k, v, the decay
 * parameter and each segment's initial state, given its derivatives with respect to o and to each
 * segment's final state (the backward pass that the ZeCO review page lists as a consequence of the
 * forward design, pith_extraction.forward_implications; it runs the chunk recurrence in reverse for
 * the state derivative next to a forward recomputation of the states).  With G_t the derivative
 * with respect to S_t, walked from the segment's end (G = ds_out there):
 *     dq_t = S_t d_o_t,   dk_t = G_t v_t,   dv_t = G_t^T k_t,   ds_in = diag(a_first) G_first,
 * and for the decay parameter the chain rule through every a_t it sets.  Segments are independent
 * sequences exactly as in la_chunk_fwd (segment 0 from s_in, the others from zero).
 *
 *   q, k, v, decay, s_in : as passed to la_chunk_fwd (read only; the states are recomputed).
 *   d_o    : [B,H,L,dv] in_dtype, derivative with respect to o (read only).
 *   ds_out : float, derivative with respect to each segment's final state, in the s_out layout of
 *            la_chunk_fwd (state_stride), or NULL for zero.
 *   dq, dk : [B,H,L,dk] in_dtype, written.        dv : [B,H,L,dv] in_dtype, written.
 *   d_decay: NONE: must be NULL.  HEAD: float[H], the derivative with respect to lambda_h summed
 *            over batch, segments, tokens and key dims.  GATE: float[B,H,L,dk], the derivative with
 *            respect to the raw gate g.  NULL skips it (and its workspace).
 *   ds_in  : float, derivative with respect to each segment's initial state (segment 0's is s_in;
 *            the others' is what a backward state scan carries between segments), in the
 *            state_stride layout, or NULL.
 *   chunk  : 16, 32 or 64.
 * No output may overlap an input or another output.  bf16 inputs with dk = dv in {32, 64, 128}
 * and chunk 64 run on the matrix cores (bf16 operands, fp32 accumulation) in every decay mode: the
 * head-decay derivative is summed token pair by token pair (fp64 partial sums), the gate derivative
 * per chunk from rowsum(S (.) D) at the chunk's start plus an in-chunk running sum of
 * k (.) dk - q (.) dq; gate mode takes any gate value as in la_chunk_fwd (the same floor on log a,
 * the same windows for chunks too wide for one factorisation).  Every other shape and fp32 inputs
 * run in fp32 arithmetic.  bf16 outputs are rounded once, to nearest even.  May allocate temporary device
 * workspace from the same stream-ordered pool as la_chunk_fwd (per sub-segment states; for the gate
 * derivative a bf16 d_k x d_v matrix and d_k floats per chunk on the matrix cores, a float per token
 * and key dim on the fp32 path).
 * Returns LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_DECAY, LA_ERR_ALIAS,
 * LA_ERR_UNSUPPORTED or LA_ERR_LAUNCH.
 */
la_status la_chunk_bwd(const void* q, const void* k, const void* v, const float* decay,
                       const float* s_in, const void* d_o, const float* ds_out, void* dq, void* dk,
                       void* dv, float* d_decay, float* ds_in, const la_shape* shape, int32_t chunk);

/*
 * la_chunk_bwd, reusing states the forward already has: the state entering every sub-segment of
 * sub_len tokens of every segment (the ZeCO review page notes that the backward reuses the global
 * states of the forward instead of exchanging or recomputing them,
 * pith_extraction.forward_implications; within one device the same holds for the states that the
 * device step's scan leaves at its sub-segment boundaries).  On the matrix-core path the backward
 * then splits every segment at those sub-segments and runs no forward state pass and no scan for
 * dq; the results are those of la_chunk_bwd up to rounding order.
 *
 *   s_sub      : float, read only: for (b,h) block b*H + h at s_sub + (b*H + h) * sub_stride,
 *                segment p's sub-segment j (tokens p*Lseg + j*sub_len ..) at
 *                (p * ceil(Lseg / sub_len) + j) * dk * dv, a [dk][dv] state.  Entry j = 0 of every
 *                segment is not read (segment 0 starts from s_in, the others from zero).  Must not
 *                overlap an output.  Not NULL.
 *   sub_len    : tokens per sub-segment, a positive multiple of chunk (64 on the matrix-core path;
 *                with other shapes the states are validated but not needed).
 *   sub_stride : floats between consecutive (b,h) blocks of s_sub, 0 = dense
 *                (nseg * ceil(Lseg / sub_len) * dk * dv); lets the device step's scan buffer, which
 *                holds one more state per (b,h), be passed as is.
 * Every other argument, the results and the return codes are those of la_chunk_bwd; a bad sub_len
 * or sub_stride returns LA_ERR_SHAPE.
 */
la_status la_chunk_bwd_states(const void* q, const void* k, const void* v, const float* decay,
                              const float* s_in, const float* s_sub, int32_t sub_len,
                              int64_t sub_stride, const void* d_o, const float* ds_out, void* dq,
                              void* dk, void* dv, float* d_decay, float* ds_in,
                              const la_shape* shape, int32_t chunk);

/*
 * Segmented state scan: the All-Scan of ZeCO reproduced on one GPU (page "ZeCO ...",
 * pith_extraction.key_machinery: each device applies the update
 * S_p = (segment decay) * S_{p-1} + S_local,p to the state it receives and passes the result on;
 * the accumulated state is what moves on, referee_report.major_comments[3]).  For each (b,h):
 *        out[p] = diag(seg_decay[p]) out[p-1] + seg_states[p],   p = 0..P-1,   out[-1] = 0,
 * i.e. an inclusive scan; out[p] is the state at the end of segment p, the incoming state of
 * segment p+1.  Accumulates in fp32 in order of p.
 *
 *   seg_states : float[B,H,P,dk,dv]   seg_decay : float[B,H,P,dk] multiplicative per-segment
 *                total decay (a vector over key dims; broadcast a scalar yourself); the entry of
 *                segment 0 only ever multiplies the zero state and is not applied.  NULL means
 *                no decay (every entry 1), the plain running sum.
 *   out_states : float[B,H,P,dk,dv]; may be the same pointer as seg_states (in place), must not
 *                otherwise overlap it, nor seg_decay.
 * Uses shape->B, H, dk, dv, stream; P is the argument (not shape->nseg).
 * Returns LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_ALIAS, LA_ERR_UNSUPPORTED or LA_ERR_LAUNCH.
 */
la_status la_state_scan(const float* seg_states, const float* seg_decay, int32_t P,
                        float* out_states, const la_shape* shape);

/*
 * Output correction with an incoming state: the rank-dk term of the decomposition identity
 * (page "ZeCO ...", pith_extraction.key_machinery).  For every segment p >= shape->seg_begin and
 * every token t of it:
 *        o_t += (q_t (*) cum_t)^T s_recv[b,h,p - seg_begin]
 * where cum_t[d] is the product of a_s[d] from the segment's first token to t inclusive.
 *
 *   q        : [B,H,L,dk] in_dtype (read only)
 *   cumdecay : by decay_mode -- NONE: NULL (cum = 1);  HEAD: float[H] log-decays lambda_h, the
 *              cumulative decay exp(lambda_h * (t - segment start + 1)) is formed in the kernel;
 *              GATE: float[B,H,L,dk] cumulative decay values as written by la_cumdecay.
 *   s_recv   : float, incoming state of segment p of (b,h) at
 *              s_recv + (b*H + h) * state_stride + (p - seg_begin) * dk * dv, each dk x dv row-major.
 *   o        : [B,H,L,dv] out_dtype, updated in place (o = round(o + correction) in fp32);
 *              must not overlap q, cumdecay, s_recv.
 * Tokens whose cumulative decay is exactly zero in fp32 receive an exactly-zero correction.
 * Returns LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_DECAY, LA_ERR_ALIAS,
 * LA_ERR_UNSUPPORTED or LA_ERR_LAUNCH.
 */
la_status la_state_correct(const void* q, const float* cumdecay, const float* s_recv, void* o,
                           const la_shape* shape);

/*
 * la_state_correct that may skip the 64-token tiles (of the segments it corrects) whose tile_live
 * entry is zero: there q_t (*) cum_t is exactly zero, so the correction is exactly zero and O is
 * bit-identical either way (the decomposition identity's correction term, page "ZeCO ...",
 * pith_extraction.key_machinery, vanishes where the cumulative decay has underflowed).
 *   tile_live : uint32[B,H,nseg,ceil(L/nseg/64)] as la_chunk_fwd_decayed writes it for the same
 *               B, H, L, nseg (all segments, including those before seg_begin), or NULL (no tile
 *               skipped: exactly la_state_correct).  Read only; must not overlap o.
 * Every other argument as for la_state_correct.  A zero entry over rows whose q (*) cum is not
 * zero is a caller error: those rows then miss their correction.
 * Returns as la_state_correct.
 */
la_status la_state_correct_live(const void* q, const float* cumdecay, const float* s_recv, void* o,
                                const uint32_t* tile_live, const la_shape* shape);

/*
 * Cumulative decay helper (not one of the three core calls; it prepares their decay inputs).
 * For every segment p of every (b,h):
 *   cumdecay[b,h,t,d] = prod_{s = first token of p .. t} a_s[d]          (inclusive)
 *   total[b,h,p,d]    = prod over all tokens of segment p of a_s[d]      (= Lambda of segment p)
 * Either output may be NULL.  In HEAD mode the values are the closed forms exp(lambda_h * n);
 * in GATE mode they are exp of an fp32 running sum of log a within the segment; in NONE mode 1.
 *   decay    : as for la_chunk_fwd
 *   cumdecay : float[B,H,L,dk] or NULL
 *   total    : float or NULL; segment p of (b,h) at total + (b*H + h) * total_stride + p * dk
 *              (dense [B,H,nseg,dk] when total_stride = 0)
 * Returns LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DECAY, LA_ERR_ALIAS or LA_ERR_LAUNCH.
 */
la_status la_cumdecay(const float* decay, float* cumdecay, float* total, const la_shape* shape);

/* Releases the current device's workspace: when the device holds buffers kept between calls, it
 * waits for the device to be idle and frees them; then it returns the pool's memory that no
 * enqueued call still uses to the device (later calls obtain it again).  Not to be called while
 * another thread enqueues work on the device or during graph capture.
 * Returns LA_OK or LA_ERR_LAUNCH. */
la_status la_trim_workspace(void);

/* Give-up counter of the chained forward (fwd_schedule = 2).  Its workgroups wait for each other's
 * flags; every wait is bounded, and a compute wave that polls a flag la_set_chain_spin_limit's
 * number of times without seeing it set stops waiting, computes on a NaN state (so its outputs are
 * NaN rather than the GPU hanging) and adds one to a per-device counter.  This call synchronises
 * the current device (do not call it while a stream of that device is being captured), stores the
 * counter in *give_ups (if not NULL) and, when clear != 0, resets it to zero.  A chained launch
 * whose workgroups are all resident (the library only chains grids that fit the device) does not
 * give up at the default limit.
 * Returns LA_OK if the counter was zero, LA_ERR_TIMEOUT if not, LA_ERR_LAUNCH if the runtime failed. */
la_status la_chain_status(int32_t clear, int64_t* give_ups);

/* Polls per flag before a chained wave gives up (default 4194304, about four seconds); limit >= 0
 * sets it for launches enqueued afterwards in this process, a negative limit only reads it.
 * Returns the previous value.  A small limit forces the give-up path (failure-handling tests: with
 * 0 every wave that waits gives up at once).  Not synchronised with concurrent launching threads. */
int32_t la_set_chain_spin_limit(int32_t limit);

/* Static description of a status code (any int32_t: codes that are not a la_status give
 * "unknown status"); never NULL. */
const char* la_status_str(int32_t status);

/* 1 if la_chunk_fwd has a kernel for this shape and chunk (validation passes), else 0. */
int32_t la_supported(const la_shape* shape, int32_t chunk);

/* Library ABI version, (major << 16) | minor. */
int32_t la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_CHUNK_H */
