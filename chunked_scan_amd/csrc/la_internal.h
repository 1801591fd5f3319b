// la_internal.h -- host-side interface between the C-ABI layer (la_api.hip) and the kernel
// launchers.  Arguments have already been validated when a launcher is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_chunk.h"

namespace la {



// Brackets each enqueued kernel with the caller's trace events (no-op without a trace).
struct Tracer {
    la_trace* t = nullptr;
    hipStream_t s = nullptr;
    bool open = false;
    void begin(const char* name) {
        open = t && t->count < t->capacity;
        if (open) {
            t->name[t->count] = name;
            (void)hipEventRecord((hipEvent_t)t->start[t->count], s);
        }
    }
    void end() {
        if (open) {
            (void)hipEventRecord((hipEvent_t)t->stop[t->count], s);
            t->count++;
            open = false;
        }
    }
};

// Launches a kernel between the tracer's events: LA_TRACED(tr, "name", kernel<<<...>>>(...));
#define LA_TRACED(tr, name, ...)        \
    do {                                \
        if (tr) (tr)->begin(name);      \
        __VA_ARGS__;                    \
        if (tr) (tr)->end();            \
    } while (0)

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* decay;
    const float* s_in;
    void* o;
    float* s_out;
    int64_t s_out_stride;  // elements between (b,h) blocks of s_out
    int64_t B, H, L;
    int dk, dv, nseg, chunk;
    bool bf16;
    int mode;
    float inv_norm;      // 1 / gate_norm (gate mode)
    int subseg_chunks;   // 0 = automatic
    int schedule = 0;    // la_shape.fwd_schedule: 0 = library choice (passes), 1 = passes, 2 = chained where available
    hipStream_t stream;
    Tracer* tr;
    void* q_dec = nullptr;     // optional: q times its cumulative decay from the segment start
    float* total = nullptr;    // optional: each segment's total decay
    int64_t total_stride = 0;  // elements between (b,h) blocks of total
    uint32_t* tile_live = nullptr;  // optional: [B,H,nseg,ceil(L/nseg/64)], 0 = the 64-token tile of q_dec is zero
};

struct CorrectArgs {
    const void* q;
    const float* cum;    // NONE: null; HEAD: [H] log-decay; GATE: [B,H,L,dk] cumulative decay
    const float* s_recv;
    void* o;
    int64_t B, H, L;
    int dk, dv, nseg, seg_begin;
    int64_t state_stride;
    bool bf16;
    int mode;
    hipStream_t stream;
    Tracer* tr;
    const uint32_t* tile_live = nullptr;  // optional: [B,H,nseg,ceil(L/nseg/64)]; 0 = skip the tile (q rows zero)
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* decay;
    const float* s_in;
    const void* d_o;
    const float* ds_out;   // [b,h] blocks of state_stride elements, segment p at p * dk * dv; may be null
    void* dq;
    void* dk_out;
    void* dv_out;
    float* d_decay;        // HEAD: [H]; GATE: [B,H,L,dk]; may be null
    float* ds_in;          // same layout as ds_out; may be null
    int64_t state_stride;
    int64_t B, H, L;
    int dk, dv, nseg, chunk;
    bool bf16;
    int mode;
    float inv_norm;
    int subseg_chunks;     // matrix-core path: chunks per sub-segment, 0 = automatic
    // optional: the state entering every sub-segment of sub_len tokens of every segment, (b,h)
    // blocks of sub_stride floats, segment p's sub-segment j at (p * ceil(Lseg / sub_len) + j) * dk * dv
    // (j = 0 unused: the segment's initial state is s_in or zero); the matrix-core path then splits
    // at those sub-segments and needs no forward state pass
    const float* s_sub;
    int64_t sub_stride;
    int sub_len;
    hipStream_t stream;
    Tracer* tr;
};

// Stream-ordered workspace pool of a device (chunk_fwd_split.hip), which keeps its memory.
hipMemPool_t workspace_pool(int dev);
// Temporary workspace on the current device's pool, stream-ordered on `stream` (free it with
// hipFreeAsync on the same stream).
hipError_t workspace_alloc(void** p, size_t bytes, hipStream_t stream);
// Workspace that stays with (current device, stream, slot) between calls (chunk_fwd_split.hip):
// *owned = false, and the next call on that stream with the same slot gets the same memory; on a
// stream under graph capture a per-call pool allocation, *owned = true.  Release with
// workspace_release either way.  Each call site has its own slot.
enum WorkspaceSlot { WS_FORWARD = 0, WS_BACKWARD = 1 };
hipError_t workspace_acquire(int slot, void** p, size_t bytes, hipStream_t stream, bool* owned);
hipError_t workspace_release(void* p, hipStream_t stream, bool owned);
// Synchronises the device if it holds cached workspace, frees that, and returns the pool memory
// not in use to the device.
hipError_t workspace_trim();

// Chunked backward with fp32 arithmetic on VALU (chunk_bwd_generic.hip): every shape the generic
// forward takes.
hipError_t launch_chunk_bwd_generic(const BwdArgs& a);
// bf16 MFMA backward (chunk_bwd_mfma*.hip): dk = dv in {32, 64, 128}, chunk 64, no decay or head decay.
bool chunk_bwd_mfma_supported(const BwdArgs& a);
hipError_t launch_chunk_bwd_mfma(const BwdArgs& a);

// Generic chunked forward: fp32 arithmetic on VALU, q/k/v/o in f32 or bf16, dk, dv in
// {16,32,64,128}, chunk in {16,32,64}.
hipError_t launch_chunk_fwd_generic(const FwdArgs& a);

// bf16 MFMA chunked forward for dk = dv in {32, 64, 128} with chunk = 64, or dk = dv in {32, 64}
// with chunk = 128, with intra-GPU sub-segment splitting (chunk_fwd_split.hip), all decay modes.
// The workspace of the split comes from the device's workspace pool.
hipError_t launch_chunk_fwd_mfma(const FwdArgs& a);
// The same with the workspace in the library's fixed device array (nothing allocated): fails with
// hipErrorInvalidValue when fwd_noalloc_bytes(a) exceeds LA_NOALLOC_SCRATCH_BYTES.
hipError_t launch_chunk_fwd_mfma_noalloc(const FwdArgs& a);
// Workspace bytes the matrix-core forward needs for this call (0 when it does not split).
size_t fwd_noalloc_bytes(const FwdArgs& a);
// A split of each segment into G sub-segments of cps chunks (uses B, H, L, nseg, subseg_chunks).
// target: about how many workgroups to aim for when the length is chosen automatically.
void mfma_split(const FwdArgs& a, int* G_out, int* cps_out, int64_t target = 256);
// The matrix-core forward's own split (by chunk length and head dim) and its workspace size.
void fwd_split_plan(const FwdArgs& a, int* G_out, int* cps_out);
size_t fwd_split_workspace_floats(const FwdArgs& a, int G);
// Its kernels: G sub-segments of cps chunks; part_state / part_decay the workspace of the
// sub-segment scan (unused when G == 1); gate mode: wide the 4 * B*H*nseg * (2G - 1) ints of the
// per-unit flags that send a unit to the windowed redo (unused otherwise).
// The dv-tiled matrix-core forward (no decay or head decay): dk = dv = 256 with 64-token chunks
// (four 64-column value tiles), and dk = dv = 128 with 128-token chunks.  Same split and workspace
// as the other matrix-core kernels.
hipError_t launch_chunk_fwd_tiled(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay);
// The chained d = 128 forward (no decay or head decay, G > 1 sub-segments): one launch (after a
// small flag reset) whose workgroups hand their sub-segment states on through the workspace
// (chain_workspace_floats floats).
size_t chain_workspace_floats(const FwdArgs& a, int G);
hipError_t launch_chunk_fwd_chain(const FwdArgs& a, int G, int cps, float* ws);
// polls per flag before a chained wave gives up (host-side setting, read at each launch)
extern int chain_spin_limit;
// synchronises the current device, then reads (and optionally clears) its give-up counter
hipError_t chain_status(unsigned int* give_ups, bool clear);
hipError_t launch_chunk_fwd_pipe(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay, int* wide);
// dq of the bf16 matrix-core backward at dk = dv = 128 with no or head decay, on the forward's
// d = 128 kernel: dq_t = S_t d_o_t with S_t = a S_{t-1} + k_t v_t^T is this forward with queries
// d_o, keys v and values k, whose state is S^T.  G sub-segments of cps chunks per (b, h, segment).
// With init null (and G > 1): a state pass into part_state / part_decay (units * (G - 1) states
// and decay vectors), their scan, then the output pass; else the output pass alone from the
// states entering sub-segments g >= 1 at init + bh * ist_bh + (seg * ist_g + g + ist_off) * 128 * 128.
// Every state in memory is in the forward's layout (key rows, value columns).
hipError_t launch_pipe_dq(const BwdArgs& a, int G, int cps, float* part_state, float* part_decay,
                          const float* init, int64_t ist_bh, int ist_g, int ist_off);
// The same for dk = dv = 32 or 64 (chunk_fwd_small.hip).
hipError_t launch_chunk_fwd_small(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay);
// The d = 128 gate output pass (or state pass) on the small-head kernel for the units whose four
// int flags (flags + 4 * unit) are not all zero; the others are left as they are.
hipError_t launch_small_gate128_redo(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay,
                                     bool state_only, const int* flags);
// The same with 128-token chunks (cps counts 128-token chunks).
hipError_t launch_chunk_fwd_small_ch128(const FwdArgs& a, int G, int cps, float* part_state, float* part_decay);

// out[n,p] = diag(lam[n,p]) out[n,p-1] + x[n,p] for n < nstates, p < P.  x may equal out.
hipError_t launch_state_scan(const float* x, const float* lam, float* out, int64_t nstates, int P,
                             int dk, int dv, hipStream_t stream, Tracer* tr);

// Output correction: MFMA kernel for bf16 with dk = dv = 128, generic fp32-arithmetic kernel otherwise.
hipError_t launch_state_correct(const CorrectArgs& a);
hipError_t launch_state_correct_generic(const CorrectArgs& a);

// total of segment p of (b,h) goes to total[bh * total_stride + p * dk].
hipError_t launch_cumdecay(const float* decay, float* cum, float* total, int64_t total_stride, int64_t B, int64_t H,
                           int64_t L, int dk, int nseg, int mode, float inv_norm, hipStream_t stream, Tracer* tr);

// a.q_dec = q times its cumulative decay from the segment start and a.total = each segment's
// total decay (either may be null), for the shapes whose forward does not emit them itself.
hipError_t launch_decayed_q(const FwdArgs& a);

// s_out[b,h,p] = (p == 0 && s_in) ? s_in[b,h] : 0 -- the final states of empty segments.
hipError_t launch_empty_states(const float* s_in, float* s_out, int64_t s_out_stride, int64_t BH, int nseg, int dk,
                               int dv, hipStream_t stream, Tracer* tr);

}  // namespace la
