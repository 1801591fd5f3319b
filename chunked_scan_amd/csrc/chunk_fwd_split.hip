// chunk_fwd_split.hip -- the bf16 MFMA forward for dk = dv in {32, 64, 128}, chunk = 64: how a
// segment is spread over the GPU, and the workspace that takes.
//
// A (b,h) sequence alone offers one serial chain of chunks, far too few workgroups for 256
// compute units, so each segment is cut into G sub-segments and the linear-decomposition identity
// of the ZeCO review page (pith_extraction.key_machinery) is applied inside the GPU:
//   pass 1 (state only): every sub-segment but the last computes its local end state from zero
//          (sub-segment 0 of segment 0 from s_in) and its total decay;
//   scan:  an inclusive state scan over the sub-segments turns those into exact incoming states;
//   pass 2 (outputs):  every sub-segment re-runs its chunks from its exact incoming state and
//          writes O; the last one writes s_out.
// Pass 2 therefore needs no output correction.  The cost is one extra read of K and V (and g).
// The kernels themselves are in chunk_fwd_pipe.hip (d = 128) and chunk_fwd_small.hip (d = 32, 64).
#include "la_device.h"
#include "la_internal.h"

#include <mutex>
#include <vector>

namespace la {
namespace {

constexpr int C = 64;  // chunk length

}  // namespace

// One stream-ordered memory pool per device for temporary workspace; it keeps what it has
// allocated (release threshold = max), so after the first call no allocation reaches the driver.
// la_trim_workspace hands what is not in use back to the device.
hipMemPool_t workspace_pool(int dev) {
    static std::mutex mu;
    static hipMemPool_t pools[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 0 || dev >= 64) return nullptr;
    if (!pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        if (hipMemPoolCreate(&p, &props) != hipSuccess) return nullptr;
        uint64_t keep = ~0ull;
        (void)hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
        pools[dev] = p;
    }
    return pools[dev];
}

hipError_t workspace_alloc(void** p, size_t bytes, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipMemPool_t pool = workspace_pool(dev);
    if (!pool) return hipErrorOutOfMemory;
    return hipMallocFromPoolAsync(p, bytes, pool, stream);
}

// Workspace kept between calls, one buffer per (device, stream, call site), grown when a call
// needs more.  Calls on one stream run in order, so the buffer a call leaves is free for the next
// call on that stream; calls on different streams get different buffers.  Taking it costs nothing
// on the GPU, where a pool allocation and its stream-ordered free per call put ≈2.5 µs of queue
// bubbles into the headline step (82.5 against 85 µs).  A stream under graph capture takes a
// per-call pool allocation instead (owned: the caller frees it), so a graph never holds a cached
// buffer.  A slot is taken by one call site only, so nested calls never share a buffer.
namespace {
struct CachedWorkspace {
    int dev, slot;
    hipStream_t stream;
    void* p;
    size_t bytes;
};
std::mutex cache_mu;
std::vector<CachedWorkspace> cache;
}  // namespace

hipError_t workspace_acquire(int slot, void** p, size_t bytes, hipStream_t stream, bool* owned) {
    *owned = true;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess || st != hipStreamCaptureStatusNone)
        return workspace_alloc(p, bytes, stream);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(cache_mu);
    for (size_t i = 0; i < cache.size(); i++) {
        CachedWorkspace& c = cache[i];
        if (c.dev != dev || c.slot != slot || c.stream != stream) continue;
        if (c.bytes < bytes) {  // grow: the old buffer goes back once the stream's earlier work is done
            e = hipFreeAsync(c.p, stream);
            if (e == hipSuccess) e = workspace_alloc(&c.p, bytes, stream);
            if (e != hipSuccess) {
                cache.erase(cache.begin() + i);
                return e;
            }
            c.bytes = bytes;
        }
        *p = c.p;
        *owned = false;
        return hipSuccess;
    }
    void* q = nullptr;
    e = workspace_alloc(&q, bytes, stream);
    if (e != hipSuccess) return e;
    cache.push_back({dev, slot, stream, q, bytes});
    *p = q;
    *owned = false;
    return hipSuccess;
}

hipError_t workspace_release(void* p, hipStream_t stream, bool owned) {
    return owned && p ? hipFreeAsync(p, stream) : hipSuccess;
}

hipError_t workspace_trim() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipMemPool_t pool = workspace_pool(dev);
    if (!pool) return hipErrorOutOfMemory;
    {
        // the cached buffers of this device: once the device is idle none is in use
        std::lock_guard<std::mutex> lock(cache_mu);
        bool any = false;
        for (const CachedWorkspace& c : cache) any |= c.dev == dev;
        if (any) {
            if ((e = hipDeviceSynchronize()) != hipSuccess) return e;
            for (size_t i = cache.size(); i-- > 0;)
                if (cache[i].dev == dev) {
                    if ((e = hipFreeAsync(cache[i].p, nullptr)) != hipSuccess) return e;
                    cache.erase(cache.begin() + i);
                }
            if ((e = hipDeviceSynchronize()) != hipSuccess) return e;
        }
    }
    return hipMemPoolTrimTo(pool, 0);
}

// Sub-segments: about `target` workgroups in total (256: one round on the compute units), at
// least 4 chunks each, unless the caller fixes the sub-segment length.
void mfma_split(const FwdArgs& a, int* G_out, int* cps_out, int64_t target) {
    const int64_t units = a.B * a.H * a.nseg;
    const int64_t Lseg = a.L / a.nseg;
    const int64_t nch = (Lseg + C - 1) / C;
    int64_t cps;
    if (a.subseg_chunks > 0) {
        cps = a.subseg_chunks;
    } else {
        const int64_t g_want = (target + units - 1) / units;
        cps = (nch + g_want - 1) / g_want;
        if (cps < 4) cps = 4;
    }
    if (cps > nch) cps = nch > 0 ? nch : 1;
    *G_out = (int)((nch + cps - 1) / cps);
    if (*G_out < 1) *G_out = 1;
    *cps_out = (int)cps;
}

// The split of the matrix-core forward.  64-token chunks: 512 workgroups for small heads (their
// kernels are latency-bound and several share a compute unit), 256 for d = 128 and for d = 256
// (whose sub-segments take four workgroups each, one per value tile).  128-token
// chunks (small heads): about 256 workgroups, at least two chunks per sub-segment; the
// sub-segment length a caller gives counts chunks of the call's own length.
void fwd_split_plan(const FwdArgs& a, int* G_out, int* cps_out) {
    if (a.chunk != 128) {
        // d = 256: four value tiles per sub-segment, so a quarter as many sub-segments
        mfma_split(a, G_out, cps_out, a.dk < 128 ? 512 : a.dk == 256 ? 64 : 256);
        return;
    }
    constexpr int CH = 128;
    const int64_t units = a.B * a.H * a.nseg;
    const int64_t nch = (a.L / a.nseg + CH - 1) / CH;
    int64_t cps;
    if (a.subseg_chunks > 0) {
        cps = a.subseg_chunks;
    } else {
        const int64_t g_want = (256 + units - 1) / units;
        cps = max((int64_t)2, (nch + g_want - 1) / g_want);
    }
    if (cps > nch) cps = nch > 0 ? nch : 1;
    *G_out = (int)max((int64_t)1, (nch + cps - 1) / cps);
    *cps_out = (int)cps;
}

// Floats of workspace for G sub-segments per segment: a state and a decay vector for every
// sub-segment but the last of every (b, h, segment); with the d = 128 gate kernel also four int flags
// per workgroup of its two passes (the units it hands to the windowed redo).
static size_t gate_flag_words(const FwdArgs& a, int G) {
    return (a.mode == DECAY_GATE && a.dk == 128 && a.chunk == 64) ? 4 * (size_t)(a.B * a.H * a.nseg) * (2 * G - 1)
                                                                   : 0;
}
// The chained single launch replaces the passes when the caller asks for it (fwd_schedule 2) and
// it exists: bf16 d = 128, 64-token chunks, no or head decay, a segment split at all.  It is not
// the default: on MI355X at B1 H16 L16384 the passes take 84.5 us (state pass, scan, output pass)
// and the chained kernel 84.8 us plus its flag reset, about 6 us.
// Its workgroups wait on one another across the whole chain, so all of them must be resident at
// once: one per compute unit.
static int compute_units() {
    static std::mutex mu;
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus[dev] = 0;
    return cus[dev];
}
static bool use_chain(const FwdArgs& a, int G) {
    return G > 1 && a.schedule == 2 && a.dk == 128 && a.dv == 128 && a.chunk == 64 && a.mode != DECAY_GATE &&
           a.B * a.H * a.nseg * G <= compute_units();
}
size_t fwd_split_workspace_floats(const FwdArgs& a, int G) {
    if (use_chain(a, G)) return chain_workspace_floats(a, G);
    const size_t flags = gate_flag_words(a, G);
    if (G <= 1) return flags;
    const size_t n = (size_t)(a.B * a.H * a.nseg) * (size_t)(G - 1);
    const size_t D = (size_t)a.dk;
    return n * D * D + n * D + flags;
}

namespace {

// The kernels of the split forward with the workspace at ws (fwd_split_workspace_floats floats;
// unused when G == 1).
hipError_t fwd_split_run(const FwdArgs& a, int G, int cps, float* ws) {
    if (use_chain(a, G)) return launch_chunk_fwd_chain(a, G, cps, ws);
    const size_t n = G > 1 ? (size_t)(a.B * a.H * a.nseg) * (size_t)(G - 1) : 0;
    float* part_state = G > 1 ? ws : nullptr;
    float* part_decay = G > 1 ? ws + n * a.dk * a.dk : nullptr;
    int* flags = gate_flag_words(a, G) ? (int*)(ws + n * a.dk * a.dk + n * a.dk) : nullptr;
    if (a.dk == 256 || (a.chunk == 128 && a.dk == 128)) return launch_chunk_fwd_tiled(a, G, cps, part_state, part_decay);
    if (a.chunk == 128) return launch_chunk_fwd_small_ch128(a, G, cps, part_state, part_decay);
    return a.dk == 128 ? launch_chunk_fwd_pipe(a, G, cps, part_state, part_decay, flags)
                       : launch_chunk_fwd_small(a, G, cps, part_state, part_decay);
}

}  // namespace

hipError_t launch_chunk_fwd_mfma(const FwdArgs& a) {
    int G, cps;
    fwd_split_plan(a, &G, &cps);
    const size_t nf = fwd_split_workspace_floats(a, G);
    float* ws = nullptr;
    bool owned = false;
    if (nf > 0) {
        hipError_t e = workspace_acquire(WS_FORWARD, (void**)&ws, nf * sizeof(float), a.stream, &owned);
        if (e != hipSuccess) return e;
    }
    hipError_t e = fwd_split_run(a, G, cps, ws);
    const hipError_t f = workspace_release(ws, a.stream, owned);
    return e == hipSuccess ? f : e;
}

// ---- the allocation-free forward (la_chunk_fwd_noalloc)
//
// Its workspace is this fixed device array: every device the library runs on holds one copy,
// from the code object's load until the process ends.  Host code never uses the array's name
// as an address (on the host it only names the symbol): the device address of each device's
// copy is looked up once per device and kept in noalloc_ptr.  Every call on a device shares that
// copy; nothing in it needs to start at zero (the state pass writes every entry the scan and the
// output pass read), and calls that overlap in time on one device race on it.
static __device__ __align__(256) float scratch[LA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

// The device address of `scratch` on the current device (looked up on the first call for that
// device), or null if the lookup failed.
float* noalloc_ptr(hipError_t* err) {
    static std::mutex mu;
    static float* ptrs[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        ptrs[dev] = (float*)p;
    }
    *err = hipSuccess;
    return ptrs[dev];
}

}  // namespace

size_t fwd_noalloc_bytes(const FwdArgs& a) {
    int G, cps;
    fwd_split_plan(a, &G, &cps);
    return fwd_split_workspace_floats(a, G) * sizeof(float);
}

hipError_t launch_chunk_fwd_mfma_noalloc(const FwdArgs& a) {
    int G, cps;
    fwd_split_plan(a, &G, &cps);
    if (fwd_split_workspace_floats(a, G) * sizeof(float) > LA_NOALLOC_SCRATCH_BYTES) return hipErrorInvalidValue;
    float* ws = nullptr;
    if (fwd_split_workspace_floats(a, G) > 0) {
        hipError_t e = hipSuccess;
        ws = noalloc_ptr(&e);
        if (!ws) return e;
    }
    return fwd_split_run(a, G, cps, ws);
}

}  // namespace la
