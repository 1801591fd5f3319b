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

namespace la {
namespace {

constexpr int C = 64;  // chunk length

}  // namespace

// One stream-ordered memory pool per device for temporary workspace; it keeps what it has
// allocated (release threshold = max), so after the first call no allocation reaches the driver.
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

hipError_t launch_chunk_fwd_mfma(const FwdArgs& a) {
    int G, cps;
    // small heads: 512 workgroups (latency-bound kernels, several share a compute unit)
    mfma_split(a, &G, &cps, a.dk < 128 ? 512 : 256);
    float* part_state = nullptr;
    float* part_decay = nullptr;
    if (G > 1) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        hipMemPool_t pool = workspace_pool(dev);
        if (!pool) return hipErrorOutOfMemory;
        const size_t n = (size_t)(a.B * a.H * a.nseg) * (G - 1);
        const size_t D = (size_t)a.dk;
        e = hipMallocFromPoolAsync((void**)&part_state, n * D * D * sizeof(float) + n * D * sizeof(float), pool,
                                   a.stream);
        if (e != hipSuccess) return e;
        part_decay = part_state + n * D * D;
    }
    hipError_t e = a.dk == 128 ? launch_chunk_fwd_pipe(a, G, cps, part_state, part_decay)
                               : launch_chunk_fwd_small(a, G, cps, part_state, part_decay);
    if (part_state) {
        hipError_t f = hipFreeAsync(part_state, a.stream);
        if (e == hipSuccess) e = f;
    }
    return e;
}

}  // namespace la
