// stem_score_noalloc: stem_score for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its scratch -- the pooled representations qbar, kbar
// and lvn that stem_score writes to a caller's workspace -- lives in a
// file-scope device array of fixed size instead.  Every device the library
// runs on holds its own copy of the array until the process ends; all calls
// on one device share it, so calls that overlap on one device race.  The
// pooling kernels write every scratch byte the score GEMM reads, so nothing
// has to be cleared between calls.
#include <mutex>

#include "stem_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[STEM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Device address of the current device's copy of `scratch`.  In host code the
// array's name is only a stand-in for the symbol, so the address is looked up
// once per device, with that device current, and kept.
hipError_t scratch_of(int device, void **ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[device],
                   [device] { g_lookup[device] = hipGetSymbolAddress(&g_scratch[device], HIP_SYMBOL(scratch)); });
    *ptr = g_scratch[device];
    return g_lookup[device];
}

}  // namespace

using namespace stem;

extern "C" int stem_score_noalloc(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                                  float *scores, void *stream) {
    Shape s;
    KvView v;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if ((rc = check_kv(kv, s, &v))) return rc;
    if (!q || !scores) return fail(STEM_EINVAL, "q or scores is NULL");
    size_t oq, ok_, ol, total;
    workspace_layout(s, &oq, &ok_, &ol, &total);
    if (total > (size_t)STEM_NOALLOC_SCRATCH_BYTES)
        return fail(STEM_EWORKSPACE, "the problem needs %zu bytes of scratch; stem_score_noalloc holds %zu "
                    "(use stem_score with a workspace)", total, (size_t)STEM_NOALLOC_SCRATCH_BYTES);
    if ((rc = hip_precheck())) return rc;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "stem_score_noalloc: hipGetDevice");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (st) {
        int sdev = -1;
        if ((e = hipStreamGetDevice(st, &sdev)) != hipSuccess) return hip_status(e, "stem_score_noalloc: stream");
        if (sdev != dev)
            return fail(STEM_EINVAL, "the stream belongs to device %d, the current device is %d", sdev, dev);
    }
    void *ws = nullptr;
    if ((e = scratch_of(dev, &ws)) != hipSuccess) return hip_status(e, "stem_score_noalloc: scratch address");
    return score_launch(s, q, &v, scores, ws, false, st, "stem_score_noalloc launch");
}
