// Launcher of the attention kernels with the online skip (BLASST summary,
// §2.1 running-maximum pruning): bsa_fp8_kernel and bsa_bf16_kernel with
// SKIP = true.  Built as its own translation unit with machine-code
// sinking disabled: the skip puts wave-uniform branches around the softmax
// slices of the pipelined region, and sinking would move every MFMA of the
// region below them, keeping all their operands live at once.
#include "bsa_kernels.h"

namespace stem {
namespace {

// The pipelined kernels with the online skip (d = 128, 128-token blocks).
template <int DT>
hipError_t launch_skip(const BsaArgs &a, bool sparse, hipStream_t st) {
    const dim3 pgrid(persistent_grid(a.batch * a.hq * a.nb));  // persistent: one workgroup per CU
    const bool paged = a.table != nullptr;
    if constexpr (DT == kFP8) {
        if (sparse && paged) hipLaunchKernelGGL((bsa_fp8_kernel<true, true, true>), pgrid, dim3(fp8p::NT), 0, st, a);
        else if (sparse) hipLaunchKernelGGL((bsa_fp8_kernel<true, false, true>), pgrid, dim3(fp8p::NT), 0, st, a);
        else if (paged) hipLaunchKernelGGL((bsa_fp8_kernel<false, true, true>), pgrid, dim3(fp8p::NT), 0, st, a);
        else hipLaunchKernelGGL((bsa_fp8_kernel<false, false, true>), pgrid, dim3(fp8p::NT), 0, st, a);
    } else {
        if (sparse && paged) hipLaunchKernelGGL((bsa_bf16_kernel<true, true, true>), pgrid, dim3(bf16p::NT), 0, st, a);
        else if (sparse) hipLaunchKernelGGL((bsa_bf16_kernel<true, false, true>), pgrid, dim3(bf16p::NT), 0, st, a);
        else if (paged) hipLaunchKernelGGL((bsa_bf16_kernel<false, true, true>), pgrid, dim3(bf16p::NT), 0, st, a);
        else hipLaunchKernelGGL((bsa_bf16_kernel<false, false, true>), pgrid, dim3(bf16p::NT), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bsa_skip(const Shape &s, const void *q, const KvView &kv, const uint32_t *mask,
                           float skip_log2, void *o, float *lse, int32_t *skipped, hipStream_t st) {
    BsaArgs a = make_args(s, q, kv, mask, o, lse);
    a.skip_log2 = skip_log2;
    a.skipped = skipped;
    if (s.d != 128 || s.blk != 128 || s.dtype == STEM_F32) return hipErrorNotSupported;
    return s.dtype == STEM_BF16 ? launch_skip<kBF16>(a, mask != nullptr, st) : launch_skip<kFP8>(a, mask != nullptr, st);
}

}  // namespace stem
