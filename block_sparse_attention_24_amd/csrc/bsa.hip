// Launchers of the attention kernels (bsa_kernels.h) without the online
// skip: bsa_fp8_kernel and bsa_bf16_kernel for d = 128 and 128-token
// blocks, bsa_kernel for every other shape.
#include "bsa_kernels.h"

namespace stem {
namespace {

template <int DT, int D, int BLK>
hipError_t launch_cfg(const BsaArgs &a, bool sparse, hipStream_t st) {
    using G = Geo<DT, D, BLK>;
    const dim3 grid((unsigned)(a.batch * a.hq * a.nb));       // one workgroup per row
    const dim3 pgrid(persistent_grid(a.batch * a.hq * a.nb));  // persistent: one workgroup per CU
    const bool paged = a.table != nullptr;
    if constexpr (DT == kFP8 && D == 128 && BLK == 128) {
        if (sparse && paged) hipLaunchKernelGGL((bsa_fp8_kernel<true, true, false>), pgrid, dim3(fp8p::NT), 0, st, a);
        else if (sparse) hipLaunchKernelGGL((bsa_fp8_kernel<true, false, false>), pgrid, dim3(fp8p::NT), 0, st, a);
        else if (paged) hipLaunchKernelGGL((bsa_fp8_kernel<false, true, false>), pgrid, dim3(fp8p::NT), 0, st, a);
        else hipLaunchKernelGGL((bsa_fp8_kernel<false, false, false>), pgrid, dim3(fp8p::NT), 0, st, a);
    } else if constexpr (DT == kBF16 && D == 128 && BLK == 128) {
        if (sparse && paged) hipLaunchKernelGGL((bsa_bf16_kernel<true, true, false>), pgrid, dim3(bf16p::NT), 0, st, a);
        else if (sparse) hipLaunchKernelGGL((bsa_bf16_kernel<true, false, false>), pgrid, dim3(bf16p::NT), 0, st, a);
        else if (paged) hipLaunchKernelGGL((bsa_bf16_kernel<false, true, false>), pgrid, dim3(bf16p::NT), 0, st, a);
        else hipLaunchKernelGGL((bsa_bf16_kernel<false, false, false>), pgrid, dim3(bf16p::NT), 0, st, a);
    } else {
        if (sparse && paged) hipLaunchKernelGGL((bsa_kernel<DT, D, BLK, true, true>), grid, dim3(G::NT), 0, st, a);
        else if (sparse) hipLaunchKernelGGL((bsa_kernel<DT, D, BLK, true, false>), grid, dim3(G::NT), 0, st, a);
        else if (paged) hipLaunchKernelGGL((bsa_kernel<DT, D, BLK, false, true>), grid, dim3(G::NT), 0, st, a);
        else hipLaunchKernelGGL((bsa_kernel<DT, D, BLK, false, false>), grid, dim3(G::NT), 0, st, a);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const Shape &s, const BsaArgs &a, bool sparse, hipStream_t st) {
    if (s.d == 64 && s.blk == 64) return launch_cfg<DT, 64, 64>(a, sparse, st);
    if (s.d == 64 && s.blk == 128) return launch_cfg<DT, 64, 128>(a, sparse, st);
    if (s.d == 128 && s.blk == 64) return launch_cfg<DT, 128, 64>(a, sparse, st);
    return launch_cfg<DT, 128, 128>(a, sparse, st);
}

}  // namespace

hipError_t launch_bsa(const Shape &s, const void *q, const KvView &kv, const uint32_t *mask, void *o,
                      float *lse, hipStream_t st) {
    const BsaArgs a = make_args(s, q, kv, mask, o, lse);
    const bool sparse = mask != nullptr;
    switch (s.dtype) {
        case STEM_F32: return launch_dt<kF32>(s, a, sparse, st);
        case STEM_BF16: return launch_dt<kBF16>(s, a, sparse, st);
        default: return launch_dt<kFP8>(s, a, sparse, st);
    }
}

}  // namespace stem
