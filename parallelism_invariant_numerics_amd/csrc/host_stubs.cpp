// host_stubs.cpp -- the kernel launchers of kernels.h as stubs that launch
// nothing and return hipErrorNotSupported.  Linked only into the CPU build
// of the host code (iso_host.cpp, identity.cpp, sha256.cpp) that runs under
// AddressSanitizer and UndefinedBehaviorSanitizer: every host check of the C
// ABI, the contract identities and the SHA-256 code run there as in the
// real library, and a call that passes every check reports ISO_ERR_LAUNCH
// instead of reaching a GPU.  Never part of libiso.so.
#include "kernels.h"

namespace iso {

int device_cus() { return 256; }

hipError_t launch_gemm_partials(const uint16_t *, const uint16_t *, void *, int, int64_t, int64_t,
                                int64_t, int, int, int, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_gemm_rows(const uint16_t *, const uint16_t *, void *, int, int64_t, int64_t,
                            int64_t, int, int, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_partition_combine(const float *, void *, int, int64_t, int, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_partition_combine_tiles(const float *, void *, int, int64_t, int64_t, int,
                                          hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_lmhead_stats(const uint16_t *, const uint16_t *, const int32_t *, float *,
                               float *, float *, int64_t, int64_t, int64_t, int, int, int, int64_t,
                               int64_t, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_lmhead_finish(const float *, const float *, const int32_t *, float *, int64_t,
                                int64_t, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_rmsnorm(const uint16_t *, const uint16_t *, uint16_t *, const uint16_t *, void *,
                          int, int64_t, int64_t, int, int, float, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_cpr_prefill(const uint16_t *, const uint16_t *, const uint16_t *, const float *,
                              const float *, const float *, float *, float *, float *, int64_t,
                              int64_t, int, float *, float *, float *, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_cpr_decode(const uint16_t *, const uint16_t *, const uint16_t *, const float *,
                             const float *, int64_t, float *, float *, float *, int64_t, int,
                             float *, float *, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_moe(const uint16_t *, const float *, const uint16_t *, const uint16_t *,
                      const uint16_t *, float *, int64_t, int64_t, int64_t, int64_t, int, int, int,
                      int, int, const MoeBuffers &, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t lmhead_noalloc_scratch(void **) { return hipErrorNotSupported; }

hipError_t launch_swiglu(const float *, const float *, float *, uint16_t *, int64_t, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace iso
