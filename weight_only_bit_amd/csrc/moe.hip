// MoE stage 1 BF16 x MXFP4 (placeholder until the grouped kernel lands).
#include "wob_device.hpp"
#include "wob_internal.hpp"

namespace wob {
size_t moe_workspace_bytes(int64_t T, int64_t topk, int64_t E)
{
    return (size_t)(E + 1) * 4 + (size_t)T * topk * 4 + 64;
}
hipError_t launch_mxfp4_moe(const void *, const int32_t *, const uint8_t *, const uint8_t *, void *,
                            int, int, int, int, int, void *, hipStream_t)
{
    return hipErrorNotSupported;
}
} // namespace wob
