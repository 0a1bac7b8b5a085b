// Cooperative-tile MFMA GEMM (placeholder until the tiled kernel lands).
#include "wob_device.hpp"
#include "wob_internal.hpp"

namespace wob {
hipError_t launch_w4a16_tiled(const W4Args &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_w4a16_grouped(const W4Args &, const int64_t *, int, hipStream_t)
{
    return hipErrorNotSupported;
}
} // namespace wob
