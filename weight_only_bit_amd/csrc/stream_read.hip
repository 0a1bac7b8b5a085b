// HBM streaming-read reference: a plain read of a byte range, timed beside
// the GEMV kernels so that their rate can be set against what a kernel that
// does nothing but read achieves on the same device for the same byte count.
// It is a measurement aid, not a step of any product.
//
// Each lane reads 16-byte blocks with non-temporal loads over a grid-stride
// loop, one block per iteration (at every step the whole grid reads one
// contiguous window), with 8 workgroups of 256 lanes per compute unit.  This
// is the fastest form found in a sweep on MI355X at the decode call's 133.8
// MB (loads per lane per iteration 1..16, 4..64 workgroups per compute unit,
// 256 or 512 lanes, grid-stride against one contiguous chunk per workgroup):
// 19.5-20.0 us (6.7-6.8 TB/s) for the best forms, against 23-32 us for
// eight or sixteen blocks per lane per iteration at this grid.  The blocks
// are folded into a checksum that is stored only if it equals a constant the
// data never produces in practice, so the loads cannot be removed; the store
// is a per-lane vector store.
#include "wob_device.hpp"
#include "wob_internal.hpp"

namespace wob {
namespace {

constexpr int SR_THREADS = 256;
constexpr int SR_WGS_PER_CU = 8; // workgroups per compute unit
constexpr uint32_t SR_NEVER = 0x9E3779B9u;

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4 *__restrict__ p,
                                                                 size_t n16,
                                                                 uint32_t *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * SR_THREADS;
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * SR_THREADS + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == SR_NEVER)
        sink[threadIdx.x] = acc;
}

} // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    const size_t n16 = bytes / 16;
    const size_t want = (n16 + SR_THREADS - 1) / SR_THREADS;
    const unsigned grid =
        (unsigned)std::min<size_t>(want, (size_t)device_topology().cus * SR_WGS_PER_CU);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(SR_THREADS), 0, stream,
                       static_cast<const u32x4 *>(buf), n16, sink);
    return hipGetLastError();
}

} // namespace wob
