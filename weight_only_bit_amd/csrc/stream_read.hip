// HBM streaming-read reference: a plain read of a byte range, timed beside
// the GEMV kernels so that their rate can be set against what a kernel that
// does nothing but read achieves on the same device for the same byte count.
// It is a measurement aid, not a step of any product.
//
// Each lane reads 16-byte blocks with non-temporal loads, SR_U of them in
// flight at a time, over a grid-stride loop (at every step the whole grid
// reads one contiguous window).  The blocks are folded into a checksum that is
// stored only if it equals a constant the data never produces in practice, so
// the loads cannot be removed; the store is a per-lane vector store.
#include "wob_device.hpp"
#include "wob_internal.hpp"

namespace wob {
namespace {

constexpr int SR_THREADS = 256;
constexpr int SR_U = 8;          // loads in flight per lane
constexpr int SR_WGS_PER_CU = 8; // workgroups per compute unit (256 CUs)
constexpr uint32_t SR_NEVER = 0x9E3779B9u;

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4 *__restrict__ p,
                                                                 size_t n16,
                                                                 uint32_t *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * SR_THREADS;
    size_t i = (size_t)blockIdx.x * SR_THREADS + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (SR_U - 1) * stride < n16; i += SR_U * stride) {
        u32x4 v[SR_U];
#pragma unroll
        for (int u = 0; u < SR_U; ++u)
            v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < SR_U; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
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
    const unsigned grid = (unsigned)std::min<size_t>(want, (size_t)256 * SR_WGS_PER_CU);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(SR_THREADS), 0, stream,
                       static_cast<const u32x4 *>(buf), n16, sink);
    return hipGetLastError();
}

} // namespace wob
