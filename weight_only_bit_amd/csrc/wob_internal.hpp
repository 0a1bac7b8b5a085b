// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace wob {

// A kernel that uses more than 64 KB of dynamic LDS (gfx950 has 160 KB per
// CU) must raise its limit with hipFuncSetAttribute, once for every device it
// runs on (the attribute belongs to the device's context).  `done` holds one
// bit per device ordinal already set; the caller keeps one per kernel.
inline hipError_t lds_optin(const void *kern, int bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

// Compute units and XCDs of the current device (the XCD count is the number
// of L2 domains that workgroups are dealt to round-robin).  Queried once per
// device; {256, 8} (MI355X) when the device cannot be queried.
struct DevTopo {
    int cus, xcds;
};
DevTopo device_topology();

struct W4Args {
    const void *x;
    const uint32_t *qweight;
    const void *scales;
    const uint32_t *qzeros; // nullptr: symmetric (z = 8)
    void *y;
    int dt; // DT_F16 / DT_BF16
    int M, N, K, g;
};

// Skinny split-K GEMV (M <= 8).
bool skinny_fits(int M, int N, int K, int g);
hipError_t launch_w4a16_skinny(const W4Args &a, hipStream_t stream);

// Cooperative-tile MFMA GEMM (any M).
hipError_t launch_w4a16_tiled(const W4Args &a, hipStream_t stream);

// Ragged grouped form of the tiled GEMM.
hipError_t launch_w4a16_grouped(const W4Args &a, const int64_t *m_offsets, int num_groups,
                                hipStream_t stream);

// MoE stage 1, BF16 x MXFP4.
size_t moe_workspace_bytes(int64_t T, int64_t topk, int64_t E);
// MoE stage 2: routing scratch plus the fp32 per-pair rows `pre` [T*topk][H].
size_t moe_stage2_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t H);
hipError_t launch_mxfp4_moe_stage2(const void *a, const int32_t *ids, const float *w,
                                   const uint8_t *w_fp4, const uint8_t *w_scale, void *y, int T,
                                   int topk, int E, int H, int I, void *workspace,
                                   hipStream_t stream);
// The static routing scratch of the allocation-free entry point: its size,
// and its address on the current device (looked up on first use per device).
size_t moe_scratch_bytes();
hipError_t moe_scratch(void **ptr);
// tile_m: 32 or 16 (MFMA block height of the expert tiles; T <= 8 ignores it).
hipError_t launch_mxfp4_moe(const void *x, const int32_t *ids, const uint8_t *w_fp4,
                            const uint8_t *w_scale, void *y, int T, int topk, int E, int N, int K,
                            int act, int tile_m, void *workspace, hipStream_t stream);

// Dequantization probes.
hipError_t launch_w4a16_dequant(const uint32_t *qweight, const void *scales, const uint32_t *qzeros,
                                void *out, int dt, bool out_f32, int N, int K, int g,
                                hipStream_t stream);
// Streaming-read reference (measurement aid): reads `bytes` (a multiple of
// 16) of `buf`; `sink` is 256 words of scratch the kernel may write.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

hipError_t launch_mxfp4_dequant(const uint8_t *w_fp4, const uint8_t *w_scale, void *out, int N,
                                int K, hipStream_t stream);

} // namespace wob
