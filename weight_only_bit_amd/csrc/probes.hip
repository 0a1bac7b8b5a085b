// Dequantization probes: write out the weights exactly as the GEMM kernels
// form them in registers, using the same helpers (wob_device.hpp), so the
// unpack/dequant stage can be compared bit for bit with the definition.
//
//  * W4A16, fp32 form: the skinny kernel's exact (q - z) pairs (the helpers
//    that kernel calls) times the fp32 scale.  The kernel itself scales each
//    chunk's sum of products rather than each weight; the product (q - z) * s
//    is exact in fp32, so this form is the definition's value either way.
//  * W4A16, activation form: the tiled kernels' MFMA weight-operand values
//    (w4_word_act8, the helper those kernels call).
//  * MXFP4: the MoE kernel's B-operand values.
// One thread per packed word; outputs are written in natural k order.
#include "wob_device.hpp"
#include "wob_internal.hpp"

namespace wob {
namespace {

template <int DT, bool OUT_F32>
__global__ __launch_bounds__(256) void w4a16_dequant_kernel(
    const uint32_t *__restrict__ qweight, const uint16_t *__restrict__ scales,
    const uint32_t *__restrict__ qzeros, void *__restrict__ out, int N, int K, int g)
{
    const int words = K >> 3;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)N * words)
        return;
    const int n = (int)(idx / words);
    const int wi = (int)(idx % words);
    const int G = K / g;
    const int j = (wi * 8) / g;
    const uint32_t w = qweight[idx];
    const uint32_t z = qzeros ? nib(qzeros[(size_t)(n >> 3) * G + j], n & 7) : 8u;
    const uint16_t sbits = scales[(size_t)n * G + j];
    float vals[8];
    if constexpr (OUT_F32) {
        // the skinny kernel's exact (q - z) pairs (word order, its helpers),
        // times the scale in fp32 here: that kernel applies the scale to each
        // chunk's sum of products instead, and (q - z) * s is exact either way
        const float s = act_to_f32<DT>(sbits);
        u32x4 d;
        if constexpr (DT == DT_F16)
            d = w4_diff_pairs_f16(w, f16_neg_bias2(z), f16_neg_bias2_hi(z));
        else
            d = w4_diff_pairs_bf16(w, (float)z);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float lo, hi;
            if constexpr (DT == DT_F16) {
                const half2_t h = bitcast<half2_t>(d[p]);
                lo = (float)h.x;
                hi = (float)h.y;
            } else {
                lo = bitcast<float>(d[p] << 16);
                hi = bitcast<float>(d[p] & 0xFFFF0000u);
            }
            vals[word_order_value(2 * p)] = lo * s;
            vals[word_order_value(2 * p + 1)] = hi * s;
        }
        float *o = static_cast<float *>(out) + (size_t)idx * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = vals[i];
    } else {
        const u32x4 v = w4_word_act8<DT>(w, sbits, z); // natural k order
        uint16_t o16[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            o16[2 * p] = (uint16_t)(v[p] & 0xFFFFu);
            o16[2 * p + 1] = (uint16_t)(v[p] >> 16);
        }
        uint16_t *o = static_cast<uint16_t *>(out) + (size_t)idx * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = o16[i];
    }
}

__global__ __launch_bounds__(256) void mxfp4_dequant_kernel(const uint32_t *__restrict__ w_fp4,
                                                            const uint8_t *__restrict__ w_scale,
                                                            uint32_t *__restrict__ out, int N, int K)
{
    const int words = K >> 3;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)N * words)
        return;
    const int n = (int)(idx / words);
    const int wi = (int)(idx % words);
    const float scale = e8m0_to_f32(w_scale[(size_t)n * (K >> 5) + (wi >> 2)]);
    const u32x4 v = fp4_word_bf16x8(w_fp4[idx], scale);
    u32x4 *o = reinterpret_cast<u32x4 *>(out) + idx;
    *o = v;
}

} // namespace

hipError_t launch_w4a16_dequant(const uint32_t *qweight, const void *scales, const uint32_t *qzeros,
                                void *out, int dt, bool out_f32, int N, int K, int g,
                                hipStream_t stream)
{
    const int64_t total = (int64_t)N * (K / 8);
    const int grid = (int)((total + 255) / 256);
    const uint16_t *sc = static_cast<const uint16_t *>(scales);
    if (dt == DT_F16) {
        if (out_f32)
            hipLaunchKernelGGL((w4a16_dequant_kernel<DT_F16, true>), dim3(grid), dim3(256), 0, stream,
                               qweight, sc, qzeros, out, N, K, g);
        else
            hipLaunchKernelGGL((w4a16_dequant_kernel<DT_F16, false>), dim3(grid), dim3(256), 0,
                               stream, qweight, sc, qzeros, out, N, K, g);
    } else {
        if (out_f32)
            hipLaunchKernelGGL((w4a16_dequant_kernel<DT_BF16, true>), dim3(grid), dim3(256), 0,
                               stream, qweight, sc, qzeros, out, N, K, g);
        else
            hipLaunchKernelGGL((w4a16_dequant_kernel<DT_BF16, false>), dim3(grid), dim3(256), 0,
                               stream, qweight, sc, qzeros, out, N, K, g);
    }
    return hipGetLastError();
}

hipError_t launch_mxfp4_dequant(const uint8_t *w_fp4, const uint8_t *w_scale, void *out, int N,
                                int K, hipStream_t stream)
{
    const int64_t total = (int64_t)N * (K / 8);
    const int grid = (int)((total + 255) / 256);
    hipLaunchKernelGGL(mxfp4_dequant_kernel, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t *>(w_fp4), w_scale,
                       static_cast<uint32_t *>(out), N, K);
    return hipGetLastError();
}

} // namespace wob
