// C-ABI layer: argument validation, architecture gate and kernel dispatch for
// the entry points declared in include/weight_only_bit.h.  Every check runs
// before any device call, so a non-OK status means nothing was enqueued.
#include "weight_only_bit.h"
#include "wob_device.hpp"
#include "wob_internal.hpp"

#include <limits.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_last_error[0] = 0;
    return WOB_OK;
}

// Per-device cache of the architecture check: 0 unknown, 1 gfx950, 2 other
// (atomic: calls may come from several host threads).
std::atomic<int> g_arch[64];

int arch_gate()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(WOB_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64)
        return fail(WOB_UNSUPPORTED, "device ordinal %d out of range", dev);
    int arch = g_arch[dev].load(std::memory_order_relaxed);
    if (arch == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(WOB_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        arch = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch[dev].store(arch, std::memory_order_relaxed);
    }
    if (arch != 1)
        return fail(WOB_UNSUPPORTED, "device %d is not gfx950", dev);
    return WOB_OK;
}

int launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(WOB_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared W4A16 operand checks.  M may be 0 (no-op) for the dense form.
int check_w4(const void *x, int x_dtype, const int32_t *qweight, const void *scales,
             int scales_dtype, const void *qzeros, int zeros_dtype, const void *y, int64_t M,
             int64_t N, int64_t K, int64_t g)
{
    if (x_dtype != WOB_F16 && x_dtype != WOB_BF16)
        return fail(WOB_DTYPE, "x dtype tag %d is not F16 or BF16", x_dtype);
    if (scales_dtype != x_dtype)
        return fail(WOB_DTYPE, "scales dtype tag %d differs from x dtype tag %d", scales_dtype,
                    x_dtype);
    if (qzeros && zeros_dtype != WOB_U4X8_I32)
        return fail(WOB_DTYPE,
                    "zero-points must be packed 4-bit (U4X8_I32); dtype tag %d is refused",
                    zeros_dtype);
    if (M < 0 || N < 0 || K < 32)
        return fail(WOB_INVALID_ARG, "bad shape M=%lld N=%lld K=%lld", (long long)M, (long long)N,
                    (long long)K);
    if (g != 32 && g != 64 && g != 128)
        return fail(WOB_UNSUPPORTED, "group size %lld is not 32, 64 or 128", (long long)g);
    if (K % g != 0 || K % 32 != 0)
        return fail(WOB_INVALID_ARG, "K=%lld is not a multiple of the group size %lld and of 32",
                    (long long)K, (long long)g);
    if (N % 8 != 0)
        return fail(WOB_INVALID_ARG, "N=%lld is not a multiple of 8", (long long)N);
    // 32-bit in-kernel offsets into one matrix of packed codes (N*K/2 bytes)
    if (M > INT_MAX / 2 || N > INT_MAX / 2 || K > INT_MAX / 2 || N * (K / 2) > (int64_t)UINT32_MAX)
        return fail(WOB_INVALID_ARG, "shape too large");
    if (M == 0 || N == 0)
        return WOB_OK;
    if (!x || !qweight || !scales || !y)
        return fail(WOB_INVALID_ARG, "null operand pointer");
    if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y) ||
        (qzeros && !aligned16(qzeros)))
        return fail(WOB_INVALID_ARG, "operand pointers must be 16-byte aligned");
    return WOB_OK;
}

// The tile kernels address a tile's activation rows with 32-bit byte offsets
// from the tile's first row: up to 2 K (rows - 1) plus a row's last 16 bytes,
// rows <= 256.  Refuse shapes whose offsets would not fit.
int check_tile_offsets(int64_t M, int64_t K)
{
    const int64_t rows = M < 256 ? M : 256;
    if (rows > 0 && 2 * K * rows > (int64_t)UINT32_MAX)
        return fail(WOB_INVALID_ARG,
                    "K=%lld too long for the tiled path (2*K*min(M,256) must stay below 2^32)",
                    (long long)K);
    return WOB_OK;
}

wob::W4Args make_args(const void *x, int dt, const int32_t *qweight, const void *scales,
                      const void *qzeros, void *y, int64_t M, int64_t N, int64_t K, int64_t g)
{
    wob::W4Args a;
    a.x = x;
    a.qweight = reinterpret_cast<const uint32_t *>(qweight);
    a.scales = scales;
    a.qzeros = static_cast<const uint32_t *>(qzeros);
    a.y = y;
    a.dt = dt == WOB_F16 ? wob::DT_F16 : wob::DT_BF16;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.g = (int)g;
    return a;
}

} // namespace

namespace wob {

DevTopo device_topology()
{
    static std::atomic<uint64_t> cache[64]; // cus << 32 | xcds, 0 = not queried
    constexpr DevTopo fallback{256, 8};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fallback;
    uint64_t v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, xcds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
            cus <= 0 || xcds <= 0)
            return fallback;
        v = ((uint64_t)cus << 32) | (uint32_t)xcds;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return DevTopo{(int)(v >> 32), (int)(uint32_t)v};
}

} // namespace wob

extern "C" {

const char *wob_status_str(int status)
{
    switch (status) {
    case WOB_OK: return "ok";
    case WOB_INVALID_ARG: return "invalid argument";
    case WOB_DTYPE: return "unsupported dtype for this operand";
    case WOB_UNSUPPORTED: return "unsupported device or parameter";
    case WOB_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *wob_last_error(void) { return g_last_error; }

int wob_device_check(void)
{
    int s = arch_gate();
    return s == WOB_OK ? ok() : s;
}

int w4a16_gemm_ex(const void *x, int x_dtype, const int32_t *qweight, const void *scales,
                  int scales_dtype, const void *qzeros, int zeros_dtype, void *y, int64_t M,
                  int64_t N, int64_t K, int64_t group_size, int path, void *stream)
{
    int s = check_w4(x, x_dtype, qweight, scales, scales_dtype, qzeros, zeros_dtype, y, M, N, K,
                     group_size);
    if (s != WOB_OK)
        return s;
    if (path != WOB_PATH_AUTO && path != WOB_PATH_SKINNY && path != WOB_PATH_TILED)
        return fail(WOB_INVALID_ARG, "unknown path %d", path);
    if (path == WOB_PATH_SKINNY && !wob::skinny_fits((int)(M ? M : 1), (int)(N ? N : 8), (int)K, (int)group_size))
        return fail(WOB_INVALID_ARG, "skinny path needs M <= 8 and M*K small enough for LDS");
    if (M == 0 || N == 0)
        return ok();
    const bool skinny = path == WOB_PATH_SKINNY ||
                        (path == WOB_PATH_AUTO &&
                         wob::skinny_fits((int)M, (int)N, (int)K, (int)group_size));
    if (!skinny && (s = check_tile_offsets(M, K)) != WOB_OK)
        return s;
    s = arch_gate();
    if (s != WOB_OK)
        return s;
    wob::W4Args a = make_args(x, x_dtype, qweight, scales, qzeros, y, M, N, K, group_size);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (skinny)
        return launched(wob::launch_w4a16_skinny(a, st), "w4a16 skinny");
    return launched(wob::launch_w4a16_tiled(a, st), "w4a16 tiled");
}

int w4a16_gemm(const void *x, int x_dtype, const int32_t *qweight, const void *scales,
               int scales_dtype, const void *qzeros, int zeros_dtype, void *y, int64_t M,
               int64_t N, int64_t K, int64_t group_size, void *stream)
{
    return w4a16_gemm_ex(x, x_dtype, qweight, scales, scales_dtype, qzeros, zeros_dtype, y, M, N,
                         K, group_size, WOB_PATH_AUTO, stream);
}

int w4a16_gemm_grouped(const void *x, int x_dtype, const int64_t *m_offsets, int64_t num_groups,
                       int64_t total_M, const int32_t *qweight, const void *scales,
                       int scales_dtype, const void *qzeros, int zeros_dtype, void *y, int64_t N,
                       int64_t K, int64_t group_size, void *stream)
{
    int s = check_w4(x, x_dtype, qweight, scales, scales_dtype, qzeros, zeros_dtype, y, total_M,
                     N, K, group_size);
    if (s != WOB_OK)
        return s;
    if (num_groups < 0 || num_groups > 65535)
        return fail(WOB_INVALID_ARG, "num_groups=%lld outside [0, 65535]", (long long)num_groups);
    if (total_M == 0 || N == 0 || num_groups == 0)
        return ok();
    if (!m_offsets || !aligned16(m_offsets))
        return fail(WOB_INVALID_ARG, "m_offsets must be a 16-byte aligned device pointer");
    if ((s = check_tile_offsets(total_M, K)) != WOB_OK)
        return s;
    s = arch_gate();
    if (s != WOB_OK)
        return s;
    wob::W4Args a = make_args(x, x_dtype, qweight, scales, qzeros, y, total_M, N, K, group_size);
    return launched(wob::launch_w4a16_grouped(a, m_offsets, (int)num_groups,
                                              static_cast<hipStream_t>(stream)),
                    "w4a16 grouped");
}

size_t mxfp4_moe_gemm_workspace_size(int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K)
{
    // The routing scratch depends on the pair count and the experts only.
    if (T < 0 || topk < 1 || E < 1 || N < 0 || K < 0 || T > INT_MAX / 64 || topk > 64 ||
        E > 4096)
        return 0;
    return wob::moe_workspace_bytes(T, topk, E);
}

namespace {

// MoE argument checks shared by both MoE entry points (everything but the
// workspace).  Sets *noop when the problem is empty.
int check_moe(const void *x, const int32_t *topk_ids, const uint8_t *w_fp4, const uint8_t *w_scale,
              const void *y, int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K, int act,
              bool *noop)
{
    *noop = false;
    if (act != WOB_ACT_NONE && act != WOB_ACT_SILU_MUL)
        return fail(WOB_INVALID_ARG, "unknown activation %d", act);
    if (T < 0 || topk < 1 || E < 1 || N < 0 || K < 32)
        return fail(WOB_INVALID_ARG, "bad shape T=%lld topk=%lld E=%lld N=%lld K=%lld",
                    (long long)T, (long long)topk, (long long)E, (long long)N, (long long)K);
    if (K % 64 != 0 || N % 16 != 0)
        return fail(WOB_INVALID_ARG, "need K %% 64 == 0 and N %% 16 == 0 (K=%lld N=%lld)",
                    (long long)K, (long long)N);
    if (act == WOB_ACT_SILU_MUL && N % 32 != 0)
        return fail(WOB_INVALID_ARG, "the silu(gate) * up activation needs N %% 32 == 0 (N=%lld)",
                    (long long)N);
    // 32-bit in-kernel offsets: x rows (T*K*2 bytes), one expert's codes
    // (N*K/2 bytes) and the routed pair count T*topk.
    if (T > INT_MAX / 64 || topk > 64 || E > 4096 || N > INT_MAX / 2 || K > INT_MAX / 2 ||
        T * K * 2 > (int64_t)UINT32_MAX || N * (K / 2) > (int64_t)UINT32_MAX ||
        E * N * (K / 2) > ((int64_t)1 << 40))
        return fail(WOB_INVALID_ARG, "shape too large");
    if (T == 0 || N == 0) {
        *noop = true;
        return WOB_OK;
    }
    if (!x || !topk_ids || !w_fp4 || !w_scale || !y)
        return fail(WOB_INVALID_ARG, "null operand pointer");
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(w_fp4) || !aligned16(w_scale) ||
        !aligned16(y))
        return fail(WOB_INVALID_ARG, "operand pointers must be 16-byte aligned");
    return WOB_OK;
}

} // namespace

namespace {

int moe_gemm_impl(const void *x, const int32_t *topk_ids, const uint8_t *w_fp4,
                  const uint8_t *w_scale, void *y, int64_t T, int64_t topk, int64_t E, int64_t N,
                  int64_t K, int act, int tile_m, void *workspace, size_t workspace_bytes,
                  void *stream)
{
    if (tile_m != 16 && tile_m != 32)
        return fail(WOB_INVALID_ARG, "tile_m %d is not 16 or 32", tile_m);
    bool noop;
    int s = check_moe(x, topk_ids, w_fp4, w_scale, y, T, topk, E, N, K, act, &noop);
    if (s != WOB_OK)
        return s;
    if (noop)
        return ok();
    const size_t need = wob::moe_workspace_bytes(T, topk, E);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need)
        return fail(WOB_INVALID_ARG, "workspace needs %zu bytes, 16-byte aligned (got %zu)", need,
                    workspace_bytes);
    s = arch_gate();
    if (s != WOB_OK)
        return s;
    return launched(wob::launch_mxfp4_moe(x, topk_ids, w_fp4, w_scale, y, (int)T, (int)topk,
                                          (int)E, (int)N, (int)K, act, tile_m, workspace,
                                          static_cast<hipStream_t>(stream)),
                    "mxfp4 moe");
}

} // namespace

int mxfp4_moe_gemm(const void *x, const int32_t *topk_ids, const uint8_t *w_fp4,
                   const uint8_t *w_scale, void *y, int64_t T, int64_t topk, int64_t E, int64_t N,
                   int64_t K, int act, void *workspace, size_t workspace_bytes, void *stream)
{
    return moe_gemm_impl(x, topk_ids, w_fp4, w_scale, y, T, topk, E, N, K, act, 32, workspace,
                         workspace_bytes, stream);
}

int mxfp4_moe_gemm_tile_m(const void *x, const int32_t *topk_ids, const uint8_t *w_fp4,
                          const uint8_t *w_scale, void *y, int64_t T, int64_t topk, int64_t E,
                          int64_t N, int64_t K, int act, int tile_m, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    return moe_gemm_impl(x, topk_ids, w_fp4, w_scale, y, T, topk, E, N, K, act, tile_m,
                         workspace, workspace_bytes, stream);
}

size_t mxfp4_moe_stage2_workspace_size(int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I)
{
    if (T < 0 || topk < 1 || E < 1 || H < 0 || I < 0 || T > INT_MAX / 64 || topk > 64 ||
        E > 4096 || H > INT_MAX / 2)
        return 0;
    return wob::moe_stage2_workspace_bytes(T, topk, E, H);
}

int mxfp4_moe_stage2(const void *a, const int32_t *topk_ids, const float *topk_weights,
                     const uint8_t *w2_fp4, const uint8_t *w2_scale, void *y, int64_t T,
                     int64_t topk, int64_t E, int64_t H, int64_t I, void *workspace,
                     size_t workspace_bytes, void *stream)
{
    if (T < 0 || topk < 1 || E < 1 || H < 0 || I < 64)
        return fail(WOB_INVALID_ARG, "bad shape T=%lld topk=%lld E=%lld H=%lld I=%lld",
                    (long long)T, (long long)topk, (long long)E, (long long)H, (long long)I);
    if (I % 64 != 0 || H % 16 != 0)
        return fail(WOB_INVALID_ARG, "need I %% 64 == 0 and H %% 16 == 0 (I=%lld H=%lld)",
                    (long long)I, (long long)H);
    // 32-bit in-kernel offsets: gathered rows of a (T*topk*I*2 bytes) and one
    // expert's codes (H*I/2 bytes).
    if (T > INT_MAX / 64 || topk > 64 || E > 4096 || H > INT_MAX / 2 || I > INT_MAX / 2 ||
        T * topk * I * 2 > (int64_t)UINT32_MAX || H * (I / 2) > (int64_t)UINT32_MAX ||
        E * H * (I / 2) > ((int64_t)1 << 40))
        return fail(WOB_INVALID_ARG, "shape too large");
    if (T == 0 || H == 0)
        return ok();
    if (!a || !topk_ids || !topk_weights || !w2_fp4 || !w2_scale || !y)
        return fail(WOB_INVALID_ARG, "null operand pointer");
    if (!aligned16(a) || !aligned16(topk_ids) || !aligned16(topk_weights) || !aligned16(w2_fp4) ||
        !aligned16(w2_scale) || !aligned16(y))
        return fail(WOB_INVALID_ARG, "operand pointers must be 16-byte aligned");
    const size_t need = wob::moe_stage2_workspace_bytes(T, topk, E, H);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need)
        return fail(WOB_INVALID_ARG, "workspace needs %zu bytes, 16-byte aligned (got %zu)", need,
                    workspace_bytes);
    int s = arch_gate();
    if (s != WOB_OK)
        return s;
    return launched(wob::launch_mxfp4_moe_stage2(a, topk_ids, topk_weights, w2_fp4, w2_scale, y,
                                                 (int)T, (int)topk, (int)E, (int)H, (int)I,
                                                 workspace, static_cast<hipStream_t>(stream)),
                    "mxfp4 moe stage 2");
}

int mxfp4_moe_gemm_noalloc(const void *x, const int32_t *topk_ids, const uint8_t *w_fp4,
                           const uint8_t *w_scale, void *y, int64_t T, int64_t topk, int64_t E,
                           int64_t N, int64_t K, int act, void *stream)
{
    bool noop;
    int s = check_moe(x, topk_ids, w_fp4, w_scale, y, T, topk, E, N, K, act, &noop);
    if (s != WOB_OK)
        return s;
    if (noop)
        return ok();
    const size_t need = wob::moe_workspace_bytes(T, topk, E);
    if (need > wob::moe_scratch_bytes())
        return fail(WOB_INVALID_ARG,
                    "routing scratch of %zu bytes (T*topk=%lld pairs, E=%lld) exceeds the "
                    "%zu-byte static scratch of the allocation-free entry point",
                    need, (long long)(T * topk), (long long)E, wob::moe_scratch_bytes());
    s = arch_gate();
    if (s != WOB_OK)
        return s;
    void *scratch = nullptr;
    const hipError_t e = wob::moe_scratch(&scratch);
    if (e != hipSuccess)
        return fail(WOB_HIP, "static scratch lookup: %s", hipGetErrorString(e));
    return launched(wob::launch_mxfp4_moe(x, topk_ids, w_fp4, w_scale, y, (int)T, (int)topk,
                                          (int)E, (int)N, (int)K, act, 32, scratch,
                                          static_cast<hipStream_t>(stream)),
                    "mxfp4 moe (static scratch)");
}

int w4a16_dequant(const int32_t *qweight, const void *scales, int scales_dtype,
                  const void *qzeros, int zeros_dtype, void *out, int out_dtype, int64_t N,
                  int64_t K, int64_t group_size, void *stream)
{
    // x is not an operand of the probe; validate the weights as for a GEMM.
    int s = check_w4(qweight, scales_dtype, qweight, scales, scales_dtype, qzeros, zeros_dtype,
                     out, 1, N, K, group_size);
    if (s != WOB_OK)
        return s;
    if (out_dtype != WOB_F32 && out_dtype != scales_dtype)
        return fail(WOB_DTYPE, "probe output dtype %d must be F32 or the scales dtype", out_dtype);
    if (N == 0)
        return ok();
    s = arch_gate();
    if (s != WOB_OK)
        return s;
    return launched(wob::launch_w4a16_dequant(reinterpret_cast<const uint32_t *>(qweight), scales,
                                              static_cast<const uint32_t *>(qzeros), out,
                                              scales_dtype == WOB_F16 ? wob::DT_F16 : wob::DT_BF16,
                                              out_dtype == WOB_F32, (int)N, (int)K,
                                              (int)group_size, static_cast<hipStream_t>(stream)),
                    "w4a16 dequant probe");
}

int mxfp4_dequant(const uint8_t *w_fp4, const uint8_t *w_scale, void *out, int64_t N, int64_t K,
                  void *stream)
{
    if (N < 0 || K < 32 || K % 32 != 0 || N > INT_MAX / 2 || K > INT_MAX / 2)
        return fail(WOB_INVALID_ARG, "bad shape N=%lld K=%lld", (long long)N, (long long)K);
    if (N == 0)
        return ok();
    if (!w_fp4 || !w_scale || !out)
        return fail(WOB_INVALID_ARG, "null operand pointer");
    if (!aligned16(w_fp4) || !aligned16(out))
        return fail(WOB_INVALID_ARG, "operand pointers must be 16-byte aligned");
    int s = arch_gate();
    if (s != WOB_OK)
        return s;
    return launched(wob::launch_mxfp4_dequant(w_fp4, w_scale, out, (int)N, (int)K,
                                              static_cast<hipStream_t>(stream)),
                    "mxfp4 dequant probe");
}

int wob_stream_read(const void *buf, size_t bytes, void *sink, void *stream)
{
    if (bytes % 16 != 0)
        return fail(WOB_INVALID_ARG, "bytes %zu is not a multiple of 16", bytes);
    if (bytes == 0)
        return ok();
    if (!buf || !sink)
        return fail(WOB_INVALID_ARG, "null pointer");
    if (!aligned16(buf) || !aligned16(sink))
        return fail(WOB_INVALID_ARG, "pointers must be 16-byte aligned");
    int s = arch_gate();
    if (s != WOB_OK)
        return s;
    return launched(wob::launch_stream_read(buf, bytes, static_cast<uint32_t *>(sink),
                                            static_cast<hipStream_t>(stream)),
                    "stream read");
}

} // extern "C"
