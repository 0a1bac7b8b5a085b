// MoE stage 1, BF16 activations x MXFP4 weights, on gfx950 ("Add BF16xFP4 MoE
// GEMM stage1 kernel", summary and Technical Details).
//
// For every routed pair p = t * topk + s with expert e = topk_ids[t][s]:
//     y[p][n] = sum_k x[t][k] * e2m1(code_e(n, k)) * 2^(w_scale[e][n][k/32] - 127)
//
// Two kernels on the caller's stream:
//  1. Routing (one workgroup): histogram of the expert ids in LDS, prefix sums
//     of the rows and of the TM-row tiles per expert, a tile table
//     {expert, first sorted row, rows} and the pairs sorted by expert (order
//     inside an expert is arbitrary; every output row is computed the same
//     way wherever it sits in a tile).  Ids outside [0, E) form one extra
//     "expert" whose tiles write zero rows.
//  2. Grouped MFMA GEMM: the cooperative-tile pipeline of wob_tile.hpp with the
//     MXFP4 weight format.  A workgroup takes one (expert tile, weight-row
//     tile) pair; its activation rows are gathered from x by token, the FP4
//     words are expanded to bfloat16 with v_cvt_scalef32_pk_bf16_fp4 (one
//     conversion per byte, two elements each, the E8M0 byte placed in the
//     binary32 exponent as the scale), v_mfma_f32_32x32x16_bf16 multiplies,
//     and the epilogue scatters rows to their pair index.  Stores are guarded
//     by the tile's row count and by N, so a tile that overhangs the weight
//     rows (N not a multiple of the tile) never writes into neighbouring
//     cells: the failure the page's store guard fixes.
//
// Tiles: 384 weight rows x up to 160 activation rows for the pre-activation
// output, 256 x 256 for the fused activation (see moe_nb).  An expert's rows
// form one tile when they fit (the average expert of a 1024-token, 32-expert,
// top-4 batch has 128), so its weights stream from memory once; the tile
// multiplies only the 32-row blocks its row count needs.
#include "wob_internal.hpp"
#include "wob_tile.hpp"

namespace wob {
namespace {

// Weight blocks per wave: 3 (384-row weight tiles, up to 160 activation
// rows) for the pre-activation output, whose per-span fixed costs (barrier,
// scale loads, code copies) then spread over 1.5x the MFMAs of a 256-row tile
// at the ~128 rows of a typical expert; 2 (256 rows, up to 256 activation
// rows) for the fused gate / up activation, which pairs weight blocks.
template <bool ACT>
constexpr int moe_nb() { return ACT ? 2 : 3; }
template <bool ACT>
constexpr int moe_tm() { return TileGeo<moe_nb<ACT>()>::TM_MAX; } // rows per expert tile
template <bool ACT>
constexpr int moe_tn() { return TileGeo<moe_nb<ACT>()>::TN; } // weight rows per tile
constexpr int MOE_TM_MIN = moe_tm<false>() < moe_tm<true>() ? moe_tm<false>() : moe_tm<true>();
constexpr int ROUTE_THREADS = 1024;

struct MoeWs {
    int32_t *hdr;    // [0]: number of expert tiles
    int4 *tiles;     // {expert (E = invalid ids), first sorted row, rows, 0}
    int32_t *sorted; // pair indices grouped by expert
};

// Expert tiles of any launch: sum over experts (and the invalid-id bucket) of
// ceil(rows / TM) <= P / TM + E + 1, for the smaller TM.
size_t max_tiles(int64_t P, int64_t E) { return (size_t)(P / MOE_TM_MIN + E + 2); }

MoeWs carve(void *ws, int64_t P, int64_t E)
{
    uint8_t *b = static_cast<uint8_t *>(ws);
    MoeWs w;
    w.hdr = reinterpret_cast<int32_t *>(b);
    w.tiles = reinterpret_cast<int4 *>(b + 16);
    w.sorted = reinterpret_cast<int32_t *>(b + 16 + 16 * max_tiles(P, E));
    return w;
}

__device__ __forceinline__ int block_excl_scan(int v, int *wsum, int &total)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d)
            incl += o;
    }
    if (lane == 63)
        wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < ROUTE_THREADS / 64; ++w) {
        const int s = wsum[w];
        if (w < wave)
            before += s;
        total += s;
    }
    __syncthreads();
    return before + incl - v;
}

__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(const int32_t *__restrict__ ids,
                                                                  int P, int E, int tm, int32_t *hdr,
                                                                  int4 *tiles, int32_t *sorted)
{
    extern __shared__ int lds_i[];
    int *cnt = lds_i;             // [E + 1]
    int *off = cnt + (E + 1);     // [E + 1]
    int *toff = off + (E + 1);    // [E + 1]
    int *wsum = toff + (E + 1);   // [16]
    const int tid = threadIdx.x;

    for (int e = tid; e <= E; e += ROUTE_THREADS)
        cnt[e] = 0;
    __syncthreads();
    for (int i = tid; i < P; i += ROUTE_THREADS) {
        int e = ids[i];
        if ((unsigned)e >= (unsigned)E)
            e = E;
        atomicAdd(&cnt[e], 1);
    }
    __syncthreads();

    // Exclusive prefix sums of rows and of tiles over the E + 1 buckets; each
    // thread owns a run of consecutive buckets.
    const int per = (E + 1 + ROUTE_THREADS - 1) / ROUTE_THREADS;
    const int e0 = min(tid * per, E + 1), e1 = min(e0 + per, E + 1);
    int srows = 0, stiles = 0;
    for (int e = e0; e < e1; ++e) {
        srows += cnt[e];
        stiles += (cnt[e] + tm - 1) / tm;
    }
    int total_rows, total_tiles;
    int rb = block_excl_scan(srows, wsum, total_rows);
    int tb = block_excl_scan(stiles, wsum, total_tiles);
    for (int e = e0; e < e1; ++e) {
        off[e] = rb;
        toff[e] = tb;
        rb += cnt[e];
        tb += (cnt[e] + tm - 1) / tm;
    }
    if (tid == 0)
        hdr[0] = total_tiles;
    __syncthreads();

    for (int e = tid; e <= E; e += ROUTE_THREADS) {
        const int c = cnt[e];
        for (int j = 0; j * tm < c; ++j)
            tiles[toff[e] + j] = int4{e, off[e] + j * tm, min(tm, c - j * tm), 0};
    }
    __syncthreads();
    for (int e = tid; e <= E; e += ROUTE_THREADS)
        cnt[e] = 0; // reused as the per-bucket cursor
    __syncthreads();
    for (int i = tid; i < P; i += ROUTE_THREADS) {
        int e = ids[i];
        if ((unsigned)e >= (unsigned)E)
            e = E;
        sorted[off[e] + atomicAdd(&cnt[e], 1)] = i;
    }
}

// Gathered activation rows of one expert tile: row r is sorted pair
// sorted[first + r], token pair / topk.  Offsets of this lane's DMA rows are
// kept in registers for the whole tile.
template <int MB>
struct GatherRows {
    uint32_t xo[2 * MB];
    const int32_t *pairs; // sorted + first
    uint16_t *y;
    int N;
    __device__ __forceinline__ uint32_t off(int i) const { return xo[i]; }
    __device__ __forceinline__ uint16_t *row(int r) const { return y + (size_t)pairs[r] * N; }
};

// The tile with MB 32-row blocks; ACT: the paired gate/up layout and the
// fused silu(gate) * up store (I = N / 2 output columns), else the plain
// pre-activation store.
template <bool ACT, int MB>
__device__ __forceinline__ void moe_run(const FmtFP4<ACT, moe_nb<ACT>()> &fmt, const int32_t *pairs,
                                        int rows, int topk, const uint16_t *x, uint16_t *y, int K,
                                        int N, int n0, uint8_t *smem, const TileLane &tl)
{
    GatherRows<MB> g;
    g.pairs = pairs;
    g.y = y;
    g.N = ACT ? N / 2 : N;
#pragma unroll
    for (int i = 0; i < 2 * MB; ++i) {
        const int p = pairs[min(16 * i + tl.rl, rows - 1)];
        g.xo[i] = (uint32_t)(p / topk) * (uint32_t)K * 2u;
    }
    constexpr int NB = moe_nb<ACT>();
    float16_t acc[NB][MB];
    tile_mainloop<DT_BF16, NB, MB>(fmt, g, reinterpret_cast<const uint8_t *>(x), K, n0, N,
                                       smem, tl, acc);
    if constexpr (ACT)
        tile_store_silu_mul<DT_BF16, NB, MB>(acc, g, rows, n0, N / 2, tl, smem);
    else
        tile_store<DT_BF16, NB, MB>(acc, g, rows, n0, N, tl, smem);
}

template <bool ACT, int MB>
__device__ __forceinline__ void moe_dispatch(int mb, const FmtFP4<ACT, moe_nb<ACT>()> &fmt,
                                             const int32_t *pairs, int rows, int topk,
                                             const uint16_t *x, uint16_t *y, int K, int N, int n0,
                                             uint8_t *smem, const TileLane &tl)
{
    if constexpr (MB > 1) {
        if (mb < MB) {
            moe_dispatch<ACT, MB - 1>(mb, fmt, pairs, rows, topk, x, y, K, N, n0, smem, tl);
            return;
        }
    }
    moe_run<ACT, MB>(fmt, pairs, rows, topk, x, y, K, N, n0, smem, tl);
}

struct ZeroRows {
    const int32_t *pairs;
    uint16_t *y;
    int N;
    __device__ __forceinline__ uint16_t *row(int r) const { return y + (size_t)pairs[r] * N; }
};

// One (expert tile, weight-row tile) pair per workgroup.  ACT: tiles of 256
// output columns (256 gate rows + the matching 256 up rows), else 512.
template <bool ACT>
__global__ __launch_bounds__(TL_THREADS, 1) void moe_gemm_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w_fp4,
    const uint8_t *__restrict__ w_scale, uint16_t *__restrict__ y, const int32_t *__restrict__ hdr,
    const int4 *__restrict__ tiles, const int32_t *__restrict__ sorted, int topk, int E, int N,
    int K, int n_nt)
{
    constexpr int NB = moe_nb<ACT>();
    constexpr int TW = ACT ? moe_tn<ACT>() / 2 : moe_tn<ACT>(); // output columns per tile
    extern __shared__ __align__(16) uint8_t smem[];
    const int t = xcd_tile(hdr[0] * n_nt);
    if (t < 0)
        return;
    const int i = t / n_nt;
    const int n0 = (t - i * n_nt) * TW;
    const int4 te = tiles[i];
    const int e = te.x, rows = te.z;
    const int32_t *pairs = sorted + te.y;
    const int Nout = ACT ? N / 2 : N;
    if (e >= E) {
        tile_store_zero<TW>(ZeroRows{pairs, y, Nout}, rows, n0, Nout);
        return;
    }
    const TileLane tl;
    const FmtFP4<ACT, NB> fmt(w_fp4 + (size_t)e * N * (K >> 1),
                                  w_scale + (size_t)e * N * (K >> 5), N, K, n0, tl);
    moe_dispatch<ACT, TileGeo<NB>::MB_MAX>((rows + 31) >> 5, fmt, pairs, rows, topk, x, y, K,
                                               N, n0, smem, tl);
}

template <bool ACT>
hipError_t launch_gemm(const void *x, const uint8_t *w_fp4, const uint8_t *w_scale, void *y,
                       const MoeWs &w, int64_t P, int topk, int E, int N, int K,
                       hipStream_t stream)
{
    constexpr int NB = moe_nb<ACT>();
    constexpr int LDS = TileGeo<NB>::lds_bytes(TileGeo<NB>::MB_MAX);
    static_assert(LDS <= 160 * 1024, "tile fits the LDS");
    auto kern = moe_gemm_kernel<ACT>;
    static hipError_t attr = hipErrorNotReady;
    if (attr != hipSuccess)
        attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (attr != hipSuccess)
        return attr;
    const int tw = ACT ? moe_tn<ACT>() / 2 : moe_tn<ACT>();
    const int nout = ACT ? N / 2 : N;
    const int n_nt = (nout + tw - 1) / tw;
    const int64_t grid = 8 * (((int64_t)max_tiles(P, E) * n_nt + 7) / 8);
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(TL_THREADS), (size_t)LDS, stream,
                       static_cast<const uint16_t *>(x), w_fp4, w_scale, static_cast<uint16_t *>(y),
                       w.hdr, w.tiles, w.sorted, topk, E, N, K, n_nt);
    return hipGetLastError();
}

} // namespace

size_t moe_workspace_bytes(int64_t T, int64_t topk, int64_t E)
{
    const int64_t P = T * topk;
    return 16 + 16 * max_tiles(P, E) + 4 * (size_t)P;
}

hipError_t launch_mxfp4_moe(const void *x, const int32_t *ids, const uint8_t *w_fp4,
                            const uint8_t *w_scale, void *y, int T, int topk, int E, int N, int K,
                            int act, void *workspace, hipStream_t stream)
{
    const int64_t P = (int64_t)T * topk;
    const MoeWs w = carve(workspace, P, E);
    const size_t route_lds = (size_t)(3 * (E + 1) + ROUTE_THREADS / 64) * sizeof(int);
    const int tm = act ? moe_tm<true>() : moe_tm<false>();
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(ROUTE_THREADS), route_lds, stream, ids,
                       (int)P, E, tm, w.hdr, w.tiles, w.sorted);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    return act ? launch_gemm<true>(x, w_fp4, w_scale, y, w, P, topk, E, N, K, stream)
               : launch_gemm<false>(x, w_fp4, w_scale, y, w, P, topk, E, N, K, stream);
}

} // namespace wob
