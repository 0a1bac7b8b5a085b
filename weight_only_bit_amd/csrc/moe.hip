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
//     binary32 exponent as the scale), v_mfma_f32_32x32x16_bf16 (or, with
//     a 16-row tile height, v_mfma_f32_16x16x32_bf16) multiplies, and the
//     epilogue scatters rows to their pair index.  Stores are guarded
//     by the tile's row count and by N, so a tile that overhangs the weight
//     rows (N not a multiple of the tile) never writes into neighbouring
//     cells: the failure the page's store guard fixes.
//
// Tiles: 384 weight rows x up to 160 activation rows for the pre-activation
// output, 256 x up to 224 (160 with 16-row blocks) for the fused activation
// (see moe_nb).  An expert's rows form one tile when they fit (the average
// expert of a 1024-token, 32-expert, top-4 batch has 128), so its weights
// stream from memory once; the tile multiplies only the blocks its row count
// needs, so an expert's rows are padded to a multiple of the tile height
// (the MFMA block height): 32 rows by default, 16 on request.  Measured on
// MI355X, the 16-row form is the slower one at every batch size tried (16 to
// 1024 tokens: 4 to 16 %), although it pads less: its accumulators are four
// times as many 4-register blocks, which the compiler shuffles between the
// two register files inside the K loop.
#include "wob_internal.hpp"
#include "wob_tile.hpp"

#include <algorithm>

// Static routing scratch of the allocation-free entry point (see
// moe_scratch below); file scope, one copy per device.
static constexpr size_t MOE_SCRATCH_BYTES = (size_t)1 << 20;
static __device__ __align__(256) uint8_t moe_static_scratch[MOE_SCRATCH_BYTES];

namespace wob {
namespace {

// Weight blocks per wave (tile height BR = MFMA block rows): 384-row weight
// tiles (3 blocks of 32 or 6 of 16) for the pre-activation output, whose
// per-span fixed costs (barrier, scale loads, code copies) then spread over
// 1.5x the MFMAs of a 256-row tile at the ~128 rows of a typical expert;
// 256 rows (128 gate rows and the matching 128 up rows) for the fused
// gate / up activation, which pairs weight blocks.
template <bool ACT, int BR>
constexpr int moe_nb() { return (ACT ? 256 : 384) / (4 * BR); }
template <bool ACT, int BR>
using MoeGeo = TileGeo<moe_nb<ACT, BR>(), BR>;
// Activation blocks per expert tile, at most: 160 rows (the 240 accumulator
// registers of the 384-row tile); the fused-activation tile stops at 224
// rows with 32-row blocks (its 256-row form spilled a register) and at 160
// rows with 16-row blocks (more spilled); a larger expert takes two tiles.
template <bool ACT, int BR>
constexpr int moe_mb_max() { return (ACT && BR == 32) ? 7 : 160 / BR; }
template <bool ACT, int BR>
constexpr int moe_tm() { return BR * moe_mb_max<ACT, BR>(); } // rows per expert tile
template <bool ACT, int BR>
constexpr int moe_tn() { return MoeGeo<ACT, BR>::TN; } // weight rows per tile
constexpr int MOE_TM_MIN = 160; // the smallest moe_tm of any variant
static_assert(moe_tm<false, 32>() >= MOE_TM_MIN && moe_tm<true, 32>() >= MOE_TM_MIN &&
                  moe_tm<false, 16>() >= MOE_TM_MIN && moe_tm<true, 16>() >= MOE_TM_MIN,
              "workspace bound");
constexpr int ROUTE_THREADS = 1024;
constexpr int ROUTE_IPT = 4; // ids per thread per batch (P = 4096 in one)

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

__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(const int32_t *__restrict__ ids,
                                                                  int P, int E, int tm, int32_t *hdr,
                                                                  int4 *tiles, int32_t *sorted)
{
    extern __shared__ int lds_i[];
    int *cnt = lds_i;             // [E + 1]
    int *off = cnt + (E + 1);     // [E + 1]
    int *toff = off + (E + 1);    // [E + 1]
    const int tid = threadIdx.x;

    for (int e = tid; e <= E; e += ROUTE_THREADS)
        cnt[e] = 0;
    __syncthreads();
    // The ids are read ROUTE_IPT per thread at a time, all requested before
    // any is used (a loop of one load and one LDS atomic waited a full memory
    // round trip per id), and with P <= ROUTE_IPT x ROUTE_THREADS kept in
    // registers for the scatter below.
    auto bucket = [&](int e) { return (unsigned)e < (unsigned)E ? e : E; };
    int eb[ROUTE_IPT];
    for (int base = 0; base < P; base += ROUTE_IPT * ROUTE_THREADS) {
        int v[ROUTE_IPT];
#pragma unroll
        for (int b = 0; b < ROUTE_IPT; ++b) {
            const int i = base + b * ROUTE_THREADS + tid;
            v[b] = ids[min(i, P - 1)]; // unconditional (clamped): issued together
        }
#pragma unroll
        for (int b = 0; b < ROUTE_IPT; ++b) {
            eb[b] = bucket(v[b]);
            if (base + b * ROUTE_THREADS + tid < P)
                atomicAdd(&cnt[eb[b]], 1);
        }
    }
    __syncthreads();

    // Exclusive prefix sums of rows and of tiles over the E + 1 buckets, by
    // wave 0 alone: lane l owns a run of consecutive buckets, and one
    // wave-wide scan joins the runs (measured: two workgroup-wide scans, each
    // with two barriers and a serial pass over the 16 wave sums, took 1.8 us).
    if (tid < 64) {
        const int per = (E + 1 + 63) / 64;
        const int e0 = min(tid * per, E + 1), e1 = min(e0 + per, E + 1);
        int srows = 0, stiles = 0;
        for (int e = e0; e < e1; ++e) {
            srows += cnt[e];
            stiles += (cnt[e] + tm - 1) / tm;
        }
        int ir = srows, it = stiles;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int orows = __shfl_up(ir, d), otiles = __shfl_up(it, d);
            if (tid >= d) {
                ir += orows;
                it += otiles;
            }
        }
        int rb = ir - srows, tb = it - stiles;
        for (int e = e0; e < e1; ++e) {
            off[e] = rb;
            toff[e] = tb;
            rb += cnt[e];
            tb += (cnt[e] + tm - 1) / tm;
        }
        if (tid == 63)
            hdr[0] = it;
    }
    __syncthreads();

    // Tile table; each bucket's count, read here by its one thread, becomes
    // that bucket's cursor for the scatter.
    for (int e = tid; e <= E; e += ROUTE_THREADS) {
        const int c = cnt[e];
        for (int j = 0; j * tm < c; ++j)
            tiles[toff[e] + j] = int4{e, off[e] + j * tm, min(tm, c - j * tm), 0};
        cnt[e] = 0;
    }
    __syncthreads();
    if (P <= ROUTE_IPT * ROUTE_THREADS) {
#pragma unroll
        for (int b = 0; b < ROUTE_IPT; ++b) {
            const int i = b * ROUTE_THREADS + tid;
            if (i < P)
                sorted[off[eb[b]] + atomicAdd(&cnt[eb[b]], 1)] = i;
        }
        return;
    }
    for (int base = 0; base < P; base += ROUTE_IPT * ROUTE_THREADS) {
        int v[ROUTE_IPT];
#pragma unroll
        for (int b = 0; b < ROUTE_IPT; ++b) {
            const int i = base + b * ROUTE_THREADS + tid;
            v[b] = ids[min(i, P - 1)]; // unconditional (clamped): issued together
        }
#pragma unroll
        for (int b = 0; b < ROUTE_IPT; ++b) {
            const int i = base + b * ROUTE_THREADS + tid;
            if (i < P) {
                const int e = bucket(v[b]);
                sorted[off[e] + atomicAdd(&cnt[e], 1)] = i;
            }
        }
    }
}

// Gathered activation rows of one expert tile: row r is sorted pair
// sorted[first + r], token pair / topk.  Offsets of this lane's DMA rows
// (NX = rows / 16 copies) are kept in registers for the whole tile.
template <int NX>
struct GatherRows {
    uint32_t xo[NX];
    const int32_t *pairs; // sorted + first
    uint16_t *base;       // y
    int ld;               // output row length
    __device__ __forceinline__ uint32_t off(int i) const { return xo[i]; }
    __device__ __forceinline__ uint32_t index(int r) const { return (uint32_t)pairs[r]; }
};

// The tile with MB 32-row blocks; ACT: the paired gate/up layout and the
// fused silu(gate) * up store (I = N / 2 output columns), else the plain
// pre-activation store.
template <bool ACT, int BR, int MB>
__device__ __forceinline__ void moe_run(const FmtFP4<ACT, moe_nb<ACT, BR>(), BR> &fmt,
                                        const int32_t *pairs, int rows, int topk,
                                        const uint16_t *x, uint16_t *y, int K, int N, int n0,
                                        uint8_t *smem, const TileLane<BR> &tl)
{
    constexpr int NX = BR * MB / 16;
    GatherRows<NX> g;
    g.pairs = pairs;
    g.base = y;
    g.ld = ACT ? N / 2 : N;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int p = pairs[min(16 * i + tl.rl, rows - 1)];
        g.xo[i] = (uint32_t)(p / topk) * (uint32_t)K * 2u;
    }
    constexpr int NB = moe_nb<ACT, BR>();
    typename AccT<BR>::type acc[NB][MB];
    tile_mainloop<DT_BF16, NB, MB, BR>(fmt, g, reinterpret_cast<const uint8_t *>(x), K, n0, N,
                                       smem, tl, acc);
    if constexpr (ACT)
        tile_store_silu_mul<DT_BF16, NB, MB, BR>(acc, g, rows, n0, N / 2, tl, smem);
    else
        tile_store<DT_BF16, NB, MB, BR>(acc, g, rows, n0, N, tl, smem);
}

template <bool ACT, int BR, int MB>
__device__ __forceinline__ void moe_dispatch(int mb, const FmtFP4<ACT, moe_nb<ACT, BR>(), BR> &fmt,
                                             const int32_t *pairs, int rows, int topk,
                                             const uint16_t *x, uint16_t *y, int K, int N, int n0,
                                             uint8_t *smem, const TileLane<BR> &tl)
{
    if constexpr (MB > 1) {
        if (mb < MB) {
            moe_dispatch<ACT, BR, MB - 1>(mb, fmt, pairs, rows, topk, x, y, K, N, n0, smem, tl);
            return;
        }
    }
    moe_run<ACT, BR, MB>(fmt, pairs, rows, topk, x, y, K, N, n0, smem, tl);
}

struct ZeroRows {
    const int32_t *pairs;
    uint16_t *y;
    int N;
    __device__ __forceinline__ uint16_t *row(int r) const { return y + (size_t)pairs[r] * N; }
};

// One (expert tile, weight-row tile) pair per workgroup.  ACT: tiles of 128
// output columns (128 gate rows + the matching 128 up rows), else 384.
template <bool ACT, int BR>
__global__ __launch_bounds__(TL_THREADS, 1) void moe_gemm_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w_fp4,
    const uint8_t *__restrict__ w_scale, uint16_t *__restrict__ y, const int32_t *__restrict__ hdr,
    const int4 *__restrict__ tiles, const int32_t *__restrict__ sorted, int topk, int E, int N,
    int K, int n_nt, int nxcd)
{
    constexpr int NB = moe_nb<ACT, BR>();
    constexpr int TW = ACT ? moe_tn<ACT, BR>() / 2 : moe_tn<ACT, BR>(); // output columns per tile
    extern __shared__ __align__(16) uint8_t smem[];
    const int t = xcd_tile(hdr[0] * n_nt, nxcd);
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
    const TileLane<BR> tl;
    const FmtFP4<ACT, NB, BR> fmt(w_fp4 + (size_t)e * N * (K >> 1),
                                  w_scale + (size_t)e * N * (K >> 5), N, K, n0, tl);
    moe_dispatch<ACT, BR, moe_mb_max<ACT, BR>()>((rows + BR - 1) / BR, fmt, pairs, rows, topk, x,
                                                 y, K, N, n0, smem, tl);
}

// ---- Stage 2: down projection with the routing-weight combine ------------
//
// Reading (the pages define stage 1 only): for token t and slot s with
// expert e = ids[t][s] in [0, E),
//     pre[t*topk + s][h] = sum_i a[t][s][i] * w2_e[h][i]
//     y[t][h] = sum over valid s of w[t][s] * pre[t*topk + s][h]
// The GEMM is the stage-1 tile kernel with activation rows gathered by routed
// pair (row p of a [T*topk][I]) instead of by token, and an fp32 epilogue
// into `pre` (workspace).  A second kernel sums each token's slots in slot
// order, so the result does not depend on timing.

// A tile's rows of pre straight from the accumulators: the lane holds
// D[n = BR NB w + BR nb + 4 G g4 + 4 g + j][m = BR mb + nl] in register
// 4 g4 + j of block (nb, mb), i.e. four consecutive outputs of one row: one
// 16-byte store each.  Rows past the tile's count and columns past H are not
// written.
template <int NB, int MB, int BR>
__device__ __forceinline__ void tile_store_rows_f32(const typename AccT<BR>::type (&acc)[NB][MB],
                                                    float *pre, const int32_t *pairs, int rows,
                                                    int n0, int H, const TileLane<BR> &tl)
{
    using GEO = TileGeo<NB, BR>;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = BR * mb + tl.nl;
        if (r >= rows)
            continue;
        float *row = pre + (size_t)pairs[r] * H;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int g4 = 0; g4 < GEO::ACC / 4; ++g4) {
                const int n = n0 + BR * NB * tl.wave + BR * nb + 4 * GEO::G * g4 + 4 * tl.g;
                if (n < H) {
                    const auto &v = acc[nb][mb];
                    *reinterpret_cast<float4_t *>(row + n) =
                        float4_t{v[4 * g4 + 0], v[4 * g4 + 1], v[4 * g4 + 2], v[4 * g4 + 3]};
                }
            }
    }
}

// 384-row weight tiles of 32-row blocks, as stage 1 (measured on MI355X at
// H = 2880: faster than 320-row tiles, which split the width evenly but make
// 288 tiles for 32 experts, more than one round of the 256 compute units,
// and faster than 16-row blocks).
constexpr int MOE2_BR = 32;
constexpr int MOE2_NB = 3;
using Moe2Geo = TileGeo<MOE2_NB, MOE2_BR>;

template <int MB>
__device__ __forceinline__ void moe2_run(const FmtFP4<false, MOE2_NB, MOE2_BR> &fmt,
                                         const int32_t *pairs, int rows, const uint16_t *a,
                                         float *pre, int I, int H, int n0, uint8_t *smem,
                                         const TileLane<MOE2_BR> &tl)
{
    constexpr int NX = MOE2_BR * MB / 16;
    GatherRows<NX> g;
    g.pairs = pairs;
    g.base = nullptr;
    g.ld = 0;
#pragma unroll
    for (int i = 0; i < NX; ++i)
        g.xo[i] = (uint32_t)pairs[min(16 * i + tl.rl, rows - 1)] * (uint32_t)I * 2u;
    typename AccT<MOE2_BR>::type acc[MOE2_NB][MB];
    tile_mainloop<DT_BF16, MOE2_NB, MB, MOE2_BR>(fmt, g, reinterpret_cast<const uint8_t *>(a), I,
                                                 n0, H, smem, tl, acc);
    tile_store_rows_f32<MOE2_NB, MB, MOE2_BR>(acc, pre, pairs, rows, n0, H, tl);
}

template <int MB>
__device__ __forceinline__ void moe2_dispatch(int mb, const FmtFP4<false, MOE2_NB, MOE2_BR> &fmt,
                                              const int32_t *pairs, int rows, const uint16_t *a,
                                              float *pre, int I, int H, int n0, uint8_t *smem,
                                              const TileLane<MOE2_BR> &tl)
{
    if constexpr (MB > 1) {
        if (mb < MB) {
            moe2_dispatch<MB - 1>(mb, fmt, pairs, rows, a, pre, I, H, n0, smem, tl);
            return;
        }
    }
    moe2_run<MB>(fmt, pairs, rows, a, pre, I, H, n0, smem, tl);
}

// One (expert tile, weight-row tile) pair per workgroup, as in stage 1.
__global__ __launch_bounds__(TL_THREADS, 1) void moe_stage2_kernel(
    const uint16_t *__restrict__ a, const uint8_t *__restrict__ w_fp4,
    const uint8_t *__restrict__ w_scale, float *__restrict__ pre, const int32_t *__restrict__ hdr,
    const int4 *__restrict__ tiles, const int32_t *__restrict__ sorted, int E, int H, int I,
    int n_nt, int nxcd)
{
    constexpr int TW = Moe2Geo::TN;
    extern __shared__ __align__(16) uint8_t smem[];
    const int t = xcd_tile(hdr[0] * n_nt, nxcd);
    if (t < 0)
        return;
    const int i = t / n_nt;
    const int n0 = (t - i * n_nt) * TW;
    const int4 te = tiles[i];
    const int e = te.x, rows = te.z;
    if (e >= E)
        return; // ids outside [0, E): the combine skips these slots
    const TileLane<MOE2_BR> tl;
    const FmtFP4<false, MOE2_NB, MOE2_BR> fmt(w_fp4 + (size_t)e * H * (I >> 1),
                                              w_scale + (size_t)e * H * (I >> 5), H, I, n0, tl);
    moe2_dispatch<moe_mb_max<false, MOE2_BR>()>((rows + MOE2_BR - 1) / MOE2_BR, fmt,
                                                sorted + te.y, rows, a, pre, I, H, n0, smem, tl);
}

// y[t][h .. h+7] = sum over valid slots s (in order) of w[t][s] * pre[t*topk + s][h ..],
// rounded once to bfloat16.  One thread per 8 outputs (H % 16 == 0).
constexpr int CB_THREADS = 256;

__global__ __launch_bounds__(CB_THREADS) void moe_combine_kernel(
    const float *__restrict__ pre, const int32_t *__restrict__ ids, const float *__restrict__ w,
    uint16_t *__restrict__ y, int T, int topk, int E, int H)
{
    const int H8 = H >> 3;
    const int64_t idx = (int64_t)blockIdx.x * CB_THREADS + threadIdx.x;
    if (idx >= (int64_t)T * H8)
        return;
    const int t = (int)(idx / H8);
    const int c = (int)(idx - (int64_t)t * H8) * 8;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc[j] = 0.f;
    for (int s = 0; s < topk; ++s) {
        const int p = t * topk + s;
        if ((unsigned)ids[p] >= (unsigned)E)
            continue;
        const float ws = w[p];
        const float4_t *src = reinterpret_cast<const float4_t *>(pre + (size_t)p * H + c);
        const float4_t v0 = src[0], v1 = src[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[j] = fmaf(ws, v0[j], acc[j]);
            acc[4 + j] = fmaf(ws, v1[j], acc[4 + j]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = f32x2_to_act2<DT_BF16>(acc[2 * j], acc[2 * j + 1]);
    *reinterpret_cast<u32x4 *>(y + (size_t)t * H + c) = o;
}

// ---- Decode path: at most MG_TOKENS tokens --------------------------------
//
// With a handful of tokens every expert holds one or two routed rows, so the
// tile kernel would run a few dozen single-block workgroups, each streaming a
// whole weight tile on its own.  This kernel splits the weight rows finely
// instead (memory-bound, like the skinny W4A16 path): a workgroup takes one
// expert tile and MG_WAVES x 8 weight rows; wave lane (r, q) = (lane / 8,
// lane % 8) owns weight row r of the wave and the 16-byte code chunks
// q, q + 8, ... of it (32 E2M1 codes and one E8M0 scale byte each).  The
// tile's activation rows are gathered by token into LDS; each code word is
// expanded with v_cvt_scalef32_pk_bf16_fp4 (the same conversion as the tile
// kernel) and multiplied with v_dot2_f32_bf16 against the activation pairs
// (exact products, fp32 accumulation).  As soon as the expert is known the
// workgroup requests its rows' E8M0 scale bytes (a few coalesced 2-byte loads
// per thread, stored in LDS after the listing) and then the first MG_D code
// chunks of every lane; a lane's chunks stream through that ring of MG_D
// slots.  Measured on 4 tokens x top-4 of 32 experts (K 2880, N 5760): a
// scale byte loaded per chunk beside the codes cost about 15 % (a copy of
// the kernel without scale loads ran 26.8 against 31.4 us); staging them in
// LDS after the listing was slower (33.5), staging them ahead of the codes
// faster (30.4); with staged scales a ring of 3 chunks beat 6 and 12 (33.6,
// 33.4), and 8-wave workgroups matched 4-wave ones.  With the fused
// activation a wave's rows are 4 gate rows and the matching 4 up rows.
constexpr int MG_TOKENS = 8;  // decode path: T <= 8
constexpr int MG_WAVES = 4;
constexpr int MG_THREADS = 64 * MG_WAVES;
constexpr int MG_D = 3;       // chunk slots per lane in the load ring
constexpr int MG_LDS = 64 * 1024;
constexpr int MG_BATCH = 4;   // staging loads per thread in flight
// Scale units (2 bytes) per thread requested with the first code chunks:
// all of them for K <= 3072 (MG_ROWS rows x K / 64 units).
constexpr int MG_SB = 6;

template <bool ACT>
constexpr int mg_cols() { return ACT ? 4 * MG_WAVES : 8 * MG_WAVES; } // output columns per workgroup

// Weight rows per workgroup (8 per wave) and the bytes of their staged E8M0
// scales (K / 32 per row, padded to 16 bytes).
constexpr int MG_ROWS = 8 * MG_WAVES;
inline int mg_scale_bytes(int K) { return (MG_ROWS * (K >> 5) + 15) & ~15; }

// Activation rows per pass for this K: the largest power of two <= 8 whose
// rows fit the LDS budget beside the staged scales (0: K too long for this
// path).
int mg_rows(int K)
{
    int mr = 8;
    while (mr > 0 && mr * 2 * K + mg_scale_bytes(K) > MG_LDS)
        mr >>= 1;
    return mr;
}

// A lane's code chunk i (chunk q + 8 i of its row, clamped into the row).
// The chunk's E8M0 scale byte comes from the workgroup's staged scale rows.
struct MgRow {
    const uint8_t *w; // the row's codes
    const uint8_t *s; // the row's staged scale bytes (LDS)
    int CK, q;        // chunks per row, this lane's first chunk
    __device__ __forceinline__ void load(int i, u32x4 &wv) const
    {
        int j = min(q + 8 * i, CK - 1);
        // opaque to the optimizer: otherwise every ring slot keeps its own
        // pair of 64-bit address registers (one strength-reduced pointer per
        // slot), which costs more registers than the slots themselves
        asm volatile("" : "+v"(j));
        wv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w) + j);
    }
};

// Chunk j of the row times rows 0 .. mr-1 of the staged activations (mr <= MR;
// rows past mr are skipped by a uniform branch).
template <int MR>
__device__ __forceinline__ void mg_chunk(const u32x4 &w, uint32_t sb, const uint8_t *xl, int j,
                                         int K2, int mr, float (&acc)[MR])
{
    const float sc = e8m0_to_f32(sb);
    u32x4 wp[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        wp[c] = fp4_word_bf16x8(w[c], sc); // k = 32 j + 8 c + 2 p, +1
    const uint8_t *xc = xl + 64 * j;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m >= mr)
            break;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 xv = *reinterpret_cast<const u32x4 *>(xc + m * K2 + 16 * c);
#pragma unroll
            for (int p = 0; p < 4; ++p)
                acc[m] = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf162_t>(wp[c][p]),
                                                         bitcast<bf162_t>(xv[p]), acc[m], false);
        }
    }
}

// One pass over the staged rows 0 .. mr-1 (MR >= mr): stream the lane's
// chunks (the ring holds chunks 0 .. MG_D-1 on entry), reduce, store.
template <bool ACT, int MR>
__device__ __forceinline__ void mg_pass(const MgRow &wr, u32x4 (&rw)[MG_D], const uint8_t *smem, int K2,
                                        const int32_t *pairs, int mr, int col, bool cvalid,
                                        int lane, uint16_t *y, int Nout)
{
    const int nch = (wr.CK - wr.q + 7) >> 3; // chunks q + 8 i of this lane (CK >= 2)
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
        acc[m] = 0.f;
    // Steady state (rows longer than the ring): compute chunk i + d from
    // slot d, then refill the slot with chunk i + d + MG_D.
    int i = 0;
    for (; i + 2 * MG_D <= nch; i += MG_D) {
#pragma unroll
        for (int d = 0; d < MG_D; ++d) {
            mg_chunk<MR>(rw[d], wr.s[wr.q + 8 * (i + d)], smem, wr.q + 8 * (i + d), K2, mr, acc);
            __builtin_amdgcn_sched_barrier(0);
            wr.load(i + d + MG_D, rw[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // Drain: the ring holds chunks i .. i + MG_D - 1 (those below nch);
    // fewer than MG_D follow, loaded into the slots as these free up.
    if (__any(i + MG_D < nch)) {
#pragma unroll
        for (int d = 0; d < MG_D; ++d) {
            if (i + d < nch)
                mg_chunk<MR>(rw[d], wr.s[wr.q + 8 * (i + d)], smem, wr.q + 8 * (i + d), K2, mr, acc);
            __builtin_amdgcn_sched_barrier(0);
            wr.load(min(i + MG_D + d, max(nch - 1, 0)), rw[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
        i += MG_D;
    }
#pragma unroll
    for (int d = 0; d < MG_D; ++d) {
        if (i + d < nch)
            mg_chunk<MR>(rw[d], wr.s[wr.q + 8 * (i + d)], smem, wr.q + 8 * (i + d), K2, mr, acc);
        __builtin_amdgcn_sched_barrier(0); // one chunk's unpacked words live at a time
    }
    // Sum over the 8 lanes of a row; lane q = 0 holds row r's dot products.
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        float v = acc[m];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        if constexpr (ACT) {
            const float u = __shfl_xor(v, 32); // up row r + 4 of the gate row r
            v = v / (1.0f + expf(-v)) * u;
        }
        const int r = lane >> 3;
        if ((lane & 7) == 0 && (!ACT || r < 4) && cvalid && m < mr)
            y[(size_t)pairs[m] * Nout + col] = f32_to_act<DT_BF16>(v);
    }
}

// Routing is folded in (no separate kernel, no workspace): workgroup
// (slot p, slice) reads the P <= MG_PMAX ids and keeps going only when pair p
// is the first pair of its bucket (its expert, or the bucket of ids outside
// [0, E)); it then lists that bucket's pairs in LDS.  The order of the list
// does not change any output value: each pair's row is computed on its own.
// All ids are read in one round trip, and the first code batch is requested
// as soon as the bucket is known, so the listing and the activation staging
// overlap the weight stream instead of preceding it.
// MR: activation rows per pass (a bucket with more pairs takes several passes).
constexpr int MG_PMAX = MG_TOKENS * 64; // T <= 8 tokens, topk <= 64
static_assert(MG_PMAX <= 2 * MG_THREADS, "two ids per thread");

template <bool ACT, int MR>
__global__ __launch_bounds__(MG_THREADS) void moe_gemv_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ ids,
    const uint8_t *__restrict__ w_fp4, const uint8_t *__restrict__ w_scale,
    uint16_t *__restrict__ y, int P, int topk, int E, int N, int K, int n_slices)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int32_t list[MG_PMAX];
    __shared__ int count;
    constexpr int COLS = mg_cols<ACT>();
    const int p = blockIdx.x / n_slices;
    const int slice = blockIdx.x - p * n_slices;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane >> 3, q = lane & 7;
    auto bucket = [&](int32_t id) { return (uint32_t)id < (uint32_t)E ? id : E; };
    const int j0 = tid, j1 = tid + MG_THREADS;
    const int e = bucket(ids[p]);
    const int b0 = j0 < P ? bucket(ids[j0]) : -1;
    const int b1 = j1 < P ? bucket(ids[j1]) : -1;
    if (tid == 0)
        count = 0;
    if (__syncthreads_or((j0 < p && b0 == e) || (j1 < p && b1 == e)))
        return; // an earlier workgroup slot owns this bucket
    const int Nout = ACT ? N / 2 : N;
    // Weight row and output column of the workgroup's row rho = 8 wave + r
    // (rows past the matrix are clamped and never stored).
    auto row_col = [&](int rho, int &col_, int &n_) {
        const int w_ = rho >> 3, r_ = rho & 7;
        if constexpr (ACT) {
            col_ = slice * COLS + 4 * w_ + (r_ & 3);
            n_ = (r_ >> 2) * (N / 2) + min(col_, N / 2 - 1);
        } else {
            col_ = slice * COLS + 8 * w_ + r_;
            n_ = min(col_, N - 1);
        }
    };
    int col, n;
    row_col(8 * wave + r, col, n);
    const bool cvalid = col < Nout;
    const int CK = K >> 5;
    const int ee = min(e, E - 1); // the invalid bucket streams nothing (loads clamped, unused)
    const int K2 = 2 * K;
    uint8_t *const sl = smem + (size_t)MR * K2; // staged scale rows, CK bytes each
    MgRow wr;
    wr.w = w_fp4 + ((size_t)ee * N + n) * (size_t)(K >> 1);
    wr.s = sl + (size_t)(8 * wave + r) * CK;
    wr.CK = CK;
    wr.q = q;
    u32x4 rw[MG_D];
    auto fill = [&]() {
        // this lane's last chunk (a lane with no chunk, K < 256, loads chunk 0 unused)
        const int last = max(((CK - q + 7) >> 3) - 1, 0);
#pragma unroll
        for (int d = 0; d < MG_D; ++d)
            wr.load(min(d, last), rw[d]);
    };
    // Cooperative copy of `tot` units, MG_BATCH loads per thread in flight
    // before their stores (a plain loop waits one round trip per unit).
    auto stage = [&](int tot, auto &&ld, auto &&st) __attribute__((always_inline)) {
        for (int base = tid; base < tot; base += MG_BATCH * MG_THREADS) {
            decltype(ld(0)) v[MG_BATCH];
#pragma unroll
            for (int b = 0; b < MG_BATCH; ++b)
                v[b] = ld(min(base + b * MG_THREADS, tot - 1));
#pragma unroll
            for (int b = 0; b < MG_BATCH; ++b)
                if (base + b * MG_THREADS < tot)
                    st(base + b * MG_THREADS, v[b]);
        }
    };
    // The E8M0 scale bytes of the workgroup's rows go to LDS once, in 2-byte
    // units (CK is even): requested before the first code chunks, so they
    // land first, and stored after the listing.  The main loop then reads one
    // byte per chunk from LDS instead of a scattered global byte load next to
    // each code load.
    const int CKh = CK >> 1, stot = MG_ROWS * CKh;
    auto sld = [&](int idx) {
        const int rho = idx / CKh, u = idx - rho * CKh;
        int c_, n_;
        row_col(rho, c_, n_);
        return *reinterpret_cast<const uint16_t *>(w_scale + ((size_t)ee * N + n_) * CK + 2 * u);
    };
    auto sst = [&](int idx, uint16_t v) {
        const int rho = idx / CKh, u = idx - rho * CKh;
        *reinterpret_cast<uint16_t *>(sl + (size_t)rho * CK + 2 * u) = v;
    };
    uint16_t sv[MG_SB];
    if (e < E) {
#pragma unroll
        for (int b = 0; b < MG_SB; ++b)
            sv[b] = sld(min(tid + b * MG_THREADS, stot - 1));
        fill();
    }
    if (j0 >= p && b0 == e)
        list[atomicAdd(&count, 1)] = j0;
    if (j1 >= p && b1 == e)
        list[atomicAdd(&count, 1)] = j1;
    __syncthreads();
    const int rows = count;
    if (e >= E) { // ids out of range: zero rows
        for (int idx = tid; idx < rows * COLS; idx += MG_THREADS) {
            const int c = slice * COLS + idx % COLS;
            if (c < Nout)
                y[(size_t)list[idx / COLS] * Nout + c] = 0;
        }
        return;
    }
#pragma unroll
    for (int b = 0; b < MG_SB; ++b)
        if (tid + b * MG_THREADS < stot)
            sst(tid + b * MG_THREADS, sv[b]);
    if (stot > MG_SB * MG_THREADS) // long rows: the rest, batched
        stage(stot - MG_SB * MG_THREADS, [&](int idx) { return sld(idx + MG_SB * MG_THREADS); },
              [&](int idx, uint16_t v) { sst(idx + MG_SB * MG_THREADS, v); });
    const int nv = K >> 3; // 16-byte blocks per activation row
    for (int m0 = 0; m0 < rows; m0 += MR) {
        const int mr = min(MR, rows - m0);
        if (m0 > 0) {
            __syncthreads(); // the previous pass's reads of the staged rows are done
            fill();
        }
        stage(
            mr * nv,
            [&](int idx) {
                const int m = idx / nv, b = idx - m * nv;
                const int tok = list[m0 + m] / topk;
                return reinterpret_cast<const u32x4 *>(x + (size_t)tok * K)[b];
            },
            [&](int idx, const u32x4 &v) {
                const int m = idx / nv, b = idx - m * nv;
                reinterpret_cast<u32x4 *>(smem + (size_t)m * K2)[b] = v;
            });
        __syncthreads();
        mg_pass<ACT, MR>(wr, rw, smem, K2, list + m0, mr, col, cvalid, lane, y, Nout);
    }
}

template <bool ACT, int MR>
hipError_t launch_gemv(const void *x, const int32_t *ids, const uint8_t *w_fp4,
                       const uint8_t *w_scale, void *y, int P, int topk, int E, int N, int K,
                       hipStream_t stream)
{
    auto kern = moe_gemv_kernel<ACT, MR>;
    static std::atomic<uint64_t> lds_set{0};
    if (const hipError_t e = lds_optin(reinterpret_cast<const void *>(kern), MG_LDS, lds_set);
        e != hipSuccess)
        return e;
    const int nout = ACT ? N / 2 : N;
    const int n_slices = (nout + mg_cols<ACT>() - 1) / mg_cols<ACT>();
    const int64_t grid = (int64_t)P * n_slices; // one slot per pair; non-first pairs exit
    if (P > MG_PMAX || grid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(MG_THREADS),
                       (size_t)MR * 2 * (size_t)K + (size_t)mg_scale_bytes(K),
                       stream, static_cast<const uint16_t *>(x), ids, w_fp4, w_scale,
                       static_cast<uint16_t *>(y), P, topk, E, N, K, n_slices);
    return hipGetLastError();
}

// Rows per pass: distinct ids per token give an expert at most T rows.
template <bool ACT>
hipError_t launch_gemv_t(const void *x, const int32_t *ids, const uint8_t *w_fp4,
                         const uint8_t *w_scale, void *y, int T, int P, int topk, int E, int N,
                         int K, int mrmax, hipStream_t stream)
{
    const int mr = std::min(T, mrmax);
    if (mr > 4)
        return launch_gemv<ACT, 8>(x, ids, w_fp4, w_scale, y, P, topk, E, N, K, stream);
    if (mr > 2)
        return launch_gemv<ACT, 4>(x, ids, w_fp4, w_scale, y, P, topk, E, N, K, stream);
    if (mr > 1)
        return launch_gemv<ACT, 2>(x, ids, w_fp4, w_scale, y, P, topk, E, N, K, stream);
    return launch_gemv<ACT, 1>(x, ids, w_fp4, w_scale, y, P, topk, E, N, K, stream);
}

template <bool ACT, int BR>
hipError_t launch_gemm(const void *x, const uint8_t *w_fp4, const uint8_t *w_scale, void *y,
                       const MoeWs &w, int64_t P, int topk, int E, int N, int K,
                       hipStream_t stream)
{
    constexpr int LDS = MoeGeo<ACT, BR>::lds_bytes(moe_mb_max<ACT, BR>());
    static_assert(LDS <= 160 * 1024, "tile fits the LDS");
    auto kern = moe_gemm_kernel<ACT, BR>;
    static std::atomic<uint64_t> lds_set{0};
    if (const hipError_t e = lds_optin(reinterpret_cast<const void *>(kern), LDS, lds_set);
        e != hipSuccess)
        return e;
    const int tw = ACT ? moe_tn<ACT, BR>() / 2 : moe_tn<ACT, BR>();
    const int nout = ACT ? N / 2 : N;
    const int n_nt = (nout + tw - 1) / tw;
    const int nxcd = device_topology().xcds;
    const int64_t grid = (int64_t)nxcd * (((int64_t)max_tiles(P, E) * n_nt + nxcd - 1) / nxcd);
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(TL_THREADS), (size_t)LDS, stream,
                       static_cast<const uint16_t *>(x), w_fp4, w_scale, static_cast<uint16_t *>(y),
                       w.hdr, w.tiles, w.sorted, topk, E, N, K, n_nt, nxcd);
    return hipGetLastError();
}

} // namespace

// ---- Allocation-free form: routing scratch in a static device array -------

// One copy per GPU the library runs on, kept until the process ends; its
// device address is looked up once per device (below).  Every call on a GPU
// shares it: the routing kernel rewrites everything the GEMM reads from it
// (tile count, tile table, sorted pairs) before the GEMM runs, so nothing has
// to be cleared, but calls that overlap on one GPU race.
size_t moe_scratch_bytes() { return MOE_SCRATCH_BYTES; }

hipError_t moe_scratch(void **ptr)
{
    static std::atomic<void *> dev_ptr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    void *p = dev_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // with `dev` current: this device's copy of the array (the array's
        // name in host code is only a stand-in, not a device address)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(moe_static_scratch));
        if (e != hipSuccess)
            return e;
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
            return hipErrorInvalidSymbol;
        dev_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

size_t moe_stage2_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t H)
{
    const size_t route = (moe_workspace_bytes(T, topk, E) + 255) & ~(size_t)255;
    return route + (size_t)(T * topk) * (size_t)H * sizeof(float);
}

hipError_t launch_mxfp4_moe_stage2(const void *a, const int32_t *ids, const float *w,
                                   const uint8_t *w_fp4, const uint8_t *w_scale, void *y, int T,
                                   int topk, int E, int H, int I, void *workspace,
                                   hipStream_t stream)
{
    const int64_t P = (int64_t)T * topk;
    const MoeWs ws = carve(workspace, P, E);
    float *pre = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                           ((moe_workspace_bytes(T, topk, E) + 255) & ~(size_t)255));
    const size_t route_lds = (size_t)(3 * (E + 1)) * sizeof(int);
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(ROUTE_THREADS), route_lds, stream, ids,
                       (int)P, E, moe_tm<false, MOE2_BR>(), ws.hdr, ws.tiles, ws.sorted);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    constexpr int MB2 = moe_mb_max<false, MOE2_BR>();
    static_assert(MB2 <= Moe2Geo::MB_MAX, "routing tile fits the stage-2 tile");
    constexpr int LDS = Moe2Geo::lds_bytes(MB2);
    static_assert(LDS <= 160 * 1024, "tile fits the LDS");
    static std::atomic<uint64_t> lds_set{0};
    if (const hipError_t e = lds_optin(reinterpret_cast<const void *>(moe_stage2_kernel), LDS,
                                       lds_set);
        e != hipSuccess)
        return e;
    const int tw = Moe2Geo::TN;
    const int n_nt = (H + tw - 1) / tw;
    const int nxcd = device_topology().xcds;
    const int64_t grid = (int64_t)nxcd * (((int64_t)max_tiles(P, E) * n_nt + nxcd - 1) / nxcd);
    if (grid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(moe_stage2_kernel, dim3((unsigned)grid), dim3(TL_THREADS), (size_t)LDS,
                       stream, static_cast<const uint16_t *>(a), w_fp4, w_scale, pre, ws.hdr,
                       ws.tiles, ws.sorted, E, H, I, n_nt, nxcd);
    err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t outs = (int64_t)T * (H / 8);
    const int64_t cgrid = (outs + CB_THREADS - 1) / CB_THREADS;
    if (cgrid > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)cgrid), dim3(CB_THREADS), 0, stream, pre,
                       ids, w, static_cast<uint16_t *>(y), T, topk, E, H);
    return hipGetLastError();
}

size_t moe_workspace_bytes(int64_t T, int64_t topk, int64_t E)
{
    const int64_t P = T * topk;
    return 16 + 16 * max_tiles(P, E) + 4 * (size_t)P;
}

hipError_t launch_mxfp4_moe(const void *x, const int32_t *ids, const uint8_t *w_fp4,
                            const uint8_t *w_scale, void *y, int T, int topk, int E, int N, int K,
                            int act, int tile_m, void *workspace, hipStream_t stream)
{
    const int64_t P = (int64_t)T * topk;
    const int mrmax = mg_rows(K);
    if (T <= MG_TOKENS && mrmax > 0)
        return act ? launch_gemv_t<true>(x, ids, w_fp4, w_scale, y, T, (int)P, topk, E, N, K,
                                         mrmax, stream)
                   : launch_gemv_t<false>(x, ids, w_fp4, w_scale, y, T, (int)P, topk, E, N, K,
                                          mrmax, stream);
    const MoeWs w = carve(workspace, P, E);
    const size_t route_lds = (size_t)(3 * (E + 1)) * sizeof(int);
    const bool br16 = tile_m == 16;
    const int tm = br16 ? (act ? moe_tm<true, 16>() : moe_tm<false, 16>())
                        : (act ? moe_tm<true, 32>() : moe_tm<false, 32>());
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(ROUTE_THREADS), route_lds, stream, ids,
                       (int)P, E, tm, w.hdr, w.tiles, w.sorted);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    if (br16)
        return act ? launch_gemm<true, 16>(x, w_fp4, w_scale, y, w, P, topk, E, N, K, stream)
                   : launch_gemm<false, 16>(x, w_fp4, w_scale, y, w, P, topk, E, N, K, stream);
    return act ? launch_gemm<true, 32>(x, w_fp4, w_scale, y, w, P, topk, E, N, K, stream)
               : launch_gemm<false, 32>(x, w_fp4, w_scale, y, w, P, topk, E, N, K, stream);
}

} // namespace wob
