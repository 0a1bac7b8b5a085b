// Cooperative-tile MFMA W4A16 GEMM on gfx950 (prefill, M >= 9; any M works)
// and its ragged grouped form.
//
// One workgroup computes a TN x TM output tile (weight rows x activation
// rows) with the shared pipeline of wob_tile.hpp: the TN weight rows are
// dequantized once per tile, the activation rows stream through LDS, and
// v_mfma_f32_32x32x16_{f16,bf16} does the products.  Tiles are 256 weight
// rows by up to 256 activation rows (TILED_NB = 2 weight blocks per wave,
// eight 32-row activation blocks); the number of activation blocks actually
// multiplied follows the tile's row count, so a short last tile (or a short
// group) costs only the blocks it needs.
//
// Dense form: tiles cover rows [TM_MAX * mt, ...) of x and y.
// Grouped form ("contiguous grouped" GEMM): group e owns rows
// [m_offsets[e], m_offsets[e+1]) of x and y and its own packed weights; each
// group is cut into tiles of TM_MAX rows.  The group table stays on the device:
// every workgroup derives its (group, tile) from the offsets with wave-wide
// prefix sums, so no host synchronization or workspace is needed.
#include "wob_internal.hpp"
#include "wob_tile.hpp"

#include <limits.h>

namespace wob {
namespace {

constexpr int TILED_NB = 2; // 32-row weight blocks per wave: 256 x 256 tiles
constexpr int TILE_BAND = 4; // activation tiles per band of the dense tile order

// Contiguous activation rows m0 .. m0 + rows - 1 of x[.][K] and y[.][N].
// Byte offset of row min(16 i + rl, rows - 1): rowb (16 i + rl) clamped to
// rowb (rows - 1), one add and one min per copy.
struct ContigRows {
    int rows;
    uint32_t o0;    // rowb * rl (this lane's first row)
    uint32_t s16;   // rowb * 16
    uint32_t omax;  // rowb * (rows - 1)
    uint16_t *base; // output row m0
    int ld;         // N
    __device__ __forceinline__ uint32_t off(int i) const { return min(o0 + (uint32_t)i * s16, omax); }
    __device__ __forceinline__ uint32_t index(int r) const { return (uint32_t)r; }
};

__device__ __forceinline__ int wave_sum_dev(int v)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1)
        v += __shfl_xor(v, d);
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d);
        if (lane >= d)
            v += o;
    }
    return v;
}

// Row range [lo, hi) of group g, clamped into [0, total_M].
__device__ __forceinline__ void group_range(const int64_t *off, int g, int total_M, int &lo, int &hi)
{
    const int64_t a = off[g], b = off[g + 1];
    lo = (int)min<int64_t>(max<int64_t>(a, 0), total_M);
    hi = (int)min<int64_t>(max<int64_t>(b, lo), total_M);
}

// Locate this workgroup's tile in the grouped problem.  Every wave runs the
// same wave-uniform computation (no LDS, no barrier).  Returns false when
// the workgroup has no tile.
__device__ bool grouped_tile(const int64_t *off, int G, int total_M, int TM, int n_nt, int nxcd,
                             int &e, int &m0, int &rows, int &nt)
{
    const int lane = threadIdx.x & 63;
    int total = 0;
    for (int c = 0; c < G; c += 64) {
        const int g = c + lane;
        int tiles = 0;
        if (g < G) {
            int lo, hi;
            group_range(off, g, total_M, lo, hi);
            tiles = (hi - lo + TM - 1) / TM;
        }
        total += wave_sum_dev(tiles);
    }
    const int t = xcd_tile(total * n_nt, nxcd);
    if (t < 0)
        return false;
    const int i = t / n_nt;
    nt = t - i * n_nt;
    int base = 0;
    for (int c = 0; c < G; c += 64) {
        const int g = c + lane;
        int tiles = 0, lo = 0, hi = 0;
        if (g < G) {
            group_range(off, g, total_M, lo, hi);
            tiles = (hi - lo + TM - 1) / TM;
        }
        const int incl = wave_incl_scan(tiles);
        const int excl = incl - tiles;
        const bool hit = g < G && base + excl <= i && i < base + incl;
        const uint64_t mask = __ballot(hit);
        if (mask) {
            const int src = __ffsll((unsigned long long)mask) - 1;
            e = __shfl(g, src);
            const int first = __shfl(lo, src);
            const int last = __shfl(hi, src);
            m0 = first + (i - base - __shfl(excl, src)) * TM;
            rows = min(TM, last - m0);
            return true;
        }
        base += __shfl(incl, 63);
    }
    return false;
}

template <int DT, int NB, int MB, class Fmt>
__device__ __forceinline__ void run_tile(const Fmt &fmt, const ContigRows &rws, const uint8_t *xbase,
                                         int K, int N, int n0, uint8_t *smem, const TileLane<> &tl)
{
    float16_t acc[NB][MB];
    tile_mainloop<DT, NB, MB, 32>(fmt, rws, xbase, K, n0, N, smem, tl, acc);
    tile_store<DT, NB, MB, 32>(acc, rws, rws.rows, n0, N, tl, smem);
}

// Runs the tile with the smallest block count that covers `rows`.
template <int DT, int NB, int MB, class Fmt>
__device__ __forceinline__ void dispatch_tile(int mb, const Fmt &fmt, const ContigRows &rws,
                                              const uint8_t *xbase, int K, int N, int n0,
                                              uint8_t *smem, const TileLane<> &tl)
{
    if constexpr (MB > 1) {
        if (mb < MB) {
            dispatch_tile<DT, NB, MB - 1>(mb, fmt, rws, xbase, K, N, n0, smem, tl);
            return;
        }
    }
    run_tile<DT, NB, MB>(fmt, rws, xbase, K, N, n0, smem, tl);
}

// m_offsets == nullptr: dense problem of M rows (n_mt tiles of TM_MAX rows).
// GM: group mode of the W4A16 format (0: g = 32; 1: g >= 64, one scale /
// zero-point load per slice pair; 2: g = 128 with an even G >= 4, scales of
// four spans per load).
template <int DT, int NB, bool HAS_Z, int GM>
__global__ __launch_bounds__(TL_THREADS, 1) void w4a16_tiled_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros,
    uint16_t *__restrict__ y, const int64_t *__restrict__ m_offsets, int num_groups, int M, int N,
    int K, int gshift, int n_mt, int n_nt, int nxcd)
{
    using GEO = TileGeo<NB>;
    constexpr int TMX = GEO::TM_MAX;
    extern __shared__ __align__(16) uint8_t smem[];

    int e = 0, m0, rows, nt;
    if (!m_offsets) {
        // Dense: tiles in bands of TILE_BAND activation tiles; within a band
        // the weight tiles advance every TILE_BAND tiles (activation tiles
        // fastest).  An XCD's contiguous run of tile indices is then a 2-D
        // block (at the prefill shape, 4 activation tiles x 16 weight tiles,
        // 4 x 8 of them resident at once), so both operands are shared in
        // its L2: 4 x 2.75 MB of activations and 8 x 0.69 MB of weights per
        // round, where a run along one operand shares only that one.
        const int t = xcd_tile(n_mt * n_nt, nxcd);
        if (t < 0)
            return;
        const int band = t / (TILE_BAND * n_nt);
        const int mt0 = band * TILE_BAND;
        const int bw = min(TILE_BAND, n_mt - mt0); // the last band may be narrower
        const int local = t - mt0 * n_nt;
        nt = local / bw;
        const int mt = mt0 + (local - nt * bw);
        m0 = mt * TMX;
        rows = min(TMX, M - m0);
    } else if (!grouped_tile(m_offsets, num_groups, M, TMX, n_nt, nxcd, e, m0, rows, nt)) {
        return;
    }
    if (rows <= 0)
        return;
    const int n0 = nt * GEO::TN;
    const int G = K >> (5 + gshift);
    const TileLane<> tl;
    const FmtW4<DT, HAS_Z, NB, GM> fmt(qweight + (size_t)e * N * (K >> 3),
                                   scales + (size_t)e * N * G,
                                   HAS_Z ? qzeros + (size_t)e * (N >> 3) * G : qzeros, N, K,
                                   gshift, n0, tl);
    ContigRows rws;
    const uint32_t rowb = 2u * (uint32_t)K;
    rws.o0 = rowb * (uint32_t)tl.rl;
    rws.s16 = rowb * 16u;
    rws.omax = rowb * (uint32_t)(rows - 1);
    rws.rows = rows;
    rws.base = y + (size_t)m0 * N;
    rws.ld = N;
    const uint8_t *xbase = reinterpret_cast<const uint8_t *>(x + (size_t)m0 * K);
    dispatch_tile<DT, NB, GEO::MB_MAX>((rows + 31) >> 5, fmt, rws, xbase, K, N, n0, smem, tl);
}

template <int DT, int NB, bool HAS_Z, int GM>
hipError_t launch_k(const W4Args &a, const int64_t *m_offsets, int num_groups, int grid, int n_mt,
                    int n_nt, int nxcd, size_t lds, hipStream_t stream)
{
    const int gshift = a.g == 32 ? 0 : a.g == 64 ? 1 : 2;
    auto kern = w4a16_tiled_kernel<DT, NB, HAS_Z, GM>;
    static std::atomic<uint64_t> lds_set{0};
    if (const hipError_t e = lds_optin(reinterpret_cast<const void *>(kern),
                                       TileGeo<NB>::lds_bytes(TileGeo<NB>::MB_MAX), lds_set);
        e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(TL_THREADS), lds, stream,
                       static_cast<const uint16_t *>(a.x), a.qweight,
                       static_cast<const uint16_t *>(a.scales), a.qzeros,
                       static_cast<uint16_t *>(a.y), m_offsets, num_groups, a.M, a.N, a.K, gshift,
                       n_mt, n_nt, nxcd);
    return hipGetLastError();
}

template <int DT, bool HAS_Z, int GM>
hipError_t launch_zg(const W4Args &a, const int64_t *m_offsets, int num_groups, hipStream_t stream)
{
    using GEO = TileGeo<TILED_NB>;
    constexpr int TMX = GEO::TM_MAX;
    const int n_nt = (a.N + GEO::TN - 1) / GEO::TN;
    const int nxcd = device_topology().xcds;
    if (!m_offsets) {
        // One tile row when M fits in it: size LDS for the blocks it needs.
        const int n_mt = (a.M + TMX - 1) / TMX;
        const int mb = n_mt == 1 ? (a.M + 31) / 32 : GEO::MB_MAX;
        const int grid = nxcd * ((n_mt * n_nt + nxcd - 1) / nxcd);
        return launch_k<DT, TILED_NB, HAS_Z, GM>(a, nullptr, 0, grid, n_mt, n_nt, nxcd,
                                                 (size_t)GEO::lds_bytes(mb), stream);
    }
    // Upper bound on the tiles of all groups: sum of ceil(rows_e / TMX).
    const int64_t max_mt = (a.M + TMX - 1) / TMX + num_groups;
    const int64_t grid = (int64_t)nxcd * ((max_mt * n_nt + nxcd - 1) / nxcd);
    if (grid > INT_MAX)
        return hipErrorInvalidValue;
    return launch_k<DT, TILED_NB, HAS_Z, GM>(a, m_offsets, num_groups, (int)grid, 0, n_nt, nxcd,
                                             (size_t)GEO::lds_bytes(GEO::MB_MAX), stream);
}

template <int DT, bool HAS_Z>
hipError_t launch_z(const W4Args &a, const int64_t *m_offsets, int num_groups, hipStream_t stream)
{
    // g = 128 with an even G >= 4: the scales of four spans per load (GM 2)
    const int G = (int)(a.K / a.g);
    if (a.g == 128 && G % 2 == 0 && G >= 4)
        return launch_zg<DT, HAS_Z, 2>(a, m_offsets, num_groups, stream);
    return a.g >= 64 ? launch_zg<DT, HAS_Z, 1>(a, m_offsets, num_groups, stream)
                     : launch_zg<DT, HAS_Z, 0>(a, m_offsets, num_groups, stream);
}

hipError_t launch_any(const W4Args &a, const int64_t *m_offsets, int num_groups, hipStream_t stream)
{
    if (a.dt == DT_F16)
        return a.qzeros ? launch_z<DT_F16, true>(a, m_offsets, num_groups, stream)
                        : launch_z<DT_F16, false>(a, m_offsets, num_groups, stream);
    return a.qzeros ? launch_z<DT_BF16, true>(a, m_offsets, num_groups, stream)
                    : launch_z<DT_BF16, false>(a, m_offsets, num_groups, stream);
}

} // namespace

hipError_t launch_w4a16_tiled(const W4Args &a, hipStream_t stream)
{
    return launch_any(a, nullptr, 0, stream);
}

hipError_t launch_w4a16_grouped(const W4Args &a, const int64_t *m_offsets, int num_groups,
                                hipStream_t stream)
{
    return launch_any(a, m_offsets, num_groups, stream);
}

} // namespace wob
