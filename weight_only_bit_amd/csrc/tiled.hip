// Cooperative-tile W4A16 GEMM on gfx950 MFMA (prefill, M >= 9; any M works).
//
// Mechanism (cooperative shared tile: "ROCm KQuantGemmKWmmaQ4K/Q6K: redesign
// around a cooperative shared tile, matching llama.cpp's mul_mat_q
// mechanism", sections Confirmed mechanism and The work): one workgroup owns
// a TN x TM output tile (weight rows x activation rows).  The packed weights
// of its TN rows are loaded and dequantized exactly once, split across the
// waves so no wave repeats another's work; one copy of the activation tile in
// LDS serves every wave; each wave multiplies its own weight rows against the
// whole activation range.  Dequantization and the matrix multiply are
// separate steps ("ROCm IQ4_XS keep-quant GEMM is 8.8x behind...", section
// Cause), here registers -> MFMA.
//
// gfx950 realisation:
//  * Matrix core: v_mfma_f32_32x32x16_{f16,bf16}.  Measured on MI355X it
//    sustains about 2.2-2.3 PFLOP/s even at one wave per SIMD, twice the
//    16x16x32 form, so every tile is built from 32 x 32 blocks.
//  * 4 waves; wave w owns weight rows n0 + 64 w .. +63 (two 32-row blocks)
//    and all TM = 32 * MB activation rows of the tile: 2 x MB accumulator
//    blocks of 16 fp32 registers (kept in AGPRs).
//  * K advances in spans of 128 (8 MFMA steps of 16).  Lane (nl, h) =
//    (lane%32, lane/32) loads 32 bytes of weight row nl of each block: words
//    8h..8h+7 of the span, i.e. k = 64h .. 64h+63 (one or two quantization
//    groups).  MFMA step s uses word s of that load: operand slot (h, e)
//    holds k = 64h + 8s + e.  The activation operand uses the same slots.
//  * The activation tile (TM rows x 128 k, 256 bytes per row) is copied from
//    global memory straight into LDS with global_load_lds_dwordx4 (no
//    staging registers), double buffered across spans.  Within a row the
//    16-byte block b is stored at position b ^ (row % 16), which makes the
//    operand reads (32 rows x one block each) bank-conflict free.
//  * Software pipeline: within a span the loop runs over the 8 MFMA steps;
//    each step dequantizes the two weight words it needs (one per 32-row
//    block) and issues its 2 x MB MFMAs, while the next step's activation
//    operands are read from LDS and its two words are dequantized.  The raw
//    packed weights are double buffered in registers and loaded a whole span
//    ahead; the next span's activation tile streams into the other LDS buffer.
//  * Tiles are mapped so that the workgroups running on one XCD share one
//    activation M-tile in its L2.
//  * Tails: weight rows >= N and activation rows >= M are clamped to valid
//    addresses and never stored; a 32-wide K slice past K gets zero weights
//    and its activation loads are clamped inside the row.
#include "wob_device.hpp"
#include "wob_internal.hpp"

namespace wob {
namespace {

typedef __attribute__((address_space(3))) void lds_ptr_t;

constexpr int TL_WAVES = 4;
constexpr int TL_THREADS = 64 * TL_WAVES;
constexpr int TL_TN = 64 * TL_WAVES; // weight rows per workgroup
constexpr int TL_SPAN = 128;         // K per span
constexpr int TL_ROWB = 256;         // LDS bytes per activation row of a span

// binary16 MFMA operand, natural k order: eight values of one packed word,
// each RNE((q - z) * s).  Byte p of the word holds values 2p (low nibble)
// and 2p+1 (high nibble); one permute places it twice next to the binary16
// exponent byte 0x64 and one mask keeps the low nibble in the first half and
// the high nibble (times 16) in the second: the exact halves (1024 + q_even,
// 1024 + 16 q_odd).  A packed fma with (1, 1/16) and -(1024 + z, 64 + z)
// gives the exact (q - z) pair, and a packed multiply by the scale rounds once.
__device__ __forceinline__ u32x4 w4_word_f16x8_nat(uint32_t w, half2_t negb, half2_t s2)
{
    const half2_t mul = half2_t{(_Float16)1.0f, (_Float16)0.0625f};
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t sel = 0x04000400u | (uint32_t)p | ((uint32_t)p << 16);
        const uint32_t t = __builtin_amdgcn_perm(MAGIC4_F16, w, sel) & 0xFFF0FF0Fu;
        const half2_t d = __builtin_elementwise_fma(bitcast<half2_t>(t), mul, negb);
        o[p] = bitcast<uint32_t>(d * s2);
    }
    return o;
}

// bfloat16 MFMA operand, natural k order: values from byte lanes as fp32,
// (q - z) * s exact in fp32, one rounding to bfloat16 per value.
__device__ __forceinline__ u32x4 w4_word_bf16x8_nat(uint32_t w, float s, float zf)
{
    const uint32_t lo = w & 0x0F0F0F0Fu;        // values 0, 2, 4, 6
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu; // values 1, 3, 5, 7
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float qe = (float)((lo >> (8 * p)) & 0xFFu);
        const float qo = (float)((hi >> (8 * p)) & 0xFFu);
        o[p] = f32x2_to_act2<DT_BF16>((qe - zf) * s, (qo - zf) * s);
    }
    return o;
}

typedef float float16_t __attribute__((ext_vector_type(16)));

// s_waitcnt that waits until at most `n` vector-memory operations are
// outstanding (expcnt and lgkmcnt left alone; gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the full memory wait __syncthreads() implies;
// callers wait for exactly the operations the barrier must cover first.
__device__ __forceinline__ void barrier_only()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS: lane L's bytes land
// at LDS byte address `lds_addr` + 16 L (global_load_lds_dwordx4, address =
// `sbase` + `voff`).  Issued through inline asm on purpose: the compiler's
// wait-count bookkeeping, once it sees an LDS DMA in flight, stops trusting
// in-order completion and waits for everything before any later load result
// or LDS read is used, which serializes the software pipeline.  The hardware
// tracks the DMA with vmcnt only; every caller waits for it explicitly
// (s_waitcnt vmcnt) before the destination is read.  M0 is saved and restored.
__device__ __forceinline__ void lds_dma16(const void *sbase_any, uint32_t voff, uint32_t lds_addr)
{
    // the base must live in scalar registers: make its (uniform) value explicit
    const uint64_t b = reinterpret_cast<uint64_t>(sbase_any);
    // readfirstlane returns a signed int: zero-extend each half explicitly
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
    const void *sbase = reinterpret_cast<const void *>(bu);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\t"
                 "global_load_lds_dwordx4 %2, %3\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(sbase)
                 : "memory");
}

template <int DT>
__device__ __forceinline__ float16_t mfma32x32x16(const u32x4 &a, const u32x4 &b, const float16_t &c)
{
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<half8_t>(a), bitcast<half8_t>(b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf168_t>(a), bitcast<bf168_t>(b), c, 0, 0, 0);
}

// One weight word (8 k values) of the B-operand form, per dtype.
template <int DT>
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, uint32_t sbits, uint32_t z)
{
    if constexpr (DT == DT_F16) {
        const _Float16 sh = bitcast<_Float16>((uint16_t)sbits);
        const half2_t negb = bitcast<half2_t>(
            (0xE400u | z) | ((uint32_t)bitcast<uint16_t>((_Float16)(-(64.f + (float)z))) << 16));
        return w4_word_f16x8_nat(w, negb, half2_t{sh, sh});
    } else {
        return w4_word_bf16x8_nat(w, act_to_f32<DT_BF16>((uint16_t)sbits), (float)z);
    }
}

template <int DT, int MB, bool HAS_Z>
__global__ __launch_bounds__(TL_THREADS, 1) void w4a16_tiled_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros,
    uint16_t *__restrict__ y, int M, int N, int K, int gshift, int n_mt, int n_nt,
    int tiles_per_xcd)
{
    constexpr int TM = 32 * MB;
    extern __shared__ __align__(16) uint8_t smem[]; // 2 x TM x 256 bytes

    // XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD takes a
    // contiguous run of tiles (N fastest), so its workgroups share M-tiles.
    const int t = (blockIdx.x & 7) * tiles_per_xcd + (blockIdx.x >> 3);
    if (t >= n_mt * n_nt)
        return;
    const int mt = t / n_nt;
    const int nt = t - mt * n_nt;
    const int m0 = mt * TM;
    const int n0 = nt * TL_TN;

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int nl = lane & 31;
    const int h = lane >> 5;
    const int S = (K + TL_SPAN - 1) / TL_SPAN;
    const int G = K >> (5 + gshift);

    // ---- per-lane weight rows: uniform bases + 32-bit byte offsets ----
    // Row n = n0 + 64 wave + 32 nb + nl (clamped to N - 1); rows of one lane
    // share n % 8, so one zero-point nibble shift serves both blocks.
    const uint8_t *wbase = reinterpret_cast<const uint8_t *>(qweight);
    const uint8_t *sbase = reinterpret_cast<const uint8_t *>(scales);
    const uint8_t *zbase = reinterpret_cast<const uint8_t *>(qzeros);
    uint32_t woff[2], soff[2], zoff[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int n = min(n0 + 64 * wave + 32 * nb + nl, N - 1);
        woff[nb] = (uint32_t)n * (uint32_t)(K >> 1); // row start
        soff[nb] = (uint32_t)n * (uint32_t)G * 2u;
        zoff[nb] = (uint32_t)(n >> 3) * (uint32_t)G * 4u;
    }
    const int zsh = 4 * (nl & 7);

    // Raw weights of one span: [block][half] 16-byte loads (words 8h+4half ..),
    // with the scale and zero-point word of each 32-wide half slice.
    struct Raw {
        u32x4 w[2][2];
        uint32_t s[2][2], z[2][2];
    };
    auto load_w = [&](int span, Raw &r) __attribute__((always_inline)) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int k = span * TL_SPAN + 64 * h + 32 * hf;
            const int kc = min(k, K - 32); // slice past K: clamped load, zeroed at dequant
            const uint32_t kb = (uint32_t)kc >> 1;
            const uint32_t grp = (uint32_t)(kc >> (5 + gshift));
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                r.w[nb][hf] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wbase + woff[nb] + kb));
                r.s[nb][hf] = *reinterpret_cast<const uint16_t *>(sbase + soff[nb] + 2u * grp);
                r.z[nb][hf] = HAS_Z ? *reinterpret_cast<const uint32_t *>(zbase + zoff[nb] + 4u * grp)
                                    : 0x88888888u;
            }
        }
    };
    // Operand of block nb, step st of a span: one weight word as 8 values.
    // Only a span that crosses K (uniform test) needs the per-lane zeroing of
    // the 32-wide slices past K.
    auto dequant_op = [&](const Raw &r, int span, int nb, int st) __attribute__((always_inline)) {
        const int hf = st >> 2;
        const uint32_t z = (r.z[nb][hf] >> zsh) & 0xFu;
        u32x4 v = dequant_word<DT>(r.w[nb][hf][st & 3], r.s[nb][hf], z);
        if (span * TL_SPAN + TL_SPAN > K) {
            if (span * TL_SPAN + 64 * h + 32 * hf >= K)
                v = u32x4{0, 0, 0, 0};
        }
        return v;
    };

    // ---- activation tile DMA: TM rows x 16 blocks per span, 1 KB per wave instruction ----
    // Instruction i of wave w fills LDS rows 16 i + 4 w .. +3; lane L takes row
    // 16 i + rl (rl = 4 w + L/16) and position p = L % 16, which holds global
    // block p ^ rl of that row (rl = row % 16 for every i).  Fast path (tile
    // inside M, span inside K): uniform base stepped per instruction plus one
    // per-lane offset.  Otherwise rows and blocks are clamped per lane.
    const int rl = 4 * wave + (lane >> 4);
    const int xblk = (lane & 15) ^ rl;
    const uint8_t *xbase = reinterpret_cast<const uint8_t *>(x);
    const uint32_t lds0 = (uint32_t)(size_t)(lds_ptr_t *)smem;
    const uint32_t xfast = 2u * ((uint32_t)rl * (uint32_t)K + 8u * (uint32_t)xblk);
    const bool mfull = m0 + TM <= M;
    auto issue_x = [&](int span, int buf) __attribute__((always_inline)) {
        const uint32_t ldsb = lds0 + (uint32_t)(buf * TM * TL_ROWB);
        if (mfull && span * TL_SPAN + TL_SPAN <= K) {
            const uint8_t *b0 = xbase + 2 * ((size_t)m0 * K + (size_t)span * TL_SPAN);
#pragma unroll
            for (int i = 0; i < TM / 16; ++i)
                lds_dma16(b0 + (size_t)32 * K * i, xfast,
                          __builtin_amdgcn_readfirstlane(ldsb + (uint32_t)((16 * i + 4 * wave) * TL_ROWB)));
        } else {
            const uint32_t k = (uint32_t)min(span * TL_SPAN + 8 * xblk, K - 8);
#pragma unroll
            for (int i = 0; i < TM / 16; ++i) {
                const uint32_t m = (uint32_t)min(m0 + 16 * i + rl, M - 1);
                lds_dma16(xbase, 2u * (m * (uint32_t)K + k),
                          __builtin_amdgcn_readfirstlane(ldsb + (uint32_t)((16 * i + 4 * wave) * TL_ROWB)));
            }
        }
    };

    float16_t acc[2][MB];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[nb][mb][e] = 0.f;

    // Raw weights double buffered: rA / rB alternate between "this span"
    // (complete) and "next span" (loads in flight).
    Raw rA, rB;
    load_w(0, rA);
    load_w(min(1, S - 1), rB);
    issue_x(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    barrier_only();

    // One span: MFMAs on LDS buffer span & 1 with the weights in `cur`.  At
    // entry `nxt`'s loads (span + 1) have landed; they are re-issued for
    // span + 2 after this span's computation has read `cur`... the roles
    // swap every span, so `cur` of this span is refilled for span + 2.
    auto run_span = [&](int span, Raw &cur, Raw &nxt) __attribute__((always_inline)) {
        (void)nxt;
        const int buf = span & 1;
        issue_x(min(span + 1, S - 1), buf ^ 1);
        const uint8_t *xb = smem + (size_t)buf * TM * TL_ROWB;
        // Activation operand of block mb, step st: 32 rows (nl), 16-byte
        // block 8h + st of the span.
        auto read_x = [&](int mb, int st) __attribute__((always_inline)) {
            const int R = 32 * mb + nl;
            const int p = (8 * h + st) ^ (R & 15);
            return *reinterpret_cast<const u32x4 *>(xb + R * TL_ROWB + 16 * p);
        };
        u32x4 wc[2], wn[2], xc[MB], xn[MB];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            wc[nb] = dequant_op(cur, span, nb, 0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            xc[mb] = read_x(mb, 0);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            if (st < 7) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    xn[mb] = read_x(mb, st + 1);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    wn[nb] = dequant_op(cur, span, nb, st + 1);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[nb][mb] = mfma32x32x16<DT>(wc[nb], xc[mb], acc[nb][mb]);
            __builtin_amdgcn_sched_barrier(0);
            if (st < 7) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    wc[nb] = wn[nb];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    xc[mb] = xn[mb];
            }
        }
        // `cur` is consumed: refill it for span + 2 (clamped, so the wait
        // counts stay exact), then the barrier that publishes the next tile.
        load_w(min(span + 2, S - 1), cur);
        wait_vmcnt<HAS_Z ? 12 : 8>(); // everything but the refill: next tile + nxt
        barrier_only();
    };

    int span = 0;
    for (; span + 1 < S; span += 2) {
        run_span(span, rA, rB);
        run_span(span + 1, rB, rA);
    }
    if (span < S)
        run_span(span, rA, rB);

    // ---- epilogue: lane holds D[n = 8 g + 4 h + j][m = nl], register 4 g + j ----
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + 32 * mb + nl;
        if (m >= M)
            continue;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int n = n0 + 64 * wave + 32 * nb + 8 * g4 + 4 * h;
                if (n >= N)
                    continue;
                const float16_t &v = acc[nb][mb];
                uint2 o;
                o.x = f32x2_to_act2<DT>(v[4 * g4 + 0], v[4 * g4 + 1]);
                o.y = f32x2_to_act2<DT>(v[4 * g4 + 2], v[4 * g4 + 3]);
                *reinterpret_cast<uint2 *>(y + (size_t)m * N + n) = o;
            }
        }
    }
}

template <int DT, int MB>
hipError_t launch_mb(const W4Args &a, hipStream_t stream)
{
    constexpr int TM = 32 * MB;
    const int n_mt = (a.M + TM - 1) / TM;
    const int n_nt = (a.N + TL_TN - 1) / TL_TN;
    const int tiles = n_mt * n_nt;
    const int tiles_per_xcd = (tiles + 7) / 8;
    const int grid = 8 * tiles_per_xcd;
    const int gshift = a.g == 32 ? 0 : a.g == 64 ? 1 : 2;
    const size_t lds = (size_t)2 * TM * TL_ROWB;
    auto kern = a.qzeros ? w4a16_tiled_kernel<DT, MB, true> : w4a16_tiled_kernel<DT, MB, false>;
    // More than 64 KB of dynamic LDS must be requested per kernel (gfx950 has 160 KB per CU).
    static hipError_t attr[2] = {hipErrorNotReady, hipErrorNotReady};
    hipError_t &ae = attr[a.qzeros ? 1 : 0];
    if (ae != hipSuccess)
        ae = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (ae != hipSuccess)
        return ae;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(TL_THREADS), lds, stream,
                       static_cast<const uint16_t *>(a.x), a.qweight,
                       static_cast<const uint16_t *>(a.scales), a.qzeros,
                       static_cast<uint16_t *>(a.y), a.M, a.N, a.K, gshift, n_mt, n_nt,
                       tiles_per_xcd);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const W4Args &a, hipStream_t stream)
{
    // Tile height by M: the 256-row tile amortizes dequantization best; small
    // M uses shorter tiles so fewer padded rows are multiplied.
    if (a.M > 128)
        return launch_mb<DT, 8>(a, stream);
    if (a.M > 64)
        return launch_mb<DT, 4>(a, stream);
    if (a.M > 32)
        return launch_mb<DT, 2>(a, stream);
    return launch_mb<DT, 1>(a, stream);
}

} // namespace

hipError_t launch_w4a16_tiled(const W4Args &a, hipStream_t stream)
{
    return a.dt == DT_F16 ? launch_dt<DT_F16>(a, stream) : launch_dt<DT_BF16>(a, stream);
}

hipError_t launch_w4a16_grouped(const W4Args &, const int64_t *, int, hipStream_t)
{
    return hipErrorNotSupported;
}

} // namespace wob
