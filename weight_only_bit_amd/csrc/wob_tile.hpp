// Cooperative-tile MFMA pipeline for gfx950, shared by the dense W4A16 GEMM,
// its ragged grouped form and the MXFP4 MoE stage-1 GEMM.
//
// Mechanism (cooperative shared tile: "ROCm KQuantGemmKWmmaQ4K/Q6K: redesign
// around a cooperative shared tile, matching llama.cpp's mul_mat_q
// mechanism", sections Confirmed mechanism and The work): one workgroup owns
// a TN x TM output tile (weight rows x activation rows).  The packed weights
// of its TN rows are loaded and dequantized exactly once, split across the
// waves so no wave repeats another's work; one copy of the activation tile in
// LDS serves every wave; each wave multiplies its own weight rows against the
// whole activation range.  Dequantization and the matrix multiply are
// separate steps ("ROCm IQ4_XS keep-quant GEMM is 8.8x behind llama.cpp's
// WMMA path", section Cause), here registers -> MFMA operands.
//
// gfx950 realisation:
//  * Matrix core: blocks of BR x BR outputs, BR = 32 with
//    v_mfma_f32_32x32x16_{f16,bf16} (32 busy cycles each, measured with the
//    MFMA busy counter) or BR = 16 with v_mfma_f32_16x16x32_{f16,bf16} (16
//    cycles for half the products: the same rate).  Both forms cost the same
//    dequantization and LDS reads per product; BR = 16 halves the row
//    granularity of a tile (the grouped and MoE forms pad a group's rows to
//    whole blocks).
//  * 4 waves; wave w owns weight rows n0 + BR NB w .. +BR NB - 1 (NB BR-row
//    blocks nb) and all TM = BR MB activation rows of the tile: NB x MB
//    accumulator blocks of BR^2 / 64 fp32 registers (at most 256 of a lane's
//    512 registers in all).  TN = 4 BR NB.
//    One activation operand read from LDS feeds NB MFMAs and one dequantized
//    weight word feeds MB, so NB trades LDS reads for dequantization work.
//    Measured on MI355X, the dequantization weighs more: NB = 2 (256 x 256)
//    for W4A16; 384 weight rows for MoE experts of ~128 rows; 512 x 128 was
//    slower for both, although it moves the fewest bytes into LDS per MFMA
//    (2 TM + TN / 2 bytes per k is smallest at TN = 4 TM).
//  * K advances in spans of 128.  The G = 64 / BR lane groups g = lane / BR
//    split the span's k: lane (nl, g) = (lane % BR, lane / BR) takes the
//    128 / G k of group g of weight row nl of each block, i.e. PPL = 4 / G
//    16-byte pieces hf (32 k each): words 4 PPL g .. 4 PPL g + 4 PPL - 1 of
//    the row's span.  The span takes NS = 4 PPL MFMA steps; step s uses word
//    s of the lane's pieces: operand slot (g, e) holds k = (128 / G) g + 8 s
//    + e (BR = 32: 64 h + 8 s + e over 8 steps of 16 k; BR = 16: 32 g + 8 s
//    + e over 4 steps of 32 k).  The activation operand uses the same slots,
//    so the pairing of k values is the same on both sides.
//  * The activation tile (TM rows x 128 k, 256 bytes per row) is copied from
//    global memory straight into LDS with global_load_lds_dwordx4 (no staging
//    registers), double buffered across spans.  Within a row the 16-byte block
//    b is stored at position b ^ (row % 16), which makes the operand reads
//    (32 rows x one block each) bank-conflict free.  Rows come from a per-lane
//    byte offset supplied by the caller, so the same copy serves contiguous
//    rows and gathered (routed) rows.
//  * The packed codes of the TN weight rows (64 bytes per row per span) are
//    copied into LDS the same way, 16 rows per wave instruction, so each
//    instruction reads sixteen contiguous 64-byte row segments instead of
//    scattering 16-byte pieces of 32 rows (measured: the scattered per-lane
//    code loads cost more than a fifth of the kernel).  A lane reads back its
//    NB rows' pieces with PPL NB ds_read_b128; LDS row R keeps its 16-byte
//    piece p at position p ^ ((R >> 2) & 3), which makes those reads
//    bank-conflict free.
//  * Software pipeline: within a span the loop runs over the NS MFMA steps;
//    each step dequantizes the NB weight words it needs (one per 32-row
//    block) and issues its NB x MB MFMAs, while the next step's activation
//    operands are read from LDS and its words are dequantized.  The per-row
//    scales and zero-points are double buffered in registers and loaded a
//    whole span ahead; the next span's activation and code tiles stream into
//    the other LDS buffers.  Those copies are spread over the first steps
//    of the span, a few per step (measured: issued in one burst at the start
//    of the span they stalled the wave for a fifth of the loop), with scalar
//    LDS addresses and one vector add per copy.
//  * Tails: weight rows past the matrix are clamped to valid addresses and
//    never stored; activation rows past the tile's row count are clamped to a
//    valid row and never stored; a 32-wide K slice past K gets zero weights.
//
// Weight formats (4-bit codes, K/2 bytes per row, at `wq`) plug in as a
// policy with:
//    const uint8_t *wq;                   codes of row 0 of the matrix
//    int tile_row(int n0, int N, int t) const;  matrix row of tile row t (clamped)
//    (the policy is built for one NB and BR and addresses rows
//    BR NB w + BR nb + nl)
//    struct Meta;                         a lane's scales / zero-points of a span
//    static constexpr int NLOADS;         vector-memory operations per load_meta()
//    void begin_span(int span) const;     at a span's start, before its copies
//                                         (loads issued here are older than them)
//    static void pin(Meta &m);            at a span's start, on that span's meta
//    void load_meta(int span, Meta &m) const;
//    void zero_past_k(int span, u32x4 (&cw)[NB][PPL], Meta &m) const;
//                                         weights of slices past K -> 0 (codes or scales)
//    u32x4 dequant(uint32_t word, const Meta &m, int nb, int st) const;
#pragma once

#include "wob_device.hpp"

namespace wob {

typedef __attribute__((address_space(3))) void lds_ptr_t;
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int TL_WAVES = 4;
constexpr int TL_THREADS = 64 * TL_WAVES;
constexpr int TL_SPAN = 128; // K per span
constexpr int TL_ROWB = 256; // LDS bytes per activation row of a span

// Tile geometry for NB weight blocks of BR rows per wave.
template <int NB, int BR = 32>
struct TileGeo {
    static_assert(BR == 32 || BR == 16, "MFMA block height");
    static_assert(NB >= 2 && NB * BR <= 128, "weight blocks per wave");
    static constexpr int G = 64 / BR;               // lane groups splitting a span's k
    static constexpr int PPL = 4 / G;               // 16-byte code pieces per lane per span
    static constexpr int NS = 4 * PPL;              // MFMA steps per span
    static constexpr int ACC = BR * BR / 64;        // accumulator registers per block
    static constexpr int TN = BR * NB * TL_WAVES;   // weight rows per tile
    static constexpr int MB_MAX = 256 / (NB * ACC); // activation blocks per tile, at most
    static constexpr int TM_MAX = BR * MB_MAX;
    static constexpr int WBUF = TN * 64;            // LDS bytes of one span's code tile
    static constexpr int WDMA = TN / 64;            // code copies per wave per span
    static_assert(TN % 64 == 0, "whole code copies");
    // LDS bytes of a tile with mb BR-row blocks: two span buffers of each
    // operand, or the epilogue's staging of the output tile if larger.
    __host__ __device__ static constexpr int lds_bytes(int mb)
    {
        const int main = 2 * BR * mb * TL_ROWB + 2 * WBUF;
        const int stage = BR * mb * (2 * TN + 16 + 4); // staged rows + row-index table
        return main > stage ? main : stage;
    }
};

// Accumulator block of BR x BR outputs: BR^2 / 64 fp32 registers per lane.
template <int BR>
struct AccT {
    typedef float type __attribute__((ext_vector_type(BR * BR / 64)));
};

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

// One MFMA of a BR x BR block: A = 8 weight values of row nl (slot g), B = 8
// activation values of row nl (slot g), D[weight row][activation row].
template <int DT, int BR>
__device__ __forceinline__ typename AccT<BR>::type mfma_blk(const u32x4 &a, const u32x4 &b,
                                                            const typename AccT<BR>::type &c)
{
    if constexpr (BR == 32) {
        if constexpr (DT == DT_F16)
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<half8_t>(a), bitcast<half8_t>(b),
                                                          c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf168_t>(a),
                                                           bitcast<bf168_t>(b), c, 0, 0, 0);
    } else {
        if constexpr (DT == DT_F16)
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(a), bitcast<half8_t>(b),
                                                          c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf168_t>(a),
                                                           bitcast<bf168_t>(b), c, 0, 0, 0);
    }
}

// Lane coordinates inside the tile.
template <int BR = 32>
struct TileLane {
    int wave, lane, nl, g;
    int rl;   // activation row (mod 16) this lane copies in every DMA instruction
    int xblk; // 16-byte block of that row this lane copies
    __device__ TileLane()
    {
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // uniform: scalar LDS addresses
        lane = threadIdx.x & 63;
        nl = lane & (BR - 1);
        g = lane / BR;
        rl = 4 * wave + (lane >> 4);
        xblk = (lane & 15) ^ rl;
    }
};

// Compile-time tag of a K-loop span: the tail span (last of an odd count) or not.
template <bool TAIL>
struct SpanTail {
    static constexpr bool value = TAIL;
};

// First activation row of DMA instruction i for this lane is row 16 i + rl.
// `XRows` supplies the byte offset (from `xbase`) of activation row r of the
// tile, already clamped to a valid row:  uint32_t XRows::off(int i) const
// returns the offset of row 16 i + rl for this lane.
//
// The tile body: runs the whole K loop for one (4 BR NB) x (BR MB) tile and
// leaves the accumulators in `acc`.  `Fmt` holds this lane's weight
// addressing.
template <int DT, int NB, int MB, int BR, class Fmt, class XRows>
__device__ __forceinline__ void tile_mainloop(const Fmt &fmt, const XRows &xr,
                                              const uint8_t *xbase, int K, int n0, int N,
                                              uint8_t *smem, const TileLane<BR> &tl,
                                              typename AccT<BR>::type (&acc)[NB][MB])
{
    using GEO = TileGeo<NB, BR>;
    static_assert(MB >= 1 && MB <= GEO::MB_MAX, "accumulator budget");
    constexpr int TM = BR * MB;
    static_assert(TM % 16 == 0, "whole activation copies");
    constexpr int WD = GEO::WDMA;
    constexpr int PPL = GEO::PPL;
    constexpr int NS = GEO::NS;
    const int S = (K + TL_SPAN - 1) / TL_SPAN;
    const uint32_t lds0 = (uint32_t)(size_t)(lds_ptr_t *)smem;
    const uint32_t wlds0 = lds0 + (uint32_t)(2 * TM * TL_ROWB);
    const uint8_t *wsm = smem + 2 * TM * TL_ROWB;

    // Code tile DMA: TN rows x 64 bytes per span, 16 rows (1 KB) per wave
    // instruction, instructions WD w .. WD w + WD - 1 for wave w (WD = TN / 64).
    // Lane L writes row L / 4 of the instruction's 16 at position L % 4, so it
    // copies piece (L % 4) ^ (L / 16) of that row.  Rows past N are clamped
    // (never stored); pieces past the end of a row are clamped inside it
    // (zeroed at dequant).
    const uint32_t rowb = (uint32_t)K >> 1;
    uint32_t crow[WD];
#pragma unroll
    for (int jj = 0; jj < WD; ++jj)
        crow[jj] = (uint32_t)fmt.tile_row(n0, N, 16 * (WD * tl.wave + jj) + (tl.lane >> 2)) * rowb;
    const uint32_t cpiece = 16u * (uint32_t)((tl.lane & 3) ^ (tl.lane >> 4));

    // Activation tile DMA: TM rows x 16 blocks per span, 1 KB per wave
    // instruction.  Instruction i of wave w fills LDS rows 16 i + 4 w .. +3;
    // lane L takes row 16 i + rl and position L % 16, which holds global block
    // (L % 16) ^ rl of that row.  Blocks past K are clamped inside the row
    // (they meet zero weights).
    //
    // Copy d of a span (d < TM / 16: activation instruction d, else code
    // instruction d - TM / 16).  The per-span lane offsets kx / kw are
    // computed once per span; LDS addresses are wave-uniform (scalar).
    constexpr int ND = TM / 16 + WD;
    auto dma = [&](int d, int buf, uint32_t kx, uint32_t kw) __attribute__((always_inline)) {
        if (d < TM / 16) {
            const uint32_t ldsb = lds0 + (uint32_t)(buf * TM * TL_ROWB);
            lds_dma16(xbase, xr.off(d) + kx,
                      ldsb + (uint32_t)((16 * d + 4 * tl.wave) * TL_ROWB));
        } else {
            const int jj = d - TM / 16;
            lds_dma16(fmt.wq, crow[jj] + kw,
                      wlds0 + (uint32_t)(buf * GEO::WBUF + (WD * tl.wave + jj) * 1024));
        }
    };
    auto koff = [&](int span, uint32_t &kx, uint32_t &kw) __attribute__((always_inline)) {
        kx = 2u * (uint32_t)min(span * TL_SPAN + 8 * tl.xblk, K - 8);
        kw = min((uint32_t)span * 64u + cpiece, rowb - 16u);
    };

#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < GEO::ACC; ++e)
                acc[nb][mb][e] = 0.f;

    // Scales / zero-points double buffered: mA / mB alternate between "this
    // span" (complete) and "next span" (loads in flight).
    typename Fmt::Meta mA, mB;
    fmt.load_meta(0, mA);
    fmt.load_meta(min(1, S - 1), mB);
    {
        uint32_t kx, kw;
        koff(0, kx, kw);
#pragma unroll
        for (int d = 0; d < ND; ++d)
            dma(d, 0, kx, kw);
    }
    __builtin_amdgcn_s_waitcnt(0);
    barrier_only();

    // BR = 32: MFMAs of one step in GR groups; with group g of step st goes
    // copy GR st + g of the next span (all copies land in the first five of
    // the eight steps at the largest tiles), so the copies are spread over
    // the span instead of issued in one burst.
    constexpr int NM = NB * MB;
    constexpr int GR = NM < 4 ? NM : 4; // group g: MFMAs [g NM / GR, (g + 1) NM / GR)
    static_assert(BR != 32 || ND <= NS * GR, "every copy of the next span gets a slot");

    // One span: MFMAs on LDS buffers span & 1 with the scales in `cur`.  At
    // entry the next span's scales (the other buffer) have landed or are in
    // flight; this span's `cur` is refilled for span + 2 once consumed.
    // TAIL: the last span of an odd span count, run after the paired loop
    // (see the end of the span).
    auto run_span = [&](int span, typename Fmt::Meta &cur, auto tail) __attribute__((always_inline)) {
        const int buf = span & 1;
        fmt.begin_span(span); // loads ahead of this span's copies (see the format)
        Fmt::pin(cur);        // (see the format)
        // The next span's tiles (the last span copies itself again: no branch
        // splits the step, and the copy is waited for before the last barrier).
        uint32_t kx, kw;
        koff(min(span + 1, S - 1), kx, kw);
        const uint8_t *xb = smem + (size_t)buf * TM * TL_ROWB;
        // This lane's packed codes of the span: rows BR NB w + BR nb + nl,
        // pieces PPL g + hf (k = 32 (PPL g + hf) .. +31 of the span).
        const uint8_t *wb = wsm + buf * GEO::WBUF;
        // Activation operand of block mb, step st: BR rows (nl), 16-byte
        // block NS g + st of the span.
        auto read_x = [&](int mb, int st) __attribute__((always_inline)) {
            const int R = BR * mb + tl.nl;
            const int p = (NS * tl.g + st) ^ (R & 15);
            return *reinterpret_cast<const u32x4 *>(xb + R * TL_ROWB + 16 * p);
        };
        if constexpr (BR == 32) {
            u32x4 cw[NB][PPL];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int hf = 0; hf < PPL; ++hf) {
                    const int R = BR * NB * tl.wave + BR * nb + tl.nl;
                    const int pos = (PPL * tl.g + hf) ^ ((tl.nl >> 2) & 3);
                    cw[nb][hf] = *reinterpret_cast<const u32x4 *>(wb + R * 64 + 16 * pos);
                }
            // Only a span that crosses K (uniform test) has slices past K;
            // the format zeroes their weights once (codes or scales).
            if (span * TL_SPAN + TL_SPAN > K)
                fmt.zero_past_k(span, cw, cur);
            auto dq = [&](int nb, int st) __attribute__((always_inline)) {
                return fmt.dequant(cw[nb][st >> 2][st & 3], cur, nb, st);
            };
            u32x4 wc[NB], wn[NB], xc[MB], xn[MB];
    #pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                wc[nb] = dq(nb, 0);
    #pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                xc[mb] = read_x(mb, 0);
    #pragma unroll
            for (int st = 0; st < NS; ++st) {
                if (st < NS - 1) {
    #pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        xn[mb] = read_x(mb, st + 1);
    #pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        wn[nb] = dq(nb, st + 1);
                }
    #pragma unroll
                for (int g = 0; g < GR; ++g) {
    #pragma unroll
                    for (int j = g * NM / GR; j < (g + 1) * NM / GR; ++j)
                        acc[j % NB][j / NB] =
                            mfma_blk<DT, BR>(wc[j % NB], xc[j / NB], acc[j % NB][j / NB]);
                    if (GR * st + g < ND)
                        dma(GR * st + g, buf ^ 1, kx, kw);
                }
                // Issue order inside the step: every MFMA followed by two of the
                // next step's dequantization ops and, every second MFMA, one of its
                // LDS operand reads (measured: the compiler's own order clustered
                // up to a dozen VALU ops between two MFMAs; this order was ~1 %
                // faster on the prefill shape).
    #pragma unroll
                for (int j = 0; j < NM; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0); // two VALU
                    if (j % 2 == 1)
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // one LDS read
                }
                __builtin_amdgcn_sched_barrier(0);
                if (st < NS - 1) {
    #pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        wc[nb] = wn[nb];
    #pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        xc[mb] = xn[mb];
                }
            }
        } else {
            // BR = 16: the step's MB activation operands would double the
            // registers of the BR = 32 form, so they stream through a ring of
            // XR operands instead, read LA positions ahead along the flattened
            // order q = MB st + mb (LA = 4 measured fastest of 2 and 4); the
            // next step's weight words are dequantized across the step's
            // positions, and the copies of the next span go out over the
            // first half of the span.
            constexpr int LA = 4, XR = LA + 1;
            constexpr int NQ = NS * MB;
            constexpr int HALF = NQ / 2 > 0 ? NQ / 2 : 1;
            // The lane's single piece per block is read one 4-byte word (one
            // step) at a time, a step ahead of its dequantization, so only
            // NB code words are live instead of NB pieces.  Slices past K:
            // zero codes (a per-lane mask) or zero scales, as the format says.
            static_assert(PPL == 1, "one piece per lane");
            if (span * TL_SPAN + TL_SPAN > K) {
                if constexpr (!Fmt::ZERO_CODES) {
                    u32x4 none[NB][PPL];
                    fmt.zero_past_k(span, none, cur);
                }
            }
            const uint32_t cmask =
                (Fmt::ZERO_CODES && span * TL_SPAN + 32 * tl.g >= K) ? 0u : ~0u;
            const uint8_t *wl =
                wb + (BR * NB * tl.wave + tl.nl) * 64 + 16 * (tl.g ^ ((tl.nl >> 2) & 3));
            auto word = [&](int nb, int st) __attribute__((always_inline)) {
                return *reinterpret_cast<const uint32_t *>(wl + BR * nb * 64 + 4 * st) & cmask;
            };
            uint32_t cn[NB];
            u32x4 wc[NB], wn[NB], xr[XR];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                wc[nb] = fmt.dequant(word(nb, 0), cur, nb, 0);
                cn[nb] = word(nb, 1);
            }
#pragma unroll
            for (int q = 0; q < LA && q < NQ; ++q)
                xr[q % XR] = read_x(q % MB, q / MB);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int st = q / MB, mb = q % MB;
                if (q + LA < NQ)
                    xr[(q + LA) % XR] = read_x((q + LA) % MB, (q + LA) / MB);
                if (st < NS - 1) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        if (nb * MB / NB == mb) {
                            wn[nb] = fmt.dequant(cn[nb], cur, nb, st + 1);
                            if (st + 2 < NS)
                                cn[nb] = word(nb, st + 2);
                        }
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb][mb] = mfma_blk<DT, BR>(wc[nb], xr[q % XR], acc[nb][mb]);
#pragma unroll
                for (int d = 0; d < ND; ++d)
                    if (d * HALF / ND == q)
                        dma(d, buf ^ 1, kx, kw);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 1, 0); // one VALU
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // one LDS read
                if (mb == MB - 1) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (st < NS - 1) {
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            wc[nb] = wn[nb];
                    }
                }
            }
        }
        // `cur` is consumed: refill it for span + 2 (clamped, so the wait
        // counts stay exact), then the barrier that publishes the next tiles:
        // wait for everything but that refill (next activation and code
        // tiles + the next span's scales).  The tail span refills nothing and
        // waits for everything: its refill would be dead, the compiler drops
        // dead loads, and the count of NLOADS would then leave that many of
        // the span's copies in flight past the last barrier, landing in LDS
        // the epilogue has already reused (staged outputs, row indices).
        if constexpr (decltype(tail)::value) {
            wait_vmcnt<0>();
        } else {
            fmt.load_meta(min(span + 2, S - 1), cur);
            wait_vmcnt<Fmt::NLOADS>();
        }
        barrier_only();
    };

    int span = 0;
    for (; span + 1 < S; span += 2) {
        run_span(span, mA, SpanTail<false>{});
        run_span(span + 1, mB, SpanTail<false>{});
    }
    if (span < S)
        run_span(span, mA, SpanTail<true>{});
    // Only the last pair's (clamped, duplicate) scale refills can still be in
    // flight here; they target registers, which the compiler's own wait
    // counts cover.  Every copy into LDS has been waited for.
}

// Store one tile's accumulators through LDS, so that every global store
// instruction writes whole 512-byte row segments of y (measured: storing the
// accumulator layout directly, 8 bytes per lane across 32 rows, took about a
// twelfth of the prefill kernel).  Lane (nl, g) holds D[n = 4 G g4 + 4 g +
// j][m = nl] of block (nb, mb) in register 4 g4 + j (G = 64 / BR lane groups;
// BR = 32: n = 8 g4 + 4 g + j, g4 < 4; BR = 16: n = 4 g + j); the tile is
// staged as TM rows of TN activation-dtype values (row stride padded by 16
// bytes against bank conflicts) in the LDS the main loop has released.  The
// output rows: yr.base + yr.index(r) * yr.ld for tile row r < rows; the
// indices are read once into LDS (for gathered MoE rows each is a global
// load, which the copy loop would otherwise repeat for every 16-byte chunk).
template <int TM, class YRows>
__device__ __forceinline__ uint32_t *stage_row_index(const YRows &yr, int rows, uint8_t *tbl_lds)
{
    uint32_t *tbl = reinterpret_cast<uint32_t *>(tbl_lds);
    static_assert(TM <= TL_THREADS, "one row index per thread");
    if ((int)threadIdx.x < rows)
        tbl[threadIdx.x] = yr.index(threadIdx.x);
    return tbl;
}

template <int DT, int NB, int MB, int BR, class YRows>
__device__ __forceinline__ void tile_store(const typename AccT<BR>::type (&acc)[NB][MB],
                                          const YRows &yr, int rows, int n0, int N,
                                          const TileLane<BR> &tl, uint8_t *smem)
{
    using GEO = TileGeo<NB, BR>;
    constexpr int TN = GEO::TN;
    constexpr int TM = BR * MB;
    constexpr int RS = TN * 2 + 16; // LDS bytes per staged row
    static_assert(TM * RS + 4 * TM <= GEO::lds_bytes(MB), "staging fits the tile's LDS");
    const uint32_t *tbl = stage_row_index<TM>(yr, rows, smem + TM * RS);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = BR * mb + tl.nl;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int g4 = 0; g4 < GEO::ACC / 4; ++g4) {
                const int c = BR * NB * tl.wave + BR * nb + 4 * GEO::G * g4 + 4 * tl.g;
                const auto &v = acc[nb][mb];
                uint2 o;
                o.x = f32x2_to_act2<DT>(v[4 * g4 + 0], v[4 * g4 + 1]);
                o.y = f32x2_to_act2<DT>(v[4 * g4 + 2], v[4 * g4 + 3]);
                *reinterpret_cast<uint2 *>(smem + m * RS + 2 * c) = o;
            }
        }
    }
    __syncthreads();
    // TN / 8 chunks of 16 bytes (8 values) per staged row; N % 8 == 0, so a
    // chunk is either wholly inside the matrix or wholly past it.
    constexpr int CPR = TN / 8;
    for (int i = threadIdx.x; i < TM * CPR; i += TL_THREADS) {
        const int r = i / CPR, c = i % CPR;
        const int n = n0 + 8 * c;
        if (r < rows && n < N)
            *reinterpret_cast<u32x4 *>(yr.base + (size_t)tbl[r] * yr.ld + n) =
                *reinterpret_cast<const u32x4 *>(smem + r * RS + 16 * c);
    }
}

// Store with the fused stage-1 activation (paired layout, see FmtFP4): the
// same accumulator register of blocks nb = 2 p and 2 p + 1 holds gate and up
// of one output column, n = n0 + (BR NB / 2) w + BR p + 4 G g4 + 4 g + j, so
// out = silu(gate) * up in fp32 with silu(v) = v / (1 + e^-v), rounded once
// to the activation dtype.  Staged through LDS as for tile_store: TN / 2
// output columns per tile row.
template <int DT, int NB, int MB, int BR, class YRows>
__device__ __forceinline__ void tile_store_silu_mul(const typename AccT<BR>::type (&acc)[NB][MB],
                                                   const YRows &yr, int rows, int n0, int I,
                                                   const TileLane<BR> &tl, uint8_t *smem)
{
    using GEO = TileGeo<NB, BR>;
    constexpr int TN = GEO::TN;
    constexpr int TM = BR * MB;
    constexpr int RS = TN + 16; // LDS bytes per staged row (TN / 2 values + pad)
    const uint32_t *tbl = stage_row_index<TM>(yr, rows, smem + TM * RS);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = BR * mb + tl.nl;
#pragma unroll
        for (int p = 0; p < NB / 2; ++p)
#pragma unroll
            for (int g4 = 0; g4 < GEO::ACC / 4; ++g4) {
                const int c = (BR * NB / 2) * tl.wave + BR * p + 4 * GEO::G * g4 + 4 * tl.g;
                float o4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float g = acc[2 * p][mb][4 * g4 + j];
                    const float u = acc[2 * p + 1][mb][4 * g4 + j];
                    o4[j] = g / (1.0f + expf(-g)) * u;
                }
                uint2 o;
                o.x = f32x2_to_act2<DT>(o4[0], o4[1]);
                o.y = f32x2_to_act2<DT>(o4[2], o4[3]);
                *reinterpret_cast<uint2 *>(smem + m * RS + 2 * c) = o;
            }
    }
    __syncthreads();
    constexpr int CPR = TN / 16;
    for (int i = threadIdx.x; i < TM * CPR; i += TL_THREADS) {
        const int r = i / CPR, c = i % CPR;
        const int n = n0 + 8 * c;
        if (r < rows && n < I)
            *reinterpret_cast<u32x4 *>(yr.base + (size_t)tbl[r] * yr.ld + n) =
                *reinterpret_cast<const u32x4 *>(smem + r * RS + 16 * c);
    }
}

// Zero rows [0, rows) of a tile's WIDTH-column range (expert rows whose id is
// out of range).
template <int WIDTH, class YRows>
__device__ __forceinline__ void tile_store_zero(const YRows &yr, int rows, int n0, int N)
{
    for (int i = threadIdx.x; i < rows * (WIDTH / 4); i += TL_THREADS) {
        const int r = i / (WIDTH / 4);
        const int n = n0 + 4 * (i % (WIDTH / 4));
        if (n < N)
            *reinterpret_cast<uint2 *>(yr.row(r) + n) = uint2{0u, 0u};
    }
}

// XCD-aware tile order: workgroups are dealt to the device's `nxcd` XCDs
// round-robin (workgroup b runs on XCD b % nxcd); each XCD takes a contiguous
// run of the `tiles` tile indices, so the tiles that share an operand (as the
// caller orders them) share it in that XCD's L2.  The grid holds
// nxcd * ceil(tiles / nxcd) workgroups; returns -1 for those beyond the run.
__device__ __forceinline__ int xcd_tile(int tiles, int nxcd)
{
    const int per_xcd = (tiles + nxcd - 1) / nxcd;
    const int b = blockIdx.x;
    const int j = b / nxcd;
    if (j >= per_xcd)
        return -1;
    const int t = (b - j * nxcd) * per_xcd + j;
    return t < tiles ? t : -1;
}

// Weight format policies -------------------------------------------------------

// W4A16: packed codes qweight[N][K/8], scales[N][K/g] in DT, packed
// zero-points qzeros[N/8][K/g] (or none: z = 8).  Each lane handles rows
// n_nb = n0 + BR NB wave + BR nb + nl, which share n % 8, so one nibble shift
// of the zero-point words serves all its blocks.  A lane's k of a span are
// PPL 32-wide slices hf (k = 32 (PPL g + hf) ..), each inside one group.
// GM (group mode): 0 for g = 32; 1 for g >= 64; 2 for g = 128 with an even
// number of groups G >= 4 per row.
template <int DT, bool HAS_Z, int NB, int GM, int BR = 32>
struct FmtW4 {
    static constexpr int PPL = TileGeo<NB, BR>::PPL;
    // GW: every group spans at least 64 k (g >= 64), so a lane's two 32-wide
    // slices of a span (BR = 32) share one scale and one zero-point word: one
    // load each.
    static constexpr bool GW = GM >= 1;
    // S4 (g = 128, BR = 32: a span is one group): a lane's scales of four
    // consecutive spans are 8 contiguous bytes of its row, loaded together
    // every four spans into `sb` (two dword loads per block, issued before the
    // span's tile copies) instead of one 2-byte load per span, each of which
    // touches a cache line per row of the block.
    static constexpr bool S4 = GM == 2;
    static_assert(!S4 || BR == 32, "a span is one group");
    static constexpr int LPS = GW ? 1 : PPL; // loads per block per span
    static constexpr int NLOADS = NB * ((HAS_Z ? 1 : 0) + (S4 ? 0 : 1)) * LPS;
    static constexpr bool ZERO_CODES = false; // slices past K: zero scales
    struct Meta {
        uint32_t s[NB][PPL], z[NB][PPL];
    };
    // bfloat16, g = 32: the span's meta (loaded at the end of span - 2) is
    // pinned at the start of its span (no instruction), so the compiler
    // cannot compute its zero-point bias pairs and scales at the start of
    // span - 1, right after the barrier that follows the loads, where that
    // waited for them.  (Pinned in binary16, or with g = 128, the loads went
    // through copies placed at the same spot instead.)
    __device__ __forceinline__ static void pin(Meta &m)
    {
        if constexpr (SDW) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int hf = 0; hf < PPL; ++hf)
                    asm volatile("" : "+v"(m.s[nb][hf]), "+v"(m.z[nb][hf]));
        }
    }
    const uint8_t *wq, *ws, *wz;
    uint32_t soff[NB], zoff[NB];
    // bfloat16 with g = 32: each scale is loaded as the aligned dword holding
    // it, so the value stays 32 bits wide (a 2-byte load was narrowed and
    // widened again right after the span barrier, which waited for the load
    // there).  ssh: bit offset of slice 0's scale in its dword, the same for
    // every span (its group 4 span + 2 g is even); slice 1's is 16 - ssh.
    static constexpr bool SDW = DT == DT_BF16 && GM == 0;
    uint32_t ssh[NB];
    int K, gshift, g, zsh, G;
    // S4: scales of groups sb_base .. sb_base + 3 (binary16 pairs per block)
    mutable uint32_t sb[NB][2];
    mutable int sb_base;

    __device__ FmtW4(const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                     int N, int K_, int gshift_, int n0, const TileLane<BR> &tl)
    {
        wq = reinterpret_cast<const uint8_t *>(qweight);
        ws = reinterpret_cast<const uint8_t *>(scales);
        wz = reinterpret_cast<const uint8_t *>(qzeros);
        K = K_;
        gshift = gshift_;
        g = tl.g;
        zsh = 4 * (tl.nl & 7);
        G = K >> (5 + gshift);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = min(n0 + BR * NB * tl.wave + BR * nb + tl.nl, N - 1);
            soff[nb] = (uint32_t)n * (uint32_t)G * 2u;
            zoff[nb] = (uint32_t)(n >> 3) * (uint32_t)G * 4u;
            ssh[nb] = 16u * ((soff[nb] >> 1) & 1u);
        }
        if constexpr (S4)
            load_batch(0);
    }

    // S4: the scales of groups b .. b + 3 (b = min(4 t, G - 4): inside the row).
    // Rows are 2 G bytes (G even) and b is even, so both dwords are aligned.
    __device__ __forceinline__ void load_batch(int b) const
    {
        sb_base = b;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(ws + soff[nb] + 2u * (uint32_t)b);
            sb[nb][0] = p[0];
            sb[nb][1] = p[1];
        }
    }

    // Called at the start of every span, before its tile copies.  S4: span
    // 4 t + 2 refills `sb` with the batch of spans 4 t + 4 .. 4 t + 7, whose
    // meta load_meta reads from the end of that span on; the last read of the
    // previous batch (meta of span 4 t + 3) happened at the end of span 4 t + 1.
    __device__ __forceinline__ void begin_span(int span) const
    {
        if constexpr (S4) {
            if ((span & 3) == 2)
                load_batch(min(4 * ((span >> 2) + 1), G - 4));
        }
    }

    __device__ __forceinline__ int tile_row(int n0, int N, int t) const { return min(n0 + t, N - 1); }

    __device__ __forceinline__ void load_meta(int span, Meta &m) const
    {
#pragma unroll
        for (int hf = 0; hf < LPS; ++hf) {
            const int k = span * TL_SPAN + 32 * (PPL * g + hf);
            const int kc = min(k, K - 32); // slice past K: clamped load, scale zeroed at use
            const uint32_t grp = (uint32_t)(kc >> (5 + gshift));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if constexpr (S4) {
                    // group `span` (< G: the caller clamps the span) of the batch
                    const int idx = span - sb_base;
                    const uint32_t w2 = (idx & 2) ? sb[nb][1] : sb[nb][0];
                    m.s[nb][hf] = (idx & 1) ? w2 >> 16 : w2 & 0xFFFFu;
                } else if constexpr (SDW) {
                    // In bounds: the scale array is a multiple of 16 bytes.
                    m.s[nb][hf] = *reinterpret_cast<const uint32_t *>(ws + ((soff[nb] + 2u * grp) & ~3u));
                } else {
                    m.s[nb][hf] = *reinterpret_cast<const uint16_t *>(ws + soff[nb] + 2u * grp);
                }
                m.z[nb][hf] = HAS_Z ? *reinterpret_cast<const uint32_t *>(wz + zoff[nb] + 4u * grp)
                                    : 0x88888888u;
            }
        }
#pragma unroll
        for (int hf = LPS; hf < PPL; ++hf)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                m.s[nb][hf] = m.s[nb][0]; // separate copies: the tail zeroes them per slice
                m.z[nb][hf] = m.z[nb][0];
            }
    }

    // Slices past K: zero scales ((q - z) * 0 is a zero of either sign).
    __device__ __forceinline__ void zero_past_k(int span, u32x4 (&)[NB][PPL], Meta &m) const
    {
#pragma unroll
        for (int hf = 0; hf < PPL; ++hf)
            if (span * TL_SPAN + 32 * (PPL * g + hf) >= K)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    m.s[nb][hf] = 0u;
    }

    __device__ __forceinline__ u32x4 dequant(uint32_t word, const Meta &m, int nb, int st) const
    {
        const int hf = st >> 2;
        const uint32_t z = (m.z[nb][hf] >> zsh) & 0xFu;
        uint32_t sbits = m.s[nb][hf];
        if constexpr (SDW)
            sbits >>= hf == 0 ? ssh[nb] : 16u - ssh[nb];
        return w4_word_act8<DT>(word, sbits, z);
    }
};

// MXFP4: E2M1 codes w_fp4[N][K/2] (even k in the low nibble), E8M0 scales
// w_scale[N][K/32]; needs K % 64 == 0, so that with BR = 32 a lane's two
// 32-wide slices share one aligned 16-bit scale load (BR = 16: one slice,
// one byte).
//
// Paired layout (PAIRED, for the fused gate/up activation): the tile's
// weight rows come in pairs, gate row j and up row N/2 + j, so that block
// nb = 2 p of wave w holds gate rows n0 + (BR NB / 2) w + BR p .. +BR-1 and
// block 2 p + 1 the matching up rows; tile row t = BR NB w + BR nb + i maps
// to matrix row (nb % 2) * N/2 + n0 + (BR NB / 2) w + BR (nb / 2) + i.
template <bool PAIRED, int NB, int BR = 32>
struct FmtFP4 {
    static_assert(!PAIRED || NB % 2 == 0, "gate / up blocks come in pairs");
    static constexpr int PPL = TileGeo<NB, BR>::PPL;
    static constexpr int NLOADS = NB;
    static constexpr bool ZERO_CODES = true; // slices past K: zero codes
    struct Meta {
        // BR = 32: the aligned dword holding the lane's E8M0 pair (slices
        // hf = 0, 1 at bytes sh / 8, sh / 8 + 1); BR = 16: the byte
        uint32_t s[NB];
    };
    __device__ __forceinline__ static void pin(Meta &) {}
    const uint8_t *wq, *ws;
    uint32_t soff[NB];
    uint32_t sh[NB]; // BR = 32: bit offset of the pair in its dword (0 or 16)
    // BR = 32: the lane reads the pair of lane group gs (its own group g,
    // except at K = 64, where group 1 has no pair inside K and reads group
    // 0's), up to span slast, the last with that pair inside K; later spans
    // reuse that dword (their codes are zero).  Clamping the span, not k,
    // keeps the pair's offset in its dword: a pair clamped to the row's last
    // k of the other lane group sat 2 bytes off, which made the load
    // unaligned and 2 bytes past the row (past the array on its last row, and
    // before it on its first row at K = 64).
    int gs, slast;
    int K, g;

    __device__ FmtFP4(const uint8_t *w_fp4, const uint8_t *w_scale, int N, int K_, int n0,
                      const TileLane<BR> &tl)
    {
        wq = w_fp4;
        ws = w_scale;
        K = K_;
        g = tl.g;
        gs = K >= 128 ? g : 0;
        slast = ((K >> 5) - 2 - 2 * gs) >> 2; // pair 4 s + 2 gs <= K / 32 - 2
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = tile_row(n0, N, BR * NB * tl.wave + BR * nb + tl.nl);
            soff[nb] = (uint32_t)n * (uint32_t)(K >> 5);
            // The pair's address soff + 4 span + 2 gs is even; its dword starts
            // 0 or 2 bytes before it, the same for every span of the lane.
            sh[nb] = 8u * ((soff[nb] + 2u * (uint32_t)gs) & 2u);
        }
    }

    // Matrix row of tile row t; PAIRED: t = BR NB w + BR nb + i is row
    // (nb % 2) * N/2 + n0 + (BR NB / 2) w + BR (nb / 2) + i (gate rows, then
    // the matching up rows).
    __device__ __forceinline__ int tile_row(int n0, int N, int t) const
    {
        if constexpr (!PAIRED) {
            return min(n0 + t, N - 1);
        } else {
            const int half = N >> 1;
            const int w = t / (BR * NB), nb = (t / BR) % NB;
            return (nb & 1) * half +
                   min(n0 + (BR * NB / 2) * w + BR * (nb >> 1) + (t & (BR - 1)), half - 1);
        }
    }

    __device__ __forceinline__ void begin_span(int) const {}

    __device__ __forceinline__ void load_meta(int span, Meta &m) const
    {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            // BR = 32: the whole aligned dword, so the value stays 32 bits wide
            // (a 2-byte load was narrowed and widened again right after the
            // span barrier, which waited for the load there).  In bounds: the
            // pair lies in the row and the scale array is a multiple of 32
            // bytes, so a pair at a multiple of 4 is never its last 2 bytes.
            if constexpr (PPL == 2) {
                const uint32_t kg = 4u * (uint32_t)min(span, slast) + 2u * (uint32_t)gs;
                m.s[nb] = *reinterpret_cast<const uint32_t *>(ws + soff[nb] + kg - sh[nb] / 8u);
            } else {
                // past K: clamped to the row's last byte, zeroed codes
                const int k = min(span * TL_SPAN + 32 * g, K - 32);
                m.s[nb] = ws[soff[nb] + ((uint32_t)k >> 5)];
            }
        }
    }

    // Slices past K: zero codes (E2M1 code 0 is +0).  K % 64 == 0, so with
    // BR = 32 both 32-wide slices of a lane are inside K or both past it.
    __device__ __forceinline__ void zero_past_k(int span, u32x4 (&cw)[NB][PPL], Meta &) const
    {
        if (span * TL_SPAN + 32 * PPL * g >= K)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int hf = 0; hf < PPL; ++hf)
                    cw[nb][hf] = u32x4{0u, 0u, 0u, 0u};
    }

    __device__ __forceinline__ u32x4 dequant(uint32_t word, const Meta &m, int nb, int st) const
    {
        const int hf = st >> 2;
        const uint32_t bit = PPL == 2 ? sh[nb] + 8u * (uint32_t)hf : 0u;
        const float scale = e8m0_to_f32((m.s[nb] >> bit) & 0xFFu);
        return fp4_word_bf16x8(word, scale);
    }
};

} // namespace wob
