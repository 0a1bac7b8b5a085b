// Skinny W4A16 GEMV for M <= 8 (decode and small batch) on gfx950.
//
// The zero-point page ("Keep W4A16 zero-points packed at 4 bits instead of
// expanding to 2 bytes", sections Problem and Known regression) establishes
// that this kernel sits at the memory roofline: its time follows the bytes it
// streams (packed codes, scales and packed zero-points), and at batch 4 with
// g = 128 the nibble extraction shows up as compute when loads and math do not
// overlap.  The design below therefore
//   * reads every weight byte exactly once with 16-byte coalesced loads,
//   * issues a batch of U independent loads per lane before any math on them,
//     so U * 16 bytes per lane stay in flight,
//   * keeps the zero-points packed and extracts the nibble in registers,
//   * forms each weight's exact (q - z) in registers and multiplies it with
//     packed binary16 or bfloat16 dot products, so every product is exact
//     and the sums round only at the size of their own terms.
//
// Work decomposition.  A wavefront owns RO row octets (an octet is 8
// consecutive rows, the rows that share one packed zero-point word) and one
// contiguous range of 32-value K chunks; `ksplit` waves of a workgroup split K
// for the same octets.  Lane (r, q) = (lane/8, lane%8) handles row r of each of
// its octets and the chunks c0 + q + 8*i of its range, so each load
// instruction covers eight 128-byte row segments, and the activations of a
// chunk are read from LDS once for all RO rows of the lane.  One chunk is one 16-byte load (four words, 32 codes) and
// lies inside a single quantization group for every g in {32, 64, 128}.
//
// Prologue.  The workgroup stages X (in word order, see wob_device.hpp) and
// the scales and packed zero-point words of its rows in LDS with a few coalesced 16-byte loads per thread.  Each wave issues its
// first batch of weight loads before it waits for the staging loads, so the
// prologue latency hides behind weight traffic.  The per-chunk metadata then
// costs two LDS reads instead of two small global loads.  With K split over
// the waves (few rows, long rows) the scales are not staged: each lane loads
// its chunk's scale next to the weights, through the ring, with an ordinary
// cached load (a non-temporal one refetched the line for every 16 bytes and
// ran slower).  On the 1 x 5376 x 21504 shape this is what lets three
// workgroups share a CU instead of two (LDS), so the grid of 672 workgroups
// runs in one generation (21.1 -> 16.8 us measured).
//
// Arithmetic: each word becomes four pairs of exact (q - z) values in the
// activation dtype (binary16: one and-or per pair places two codes under the
// exponent byte of 1024 and one packed add of -(1024 + z) per pair removes
// the bias; bfloat16: byte-to-float conversions, an fp32 subtract and a pack),
// which v_dot2_f32_f16 / v_dot2_f32_bf16 multiply with the activation pairs.
// The odd codes stay in their high nibbles (16 q, no shift) and are read at
// their plain value (under the binary16 exponent of 64, or by an exact fma
// with 1/16 in fp32).
// |q - z| <= 15 has four significant bits, so every product is exact in fp32;
// each chunk's sum of products sum_k (q_k - z) x_k is scaled once by its s.
// The sums round only at the size of their own terms: weights that dequantize
// to zero give exact zeros whatever the activations.  About 1.9 vector
// operations per weight at M = 1 (binary16), counting the scale, zero-point
// and address work.
//
// Measured alternatives (MI355X, one box, decode 1 x 43008 x 5376): folding
// the zero-point out of the sums as sum (B + q) x - (B + z) sum x with the
// biased codes as operands costs 1.4 operations per weight (23.5 us against
// 25.9 us) but rounds at B times the size of the terms: with B = 1024 (the
// exponent-byte trick) weights that dequantize to zero under activations with
// 1e3 outliers miss the parity bound 15-fold; B = 16 (codes shifted under the
// exponent of 16) stays inside it at half the bound and runs slower (26.7 us:
// its and-or pairs do not fuse); B = 0 (codes as binary16 subnormals) runs
// into v_dot2c_f32_f16's reduced precision on subnormal operands (errors of
// 2^-16 relative to the activations, against 2^-24 with normal operands).
//
// Weight loads stream through a ring of D chunk slots: computing chunk i frees
// its slot, which immediately receives the load of chunk i + D.  One load is
// issued per chunk computed, so each wave's requests stay smooth instead of
// bursty (measured: batches of several chunks per issue point run slower),
// and D - 1 chunks per row stay in flight while a chunk is computed (D = 3;
// 6 ran slower on the split-K shapes measured).  When fewer than D chunks remain
// after the ring's contents, they are loaded into slots as these free up, so
// a short row's last chunks are not fetched one round trip at a time.
// Partial sums are reduced over the 8 lanes of a row with cross-lane moves
// and, for ksplit > 1, over waves through LDS.
#include "wob_device.hpp"
#include "wob_internal.hpp"

namespace wob {
namespace {

constexpr int SK_WAVES = 4;     // waves per workgroup when K is split
constexpr int SK_MAX_WAVES = 8; // largest workgroup
constexpr int SK_MAX_THREADS = 64 * SK_MAX_WAVES;
constexpr int SK_LDS_BUDGET = 64 * 1024;
constexpr int SK_RING = 3; // chunk slots per row in the load ring

// Prologue register budget: loads per thread issued before the first wait.
constexpr int SK_XR = 4; // X blocks (covers M*K <= 8192)
constexpr int SK_SR = 3; // 16-byte scale blocks
constexpr int SK_ZR = 3; // zero-point words

// LDS carve-up, in bytes, shared by the kernel and the host-side size check.
// Scales are staged only when `sc_lds` (see the kernel's SG parameter).
struct SkLds {
    int x, sc, zp, red, total;
    __host__ __device__ SkLds(int M, int K, int G, int octs_per_wg, bool sc_lds)
    {
        const int RB = ((K + 255) >> 8) * 32; // 16-byte blocks per X row
        x = 0;
        sc = x + M * RB * 16;
        zp = sc + (sc_lds ? ((octs_per_wg * 8 * G * 2 + 15) & ~15) : 0);
        red = zp + ((octs_per_wg * G * 4 + 15) & ~15);
        total = red + SK_MAX_WAVES * 2 * M * 8 * 4; // up to two octets per wave
    }
};

// Occupancy target per SIMD: enough resident waves for one wave generation on
// the decode shapes (fewer for the register-heavy larger M).
template <int M, int RO>
constexpr int sk_min_waves() { return RO == 2 ? 3 : (M <= 2 ? 4 : 2); }

// SG: scales are read from global memory with the weights (one 2-byte load
// per row and chunk, through the same ring) instead of being staged in LDS.
// Used with split K, where the staged scales would cost a resident
// workgroup per CU on long rows.
template <int DT, int M, int D, int GS, bool HAS_Z, int RO, bool SG>
__global__ __launch_bounds__(SK_MAX_THREADS, (sk_min_waves<M, RO>())) void w4a16_skinny_kernel(
    const uint16_t *__restrict__ x, const uint32_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros,
    uint16_t *__restrict__ y, int N, int K, int ksplit)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int C = K >> 5;  // chunks per row
    const int G = C >> GS; // groups per row
    const int RB = ((K + 255) >> 8) * 32;
    const int NO = N >> 3; // row octets
    const int nthr = blockDim.x; // 64 * waves of this workgroup
    const int octs_per_wg = (nthr >> 6) / ksplit * RO;
    const SkLds L(M, K, G, octs_per_wg, !SG);
    u32x4 *xl = reinterpret_cast<u32x4 *>(smem + L.x);
    uint16_t *sl = reinterpret_cast<uint16_t *>(smem + L.sc);
    uint32_t *zl = reinterpret_cast<uint32_t *>(smem + L.zp);
    float *red = reinterpret_cast<float *>(smem + L.red);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int oct0 = blockIdx.x * octs_per_wg;
    const int nocts = min(octs_per_wg, NO - oct0);

    // ---- prologue loads: X, scales, zero-points (unconditional, clamped) ----
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(x);
    const int nvec = (M * K) >> 3;
    u32x4 xr[SK_XR];
#pragma unroll
    for (int t = 0; t < SK_XR; ++t)
        xr[t] = xs[min(tid + nthr * t, nvec - 1)];
    const u32x4 *ss = reinterpret_cast<const u32x4 *>(scales + (size_t)oct0 * 8 * G);
    const int nsb = nocts * G; // 16-byte blocks of this workgroup's scales
    u32x4 sr[SK_SR];
    if constexpr (!SG) {
#pragma unroll
        for (int t = 0; t < SK_SR; ++t)
            sr[t] = ss[min(tid + nthr * t, nsb - 1)];
    }
    const uint32_t *zs = HAS_Z ? qzeros + (size_t)oct0 * G : nullptr;
    const int nzw = nocts * G;
    uint32_t zr[SK_ZR];
    if constexpr (HAS_Z) {
#pragma unroll
        for (int t = 0; t < SK_ZR; ++t)
            zr[t] = zs[min(tid + nthr * t, nzw - 1)];
    }

    // ---- this wave's work ----
    const int woct = (wave / ksplit) * RO; // first octet of this wave within the workgroup
    const int oct = oct0 + woct;
    const int ks = wave % ksplit;
    const int r = lane >> 3;
    const int q = lane & 7;
    const int cper = ((C + ksplit - 1) / ksplit + 7) & ~7;
    const int c0 = ks * cper;
    const int c1 = min(C, c0 + cper);
    const int jf = c0 + q; // this lane's first chunk
    const int n_it = (oct < NO && jf < c1) ? (c1 - jf + 7) >> 3 : 0;
    const int jfc = min(jf, C - 1);
    const u32x4 *wp[RO];    // row r of each octet (clamped into the matrix)
    const uint16_t *sg[RO]; // its scale of chunk jfc (SG)
#pragma unroll
    for (int o = 0; o < RO; ++o) {
        const size_t row = (size_t)(min(oct + o, NO - 1) * 8 + r);
        wp[o] = reinterpret_cast<const u32x4 *>(qweight + row * (K >> 3)) + jfc;
        sg[o] = scales + row * G + (jfc >> GS);
    }
    constexpr int SU = 8 >> GS; // scale / zero-point index step per chunk step of 8

    // Weight (and, with SG, scale) loads of this lane's chunk i into a ring slot.
    auto load_chunk = [&](u32x4(&w)[RO], uint32_t(&sv)[RO], int i) {
#pragma unroll
        for (int o = 0; o < RO; ++o) {
            w[o] = __builtin_nontemporal_load(wp[o] + 8 * i);
            if constexpr (SG)
                sv[o] = sg[o][SU * i]; // cached: later chunks of the wave read the same line
        }
    };
    // Fill the ring with chunks 0..D-1 before any wait (clamped into the row).
    u32x4 ring[D][RO];
    uint32_t sring[D][RO]; // raw scale bits (SG only)
#pragma unroll
    for (int d = 0; d < D; ++d)
        load_chunk(ring[d], sring[d], min(d, max(n_it - 1, 0)));
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage X (word order, conflict-free block layout) ----
    const int rowblk = K >> 3;
#pragma unroll
    for (int t = 0; t < SK_XR; ++t) {
        const int i = tid + nthr * t;
        if (i < nvec) {
            const int m = i / rowblk;
            const int tb = i - m * rowblk;
            const int j = tb >> 2, wi = tb & 3;
            xl[m * RB + (j >> 3) * 32 + wi * 8 + (j & 7)] = to_word_order(xr[t]);
        }
    }
    {
        if constexpr (!SG) {
            u32x4 *sd = reinterpret_cast<u32x4 *>(sl);
#pragma unroll
            for (int t = 0; t < SK_SR; ++t) {
                const int i = tid + nthr * t;
                if (i < nsb)
                    sd[i] = sr[t];
            }
        }
        if constexpr (HAS_Z) {
#pragma unroll
            for (int t = 0; t < SK_ZR; ++t) {
                const int i = tid + nthr * t;
                if (i < nzw)
                    zl[i] = zr[t];
            }
        }
    }
    // Large M * K (long rows): whatever did not fit the prologue registers,
    // SK_XR loads per thread at a time so their latencies overlap (one load
    // per iteration serialized a dozen L2 round trips on 1 x 21504 rows).
    for (int i0 = tid + nthr * SK_XR; i0 < nvec; i0 += nthr * SK_XR) {
        u32x4 v[SK_XR];
#pragma unroll
        for (int t = 0; t < SK_XR; ++t)
            v[t] = xs[min(i0 + nthr * t, nvec - 1)];
#pragma unroll
        for (int t = 0; t < SK_XR; ++t) {
            const int i = i0 + nthr * t;
            if (i < nvec) {
                const int m = i / rowblk;
                const int tb = i - m * rowblk;
                const int j = tb >> 2, wi = tb & 3;
                xl[m * RB + (j >> 3) * 32 + wi * 8 + (j & 7)] = to_word_order(v[t]);
            }
        }
    }
    if constexpr (!SG) {
        for (int i = tid + nthr * SK_SR; i < nsb; i += nthr)
            reinterpret_cast<u32x4 *>(sl)[i] = ss[i];
    }
    if constexpr (HAS_Z) {
        for (int i = tid + nthr * SK_ZR; i < nzw; i += nthr)
            zl[i] = zs[i];
    }
    __syncthreads();

    float acc[RO][M];
#pragma unroll
    for (int o = 0; o < RO; ++o)
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[o][m] = 0.f;
    // octets of this wave that exist (the last workgroup may be partial)
    const int ro_valid = min(RO, NO - oct);

    if (n_it > 0) {
        // this lane's LDS data: X blocks of chunk jf + 8 i, word wi at 32 i + 8 wi
        const u32x4 *xb0 = xl + (jf >> 3) * 32 + (jf & 7);
        const uint16_t *sp = sl + (woct * 8 + r) * G + (jf >> GS); // octet o: + 8 G o
        const uint32_t *zp = zl + woct * G + (jf >> GS);            // octet o: + G o

        auto chunk = [&](int i, const u32x4(&wv)[RO], const uint32_t(&sv)[RO]) {
            // unpack every row's (q - z) pairs first; then, per activation
            // row, read that row's X blocks once and use them for all RO rows
            u32x4 pr[RO][4];
            float sc[RO];
#pragma unroll
            for (int o = 0; o < RO; ++o) {
                sc[o] = act_to_f32<DT>(SG ? (uint16_t)sv[o] : sp[8 * G * o + SU * i]);
                const uint32_t z = HAS_Z ? nib(zp[G * o + SU * i], r) : 8u;
                if constexpr (DT == DT_F16) {
                    const uint32_t nb2 = f16_neg_bias2(z), nb2h = f16_neg_bias2_hi(z);
#pragma unroll
                    for (int wi = 0; wi < 4; ++wi)
                        pr[o][wi] = w4_diff_pairs_f16(wv[o][wi], nb2, nb2h);
                } else {
                    const float zf = (float)z;
#pragma unroll
                    for (int wi = 0; wi < 4; ++wi)
                        pr[o][wi] = w4_diff_pairs_bf16(wv[o][wi], zf);
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                u32x4 xv[4];
#pragma unroll
                for (int wi = 0; wi < 4; ++wi)
                    xv[wi] = xb0[m * RB + 32 * i + 8 * wi];
#pragma unroll
                for (int o = 0; o < RO; ++o) {
                    float a = 0.f;
#pragma unroll
                    for (int wi = 0; wi < 4; ++wi) {
                        const u32x4 x4 = xv[wi];
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            if constexpr (DT == DT_F16)
                                a = __builtin_amdgcn_fdot2(bitcast<half2_t>(pr[o][wi][p]), bitcast<half2_t>(x4[p]), a, false);
                            else
                                a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf162_t>(pr[o][wi][p]), bitcast<bf162_t>(x4[p]), a, false);
                        }
                    }
                    acc[o][m] = fmaf(sc[o], a, acc[o][m]);
                }
            }
        };
        // Steady state: compute chunk i + d from slot d, then refill the slot
        // with chunk i + d + D.  Loads here are unconditional so the wait
        // counts stay exact; the scheduling barriers keep the compiler from
        // moving a refill across the computation it should overlap.
        // The refill addresses advance by one pointer step per iteration, so
        // the D loads of an iteration differ by immediate offsets.
        int i = 0;
        const u32x4 *wq[RO];
        const uint16_t *sq[RO];
#pragma unroll
        for (int o = 0; o < RO; ++o) {
            wq[o] = wp[o] + 8 * D; // chunk i + D of this lane at i = 0
            sq[o] = sg[o] + SU * D;
        }
        for (; i + 2 * D <= n_it; i += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                chunk(i + d, ring[d], sring[d]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int o = 0; o < RO; ++o) {
                    ring[d][o] = __builtin_nontemporal_load(wq[o] + 8 * d); // chunk i + d + D
                    if constexpr (SG)
                        sring[d][o] = sq[o][SU * d];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int o = 0; o < RO; ++o) {
                wq[o] += 8 * D;
                sq[o] += SU * D;
            }
        }
        // Drain: the ring holds chunks i .. i+D-1 (those below n_it) and fewer
        // than D chunks follow them.  Those are loaded into the slots as they
        // free up (addresses clamped to the last chunk, so the loads stay
        // unconditional), so they too are in flight together rather than
        // one round trip each.
        if (__any(i + D < n_it)) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (i + d < n_it)
                    chunk(i + d, ring[d], sring[d]);
                __builtin_amdgcn_sched_barrier(0);
                load_chunk(ring[d], sring[d], min(i + D + d, n_it - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (i + D + d < n_it)
                    chunk(i + D + d, ring[d], sring[d]);
        } else {
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (i + d < n_it)
                    chunk(i + d, ring[d], sring[d]);
        }
    }

    // Reduce over the 8 lanes of a row.
#pragma unroll
    for (int o = 0; o < RO; ++o)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float v = acc[o][m];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            acc[o][m] = v;
        }

    if (ksplit == 1) {
        if (q == 0) {
#pragma unroll
            for (int o = 0; o < RO; ++o) {
                if (o >= ro_valid)
                    break;
#pragma unroll
                for (int m = 0; m < M; ++m)
                    y[(size_t)m * N + (oct + o) * 8 + r] = f32_to_act<DT>(acc[o][m]);
            }
        }
        return;
    }
    if (q == 0) {
#pragma unroll
        for (int o = 0; o < RO; ++o)
#pragma unroll
            for (int m = 0; m < M; ++m)
                red[((wave * RO + o) * M + m) * 8 + r] = acc[o][m];
    }
    __syncthreads();
    if (ks == 0 && q == 0) {
#pragma unroll
        for (int o = 0; o < RO; ++o) {
            if (o >= ro_valid)
                break;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float v = 0.f;
                for (int w = 0; w < ksplit; ++w)
                    v += red[(((wave + w) * RO + o) * M + m) * 8 + r];
                y[(size_t)m * N + (oct + o) * 8 + r] = f32_to_act<DT>(v);
            }
        }
    }
}

// Launch shape: RO octets per wave, `waves` waves per workgroup, K split
// `ksplit` ways across the waves of a workgroup.
struct SkCfg {
    int ro, waves, ksplit;
};

// `cus`: compute units of the device (the workgroups are spread over them).
SkCfg sk_config(int M, int N, int K, int cus)
{
    const int octs = N / 8;
    const int C = K / 32;
    // Enough row octets to fill the chip without splitting K: pick the
    // octets-per-wave and workgroup size that spread the work most evenly over
    // the compute units (each CU streams at a bounded rate, so the CU with the
    // most workgroups sets the kernel time; measured on the decode shape, the
    // CUs holding one workgroup more than the others finished last).
    if (octs >= 16 * cus) {
        SkCfg best{1, SK_WAVES, 1};
        double best_eff = -1.0;
        for (int ro = 1; ro <= (M <= 2 ? 2 : 1); ++ro) {
            const int units = (octs + ro - 1) / ro;
            for (int w = SK_MAX_WAVES; w >= 2; --w) {
                const int wgs = (units + w - 1) / w;
                const int per_cu = (wgs + cus - 1) / cus;
                const double eff = (double)octs / ((double)cus * per_cu * w * ro);
                if (eff > best_eff + 1e-9) {
                    best_eff = eff;
                    best = SkCfg{ro, w, 1};
                }
            }
        }
        return best;
    }
    // Few row octets: split K across the waves of a workgroup (up to 8 ways,
    // one octet per workgroup beyond 4), keeping at least two chunks per
    // lane.  On 1 x 5376 x 21504 the 8-way split (21 waves per CU instead of
    // 10.5) ran 17.3 -> 15.9 us; splitting the 1 x 16384 x 5376 shape 3 or 4
    // ways instead of 2 was slower (12.7 and 13.6 against 11.5 us).
    int ksplit = 1;
    while (ksplit < SK_MAX_WAVES && octs * ksplit < 4096 && C >= 16 * ksplit * 2)
        ksplit *= 2;
    // Enough work for two 8-wave workgroups per CU: take 8 waves (more
    // octets per workgroup), so fewer workgroups each stage the whole of X
    // (1 x 16384 x 5376: 512 instead of 1024 copies of 10.7 KB; 11.29 ->
    // 11.10 us).
    if (ksplit < SK_MAX_WAVES && octs * ksplit / SK_MAX_WAVES >= 2 * cus)
        return SkCfg{1, SK_MAX_WAVES, ksplit};
    return SkCfg{1, max(SK_WAVES, ksplit), ksplit};
}

int lds_bytes(int M, int N, int K, int g)
{
    const SkCfg c = sk_config(M, N, K, device_topology().cus);
    return SkLds(M, K, K / g, c.waves / c.ksplit * c.ro, c.ksplit == 1).total;
}

template <int DT, int M, int GS, int RO, int D, bool SG>
hipError_t launch_r(const W4Args &a, const SkCfg &c, size_t lds, hipStream_t stream)
{
    const int octs_per_wg = c.waves / c.ksplit * RO;
    const int grid = (a.N / 8 + octs_per_wg - 1) / octs_per_wg;
    if (a.qzeros)
        hipLaunchKernelGGL((w4a16_skinny_kernel<DT, M, D, GS, true, RO, SG>), dim3(grid),
                           dim3(64 * c.waves), lds, stream, static_cast<const uint16_t *>(a.x),
                           a.qweight, static_cast<const uint16_t *>(a.scales), a.qzeros,
                           static_cast<uint16_t *>(a.y), a.N, a.K, c.ksplit);
    else
        hipLaunchKernelGGL((w4a16_skinny_kernel<DT, M, D, GS, false, RO, SG>), dim3(grid),
                           dim3(64 * c.waves), lds, stream, static_cast<const uint16_t *>(a.x),
                           a.qweight, static_cast<const uint16_t *>(a.scales), a.qzeros,
                           static_cast<uint16_t *>(a.y), a.N, a.K, c.ksplit);
    return hipGetLastError();
}

// Split K: scales from global memory (on the 1 x 5376 x 21504 down shape this
// lets three workgroups share a CU instead of two, so the grid runs in one
// generation).  Otherwise: scales staged in LDS.
template <int DT, int M, int GS>
hipError_t launch_g(const W4Args &a, const SkCfg &c, size_t lds, hipStream_t stream)
{
    if (c.ksplit > 1)
        return launch_r<DT, M, GS, 1, SK_RING, true>(a, c, lds, stream);
    if constexpr (M <= 2) {
        if (c.ro == 2)
            return launch_r<DT, M, GS, 2, SK_RING, false>(a, c, lds, stream);
    }
    return launch_r<DT, M, GS, 1, SK_RING, false>(a, c, lds, stream);
}

template <int DT, int M>
hipError_t launch_m(const W4Args &a, hipStream_t stream)
{
    const SkCfg c = sk_config(M, a.N, a.K, device_topology().cus);
    const size_t lds = (size_t)lds_bytes(M, a.N, a.K, a.g);
    switch (a.g) {
    case 32: return launch_g<DT, M, 0>(a, c, lds, stream);
    case 64: return launch_g<DT, M, 1>(a, c, lds, stream);
    default: return launch_g<DT, M, 2>(a, c, lds, stream);
    }
}

template <int DT>
hipError_t launch_dt(const W4Args &a, hipStream_t stream)
{
    switch (a.M) {
    case 1: return launch_m<DT, 1>(a, stream);
    case 2: return launch_m<DT, 2>(a, stream);
    case 3: return launch_m<DT, 3>(a, stream);
    case 4: return launch_m<DT, 4>(a, stream);
    case 5: return launch_m<DT, 5>(a, stream);
    case 6: return launch_m<DT, 6>(a, stream);
    case 7: return launch_m<DT, 7>(a, stream);
    case 8: return launch_m<DT, 8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

bool skinny_fits(int M, int N, int K, int g)
{
    return M >= 1 && M <= 8 && lds_bytes(M, N, K, g) <= SK_LDS_BUDGET;
}

hipError_t launch_w4a16_skinny(const W4Args &a, hipStream_t stream)
{
    if (!skinny_fits(a.M, a.N, a.K, a.g))
        return hipErrorInvalidValue;
    return a.dt == DT_F16 ? launch_dt<DT_F16>(a, stream) : launch_dt<DT_BF16>(a, stream);
}

} // namespace wob
