// gla_prefill.hpp -- chunkwise block-parallel prefill kernel for gfx950.
//
// The chunkwise form ("Gated Linear Attention", Summary and Methodology: chunks of
// C tokens, cost O(L/C (C^2 d + C d^2))) of the gated recurrence ("Attention is
// recurrent", Gated linear attention: a write at position s reaches position t
// scaled by the product of the gates after it).  For one head and one chunk, with
// rows t, s in [0, C), in-chunk inclusive cumulative log-gates B[t] = sum_{u<=t} g[u]
// and chunk total Gamma = B[C-1]:
//
//   Q~ = phi(Q) * exp(B),   K^ = phi(K) * exp(-B)       (so Q~_t K^_s = prod of gates)
//   P  = (Q~ K^^T) masked to s <= t
//   O  = P V + Q~ S                                       (intra-chunk + carried state)
//   S <- Diag(exp Gamma) (S + K^^T V)                     (the weighted scan step)
//
// Scalar gates (one log-gate b per token, the same in every key dimension) take the
// same form with one factor per row, exp(+-b_t), computed once per row.  The
// factorisation needs exp(-B) well inside the fp32 range: a chunk whose cumulative
// log2-gate falls below -kFastLim in some key dimension (flagged by the producers) is
// computed token by token instead, by the consumer waves (gla_slow.hpp), which is
// exact for any gate in [0, 1].
//
// Outer-product gate ("Gated Linear Attention", GLA / Recurrent Form: G_t = alpha_t
// beta_t^T, a key-side and a value-side gate): the gate products between s and t
// factorise per key dimension and per value dimension, so with the value side's
// in-chunk cumulative log-gates Bv[t][j] and totals GB[j] the same chunk step becomes
//   V^ = V * exp(-Bv),   O = (P V^ + Q~ S) (.) exp(Bv),
//   S <- Diag(exp Gamma) (S + K^^T V^) Diag(exp GB).
// The producers scan the value gates of their value columns as they scan the key
// gates (a lane holds four value columns of a few rows); a chunk whose lowest key
// and value totals add up to less than -kFastLim runs token by token.
//
// Decomposition: one workgroup per (batch*head, tile of DVT value columns) walks the
// chunks of its head in order, with two kinds of wavefronts:
//   producers (NP waves)  turn raw q, k, g, v rows into matrix-core operands in LDS:
//       each owns DK/NP key columns of all C rows; a lane holds one 16-byte piece of
//       q and k (8 bf16 columns) for RPS consecutive rows, so loads read whole row
//       pieces; it sums the gates of its rows serially and finishes the cumulative
//       sum with a cross-lane scan; Q~ and K^ (scalar gate: also K~) are written
//       row-major, and V rows are copied as they are.  Raw rows are requested two
//       chunks ahead, and each part of a lane's raw registers (gates, q and k, v) is
//       requested again as soon as it has been consumed, so the loads overlap the
//       arithmetic.
//   consumers (NC waves)  hold the fp32 state slice S[d_k][DVT] in accumulator
//       registers (16x16 tiles) and, for the 16-row block of the chunk they own,
//       compute the score tiles P^T[s-block <= tb][tb] in registers and
//       O^T = S^T Q~^T + V^T P^T per 16-column value tile; the output block goes
//       through a private LDS staging area so it is stored with 16-byte row-contiguous
//       writes; then S += K^^T V and the gate decay.  The products that contract over
//       tokens (V^T P^T, K^^T V) read their operands from the row-major arrays with
//       transposing LDS reads.  The state is shared between consumers as a bf16
//       operand copy in LDS.
// With two LDS operand buffers the producers prepare chunk n+1 while the consumers
// compute chunk n (one barrier per chunk); where two buffers do not fit in LDS the
// phases alternate on one buffer.  Barriers wait only for LDS traffic, so requested
// global rows stay in flight.  bf16 inputs use bf16 MFMA operands with fp32
// accumulation; fp32 inputs use fp32 MFMA.
//
// LDS layout: operand rows are not padded; the 16-byte chunks of a row are
// XOR-swizzled by a permutation of (row mod 8), so the rows that one fragment read or
// one transposing read touches, and the producers' writes, spread over all banks.
#pragma once

#include <type_traits>
#include <utility>

#include "gla_device.hpp"
#include "gla_launch.hpp"
#include "gla_slow.hpp"

namespace gla {


template <typename T, int N> struct VecN { typedef T type __attribute__((ext_vector_type(N))); };
template <typename T> struct VecN<T, 1> { typedef T type; };
template <typename T> using Vec4 = VecN<T, 4>;

template <typename T, int N>
__device__ __forceinline__ void widen(const typename VecN<T, N>::type &v, float (&f)[N])
{
#pragma unroll
    for (int e = 0; e < N; ++e) f[e] = (float)v[e];
}

template <typename E> __device__ __forceinline__ typename Vec4<E>::type narrow4(f32x4 v)
{
    return typename Vec4<E>::type{from_f32<E>(v[0]), from_f32<E>(v[1]), from_f32<E>(v[2]), from_f32<E>(v[3])};
}

// Operand fragment of one matrix-core step (see gla_device.hpp for the lane layout).
// bf16: one 16x16x32 step covers a 32-wide slice of the contraction index (8 values
// per lane); fp32: one 16-wide block, 4 steps of 16x16x4 (4 values per lane).  A
// fragment is one 16-byte chunk of an LDS row.
template <typename E> struct Op;

template <> struct Op<bf16> {
    typedef bf16x8 frag;
    static constexpr int W = 32;                   // contraction width of one step
    static __device__ __forceinline__ frag from_acc(f32x4 a, f32x4 b)
    {
        return frag{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                    (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
    }
    static __device__ __forceinline__ frag zero() { return frag{}; }
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Op<float> {
    typedef f32x4 frag;
    static constexpr int W = 16;
    static __device__ __forceinline__ frag from_acc(f32x4 a) { return a; }
    static __device__ __forceinline__ frag zero() { return frag{0.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
};

constexpr int cmin(int a, int b) { return a < b ? a : b; }

// swizzle codes of PrefillShape::swz beyond plain row masks
constexpr int kSwz16 = 0x100, kSwz8 = 0x101, kSwzO8 = 0x102;
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename T, int DK, int C, int DVT, bool OUTER = false>
struct PrefillShape {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int CE = 16 / sizeof(T);      // elements per 16-byte chunk
    static constexpr int NP = cmin(4, DK / CE);    // producer waves
    static constexpr int NTB = C / 16;             // 16-row blocks per chunk
    static constexpr int NKB = DK / 16;            // 16-blocks of the key dim
    static constexpr int NJT = DVT / 16;           // 16-column value tiles
    static constexpr int NC = 4;                   // consumer waves
    static constexpr int NT = 64 * (NP + NC);
    // output blocks: consumer c computes t-block c % NTB for value tiles
    // [(c / NTB) * NJC, +NJC); with more consumers than t-blocks, JS consumers share a
    // t-block (each recomputes its score tiles) and split its value tiles
    static constexpr int JS = (NC > NTB && NJT % (NC / NTB) == 0) ? NC / NTB : 1;
    static constexpr int NJC = NJT / JS;
    static constexpr int DVS = DVT / JS;           // staged output columns per consumer
    static_assert(NC * DVS <= 4 * DVT, "output staging within the LDS budget");
    static constexpr int SW = Op<T>::W;            // contraction width per MFMA step
    static constexpr int KSTEPS = (DK + SW - 1) / SW;
    static constexpr int CSTEPS = (C + SW - 1) / SW;
    static constexpr int KCH = DK / CE, VCH = DVT / CE;   // 16-byte chunks per row
    // swizzle codes (see swz): rows of at least 16 chunks use kSwz16, operand rows of
    // 8 chunks kSwz8; narrower rows mask the row bits
    static constexpr int SWK = KCH >= 16 ? kSwz16 : (KCH == 8 ? kSwz8 : KCH - 1);
    static constexpr int SWV = VCH >= 16 ? kSwz16 : (VCH == 8 ? kSwz8 : VCH - 1);
    // producer gate mapping: producer p owns key columns [p*CW, (p+1)*CW); a lane
    // has column group cg (one 16-byte chunk, CE columns) and row segment rs (RPS
    // consecutive rows); column groups vary fastest across lanes
    static constexpr int CW = DK / NP;
    static constexpr int CG = CW / CE;
    static constexpr int RSEG = cmin(64 / CG, C);
    static constexpr int RPS = C / RSEG;
    // producer value mapping: the C x VCH 16-byte pieces of a chunk's value tile are
    // dealt to the 64*NP producer lanes in order, NVL per lane
    static constexpr int NVP = C * VCH;
    static constexpr int NVL = NVP >= 64 * NP ? NVP / (64 * NP) : 1;
    static constexpr int NU = NKB * NJT;          // 16x16 state tiles
    // output staging: 16 rows x DVS, stored by 64 lanes in 16-byte chunks
    static constexpr int SCH = DVS / CE, SWS = SCH >= 16 ? kSwz16 : (SCH == 8 ? kSwzO8 : SCH - 1);
    static constexpr int OCH = 16 * SCH;           // chunks per staged block
    static constexpr int OCPL = cmax(1, OCH / 64); // chunks per lane
    // outer-product gate, value side: producer p owns value columns [p*CWV, (p+1)*CWV)
    // of the tile; a lane has four of them (column group cgv: one f32x4 of gates) for
    // RPSV consecutive rows (row segment rsv); column groups vary fastest across lanes
    static constexpr int CWV = DVT / NP;
    static constexpr int CGV = cmax(1, CWV / 4);
    static constexpr int RSEGV = cmin(64 / CGV, C);
    static constexpr int RPSV = C / RSEGV;
    static constexpr int LEV = DVT + 4;            // fp32 row length of exp(Bv) in LDS
    static constexpr int NBUF = prefill_nbuf((int)sizeof(T), DK, C, DVT, OUTER);
    static_assert(NBUF >= 1, "LDS budget");
    static_assert(!OUTER || (CWV >= 4 && CWV % 4 == 0 && 16 % CGV == 0 && RPSV >= 1), "value gate mapping");
    static_assert(CW >= CE && CW % CE == 0 && 64 % CG == 0, "producer gate mapping");
    static_assert(NVP < 64 * NP || NVP % (64 * NP) == 0, "producer value mapping");
    static_assert(RPS >= 1, "rows per lane");
    static_assert(16 % CG == 0, "gate scan: column groups per 16-lane row");

    // element offset of (row, col) in a row-major array of rows of `len` elements
    // whose 16-byte chunks are XOR-swizzled by a function of the row.  The functions
    // follow gfx950's LDS banking (64 banks of 4 bytes): a 16-byte read serves 16
    // lanes at a time, the four lanes of each quad whose index has even (or odd) bit
    // parity within a 32-lane half, over 256 bytes; a transposing 8-byte read serves
    // 32 lanes over 256 bytes; a 16-byte write serves 8 lanes and an 8-byte access 16
    // lanes, over 128 bytes.  With r0..r3 the low row bits:
    //   kSwz16 (rows of 16 or more chunks): r0 | r1 << 1 | (r0 ^ r2) << 2 | (r0 ^ r3) << 3
    //     -- fragment reads of 16 rows, transposing reads of 8 rows and the producers'
    //        row-piece writes touch every bank once;
    //   kSwz8 (operand rows of 8 chunks): row & 6 -- transposing reads of 8 rows hit
    //     distinct 32-byte bank groups, and fragment reads and row-piece writes touch
    //     every bank once;
    //   kSwzO8 (output staging rows of 8 chunks): row & 7 -- the 16-byte read-back of
    //     two rows per 16 lanes hits every bank once;
    //   otherwise row & sw.
    static __device__ __forceinline__ int swz(int row, int sw)
    {
        if (sw == kSwz16) return (row & 3) | ((((row >> 2) ^ row) & 1) << 2) | ((((row >> 3) ^ row) & 1) << 3);
        if (sw == kSwz8) return row & 6;
        if (sw == kSwzO8) return row & 7;
        return row & sw;
    }
    static __device__ __forceinline__ int sw_off(int row, int col, int len, int sw)
    {
        return row * len + (((col / CE) ^ swz(row, sw)) * CE) + col % CE;
    }
    static __device__ __forceinline__ int rk(int row, int col) { return sw_off(row, col, DK, SWK); }
    static __device__ __forceinline__ int rv(int row, int col) { return sw_off(row, col, DVT, SWV); }
    static __device__ __forceinline__ int ro(int row, int col) { return sw_off(row, col, DVS, SWS); }
};

// Calls fn(std::integral_constant<int, I>) for I = 0 .. N-1.
template <typename Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn &&fn, std::integer_sequence<int, I...>)
{
    (fn(std::integral_constant<int, I>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn &&fn)
{
    static_for_impl(fn, std::make_integer_sequence<int, N>{});
}

// Inclusive scan of v over the RSEG lanes of a segment group: the lanes
// rs * STRIDE + cg (rs = 0 .. RSEG-1, STRIDE divides 16) for a fixed cg, in order of
// rs.  Inside each 16-lane row the segments are scanned with DPP row shifts (a
// source outside the row reads 0, which is exactly the row-local scan); the rows are
// then combined by adding the running total at the last segment of earlier rows.
template <int DPPSHIFT>
__device__ __forceinline__ float row_shr(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                  0x110 + DPPSHIFT, 0xf, 0xf, true));
}
template <int RSEG, int STRIDE>
__device__ __forceinline__ float group_scan(float v, int lane)
{
    constexpr int SPR = 16 / STRIDE;                   // segments per 16-lane row
    constexpr int NR = (RSEG * STRIDE + 15) / 16;      // rows of the group
    if constexpr (SPR > 1) v += row_shr<STRIDE>(v);
    if constexpr (SPR > 2) v += row_shr<2 * STRIDE>(v);
    if constexpr (SPR > 4) v += row_shr<4 * STRIDE>(v);
    if constexpr (SPR > 8) v += row_shr<8 * STRIDE>(v);
    const int row = lane >> 4, last = 16 - STRIDE + (lane & (STRIDE - 1));
    if constexpr (NR > 1) {
        const float up = __shfl(v, 16 * (row - 1) + last, 64);
        v += row >= 1 ? up : 0.f;
    }
    if constexpr (NR > 2) {
        const float up = __shfl(v, 16 * (row - 2) + last, 64);
        v += row >= 2 ? up : 0.f;
    }
    return v;
}

// The same scan for NE columns at once, with the group totals: v[e] becomes the
// inclusive scan and tot[e] the total over all RSEG segments.  Inside each 16-lane row
// DPP row shifts as above; the rows' totals then go through a small LDS area of this
// wave (scr, STRIDE * NE * 4 floats): the last segment of each row writes its row
// total, and every lane reads the (at most four) totals of its column group in one
// access, so all columns take one LDS round trip instead of one shuffle per row step.
// (A wave's LDS accesses complete in order, so the reads see this wave's writes.)
template <int RSEG, int STRIDE, int NE>
__device__ __forceinline__ void group_scan_tot(float (&v)[NE], float (&tot)[NE], int lane, float *scr)
{
    constexpr int SPR = 16 / STRIDE;                   // segments per 16-lane row
    constexpr int NR = (RSEG * STRIDE + 15) / 16;      // rows of the group
    static_assert(NR <= 4 && (RSEG * STRIDE) % 16 == 0, "group scan: whole 16-lane rows");
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        if constexpr (SPR > 1) v[e] += row_shr<STRIDE>(v[e]);
        if constexpr (SPR > 2) v[e] += row_shr<2 * STRIDE>(v[e]);
        if constexpr (SPR > 4) v[e] += row_shr<4 * STRIDE>(v[e]);
        if constexpr (SPR > 8) v[e] += row_shr<8 * STRIDE>(v[e]);
    }
    const int row = lane >> 4, cg = lane & (STRIDE - 1);
    if ((lane & 15) >= 16 - STRIDE) {                  // the row's last segment
#pragma unroll
        for (int e = 0; e < NE; ++e) scr[(cg * NE + e) * 4 + row] = v[e];
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const f32x4 t = *(const f32x4 *)(scr + (cg * NE + e) * 4);
        float before = 0.f, all = 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            all += t[r];
            before += r < row ? t[r] : 0.f;
        }
        v[e] += before;
        tot[e] = all;
    }
}


// SO (state only): the first pass of a segmented prefill, launched over pieces of the
// segments (its own "segments").  Each workgroup computes its piece's state from a
// zero start and the piece's gate totals; no outputs, no Q~.  It walks the piece's
// chunks last to first and adds each chunk's writes already decayed to the piece's
// end, S += (phi(K) * exp(Gamma_c - B + later))^T V, with `later` the gate total of
// the chunks after it: every exponent is <= 0, so no chunk leaves the factorised
// range and this pass needs no token-by-token chunks.
// NM (normalised, "Transformers are RNNs" notes: the weighted sum of values over the
// sum of the same weights): the state's owners also carry the normaliser state z, the
// state of a value that is 1 in every token, z <- Diag(e^Gamma)(z + K^^T 1), with the
// matrix cores (a fragment of ones as the value operand); each output row is divided
// by its denominator Q~_t . z + sum_{s<=t} P_ts.
template <typename T, int DK, int C, int DVT, int GATE, bool ELU1, bool SO, bool NM>
__global__ __launch_bounds__((PrefillShape<T, DK, C, DVT>::NT)) void prefill_kernel(const PrefillArgs a)
{
    using SH = PrefillShape<T, DK, C, DVT, GATE == kGateOuter>;
    using O = Op<T>;
    using V4 = typename Vec4<T>::type;
    using VC = typename VecN<T, SH::CE>::type;       // one 16-byte chunk
    using F = typename O::frag;
    constexpr int NP = SH::NP, NC = SH::NC, NBUF = SH::NBUF, CE = SH::CE;
    constexpr int NTB = SH::NTB, NKB = SH::NKB, NJT = SH::NJT;
    constexpr int CW = SH::CW, RSEG = SH::RSEG, RPS = SH::RPS;
    constexpr int NVL = SH::NVL, NU = SH::NU;

    __shared__ __attribute__((aligned(16))) T sQ[NBUF][C * DK];      // Q~ [t][i]
    __shared__ __attribute__((aligned(16))) T sK[NBUF][C * DK];      // K^ [s][i]
    constexpr bool OG = GATE == kGateOuter;         // outer-product gate: value-side gates too
    constexpr bool KG = GATE == kGateKeydim || OG;  // gates per key dimension
    constexpr bool FG = GATE != kGateNone;          // factorised: Q~ = q e^B, K^ = k e^-B
    __shared__ __attribute__((aligned(16))) T sV[NBUF][C * DVT];     // V [s][j]
    __shared__ __attribute__((aligned(16))) T sS[2][DVT * DK];       // state^T [j][i], by parity
    __shared__ __attribute__((aligned(16))) T sO[NC][16 * SH::DVS];  // output staging, per consumer
    __shared__ __attribute__((aligned(16))) float sEG[NBUF][DK];     // exp(Gamma_i)
    __shared__ __attribute__((aligned(16))) float sZ[NM ? 2 : 1][NM ? DK : 4];   // normaliser z, by parity
    __shared__ __attribute__((aligned(16))) int sFlag[NBUF][4];      // per producer: chunk out of range
    // outer gate, per producer: the gate scan's row totals
    __shared__ __attribute__((aligned(16))) float sScan[OG || NM ? SH::NP : 1][OG || NM ? SH::CG * SH::CE * 4 : 4];
    // outer-product gate: exp(Bv) [t][j] for the outputs, exp of the value-side chunk
    // totals, and per producer the lowest key-side and value-side log2 totals
    __shared__ __attribute__((aligned(16))) float sEV[OG ? NBUF : 1][OG ? C * SH::LEV : 4];
    __shared__ __attribute__((aligned(16))) float sEGV[OG ? NBUF : 1][OG ? DVT : 4];
    __shared__ __attribute__((aligned(16))) float sMin[OG ? NBUF : 1][2][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;
    const bool producer = w < NP;

    int wg = blockIdx.x;
    if (a.xcd_remap) wg = (wg & 7) * (gridDim.x >> 3) + (wg >> 3);
    const int bhs = wg / a.n_vt;                   // (head, segment)
    const int vt = wg - bhs * a.n_vt;
    const int bh = bhs / a.nseg, seg = bhs - bh * a.nseg;
    const int DV = a.d_v;
    // this workgroup's rows: [row0, row0 + L) of its head
    const int row0 = seg * a.seg_len;
    const int L = max(0, min(a.L - row0, a.seg_len));
    const size_t hrow = (size_t)bh * a.L + row0;   // first row, counted over all heads

    // per-segment buffer views (host code guarantees each head's bytes fit in 31 bits)
    constexpr int ES = sizeof(T);
    const Rsrc rq = make_rsrc((const T *)a.q + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rk = make_rsrc((const T *)a.k + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rvv = make_rsrc((const T *)a.v + hrow * DV, (unsigned)(L * DV * ES));
    T *__restrict__ oh = SO ? nullptr : (T *)a.o + hrow * DV + vt * DVT;
    Rsrc rg = make_rsrc(a.g, 0u);                  // no gates: never read
    if constexpr (KG) rg = make_rsrc(a.g + hrow * DK, (unsigned)(L * DK * 4));
    if constexpr (GATE == kGateScalar) rg = make_rsrc(a.g + hrow, (unsigned)(L * 4));
    Rsrc rgv = make_rsrc(a.gv, 0u);                // value-side gates (outer-product gate only)
    if constexpr (OG) rgv = make_rsrc(a.gv + hrow * DV, (unsigned)(L * DV * 4));
    const int nchunks = (L + C - 1) / C;

    // ---------------- producers -------------------------------------------------------
    const int p = w;
    const int cg = lane % SH::CG, rs = lane / SH::CG;   // column group, row segment
    // lanes with work in the gate / value mappings (all of them for the common shapes,
    // known at compile time so that no branch surrounds the loads)
    const bool gate_lane = (SH::CG * RSEG == 64) || rs < RSEG;
    const int ic = p * CW + CE * cg;               // first of this lane's CE key columns
    const bool v_lane = SH::NVP >= 64 * NP || tid < SH::NVP;
    // outer-product gate: the value mapping follows the value-gate scan instead
    const int cgv = lane % SH::CGV, rsv = lane / SH::CGV;
    const bool vg_lane = SH::CGV * SH::RSEGV == 64 || rsv < SH::RSEGV;
    const int jc = p * SH::CWV + 4 * cgv;          // first of this lane's four value columns

    struct Raw {
        VC q[RPS], k[RPS];
        f32x4 g[RPS][CE / 4];
        VC v[OG ? 1 : NVL];
        V4 vv[OG ? SH::RPSV : 1];                  // outer: four value columns of RPSV rows
        f32x4 gv[OG ? SH::RPSV : 1];               // outer: their value-side log-gates
    };
    float gsum[CE];                                // state-only pass: gate totals so far
#pragma unroll
    for (int e = 0; e < CE; ++e) gsum[e] = 0.f;
    // Who holds the fp32 state (see "state owners" below): the producers (POWN) where
    // that measured faster -- scalar gates, the normalised form, the outer gate at
    // 64-row chunks -- else the consumers.
    constexpr bool POWN = !SO && (GATE == kGateScalar || NM || (OG && C == 64));
    // raw register sets: with two operand buffers the rows are requested two chunks
    // ahead, except where the producers also hold the state and per-key-dimension
    // gates (one chunk ahead, which leaves room in their registers) and in the
    // state-only pass (one set, so that three of its workgroups fit a CU)
    constexpr int NRAW = NBUF == 2 && !(POWN && KG) && !SO ? 2 : 1;
    Raw R[NRAW];

    // Raw rows of the chunk starting at t0, requested in three parts so that each
    // part of a register set can be refilled as soon as it has been consumed.  Rows
    // past L read as zeros (buffer range check), which is exactly the masking the
    // tail chunk needs: zero log-gates leave the cumulative gate flat, zero keys and
    // values add nothing to the state, and those rows' outputs are never stored.
    const int qk_off = (rs * RPS) * DK * ES + ic * ES;
    auto load_g = [&](Raw &r_, int t0) __attribute__((always_inline)) {
        if (gate_lane) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                if constexpr (KG) {
#pragma unroll
                    for (int h = 0; h < CE / 4; ++h)
                        r_.g[r][h] = buf_load16<f32x4>(rg, (t0 + rs * RPS + r) * DK * 4 + (ic + 4 * h) * 4);
                } else if constexpr (GATE == kGateScalar) {
                    const float gv = buf_load4(rg, (t0 + rs * RPS + r) * 4);
                    r_.g[r][0] = f32x4{gv, gv, gv, gv};
                }
            }
        }
    };
    auto load_qk = [&](Raw &r_, int t0) __attribute__((always_inline)) {
        if (gate_lane) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                if constexpr (!SO) r_.q[r] = buf_load16<VC>(rq, qk_off + (t0 + r) * DK * ES);
                r_.k[r] = buf_load16<VC>(rk, qk_off + (t0 + r) * DK * ES);
            }
        }
    };
    auto load_v = [&](Raw &r_, int t0) __attribute__((always_inline)) {
        if constexpr (OG) {
            if (vg_lane) {
#pragma unroll
                for (int r = 0; r < SH::RPSV; ++r)
                    r_.vv[r] = buf_load<V4>(rvv, (t0 + rsv * SH::RPSV + r) * DV * ES + (vt * DVT + jc) * ES);
            }
        } else if (v_lane) {
#pragma unroll
            for (int h = 0; h < NVL; ++h) {
                const int id = tid + 64 * NP * h;
                r_.v[h] = buf_load16<VC>(rvv, (t0 + id / SH::VCH) * DV * ES + (vt * DVT + (id % SH::VCH) * CE) * ES);
            }
        }
    };
    auto load_gv = [&](Raw &r_, int t0) __attribute__((always_inline)) {
        if constexpr (OG) {
            if (vg_lane) {
#pragma unroll
                for (int r = 0; r < SH::RPSV; ++r)
                    r_.gv[r] = buf_load16<f32x4>(rgv, ((t0 + rsv * SH::RPSV + r) * DV + vt * DVT + jc) * 4);
            }
        }
    };
    auto load_raw = [&](Raw &r_, int t0) __attribute__((always_inline)) {
        load_g(r_, t0);
        load_gv(r_, t0);
        load_qk(r_, t0);
        load_v(r_, t0);
    };

    // Turn the raw rows of the chunk starting at t0 into the operands of buffer `buf`,
    // refilling each part of the register set with the rows of the chunk at t_next
    // as soon as that part has been consumed.
    auto produce = [&](Raw &r_, int t0, int buf, int t_next) __attribute__((always_inline)) {
        // No branch here depends on a pending load: a branch would make the compiler's
        // wait analysis wait for every outstanding load at the join.
        [[maybe_unused]] float kmin = 0.f, vmin = 0.f;   // outer: lowest key / value log2 totals
        if (gate_lane) {
            float bc[RPS][CE];
            float excl[CE], tot[CE];
#pragma unroll
            for (int e = 0; e < CE; ++e) excl[e] = tot[e] = 0.f;
            if constexpr (GATE != kGateNone) {
                constexpr int NE = GATE == kGateScalar ? 1 : CE;
                float run[NE];
#pragma unroll
                for (int e = 0; e < NE; ++e) run[e] = 0.f;
#pragma unroll
                for (int r = 0; r < RPS; ++r) {
#pragma unroll
                    for (int e = 0; e < NE; ++e) {             // cumulative sums in log2 units
                        run[e] += r_.g[r][e / 4][e % 4] * kLog2e;
                        bc[r][e] = run[e];
                    }
                }
                load_g(r_, t_next);                // gates consumed: refill them now
                if constexpr (OG || NM) {
                    // outer gate and normalised form (their producers carry the
                    // longer role; measured faster there): the rows' totals through LDS
                    float incl[NE], totn[NE];
#pragma unroll
                    for (int e = 0; e < NE; ++e) incl[e] = run[e];
                    group_scan_tot<RSEG, SH::CG, NE>(incl, totn, lane, sScan[OG || NM ? p : 0]);
#pragma unroll
                    for (int e = 0; e < NE; ++e) {
                        excl[e] = incl[e] - run[e];
                        tot[e] = totn[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < NE; ++e) {
                        const float incl = group_scan<RSEG, SH::CG>(run[e], lane);
                        excl[e] = incl - run[e];
                        tot[e] = __shfl(incl, (RSEG - 1) * SH::CG + cg, 64);
                    }
                }
                if constexpr (GATE == kGateScalar) {     // one gate per row: the same in every column
#pragma unroll
                    for (int e = 1; e < CE; ++e) { excl[e] = excl[0]; tot[e] = tot[0]; }
#pragma unroll
                    for (int r = 0; r < RPS; ++r)
#pragma unroll
                        for (int e = 1; e < CE; ++e) bc[r][e] = bc[r][0];
                }
                if constexpr (FG) {
                    // the chunk total is the lowest cumulative log2-gate of a column
                    // (gates are <= 0); below -kFastLim the chunk runs token by token
                    // (outer gate: the key-side and value-side lowest totals together)
                    float m = tot[0];
#pragma unroll
                    for (int e = 1; e < CE; ++e) m = fminf(m, tot[e]);
                    if constexpr (OG) {
                        kmin = m;
                    } else {
                        const bool far = __ballot(m < -kFastLim) != 0;
                        if (lane == 0) sFlag[buf][p] = far ? 1 : 0;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int t = rs * RPS + r;
                if constexpr (!FG && !ELU1) {
                    // q and k enter the products as they are
                    if constexpr (!SO) *(VC *)(sQ[buf] + SH::rk(t, ic)) = r_.q[r];
                    *(VC *)(sK[buf] + SH::rk(t, ic)) = r_.k[r];
                } else {
                    float q[CE], kk[CE];
                    if constexpr (!SO) widen<T, CE>(r_.q[r], q);
                    widen<T, CE>(r_.k[r], kk);
#pragma unroll
                    for (int e = 0; e < CE; ++e) {
                        // key exponent: -b, or for the state-only pass (chunks last to
                        // first) Gamma - b + the later chunks' total, which is <= 0
                        [[maybe_unused]] const float kb =
                            SO ? tot[e] - (excl[e] + bc[r][e]) + gsum[e] : -(excl[e] + bc[r][e]);
                        if constexpr (ELU1 && FG) {
                            // phi(x) 2^(+-b) with one exponential: (x + 1) 2^(+-b) for
                            // x > 0, else 2^(x log2(e) +- b), i.e. with
                            // f = 2^(min(x, 0) log2(e) +- b), max(x, 0) f + f (no
                            // compare-and-select, one fused multiply-add)
                            const float b = excl[e] + bc[r][e];
                            if constexpr (!SO) {
                                const float x = q[e];
                                const float f = exp2_fast(fmaf(fminf(x, 0.f), kLog2e, b));
                                q[e] = fmaf(fmaxf(x, 0.f), f, f);
                            }
                            const float x = kk[e];
                            const float f = exp2_fast(fmaf(fminf(x, 0.f), kLog2e, kb));
                            kk[e] = fmaf(fmaxf(x, 0.f), f, f);
                        } else {
                            if constexpr (ELU1) {
                                if constexpr (!SO) q[e] = feature(q[e], true);
                                kk[e] = feature(kk[e], true);
                            }
                            if constexpr (FG) {
                                // (a scalar gate's b is the same in every column: its two
                                // exponentials are computed once per row)
                                const float b = excl[e] + bc[r][e];
                                if constexpr (!SO) q[e] *= exp2_fast(b);
                                kk[e] *= exp2_fast(kb);
                            }
                        }
                    }
                    VC qv, kv;
#pragma unroll
                    for (int e = 0; e < CE; ++e) {
                        if constexpr (!SO) qv[e] = from_f32<T>(q[e]);
                        kv[e] = from_f32<T>(kk[e]);
                    }
                    if constexpr (!SO) *(VC *)(sQ[buf] + SH::rk(t, ic)) = qv;
                    *(VC *)(sK[buf] + SH::rk(t, ic)) = kv;
                }
            }
            load_qk(r_, t_next);                   // q, k consumed: refill them now
            if constexpr (SO) {
#pragma unroll
                for (int e = 0; e < CE; ++e) gsum[e] += tot[e];
            }
            if (rs == 0) {
#pragma unroll
                for (int e = 0; e < CE; ++e)
                    sEG[buf][ic + e] = GATE == kGateNone ? 1.f : exp2_fast(tot[e]);
            }
        }
        if constexpr (OG) {
            // value side of the outer-product gate: cumulative log2-gates Bv down the
            // rows of each value column (the key side's scan on this mapping), then
            // V^ = v exp(-Bv), exp(Bv) for the outputs and exp of the chunk totals
            if (vg_lane) {
                float bcv[SH::RPSV][4], run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < SH::RPSV; ++r) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        run[e] += r_.gv[r][e] * kLog2e;
                        bcv[r][e] = run[e];
                    }
                }
                load_gv(r_, t_next);               // value gates consumed: refill them now
                float exv[4], totv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float incl = group_scan<SH::RSEGV, SH::CGV>(run[e], lane);
                    exv[e] = incl - run[e];
                    totv[e] = __shfl(incl, (SH::RSEGV - 1) * SH::CGV + cgv, 64);
                }
                vmin = fminf(fminf(totv[0], totv[1]), fminf(totv[2], totv[3]));
#pragma unroll
                for (int r = 0; r < SH::RPSV; ++r) {
                    const int t = rsv * SH::RPSV + r;
                    f32x4 ev;
                    V4 vh;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float b = exv[e] + bcv[r][e];
                        ev[e] = exp2_fast(b);
                        vh[e] = from_f32<T>((float)r_.vv[r][e] * exp2_fast(-b));
                    }
                    *(V4 *)(sV[buf] + SH::rv(t, jc)) = vh;
                    *(f32x4 *)(sEV[buf] + t * SH::LEV + jc) = ev;
                }
                load_v(r_, t_next);                // v consumed: refill it now
                if (rsv == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sEGV[buf][jc + e] = exp2_fast(totv[e]);
                }
            }
            // all lanes again: the wave's lowest totals for the range check
            kmin = wave_min(kmin);
            vmin = wave_min(vmin);
            if (lane == 0) {
                sMin[buf][0][p] = kmin;
                sMin[buf][1][p] = vmin;
            }
        } else if (v_lane) {
            // store first, then refill the same registers (a load issued while the old
            // values are still live would land in other registers and need a copy,
            // and the copy a wait for the load)
#pragma unroll
            for (int h = 0; h < NVL; ++h) {
                const int id = tid + 64 * NP * h;
                *(VC *)(sV[buf] + SH::rv(id / SH::VCH, (id % SH::VCH) * CE)) = r_.v[h];
            }
            load_v(r_, t_next);                    // v consumed: refill it now
        }
    };

    // ---------------- state owners and consumers ----------------------------------------
    // The fp32 state tiles sit in the registers of their owner waves.  With POWN these
    // are the producers: while the consumers compute chunk n's outputs from the bf16
    // copy of the state before it, the producers prepare chunk n+1's operands and
    // update S with chunk n's K^ and V, then write the next copy.  Otherwise the
    // consumers update S after their outputs (and alone in the state-only pass).
    // Owner ow holds the 16x16 tiles (key block ow + NOW a, every value tile) when
    // NKB % NOW == 0, so that its key fragments are shared across value tiles;
    // otherwise tiles are dealt round-robin.
    const int c = w - NP;
    constexpr int NOW = POWN ? NP : NC;              // owner waves
    const int ow = POWN ? w : c;                      // this wave's index among them
    constexpr bool BLK = NKB % NOW == 0;
    constexpr int IPC = BLK ? NKB / NOW : 1;
    constexpr int NSLOT = BLK ? IPC * NJT : (NU + NOW - 1) / NOW;
    auto tile_i = [&](int k) __attribute__((always_inline)) -> int {
        if constexpr (BLK) return ow + NOW * (k % IPC);
        else return (k * NOW + ow) % NKB;
    };
    auto tile_j = [&](int k) __attribute__((always_inline)) -> int {
        if constexpr (BLK) return k / IPC;
        else return (k * NOW + ow) / NKB;
    };
    auto tile_ok = [&](int k) __attribute__((always_inline)) -> bool {
        if constexpr (BLK) return true;
        else return k * NOW + ow < NU;
    };

    f32x4 S[NSLOT];
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // normaliser tiles: owner ow holds z rows 16 it + 4 grp + r for it = ow + NOW m
    constexpr int NZ = NM ? (NKB + NOW - 1) / NOW : 0;
    f32x4 Z[NZ > 0 ? NZ : 1];
#pragma unroll
    for (int m = 0; m < NZ; ++m) Z[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto z_ok = [&](int m) __attribute__((always_inline)) -> bool { return ow + NOW * m < NKB; };
    // initial state (by the owners)
    // In the full pass of a segmented prefill (a.seg_ds set) the segment's initial
    // state is the weighted scan over the states from zero of the pieces before it
    // (a.seg_sub per segment): S = s0, then S = Diag(exp2(gam_p)) S + ds_p for
    // p = 0 .. seg * seg_sub - 1.
    auto load_s0 = [&]() __attribute__((always_inline)) {
        if (SO || !a.seg_ds) {
            if (a.s0) {
#pragma unroll
                for (int k = 0; k < NSLOT; ++k) {
                    const bool ok = tile_ok(k);
                    const int it = ok ? tile_i(k) : 0, jt = ok ? tile_j(k) : 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * it + 4 * grp + r;
                        const float v = a.s0[((size_t)bhs * DK + i) * DV + vt * DVT + 16 * jt + x];
                        S[k][r] = ok ? v : 0.f;
                    }
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < NSLOT; ++k) {
                S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (a.s0 && tile_ok(k)) {
                    const int it = tile_i(k), j = vt * DVT + 16 * tile_j(k) + x;
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[k][r] = a.s0[((size_t)bh * DK + 16 * it + 4 * grp + r) * DV + j];
                }
            }
            // pieces two at a time, their loads for every tile requested before the steps
            // (one memory round trip per two pieces); the gate totals depend on the key
            // block only, shared by the tiles of one key block
            const int np = seg * a.seg_sub;
            const size_t hp0 = (size_t)bh * (a.nseg - 1) * a.seg_sub;
            constexpr int PB = 2, NG = BLK ? IPC : NSLOT;
            auto gidx = [&](int k) __attribute__((always_inline)) -> int { return BLK ? k % IPC : k; };
            for (int sp0 = 0; sp0 < np; sp0 += PB) {
                f32x4 d[PB][NSLOT], gm[PB][NG];
#pragma unroll
                for (int u = 0; u < PB; ++u) {
                    const size_t hp = hp0 + sp0 + u;
#pragma unroll
                    for (int k = 0; k < NSLOT; ++k) {
                        d[u][k] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (sp0 + u < np && tile_ok(k)) {
                            const int it = tile_i(k), j = vt * DVT + 16 * tile_j(k) + x;
                            const float *ds = a.seg_ds + (hp * DK + 16 * it + 4 * grp) * DV + j;
#pragma unroll
                            for (int r = 0; r < 4; ++r) d[u][k][r] = ds[(size_t)r * DV];
                        }
                    }
#pragma unroll
                    for (int g = 0; g < NG; ++g) {
                        gm[u][g] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (a.seg_gam && sp0 + u < np && tile_ok(g)) {
                            const int it = tile_i(g);
                            gm[u][g] = *(const f32x4 *)(a.seg_gam + hp * DK + 16 * it + 4 * grp);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < PB; ++u) {
                    if (sp0 + u < np) {
#pragma unroll
                        for (int g = 0; g < NG; ++g)
#pragma unroll
                            for (int r = 0; r < 4; ++r) gm[u][g][r] = exp2_fast(gm[u][g][r]);
#pragma unroll
                        for (int k = 0; k < NSLOT; ++k)
#pragma unroll
                            for (int r = 0; r < 4; ++r) S[k][r] = fmaf(gm[u][gidx(k)][r], S[k][r], d[u][k][r]);
                    }
                }
            }
        }
    };

    auto load_z0 = [&]() __attribute__((always_inline)) {
        if constexpr (NM) {
            if (a.z0) {
#pragma unroll
                for (int m = 0; m < NZ; ++m) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * (z_ok(m) ? ow + NOW * m : 0) + 4 * grp + r;
                        const float v = a.z0[(size_t)bhs * DK + i];
                        Z[m][r] = z_ok(m) ? v : 0.f;
                    }
                }
            }
        }
    };
    auto write_z = [&](int par) __attribute__((always_inline)) {     // -> fp32 rows for the denominators
        if constexpr (NM) {
#pragma unroll
            for (int m = 0; m < NZ; ++m)
                if (z_ok(m) && x == 0) *(f32x4 *)(sZ[par] + 16 * (ow + NOW * m) + 4 * grp) = Z[m];
        }
    };

    auto write_state = [&](int par) __attribute__((always_inline)) {   // -> bf16 operand rows
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            if (tile_ok(k)) {
                const int it = tile_i(k), jt = tile_j(k);
                *(V4 *)(sS[par] + SH::rk(16 * jt + x, 16 * it + 4 * grp)) = narrow4<T>(S[k]);
            }
        }
    };

    // fragment k-step `ks` of a row of length d_k (contraction over d_k)
    auto frag_k = [&](const T *base, int row, int ks) __attribute__((always_inline)) -> F {
        const int col = SH::SW * ks + CE * grp;
        if constexpr (SH::BF && DK % 32 != 0) {
            if (col >= DK) return O::zero();
        }
        return *(const F *)(base + SH::rk(row, col));
    };
    // fragment k-step `ks` of column n0 + x of a row-major array [C][len] (swizzle sw),
    // contracting over tokens.  bf16: a lane of group grp holds tokens 32ks + 4grp + 0..3
    // and 32ks + 16 + 4grp + 0..3, the order in which a score accumulator tile pair
    // feeds the next product (Op::from_acc); fp32: tokens 16ks + 4grp + 0..3.
    auto frag_tr = [&](const T *base, int len, int sw, int n0, int ks) __attribute__((always_inline)) -> F {
        if constexpr (SH::BF) {
            const int col = n0 + 4 * (x & 3);
            const int r0 = 32 * ks + 4 * grp + (x >> 2);
            const bf16x4 lo = lds_read_tr16(base + SH::sw_off(r0, col, len, sw));
            bf16x4 hi = {};
            if constexpr (C % 32 == 0) hi = lds_read_tr16(base + SH::sw_off(r0 + 16, col, len, sw));
            return F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
            F f;
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = base[SH::sw_off(16 * ks + 4 * grp + r, n0 + x, len, sw)];
            return f;
        }
    };

    // Outputs of the 16-row block TB of the chunk starting at t0 (straight-line code:
    // TB is a compile-time constant, so every tile loop below is unrolled).
    auto out_block = [&](auto tbc, int j0, int t0, int nvalid, int buf, int par, const T *Q, const T *K,
                         const T *V, const T *SS) __attribute__((always_inline)) {
        constexpr int TB = decltype(tbc)::value;
        const int t = 16 * TB + x;
        F qf[SH::KSTEPS];
#pragma unroll
        for (int k = 0; k < SH::KSTEPS; ++k) qf[k] = frag_k(Q, t, k);
        // normalised: this lane's share of Q~_t . z, formed before the score products
        // so that it overlaps them, as four partial sums (a short dependent chain)
        float dz = 0.f;
        if constexpr (NM) {
            float dzp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < SH::KSTEPS; ++k) {
                constexpr int NE = sizeof(F) / sizeof(T);
                const int i0 = SH::SW * k + (SH::BF ? 8 : 4) * grp;
#pragma unroll
                for (int e = 0; e < NE; ++e)
                    if (!SH::BF || DK % 32 == 0 || i0 + e < DK) dzp[e & 3] += to_f32(qf[k][e]) * sZ[par][i0 + e];
            }
            dz = (dzp[0] + dzp[1]) + (dzp[2] + dzp[3]);
        }
        // score tiles P^T[s-block sb][t-block TB]: lane holds P[t][16sb + 4grp + r]
        f32x4 pt[TB + 2];
        // the next s-block's key fragments are requested before the current block's
        // products
        F kf[2][SH::KSTEPS];
#pragma unroll
        for (int k = 0; k < SH::KSTEPS; ++k) kf[0][k] = frag_k(K, x, k);
#pragma unroll
        for (int sb = 0; sb <= TB; ++sb) {
            if (sb < TB) {
#pragma unroll
                for (int k = 0; k < SH::KSTEPS; ++k) kf[(sb + 1) & 1][k] = frag_k(K, 16 * (sb + 1) + x, k);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < SH::KSTEPS; ++k) acc = O::mma(kf[sb & 1][k], qf[k], acc);
            if (sb == TB) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = 4 * grp + r <= x ? acc[r] : 0.f;
            }
            pt[sb] = acc;
        }
        pt[TB + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
        // normalised: denominator of row t = Q~_t . z + sum_{s <= t} P_ts; a lane sums
        // its share, the four lane groups of column x are then added
        float rden = 1.f;
        if constexpr (NM) {
            float dp = 0.f;
#pragma unroll
            for (int sb = 0; sb <= TB; ++sb) dp += pt[sb][0] + pt[sb][1] + pt[sb][2] + pt[sb][3];
            float den = dz + dp;
            den += __shfl_xor(den, 16, 64);
            den += __shfl_xor(den, 32, 64);
            rden = 1.f / den;
        }
        T *stage = sO[c];
        // value tiles in order; the next tile's state and value fragments are requested
        // before the current tile's products (two register slots), so LDS latency
        // overlaps the matrix cores
        constexpr int NSP = SH::BF ? TB / 2 + 1 : TB + 1;
        F sf[2][SH::KSTEPS], vf[2][NSP];
        auto load_j = [&](int jj, int slot) __attribute__((always_inline)) {
            const int jt = j0 + jj;
#pragma unroll
            for (int k = 0; k < SH::KSTEPS; ++k) sf[slot][k] = frag_k(SS, 16 * jt + x, k);
#pragma unroll
            for (int sp = 0; sp < NSP; ++sp) vf[slot][sp] = frag_tr(V, DVT, SH::SWV, 16 * jt, sp);
        };
        load_j(0, 0);
#pragma unroll
        for (int jj = 0; jj < SH::NJC; ++jj) {
            if (jj + 1 < SH::NJC) load_j(jj + 1, (jj + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            const int sl = jj & 1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < SH::KSTEPS; ++k) acc = O::mma(sf[sl][k], qf[k], acc);
            if constexpr (SH::BF) {
#pragma unroll
                for (int sp = 0; 2 * sp <= TB; ++sp)
                    acc = O::mma(vf[sl][sp], O::from_acc(pt[2 * sp], pt[2 * sp + 1]), acc);
            } else {
#pragma unroll
                for (int sb = 0; sb <= TB; ++sb) acc = O::mma(vf[sl][sb], O::from_acc(pt[sb]), acc);
            }
            if constexpr (NM) acc *= rden;
            if constexpr (OG) acc *= *(const f32x4 *)(sEV[buf] + t * SH::LEV + 16 * (j0 + jj) + 4 * grp);
            *(V4 *)(stage + SH::ro(x, 16 * jj + 4 * grp)) = narrow4<T>(acc);
        }
        // read the block back row-contiguous and store 16-byte chunks (wave-local:
        // LDS operations of one wave complete in order)
#pragma unroll
        for (int h = 0; h < SH::OCPL; ++h) {
            const int chunk = lane + 64 * h;       // 8 lanes read one 128-byte row
            if (chunk < SH::OCH) {
                const int row = chunk / SH::SCH, col = (chunk % SH::SCH) * CE;
                const VC val = *(const VC *)(stage + SH::ro(row, col));
                if (16 * TB + row < nvalid)
                    *(VC *)(oh + (size_t)(t0 + 16 * TB + row) * DV + 16 * j0 + col) = val;
            }
        }
    };

    // State step of the chunk starting at t0 in operand buffer `buf`, by the owners:
    // S <- Diag(exp Gamma) (S + K^^T V) (outer gate: times Diag(exp GB) on the right;
    // state-only pass: S += K'^T V, the keys already decayed to the segment end).
    auto state_step = [&](int t0, int buf) __attribute__((always_inline)) {
        const int nvalid = min(L - t0, C);
        const T *KS = sK[buf], *V = sV[buf];
        auto vfrag = [&](int jt, int cs) __attribute__((always_inline)) -> F {
            return frag_tr(V, DVT, SH::SWV, 16 * jt, cs);
        };
        if constexpr (BLK) {
            F af[IPC][SH::CSTEPS];
#pragma unroll
            for (int ia = 0; ia < IPC; ++ia)
#pragma unroll
                for (int cs = 0; cs < SH::CSTEPS; ++cs) af[ia][cs] = frag_tr(KS, DK, SH::SWK, 16 * (ow + NOW * ia), cs);
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) {
                F bfr[SH::CSTEPS];
#pragma unroll
                for (int cs = 0; cs < SH::CSTEPS; ++cs) bfr[cs] = vfrag(jt, cs);
#pragma unroll
                for (int ia = 0; ia < IPC; ++ia) {
                    const int k = jt * IPC + ia;
                    f32x4 acc = S[k];
#pragma unroll
                    for (int cs = 0; cs < SH::CSTEPS; ++cs) acc = O::mma(af[ia][cs], bfr[cs], acc);
                    if constexpr (FG && !SO) acc *= *(const f32x4 *)(sEG[buf] + 16 * (ow + NOW * ia) + 4 * grp);
                    if constexpr (OG) acc *= sEGV[buf][16 * jt + x];
                    S[k] = acc;
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < NSLOT; ++k) {
                if (tile_ok(k)) {
                    const int it = tile_i(k), jt = tile_j(k);
                    f32x4 acc = S[k];
#pragma unroll
                    for (int cs = 0; cs < SH::CSTEPS; ++cs)
                        acc = O::mma(frag_tr(KS, DK, SH::SWK, 16 * it, cs), vfrag(jt, cs), acc);
                    if constexpr (FG && !SO) acc *= *(const f32x4 *)(sEG[buf] + 16 * it + 4 * grp);
                    if constexpr (OG) acc *= sEGV[buf][16 * jt + x];
                    S[k] = acc;
                }
            }
        }
        if constexpr (NM) {                        // z <- Diag(e^Gamma)(z + K^^T 1)
            // the value-1 operand, 0 for rows past L (their keys are phi(0), not 0,
            // under elu+1)
            F ones[SH::CSTEPS];
#pragma unroll
            for (int cs = 0; cs < SH::CSTEPS; ++cs) {
#pragma unroll
                for (int e = 0; e < (int)(sizeof(F) / sizeof(T)); ++e) {
                    const int s = SH::BF ? 32 * cs + 4 * grp + (e & 3) + 16 * (e >> 2) : 16 * cs + 4 * grp + e;
                    ones[cs][e] = from_f32<T>(s < nvalid ? 1.f : 0.f);
                }
            }
#pragma unroll
            for (int m = 0; m < NZ; ++m) {
                if (z_ok(m)) {
                    const int it = ow + NOW * m;
                    f32x4 acc = Z[m];
#pragma unroll
                    for (int cs = 0; cs < SH::CSTEPS; ++cs) acc = O::mma(frag_tr(KS, DK, SH::SWK, 16 * it, cs), ones[cs], acc);
                    if constexpr (FG) acc *= *(const f32x4 *)(sEG[buf] + 16 * it + 4 * grp);
                    Z[m] = acc;
                }
            }
        }
    };

    // Outputs of the chunk starting at t0 from operand buffer `buf` and state copy `par`
    // (consumers), then, where the consumers own the state, its step and next copy.
    auto consume = [&](int t0, int buf, int par) __attribute__((always_inline)) {
        if constexpr (!SO) {
            const int nvalid = min(L - t0, C);
            const T *Q = sQ[buf], *K = sK[buf], *V = sV[buf], *SS = sS[par];
            // consumer c owns t-block c % NTB (value tiles from (c / NTB) * NJC), or the
            // t-blocks tb with tb % NC == c when there are more t-blocks than consumers
            static_for<NTB>([&](auto tbc) __attribute__((always_inline)) {
                constexpr int TB = decltype(tbc)::value;
                if constexpr (NTB <= NC) {
                    if (c < NTB * SH::JS && TB == c % NTB)
                        out_block(tbc, (c / NTB) * SH::NJC, t0, nvalid, buf, par, Q, K, V, SS);
                } else {
                    if (TB % NC == c) out_block(tbc, 0, t0, nvalid, buf, par, Q, K, V, SS);
                }
            });
        }
        if constexpr (!POWN) {
            state_step(t0, buf);
            if constexpr (!SO) write_state(par ^ 1);
            write_z(par ^ 1);
        }
    };

    // ---------------- chunks out of the factorised form's range -------------------------
    // Whether the chunk in operand buffer `buf` has a cumulative log2-gate below
    // -kFastLim (the producers' flags, read after the barrier that publishes them, so
    // every wave takes the same decision).
    auto chunk_far = [&](int buf) __attribute__((always_inline)) -> bool {
        int f = 0;
        if constexpr (OG) {
            float mk = sMin[buf][0][0], mv = sMin[buf][1][0];
#pragma unroll
            for (int i = 1; i < NP; ++i) {
                mk = fminf(mk, sMin[buf][0][i]);
                mv = fminf(mv, sMin[buf][1][i]);
            }
            f = mk + mv < -kFastLim ? 1 : 0;
        } else {
#pragma unroll
            for (int i = 0; i < NP; ++i) f |= sFlag[buf][i];
        }
        return __builtin_amdgcn_readfirstlane(f) != 0;
    };
    // The chunk starting at t0, token by token (gla_slow.hpp), by the consumer waves.
    // The state's owners hand their fp32 tiles over through the space of the bf16
    // state copies (as [j][i]) before the first barrier and take them back after the
    // last, then write the next copy; the operand buffers stage the rows.  Neither is
    // needed otherwise at this point: the chunk's own operands are not used, and the
    // producers fill the next chunk's buffer only afterwards.  Barriers: A, 2 per
    // staged group, B, C, on both roles (slow_run, slow_pass).  (The state-only pass
    // has no such chunks.)
    constexpr int SR = NBUF == 2 ? C : C / 2;        // rows staged at a time
    static_assert(SR * DK * 4 <= (int)sizeof(sQ) && 2 * SR * DK * ES <= (int)sizeof(sK) &&
                  SR * DVT * ES <= (int)sizeof(sV) && DVT * DK * 4 <= (int)sizeof(sS) &&
                  (!NM || DK * 4 <= (int)sizeof(sZ)) && (!OG || SR * DVT * 4 <= (int)sizeof(sEV)),
                  "token-loop staging within the operand buffers");
    float *const PS = (float *)&sS[0][0];
    float *const PZ = &sZ[0][0];
    auto slow_give = [&]() __attribute__((always_inline)) {          // owners
        // S[16it + 4grp + r][16jt + x] -> PS[16jt + x][16it + 4grp + r]
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            if (tile_ok(k)) {
                const int it = tile_i(k), jt = tile_j(k);
                *(f32x4 *)(PS + (16 * jt + x) * DK + 16 * it + 4 * grp) = S[k];
            }
        }
        if constexpr (NM) {
#pragma unroll
            for (int m = 0; m < NZ; ++m)
                if (z_ok(m) && x == 0) *(f32x4 *)(PZ + 16 * (ow + NOW * m) + 4 * grp) = Z[m];
        }
    };
    // (PS lies over the bf16 state copies: every owner has read its tiles back, barrier
    // C, before any writes the next copy)
    auto slow_take = [&](int par) __attribute__((always_inline)) {   // owners
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            if (tile_ok(k)) {
                const int it = tile_i(k), jt = tile_j(k);
                S[k] = *(const f32x4 *)(PS + (16 * jt + x) * DK + 16 * it + 4 * grp);
            }
        }
        if constexpr (NM) {
#pragma unroll
            for (int m = 0; m < NZ; ++m)
                if (z_ok(m)) Z[m] = *(const f32x4 *)(PZ + 16 * (ow + NOW * m) + 4 * grp);
        }
        lds_barrier();                                               // C
        write_state(par);
        write_z(par);
    };
    // consumers: the token loop between barriers A and B
    auto slow_run = [&](int t0, int par) __attribute__((always_inline)) {
        const int nvalid = min(L - t0, C);
        if constexpr (!POWN) slow_give();
        lds_barrier();                                               // A: state handed over
        const SlowStage<T> st{(float *)&sQ[0][0], OG ? &sEV[0][0] : nullptr, &sK[0][0], &sK[0][0] + SR * DK,
                              &sV[0][0]};
        slow_chunk_lds<T, DK, DVT, SR, 64 * NC, ELU1, !SO, NM, OG, GATE == kGateScalar>(
            PS, PZ, st, rq, rk, rvv, rg, rgv, t0, nvalid, DV, vt * DVT, SO ? nullptr : oh + (size_t)t0 * DV, tid - 64 * NP);
        lds_barrier();                                               // B: state back in PS / PZ
        if constexpr (!POWN) slow_take(par);
        else lds_barrier();                                          // C
    };
    // producers: the same barriers
    auto slow_pass = [&](int t0, int par) __attribute__((always_inline)) {
        if constexpr (POWN) slow_give();
        lds_barrier();                                               // A
        const int groups = (min(L - t0, C) + SR - 1) / SR;
        for (int i = 0; i < 2 * groups; ++i) lds_barrier();
        lds_barrier();                                               // B
        if constexpr (POWN) slow_take(par);
        else lds_barrier();                                          // C
    };
    // the owners' step for the chunk starting at t0 in buffer `buf`, then the copy of
    // the new state for the next chunk (parity `par`)
    auto own_step = [&](int t0, int buf, int par) __attribute__((always_inline)) {
        state_step(t0, buf);
        write_state(par);
        write_z(par);
    };
    auto store_final = [&]() __attribute__((always_inline)) {        // owners
        if (a.s_final && (!a.final_last_seg || seg == a.nseg - 1)) {
            const size_t sh = a.final_last_seg ? (size_t)bh : (size_t)bhs;
#pragma unroll
            for (int k = 0; k < NSLOT; ++k) {
                if (tile_ok(k)) {
                    const int it = tile_i(k), jt = tile_j(k);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * it + 4 * grp + r;
                        a.s_final[(sh * DK + i) * DV + vt * DVT + 16 * jt + x] = S[k][r];
                    }
                }
            }
        }
        if constexpr (NM) {
            if (a.z_final && vt == 0 && x == 0) {
#pragma unroll
                for (int m = 0; m < NZ; ++m)
                    if (z_ok(m)) *(f32x4 *)(a.z_final + (size_t)bhs * DK + 16 * (ow + NOW * m) + 4 * grp) = Z[m];
            }
        }
    };
    // chunks may leave the factorised range (not in the state-only pass, whose key
    // exponents are <= 0)
    constexpr bool KD = FG && !SO;
    // first row of the n-th chunk in processing order: the state-only pass walks its
    // segment last chunk first; past the last chunk, rows beyond the end (zeros)
    auto row_of = [&](int n) __attribute__((always_inline)) -> int {
        if constexpr (SO) return n < nchunks ? (nchunks - 1 - n) * C : n * C;
        else return n * C;
    };

    // ---------------- pipeline ---------------------------------------------------------
    // The two roles run separate loops (so their registers are not live at the same
    // time) that meet at the same number of barriers.  With two buffers both run
    // 1 + 2*npairs barriers over chunk pairs; producers always request and prepare
    // (rows past the end read as zeros, surplus operands are never read), so the loop
    // has no branch around its global loads.  With one buffer: 2 * nchunks barriers.
    // A chunk out of the factorised range adds the same barriers on both sides.
    if (producer) {
        if constexpr (NBUF == 2) {
            const int npairs = (nchunks + 1) / 2;
            // operands one chunk ahead of the consumers, raw rows NRAW chunks ahead (raw
            // set n % NRAW holds chunk n)
            if constexpr (POWN) {                  // the producers own the state
                load_s0();
                load_z0();
            }
            if (nchunks > 0) {
                load_raw(R[0], row_of(0));
                if constexpr (NRAW == 2) load_raw(R[NRAW - 1], row_of(1));
                produce(R[0], row_of(0), 0, row_of(NRAW));
            }
            if constexpr (POWN) {
                write_state(0);
                write_z(0);
            }
            lds_barrier();
            for (int n = 0; n < 2 * npairs; n += 2) {
                // chunk n (buffer 0) out of range: the consumers compute it token by token
                bool far = false;
                if constexpr (KD) {
                    far = n < nchunks && chunk_far(0);
                    if (far) slow_pass(n * C, 1);
                }
                produce(R[1 % NRAW], row_of(n + 1), 1, row_of(n + 1 + NRAW));
                if constexpr (POWN) {
                    if (n < nchunks && !far) own_step(n * C, 0, 1);
                }
                lds_barrier();
                far = false;
                if constexpr (KD) {
                    far = n + 1 < nchunks && chunk_far(1);
                    if (far) slow_pass((n + 1) * C, 0);
                }
                produce(R[0], row_of(n + 2), 0, row_of(n + 2 + NRAW));
                if constexpr (POWN) {
                    if (n + 1 < nchunks && !far) own_step((n + 1) * C, 1, 0);
                }
                lds_barrier();
            }
        } else {
            if constexpr (POWN) {
                load_s0();
                load_z0();
            }
            if (nchunks > 0) load_raw(R[0], row_of(0));
            if constexpr (POWN) {
                write_state(0);
                write_z(0);
            }
            for (int n = 0; n < nchunks; ++n) {
                produce(R[0], row_of(n), 0, row_of(n + 1));
                lds_barrier();
                if (KD && chunk_far(0)) slow_pass(n * C, (n & 1) ^ 1);
                else if constexpr (POWN) own_step(n * C, 0, (n & 1) ^ 1);
                lds_barrier();
            }
        }
        if constexpr (SO && GATE != kGateNone) {   // segment gate totals (log2 units)
            if (vt == 0 && gate_lane && rs == 0) {
#pragma unroll
                for (int e = 0; e < CE; ++e) a.gam[(size_t)bhs * DK + ic + e] = gsum[e];
            }
        }
        if constexpr (POWN) store_final();
    } else {
        if constexpr (!POWN) {                     // the consumers own the state
            load_s0();
            load_z0();
            if constexpr (!SO) write_state(0);
            write_z(0);
        }
        if constexpr (NBUF == 2) {
            const int npairs = (nchunks + 1) / 2;
            lds_barrier();
            // a chunk out of range leaves the loop for the token-by-token block below,
            // which rejoins it at the next chunk (keeps that block out of the loop body)
            int n = 0;
            for (;;) {
                for (; n < 2 * npairs; ++n) {
                    if (n < nchunks) {
                        if (KD && chunk_far(n & 1)) break;
                        consume(n * C, n & 1, n & 1);
                    }
                    lds_barrier();
                }
                if (n >= 2 * npairs) break;
                slow_run(n * C, (n & 1) ^ 1);
                lds_barrier();
                ++n;
            }
        } else {
            int n = 0;
            for (;;) {
                for (; n < nchunks; ++n) {
                    lds_barrier();
                    if (KD && chunk_far(0)) break;
                    consume(n * C, 0, n & 1);
                    lds_barrier();
                }
                if (n >= nchunks) break;
                slow_run(n * C, (n & 1) ^ 1);
                lds_barrier();
                ++n;
            }
        }
        if constexpr (!POWN) store_final();
    }
}

template <typename T, int DK, int C, int DVT, int GATE, bool ELU1, bool SO, bool NM>
hipError_t launch_prefill_inst(const PrefillArgs &a, hipStream_t stream)
{
    const int grid = a.BH * a.nseg * a.n_vt;
    hipLaunchKernelGGL((prefill_kernel<T, DK, C, DVT, GATE, ELU1, SO, NM>), dim3(grid),
                       dim3(PrefillShape<T, DK, C, DVT>::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gla
