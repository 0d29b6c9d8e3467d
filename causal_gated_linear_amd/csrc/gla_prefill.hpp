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
// Scalar gates (one log-gate b per token) use the exact mask form instead, so no
// factor exceeds 1: P = (phi(Q) phi(K)^T) * exp(b_t - b_s), O_inter = exp(b_t) phi(Q) S,
// S <- exp(Gamma) S + (phi(K) * exp(Gamma - b))^T V.  The key-dim factorisation needs
// exp(-B) finite: the in-chunk cumulative log-gate must stay above about -80.
//
// Decomposition: one workgroup per (batch*head, tile of DVT value columns) walks the
// chunks of its head in order, with two kinds of wavefronts:
//   producers (NP waves)  turn raw q, k, g, v rows into matrix-core operands in LDS:
//       each owns DK/NP key columns of all C rows, forms the cumulative gate sums
//       with an in-register scan plus a cross-lane scan, and writes Q~ and K^
//       row-major and K^ (scalar gate: K~) and V transposed.  Raw rows are requested
//       two chunks ahead into registers.
//   consumers (NC waves)  hold the fp32 state slice S[d_k][DVT] in accumulator
//       registers (16x16 tiles dealt round-robin) and, per 16-row block tb of the
//       chunk they own, compute the score tiles P^T[s-block <= tb][tb] in registers
//       and O^T = S^T Q~^T + V^T P^T per 16-column value tile, stored to global
//       memory; then S += K^^T V and the gate decay.  The state is shared between
//       consumers as a bf16 operand copy in LDS.
// With two LDS operand buffers the producers prepare chunk n+1 while the consumers
// compute chunk n (one barrier per chunk); where two buffers do not fit in LDS the
// phases alternate on one buffer.  Barriers wait only for LDS traffic, so requested
// global rows stay in flight.  bf16 inputs use bf16 MFMA operands with fp32
// accumulation; fp32 inputs use fp32 MFMA.
#pragma once

#include <type_traits>

#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

// Barrier for LDS communication only: waits for this wave's LDS operations, not
// for its outstanding global loads.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

__device__ __forceinline__ f32x4 widen(bf16x4 v) { return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }
__device__ __forceinline__ f32x4 widen(f32x4 v) { return v; }

template <typename E> __device__ __forceinline__ typename Vec4<E>::type narrow4(f32x4 v);
template <> __device__ __forceinline__ bf16x4 narrow4<bf16>(f32x4 v)
{
    return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
template <> __device__ __forceinline__ f32x4 narrow4<float>(f32x4 v) { return v; }

// Operand fragment of one matrix-core step (see gla_device.hpp for the lane layout).
// bf16: one 16x16x32 step covers a 32-wide slice of the contraction index; lane
// group grp holds 8 values.  fp32: a 16-wide block is 4 steps of 16x16x4.
template <typename E> struct Op;

template <> struct Op<bf16> {
    typedef bf16x8 frag;                           // one step
    static constexpr int W = 32;                   // contraction width of one step
    // contiguous convention: elements [32k + 8grp, 32k + 8grp + 7] of an LDS row
    static __device__ __forceinline__ frag contig(const bf16 *row, int k, int grp)
    {
        return *(const bf16x8 *)(row + 32 * k + 8 * grp);
    }
    // split convention (matches the accumulator layout): elements
    // [32k + 4grp, +3] and [32k + 16 + 4grp, +3]
    static __device__ __forceinline__ frag split(const bf16 *row, int k, int grp)
    {
        const bf16x4 a = *(const bf16x4 *)(row + 32 * k + 4 * grp);
        const bf16x4 b = *(const bf16x4 *)(row + 32 * k + 16 + 4 * grp);
        return frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    static __device__ __forceinline__ frag split_lo(const bf16 *row, int k, int grp)
    {
        const bf16x4 a = *(const bf16x4 *)(row + 32 * k + 4 * grp);
        return frag{a[0], a[1], a[2], a[3], (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    }
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
    typedef f32x4 frag;                            // 4 steps of 16x16x4 (one 16-block)
    static constexpr int W = 16;
    static __device__ __forceinline__ frag contig(const float *row, int k, int grp)
    {
        return *(const f32x4 *)(row + 16 * k + 4 * grp);
    }
    static __device__ __forceinline__ frag split(const float *row, int k, int grp)
    {
        return contig(row, k, grp);
    }
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

template <typename T, int DK, int C, int DVT>
struct PrefillShape {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int NP = 4, NC = 4;           // producer / consumer waves
    static constexpr int NT = 64 * (NP + NC);
    static constexpr int NTB = C / 16;             // 16-row blocks per chunk
    static constexpr int NKB = DK / 16;            // 16-blocks of the key dim
    static constexpr int NJT = DVT / 16;           // 16-column value tiles
    static constexpr int SW = Op<T>::W;            // contraction width per MFMA step
    static constexpr int KSTEPS = (DK + SW - 1) / SW;
    static constexpr int CSTEPS = (C + SW - 1) / SW;
    static constexpr int PAD = 16 / sizeof(T);     // 16 bytes of row padding in LDS
    static constexpr int LDK = DK + PAD;           // rows of length d_k
    static constexpr int LDC = C + PAD;            // rows of length C
    // producer gate mapping: producer p owns key columns [p*CW, (p+1)*CW)
    static constexpr int CW = DK / NP;
    static constexpr int CG = CW / 4;              // 4-column groups
    static constexpr int RSEG = (64 / CG) < C ? (64 / CG) : C;
    static constexpr int RPS = C / RSEG;           // rows per lane
    // producer value mapping: 64*NP lanes cover C x DVT, a lane 4 columns x RV rows
    static constexpr int CGV = DVT / 4;
    static constexpr int RGV = (64 * NP / CGV) < C ? (64 * NP / CGV) : C;
    static constexpr int RV = C / RGV;
    // consumer state tiles, dealt round-robin
    static constexpr int NU = NKB * NJT;
    static constexpr int NSLOT = (NU + NC - 1) / NC;
    // LDS: operand buffers (Q~, K^, K^T, V^T, exp Gamma, B) and the state copies
    static constexpr int NBUF = prefill_nbuf((int)sizeof(T), DK, C, DVT);
    static_assert(NBUF >= 1, "LDS budget");
    static_assert(CW >= 4 && CW % 4 == 0 && 64 % CG == 0, "producer gate mapping");
    static_assert((64 * NP) % CGV == 0, "producer value mapping");
    static_assert(RPS >= 1 && RV >= 1, "rows per lane");
};

template <typename T, int N> struct VecN { typedef T type __attribute__((ext_vector_type(N))); };
template <typename T> struct VecN<T, 1> { typedef T type; };

template <typename T, int DK, int C, int DVT, int GATE, bool ELU1>
__global__ __launch_bounds__(512) void prefill_kernel(const PrefillArgs a)
{
    using SH = PrefillShape<T, DK, C, DVT>;
    using O = Op<T>;
    using V4 = typename Vec4<T>::type;
    constexpr int NP = SH::NP, NC = SH::NC, NBUF = SH::NBUF;
    constexpr int NTB = SH::NTB, NKB = SH::NKB, NJT = SH::NJT, LDK = SH::LDK, LDC = SH::LDC;
    constexpr int CW = SH::CW, CG = SH::CG, RSEG = SH::RSEG, RPS = SH::RPS;
    constexpr int CGV = SH::CGV, RGV = SH::RGV, RV = SH::RV, NSLOT = SH::NSLOT, NU = SH::NU;

    __shared__ __attribute__((aligned(16))) T sQ[NBUF][C * LDK];     // Q~ [t][i]
    __shared__ __attribute__((aligned(16))) T sK[NBUF][C * LDK];     // K^ [s][i]
    __shared__ __attribute__((aligned(16))) T sKT[NBUF][DK * LDC];   // K^ (scalar: K~) [i][s]
    __shared__ __attribute__((aligned(16))) T sVT[NBUF][DVT * LDC];  // V^T [j][s]
    __shared__ __attribute__((aligned(16))) T sS[2][DVT * LDK];      // state^T [j][i], by parity
    __shared__ float sEG[NBUF][DK];                                  // exp(Gamma_i)
    __shared__ float sB[NBUF][C];                                    // scalar gate: B_t (log2)

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;
    const bool producer = w < NP;

    int wg = blockIdx.x;
    if (a.xcd_remap) wg = (wg & 7) * (gridDim.x >> 3) + (wg >> 3);
    const int bh = wg / a.n_vt;
    const int vt = wg - bh * a.n_vt;
    const int L = a.L, DV = a.d_v;

    const T *__restrict__ qh = (const T *)a.q + (size_t)bh * L * DK;
    const T *__restrict__ kh = (const T *)a.k + (size_t)bh * L * DK;
    const T *__restrict__ vh = (const T *)a.v + (size_t)bh * L * DV + vt * DVT;
    T *__restrict__ oh = (T *)a.o + (size_t)bh * L * DV + vt * DVT;
    const float *__restrict__ gk = a.g + (size_t)bh * L * DK;   // key-dim gates
    const float *__restrict__ gs = a.g + (size_t)bh * L;        // scalar gates
    const int nchunks = (L + C - 1) / C;

    // ---------------- producer state ------------------------------------------------
    const int p = w;                               // producer index (when producer)
    const int cg = lane % CG, rs = lane / CG;
    const bool gate_lane = producer && rs < RSEG;
    const int ic = p * CW + 4 * cg;                // first of this lane's 4 key columns
    const int ptid = tid;                          // producer thread index (< 64*NP)
    const int cgv = ptid % CGV, rgv = ptid / CGV;
    const bool v_lane = producer && rgv < RGV;

    struct Raw {
        V4 q[RPS], k[RPS], v[RV];
        f32x4 g[RPS];
    };
    Raw R[NBUF];

    auto load_raw = [&](Raw &r_, int t0) __attribute__((always_inline)) {
        if (gate_lane) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int row = min(t0 + rs * RPS + r, L - 1);   // clamp: always in bounds
                r_.q[r] = *(const V4 *)(qh + (size_t)row * DK + ic);
                r_.k[r] = *(const V4 *)(kh + (size_t)row * DK + ic);
                if constexpr (GATE == kGateKeydim) {
                    r_.g[r] = *(const f32x4 *)(gk + (size_t)row * DK + ic);
                } else if constexpr (GATE == kGateScalar) {
                    const float gv = gs[row];
                    r_.g[r] = f32x4{gv, gv, gv, gv};
                }
            }
        }
        if (v_lane) {
#pragma unroll
            for (int r = 0; r < RV; ++r) {
                const int row = min(t0 + rgv * RV + r, L - 1);
                r_.v[r] = *(const V4 *)(vh + (size_t)row * DV + 4 * cgv);
            }
        }
    };

    // Turn the raw rows of the chunk starting at t0 into the operands of buffer `buf`.
    auto produce = [&](Raw &r_, int t0, int buf) __attribute__((always_inline)) {
        const int nvalid = min(L - t0, C);
        if (nvalid < C) {                          // ragged tail: rows past L carry no gate
#pragma unroll                                     // and no value (their q, k are finite copies)
            for (int r = 0; r < RPS; ++r)
                if (rs * RPS + r >= nvalid) r_.g[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RV; ++r)
                if (rgv * RV + r >= nvalid) r_.v[r] = narrow4<T>(f32x4{0.f, 0.f, 0.f, 0.f});
        }
        if (gate_lane) {
            f32x4 bc[RPS];
            f32x4 incl = {0.f, 0.f, 0.f, 0.f}, excl = incl, tot = incl;
            if constexpr (GATE != kGateNone) {
                f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < RPS; ++r) {
                    run += r_.g[r];
                    bc[r] = run;
                }
                incl = run;
#pragma unroll
                for (int off = 1; off < RSEG; off <<= 1) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float up = __shfl_up(incl[e], off * CG, 64);
                        if (rs >= off) incl[e] += up;
                    }
                }
                excl = incl - run;
#pragma unroll
                for (int e = 0; e < 4; ++e) tot[e] = __shfl(incl[e], (RSEG - 1) * CG + cg, 64) * kLog2e;
            }
            typedef typename VecN<T, RPS>::type KTv;
            KTv ktv[4];
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int t = rs * RPS + r;
                f32x4 q = widen(r_.q[r]), kk = widen(r_.k[r]);
                if constexpr (ELU1) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        q[e] = feature(q[e], true);
                        kk[e] = feature(kk[e], true);
                    }
                }
                f32x4 qt = q, kt = kk, kT = kk;
                if constexpr (GATE == kGateKeydim) {
                    const f32x4 b = (excl + bc[r]) * kLog2e;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        qt[e] = q[e] * exp2_fast(b[e]);
                        kt[e] = kk[e] * exp2_fast(-b[e]);
                    }
                    kT = kt;
                } else if constexpr (GATE == kGateScalar) {
                    const float b = (excl[0] + bc[r][0]) * kLog2e;
                    kT = kk * exp2_fast(tot[0] - b);
                    if (p == 0 && cg == 0) sB[buf][t] = b;
                }
                *(V4 *)(sQ[buf] + t * LDK + ic) = narrow4<T>(qt);
                *(V4 *)(sK[buf] + t * LDK + ic) = narrow4<T>(kt);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (RPS == 1) ktv[e] = from_f32<T>(kT[e]);
                    else ktv[e][r] = from_f32<T>(kT[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) *(KTv *)(sKT[buf] + (ic + e) * LDC + rs * RPS) = ktv[e];
            if (rs == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sEG[buf][ic + e] = GATE == kGateNone ? 1.f : exp2_fast(tot[e]);
            }
        }
        if (v_lane) {
            typedef typename VecN<T, RV>::type Vv;
            Vv vv[4];
#pragma unroll
            for (int r = 0; r < RV; ++r) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (RV == 1) vv[e] = r_.v[r][e];
                    else vv[e][r] = r_.v[r][e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) *(Vv *)(sVT[buf] + (4 * cgv + e) * LDC + rgv * RV) = vv[e];
        }
    };

    // ---------------- consumer state ------------------------------------------------
    const int c = w - NP;                          // consumer index (when consumer)
    f32x4 S[NSLOT];
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!producer && a.s0) {                       // branch-free loads, issued together
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int u = k * NC + c;
            const int uc = u < NU ? u : NU - 1;
            const int it = uc % NKB, jt = uc / NKB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * grp + r;
                const float v = a.s0[((size_t)bh * DK + i) * DV + vt * DVT + 16 * jt + x];
                S[k][r] = u < NU ? v : 0.f;
            }
        }
    }

    auto write_state = [&](int par) __attribute__((always_inline)) {              // state tiles -> bf16 operand rows
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int u = k * NC + c;
            if (u < NU) {
                const int it = u % NKB, jt = u / NKB;
                *(V4 *)(sS[par] + (16 * jt + x) * LDK + 16 * it + 4 * grp) = narrow4<T>(S[k]);
            }
        }
    };

    // Outputs of chunk starting at t0 from operand buffer `buf`, then the state step.
    auto consume = [&](int t0, int buf, int par) __attribute__((always_inline)) {
        const int nvalid = min(L - t0, C);
        const T *Q = sQ[buf], *K = sK[buf], *KT = sKT[buf], *VT = sVT[buf], *SS = sS[par];
        for (int tb = c; tb < NTB; tb += NC) {
            const int t = 16 * tb + x;
            typename O::frag qf[SH::KSTEPS];
#pragma unroll
            for (int k = 0; k < SH::KSTEPS; ++k) {
                if constexpr (SH::BF && DK % 32 != 0)
                    qf[k] = (32 * k + 8 * grp < DK) ? O::contig(Q + t * LDK, k, grp) : O::zero();
                else
                    qf[k] = O::contig(Q + t * LDK, k, grp);
            }
            // score tiles P^T[s-block sb][t-block tb]: lane holds P[t][16sb + 4grp + r]
            f32x4 pt[NTB];
#pragma unroll
            for (int sb = 0; sb < NTB; ++sb) {
                if (sb > tb) break;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int srow = 16 * sb + x;
#pragma unroll
                for (int k = 0; k < SH::KSTEPS; ++k) {
                    typename O::frag af;
                    if constexpr (SH::BF && DK % 32 != 0)
                        af = (32 * k + 8 * grp < DK) ? O::contig(K + srow * LDK, k, grp) : O::zero();
                    else
                        af = O::contig(K + srow * LDK, k, grp);
                    acc = O::mma(af, qf[k], acc);
                }
                if constexpr (GATE == kGateScalar) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int s = 16 * sb + 4 * grp + r;
                        acc[r] = s <= t ? acc[r] * exp2_fast(sB[buf][t] - sB[buf][s]) : 0.f;
                    }
                } else if (sb == tb) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] = 4 * grp + r <= x ? acc[r] : 0.f;
                }
                pt[sb] = acc;
            }
            float inter_scale = 1.f;
            if constexpr (GATE == kGateScalar) inter_scale = exp2_fast(sB[buf][t]);
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) {
                const int jrow = 16 * jt + x;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                // inter-chunk: O^T += S^T Q~^T
#pragma unroll
                for (int k = 0; k < SH::KSTEPS; ++k) {
                    typename O::frag af;
                    if constexpr (SH::BF && DK % 32 != 0)
                        af = (32 * k + 8 * grp < DK) ? O::contig(SS + jrow * LDK, k, grp) : O::zero();
                    else
                        af = O::contig(SS + jrow * LDK, k, grp);
                    acc = O::mma(af, qf[k], acc);
                }
                if constexpr (GATE == kGateScalar) acc *= inter_scale;
                // intra-chunk: O^T += V^T P^T over s-blocks 0..tb
                if constexpr (SH::BF) {
#pragma unroll
                    for (int sp = 0; sp < (NTB + 1) / 2; ++sp) {
                        if (2 * sp > tb) break;
                        if (2 * sp + 1 <= tb) {
                            acc = O::mma(O::split(VT + jrow * LDC, sp, grp),
                                         O::from_acc(pt[2 * sp], pt[2 * sp + 1]), acc);
                        } else {            // only the first 16-block of this pair is in range
                            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                            acc = O::mma(O::split_lo(VT + jrow * LDC, sp, grp),
                                         O::from_acc(pt[2 * sp], z), acc);
                        }
                    }
                } else {
#pragma unroll
                    for (int sb = 0; sb < NTB; ++sb) {
                        if (sb > tb) break;
                        acc = O::mma(O::split(VT + jrow * LDC, sb, grp), O::from_acc(pt[sb]), acc);
                    }
                }
                if (t < nvalid) store4(oh + (size_t)(t0 + t) * DV + 16 * jt + 4 * grp, acc);
            }
        }
        // state tiles: S <- Diag(exp Gamma) (S + K^^T V)  (scalar gate: exp(Gamma) S + K~^T V)
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int u = k * NC + c;
            if (u < NU) {
                const int it = u % NKB, jt = u / NKB;
                const T *arow = KT + (16 * it + x) * LDC;
                const T *brow = VT + (16 * jt + x) * LDC;
                f32x4 acc = S[k];
                if constexpr (GATE == kGateScalar) acc *= sEG[buf][0];
#pragma unroll
                for (int cs = 0; cs < SH::CSTEPS; ++cs) {
                    typename O::frag af, bfr;
                    if constexpr (SH::BF && C % 32 != 0) {
                        const bool in = 32 * cs + 8 * grp < C;
                        af = in ? O::contig(arow, cs, grp) : O::zero();
                        bfr = in ? O::contig(brow, cs, grp) : O::zero();
                    } else {
                        af = O::contig(arow, cs, grp);
                        bfr = O::contig(brow, cs, grp);
                    }
                    acc = O::mma(af, bfr, acc);
                }
                if constexpr (GATE == kGateKeydim) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] *= sEG[buf][16 * it + 4 * grp + r];
                }
                S[k] = acc;
            }
        }
        write_state(par ^ 1);
    };

    // ---------------- pipeline ---------------------------------------------------------
    // The two roles run separate loops (so their registers are not live at the same
    // time) that meet at the same number of barriers: 1 + nchunks with two buffers,
    // 2 * nchunks with one.
    if (producer) {
        if constexpr (NBUF == 2) {
            // operands one chunk ahead of the consumers, raw rows two chunks ahead
            if (nchunks > 0) {
                load_raw(R[0], 0);
                if (nchunks > 1) load_raw(R[1], C);
                produce(R[0], 0, 0);
                if (nchunks > 2) load_raw(R[0], 2 * C);
            }
            lds_barrier();
            auto step = [&](auto pi, int n) __attribute__((always_inline)) {
                constexpr int PI = decltype(pi)::value;        // n % 2
                if (n + 1 < nchunks) {
                    produce(R[1 - PI], (n + 1) * C, 1 - PI);
                    if (n + 3 < nchunks) load_raw(R[1 - PI], (n + 3) * C);
                }
                lds_barrier();
            };
            for (int n = 0; n < nchunks; n += 2) {
                step(std::integral_constant<int, 0>{}, n);
                if (n + 1 < nchunks) step(std::integral_constant<int, 1>{}, n + 1);
            }
        } else {
            if (nchunks > 0) load_raw(R[0], 0);
            for (int n = 0; n < nchunks; ++n) {
                produce(R[0], n * C, 0);
                if (n + 1 < nchunks) load_raw(R[0], (n + 1) * C);
                lds_barrier();
                lds_barrier();
            }
        }
    } else {
        write_state(0);
        if constexpr (NBUF == 2) {
            lds_barrier();
            for (int n = 0; n < nchunks; ++n) {
                consume(n * C, n & 1, n & 1);
                lds_barrier();
            }
        } else {
            for (int n = 0; n < nchunks; ++n) {
                lds_barrier();
                consume(n * C, 0, n & 1);
                lds_barrier();
            }
        }
        if (a.s_final) {
#pragma unroll
            for (int k = 0; k < NSLOT; ++k) {
                const int u = k * NC + c;
                if (u < NU) {
                    const int it = u % NKB, jt = u / NKB;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * it + 4 * grp + r;
                        a.s_final[((size_t)bh * DK + i) * DV + vt * DVT + 16 * jt + x] = S[k][r];
                    }
                }
            }
        }
    }
}

template <typename T, int DK, int C, int DVT, int GATE, bool ELU1>
hipError_t launch_prefill_inst(const PrefillArgs &a, hipStream_t stream)
{
    const int grid = a.BH * a.n_vt;
    hipLaunchKernelGGL((prefill_kernel<T, DK, C, DVT, GATE, ELU1>), dim3(grid),
                       dim3(PrefillShape<T, DK, C, DVT>::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gla
