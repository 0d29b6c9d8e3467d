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
// Decomposition: one workgroup of NW wavefronts per (batch*head, tile of DVT value
// columns) walks the chunks of its head in order.  The fp32 state slice
// S[d_k][DVT] lives in MFMA accumulator registers, split into 16x16 tiles dealt
// round-robin to the waves.  Per chunk:
//   A/B (all waves)  raw q, k, g rows prefetched into registers during the previous
//       chunk are turned into LDS operands: each wave owns DK/NW key columns for all
//       C rows, forms the cumulative gate sums with an in-register scan plus a
//       cross-lane scan, and writes Q~, K^ (row-major) and K^ (or the scalar-gate
//       K~) transposed; v is written transposed; each wave writes its state tiles
//       as bf16 for the read-out.  Then the next chunk's raw rows are requested.
//   D   (per wave)   for its 16-row blocks tb of the chunk: the score tiles
//       P^T[s-block <= tb][tb] (kept in registers), then per 16-column value tile
//       O^T = S^T Q~^T + V^T P^T, stored to global memory; then its state tiles
//       S += K^^T V and the gate decay.
// Two LDS barriers per chunk; the barrier waits only for LDS traffic, so the
// prefetched global loads stay in flight across it.  bf16 inputs use bf16 MFMA
// operands with fp32 accumulation; fp32 inputs use fp32 MFMA.
#pragma once

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

template <typename T, int DK, int C, int DVT, int NW>
struct PrefillShape {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int NT = 64 * NW;
    static constexpr int NTB = C / 16;             // 16-row blocks per chunk
    static constexpr int NKB = DK / 16;            // 16-blocks of the key dim
    static constexpr int NJT = DVT / 16;           // 16-column value tiles
    static constexpr int SW = Op<T>::W;            // contraction width per MFMA step
    static constexpr int KSTEPS = (DK + SW - 1) / SW;   // steps over the key dim
    static constexpr int PAD = 16 / sizeof(T);     // 16 bytes of row padding in LDS
    static constexpr int LDK = DK + PAD;           // rows of length d_k
    static constexpr int LDC = C + PAD;            // rows of length C
    // gate stage: wave w owns key columns [w*CW, (w+1)*CW) for all C rows
    static constexpr int CW = DK / NW;
    static constexpr int CG = CW / 4;              // 4-column groups per wave
    static constexpr int RSEG = (64 / CG) < C ? (64 / CG) : C;
    static constexpr int RPS = C / RSEG;           // rows per lane
    // value stage: the whole workgroup covers C x DVT, a lane 4 columns x RV rows
    static constexpr int CGV = DVT / 4;
    static constexpr int RGV = (NT / CGV) < C ? (NT / CGV) : C;
    static constexpr int RV = C / RGV;
    // state tiles dealt round-robin to the waves
    static constexpr int NU = NKB * NJT;
    static constexpr int NSLOT = (NU + NW - 1) / NW;
    static_assert(CW >= 4 && CW % 4 == 0 && 64 % CG == 0, "gate-stage mapping");
    static_assert(NT % CGV == 0, "value-stage mapping");
    static_assert(RPS >= 1 && RV >= 1, "rows per lane");
};

template <typename T, int DK, int C, int DVT, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(const PrefillArgs a)
{
    using SH = PrefillShape<T, DK, C, DVT, NW>;
    using O = Op<T>;
    using V4 = typename Vec4<T>::type;
    constexpr int NTB = SH::NTB, NKB = SH::NKB, NJT = SH::NJT, LDK = SH::LDK, LDC = SH::LDC;
    constexpr int CW = SH::CW, CG = SH::CG, RSEG = SH::RSEG, RPS = SH::RPS;
    constexpr int CGV = SH::CGV, RGV = SH::RGV, RV = SH::RV, NSLOT = SH::NSLOT, NU = SH::NU;

    __shared__ __attribute__((aligned(16))) T sQ[C * LDK];     // Q~ [t][i]
    __shared__ __attribute__((aligned(16))) T sK[C * LDK];     // K^ [s][i]
    __shared__ __attribute__((aligned(16))) T sKT[DK * LDC];   // K^ (scalar gate: K~) [i][s]
    __shared__ __attribute__((aligned(16))) T sVT[DVT * LDC];  // V^T [j][s]
    __shared__ __attribute__((aligned(16))) T sS[DVT * LDK];   // state^T [j][i] (operand copy)
    __shared__ float sEG[DK];                                  // exp(Gamma_i)
    __shared__ float sB[C];                                    // scalar gate: B_t (log2 units)

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;

    int wg = blockIdx.x;
    if (a.xcd_remap) wg = (wg & 7) * (gridDim.x >> 3) + (wg >> 3);
    const int bh = wg / a.n_vt;
    const int vt = wg - bh * a.n_vt;
    const int L = a.L, DV = a.d_v;
    const bool elu1 = a.elu1 != 0;
    const int gate = a.gate;

    const T *__restrict__ qh = (const T *)a.q + (size_t)bh * L * DK;
    const T *__restrict__ kh = (const T *)a.k + (size_t)bh * L * DK;
    const T *__restrict__ vh = (const T *)a.v + (size_t)bh * L * DV + vt * DVT;
    T *__restrict__ oh = (T *)a.o + (size_t)bh * L * DV + vt * DVT;
    const float *__restrict__ gk = a.g + (size_t)bh * L * DK;   // key-dim gates
    const float *__restrict__ gs = a.g + (size_t)bh * L;        // scalar gates

    // ---- state tiles owned by this wave: tile u = slot*NW + w, (i-tile, j-tile) -----
    f32x4 S[NSLOT];
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) S[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.s0) {                                     // branch-free loads, issued together
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int u = k * NW + w;
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

    // ---- gate-stage lane coordinates ------------------------------------------------
    const int cg = lane % CG, rs = lane / CG;
    const bool gate_lane = rs < RSEG;
    const int ic = w * CW + 4 * cg;                 // first of this lane's 4 key columns
    const int cgv = tid % CGV, rgv = tid / CGV;
    const bool v_lane = rgv < RGV;

    V4 qr[RPS], kr[RPS], vr[RV];
    f32x4 gr[RPS];

    auto load_raw = [&](int t0) {
        if (gate_lane) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int row = min(t0 + rs * RPS + r, L - 1);   // clamp: always in bounds
                qr[r] = *(const V4 *)(qh + (size_t)row * DK + ic);
                kr[r] = *(const V4 *)(kh + (size_t)row * DK + ic);
            }
            if (gate == kGateKeydim) {
#pragma unroll
                for (int r = 0; r < RPS; ++r) {
                    const int row = min(t0 + rs * RPS + r, L - 1);
                    gr[r] = *(const f32x4 *)(gk + (size_t)row * DK + ic);
                }
            } else if (gate == kGateScalar) {
#pragma unroll
                for (int r = 0; r < RPS; ++r) {
                    const int row = min(t0 + rs * RPS + r, L - 1);
                    const float gv = gs[row];
                    gr[r] = f32x4{gv, gv, gv, gv};
                }
            }
        }
        if (v_lane) {
#pragma unroll
            for (int r = 0; r < RV; ++r) {
                const int row = min(t0 + rgv * RV + r, L - 1);
                vr[r] = *(const V4 *)(vh + (size_t)row * DV + 4 * cgv);
            }
        }
    };

    const int nchunks = (L + C - 1) / C;
    if (nchunks > 0) load_raw(0);

    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * C;
        const int nvalid = min(L - t0, C);

        // ================= A/B: operands of chunk n into LDS ==========================
        // state tiles as bf16 (or fp32) operand rows S^T[j][i]
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int u = k * NW + w;
            if (u < NU) {
                const int it = u % NKB, jt = u / NKB;
                *(V4 *)(sS + (16 * jt + x) * LDK + 16 * it + 4 * grp) = narrow4<T>(S[k]);
            }
        }
        if (gate_lane) {
            // cumulative log2-gates: serial within this lane's rows, then across lanes
            f32x4 bc[RPS];
            f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const bool valid = rs * RPS + r < nvalid;
                const f32x4 gl = (gate != kGateNone && valid) ? gr[r] * kLog2e : f32x4{0.f, 0.f, 0.f, 0.f};
                run += gl;
                bc[r] = run;
            }
            f32x4 incl = run;
#pragma unroll
            for (int off = 1; off < RSEG; off <<= 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float up = __shfl_up(incl[e], off * CG, 64);
                    if (rs >= off) incl[e] += up;
                }
            }
            f32x4 excl = incl - run, tot;
#pragma unroll
            for (int e = 0; e < 4; ++e) tot[e] = __shfl(incl[e], (RSEG - 1) * CG + cg, 64);

            typedef T KTvec __attribute__((ext_vector_type(RPS)));
            KTvec ktv[4];
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int t = rs * RPS + r;
                const bool valid = t < nvalid;
                const f32x4 b = excl + bc[r];
                const f32x4 q = widen(qr[r]), kk = widen(kr[r]);
                f32x4 qt, kt, kT;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float fq = valid ? feature(q[e], elu1) : 0.f;
                    const float fk = valid ? feature(kk[e], elu1) : 0.f;
                    if (gate == kGateKeydim) {
                        qt[e] = fq * exp2_fast(b[e]);
                        kt[e] = fk * exp2_fast(-b[e]);
                        kT[e] = kt[e];
                    } else if (gate == kGateScalar) {
                        qt[e] = fq;
                        kt[e] = fk;
                        kT[e] = fk * exp2_fast(tot[e] - b[e]);
                    } else {
                        qt[e] = fq;
                        kt[e] = fk;
                        kT[e] = fk;
                    }
                    ktv[e][r] = from_f32<T>(kT[e]);
                }
                *(V4 *)(sQ + t * LDK + ic) = narrow4<T>(qt);
                *(V4 *)(sK + t * LDK + ic) = narrow4<T>(kt);
                if (gate == kGateScalar && w == 0 && cg == 0) sB[t] = b[0];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) *(KTvec *)(sKT + (ic + e) * LDC + rs * RPS) = ktv[e];
            if (rs == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sEG[ic + e] = gate == kGateNone ? 1.f : exp2_fast(tot[e]);
            }
        }
        if (v_lane) {
            typedef T Vvec __attribute__((ext_vector_type(RV)));
            Vvec vv[4];
#pragma unroll
            for (int r = 0; r < RV; ++r) {
                const bool valid = rgv * RV + r < nvalid;
                const f32x4 vf = widen(vr[r]);
#pragma unroll
                for (int e = 0; e < 4; ++e) vv[e][r] = from_f32<T>(valid ? vf[e] : 0.f);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) *(Vvec *)(sVT + (4 * cgv + e) * LDC + rgv * RV) = vv[e];
        }
        // request the next chunk's rows; they arrive while this chunk is computed
        if (n + 1 < nchunks) load_raw(t0 + C);
        lds_barrier();

        // ================= D: outputs and the state step ===============================
        for (int tb = w; tb < NTB; tb += NW) {
            const int t = 16 * tb + x;
            typename O::frag qf[SH::KSTEPS];
#pragma unroll
            for (int k = 0; k < SH::KSTEPS; ++k) {
                if constexpr (SH::BF) {
                    qf[k] = (32 * k + 8 * grp < DK) ? O::contig(sQ + t * LDK, k, grp) : O::zero();
                } else {
                    qf[k] = O::contig(sQ + t * LDK, k, grp);
                }
            }
            // score tiles P^T[s-block sb][t-block tb], lane holds P[t][16sb + 4grp + r]
            f32x4 pt[NTB];
#pragma unroll
            for (int sb = 0; sb < NTB; ++sb) {
                if (sb > tb) break;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int srow = 16 * sb + x;
#pragma unroll
                for (int k = 0; k < SH::KSTEPS; ++k) {
                    typename O::frag af;
                    if constexpr (SH::BF) af = (32 * k + 8 * grp < DK) ? O::contig(sK + srow * LDK, k, grp) : O::zero();
                    else af = O::contig(sK + srow * LDK, k, grp);
                    acc = O::mma(af, qf[k], acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * sb + 4 * grp + r;
                    float p = s <= t ? acc[r] : 0.f;
                    if (gate == kGateScalar && s <= t) p *= exp2_fast(sB[t] - sB[s]);
                    acc[r] = p;
                }
                pt[sb] = acc;
            }
            const float inter_scale = gate == kGateScalar ? exp2_fast(sB[t]) : 1.f;
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) {
                const int jrow = 16 * jt + x;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                // inter-chunk: O^T += S^T Q~^T
#pragma unroll
                for (int k = 0; k < SH::KSTEPS; ++k) {
                    typename O::frag af;
                    if constexpr (SH::BF) af = (32 * k + 8 * grp < DK) ? O::contig(sS + jrow * LDK, k, grp) : O::zero();
                    else af = O::contig(sS + jrow * LDK, k, grp);
                    acc = O::mma(af, qf[k], acc);
                }
                acc *= inter_scale;
                // intra-chunk: O^T += V^T P^T over s-blocks 0..tb
                if constexpr (SH::BF) {
#pragma unroll
                    for (int sp = 0; sp < (NTB + 1) / 2; ++sp) {
                        if (2 * sp > tb) break;
                        const bool hi = 2 * sp + 1 <= tb;
                        typename O::frag af, bf;
                        if (hi) {
                            af = O::split(sVT + jrow * LDC, sp, grp);
                            bf = O::from_acc(pt[2 * sp], pt[2 * sp + 1]);
                        } else {    // only the first 16-block of this pair is in range
                            const bf16x4 lo = *(const bf16x4 *)(sVT + jrow * LDC + 32 * sp + 4 * grp);
                            af = typename O::frag{lo[0], lo[1], lo[2], lo[3], (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
                            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                            bf = O::from_acc(pt[2 * sp], z);
                        }
                        acc = O::mma(af, bf, acc);
                    }
                } else {
#pragma unroll
                    for (int sb = 0; sb < NTB; ++sb) {
                        if (sb > tb) break;
                        acc = O::mma(O::split(sVT + jrow * LDC, sb, grp), O::from_acc(pt[sb]), acc);
                    }
                }
                if (t < nvalid) store4(oh + (size_t)(t0 + t) * DV + 16 * jt + 4 * grp, acc);
            }
        }
        // state tiles: S <- Diag(exp Gamma) (S + K^^T V)  (scalar gate: exp(Gamma) S + K~^T V)
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int u = k * NW + w;
            if (u < NU) {
                const int it = u % NKB, jt = u / NKB;
                const T *arow = sKT + (16 * it + x) * LDC;
                const T *brow = sVT + (16 * jt + x) * LDC;
                f32x4 acc = S[k];
                if (gate == kGateScalar) acc *= sEG[0];
                constexpr int CSTEPS = (C + SH::SW - 1) / SH::SW;
#pragma unroll
                for (int c = 0; c < CSTEPS; ++c) {
                    typename O::frag af, bfr;
                    if constexpr (SH::BF) {
                        const bool in = 32 * c + 8 * grp < C;
                        af = in ? O::contig(arow, c, grp) : O::zero();
                        bfr = in ? O::contig(brow, c, grp) : O::zero();
                    } else {
                        af = O::contig(arow, c, grp);
                        bfr = O::contig(brow, c, grp);
                    }
                    acc = O::mma(af, bfr, acc);
                }
                if (gate == kGateKeydim) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] *= sEG[16 * it + 4 * grp + r];
                }
                S[k] = acc;
            }
        }
        lds_barrier();
    }

    if (a.s_final) {
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
            const int u = k * NW + w;
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

template <typename T, int DK, int C, int DVT, int NW>
hipError_t launch_prefill_inst(const PrefillArgs &a, hipStream_t stream)
{
    const int grid = a.BH * a.n_vt;
    hipLaunchKernelGGL((prefill_kernel<T, DK, C, DVT, NW>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gla
