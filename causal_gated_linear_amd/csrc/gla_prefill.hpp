// gla_prefill.hpp -- chunkwise block-parallel prefill kernel for gfx950.
//
// The chunkwise form ("Gated Linear Attention", Summary and Methodology: chunks of
// C tokens, cost O(L/C (C^2 d + C d^2))) of the gated recurrence
// ("Attention is recurrent", Gated linear attention: a write at position s reaches
// position t scaled by the product of the gates after it).  For one head and a
// chunk of rows t, s in [0, C) with in-chunk inclusive cumulative log-gates
// B[t] = sum_{u<=t} g[u] and chunk total Gamma = B[C-1]:
//
//   Q~ = phi(Q) * exp(B),  K^ = phi(K) * exp(-B),  K~ = phi(K) * exp(Gamma - B)
//   P  = (Q~ K^^T) masked to s <= t                   (exp(B_t - B_s) = prod of gates)
//   O  = P V + Q~ S_in                                (intra-chunk + carried state)
//   S_out = Diag(exp(Gamma)) S_in + K~^T V            (the weighted scan step)
//
// Scalar gates use the exact mask form instead: P = (phi(Q) phi(K)^T) * exp(b_t - b_s)
// and O_inter = exp(b_t) phi(Q) S_in, so no factor ever exceeds 1.  For key-dim
// gates the factorised form needs exp(-B) to stay finite: the in-chunk cumulative
// log-gate must stay above about -80 (e.g. alpha >= 0.29 everywhere at C = 64).
//
// Work decomposition: one workgroup per (batch*head, value-column tile); NW
// wavefronts, each owning 16 value columns.  The workgroup walks the chunks of its
// head in order, keeping its d_k x 16*NW slice of the fp32 state in registers
// (accumulator layout).  Per chunk:
//   A  global loads: q, k, g rows (each thread a column pair and a row segment,
//      serial cumulative sum over its rows) and the v tile;
//   B  gated operands into LDS: Q~ and K^ row-major, K~ and V transposed;
//   C  the causal score tiles P (16x16 MFMA tiles with s-block <= t-block) shared
//      through LDS;
//   D  per wave: O^T = V^T P^T + S^T Q~^T for its 16 columns (stored straight to
//      global memory), then S <- Diag(exp Gamma) S + K~^T V.
// All products run on the matrix cores: bf16 operands with fp32 accumulation for
// bf16 inputs, fp32 operands for fp32 inputs.
#pragma once

#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

template <typename T, int DK, int C, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(const PrefillArgs a)
{
    using E = T;                                  // matrix-core operand type
    constexpr int NT = NW * 64;                   // threads
    constexpr int DVT = NW * 16;                  // value columns of this workgroup
    constexpr int NTB = C / 16;                   // 16-row blocks per chunk
    constexpr int NKB = DK / 16;                  // 16-blocks of the key dimension
    constexpr int PAD = 4;                        // LDS row padding (elements)
    constexpr int LDQ = DK + PAD;                 // Q~, K^ rows (length d_k)
    constexpr int LDT = C + PAD;                  // K~^T, V^T, P rows (length C)
    // gate stage: a thread owns a column pair and a segment of RPS rows
    constexpr int CP = DK / 2;
    constexpr int NSG = (NT / CP) < C ? (NT / CP) : C;
    constexpr int RPS = C / NSG;
    constexpr bool CACHE = RPS <= 16;             // keep a segment's loads in registers
    // value stage: same scheme over the workgroup's value columns
    constexpr int CPV = DVT / 2;
    constexpr int NSGV = (NT / CPV) < C ? (NT / CPV) : C;
    constexpr int RPSV = C / NSGV;
    static_assert(NT % CP == 0 && NT % CPV == 0, "thread mapping");

    __shared__ E sQ[C * LDQ];                     // Q~ [t][i]
    __shared__ E sKh[C * LDQ];                    // K^ [s][i]
    __shared__ E sKtT[DK * LDT];                  // K~^T [i][s]
    __shared__ E sVT[DVT * LDT];                  // V^T [j][s]
    __shared__ E sP[C * LDT];                     // P [t][s]
    __shared__ float sTot[NSG * DK];              // per-segment gate sums (log2 units)
    __shared__ float sEG[DK];                     // exp(Gamma_i)
    __shared__ float sB[C];                       // scalar gate: cumulative log2-gate per row

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;

    // workgroup -> (head, value tile); optionally keep a head's tiles on one XCD
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
    const float *__restrict__ gk = a.g ? a.g + (size_t)bh * L * DK : nullptr;  // key-dim
    const float *__restrict__ gs = a.g ? a.g + (size_t)bh * L : nullptr;       // scalar

    // state slice: tile kb holds S[16kb + 4grp + r][col0 + x], col0 = vt*DVT + 16w
    const int jw = 16 * w;
    const int scol = vt * DVT + jw + x;
    f32x4 S[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * kb + 4 * grp + r;
            S[kb][r] = a.s0 ? a.s0[((size_t)bh * DK + i) * DV + scol] : 0.f;
        }
    }

    const int cp = tid % CP, sg = tid / CP;       // gate-stage coordinates
    const int cpv = tid % CPV, sgv = tid / CPV;   // value-stage coordinates
    const int nchunks = (L + C - 1) / C;

    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * C;
        const int nvalid = (L - t0) < C ? (L - t0) : C;

        // ---- A: global loads and per-segment cumulative gate sums -------------
        // log2-domain gate of row t for this thread's column pair (0 past the end)
        auto load_gate = [&](int t) -> f32x2 {
            if (t >= nvalid || gate == kGateNone) return f32x2{0.f, 0.f};
            if (gate == kGateKeydim) return load2(gk + (size_t)(t0 + t) * DK + 2 * cp) * kLog2e;
            const float gv = gs[t0 + t] * kLog2e;
            return f32x2{gv, gv};
        };
        auto load_qk = [&](const T *base, int t) -> f32x2 {
            return t < nvalid ? load2(base + (size_t)(t0 + t) * DK + 2 * cp) : f32x2{0.f, 0.f};
        };
        f32x2 qv[CACHE ? RPS : 1], kv[CACHE ? RPS : 1], bc[CACHE ? RPS : 1];
        if (sg < NSG) {
            f32x2 run = {0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int t = sg * RPS + r;
                run += load_gate(t);
                if constexpr (CACHE) {
                    bc[r] = run;
                    qv[r] = load_qk(qh, t);
                    kv[r] = load_qk(kh, t);
                }
            }
            sTot[sg * DK + 2 * cp] = run[0];
            sTot[sg * DK + 2 * cp + 1] = run[1];
        }
        f32x2 vv[RPSV];
        if (sgv < NSGV) {
#pragma unroll
            for (int r = 0; r < RPSV; ++r) {
                const int t = sgv * RPSV + r;
                vv[r] = t < nvalid ? load2(vh + (size_t)(t0 + t) * DV + 2 * cpv) : f32x2{0.f, 0.f};
            }
        }
        __syncthreads();

        // ---- B: gated operands into LDS ------------------------------------------
        if (sg < NSG) {
            f32x2 pre = {0.f, 0.f}, tot = {0.f, 0.f};
            for (int s = 0; s < NSG; ++s) {
                const f32x2 ts = {sTot[s * DK + 2 * cp], sTot[s * DK + 2 * cp + 1]};
                if (s < sg) pre += ts;
                tot += ts;
            }
            f32x2 run = pre;
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const int t = sg * RPS + r;
                const bool valid = t < nvalid;
                f32x2 b, q2, k2;
                if constexpr (CACHE) {
                    b = pre + bc[r];
                    q2 = qv[r];
                    k2 = kv[r];
                } else {            // segment too long to keep in registers: reload
                    run += load_gate(t);
                    b = run;
                    q2 = load_qk(qh, t);
                    k2 = load_qk(kh, t);
                }
                f32x2 qt, khat, ktil;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float fq = valid ? feature(q2[e], elu1) : 0.f;
                    const float fk = valid ? feature(k2[e], elu1) : 0.f;
                    if (gate == kGateKeydim) {
                        qt[e] = fq * exp2_fast(b[e]);
                        khat[e] = fk * exp2_fast(-b[e]);
                        ktil[e] = fk * exp2_fast(tot[e] - b[e]);
                    } else if (gate == kGateScalar) {
                        qt[e] = fq;
                        khat[e] = fk;
                        ktil[e] = fk * exp2_fast(tot[e] - b[e]);
                    } else {
                        qt[e] = fq;
                        khat[e] = fk;
                        ktil[e] = fk;
                    }
                }
                E *q_dst = sQ + t * LDQ + 2 * cp;
                E *kh_dst = sKh + t * LDQ + 2 * cp;
                q_dst[0] = from_f32<E>(qt[0]);
                q_dst[1] = from_f32<E>(qt[1]);
                kh_dst[0] = from_f32<E>(khat[0]);
                kh_dst[1] = from_f32<E>(khat[1]);
                sKtT[(2 * cp) * LDT + t] = from_f32<E>(ktil[0]);
                sKtT[(2 * cp + 1) * LDT + t] = from_f32<E>(ktil[1]);
                if (gate == kGateScalar && cp == 0) sB[t] = b[0];
            }
            if (sg == NSG - 1) {
                sEG[2 * cp] = gate == kGateNone ? 1.f : exp2_fast(tot[0]);
                sEG[2 * cp + 1] = gate == kGateNone ? 1.f : exp2_fast(tot[1]);
            }
        }
        if (sgv < NSGV) {
#pragma unroll
            for (int r = 0; r < RPSV; ++r) {
                const int t = sgv * RPSV + r;
                sVT[(2 * cpv) * LDT + t] = from_f32<E>(vv[r][0]);
                sVT[(2 * cpv + 1) * LDT + t] = from_f32<E>(vv[r][1]);
            }
        }
        __syncthreads();

        // ---- C: causal score tiles P[t][s] (s-block <= t-block), shared in LDS ----
        {
            constexpr int NTILES = NTB * (NTB + 1) / 2;
            for (int tile = w; tile < NTILES; tile += NW) {
                int tb = 0, sb = tile;
                while (sb > tb) { sb -= tb + 1; ++tb; }
                // P^T tile = K^[s-block] Q~[t-block]^T: lane holds P[16tb+x][16sb+4grp+r]
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = contract_rows<E>(sKh + (16 * sb + x) * LDQ, sQ + (16 * tb + x) * LDQ, NKB,
                                       grp, acc);
                const int t = 16 * tb + x;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * sb + 4 * grp + r;
                    float pv = s <= t ? acc[r] : 0.f;
                    if (gate == kGateScalar && s <= t) pv *= exp2_fast(sB[t] - sB[s]);
                    acc[r] = pv;
                }
                E *dst = sP + t * LDT + 16 * sb + 4 * grp;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r] = from_f32<E>(acc[r]);
            }
        }
        __syncthreads();

        // ---- D: outputs of this wave's 16 columns, then the state step -----------
        {
            const E *vrow = sVT + (jw + x) * LDT;             // V^T row j = jw + x
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                const int t = 16 * tb + x;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                // inter-chunk: O^T += S^T Q~^T (contraction over the key dim)
                acc = contract_regs_rows<E, NKB>(S, sQ + t * LDQ, grp, acc);
                if (gate == kGateScalar) acc *= exp2_fast(sB[t]);
                // intra-chunk: O^T += V^T P^T over s-blocks 0..tb
                acc = contract_rows<E>(vrow, sP + t * LDT, tb + 1, grp, acc);
                if (t < nvalid) store4(oh + (size_t)(t0 + t) * DV + jw + 4 * grp, acc);
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[kb][r] *= sEG[16 * kb + 4 * grp + r];
                S[kb] = contract_rows<E>(sKtT + (16 * kb + x) * LDT, vrow, NTB, grp, S[kb]);
            }
        }
    }

    if (a.s_final) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * kb + 4 * grp + r;
                a.s_final[((size_t)bh * DK + i) * DV + scol] = S[kb][r];
            }
        }
    }
}

template <typename T, int DK, int C, int NW>
hipError_t launch_prefill_inst(const PrefillArgs &a, hipStream_t stream)
{
    const int grid = a.BH * a.n_vt;
    hipLaunchKernelGGL((prefill_kernel<T, DK, C, NW>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gla
