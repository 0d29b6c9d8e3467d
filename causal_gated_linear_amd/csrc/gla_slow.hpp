// gla_slow.hpp -- the token-by-token form of one chunk, for the chunks whose gates
// leave the range of the factorised chunk form.
//
// The chunkwise kernels scale keys by exp(-B) and queries by exp(B), with B a
// cumulative log-gate inside the chunk ("Gated Linear Attention", Summary: the
// chunk form; "Attention is recurrent", Gated linear attention: a write reaches a
// later token scaled by the product of the gates in between).  The products of the
// two factors are the exact gate products, but each factor alone must stay inside
// the fp32/bf16 exponent range.  A chunk whose cumulative log2-gate falls below
// -kFastLim in some dimension is therefore computed here instead, straight from the
// recurrence of the same pages:
//
//     S_t[i][j] = alpha_t[i] beta_t[j] S_{t-1}[i][j] + phi(k_t)[i] v_t[j]
//     o_t[j]    = sum_i phi(q_t)[i] S_t[i][j]            (beta = 1 without value gates)
//
// one token at a time, in fp32, which holds for any gate in [0, 1] (alpha = 0
// included).  The normalised form also carries z_t = alpha_t (*) z_{t-1} + phi(k_t)
// and divides o_t by phi(q_t) . z_t ("Transformers are RNNs" notes).
//
// The staging threads (the caller's consumer waves) copy SR rows at a time into LDS
// (alpha = exp(g) and beta = exp(gv) in fp32, phi(q), phi(k) and v in the input type)
// from global memory; then the token loop runs on lanes that each own one value column j and
// NG groups of four key rows, so the sum over i is a reduction over the lanes that
// share j (lanes JPW apart).  Each staged group ends with a workgroup barrier;
// callers call the staging and the token loop in the same order on every wave.
#pragma once

#include "gla_device.hpp"

namespace gla {

template <typename T> struct Piece16;              // one 16-byte piece of T elements
template <> struct Piece16<bf16> { typedef bf16x8 type; };
template <> struct Piece16<float> { typedef f32x4 type; };

// Chunks are computed token by token once a cumulative log2-gate (the exponent of
// the factorised form's key factor, and of the query factor's inverse) falls below
// -kFastLim: keys then stay below 2^100 times their size, queries above 2^-100
// times theirs, and the chunk's key-value sums far from fp32 overflow.
constexpr float kFastLim = 100.f;

// Lane mapping of the token loop for a tile of DVT value columns and DK key rows
// on NW waves: JPW columns per wave (a power of two) and 64 / JPW row slabs per
// column, each of 4 to 16 rows (so a lane holds at most 16 state values); the tile's
// columns are covered in passes of (waves used) * JPW columns.
constexpr int slow_jpw(int dvt, int nw, int dk)
{
    int j = 256 / dk;                              // at least 4 rows per lane
    while (j * 2 * dk <= 1024 && j * 2 * nw <= dvt) j *= 2;
    return j;
}
constexpr int slow_waves(int dvt, int nw, int dk)
{
    return dvt / slow_jpw(dvt, nw, dk) < nw ? dvt / slow_jpw(dvt, nw, dk) : nw;
}

template <typename T> struct SlowStage {
    float *a;      // [SR][DK]  alpha = exp(g)
    float *b;      // [SR][dvt] beta = exp(gv) (value gates only)
    T *q, *k;      // [SR][DK]  phi(q), phi(k)
    T *v;          // [SR][dvt]
};

// Stage rows [row, row + SR) of the views (rows past the end read as zeros) with
// all NT threads.  Key-side rows are DK long (SG: one gate per row, the same for
// every key dimension); value-side rows are the dvt columns of this tile, starting at
// column vcol of rows DV long.
template <typename T, int DK, int SR, int NT, bool ELU1, bool OUT, bool VG, bool SG = false>
__device__ __forceinline__ void slow_stage(const SlowStage<T> &st, Rsrc rq, Rsrc rk, Rsrc rv, Rsrc rg,
                                           Rsrc rgv, int row, int DV, int vcol, int dvt, int tid)
{
    constexpr int ES = sizeof(T), CE = 16 / ES;
    typedef typename Piece16<T>::type VC;
#pragma unroll 1
    for (int p = tid; p < SR * DK / 4; p += NT) {
        const int r = p / (DK / 4), c = (p % (DK / 4)) * 4;
        f32x4 g;
        if constexpr (SG) {
            const float gs = buf_load4(rg, (row + r) * 4);
            g = f32x4{gs, gs, gs, gs};
        } else {
            g = buf_load16<f32x4>(rg, ((row + r) * DK + c) * 4);
        }
        f32x4 al;
#pragma unroll
        for (int e = 0; e < 4; ++e) al[e] = exp2_fast(g[e] * kLog2e);
        *(f32x4 *)(st.a + r * DK + c) = al;
    }
#pragma unroll 1
    for (int p = tid; p < SR * DK / CE; p += NT) {
        const int r = p / (DK / CE), c = (p % (DK / CE)) * CE;
        const int off = ((row + r) * DK + c) * ES;
        VC kv = buf_load16<VC>(rk, off);
        if constexpr (ELU1) {
#pragma unroll
            for (int e = 0; e < CE; ++e) kv[e] = from_f32<T>(feature(to_f32(kv[e]), true));
        }
        *(VC *)(st.k + r * DK + c) = kv;
        if constexpr (OUT) {
            VC qv = buf_load16<VC>(rq, off);
            if constexpr (ELU1) {
#pragma unroll
                for (int e = 0; e < CE; ++e) qv[e] = from_f32<T>(feature(to_f32(qv[e]), true));
            }
            *(VC *)(st.q + r * DK + c) = qv;
        }
    }
    const int vpr = dvt / CE;                      // 16-byte pieces per value row
#pragma unroll 1
    for (int p = tid; p < SR * vpr; p += NT) {
        const int r = p / vpr, c = (p % vpr) * CE;
        *(VC *)(st.v + r * dvt + c) = buf_load16<VC>(rv, ((row + r) * DV + vcol + c) * ES);
    }
    if constexpr (VG) {
        const int gpr = dvt / 4;
#pragma unroll 1
        for (int p = tid; p < SR * gpr; p += NT) {
            const int r = p / gpr, c = (p % gpr) * 4;
            const f32x4 g = buf_load16<f32x4>(rgv, ((row + r) * DV + vcol + c) * 4);
            f32x4 be;
#pragma unroll
            for (int e = 0; e < 4; ++e) be[e] = exp2_fast(g[e] * kLog2e);
            *(f32x4 *)(st.b + r * dvt + c) = be;
        }
    }
}

// Token loop over `nrows` staged rows.  The lane owns value column j (of the
// tile) and the key rows r0 + GS * g + e (g < NG, e < 4); S[g][e] is S[r0 + GS g + e][j]
// and Z[g][e] the normaliser z[r0 + GS g + e] (normalised form).  Lanes JPW apart
// share j; the lanes with lane < JPW store o[t][j] to orow + t * DV when `OUT`.
template <typename T, int DK, int NG, int GS, int JPW, bool OUT, bool NM, bool VG>
__device__ __forceinline__ void slow_tokens(const SlowStage<T> &st, f32x4 (&S)[NG], f32x4 (&Z)[NG], int r0, int j,
                                            int dvt, int nrows, T *orow, int DV, bool writer)
{
    typedef typename Frag<T>::type F4;
    for (int t = 0; t < nrows; ++t) {
        const float vj = to_f32(st.v[t * dvt + j]);
        float bj = 1.f;
        if constexpr (VG) bj = st.b[t * dvt + j];
        // row pointers of this token; the groups sit at fixed offsets from them
        const float *pa = st.a + t * DK + r0;
        const T *pk = st.k + t * DK + r0, *pq = st.q + t * DK + r0;
        float op[2] = {0.f, 0.f}, dp[2] = {0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            // one group of rows at a time keeps the loop's registers few
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 al = *(const f32x4 *)(pa + GS * g);
            const f32x4 kk = widen4(*(const F4 *)(pk + GS * g));
            f32x4 qq = {0.f, 0.f, 0.f, 0.f};
            if constexpr (OUT) qq = widen4(*(const F4 *)(pq + GS * g));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float d = VG ? al[e] * bj : al[e];
                S[g][e] = fmaf(d, S[g][e], kk[e] * vj);
                if constexpr (NM) Z[g][e] = fmaf(al[e], Z[g][e], kk[e]);
                if constexpr (OUT) {
                    op[e & 1] = fmaf(qq[e], S[g][e], op[e & 1]);
                    if constexpr (NM) dp[e & 1] = fmaf(qq[e], Z[g][e], dp[e & 1]);
                }
            }
        }
        if constexpr (OUT) {
            float o = op[0] + op[1], den = dp[0] + dp[1];
#pragma unroll
            for (int off = JPW; off < 64; off <<= 1) {
                o += __shfl_xor(o, off, 64);
                if constexpr (NM) den += __shfl_xor(den, off, 64);
            }
            if (writer) orow[(size_t)t * DV] = from_f32<T>(NM ? o / den : o);
        }
    }
}

// One chunk token by token, with the state handed over in LDS: PS holds S^T as
// fp32 [DVT][DK] (PS[j * DK + i] = S[i][j]) and PZ the normaliser z [DK] (normalised
// form); both are read and rewritten here.  The chunk covers rows [t0, t0 + nvalid)
// of the views; output row t of the tile goes to out + t * DV (its first column).
// NTS threads stage the rows (`sw`: this thread's index among them, -1 for none);
// the token loop runs on the first slow_waves(DVT, NTS / 64, DK) of those waves, in
// passes over the tile's columns.  Every staging thread passes 2 * ceil(nvalid / SR)
// workgroup barriers here; the caller passes one more before it reads PS or PZ.
template <typename T, int DK, int DVT, int SR, int NTS, bool ELU1, bool OUT, bool NM, bool VG, bool SG = false>
__device__ __forceinline__ void slow_chunk_lds(float *PS, float *PZ, const SlowStage<T> &st, Rsrc rq, Rsrc rk,
                                               Rsrc rv, Rsrc rg, Rsrc rgv, int t0, int nvalid, int DV, int vcol,
                                               T *out, int sw)
{
    constexpr int JPW = slow_jpw(DVT, NTS / 64, DK), NTL = slow_waves(DVT, NTS / 64, DK);
    constexpr int RPL = DK * JPW / 64, NG = RPL / 4, NPASS = DVT / (NTL * JPW);
    static_assert(RPL % 4 == 0 && NG <= 4 && NPASS * NTL * JPW == DVT, "token-loop lane mapping");
    const int tw = sw >> 6, lane = sw & 63;
    const bool tl = tw < NTL;                      // wave-uniform
    const int jl = lane % JPW, isub = lane / JPW;
    for (int r0 = 0; r0 < nvalid; r0 += SR) {
        slow_stage<T, DK, SR, NTS, ELU1, OUT, VG, SG>(st, rq, rk, rv, rg, rgv, t0 + r0, DV, vcol, DVT, sw);
        lds_barrier();
        f32x4 Z[NG];                               // normaliser rows: the same in every pass
        const int rb = isub * RPL;                 // first key row of this lane
        if (tl) {
#pragma unroll 1
            for (int ps = 0; ps < NPASS; ++ps) {
                const int j = (ps * NTL + tw) * JPW + jl;
                f32x4 S[NG];
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    S[g] = *(const f32x4 *)(PS + j * DK + rb + 4 * g);
                    Z[g] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (NM) Z[g] = *(const f32x4 *)(PZ + rb + 4 * g);
                }
                slow_tokens<T, DK, NG, 4, JPW, OUT, NM, VG>(st, S, Z, rb, j, DVT, min(SR, nvalid - r0),
                                                            OUT ? out + (size_t)r0 * DV + j : nullptr, DV, lane < JPW);
#pragma unroll
                for (int g = 0; g < NG; ++g) *(f32x4 *)(PS + j * DK + rb + 4 * g) = S[g];
            }
        }
        lds_barrier();
        if constexpr (NM) {
            // every pass of every token-loop lane read z at the group's start; one lane per
            // row slab writes the group's end value back, read after the next barrier
            if (tl && tw == 0 && jl == 0) {
#pragma unroll
                for (int g = 0; g < NG; ++g) *(f32x4 *)(PZ + rb + 4 * g) = Z[g];
            }
        }
    }
}

}  // namespace gla
