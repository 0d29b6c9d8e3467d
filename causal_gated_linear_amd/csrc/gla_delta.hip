// gla_delta.hip -- the delta rule ("Attention is recurrent", Delta attention and the
// Prefill section after it) on gfx950.
//
// Per head, token t:  u_t = beta_t (v_t - S_{t-1}^T k_t),  S_t = S_{t-1} + k_t u_t^T,
// o_t = S_t^T q_t.  The writes u depend on the state, so a chunk of C tokens that
// starts from state S solves one unit lower-triangular system for its writes (the
// page's whole-prompt argument, applied to a chunk with a nonzero starting state):
//
//     T U = diag(beta) (V - K S),      T = I + tril(diag(beta) K K^T, -1)
//
// With X = T^{-1}, W = X diag(beta) K and U~ = X diag(beta) V:
//
//     U = U~ - W S,   O = Q S + tril(Q K^T) U  (diagonal included: o_t reads S_t),
//     S <- S + K^T U.
//
// X, W and U~ depend only on the chunk's own keys, values and strengths.  Chunks of
// 64 tokens use two kernels with a workspace between them:
//   delta_prep_kernel  one workgroup per (head, chunk), all chunks in parallel:
//       N = tril(diag(beta) K K^T, -1) on the matrix cores; the inverses of the 16x16
//       diagonal blocks of I + N by substitution in fp32 (one lane per column); the
//       blocks below the diagonal one block row at a time,
//       X_ij = -X_ii sum_{k=j}^{i-1} N_ik X_kj, with fp32 matrix-core products; then
//       -W and U~ on the matrix cores, stored to the workspace in the layouts the scan
//       reads directly (-W row-major per token, U~ transposed per chunk).
//   delta_scan_kernel  one workgroup per (head, 64 value columns) walks the chunks in
//       order.  Each wave owns 16 value columns and their state slice S[d_k][16] in
//       accumulator registers.  Per chunk: U = U~ + (-W) S for every 16-row block (the
//       accumulator tiles of U are at once the operand fragments of the next two
//       products), the score tiles P^T = K Q^T masked to s <= t, O^T = S^T Q^T + U^T P^T
//       stored per block, then S += K^T U.  The chunk's Q, K, -W and U~ rows are staged
//       in LDS; the next chunk's rows are requested before the current one is
//       computed, into a second LDS buffer where two fit.
// Chunks of 16 or 32 tokens use one kernel, delta_fused_kernel, which interleaves
// the two: between the barriers that separate the steps of chunk n's state pass it
// solves chunk n+1's system into the other LDS buffer (see its own comment).
// bf16 inputs: bf16 matrix-core operands, fp32 accumulation and fp32 X; fp32 inputs:
// fp32 matrix-core products throughout.
#include <type_traits>

#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// row padding (elements): 32 bytes for bf16 rows, 16 bytes for fp32 rows
template <typename T> constexpr int row_pad() { return sizeof(T) == 2 ? 16 : 4; }

__device__ __forceinline__ void store4_if(bf16 *p, f32x4 v, bool ok) { if (ok) store4(p, v); }
__device__ __forceinline__ void store4_if(float *p, f32x4 v, bool ok) { if (ok) store4(p, v); }

}  // namespace

// ------------------------------------------------------------------------------------
// delta_prep_kernel: X, -W and U~ of one chunk of one head
// ------------------------------------------------------------------------------------
template <typename T, int C>
__global__ __launch_bounds__(256) void delta_prep_kernel(const DeltaArgs a)
{
    constexpr int NB = C / 16, CE = 16 / sizeof(T), PAD = row_pad<T>();
    // K rows (8-byte row reads and transposing reads; with bf16 a pad of 12 gives an
    // odd multiple of 8 bytes, conflict-free for the row reads on gfx950) and V rows
    // (transposing reads only, conflict-free with a pad of 16); d_k, d_v <= 128
    constexpr int LDMK = 128 + (sizeof(T) == 2 ? 12 : PAD), LDMV = 128 + PAD;
    constexpr int LDC = C + 4;                     // N and X row stride (fp32)
    typedef typename Frag<T>::type F4;
    __shared__ __align__(16) T sK[C * LDMK];
    __shared__ __align__(16) T sV[C * LDMV];
    __shared__ __align__(16) float sN[C * LDC];
    __shared__ __align__(16) float sX[C * LDC];
    __shared__ __align__(16) float sB[C];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;
    const int dk = a.d_k, dv = a.d_v, L = a.L;
    const int nch = (L + C - 1) / C;
    const int bh = blockIdx.x / nch, n = blockIdx.x - bh * nch;
    const int nvalid = min(C, L - n * C);
    const size_t hrow = (size_t)bh * L + (size_t)n * C;   // first row of this chunk

    // K and V rows (zero past the end of the sequence) and the strengths
    {
        const int kc = dk / CE, vc = dv / CE;
        const T *kg = (const T *)a.k + hrow * dk, *vg = (const T *)a.v + hrow * dv;
        for (int e = tid; e < C * kc; e += 256) {
            const int r = e / kc, c = (e - r * kc) * CE;
            i32x4 val = {0, 0, 0, 0};
            if (r < nvalid) val = *(const i32x4 *)(kg + (size_t)r * dk + c);
            typedef int i32x2 __attribute__((ext_vector_type(2)));
            *(i32x2 *)(sK + r * LDMK + c) = i32x2{val[0], val[1]};          // 8-byte aligned rows
            *(i32x2 *)(sK + r * LDMK + c + CE / 2) = i32x2{val[2], val[3]};
        }
        for (int e = tid; e < C * vc; e += 256) {
            const int r = e / vc, c = (e - r * vc) * CE;
            i32x4 val = {0, 0, 0, 0};
            if (r < nvalid) val = *(const i32x4 *)(vg + (size_t)r * dv + c);
            *(i32x4 *)(sV + r * LDMV + c) = val;
        }
        if (tid < C) sB[tid] = tid < nvalid ? a.beta[hrow + tid] : 0.f;
    }
    __syncthreads();

    // N = tril(diag(beta) K K^T, -1) on the 16x16 tiles on and below the diagonal
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int id = w; id < NB * (NB + 1) / 2; id += 4) {
        int tb = 0;
        while ((tb + 1) * (tb + 2) / 2 <= id) ++tb;
        const int sb = id - tb * (tb + 1) / 2;
        // lane (x, grp) element e: (K K^T)[16 tb + 4 grp + e][16 sb + x]
        const f32x4 g = contract_rows(sK + (16 * tb + x) * LDMK, sK + (16 * sb + x) * LDMK, dk / 16, grp, zero);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * tb + 4 * grp + e, s = 16 * sb + x;
            sN[t * LDC + s] = s < t ? sB[t] * g[e] : 0.f;
        }
    }
    __syncthreads();

    // inverses of the diagonal blocks I + N_bb: lane 16 b + j solves for column j of
    // block b by substitution, x_r = [r == j] - sum_{m<r} N_rm x_m
    if (w == 0) {
        const int b = lane >> 4, j = lane & 15;
        if (b < NB) {
            const float *nb = sN + 16 * b * LDC + 16 * b;
            // column-wise (right-looking): once x_m is final, its multiples are
            // subtracted from every later row, so the dependent chain is 16 steps long
            float xs[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) xs[r] = r == j ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m)
#pragma unroll
                for (int r = m + 1; r < 16; ++r) xs[r] -= nb[r * LDC + m] * xs[m];
#pragma unroll
            for (int r = 0; r < 16; ++r) sX[(16 * b + r) * LDC + 16 * b + j] = xs[r];
        }
    }
    __syncthreads();

    // blocks below the diagonal, one block row i at a time; wave j computes
    // X_ij = -X_ii R with R = sum_{k=j}^{i-1} N_ik X_kj (fp32 products)
    for (int i = 1; i < NB; ++i) {
        if (w < i) {
            const int j = w;
            f32x4 r = zero;
            for (int k = j; k < i; ++k)
                r = mma1(lds_frag(sN + (16 * i + x) * LDC + 16 * k, 0, grp),
                         col_frag(sX, LDC, 16 * k + 4 * grp, 16 * j, x), r);
            const f32x4 xr = mma1(lds_frag(sX + (16 * i + x) * LDC + 16 * i, 0, grp), r, zero);
#pragma unroll
            for (int e = 0; e < 4; ++e) sX[(16 * i + 4 * grp + e) * LDC + 16 * j + x] = -xr[e];
        }
        __syncthreads();
    }

    // (X diag(beta)) fragment of row t = 16 tb + x over the 16-block sb of s
    auto xb = [&](int tb, int sb) -> F4 {
        const f32x4 xv = lds_frag(sX + (16 * tb + x) * LDC, sb, grp);
        const f32x4 bv = *(const f32x4 *)(sB + 16 * sb + 4 * grp);
        return cvt4<T>(xv * bv);
    };
    // -W^T tiles (i-block ib, t-block tb) and U~ tiles (t-block tb, j-block jb); X is
    // lower triangular, so the contraction over s stops at block tb
    const int nkb = dk / 16, nvb = dv / 16;
    const size_t lp = (size_t)nch * C;
    T *wg = (T *)a.ws_w + ((size_t)bh * lp + (size_t)n * C) * dk;
    T *ug = (T *)a.ws_u + ((size_t)bh * nch + n) * dv * C;
    for (int id = w; id < (nkb + nvb) * NB; id += 4) {
        const int tb = id % NB, cb = id / NB;
        f32x4 acc = zero;
        if (cb < nkb) {
            // lane (x, grp) element e: W^T[16 cb + 4 grp + e][16 tb + x] = W[t][i..i+3]
            int sb = 0;
            for (; sb + 1 <= tb; sb += 2)
                acc = mac2(col_frag(sK, LDMK, 16 * sb + 4 * grp, 16 * cb, x),
                           col_frag(sK, LDMK, 16 * (sb + 1) + 4 * grp, 16 * cb, x), xb(tb, sb), xb(tb, sb + 1), acc);
            if (sb <= tb) acc = mac1(col_frag(sK, LDMK, 16 * sb + 4 * grp, 16 * cb, x), xb(tb, sb), acc);
            store4(wg + (size_t)(16 * tb + x) * dk + 16 * cb + 4 * grp, -acc);
        } else {
            const int jb = cb - nkb;
            // lane (x, grp) element e: U~[16 tb + 4 grp + e][16 jb + x] = U~^T[j][t..t+3]
            int sb = 0;
            for (; sb + 1 <= tb; sb += 2)
                acc = mac2(xb(tb, sb), xb(tb, sb + 1), col_frag(sV, LDMV, 16 * sb + 4 * grp, 16 * jb, x),
                           col_frag(sV, LDMV, 16 * (sb + 1) + 4 * grp, 16 * jb, x), acc);
            if (sb <= tb) acc = mac1(xb(tb, sb), col_frag(sV, LDMV, 16 * sb + 4 * grp, 16 * jb, x), acc);
            store4(ug + (size_t)(16 * jb + x) * C + 16 * tb + 4 * grp, acc);
        }
    }
}

// ------------------------------------------------------------------------------------
// delta_scan_kernel: the chunks of one head in order, state in registers
// ------------------------------------------------------------------------------------
template <typename T, int DK, int C>
struct DeltaScanShape {
    static constexpr int ES = sizeof(T), CE = 16 / ES, PAD = row_pad<T>();
    static constexpr int NB = C / 16, NKB = DK / 16;
    // Q, K, -W rows: with bf16 a pad of 12 gives an odd multiple of 8 bytes, so the
    // 8-byte row reads are conflict-free on gfx950; every access to them is 8 bytes
    static constexpr int LDK = DK + (ES == 2 ? 12 : PAD);
    static constexpr int LDU = C + PAD;            // U~^T row stride
    static constexpr int DVT_MAX = 64;
    static constexpr int BUF = 3 * C * LDK + DVT_MAX * LDU;   // elements per buffer
    static constexpr int NBUF = 2 * BUF * ES <= kLdsBytes ? 2 : 1;
    static constexpr int QP = C * DK / CE;         // 16-byte pieces of one C x DK array
    static constexpr int QPT = (QP + 255) / 256;
    static constexpr int UPT = (DVT_MAX * C / CE + 255) / 256;
};

template <typename T, int DK, int C>
__global__ __launch_bounds__(256) void delta_scan_kernel(const DeltaArgs a)
{
    typedef DeltaScanShape<T, DK, C> SH;
    constexpr int ES = SH::ES, CE = SH::CE, NB = SH::NB, NKB = SH::NKB;
    constexpr int LDK = SH::LDK, LDU = SH::LDU, QP = SH::QP;
    __shared__ __align__(16) T smem[SH::NBUF * SH::BUF];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;
    int wgi = blockIdx.x;
    if (a.xcd_remap) wgi = (wgi & 7) * (gridDim.x >> 3) + (wgi >> 3);
    const int bh = wgi / a.n_vt, vt = wgi - bh * a.n_vt;
    const int L = a.L, DV = a.d_v, DVT = a.dvt;
    const int nch = (L + C - 1) / C;
    const size_t hrow = (size_t)bh * L, lp = (size_t)nch * C;
    const int j0 = vt * DVT + 16 * w;              // this wave's first value column
    const bool active = 16 * w < DVT;              // wave-uniform
    const int UP = DVT * C / CE;                   // pieces of this tile's U~^T block

    // head views (host code guarantees each head's bytes fit in 31 bits); rows past
    // the end of the sequence read as zeros
    const Rsrc rq = make_rsrc((const T *)a.q + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rk = make_rsrc((const T *)a.k + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rw = make_rsrc((const T *)a.ws_w + bh * lp * DK, (unsigned)(lp * DK * ES));
    const Rsrc ru = make_rsrc((const T *)a.ws_u + bh * lp * DV, (unsigned)(lp * DV * ES));

    i32x4 gq[SH::QPT], gk[SH::QPT], gw[SH::QPT], gu[SH::UPT];
    auto fetch = [&](int n) {
        const int base = n * C * DK * ES;
#pragma unroll
        for (int i = 0; i < SH::QPT; ++i) {
            const int p = tid + 256 * i;
            if (QP % 256 == 0 || p < QP) {
                gq[i] = buf_load16<i32x4>(rq, base + 16 * p);
                gk[i] = buf_load16<i32x4>(rk, base + 16 * p);
                gw[i] = buf_load16<i32x4>(rw, base + 16 * p);
            }
        }
        const int ubase = (n * DV + vt * DVT) * C * ES;
#pragma unroll
        for (int i = 0; i < SH::UPT; ++i) {
            const int p = tid + 256 * i;
            if (p < UP) gu[i] = buf_load16<i32x4>(ru, ubase + 16 * p);
        }
    };
    auto stash = [&](T *buf) {
        T *sQ = buf, *sK = buf + C * LDK, *sW = buf + 2 * C * LDK, *sU = buf + 3 * C * LDK;
#pragma unroll
        for (int i = 0; i < SH::QPT; ++i) {
            const int p = tid + 256 * i;
            if (QP % 256 == 0 || p < QP) {
                const int r = p / (DK / CE), c = (p - r * (DK / CE)) * CE;
                typedef int i32x2 __attribute__((ext_vector_type(2)));
                *(i32x2 *)(sQ + r * LDK + c) = i32x2{gq[i][0], gq[i][1]};    // 8-byte aligned rows
                *(i32x2 *)(sQ + r * LDK + c + CE / 2) = i32x2{gq[i][2], gq[i][3]};
                *(i32x2 *)(sK + r * LDK + c) = i32x2{gk[i][0], gk[i][1]};
                *(i32x2 *)(sK + r * LDK + c + CE / 2) = i32x2{gk[i][2], gk[i][3]};
                *(i32x2 *)(sW + r * LDK + c) = i32x2{gw[i][0], gw[i][1]};
                *(i32x2 *)(sW + r * LDK + c + CE / 2) = i32x2{gw[i][2], gw[i][3]};
            }
        }
#pragma unroll
        for (int i = 0; i < SH::UPT; ++i) {
            const int p = tid + 256 * i;
            if (p < UP) {
                const int r = p / (C / CE), c = (p - r * (C / CE)) * CE;
                *(i32x4 *)(sU + r * LDU + c) = gu[i];
            }
        }
    };

    // state slice: tile ib, lane (x, grp) element e holds S[16 ib + 4 grp + e][j0 + x]
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 s[NKB];
#pragma unroll
    for (int ib = 0; ib < NKB; ++ib) {
        s[ib] = zero;
        if (active && a.s0) {
            const float *p = a.s0 + ((size_t)bh * DK + 16 * ib + 4 * grp) * DV + j0 + x;
            s[ib] = f32x4{p[0], p[DV], p[2 * DV], p[3 * DV]};
        }
    }

    if (nch > 0) fetch(0);
    for (int n = 0; n < nch; ++n) {
        T *buf = smem + (SH::NBUF == 2 ? (n & 1) * SH::BUF : 0);
        if (SH::NBUF == 1 && n > 0) lds_barrier();    // the buffer's last readers are done
        stash(buf);
        lds_barrier();
        if (n + 1 < nch) fetch(n + 1);
        if (!active) continue;

        const T *sQ = buf, *sK = buf + C * LDK, *sW = buf + 2 * C * LDK;
        const T *sU = buf + 3 * C * LDK + 16 * w * LDU;
        const int nvalid = min(C, L - n * C);

        // U = U~ + (-W) S; tile tb, lane (x, grp) element e: U[16 tb + 4 grp + e][j0 + x]
        f32x4 u[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            f32x4 acc = widen4(lds_frag(sU + x * LDU, tb, grp));
            const T *wrow = sW + (16 * tb + x) * LDK;
#pragma unroll
            for (int ib = 0; ib + 1 < NKB; ib += 2)
                acc = mac2(lds_frag(wrow, ib, grp), lds_frag(wrow, ib + 1, grp), cvt4<T>(s[ib]),
                           cvt4<T>(s[ib + 1]), acc);
            if (NKB % 2) acc = mac1(lds_frag(wrow, NKB - 1, grp), cvt4<T>(s[NKB - 1]), acc);
            u[tb] = acc;
        }

        // O^T = S^T Q^T + U^T P^T; lane (x, grp) element e: O[16 tb + x][j0 + 4 grp + e]
        T *og = (T *)a.o + (hrow + (size_t)n * C) * DV + j0 + 4 * grp;
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const T *qrow = sQ + (16 * tb + x) * LDK;
            f32x4 o = contract_regs_rows<T, NKB>(s, qrow, grp, zero);
            // P^T[s][t] = k_s . q_t for s <= t; lane (x, grp) element e: s = 16 sb + 4 grp + e
            auto score = [&](int sb) {
                f32x4 p = contract_rows(sK + (16 * sb + x) * LDK, qrow, NKB, grp, zero);
                if (sb == tb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * grp + e > x) p[e] = 0.f;
                }
                return p;
            };
#pragma unroll
            for (int sb = 0; sb <= tb; sb += 2) {
                if (sb + 1 <= tb)
                    o = mac2(cvt4<T>(u[sb]), cvt4<T>(u[sb + 1]), cvt4<T>(score(sb)), cvt4<T>(score(sb + 1)), o);
                else
                    o = mac1(cvt4<T>(u[sb]), cvt4<T>(score(sb)), o);
            }
            store4_if(og + (size_t)(16 * tb + x) * DV, o, 16 * tb + x < nvalid);
        }

        // S += K^T U
#pragma unroll
        for (int ib = 0; ib < NKB; ++ib) {
#pragma unroll
            for (int sb = 0; sb + 1 < NB; sb += 2)
                s[ib] = mac2(col_frag(sK, LDK, 16 * sb + 4 * grp, 16 * ib, x),
                             col_frag(sK, LDK, 16 * (sb + 1) + 4 * grp, 16 * ib, x), cvt4<T>(u[sb]),
                             cvt4<T>(u[sb + 1]), s[ib]);
            if (NB % 2)
                s[ib] = mac1(col_frag(sK, LDK, 16 * (NB - 1) + 4 * grp, 16 * ib, x), cvt4<T>(u[NB - 1]), s[ib]);
        }
    }

    if (active && a.s_final) {
#pragma unroll
        for (int ib = 0; ib < NKB; ++ib) {
            float *p = a.s_final + ((size_t)bh * DK + 16 * ib + 4 * grp) * DV + j0 + x;
#pragma unroll
            for (int e = 0; e < 4; ++e) p[(size_t)e * DV] = s[ib][e];
        }
    }
}

// ------------------------------------------------------------------------------------
// delta_fused_kernel: both halves in one workgroup (chunks of 16 or 32 tokens)
// ------------------------------------------------------------------------------------
// One workgroup per (head, 64 value columns) walks the chunks in order.  While four
// waves carry the state through chunk n (U = U~ + (-W) S, the outputs, S += K^T U,
// as delta_scan_kernel), four other waves solve chunk n+1's triangular system (N,
// the diagonal-block inverses, the block below the diagonal, then -W and U~ into
// LDS, as delta_prep_kernel), one step of each between consecutive barriers, so the
// two run side by side and nothing goes through global memory.  N (strictly lower) and X^T
// (upper triangle with the diagonal) share one fp32 array: the inverse of a unit
// lower-triangular block is lower triangular, so its transpose fills exactly the
// positions N leaves free.
template <typename T, int DK, int C>
struct DeltaFusedShape {
    static constexpr int ES = sizeof(T), CE = 16 / ES, PAD = row_pad<T>();
    static constexpr int NB = C / 16, NKB = DK / 16, DVT = 64;
    // Q, K, -W rows.  With bf16 a pad of 12 makes the row stride an odd multiple of 8
    // bytes, so the 16 lanes of an 8-byte row read (served together over 128 bytes on
    // gfx950) hit 16 different bank pairs; rows are then only 8-byte aligned, and every
    // access to them is 8 bytes wide
    static constexpr int LDK = DK + (ES == 2 ? 12 : PAD);
    static constexpr int LDU = C + PAD;            // U~^T rows
    static constexpr int LDV = DVT + 16 / ES;      // raw V rows
    static constexpr int LDC = C + 4;              // N / X^T rows (fp32)
    static constexpr int BUF = 3 * C * LDK + DVT * LDU;       // elements per chunk buffer
    static constexpr int QP = C * DK / CE, QPT = (QP + 255) / 256;
    static constexpr int VPT = (C * DVT / CE + 255) / 256;
    static_assert(NB <= 2, "fused path: chunks of 16 or 32 tokens");
};

template <typename T, int DK, int C>
constexpr int delta_fused_lds()
{
    typedef DeltaFusedShape<T, DK, C> SH;
    return (2 * SH::BUF + 2 * C * SH::LDV) * (int)sizeof(T) + (C * SH::LDC + 2 * C) * 4;
}

template <typename T, int DK, int C>
__global__ __launch_bounds__(512) void delta_fused_kernel(const DeltaArgs a)
{
    typedef DeltaFusedShape<T, DK, C> SH;
    constexpr int ES = SH::ES, CE = SH::CE, NB = SH::NB, NKB = SH::NKB;
    constexpr int LDK = SH::LDK, LDU = SH::LDU, LDV = SH::LDV, LDC = SH::LDC, QP = SH::QP;
    typedef typename Frag<T>::type F4;
    __shared__ __align__(16) T sbuf[2 * SH::BUF];      // per chunk: Q, K, -W rows, U~^T
    __shared__ __align__(16) T sVr[2][C * LDV];        // raw V rows of the chunk being solved
    __shared__ __align__(16) float sNX[C * LDC];       // N (strictly lower) and X^T (upper)
    __shared__ __align__(16) float sBt[2][C];          // write strengths

    // waves 0-3 solve the chunks' systems (and load their rows); waves 4-7 carry the
    // state, wave 4 + c owning value columns 16 c .. 16 c + 15 of the tile
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;
    const bool solver = w < 4;                         // wave-uniform
    const int wc = w - 4;
    int wgi = blockIdx.x;
    if (a.xcd_remap) wgi = (wgi & 7) * (gridDim.x >> 3) + (wgi >> 3);
    const int bh = wgi / a.n_vt, vt = wgi - bh * a.n_vt;
    const int L = a.L, DV = a.d_v, DVT = a.dvt;
    const int nch = (L + C - 1) / C;
    const size_t hrow = (size_t)bh * L;
    const int j0 = vt * DVT + 16 * wc;
    const bool active = !solver && 16 * wc < DVT;      // wave-uniform
    const int VP = C * DVT / CE;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    const Rsrc rq = make_rsrc((const T *)a.q + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rk = make_rsrc((const T *)a.k + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rv = make_rsrc((const T *)a.v + hrow * DV, (unsigned)(L * DV * ES));
    auto bQ = [&](int n) { return sbuf + (n & 1) * SH::BUF; };
    auto bK = [&](int n) { return sbuf + (n & 1) * SH::BUF + C * LDK; };
    auto bW = [&](int n) { return sbuf + (n & 1) * SH::BUF + 2 * C * LDK; };
    auto bU = [&](int n) { return sbuf + (n & 1) * SH::BUF + 3 * C * LDK; };

    // raw rows of a chunk: requested into registers, later written to LDS
    i32x4 gq[SH::QPT], gk[SH::QPT], gv[SH::VPT];
    float gb = 0.f;
    auto fetch = [&](int n) {
        const int base = n * C * DK * ES;
#pragma unroll
        for (int i = 0; i < SH::QPT; ++i) {
            const int p = tid + 256 * i;
            if (QP % 256 == 0 || p < QP) {
                gq[i] = buf_load16<i32x4>(rq, base + 16 * p);
                gk[i] = buf_load16<i32x4>(rk, base + 16 * p);
            }
        }
#pragma unroll
        for (int i = 0; i < SH::VPT; ++i) {
            const int p = tid + 256 * i;
            if (p < VP) {
                const int r = p / (DVT / CE), c = (p - r * (DVT / CE)) * CE;
                gv[i] = buf_load16<i32x4>(rv, ((n * C + r) * DV + vt * DVT + c) * ES);
            }
        }
        gb = (tid < C && n * C + tid < L) ? a.beta[hrow + n * C + tid] : 0.f;
    };
    auto stash = [&](int n) {
        T *sQ = bQ(n), *sK = bK(n), *sV = sVr[n & 1];
#pragma unroll
        for (int i = 0; i < SH::QPT; ++i) {
            const int p = tid + 256 * i;
            if (QP % 256 == 0 || p < QP) {
                const int r = p / (DK / CE), c = (p - r * (DK / CE)) * CE;
                typedef int i32x2 __attribute__((ext_vector_type(2)));
                *(i32x2 *)(sQ + r * LDK + c) = i32x2{gq[i][0], gq[i][1]};    // 8-byte aligned rows
                *(i32x2 *)(sQ + r * LDK + c + CE / 2) = i32x2{gq[i][2], gq[i][3]};
                *(i32x2 *)(sK + r * LDK + c) = i32x2{gk[i][0], gk[i][1]};
                *(i32x2 *)(sK + r * LDK + c + CE / 2) = i32x2{gk[i][2], gk[i][3]};
            }
        }
#pragma unroll
        for (int i = 0; i < SH::VPT; ++i) {
            const int p = tid + 256 * i;
            if (p < VP) {
                const int r = p / (DVT / CE), c = (p - r * (DVT / CE)) * CE;
                *(i32x4 *)(sV + r * LDV + c) = gv[i];
            }
        }
        if (tid < C) sBt[n & 1][tid] = gb;
    };

    // ---- the triangular solve of chunk m, in four steps ------------------------------
    // A: N = tril(diag(beta) K K^T, -1), strictly lower entries only
    // With two blocks, the full block N_10 is split over its key blocks between waves
    // 1 and 3: wave 3 stores its part transposed in the X^T block (0, 1), which is free
    // until the off-diagonal step adds it back in and then overwrites it.
    auto solveA = [&](int m) {
        const T *sK = bK(m);
        const float *bt = sBt[m & 1];
        // block (tb, sb) of N over key blocks [k0, k0 + NK); `tr`: store transposed
        auto part = [&](int tb, int sb, int k0, auto nkc, bool tr) {
            constexpr int NK = decltype(nkc)::value;
            const f32x4 g = contract_rows(sK + (16 * tb + x) * LDK + 16 * k0, sK + (16 * sb + x) * LDK + 16 * k0,
                                          NK, grp, zero);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tb + 4 * grp + e, s = 16 * sb + x;
                if (tr) sNX[s * LDC + t] = bt[t] * g[e];
                else if (s < t) sNX[t * LDC + s] = bt[t] * g[e];
            }
        };
        if constexpr (NB == 2) {
            constexpr int H1 = (NKB + 1) / 2;         // wave 1's key blocks of N_10
            if (w == 0) part(0, 0, 0, std::integral_constant<int, NKB>{}, false);
            else if (w == 1) part(1, 0, 0, std::integral_constant<int, H1>{}, false);
            else if (w == 2) part(1, 1, 0, std::integral_constant<int, NKB>{}, false);
            else part(1, 0, H1, std::integral_constant<int, NKB - H1>{}, true);
        } else {
            if (w == 0) part(0, 0, 0, std::integral_constant<int, NKB>{}, false);
        }
    };
    // B: the diagonal blocks' inverses, stored transposed (upper triangle with diagonal)
    auto solveB = [&]() {
        if (w < NB && lane < 16) {
            const int b = w, j = lane;
            const float *nb = sNX + 16 * b * LDC + 16 * b;
            float xs[16];                              // column-wise, as in delta_prep_kernel
#pragma unroll
            for (int r = 0; r < 16; ++r) xs[r] = r == j ? 1.f : 0.f;
#pragma unroll
            for (int mm = 0; mm < 16; ++mm)
#pragma unroll
                for (int r = mm + 1; r < 16; ++r) xs[r] -= nb[r * LDC + mm] * xs[mm];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (r >= j) sNX[(16 * b + j) * LDC + 16 * b + r] = xs[r];
        }
    };
    // fragment of X[row][16 cb + 4 grp + e] for row = 16 rb + x (the lower triangle of
    // X, read from its transpose); zero above the diagonal
    auto xrow = [&](int rb, int cb) {
        f32x4 v = col_frag(sNX, LDC, 16 * cb + 4 * grp, 16 * rb, x);
        if (rb == cb) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * grp + e > x) v[e] = 0.f;
        }
        return v;
    };
    // C: the block below the diagonal (two blocks): X_10 = -X_11 N_10 X_00
    auto solveC = [&]() {
        if (NB == 2 && w == 3) {
            // R = N_10 X_00: A = N_10 rows, B = X_00 columns = X_00^T rows (masked)
            f32x4 b0 = lds_frag(sNX + x * LDC, 0, grp);       // X^T[x][4 grp + e] = X[4 grp + e][x]
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * grp + e < x) b0[e] = 0.f;            // X_00 is zero above its diagonal
            // N_10 = the part in place + wave 3's part, stored transposed in block (0, 1)
            const f32x4 n10 = lds_frag(sNX + (16 + x) * LDC, 0, grp) + col_frag(sNX, LDC, 4 * grp, 16, x);
            const f32x4 r = mma1(n10, b0, zero);
            const f32x4 xr = mma1(xrow(1, 1), r, zero);       // X_11 R
            *(f32x4 *)(sNX + x * LDC + 16 + 4 * grp) = -xr;  // X^T block (0, 1)
        }
    };
    // D: -W and U~ of chunk m into its buffer, by all eight waves (the state waves
    // would otherwise wait for it); the fragments of X diag(beta) are formed once
    auto solveD = [&](int m) {
        const T *sK = bK(m), *sV = sVr[m & 1];
        T *sW = bW(m), *sU = bU(m);
        const float *bt = sBt[m & 1];
        auto xb = [&](int tb, int sb) -> F4 {
            return cvt4<T>(xrow(tb, sb) * *(const f32x4 *)(bt + 16 * sb + 4 * grp));
        };
        const F4 x00 = xb(0, 0);
        F4 x10 = x00, x11 = x00;
        if (NB == 2) {
            x10 = xb(1, 0);
            x11 = xb(1, 1);
        }
        const int nvb = DVT / 16, ntile = (NKB + nvb) * NB;
        auto tile = [&](int id) {
            const int tb = id % NB, cb = id / NB;
            f32x4 acc = zero;
            if (cb < NKB) {       // lane (x, grp) element e: W[16 tb + x][16 cb + 4 grp + e]
                if (tb == 1)
                    acc = mac2(col_frag(sK, LDK, 4 * grp, 16 * cb, x), col_frag(sK, LDK, 16 + 4 * grp, 16 * cb, x),
                               x10, x11, acc);
                else
                    acc = mac1(col_frag(sK, LDK, 4 * grp, 16 * cb, x), x00, acc);
                store4(sW + (16 * tb + x) * LDK + 16 * cb + 4 * grp, -acc);
            } else {              // lane (x, grp) element e: U~[16 tb + 4 grp + e][16 jb + x]
                const int jb = cb - NKB;
                if (tb == 1)
                    acc = mac2(x10, x11, col_frag(sV, LDV, 4 * grp, 16 * jb, x),
                               col_frag(sV, LDV, 16 + 4 * grp, 16 * jb, x), acc);
                else
                    acc = mac1(x00, col_frag(sV, LDV, 4 * grp, 16 * jb, x), acc);
                store4(sU + (16 * jb + x) * LDU + 16 * tb + 4 * grp, acc);
            }
        };
        if constexpr (NB == 2) {
            // at most (NKB + 4) * 2 tiles, dealt round-robin: a fixed trip count lets
            // the compiler interleave the tiles' reads and products (with one 16-row
            // block this measured slower than the plain loop)
            constexpr int ROUNDS = ((NKB + 4) * NB + 7) / 8;
#pragma unroll
            for (int r = 0; r < ROUNDS; ++r)
                if (w + 8 * r < ntile) tile(w + 8 * r);
        } else {
            for (int id = w; id < ntile; id += 8) tile(id);
        }
    };

    // ---- the state pass over chunk n ---------------------------------------------------
    f32x4 s[NKB], u[2];
#pragma unroll
    for (int ib = 0; ib < NKB; ++ib) {
        s[ib] = zero;
        if (active && a.s0) {
            const float *p = a.s0 + ((size_t)bh * DK + 16 * ib + 4 * grp) * DV + j0 + x;
            s[ib] = f32x4{p[0], p[DV], p[2 * DV], p[3 * DV]};
        }
    }
    auto scanU = [&](int n) {            // U = U~ + (-W) S
        const T *sW = bW(n), *sU = bU(n) + 16 * wc * LDU;
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            f32x4 acc = widen4(lds_frag(sU + x * LDU, tb, grp));
            const T *wrow = sW + (16 * tb + x) * LDK;
#pragma unroll
            for (int ib = 0; ib + 1 < NKB; ib += 2)
                acc = mac2(lds_frag(wrow, ib, grp), lds_frag(wrow, ib + 1, grp), cvt4<T>(s[ib]),
                           cvt4<T>(s[ib + 1]), acc);
            if (NKB % 2) acc = mac1(lds_frag(wrow, NKB - 1, grp), cvt4<T>(s[NKB - 1]), acc);
            u[tb] = acc;
        }
    };
    auto scanO = [&](int n) {            // O^T = S^T Q^T + U^T P^T, stored
        const T *sQ = bQ(n), *sK = bK(n);
        const int nvalid = min(C, L - n * C);
        T *og = (T *)a.o + (hrow + (size_t)n * C) * DV + j0 + 4 * grp;
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const T *qrow = sQ + (16 * tb + x) * LDK;
            f32x4 o = contract_regs_rows<T, NKB>(s, qrow, grp, zero);
            auto score = [&](int sb) {
                f32x4 p = contract_rows(sK + (16 * sb + x) * LDK, qrow, NKB, grp, zero);
                if (sb == tb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * grp + e > x) p[e] = 0.f;
                }
                return p;
            };
            if (tb == 1)
                o = mac2(cvt4<T>(u[0]), cvt4<T>(u[1]), cvt4<T>(score(0)), cvt4<T>(score(1)), o);
            else
                o = mac1(cvt4<T>(u[0]), cvt4<T>(score(0)), o);
            if (16 * tb + x < nvalid) store4(og + (size_t)(16 * tb + x) * DV, o);
        }
    };
    auto scanS = [&](int n) {            // S += K^T U
        const T *sK = bK(n);
#pragma unroll
        for (int ib = 0; ib < NKB; ++ib) {
            if (NB == 2)
                s[ib] = mac2(col_frag(sK, LDK, 4 * grp, 16 * ib, x), col_frag(sK, LDK, 16 + 4 * grp, 16 * ib, x),
                             cvt4<T>(u[0]), cvt4<T>(u[1]), s[ib]);
            else
                s[ib] = mac1(col_frag(sK, LDK, 4 * grp, 16 * ib, x), cvt4<T>(u[0]), s[ib]);
        }
    };

    if (nch > 0) {
        if (solver) {
            fetch(0);
            stash(0);
        }
        lds_barrier();
        if (solver) solveA(0);
        lds_barrier();
        if (solver) solveB();
        lds_barrier();
        if (solver) solveC();
        lds_barrier();
        solveD(0);                                     // all eight waves
        if (solver && nch > 1) fetch(1);
    }
    // The rows of chunk n+2 are requested by each solver wave in a step where it has
    // no part of the solve: waves NB.. while waves 0..NB-1 invert the diagonal blocks,
    // waves 0..NB-1 while wave 3 forms the block below the diagonal.
    const bool early = w >= NB;
    for (int n = 0; n < nch; ++n) {
        const bool more = solver && n + 1 < nch;       // wave-uniform
        const bool ahead = solver && n + 2 < nch;
        if (more) stash(n + 1);
        lds_barrier();                                 // chunk n's -W, U~ and chunk n+1's rows visible
        if (more) solveA(n + 1);
        if (active) scanU(n);
        lds_barrier();
        if (more) solveB();
        if (ahead && early) fetch(n + 2);
        if (active) scanO(n);
        lds_barrier();
        if (more) solveC();
        if (ahead && !early) fetch(n + 2);
        if (active) scanS(n);
        lds_barrier();
        if (n + 1 < nch) solveD(n + 1);
    }

    if (active && a.s_final) {
#pragma unroll
        for (int ib = 0; ib < NKB; ++ib) {
            float *p = a.s_final + ((size_t)bh * DK + 16 * ib + 4 * grp) * DV + j0 + x;
#pragma unroll
            for (int e = 0; e < 4; ++e) p[(size_t)e * DV] = s[ib][e];
        }
    }
}

// ------------------------------------------------------------------------------------
// delta_decode_kernel: one token on a resident fp32 state, in place
// ------------------------------------------------------------------------------------
// One workgroup per head; a thread owns a float4 column group and every RS-th row.
// The prediction S^T k and the read-out S^T q are column sums reduced across rows
// through LDS; the state is read once and written once.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void delta_decode_kernel(const DeltaArgs a)
{
    constexpr int CQ = DV / 4;
    constexpr int NT = (DK * CQ) < 256 ? (DK * CQ) : 256;
    constexpr int RS = NT / CQ;
    constexpr int NPASS = DK / RS;
    static_assert(NT >= DK && NT >= CQ && DK % RS == 0, "decode mapping");

    __shared__ float sq[DK], sk[DK];
    __shared__ f32x4 sred[RS][CQ];
    __shared__ f32x4 su[CQ];

    const int tid = threadIdx.x;
    const size_t bh = blockIdx.x;
    if (tid < DK) {
        sq[tid] = to_f32(((const T *)a.q)[bh * DK + tid]);
        sk[tid] = to_f32(((const T *)a.k)[bh * DK + tid]);
    }
    const int c = tid % CQ, r0 = tid / CQ;
    f32x4 *st = (f32x4 *)(a.s_final + bh * DK * DV) + c;
    f32x4 s[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) s[p] = __builtin_nontemporal_load(st + (size_t)(r0 + p * RS) * CQ);
    __syncthreads();

    f32x4 pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NPASS; ++p) pr += sk[r0 + p * RS] * s[p];
    sred[r0][c] = pr;
    __syncthreads();
    if (tid < CQ) {                                // u = beta (v - S^T k)
        f32x4 acc = sred[0][tid];
#pragma unroll
        for (int r = 1; r < RS; ++r) acc += sred[r][tid];
        const T *vp = (const T *)a.v + bh * DV + 4 * tid;
        const f32x4 v = {to_f32(vp[0]), to_f32(vp[1]), to_f32(vp[2]), to_f32(vp[3])};
        su[tid] = a.beta[bh] * (v - acc);
    }
    __syncthreads();

    const f32x4 u = su[c];
    f32x4 op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int i = r0 + p * RS;
        s[p] += sk[i] * u;
        __builtin_nontemporal_store(s[p], st + (size_t)i * CQ);
        op += sq[i] * s[p];
    }
    sred[r0][c] = op;
    __syncthreads();
    if (tid < CQ) {
        f32x4 acc = sred[0][tid];
#pragma unroll
        for (int r = 1; r < RS; ++r) acc += sred[r][tid];
        store4((T *)a.o + bh * DV + 4 * tid, acc);
    }
}

// ------------------------------------------------------------------------------------
// launches
// ------------------------------------------------------------------------------------
// Chunks of 16 or 32 tokens run in the fused kernel (its LDS fits for every d_k and
// both element types); chunks of 64 in the two kernels with the workspace between.
bool delta_fused(int chunk) { return chunk == 16 || chunk == 32; }

size_t delta_workspace(int BH, int L, int d_k, int d_v, int chunk, int elem_bytes)
{
    if (delta_fused(chunk)) return 0;
    const size_t lp = (size_t)(L + chunk - 1) / chunk * chunk;
    return (size_t)BH * lp * (d_k + d_v) * elem_bytes;
}

template <typename T, int C>
static hipError_t launch_delta_fused(const DeltaArgs &a, hipStream_t stream)
{
    const int grid = a.BH * a.n_vt;
#define GLA_FUSED(DK)                                                                                \
    case DK:                                                                                         \
        static_assert(delta_fused_lds<T, DK, C>() <= kLdsBytes, "fused delta LDS");                 \
        hipLaunchKernelGGL((delta_fused_kernel<T, DK, C>), dim3(grid), dim3(512), 0, stream, a);     \
        break;
    switch (a.d_k) {
    GLA_FUSED(16) GLA_FUSED(32) GLA_FUSED(64) GLA_FUSED(128)
    default: return hipErrorInvalidValue;
    }
#undef GLA_FUSED
    return hipGetLastError();
}

template <typename T, int C>
static hipError_t launch_delta_c(const DeltaArgs &a, hipStream_t stream)
{
    const int nch = (a.L + C - 1) / C;
    if (nch > 0) {
        hipLaunchKernelGGL((delta_prep_kernel<T, C>), dim3(a.BH * nch), dim3(256), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int grid = a.BH * a.n_vt;
    switch (a.d_k) {
    case 16: hipLaunchKernelGGL((delta_scan_kernel<T, 16, C>), dim3(grid), dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((delta_scan_kernel<T, 32, C>), dim3(grid), dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((delta_scan_kernel<T, 64, C>), dim3(grid), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((delta_scan_kernel<T, 128, C>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_delta_t(const DeltaArgs &a, int chunk, hipStream_t stream)
{
    if (chunk == 16) return launch_delta_fused<T, 16>(a, stream);
    if (chunk == 32) return launch_delta_fused<T, 32>(a, stream);
    if (chunk == 64) return launch_delta_c<T, 64>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_delta_prefill(const DeltaArgs &a, int dtype, int chunk, hipStream_t stream)
{
    if (dtype == 1) return launch_delta_t<bf16>(a, chunk, stream);
    return launch_delta_t<float>(a, chunk, stream);
}

template <typename T>
static hipError_t launch_delta_decode_t(const DeltaArgs &a, hipStream_t stream)
{
#define GLA_DELTA_DECODE(DK, DV)                                                                   \
    if (a.d_k == DK && a.d_v == DV) {                                                              \
        constexpr int NT = (DK * (DV / 4)) < 256 ? (DK * (DV / 4)) : 256;                          \
        hipLaunchKernelGGL((delta_decode_kernel<T, DK, DV>), dim3(a.BH), dim3(NT), 0, stream, a);  \
        return hipGetLastError();                                                                  \
    }
#define GLA_DELTA_DECODE_DV(DK) \
    GLA_DELTA_DECODE(DK, 16) GLA_DELTA_DECODE(DK, 32) GLA_DELTA_DECODE(DK, 64) GLA_DELTA_DECODE(DK, 128)
    GLA_DELTA_DECODE_DV(16) GLA_DELTA_DECODE_DV(32) GLA_DELTA_DECODE_DV(64) GLA_DELTA_DECODE_DV(128)
#undef GLA_DELTA_DECODE_DV
#undef GLA_DELTA_DECODE
    return hipErrorInvalidValue;
}

hipError_t launch_delta_decode(const DeltaArgs &a, int dtype, hipStream_t stream)
{
    if (dtype == 1) return launch_delta_decode_t<bf16>(a, stream);
    return launch_delta_decode_t<float>(a, stream);
}

}  // namespace gla
