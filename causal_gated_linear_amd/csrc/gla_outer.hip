// gla_outer.hip -- gated linear attention with the outer-product gate on gfx950.
//
// "Gated Linear Attention", section "GLA / Recurrent Form": of the general gate
// G_t (.) S_{t-1}, the low-rank parameterisation G_t = alpha_t beta_t^T decays the
// state along both dimensions:
//
//     S_t[i][j] = alpha_t[i] beta_t[j] S_{t-1}[i][j] + phi(k_t)[i] v_t[j],
//     o_t = S_t^T phi(q_t)
//
// with natural-log gates g (alpha, [L][d_k]) and gv (beta, [L][d_v]).  Chunkwise, with
// in-chunk inclusive cumulative log-gates A[t][i], Bv[t][j] and chunk totals
// GA = A[C-1], GB = Bv[C-1]:
//
//     Q~ = phi(Q) e^A,  K^ = phi(K) e^-A,  V^ = V e^-Bv
//     O  = ((Q~ K^^T masked to s <= t) V^ + Q~ S) (.) e^Bv
//     S <- Diag(e^GA) (S + K^^T V^) Diag(e^GB)
//
// (the product of the gates between s and t factorises per key dimension and per
// value dimension).  The factors e^-A and e^-Bv, and their product in K^^T V^, must
// stay well inside the fp32 range: a chunk whose lowest key-side and lowest
// value-side cumulative log2-gates add up to less than -kFastLim is computed token
// by token instead (gla_slow.hpp), exact for any gate in [0, 1].  The consumer waves
// run that loop on their own state registers; the rows are staged in LDS.
//
// One workgroup per (head, value tile of up to 64 columns); wave w owns 16 value
// columns and their state slice S[d_k][16] in accumulator registers.  Per chunk the
// workgroup stages the raw rows (q, k, v, both gates) in LDS, then
//   1. computes the cumulative sums A and Bv: a thread owns four columns of a segment
//      of rows, sums them serially, and the segments finish the scan with shuffles
//      across consecutive lanes; it then scales its rows' q, k, v elements in place
//      and writes e^Bv for the output and the chunk totals;
//   2. computes the masked scores, O^T = (S^T Q~^T + V^^T P^T) (.) e^Bv^T and the
//      two-sided state update, as in the other prefill kernels.
// The next chunk's raw rows are requested before the current chunk is computed.
#include "gla_device.hpp"
#include "gla_launch.hpp"
#include "gla_slow.hpp"

namespace gla {

namespace {
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <typename T> constexpr int pad_of() { return sizeof(T) == 2 ? 16 : 4; }

// Minimum over the 64 lanes, in registers only: DPP shifts within each 16-lane row
// (a lane whose source is outside the row keeps its own value), then the rows' last
// lanes read as scalars.
template <int SHIFT> __device__ __forceinline__ float row_shr_keep(float v)
{
    const int b = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x110 + SHIFT, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_min(float v)
{
    v = fminf(v, row_shr_keep<1>(v));
    v = fminf(v, row_shr_keep<2>(v));
    v = fminf(v, row_shr_keep<4>(v));
    v = fminf(v, row_shr_keep<8>(v));
    const int b = __builtin_bit_cast(int, v);
    return fminf(fminf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 15)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 31))),
                 fminf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 47)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63))));
}
}  // namespace

template <typename T, int DK, int C>
struct OuterShape {
    static constexpr int ES = sizeof(T), CE = 16 / ES, PAD = pad_of<T>();
    static constexpr int NB = C / 16, NKB = DK / 16, DVT = 64;
    static constexpr int LDK = DK + PAD, LDV = DVT + PAD;      // T rows
    // key rows of the producer/consumer kernel, whose accesses to them are all 8 bytes
    // wide: with bf16 a pad of 12 makes the row stride an odd multiple of 8 bytes, so
    // the 16 lanes of an 8-byte row read hit 16 different bank pairs (gfx950 serves
    // them together over 128 bytes); transposing reads and the producers' writes stay
    // within 2-way conflicts
    static constexpr int LDKP = DK + (ES == 2 ? 12 : PAD);
    static constexpr int LDG = DK + 4, LDGV = DVT + 4;         // fp32 rows
    // 16-byte pieces per chunk, and per thread (256 threads)
    static constexpr int PQ = C * DK / CE, PG = C * DK / 4;
    static constexpr int PVM = C * DVT / CE, PGVM = C * DVT / 4;   // at the widest tile
    static constexpr int TQ = (PQ + 255) / 256, TG = (PG + 255) / 256;
    static constexpr int TV = (PVM + 255) / 256, TGV = (PGVM + 255) / 256;
    // cumulative-gate scan: row segments per four-column group (key side, value side)
    static constexpr int KSEG = C < 256 / (DK / 4) ? C : 256 / (DK / 4);
    static constexpr int VSEG = C < 256 / (DVT / 4) ? C : 256 / (DVT / 4);
    static_assert(KSEG <= 64 && VSEG <= 64, "a segment group stays within one wave");
};

template <typename T, int DK, int C, bool ELU1>
__global__ __launch_bounds__(256) void outer_prefill_kernel(const OuterArgs a)
{
    typedef OuterShape<T, DK, C> SH;
    constexpr int ES = SH::ES, CE = SH::CE, NB = SH::NB, NKB = SH::NKB;
    constexpr int LDK = SH::LDK, LDV = SH::LDV, LDG = SH::LDG, LDGV = SH::LDGV;
    __shared__ __align__(16) T sQ[C * LDK];
    __shared__ __align__(16) T sK[C * LDK];
    __shared__ __align__(16) T sV[C * LDV];
    __shared__ __align__(16) float sG[C * LDG];       // raw key-dimension log-gates
    __shared__ __align__(16) float sGV[C * LDGV];     // raw value-dimension log-gates
    __shared__ __align__(16) float sEV[C * LDGV];     // e^Bv[t][j]
    __shared__ __align__(16) float sEA[DK];           // e^GA
    __shared__ __align__(16) float sEB[SH::DVT];      // e^GB
    __shared__ __align__(16) float sMin[4][2];        // per wave: lowest key / value chunk total

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;
    int wgi = blockIdx.x;
    if (a.xcd_remap) wgi = (wgi & 7) * (gridDim.x >> 3) + (wgi >> 3);
    const int bh = wgi / a.n_vt, vt = wgi - bh * a.n_vt;
    const int L = a.L, DV = a.d_v, DVT = a.dvt;
    const int nch = (L + C - 1) / C;
    const size_t hrow = (size_t)bh * L;
    const int j0 = vt * DVT + 16 * w;                  // this wave's first value column
    const bool active = 16 * w < DVT;                  // wave-uniform
    const int PV = C * DVT / CE, PGV = C * DVT / 4;    // pieces of this tile's v and gv rows

    // head views; rows past the end of the sequence read as zeros (zero log-gates)
    const Rsrc rq = make_rsrc((const T *)a.q + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rk = make_rsrc((const T *)a.k + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rv = make_rsrc((const T *)a.v + hrow * DV, (unsigned)(L * DV * ES));
    const Rsrc rg = make_rsrc(a.g + hrow * DK, (unsigned)(L * DK * 4));
    const Rsrc rgv = make_rsrc(a.gv + hrow * DV, (unsigned)(L * DV * 4));

    i32x4 gq[SH::TQ], gk[SH::TQ], gg[SH::TG], gvv[SH::TV], ggv[SH::TGV];
    auto fetch = [&](int n) {
        const int r0 = n * C;
#pragma unroll
        for (int i = 0; i < SH::TQ; ++i) {
            const int p = tid + 256 * i;
            if (SH::PQ % 256 == 0 || p < SH::PQ) {
                gq[i] = buf_load16<i32x4>(rq, (r0 * DK + p * CE) * ES);
                gk[i] = buf_load16<i32x4>(rk, (r0 * DK + p * CE) * ES);
            }
        }
#pragma unroll
        for (int i = 0; i < SH::TG; ++i) {
            const int p = tid + 256 * i;
            if (SH::PG % 256 == 0 || p < SH::PG) gg[i] = buf_load16<i32x4>(rg, (r0 * DK + p * 4) * 4);
        }
#pragma unroll
        for (int i = 0; i < SH::TV; ++i) {
            const int p = tid + 256 * i;
            if (p < PV) {
                const int r = p / (DVT / CE), c = (p - r * (DVT / CE)) * CE;
                gvv[i] = buf_load16<i32x4>(rv, ((r0 + r) * DV + vt * DVT + c) * ES);
            }
        }
#pragma unroll
        for (int i = 0; i < SH::TGV; ++i) {
            const int p = tid + 256 * i;
            if (p < PGV) {
                const int r = p / (DVT / 4), c = (p - r * (DVT / 4)) * 4;
                ggv[i] = buf_load16<i32x4>(rgv, ((r0 + r) * DV + vt * DVT + c) * 4);
            }
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < SH::TQ; ++i) {
            const int p = tid + 256 * i;
            if (SH::PQ % 256 == 0 || p < SH::PQ) {
                const int r = p / (DK / CE), c = (p - r * (DK / CE)) * CE;
                *(i32x4 *)(sQ + r * LDK + c) = gq[i];
                *(i32x4 *)(sK + r * LDK + c) = gk[i];
            }
        }
#pragma unroll
        for (int i = 0; i < SH::TG; ++i) {
            const int p = tid + 256 * i;
            if (SH::PG % 256 == 0 || p < SH::PG) {
                const int r = p / (DK / 4), c = (p - r * (DK / 4)) * 4;
                *(i32x4 *)(sG + r * LDG + c) = gg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < SH::TV; ++i) {
            const int p = tid + 256 * i;
            if (p < PV) {
                const int r = p / (DVT / CE), c = (p - r * (DVT / CE)) * CE;
                *(i32x4 *)(sV + r * LDV + c) = gvv[i];
            }
        }
#pragma unroll
        for (int i = 0; i < SH::TGV; ++i) {
            const int p = tid + 256 * i;
            if (p < PGV) {
                const int r = p / (DVT / 4), c = (p - r * (DVT / 4)) * 4;
                *(i32x4 *)(sGV + r * LDGV + c) = ggv[i];
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
        if (n > 0) lds_barrier();                      // the previous chunk's readers are done
        stash();
        lds_barrier();
        if (n + 1 < nch) fetch(n + 1);
        const int nvalid = min(C, L - n * C);

        // 1. cumulative gates; scale q, k (key side) and v (value side) in place.
        //    A thread owns four columns of a segment of rows: it sums its rows serially,
        //    the segments of a column group (consecutive lanes) finish the scan with
        //    shuffles, then it scales its rows' elements.  kmin / vmin: the lowest
        //    cumulative log2-gate of the thread's columns (gates <= 0: the chunk totals).
        float kmin = 0.f, vmin = 0.f;
        {
            constexpr int NCG = DK / 4, NSEG = SH::KSEG, RPT = C / NSEG;
            const int cg = tid / NSEG, seg = tid % NSEG;
            if (cg < NCG) {                                    // whole waves
                float pre[RPT][4], run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    const f32x4 g = *(const f32x4 *)(sG + (seg * RPT + r) * LDG + 4 * cg);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pre[r][e] = run[e] += g[e] * kLog2e;
                }
                float excl[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float incl = run[e];
#pragma unroll
                    for (int off = 1; off < NSEG; off <<= 1) {
                        const float up = __shfl_up(incl, off, NSEG);
                        if (seg >= off) incl += up;
                    }
                    excl[e] = incl - run[e];
                    kmin = fminf(kmin, excl[e] + pre[RPT - 1][e]);
                }
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    const int t = seg * RPT + r;
                    T *qp = sQ + t * LDK + 4 * cg, *kp = sK + t * LDK + 4 * cg;
                    const f32x4 qv = widen4(*(const typename Frag<T>::type *)qp);
                    const f32x4 kv = widen4(*(const typename Frag<T>::type *)kp);
                    f32x4 qo, ko, up;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float b = excl[e] + pre[r][e];
                        up[e] = exp2_fast(b);
                        qo[e] = feature(qv[e], ELU1) * up[e];
                        ko[e] = feature(kv[e], ELU1) * exp2_fast(-b);
                    }
                    *(typename Frag<T>::type *)qp = cvt4<T>(qo);
                    *(typename Frag<T>::type *)kp = cvt4<T>(ko);
                    if (t == C - 1) *(f32x4 *)(sEA + 4 * cg) = up;
                }
            }
        }
        {
            constexpr int NCG = SH::DVT / 4, NSEG = SH::VSEG, RPT = C / NSEG;
            const int cg = tid / NSEG, seg = tid % NSEG;
            if (cg < NCG && 4 * cg < DVT) {                    // all lanes of a segment group agree
                float pre[RPT][4], run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    const f32x4 g = *(const f32x4 *)(sGV + (seg * RPT + r) * LDGV + 4 * cg);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pre[r][e] = run[e] += g[e] * kLog2e;
                }
                float excl[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float incl = run[e];
#pragma unroll
                    for (int off = 1; off < NSEG; off <<= 1) {
                        const float up = __shfl_up(incl, off, NSEG);
                        if (seg >= off) incl += up;
                    }
                    excl[e] = incl - run[e];
                    vmin = fminf(vmin, excl[e] + pre[RPT - 1][e]);
                }
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    const int t = seg * RPT + r;
                    T *vp = sV + t * LDV + 4 * cg;
                    const f32x4 vv = widen4(*(const typename Frag<T>::type *)vp);
                    f32x4 vo, up;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float b = excl[e] + pre[r][e];
                        up[e] = exp2_fast(b);
                        vo[e] = vv[e] * exp2_fast(-b);
                    }
                    *(typename Frag<T>::type *)vp = cvt4<T>(vo);
                    *(f32x4 *)(sEV + t * LDGV + 4 * cg) = up;
                    if (t == C - 1) *(f32x4 *)(sEB + 4 * cg) = up;
                }
            }
        }
        kmin = wave_min(kmin);
        vmin = wave_min(vmin);
        if (lane == 0) {
            sMin[w][0] = kmin;
            sMin[w][1] = vmin;
        }
        lds_barrier();
        {
            float km = sMin[0][0], vm = sMin[0][1];
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                km = fminf(km, sMin[i][0]);
                vm = fminf(vm, sMin[i][1]);
            }
            if (__builtin_amdgcn_readfirstlane(km + vm < -kFastLim ? 1 : 0)) {
                // out of the factorised range: the chunk token by token (the staged rows
                // were scaled in place, so they are staged again from memory)
                const SlowStage<T> st{sG, sGV, sQ, sK, sV};
                T *out = (T *)a.o + (hrow + (size_t)n * C) * DV + vt * DVT;
                f32x4 zz[NKB] = {};
                for (int r0 = 0; r0 < nvalid; r0 += C) {
                    slow_stage<T, DK, C, 256, ELU1, true, true>(st, rq, rk, rv, rg, rgv, n * C + r0, DV, vt * DVT,
                                                                DVT, tid);
                    lds_barrier();
                    if (active)
                        slow_tokens<T, DK, NKB, 16, 16, true, false, true>(st, s, zz, 4 * grp, 16 * w + x, DVT,
                                                                       min(C, nvalid - r0), out + (size_t)r0 * DV
                                                                       + 16 * w + x, DV, lane < 16);
                    lds_barrier();
                }
                continue;
            }
        }
        if (!active) continue;

        // 2. O^T = (S^T Q~^T + V^^T P^T) (.) e^Bv^T; lane (x, grp) element e:
        //    O[16 tb + x][j0 + 4 grp + e]
        T *og = (T *)a.o + (hrow + (size_t)n * C) * DV + j0 + 4 * grp;
        const int jl = 16 * w;                         // this wave's columns within the tile
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const T *qrow = sQ + (16 * tb + x) * LDK;
            f32x4 o = contract_regs_rows<T, NKB>(s, qrow, grp, zero);
            auto score = [&](int sb) {                 // P^T[s][t], s = 16 sb + 4 grp + e
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
                    o = mac2(col_frag(sV, LDV, 16 * sb + 4 * grp, jl, x),
                             col_frag(sV, LDV, 16 * (sb + 1) + 4 * grp, jl, x), cvt4<T>(score(sb)),
                             cvt4<T>(score(sb + 1)), o);
                else
                    o = mac1(col_frag(sV, LDV, 16 * sb + 4 * grp, jl, x), cvt4<T>(score(sb)), o);
            }
            o *= *(const f32x4 *)(sEV + (16 * tb + x) * LDGV + jl + 4 * grp);
            if (16 * tb + x < nvalid) store4(og + (size_t)(16 * tb + x) * DV, o);
        }

        // 3. S <- Diag(e^GA) (S + K^^T V^) Diag(e^GB)
        const float eb = sEB[jl + x];
#pragma unroll
        for (int ib = 0; ib < NKB; ++ib) {
#pragma unroll
            for (int sb = 0; sb + 1 < NB; sb += 2)
                s[ib] = mac2(col_frag(sK, LDK, 16 * sb + 4 * grp, 16 * ib, x),
                             col_frag(sK, LDK, 16 * (sb + 1) + 4 * grp, 16 * ib, x),
                             col_frag(sV, LDV, 16 * sb + 4 * grp, jl, x),
                             col_frag(sV, LDV, 16 * (sb + 1) + 4 * grp, jl, x), s[ib]);
            if (NB % 2)
                s[ib] = mac1(col_frag(sK, LDK, 16 * (NB - 1) + 4 * grp, 16 * ib, x),
                             col_frag(sV, LDV, 16 * (NB - 1) + 4 * grp, jl, x), s[ib]);
            s[ib] *= *(const f32x4 *)(sEA + 16 * ib + 4 * grp) * eb;
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

// Producer/consumer form of the same computation, for the sizes whose two operand
// buffers fit in LDS.  Eight waves: the four producer waves load the raw rows of
// chunk n+1 straight into registers in the scan's own layout (a thread owns four
// columns of a segment of rows), run the cumulative gates and write Q~, K^, V^,
// e^Bv and the chunk totals into one LDS buffer, while the four consumer waves run
// chunk n's products from the other buffer; one barrier per chunk.
template <typename T, int DK, int C>
constexpr int outer_pc_lds()
{
    typedef OuterShape<T, DK, C> SH;
    return 2 * ((2 * C * SH::LDKP + C * SH::LDV) * (int)sizeof(T) + (C * SH::LDGV + DK + SH::DVT) * 4);
}

// Rows staged at a time by the producer/consumer kernel's token-by-token chunks: the
// largest of C, 32, 16, 8 whose phi(q) and phi(k) rows fit in the Q~ buffers and whose
// alpha, beta and v rows fit in the e^Bv buffers.
constexpr int outer_slow_rows(int c, int q_bytes, int ev_bytes, int dk, int es)
{
    for (int sr : {64, 32, 16, 8})
        if (sr <= c && 2 * sr * dk * es <= q_bytes && sr * (dk * 4 + 64 * 4 + 64 * es) <= ev_bytes) return sr;
    return 0;
}

template <typename T> __device__ __forceinline__ typename Frag<T>::type buf_load_frag(Rsrc r, int off);
template <> __device__ __forceinline__ bf16x4 buf_load_frag<bf16>(Rsrc r, int off)
{
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(bf16x4, __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0)));
}
template <> __device__ __forceinline__ f32x4 buf_load_frag<float>(Rsrc r, int off)
{
    return buf_load16<f32x4>(r, off);
}

template <typename T, int DK, int C, bool ELU1>
__global__ __launch_bounds__(512) void outer_pc_kernel(const OuterArgs a)
{
    typedef OuterShape<T, DK, C> SH;
    constexpr int ES = SH::ES, NB = SH::NB, NKB = SH::NKB;
    constexpr int LDK = SH::LDKP, LDV = SH::LDV, LDGV = SH::LDGV;
    constexpr int KNCG = DK / 4, KSEG = SH::KSEG, KRPT = C / KSEG;
    constexpr int VNCG = SH::DVT / 4, VSEG = SH::VSEG, VRPT = C / VSEG;
    typedef typename Frag<T>::type F4;
    __shared__ __align__(16) T sQ[2][C * LDK];
    __shared__ __align__(16) T sK[2][C * LDK];
    __shared__ __align__(16) T sV[2][C * LDV];
    __shared__ __align__(16) float sEV[2][C * LDGV];
    __shared__ __align__(16) float sEA[2][DK];
    __shared__ __align__(16) float sEB[2][SH::DVT];
    __shared__ __align__(16) float sMin[2][4][2];     // per producer wave: lowest key / value chunk total

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;
    const bool producer = w < 4;                       // wave-uniform
    int wgi = blockIdx.x;
    if (a.xcd_remap) wgi = (wgi & 7) * (gridDim.x >> 3) + (wgi >> 3);
    const int bh = wgi / a.n_vt, vt = wgi - bh * a.n_vt;
    const int L = a.L, DV = a.d_v, DVT = a.dvt;
    const int nch = (L + C - 1) / C;
    const size_t hrow = (size_t)bh * L;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // ---- producers ---------------------------------------------------------------------
    const Rsrc rq = make_rsrc((const T *)a.q + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rk = make_rsrc((const T *)a.k + hrow * DK, (unsigned)(L * DK * ES));
    const Rsrc rv = make_rsrc((const T *)a.v + hrow * DV, (unsigned)(L * DV * ES));
    const Rsrc rg = make_rsrc(a.g + hrow * DK, (unsigned)(L * DK * 4));
    const Rsrc rgv = make_rsrc(a.gv + hrow * DV, (unsigned)(L * DV * 4));
    const int kcg = tid / KSEG, kseg = tid % KSEG, vcg = tid / VSEG, vseg = tid % VSEG;
    const bool klane = producer && kcg < KNCG;                 // whole waves
    const bool vlane = producer && vcg < VNCG && 4 * vcg < DVT;   // whole segment groups
    f32x4 rgk[KRPT], rgvv[VRPT];
    F4 rqq[KRPT], rkk[KRPT], rvv[VRPT];
    auto load = [&](int n) {
        if (klane) {
#pragma unroll
            for (int r = 0; r < KRPT; ++r) {
                const int t = n * C + kseg * KRPT + r;         // rows past L read as zeros
                rgk[r] = buf_load16<f32x4>(rg, (t * DK + 4 * kcg) * 4);
                rqq[r] = buf_load_frag<T>(rq, (t * DK + 4 * kcg) * ES);
                rkk[r] = buf_load_frag<T>(rk, (t * DK + 4 * kcg) * ES);
            }
        }
        if (vlane) {
#pragma unroll
            for (int r = 0; r < VRPT; ++r) {
                const int t = n * C + vseg * VRPT + r;
                rgvv[r] = buf_load16<f32x4>(rgv, (t * DV + vt * DVT + 4 * vcg) * 4);
                rvv[r] = buf_load_frag<T>(rv, (t * DV + vt * DVT + 4 * vcg) * ES);
            }
        }
    };
    // inclusive prefix sums (log2 units) of a thread's rows, and the exclusive offset
    // of its segment within the column group (segments on consecutive lanes)
    auto scan = [&](const f32x4 *g, int nr, int nseg, int seg, float (*pre)[4], float *excl) {
        float run[4] = {0.f, 0.f, 0.f, 0.f};
        for (int r = 0; r < nr; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) pre[r][e] = run[e] += g[r][e] * kLog2e;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float incl = run[e];
            for (int off = 1; off < nseg; off <<= 1) {
                const float up = __shfl_up(incl, off, nseg);
                if (seg >= off) incl += up;
            }
            excl[e] = incl - run[e];
        }
    };
    auto produce = [&](int n) {
        const int b = n & 1;
        float kmin = 0.f, vmin = 0.f;                  // lowest cumulative log2-gates (chunk totals)
        if (klane) {
            float pre[KRPT][4], excl[4];
            scan(rgk, KRPT, KSEG, kseg, pre, excl);
#pragma unroll
            for (int e = 0; e < 4; ++e) kmin = fminf(kmin, excl[e] + pre[KRPT - 1][e]);
#pragma unroll
            for (int r = 0; r < KRPT; ++r) {
                const int t = kseg * KRPT + r;
                const f32x4 qv = widen4(rqq[r]), kv = widen4(rkk[r]);
                f32x4 qo, ko, up;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float bb = excl[e] + pre[r][e];
                    up[e] = exp2_fast(bb);
                    qo[e] = feature(qv[e], ELU1) * up[e];
                    ko[e] = feature(kv[e], ELU1) * exp2_fast(-bb);
                }
                *(F4 *)(sQ[b] + t * LDK + 4 * kcg) = cvt4<T>(qo);
                *(F4 *)(sK[b] + t * LDK + 4 * kcg) = cvt4<T>(ko);
                if (t == C - 1) *(f32x4 *)(sEA[b] + 4 * kcg) = up;
            }
        }
        if (vlane) {
            float pre[VRPT][4], excl[4];
            scan(rgvv, VRPT, VSEG, vseg, pre, excl);
#pragma unroll
            for (int e = 0; e < 4; ++e) vmin = fminf(vmin, excl[e] + pre[VRPT - 1][e]);
#pragma unroll
            for (int r = 0; r < VRPT; ++r) {
                const int t = vseg * VRPT + r;
                const f32x4 vv = widen4(rvv[r]);
                f32x4 vo, up;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float bb = excl[e] + pre[r][e];
                    up[e] = exp2_fast(bb);
                    vo[e] = vv[e] * exp2_fast(-bb);
                }
                *(F4 *)(sV[b] + t * LDV + 4 * vcg) = cvt4<T>(vo);
                *(f32x4 *)(sEV[b] + t * LDGV + 4 * vcg) = up;
                if (t == C - 1) *(f32x4 *)(sEB[b] + 4 * vcg) = up;
            }
        }
        kmin = wave_min(kmin);
        vmin = wave_min(vmin);
        if (lane == 0) {
            sMin[b][w][0] = kmin;
            sMin[b][w][1] = vmin;
        }
    };
    // the chunk in buffer b is out of the factorised range (read after the barrier
    // that publishes the producers' totals: every wave takes the same decision)
    auto chunk_far = [&](int b) -> bool {
        float km = sMin[b][0][0], vm = sMin[b][0][1];
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            km = fminf(km, sMin[b][i][0]);
            vm = fminf(vm, sMin[b][i][1]);
        }
        return __builtin_amdgcn_readfirstlane(km + vm < -kFastLim ? 1 : 0) != 0;
    };
    // Such a chunk runs token by token on the consumers' state registers; the consumer
    // waves stage its rows from memory in groups of SR rows into the two operand
    // buffers' space (both free here: the producers fill the next one afterwards), and
    // the producers pass the same barriers.
    constexpr int SR = outer_slow_rows(C, (int)sizeof(sQ), (int)sizeof(sEV), DK, ES);
    static_assert(SR > 0, "token-loop staging within the operand buffers");

    // ---- consumers ---------------------------------------------------------------------
    const int c = w - 4, jl = 16 * c, j0 = vt * DVT + jl;
    const bool active = !producer && jl < DVT;          // wave-uniform
    f32x4 s[NKB];
#pragma unroll
    for (int ib = 0; ib < NKB; ++ib) {
        s[ib] = zero;
        if (active && a.s0) {
            const float *p = a.s0 + ((size_t)bh * DK + 16 * ib + 4 * grp) * DV + j0 + x;
            s[ib] = f32x4{p[0], p[DV], p[2 * DV], p[3 * DV]};
        }
    }
    auto consume = [&](int n) {
        const int b = n & 1;
        const T *Q = sQ[b], *K = sK[b], *V = sV[b];
        const int nvalid = min(C, L - n * C);
        T *og = (T *)a.o + (hrow + (size_t)n * C) * DV + j0 + 4 * grp;
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {               // O^T = (S^T Q~^T + V^^T P^T) (.) e^Bv^T
            const T *qrow = Q + (16 * tb + x) * LDK;
            f32x4 o = contract_regs_rows<T, NKB>(s, qrow, grp, zero);
            auto score = [&](int sb) {
                f32x4 p = contract_rows(K + (16 * sb + x) * LDK, qrow, NKB, grp, zero);
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
                    o = mac2(col_frag(V, LDV, 16 * sb + 4 * grp, jl, x), col_frag(V, LDV, 16 * (sb + 1) + 4 * grp, jl, x),
                             cvt4<T>(score(sb)), cvt4<T>(score(sb + 1)), o);
                else
                    o = mac1(col_frag(V, LDV, 16 * sb + 4 * grp, jl, x), cvt4<T>(score(sb)), o);
            }
            o *= *(const f32x4 *)(sEV[b] + (16 * tb + x) * LDGV + jl + 4 * grp);
            if (16 * tb + x < nvalid) store4(og + (size_t)(16 * tb + x) * DV, o);
        }
        const float eb = sEB[b][jl + x];                 // S <- Diag(e^GA)(S + K^^T V^)Diag(e^GB)
#pragma unroll
        for (int ib = 0; ib < NKB; ++ib) {
#pragma unroll
            for (int sb = 0; sb + 1 < NB; sb += 2)
                s[ib] = mac2(col_frag(K, LDK, 16 * sb + 4 * grp, 16 * ib, x),
                             col_frag(K, LDK, 16 * (sb + 1) + 4 * grp, 16 * ib, x),
                             col_frag(V, LDV, 16 * sb + 4 * grp, jl, x),
                             col_frag(V, LDV, 16 * (sb + 1) + 4 * grp, jl, x), s[ib]);
            if (NB % 2)
                s[ib] = mac1(col_frag(K, LDK, 16 * (NB - 1) + 4 * grp, 16 * ib, x),
                             col_frag(V, LDV, 16 * (NB - 1) + 4 * grp, jl, x), s[ib]);
            s[ib] *= *(const f32x4 *)(sEA[b] + 16 * ib + 4 * grp) * eb;
        }
    };

    // The two roles run separate loops that meet at the same barriers.  A chunk out of
    // range takes the consumers out of their loop into the token-by-token block after
    // it, which rejoins the loop at the next chunk; the producers pass the same
    // barriers and then prepare the next chunk as usual.
    if (producer) {
        if (nch > 0) {
            load(0);
            produce(0);
            if (nch > 1) load(1);
        }
        for (int n = 0; n < nch; ++n) {
            lds_barrier();                               // buffer n ready, buffer n+1 free
            if (chunk_far(n & 1)) {
                for (int r0 = 0; r0 < min(C, L - n * C); r0 += SR) {
                    lds_barrier();
                    lds_barrier();
                }
            }
            if (n + 1 < nch) {
                produce(n + 1);
                if (n + 2 < nch) load(n + 2);
            }
        }
    } else {
        int n = 0;
        for (;;) {
            for (; n < nch; ++n) {
                lds_barrier();                           // buffer n ready
                if (chunk_far(n & 1)) break;
                if (active) consume(n);
            }
            if (n >= nch) break;
            const int nvalid = min(C, L - n * C);
            float *const ev = &sEV[0][0];
            const SlowStage<T> st{ev, ev + SR * DK, &sQ[0][0], &sQ[0][0] + SR * DK,
                                  (T *)(ev + SR * DK + SR * SH::DVT)};
            T *out = (T *)a.o + (hrow + (size_t)n * C) * DV + vt * DVT;
            f32x4 zz[NKB] = {};
            for (int r0 = 0; r0 < nvalid; r0 += SR) {
                slow_stage<T, DK, SR, 256, ELU1, true, true>(st, rq, rk, rv, rg, rgv, n * C + r0, DV, vt * DVT, DVT,
                                                             tid - 256);
                lds_barrier();
                if (active)
                    slow_tokens<T, DK, NKB, 16, 16, true, false, true>(st, s, zz, 4 * grp, jl + x, DVT,
                                                                       min(SR, nvalid - r0),
                                                                       out + (size_t)r0 * DV + jl + x, DV, lane < 16);
                lds_barrier();
            }
            ++n;
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

// One token on a resident fp32 state, in place: S <- (alpha beta^T) (.) S + phi(k) v^T,
// o = S^T phi(q).  One workgroup per head; a thread owns a float4 column group (with its
// four value gates) and every RS-th row; o is reduced across rows through LDS.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void outer_decode_kernel(const OuterArgs a)
{
    constexpr int CQ = DV / 4;
    constexpr int NT = (DK * CQ) < 256 ? (DK * CQ) : 256;
    constexpr int RS = NT / CQ;
    constexpr int NPASS = DK / RS;
    static_assert(NT >= DK && NT >= CQ && DK % RS == 0, "decode mapping");
    __shared__ float sq[DK], sk[DK], sa[DK];
    __shared__ f32x4 sred[RS][CQ];

    const int tid = threadIdx.x;
    const size_t bh = blockIdx.x;
    const bool elu1 = a.elu1 != 0;
    if (tid < DK) {
        sq[tid] = feature(to_f32(((const T *)a.q)[bh * DK + tid]), elu1);
        sk[tid] = feature(to_f32(((const T *)a.k)[bh * DK + tid]), elu1);
        sa[tid] = exp2_fast(a.g[bh * DK + tid] * kLog2e);
    }
    const int c = tid % CQ, r0 = tid / CQ;
    const T *vp = (const T *)a.v + bh * DV + 4 * c;
    const f32x4 v = {to_f32(vp[0]), to_f32(vp[1]), to_f32(vp[2]), to_f32(vp[3])};
    const f32x4 gb = *(const f32x4 *)(a.gv + bh * DV + 4 * c);
    const f32x4 bv = {exp2_fast(gb[0] * kLog2e), exp2_fast(gb[1] * kLog2e), exp2_fast(gb[2] * kLog2e),
                      exp2_fast(gb[3] * kLog2e)};
    f32x4 *st = (f32x4 *)(a.s_final + bh * DK * DV) + c;
    f32x4 s[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) s[p] = __builtin_nontemporal_load(st + (size_t)(r0 + p * RS) * CQ);
    __syncthreads();

    f32x4 op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int i = r0 + p * RS;
        s[p] = sa[i] * (bv * s[p]) + sk[i] * v;
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

// The producer/consumer kernel where its two buffers fit in LDS, else the
// single-role kernel (fp32 with d_k = 128 and chunks of 64).
template <typename T, int DK, int C, bool ELU1>
static void launch_outer_dk(const OuterArgs &a, int grid, hipStream_t stream)
{
    if constexpr (outer_pc_lds<T, DK, C>() <= kLdsBytes)
        hipLaunchKernelGGL((outer_pc_kernel<T, DK, C, ELU1>), dim3(grid), dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL((outer_prefill_kernel<T, DK, C, ELU1>), dim3(grid), dim3(256), 0, stream, a);
}

template <typename T, int C, bool ELU1>
static hipError_t launch_outer_c(const OuterArgs &a, hipStream_t stream)
{
    const int grid = a.BH * a.n_vt;
    switch (a.d_k) {
    case 16: launch_outer_dk<T, 16, C, ELU1>(a, grid, stream); break;
    case 32: launch_outer_dk<T, 32, C, ELU1>(a, grid, stream); break;
    case 64: launch_outer_dk<T, 64, C, ELU1>(a, grid, stream); break;
    case 128: launch_outer_dk<T, 128, C, ELU1>(a, grid, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool ELU1>
static hipError_t launch_outer_t(const OuterArgs &a, int chunk, hipStream_t stream)
{
    if (chunk == 16) return launch_outer_c<T, 16, ELU1>(a, stream);
    if (chunk == 32) return launch_outer_c<T, 32, ELU1>(a, stream);
    if (chunk == 64) return launch_outer_c<T, 64, ELU1>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_outer_prefill(const OuterArgs &a, int dtype, int chunk, hipStream_t stream)
{
    if (dtype == 1) return a.elu1 ? launch_outer_t<bf16, true>(a, chunk, stream) : launch_outer_t<bf16, false>(a, chunk, stream);
    return a.elu1 ? launch_outer_t<float, true>(a, chunk, stream) : launch_outer_t<float, false>(a, chunk, stream);
}

template <typename T>
static hipError_t launch_outer_decode_t(const OuterArgs &a, hipStream_t stream)
{
#define GLA_OUTER_DECODE(DK, DV)                                                                   \
    if (a.d_k == DK && a.d_v == DV) {                                                              \
        constexpr int NT = (DK * (DV / 4)) < 256 ? (DK * (DV / 4)) : 256;                          \
        hipLaunchKernelGGL((outer_decode_kernel<T, DK, DV>), dim3(a.BH), dim3(NT), 0, stream, a);  \
        return hipGetLastError();                                                                  \
    }
#define GLA_OUTER_DECODE_DV(DK) \
    GLA_OUTER_DECODE(DK, 16) GLA_OUTER_DECODE(DK, 32) GLA_OUTER_DECODE(DK, 64) GLA_OUTER_DECODE(DK, 128)
    GLA_OUTER_DECODE_DV(16) GLA_OUTER_DECODE_DV(32) GLA_OUTER_DECODE_DV(64) GLA_OUTER_DECODE_DV(128)
#undef GLA_OUTER_DECODE_DV
#undef GLA_OUTER_DECODE
    return hipErrorInvalidValue;
}

hipError_t launch_outer_decode(const OuterArgs &a, int dtype, hipStream_t stream)
{
    if (dtype == 1) return launch_outer_decode_t<bf16>(a, stream);
    return launch_outer_decode_t<float>(a, stream);
}

}  // namespace gla
