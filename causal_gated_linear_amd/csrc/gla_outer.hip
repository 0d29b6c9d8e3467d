// gla_outer.hip -- one decode step of gated linear attention with the outer-product
// gate on gfx950.
//
// "Gated Linear Attention", section "GLA / Recurrent Form": of the general gate
// G_t (.) S_{t-1}, the low-rank parameterisation G_t = alpha_t beta_t^T decays the
// state along both dimensions:
//
//     S_t[i][j] = alpha_t[i] beta_t[j] S_{t-1}[i][j] + phi(k_t)[i] v_t[j],
//     o_t = S_t^T phi(q_t)
//
// with natural-log gates g (alpha, [d_k]) and gv (beta, [d_v]) per head.  The chunkwise
// prefill of the same gate is the prefill kernel's outer-gate mode (gla_prefill.hpp).
#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

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
