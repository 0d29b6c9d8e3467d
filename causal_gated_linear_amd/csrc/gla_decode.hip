// gla_decode.hip -- one token of the gated recurrence on a resident fp32 state.
//
// "Attention is recurrent", Linear attention / Gated linear attention: the output
// of token n depends only on the cached state S_{n-1} and token n's q, k, v and
// gate; "Gated Linear Attention", Recurrent Form: S_t = Diag(alpha_t) S_{t-1} +
// (key-value outer product), then the read-out with q.  Per head:
//     S[i][:] <- alpha_i * S[i][:] + phi(k)_i * v        (in place)
//     o[j]     = sum_i phi(q)_i * S[i][j]
//
// The step is bound by HBM: every state element is read and written once
// (8 bytes per 5 flops).  One workgroup per head; a thread owns a float4 column
// group and every RS-th row, issues all of its state loads before using any
// (the row loop is fully unrolled), and the column partial sums of o are reduced
// across rows through LDS.  Row accesses are contiguous 16-byte vectors, and the
// state's loads and stores are non-temporal: the state of a step is touched once
// and is far larger than the caches, so keeping it out of them leaves the memory
// path to the stream (15 % faster at the decode workload's size).
//
// Normalised form ("Transformers are RNNs" notes, numerator over denominator): the
// normaliser state z, the state of a value that is 1 in every token, is updated in
// place beside S, z_i <- alpha_i z_i + phi(k)_i, and o is divided by phi(q) . z.
#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

template <typename T, int DK, int DV, bool NM>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a)
{
    constexpr int CQ = DV / 4;                               // float4 groups per row
    constexpr int NT = (DK * CQ) < 256 ? (DK * CQ) : 256;    // threads
    constexpr int RS = NT / CQ;                              // rows per pass
    constexpr int NPASS = DK / RS;
    static_assert(NT >= DK && NT >= DV && DK % RS == 0, "decode mapping");

    __shared__ float sq[DK], sk[DK], sa[DK];
    __shared__ f32x4 sred[RS][CQ];
    __shared__ float sden[NM ? DK : 1];

    const int tid = threadIdx.x;
    const size_t bh = blockIdx.x;
    const bool elu1 = a.elu1 != 0;

    if (tid < DK) {
        const T *q = (const T *)a.q + bh * DK;
        const T *k = (const T *)a.k + bh * DK;
        sq[tid] = feature(to_f32(q[tid]), elu1);
        sk[tid] = feature(to_f32(k[tid]), elu1);
        float al = 1.f;
        if (a.gate == kGateKeydim) al = exp2_fast(a.g[bh * DK + tid] * kLog2e);
        else if (a.gate == kGateScalar) al = exp2_fast(a.g[bh] * kLog2e);
        sa[tid] = al;
        if constexpr (NM) {                        // z_i <- alpha_i z_i + phi(k)_i; q~_i z_i
            float *zp = a.z + bh * DK + tid;
            const float z = al * *zp + sk[tid];
            *zp = z;
            sden[tid] = sq[tid] * z;
        }
    }

    const int c = tid % CQ, r0 = tid / CQ;
    const T *vp = (const T *)a.v + bh * DV + 4 * c;
    const f32x4 v = {to_f32(vp[0]), to_f32(vp[1]), to_f32(vp[2]), to_f32(vp[3])};
    f32x4 *st = (f32x4 *)(a.state + bh * DK * DV) + c;
    f32x4 s[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) s[p] = __builtin_nontemporal_load(st + (size_t)(r0 + p * RS) * CQ);
    __syncthreads();

    f32x4 op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int i = r0 + p * RS;
        s[p] = sa[i] * s[p] + sk[i] * v;
        __builtin_nontemporal_store(s[p], st + (size_t)i * CQ);
        op += sq[i] * s[p];
    }
    sred[r0][c] = op;
    __syncthreads();

    if (tid < CQ) {
        f32x4 acc = sred[0][tid];
#pragma unroll
        for (int r = 1; r < RS; ++r) acc += sred[r][tid];
        if constexpr (NM) {
            float den = 0.f;
            for (int i = 0; i < DK; ++i) den += sden[i];
            acc *= 1.f / den;
        }
        store4((T *)a.o + bh * DV + 4 * tid, acc);
    }
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_inst(const DecodeArgs &a, hipStream_t stream)
{
    constexpr int CQ = DV / 4;
    constexpr int NT = (DK * CQ) < 256 ? (DK * CQ) : 256;
    if (a.z) hipLaunchKernelGGL((decode_kernel<T, DK, DV, true>), dim3(a.BH), dim3(NT), 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<T, DK, DV, false>), dim3(a.BH), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_t(const DecodeArgs &a, int d_k, int d_v, hipStream_t stream)
{
#define GLA_DV_CASES(DK)                                                            \
    if (d_k == DK) {                                                                \
        if (d_v == 16) return launch_decode_inst<T, DK, 16>(a, stream);             \
        if (d_v == 32) return launch_decode_inst<T, DK, 32>(a, stream);             \
        if (d_v == 64) return launch_decode_inst<T, DK, 64>(a, stream);             \
        if (d_v == 128) return launch_decode_inst<T, DK, 128>(a, stream);           \
    }
    GLA_DV_CASES(16) GLA_DV_CASES(32) GLA_DV_CASES(64) GLA_DV_CASES(128)
#undef GLA_DV_CASES
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, int d_k, int d_v, hipStream_t stream)
{
    if (dtype == 1) return launch_decode_t<bf16>(a, d_k, d_v, stream);
    return launch_decode_t<float>(a, d_k, d_v, stream);
}

}  // namespace gla
