// gla_gate.hip -- the input-side gate producer on gfx950.
//
// "Gated Linear Attention", section "GLA / Recurrent Form" and its flow chart: the
// key-dimension gate of token t is alpha_t = sigmoid(W_up W_down x_t), a low-rank
// map from the token's input x_t (d_model) down to r dimensions and up to one value
// per key dimension of every head.  The prefill takes natural-log gates, so this
// kernel writes
//
//     g[b][h][t][i] = log(sigmoid(z_t[h d_k + i])) / tau,   z_t = W_up (W_down x_t)
//
// straight into the prefill's [B][H][L][d_k] layout.
//
// One workgroup per 64 tokens (16 per wave) and group of 16-output tiles.  Each
// wave first computes its tokens' rank-r codes zd^T = W_down x^T on the matrix
// cores, from x and W_down row chunks that the workgroup stages in LDS with
// row-contiguous loads (x comes from HBM once; W_down stays in cache).  The
// accumulator tiles of zd^T are then, unchanged, the right operand of the
// up-projection z^T = W_up zd^T, which runs on the matrix cores one 16-row tile of
// W_up at a time; each tile's outputs go through log-sigmoid and are stored
// as 16-byte row pieces, non-temporally (g is written once and read by a later
// kernel, far beyond the caches).  The write of g (4 bytes per token and key
// dimension) dominates the traffic.
#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

namespace {

// log(sigmoid(z)) = min(z, 0) - log(1 + e^-|z|), with the hardware base-2 exp and
// log.  Where e^-|z| is below fp32's epsilon, 1 + e^-|z| rounds to 1 and the term it
// drops is below 6e-8 in absolute value.
__device__ __forceinline__ float log_sigmoid(float z)
{
    constexpr float kLn2 = 0.6931471805599453f;
    const float e = exp2_fast(-fabsf(z) * kLog2e);
    return fminf(z, 0.f) - __builtin_amdgcn_logf(1.f + e) * kLn2;
}

// 16-byte operand piece: 8 bf16 or 4 fp32 consecutive elements of a row.
template <typename T> struct Piece;
template <> struct Piece<bf16> { typedef bf16x8 type; };
template <> struct Piece<float> { typedef f32x4 type; };

__device__ __forceinline__ f32x4 mma_piece(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_piece(f32x4 a, f32x4 b, f32x4 c) { return mma1(a, b, c); }

// Up-projection step: z += W_up[n][4 grp + e, 16 + 4 grp + e] x zd over one or two
// 16-blocks of the rank, from the accumulator tiles of zd^T.  bf16 weights: bf16
// matrix-core operands (the rank-r code rounded to bf16); fp32 weights: fp32.
__device__ __forceinline__ f32x4 up_step(const bf16 *w, const f32x4 *zd, int nr, f32x4 acc)
{
    const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    bf16x4 *tag = nullptr;
    const bf16x4 a0 = *(const bf16x4 *)w;
    if (nr == 1) return mma2(a0, z, frag_from_acc(tag, zd[0]), z, acc);
    return mma2(a0, *(const bf16x4 *)(w + 16), frag_from_acc(tag, zd[0]), frag_from_acc(tag, zd[1]), acc);
}
__device__ __forceinline__ f32x4 up_step(const float *w, const f32x4 *zd, int nr, f32x4 acc)
{
    acc = mma1(*(const f32x4 *)w, zd[0], acc);
    if (nr == 2) acc = mma1(*(const f32x4 *)(w + 16), zd[1], acc);
    return acc;
}

}  // namespace

template <typename T, int R>
__global__ __launch_bounds__(256) void gate_project_kernel(const GateArgs a)
{
    constexpr int ES = sizeof(T);
    constexpr int KW = 16 / ES;                    // contraction elements per lane per step
    constexpr int KSTEP = 4 * KW;                  // contraction width of one step (32 or 16)
    constexpr int NR = R / 16;                     // 16-row tiles of the rank
    typedef typename Piece<T>::type P;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int x = lane & 15, grp = lane >> 4;
    const long row0 = (long)blockIdx.x * 64 + 16 * w;        // this wave's first token
    const int og = blockIdx.y;                                 // group of 16-output tiles
    const int dm = a.d_model;
    const long ntok = (long)a.B * a.L;
    const int nrows = (int)max(0L, min(16L, ntok - row0));  // 0 for idle waves of the last block

    // down-projection: zd^T[j][t] = sum_m W_down[j][m] x[t][m]; lane (x, grp) element e
    // of tile jt holds zd[t = row0 + x][j = 16 jt + 4 grp + e].
    // The contraction runs in chunks of MB columns (512 bytes of a row).  The
    // workgroup stages the chunk of its 64 tokens' x rows and of W_down in LDS, each
    // 32 lanes reading one 512-byte row piece; the next chunk is requested into
    // registers before the current one is multiplied.  Pieces past d_model (or past
    // the last token) read as zeros through the range checks.
    constexpr int MB = 512 / ES, LDX = MB + KW, NU = MB / KSTEP;
    constexpr int PPR = MB / KW;                               // 16-byte pieces per row chunk
    constexpr int XP = 64 * PPR / 256, WP = (R * PPR + 255) / 256;
    __shared__ __align__(16) T sX[64 * LDX];
    __shared__ __align__(16) T sW[R * LDX];
    const long tok0 = (long)blockIdx.x * 64;
    const int brows = (int)max(0L, min(64L, ntok - tok0));
    const Rsrc rx = make_rsrc((const T *)a.x + tok0 * dm, (unsigned)(brows * dm * ES));
    const Rsrc rwd = make_rsrc(a.w_down, (unsigned)(R * dm * ES));
    const int tid = threadIdx.x;
    P gx[XP], gw[WP];
    auto fetch = [&](int m0) {
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = tid + 256 * i, r = p / PPR, c = m0 + (p - r * PPR) * KW;
            gx[i] = buf_load16<P>(rx, (c < dm ? r * dm + c : brows * dm) * ES);
        }
#pragma unroll
        for (int i = 0; i < WP; ++i) {
            const int p = tid + 256 * i, r = p / PPR, c = m0 + (p - r * PPR) * KW;
            if (R * PPR % 256 == 0 || p < R * PPR) gw[i] = buf_load16<P>(rwd, (c < dm ? r * dm + c : R * dm) * ES);
        }
    };
    f32x4 zd[NR];
#pragma unroll
    for (int jt = 0; jt < NR; ++jt) zd[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    fetch(0);
    for (int m0 = 0; m0 < dm; m0 += MB) {
        __syncthreads();                                       // previous chunk consumed
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = tid + 256 * i, r = p / PPR;
            *(P *)(sX + r * LDX + (p - r * PPR) * KW) = gx[i];
        }
#pragma unroll
        for (int i = 0; i < WP; ++i) {
            const int p = tid + 256 * i, r = p / PPR;
            if (R * PPR % 256 == 0 || p < R * PPR) *(P *)(sW + r * LDX + (p - r * PPR) * KW) = gw[i];
        }
        __syncthreads();
        fetch(m0 + MB);                                        // past the end: zeros, unused
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const P xb = *(const P *)(sX + (16 * w + x) * LDX + u * KSTEP + KW * grp);
#pragma unroll
            for (int jt = 0; jt < NR; ++jt)
                zd[jt] = mma_piece(*(const P *)(sW + (16 * jt + x) * LDX + u * KSTEP + KW * grp), xb, zd[jt]);
        }
    }

    if (nrows == 0) return;                                    // wave-uniform; no barrier follows

    // up-projection per 16-row tile of W_up (outputs n), then log-sigmoid and store;
    // batches of NV tiles request their W_up fragments before the first product
    const int ntile = min(a.H * a.d_k / 16, (og + 1) * a.tiles_per_group);
    const T *wu = (const T *)a.w_up;
    const float inv_tau = a.inv_tau;
    const long tok = row0 + x;
    const long b = tok / a.L, l = tok - b * a.L;
    const bool store = x < nrows;
    float *gt = a.g + ((size_t)b * a.H * a.L + l) * a.d_k;    // g[b][0][l][0]
    const size_t hstride = (size_t)a.L * a.d_k;
    // Two adjacent tiles of one head cover 128 bytes of each token's row.  Lanes x and
    // x ^ 8 swap their second tile's values, so that each store instruction writes
    // whole 128-byte row pieces of 8 tokens (half-line non-temporal writes cost extra
    // HBM traffic): the first store holds tokens 0..7 of the wave, the second 8..15.
    const bool pairable = a.d_k >= 32;                         // both tiles in one head
    const long tok8 = row0 + (x ^ 8);
    const long b8 = tok8 / a.L, l8 = tok8 - b8 * a.L;
    float *gt8 = a.g + ((size_t)b8 * a.H * a.L + l8) * a.d_k;   // row of token x ^ 8
    const bool lo = x < 8;
    const bool store_a = (x & 7) < nrows, store_b = (x & 7) + 8 < nrows;
    auto tile_gates = [&](int tile) __attribute__((always_inline)) -> f32x4 {
        const f32x4 z = up_step(wu + (size_t)(16 * tile + x) * R + 4 * grp, zd, NR, f32x4{0.f, 0.f, 0.f, 0.f});
        // lane (x, grp) element e: z[t = row0 + x][n = 16 tile + 4 grp + e]
        f32x4 g;
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = log_sigmoid(z[e]) * inv_tau;
        return g;
    };
    for (int t0 = og * a.tiles_per_group; t0 < ntile; t0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
            if (t0 + u >= ntile) break;                            // wave-uniform
            const int n0 = 16 * (t0 + u) + 4 * grp, h0 = n0 >> a.dk_shift, i0 = n0 & (a.d_k - 1);
            const f32x4 g0 = tile_gates(t0 + u);
            if (!pairable || t0 + u + 1 >= ntile) {                // wave-uniform
                if (store) __builtin_nontemporal_store(g0, (f32x4 *)(gt + h0 * hstride + i0));
                if (t0 + u + 1 < ntile) {
                    const int n1 = n0 + 16, h1 = n1 >> a.dk_shift, i1 = n1 & (a.d_k - 1);
                    const f32x4 g1 = tile_gates(t0 + u + 1);
                    if (store) __builtin_nontemporal_store(g1, (f32x4 *)(gt + h1 * hstride + i1));
                }
                continue;
            }
            const f32x4 g1 = tile_gates(t0 + u + 1);
            f32x4 r;                                               // tile u+1 of token x ^ 8
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = __shfl_xor(g1[e], 8, 64);
            float *own = gt + h0 * hstride + i0;                   // token x, tile u
            float *oth = gt8 + h0 * hstride + i0 + 16;             // token x ^ 8, tile u+1
            if (store_a) __builtin_nontemporal_store(lo ? g0 : r, (f32x4 *)(lo ? own : oth));
            if (store_b) __builtin_nontemporal_store(lo ? r : g0, (f32x4 *)(lo ? oth : own));
        }
    }
}

hipError_t launch_gate_project(const GateArgs &a, int dtype, int rank, hipStream_t stream)
{
    const long ntok = (long)a.B * a.L;
    const unsigned grid = (unsigned)((ntok + 63) / 64);
    if (grid == 0) return hipSuccess;
    const int ntile = a.H * a.d_k / 16;
    const dim3 g2(grid, (ntile + a.tiles_per_group - 1) / a.tiles_per_group);
#define GLA_GATE_LAUNCH(T, R) \
    hipLaunchKernelGGL((gate_project_kernel<T, R>), g2, dim3(256), 0, stream, a)
    if (dtype == 1) {
        if (rank == 16) GLA_GATE_LAUNCH(bf16, 16);
        else if (rank == 32) GLA_GATE_LAUNCH(bf16, 32);
        else return hipErrorInvalidValue;
    } else {
        if (rank == 16) GLA_GATE_LAUNCH(float, 16);
        else if (rank == 32) GLA_GATE_LAUNCH(float, 32);
        else return hipErrorInvalidValue;
    }
#undef GLA_GATE_LAUNCH
    return hipGetLastError();
}

}  // namespace gla
