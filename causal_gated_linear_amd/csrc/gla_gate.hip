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
// Persistent workgroups (one per CU and group of 16-output tiles) walk the token
// blocks of 64 tokens with a stride of the grid.  Four reader waves compute the
// next block's rank-r codes zd^T = W_down x^T on the matrix cores, with operand
// fragments loaded straight from memory (x from HBM once, W_down from the cache),
// while four writer waves turn the current block's codes into gates: the
// up-projection z^T = W_up zd^T on the matrix cores, one 16-row tile of W_up at a
// time from the workgroup's rows of W_up staged in LDS (64 KB) at the start, then
// log-sigmoid, and stores as 16-byte row pieces, non-temporally (g is written once
// and read by a later kernel, far beyond the caches).  The codes pass through LDS,
// double-buffered, with one barrier per block.  Reading x and writing g thus overlap
// across the chip, and no wave issues both loads and stores: loads and stores share
// one in-order completion counter, so a load issued after a store would wait for
// that store's write.  The write of g (4 bytes per token and key dimension)
// dominates the traffic.
#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

namespace {

// log(sigmoid(z)) / tau = min(z, 0) / tau - log(1 + e^-|z|) / tau, with the hardware
// base-2 exp and log (c = -ln 2 / tau).  Where e^-|z| is below fp32's epsilon,
// 1 + e^-|z| rounds to 1 and the term it drops is below 6e-8 / tau in absolute value.
// min(z, 0) / tau is taken as min(z / tau, 0) (tau > 0).
__device__ __forceinline__ float log_sigmoid_scaled(float z, float inv_tau, float c)
{
    const float e = exp2_fast(-fabsf(z) * kLog2e);
    return fmaf(c, __builtin_amdgcn_logf(1.f + e), fminf(z * inv_tau, 0.f));
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

// Staged W_up rows in LDS: row r (R elements, no padding).  For bf16 the 8-byte
// pieces of a row are permuted by an even XOR of the row index, so that the 16
// lanes of one ds_read_b64 (rows x = 0..15, one piece) hit distinct banks, while
// each 16-byte piece of the staging copy stays contiguous.
template <typename T, int R>
__device__ __forceinline__ int up_off(int row, int elem)
{
    if constexpr (sizeof(T) == 2) {
        const int sw = R == 16 ? 2 * ((row >> 3) & 1) : 2 * ((row >> 2) & 3);
        return row * R + ((((elem >> 2) ^ sw)) << 2) + (elem & 3);
    } else {
        return row * R + elem;
    }
}

// Up-projection step: z = W_up[row][:] x zd over the rank (one or two 16-blocks),
// with row = 16 tile + x of the staged rows and the accumulator tiles of zd^T.  bf16
// weights: bf16 matrix-core operands (the rank-r code rounded to bf16); fp32 weights:
// fp32.
template <int R>
__device__ __forceinline__ f32x4 up_step(const bf16 *su, int row, int grp, const f32x4 *zd)
{
    const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    const f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    bf16x4 *tag = nullptr;
    const bf16x4 a0 = *(const bf16x4 *)(su + up_off<bf16, R>(row, 4 * grp));
    if constexpr (R == 16) return mma2(a0, z, frag_from_acc(tag, zd[0]), z, acc);
    else return mma2(a0, *(const bf16x4 *)(su + up_off<bf16, R>(row, 16 + 4 * grp)),
                     frag_from_acc(tag, zd[0]), frag_from_acc(tag, zd[1]), acc);
}
template <int R>
__device__ __forceinline__ f32x4 up_step(const float *su, int row, int grp, const f32x4 *zd)
{
    f32x4 acc = mma1(*(const f32x4 *)(su + up_off<float, R>(row, 4 * grp)), zd[0], f32x4{0.f, 0.f, 0.f, 0.f});
    if constexpr (R == 32) acc = mma1(*(const f32x4 *)(su + up_off<float, R>(row, 16 + 4 * grp)), zd[1], acc);
    return acc;
}

}  // namespace

template <typename T, int R>
__global__ __launch_bounds__(512) void gate_project_kernel(const GateArgs a)
{
    constexpr int ES = sizeof(T);
    constexpr int KW = 16 / ES;                    // contraction elements per lane per step
    constexpr int KSTEP = 4 * KW;                  // contraction width of one step (32 or 16)
    constexpr int NR = R / 16;                     // 16-row tiles of the rank
    constexpr int LDZ = R + 4;                     // row stride of the staged codes (floats)
    constexpr int TPG = gate_tiles_per_group(ES, R);
    typedef typename Piece<T>::type P;
    __shared__ __align__(16) T sU[TPG * 16 * R];              // the group's rows of W_up
    __shared__ __align__(16) float sZ[2][64 * LDZ];            // codes of two token blocks

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int x = lane & 15, grp = lane >> 4;
    const bool reader = w < 4;                                 // wave-uniform
    const int wr = w & 3;                                      // token rows 16 wr .. of a block
    const int og = blockIdx.y;                                 // group of 16-output tiles
    const int dm = a.d_model;
    const long ntok = (long)a.B * a.L;
    const long nblk = (ntok + 63) / 64;
    const int nk = (int)((nblk - blockIdx.x + gridDim.x - 1) / gridDim.x);   // blocks of this workgroup
    const int tile0 = og * TPG;
    const int ntile = min(a.H * a.d_k / 16, tile0 + TPG);

    // stage rows [16 tile0, 16 ntile) of W_up, 16-byte pieces, all waves
    {
        constexpr int PPU = R * ES / 16, UP = TPG * 16 * PPU / 512;
        const int npiece = 16 * (ntile - tile0) * PPU;
        const char *wsrc = (const char *)a.w_up + (size_t)16 * tile0 * R * ES;
        P gu[UP];
#pragma unroll
        for (int i = 0; i < UP; ++i) {
            const int p = tid + 512 * i;
            if (p < npiece) gu[i] = *(const P *)(wsrc + (size_t)p * 16);
        }
#pragma unroll
        for (int i = 0; i < UP; ++i) {
            const int p = tid + 512 * i, r = p / PPU;
            if (p < npiece) *(P *)(sU + up_off<T, R>(r, (p - r * PPU) * KW)) = gu[i];
        }
    }

    // Readers: rank-r codes zd[t][j] = sum_m W_down[j][m] x[t][m] of one 64-token block
    // on the matrix cores, reader wr taking tokens 16 wr .. 16 wr + 15.  Operand
    // fragments come straight from memory (x once from HBM, W_down from the cache),
    // D steps ahead of their products; pieces past d_model or past the last token read
    // as zeros through the range checks.  The accumulator tiles go to sZ[buf] in their
    // lane layout: lane (x, grp) element e of tile jt is zd[16 wr + x][16 jt + 4 grp + e].
    const Rsrc rwd = make_rsrc(a.w_down, (unsigned)(R * dm * ES));
    auto codes = [&](long blk, int buf) __attribute__((always_inline)) {
        constexpr int D = 8;
        const long tok0 = blk * 64;
        const int brows = (int)max(0L, min(64L, ntok - tok0));
        const Rsrc rx = make_rsrc((const T *)a.x + tok0 * dm, (unsigned)(brows * dm * ES));
        const int xrow = 16 * wr + x, nstep = dm / KSTEP;
        P xc[D], wc[D][NR], xn[D], wn[D][NR];
        auto load = [&](int u, P &xv, P (&wv)[NR]) __attribute__((always_inline)) {
            const int m = u * KSTEP + KW * grp;
            xv = buf_load16<P>(rx, (m < dm ? xrow * dm + m : brows * dm) * ES);
#pragma unroll
            for (int jt = 0; jt < NR; ++jt) wv[jt] = buf_load16<P>(rwd, (m < dm ? (16 * jt + x) * dm + m : R * dm) * ES);
        };
        f32x4 acc[NR];
#pragma unroll
        for (int jt = 0; jt < NR; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < D; ++i) load(i, xc[i], wc[i]);
        for (int s0 = 0; s0 < nstep; s0 += D) {
#pragma unroll
            for (int i = 0; i < D; ++i) load(s0 + D + i, xn[i], wn[i]);      // zeros past the end
#pragma unroll
            for (int i = 0; i < D; ++i)
#pragma unroll
                for (int jt = 0; jt < NR; ++jt) acc[jt] = mma_piece(wc[i][jt], xc[i], acc[jt]);
#pragma unroll
            for (int i = 0; i < D; ++i) {
                xc[i] = xn[i];
#pragma unroll
                for (int jt = 0; jt < NR; ++jt) wc[i][jt] = wn[i][jt];
            }
        }
#pragma unroll
        for (int jt = 0; jt < NR; ++jt) *(f32x4 *)(sZ[buf] + (16 * wr + x) * LDZ + 16 * jt + 4 * grp) = acc[jt];
    };

    // Writers: up-projection of one block from its staged codes, log-sigmoid, stores.
    const float inv_tau = a.inv_tau, c_log = -0.6931471805599453f * a.inv_tau;
    const size_t hstride = (size_t)a.L * a.d_k;
    const bool pairable = a.d_k >= 32;                         // both tiles of a pair in one head
    const bool lo = x < 8;
    auto gates = [&](const f32x4 &z) __attribute__((always_inline)) -> f32x4 {
        // lane (x, grp) element e: z[t = row0 + x][n = 16 tile + 4 grp + e]
        f32x4 g;
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = log_sigmoid_scaled(z[e], inv_tau, c_log);
        return g;
    };
    auto outputs = [&](long blk, int buf) __attribute__((always_inline)) {
        const long row0 = blk * 64 + 16 * wr;                  // this wave's first token
        const int nrows = (int)max(0L, min(16L, ntok - row0));
        if (nrows == 0) return;                                // wave-uniform
        f32x4 zd[NR];
#pragma unroll
        for (int jt = 0; jt < NR; ++jt) zd[jt] = *(const f32x4 *)(sZ[buf] + (16 * wr + x) * LDZ + 16 * jt + 4 * grp);
        const long tok = row0 + x;
        const long b = tok / a.L, l = tok - b * a.L;
        const bool store = x < nrows;
        float *gt = a.g + ((size_t)b * a.H * a.L + l) * a.d_k;    // g[b][0][l][0]
        // Two adjacent tiles of one head cover 128 bytes of each token's row.  Lanes x
        // and x ^ 8 swap their second tile's values, so that each store instruction
        // writes whole 128-byte row pieces of 8 tokens (half-line non-temporal writes
        // cost extra HBM traffic): the first store holds tokens 0..7 of the wave, the
        // second 8..15.
        const long tok8 = row0 + (x ^ 8);
        const long b8 = tok8 / a.L, l8 = tok8 - b8 * a.L;
        float *gt8 = a.g + ((size_t)b8 * a.H * a.L + l8) * a.d_k;   // row of token x ^ 8
        const bool store_a = (x & 7) < nrows, store_b = (x & 7) + 8 < nrows;
        for (int t0 = tile0; t0 < ntile; t0 += 8) {
            // the batch's 8 products first (tile index clamped to the staged rows), so
            // that their LDS reads and matrix-core latencies overlap
            f32x4 zz[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) zz[u] = up_step<R>(sU, 16 * (min(t0 + u, ntile - 1) - tile0) + x, grp, zd);
#pragma unroll
            for (int u = 0; u < 8; u += 2) {
                if (t0 + u >= ntile) break;                        // wave-uniform
                const int n0 = 16 * (t0 + u) + 4 * grp, h0 = n0 >> a.dk_shift, i0 = n0 & (a.d_k - 1);
                const f32x4 g0 = gates(zz[u]);
                if (!pairable || t0 + u + 1 >= ntile) {            // wave-uniform
                    if (store) __builtin_nontemporal_store(g0, (f32x4 *)(gt + h0 * hstride + i0));
                    if (t0 + u + 1 < ntile) {
                        const int n1 = n0 + 16, h1 = n1 >> a.dk_shift, i1 = n1 & (a.d_k - 1);
                        const f32x4 g1 = gates(zz[u + 1]);
                        if (store) __builtin_nontemporal_store(g1, (f32x4 *)(gt + h1 * hstride + i1));
                    }
                    continue;
                }
                const f32x4 g1 = gates(zz[u + 1]);
                f32x4 r;                                           // tile u+1 of token x ^ 8
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = __shfl_xor(g1[e], 8, 64);
                float *own = gt + h0 * hstride + i0;               // token x, tile u
                float *oth = gt8 + h0 * hstride + i0 + 16;         // token x ^ 8, tile u+1
                if (store_a) __builtin_nontemporal_store(lo ? g0 : r, (f32x4 *)(lo ? own : oth));
                if (store_b) __builtin_nontemporal_store(lo ? r : g0, (f32x4 *)(lo ? oth : own));
            }
        }
    };

    // Blocks blockIdx.x + k gridDim.x, k < nk: the readers compute block k + 1's codes
    // while the writers emit block k's gates; one barrier per block hands over the
    // codes and frees their buffer.
    if (reader) codes(blockIdx.x, 0);
    __syncthreads();                                           // W_up staged, first codes ready
    for (int k = 0; k < nk; ++k) {
        if (reader) {
            if (k + 1 < nk) codes(blockIdx.x + (long)(k + 1) * gridDim.x, (k + 1) & 1);
        } else {
            outputs(blockIdx.x + (long)k * gridDim.x, k & 1);
        }
        __syncthreads();
    }
}

hipError_t launch_gate_project(const GateArgs &a, int dtype, int rank, hipStream_t stream)
{
    const long ntok = (long)a.B * a.L;
    const long nblk = (ntok + 63) / 64;
    if (nblk == 0) return hipSuccess;
    const int ntile = a.H * a.d_k / 16, tpg = gate_tiles_per_group(dtype == 1 ? 2 : 4, rank);
    // persistent workgroups, one per CU and group of output tiles, each walking the
    // token blocks with a stride of the grid
    const dim3 g2((unsigned)min(nblk, 256L), (ntile + tpg - 1) / tpg);
#define GLA_GATE_LAUNCH(T, R) \
    hipLaunchKernelGGL((gate_project_kernel<T, R>), g2, dim3(512), 0, stream, a)
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
