// gla_device.hpp -- device-side building blocks for the gfx950 kernels:
// vector types, bf16 conversion, exp2, the elu+1 feature map and the matrix-core
// (MFMA) contraction helpers.
//
// Fragment convention used by every contraction in this library.  For a 16x16
// output tile computed by one wavefront, lane l has x = l % 16 and grp = l / 16.
//  * Operand fragments: along the contraction index, cut into 16-wide blocks,
//    lane (x, grp) supplies elements [16*blk + 4*grp, 16*blk + 4*grp + 3] of row x
//    of the left operand (and of column x of the right operand).
//  * Accumulators (the MFMA "C/D" layout): lane (x, grp) holds rows
//    4*grp .. 4*grp+3 of column x.
// A 16x16 accumulator tile therefore already *is* an operand fragment for a
// contraction over its row index, which lets results (attention scores, the
// state) feed the next product from registers.  bf16 instructions consume two
// 16-blocks at once (8 values per lane), fp32 ones a single value per lane; both
// sides of a product always enumerate the contraction index the same way, so
// the hardware's internal k ordering does not matter.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// phi(x) = elu(x) + 1 (elu's alpha = 1): x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float feature(float x, bool elu1)
{
    if (!elu1) return x;
    return x > 0.f ? x + 1.f : exp2_fast(x * kLog2e);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Two consecutive elements of T, loaded as one access and widened to fp32.
__device__ __forceinline__ f32x2 load2(const float *p) { return *(const f32x2 *)p; }
__device__ __forceinline__ f32x2 load2(const bf16 *p)
{
    bf16x2 v = *(const bf16x2 *)p;
    return f32x2{(float)v[0], (float)v[1]};
}

// Four consecutive elements stored from fp32 (vector store of 8 or 16 bytes).
__device__ __forceinline__ void store4(float *p, f32x4 v) { *(f32x4 *)p = v; }
__device__ __forceinline__ void store4(bf16 *p, f32x4 v)
{
    *(bf16x4 *)p = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

template <typename E> struct Frag;                                  // 4 operand values per lane
template <> struct Frag<bf16> { typedef bf16x4 type; };
template <> struct Frag<float> { typedef f32x4 type; };

template <typename E>
__device__ __forceinline__ typename Frag<E>::type lds_frag(const E *row, int blk, int grp)
{
    return *(const typename Frag<E>::type *)(row + 16 * blk + 4 * grp);
}

__device__ __forceinline__ bf16x4 frag_from_acc(bf16x4 *, f32x4 a)
{
    return bf16x4{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
}
__device__ __forceinline__ f32x4 frag_from_acc(f32x4 *, f32x4 a) { return a; }

// acc += A(16 x 32) * B(32 x 16) for two 16-blocks of the contraction index.
__device__ __forceinline__ f32x4 mma2(bf16x4 a0, bf16x4 a1, bf16x4 b0, bf16x4 b1, f32x4 acc)
{
    bf16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    bf16x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// acc += A(16 x 16) * B(16 x 16), one 16-block of the contraction index, fp32.
__device__ __forceinline__ f32x4 mma1(f32x4 a, f32x4 b, f32x4 acc)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
}

// acc += sum over 16-blocks blk in [0, nblk) of A[x][blk] * B[x][blk], with A and B
// given as LDS rows (row x of each operand for this lane).  bf16 pairs blocks; an
// odd last block is paired with zeros.
template <typename E>
__device__ __forceinline__ f32x4 contract_rows(const E *arow, const E *brow, int nblk, int grp,
                                               f32x4 acc)
{
    if constexpr (sizeof(E) == 2) {
        const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
        int blk = 0;
        for (; blk + 1 < nblk; blk += 2)
            acc = mma2(lds_frag(arow, blk, grp), lds_frag(arow, blk + 1, grp),
                       lds_frag(brow, blk, grp), lds_frag(brow, blk + 1, grp), acc);
        if (blk < nblk)
            acc = mma2(lds_frag(arow, blk, grp), z, lds_frag(brow, blk, grp), z, acc);
    } else {
        for (int blk = 0; blk < nblk; ++blk)
            acc = mma1(lds_frag(arow, blk, grp), lds_frag(brow, blk, grp), acc);
    }
    return acc;
}

// Same, with the left operand given as accumulator tiles held in registers
// (tile blk holds the 16-block blk of the contraction index), e.g. a state
// S[i][j] whose tiles are S^T fragments for a contraction over i.
template <typename E, int NBLK>
__device__ __forceinline__ f32x4 contract_regs_rows(const f32x4 (&atiles)[NBLK], const E *brow,
                                                    int grp, f32x4 acc)
{
    if constexpr (sizeof(E) == 2) {
        bf16x4 *tag = nullptr;
        const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
#pragma unroll
        for (int blk = 0; blk < NBLK; blk += 2) {
            if (blk + 1 < NBLK)
                acc = mma2(frag_from_acc(tag, atiles[blk]), frag_from_acc(tag, atiles[blk + 1]),
                           lds_frag(brow, blk, grp), lds_frag(brow, blk + 1, grp), acc);
            else
                acc = mma2(frag_from_acc(tag, atiles[blk]), z, lds_frag(brow, blk, grp), z, acc);
        }
    } else {
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) acc = mma1(atiles[blk], lds_frag(brow, blk, grp), acc);
    }
    return acc;
}

// Barrier for LDS communication only: waits for this wave's LDS operations, not
// for its outstanding global loads.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Transposed operand reads from row-major LDS arrays (rows = tokens s, columns =
// i or j), for the products that contract over tokens.  One ds_read_b64_tr_b16
// serves a 16-lane group: lane l of the group gives the address of row s0 + l/4,
// columns n0 + 4(l%4) .. +3, and receives column n0 + l of rows s0 .. s0+3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16 *p)
{
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// Raw buffer access over `bytes` bytes from p: a load at a byte offset at or past
// `bytes` returns zeros and touches no memory.  Rows past the end of a sequence
// therefore read as zero q, k, v and zero log-gates.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void *p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
template <typename V>
__device__ __forceinline__ V buf_load16(Rsrc r, int off)
{
    static_assert(sizeof(V) == 16, "16-byte load");
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load4(Rsrc r, int off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// one load of sizeof(V) bytes (8 or 16)
template <typename V>
__device__ __forceinline__ V buf_load(Rsrc r, int off)
{
    static_assert(sizeof(V) == 8 || sizeof(V) == 16, "8- or 16-byte load");
    if constexpr (sizeof(V) == 16) return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    else return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Minimum over the 64 lanes (all active), in registers only: DPP shifts within each
// 16-lane row (a lane whose source is outside the row keeps its own value), then the
// rows' last lanes read as scalars.
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


// Accumulator tile -> operand fragment of element type T (bf16 rounds to nearest even).
template <typename T> __device__ __forceinline__ typename Frag<T>::type cvt4(f32x4 v)
{
    typename Frag<T>::type *tag = nullptr;
    return frag_from_acc(tag, v);
}
__device__ __forceinline__ f32x4 widen4(bf16x4 v) { return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }
__device__ __forceinline__ f32x4 widen4(f32x4 v) { return v; }

// acc += A B over one 16-block (mac1) or two 16-blocks (mac2) of the contraction index
__device__ __forceinline__ f32x4 mac1(bf16x4 a, bf16x4 b, f32x4 acc)
{
    const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    return mma2(a, z, b, z, acc);
}
__device__ __forceinline__ f32x4 mac1(f32x4 a, f32x4 b, f32x4 acc) { return mma1(a, b, acc); }
__device__ __forceinline__ f32x4 mac2(bf16x4 a0, bf16x4 a1, bf16x4 b0, bf16x4 b1, f32x4 acc)
{
    return mma2(a0, a1, b0, b1, acc);
}
__device__ __forceinline__ f32x4 mac2(f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1, f32x4 acc)
{
    return mma1(a1, b1, mma1(a0, b0, acc));
}

// Fragment of a column of a row-major LDS array: lane (x, grp) receives
// base[(s0 + e) * ld + c0 + x], e = 0..3, where s0 already includes 4 * grp.
__device__ __forceinline__ bf16x4 col_frag(const bf16 *base, int ld, int s0, int c0, int x)
{
    return lds_read_tr16(base + (s0 + (x >> 2)) * ld + c0 + 4 * (x & 3));
}
__device__ __forceinline__ f32x4 col_frag(const float *base, int ld, int s0, int c0, int x)
{
    const float *p = base + s0 * ld + c0 + x;
    return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

}  // namespace gla
