// gla_launch.hpp -- internal interface between the C ABI (gla_api.cpp) and the
// kernel translation units.  Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

enum { kGateNone = 0, kGateKeydim = 1, kGateScalar = 2 };

struct PrefillArgs {
    const void *q, *k, *v;   // [B][H][L][d_k] / [B][H][L][d_v], element type T
    const float *g;          // log-gates (natural log), layout per gate mode, or null
    const float *s0;         // [B][H][d_k][d_v] or null
    void *o;                 // [B][H][L][d_v], T
    float *s_final;          // [B][H][d_k][d_v] or null
    int BH, L, d_v;
    int gate, elu1;
    int n_vt;                // value-column tiles per head (d_v / tile width)
    int xcd_remap;           // 1: map workgroups so a head's tiles share one XCD
};

struct DecodeArgs {
    const void *q, *k, *v;   // [B][H][d_k] / [B][H][d_v], element type T
    const float *g;          // [B][H][d_k] / [B][H] / null
    float *state;            // [B][H][d_k][d_v], in/out
    void *o;                 // [B][H][d_v], T
    int BH;
    int gate, elu1;
};

// LDS bytes of a prefill workgroup (an upper bound, alignment included): `nbuf`
// operand buffers (Q~ and K^ rows of length d_k, V rows of length dvt, exp(Gamma)
// and the scalar-gate sums), the two parity copies of the state operand, and the
// output staging rows of the consumer waves (at most 4 x 16 x dvt).
constexpr int kLdsBytes = 163840;                  // LDS per compute unit on gfx950
constexpr int prefill_lds_bytes(int es, int dk, int c, int dvt, int nbuf)
{
    const int buf = (2 * c * dk + dvt * c) * es + 4 * (dk + c + 4);
    return nbuf * buf + 2 * dvt * dk * es + 4 * 16 * dvt * es + 128;
}
// Operand buffers that fit (2: producer/consumer overlap, 1: alternating, 0: none).
constexpr int prefill_nbuf(int es, int dk, int c, int dvt)
{
    return prefill_lds_bytes(es, dk, c, dvt, 2) <= kLdsBytes ? 2
           : prefill_lds_bytes(es, dk, c, dvt, 1) <= kLdsBytes ? 1 : 0;
}

// Value columns per prefill workgroup (16, 32 or 64) for these sizes.
int prefill_tile(int BH, int d_k, int d_v, int chunk, int elem_bytes);

// Enqueue the prefill kernel.  dtype: 0 fp32, 1 bf16.  Sizes must already be valid.
hipError_t launch_prefill(const PrefillArgs &a, int dtype, int d_k, int chunk, int dvt,
                          hipStream_t stream);

// Enqueue one decode step.  Sizes must already be valid.
hipError_t launch_decode(const DecodeArgs &a, int dtype, int d_k, int d_v, hipStream_t stream);

}  // namespace gla
