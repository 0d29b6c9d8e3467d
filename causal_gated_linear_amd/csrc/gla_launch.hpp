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

// Prefill launch shape: value columns per workgroup (16, 32 or 64) and waves per
// workgroup (4, or 8 with 64 columns and d_k >= 32).
struct PrefillTile {
    int dvt, nw;
};
PrefillTile prefill_tile(int BH, int d_k, int d_v);

// Enqueue the prefill kernel.  dtype: 0 fp32, 1 bf16.  Sizes must already be valid.
hipError_t launch_prefill(const PrefillArgs &a, int dtype, int d_k, int chunk, PrefillTile tile,
                          hipStream_t stream);

// Enqueue one decode step.  Sizes must already be valid.
hipError_t launch_decode(const DecodeArgs &a, int dtype, int d_k, int d_v, hipStream_t stream);

}  // namespace gla
