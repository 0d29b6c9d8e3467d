// gla_launch.hpp -- internal interface between the C ABI (gla_api.cpp) and the
// kernel translation units.  Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

// gate modes of the prefill kernel: none, key-dimension gates, one scalar gate per
// token, and the outer-product gate (key-dimension gates g and value-dimension gates
// gv, the latter only through gla_prefill_outer)
enum { kGateNone = 0, kGateKeydim = 1, kGateScalar = 2, kGateOuter = 3 };

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
    // sequence segments: workgroup (head, segment, tile) covers rows
    // [seg * seg_len, min(L, (seg + 1) * seg_len)) of its head; s0 and s_final are
    // then indexed [BH][nseg][d_k][d_v].  nseg = 1, seg_len = L: whole sequences.
    int nseg, seg_len;
    float *gam;              // state-only pass: segment totals of the log2-gates [BH][nseg][d_k]
    // 1: only the last segment's workgroups store their final state, into s_final
    // indexed [BH][d_k][d_v] (the full pass of a segmented prefill)
    int final_last_seg = 0;
    // normalised form: outputs divided by phi(q) . z, z the normaliser state
    int norm;
    const float *z0;         // [B][H][d_k] or null
    float *z_final;          // [B][H][d_k] or null
    // outer-product gate: value-dimension log-gates (natural log) [B][H][L][d_v]
    const float *gv = nullptr;
    // full pass of a segmented prefill: the states from zero of the pieces that cover
    // segments 0 .. nseg-2, seg_sub equal pieces per segment ([BH][(nseg - 1) seg_sub]
    // [d_k][d_v]), and their log2 gate totals ([BH][(nseg - 1) seg_sub][d_k], null
    // without gates); each workgroup scans the pieces before its segment into its
    // initial state, and s0 is then the sequence's own initial state [BH][d_k][d_v]
    // (or null)
    const float *seg_ds = nullptr, *seg_gam = nullptr;
    int seg_sub = 1;
};

struct DecodeArgs {
    const void *q, *k, *v;   // [B][H][d_k] / [B][H][d_v], element type T
    const float *g;          // [B][H][d_k] / [B][H] / null
    float *state;            // [B][H][d_k][d_v], in/out
    void *o;                 // [B][H][d_v], T
    int BH;
    int gate, elu1;
    float *z;                // normalised form: [B][H][d_k], in/out; null otherwise
};

// LDS bytes of a prefill workgroup (an upper bound, alignment included): `nbuf`
// operand buffers (Q~ and K^ rows of length d_k, the scalar gate's K~ rows, V rows
// of length dvt, exp(Gamma) and the scalar-gate sums), the two parity copies of the
// state operand, and the output staging rows of the consumer waves (at most
// 4 x 16 x dvt).
constexpr int kLdsBytes = 163840;                  // LDS per compute unit on gfx950
// The outer-product gate has no K~ rows but adds, per buffer, exp(Bv) for every
// (row, value column) in fp32 rows of dvt + 4, exp of the value-side chunk totals and
// the producers' gate minima.
constexpr int prefill_lds_bytes(int es, int dk, int c, int dvt, int nbuf, bool outer = false)
{
    const int buf = outer ? (2 * c * dk + dvt * c) * es + 4 * (dk + c + 4) + 4 * (c * (dvt + 4) + dvt + 8)
                          : (3 * c * dk + dvt * c) * es + 4 * (dk + c + 4);
    return nbuf * buf + 2 * dvt * dk * es + 4 * 16 * dvt * es + 128;
}
// Operand buffers that fit (2: producer/consumer overlap, 1: alternating, 0: none).
constexpr int prefill_nbuf(int es, int dk, int c, int dvt, bool outer = false)
{
    return prefill_lds_bytes(es, dk, c, dvt, 2, outer) <= kLdsBytes ? 2
           : prefill_lds_bytes(es, dk, c, dvt, 1, outer) <= kLdsBytes ? 1 : 0;
}

// Launch plan of a prefill: value columns per workgroup (16, 32 or 64) and, for
// few long sequences, the number of sequence segments, their length in rows, and into
// how many equal pieces the state-only pass splits each segment but the last.
struct PrefillPlan {
    int dvt, nseg, seg_len, sub;
};
PrefillPlan prefill_plan(int BH, int L, int d_k, int d_v, int chunk, int elem_bytes);

// Device workspace of a segmented prefill: the states from zero of the pieces of all
// segments but the last (fp32 [BH][(nseg - 1) sub][d_k][d_v]), their gate totals
// (fp32 [BH][(nseg - 1) sub][d_k]) and room for a copy of s0 (fp32 [BH][d_k][d_v],
// used when the state is updated in place), each rounded up to 256 bytes; 0 when
// nseg == 1.
size_t prefill_workspace(const PrefillPlan &p, int BH, int d_k, int d_v);

// Enqueue the prefill kernel.  dtype: 0 fp32, 1 bf16.  state_only: compute only
// each segment's final state from a zero start and its gate totals (a.gam), with no
// outputs.  Sizes must already be valid.
hipError_t launch_prefill(const PrefillArgs &a, int dtype, int d_k, int chunk, int dvt,
                          bool state_only, hipStream_t stream);

// Enqueue one decode step.  Sizes must already be valid.
hipError_t launch_decode(const DecodeArgs &a, int dtype, int d_k, int d_v, hipStream_t stream);

// The delta rule (gla_delta.hip).  Workspace per head, element type T: the negated
// write weights -W = -X diag(beta) K as rows [lp][d_k] (lp = chunks * chunk), then the
// state-free writes U~ = X diag(beta) V transposed per chunk, [chunks][d_v][chunk];
// X is the inverse of the chunk's unit lower-triangular system.
struct DeltaArgs {
    const void *q, *k, *v;   // [B][H][L][d_k] / [B][H][L][d_v], element type T
    const float *beta;       // [B][H][L] write strengths
    const float *s0;         // [B][H][d_k][d_v] or null
    void *o;                 // [B][H][L][d_v], T
    float *s_final;          // [B][H][d_k][d_v] or null
    void *ws_w, *ws_u;       // workspace parts (see above)
    int BH, L, d_k, d_v;
    int dvt, n_vt;           // value columns per scan workgroup (16, 32 or 64), tiles per head
    int xcd_remap;
};
size_t delta_workspace(int BH, int L, int d_k, int d_v, int chunk, int elem_bytes);

// The input-side gate producer (gla_gate.hip): g = log(sigmoid(W_up W_down x)) / tau.
struct GateArgs {
    const void *x;           // [B][L][d_model], element type T
    const void *w_down;      // [rank][d_model], T
    const void *w_up;        // [H * d_k][rank], T
    float *g;                // [B][H][L][d_k] fp32 log-gates
    int B, L, d_model, H, d_k;
    int dk_shift;            // log2(d_k)
    float inv_tau;
};
// 16-output tiles per workgroup of the gate producer (grid.y splits H*d_k/16): as
// many as 64 KB of W_up rows hold.
constexpr int gate_tiles_per_group(int elem_size, int rank) { return 65536 / (16 * rank * elem_size); }
hipError_t launch_gate_project(const GateArgs &a, int dtype, int rank, hipStream_t stream);

// One decode step with the outer-product gate (gla_outer.hip):
// S <- (alpha beta^T) (.) S + phi(k) v^T, o = S^T phi(q).  Its chunkwise prefill is the
// prefill kernel's kGateOuter mode.
struct OuterArgs {
    const void *q, *k, *v;   // [B][H][d_k] / [B][H][d_v], element type T
    const float *g, *gv;     // natural-log gates [B][H][d_k] and [B][H][d_v]
    void *o;                 // [B][H][d_v], T
    float *s_final;          // the state [B][H][d_k][d_v], updated in place
    int BH, d_k, d_v, elu1;
};
hipError_t launch_outer_decode(const OuterArgs &a, int dtype, hipStream_t stream);
hipError_t launch_delta_prefill(const DeltaArgs &a, int dtype, int chunk, hipStream_t stream);
hipError_t launch_delta_decode(const DeltaArgs &a, int dtype, hipStream_t stream);

}  // namespace gla
