// gla_api.cpp -- the C ABI declared in include/gla.h: host-only argument
// validation (no HIP call happens before it passes), launch configuration, and the
// state allocation helpers.  The operations themselves are the gated recurrence of
// "Attention is recurrent" (Linear attention, Gated linear attention) and "Gated
// Linear Attention" (Recurrent Form), computed by the kernels in gla_prefill.hpp
// (chunkwise form) and gla_decode.hip (one recurrent step).
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "gla.h"
#include "gla_launch.hpp"
#include "gla_testing.h"

namespace gla {
// Launch-plan choices forced by gla_testing_set_plan (0: automatic).
static int g_force_prefill_tile = 0, g_force_prefill_segments = 0, g_force_delta_tile = 0;

hipError_t launch_prefill_0_16(const PrefillArgs &, int, int, bool, hipStream_t);
hipError_t launch_prefill_0_32(const PrefillArgs &, int, int, bool, hipStream_t);
hipError_t launch_prefill_0_64(const PrefillArgs &, int, int, bool, hipStream_t);
hipError_t launch_prefill_0_128(const PrefillArgs &, int, int, bool, hipStream_t);
hipError_t launch_prefill_1_16(const PrefillArgs &, int, int, bool, hipStream_t);
hipError_t launch_prefill_1_32(const PrefillArgs &, int, int, bool, hipStream_t);
hipError_t launch_prefill_1_64(const PrefillArgs &, int, int, bool, hipStream_t);
hipError_t launch_prefill_1_128(const PrefillArgs &, int, int, bool, hipStream_t);

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int d_k, int chunk, int dvt,
                          bool state_only, hipStream_t stream)
{
    if (dtype == 1) {
        switch (d_k) {
        case 16: return launch_prefill_1_16(a, chunk, dvt, state_only, stream);
        case 32: return launch_prefill_1_32(a, chunk, dvt, state_only, stream);
        case 64: return launch_prefill_1_64(a, chunk, dvt, state_only, stream);
        case 128: return launch_prefill_1_128(a, chunk, dvt, state_only, stream);
        }
    } else {
        switch (d_k) {
        case 16: return launch_prefill_0_16(a, chunk, dvt, state_only, stream);
        case 32: return launch_prefill_0_32(a, chunk, dvt, state_only, stream);
        case 64: return launch_prefill_0_64(a, chunk, dvt, state_only, stream);
        case 128: return launch_prefill_0_128(a, chunk, dvt, state_only, stream);
        }
    }
    return hipErrorInvalidValue;
}

// Launch shape: the widest value tile (64, 32 or 16 columns) that fits in LDS and
// still gives at least 256 workgroups for the 256 compute units (a test can force
// another usable width through gla_testing_set_plan).
static bool tile_usable(int dvt, int d_k, int d_v, int chunk, int elem_bytes, bool outer = false)
{
    return dvt <= d_v && d_v % dvt == 0 && prefill_nbuf(elem_bytes, d_k, chunk, dvt, outer) > 0;
}

int prefill_tile(int BH, int d_k, int d_v, int chunk, int elem_bytes, bool outer = false)
{
    const int forced = g_force_prefill_tile;
    if (forced && tile_usable(forced, d_k, d_v, chunk, elem_bytes, outer)) return forced;
    const long bh = BH;
    if (tile_usable(64, d_k, d_v, chunk, elem_bytes, outer) && bh * (d_v / 64) >= 256) return 64;
    if (tile_usable(32, d_k, d_v, chunk, elem_bytes, outer) && bh * (d_v / 32) >= 256) return 32;
    return 16;
}

// Few long sequences: rather than narrowing the value tile (which repeats the per-
// token gate and score work in every tile of a head), split each sequence into
// segments at the widest tile.  A state-only pass computes every segment's state
// from zero, and the full pass then runs all segments in parallel, each workgroup
// first scanning the earlier segments' states into its own initial state.  Used when
// the widest tile gives fewer than 256 workgroups and the sequences have at least 64
// chunks; segments keep at least 16 chunks.  Sequences of 32 to 63 chunks are split
// too when even the narrowest tile leaves CUs idle (fewer than 256 workgroups), at a
// 32-column tile into at most four segments of at least 4 chunks.
// gla_testing_set_plan can force the count.
constexpr int kSegMinChunks = 16, kSegMinSeqChunks = 64;
constexpr int kSegShortMinChunks = 4, kSegShortSeqChunks = 32;
// The state-only pass runs alone ahead of the full pass: it splits each segment into
// equal pieces (each at least kPieceMinChunks chunks) until up to three of its
// workgroups share each CU (as many as its registers allow without gates or with a
// scalar gate), and the full pass scans the pieces' states.
constexpr int kPieceMinChunks = 4, kPieceMaxWorkgroups = 768;

PrefillPlan prefill_plan(int BH, int L, int d_k, int d_v, int chunk, int elem_bytes)
{
    PrefillPlan p{prefill_tile(BH, d_k, d_v, chunk, elem_bytes), 1, L, 1};
    const int nchunks = (L + chunk - 1) / chunk;
    int dvt = 16;
    for (int t : {64, 32})
        if (dvt == 16 && tile_usable(t, d_k, d_v, chunk, elem_bytes)) dvt = t;
    if (g_force_prefill_tile && tile_usable(g_force_prefill_tile, d_k, d_v, chunk, elem_bytes))
        dvt = g_force_prefill_tile;
    const long wgs = (long)BH * (d_v / dvt);
    int nseg = 1;
    if (nchunks >= kSegMinSeqChunks) {
        while (wgs * nseg < 256 && nchunks / (2 * nseg) >= kSegMinChunks) nseg *= 2;
    } else if (nchunks >= kSegShortSeqChunks && (long)BH * (d_v / 16) < 256) {
        // a 32-column tile with at most four segments: each workgroup scans the earlier
        // segments' states before its first chunk, and with chains this short a deeper
        // split costs more than the repeated per-token work of a narrower tile
        if (tile_usable(32, d_k, d_v, chunk, elem_bytes)) dvt = 32;
        const long w32 = (long)BH * (d_v / dvt);
        while (w32 * nseg * 2 <= 256 && nseg < 4 && nchunks / (2 * nseg) >= kSegShortMinChunks) nseg *= 2;
    }
    const int forced = g_force_prefill_segments;
    if (forced >= 1) nseg = forced < nchunks ? forced : (nchunks > 0 ? nchunks : 1);
    if (nseg > 1) {
        const int cps = (nchunks + nseg - 1) / nseg;   // chunks per segment
        p.nseg = (nchunks + cps - 1) / cps;
        p.seg_len = cps * chunk;
        p.dvt = dvt;
        const long pass1 = (long)BH * (d_v / dvt) * (p.nseg - 1);
        while (pass1 * p.sub * 2 <= kPieceMaxWorkgroups && cps % (2 * p.sub) == 0 &&
               cps / (2 * p.sub) >= kPieceMinChunks)
            p.sub *= 2;
    }
    return p;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

size_t prefill_workspace(const PrefillPlan &p, int BH, int d_k, int d_v)
{
    if (p.nseg <= 1) return 0;
    const size_t pieces = (size_t)BH * (p.nseg - 1) * p.sub;
    return round256(pieces * d_k * d_v * 4) + round256(pieces * d_k * 4) + round256((size_t)BH * d_k * d_v * 4);
}
}  // namespace gla

namespace {

thread_local std::string g_detail;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_detail = buf;
    return status;
}

int ok()
{
    g_detail.clear();
    return GLA_OK;
}

bool dim_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_supported(int c) { return c == 16 || c == 32 || c == 64; }
// the GLA prefills also take chunks of 128 rows when d_k <= 64
bool prefill_chunk_supported(int c, int d_k) { return chunk_supported(c) || (c == 128 && d_k <= 64); }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t elem_size(gla_dtype dt) { return dt == GLA_BF16 ? 2 : 4; }

struct Span {
    uintptr_t lo, hi;   // [lo, hi); empty when lo == hi
    const char *name;
};
Span span(const void *p, size_t bytes, const char *name)
{
    const uintptr_t lo = (uintptr_t)p;
    return Span{lo, p ? lo + bytes : lo, name};
}
bool overlap(const Span &a, const Span &b)
{
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

int check_common(int B, int H, int d_k, int d_v, gla_dtype dtype, gla_gate_mode gate,
                 gla_feature_map phi, const float *g, bool g_required)
{
    if (B <= 0 || H <= 0) return fail(GLA_ERR_SHAPE, "B=%d and H=%d must be positive", B, H);
    if (d_k <= 0 || d_v <= 0)
        return fail(GLA_ERR_SHAPE, "d_k=%d and d_v=%d must be positive", d_k, d_v);
    if (!dim_supported(d_k) || !dim_supported(d_v))
        return fail(GLA_ERR_UNSUPPORTED, "d_k=%d, d_v=%d: each must be 16, 32, 64 or 128", d_k, d_v);
    if (dtype != GLA_F32 && dtype != GLA_BF16)
        return fail(GLA_ERR_UNSUPPORTED, "dtype %d is not GLA_F32 or GLA_BF16", (int)dtype);
    if (gate != GLA_GATE_NONE && gate != GLA_GATE_KEYDIM && gate != GLA_GATE_SCALAR)
        return fail(GLA_ERR_UNSUPPORTED, "gate mode %d", (int)gate);
    if (phi != GLA_PHI_IDENTITY && phi != GLA_PHI_ELU1)
        return fail(GLA_ERR_UNSUPPORTED, "feature map %d", (int)phi);
    if (gate == GLA_GATE_NONE && g != nullptr)
        return fail(GLA_ERR_UNSUPPORTED, "g must be NULL with GLA_GATE_NONE");
    if (gate != GLA_GATE_NONE && g == nullptr && g_required)
        return fail(GLA_ERR_NULL, "g is NULL but a gate mode is set");
    if (g && ((uintptr_t)g & (gate == GLA_GATE_SCALAR ? 3u : 15u)))
        return fail(GLA_ERR_ALIGN, "g=%p is not %d-byte aligned", (const void *)g,
                    gate == GLA_GATE_SCALAR ? 4 : 16);
    return GLA_OK;
}

// ---- scratch of the allocation-free prefill (gla_prefill_chunked_noalloc) ----------
// A segmented prefill's workspace (segment states and gate totals) comes from this
// array: each device the library runs on holds its own copy until the process ends.
// Its device address is looked up once per device, with that device current; host
// code uses only that address, never the array's name.  Nothing in it must start at
// zero: every byte a launch reads was written earlier in the same call.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

int scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GLA_ERR_HIP, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GLA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return GLA_OK;
}

}  // namespace

extern "C" {

const char *gla_strerror(int status)
{
    switch (status) {
    case GLA_OK: return "success";
    case GLA_ERR_NULL: return "required pointer is NULL";
    case GLA_ERR_SHAPE: return "invalid size";
    case GLA_ERR_UNSUPPORTED: return "unsupported size, dtype, gate mode or feature map";
    case GLA_ERR_ALIGN: return "pointer not suitably aligned";
    case GLA_ERR_ALIAS: return "output overlaps an input";
    case GLA_ERR_HIP: return "HIP runtime error";
    case GLA_ERR_OOM: return "out of device memory";
    case GLA_ERR_WORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

const char *gla_last_error_detail(void) { return g_detail.c_str(); }

int gla_testing_set_plan(int prefill_tile, int prefill_segments, int delta_tile)
{
    auto tile_ok = [](int t) { return t == 0 || t == 16 || t == 32 || t == 64; };
    if (!tile_ok(prefill_tile) || !tile_ok(delta_tile) || prefill_segments < 0)
        return fail(GLA_ERR_UNSUPPORTED, "gla_testing_set_plan(%d, %d, %d): tiles must be 0, 16, 32 or 64 and "
                    "segments >= 0", prefill_tile, prefill_segments, delta_tile);
    gla::g_force_prefill_tile = prefill_tile;
    gla::g_force_prefill_segments = prefill_segments;
    gla::g_force_delta_tile = delta_tile;
    return ok();
}

int gla_state_alloc(int B, int H, int d_k, int d_v, float **state, gla_stream_t stream)
{
    if (!state) return fail(GLA_ERR_NULL, "state out-pointer is NULL");
    if (B <= 0 || H <= 0 || d_k <= 0 || d_v <= 0)
        return fail(GLA_ERR_SHAPE, "B=%d H=%d d_k=%d d_v=%d must be positive", B, H, d_k, d_v);
    if (!dim_supported(d_k) || !dim_supported(d_v))
        return fail(GLA_ERR_UNSUPPORTED, "d_k=%d, d_v=%d: each must be 16, 32, 64 or 128", d_k, d_v);
    const size_t bytes = (size_t)B * H * d_k * d_v * sizeof(float);
    void *p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e == hipErrorOutOfMemory) {
        (void)hipGetLastError();
        return fail(GLA_ERR_OOM, "hipMalloc(%zu) failed: out of memory", bytes);
    }
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "hipMalloc: %s", hipGetErrorString(e));
    e = hipMemsetAsync(p, 0, bytes, (hipStream_t)stream);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return fail(GLA_ERR_HIP, "hipMemsetAsync: %s", hipGetErrorString(e));
    }
    *state = (float *)p;
    return ok();
}

int gla_state_free(float *state, gla_stream_t stream)
{
    if (!state) return ok();
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
    e = hipFree(state);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "hipFree: %s", hipGetErrorString(e));
    return ok();
}

size_t gla_prefill_workspace_bytes(int B, int H, int L, int d_k, int d_v, int chunk,
                                   gla_dtype dtype)
{
    if (B <= 0 || H <= 0 || L < 0 || !dim_supported(d_k) || !dim_supported(d_v) ||
        !prefill_chunk_supported(chunk, d_k) || (dtype != GLA_F32 && dtype != GLA_BF16) ||
        (long long)B * H > 0x7fffffffLL)
        return 0;
    const int BH = B * H;
    const gla::PrefillPlan p = gla::prefill_plan(BH, L, d_k, d_v, chunk, (int)elem_size(dtype));
    return gla::prefill_workspace(p, BH, d_k, d_v);
}

// Both prefill entry points.  norm: the normalised form, with the normaliser state
// z0 (nullable) / z_final (nullable); it runs unsegmented and needs no workspace.
static int prefill_impl(const void *q, const void *k, const void *v, const float *g,
                        gla_gate_mode gate, const float *s0, const float *z0, void *o, float *s_final,
                        float *z_final, int B, int H, int L, int d_k, int d_v, int chunk,
                        gla_dtype dtype, gla_feature_map phi, void *workspace,
                        size_t workspace_bytes, gla_stream_t stream, bool norm, bool use_scratch = false)
{
    if (L < 0) return fail(GLA_ERR_SHAPE, "L=%d must be >= 0", L);
    int st = check_common(B, H, d_k, d_v, dtype, gate, phi, g, L > 0);
    if (st != GLA_OK) return st;
    if (!prefill_chunk_supported(chunk, d_k))
        return fail(GLA_ERR_UNSUPPORTED, "chunk=%d: must be 16, 32 or 64, or 128 when d_k <= 64 (d_k=%d)",
                    chunk, d_k);
    // the kernel addresses one head's rows (and the rows of its last chunk past L)
    // with 32-bit byte offsets: (L + chunk) * max(d_k, d_v) * 4 must stay below 2^31
    if ((long long)(L + chunk) * (d_k > d_v ? d_k : d_v) * 4 > 0x7fffffffLL)
        return fail(GLA_ERR_SHAPE, "L=%d too long for one head (limit (L + chunk) * max(d_k, d_v) * 4 < 2^31)", L);
    if (L > 0 && (!q || !k || !v || !o))
        return fail(GLA_ERR_NULL, "q, k, v and o are required when L > 0");
    const void *ptrs[] = {q, k, v, s0, o, s_final, workspace, z0, z_final};
    const char *names[] = {"q", "k", "v", "s0", "o", "s_final", "workspace", "z0", "z_final"};
    for (int i = 0; i < 9; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GLA_ERR_ALIGN, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    const size_t need = norm ? 0 : gla_prefill_workspace_bytes(B, H, L, d_k, d_v, chunk, dtype);
    if (use_scratch && need > kScratchBytes)
        return fail(GLA_ERR_WORKSPACE, "these sizes need %zu bytes of scratch; the allocation-free prefill "
                    "holds %zu (use gla_prefill_chunked with a workspace)", need, kScratchBytes);
    if (!use_scratch && need > 0 && (!workspace || workspace_bytes < need))
        return fail(GLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);

    const size_t BH = (size_t)B * H, es = elem_size(dtype);
    const size_t gbytes = gate == GLA_GATE_KEYDIM ? BH * L * d_k * 4 : BH * L * 4;
    const size_t sbytes = BH * d_k * d_v * 4;
    const Span sq = span(q, BH * L * d_k * es, "q"), sk = span(k, BH * L * d_k * es, "k");
    const Span sv = span(v, BH * L * d_v * es, "v"), sg = span(g, g ? gbytes : 0, "g");
    const Span ss0 = span(s0, sbytes, "s0"), so = span(o, BH * L * d_v * es, "o");
    const Span ssf = span(s_final, sbytes, "s_final"), sw = span(workspace, need, "workspace");
    const size_t zbytes = BH * d_k * 4;
    const Span sz0 = span(z0, zbytes, "z0"), szf = span(z_final, zbytes, "z_final");
    const Span o_forbidden[] = {sq, sk, sv, sg, ss0, ssf, sw, sz0, szf};
    for (const Span &x : o_forbidden)
        if (overlap(so, x)) return fail(GLA_ERR_ALIAS, "o overlaps %s", x.name);
    const Span sf_forbidden[] = {sq, sk, sv, sg, sw, sz0, szf};
    for (const Span &x : sf_forbidden)
        if (overlap(ssf, x)) return fail(GLA_ERR_ALIAS, "s_final overlaps %s", x.name);
    if (overlap(ssf, ss0) && s_final != s0)
        return fail(GLA_ERR_ALIAS, "s_final partially overlaps s0");
    const Span w_forbidden[] = {sq, sk, sv, sg, ss0, sz0};
    for (const Span &x : w_forbidden)
        if (overlap(sw, x)) return fail(GLA_ERR_ALIAS, "workspace overlaps %s", x.name);
    const Span zf_forbidden[] = {sq, sk, sv, sg, sw, ss0};
    for (const Span &x : zf_forbidden)
        if (overlap(szf, x)) return fail(GLA_ERR_ALIAS, "z_final overlaps %s", x.name);
    // every value-column workgroup of a head reads all of z0 when it starts, and one of
    // them writes z_final when it ends: an in-place z would race between workgroups
    if (overlap(szf, sz0))
        return fail(GLA_ERR_ALIAS, "z_final overlaps z0 (in-place normaliser state is not supported)");

    gla::PrefillPlan plan = gla::prefill_plan((int)BH, L, d_k, d_v, chunk, (int)es);
    if (norm) plan = {gla::prefill_tile((int)BH, d_k, d_v, chunk, (int)es), 1, L, 1};
    gla::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s0 = s0; a.o = o; a.s_final = s_final;
    a.BH = (int)BH; a.L = L; a.d_v = d_v;
    a.gate = (int)gate; a.elu1 = phi == GLA_PHI_ELU1;
    a.n_vt = d_v / plan.dvt;
    a.nseg = plan.nseg; a.seg_len = plan.seg_len; a.gam = nullptr;
    a.norm = norm ? 1 : 0; a.z0 = z0; a.z_final = z_final;
    const long grid = (long)BH * a.nseg * a.n_vt;
    if (grid > 0x7fffffffL) return fail(GLA_ERR_SHAPE, "B*H too large");
    a.xcd_remap = (a.n_vt > 1 && grid % 8 == 0) ? 1 : 0;
    if (L == 0 && !s_final && !z_final) return ok();
    if (use_scratch && plan.nseg > 1) {             // validation done: now the HIP lookup
        st = scratch_address(&workspace);
        if (st != GLA_OK) return st;
    }
    const int dt = dtype == GLA_BF16 ? 1 : 0;
    const hipStream_t hs = (hipStream_t)stream;
    hipError_t e;
    if (plan.nseg == 1) {
        e = gla::launch_prefill(a, dt, d_k, chunk, plan.dvt, false, hs);
    } else {
        // workspace: the states from zero and gate totals of the pieces of all segments
        // but the last, then room for a copy of s0
        const size_t pieces = (size_t)BH * (plan.nseg - 1) * plan.sub;
        float *ds = (float *)workspace;
        float *gam = (float *)((char *)ds + gla::round256(pieces * d_k * d_v * 4));
        float *s0c = (float *)((char *)gam + gla::round256(pieces * d_k * 4));
        // in place (s_final == s0): every segment's workgroups read s0 while the last
        // segment's write s_final, and they need not all be running at once, so the
        // full pass reads a copy taken before either launch
        const float *s0_full = s0;
        e = hipSuccess;
        if (s0 && s_final == s0) {
            e = hipMemcpyAsync(s0c, s0, sbytes, hipMemcpyDeviceToDevice, hs);
            s0_full = s0c;
        }
        // pass 1: the states from zero of the pieces of every segment but the last
        // (whose state only feeds s_final, which pass 2 writes)
        gla::PrefillArgs a1 = a;
        a1.s0 = nullptr; a1.s_final = ds; a1.o = nullptr; a1.gam = gam;
        a1.nseg = (plan.nseg - 1) * plan.sub;
        a1.seg_len = plan.seg_len / plan.sub;
        a1.xcd_remap = (a1.n_vt > 1 && ((long)BH * a1.nseg * a1.n_vt) % 8 == 0) ? 1 : 0;
        if (e == hipSuccess) e = gla::launch_prefill(a1, dt, d_k, chunk, plan.dvt, true, hs);
        // pass 2: outputs of every segment, each workgroup scanning the earlier
        // segments' states into its own initial state
        gla::PrefillArgs a2 = a;
        a2.s0 = s0_full; a2.s_final = s_final; a2.final_last_seg = 1;
        a2.seg_ds = ds; a2.seg_gam = gate == GLA_GATE_NONE ? nullptr : gam;
        a2.seg_sub = plan.sub;
        if (e == hipSuccess) e = gla::launch_prefill(a2, dt, d_k, chunk, plan.dvt, false, hs);
    }
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return ok();
}

int gla_prefill_chunked(const void *q, const void *k, const void *v, const float *g,
                        gla_gate_mode gate, const float *s0, void *o, float *s_final,
                        int B, int H, int L, int d_k, int d_v, int chunk, gla_dtype dtype,
                        gla_feature_map phi, void *workspace, size_t workspace_bytes,
                        gla_stream_t stream)
{
    return prefill_impl(q, k, v, g, gate, s0, nullptr, o, s_final, nullptr, B, H, L, d_k, d_v, chunk,
                        dtype, phi, workspace, workspace_bytes, stream, false);
}

int gla_prefill_chunked_noalloc(const void *q, const void *k, const void *v, const float *g,
                                gla_gate_mode gate, const float *s0, void *o, float *s_final, int B, int H,
                                int L, int d_k, int d_v, int chunk, gla_dtype dtype, gla_feature_map phi,
                                gla_stream_t stream)
{
    return prefill_impl(q, k, v, g, gate, s0, nullptr, o, s_final, nullptr, B, H, L, d_k, d_v, chunk, dtype, phi,
                        nullptr, 0, stream, false, true);
}

int gla_prefill_chunked_norm(const void *q, const void *k, const void *v, const float *g,
                             gla_gate_mode gate, const float *s0, const float *z0, void *o,
                             float *s_final, float *z_final, int B, int H, int L, int d_k,
                             int d_v, int chunk, gla_dtype dtype, gla_feature_map phi,
                             gla_stream_t stream)
{
    return prefill_impl(q, k, v, g, gate, s0, z0, o, s_final, z_final, B, H, L, d_k, d_v, chunk, dtype,
                        phi, nullptr, 0, stream, true);
}

// Both decode entry points; z non-null selects the normalised form.
static int decode_impl(const void *q, const void *k, const void *v, const float *g,
                       gla_gate_mode gate, float *state, float *z, void *o, int B, int H, int d_k,
                       int d_v, gla_dtype dtype, gla_feature_map phi, gla_stream_t stream)
{
    int st = check_common(B, H, d_k, d_v, dtype, gate, phi, g, true);
    if (st != GLA_OK) return st;
    if (!q || !k || !v || !state || !o)
        return fail(GLA_ERR_NULL, "q, k, v, state and o are required");
    const void *ptrs[] = {q, k, v, state, o, z};
    const char *names[] = {"q", "k", "v", "state", "o", "z"};
    for (int i = 0; i < 6; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GLA_ERR_ALIGN, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    const size_t BH = (size_t)B * H, es = elem_size(dtype);
    const size_t gbytes = gate == GLA_GATE_KEYDIM ? BH * d_k * 4 : BH * 4;
    const Span sq = span(q, BH * d_k * es, "q"), sk = span(k, BH * d_k * es, "k");
    const Span sv = span(v, BH * d_v * es, "v"), sg = span(g, g ? gbytes : 0, "g");
    const Span sst = span(state, BH * d_k * d_v * 4, "state"), so = span(o, BH * d_v * es, "o");
    const Span sz = span(z, BH * d_k * 4, "z");
    const Span o_forbidden[] = {sq, sk, sv, sg, sst, sz};
    for (const Span &x : o_forbidden)
        if (overlap(so, x)) return fail(GLA_ERR_ALIAS, "o overlaps %s", x.name);
    const Span st_forbidden[] = {sq, sk, sv, sg, sz};
    for (const Span &x : st_forbidden)
        if (overlap(sst, x)) return fail(GLA_ERR_ALIAS, "state overlaps %s", x.name);
    const Span z_forbidden[] = {sq, sk, sv, sg};
    for (const Span &x : z_forbidden)
        if (overlap(sz, x)) return fail(GLA_ERR_ALIAS, "z overlaps %s", x.name);
    if (BH > 0x7fffffffUL) return fail(GLA_ERR_SHAPE, "B*H too large");

    gla::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.state = state; a.o = o;
    a.BH = (int)BH; a.gate = (int)gate; a.elu1 = phi == GLA_PHI_ELU1; a.z = z;
    hipError_t e = gla::launch_decode(a, dtype == GLA_BF16 ? 1 : 0, d_k, d_v, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

int gla_decode_step(const void *q, const void *k, const void *v, const float *g,
                    gla_gate_mode gate, float *state, void *o, int B, int H, int d_k, int d_v,
                    gla_dtype dtype, gla_feature_map phi, gla_stream_t stream)
{
    return decode_impl(q, k, v, g, gate, state, nullptr, o, B, H, d_k, d_v, dtype, phi, stream);
}

int gla_decode_step_norm(const void *q, const void *k, const void *v, const float *g,
                         gla_gate_mode gate, float *state, float *z, void *o, int B, int H, int d_k,
                         int d_v, gla_dtype dtype, gla_feature_map phi, gla_stream_t stream)
{
    if (!z) return fail(GLA_ERR_NULL, "z (the normaliser state) is required");
    return decode_impl(q, k, v, g, gate, state, z, o, B, H, d_k, d_v, dtype, phi, stream);
}

// ---- the delta rule ----------------------------------------------------------------

size_t gla_delta_workspace_bytes(int B, int H, int L, int d_k, int d_v, int chunk, gla_dtype dtype)
{
    if (B <= 0 || H <= 0 || L < 0 || !dim_supported(d_k) || !dim_supported(d_v) || !chunk_supported(chunk) ||
        (dtype != GLA_F32 && dtype != GLA_BF16) || (long long)B * H > 0x7fffffffLL)
        return 0;
    return gla::delta_workspace(B * H, L, d_k, d_v, chunk, (int)elem_size(dtype));
}

int gla_prefill_delta(const void *q, const void *k, const void *v, const float *beta, const float *s0,
                      void *o, float *s_final, int B, int H, int L, int d_k, int d_v, int chunk,
                      gla_dtype dtype, void *workspace, size_t workspace_bytes, gla_stream_t stream)
{
    if (L < 0) return fail(GLA_ERR_SHAPE, "L=%d must be >= 0", L);
    int st = check_common(B, H, d_k, d_v, dtype, GLA_GATE_NONE, GLA_PHI_IDENTITY, nullptr, false);
    if (st != GLA_OK) return st;
    if (!chunk_supported(chunk))
        return fail(GLA_ERR_UNSUPPORTED, "chunk=%d: must be 16, 32 or 64", chunk);
    if ((long long)(L + chunk) * (d_k > d_v ? d_k : d_v) * 4 > 0x7fffffffLL)
        return fail(GLA_ERR_SHAPE, "L=%d too long for one head (limit (L + chunk) * max(d_k, d_v) * 4 < 2^31)", L);
    if (L > 0 && (!q || !k || !v || !beta || !o))
        return fail(GLA_ERR_NULL, "q, k, v, beta and o are required when L > 0");
    const void *ptrs[] = {q, k, v, s0, o, s_final, workspace};
    const char *names[] = {"q", "k", "v", "s0", "o", "s_final", "workspace"};
    for (int i = 0; i < 7; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GLA_ERR_ALIGN, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    if (beta && ((uintptr_t)beta & 3u)) return fail(GLA_ERR_ALIGN, "beta=%p is not 4-byte aligned", (const void *)beta);
    const size_t need = gla_delta_workspace_bytes(B, H, L, d_k, d_v, chunk, dtype);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);

    const size_t BH = (size_t)B * H, es = elem_size(dtype);
    const size_t sbytes = BH * d_k * d_v * 4;
    const Span sq = span(q, BH * L * d_k * es, "q"), sk = span(k, BH * L * d_k * es, "k");
    const Span sv = span(v, BH * L * d_v * es, "v"), sb = span(beta, BH * L * 4, "beta");
    const Span ss0 = span(s0, sbytes, "s0"), so = span(o, BH * L * d_v * es, "o");
    const Span ssf = span(s_final, sbytes, "s_final"), sw = span(workspace, need, "workspace");
    const Span o_forbidden[] = {sq, sk, sv, sb, ss0, ssf, sw};
    for (const Span &x : o_forbidden)
        if (overlap(so, x)) return fail(GLA_ERR_ALIAS, "o overlaps %s", x.name);
    const Span sf_forbidden[] = {sq, sk, sv, sb, sw};
    for (const Span &x : sf_forbidden)
        if (overlap(ssf, x)) return fail(GLA_ERR_ALIAS, "s_final overlaps %s", x.name);
    if (overlap(ssf, ss0) && s_final != s0)
        return fail(GLA_ERR_ALIAS, "s_final partially overlaps s0");
    const Span w_forbidden[] = {sq, sk, sv, sb, ss0};
    for (const Span &x : w_forbidden)
        if (overlap(sw, x)) return fail(GLA_ERR_ALIAS, "workspace overlaps %s", x.name);

    const long nch = (L + chunk - 1) / chunk;
    if ((long)BH * (nch > 1 ? nch : 1) > 0x7fffffffL) return fail(GLA_ERR_SHAPE, "B*H*chunks too large");
    gla::DeltaArgs a;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.s0 = s0; a.o = o; a.s_final = s_final;
    const size_t lp = (size_t)nch * chunk;
    a.ws_w = workspace;
    a.ws_u = workspace ? (char *)workspace + BH * lp * d_k * es : nullptr;
    a.BH = (int)BH; a.L = L; a.d_k = d_k; a.d_v = d_v;
    a.dvt = d_v < 64 ? d_v : 64;
    if (gla::g_force_delta_tile && gla::g_force_delta_tile <= d_v) a.dvt = gla::g_force_delta_tile;
    a.n_vt = d_v / a.dvt;
    const long grid = (long)BH * a.n_vt;
    a.xcd_remap = (a.n_vt > 1 && grid % 8 == 0) ? 1 : 0;
    if (L == 0 && !s_final) return ok();
    const hipError_t e = gla::launch_delta_prefill(a, dtype == GLA_BF16 ? 1 : 0, chunk, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "delta prefill launch: %s", hipGetErrorString(e));
    return ok();
}

int gla_decode_step_delta(const void *q, const void *k, const void *v, const float *beta, float *state,
                          void *o, int B, int H, int d_k, int d_v, gla_dtype dtype, gla_stream_t stream)
{
    int st = check_common(B, H, d_k, d_v, dtype, GLA_GATE_NONE, GLA_PHI_IDENTITY, nullptr, false);
    if (st != GLA_OK) return st;
    if (!q || !k || !v || !beta || !state || !o)
        return fail(GLA_ERR_NULL, "q, k, v, beta, state and o are required");
    const void *ptrs[] = {q, k, v, state, o};
    const char *names[] = {"q", "k", "v", "state", "o"};
    for (int i = 0; i < 5; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    if ((uintptr_t)beta & 3u) return fail(GLA_ERR_ALIGN, "beta=%p is not 4-byte aligned", (const void *)beta);
    const size_t BH = (size_t)B * H, es = elem_size(dtype);
    const Span sq = span(q, BH * d_k * es, "q"), sk = span(k, BH * d_k * es, "k");
    const Span sv = span(v, BH * d_v * es, "v"), sb = span(beta, BH * 4, "beta");
    const Span sst = span(state, BH * d_k * d_v * 4, "state"), so = span(o, BH * d_v * es, "o");
    const Span o_forbidden[] = {sq, sk, sv, sb, sst};
    for (const Span &x : o_forbidden)
        if (overlap(so, x)) return fail(GLA_ERR_ALIAS, "o overlaps %s", x.name);
    const Span st_forbidden[] = {sq, sk, sv, sb};
    for (const Span &x : st_forbidden)
        if (overlap(sst, x)) return fail(GLA_ERR_ALIAS, "state overlaps %s", x.name);
    if (BH > 0x7fffffffUL) return fail(GLA_ERR_SHAPE, "B*H too large");
    gla::DeltaArgs a = {};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.s0 = state; a.s_final = state; a.o = o;
    a.BH = (int)BH; a.d_k = d_k; a.d_v = d_v;
    const hipError_t e = gla::launch_delta_decode(a, dtype == GLA_BF16 ? 1 : 0, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "delta decode launch: %s", hipGetErrorString(e));
    return ok();
}

// ---- the input-side gate producer ------------------------------------------------

int gla_gate_project(const void *x, const void *w_down, const void *w_up, float *g, int B, int L,
                     int d_model, int rank, int H, int d_k, float tau, gla_dtype dtype,
                     gla_stream_t stream)
{
    if (B <= 0 || H <= 0 || L < 0) return fail(GLA_ERR_SHAPE, "B=%d, H=%d must be positive and L=%d >= 0", B, H, L);
    if (d_model <= 0) return fail(GLA_ERR_SHAPE, "d_model=%d must be positive", d_model);
    if (d_model % 32 != 0 || d_model > 65536)
        return fail(GLA_ERR_UNSUPPORTED, "d_model=%d: must be a multiple of 32, at most 65536", d_model);
    if (rank != 16 && rank != 32) return fail(GLA_ERR_UNSUPPORTED, "rank=%d: must be 16 or 32", rank);
    if (!dim_supported(d_k)) return fail(GLA_ERR_UNSUPPORTED, "d_k=%d: must be 16, 32, 64 or 128", d_k);
    if (dtype != GLA_F32 && dtype != GLA_BF16)
        return fail(GLA_ERR_UNSUPPORTED, "dtype %d is not GLA_F32 or GLA_BF16", (int)dtype);
    if (!(tau > 0.f) || tau > 3.0e38f) return fail(GLA_ERR_SHAPE, "tau=%g must be positive and finite", (double)tau);
    if ((long long)H * d_k > (1LL << 20)) return fail(GLA_ERR_SHAPE, "H*d_k=%lld too large", (long long)H * d_k);
    if ((long long)B * L > (1LL << 40)) return fail(GLA_ERR_SHAPE, "B*L too large");
    if (L > 0 && (!x || !w_down || !w_up || !g))
        return fail(GLA_ERR_NULL, "x, w_down, w_up and g are required when L > 0");
    const void *ptrs[] = {x, w_down, w_up, g};
    const char *names[] = {"x", "w_down", "w_up", "g"};
    for (int i = 0; i < 4; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GLA_ERR_ALIGN, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    const size_t es = elem_size(dtype), ntok = (size_t)B * L;
    const Span sx = span(x, ntok * d_model * es, "x"), swd = span(w_down, (size_t)rank * d_model * es, "w_down");
    const Span swu = span(w_up, (size_t)H * d_k * rank * es, "w_up"), sg = span(g, ntok * H * d_k * 4, "g");
    const Span g_forbidden[] = {sx, swd, swu};
    for (const Span &s : g_forbidden)
        if (overlap(sg, s)) return fail(GLA_ERR_ALIAS, "g overlaps %s", s.name);
    if (L == 0) return ok();
    if ((ntok + 63) / 64 > 0x7fffffffUL) return fail(GLA_ERR_SHAPE, "B*L too large");
    gla::GateArgs a;
    a.x = x; a.w_down = w_down; a.w_up = w_up; a.g = g;
    a.B = B; a.L = L; a.d_model = d_model; a.H = H; a.d_k = d_k; a.inv_tau = 1.f / tau;
    a.dk_shift = 0;
    while ((1 << a.dk_shift) < d_k) ++a.dk_shift;           // d_k is a power of two
    const hipError_t e = gla::launch_gate_project(a, dtype == GLA_BF16 ? 1 : 0, rank, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "gate producer launch: %s", hipGetErrorString(e));
    return ok();
}

// ---- the outer-product gate --------------------------------------------------------

int gla_prefill_outer(const void *q, const void *k, const void *v, const float *g, const float *gv,
                      const float *s0, void *o, float *s_final, int B, int H, int L, int d_k, int d_v,
                      int chunk, gla_dtype dtype, gla_feature_map phi, gla_stream_t stream)
{
    if (L < 0) return fail(GLA_ERR_SHAPE, "L=%d must be >= 0", L);
    int st = check_common(B, H, d_k, d_v, dtype, GLA_GATE_KEYDIM, phi, g, L > 0);
    if (st != GLA_OK) return st;
    if (!chunk_supported(chunk))
        return fail(GLA_ERR_UNSUPPORTED, "chunk=%d: must be 16, 32 or 64", chunk);
    if ((long long)(L + chunk) * (d_k > d_v ? d_k : d_v) * 4 > 0x7fffffffLL)
        return fail(GLA_ERR_SHAPE, "L=%d too long for one head (limit (L + chunk) * max(d_k, d_v) * 4 < 2^31)", L);
    if (L > 0 && (!q || !k || !v || !gv || !o))
        return fail(GLA_ERR_NULL, "q, k, v, g, gv and o are required when L > 0");
    const void *ptrs[] = {q, k, v, gv, s0, o, s_final};
    const char *names[] = {"q", "k", "v", "gv", "s0", "o", "s_final"};
    for (int i = 0; i < 7; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GLA_ERR_ALIGN, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    const size_t BH = (size_t)B * H, es = elem_size(dtype);
    const size_t sbytes = BH * d_k * d_v * 4;
    const Span sq = span(q, BH * L * d_k * es, "q"), sk = span(k, BH * L * d_k * es, "k");
    const Span sv = span(v, BH * L * d_v * es, "v"), sg = span(g, BH * L * d_k * 4, "g");
    const Span sgv = span(gv, BH * L * d_v * 4, "gv"), ss0 = span(s0, sbytes, "s0");
    const Span so = span(o, BH * L * d_v * es, "o"), ssf = span(s_final, sbytes, "s_final");
    const Span o_forbidden[] = {sq, sk, sv, sg, sgv, ss0, ssf};
    for (const Span &x : o_forbidden)
        if (overlap(so, x)) return fail(GLA_ERR_ALIAS, "o overlaps %s", x.name);
    const Span sf_forbidden[] = {sq, sk, sv, sg, sgv};
    for (const Span &x : sf_forbidden)
        if (overlap(ssf, x)) return fail(GLA_ERR_ALIAS, "s_final overlaps %s", x.name);
    if (overlap(ssf, ss0) && s_final != s0)
        return fail(GLA_ERR_ALIAS, "s_final partially overlaps s0");
    if (BH > 0x7fffffffUL) return fail(GLA_ERR_SHAPE, "B*H too large");
    // the prefill kernel with value-side gates: one workgroup per (head, value tile)
    gla::PrefillArgs a = {};
    a.q = q; a.k = k; a.v = v; a.g = g; a.gv = gv; a.s0 = s0; a.o = o; a.s_final = s_final;
    a.BH = (int)BH; a.L = L; a.d_v = d_v;
    a.gate = gla::kGateOuter; a.elu1 = phi == GLA_PHI_ELU1;
    const int dvt = gla::prefill_tile((int)BH, d_k, d_v, chunk, (int)es, true);
    a.n_vt = d_v / dvt;
    a.nseg = 1; a.seg_len = L; a.gam = nullptr;
    a.norm = 0; a.z0 = nullptr; a.z_final = nullptr;
    const long grid = (long)BH * a.n_vt;
    if (grid > 0x7fffffffL) return fail(GLA_ERR_SHAPE, "B*H too large");
    a.xcd_remap = (a.n_vt > 1 && grid % 8 == 0) ? 1 : 0;
    if (L == 0 && !s_final) return ok();
    const hipError_t e = gla::launch_prefill(a, dtype == GLA_BF16 ? 1 : 0, d_k, chunk, dvt, false, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "outer-gate prefill launch: %s", hipGetErrorString(e));
    return ok();
}

int gla_decode_step_outer(const void *q, const void *k, const void *v, const float *g, const float *gv,
                          float *state, void *o, int B, int H, int d_k, int d_v, gla_dtype dtype,
                          gla_feature_map phi, gla_stream_t stream)
{
    int st = check_common(B, H, d_k, d_v, dtype, GLA_GATE_KEYDIM, phi, g, true);
    if (st != GLA_OK) return st;
    if (!q || !k || !v || !gv || !state || !o)
        return fail(GLA_ERR_NULL, "q, k, v, g, gv, state and o are required");
    const void *ptrs[] = {q, k, v, gv, state, o};
    const char *names[] = {"q", "k", "v", "gv", "state", "o"};
    for (int i = 0; i < 6; ++i)
        if (!aligned16(ptrs[i])) return fail(GLA_ERR_ALIGN, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    const size_t BH = (size_t)B * H, es = elem_size(dtype);
    const Span sq = span(q, BH * d_k * es, "q"), sk = span(k, BH * d_k * es, "k");
    const Span sv = span(v, BH * d_v * es, "v"), sg = span(g, BH * d_k * 4, "g");
    const Span sgv = span(gv, BH * d_v * 4, "gv");
    const Span sst = span(state, BH * d_k * d_v * 4, "state"), so = span(o, BH * d_v * es, "o");
    const Span o_forbidden[] = {sq, sk, sv, sg, sgv, sst};
    for (const Span &x : o_forbidden)
        if (overlap(so, x)) return fail(GLA_ERR_ALIAS, "o overlaps %s", x.name);
    const Span st_forbidden[] = {sq, sk, sv, sg, sgv};
    for (const Span &x : st_forbidden)
        if (overlap(sst, x)) return fail(GLA_ERR_ALIAS, "state overlaps %s", x.name);
    if (BH > 0x7fffffffUL) return fail(GLA_ERR_SHAPE, "B*H too large");
    gla::OuterArgs a = {};
    a.q = q; a.k = k; a.v = v; a.g = g; a.gv = gv; a.s_final = state; a.o = o;
    a.BH = (int)BH; a.d_k = d_k; a.d_v = d_v; a.elu1 = phi == GLA_PHI_ELU1;
    const hipError_t e = gla::launch_outer_decode(a, dtype == GLA_BF16 ? 1 : 0, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GLA_ERR_HIP, "outer-gate decode launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
