// gla_scan.hip -- the scan over sequence segments of a segmented prefill.
//
// A long sequence split into segments is a weighted scan over the segments' states
// ("Attention is recurrent", Prefill: the prefix states form a scan; with gates the
// state before segment p is the decayed state before segment p-1 plus what segment
// p-1 wrote).  Each segment's state from a zero start (ds) and gate totals (gam,
// log2 units) come from the state-only pass of the prefill kernel, for every segment
// but the last; this kernel walks the segments of every head in order, one thread per
// 4 consecutive state elements:
//
//   S = s0 (or 0);  for p < nseg: sin[p] = S;  if p < nseg - 1: S = exp2(gam[p][i]) * S + ds[p]
//
// The full pass then runs every segment from sin[p]; the last segment's final state
// is the sequence's.
// It reads and writes each segment state once: a memory-bound pass.
#include <hip/hip_runtime.h>

#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

__global__ __launch_bounds__(256) void segment_scan_kernel(const float *__restrict__ ds,
                                                           const float *__restrict__ gam,
                                                           const float *s0, float *__restrict__ sin,
                                                           int BH, int nseg, int DK, int DV)
{
    const size_t per_head = (size_t)DK * DV;
    const size_t idx = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (idx >= (size_t)BH * per_head) return;
    const size_t bh = idx / per_head, e = idx - bh * per_head;
    const int i = (int)(e / DV);
    const int ns = nseg - 1;                       // segments with a stored state
    f32x4 S = s0 ? *(const f32x4 *)(s0 + idx) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < nseg; ++p) {
        *(f32x4 *)(sin + (bh * nseg + p) * per_head + e) = S;
        if (p < ns) {
            const size_t o = (bh * ns + p) * per_head + e;
            const float a = gam ? exp2_fast(gam[(bh * ns + p) * DK + i]) : 1.f;
            S = a * S + *(const f32x4 *)(ds + o);
        }
    }
}

hipError_t launch_segment_scan(const float *ds, const float *gam, const float *s0, float *sin,
                               int BH, int nseg, int d_k, int d_v, hipStream_t stream)
{
    const size_t threads = (size_t)BH * d_k * d_v / 4;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(segment_scan_kernel, dim3(blocks), dim3(256), 0, stream, ds, gam, s0, sin,
                       BH, nseg, d_k, d_v);
    return hipGetLastError();
}

}  // namespace gla
