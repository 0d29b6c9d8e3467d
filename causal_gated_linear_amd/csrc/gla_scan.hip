// gla_scan.hip -- the scan over sequence segments of a segmented prefill.
//
// A long sequence split into segments is a weighted scan over the segments' states
// ("Attention is recurrent", Prefill: the prefix states form a scan; with gates the
// state before segment p is the decayed state before segment p-1 plus what segment
// p-1 wrote).  Each segment's state from a zero start (ds) and gate totals (gam,
// log2 units) come from the state-only pass of the prefill kernel; this kernel walks
// the segments of every head in order, one thread per 4 consecutive state elements:
//
//   S = s0 (or 0);  for p: sin[p] = S;  S = exp2(gam[p][i]) * S + ds[p]
//   s_final = S
//
// It reads and writes each segment state once: a memory-bound pass.
#include <hip/hip_runtime.h>

#include "gla_device.hpp"
#include "gla_launch.hpp"

namespace gla {

__global__ __launch_bounds__(256) void segment_scan_kernel(const float *__restrict__ ds,
                                                           const float *__restrict__ gam,
                                                           const float *s0, float *__restrict__ sin,
                                                           float *s_final, int BH, int nseg, int DK,
                                                           int DV)
{
    const size_t per_head = (size_t)DK * DV;
    const size_t idx = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (idx >= (size_t)BH * per_head) return;
    const size_t bh = idx / per_head, e = idx - bh * per_head;
    const int i = (int)(e / DV);
    f32x4 S = s0 ? *(const f32x4 *)(s0 + idx) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < nseg; ++p) {
        const size_t o = (bh * nseg + p) * per_head + e;
        *(f32x4 *)(sin + o) = S;
        const float a = gam ? exp2_fast(gam[(bh * nseg + p) * DK + i]) : 1.f;
        S = a * S + *(const f32x4 *)(ds + o);
    }
    if (s_final) *(f32x4 *)(s_final + idx) = S;   // after the s0 read: s_final may be s0
}

hipError_t launch_segment_scan(const float *ds, const float *gam, const float *s0, float *sin,
                               float *s_final, int BH, int nseg, int d_k, int d_v,
                               hipStream_t stream)
{
    const size_t threads = (size_t)BH * d_k * d_v / 4;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(segment_scan_kernel, dim3(blocks), dim3(256), 0, stream, ds, gam, s0, sin,
                       s_final, BH, nseg, d_k, d_v);
    return hipGetLastError();
}

}  // namespace gla
