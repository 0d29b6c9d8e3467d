// bench_peaks.hip -- achievable peaks of the card, measured by bench.py in the same
// run as the GLA kernels, so that their fractions can be read against what this card
// delivers as well as against its datasheet:
//   peaks_stream  a streaming kernel with the headline prefill's traffic mix (five
//                 bytes read per byte written; 16-byte non-temporal accesses), in GB/s;
//   peaks_inplace an in-place scaling of 512 MiB with 16-byte non-temporal loads and
//                 stores, four per thread: the decode step's access pattern without its
//                 arithmetic, in GB/s (bytes read plus bytes written);
//   peaks_mfma    a loop of independent bf16 16x16x32 matrix-core products on
//                 register operands (no memory traffic), in TFLOP/s.
// Measurement infrastructure only: not part of the library's entry points.
#include <hip/hip_runtime.h>

#include <cstddef>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kReads = 5;                          // float4 read per float4 written

__global__ __launch_bounds__(256) void stream_mix(const f4 *in, f4 *out, size_t nout)
{
    const size_t j = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= nout) return;
    f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < kReads; ++r) s += __builtin_nontemporal_load(in + (size_t)r * nout + j);
    __builtin_nontemporal_store(s, out + j);
}

constexpr int kInplacePer = 4;                     // float4 per thread

__global__ __launch_bounds__(256) void stream_inplace(f4 *buf, size_t n)
{
    const size_t j0 = (size_t)blockIdx.x * 256 * kInplacePer + threadIdx.x;
    f4 v[kInplacePer];
#pragma unroll
    for (int r = 0; r < kInplacePer; ++r) {
        const size_t j = j0 + (size_t)r * 256;
        v[r] = j < n ? __builtin_nontemporal_load(buf + j) : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int r = 0; r < kInplacePer; ++r) {
        const size_t j = j0 + (size_t)r * 256;
        if (j < n) __builtin_nontemporal_store(v[r] * 0.5f, buf + j);
    }
}

__global__ __launch_bounds__(256) void mfma_loop(float *sink, int iters)
{
    const float t = (float)threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1e-3f * (t + e));
        b[e] = (__bf16)(1e-3f * (t - e));
    }
    f4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int i = 0; i < iters; ++i) {            // four independent accumulation chains
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
    }
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = c0[0] + c1[1] + c2[2] + c3[3];
}

// best (shortest) per-launch time in ms over `batches` timed batches of `n` launches
template <typename Launch>
int best_ms(Launch launch, int n, int batches, double *ms_out)
{
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1;
    for (int i = 0; i < n; ++i) launch();         // warm-up
    double best = 1e30;
    for (int bt = 0; bt < batches; ++bt) {
        if (hipEventRecord(e0, 0) != hipSuccess) return -1;
        for (int i = 0; i < n; ++i) launch();
        if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return -1;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return -1;
        if (ms / n < best) best = ms / n;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    *ms_out = best;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

extern "C" {

// Streaming rate of the prefill's traffic mix over 136 MiB written (816 MiB read), in
// GB/s (10^9 bytes per second).  Returns 0, or -1 on a HIP error.
int peaks_stream(double *gbs)
{
    const size_t nout = (size_t)136 << 20 >> 4;
    f4 *in = nullptr, *out = nullptr;
    if (hipMalloc(&in, kReads * nout * sizeof(f4)) != hipSuccess) return -1;
    if (hipMalloc(&out, nout * sizeof(f4)) != hipSuccess) { (void)hipFree(in); return -1; }
    int rc = hipMemset(in, 0, kReads * nout * sizeof(f4)) == hipSuccess ? 0 : -1;
    const unsigned grid = (unsigned)((nout + 255) / 256);
    double ms = 0.0;
    if (rc == 0)
        rc = best_ms([&] { hipLaunchKernelGGL(stream_mix, dim3(grid), dim3(256), 0, 0, in, out, nout); },
                     20, 5, &ms);
    (void)hipDeviceSynchronize();
    (void)hipFree(in);
    (void)hipFree(out);
    if (rc == 0) *gbs = (double)(kReads + 1) * nout * sizeof(f4) / (ms * 1e-3) / 1e9;
    return rc;
}

// In-place streaming rate over a 512 MiB buffer (read and written once per launch), in
// GB/s counting both directions.  Returns 0, or -1 on a HIP error.
int peaks_inplace(double *gbs)
{
    const size_t n = (size_t)512 << 20 >> 4;
    f4 *buf = nullptr;
    if (hipMalloc(&buf, n * sizeof(f4)) != hipSuccess) return -1;
    int rc = hipMemset(buf, 0, n * sizeof(f4)) == hipSuccess ? 0 : -1;
    const unsigned grid = (unsigned)((n + 256 * kInplacePer - 1) / (256 * kInplacePer));
    double ms = 0.0;
    if (rc == 0)
        rc = best_ms([&] { hipLaunchKernelGGL(stream_inplace, dim3(grid), dim3(256), 0, 0, buf, n); }, 20, 5, &ms);
    (void)hipDeviceSynchronize();
    (void)hipFree(buf);
    if (rc == 0) *gbs = 2.0 * n * sizeof(f4) / (ms * 1e-3) / 1e9;
    return rc;
}

// Dense bf16 matrix-core rate in TFLOP/s: 8 workgroups of 4 waves per CU, each wave
// issuing four independent 16x16x32 products per iteration.
int peaks_mfma(double *tflops)
{
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || cus <= 0) return -1;
    const unsigned grid = (unsigned)cus * 8;
    const int iters = 2000;
    float *sink = nullptr;
    if (hipMalloc(&sink, (size_t)grid * 256 * sizeof(float)) != hipSuccess) return -1;
    double ms = 0.0;
    const int rc = best_ms([&] { hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(256), 0, 0, sink, iters); },
                           5, 5, &ms);
    (void)hipDeviceSynchronize();
    (void)hipFree(sink);
    if (rc == 0) *tflops = (double)grid * 4 * iters * 4 * (16.0 * 16 * 32 * 2) / (ms * 1e-3) / 1e12;
    return rc;
}

}  // extern "C"
