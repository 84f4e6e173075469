// Issue-rate probe for gfx950: how many fp32 FMA and transcendental lane
// operations a compute unit completes per second, alone and mixed.
//
// The selective scan spends one exp2 and a handful of FMA-class operations
// per token and state coordinate, so its arithmetic ceiling is set by these
// two rates and by whether a transcendental overlaps ordinary VALU work.
// Each kernel below runs NE independent exp2 chains and NF independent FMA
// chains per loop iteration in every lane, at 8 waves per SIMD (2048 blocks
// of 256 threads on 256 compute units), with no memory traffic inside the
// loop. The exp2 chains iterate a <- 2^(-a), which stays in [0.5, 0.71]; the
// FMA chains a <- a * c1 + c2 with c1 = 0.5, c2 = 0.25, which stays in
// [0.25, 0.75]. Comparing the mixed kernels' times with the sum and the max
// of the pure ones tells whether the two kinds of work overlap.
//
// A separate small library (libssprobe.so): it is measurement support for the
// benchmark, not part of the scan's API.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

template <int NE, int NF>
__global__ __launch_bounds__(kThreads) void issue_probe_kernel(float* sink, unsigned long long* clocks, int iters,
                                                               float c1, float c2) {
  float e[NE > 0 ? NE : 1], f[NF > 0 ? NF : 1];
  const float seed = 0.001f * (threadIdx.x & 63);
#pragma unroll
  for (int i = 0; i < NE; ++i) e[i] = 0.55f + seed + 0.01f * i;
#pragma unroll
  for (int i = 0; i < NF; ++i) f[i] = 0.3f + seed + 0.01f * i;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
#pragma unroll 4
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NE; ++i) e[i] = __builtin_amdgcn_exp2f(-e[i]);
#pragma unroll
    for (int i = 0; i < NF; ++i) f[i] = __builtin_fmaf(f[i], c1, c2);
  }
  if (timer) {
    clocks[0] = __builtin_amdgcn_s_memtime() - t0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NE; ++i) s += e[i];
#pragma unroll
  for (int i = 0; i < NF; ++i) s += f[i];
  // never true for the values above; keeps the chains live
  if (s == -1.0f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

using KernelFn = void (*)(float*, unsigned long long*, int, float, float);

struct Entry {
  int ne, nf;
  KernelFn fn;
};

const Entry kEntries[] = {
    {0, 8, issue_probe_kernel<0, 8>},  {8, 0, issue_probe_kernel<8, 0>},  {1, 8, issue_probe_kernel<1, 8>},
    {2, 8, issue_probe_kernel<2, 8>},  {4, 8, issue_probe_kernel<4, 8>},  {8, 8, issue_probe_kernel<8, 8>},
    {1, 4, issue_probe_kernel<1, 4>},  {1, 5, issue_probe_kernel<1, 5>},  {4, 4, issue_probe_kernel<4, 4>},
    {0, 16, issue_probe_kernel<0, 16>}, {16, 0, issue_probe_kernel<16, 0>},
    // few chains: with few waves per SIMD these expose the dependent-issue latency
    {0, 1, issue_probe_kernel<0, 1>},  {0, 2, issue_probe_kernel<0, 2>},  {0, 4, issue_probe_kernel<0, 4>},
    {1, 0, issue_probe_kernel<1, 0>},  {2, 0, issue_probe_kernel<2, 0>},  {4, 0, issue_probe_kernel<4, 0>},
};

}  // namespace

extern "C" {

// Runs the probe with ne exp2 chains and nf FMA chains per iteration (one of
// the instantiated pairs; else returns 1) over `blocks` blocks of 256
// threads and `iters` iterations, once untimed and then timed with HIP
// events on the null stream. Outputs: *ms the kernel time, *clock_mhz the
// shader clock measured inside the timed launch (s_memtime against the
// 100 MHz s_memrealtime). Returns 0 on success, 2 on a HIP error.
int ssprobe_issue(int ne, int nf, int iters, int blocks, double* ms, double* clock_mhz) {
  KernelFn fn = nullptr;
  for (const Entry& e : kEntries)
    if (e.ne == ne && e.nf == nf) fn = e.fn;
  if (!fn || iters <= 0 || blocks <= 0) return 1;
  float* sink = nullptr;
  unsigned long long* clocks = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  int rc = 2;
  if (hipMalloc(&sink, sizeof(float) * (size_t)blocks * kThreads) != hipSuccess) return 2;
  if (hipMalloc(&clocks, 2 * sizeof(unsigned long long)) != hipSuccess) goto done;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) goto done;
  {
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(kThreads), 0, 0, sink, clocks, iters, 0.5f, 0.25f);
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) goto done;
    if (hipEventRecord(a, 0) != hipSuccess) goto done;
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(kThreads), 0, 0, sink, clocks, iters, 0.5f, 0.25f);
    if (hipEventRecord(b, 0) != hipSuccess) goto done;
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(b) != hipSuccess) goto done;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, a, b) != hipSuccess) goto done;
    unsigned long long c[2] = {0, 0};
    if (hipMemcpy(c, clocks, sizeof(c), hipMemcpyDeviceToHost) != hipSuccess) goto done;
    *ms = t;
    *clock_mhz = c[1] ? 100.0 * (double)c[0] / (double)c[1] : 0.0;
    rc = 0;
  }
done:
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  if (clocks) (void)hipFree(clocks);
  if (sink) (void)hipFree(sink);
  return rc;
}

}  // extern "C"
