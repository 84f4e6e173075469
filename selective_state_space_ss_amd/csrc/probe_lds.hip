// LDS bank probe for gfx950: one wave reads or writes 4, 8 or 16 bytes per
// lane at per-lane byte offsets from a table, `iters` times, each access
// waited for before the next. Run under rocprofv3 --pmc SQ_LDS_BANK_CONFLICT
// SQ_INSTS_LDS, one launch per offset pattern, it gives the conflict cycles
// each pattern costs per instruction: how many lanes the LDS serves at once
// for each access width, over how many banks. The scan's and dt_proj's LDS
// layouts are checked against these measurements.
//
// Part of libssprobe.so (measurement support for the benchmark, not part of
// the scan's API).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWords = 16384;  // 64 KB of LDS; offsets must stay below 64 KB - 16

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

template <int WIDTH, bool WRITE>
__global__ __launch_bounds__(64) void lds_probe_kernel(const int* __restrict__ offsets, int iters, float* out) {
  __shared__ __align__(16) float lds[kWords];
  const int l = threadIdx.x;
  for (int i = l; i < kWords; i += 64) lds[i] = static_cast<float>(i);
  __syncthreads();
  // (an offset outside the array is clamped into it, aligned to the width)
  int off = offsets[l];
  off = off < 0 ? 0 : (off > 4 * kWords - 16 ? 4 * kWords - 16 : off);
  off &= ~(WIDTH - 1);
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + static_cast<uint32_t>(off);
  float acc = 0.0f;
  for (int it = 0; it < iters; ++it) {
    // (each access in its own asm block with its wait, so that neither is
    // moved, merged or hoisted out of the loop)
    if constexpr (WRITE) {
      if constexpr (WIDTH == 16) {
        const f4 v = {acc, acc, acc, acc};
        asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(v) : "memory");
      } else if constexpr (WIDTH == 8) {
        const f2 v = {acc, acc};
        asm volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(v) : "memory");
      } else {
        asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(acc) : "memory");
      }
    } else {
      if constexpr (WIDTH == 16) {
        f4 v;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
        acc += v.x + v.w;
      } else if constexpr (WIDTH == 8) {
        f2 v;
        asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
        acc += v.x + v.y;
      } else {
        float v;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
        acc += v;
      }
    }
    acc += 1.0f;
  }
  out[l] = acc;
}

template <int WIDTH>
hipError_t launch(const int* offsets, int iters, bool write, float* out, hipStream_t s) {
  void* args[] = {&offsets, &iters, &out};
  const void* fn = write ? reinterpret_cast<const void*>(&lds_probe_kernel<WIDTH, true>)
                         : reinterpret_cast<const void*>(&lds_probe_kernel<WIDTH, false>);
  return hipLaunchKernel(fn, dim3(1), dim3(64), args, 0, s);
}

}  // namespace

// offsets_dev: 64 device ints, byte offsets (multiples of width, below 64 KB -
// 16); width 4, 8 or 16; out_dev: 64 device floats. Returns 0, or -1 for a
// bad argument, or the HIP error of the launch.
extern "C" int ssprobe_lds(const int* offsets_dev, int width, int iters, int write, float* out_dev, void* stream) {
  if (!offsets_dev || !out_dev || iters < 0) return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (width == 16) e = launch<16>(offsets_dev, iters, write != 0, out_dev, s);
  else if (width == 8) e = launch<8>(offsets_dev, iters, write != 0, out_dev, s);
  else if (width == 4) e = launch<4>(offsets_dev, iters, write != 0, out_dev, s);
  else return -1;
  return static_cast<int>(e);
}
