// Measured throughput ceilings (dense bf16 MFMA, HBM streaming in the block-diagonal mix) that
// serve as the second denominator of the attention kernels' roofline.  Calibration only; the
// attention library does not link or call this file.
#include <hip/hip_runtime.h>

#include "../../include/attn_ceilings.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned int u32x4 __attribute__((__vector_size__(16)));

constexpr int kMfmaPerWave = 4096;
constexpr int kThreads = 256;              // four waves per workgroup, one per SIMD
constexpr int kMfmaGroupsPerCu = 2;        // two workgroups per CU: two waves per SIMD
constexpr int kStreamGroupsPerCu = 16;
constexpr int kStreamUnroll = 2;

// Integer hash (xorshift-multiply) that turns thread and slot indices into operand bits.
__device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ float uniform_pm2(unsigned bits) {
  return (float)(bits >> 8) * (4.0f / 16777216.0f) - 2.0f;   // [-2, 2)
}

// Eight operand pairs held in registers and used in rotation, so consecutive MFMAs read
// different registers; four independent accumulator chains.
__global__ __launch_bounds__(kThreads) void mfma_burn(float* out, unsigned seed) {
  bf16x8 a[8], b[8];
  const unsigned t = blockIdx.x * kThreads + threadIdx.x;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[j][i] = (__bf16)uniform_pm2(mix(t * 131u + j * 17u + i + seed));
      b[j][i] = (__bf16)uniform_pm2(mix(t * 257u + j * 29u + i + 3u * seed));
    }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < kMfmaPerWave / 8; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + 3) & 7], acc[j & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[t] = s;   // keeps the MFMAs live
}

// d = a ^ b ^ c over n 16-byte elements, grid-stride.
__global__ __launch_bounds__(kThreads) void stream_3r1w(const u32x4* __restrict__ a,
                                                        const u32x4* __restrict__ b,
                                                        const u32x4* __restrict__ c,
                                                        u32x4* __restrict__ d, size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads * kStreamUnroll;
  for (size_t i = (size_t)blockIdx.x * kThreads * kStreamUnroll + threadIdx.x; i < n; i += stride) {
    u32x4 x[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t j = i + (size_t)u * kThreads;
      if (j < n)
        x[u] = __builtin_nontemporal_load(&a[j]) ^ __builtin_nontemporal_load(&b[j]) ^
               __builtin_nontemporal_load(&c[j]);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t j = i + (size_t)u * kThreads;
      if (j < n) __builtin_nontemporal_store(x[u], &d[j]);
    }
  }
}

int compute_units(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  return (int)e;
}

// warmup untimed launches, then `launches` timed ones between two events on the default stream.
template <class Launch>
int time_launches(int warmup, int launches, Launch launch, float* ms) {
  for (int i = 0; i < warmup; ++i) launch();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if ((e = hipEventCreate(&e0)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&e1)) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return (int)e;
  }
  e = hipEventRecord(e0, nullptr);
  for (int i = 0; i < launches && e == hipSuccess; ++i) launch();
  if (e == hipSuccess) e = hipGetLastError();
  if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return (int)e;
}

}  // namespace

extern "C" {

int attn_ceiling_mfma_bf16(int warmup, int launches, double* tflops) {
  if (warmup < 0 || launches < 1 || tflops == nullptr) return (int)hipErrorInvalidValue;
  int cus = 0;
  int st = compute_units(&cus);
  if (st != 0) return st;
  const int grid = cus * kMfmaGroupsPerCu;
  float* out = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)grid * kThreads * sizeof(float));
  if (e != hipSuccess) return (int)e;
  unsigned seed = 12345u;
  float ms = 0.f;
  st = time_launches(warmup, launches, [&] {
    hipLaunchKernelGGL(mfma_burn, dim3(grid), dim3(kThreads), 0, nullptr, out, seed++);
  }, &ms);
  const hipError_t ef = hipFree(out);
  if (st != 0) return st;
  if (ef != hipSuccess) return (int)ef;
  const double flops = (double)grid * (kThreads / 64) * kMfmaPerWave * (32.0 * 32.0 * 16.0 * 2.0);
  *tflops = launches * flops / (ms * 1e-3) / 1e12;
  return 0;
}

int attn_ceiling_hbm_3r1w(int warmup, int launches, size_t bytes_per_array, double* gbs) {
  if (warmup < 0 || launches < 1 || gbs == nullptr || bytes_per_array == 0 || bytes_per_array % 16 != 0)
    return (int)hipErrorInvalidValue;
  int cus = 0;
  int st = compute_units(&cus);
  if (st != 0) return st;
  u32x4* buf[4] = {nullptr, nullptr, nullptr, nullptr};
  hipError_t e = hipSuccess;
  for (int i = 0; i < 4 && e == hipSuccess; ++i) {
    e = hipMalloc(&buf[i], bytes_per_array);
    if (e == hipSuccess && i < 3) e = hipMemset(buf[i], 0x11 * (i + 1), bytes_per_array);
  }
  float ms = 0.f;
  if (e == hipSuccess) {
    const size_t n = bytes_per_array / 16;
    const int grid = cus * kStreamGroupsPerCu;
    st = time_launches(warmup, launches, [&] {
      hipLaunchKernelGGL(stream_3r1w, dim3(grid), dim3(kThreads), 0, nullptr, buf[0], buf[1], buf[2],
                         buf[3], n);
    }, &ms);
  } else {
    st = (int)e;
  }
  for (int i = 0; i < 4; ++i)
    if (buf[i] != nullptr) {
      const hipError_t ef = hipFree(buf[i]);
      if (st == 0 && ef != hipSuccess) st = (int)ef;
    }
  if (st != 0) return st;
  *gbs = launches * 4.0 * (double)bytes_per_array / (ms * 1e-3) / 1e9;
  return 0;
}

}  // extern "C"
