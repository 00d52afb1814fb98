// Measured roofline denominators on the running GPU, printed as one JSON line:
//   hbm_read_gbs   streaming 128-bit reads of a 4 GiB buffer (every CU busy)
//   copy_gbs       a plain 4 GiB -> 4 GiB copy (also the known-size kernel used
//                  to calibrate the FETCH_SIZE / WRITE_SIZE counters)
//   mfma_bf16_tflops  independent v_mfma_f32_32x32x16_bf16 chains, 4 per wave
//   lds_read_bytes_per_clk_cu  conflict-free ds_read_b128 per CU per clock
//   graph_node_us  per-node time of a hipGraph of empty kernels
// Usage: mla_peaks [copy_only]

#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define CK(x)                                                                              \
  do {                                                                                     \
    hipError_t e_ = (x);                                                                   \
    if (e_ != hipSuccess) {                                                                \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(1);                                                                             \
    }                                                                                      \
  } while (0)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void read_kernel(const float4* __restrict__ src, size_t n, float* sink) {
  float acc = 0.f;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride * 4) {
    float4 a = src[i];
    float4 b = i + stride < n ? src[i + stride] : float4{};
    float4 c = i + 2 * stride < n ? src[i + 2 * stride] : float4{};
    float4 d = i + 3 * stride < n ? src[i + 3 * stride] : float4{};
    acc += a.x + b.y + c.z + d.w;
  }
  if (acc == 12345.678f) sink[0] = acc;  // keeps the loads alive
}

__global__ __launch_bounds__(256) void copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                   size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* sink) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * (threadIdx.x + i));
    b[i] = static_cast<__bf16>(0.002f * (threadIdx.x - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == 12345.678f) sink[0] = s;
}

__global__ __launch_bounds__(256) void lds_kernel(int iters, float* sink) {
  __shared__ __attribute__((aligned(16))) float4 buf[4096];  // 64 KiB
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = float4{1.f * i, 0.f, 0.f, 0.f};
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float4 acc = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 v = buf[((it * 8 + k + wave * 16) & 63) * 64 + lane];  // 1 KiB contiguous per wave read
      acc.x += v.x;
      acc.y += v.y;
    }
  }
  if (acc.x + acc.y == 12345.678f) sink[0] = acc.x;
}

__global__ void empty_kernel() {}

static float time_ms(hipEvent_t a, hipEvent_t b) {
  float ms = 0.f;
  CK(hipEventElapsedTime(&ms, a, b));
  return ms;
}

int main(int argc, char** argv) {
  const bool copy_only = argc > 1 && strcmp(argv[1], "copy_only") == 0;
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const double clk_ghz = prop.clockRate / 1e6;
  const size_t bytes = 4ull << 30;
  const size_t n = bytes / 16;
  float4 *src = nullptr, *dst = nullptr;
  float* sink = nullptr;
  CK(hipMalloc(&src, bytes));
  CK(hipMalloc(&dst, bytes));
  CK(hipMalloc(&sink, 64));
  CK(hipMemset(src, 0, bytes));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  const int grid = cus * 16;

  // plain copy (also the counter calibration kernel: 4 GiB read, 4 GiB written)
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, 0, src, dst, n);
  CK(hipDeviceSynchronize());
  const int copy_reps = 3;
  CK(hipEventRecord(e0));
  for (int r = 0; r < copy_reps; ++r) hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, 0, src, dst, n);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  const double copy_gbs = 2.0 * bytes * copy_reps / (time_ms(e0, e1) * 1e-3) / 1e9;
  if (copy_only) {
    printf("{\"copy_bytes_read\": %zu, \"copy_bytes_written\": %zu, \"copy_gbs\": %.1f}\n", bytes, bytes, copy_gbs);
    return 0;
  }

  // streaming read
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, 0, src, n, sink);
  CK(hipDeviceSynchronize());
  const int read_reps = 5;
  CK(hipEventRecord(e0));
  for (int r = 0; r < read_reps; ++r) hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, 0, src, n, sink);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  const double read_gbs = static_cast<double>(bytes) * read_reps / (time_ms(e0, e1) * 1e-3) / 1e9;

  // MFMA: 4 waves per CU (one per SIMD), 4 independent accumulators each
  const int iters = 20000;
  hipLaunchKernelGGL(mfma_kernel, dim3(cus), dim3(256), 0, 0, 10, sink);
  CK(hipDeviceSynchronize());
  CK(hipEventRecord(e0));
  hipLaunchKernelGGL(mfma_kernel, dim3(cus * 2), dim3(256), 0, 0, iters, sink);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  const double flops = static_cast<double>(cus) * 2 * 4 * iters * 4 * 32.0 * 32 * 16 * 2;
  const double mfma_tflops = flops / (time_ms(e0, e1) * 1e-3) / 1e12;

  // LDS reads: 2 workgroups of 4 waves per CU
  const int lds_iters = 20000;
  hipLaunchKernelGGL(lds_kernel, dim3(cus), dim3(256), 0, 0, 10, sink);
  CK(hipDeviceSynchronize());
  CK(hipEventRecord(e0));
  hipLaunchKernelGGL(lds_kernel, dim3(cus * 2), dim3(256), 0, 0, lds_iters, sink);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  const double lds_ms = time_ms(e0, e1);
  const double lds_bytes = static_cast<double>(cus) * 2 * 4 * lds_iters * 8 * 1024.0;
  const double lds_bpc = lds_bytes / (lds_ms * 1e-3) / (clk_ghz * 1e9) / cus;

  // hipGraph of empty kernels
  hipStream_t st;
  CK(hipStreamCreate(&st));
  hipGraph_t g;
  hipGraphExec_t ge;
  const int nodes = 1000;
  CK(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
  for (int i = 0; i < nodes; ++i) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, st);
  CK(hipStreamEndCapture(st, &g));
  CK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
  CK(hipGraphLaunch(ge, st));
  CK(hipStreamSynchronize(st));
  CK(hipEventRecord(e0, st));
  CK(hipGraphLaunch(ge, st));
  CK(hipEventRecord(e1, st));
  CK(hipEventSynchronize(e1));
  const double node_us = time_ms(e0, e1) * 1e3 / nodes;

  printf("{\"device\": \"%s\", \"cus\": %d, \"clock_ghz\": %.3f, \"hbm_read_gbs\": %.1f, \"copy_gbs\": %.1f, "
         "\"mfma_bf16_tflops\": %.1f, \"lds_read_bytes_per_clk_cu\": %.1f, \"graph_node_us\": %.3f}\n",
         prop.gcnArchName, cus, clk_ghz, read_gbs, copy_gbs, mfma_tflops, lds_bpc, node_us);
  CK(hipGraphExecDestroy(ge));
  CK(hipGraphDestroy(g));
  CK(hipStreamDestroy(st));
  CK(hipFree(src));
  CK(hipFree(dst));
  CK(hipFree(sink));
  return 0;
}
