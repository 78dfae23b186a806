// mfma_ceiling: what the matrix cores sustain on this GPU when nothing but
// MFMAs and their LDS operand reads run -- the ceiling a GEMM k loop could
// reach if its global loads, barriers and epilogue were free.
//
// One workgroup per compute unit (256 threads, four waves, one per SIMD),
// each wave computing a 128 x 128 tile with a 32-deep k step per iteration,
// the wave tile of the grouped GEMM.  Every iteration reads fresh operand
// fragments (16 bytes per lane each) from a 64 KB LDS array filled once
// from device memory, so the operands change every step as in a GEMM.
// Variants:
//   - 32x32x16 bf16 MFMAs (the GEMM's instruction): 32 per iteration;
//   - 16x16x32 bf16 MFMAs: 64 per iteration, the same FLOPs;
//   - 32x32x16 on all-zero operands: the same instruction stream with
//     nothing toggling in the multipliers.
// If the rate depends on the operand values, the clock is set by power, not
// by the instruction count.
//
// Every LDS index is masked to the array; global reads are reduced modulo the
// source length; each thread writes its own output word once.  Prints one
// JSON object per measurement.
//
// Usage: mfma_ceiling [iterations per launch] (default 200000)

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLds = 4096;          // 16-byte entries: 64 KB
constexpr int kSrc = 1 << 20;       // 16-byte entries: 16 MB source
constexpr int kGrid = 256;          // one workgroup per compute unit
constexpr int kThreads = 256;

template <int MODE>  // 0: 32x32x16, 1: 16x16x32
__global__ __launch_bounds__(kThreads) void mfma_loop(const u32x4* src, float* out, int iters) {
  __shared__ u32x4 lds[kLds];
  for (int i = threadIdx.x; i < kLds; i += kThreads) lds[i] = src[(blockIdx.x * kLds + i) % kSrc];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float s = 0.0f;
  if constexpr (MODE == 0) {
    f32x16 acc[4][4];
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int base = (it * 2 + ks) * 512 + wave * 64 + lane;
        bf16x8 fa[4], fb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          fa[q] = __builtin_bit_cast(bf16x8, lds[(base + q * 256) & (kLds - 1)]);
          fb[q] = __builtin_bit_cast(bf16x8, lds[(base + 1024 + q * 256 + 128) & (kLds - 1)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[i], fa[j], acc[i][j], 0, 0, 0);
      }
    }
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  } else {
    f32x4 acc[8][8];
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};
    for (int it = 0; it < iters; ++it) {
      const int base = it * 1024 + wave * 64 + lane;
      bf16x8 fa[8], fb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        fa[q] = __builtin_bit_cast(bf16x8, lds[(base + q * 256) & (kLds - 1)]);
        fb[q] = __builtin_bit_cast(bf16x8, lds[(base + 2048 + q * 256 + 128) & (kLds - 1)]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[i], fa[j], acc[i][j], 0, 0, 0);
    }
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 8; ++j)
        for (int e = 0; e < 4; ++e) s += acc[i][j][e];
  }
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 200000;
  if (iters < 1) {
    std::fprintf(stderr, "iterations must be positive\n");
    return 2;
  }
  // bf16 N(0, 1) operands (the upper half of the float's bits)
  std::vector<uint16_t> h(static_cast<size_t>(kSrc) * 8);
  std::mt19937 rng(1);
  std::normal_distribution<float> nd(0.0f, 1.0f);
  for (auto& x : h) {
    const float f = nd(rng);
    uint32_t u;
    std::memcpy(&u, &f, 4);
    x = static_cast<uint16_t>(u >> 16);
  }
  u32x4 *rnd = nullptr, *zero = nullptr;
  float* out = nullptr;
  CHECK(hipMalloc(&rnd, sizeof(u32x4) * kSrc));
  CHECK(hipMalloc(&zero, sizeof(u32x4) * kSrc));
  CHECK(hipMalloc(&out, sizeof(float) * kGrid * kThreads));
  CHECK(hipMemcpy(rnd, h.data(), sizeof(u32x4) * kSrc, hipMemcpyHostToDevice));
  CHECK(hipMemset(zero, 0, sizeof(u32x4) * kSrc));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  struct Variant { const char* mfma; const char* operands; int mode; const u32x4* src; };
  const Variant vars[] = {{"32x32x16", "random bf16 N(0,1)", 0, rnd},
                          {"16x16x32", "random bf16 N(0,1)", 1, rnd},
                          {"32x32x16", "zeros", 0, zero}};
  constexpr int kLaunches = 3, kReps = 3;
  const double flops = double(kLaunches) * kGrid * 4 * double(iters) * 128 * 128 * 32 * 2;
  for (int rep = 0; rep < kReps; ++rep) {
    for (const Variant& v : vars) {
      CHECK(hipEventRecord(e0));
      for (int l = 0; l < kLaunches; ++l) {
        if (v.mode == 0)
          hipLaunchKernelGGL(mfma_loop<0>, dim3(kGrid), dim3(kThreads), 0, 0, v.src, out, iters);
        else
          hipLaunchKernelGGL(mfma_loop<1>, dim3(kGrid), dim3(kThreads), 0, 0, v.src, out, iters);
      }
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0.0f;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      std::printf("{\"rep\": %d, \"mfma\": \"%s\", \"operands\": \"%s\", \"ms\": %.3f, "
                  "\"TFLOP/s\": %.1f}\n",
                  rep, v.mfma, v.operands, ms, flops / (ms * 1e-3) / 1e12);
      std::fflush(stdout);
    }
  }
  CHECK(hipFree(rnd));
  CHECK(hipFree(zero));
  CHECK(hipFree(out));
  return 0;
}
