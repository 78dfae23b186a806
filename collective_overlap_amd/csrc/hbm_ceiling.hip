// hbm_ceiling: what HBM sustains on this GPU for plain streaming kernels --
// the ceiling an HBM-bound kernel such as the fused reduce epilogue could
// reach if it did nothing but move its bytes.
//
// Each kernel reads R streams and writes W (0 or 1) stream of 16-byte
// vectors, element i of the output being the XOR of element i of the
// inputs, in a grid-stride loop that issues U vectors per stream and thread
// before using any of them.  Mixes:
//   - read only (R = 1, W = 0; the XOR is kept in a register and written
//     only if it equals a value it never takes, so the loads stay);
//   - write only (R = 0, W = 1);
//   - copy (R = 1, W = 1);
//   - R = 3, 5, 9 reads per write: the byte mixes of the fused epilogue
//     (one fp32 accumulator and a bf16 residual per bf16 output; two fp32
//     accumulators and a residual; eight bf16 partials and a residual).
// Swept: U in {1, 2, 4, 8} (at most 32 vectors in flight per thread),
// plain or nontemporal accesses, and the grid: 512 .. 8192 workgroups of 256
// threads looping over the streams, or one vector per thread with no loop.
// Every stream is 1 GiB, four times the 256 MB memory-side cache.
//
// Every index is below the stream length; prints one JSON object per
// measurement (GB/s = bytes moved / time, over `reps` back-to-back launches).
//
// Usage: hbm_ceiling [reps] (default 5)

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
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

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxR = 9;
constexpr int kThreads = 256;
constexpr int64_t kVecs = int64_t{1} << 26;   // 16-byte vectors per stream: 1 GiB
constexpr unsigned kNever = 0x9e3779b9u;      // the read-only XOR never equals this in every word

struct Args {
  const u32x4* src[kMaxR];
  u32x4* dst;
  int64_t n;
};

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int R, bool W, int U, bool NT>
__global__ __launch_bounds__(kThreads) void stream_kernel(Args a) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  u32x4 keep = {0u, 0u, 0u, 0u};
  auto one = [&](int64_t j, const u32x4 (&v)[R > 0 ? R : 1]) {
    u32x4 x = {static_cast<unsigned>(j), 1u, 2u, 3u};
#pragma unroll
    for (int r = 0; r < R; ++r) x ^= v[r];
    if constexpr (W) st<NT>(a.dst + j, x);
    else keep ^= x;
  };
  for (; i + (U - 1) * stride < a.n; i += U * stride) {
    u32x4 v[U][R > 0 ? R : 1];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) v[u][r] = ld<NT>(a.src[r] + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) one(i + u * stride, v[u]);
  }
  for (; i < a.n; i += stride) {
    u32x4 v[R > 0 ? R : 1];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = ld<NT>(a.src[r] + i);
    one(i, v);
  }
  if constexpr (!W) {
    if (keep.x == kNever && keep.y == kNever && keep.z == kNever && keep.w == kNever)
      a.dst[threadIdx.x] = keep;
  }
}

using Kernel = void (*)(Args);

struct Variant {
  int r, w, u, nt;
  Kernel k;
};

template <int R, bool W, int U>
void add(std::vector<Variant>& v) {
  if constexpr (U * (R > 0 ? R : 1) <= 32) {
    v.push_back({R, W, U, 0, stream_kernel<R, W, U, false>});
    v.push_back({R, W, U, 1, stream_kernel<R, W, U, true>});
  }
}

template <int R, bool W>
void add_u(std::vector<Variant>& v) {
  add<R, W, 1>(v);
  add<R, W, 2>(v);
  add<R, W, 4>(v);
  add<R, W, 8>(v);
}

const char* mix_name(int r, int w) {
  if (w == 0) return "read";
  if (r == 0) return "write";
  if (r == 1) return "copy";
  if (r == 3) return "3:1";
  if (r == 5) return "5:1";
  return "9:1";
}

}  // namespace

int main(int argc, char** argv) {
  const int reps = argc > 1 ? std::atoi(argv[1]) : 5;
  if (reps < 1) {
    std::fprintf(stderr, "reps must be >= 1\n");
    return 1;
  }
  std::vector<Variant> vars;
  add_u<1, false>(vars);
  add_u<0, true>(vars);
  add_u<1, true>(vars);
  add_u<3, true>(vars);
  add_u<5, true>(vars);
  add_u<9, true>(vars);

  const size_t bytes = static_cast<size_t>(kVecs) * 16;
  Args a{};
  std::vector<void*> bufs;
  for (int r = 0; r < kMaxR + 1; ++r) {
    void* p = nullptr;
    CHECK(hipMalloc(&p, bytes));
    CHECK(hipMemset(p, r + 1, bytes));
    bufs.push_back(p);
  }
  for (int r = 0; r < kMaxR; ++r) a.src[r] = static_cast<const u32x4*>(bufs[r]);
  a.dst = static_cast<u32x4*>(bufs[kMaxR]);
  a.n = kVecs;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  // 0: one vector per thread, no loop
  const int grids[] = {512, 1024, 2048, 4096, 8192, 0};
  for (const Variant& v : vars) {
    for (int g : grids) {
      if (g == 0 && v.u != 1) continue;
      const int64_t blocks = g ? g : (kVecs + kThreads - 1) / kThreads;
      const dim3 grid(static_cast<unsigned>(blocks));
      hipLaunchKernelGGL(v.k, grid, dim3(kThreads), 0, 0, a);   // warm-up
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e0, 0));
      for (int i = 0; i < reps; ++i) hipLaunchKernelGGL(v.k, grid, dim3(kThreads), 0, 0, a);
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1, 0));
      CHECK(hipEventSynchronize(e1));
      float ms = 0.0f;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      const double moved = static_cast<double>(v.r + v.w) * bytes * reps;
      std::printf("{\"mix\": \"%s\", \"reads\": %d, \"writes\": %d, \"unroll\": %d, \"nontemporal\": %s, "
                  "\"workgroups\": %lld, \"loop\": %s, \"ms_per_launch\": %.4f, \"GB/s\": %.1f}\n",
                  mix_name(v.r, v.w), v.r, v.w, v.u, v.nt ? "true" : "false",
                  static_cast<long long>(blocks), g ? "true" : "false", ms / reps,
                  moved / (ms * 1e-3) / 1e9);
      std::fflush(stdout);
    }
  }
  for (void* p : bufs) CHECK(hipFree(p));
  return 0;
}
