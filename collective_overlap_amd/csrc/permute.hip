// Ring-permute copies for gfx950: one launch moves every shard (or
// accumulator) of one permute step -- the CollectivePermute of the looped
// CollectiveEinsum (Wang et al., ASPLOS'23, Sections 5.1 and 5.2), rank r's
// buffer to rank r-1's (and, two-way, r+1's) -- on the copy stream, beside the
// partial GEMM of the same iteration.
//
// A GEMM workgroup takes a whole compute unit (one wave per SIMD holding
// 352-512 of each lane's 512 registers), so the copy takes units from the
// GEMM for as long as its workgroups live: few workgroups (128), each with
// many bytes in flight (16 waves, four 16-byte loads per lane), no LDS and few
// registers.  A copy with nothing beside it (the two-way AllGather's
// prologue, the ReduceScatter's last permute) takes the whole GPU instead, one
// vector per thread.  Data is read once and written once, with nontemporal
// loads and stores.
//
// Item layout: one contiguous span of `width` bytes (a multiple of 16) at
// 16-byte aligned src and dst.  Every permute the plans make is one: a
// looped shard and its receive buffer share a row stride, and accumulators
// are whole buffers.  Anything else goes to the runtime's copy.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "cce_internal.hpp"

namespace cce {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct PermArgs {
  int n;
  PermuteItem it[kMaxPermuteItems];
};

constexpr int kThreads = 1024;
constexpr int kUnroll = 4;   // 16-byte loads in flight per lane

// Chunks [c0, c1) of one row (16-byte units), kUnroll loads in flight per
// lane before their stores.
__device__ __forceinline__ void copy_chunks(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                            int64_t c0, int64_t c1) {
  for (int64_t c = c0 + threadIdx.x; c < c1; c += kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (c + u * kThreads < c1) v[u] = __builtin_nontemporal_load(src + c + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (c + u * kThreads < c1) __builtin_nontemporal_store(v[u], dst + c + u * kThreads);
  }
}

// A copy with nothing beside it: one 16-byte vector per thread in many short
// workgroups, the fastest form of a plain copy on this chip (grid-stride
// loops measured 6-20% slower for every read/write mix that writes; against
// the loop over 1024 workgroups it replaced, the MLP step -0.4%, the GPT-3
// FFN step unchanged).
constexpr int kAloneThreads = 256;
__global__ __launch_bounds__(kAloneThreads) void permute_copy_alone_kernel(PermArgs a) {
  const PermuteItem& it = a.it[blockIdx.y];
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kAloneThreads + threadIdx.x;
  if (c < (it.width >> 4))
    __builtin_nontemporal_store(__builtin_nontemporal_load(static_cast<const u32x4*>(it.src) + c),
                                static_cast<u32x4*>(it.dst) + c);
}

__global__ __launch_bounds__(kThreads) void permute_copy_kernel(PermArgs a) {
  const PermuteItem& it = a.it[blockIdx.y];
  const int64_t chunks = it.width >> 4;
  // the span split evenly over the item's workgroups
  const int64_t per = (chunks + gridDim.x - 1) / gridDim.x;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t c1 = c0 + per < chunks ? c0 + per : chunks;
  copy_chunks(static_cast<const u32x4*>(it.src), static_cast<u32x4*>(it.dst), c0, c1);
}

}  // namespace

bool permute_item_ok(const PermuteItem& it) {
  const auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  return al(it.src) && al(it.dst) && it.rows == 1 && it.width >= 0 && (it.width & 15) == 0;
}

cce_status launch_permute_copy(const PermuteItem* items, int n, void* stream, bool alone) {
  if (n <= 0) return CCE_OK;
  if (n > kMaxPermuteItems) return fail(CCE_EINVAL, "permute copy: too many items");
  PermArgs k{};
  k.n = n;
  int64_t biggest = 0;
  for (int i = 0; i < n; ++i) {
    k.it[i] = items[i];
    biggest = items[i].width > biggest ? items[i].width : biggest;
  }
  if (biggest == 0) return CCE_OK;
  // 128 workgroups in all, over the items: the copy shares the GPU with the
  // GEMM beside it and spreads its HBM traffic over the GEMM's duration.
  // (256 finished sooner but slowed the GEMM's accumulate epilogues more; 64
  // or 32 made the copy outlast the GEMM it hides behind.  GPT-3 FFN two-way
  // stream form, 256-thread workgroups: 18.13 / 18.03 / 18.99 / 19.55 ms for
  // 256 / 128 / 64 / 32.)  1024-thread workgroups (four waves per SIMD, more
  // bytes in flight per compute unit) measured 18.09 against 18.22 ms for 256
  // threads in the same process; many short-lived workgroups of 512 KB or
  // 2 MB each were slower (18.26 and 18.44 ms; 3.34 and 3.41 against 3.03 ms
  // on the 8-way fp32 ReduceScatter).
  constexpr int kUnits = 128;
  const int64_t chunks = biggest / 16;
  if (alone) {
    // A copy with nothing beside it takes the whole GPU, one vector per thread.
    const int64_t blocks = (chunks + kAloneThreads - 1) / kAloneThreads;
    if (blocks > 0x7fffffff) return fail(CCE_EUNSUPPORTED, "permute copy: item too large");
    hipLaunchKernelGGL(permute_copy_alone_kernel, dim3(static_cast<unsigned>(blocks), n),
                       dim3(kAloneThreads), 0, static_cast<hipStream_t>(stream), k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CCE_EHIP, std::string("permute copy launch: ") + hipGetErrorString(e));
    return CCE_OK;
  }
  int per_item = (kUnits + n - 1) / n;
  if (per_item > chunks / (kThreads * kUnroll) + 1) per_item = static_cast<int>(chunks / (kThreads * kUnroll) + 1);
  hipLaunchKernelGGL(permute_copy_kernel, dim3(per_item, n), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), k);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CCE_EHIP, std::string("permute copy launch: ") + hipGetErrorString(e));
  return CCE_OK;
}

}  // namespace cce
