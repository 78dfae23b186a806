// Philox4x32-10 on the device (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11): ten rounds of the 4x32 bijection
// with the published multipliers, the key bumped by the Weyl increments (the
// 32-bit fractions of the golden ratio and of sqrt(3)) between rounds.
//
// The dropout keep mask of the fused reduce epilogue draws from it: element
// e (a global element index) takes word e & 3 of the block whose counter is
// (lo(e >> 2), hi(e >> 2), lo(offset), hi(offset)) under the key
// (lo(seed), hi(seed)), and is kept iff that word >= floor(p * 2^32).
// Shared by the standalone epilogue kernels and the consumer that runs inside
// the ReduceScatter's last GEMM launch, so both draw the same mask.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cce {

struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(kM0) * c0;
    const uint64_t p1 = static_cast<uint64_t>(kM1) * c2;
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
    k0 += kW0;
    k1 += kW1;
  }
  return Philox4{{c0, c1, c2, c3}};
}

__device__ __forceinline__ uint32_t philox_pick(const Philox4& x, uint32_t i) {
  return i == 0 ? x.w[0] : (i == 1 ? x.w[1] : (i == 2 ? x.w[2] : x.w[3]));
}

// The block of mask words for block index blk (= e >> 2).
__device__ __forceinline__ Philox4 philox_block(uint64_t blk, uint32_t off0, uint32_t off1,
                                                uint32_t key0, uint32_t key1) {
  return philox10(static_cast<uint32_t>(blk), static_cast<uint32_t>(blk >> 32), off0, off1, key0,
                  key1);
}

}  // namespace cce
