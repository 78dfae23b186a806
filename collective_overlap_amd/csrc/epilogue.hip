// Fused reduce epilogue for gfx950:
//
//   out = residual + keep * (sum_k partials[k] + bias) * scale
//
// CoCoNet (Jangda et al., ASPLOS'22), the Figure 3 program and its
// FusedAllReduce: the sum that the AllReduce produces is consumed by the bias
// add, the dropout and the residual add while it is still in registers, so
// the reduced tensor is never stored and reloaded.  Here the N partials are
// N rank buffers in one HBM: every operand is read exactly once and the
// output written exactly once; the keep mask costs no memory traffic.
//
// Work unit: 8 consecutive columns of one row ("vector").  A 64-lane wave
// covers 512 consecutive columns, so every operand load is a fully coalesced
// 16-byte-per-lane access (two for fp32), and all N partial loads plus the
// residual load of a lane are issued before the first add.
//
// Arithmetic order is fixed and contraction is off: ((p0 + p1) + ...) + bias,
// times scale if kept (else 0), plus residual, each in fp32; one
// round-to-nearest-even conversion to the output type.
//
// Keep mask: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11) keyed by the seed, with counter
// (e >> 2, offset) for the global element index e; word e & 3 decides e.
// When 8 | row stride and 4 | start column, one vector needs exactly two
// Philox blocks.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "cce_internal.hpp"
#include "philox.hpp"

#pragma clang fp contract(off)

namespace cce {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct EArgs {
  const void* parts[kMaxGroups];   // [batch * n + k]
  const void* res[kMaxGroups];     // per batch entry (NULL: no residual)
  void* out[kMaxGroups];           // [batch * n_rep + q]: every replica gets the result
  int n_rep;
  uint8_t* mask[kMaxGroups];       // per batch entry (NULL: no mask output)
  int64_t mrow0[kMaxGroups];
  int n;
  int rows, cols;
  int64_t ld_part, ld_res, ld_out;
  const void* bias;
  uint32_t threshold;
  int mode;                 // 0: no dropout, 1: dropout, 2: drop everything
  float scale;
  uint32_t key0, key1, off0, off1;
  int64_t mcol0, mld;
  bool aligned;             // 4 | mld and 4 | mcol0: two Philox blocks per vector
};

// ---- Philox4x32-10 (philox.hpp) -------------------------------------------
__device__ __forceinline__ uint32_t pick(const Philox4& x, uint32_t i) { return philox_pick(x, i); }

__device__ __forceinline__ Philox4 block_for(const EArgs& a, uint64_t blk) {
  return philox_block(blk, a.off0, a.off1, a.key0, a.key1);
}

// ---- typed loads / stores -------------------------------------------------
// Partials, residual and output are touched exactly once: their vector loads
// and stores are nontemporal (streamed past the caches).  The bias, reused by
// every row, takes plain loads.
template <typename T, bool NT>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + idx);
    f32x4 x, y;
    if constexpr (NT) {
      x = __builtin_nontemporal_load(p);
      y = __builtin_nontemporal_load(p + 1);
    } else {
      x = p[0];
      y = p[1];
    }
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
    v[4] = y[0]; v[5] = y[1]; v[6] = y[2]; v[7] = y[3];
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(base) + idx);
    u32x4 w;
    if constexpr (NT) w = __builtin_nontemporal_load(p);
    else w = *p;
    const bf16x8 x = __builtin_bit_cast(bf16x8, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(x[e]);
  }
}

template <typename T>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (sizeof(T) == 4) return reinterpret_cast<const float*>(base)[idx];
  else return static_cast<float>(reinterpret_cast<const __bf16*>(base)[idx]);
}

template <typename T>
__device__ __forceinline__ void store8(void* base, int64_t idx, const float (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, p);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, p + 1);
  } else {
    bf16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = static_cast<__bf16>(v[e]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h),
                                reinterpret_cast<u32x4*>(reinterpret_cast<__bf16*>(base) + idx));
  }
}

template <typename T>
__device__ __forceinline__ void store1(void* base, int64_t idx, float v) {
  if constexpr (sizeof(T) == 4) reinterpret_cast<float*>(base)[idx] = v;
  else reinterpret_cast<__bf16*>(base)[idx] = static_cast<__bf16>(v);
}

// NP > 0: compile-time partial count; NP == 0: runtime count a.n.
// T is the type of the bias, the residual and the output.
template <int NP, typename TP, typename T>
__global__ __launch_bounds__(256) void epilogue_kernel(EArgs a) {
  using TB = T;
  using TR = T;
  using TO = T;
  const bool ALIGNED = a.aligned;
  const int vpr = (a.cols + 7) >> 3;
  const int jv = blockIdx.x * 256 + threadIdx.x;
  if (jv >= vpr) return;
  const int j = jv * 8;
  const bool full = (j + 8 <= a.cols);
  const int bz = blockIdx.z;
  const int n = NP > 0 ? NP : a.n;
  const void* const* parts = a.parts + bz * n;
  const void* res = a.res[bz];
  void* const* outs = a.out + bz * a.n_rep;
  uint8_t* mask = a.mask[bz];
  const int64_t mrow0 = a.mrow0[bz];
  for (int i = blockIdx.y; i < a.rows; i += gridDim.y) {
    float s[8];
    bool keep[8];
    const int64_t e0 = (mrow0 + i) * a.mld + a.mcol0 + j;
    if (full) {
      // ---- vector path: 8 columns ----
      const int64_t ip = static_cast<int64_t>(i) * a.ld_part + j;
      float r[8];
      if (res) load8<TR, true>(res, static_cast<int64_t>(i) * a.ld_res + j, r);
      load8<TP, true>(parts[0], ip, s);
      if constexpr (NP > 0) {
        float t[NP > 1 ? NP - 1 : 1][8];
#pragma unroll
        for (int k = 1; k < NP; ++k) load8<TP, true>(parts[k], ip, t[k - 1]);
#pragma unroll
        for (int k = 1; k < NP; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] = s[e] + t[k - 1][e];
      } else {
        for (int k = 1; k < n; ++k) {
          float t[8];
          load8<TP, true>(parts[k], ip, t);
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] = s[e] + t[e];
        }
      }
      if (a.bias) {
        float b[8];
        load8<TB, false>(a.bias, j, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = s[e] + b[e];
      }
      if (a.mode == 1) {
        if (ALIGNED) {
          const uint64_t blk = static_cast<uint64_t>(e0) >> 2;
          const Philox4 x = block_for(a, blk), y = block_for(a, blk + 1);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            keep[e] = x.w[e] >= a.threshold;
            keep[e + 4] = y.w[e] >= a.threshold;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint64_t ee = static_cast<uint64_t>(e0 + e);
            const Philox4 x = block_for(a, ee >> 2);
            keep[e] = pick(x, static_cast<uint32_t>(ee & 3)) >= a.threshold;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = keep[e] ? s[e] * a.scale : 0.0f;
      } else if (a.mode == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          keep[e] = false;
          s[e] = 0.0f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) keep[e] = true;
      }
      if (res) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = s[e] + r[e];
      }
      for (int q = 0; q < a.n_rep; ++q) store8<TO>(outs[q], static_cast<int64_t>(i) * a.ld_out + j, s);
      if (mask) {
        uint64_t bits = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) bits |= static_cast<uint64_t>(keep[e] ? 1 : 0) << (8 * e);
        uint8_t* mp = mask + static_cast<int64_t>(i) * a.cols + j;
        if ((a.cols & 7) == 0) {
          *reinterpret_cast<uint64_t*>(mp) = bits;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) mp[e] = static_cast<uint8_t>(bits >> (8 * e));
        }
      }
    } else {
      // ---- ragged tail of a row: element by element ----
      for (int e = 0; j + e < a.cols; ++e) {
        const int c = j + e;
        const int64_t ip = static_cast<int64_t>(i) * a.ld_part + c;
        float v = load1<TP>(parts[0], ip);
        for (int k = 1; k < n; ++k) v = v + load1<TP>(parts[k], ip);
        if (a.bias) v = v + load1<TB>(a.bias, c);
        bool kp = true;
        if (a.mode == 1) {
          const uint64_t ee = static_cast<uint64_t>(e0 + e);
          const Philox4 x = block_for(a, ee >> 2);
          kp = pick(x, static_cast<uint32_t>(ee & 3)) >= a.threshold;
          v = kp ? v * a.scale : 0.0f;
        } else if (a.mode == 2) {
          kp = false;
          v = 0.0f;
        }
        if (res) v = v + load1<TR>(res, static_cast<int64_t>(i) * a.ld_res + c);
        for (int q = 0; q < a.n_rep; ++q) store1<TO>(outs[q], static_cast<int64_t>(i) * a.ld_out + c, v);
        if (mask) mask[static_cast<int64_t>(i) * a.cols + c] = kp ? 1 : 0;
      }
    }
  }
}

// Eight elements as loaded: two 16-byte fp32 vectors, or one of bf16 kept
// packed until the arithmetic needs them (half the registers).
template <typename T>
struct Raw8;
template <>
struct Raw8<float> {
  f32x4 x, y;
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? x[e] : y[e - 4]; }
};
template <>
struct Raw8<__bf16> {
  u32x4 w;
  __device__ __forceinline__ float operator[](int e) const {
    return static_cast<float>(__builtin_bit_cast(bf16x8, w)[e]);
  }
};

// Load at byte offset `off` (32 bits) from a wave-uniform row base: the
// loads of all operands then share one offset register.
template <typename T, bool NT>
__device__ __forceinline__ Raw8<T> load_raw8(const void* row, uint32_t off) {
  Raw8<T> r;
  const char* p = reinterpret_cast<const char*>(row) + off;
  if constexpr (sizeof(T) == 4) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    if constexpr (NT) {
      r.x = __builtin_nontemporal_load(q);
      r.y = __builtin_nontemporal_load(q + 1);
    } else {
      r.x = q[0];
      r.y = q[1];
    }
  } else {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    if constexpr (NT) r.w = __builtin_nontemporal_load(q);
    else r.w = *q;
  }
  return r;
}

// Vector kernel for one or two partials in the common shape: every row a
// whole number of 8-column vectors, the mask's element index a multiple of 4
// at every vector start (two Philox blocks per vector), no mask output and at
// most 65535 rows.  The arithmetic is the general kernel's, step for step, so
// both give the same bits.  Without the ragged and debug paths, with loads
// kept packed until they are summed and row bases kept scalar, one fp32
// partial needs 28 VGPRs instead of 70: eight waves per SIMD then keep enough
// loads in flight to stream HBM, and the mask's integer work hides under the
// loads (the GPT-3 FFN shape, 8 x [1024, 12288]: 5.75 -> 6.11 TB/s in an A/B
// run).  Eight partials stay on the general kernel: the same structure was 3%
// slower there, with or without an occupancy cap.  MODE: 0 no dropout,
// 1 dropout, 2 drop everything.
template <int NP, typename TP, typename T, int MODE>
__global__ __launch_bounds__(256) void epilogue_vec_kernel(EArgs a) {
  const int jv = blockIdx.x * 256 + threadIdx.x;
  if (jv >= (a.cols >> 3)) return;
  const int j = jv * 8;
  const int i = blockIdx.y;     // one row per grid row (rows <= 65535)
  const int bz = blockIdx.z;
  // Row bases are wave-uniform (scalar); a lane adds its vector's byte offset.
  const uint32_t op = static_cast<uint32_t>(j) * sizeof(TP), ot = static_cast<uint32_t>(j) * sizeof(T);
  const int64_t rp = static_cast<int64_t>(i) * a.ld_part * static_cast<int64_t>(sizeof(TP));
  const void* res = a.res[bz];
  Raw8<T> r{}, b{};
  if (res)
    r = load_raw8<T, true>(reinterpret_cast<const char*>(res) +
                               static_cast<int64_t>(i) * a.ld_res * static_cast<int64_t>(sizeof(T)),
                           ot);
  Raw8<TP> p[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k)
    p[k] = load_raw8<TP, true>(reinterpret_cast<const char*>(a.parts[bz * NP + k]) + rp, op);
  if (a.bias) b = load_raw8<T, false>(a.bias, ot);
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s[e] = p[0][e];
#pragma unroll
    for (int k = 1; k < NP; ++k) s[e] = s[e] + p[k][e];
  }
  if (a.bias) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + b[e];
  }
  if constexpr (MODE == 1) {
    const int64_t e0 = (a.mrow0[bz] + i) * a.mld + a.mcol0 + j;
    const uint64_t blk = static_cast<uint64_t>(e0) >> 2;
    const Philox4 x = block_for(a, blk), y = block_for(a, blk + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] = x.w[e] >= a.threshold ? s[e] * a.scale : 0.0f;
      s[e + 4] = y.w[e] >= a.threshold ? s[e + 4] * a.scale : 0.0f;
    }
  } else if constexpr (MODE == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0f;
  }
  if (res) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + r[e];
  }
  const int64_t oi = static_cast<int64_t>(i) * a.ld_out + j;
  for (int q = 0; q < a.n_rep; ++q) store8<T>(a.out[bz * a.n_rep + q], oi, s);
}

template <int NP, typename TP, typename T>
hipError_t launch_np(const EArgs& k, dim3 grid, hipStream_t s, bool vec) {
  if constexpr (NP > 0 && NP <= 2) {
    if (vec) {
      if (k.mode == 1) hipLaunchKernelGGL((epilogue_vec_kernel<NP, TP, T, 1>), grid, dim3(256), 0, s, k);
      else if (k.mode == 2) hipLaunchKernelGGL((epilogue_vec_kernel<NP, TP, T, 2>), grid, dim3(256), 0, s, k);
      else hipLaunchKernelGGL((epilogue_vec_kernel<NP, TP, T, 0>), grid, dim3(256), 0, s, k);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((epilogue_kernel<NP, TP, T>), grid, dim3(256), 0, s, k);
  return hipGetLastError();
}
template <typename TP, typename T>
hipError_t launch_t(const EArgs& k, dim3 grid, hipStream_t s, bool vec) {
  switch (k.n) {
    case 1: return launch_np<1, TP, T>(k, grid, s, vec);
    case 2: return launch_np<2, TP, T>(k, grid, s, vec);
    case 8: return launch_np<8, TP, T>(k, grid, s, vec);
    default: return launch_np<0, TP, T>(k, grid, s, false);
  }
}

}  // namespace

cce_status launch_fused_epilogue(const EpilogueLaunch& L, void* stream) {
  if (L.rows <= 0 || L.cols <= 0 || L.batch <= 0) return CCE_OK;
  EArgs k{};
  for (int i = 0; i < L.n * L.batch; ++i) k.parts[i] = L.parts[i];
  for (int q = 0; q < L.batch * L.n_rep; ++q) k.out[q] = L.out[q];
  k.n_rep = L.n_rep;
  for (int b = 0; b < L.batch; ++b) {
    k.res[b] = L.res[b];
    k.mask[b] = L.mask[b];
    k.mrow0[b] = L.mrow0[b];
  }
  k.n = L.n;
  k.rows = static_cast<int>(L.rows);
  k.cols = static_cast<int>(L.cols);
  k.ld_part = L.ld_part;
  k.ld_res = L.ld_res;
  k.ld_out = L.ld_out;
  k.bias = L.bias;
  k.threshold = L.threshold;
  k.mode = L.drop_all ? 2 : (L.dropout ? 1 : 0);
  k.scale = L.scale;
  k.key0 = static_cast<uint32_t>(L.seed);
  k.key1 = static_cast<uint32_t>(L.seed >> 32);
  k.off0 = static_cast<uint32_t>(L.offset);
  k.off1 = static_cast<uint32_t>(L.offset >> 32);
  k.mcol0 = L.mcol0;
  k.mld = L.mld;
  k.aligned = (L.mld % 4 == 0) && (L.mcol0 % 4 == 0);
  const int vpr = static_cast<int>((L.cols + 7) / 8);
  dim3 grid((vpr + 255) / 256, static_cast<unsigned>(L.rows < 65535 ? L.rows : 65535),
            static_cast<unsigned>(L.batch));
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The vector kernel takes whole vectors with an aligned mask index, no mask
  // output and one grid row per row (pointers are 16-byte aligned and every
  // ld a multiple of 8, so each vector is one or two aligned 16-byte
  // accesses).
  bool vec = (L.cols % 8 == 0) && (k.mode != 1 || k.aligned) && L.rows <= 65535;
  for (int b = 0; b < L.batch; ++b) vec = vec && L.mask[b] == nullptr;
  // bias and residual share the output type (checked by the caller).
  hipError_t e;
  if (L.part_t == CCE_F32)
    e = (L.out_t == CCE_F32) ? launch_t<float, float>(k, grid, s, vec) : launch_t<float, __bf16>(k, grid, s, vec);
  else
    e = (L.out_t == CCE_F32) ? launch_t<__bf16, float>(k, grid, s, vec) : launch_t<__bf16, __bf16>(k, grid, s, vec);
  if (e != hipSuccess) return fail(CCE_EHIP, std::string("epilogue launch: ") + hipGetErrorString(e));
  return CCE_OK;
}

}  // namespace cce
