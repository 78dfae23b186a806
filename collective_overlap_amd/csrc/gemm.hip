// Grouped GEMM kernels for gfx950 (CDNA4): C_g = epi(A_g * B_g^T [, Cin_g]).
//
// These are the per-iteration partial einsums of the looped CollectiveEinsum
// (Wang et al., ASPLOS'23, Section 5.1): one launch covers the partial GEMM of
// every rank of one iteration (or half-step), and the update -- a store into
// the strided result slice (DynamicUpdateSlice) or an addition into the
// travelling accumulator -- is fused into the GEMM's epilogue, as the fusion
// of Section 5.4.3 fuses the Addition into the Einsum.
//
// bf16 path: 256 threads = 4 waves of 64 lanes.  A macro-tile BM x BN x 64 is
// staged through LDS (double-buffered, XOR-swizzled 16-byte chunks so that the
// ds_read_b128 of 32 consecutive rows hit distinct banks).  Each wave owns a
// (BM/WM) x (BN/WN) sub-tile of 32x32 blocks computed with
// v_mfma_f32_32x32x16_bf16.  The MFMA's first operand is fed with rows of the
// B^T tile and the second with rows of the A tile, so the 32x32 result block
// is C^T: each lane then holds 4 consecutive output columns of one row per
// register quad, which the epilogue stores (and, for the accumulate mode,
// loads) as one 16-byte (fp32) or 8-byte (bf16) vector.
//
// Global loads are raw buffer loads with the range of the operand block as the
// buffer size: rows past M / N read as zero; chunks past K are steered out of
// range, so ragged tails need no separate path.
//
// Workgroups are dealt to the 8 XCDs round-robin by workgroup ID; the tile
// index is remapped so that every XCD works through a contiguous range of
// tiles (for 8 groups of equal size, one rank per XCD), walked in bands of
// 4 tile rows so that 32 co-resident tiles share A rows and B^T rows in the
// XCD's L2.

#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "cce_internal.hpp"
#include "philox.hpp"

namespace cce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kOob = 0x40000000;

// Pipeline shape of the bf16 kernel: k-tile depth and LDS stages (build-time
// tuning knobs; 256x256 tiles need NS * (BM + BN) * BK * 2 <= 160 KB of LDS).
#ifndef CCE_GEMM_BK
#define CCE_GEMM_BK 64
#endif
#ifndef CCE_GEMM_NS
#define CCE_GEMM_NS 2
#endif
constexpr int kBK = CCE_GEMM_BK;
constexpr int kNS = CCE_GEMM_NS;
#ifndef CCE_GEMM_STAGED_STORE
#define CCE_GEMM_STAGED_STORE 1
#endif
constexpr bool kStagedStore = CCE_GEMM_STAGED_STORE;
// added to steer a load past num_records
constexpr int64_t kMaxRsrcBytes = kOob - 256;

struct KArgs {
  int groups;
  int M, N, K;
  int lda, ldb, ldc, ldcin;   // elements
  int tiles_m, tiles_n, tiles_per_group, total_tiles;
  int fwd, ldfwd;             // fused permute: operand to forward, its destination ld
  GemmGroupPtrs p;
  FinalArgs fin;              // EPI_FINAL: the chunk consumer
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  int n = bytes > kMaxRsrcBytes ? static_cast<int>(kMaxRsrcBytes) : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferFlags);
}

// Tile index -> (group, tile row, tile col), XCD-aware (see header).
__device__ __forceinline__ void map_tile(const KArgs& a, int& g, int& tm, int& tn) {
  const int w = blockIdx.x;
  const int nwg = gridDim.x;
  const int per = nwg / 8;
  int t = (w < per * 8) ? (w % 8) * per + (w / 8) : w;
  g = t / a.tiles_per_group;
  const int rem = t - g * a.tiles_per_group;
  constexpr int kBand = 4;
  const int band = rem / (kBand * a.tiles_n);
  const int first = band * kBand;
  const int rows = min(a.tiles_m - first, kBand);
  const int in_band = rem - band * kBand * a.tiles_n;
  tm = first + in_band % rows;
  tn = in_band / rows;
}

// 16-byte global->LDS load: lane L of the wave writes bytes [16 L, 16 L + 16)
// after the wave-uniform LDS address `lds`.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voffset, 0, 0, 0);
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maxima (gfx9
// encoding: vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8,
// vmcnt[5:4] bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Exact (erf) GELU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)).  erf comes from
// the rational approximation of Abramowitz and Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (absolute error <= 1.5e-7):
//   erfc(a) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-a^2),
//   t = 1 / (1 + p a), a >= 0,
// and 1 + erf(u) is formed as 2 - erfc(|u|) for u >= 0 and erfc(|u|) for
// u < 0, so the negative tail has no cancellation.  About a dozen VALU
// operations against several dozen for the library erff; the epilogue runs
// while the matrix cores idle, so its length shows in the kernel time.
__device__ __forceinline__ float gelu_exact(float x) {
  const float u = x * 0.70710678118654752f;
  const float a = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * a);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f +
                                                                          t * 1.061405429f))));
  const float q = poly * __expf(-(a * a));
  return 0.5f * x * (u >= 0.0f ? 2.0f - q : q);
}

// Accumulator input of 4 consecutive columns [n, n+4) of row m (zeros past
// the edges; store_quad skips those).  The input is read once, so the load
// is nontemporal and leaves the L2 to the operand tiles.
__device__ __forceinline__ f32x4 load_cin_quad(const KArgs& a, const float* cinbase, int m, int n) {
  f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
  if (m >= a.M || n >= a.N) return r;
  const float* cin = cinbase + static_cast<int64_t>(m) * a.ldcin + n;
  if (n + 3 < a.N) {
    r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(cin));
  } else {
    for (int e = 0; e < 4; ++e)
      if (n + e < a.N) r[e] = cin[e];
  }
  return r;
}

// Epilogue for 4 consecutive columns [n, n+4) of row m; cinv is the
// accumulator input (EPI_ACCUM) loaded by load_cin_quad.
template <typename TOut, int EPI, bool GELU>
__device__ __forceinline__ void store_quad(const KArgs& a, void* cbase, int m, int n, f32x4 v,
                                           f32x4 cinv) {
  if (m >= a.M || n >= a.N) return;
  const bool full = (n + 3 < a.N);
  if (EPI == EPI_ACCUM) v = cinv + v;
  if (GELU) {
    for (int e = 0; e < 4; ++e) v[e] = gelu_exact(v[e]);
  }
  if constexpr (sizeof(TOut) == 4) {
    float* c = reinterpret_cast<float*>(cbase) + static_cast<int64_t>(m) * a.ldc + n;
    if (full) {
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(c));
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < a.N) c[e] = v[e];
    }
  } else {
    __bf16* c = reinterpret_cast<__bf16*>(cbase) + static_cast<int64_t>(m) * a.ldc + n;
    bf16x4 h;
    for (int e = 0; e < 4; ++e) h[e] = static_cast<__bf16>(v[e]);
    if (full) {
      __builtin_nontemporal_store(h, reinterpret_cast<bf16x4*>(c));
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < a.N) c[e] = h[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk consumer of EPI_FINAL launches (fine-grained overlap; FinalArgs in
// cce_internal.hpp).  Four consecutive columns [n, n+4) of row m at a time,
// n a multiple of 4: loads of the other partial and of the residual (zeros
// past column N), and the consumer arithmetic.
// ---------------------------------------------------------------------------
template <bool WHOLE = false>
__device__ __forceinline__ f32x4 load_f32x4_nt(const float* p, int n, int N) {
  if (WHOLE || n + 3 < N) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int e = 0; e < 4; ++e)
    if (n + e < N) r[e] = p[e];
  return r;
}

template <typename T, bool WHOLE = false>
__device__ __forceinline__ f32x4 load_t4(const void* base, int64_t idx, int n, int N, bool nt) {
  f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (sizeof(T) == 4) {
    const float* p = reinterpret_cast<const float*>(base) + idx;
    if (WHOLE || n + 3 < N) return nt ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p))
                             : *reinterpret_cast<const f32x4*>(p);
    for (int e = 0; e < 4; ++e)
      if (n + e < N) r[e] = p[e];
  } else {
    const __bf16* p = reinterpret_cast<const __bf16*>(base) + idx;
    if (WHOLE || n + 3 < N) {
      const u32x2 w = nt ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p))
                         : *reinterpret_cast<const u32x2*>(p);
      const bf16x4 h = __builtin_bit_cast(bf16x4, w);
      for (int e = 0; e < 4; ++e) r[e] = static_cast<float>(h[e]);
      return r;
    }
    for (int e = 0; e < 4; ++e)
      if (n + e < N) r[e] = static_cast<float>(p[e]);
  }
  return r;
}

// Keep decisions of the 4 elements [n, n+4) of output row m (bit e: element
// n+e kept), from the Philox mask of the standalone epilogue: element index
// e = (mrow0 + m) * mld + mcol0 + n + e.
__device__ __forceinline__ unsigned keep_bits4(const FinalArgs& f, int64_t mrow0, int m, int n) {
  const int64_t e0 = (mrow0 + m) * f.mld + f.mcol0 + n;
  unsigned bits = 0;
  if (f.aligned) {
    const Philox4 k = philox_block(static_cast<uint64_t>(e0) >> 2, f.off0, f.off1, f.key0, f.key1);
    for (int e = 0; e < 4; ++e) bits |= (k.w[e] >= f.threshold ? 1u : 0u) << e;
  } else {
    for (int e = 0; e < 4; ++e) {
      const uint64_t ee = static_cast<uint64_t>(e0 + e);
      const Philox4 k = philox_block(ee >> 2, f.off0, f.off1, f.key0, f.key1);
      bits |= (philox_pick(k, static_cast<uint32_t>(ee & 3)) >= f.threshold ? 1u : 0u) << e;
    }
  }
  return bits;
}

// out[m, n..n+3] = r + keep * ((v + w) + b) * scale, in the order of the
// standalone epilogue kernel (the sum of the partials, the bias, the mask
// and scale, the residual; each step one fp32 operation, no contraction),
// rounded once to TOut.  v is this producer's partial; w the other one
// (has_w), b the bias (f.bias), r the residual (has_r); keep holds the keep
// bits (keep_bits4) when f.mode is 1.
template <typename TOut, bool WHOLE = false>
__device__ __forceinline__ void consume4(const FinalArgs& f, int m, int n, int N, f32x4 v,
                                         bool has_w, f32x4 w, f32x4 b, bool has_r, f32x4 r,
                                         unsigned keep, void* out) {
#pragma clang fp contract(off)
  float x[4] = {v[0], v[1], v[2], v[3]};
  if (has_w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = x[e] + w[e];
  }
  if (f.bias) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = x[e] + b[e];
  }
  if (f.mode == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = ((keep >> e) & 1u) ? x[e] * f.scale : 0.0f;
  } else if (f.mode == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = 0.0f;
  }
  if (has_r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = x[e] + r[e];
  }
  const int64_t oi = static_cast<int64_t>(m) * f.ld_out + n;
  if constexpr (sizeof(TOut) == 4) {
    float* o = reinterpret_cast<float*>(out) + oi;
    if (WHOLE || n + 3 < N) {
      __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(o));
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < N) o[e] = x[e];
    }
  } else {
    __bf16* o = reinterpret_cast<__bf16*>(out) + oi;
    bf16x4 h;
    for (int e = 0; e < 4; ++e) h[e] = static_cast<__bf16>(x[e]);
    if (WHOLE || n + 3 < N) {
      __builtin_nontemporal_store(__builtin_bit_cast(u32x2, h), reinterpret_cast<u32x2*>(o));
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < N) o[e] = h[e];
    }
  }
}

// The partial a first producer publishes crosses workgroups, usually on
// different XCDs, each with its own L2.  It is written and read with the
// device-coherent cache policy (sc1): such accesses are performed at the
// device's coherence point, past the XCD's L2, so neither side has to write
// back or invalidate its whole L2 -- which is what an agent-scope release or
// acquire fence does on this chip, and what made every co-running tile
// re-fetch its operands.  The ready word is stored only after every thread's
// stores have been performed (vmcnt 0, then the workgroup barrier), and the
// consumer issues its loads only after it has seen the word.
constexpr int kDevCoherent = 16;   // buffer instruction cache policy: sc1

template <bool WHOLE = false>
__device__ __forceinline__ void store_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v, int n,
                                           int N) {
  if (WHOLE || n + 3 < N) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kDevCoherent);
  } else {
    for (int e = 0; e < 4; ++e)
      if (n + e < N)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v[e]), r, off + 4 * e, 0,
                                              kDevCoherent);
  }
}

template <bool WHOLE = false>
__device__ __forceinline__ f32x4 load_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, int n, int N) {
  if (WHOLE || n + 3 < N)
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDevCoherent));
  f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int e = 0; e < 4; ++e)
    if (n + e < N)
      v[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * e, 0,
                                                                            kDevCoherent));
  return v;
}

// Chunk protocol of an EPI_FINAL workgroup, run once its partial is in
// registers.  Returns the role -- 0: the chunk's only producer in this launch
// (consume; *other is the other partial finished by an earlier launch, or
// NULL), 1: the first of two producers (store the partial at C with
// store_dev4, then publish_chunk), 2: the second (consume *other, the pair's
// partial, after its ready word) -- or -1 when the wait gave up (the
// workgroup then writes nothing).  The claim is an agent-scope atomic on the
// chunk's counter; the first producer is already running when the second
// claims, so the second's wait ends once the first has stored its partial.
// Every thread of the workgroup must call it.
// (Values read back from LDS are per-lane to the compiler: the role and the
// pointer are made wave-uniform with readfirstlane, so that branches on them
// are scalar and buffer resources built from them need no per-lane loop.)
__device__ __forceinline__ const float* uniform_ptr(const float* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const float*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// `sh`: two ints of the workgroup's LDS for the role and the wait's result.
// (They live in the kernel's one LDS array: a second LDS object makes the
// compiler wait for every global->LDS load of the k loop before the next LDS
// access, since it can no longer tell the loads' target apart from other
// LDS accesses -- which serialised the whole k loop.)
__device__ __forceinline__ int claim_chunk(const KArgs& a, int g, int slot, const float** other,
                                           int* sh) {
  int& s_role = sh[0];
  int& s_ok = sh[1];
  const int part = a.fin.partner[g];
  if (part < 0) {
    *other = a.fin.other[a.fin.oid[g]];
    return 0;
  }
  if (threadIdx.x == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(a.fin.sig + 2 * slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_role = old == 0u ? 1 : 2;
  }
  __syncthreads();
  const int role = __builtin_amdgcn_readfirstlane(s_role);
  if (role == 1) return 1;
  if (threadIdx.x == 0) {
    const unsigned* rdy = a.fin.sig + 2 * slot + 1;
    unsigned polls = 0;
    int ok = 0;
    for (;;) {
      if (__hip_atomic_load(rdy, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        ok = 1;
        break;
      }
      if (++polls >= a.fin.cap) break;
      __builtin_amdgcn_s_sleep(4);
    }
    if (!ok) __hip_atomic_fetch_add(a.fin.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_ok = ok;
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(s_ok)) return -1;
  *other = reinterpret_cast<const float*>(a.p.c[part]);
  return 2;
}

// The first producer's partial is stored (store_dev4): once every thread's
// stores have been performed, set the chunk's ready word.  Every thread of
// the workgroup must call it.
__device__ __forceinline__ void publish_chunk(const KArgs& a, int slot) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0 && !a.fin.nopub)
    __hip_atomic_store(a.fin.sig + 2 * slot + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile row of staged read instruction `it` of pass p, for thread row 0 (the
// staged epilogue of the bf16 kernel: ERI rows per instruction, EJP 32-row
// blocks per wave and pass, WTM rows per wave).
template <int ERI, int EJP, int WTM>
__device__ __forceinline__ int staged_row(int p, int it) {
  const int lr = ERI * it;
  return (lr / (32 * EJP)) * WTM + 32 * (p * EJP + (lr / 32) % EJP) + lr % 32;
}

// Chunk consumer of one staged pass of an EPI_FINAL tile: this producer's
// partial (Cin + the staged accumulators), the other partial (rpw, when
// has_pw), the residual and the bias go through consume4.  The pass's keep
// bits come first, from a rolled loop (the Philox rounds stay out of the
// unrolled loop, so that the whole pass is straight-line code).  WHOLE: the
// tile lies inside the matrix -- no per-lane edge checks, so loads and
// stores of consecutive chunks are counted exactly by the wait counters
// (a per-lane branch between them makes every wait a full drain, stores
// included).
template <typename TOut, bool WHOLE, int EIT, int ERI, int EJP, int WTM, int ERB, int ESW, int EPC>
__device__ __forceinline__ void consume_pass(const KArgs& a, const char* smem, int p, int m0, int n0,
                                             int e_r, int e_c, const float* cin,
                                             __amdgpu_buffer_rsrc_t rpw, bool has_pw,
                                             const void* resp, void* outp, int64_t mr0, f32x4 b4) {
  const int n = n0 + EPC * e_c;
  static_assert(EIT <= 32, "keep bits");
  uint64_t kb0 = 0, kb1 = 0;   // 4 bits per chunk: chunk it at bit 4 (it % 16) of kb[it / 16]
  if (a.fin.mode == 1) {
#pragma unroll 1
    for (int it = 0; it < EIT; ++it) {
      const int m = m0 + staged_row<ERI, EJP, WTM>(p, it) + e_r;
      if (!WHOLE && (m >= a.M || n >= a.N)) continue;
      const uint64_t bits = keep_bits4(a.fin, mr0, m, n);
      if (it < 16) kb0 |= bits << (4 * it);
      else kb1 |= bits << (4 * (it - 16));
    }
  }
  constexpr int CB = 4;
  static_assert(EIT % CB == 0, "consumer batch");
#pragma unroll
  for (int i0 = 0; i0 < EIT; i0 += CB) {
    // one batch at a time: loads of later batches are not hoisted here
    // (that would hold every batch's loads in registers at once)
    __builtin_amdgcn_sched_barrier(0);
    f32x4 cv[CB], wv[CB], rv[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int m = m0 + staged_row<ERI, EJP, WTM>(p, i0 + j) + e_r;
      const bool ok = WHOLE || (m < a.M && n < a.N);
      cv[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      wv[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      rv[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (ok && cin) cv[j] = load_f32x4_nt<WHOLE>(cin + static_cast<int64_t>(m) * a.ldcin + n, n, a.N);
      if (ok && has_pw) wv[j] = load_dev4<WHOLE>(rpw, static_cast<uint32_t>((m * a.ldc + n) * 4), n, a.N);
      if (ok && resp)
        rv[j] = load_t4<TOut, WHOLE>(resp, static_cast<int64_t>(m) * a.fin.ld_res + n, n, a.N, true);
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int it = i0 + j;
      const int lr = ERI * it + e_r;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(smem + lr * ERB + ((e_c ^ (lr & ESW)) << 4));
      const int m = m0 + staged_row<ERI, EJP, WTM>(p, it) + e_r;
      if (!WHOLE && (m >= a.M || n >= a.N)) continue;
      // (a first iteration's partial has no input: used as is, not added to
      // zero, which would turn -0 into +0)
      const f32x4 v = cin ? cv[j] + __builtin_bit_cast(f32x4, raw) : __builtin_bit_cast(f32x4, raw);
      const unsigned keep =
          static_cast<unsigned>((it < 16 ? kb0 >> (4 * it) : kb1 >> (4 * (it - 16))) & 15u);
      consume4<TOut, WHOLE>(a.fin, m, n, a.N, v, has_pw, wv[j], b4, resp != nullptr, rv[j], keep,
                            outp);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
//
// Software pipeline of one 64-deep k tile (4 steps of k16), with fragment
// double buffering so that the LDS reads for step kk+1 issue between the
// MFMAs of step kk:
//   kk=0: MFMA(F0) | read F1 (kk=1)
//   kk=1: MFMA(F1) | read F0 (kk=2)
//   kk=2: MFMA(F0) | read F1 (kk=3)
//   barrier (waits for the next tile's global->LDS loads)
//   kk=3: MFMA(F1) | read F0 (kk=0 of the next tile) | global->LDS loads of
//                    the tile after next into this tile's buffer
// One barrier per k tile.  It separates (a) the other buffer's loads from its
// first reads and (b) this buffer's last reads (issued in kk=2 and completed
// before the barrier) from the loads that overwrite it.  The loop body has no
// branches: loads past the end of K are steered out of range and land as
// zeros, so the tail needs no special case.
// ---------------------------------------------------------------------------
// Rows of a forwarded tile (per thread) whose LDS reads are issued together:
// all of them.  A rolled loop with one LDS wait per row had cost about 6% of
// the MLP's layer-1 launch; batched, the GPT-3 FFN step measured 16.72 ->
// 16.66 ms and the MLP's 2.012 -> 1.997 ms (A/B, interleaved; 4 per batch
// measured 16.68 / 1.998).
constexpr int kFwdBatch = 8;

// LDS swizzle of 16-byte chunks: physical chunk = logical ^ swz(row).  Rows
// of 8 chunks (k tile 64): swz = (r & 7) ^ ((r >> 3) & 1).  Rows of 4 chunks
// (k tile 32): swz = ((r >> 1) ^ (r >> 3)) & 3.  Either way the ds_read_b128
// of 32 consecutive rows at one logical chunk hits every bank once per
// 8-lane (32-bank) and per 16-lane (64-bank) service group.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

template <int BM, int BN, int WM, int WN, int BK, int NS, typename TOut, int EPI, bool GELU>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_bf16_kernel(KArgs a) {
  constexpr int NW = WM * WN;                // waves
  constexpr int ROWB = BK * 2;               // bytes per LDS row
  constexpr int CPR = BK / 8;                // 16-byte chunks per row
  constexpr int KK = BK / 16;                // k16 steps per k tile
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int RPI = 1024 / ROWB;           // rows per 1 KB load instruction
  constexpr int A_DMA = BM / (NW * RPI);     // load instructions per wave per stage
  constexpr int B_DMA = BN / (NW * RPI);
  constexpr int N_DMA = A_DMA + B_DMA;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(KK % 2 == 0 && NS >= 2 && A_DMA >= 1 && B_DMA >= 1, "tile shape");
  static_assert(NS * STAGE <= 160 * 1024, "LDS");
  static_assert((NS - 1) * N_DMA < 64, "vmcnt range");

  // (EPI_FINAL: 16 more bytes for the chunk claim's role and wait result)
  constexpr int kClaimBytes = (EPI == EPI_FINAL) ? 16 : 0;
  __shared__ __attribute__((aligned(16))) char smem[NS * STAGE + kClaimBytes];

  int g, tm, tn;
  map_tile(a, g, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform (an SGPR), so that LDS destinations of the direct loads are
  // scalar additions into M0 rather than VGPR reads.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const __bf16* A = reinterpret_cast<const __bf16*>(a.p.a[g]);
  const __bf16* B = reinterpret_cast<const __bf16*>(a.p.b[g]);
  // Buffer ranges: rows [m0, M) of A and [n0, N) of B^T.
  const int64_t a_bytes = (static_cast<int64_t>(a.M - m0 - 1) * a.lda + a.K) * 2;
  const int64_t b_bytes = (static_cast<int64_t>(a.N - n0 - 1) * a.ldb + a.K) * 2;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * a.lda, a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + static_cast<int64_t>(n0) * a.ldb, b_bytes);

  // Direct global->LDS staging (buffer_load ... lds): one instruction of a
  // wave fills 1 KB of LDS = RPI consecutive rows, lane L landing at byte
  // 16 L, i.e. row L / CPR, physical chunk L % CPR.  The lane fetches the
  // logical chunk that belongs there under the swizzle.  For wave w and
  // instruction p the rows are RPI (4 p + w) + L / CPR, and the swizzle of
  // those rows does not depend on p, so neither does the fetched chunk.
  const int dl_row = lane / CPR;
  const int dl_chunk = (lane % CPR) ^ swz<CPR>(RPI * wave + dl_row);
  uint32_t a_off[A_DMA], b_off[B_DMA];
#pragma unroll
  for (int p = 0; p < A_DMA; ++p) {
    const int r = RPI * (NW * p + wave) + dl_row;
    a_off[p] = (m0 + r < a.M) ? (r * a.lda + dl_chunk * 8) * 2u : uint32_t(kOob);
  }
#pragma unroll
  for (int p = 0; p < B_DMA; ++p) {
    const int r = RPI * (NW * p + wave) + dl_row;
    b_off[p] = (n0 + r < a.N) ? (r * a.ldb + dl_chunk * 8) * 2u : uint32_t(kOob);
  }
  // Rows past M / N start at kOob; chunks past K add kOob.  Operands are
  // smaller than kOob bytes, so either lands out of the buffer's range (the
  // sum stays below 2^32 because offsets within range are below 2^30); an
  // out-of-range lane writes zeros into its LDS slot.
  auto gload = [&](int buf, int k0) {
    const uint32_t kadd = k0 * 2u + ((k0 + dl_chunk * 8) < a.K ? 0u : uint32_t(kOob));
    char* s = smem + buf * STAGE + wave * 1024;
#pragma unroll
    for (int p = 0; p < A_DMA; ++p) dma16(ra, s + p * NW * 1024, a_off[p] + kadd);
#pragma unroll
    for (int p = 0; p < B_DMA; ++p) dma16(rb, s + BM * ROWB + p * NW * 1024, b_off[p] + kadd);
  };

  auto kadd_of = [&](int k0) {
    return k0 * 2u + ((k0 + dl_chunk * 8) < a.K ? 0u : uint32_t(kOob));
  };
  // Load instruction d of the wave's N_DMA (A first, then B).
  auto dma_one = [&](int buf, uint32_t kadd, int d) {
    char* s = smem + buf * STAGE + wave * 1024;
    if (d < A_DMA) dma16(ra, s + d * NW * 1024, a_off[d] + kadd);
    else dma16(rb, s + BM * ROWB + (d - A_DMA) * NW * 1024, b_off[d - A_DMA] + kadd);
  };

  // Fragment addressing: row r = base + 32 i + (lane & 31) with base a
  // multiple of 32, so swz(r) = swz(lane & 31); chunk 2 kk + (lane >> 5).
  const int frow = lane & 31;
  const int fk = lane >> 5;
  const int fa_base = (wm * WTM + frow) * ROWB;
  const int fb_base = BM * ROWB + (wn * WTN + frow) * ROWB;
  const int frow_sw = swz<CPR>(frow);
  int fsw[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) fsw[kk] = ((2 * kk + fk) ^ frow_sw) << 4;

  bf16x8 fa[2][FM], fb[2][FN];
  auto fread = [&](int buf, int kk, int slot) {
    const char* s = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < FN; ++i)
      fb[slot][i] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(s + fb_base + fsw[kk] + i * 32 * ROWB));
#pragma unroll
    for (int j = 0; j < FM; ++j)
      fa[slot][j] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(s + fa_base + fsw[kk] + j * 32 * ROWB));
  };

  // Fragment q of step kk: B^T blocks 0..FN-1, then A blocks.
  auto fread_one = [&](int buf, int kk, int slot, int q) {
    const char* s = smem + buf * STAGE;
    if (q < FN)
      fb[slot][q] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(s + fb_base + fsw[kk] + q * 32 * ROWB));
    else
      fa[slot][q - FN] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(s + fa_base + fsw[kk] + (q - FN) * 32 * ROWB));
  };

  // Fused permute: the looped operand (A or B) is written once to the next
  // rank's receive buffer while it sits in LDS.  k tile kt of a row block is
  // written by the one workgroup of that block whose other tile index equals
  // kt modulo the number of such workgroups, which spreads the stores evenly.
  // The next launch reads it: nontemporal stores.
  const bool fwd_a = a.fwd == FWD_A, fwd_b = a.fwd == FWD_B;
  __bf16* fdst = reinterpret_cast<__bf16*>(a.p.fwd[g]);
  auto forward = [&](int buf, int kt) {
    const int mine = fwd_a ? tn : tm;
    const int span = fwd_a ? a.tiles_n : a.tiles_m;
    // Groups without a destination (a stream that has ended) forward nothing.
    if (!(fwd_a || fwd_b) || fdst == nullptr || kt % span != mine) return;
    const char* s = smem + buf * STAGE + (fwd_a ? 0 : BM * ROWB);
    const int row0 = fwd_a ? m0 : n0;
    const int rows = fwd_a ? BM : BN;
    const int lim = fwd_a ? a.M : a.N;
    constexpr int RP = 64 * NW / CPR;            // rows per pass
    const int c = tid % CPR, r0 = tid / CPR;
    const int k = kt * BK + c * 8;
    if (k >= a.K) return;
    if (row0 + rows <= lim) {
      // Whole tile (the usual case): FB rows' LDS reads issued together,
      // then their stores, so that each batch waits for LDS once.
      auto whole = [&](auto rows_c) {
        constexpr int ROWS = decltype(rows_c)::value;
        constexpr int FB = kFwdBatch < ROWS / RP ? kFwdBatch : ROWS / RP;
        static_assert(ROWS % (RP * FB) == 0, "forward batches");
#pragma unroll
        for (int b = 0; b < ROWS / RP; b += FB) {
          u32x4 v[FB];
#pragma unroll
          for (int i = 0; i < FB; ++i) {
            const int r = r0 + (b + i) * RP;
            v[i] = *reinterpret_cast<const u32x4*>(s + r * ROWB + ((c ^ swz<CPR>(r)) << 4));
          }
#pragma unroll
          for (int i = 0; i < FB; ++i) {
            const int r = r0 + (b + i) * RP;
            __builtin_nontemporal_store(
                v[i], reinterpret_cast<u32x4*>(fdst + static_cast<int64_t>(row0 + r) * a.ldfwd + k));
          }
        }
      };
      if (fwd_a) whole(std::integral_constant<int, BM>{});
      else whole(std::integral_constant<int, BN>{});
      return;
    }
    for (int r = r0; r < rows; r += RP) {
      if (row0 + r >= lim) break;
      const u32x4 v = *reinterpret_cast<const u32x4*>(s + r * ROWB + ((c ^ swz<CPR>(r)) << 4));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(fdst + static_cast<int64_t>(row0 + r) * a.ldfwd + k));
    }
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};

  // The MFMAs of a step walk the accumulator blocks in a snake order: row i
  // of blocks left to right, row i+1 right to left, so that consecutive
  // MFMAs always share one operand.  The matrix cores run power-limited and
  // fewer operand changes cost less: 0.4% per launch, 0.9% in a loop of
  // MFMAs alone.  Each block still sees the same k sequence (same bits).
  auto mfma_one = [&](int slot, int q) {
    const int i = q / FM;
    const int j = (i & 1) ? FM - 1 - q % FM : q % FM;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][i], fa[slot][j], acc[i][j], 0, 0, 0);
  };

  // Pipeline: NS LDS buffers; tile kt in buffer kt % NS.  Per k tile kt:
  //   kk = 0 .. KK-2: MFMA(step kk) | LDS reads of step kk+1
  //   wait for tile kt+1's loads, barrier
  //   kk = KK-1:      MFMA | LDS reads of step 0 of tile kt+1
  // Tile kt's buffer is free after the barrier: its last fragments (step
  // KK-1) were read before it, and the barrier makes every wave's loads of
  // tile kt+1 visible.  The loads of tile kt+NS into that buffer are spread
  // over two steps: the first half during step KK-1 of iteration kt, the
  // second half during step 0 of iteration kt+1, one instruction per
  // NMF / C MFMAs, so that the vector memory path sees a steady stream
  // instead of one burst per k tile.  Each step is issued in a fixed order
  // (MFMA, fragment read, load), fenced by scheduling barriers.  The loop
  // body has no branches on the data path: loads past the end of K are
  // steered out of range and land as zeros, so the tail needs no special
  // case.
  constexpr int NMF = FM * FN;
  constexpr int C = (N_DMA + 1) / 2;         // loads per half
  // fragment reads: one per RS MFMAs, spread over the step
  constexpr int RS = NMF >= 2 * (FM + FN) ? 2 : 1;
  const int KT = (a.K + BK - 1) / BK;
  if (KT > 0) {
#pragma unroll
    for (int st = 0; st < NS; ++st) gload(st, st * BK);
    wait_vmcnt<(NS - 1) * N_DMA>();
    __syncthreads();
    forward(0, 0);
#pragma unroll
    for (int q = 0; q < FM + FN; ++q) fread_one(0, 0, 0, q);
  }
  // Epilogue geometry: block b = (i, j) = (b % FN, b / FN) holds C^T; the
  // lane owns row quad_m(b) and columns quad_n(b, q) .. +3 for q = 0..3.
  void* cbase = a.p.c[g];
  const float* cin = a.p.cin[g];
  constexpr int NB = FM * FN;
  auto quad_m = [&](int b) { return m0 + wm * WTM + (b / FN) * 32 + (lane & 31); };
  auto quad_n = [&](int b, int q) { return n0 + wn * WTN + (b % FN) * 32 + 8 * q + 4 * (lane >> 5); };
  // Accumulate mode with fp32 results and no GELU: staged through LDS like
  // the store mode (below).  Otherwise the accumulator input of the first
  // NPRE blocks is loaded into registers during the last k tiles -- PER_IT
  // blocks in each of two iterations, one load per MFMA slot of the step
  // after the barrier -- so that its HBM traffic overlaps MFMAs instead of
  // stalling the epilogue.
  // EPI_FINAL (the ReduceScatter's last launch with fine-grained overlap)
  // takes the staged fp32 accumulate path; its chunk consumer writes TOut.
  constexpr bool FIN = (EPI == EPI_FINAL);
  static_assert(!FIN || (kStagedStore && !GELU), "EPI_FINAL runs on the staged fp32 path");
  constexpr bool ACS = (((EPI == EPI_ACCUM) && sizeof(TOut) == 4) || FIN) && !GELU && kStagedStore;
  constexpr bool PREF = (EPI == EPI_ACCUM) && !ACS;
  constexpr int PER_IT = PREF ? NB / 8 : 0;   // blocks per prefetch iteration
  constexpr int NPRE = 2 * PER_IT;
  f32x4 cpre[NPRE > 0 ? NPRE : 1][4];
  // this lane's first accumulator input: row quad_m(0), column quad_n(0, 0)
  const float* cin_w = PREF ? cin + static_cast<int64_t>(quad_m(0)) * a.ldcin + quad_n(0, 0) : cin;

  // Store mode: the result passes through LDS on its way out.  The
  // accumulators (block (i, j) of a wave holds C^T, the lane 4 consecutive
  // columns of one row per register quad) are written to LDS row-major and
  // read back in 16-byte chunks along the rows, so that a wave's store
  // instruction writes whole rows (1 KB of consecutive bytes) instead of 32
  // rows x 16 bytes, in 8-byte pieces for bf16, a pattern that ran at about
  // a third of the HBM write bandwidth (for fp32 it stalls the address
  // path, and staging was 1% faster on the ReduceScatter).  Chunk c of
  // staged row r is kept at chunk c ^ (r & ESW) so that both the 32-row
  // writes and the row reads spread over the banks.  A tile that does not
  // fit the LDS (fp32) goes in EP passes of EJP 32-row blocks per wave.  The
  // accumulate mode with fp32 results is staged the same way, and reads its
  // input in the same 16-byte chunks along the rows, every chunk of a pass
  // issued before the pass is written to LDS; for whole tiles the first
  // pass's chunks are loaded during the last-but-one k tile (together
  // 1.3-1.7% on the ReduceScatter over loading the input block by block in
  // the registers' layout).  With GELU or bf16 results it keeps the
  // register path.
  constexpr bool STAGED = ((EPI == EPI_STORE) && kStagedStore) || ACS;
  using TS = std::conditional_t<FIN, float, TOut>;   // staged (and stored) element type
  constexpr int ESZ = static_cast<int>(sizeof(TS));
  constexpr int ERB = BN * ESZ;                  // staged row bytes
  constexpr int ECR = ERB / 16;                  // chunks per staged row
  constexpr int EPC = 16 / ESZ;                  // elements per chunk
  constexpr int EP = (BM * ERB + NS * STAGE - 1) / (NS * STAGE);
  constexpr int EJP = FM / EP;
  constexpr int EPR = BM / EP;                   // staged rows per pass
  constexpr int ERI = 64 * NW / ECR;             // rows per read instruction
  constexpr int EIT = EPR / ERI;                 // read instructions per pass
  constexpr int ESW = ECR < 32 ? ECR - 1 : 31;
  static_assert(!STAGED || (FM % EP == 0 && EPR * ERB <= NS * STAGE && 64 * NW % ECR == 0 &&
                            32 % ERI == 0 && EPR % ERI == 0),
                "staged epilogue shape");
  const bool whole = m0 + BM <= a.M && n0 + BN <= a.N;
  // 16-byte result rows: chunks inside the matrix are stored as vectors,
  // the rest element by element.
  const bool vec = (reinterpret_cast<uintptr_t>(cbase) & 15) == 0 &&
                   (static_cast<int64_t>(a.ldc) * ESZ) % 16 == 0;
  // Tile row of read instruction `it` of pass p for thread row 0: staged row
  // lr = ERI it + tid / ECR belongs to wave row lr / (32 EJP), block
  // p EJP + (lr / 32) % EJP, row lr % 32 (ERI divides 32, so `it` alone
  // fixes the block).
  auto erow = [&](int p, int it) {
    const int lr = ERI * it;
    return (lr / (32 * EJP)) * WTM + 32 * (p * EJP + (lr / 32) % EJP) + lr % 32;
  };
  const int e_r = tid / ECR, e_c = tid % ECR;

  int cur = 0;                  // buffer of tile kt
  f32x4 cinv[ACS ? EIT : 1];    // accumulate mode, staged: input chunks of a pass
  // One k tile.  PH = 1, 2: also load the accumulator input of prefetch
  // group PH-1.
  auto iteration = [&](int kt, auto ph) {
    constexpr int PH = decltype(ph)::value;
    const int nxt = (cur + 1 == NS) ? 0 : cur + 1;
    const int prv = (cur == 0) ? NS - 1 : cur - 1;   // buffer of tile kt+NS-1
    // Second half of tile kt+NS-1's loads.  At kt = 0 this repeats loads of
    // the prologue: the same bytes to the same place, first read after
    // barrier NS-2.
    const uint32_t kadd1 = kadd_of((kt + NS - 1) * BK);
#pragma unroll
    for (int kk = 0; kk + 1 < KK; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        mfma_one(kk & 1, q);
        if (q % RS == 0 && q / RS < FM + FN) fread_one(cur, kk + 1, (kk + 1) & 1, q / RS);
#pragma unroll
        for (int d = C; d < N_DMA; ++d)
          if (kk == 0 && (d - C) * NMF / C == q) dma_one(prv, kadd1, d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The compiler does not order the global->LDS loads before the barrier
    // by itself: wait until tile kt+1's have landed.  The loads of tiles
    // kt+2 .. kt+NS-1 ((NS-2) * N_DMA instructions) may stay in flight;
    // forwarded stores issued after them only make the wait stricter.
    wait_vmcnt<(NS - 2) * N_DMA>();
    __syncthreads();
    {
      const uint32_t kadd = kadd_of((kt + NS) * BK);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        mfma_one((KK - 1) & 1, q);
        if (q % RS == 0 && q / RS < FM + FN) fread_one(nxt, 0, 0, q / RS);
#pragma unroll
        for (int d = 0; d < C; ++d)
          if (d * NMF / C == q) dma_one(cur, kadd, d);
        if constexpr (ACS && PH == 3) {
          // pass 0's input chunks, a k tile ahead of the epilogue
#pragma unroll
          for (int it = 0; it < EIT; ++it)
            if (it * NMF / EIT == q)
              cinv[it] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
                  cin + static_cast<int64_t>(m0 + erow(0, it) + e_r) * a.ldcin + n0 + EPC * e_c));
        }
        if constexpr (PREF && PH > 0) {
          if (q < 4 * PER_IT) {
            // whole tiles only (peel is false at the matrix edges)
            const int bb = (PH - 1) * PER_IT + q / 4, qq = q % 4;
            cpre[bb][qq] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
                cin_w + (bb / FN) * 32 * a.ldcin + (bb % FN) * 32 + 8 * qq));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Forward tile kt+1 (fused permute) after this step's work is issued.
    if (kt + 1 < KT) forward(nxt, kt + 1);
    cur = nxt;
  };
  using P0 = std::integral_constant<int, 0>;
  const bool peel = NPRE > 0 && KT >= 3 && 4 * PER_IT <= NMF && m0 + BM <= a.M && n0 + BN <= a.N;
  // (EPI_FINAL: no early load -- a consumer tile reads its input batch by
  // batch with the other partial and the residual, see the staged epilogue)
  const bool pf = ACS && !FIN && KT >= 2 && m0 + BM <= a.M && n0 + BN <= a.N &&
                  (reinterpret_cast<uintptr_t>(cin) & 15) == 0 && a.ldcin % 4 == 0;
  const int KT_main = peel ? KT - 3 : (pf ? KT - 2 : KT);
  for (int kt = 0; kt < KT_main; ++kt) iteration(kt, P0{});
  if constexpr (ACS) {
    if (pf) {
      iteration(KT - 2, std::integral_constant<int, 3>{});
      iteration(KT - 1, P0{});
    }
  }
  if constexpr (PREF) {
    if (peel) {
      iteration(KT - 3, std::integral_constant<int, 1>{});
      iteration(KT - 2, std::integral_constant<int, 2>{});
      iteration(KT - 1, P0{});
    } else {
#pragma unroll
      for (int bb = 0; bb < NPRE; ++bb)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) cpre[bb][qq] = load_cin_quad(a, cin, quad_m(bb), quad_n(bb, qq));
    }
  }
  // The last iterations issued loads past K (they land as zeros); drain them
  // before the workgroup's LDS can be handed to another workgroup.
  wait_vmcnt<0>();

  if constexpr (STAGED) {
    // EPI_FINAL: this tile's role in its chunk (claim_chunk)
    int role = 0, slot = 0;
    const float* pw = nullptr;
    if constexpr (FIN) {
      slot = a.fin.oid[g] * a.tiles_per_group + tm * a.tiles_n + tn;
      role = claim_chunk(a, g, slot, &pw, reinterpret_cast<int*>(smem + NS * STAGE));
      if (role < 0) return;
    }
    // every wave's last fragment reads are done before LDS is overwritten
    __syncthreads();
    f32x4 b4 = {0.0f, 0.0f, 0.0f, 0.0f};
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rc = make_rsrc(cbase, kMaxRsrcBytes);
    if constexpr (FIN) {
      const int n = n0 + EPC * e_c;   // every chunk of this thread has this column
      if (role != 1 && a.fin.bias) b4 = load_t4<TOut>(a.fin.bias, n, n, a.N, false);
    }
#pragma unroll
    for (int p = 0; p < EP; ++p) {
      if (p > 0) __syncthreads();   // the previous pass's reads are done
      if constexpr (ACS) {
        // this pass's input chunks, in flight while the pass is staged (a
        // consumer tile of an EPI_FINAL launch loads them batch by batch)
        if ((p > 0 || !pf) && !(FIN && (role != 1 || cin == nullptr))) {
          if (pf) {
            // whole, aligned tile: no per-lane edge branches between the loads
#pragma unroll
            for (int it = 0; it < EIT; ++it)
              cinv[it] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
                  cin + static_cast<int64_t>(m0 + erow(p, it) + e_r) * a.ldcin + n0 + EPC * e_c));
          } else {
#pragma unroll
            for (int it = 0; it < EIT; ++it)
              cinv[it] = load_cin_quad(a, cin, m0 + erow(p, it) + e_r, n0 + EPC * e_c);
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < EJP; ++jj) {
        const int j = p * EJP + jj;
        const int lr = wm * 32 * EJP + jj * 32 + (lane & 31);
        char* srow = smem + lr * ERB;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 v = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                       acc[i][j][4 * q + 3]};
            const int byte = (wn * WTN + 32 * i + 8 * q + 4 * (lane >> 5)) * ESZ;
            char* d = srow + (((byte >> 4) ^ (lr & ESW)) << 4) + (byte & 15);
            if (GELU) {
              for (int e = 0; e < 4; ++e) v[e] = gelu_exact(v[e]);
            }
            if constexpr (ESZ == 4) {
              *reinterpret_cast<f32x4*>(d) = v;
            } else {
              bf16x4 h;
              for (int e = 0; e < 4; ++e) h[e] = static_cast<__bf16>(v[e]);
              *reinterpret_cast<bf16x4*>(d) = h;
            }
          }
        }
      }
      __syncthreads();
      if constexpr (FIN) {
        if (role != 1) {
          // Chunk consumer (consume_pass); one uniform branch on `whole`.
          const int oid = a.fin.oid[g];
          const void* resp = a.fin.res[oid];
          void* outp = a.fin.out[oid];
          const int64_t mr0 = a.fin.mrow0[oid];
          const __amdgpu_buffer_rsrc_t rpw = make_rsrc(uniform_ptr(pw), kMaxRsrcBytes);
          if (whole)
            consume_pass<TOut, true, EIT, ERI, EJP, WTM, ERB, ESW, EPC>(
                a, smem, p, m0, n0, e_r, e_c, cin, rpw, pw != nullptr, resp, outp, mr0, b4);
          else
            consume_pass<TOut, false, EIT, ERI, EJP, WTM, ERB, ESW, EPC>(
                a, smem, p, m0, n0, e_r, e_c, cin, rpw, pw != nullptr, resp, outp, mr0, b4);
          continue;
        }
      }
      if constexpr (FIN) {
        // The first producer's partial, published to the pair's consumer
        // (device-coherent stores); whole tiles take a path without per-lane
        // edge checks.
        if (whole) {
#pragma unroll
          for (int it = 0; it < EIT; ++it) {
            const int lr = ERI * it + e_r;
            const u32x4 raw = *reinterpret_cast<const u32x4*>(smem + lr * ERB + ((e_c ^ (lr & ESW)) << 4));
            const int m = m0 + erow(p, it) + e_r;
            const int n = n0 + EPC * e_c;
            const f32x4 v = cin ? cinv[it] + __builtin_bit_cast(f32x4, raw) : __builtin_bit_cast(f32x4, raw);
            store_dev4<true>(rc, static_cast<uint32_t>((m * a.ldc + n) * 4), v, n, a.N);
          }
        } else {
#pragma unroll
          for (int it = 0; it < EIT; ++it) {
            const int lr = ERI * it + e_r;
            const u32x4 raw = *reinterpret_cast<const u32x4*>(smem + lr * ERB + ((e_c ^ (lr & ESW)) << 4));
            const int m = m0 + erow(p, it) + e_r;
            const int n = n0 + EPC * e_c;
            if (m >= a.M || n >= a.N) continue;
            const f32x4 v = cin ? cinv[it] + __builtin_bit_cast(f32x4, raw) : __builtin_bit_cast(f32x4, raw);
            store_dev4(rc, static_cast<uint32_t>((m * a.ldc + n) * 4), v, n, a.N);
          }
        }
        continue;
      }
      if (whole && vec) {
        // Whole tile, 16-byte rows: straight-line code.  (A per-lane branch
        // between the stores -- vector or element by element -- leaves the
        // compiler unsure how many stores are in flight at the next use of a
        // loaded input, and it then waits for all of them: one full drain
        // per chunk.)
#pragma unroll
        for (int it = 0; it < EIT; ++it) {
          const int lr = ERI * it + e_r;
          const u32x4 raw = *reinterpret_cast<const u32x4*>(smem + lr * ERB + ((e_c ^ (lr & ESW)) << 4));
          const int m = m0 + erow(p, it) + e_r;
          const int n = n0 + EPC * e_c;
          TS* dst = reinterpret_cast<TS*>(cbase) + static_cast<int64_t>(m) * a.ldc + n;
          if constexpr (ACS) {
            const f32x4 v = cinv[it] + __builtin_bit_cast(f32x4, raw);
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
          } else {
            __builtin_nontemporal_store(raw, reinterpret_cast<u32x4*>(dst));
          }
        }
        continue;
      }
#pragma unroll
      for (int it = 0; it < EIT; ++it) {
        const int lr = ERI * it + e_r;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(smem + lr * ERB + ((e_c ^ (lr & ESW)) << 4));
        const int m = m0 + erow(p, it) + e_r;
        const int n = n0 + EPC * e_c;
        if (!whole && (m >= a.M || n >= a.N)) continue;
        TS* dst = reinterpret_cast<TS*>(cbase) + static_cast<int64_t>(m) * a.ldc + n;
        if constexpr (ACS) {
          // C = Cin + part, the register epilogue's addition.  Results are
          // read once, by a later launch: nontemporal stores, here and below.
          const f32x4 v = cinv[it] + __builtin_bit_cast(f32x4, raw);
          if (vec && (whole || n + EPC <= a.N)) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
          } else {
            for (int e = 0; e < EPC; ++e)
              if (n + e < a.N) reinterpret_cast<float*>(dst)[e] = v[e];
          }
          continue;
        }
        if (vec && (whole || n + EPC <= a.N)) {
          __builtin_nontemporal_store(raw, reinterpret_cast<u32x4*>(dst));
        } else {
          const TS* src = reinterpret_cast<const TS*>(&raw);
          for (int e = 0; e < EPC; ++e)
            if (n + e < a.N) dst[e] = src[e];
        }
      }
    }
    if constexpr (FIN) {
      if (role == 1) publish_chunk(a, slot);
    }
    return;
  }

  // Epilogue, one block at a time (register pressure).  Accumulate mode:
  // blocks below NPRE take the prefetched input; for the others the input of
  // block b+1 is loaded before block b is finished, so its latency overlaps
  // block b's stores.
  f32x4 cb[2][4];
  if (PREF && NPRE < NB) {
#pragma unroll
    for (int q = 0; q < 4; ++q) cb[NPRE & 1][q] = load_cin_quad(a, cin, quad_m(NPRE), quad_n(NPRE, q));
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int i = b % FN, j = b / FN;
    if (PREF && b + 1 > NPRE && b + 1 < NB) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        cb[(b + 1) & 1][q] = load_cin_quad(a, cin, quad_m(b + 1), quad_n(b + 1, q));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 v = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                 acc[i][j][4 * q + 3]};
      f32x4 cv = f32x4{};
      if (PREF) cv = (b < NPRE) ? cpre[b < NPRE ? b : 0][q] : cb[b & 1][q];
      store_quad<TOut, EPI, GELU>(a, cbase, quad_m(b), quad_n(b, q), v, cv);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// fp32 MFMA kernel (v_mfma_f32_32x32x2_f32): 64x64 tiles, k step 16.
// ---------------------------------------------------------------------------
template <typename TOut, int EPI, bool GELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(KArgs a) {
  // 64 x 64 tiles, 32-deep k chunks in two LDS buffers: chunk c+1's global
  // loads are in flight (in registers) while chunk c's MFMAs run, and are
  // written to the other buffer afterwards, so each chunk costs one barrier
  // and no exposed load latency beyond the first.  (With 16-deep chunks and
  // a load-barrier-compute loop, a launch of 4 x 64 x 512 x 256 took 17 us,
  // almost all of it waiting for loads.)  The MFMAs see k in the same order
  // as any other chunking, so the results do not depend on it.
  constexpr int BM = 64, BN = 64, BK = 32, LDK = BK + 1;
  __shared__ float sa[2][BM * LDK];
  __shared__ float sb[2][BN * LDK];
  int g, tm, tn;
  map_tile(a, g, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float* A = reinterpret_cast<const float*>(a.p.a[g]);
  const float* B = reinterpret_cast<const float*>(a.p.b[g]);
  float* fd = reinterpret_cast<float*>(a.p.fwd[g]);
  // loads: thread t takes rows t / 8 and t / 8 + 32 of each operand's chunk,
  // 4 consecutive k at (t % 8) * 4 (K is a multiple of 8)
  const int lr = tid >> 3, lc = (tid & 7) * 4;
  f32x4 va[2], vb[2];
  auto gload = [&](int k0) {
    const int k = k0 + lc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = m0 + lr + 32 * h, n = n0 + lr + 32 * h;
      va[h] = (m < a.M && k < a.K) ? *reinterpret_cast<const f32x4*>(A + static_cast<int64_t>(m) * a.lda + k)
                                   : f32x4{};
      vb[h] = (n < a.N && k < a.K) ? *reinterpret_cast<const f32x4*>(B + static_cast<int64_t>(n) * a.ldb + k)
                                   : f32x4{};
    }
  };
  auto lstore = [&](int buf, int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sa[buf][(lr + 32 * h) * LDK + lc + e] = va[h][e];
        sb[buf][(lr + 32 * h) * LDK + lc + e] = vb[h][e];
      }
    // fused permute: forward the looped operand's k chunk (once per row block)
    const int kt = k0 / BK, k = k0 + lc;
    if (fd == nullptr || k >= a.K) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = m0 + lr + 32 * h, n = n0 + lr + 32 * h;
      if (a.fwd == FWD_A && kt % a.tiles_n == tn && m < a.M)
        *reinterpret_cast<f32x4*>(fd + static_cast<int64_t>(m) * a.ldfwd + k) = va[h];
      if (a.fwd == FWD_B && kt % a.tiles_m == tm && n < a.N)
        *reinterpret_cast<f32x4*>(fd + static_cast<int64_t>(n) * a.ldfwd + k) = vb[h];
    }
  };
  f32x16 acc = f32x16{};
  const int nk = (a.K + BK - 1) / BK;
  if (nk > 0) {
    gload(0);
    lstore(0, 0);
  }
  for (int c = 0; c < nk; ++c) {
    const int cur = c & 1;
    if (c + 1 < nk) gload((c + 1) * BK);
    // chunk c's stores are visible; every wave is done with chunk c-1's
    // buffer, which the stores below overwrite
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      const float x = sb[cur][(wn * 32 + (lane & 31)) * LDK + k];
      const float y = sa[cur][(wm * 32 + (lane & 31)) * LDK + k];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, acc, 0, 0, 0);
    }
    if (c + 1 < nk) lstore(cur ^ 1, (c + 1) * BK);
  }
  const int m = m0 + wm * 32 + (lane & 31);
  if constexpr (EPI == EPI_FINAL) {
    // the chunk protocol of the bf16 kernel on the register path
    static_assert(!GELU, "EPI_FINAL has no GELU");
    const int slot = a.fin.oid[g] * a.tiles_per_group + tm * a.tiles_n + tn;
    const float* pw = nullptr;
    __shared__ int claim_sh[2];
    const int role = claim_chunk(a, g, slot, &pw, claim_sh);
    if (role < 0) return;
    const int oid = a.fin.oid[g];
    const float* cin = a.p.cin[g];
    f32x4 cv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      cv[q] = cin ? load_cin_quad(a, cin, m, n0 + wn * 32 + 8 * q + 4 * (lane >> 5)) : f32x4{};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + wn * 32 + 8 * q + 4 * (lane >> 5);
      if (m >= a.M || n >= a.N) continue;
      const f32x4 part = {acc[4 * q + 0], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      const f32x4 v = cin ? cv[q] + part : part;
      if (role == 1) {
        store_dev4(make_rsrc(a.p.c[g], kMaxRsrcBytes), static_cast<uint32_t>((m * a.ldc + n) * 4), v,
                   n, a.N);
        continue;
      }
      const f32x4 w = pw ? load_dev4(make_rsrc(pw, kMaxRsrcBytes),
                                     static_cast<uint32_t>((m * a.ldc + n) * 4), n, a.N)
                         : f32x4{};
      const void* resp = a.fin.res[oid];
      const f32x4 r = resp ? load_t4<TOut>(resp, static_cast<int64_t>(m) * a.fin.ld_res + n, n, a.N, true)
                           : f32x4{};
      const f32x4 b = a.fin.bias ? load_t4<TOut>(a.fin.bias, n, n, a.N, false) : f32x4{};
      const unsigned keep = a.fin.mode == 1 ? keep_bits4(a.fin, a.fin.mrow0[oid], m, n) : 0u;
      consume4<TOut>(a.fin, m, n, a.N, v, pw != nullptr, w, b, resp != nullptr, r, keep,
                     a.fin.out[oid]);
    }
    if (role == 1) publish_chunk(a, slot);
    return;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + wn * 32 + 8 * q + 4 * (lane >> 5);
      f32x4 v = {acc[4 * q + 0], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      const f32x4 cinv = EPI == EPI_ACCUM ? load_cin_quad(a, a.p.cin[g], m, n) : f32x4{};
      store_quad<TOut, EPI, GELU>(a, a.p.c[g], m, n, v, cinv);
    }
  }
}

// Zeroes n 32-bit words (the chunk signal words of a call).
__global__ __launch_bounds__(256) void zero_words_kernel(unsigned* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
template <typename TOut, int EPI, bool GELU>
hipError_t launch_typed(const GemmLaunch& L, KArgs& k, hipStream_t s) {
  bool sig_fits = true;
  auto grid_for = [&](int bm, int bn) {
    k.tiles_m = static_cast<int>((L.M + bm - 1) / bm);
    k.tiles_n = static_cast<int>((L.N + bn - 1) / bn);
    k.tiles_per_group = k.tiles_m * k.tiles_n;
    k.total_tiles = k.tiles_per_group * L.groups;
    // EPI_FINAL: each output's chunks index its signal words
    if (EPI == EPI_FINAL && k.tiles_per_group > L.fin.sig_tiles) sig_fits = false;
    return k.total_tiles;
  };
  if (L.in_t == CCE_F32) {
    const int t = grid_for(64, 64);
    if (!sig_fits) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_f32_kernel<TOut, EPI, GELU>), dim3(t), dim3(256), 0, s, k);
    return hipGetLastError();
  }
  // bf16: pick the largest tile that still gives every CU work.
  constexpr int kCUs = 256;
  auto tiles = [&](int bm, int bn) {
    return static_cast<int64_t>(L.groups) * ((L.M + bm - 1) / bm) * ((L.N + bn - 1) / bn);
  };
  if (tiles(256, 256) >= kCUs) {
    const int t = grid_for(256, 256);
    if (!sig_fits) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 2, kBK, kNS, TOut, EPI, GELU>), dim3(t), dim3(256), 0, s, k);
  } else if (tiles(256, 128) >= kCUs) {
    const int t = grid_for(256, 128);
    if (!sig_fits) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 128, 2, 2, kBK, kNS, TOut, EPI, GELU>), dim3(t), dim3(256), 0, s, k);
  } else {
    const int t = grid_for(128, 128);
    if (!sig_fits) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, kBK, kNS, TOut, EPI, GELU>), dim3(t), dim3(256), 0, s, k);
  }
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_out(const GemmLaunch& L, KArgs& k, hipStream_t s) {
  if (L.epi == EPI_FINAL) return launch_typed<TOut, EPI_FINAL, false>(L, k, s);
  if (L.epi == EPI_STORE)
    return L.gelu ? launch_typed<TOut, EPI_STORE, true>(L, k, s)
                  : launch_typed<TOut, EPI_STORE, false>(L, k, s);
  return L.gelu ? launch_typed<TOut, EPI_ACCUM, true>(L, k, s)
                : launch_typed<TOut, EPI_ACCUM, false>(L, k, s);
}

}  // namespace

cce_status launch_grouped_gemm(const GemmLaunch& L, void* stream) {
  if (L.groups <= 0 || L.M <= 0 || L.N <= 0) return CCE_OK;
  // The accumulator input is read in 16-byte vectors (load_cin_quad and the
  // staged path): every cin must be 16-byte aligned with ldcin % 4 == 0.
  // The plans only pass workspace accumulators, which are; anything else is a
  // planning error, caught here before a launch.
  if (L.epi == EPI_ACCUM || L.epi == EPI_FINAL) {
    if (L.ldcin % 4 != 0) return fail(CCE_EINVAL, "gemm launch: accumulator input ld % 4 != 0");
    for (int g = 0; g < L.groups; ++g)
      if (reinterpret_cast<uintptr_t>(L.p.cin[g]) & 15)
        return fail(CCE_EINVAL, "gemm launch: accumulator input not 16-byte aligned");
  }
  KArgs k{};
  k.groups = L.groups;
  k.M = static_cast<int>(L.M);
  k.N = static_cast<int>(L.N);
  k.K = static_cast<int>(L.K);
  k.lda = static_cast<int>(L.lda);
  k.ldb = static_cast<int>(L.ldb);
  k.ldc = static_cast<int>(L.ldc);
  k.ldcin = static_cast<int>(L.ldcin);
  k.fwd = L.fwd;
  k.ldfwd = static_cast<int>(L.ldfwd);
  k.p = L.p;
  k.fin = L.fin;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = (L.out_t == CCE_F32) ? launch_out<float>(L, k, s) : launch_out<__bf16>(L, k, s);
  if (e != hipSuccess) return fail(CCE_EHIP, std::string("gemm launch: ") + hipGetErrorString(e));
  return CCE_OK;
}

cce_status launch_zero_words(unsigned* p, int64_t n, void* stream) {
  if (n <= 0) return CCE_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p, n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CCE_EHIP, std::string("zero_words launch: ") + hipGetErrorString(e));
  return CCE_OK;
}

}  // namespace cce
