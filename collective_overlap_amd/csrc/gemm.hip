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
#include <cstdint>

#include "cce_internal.hpp"

namespace cce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kOutOfRange = 0x7ffffff0;    // offset steered past num_records

struct KArgs {
  int groups;
  int M, N, K;
  int lda, ldb, ldc, ldcin;   // elements
  int tiles_m, tiles_n, tiles_per_group, total_tiles;
  GemmGroupPtrs p;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  int n = bytes > 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes);
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

__device__ __forceinline__ float gelu_exact(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// Epilogue for 4 consecutive columns [n, n+4) of row m.
template <typename TOut, int EPI, bool GELU>
__device__ __forceinline__ void store_quad(const KArgs& a, void* cbase, const float* cinbase, int m,
                                           int n, f32x4 v) {
  if (m >= a.M || n >= a.N) return;
  const bool full = (n + 3 < a.N);
  if (EPI == EPI_ACCUM) {
    const float* cin = cinbase + static_cast<int64_t>(m) * a.ldcin + n;
    if (full) {
      f32x4 r = *reinterpret_cast<const f32x4*>(cin);
      v = r + v;
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < a.N) v[e] = cin[e] + v[e];
    }
  }
  if (GELU) {
    for (int e = 0; e < 4; ++e) v[e] = gelu_exact(v[e]);
  }
  if constexpr (sizeof(TOut) == 4) {
    float* c = reinterpret_cast<float*>(cbase) + static_cast<int64_t>(m) * a.ldc + n;
    if (full) {
      *reinterpret_cast<f32x4*>(c) = v;
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < a.N) c[e] = v[e];
    }
  } else {
    __bf16* c = reinterpret_cast<__bf16*>(cbase) + static_cast<int64_t>(m) * a.ldc + n;
    bf16x4 h;
    for (int e = 0; e < 4; ++e) h[e] = static_cast<__bf16>(v[e]);
    if (full) {
      *reinterpret_cast<bf16x4*>(c) = h;
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < a.N) c[e] = h[e];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, typename TOut, int EPI, bool GELU>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(KArgs a) {
  constexpr int BK = 64;                     // 8 chunks of 8 bf16 per row
  constexpr int ROWB = BK * 2;               // bytes per LDS row
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_CH = BM * 8 / 256;         // 16-byte chunks per thread per stage
  constexpr int B_CH = BN * 8 / 256;
  constexpr int STAGE = (BM + BN) * ROWB;
  static_assert(WM * WN == 4, "4 waves");
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  int g, tm, tn;
  map_tile(a, g, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const __bf16* A = reinterpret_cast<const __bf16*>(a.p.a[g]);
  const __bf16* B = reinterpret_cast<const __bf16*>(a.p.b[g]);
  // Buffer ranges: rows [m0, M) of A and [n0, N) of B^T.
  const int64_t a_bytes = (static_cast<int64_t>(a.M - m0 - 1) * a.lda + a.K) * 2;
  const int64_t b_bytes = (static_cast<int64_t>(a.N - n0 - 1) * a.ldb + a.K) * 2;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * a.lda, a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + static_cast<int64_t>(n0) * a.ldb, b_bytes);

  // Per-thread chunk coordinates: chunk c = tid % 8 of rows tid/8 + 32*p.
  const int lc = tid & 7;
  const int lr = tid >> 3;
  int a_off[A_CH], b_off[B_CH];       // byte offsets at k0 = 0 (row part)
  int a_lds[A_CH], b_lds[B_CH];       // LDS byte offsets (swizzled)
#pragma unroll
  for (int p = 0; p < A_CH; ++p) {
    const int r = lr + 32 * p;
    a_off[p] = (m0 + r < a.M) ? (r * a.lda + lc * 8) * 2 : kOutOfRange;
    a_lds[p] = r * ROWB + ((lc ^ (r & 7)) << 4);
  }
#pragma unroll
  for (int p = 0; p < B_CH; ++p) {
    const int r = lr + 32 * p;
    b_off[p] = (n0 + r < a.N) ? (r * a.ldb + lc * 8) * 2 : kOutOfRange;
    b_lds[p] = BM * ROWB + r * ROWB + ((lc ^ (r & 7)) << 4);
  }

  u32x4 ra_reg[A_CH], rb_reg[B_CH];
  auto gload = [&](int k0) {
    const bool kin = (k0 + lc * 8) < a.K;
#pragma unroll
    for (int p = 0; p < A_CH; ++p)
      ra_reg[p] = __builtin_amdgcn_raw_buffer_load_b128(ra, kin ? a_off[p] + k0 * 2 : kOutOfRange, 0, 0);
#pragma unroll
    for (int p = 0; p < B_CH; ++p)
      rb_reg[p] = __builtin_amdgcn_raw_buffer_load_b128(rb, kin ? b_off[p] + k0 * 2 : kOutOfRange, 0, 0);
  };
  auto lstore = [&](int stage) {
    char* s = smem + stage * STAGE;
#pragma unroll
    for (int p = 0; p < A_CH; ++p) *reinterpret_cast<u32x4*>(s + a_lds[p]) = ra_reg[p];
#pragma unroll
    for (int p = 0; p < B_CH; ++p) *reinterpret_cast<u32x4*>(s + b_lds[p]) = rb_reg[p];
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};

  // Fragment rows read by this lane.
  const int frow = lane & 31;
  const int fk = lane >> 5;           // which 8-element half of a 16-wide k step
  const int KT = (a.K + BK - 1) / BK;

  if (KT > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const char* s = smem + cur * STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + fk;
      bf16x8 bf[FN], af[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int r = wn * WTN + i * 32 + frow;
        bf[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               s + BM * ROWB + r * ROWB + ((c ^ (r & 7)) << 4)));
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int r = wm * WTM + j * 32 + frow;
        af[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               s + r * ROWB + ((c ^ (r & 7)) << 4)));
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[i], af[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: block (i, j) holds C^T; lane owns row m, columns n..n+3 per quad.
  void* cbase = a.p.c[g];
  const float* cin = a.p.cin[g];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int m = m0 + wm * WTM + j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WTN + i * 32 + 8 * q + 4 * (lane >> 5);
        f32x4 v = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                   acc[i][j][4 * q + 3]};
        store_quad<TOut, EPI, GELU>(a, cbase, cin, m, n, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 MFMA kernel (v_mfma_f32_32x32x2_f32): 64x64 tiles, k step 16.
// ---------------------------------------------------------------------------
template <typename TOut, int EPI, bool GELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(KArgs a) {
  constexpr int BM = 64, BN = 64, BK = 16, LDK = BK + 1;
  __shared__ float sa[BM * LDK];
  __shared__ float sb[BN * LDK];
  int g, tm, tn;
  map_tile(a, g, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float* A = reinterpret_cast<const float*>(a.p.a[g]);
  const float* B = reinterpret_cast<const float*>(a.p.b[g]);
  const int lr = tid >> 2, lc = (tid & 3) * 4;
  f32x16 acc = f32x16{};
  for (int k0 = 0; k0 < a.K; k0 += BK) {
    {
      const int m = m0 + lr, k = k0 + lc;
      f32x4 v = f32x4{};
      if (m < a.M && k < a.K) v = *reinterpret_cast<const f32x4*>(A + static_cast<int64_t>(m) * a.lda + k);
      for (int e = 0; e < 4; ++e) sa[lr * LDK + lc + e] = v[e];
      const int n = n0 + lr;
      f32x4 w = f32x4{};
      if (n < a.N && k < a.K) w = *reinterpret_cast<const f32x4*>(B + static_cast<int64_t>(n) * a.ldb + k);
      for (int e = 0; e < 4; ++e) sb[lr * LDK + lc + e] = w[e];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      const float x = sb[(wn * 32 + (lane & 31)) * LDK + k];
      const float y = sa[(wm * 32 + (lane & 31)) * LDK + k];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  const int m = m0 + wm * 32 + (lane & 31);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = n0 + wn * 32 + 8 * q + 4 * (lane >> 5);
    f32x4 v = {acc[4 * q + 0], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    store_quad<TOut, EPI, GELU>(a, a.p.c[g], a.p.cin[g], m, n, v);
  }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
template <typename TOut, int EPI, bool GELU>
hipError_t launch_typed(const GemmLaunch& L, KArgs& k, hipStream_t s) {
  auto grid_for = [&](int bm, int bn) {
    k.tiles_m = static_cast<int>((L.M + bm - 1) / bm);
    k.tiles_n = static_cast<int>((L.N + bn - 1) / bn);
    k.tiles_per_group = k.tiles_m * k.tiles_n;
    k.total_tiles = k.tiles_per_group * L.groups;
    return k.total_tiles;
  };
  if (L.in_t == CCE_F32) {
    const int t = grid_for(64, 64);
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
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 2, TOut, EPI, GELU>), dim3(t), dim3(256), 0, s, k);
  } else if (tiles(256, 128) >= kCUs) {
    const int t = grid_for(256, 128);
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 128, 2, 2, TOut, EPI, GELU>), dim3(t), dim3(256), 0, s, k);
  } else {
    const int t = grid_for(128, 128);
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, TOut, EPI, GELU>), dim3(t), dim3(256), 0, s, k);
  }
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_out(const GemmLaunch& L, KArgs& k, hipStream_t s) {
  if (L.epi == EPI_STORE)
    return L.gelu ? launch_typed<TOut, EPI_STORE, true>(L, k, s)
                  : launch_typed<TOut, EPI_STORE, false>(L, k, s);
  return L.gelu ? launch_typed<TOut, EPI_ACCUM, true>(L, k, s)
                : launch_typed<TOut, EPI_ACCUM, false>(L, k, s);
}

}  // namespace

cce_status launch_grouped_gemm(const GemmLaunch& L, void* stream) {
  if (L.groups <= 0 || L.M <= 0 || L.N <= 0) return CCE_OK;
  KArgs k{};
  k.groups = L.groups;
  k.M = static_cast<int>(L.M);
  k.N = static_cast<int>(L.N);
  k.K = static_cast<int>(L.K);
  k.lda = static_cast<int>(L.lda);
  k.ldb = static_cast<int>(L.ldb);
  k.ldc = static_cast<int>(L.ldc);
  k.ldcin = static_cast<int>(L.ldcin);
  k.p = L.p;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = (L.out_t == CCE_F32) ? launch_out<float>(L, k, s) : launch_out<__bf16>(L, k, s);
  if (e != hipSuccess) return fail(CCE_EHIP, std::string("gemm launch: ") + hipGetErrorString(e));
  return CCE_OK;
}

}  // namespace cce
