// C ABI of the library: argument validation, contexts, workspace layout and
// the executor that turns a plan (plan.cpp) into HIP stream operations.
//
// Stream/event discipline follows the completion-handle pattern of MCR-DL
// (Anthony et al., "MCR-DL: Mix-and-Match Communication Runtime for Deep
// Learning", its synchronization section): transfers are posted to an
// internal communication stream, an event is recorded after them, and the
// consumer waits on that event instead of synchronising the host.  A call
// forks the copy stream from the caller's stream when its first copy reads
// caller data; the last copy is always waited for by the last GEMM on the
// caller's stream, which joins the copy stream back.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "cce_internal.hpp"

struct cce_prof_slot {
  int kind = 0;
  int iter = -1;
  double flops = 0, bytes = 0;
  hipEvent_t start = nullptr, stop = nullptr;
};

struct cce_ctx {
  int device = 0;
  hipStream_t copy = nullptr;            // the stream the permute copies run on
  hipStream_t own_copy = nullptr;        // the context's own copy stream
  unsigned* err = nullptr;               // device word: chunk consumers that gave up (fine-grained overlap)
  std::vector<hipEvent_t> events;        // ordering events (no timing)
  bool profiling = false;
  std::vector<hipEvent_t> timing_pool;   // timing events, reused
  size_t timing_used = 0;
  std::vector<cce_prof_slot> prof;
};

namespace cce {

namespace {
thread_local std::string g_err;

// Error-path test hook (cce_debug_fail_op): plan operation g_fail_at of a
// looped call on this thread fails as a HIP error would.  Fires once.
thread_local int g_fail_at = 0;
thread_local int g_ops_seen = 0;

// Test hook of the fine-grained overlap's bounded wait (cce_debug_signal_giveup):
// the next fine-grained call's first producers do not publish and its
// consumers poll at most this many times.  Fires once.
thread_local int g_giveup_polls = 0;

bool fail_due() {
  if (g_fail_at <= 0) return false;
  if (++g_ops_seen != g_fail_at) return false;
  g_fail_at = 0;
  return true;
}

// GEMM operands are addressed through 32-bit buffer offsets (see gemm.hip).
constexpr int64_t kMaxOperandBytes = (int64_t{1} << 30) - 256;

size_t esize(cce_dtype t) { return t == CCE_F32 ? 4 : 2; }
bool dtype_ok(int t) { return t == CCE_F32 || t == CCE_BF16; }
int64_t align256(int64_t b) { return (b + 255) & ~int64_t{255}; }
int64_t round8(int64_t v) { return (v + 7) & ~int64_t{7}; }

int64_t span_bytes(const cce_mat& m, size_t es) {
  if (m.rows <= 0 || m.cols <= 0) return 0;
  return ((m.rows - 1) * m.ld + m.cols) * static_cast<int64_t>(es);
}

std::string mat_str(const cce_mat& m) {
  return "[" + std::to_string(m.rows) + "," + std::to_string(m.cols) + "] ld " + std::to_string(m.ld);
}

cce_status check_mat(const char* name, const cce_mat& m) {
  if (m.rows < 0 || m.cols < 0 || m.ld < m.cols || m.ld < 0)
    return fail(CCE_EINVAL, std::string(name) + ": bad extents " + mat_str(m));
  if (m.ld % 8 != 0)
    return fail(CCE_EUNSUPPORTED, std::string(name) + ": ld must be a multiple of 8, got " + mat_str(m));
  if (m.rows > 0x7fffffff || m.cols > 0x7fffffff || m.ld > 0x7fffffff)
    return fail(CCE_EUNSUPPORTED, std::string(name) + ": extent exceeds 2^31");
  return CCE_OK;
}

cce_status check_ptr(const char* name, const void* p, int64_t span) {
  if (span == 0) return CCE_OK;
  if (!p) return fail(CCE_EINVAL, std::string(name) + ": NULL pointer");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(CCE_EUNSUPPORTED, std::string(name) + ": pointer not 16-byte aligned");
  return CCE_OK;
}

struct Range {
  uintptr_t lo, hi;
  std::string name;
  bool writes;
};

// Outputs may overlap nothing; inputs may overlap each other.
cce_status check_overlaps(const std::vector<Range>& rs) {
  for (size_t i = 0; i < rs.size(); ++i) {
    if (rs[i].hi <= rs[i].lo) continue;
    for (size_t j = i + 1; j < rs.size(); ++j) {
      if (rs[j].hi <= rs[j].lo) continue;
      if (!rs[i].writes && !rs[j].writes) continue;
      if (rs[i].lo < rs[j].hi && rs[j].lo < rs[i].hi)
        return fail(CCE_EINVAL, rs[i].name + " overlaps " + rs[j].name);
    }
  }
  return CCE_OK;
}

Range range_of(const void* p, int64_t span, const std::string& name, bool writes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(span), name, writes};
}

#define CCE_TRY(expr)                       \
  do {                                      \
    cce_status _s = (expr);                 \
    if (_s != CCE_OK) return _s;            \
  } while (0)

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t _e = (expr);                                                        \
    if (_e != hipSuccess)                                                          \
      return fail(CCE_EHIP, std::string(#expr) + ": " + hipGetErrorString(_e));    \
  } while (0)

// Makes ctx->device current for the duration of a call.
class DeviceGuard {
 public:
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev_) != hipSuccess) prev_ = -1;
    if (prev_ != dev) hipSetDevice(dev);
    dev_ = dev;
  }
  ~DeviceGuard() {
    if (prev_ >= 0 && prev_ != dev_) hipSetDevice(prev_);
  }

 private:
  int prev_ = -1, dev_ = 0;
};

cce_status ensure_events(cce_ctx* ctx, int n) {
  while (static_cast<int>(ctx->events.size()) < n) {
    hipEvent_t e;
    HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    ctx->events.push_back(e);
  }
  return CCE_OK;
}

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free entry point
// (cce_looped_einsum_reducescatter_epilogue_noalloc): its workspace is this
// file-scope device array instead of caller memory.  Every GPU the library
// runs on holds its own copy, at its own address, until the process ends.
// The array's name is a host-side stand-in, never a device address: host
// code uses only the address hipGetSymbolAddress returns, looked up once per
// device (at cce_ctx_create, with that device current) and kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[CCE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
hipError_t g_scratch_err[kMaxScratchDevices] = {};

// Once per device, with `device` current.
void scratch_setup(int device) {
  if (device < 0 || device >= kMaxScratchDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] != nullptr) return;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e == hipSuccess && p != nullptr) {
    g_scratch_ptr[device] = p;
    g_scratch_err[device] = hipSuccess;
  } else {
    g_scratch_err[device] = (e == hipSuccess) ? hipErrorInvalidSymbol : e;
  }
}

cce_status scratch_of(int device, void** out) {
  if (device < 0 || device >= kMaxScratchDevices)
    return fail(CCE_EUNSUPPORTED, "the static scratch covers devices 0.." +
                                      std::to_string(kMaxScratchDevices - 1));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr)
    return fail(CCE_EHIP, std::string("hipGetSymbolAddress(scratch) failed on device ") +
                              std::to_string(device) + ": " +
                              hipGetErrorString(g_scratch_err[device]));
  *out = g_scratch_ptr[device];
  return CCE_OK;
}

// Timing brackets (only while profiling is enabled).
cce_status timing_event(cce_ctx* ctx, hipEvent_t* out) {
  if (ctx->timing_used == ctx->timing_pool.size()) {
    hipEvent_t e;
    HIP_TRY(hipEventCreate(&e));
    ctx->timing_pool.push_back(e);
  }
  *out = ctx->timing_pool[ctx->timing_used++];
  return CCE_OK;
}

cce_status prof_begin(cce_ctx* ctx, hipStream_t s, int kind, int iter, double flops, double bytes,
                      int* slot) {
  *slot = -1;
  if (!ctx->profiling) return CCE_OK;
  cce_prof_slot p;
  p.kind = kind;
  p.iter = iter;
  p.flops = flops;
  p.bytes = bytes;
  CCE_TRY(timing_event(ctx, &p.start));
  CCE_TRY(timing_event(ctx, &p.stop));
  HIP_TRY(hipEventRecord(p.start, s));
  ctx->prof.push_back(p);
  *slot = static_cast<int>(ctx->prof.size()) - 1;
  return CCE_OK;
}

cce_status prof_end(cce_ctx* ctx, hipStream_t s, int slot) {
  if (slot < 0) return CCE_OK;
  HIP_TRY(hipEventRecord(ctx->prof[slot].stop, s));
  return CCE_OK;
}

// ---------------------------------------------------------------------------
// AllGather: shapes and workspace
// ---------------------------------------------------------------------------
struct AgGeom {
  int n = 0;
  int mode = 0;
  bool case2 = false;
  bool case2_ws = false;
  int64_t M = 0, N = 0, K = 0;          // per-iteration GEMM (one batch element for case 3)
  int64_t bs = 1;                       // case 3: batch elements per shard
  int64_t recv_bytes = 0;               // one receive buffer (the looped shard, its ld included)
  int64_t acc_ld = 0, acc_bytes = 0;    // case-2 fp32 accumulator
  int64_t ccw_off = 0;                  // counter-clockwise receive buffers (bidirectional)
  int64_t total = 0;                    // enough for every flag combination
};

cce_status ag_geometry(int n, int mode, cce_dtype in_t, cce_dtype out_t, const cce_mat& looped,
                       const cce_mat* local, const cce_mat& out, AgGeom& g) {
  if (n < 1 || n > CCE_MAX_RANKS)
    return fail(n < 1 ? CCE_EINVAL : CCE_EUNSUPPORTED, "n_ranks out of range: " + std::to_string(n));
  if (mode < 0 || mode > 4) return fail(CCE_EINVAL, "bad AllGather mode");
  if (!dtype_ok(in_t) || !dtype_ok(out_t)) return fail(CCE_EINVAL, "bad dtype");
  CCE_TRY(check_mat("looped_shard", looped));
  CCE_TRY(check_mat("out_shape", out));
  if (local) CCE_TRY(check_mat("local_shape", *local));
  g.n = n;
  g.mode = mode;
  g.case2 = (mode == CCE_AG_LHS_COLS || mode == CCE_AG_RHS_ROWS);
  g.case2_ws = g.case2 && out_t == CCE_BF16 && n > 1;
  const int64_t nn = n;
  switch (mode) {
    case CCE_AG_LHS_ROWS:
      g.M = looped.rows; g.K = looped.cols; g.N = out.cols;
      if (out.rows != nn * looped.rows) return fail(CCE_EINVAL, "out rows must be n * looped rows");
      if (local && (local->rows != out.cols || local->cols != looped.cols))
        return fail(CCE_EINVAL, "local must be [out cols, looped cols] " + mat_str(*local));
      break;
    case CCE_AG_RHS_COLS:
      g.M = out.rows; g.K = looped.cols; g.N = looped.rows;
      if (out.cols != nn * looped.rows) return fail(CCE_EINVAL, "out cols must be n * looped rows");
      if (local && (local->rows != out.rows || local->cols != looped.cols))
        return fail(CCE_EINVAL, "local must be [out rows, looped cols] " + mat_str(*local));
      break;
    case CCE_AG_LHS_COLS:
      g.M = looped.rows; g.K = looped.cols; g.N = out.cols;
      if (out.rows != looped.rows) return fail(CCE_EINVAL, "out rows must equal looped rows");
      if (local && (local->rows != out.cols || local->cols != nn * looped.cols))
        return fail(CCE_EINVAL, "local must be [out cols, n * looped cols] " + mat_str(*local));
      break;
    case CCE_AG_RHS_ROWS:
      g.M = out.rows; g.K = looped.cols; g.N = looped.rows;
      if (out.cols != looped.rows) return fail(CCE_EINVAL, "out cols must equal looped rows");
      if (local && (local->rows != out.rows || local->cols != nn * looped.cols))
        return fail(CCE_EINVAL, "local must be [out rows, n * looped cols] " + mat_str(*local));
      break;
    case CCE_AG_LHS_BATCH:
      // b_s batch elements per shard, stacked row-wise; b_s comes from the
      // local operand (n * b_s stacked [N, K] factors), so the workspace
      // query, which has no local shape, sizes the receive buffers only.
      g.K = looped.cols; g.N = out.cols; g.M = looped.rows;
      if (out.rows != nn * looped.rows) return fail(CCE_EINVAL, "out rows must be n * looped rows");
      if (local) {
        if (local->cols != looped.cols)
          return fail(CCE_EINVAL, "local must have the looped shard's K " + mat_str(*local));
        if (out.cols == 0 || local->rows == 0 || local->rows % (nn * out.cols) != 0)
          return fail(CCE_EINVAL, "local rows must be n * b_s * out cols " + mat_str(*local));
        g.bs = local->rows / (nn * out.cols);
        if (looped.rows % g.bs != 0)
          return fail(CCE_EINVAL, "looped rows must be b_s * m (b_s = " + std::to_string(g.bs) + ")");
        g.M = looped.rows / g.bs;
      }
      break;
  }
  if (g.K % 8 != 0) return fail(CCE_EUNSUPPORTED, "contraction length must be a multiple of 8");
  // Receive buffers keep the caller's ld: one launch can hold a caller's
  // shard and a received one (iteration 0 of the two-way form), and a launch
  // has a single ld per operand.
  g.recv_bytes = (n > 1) ? align256(looped.rows * looped.ld * static_cast<int64_t>(esize(in_t))) : 0;
  if (g.case2_ws) {
    g.acc_ld = round8(out.cols);
    g.acc_bytes = align256(out.rows * g.acc_ld * 4);
  }
  g.ccw_off = 2 * nn * g.recv_bytes + (g.case2_ws ? nn * g.acc_bytes : 0);
  // The bidirectional form (case 1 only) adds two ccw receive buffers per rank.
  g.total = g.ccw_off + (g.case2 ? 0 : 2 * nn * g.recv_bytes);
  return CCE_OK;
}

// ---------------------------------------------------------------------------
// ReduceScatter: shapes and workspace
// ---------------------------------------------------------------------------
struct RsGeom {
  int n = 0;
  int mode = 0;
  int64_t K = 0;
  int64_t shard = 0;              // m_s (rows) or n_s (cols)
  int64_t other = 0;              // N (cols) or M (rows)
  int64_t h0 = 0, h1 = 0;         // half extents along the sliced dim
  int H = 2;                      // accumulator chains (halves) per shard
  int64_t acc_ld = 0, half_bytes = 0;
  int64_t region = 0;             // one set of accumulators (cw); the ccw set follows
  int64_t sig_off = 0;            // chunk signal words (CCE_FLAG_FINE_GRAINED) follow both sets
  int64_t sig_tiles = 0;          // chunks per output: (64 x 64)-tiles of a shard
  int64_t sig_words = 0;          // 2 per chunk, n outputs
  int64_t total = 0;              // enough for every flag combination
};

cce_status rs_geometry(int n, int mode, cce_dtype acc_t, const cce_mat& out, RsGeom& g,
                       bool one_chain = false) {
  if (n < 1 || n > CCE_MAX_RANKS)
    return fail(n < 1 ? CCE_EINVAL : CCE_EUNSUPPORTED, "n_ranks out of range: " + std::to_string(n));
  if (mode != CCE_RS_SLICE_LHS_ROWS && mode != CCE_RS_SLICE_RHS_COLS)
    return fail(CCE_EINVAL, "bad ReduceScatter mode");
  if (!dtype_ok(acc_t)) return fail(CCE_EINVAL, "bad acc dtype");
  if (acc_t != CCE_F32) return fail(CCE_EUNSUPPORTED, "the travelling accumulator is fp32 only");
  CCE_TRY(check_mat("out_shard", out));
  g.n = n;
  g.mode = mode;
  const bool rows = (mode == CCE_RS_SLICE_LHS_ROWS);
  g.shard = rows ? out.rows : out.cols;
  g.other = rows ? out.cols : out.rows;
  // The split of a shard into two chains: rows split at ceil(m/2); columns
  // split at a multiple of 8 so that the second half stays 16-byte aligned.
  auto split = [&](int64_t* h0, int64_t* h1) {
    if (rows) {
      *h0 = (g.shard + 1) / 2;
    } else {
      *h0 = round8((g.shard + 1) / 2);
      if (*h0 >= g.shard) *h0 = g.shard;
    }
    *h1 = g.shard - *h0;
  };
  auto layout = [&](int64_t h0, int64_t* ld, int64_t* slot) {
    *ld = rows ? round8(g.other) : round8(h0);
    *slot = rows ? align256(h0 * *ld * 4) : align256(g.other * *ld * 4);
  };
  // Two chains of half shards (copies beside the GEMMs), or one chain of
  // whole shards (permute fused into the GEMM epilogue, or CCE_FLAG_ONE_CHAIN).
  int64_t s0, s1, ld2, slot2, ld1, slot1;
  split(&s0, &s1);
  layout(s0, &ld2, &slot2);
  layout(g.shard, &ld1, &slot1);
  const int64_t total2 = 2LL * n * 2 * slot2, total1 = 2LL * n * slot1;
  g.region = std::max(total1, total2);
  // The bidirectional form needs a second (counter-clockwise) set; with one
  // rank there are no accumulators at all.
  g.total = (n > 1) ? 2 * g.region : 0;
  // Two words per output chunk for the fine-grained overlap, counted for the
  // smallest GEMM tile (64 x 64, the fp32 kernel's), whatever tile the
  // launch takes.
  g.sig_off = g.total;
  g.sig_tiles = ((g.shard + 63) / 64) * ((g.other + 63) / 64);
  g.sig_words = (n > 1) ? 2LL * n * g.sig_tiles : 0;
  g.total += align256(4 * g.sig_words);
  if (one_chain) {
    g.h0 = g.shard;
    g.h1 = 0;
    g.H = 1;
    g.acc_ld = ld1;
    g.half_bytes = slot1;
  } else {
    g.h0 = s0;
    g.h1 = s1;
    g.H = 2;
    g.acc_ld = ld2;
    g.half_bytes = slot2;
  }
  return CCE_OK;
}

}  // namespace

void set_error(const std::string& msg) { g_err = msg; }
void clear_error() { g_err.clear(); }
cce_status fail(cce_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// ---------------------------------------------------------------------------
// Executors
// ---------------------------------------------------------------------------
namespace {

hipMemcpyKind copy_kind(uint32_t flags) {
  return (flags & CCE_FLAG_COPY_DMA) ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
}

// Copies of the overlapped form run as the library's permute kernel, which
// shares compute units with the GEMM beside it; the DMA form keeps the DMA
// engines, and the serial form (the unoverlapped comparison) the runtime's
// full-device copy.
// The copy kernel moves device-to-device permutes, except in the serial form
// (CCE_FLAG_SERIAL), which keeps the runtime's own copies as the baseline the
// overlapped forms are measured against.  A fused plan's few copies (the
// two-way AllGather's prologue) take the kernel too.
bool use_permute_kernel(hipMemcpyKind kind, const Plan& plan) {
  return kind == hipMemcpyDeviceToDevice && (!plan.serial || plan.fused);
}

// Plan positions of the first and last GEMM op: a copy before the first or
// after the last has no GEMM beside it.
struct GemmSpan {
  size_t first = SIZE_MAX, last = 0;
  bool alone(const Plan& plan, const Op& o) const {
    const size_t j = static_cast<size_t>(&o - plan.ops.data());
    return first == SIZE_MAX || j < first || j > last;
  }
};
GemmSpan gemm_span(const Plan& plan) {
  GemmSpan g;
  for (size_t j = 0; j < plan.ops.size(); ++j)
    if (plan.ops[j].kind == OP_GEMM) {
      g.first = std::min(g.first, j);
      g.last = j;
    }
  return g;
}

hipStream_t stream_of(const Op& o, hipStream_t compute, hipStream_t copy, bool serial) {
  return (serial || o.stream == S_COMPUTE) ? compute : copy;
}

cce_status run_events(cce_ctx* ctx, const Op& o, hipStream_t s) {
  if (o.kind == OP_RECORD) HIP_TRY(hipEventRecord(ctx->events[o.event], s));
  if (o.kind == OP_WAIT) HIP_TRY(hipStreamWaitEvent(s, ctx->events[o.event], 0));
  return CCE_OK;
}

struct AgCall {
  AgGeom g;
  cce_dtype in_t, out_t;
  const void* const* looped;
  cce_mat lshape;
  const void* const* local;
  cce_mat local_shape;
  void* const* out;
  cce_mat oshape;
  char* ws;
  bool gelu;
  hipMemcpyKind copy_kind;
};

// pointer + leading dimension of a symbolic buffer
struct PtrLd {
  char* p;
  int64_t ld;
};

PtrLd ag_resolve(const AgCall& c, const BufRef& b) {
  const int r = b.rank;
  switch (b.kind) {
    case B_LOOPED: return {const_cast<char*>(static_cast<const char*>(c.looped[r])), c.lshape.ld};
    case B_LOCAL: return {const_cast<char*>(static_cast<const char*>(c.local[r])), c.local_shape.ld};
    case B_OUT: return {static_cast<char*>(c.out[r]), c.oshape.ld};
    case B_RECV:
      return {c.ws + (static_cast<int64_t>(b.parity) * c.g.n + r) * c.g.recv_bytes, c.lshape.ld};
    case B_CASE2:
      return {c.ws + 2LL * c.g.n * c.g.recv_bytes + r * c.g.acc_bytes, c.g.acc_ld};
    case B_RECV_CCW:
      return {c.ws + c.g.ccw_off + (static_cast<int64_t>(b.parity) * c.g.n + r) * c.g.recv_bytes,
              c.lshape.ld};
  }
  return {nullptr, 0};
}

// A plan that fails part-way may leave work on the copy stream that the
// caller's stream would no longer wait for.  Join the copy stream back
// (best effort: the first error is the one reported), so that the caller's
// later work, freeing the workspace included, stays ordered after it.
cce_status joined(cce_ctx* ctx, hipStream_t compute, cce_status st) {
  if (st == CCE_OK || ctx->events.empty()) return st;
  const std::string err = g_err;
  if (hipEventRecord(ctx->events[0], ctx->copy) == hipSuccess)
    (void)hipStreamWaitEvent(compute, ctx->events[0], 0);
  g_err = err;
  return st;
}

cce_status ag_execute(cce_ctx* ctx, const AgCall& c, const Plan& plan, hipStream_t compute) {
  const size_t ein = esize(c.in_t);
  g_ops_seen = 0;
  const GemmSpan gs = gemm_span(plan);
  for (const Op& o : plan.ops) {
    if (fail_due()) return fail(CCE_EHIP, "injected failure at plan op " + std::to_string(g_ops_seen));
    hipStream_t s = stream_of(o, compute, ctx->copy, plan.serial);
    if (o.kind == OP_RECORD || o.kind == OP_WAIT) {
      CCE_TRY(run_events(ctx, o, s));
      continue;
    }
    if (o.kind == OP_COPY) {
      const int64_t w = c.lshape.cols * static_cast<int64_t>(ein);
      int slot;
      CCE_TRY(prof_begin(ctx, s, 1, o.iter, 0.0,
                         2.0 * static_cast<double>(w) * c.lshape.rows * o.items.size(), &slot));
      // The shard's exact span (contiguous when both sides share the ld): no
      // read of the caller's memory past its last row.
      std::vector<PermuteItem> pitems;
      bool kernel_ok = use_permute_kernel(c.copy_kind, plan);
      for (const Item& it : o.items) {
        const PtrLd src = ag_resolve(c, it.a), dst = ag_resolve(c, it.c);
        if (c.lshape.rows == 0 || w == 0) continue;
        PermuteItem pi;
        pi.src = src.p;
        pi.dst = dst.p;
        if (src.ld == dst.ld) {
          pi.rows = 1;
          pi.width = ((c.lshape.rows - 1) * src.ld + c.lshape.cols) * ein;
        } else {
          pi.rows = c.lshape.rows;
          pi.width = w;
          pi.src_pitch = src.ld * ein;
          pi.dst_pitch = dst.ld * ein;
        }
        kernel_ok = kernel_ok && permute_item_ok(pi);
        pitems.push_back(pi);
      }
      if (kernel_ok) {
        CCE_TRY(launch_permute_copy(pitems.data(), static_cast<int>(pitems.size()), s,
                                    gs.alone(plan, o)));
      } else {
        for (const PermuteItem& pi : pitems) {
          if (pi.rows == 1)
            HIP_TRY(hipMemcpyAsync(pi.dst, pi.src, pi.width, c.copy_kind, s));
          else
            HIP_TRY(hipMemcpy2DAsync(pi.dst, pi.dst_pitch, pi.src, pi.src_pitch, pi.width, pi.rows,
                                     c.copy_kind, s));
        }
      }
      CCE_TRY(prof_end(ctx, s, slot));
      continue;
    }
    // GEMM
    GemmLaunch L;
    // one group per item (rank, direction); case 3: one per batch element
    const int per = (c.g.mode == CCE_AG_LHS_BATCH) ? static_cast<int>(c.g.bs) : 1;
    L.groups = static_cast<int>(o.items.size()) * per;
    L.M = c.g.M;
    L.N = c.g.N;
    L.K = c.g.K;
    L.in_t = c.in_t;
    L.epi = o.epi;
    const bool last = (o.iter == plan.n - 1);
    L.gelu = c.gelu && (!c.g.case2 || last);
    int gi = 0;
    for (const Item& it : o.items) {
      const int64_t s_id = it.shard;
      const PtrLd held = ag_resolve(c, it.a);
      const PtrLd loc = ag_resolve(c, it.b);
      const PtrLd dst = ag_resolve(c, it.c);
      L.out_t = (it.c.kind == B_OUT) ? c.out_t : CCE_F32;
      L.ldc = dst.ld;
      const int64_t eo = esize(L.out_t);
      const PtrLd f = it.has_fwd ? ag_resolve(c, it.fwd) : PtrLd{nullptr, 0};
      for (int e = 0; e < per; ++e) {
        const int r = gi++;
        char* cptr = dst.p;
        switch (c.g.mode) {
          case CCE_AG_LHS_ROWS:
            L.p.a[r] = held.p; L.lda = held.ld;
            L.p.b[r] = loc.p; L.ldb = loc.ld;
            cptr += s_id * c.g.M * dst.ld * eo;
            break;
          case CCE_AG_RHS_COLS:
            L.p.a[r] = loc.p; L.lda = loc.ld;
            L.p.b[r] = held.p; L.ldb = held.ld;
            cptr += s_id * c.g.N * eo;
            break;
          case CCE_AG_LHS_COLS:
            L.p.a[r] = held.p; L.lda = held.ld;
            L.p.b[r] = loc.p + s_id * c.g.K * ein; L.ldb = loc.ld;
            break;
          case CCE_AG_RHS_ROWS:
            L.p.a[r] = loc.p + s_id * c.g.K * ein; L.lda = loc.ld;
            L.p.b[r] = held.p; L.ldb = held.ld;
            break;
          case CCE_AG_LHS_BATCH: {
            // element e of shard s: its rows of the held shard, the local
            // operand's element s*b_s + e, the output's element s*b_s + e
            const int64_t j = s_id * per + e;
            L.p.a[r] = held.p + e * c.g.M * held.ld * ein; L.lda = held.ld;
            L.p.b[r] = loc.p + j * c.g.N * loc.ld * ein; L.ldb = loc.ld;
            cptr += j * c.g.M * dst.ld * eo;
            break;
          }
        }
        L.p.c[r] = cptr;
        if (it.has_fwd) {
          L.fwd = (c.g.mode == CCE_AG_LHS_ROWS || c.g.mode == CCE_AG_LHS_COLS ||
                   c.g.mode == CCE_AG_LHS_BATCH)
                      ? FWD_A
                      : FWD_B;
          // case 3: element e of the shard lands at its rows of the next buffer
          L.p.fwd[r] = f.p + (c.g.mode == CCE_AG_LHS_BATCH ? e * c.g.M * f.ld * ein : 0);
          L.ldfwd = f.ld;
        } else {
          L.p.fwd[r] = nullptr;
        }
        if (it.has_cin) {
          const PtrLd cin = ag_resolve(c, it.cin);
          L.p.cin[r] = reinterpret_cast<const float*>(cin.p);
          L.ldcin = cin.ld;
        } else {
          L.p.cin[r] = nullptr;
        }
      }
    }
    int slot;
    CCE_TRY(prof_begin(ctx, compute, 0, o.iter, 2.0 * L.M * L.N * L.K * L.groups, 0.0, &slot));
    CCE_TRY(launch_grouped_gemm(L, compute));
    CCE_TRY(prof_end(ctx, compute, slot));
  }
  return CCE_OK;
}

// The fused reduce epilogue applied to a ReduceScatter's fp32 result
// (cce_looped_einsum_reducescatter_epilogue).
struct RsEpi {
  const void* bias = nullptr;
  const void* const* res = nullptr;   // [n] or NULL
  int64_t ld_res = 0;
  bool dropout = false, drop_all = false;
  uint32_t threshold = 0;
  float scale = 1.0f;
  uint64_t seed = 0, offset = 0;
  const int64_t* mrow0 = nullptr;     // [n]
  int64_t mcol0 = 0, mld = 0;
};

struct RsCall {
  RsGeom g;
  cce_dtype in_t, out_t;
  const void* const* a;
  cce_mat ashape;
  const void* const* b;
  cce_mat bshape;
  void* const* out;
  cce_mat oshape;
  char* ws;
  hipMemcpyKind copy_kind;
  const RsEpi* epi = nullptr;
  unsigned* err = nullptr;        // the context's give-up counter (fine-grained overlap)
};

PtrLd rs_resolve(const RsCall& c, const BufRef& b) {
  const int r = b.rank;
  switch (b.kind) {
    case B_A: return {const_cast<char*>(static_cast<const char*>(c.a[r])), c.ashape.ld};
    case B_B: return {const_cast<char*>(static_cast<const char*>(c.b[r])), c.bshape.ld};
    case B_OUT: {
      const int64_t eo = esize(c.out_t);
      char* p = static_cast<char*>(c.out[r]);
      if (b.half == 1)
        p += (c.g.mode == CCE_RS_SLICE_LHS_ROWS) ? c.g.h0 * c.oshape.ld * eo : c.g.h0 * eo;
      return {p, c.oshape.ld};
    }
    case B_ACC:
      return {c.ws + ((static_cast<int64_t>(b.parity) * c.g.n + r) * c.g.H + b.half) * c.g.half_bytes,
              c.g.acc_ld};
    case B_ACC_CCW:
      return {c.ws + c.g.region +
                  ((static_cast<int64_t>(b.parity) * c.g.n + r) * c.g.H + b.half) * c.g.half_bytes,
              c.g.acc_ld};
  }
  return {nullptr, 0};
}

// One batched launch of the fused epilogue over every rank's half h of the
// output: src[r] holds rank r's fp32 partial(s) (one in the one-way form, the
// cw and ccw accumulators in the two-way form), which are summed first.
cce_status rs_epilogue(cce_ctx* ctx, const RsCall& c, int h, int n_part,
                       const std::vector<std::array<PtrLd, 2>>& src, hipStream_t s) {
  const RsEpi& x = *c.epi;
  const bool rows_mode = (c.g.mode == CCE_RS_SLICE_LHS_ROWS);
  const int64_t ext = (h == 0) ? c.g.h0 : c.g.h1;
  const int64_t base = h * c.g.h0;            // first row (or column) of the half
  const size_t eo = esize(c.out_t);
  EpilogueLaunch E;
  E.n = n_part;
  E.batch = c.g.n;
  E.part_t = CCE_F32;
  E.rows = rows_mode ? ext : c.g.other;
  E.cols = rows_mode ? c.g.other : ext;
  if (E.rows == 0 || E.cols == 0) return CCE_OK;
  E.ld_part = c.g.acc_ld;
  E.bias = x.bias ? static_cast<const char*>(x.bias) + (rows_mode ? 0 : base * eo) : nullptr;
  E.bias_t = c.out_t;
  E.res_t = c.out_t;
  E.ld_res = x.ld_res;
  E.out_t = c.out_t;
  E.ld_out = c.oshape.ld;
  E.threshold = x.threshold;
  E.drop_all = x.drop_all;
  E.dropout = x.dropout;
  E.scale = x.scale;
  E.seed = x.seed;
  E.offset = x.offset;
  E.mcol0 = x.mcol0 + (rows_mode ? 0 : base);
  E.mld = x.mld;
  for (int r = 0; r < c.g.n; ++r) {
    for (int k = 0; k < n_part; ++k) E.parts[r * n_part + k] = src[r][k].p;
    E.res[r] = x.res ? static_cast<const char*>(x.res[r]) +
                           (rows_mode ? base * x.ld_res * static_cast<int64_t>(eo) : base * eo)
                     : nullptr;
    E.out[r] = rs_resolve(c, BufRef{B_OUT, 0, static_cast<uint8_t>(h), static_cast<int16_t>(r)}).p;
    E.mask[r] = nullptr;
    E.mrow0[r] = x.mrow0[r] + (rows_mode ? base : 0);
  }
  const double bytes = static_cast<double>(E.batch) * E.rows * E.cols *
                           (4.0 * n_part + (x.res ? eo : 0) + eo) +
                       (x.bias ? static_cast<double>(E.cols) * eo : 0.0);
  int slot;
  CCE_TRY(prof_begin(ctx, s, 2, -1, 0.0, bytes, &slot));
  CCE_TRY(launch_fused_epilogue(E, s));
  return prof_end(ctx, s, slot);
}

// The chunk consumer's arguments of an EPI_FINAL launch of half h (fine-
// grained overlap): the per-launch part; the per-output part is filled item
// by item (rs_final_item).  Without the fused epilogue the consumer is the
// align-and-sum of the two ring directions: no bias, mask or residual.
void rs_final_launch(const RsCall& c, int h, FinalArgs& f) {
  const bool rows_mode = (c.g.mode == CCE_RS_SLICE_LHS_ROWS);
  const int64_t base = h * c.g.h0;   // first row (or column) of the half
  const size_t eo = esize(c.out_t);
  f.ld_out = c.oshape.ld;
  f.sig = reinterpret_cast<unsigned*>(c.ws + c.g.sig_off);
  f.sig_tiles = c.g.sig_tiles;
  f.err = c.err;
  f.cap = kSignalPollCap;
  f.nopub = 0;
  if (g_giveup_polls > 0) {
    f.cap = static_cast<unsigned>(g_giveup_polls);
    f.nopub = 1;
  }
  if (!c.epi) return;
  const RsEpi& x = *c.epi;
  f.bias = x.bias ? static_cast<const char*>(x.bias) + (rows_mode ? 0 : base * eo) : nullptr;
  f.ld_res = x.ld_res;
  f.mode = x.drop_all ? 2 : (x.dropout ? 1 : 0);
  f.threshold = x.threshold;
  f.scale = x.scale;
  f.key0 = static_cast<uint32_t>(x.seed);
  f.key1 = static_cast<uint32_t>(x.seed >> 32);
  f.off0 = static_cast<uint32_t>(x.offset);
  f.off1 = static_cast<uint32_t>(x.offset >> 32);
  f.mcol0 = x.mcol0 + (rows_mode ? 0 : base);
  f.mld = x.mld;
  f.aligned = (f.mld % 4 == 0) && (f.mcol0 % 4 == 0);
}

void rs_final_item(const RsCall& c, int h, const Item& it, FinalArgs& f) {
  const bool rows_mode = (c.g.mode == CCE_RS_SLICE_LHS_ROWS);
  const int64_t base = h * c.g.h0;
  const size_t eo = esize(c.out_t);
  const int s = it.c.rank;
  f.out[s] = rs_resolve(c, it.c).p;
  f.other[s] = (it.has_other && it.pair < 0) ? reinterpret_cast<const float*>(rs_resolve(c, it.other).p)
                                             : nullptr;
  f.res[s] = nullptr;
  f.mrow0[s] = 0;
  if (!c.epi) return;
  const RsEpi& x = *c.epi;
  f.res[s] = x.res ? static_cast<const char*>(x.res[s]) +
                         (rows_mode ? base * x.ld_res * static_cast<int64_t>(eo) : base * eo)
                   : nullptr;
  f.mrow0[s] = x.mrow0[s] + (rows_mode ? base : 0);
}

cce_status rs_execute(cce_ctx* ctx, const RsCall& c, const Plan& plan, hipStream_t compute) {
  const size_t ein = esize(c.in_t);
  const bool rows_mode = (c.g.mode == CCE_RS_SLICE_LHS_ROWS);
  // one-way form with the fused epilogue: where each rank's result half ends
  std::vector<std::array<PtrLd, 2>> final_acc[2] = {std::vector<std::array<PtrLd, 2>>(c.g.n),
                                                    std::vector<std::array<PtrLd, 2>>(c.g.n)};
  bool has_final[2] = {false, false};
  g_ops_seen = 0;
  // Fine-grained overlap: the chunk signal words start at zero (a kernel,
  // not a memset: the call may be captured in a graph).
  bool fine = false;
  for (const Op& o : plan.ops) fine = fine || (o.kind == OP_GEMM && o.epi == EPI_FINAL);
  if (fine)
    CCE_TRY(launch_zero_words(reinterpret_cast<unsigned*>(c.ws + c.g.sig_off), c.g.sig_words,
                              compute));
  const GemmSpan gs = gemm_span(plan);
  for (const Op& o : plan.ops) {
    if (fail_due()) return fail(CCE_EHIP, "injected failure at plan op " + std::to_string(g_ops_seen));
    hipStream_t s = stream_of(o, compute, ctx->copy, plan.serial);
    if (o.kind == OP_RECORD || o.kind == OP_WAIT) {
      CCE_TRY(run_events(ctx, o, s));
      continue;
    }
    const int64_t ext = (o.half == 0) ? c.g.h0 : c.g.h1;   // extent along the sliced dim
    if (o.kind == OP_SUM && c.epi) {
      // Two-way form with the fused epilogue: the cw and ccw accumulators go
      // straight into it and are summed before the bias (never stored).
      std::vector<std::array<PtrLd, 2>> src(c.g.n);
      for (const Item& it : o.items) src[it.c.rank] = {rs_resolve(c, it.a), rs_resolve(c, it.cin)};
      CCE_TRY(rs_epilogue(ctx, c, o.half, 2, src, compute));
      continue;
    }
    if (o.kind == OP_SUM) {
      // Align-and-sum of the bidirectional form: out = cw + ccw, one batched
      // epilogue launch (two fp32 partials per rank, no bias, no dropout).
      EpilogueLaunch E;
      E.n = 2;
      E.batch = static_cast<int>(o.items.size());
      E.part_t = CCE_F32;
      E.rows = rows_mode ? ext : c.g.other;
      E.cols = rows_mode ? c.g.other : ext;
      E.ld_part = c.g.acc_ld;
      E.out_t = c.out_t;
      E.ld_out = c.oshape.ld;
      E.mcol0 = 0;
      E.mld = E.cols;
      int b = 0;
      for (const Item& it : o.items) {
        E.parts[2 * b] = rs_resolve(c, it.a).p;
        E.parts[2 * b + 1] = rs_resolve(c, it.cin).p;
        E.res[b] = nullptr;
        E.out[b] = rs_resolve(c, it.c).p;
        E.mask[b] = nullptr;
        E.mrow0[b] = 0;
        ++b;
      }
      if (E.rows == 0 || E.cols == 0) continue;
      int slot;
      CCE_TRY(prof_begin(ctx, compute, 3, o.iter, 0.0,
                         static_cast<double>(E.rows) * E.cols * (8.0 + esize(c.out_t)) * E.batch,
                         &slot));
      CCE_TRY(launch_fused_epilogue(E, compute));
      CCE_TRY(prof_end(ctx, compute, slot));
      continue;
    }
    if (o.kind == OP_COPY) {
      const int64_t bytes = (rows_mode ? ext * c.g.acc_ld : c.g.other * c.g.acc_ld) * 4;
      if (bytes == 0) continue;
      int slot;
      CCE_TRY(prof_begin(ctx, s, 1, o.iter, 0.0, 2.0 * bytes * o.items.size(), &slot));
      std::vector<PermuteItem> pitems;
      bool kernel_ok = use_permute_kernel(c.copy_kind, plan);
      for (const Item& it : o.items) {
        const PtrLd src = rs_resolve(c, it.a), dst = rs_resolve(c, it.c);
        PermuteItem pi;
        pi.src = src.p;
        pi.dst = dst.p;
        pi.rows = 1;
        pi.width = bytes;
        kernel_ok = kernel_ok && permute_item_ok(pi);
        pitems.push_back(pi);
      }
      if (kernel_ok) {
        CCE_TRY(launch_permute_copy(pitems.data(), static_cast<int>(pitems.size()), s,
                                    gs.alone(plan, o)));
      } else {
        for (const PermuteItem& pi : pitems)
          HIP_TRY(hipMemcpyAsync(pi.dst, pi.src, pi.width, c.copy_kind, s));
      }
      CCE_TRY(prof_end(ctx, s, slot));
      continue;
    }
    GemmLaunch L;
    L.groups = static_cast<int>(o.items.size());   // one group per item (rank, direction)
    L.K = c.g.K;
    L.in_t = c.in_t;
    L.epi = o.epi;
    L.gelu = false;
    if (rows_mode) {
      L.M = ext;
      L.N = c.g.other;
    } else {
      L.M = c.g.other;
      L.N = ext;
    }
    const bool final_op = (o.epi == EPI_FINAL);
    if (final_op) rs_final_launch(c, o.half, L.fin);
    int gi = 0;
    for (const Item& it : o.items) {
      const int r = gi++;
      const int64_t t = it.shard;
      const PtrLd A = rs_resolve(c, it.a), B = rs_resolve(c, it.b);
      PtrLd D = rs_resolve(c, it.c);
      L.out_t = (it.c.kind == B_OUT) ? c.out_t : CCE_F32;
      if (final_op) {
        // The chunk consumer writes the output; a paired item stores its
        // partial at its own accumulator when it claims a chunk first.
        rs_final_item(c, o.half, it, L.fin);
        L.fin.oid[r] = static_cast<int8_t>(it.c.rank);
        L.fin.partner[r] = static_cast<int8_t>(it.pair);
        D = it.pair >= 0 ? rs_resolve(c, it.meet) : PtrLd{nullptr, c.g.acc_ld};
        D.ld = c.g.acc_ld;
      } else if (c.epi && it.c.kind == B_OUT) {
        // One-way form with the fused epilogue: the last partial accumulates
        // in place into the received accumulator (every element is read
        // before it is written, by the same lane), which the epilogue reads.
        D = rs_resolve(c, it.cin);
        L.out_t = CCE_F32;
        final_acc[o.half][it.c.rank] = {D, D};
        has_final[o.half] = true;
      }
      const int64_t off = t * c.g.shard + o.half * c.g.h0;     // start along the sliced dim
      if (rows_mode) {
        L.p.a[r] = A.p + off * A.ld * ein;
        L.p.b[r] = B.p;
      } else {
        L.p.a[r] = A.p;
        L.p.b[r] = B.p + off * B.ld * ein;
      }
      L.lda = A.ld;
      L.ldb = B.ld;
      L.p.c[r] = D.p;
      L.ldc = D.ld;
      if (it.has_cin) {
        const PtrLd cin = rs_resolve(c, it.cin);
        L.p.cin[r] = reinterpret_cast<const float*>(cin.p);
        L.ldcin = cin.ld;
      } else {
        L.p.cin[r] = nullptr;
      }
    }
    if (L.M > 0 && L.N > 0) {
      int slot;
      CCE_TRY(prof_begin(ctx, compute, 0, o.iter, 2.0 * L.M * L.N * L.K * L.groups, 0.0, &slot));
      CCE_TRY(launch_grouped_gemm(L, compute));
      CCE_TRY(prof_end(ctx, compute, slot));
    }
  }
  for (int h = 0; h < 2; ++h)
    if (has_final[h]) CCE_TRY(rs_epilogue(ctx, c, h, 1, final_acc[h], compute));
  return CCE_OK;
}

}  // namespace
}  // namespace cce

using namespace cce;

extern "C" {

const char* cce_status_string(cce_status s) {
  switch (s) {
    case CCE_OK: return "CCE_OK";
    case CCE_EINVAL: return "CCE_EINVAL: invalid argument";
    case CCE_EUNSUPPORTED: return "CCE_EUNSUPPORTED: unsupported argument";
    case CCE_EWORKSPACE: return "CCE_EWORKSPACE: workspace missing or too small";
    case CCE_EHIP: return "CCE_EHIP: HIP runtime error";
  }
  return "unknown cce_status";
}

const char* cce_last_error(void) { return g_err.c_str(); }

const char* cce_version(void) { return "0.1.0"; }

cce_status cce_debug_fail_op(int index) {
  if (index < 0) return fail(CCE_EINVAL, "cce_debug_fail_op: index must be >= 0");
  g_fail_at = index;
  g_ops_seen = 0;
  return CCE_OK;
}

cce_status cce_ctx_create(int device, cce_ctx** out) {
  clear_error();
  if (!out) return fail(CCE_EINVAL, "out is NULL");
  *out = nullptr;
  int count = 0;
  HIP_TRY(hipGetDeviceCount(&count));
  if (device < 0 || device >= count) return fail(CCE_EINVAL, "bad device " + std::to_string(device));
  DeviceGuard guard(device);
  scratch_setup(device);
  cce_ctx* c = new cce_ctx();
  c->device = device;
  hipError_t e = hipStreamCreateWithFlags(&c->own_copy, hipStreamNonBlocking);
  if (e != hipSuccess) {
    delete c;
    return fail(CCE_EHIP, std::string("hipStreamCreateWithFlags: ") + hipGetErrorString(e));
  }
  c->copy = c->own_copy;
  // The fine-grained overlap's give-up counter (cce_ctx_check_signals).
  e = hipMalloc(reinterpret_cast<void**>(&c->err), 256);
  if (e == hipSuccess) e = hipMemset(c->err, 0, 256);
  if (e != hipSuccess) {
    if (c->err) hipFree(c->err);
    hipStreamDestroy(c->own_copy);
    delete c;
    return fail(CCE_EHIP, std::string("context error word: ") + hipGetErrorString(e));
  }
  *out = c;
  return CCE_OK;
}

cce_status cce_ctx_set_copy_stream(cce_ctx* ctx, cce_stream copy) {
  clear_error();
  if (!ctx) return fail(CCE_EINVAL, "ctx is NULL");
  ctx->copy = copy ? static_cast<hipStream_t>(copy) : ctx->own_copy;
  return CCE_OK;
}

cce_status cce_ctx_check_signals(cce_ctx* ctx, cce_stream stream) {
  clear_error();
  if (!ctx) return fail(CCE_EINVAL, "ctx is NULL");
  DeviceGuard guard(ctx->device);
  HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  unsigned v = 0;
  HIP_TRY(hipMemcpy(&v, ctx->err, sizeof v, hipMemcpyDeviceToHost));
  if (v == 0) return CCE_OK;
  HIP_TRY(hipMemset(ctx->err, 0, sizeof v));
  return fail(CCE_EHIP, std::to_string(v) + " chunk consumer(s) gave up waiting for the other "
                                            "producer's partial; their output chunks were not written");
}

cce_status cce_debug_signal_giveup(int polls) {
  if (polls < 0) return fail(CCE_EINVAL, "cce_debug_signal_giveup: polls must be >= 0");
  g_giveup_polls = polls;
  return CCE_OK;
}

cce_status cce_ctx_destroy(cce_ctx* ctx) {
  clear_error();
  if (!ctx) return CCE_OK;
  DeviceGuard guard(ctx->device);
  hipStreamSynchronize(ctx->own_copy);
  for (hipEvent_t e : ctx->events) hipEventDestroy(e);
  for (hipEvent_t e : ctx->timing_pool) hipEventDestroy(e);
  hipStreamDestroy(ctx->own_copy);
  if (ctx->err) hipFree(ctx->err);
  delete ctx;
  return CCE_OK;
}

cce_status cce_ctx_set_profiling(cce_ctx* ctx, int enable) {
  clear_error();
  if (!ctx) return fail(CCE_EINVAL, "ctx is NULL");
  ctx->profiling = enable != 0;
  if (enable) {
    ctx->prof.clear();
    ctx->timing_used = 0;
  }
  return CCE_OK;
}

cce_status cce_ctx_read_profile(cce_ctx* ctx, int max_records, cce_prof_record* out, int* n_out) {
  clear_error();
  if (!ctx || !n_out || (max_records > 0 && !out)) return fail(CCE_EINVAL, "NULL argument");
  DeviceGuard guard(ctx->device);
  int n = 0;
  for (const cce_prof_slot& p : ctx->prof) {
    if (n >= max_records) break;
    HIP_TRY(hipEventSynchronize(p.stop));
    float ms = 0.0f;
    HIP_TRY(hipEventElapsedTime(&ms, p.start, p.stop));
    out[n].kind = p.kind;
    out[n].iter = p.iter;
    out[n].ms = ms;
    out[n].flops = p.flops;
    out[n].bytes = p.bytes;
    ++n;
  }
  *n_out = n;
  ctx->prof.clear();
  ctx->timing_used = 0;
  return CCE_OK;
}

cce_status cce_shard_schedule(int n_ranks, int kind, int32_t* table) {
  clear_error();
  if (n_ranks < 1 || n_ranks > CCE_MAX_RANKS) return fail(CCE_EINVAL, "n_ranks out of range");
  if (kind < 0 || kind > 3) return fail(CCE_EINVAL, "kind must be 0, 1, 2 or 3");
  if (!table) return fail(CCE_EINVAL, "table is NULL");
  if ((kind == 2 || kind == 3) && 2 * n_ranks > CCE_MAX_RANKS)
    return fail(CCE_EUNSUPPORTED, "the bidirectional form takes at most CCE_MAX_RANKS / 2 ranks");
  // The schedule the plans use: read it back from the built plan itself.
  Plan p;
  switch (kind) {
    case 0: p = build_allgather_plan(n_ranks, CCE_AG_LHS_ROWS, false, true); break;
    case 1: p = build_reducescatter_plan(n_ranks, CCE_RS_SLICE_LHS_ROWS, false, true); break;
    case 2: p = build_allgather_plan_bidir(n_ranks, CCE_AG_LHS_ROWS, true, false); break;
    default: p = build_reducescatter_plan_bidir(n_ranks, CCE_RS_SLICE_LHS_ROWS, false, true, false);
  }
  if (kind >= 2) {
    const int iters = bidir_cw_len(n_ranks);
    for (int k = 0; k < iters * n_ranks * 2; ++k) table[k] = -1;
  }
  for (const Op& o : p.ops) {
    if (o.kind != OP_GEMM) continue;
    if (kind < 2) {
      for (const Item& it : o.items) table[o.iter * n_ranks + it.rank] = it.shard;
    } else {
      // items: the n clockwise ones first, then (while it runs) the n
      // counter-clockwise ones
      for (size_t k = 0; k < o.items.size(); ++k) {
        const Item& it = o.items[k];
        const int d = k < static_cast<size_t>(n_ranks) ? 0 : 1;
        table[(o.iter * n_ranks + it.rank) * 2 + d] = it.shard;
      }
    }
  }
  return CCE_OK;
}

cce_status cce_looped_allgather_einsum_workspace(int n_ranks, cce_ag_mode mode, cce_dtype in_t,
                                                 cce_dtype out_t, cce_mat looped_shard,
                                                 cce_mat out_shape, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(CCE_EINVAL, "bytes is NULL");
  AgGeom g;
  CCE_TRY(ag_geometry(n_ranks, mode, in_t, out_t, looped_shard, nullptr, out_shape, g));
  *bytes = static_cast<size_t>(g.total);
  return CCE_OK;
}

cce_status cce_looped_allgather_einsum(cce_ctx* ctx, int n_ranks, cce_ag_mode mode, cce_dtype in_t,
                                       cce_dtype out_t, const void* const* looped,
                                       cce_mat looped_shard, const void* const* local,
                                       cce_mat local_shape, void* const* out, cce_mat out_shape,
                                       void* workspace, size_t workspace_bytes, uint32_t flags,
                                       cce_stream stream) {
  clear_error();
  if (!ctx) return fail(CCE_EINVAL, "ctx is NULL");
  if (flags & ~(CCE_FLAG_SERIAL | CCE_FLAG_GELU | CCE_FLAG_COPY_DMA | CCE_FLAG_FUSED_PERMUTE |
                CCE_FLAG_BIDIRECTIONAL | CCE_FLAG_ONE_CHAIN))
    return fail(CCE_EINVAL, "unknown flags");
  if (!looped || !local || !out) return fail(CCE_EINVAL, "pointer array is NULL");
  AgGeom g;
  CCE_TRY(ag_geometry(n_ranks, mode, in_t, out_t, looped_shard, &local_shape, out_shape, g));
  const bool bidir = (flags & CCE_FLAG_BIDIRECTIONAL) != 0;
  if (bidir && g.case2)
    return fail(CCE_EUNSUPPORTED, "the bidirectional form takes the case-1 modes only");
  if (bidir && 2 * n_ranks > CCE_MAX_RANKS)
    return fail(CCE_EUNSUPPORTED, "the bidirectional form takes at most CCE_MAX_RANKS / 2 ranks");
  if (static_cast<int64_t>(bidir ? 2 : 1) * n_ranks * g.bs > CCE_MAX_RANKS)
    return fail(CCE_EUNSUPPORTED, "case 3: n * b_s GEMM groups (2 * n * b_s two-way) exceed CCE_MAX_RANKS");
  const size_t ein = esize(in_t), eout = esize(out_t);
  const int64_t ls = span_bytes(looped_shard, ein), cs = span_bytes(local_shape, ein),
                os = span_bytes(out_shape, eout);
  if (ls > kMaxOperandBytes || cs > kMaxOperandBytes)
    return fail(CCE_EUNSUPPORTED, "a GEMM operand exceeds 1 GiB");
  std::vector<Range> ranges;
  for (int r = 0; r < n_ranks; ++r) {
    const std::string rs = std::to_string(r);
    CCE_TRY(check_ptr(("looped[" + rs + "]").c_str(), looped[r], ls));
    CCE_TRY(check_ptr(("local[" + rs + "]").c_str(), local[r], cs));
    CCE_TRY(check_ptr(("out[" + rs + "]").c_str(), out[r], os));
    ranges.push_back(range_of(looped[r], ls, "looped[" + rs + "]", false));
    ranges.push_back(range_of(local[r], cs, "local[" + rs + "]", false));
    ranges.push_back(range_of(out[r], os, "out[" + rs + "]", true));
  }
  if (g.total > 0) {
    if (!workspace || workspace_bytes < static_cast<size_t>(g.total))
      return fail(CCE_EWORKSPACE, "workspace needs " + std::to_string(g.total) + " bytes");
    CCE_TRY(check_ptr("workspace", workspace, g.total));
    ranges.push_back(range_of(workspace, g.total, "workspace", true));
  }
  CCE_TRY(check_overlaps(ranges));
  if (g.M == 0 || g.N == 0) return CCE_OK;

  DeviceGuard guard(ctx->device);
  const bool serial = (flags & CCE_FLAG_SERIAL) != 0;
  const bool fused = (flags & CCE_FLAG_FUSED_PERMUTE) != 0;
  const Plan plan = bidir ? build_allgather_plan_bidir(n_ranks, mode, serial, fused)
                          : build_allgather_plan(n_ranks, mode, g.case2_ws, serial, fused);
  CCE_TRY(ensure_events(ctx, std::max(plan.n_events, 1)));
  AgCall c{g, in_t, out_t, looped, looped_shard, local, local_shape, out, out_shape,
           static_cast<char*>(workspace), (flags & CCE_FLAG_GELU) != 0, copy_kind(flags)};
  return joined(ctx, static_cast<hipStream_t>(stream), ag_execute(ctx, c, plan, static_cast<hipStream_t>(stream)));
}

cce_status cce_looped_einsum_reducescatter_workspace(int n_ranks, cce_rs_mode mode, cce_dtype acc_t,
                                                     cce_mat out_shard, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(CCE_EINVAL, "bytes is NULL");
  RsGeom g;
  CCE_TRY(rs_geometry(n_ranks, mode, acc_t, out_shard, g));
  *bytes = static_cast<size_t>(g.total);
  return CCE_OK;
}

// The epilogue's arguments as the caller gives them.
struct RsEpiArgs {
  const void* bias;
  const void* const* res;
  int64_t ld_res;
  double p_drop;
  uint64_t seed, offset;
  const int64_t* mrow0;
  int64_t mcol0, mld;
};

static cce_status rs_impl(cce_ctx* ctx, int n_ranks, cce_rs_mode mode, cce_dtype in_t,
                          cce_dtype acc_t, cce_dtype out_t, const void* const* a,
                          cce_mat a_shape, const void* const* b, cce_mat b_shape,
                          void* const* out, cce_mat out_shard, void* workspace,
                          size_t workspace_bytes, uint32_t flags, cce_stream stream,
                          const RsEpiArgs* ea) {
  if (!ctx) return fail(CCE_EINVAL, "ctx is NULL");
  if (flags & ~(CCE_FLAG_SERIAL | CCE_FLAG_COPY_DMA | CCE_FLAG_FUSED_PERMUTE |
                CCE_FLAG_BIDIRECTIONAL | CCE_FLAG_FINE_GRAINED | CCE_FLAG_ONE_CHAIN))
    return fail(CCE_EINVAL, "unsupported flags for ReduceScatter");
  const bool fused = (flags & CCE_FLAG_FUSED_PERMUTE) != 0;
  const bool one_chain = fused || (flags & CCE_FLAG_ONE_CHAIN) != 0;
  const bool bidir = (flags & CCE_FLAG_BIDIRECTIONAL) != 0;
  const bool fine = (flags & CCE_FLAG_FINE_GRAINED) != 0;
  if (fine && bidir && !fused)
    return fail(CCE_EUNSUPPORTED, "CCE_FLAG_FINE_GRAINED with CCE_FLAG_BIDIRECTIONAL needs "
                                  "CCE_FLAG_FUSED_PERMUTE (with copies, the last partial of the "
                                  "counter-clockwise direction still travels after the loop)");
  if (bidir && 2 * n_ranks > CCE_MAX_RANKS)
    return fail(CCE_EUNSUPPORTED, "the bidirectional form takes at most CCE_MAX_RANKS / 2 ranks");
  if (!a || !b || !out) return fail(CCE_EINVAL, "pointer array is NULL");
  if (!dtype_ok(in_t) || !dtype_ok(out_t)) return fail(CCE_EINVAL, "bad dtype");
  RsGeom g;
  CCE_TRY(rs_geometry(n_ranks, mode, acc_t, out_shard, g, one_chain));
  // (the chunk consumers address a published partial by 32-bit offsets)
  if (fine && g.half_bytes > kMaxOperandBytes)
    return fail(CCE_EUNSUPPORTED, "CCE_FLAG_FINE_GRAINED: an accumulator exceeds 1 GiB");
  CCE_TRY(check_mat("a_shape", a_shape));
  CCE_TRY(check_mat("b_shape", b_shape));
  const int64_t nn = n_ranks;
  if (a_shape.cols != b_shape.cols) return fail(CCE_EINVAL, "a and b must share the contraction length");
  g.K = a_shape.cols;
  if (mode == CCE_RS_SLICE_LHS_ROWS) {
    if (a_shape.rows != nn * out_shard.rows) return fail(CCE_EINVAL, "a rows must be n * out rows");
    if (b_shape.rows != out_shard.cols) return fail(CCE_EINVAL, "b rows must equal out cols");
  } else {
    if (a_shape.rows != out_shard.rows) return fail(CCE_EINVAL, "a rows must equal out rows");
    if (b_shape.rows != nn * out_shard.cols) return fail(CCE_EINVAL, "b rows must be n * out cols");
  }
  if (g.K % 8 != 0) return fail(CCE_EUNSUPPORTED, "contraction length must be a multiple of 8");
  const size_t ein = esize(in_t), eout = esize(out_t);
  const int64_t as = span_bytes(a_shape, ein), bs = span_bytes(b_shape, ein),
                os = span_bytes(out_shard, eout);
  if (as > kMaxOperandBytes || bs > kMaxOperandBytes)
    return fail(CCE_EUNSUPPORTED, "a GEMM operand exceeds 1 GiB");
  RsEpi epi;
  if (ea) {
    // The epilogue reads the result from the workspace's accumulators.
    if (n_ranks < 2)
      return fail(CCE_EUNSUPPORTED, "the fused epilogue needs n_ranks >= 2 (with one rank, use "
                                    "cce_grouped_gemm and cce_fused_reduce_epilogue)");
    if (std::isnan(ea->p_drop)) return fail(CCE_EINVAL, "p_drop is NaN");
    if (!ea->mrow0) return fail(CCE_EINVAL, "mask_row0 is NULL");
    if (ea->mcol0 < 0 || ea->mld < ea->mcol0 + out_shard.cols)
      return fail(CCE_EINVAL, "mask index base must satisfy 0 <= col0, col0 + cols <= mask_ld");
    for (int r = 0; r < n_ranks; ++r)
      if (ea->mrow0[r] < 0) return fail(CCE_EINVAL, "mask row base must be >= 0");
    if (ea->res) CCE_TRY(check_mat("residual", cce_mat{out_shard.rows, out_shard.cols, ea->ld_res}));
    epi.bias = ea->bias;
    epi.res = ea->res;
    epi.ld_res = ea->ld_res;
    epi.seed = ea->seed;
    epi.offset = ea->offset;
    epi.mrow0 = ea->mrow0;
    epi.mcol0 = ea->mcol0;
    epi.mld = ea->mld;
    if (ea->p_drop >= 1.0) {
      epi.drop_all = true;
    } else if (ea->p_drop > 0.0) {
      epi.dropout = true;
      epi.threshold = static_cast<uint32_t>(std::floor(ea->p_drop * 4294967296.0));
      epi.scale = static_cast<float>(1.0 / (1.0 - ea->p_drop));
    }
  }
  std::vector<Range> ranges;
  for (int r = 0; r < n_ranks; ++r) {
    const std::string rs = std::to_string(r);
    CCE_TRY(check_ptr(("a[" + rs + "]").c_str(), a[r], as));
    CCE_TRY(check_ptr(("b[" + rs + "]").c_str(), b[r], bs));
    CCE_TRY(check_ptr(("out[" + rs + "]").c_str(), out[r], os));
    ranges.push_back(range_of(a[r], as, "a[" + rs + "]", false));
    ranges.push_back(range_of(b[r], bs, "b[" + rs + "]", false));
    ranges.push_back(range_of(out[r], os, "out[" + rs + "]", true));
    if (ea && ea->res) {
      const int64_t rsz = span_bytes(cce_mat{out_shard.rows, out_shard.cols, ea->ld_res}, eout);
      CCE_TRY(check_ptr(("residual[" + rs + "]").c_str(), ea->res[r], rsz));
      ranges.push_back(range_of(ea->res[r], rsz, "residual[" + rs + "]", false));
    }
  }
  if (ea && ea->bias) {
    const int64_t bsz = out_shard.cols * static_cast<int64_t>(eout);
    CCE_TRY(check_ptr("bias", ea->bias, bsz));
    ranges.push_back(range_of(ea->bias, bsz, "bias", false));
  }
  if (g.total > 0) {
    if (!workspace || workspace_bytes < static_cast<size_t>(g.total))
      return fail(CCE_EWORKSPACE, "workspace needs " + std::to_string(g.total) + " bytes");
    CCE_TRY(check_ptr("workspace", workspace, g.total));
    ranges.push_back(range_of(workspace, g.total, "workspace", true));
  }
  CCE_TRY(check_overlaps(ranges));
  if (out_shard.rows == 0 || out_shard.cols == 0) return CCE_OK;

  DeviceGuard guard(ctx->device);
  const bool serial = (flags & CCE_FLAG_SERIAL) != 0;
  Plan plan = bidir ? build_reducescatter_plan_bidir(n_ranks, mode, g.h1 > 0, serial, fused)
                    : build_reducescatter_plan(n_ranks, mode, g.h1 > 0, serial, fused);
  if (fine) make_fine_grained(plan, ea != nullptr);
  CCE_TRY(ensure_events(ctx, std::max(plan.n_events, 1)));
  RsCall c{g, in_t, out_t, a, a_shape, b, b_shape, out, out_shard, static_cast<char*>(workspace),
           copy_kind(flags)};
  c.epi = ea ? &epi : nullptr;
  c.err = ctx->err;
  const cce_status st =
      joined(ctx, static_cast<hipStream_t>(stream), rs_execute(ctx, c, plan, static_cast<hipStream_t>(stream)));
  if (fine) g_giveup_polls = 0;   // the test hook fires once
  return st;
}

cce_status cce_looped_einsum_reducescatter(cce_ctx* ctx, int n_ranks, cce_rs_mode mode,
                                           cce_dtype in_t, cce_dtype acc_t, cce_dtype out_t,
                                           const void* const* a, cce_mat a_shape,
                                           const void* const* b, cce_mat b_shape,
                                           void* const* out, cce_mat out_shard, void* workspace,
                                           size_t workspace_bytes, uint32_t flags,
                                           cce_stream stream) {
  clear_error();
  return rs_impl(ctx, n_ranks, mode, in_t, acc_t, out_t, a, a_shape, b, b_shape, out, out_shard,
                 workspace, workspace_bytes, flags, stream, nullptr);
}

cce_status cce_looped_einsum_reducescatter_epilogue(
    cce_ctx* ctx, int n_ranks, cce_rs_mode mode, cce_dtype in_t, cce_dtype out_t,
    const void* const* a, cce_mat a_shape, const void* const* b, cce_mat b_shape,
    const void* bias, const void* const* residuals, int64_t ld_res, double p_drop,
    uint64_t seed, uint64_t offset, const int64_t* mask_row0, int64_t mask_col0,
    int64_t mask_ld, void* const* out, cce_mat out_shard, void* workspace,
    size_t workspace_bytes, uint32_t flags, cce_stream stream) {
  clear_error();
  const RsEpiArgs ea{bias, residuals, ld_res, p_drop, seed, offset, mask_row0, mask_col0, mask_ld};
  return rs_impl(ctx, n_ranks, mode, in_t, CCE_F32, out_t, a, a_shape, b, b_shape, out, out_shard,
                 workspace, workspace_bytes, flags, stream, &ea);
}

cce_status cce_looped_einsum_reducescatter_epilogue_noalloc(
    cce_ctx* ctx, int n_ranks, cce_rs_mode mode, cce_dtype in_t, cce_dtype out_t,
    const void* const* a, cce_mat a_shape, const void* const* b, cce_mat b_shape,
    const void* bias, const void* const* residuals, int64_t ld_res, double p_drop,
    uint64_t seed, uint64_t offset, const int64_t* mask_row0, int64_t mask_col0,
    int64_t mask_ld, void* const* out, cce_mat out_shard, uint32_t flags, cce_stream stream) {
  clear_error();
  if (!ctx) return fail(CCE_EINVAL, "ctx is NULL");
  // The workspace this call needs, checked against the static maximum before
  // anything else touches the arguments' memory.
  RsGeom g;
  CCE_TRY(rs_geometry(n_ranks, mode, CCE_F32, out_shard, g));
  if (static_cast<uint64_t>(g.total) > CCE_NOALLOC_SCRATCH_BYTES)
    return fail(CCE_EUNSUPPORTED, "needs " + std::to_string(g.total) +
                                      " bytes of workspace; the static scratch holds " +
                                      std::to_string(CCE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (g.total > 0) CCE_TRY(scratch_of(ctx->device, &ws));
  const RsEpiArgs ea{bias, residuals, ld_res, p_drop, seed, offset, mask_row0, mask_col0, mask_ld};
  return rs_impl(ctx, n_ranks, mode, in_t, CCE_F32, out_t, a, a_shape, b, b_shape, out, out_shard,
                 ws, ws ? static_cast<size_t>(CCE_NOALLOC_SCRATCH_BYTES) : 0, flags, stream, &ea);
}

cce_status cce_grouped_gemm(cce_ctx* ctx, int n_groups, cce_dtype in_t, cce_dtype out_t,
                            const void* const* a, cce_mat a_shape, const void* const* b,
                            cce_mat b_shape, void* const* c, cce_mat c_shape, uint32_t flags,
                            cce_stream stream) {
  clear_error();
  if (!ctx) return fail(CCE_EINVAL, "ctx is NULL");
  if (flags & ~CCE_FLAG_GELU) return fail(CCE_EINVAL, "unsupported flags for grouped GEMM");
  if (n_groups < 1) return fail(CCE_EINVAL, "n_groups < 1");
  if (n_groups > CCE_MAX_RANKS) return fail(CCE_EUNSUPPORTED, "n_groups > CCE_MAX_RANKS");
  if (!a || !b || !c) return fail(CCE_EINVAL, "pointer array is NULL");
  if (!dtype_ok(in_t) || !dtype_ok(out_t)) return fail(CCE_EINVAL, "bad dtype");
  CCE_TRY(check_mat("a_shape", a_shape));
  CCE_TRY(check_mat("b_shape", b_shape));
  CCE_TRY(check_mat("c_shape", c_shape));
  if (a_shape.cols != b_shape.cols) return fail(CCE_EINVAL, "a and b must share the contraction length");
  if (c_shape.rows != a_shape.rows || c_shape.cols != b_shape.rows)
    return fail(CCE_EINVAL, "c must be [a rows, b rows]");
  if (a_shape.cols % 8 != 0) return fail(CCE_EUNSUPPORTED, "contraction length must be a multiple of 8");
  const size_t ein = esize(in_t), eout = esize(out_t);
  const int64_t as = span_bytes(a_shape, ein), bs = span_bytes(b_shape, ein),
                cs = span_bytes(c_shape, eout);
  if (as > kMaxOperandBytes || bs > kMaxOperandBytes)
    return fail(CCE_EUNSUPPORTED, "a GEMM operand exceeds 1 GiB");
  std::vector<Range> ranges;
  for (int r = 0; r < n_groups; ++r) {
    const std::string rs = std::to_string(r);
    CCE_TRY(check_ptr(("a[" + rs + "]").c_str(), a[r], as));
    CCE_TRY(check_ptr(("b[" + rs + "]").c_str(), b[r], bs));
    CCE_TRY(check_ptr(("c[" + rs + "]").c_str(), c[r], cs));
    ranges.push_back(range_of(a[r], as, "a[" + rs + "]", false));
    ranges.push_back(range_of(b[r], bs, "b[" + rs + "]", false));
    ranges.push_back(range_of(c[r], cs, "c[" + rs + "]", true));
  }
  CCE_TRY(check_overlaps(ranges));
  if (c_shape.rows == 0 || c_shape.cols == 0) return CCE_OK;
  DeviceGuard guard(ctx->device);
  GemmLaunch L;
  L.groups = n_groups;
  L.M = a_shape.rows;
  L.N = b_shape.rows;
  L.K = a_shape.cols;
  L.lda = a_shape.ld;
  L.ldb = b_shape.ld;
  L.ldc = c_shape.ld;
  L.in_t = in_t;
  L.out_t = out_t;
  L.epi = EPI_STORE;
  L.gelu = (flags & CCE_FLAG_GELU) != 0;
  for (int r = 0; r < n_groups; ++r) {
    L.p.a[r] = a[r];
    L.p.b[r] = b[r];
    L.p.c[r] = c[r];
    L.p.cin[r] = nullptr;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int slot;
  CCE_TRY(prof_begin(ctx, hs, 0, -1, 2.0 * L.M * L.N * L.K * L.groups, 0.0, &slot));
  CCE_TRY(launch_grouped_gemm(L, stream));
  return prof_end(ctx, hs, slot);
}

// Shared by the single and the batched epilogue entry points.  residuals and
// mask_outs are NULL or arrays of n_batch non-NULL pointers.
static cce_status epilogue_impl(cce_ctx* ctx, int n_batch, int n_partials, cce_dtype part_t,
                                const void* const* partials, cce_mat shape, const void* bias,
                                cce_dtype bias_t, const void* const* residuals, cce_dtype res_t,
                                int64_t ld_res, double p_drop, uint64_t seed, uint64_t offset,
                                const int64_t* mask_row0, int64_t mask_col0, int64_t mask_ld,
                                void* const* outs, int n_rep, cce_dtype out_t, int64_t ld_out,
                                uint8_t* const* mask_outs, uint32_t flags, cce_stream stream) {
  if (!ctx) return fail(CCE_EINVAL, "ctx is NULL");
  if (flags != 0) return fail(CCE_EINVAL, "flags must be 0");
  if (n_batch < 1) return fail(CCE_EINVAL, "n_batch < 1");
  if (n_partials < 1) return fail(CCE_EINVAL, "n_partials < 1");
  if (n_rep < 1) return fail(CCE_EINVAL, "n_rep < 1");
  if (static_cast<int64_t>(n_partials) * n_batch > CCE_MAX_RANKS ||
      static_cast<int64_t>(n_rep) * n_batch > CCE_MAX_RANKS)
    return fail(CCE_EUNSUPPORTED, "n_batch * n_partials (or outputs) > CCE_MAX_RANKS");
  if (!partials) return fail(CCE_EINVAL, "partials is NULL");
  if (!outs) return fail(CCE_EINVAL, "out is NULL");
  if (!mask_row0) return fail(CCE_EINVAL, "mask_row0 is NULL");
  if (!dtype_ok(part_t) || !dtype_ok(out_t) || (bias && !dtype_ok(bias_t)) ||
      (residuals && !dtype_ok(res_t)))
    return fail(CCE_EINVAL, "bad dtype");
  if ((bias && bias_t != out_t) || (residuals && res_t != out_t))
    return fail(CCE_EUNSUPPORTED, "bias and residual must have the output dtype");
  if (std::isnan(p_drop)) return fail(CCE_EINVAL, "p_drop is NaN");
  CCE_TRY(check_mat("shape", shape));
  const cce_mat rmat{shape.rows, shape.cols, ld_res}, omat{shape.rows, shape.cols, ld_out};
  if (residuals) CCE_TRY(check_mat("residual", rmat));
  CCE_TRY(check_mat("out", omat));
  if (mask_col0 < 0 || mask_ld < mask_col0 + shape.cols)
    return fail(CCE_EINVAL, "mask index base must satisfy 0 <= col0, col0 + cols <= mask_ld");
  for (int b = 0; b < n_batch; ++b)
    if (mask_row0[b] < 0) return fail(CCE_EINVAL, "mask row base must be >= 0");
  const size_t ep = esize(part_t), eo = esize(out_t);
  const int64_t ps = span_bytes(shape, ep), rs = residuals ? span_bytes(rmat, eo) : 0,
                os = span_bytes(omat, eo), bs = bias ? shape.cols * static_cast<int64_t>(eo) : 0,
                ms = mask_outs ? shape.rows * shape.cols : 0;
  std::vector<Range> ranges;
  for (int k = 0; k < n_partials * n_batch; ++k) {
    const std::string ks = std::to_string(k);
    CCE_TRY(check_ptr(("partials[" + ks + "]").c_str(), partials[k], ps));
    ranges.push_back(range_of(partials[k], ps, "partials[" + ks + "]", false));
  }
  if (bias) CCE_TRY(check_ptr("bias", bias, bs));
  ranges.push_back(range_of(bias, bs, "bias", false));
  for (int b = 0; b < n_batch; ++b) {
    const std::string bsx = "[" + std::to_string(b) + "]";
    if (residuals) {
      CCE_TRY(check_ptr(("residual" + bsx).c_str(), residuals[b], rs));
      ranges.push_back(range_of(residuals[b], rs, "residual" + bsx, false));
    }
    for (int q = 0; q < n_rep; ++q) {
      const std::string oq = "out[" + std::to_string(b * n_rep + q) + "]";
      CCE_TRY(check_ptr(oq.c_str(), outs[b * n_rep + q], os));
      ranges.push_back(range_of(outs[b * n_rep + q], os, oq, true));
    }
    if (mask_outs) {
      CCE_TRY(check_ptr(("mask_out" + bsx).c_str(), mask_outs[b], ms));
      ranges.push_back(range_of(mask_outs[b], ms, "mask_out" + bsx, true));
    }
  }
  CCE_TRY(check_overlaps(ranges));
  if (shape.rows == 0 || shape.cols == 0) return CCE_OK;

  EpilogueLaunch L;
  L.n = n_partials;
  L.batch = n_batch;
  L.part_t = part_t;
  for (int k = 0; k < n_partials * n_batch; ++k) L.parts[k] = partials[k];
  for (int b = 0; b < n_batch; ++b) {
    L.res[b] = residuals ? residuals[b] : nullptr;
    L.mask[b] = mask_outs ? mask_outs[b] : nullptr;
    L.mrow0[b] = mask_row0[b];
  }
  L.n_rep = n_rep;
  for (int q = 0; q < n_batch * n_rep; ++q) L.out[q] = outs[q];
  L.rows = shape.rows;
  L.cols = shape.cols;
  L.ld_part = shape.ld;
  L.bias = bias;
  L.bias_t = bias_t;
  L.res_t = res_t;
  L.ld_res = ld_res;
  L.out_t = out_t;
  L.ld_out = ld_out;
  L.seed = seed;
  L.offset = offset;
  L.mcol0 = mask_col0;
  L.mld = mask_ld;
  if (p_drop <= 0.0) {
    L.dropout = false;
    L.scale = 1.0f;
  } else if (p_drop >= 1.0) {
    L.drop_all = true;
  } else {
    L.dropout = true;
    const double t = std::floor(p_drop * 4294967296.0);
    L.threshold = static_cast<uint32_t>(t);
    L.scale = static_cast<float>(1.0 / (1.0 - p_drop));
  }
  DeviceGuard guard(ctx->device);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const double ebytes =
      n_batch * (static_cast<double>(shape.rows) * shape.cols *
                 (static_cast<double>(n_partials) * ep + (residuals ? eo : 0) +
                  static_cast<double>(n_rep) * eo)) +
      (bias ? static_cast<double>(shape.cols) * eo : 0.0);
  int slot;
  CCE_TRY(prof_begin(ctx, hs, 2, -1, 0.0, ebytes, &slot));
  CCE_TRY(launch_fused_epilogue(L, stream));
  return prof_end(ctx, hs, slot);
}

cce_status cce_fused_reduce_epilogue(cce_ctx* ctx, int n_partials, cce_dtype part_t,
                                     const void* const* partials, cce_mat shape, const void* bias,
                                     cce_dtype bias_t, const void* residual, cce_dtype res_t,
                                     int64_t ld_res, double p_drop, uint64_t seed, uint64_t offset,
                                     int64_t mask_row0, int64_t mask_col0, int64_t mask_ld,
                                     void* out, cce_dtype out_t, int64_t ld_out, uint8_t* mask_out,
                                     uint32_t flags, cce_stream stream) {
  clear_error();
  const void* res1[1] = {residual};
  void* out1[1] = {out};
  uint8_t* mask1[1] = {mask_out};
  const int64_t row1[1] = {mask_row0};
  return epilogue_impl(ctx, 1, n_partials, part_t, partials, shape, bias, bias_t,
                       residual ? res1 : nullptr, res_t, ld_res, p_drop, seed, offset, row1,
                       mask_col0, mask_ld, out1, 1, out_t, ld_out, mask_out ? mask1 : nullptr,
                       flags, stream);
}

cce_status cce_fused_reduce_epilogue_batched(
    cce_ctx* ctx, int n_batch, int n_partials, cce_dtype part_t, const void* const* partials,
    cce_mat shape, const void* bias, cce_dtype bias_t, const void* const* residuals,
    cce_dtype res_t, int64_t ld_res, double p_drop, uint64_t seed, uint64_t offset,
    const int64_t* mask_row0, int64_t mask_col0, int64_t mask_ld, void* const* outs,
    cce_dtype out_t, int64_t ld_out, uint8_t* const* mask_outs, uint32_t flags,
    cce_stream stream) {
  clear_error();
  if (residuals)
    for (int b = 0; b < n_batch && b < CCE_MAX_RANKS; ++b)
      if (!residuals[b]) return fail(CCE_EINVAL, "residuals[b] is NULL (pass a NULL array for none)");
  if (mask_outs)
    for (int b = 0; b < n_batch && b < CCE_MAX_RANKS; ++b)
      if (!mask_outs[b]) return fail(CCE_EINVAL, "mask_outs[b] is NULL (pass a NULL array for none)");
  return epilogue_impl(ctx, n_batch, n_partials, part_t, partials, shape, bias, bias_t, residuals,
                       res_t, ld_res, p_drop, seed, offset, mask_row0, mask_col0, mask_ld, outs,
                       1, out_t, ld_out, mask_outs, flags, stream);
}

cce_status cce_fused_allreduce_epilogue(cce_ctx* ctx, int n_ranks, cce_dtype part_t,
                                        const void* const* partials, cce_mat shape,
                                        const void* bias, cce_dtype bias_t, const void* residual,
                                        cce_dtype res_t, int64_t ld_res, double p_drop,
                                        uint64_t seed, uint64_t offset, int64_t mask_row0,
                                        int64_t mask_col0, int64_t mask_ld, void* const* outs,
                                        cce_dtype out_t, int64_t ld_out, uint8_t* mask_out,
                                        uint32_t flags, cce_stream stream) {
  clear_error();
  const void* res1[1] = {residual};
  uint8_t* mask1[1] = {mask_out};
  const int64_t row1[1] = {mask_row0};
  return epilogue_impl(ctx, 1, n_ranks, part_t, partials, shape, bias, bias_t,
                       residual ? res1 : nullptr, res_t, ld_res, p_drop, seed, offset, row1,
                       mask_col0, mask_ld, outs, n_ranks, out_t, ld_out,
                       mask_out ? mask1 : nullptr, flags, stream);
}

int cce_overlap_beneficial(double original_comp, double original_comm, double ring_comm,
                           double epilogue) {
  const double v[4] = {original_comp, original_comm, ring_comm, epilogue};
  for (double x : v)
    if (!(x >= 0.0)) return -1;                 // negative or NaN
  return original_comp + original_comm >= std::max(original_comp, ring_comm) + epilogue ? 1 : 0;
}

int cce_overlap_choose(double comp, double comm0, double shard_bytes0, double comm1,
                       double shard_bytes1) {
  const double v[5] = {comp, comm0, shard_bytes0, comm1, shard_bytes1};
  for (double x : v)
    if (!(x >= 0.0)) return -1;
  if (comp < comm0 && comp < comm1) return shard_bytes1 < shard_bytes0 ? 1 : 0;
  return comm1 > comm0 ? 1 : 0;
}

cce_status cce_describe_plan(int kind, int n_ranks, int mode, cce_dtype out_t, uint32_t flags,
                             char* buf, size_t buf_len, size_t* needed) {
  clear_error();
  if (n_ranks < 1 || n_ranks > CCE_MAX_RANKS) return fail(CCE_EINVAL, "n_ranks out of range");
  if (!dtype_ok(out_t)) return fail(CCE_EINVAL, "bad dtype");
  if (flags & ~(CCE_FLAG_SERIAL | CCE_FLAG_GELU | CCE_FLAG_COPY_DMA | CCE_FLAG_FUSED_PERMUTE |
                CCE_FLAG_BIDIRECTIONAL | CCE_FLAG_FINE_GRAINED | CCE_FLAG_ONE_CHAIN))
    return fail(CCE_EINVAL, "unknown flags");
  if (kind == 0 && (flags & CCE_FLAG_FINE_GRAINED))
    return fail(CCE_EINVAL, "CCE_FLAG_FINE_GRAINED applies to the ReduceScatter");
  const bool serial = (flags & CCE_FLAG_SERIAL) != 0;
  const bool fused = (flags & CCE_FLAG_FUSED_PERMUTE) != 0;
  const bool bidir = (flags & CCE_FLAG_BIDIRECTIONAL) != 0;
  if (bidir && 2 * n_ranks > CCE_MAX_RANKS)
    return fail(CCE_EUNSUPPORTED, "the bidirectional form takes at most CCE_MAX_RANKS / 2 ranks");
  Plan p;
  if (kind == 0) {
    if (mode < 0 || mode > 4) return fail(CCE_EINVAL, "bad AllGather mode");
    const bool case2 = (mode == CCE_AG_LHS_COLS || mode == CCE_AG_RHS_ROWS);
    if (bidir && case2)
      return fail(CCE_EUNSUPPORTED, "the bidirectional form takes the case-1 modes only");
    p = bidir ? build_allgather_plan_bidir(n_ranks, mode, serial, fused)
              : build_allgather_plan(n_ranks, mode, case2 && out_t == CCE_BF16 && n_ranks > 1,
                                     serial, fused);
  } else if (kind == 1 || kind == 2) {
    if (mode != 0 && mode != 1) return fail(CCE_EINVAL, "bad ReduceScatter mode");
    if ((flags & CCE_FLAG_FINE_GRAINED) && bidir && !fused)
      return fail(CCE_EUNSUPPORTED, "CCE_FLAG_FINE_GRAINED with CCE_FLAG_BIDIRECTIONAL needs "
                                    "CCE_FLAG_FUSED_PERMUTE");
    const bool halves = (flags & CCE_FLAG_ONE_CHAIN) == 0;
    p = bidir ? build_reducescatter_plan_bidir(n_ranks, mode, halves, serial, fused)
              : build_reducescatter_plan(n_ranks, mode, halves, serial, fused);
    if (flags & CCE_FLAG_FINE_GRAINED) make_fine_grained(p, kind == 2);
  } else {
    return fail(CCE_EINVAL, "kind must be 0, 1 or 2");
  }
  const std::string s = describe_plan(p);
  if (needed) *needed = s.size() + 1;
  if (buf && buf_len > 0) {
    const size_t k = std::min(buf_len - 1, s.size());
    std::memcpy(buf, s.data(), k);
    buf[k] = '\0';
  }
  return CCE_OK;
}

}  // extern "C"
