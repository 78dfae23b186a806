// Internal declarations shared by the library's translation units.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/cce.h"

namespace cce {

// ---------------------------------------------------------------------------
// Error reporting
// ---------------------------------------------------------------------------
void set_error(const std::string& msg);
void clear_error();
cce_status fail(cce_status s, const std::string& msg);

// ---------------------------------------------------------------------------
// Grouped GEMM launch description: one launch computes, for every group g,
//   C_g[M, N] = epilogue(A_g[M, K] * B_g[N, K]^T, Cin_g)
// with shared extents and leading dimensions.
// ---------------------------------------------------------------------------
enum Epi : int {
  EPI_STORE = 0,        // C = part
  EPI_ACCUM = 1,        // C = Cin + part       (Cin fp32, may alias C)
  EPI_FINAL = 2,        // Cin + part is the last partial of an output chunk: the
                        // chunk's consumer (FinalArgs) runs in the same launch
};

constexpr int kMaxGroups = CCE_MAX_RANKS;

// Fine-grained overlap of the ReduceScatter's last launch with its consumer
// (CoCoNet's fine-grained overlap of a MatMul with the collective that
// consumes it, chunk by chunk): every output tile ("chunk") of rank s is
// complete when its last partials -- one per ring direction -- are computed;
// the consumer (the align-and-sum of the two directions, or the fused reduce
// epilogue) then runs for that chunk inside the producing launch.  With two
// producers in the launch, they claim the chunk through a per-chunk counter:
// the first stores its fp32 partial at its accumulator (C) and publishes a
// ready word; the second waits for that word (a bounded poll) and consumes its
// own partial from registers plus the published one.  The consumer computes
//   out = residual + keep * ((p_own + p_other) + bias) * scale
// in the standalone epilogue's order, each step rounded to fp32.
constexpr unsigned kSignalPollCap = 1u << 18;   // polls before a consumer gives up

struct FinalArgs {
  int8_t oid[kMaxGroups];               // output (rank) of each group's chunks
  int8_t partner[kMaxGroups];           // group producing the other partial in this launch, or -1
  const float* other[kMaxGroups];       // per output: the other partial, already in memory, or NULL
  const void* res[kMaxGroups];          // per output: residual, or NULL
  void* out[kMaxGroups];                // per output
  int64_t mrow0[kMaxGroups];            // per output: global row of its first row (keep mask)
  const void* bias = nullptr;           // [N] of the output type, or NULL
  int64_t ld_res = 0, ld_out = 0;
  int mode = 0;                         // 0 no dropout, 1 dropout, 2 drop everything
  uint32_t threshold = 0;
  float scale = 1.0f;
  uint32_t key0 = 0, key1 = 0, off0 = 0, off1 = 0;
  int64_t mcol0 = 0, mld = 0;
  bool aligned = true;                  // 4 | mld and 4 | mcol0: one Philox block per 4 columns
  unsigned* sig = nullptr;              // [2 * (oid * tiles_per_group + tile)]: claim, ready
  int64_t sig_tiles = 0;                // chunks per output the signal words hold (>= tiles_per_group)
  unsigned* err = nullptr;              // counts consumers that gave up waiting
  unsigned cap = kSignalPollCap;
  int nopub = 0;                        // test hook: first producers do not publish
};

struct GemmGroupPtrs {
  const void* a[kMaxGroups];
  const void* b[kMaxGroups];
  void* c[kMaxGroups];
  const float* cin[kMaxGroups];
  void* fwd[kMaxGroups];      // forward destination of the looped operand
};

// Operand a fused-permute GEMM forwards (writes once, as it stages it).
enum Fwd : int { FWD_NONE = 0, FWD_A = 1, FWD_B = 2 };

struct GemmLaunch {
  int groups = 0;
  int64_t M = 0, N = 0, K = 0;
  int64_t lda = 0, ldb = 0, ldc = 0, ldcin = 0;
  cce_dtype in_t = CCE_BF16;
  cce_dtype out_t = CCE_BF16;
  int epi = EPI_STORE;
  bool gelu = false;
  int fwd = FWD_NONE;          // forward A or B of every group to p.fwd[g]
  int64_t ldfwd = 0;
  GemmGroupPtrs p{};
  FinalArgs fin{};             // EPI_FINAL only
};

// Ring-permute copy (permute.hip): `rows` rows of `width` bytes, row i at
// src + i * src_pitch -> dst + i * dst_pitch.  One launch copies every item
// of a permute step on the copy stream.  permute_item_ok: the kernel takes
// single spans (rows == 1) of a multiple of 16 bytes at 16-byte aligned
// pointers; the caller gives anything else to the runtime's copy.
constexpr int kMaxPermuteItems = kMaxGroups;
struct PermuteItem {
  const void* src = nullptr;
  void* dst = nullptr;
  int64_t rows = 0, width = 0, src_pitch = 0, dst_pitch = 0;
};
bool permute_item_ok(const PermuteItem& it);
// `alone`: nothing runs beside this copy (the two-way AllGather's prologue,
// the ReduceScatter's last permute), so it takes the whole GPU.
cce_status launch_permute_copy(const PermuteItem* items, int n, void* stream, bool alone);

// Enqueue a kernel that sets n 32-bit words at p to zero (the chunk signal
// words of a call, cleared by a kernel rather than a memset so that the call
// can be captured in a graph).
cce_status launch_zero_words(unsigned* p, int64_t n, void* stream);

// Enqueue one grouped GEMM on `stream` (a hipStream_t).  Returns CCE_OK or
// CCE_EHIP.  Shapes must already be validated.
cce_status launch_grouped_gemm(const GemmLaunch& g, void* stream);

// ---------------------------------------------------------------------------
// Fused reduce epilogue launch.
// ---------------------------------------------------------------------------
struct EpilogueLaunch {
  int n = 0;                  // partials per output
  int batch = 1;              // outputs in the launch (batch * n <= kMaxGroups)
  cce_dtype part_t = CCE_F32;
  const void* parts[kMaxGroups];   // [b * n + k]
  int64_t rows = 0, cols = 0, ld_part = 0;
  const void* bias = nullptr;
  cce_dtype bias_t = CCE_F32;
  const void* res[kMaxGroups];     // per output; NULL entries: no residual
  cce_dtype res_t = CCE_F32;
  int64_t ld_res = 0;
  void* out[kMaxGroups];           // [b * n_rep + q]
  int n_rep = 1;                   // replicas of each output (FusedAllReduce's AllGather)
  cce_dtype out_t = CCE_F32;
  int64_t ld_out = 0;
  uint8_t* mask[kMaxGroups];       // per output; NULL entries: no mask output
  int64_t mrow0[kMaxGroups];
  uint32_t threshold = 0;     // keep iff word >= threshold (when !drop_all)
  bool drop_all = false;
  bool dropout = false;       // p > 0
  float scale = 1.0f;
  uint64_t seed = 0, offset = 0;
  int64_t mcol0 = 0, mld = 0;
};

cce_status launch_fused_epilogue(const EpilogueLaunch& e, void* stream);

// ---------------------------------------------------------------------------
// Plan IR: the ordered operations of one looped call, independent of HIP.
// Buffers are symbolic so that the same plan can be printed and race-checked
// on the host, and resolved to device pointers by the executor.
// ---------------------------------------------------------------------------
enum BufKind : uint8_t {
  B_LOOPED = 0,   // caller's looped shard of a rank (AllGather)
  B_LOCAL = 1,    // caller's local operand of a rank
  B_OUT = 2,      // caller's output of a rank
  B_RECV = 3,     // workspace receive buffer (rank, parity)  AllGather
  B_ACC = 4,      // workspace accumulator (rank, parity, half) ReduceScatter
  B_CASE2 = 5,    // workspace fp32 accumulator (rank) AllGather case 2, bf16 out
  B_A = 6,        // caller's left factor (ReduceScatter)
  B_B = 7,        // caller's right factor (ReduceScatter)
  B_RECV_CCW = 8, // workspace receive buffer of the counter-clockwise stream (rank, parity)
  B_ACC_CCW = 9,  // workspace counter-clockwise accumulator (rank, parity, half)
};

struct BufRef {
  uint8_t kind = 0;
  uint8_t parity = 0;
  uint8_t half = 0;
  int16_t rank = 0;
};

struct Item {            // one rank's share of a GEMM or copy
  int rank = 0;
  int shard = 0;         // shard / slice ID worked on
  BufRef a, b, cin, c;   // gemm: reads a, b (and cin if has_cin), writes c
                         // copy: reads a, writes c
  BufRef fwd;            // gemm with a fused permute: writes the looped operand here
  bool has_cin = false;
  bool has_fwd = false;
  // EPI_FINAL gemm (fine-grained overlap): c is the output the chunk's
  // consumer writes; `meet` is this item's own accumulator, where it stores
  // its partial when it is the first of a pair; `other` is the other partial
  // of the same output -- the pair item's meet (pair >= 0, read after its
  // ready signal) or a buffer finished by an earlier launch.
  BufRef meet, other;
  bool has_other = false;
  int pair = -1;         // index of the pair item in the same op
};

// OP_SUM: out = a + c-side input per item (the bidirectional ReduceScatter's
// align-and-sum epilogue); reads a and cin, writes c.
enum OpKind : uint8_t { OP_GEMM = 0, OP_COPY = 1, OP_RECORD = 2, OP_WAIT = 3, OP_SUM = 4 };
enum StreamId : uint8_t { S_COMPUTE = 0, S_COPY = 1 };

struct Op {
  OpKind kind = OP_GEMM;
  StreamId stream = S_COMPUTE;
  int iter = 0;
  int half = 0;          // ReduceScatter half-step (0/1); 0 for AllGather
  int event = -1;        // record / wait
  bool hint = false;     // wait that orders dispatch only (not needed for correctness)
  int epi = EPI_STORE;   // gemm epilogue
  bool final_store = false;   // gemm writes the caller's output dtype
  std::vector<Item> items;
};

struct Plan {
  int kind = 0;          // 0 AllGather, 1 ReduceScatter
  int n = 0;
  int mode = 0;
  int n_events = 0;
  bool serial = false;
  bool fused = false;    // permutes fused into the GEMMs (no copy ops)
  bool bidir = false;    // two-way ring: items of both directions per op
  std::vector<Op> ops;
};

// Shard ID rank r uses in iteration i.
inline int ag_shard(int n, int r, int i) { return (r + i) % n; }
inline int rs_slice(int n, int r, int i) { return (r + i + 1) % n; }

// Bidirectional ring ([OV] 5.4.2): the clockwise stream (rank r sends to
// r - 1) runs ceil(n/2) iterations, the counter-clockwise one (r sends to
// r + 1) floor(n/2).  AllGather: the cw buffer starts with the own shard,
// the ccw buffer with the shard of rank r - 1 (prologue permute).
// ReduceScatter: the cw accumulator of a slice ends on its rank at loop end,
// the ccw accumulator one rank short of it (one epilogue permute).
inline int bidir_cw_len(int n) { return (n + 1) / 2; }
inline int bidir_ccw_len(int n) { return n / 2; }
inline int mod_n(int x, int n) { return ((x % n) + n) % n; }
inline int ag_shard_cw(int n, int r, int i) { return mod_n(r + i, n); }
inline int ag_shard_ccw(int n, int r, int i) { return mod_n(r - 1 - i, n); }
inline int rs_slice_cw(int n, int r, int i) { return mod_n(r + i + 1 - bidir_cw_len(n), n); }
inline int rs_slice_ccw(int n, int r, int i) { return mod_n(r - i + bidir_ccw_len(n), n); }

// Build the plan of a looped call.  `case2_ws` selects the workspace fp32
// accumulator for AllGather case 2 (bf16 output); `two_halves` is false when
// the ReduceScatter shard has a single row/column (no second chain).
Plan build_allgather_plan(int n, int mode, bool case2_ws, bool serial, bool fused = false);
Plan build_reducescatter_plan(int n, int mode, bool two_halves, bool serial, bool fused = false);
// Bidirectional forms ([OV] 5.4.2).  AllGather: case 1 modes only.
Plan build_allgather_plan_bidir(int n, int mode, bool serial, bool fused);
Plan build_reducescatter_plan_bidir(int n, int mode, bool two_halves, bool serial, bool fused);
// Fine-grained overlap (FinalArgs): the consumer of every output chunk runs
// in the launch that produces the chunk's last partials.  Two-way fused
// plans: the last GEMM op becomes EPI_FINAL and the align-and-sum op goes.
// One-way plans with `epilogue`: the final GEMM ops become EPI_FINAL.
// Returns false (plan unchanged) for a plan it does not apply to (two-way
// with copies, one-way without an epilogue).
bool make_fine_grained(Plan& p, bool epilogue);

std::string describe_plan(const Plan& p);

}  // namespace cce
