/*
 * cce.h -- C ABI of the looped CollectiveEinsum library for one MI355X (gfx950).
 *
 * The library computes an AllGather- or ReduceScatter-bound einsum as a loop
 * of N per-shard partial GEMMs, with the collective replaced by a ring of
 * point-to-point shard transfers, and a fused "sum of partials + bias +
 * dropout + residual" epilogue.  All N logical ranks are separate buffers in
 * the HBM of one GPU; a transfer is an asynchronous device-to-device copy on a
 * second stream, ordered by events and double-buffered against the GEMMs.
 *
 * Sources (cited by page title and section):
 *   [OV] Wang et al., "Overlap Communication with Dependent Computation via
 *        Decomposition in Large Deep Learning Models", ASPLOS'23.
 *   [CC] Jangda et al., "Breaking the Computation and Communication
 *        Abstraction Barrier in Distributed Machine Learning Workloads"
 *        (CoCoNet), ASPLOS'22.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Matrices are row-major: element (i, j) of a cce_mat lives at
 * base[i * ld + j]; ld >= cols, counted in elements.  A product is written
 * C = A * B^T: the left factor A is stored [M, K] and the right factor is
 * stored out-major as B^T [N, K] (the nn.Linear weight layout), so both
 * factors are contiguous along the contraction dim.  The mathematical right
 * factor [K, N] of the pages is the transpose of what is passed.
 *
 * Pointer arrays (const void* const* ...) are HOST arrays of n DEVICE
 * pointers, read only during the call.  Every device buffer (inputs,
 * outputs, workspace) is owned by the caller and must stay alive until the
 * work enqueued on `stream` has finished.  The library never writes inputs.
 * Outputs must not overlap inputs or each other.
 *
 * Alignment: every device base pointer must be 16-byte aligned and every ld
 * and every contraction length K a multiple of 8 elements, and every GEMM
 * operand (one rank's factor) must span less than 1 GiB; otherwise the call
 * returns CCE_EUNSUPPORTED.  Other extents (M, N, rows, cols) are arbitrary,
 * including ragged tile tails; a zero extent is a valid no-op.
 *
 * Ordering: calls are asynchronous.  All work of a call is ordered after the
 * work already enqueued on `stream` and before work enqueued on it later; the
 * library's internal copy stream is forked from and joined back to `stream`
 * with events.  Nothing blocks the host.
 *
 * Errors: every argument is validated before anything is enqueued, so a
 * status other than CCE_OK means no work was enqueued (except CCE_EHIP, which
 * reports a failing HIP call; cce_last_error() then names it).  Faults inside
 * kernels surface at the caller's next synchronisation, as in HIP.
 * A cce_ctx is not thread-safe; distinct contexts are independent.
 */
#ifndef CCE_H_
#define CCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cce_status {
  CCE_OK = 0,
  CCE_EINVAL = 1,        /* bad argument: NULL, negative or mismatched extent */
  CCE_EUNSUPPORTED = 2,  /* valid but outside what the kernels take (alignment, dtype combination, n_ranks) */
  CCE_EWORKSPACE = 3,    /* workspace NULL or smaller than the query returned */
  CCE_EHIP = 4           /* a HIP runtime call failed; see cce_last_error() */
} cce_status;

typedef enum cce_dtype { CCE_F32 = 0, CCE_BF16 = 1 } cce_dtype;

typedef struct cce_mat { int64_t rows, cols, ld; } cce_mat;

typedef struct cce_ctx cce_ctx;
typedef void* cce_stream;          /* a hipStream_t; NULL = the null stream */

#define CCE_MAX_RANKS 64

/* Flags (bitwise OR). */
#define CCE_FLAG_SERIAL 0x1u  /* run every copy on `stream` itself, no overlap:
                                 the same kernels and the same results, used as
                                 the unoverlapped comparison */
#define CCE_FLAG_GELU 0x2u    /* apply exact GELU, x*Phi(x), to each output
                                 element as it is stored (AllGather-Einsum and
                                 grouped GEMM only) */
#define CCE_FLAG_COPY_DMA 0x4u /* run the permute copies on the DMA engines
                                  (no compute units) instead of copy kernels */
#define CCE_FLAG_FUSED_PERMUTE 0x8u /* no copy stream: each partial GEMM sends
                                  the data itself.  AllGather: the GEMM writes
                                  the looped shard it stages through LDS to the
                                  next rank's receive buffer (each k tile once);
                                  ReduceScatter: the GEMM's accumulate epilogue
                                  stores into the next rank's accumulator.  Same
                                  results, bit for bit; no extra reads. */
#define CCE_FLAG_BIDIRECTIONAL 0x10u /* [OV] Section 5.4.2: two looped buffers
                                  (AllGather) or accumulators (ReduceScatter)
                                  per rank travel the ring in opposite
                                  directions and each iteration computes both
                                  partial einsums in one launch, so the loop
                                  runs ceil(n/2) iterations; each rank still
                                  sends n-1 shards.  The AllGather fills its
                                  second buffer with a prologue transfer; the
                                  ReduceScatter ends with an epilogue transfer
                                  and an align-and-sum of the two
                                  accumulators.  AllGather case 1 and 3 modes
                                  and both ReduceScatter modes; n_ranks <= 32.
                                  Combines with SERIAL, GELU, COPY_DMA and
                                  FUSED_PERMUTE. */
#define CCE_FLAG_FINE_GRAINED 0x20u /* [CC] fine-grained overlap: the consumer
                                  of each output chunk (tile) of a looped
                                  Einsum-ReduceScatter -- the align-and-sum of
                                  the two ring directions, or the fused reduce
                                  epilogue -- runs inside the launch that
                                  produces the chunk's last partials, as soon
                                  as that chunk is complete, instead of in a
                                  launch after the loop.  The two producers of
                                  a chunk claim it through a per-chunk counter
                                  in the workspace: the first stores its fp32
                                  partial and publishes a ready word, the
                                  second waits for that word (a bounded poll)
                                  and writes the chunk's output from its own
                                  partial and the published one.  Results are
                                  bit-identical to the form without the flag.
                                  Applies to the two-way ring with
                                  CCE_FLAG_FUSED_PERMUTE (both ReduceScatter
                                  entry points) and to the one-way ring of
                                  cce_looped_einsum_reducescatter_epilogue
                                  (any permute form); the one-way
                                  cce_looped_einsum_reducescatter already
                                  writes its output from its last launch, so
                                  the flag changes nothing there; the two-way
                                  ring with copies returns CCE_EUNSUPPORTED.
                                  A consumer that waits too long (it cannot
                                  under the protocol: the first producer is
                                  already running) gives up, leaves its chunk
                                  unwritten and counts the event for
                                  cce_ctx_check_signals. */
#define CCE_FLAG_ONE_CHAIN 0x40u /* ReduceScatter with copies (stream, serial
                                  or DMA form): keep each shard's accumulator
                                  whole, one chain of n launches, instead of
                                  the default two chains of half shards whose
                                  copies overlap the other chain's GEMM.  The
                                  fused permute always runs one chain.  With a
                                  copy stream each copy then waits for its own
                                  GEMM, so the flag is for the serial form: the
                                  unoverlapped comparison with the same GEMMs
                                  as the fused form.  Same results, bit for
                                  bit.  The AllGather entry point accepts it
                                  and is unchanged (its loop is one chain). */

/* Status text; never NULL. */
const char* cce_status_string(cce_status s);

/* Detail of the last error on the calling thread ("" if none). */
const char* cce_last_error(void);

/* Library version as "major.minor.patch". */
const char* cce_version(void);

/* Create a context on HIP device `device`: it owns a copy stream (default
 * priority, non-blocking) and a pool of events.  *out receives the context.
 * It also allocates one 256-byte device word (cce_ctx_check_signals). */
cce_status cce_ctx_create(int device, cce_ctx** out);
cce_status cce_ctx_destroy(cce_ctx* ctx);

/* The stream the context's looped calls run their permute copies on (the
 * second stream of [OV] Section 5.2's asynchronous CollectivePermute): the
 * caller's `copy` (a hipStream_t of the context's device, e.g. one created
 * with a compute-unit mask, or one the caller already synchronises with), or
 * NULL for the context's own.  Work on it is ordered against each call's
 * `stream` by events as before.  The caller keeps ownership and must keep it
 * alive while calls of this context are queued on it; the context never
 * destroys it.  Host-only. */
cce_status cce_ctx_set_copy_stream(cce_ctx* ctx, cce_stream copy);

/* Fine-grained overlap status (CCE_FLAG_FINE_GRAINED): waits for the work
 * queued on `stream`, then reads and clears the context's device error word,
 * which counts chunk consumers that gave up waiting for their pair's partial
 * (those chunks' outputs were not written).  Returns CCE_EHIP, with the count
 * in cce_last_error(), when it is nonzero, CCE_OK otherwise.  Blocks the
 * host. */
cce_status cce_ctx_check_signals(cce_ctx* ctx, cce_stream stream);

/* ------------------------------------------------------------------------
 * Kernel timing.  While profiling is enabled on a context, every GEMM launch,
 * every permute step (the batch of copies of one iteration or half-step) and
 * every epilogue launch it enqueues is bracketed by a pair of timing events
 * on the stream that runs it.  cce_ctx_read_profile waits for those events,
 * returns up to max_records records in enqueue order, and clears the list.
 * Enabling (enable != 0) also clears it.  Host memory only; no allocation on
 * the device.
 *   kind: 0 GEMM launch, 1 permute step (copies), 2 fused epilogue launch,
 *         3 align-and-sum launch (bidirectional ReduceScatter)
 *   iter: loop iteration (GEMM, copies), -1 otherwise
 *   ms:   event-to-event time on the device
 *   flops: 2*M*N*K summed over the launch's groups (GEMM), else 0
 *   bytes: bytes moved (copies: read + write), algorithmic bytes (epilogue)
 * ---------------------------------------------------------------------- */
typedef struct cce_prof_record {
  int32_t kind;
  int32_t iter;
  float ms;
  double flops;
  double bytes;
} cce_prof_record;

cce_status cce_ctx_set_profiling(cce_ctx* ctx, int enable);
cce_status cce_ctx_read_profile(cce_ctx* ctx, int max_records, cce_prof_record* out, int* n_out);

/* ------------------------------------------------------------------------
 * Ring schedule ([OV] Section 5.1).
 * Fills table[i * n_ranks + r] with the shard ID rank r works on in
 * iteration i.  kind 0: looped AllGather-Einsum (aligned with the partition
 * ID at loop start); kind 1: looped Einsum-ReduceScatter (aligned at loop
 * end).  Transfers always go from rank r to rank (r - 1) mod n, the
 * {source, destination} pairs {0, N-1}, {1, 0}, ..., {N-1, N-2}.
 * table is host memory of n_ranks * n_ranks int32.  Host-only; no device.
 * kind 2 / 3: the bidirectional forms (CCE_FLAG_BIDIRECTIONAL) of the
 * AllGather / ReduceScatter loop: table[(i * n_ranks + r) * 2 + d] is the
 * shard of rank r in iteration i for direction d (0: clockwise, sent to
 * r - 1; 1: counter-clockwise, sent to r + 1), -1 when that stream has
 * ended; table holds ceil(n_ranks / 2) * n_ranks * 2 int32; n_ranks <= 32.
 * ---------------------------------------------------------------------- */
cce_status cce_shard_schedule(int n_ranks, int kind, int32_t* table);

/* ------------------------------------------------------------------------
 * Looped AllGather-Einsum ([OV] Sections 4 and 5.1, cases 1, 2 and 3).
 *
 * looped[r] is rank r's own shard (shard ID r) of the operand the AllGather
 * would rebuild; local[r] is rank r's operand that never moves; out[r]
 * receives rank r's full result.  In iteration i rank r computes the partial
 * einsum on shard s = (r + i) mod n while that shard travels on to rank
 * r - 1; the update is a store into the result slice of shard s (cases 1
 * and 3, DynamicUpdateSlice) or an addition (case 2).  Shapes (storage
 * orientation, see the header comment):
 *
 *   CCE_AG_LHS_ROWS  case 1, looped left factor split on rows M:
 *                    looped [m_s, K], local B^T [N, K], out [n*m_s, N];
 *                    shard s fills out rows [s*m_s, (s+1)*m_s).
 *   CCE_AG_RHS_COLS  case 1, looped right factor split on columns N:
 *                    looped B^T [n_s, K], local A [M, K], out [M, n*n_s];
 *                    shard s fills out columns [s*n_s, (s+1)*n_s).
 *   CCE_AG_LHS_COLS  case 2, looped left factor split on K:
 *                    looped [M, k_s], local B^T [N, n*k_s], out [M, N];
 *                    out += shard * (B^T columns [s*k_s, (s+1)*k_s))^T.
 *   CCE_AG_RHS_ROWS  case 2, looped right factor split on K:
 *                    looped B^T [N, k_s], local A [M, n*k_s], out [M, N];
 *                    out += (A columns [s*k_s, (s+1)*k_s)) * shard^T.
 *   CCE_AG_LHS_BATCH case 3, looped left factor split on a batch dim: b_s
 *                    batch elements per shard, each stacked row-wise:
 *                    looped [b_s*m, K] (element e = rows [e*m, (e+1)*m)),
 *                    local B^T [n*b_s*N, K] (element j's B^T = rows
 *                    [j*N, (j+1)*N)), out [n*b_s*m, N] (element j = rows
 *                    [j*m, (j+1)*m)); b_s = local rows / (n * out cols).
 *                    Element e of shard s multiplies the local operand's
 *                    element s*b_s + e (a DynamicSlice along its batch dim,
 *                    of the shard's batch extent) and fills out element
 *                    s*b_s + e.  One GEMM group per batch element: n*b_s
 *                    (2*n*b_s with CCE_FLAG_BIDIRECTIONAL) must not exceed
 *                    CCE_MAX_RANKS.
 *
 * in_t: CCE_BF16 (fp32 accumulation) or CCE_F32 (both inputs the same type).
 * out_t: CCE_BF16 or CCE_F32 (round to nearest even on the final store).
 * Case 2 accumulates across iterations in fp32 (in `out` itself when out_t is
 * CCE_F32, else in the workspace).  flags: CCE_FLAG_SERIAL, CCE_FLAG_GELU,
 * CCE_FLAG_COPY_DMA, CCE_FLAG_FUSED_PERMUTE, CCE_FLAG_BIDIRECTIONAL (cases 1
 * and 3).
 * workspace: device memory of at least the size the query returns (two
 * receive buffers per rank and direction, plus the fp32 accumulators of
 * case 2 with a bf16 output; the size covers every flag combination); its
 * contents on entry do not matter.
 * ---------------------------------------------------------------------- */
typedef enum cce_ag_mode {
  CCE_AG_LHS_ROWS = 0,
  CCE_AG_RHS_COLS = 1,
  CCE_AG_LHS_COLS = 2,
  CCE_AG_RHS_ROWS = 3,
  CCE_AG_LHS_BATCH = 4
} cce_ag_mode;

cce_status cce_looped_allgather_einsum_workspace(int n_ranks, cce_ag_mode mode, cce_dtype in_t,
                                                 cce_dtype out_t, cce_mat looped_shard,
                                                 cce_mat out_shape, size_t* bytes);

cce_status cce_looped_allgather_einsum(cce_ctx* ctx, int n_ranks, cce_ag_mode mode,
                                       cce_dtype in_t, cce_dtype out_t,
                                       const void* const* looped, cce_mat looped_shard,
                                       const void* const* local, cce_mat local_shape,
                                       void* const* out, cce_mat out_shape,
                                       void* workspace, size_t workspace_bytes,
                                       uint32_t flags, cce_stream stream);

/* ------------------------------------------------------------------------
 * Looped Einsum-ReduceScatter ([OV] Sections 4, 5.1 and 5.4.1).
 *
 * a[r], b[r] are rank r's factors; out[r] receives shard r of the sum over
 * all ranks of a[q] * b[q]^T:
 *
 *   CCE_RS_SLICE_LHS_ROWS  a [n*m_s, K], b^T [N, K], out [m_s, N];
 *                          out_r = sum_q (a_q b_q^T)[rows r*m_s .. +m_s).
 *   CCE_RS_SLICE_RHS_COLS  a [M, K], b^T [n*n_s, K], out [M, n_s];
 *                          out_r = sum_q (a_q b_q^T)[cols r*n_s .. +n_s).
 *
 * The accumulator of each shard travels the ring (rank r -> r - 1) and ends
 * on the rank of its shard ID; in iteration i rank r adds its partial for
 * slice t = (r + i + 1) mod n.  As in the loop unrolling of [OV] 5.4.1, each
 * accumulator is split into two halves that form two interleaved chains, so
 * the transfer of one half overlaps the GEMM of the other.  For every element
 * of out[s] the sum runs over the partials of ranks s-1, s-2, ..., s+1, s
 * (mod n) in that order, in fp32, whatever the flags -- except with
 * CCE_FLAG_BIDIRECTIONAL, where out[s] = cw + ccw: cw sums the partials of
 * ranks s+c-1, ..., s+1, s and ccw those of ranks s-w, ..., s-1 (c =
 * ceil(n/2), w = floor(n/2), indices mod n), each chain in that order.
 * in_t: CCE_BF16 or CCE_F32; acc_t: CCE_F32 only; out_t: CCE_F32 or CCE_BF16.
 * flags: CCE_FLAG_SERIAL, CCE_FLAG_COPY_DMA, CCE_FLAG_FUSED_PERMUTE,
 * CCE_FLAG_BIDIRECTIONAL.
 * workspace: two fp32 accumulators per rank and direction (the query
 * returns the size, which covers every flag combination).
 * ---------------------------------------------------------------------- */
typedef enum cce_rs_mode { CCE_RS_SLICE_LHS_ROWS = 0, CCE_RS_SLICE_RHS_COLS = 1 } cce_rs_mode;

cce_status cce_looped_einsum_reducescatter_workspace(int n_ranks, cce_rs_mode mode,
                                                     cce_dtype acc_t, cce_mat out_shard,
                                                     size_t* bytes);

cce_status cce_looped_einsum_reducescatter(cce_ctx* ctx, int n_ranks, cce_rs_mode mode,
                                           cce_dtype in_t, cce_dtype acc_t, cce_dtype out_t,
                                           const void* const* a, cce_mat a_shape,
                                           const void* const* b, cce_mat b_shape,
                                           void* const* out, cce_mat out_shard,
                                           void* workspace, size_t workspace_bytes,
                                           uint32_t flags, cce_stream stream);

/* ------------------------------------------------------------------------
 * Looped Einsum-ReduceScatter with the fused reduce epilogue
 * ([OV] Sections 4, 5.1, 5.4.1 and 5.4.2; [CC] Figure 3 program).
 *
 *   out[r] = residual[r] + keep * (S_r + bias) * c,   c = 1 / (1 - p_drop)
 *
 * where S_r is the fp32 result that cce_looped_einsum_reducescatter gives
 * for rank r with the same a, b, mode and flags.  The result is, bit for
 * bit, that call with out_t = CCE_F32 followed by
 * cce_fused_reduce_epilogue_batched over the ranks (one partial each, the
 * same bias, residuals, dropout and mask arguments), without storing S_r in
 * the caller's memory:
 *   - with CCE_FLAG_BIDIRECTIONAL the two chains' accumulators go straight
 *     into the epilogue, which sums them (cw + ccw, the align-and-sum's
 *     order) before the bias: the sum is never stored;
 *   - in the one-way form the last iteration leaves S_r in the workspace and
 *     one batched epilogue launch reads it from there.
 * Arguments: as cce_looped_einsum_reducescatter (acc_t is CCE_F32), plus
 * the epilogue's: bias [out cols] of out_t or NULL; residuals NULL or n_ranks
 * pointers to [out rows, out cols] arrays of out_t with ld_res; dropout,
 * seed, offset and the keep mask as cce_fused_reduce_epilogue, with
 * mask_row0[r] the global row of rank r's first output row.  out[r] of
 * out_t (CCE_F32 or CCE_BF16) with out_shard.ld.  The workspace is the one
 * cce_looped_einsum_reducescatter_workspace returns.  flags: those of
 * cce_looped_einsum_reducescatter.  No mask output.
 * ---------------------------------------------------------------------- */
cce_status cce_looped_einsum_reducescatter_epilogue(
    cce_ctx* ctx, int n_ranks, cce_rs_mode mode, cce_dtype in_t, cce_dtype out_t,
    const void* const* a, cce_mat a_shape, const void* const* b, cce_mat b_shape,
    const void* bias, const void* const* residuals, int64_t ld_res, double p_drop,
    uint64_t seed, uint64_t offset, const int64_t* mask_row0, int64_t mask_col0,
    int64_t mask_ld, void* const* out, cce_mat out_shard, void* workspace,
    size_t workspace_bytes, uint32_t flags, cce_stream stream);

/* ------------------------------------------------------------------------
 * Allocation-free variant of cce_looped_einsum_reducescatter_epilogue, for
 * callers that cannot allocate device memory or hand over a workspace: code
 * under HIP graph capture, serving loops and harnesses that forbid
 * allocation.  Arguments, results and errors are those of
 * cce_looped_einsum_reducescatter_epilogue without the workspace (same
 * kernels, bit-identical outputs); the caller still passes inputs and
 * outputs.  The workspace is a static device array of
 * CCE_NOALLOC_SCRATCH_BYTES inside the library: each GPU holds its own copy
 * from the library's first context on that device until the process ends.
 * A call whose workspace (the size cce_looped_einsum_reducescatter_workspace
 * returns) exceeds it returns CCE_EUNSUPPORTED before anything is enqueued.
 * The call allocates no device memory (no hipMalloc, hipFree or allocating
 * library routine); the context's event pool grows on its first looped call,
 * as for every entry point.  The array keeps the last call's contents and
 * every call on a GPU shares it: calls on one stream are ordered, but calls
 * that overlap on one GPU (other streams, other contexts or threads) race on
 * it.  Devices 0..63.
 * ---------------------------------------------------------------------- */
#define CCE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

cce_status cce_looped_einsum_reducescatter_epilogue_noalloc(
    cce_ctx* ctx, int n_ranks, cce_rs_mode mode, cce_dtype in_t, cce_dtype out_t,
    const void* const* a, cce_mat a_shape, const void* const* b, cce_mat b_shape,
    const void* bias, const void* const* residuals, int64_t ld_res, double p_drop,
    uint64_t seed, uint64_t offset, const int64_t* mask_row0, int64_t mask_col0,
    int64_t mask_ld, void* const* out, cce_mat out_shard, uint32_t flags, cce_stream stream);

/* ------------------------------------------------------------------------
 * Grouped local GEMM: c[g] = a[g] * b[g]^T for g < n_groups, one launch.
 * This is the per-rank MatMul of two tensors sliced on the contraction dim,
 * producing one local partial per rank ([CC] Figure 3 program, the MatMul
 * before the AllReduce).  a [M, K], b^T [N, K], c [M, N].  in_t CCE_BF16 or
 * CCE_F32; out_t CCE_BF16 or CCE_F32.  flags: CCE_FLAG_GELU.
 * ---------------------------------------------------------------------- */
cce_status cce_grouped_gemm(cce_ctx* ctx, int n_groups, cce_dtype in_t, cce_dtype out_t,
                            const void* const* a, cce_mat a_shape,
                            const void* const* b, cce_mat b_shape,
                            void* const* c, cce_mat c_shape,
                            uint32_t flags, cce_stream stream);

/* ------------------------------------------------------------------------
 * Fused reduce epilogue ([CC] Figure 3 program and its FusedAllReduce):
 *
 *   out = residual + keep * (sum_k partials[k] + bias) * c,   c = 1 / (1 - p_drop)
 *
 * in one pass: each partial, the residual and the bias are read once, the
 * output is written once, and the keep mask is generated in registers.
 * partials[k] (k < n_partials) share `shape` (rows, cols, ld) and part_t;
 * bias: [cols] of bias_t, or NULL; residual: [rows, cols] with ld_res, of
 * res_t, or NULL; out: [rows, cols] with ld_out, of out_t.  The bias and the
 * residual share the output's dtype (bias_t == res_t == out_t, else
 * CCE_EUNSUPPORTED); part_t is independent (e.g. fp32 accumulators into a
 * bf16 output).
 * Sum order: ((p0 + p1) + ...) + p_{n-1} in fp32, then + bias, then the
 * dropout scale, then + residual, each rounded to fp32, no fused
 * multiply-add; the output is rounded to nearest even once.
 * Keep mask: element (i, j) has the global index
 *   e = (mask_row0 + i) * mask_ld + (mask_col0 + j);
 * Philox4x32-10 (Salmon et al., SC'11) with counter (lo(e>>2), hi(e>>2),
 * lo(offset), hi(offset)) and key (lo(seed), hi(seed)) gives word e & 3;
 * the element is kept iff word >= floor(p_drop * 2^32).  p_drop <= 0 keeps
 * everything, p_drop >= 1 drops everything (out = residual).
 * mask_out: NULL, or a device [rows, cols] uint8 array (ld = cols) that
 * receives the keep decisions (1 kept, 0 dropped), for tests.
 * 1 <= n_partials <= CCE_MAX_RANKS.  flags: must be 0.
 * ---------------------------------------------------------------------- */
cce_status cce_fused_reduce_epilogue(cce_ctx* ctx, int n_partials, cce_dtype part_t,
                                     const void* const* partials, cce_mat shape,
                                     const void* bias, cce_dtype bias_t,
                                     const void* residual, cce_dtype res_t, int64_t ld_res,
                                     double p_drop, uint64_t seed, uint64_t offset,
                                     int64_t mask_row0, int64_t mask_col0, int64_t mask_ld,
                                     void* out, cce_dtype out_t, int64_t ld_out,
                                     uint8_t* mask_out, uint32_t flags, cce_stream stream);

/* ------------------------------------------------------------------------
 * Batched fused reduce epilogue: n_batch independent epilogues of one shape
 * in a single launch, e.g. one per rank of a ReduceScatter whose shards each
 * receive bias, dropout and residual ([CC] fused collectives: the pointwise
 * tail applied to every rank's slice of the reduced tensor).
 *
 * Output b is computed exactly as cce_fused_reduce_epilogue computes it from
 *   partials[b * n_partials + k] (k < n_partials), the shared bias,
 *   residuals[b], mask row base mask_row0[b] (shared mask_col0, mask_ld),
 *   written to outs[b] (and mask_outs[b]),
 * so results are bit-identical to n_batch single calls.  residuals and
 * mask_outs are NULL (none) or host arrays of n_batch non-NULL device
 * pointers; mask_row0 is a host array of n_batch values.
 * 1 <= n_batch, n_batch * n_partials <= CCE_MAX_RANKS.  flags: must be 0.
 * ---------------------------------------------------------------------- */
cce_status cce_fused_reduce_epilogue_batched(
    cce_ctx* ctx, int n_batch, int n_partials, cce_dtype part_t, const void* const* partials,
    cce_mat shape, const void* bias, cce_dtype bias_t, const void* const* residuals,
    cce_dtype res_t, int64_t ld_res, double p_drop, uint64_t seed, uint64_t offset,
    const int64_t* mask_row0, int64_t mask_col0, int64_t mask_ld, void* const* outs,
    cce_dtype out_t, int64_t ld_out, uint8_t* const* mask_outs, uint32_t flags,
    cce_stream stream);

/* ------------------------------------------------------------------------
 * FusedAllReduce across n_ranks logical ranks ([CC] fused collective
 * communication: an AllReduce split into ReduceScatter and AllGather, with
 * the bias add, dropout and residual add applied to each rank's reduced
 * slice in between).  partials[r] is rank r's [rows, cols] partial; every
 * outs[r] (r < n_ranks) receives the whole result
 *   residual + keep * (sum_r partials[r] + bias) * c
 * computed exactly as cce_fused_reduce_epilogue computes it (same order,
 * same mask for the given index base), so all replicas are bit-identical to
 * that call's output.  On one GPU the ranks share the HBM, so the
 * ReduceScatter, the pointwise tail and the AllGather are one pass: each
 * partial and the residual are read once and the result is stored once per
 * rank.  The residual is the one replicated tensor (NULL for none);
 * mask_out (NULL or [rows, cols] uint8) receives the keep decisions once.
 * 1 <= n_ranks <= CCE_MAX_RANKS.  flags: must be 0.
 * ---------------------------------------------------------------------- */
cce_status cce_fused_allreduce_epilogue(cce_ctx* ctx, int n_ranks, cce_dtype part_t,
                                        const void* const* partials, cce_mat shape,
                                        const void* bias, cce_dtype bias_t, const void* residual,
                                        cce_dtype res_t, int64_t ld_res, double p_drop,
                                        uint64_t seed, uint64_t offset, int64_t mask_row0,
                                        int64_t mask_col0, int64_t mask_ld, void* const* outs,
                                        cce_dtype out_t, int64_t ld_out, uint8_t* mask_out,
                                        uint32_t flags, cce_stream stream);

/* ------------------------------------------------------------------------
 * Enabling rule of [OV] Section 5.5 (host-only).  The looped form replaces a
 * collective + einsum only when it is estimated not to be slower:
 *   original_comp + original_comm >= max(original_comp, ring_comm) + epilogue
 * where original_comp / original_comm are the times of the einsum and of
 * the collective as they are, ring_comm the time of the permutes along the
 * ring, and epilogue the cost of the loop's prologue or epilogue (all in the
 * same unit, each >= 0).  Returns 1 to use the loop, 0 to keep the original,
 * -1 for a negative or NaN argument.
 *
 * cce_overlap_choose: the same section's choice between two candidate
 * collectives of one einsum.  If the einsum is estimated faster than both
 * (comp < comm0 and comp < comm1) the candidate with the smaller shard
 * (fewer bytes moved outside the loop) is chosen, else the one whose
 * collective takes longer.  Ties go to candidate 0.  Returns 0 or 1, -1 for
 * a negative or NaN argument.
 * ---------------------------------------------------------------------- */
int cce_overlap_beneficial(double original_comp, double original_comm, double ring_comm,
                           double epilogue);
int cce_overlap_choose(double comp, double comm0, double shard_bytes0, double comm1,
                       double shard_bytes1);

/* ------------------------------------------------------------------------
 * Plan description, host-only (no device, no context): writes the ordered
 * list of operations that a looped call with these arguments would enqueue,
 * one per line, into buf (NUL-terminated; *needed receives the full length
 * including the NUL).  Line format:
 *   <stream> <op> [key=value ...]
 * stream is "compute" or "copy"; op is gemm, copy, record or wait; gemm and
 * copy lines list the symbolic buffers they read (r=) and write (w=); record
 * and wait lines name an event (ev=).  kind 0 = AllGather (mode is a
 * cce_ag_mode), kind 1 = ReduceScatter, kind 2 = ReduceScatter with the fused
 * epilogue (mode is a cce_rs_mode).  With CCE_FLAG_FINE_GRAINED, the gemm
 * line of the launch that runs the chunk consumers has epi=2 and lists the
 * pairs of items that claim chunks together (pairs=i:j; a paired item stores
 * its partial at its own accumulator, named among its writes, when it claims
 * the chunk first, and the other reads it only after the ready signal).  Used
 * to check the stream/event ordering for races on the CPU.
 * ---------------------------------------------------------------------- */
cce_status cce_describe_plan(int kind, int n_ranks, int mode, cce_dtype out_t,
                             uint32_t flags, char* buf, size_t buf_len, size_t* needed);

/* ------------------------------------------------------------------------
 * Error-path test hook.  Arms a failure: plan operation `index` (1-based, in
 * the order cce_describe_plan lists them: a GEMM or epilogue launch, a copy,
 * an event record or wait) of the next looped call on this thread is not
 * enqueued; the call returns CCE_EHIP as if that HIP call had failed, with
 * cce_last_error naming the operation.  The operations before it stay
 * enqueued, and the call joins the copy stream back into `stream` before it
 * returns, so the caller's later work stays ordered after them.  The hook
 * fires once; index 0 disarms it, an index past the plan's length never
 * fires.  Returns CCE_EINVAL for a negative index.  For tests of the error
 * path and of the state a failed call leaves behind.
 * ---------------------------------------------------------------------- */
cce_status cce_debug_fail_op(int index);

/* Test hook of the fine-grained overlap's bounded wait: in the next
 * CCE_FLAG_FINE_GRAINED call on this thread, the first producer of each
 * chunk does not publish its ready word and every waiting consumer gives up
 * after at most `polls` polls, so the give-up path runs while every kernel
 * still ends normally.  polls >= 1 arms the hook (it fires once), 0 disarms
 * it, a negative value returns CCE_EINVAL. */
cce_status cce_debug_signal_giveup(int polls);

#ifdef __cplusplus
}
#endif

#endif /* CCE_H_ */
