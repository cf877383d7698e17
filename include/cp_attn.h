/*
 * cp_attn.h - one context-parallel rank's share of packed variable-length
 * ("thd") causal attention with ring (P2P) KV exchange, on one MI355X (gfx950).
 *
 * The pages this follows (cited by title and section):
 *  [I1]  "thd format is not supported with hierarchical CP implementation yet"
 *        (Transformer Engine issue 2208): packed THD sequences, the P2P ring
 *        and the a2a / a2a+p2p communication types; P2P suits long sequences
 *        because the ring exchange can hide under compute.
 *  [I2]  "[PyTorch][Attention] THD P2P context-parallel regression when padded
 *        cu_seqlens are value-equal but not object-identical" (Transformer
 *        Engine issue 3487), sections "Describe the bug", "Steps/Code to
 *        reproduce bug" and "Expected behavior": cu_seqlens / padded
 *        cu_seqlens, the automatic pad_between_seqs decision (which must be
 *        taken from values, not object identity), per-rank sequence lengths
 *        recomputed per ring step, THD dQ/dK/dV tail zeroing that should only
 *        run when a tail exists, and graph-safe padding metadata.
 *  [I3]  "Hybrid / Hierarchical Context Parallel Skill", sections
 *        "Enablement" and "Code Anchors": every sequence length must divide
 *        by 2*CP; hierarchical sizes are [a2a size, p2p size] whose product is
 *        CP.
 *
 * Conventions used by every entry point:
 *  - Pointers are DEVICE pointers unless the comment says "host".
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - bf16 tensors are row-major [rows, heads, head_dim]; a rank's local
 *    tensors hold t_alloc >= T_local rows (T_local = cu_seqlens_padded[B]/CP).
 *  - LSE is the natural-log log-sum-exp of the scaled scores, fp32, laid out
 *    [heads, t_alloc] (head-major).
 *  - Local row layout of rank r (and of every KV shard s, with s in place of
 *    r): sequence b occupies local rows [cup[b]/CP, cup[b+1]/CP); the first
 *    half of that slot is chunk r of the sequence's 2*CP chunks and the second
 *    half is chunk 2*CP-1-r (the load-balanced pairing). Valid tokens fill
 *    chunks in order; padding sits at the end of a sequence's padded slot.
 *  - Every call returns a cp_attn_status. On failure nothing further is
 *    launched and cp_attn_last_error() (thread-local) describes the cause.
 *    Faults of earlier asynchronous work surface as CP_ATTN_ERR_HIP.
 *  - Caller owns every tensor and workspace; the library owns only the
 *    cp_attn_meta handle (device tables plus a pinned summary).
 */
#ifndef CP_ATTN_H_
#define CP_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CP_ATTN_OK = 0,
  CP_ATTN_ERR_INVALID_ARG = 1,   /* bad sizes / pointers / layout rules */
  CP_ATTN_ERR_UNSUPPORTED = 2,   /* e.g. head_dim not 64/128, non-causal */
  CP_ATTN_ERR_HINT_MISMATCH = 3, /* pad_hint contradicts the values */
  CP_ATTN_ERR_WORKSPACE = 4,     /* workspace missing or too small */
  CP_ATTN_ERR_HIP = 5            /* a HIP runtime call failed */
} cp_attn_status;

#define CP_ATTN_MAX_CP 16
/* Most sequences per batch that cp_attn_rank_metadata_host accepts. */
#define CP_ATTN_HOST_META_MAX_B 255

/* Opaque per-batch metadata handle (device tables + host summary). */
typedef struct cp_attn_meta cp_attn_meta;

/* Host-side summary of a metadata handle. step_kind[i]: 0 = own shard, causal
 * on local rows; 1 = source shard s < rank: all query rows x the first half of
 * shard s, no mask; 2 = s > rank: second-half query rows x all of shard s, no
 * mask. step_src[i] = (rank - i) mod CP. tiles_* are the per-step work-item
 * counts of the forward / dQ kernels and of the dK/dV kernel. */
typedef struct {
  int32_t B, cp_size, cp_rank;
  int32_t pad_between_seqs; /* 1 iff cu_seqlens != cu_seqlens_padded anywhere (by value) */
  int32_t t_local;          /* cu_seqlens_padded[B] / CP */
  int32_t has_tail;         /* 1 iff t_alloc > t_local */
  int64_t t_alloc;
  int32_t step_kind[CP_ATTN_MAX_CP];
  int32_t step_src[CP_ATTN_MAX_CP];
  int64_t tiles_fwd[CP_ATTN_MAX_CP];
  int64_t tiles_dkdv[CP_ATTN_MAX_CP];
  int64_t valid_rows;       /* valid (non-padding) local rows of this rank */
} cp_attn_summary;

/*
 * Build rank cp_rank's per-batch metadata on the device (one small kernel
 * group, then ONE host synchronisation of `stream` to read back a <1 KB
 * summary; the only synchronisation in the library). The summary lands in a
 * pinned host buffer that each calling thread keeps per device until the
 * process ends. [I2] "Describe the bug": the per-step
 * per-rank cu_seqlens; [I2] "Expected behavior": the padding decision is
 * taken from values only - the library never compares pointers, so an
 * aliased, NULL or distinct-but-equal cu_seqlens_padded all yield identical
 * tables and the same kernel sequence. [I3] "Enablement": padded lengths must
 * divide by 2*CP.
 *
 *  cu_seqlens         device int32 [B+1], cu[0] = 0, non-decreasing (valid lengths)
 *  cu_seqlens_padded  device int32 [B+1] (padded lengths); may alias cu_seqlens;
 *                     NULL means "no padding" (= cu_seqlens)
 *  B                  number of sequences, >= 1
 *  cp_size, cp_rank   ring size (1..CP_ATTN_MAX_CP) and this rank
 *  pad_hint           -1 = decide from the values; 0 / 1 = caller asserts
 *                     no padding / padding; a contradiction with the values
 *                     returns CP_ATTN_ERR_HINT_MISMATCH
 *  t_alloc            rows allocated in this rank's local tensors (>= T_local)
 *  out                receives the handle (free with cp_attn_meta_free)
 * Device-side checks (reported after the sync): cu[0] = cup[0] = 0, both
 * non-decreasing, 0 <= L_b <= P_b, P_b % (2*CP) == 0, t_alloc >= T_local.
 */
cp_attn_status cp_attn_rank_metadata(const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded,
                                     int32_t B, int32_t cp_size, int32_t cp_rank, int32_t pad_hint,
                                     int64_t t_alloc, void* stream, cp_attn_meta** out);

/*
 * cp_attn_rank_metadata from host copies of the same arrays, with no
 * synchronisation: the summary and every validation check are computed on
 * the host (the same arithmetic, so the same tables, summary, status and
 * message), and the values travel to the device in the table kernel's launch
 * arguments, so nothing the caller owns is read after the call returns. For
 * a caller that holds the batch's cu_seqlens on the host (a data loader
 * builds them there): the per-step host wait of the device path disappears
 * and the next kernels queue straight behind the metadata kernels.
 *
 *  cu_seqlens, cu_seqlens_padded  HOST int32 [B+1] (padded: NULL = none);
 *                     conditions and pad_hint as in cp_attn_rank_metadata
 *  B                  1 .. CP_ATTN_HOST_META_MAX_B, else CP_ATTN_ERR_UNSUPPORTED
 *  stream             the metadata kernels run on it; later calls with the
 *                     handle must be ordered after them (same stream, or an
 *                     event)
 * Other arguments: as cp_attn_rank_metadata.
 */
cp_attn_status cp_attn_rank_metadata_host(const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded, int32_t B,
                                          int32_t cp_size, int32_t cp_rank, int32_t pad_hint, int64_t t_alloc,
                                          void* stream, cp_attn_meta** out);

/* Copy the host summary (no device work). */
cp_attn_status cp_attn_meta_summary(const cp_attn_meta* m, cp_attn_summary* out);

/*
 * Export the integer tables to a host buffer (synchronous device->host copy;
 * for tests and tooling). Layout, all int32, in this order:
 *   header[8] = {B, CP, rank, pad_between_seqs, T_local, has_tail, n_steps=CP, 0}
 *   chunk[B]                       c_b = P_b / (2 CP)
 *   cu_padded_local[B+1]           cup / CP
 *   cu_padded_half[B+1]            cup / (2 CP)
 *   for s in 0..CP-1: cu_full_s[B+1], cu_first_s[B+1], cu_second_s[B+1]
 *                                  exclusive prefix sums of the valid rows of
 *                                  shard s (both chunks / first / second chunk)
 *   for i in 0..CP-1: {kind, src}, q_start[B], q_len[B], kv_start[B], kv_len[B]
 *                                  step i's query and key row ranges in local rows
 * n is the capacity of host_buf in int32 elements; *n_needed receives the
 * required count (call with host_buf = NULL to query).
 */
cp_attn_status cp_attn_meta_export(const cp_attn_meta* m, int32_t* host_buf, size_t n, size_t* n_needed);

/* Release the handle (synchronises the device it was built on). Its device
 * table buffer goes back to a per-device pool (at most 64 buffers, kept until
 * the process ends) from which later handles take theirs, so steady-state
 * metadata builds allocate nothing. NULL is a no-op. */
void cp_attn_meta_free(cp_attn_meta* m);

/* Workspace bytes needed by cp_attn_fwd (pass 0: one fp32 output accumulator
 * and LSE plane, 4 * (hq * d + hq) * T_local bytes rounded up) or cp_attn_bwd
 * (pass 1: two fp32 planes of hq * T_local); 0 for a NULL handle or
 * non-positive sizes. */
size_t cp_attn_workspace_bytes(const cp_attn_meta* m, int32_t hq, int32_t hkv, int32_t d, int32_t pass);

/*
 * Forward of the rank's share: for ring step i = 0..CP-1 the step's query
 * rows attend to the step's key rows of shard s = (rank - i) mod CP (flash-
 * style MFMA kernels, causal on local rows at step 0 only), and the per-step
 * partial outputs are folded through their log-sum-exp. [I1] the P2P ring;
 * [I2] "Describe the bug": per-step metadata. When every step's own launch
 * would be short (under four waves of two blocks per compute unit) all steps
 * run in one launch whose blocks carry the online softmax across the steps
 * (the fold applied tile by tile in registers; the workspace is not
 * touched); otherwise the steps run in order, one launch each, each folding
 * its normalised partial into the workspace's accumulator in its epilogue.
 * Everything runs on `stream`.
 *
 *  q                  bf16 [t_alloc, hq, d]: this rank's query rows
 *  k_shards, v_shards HOST arrays of CP device pointers, bf16 [t_alloc, hkv, d];
 *                     entry s is the shard of rank s (entry rank = own K/V)
 *  hq, hkv, d         heads (hq % hkv == 0; query head h uses KV head h/(hq/hkv)),
 *                     head_dim in {64, 128}
 *  softmax_scale      multiplies q.k (usually 1/sqrt(d))
 *  causal             must be 1
 *  out                bf16 [t_alloc, hq, d]: rows [0, T_local) written; padding
 *                     rows are 0; rows >= T_local untouched
 *  lse                fp32 [hq, t_alloc]: natural-log LSE, padding rows -inf,
 *                     columns >= T_local untouched
 *  workspace          device scratch of cp_attn_workspace_bytes(m, .., 0) bytes
 * Never synchronises; capturable in a HIP graph.
 */
cp_attn_status cp_attn_fwd(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                           const void* const* v_shards, int32_t hq, int32_t hkv, int32_t d,
                           float softmax_scale, int32_t causal, void* out, float* lse,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * Backward of the rank's share: the gradient of sum(dout * out) with respect
 * to this rank's queries (dq) and to every source shard's keys and values
 * (dk_parts[s], dv_parts[s]: the contribution of this rank's query rows only,
 * in shard s's local layout; in a real ring these are what travels back).
 * THD gradient tail zeroing ([I2] "Describe the bug" and "Expected
 * behavior"): rows [T_local, t_alloc) of dq and of every part are zeroed by
 * one extra launch, made only when the metadata shows such a tail exists.
 * Launches: one that computes D = rowsum(dout * out), one for the dK/dV of
 * every ring step (each step writes its own part), one for the dQ of every
 * step (each query tile sums its steps in registers and writes bf16 dQ
 * once), one that zeroes dQ's padding rows when the share has any, and the
 * tail zeroing. When the dQ launch is short the dK/dV launch runs on a side
 * stream forked from `stream` beside it and is joined back before the call
 * returns its work to `stream`.
 *
 *  q, k_shards, v_shards, hq, hkv, d, softmax_scale, causal: as cp_attn_fwd
 *  out, lse           the forward's outputs
 *  dout               bf16 [t_alloc, hq, d]
 *  dq                 bf16 [t_alloc, hq, d] (overwritten; padding rows 0)
 *  dk_parts, dv_parts HOST arrays of CP device pointers, bf16 [t_alloc, hkv, d]
 *                     (overwritten; rows outside the step's key range 0)
 *  workspace          device scratch of cp_attn_workspace_bytes(m, .., 1) bytes
 * Never synchronises; capturable in a HIP graph.
 */
cp_attn_status cp_attn_bwd(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                           const void* const* v_shards, const void* out, const float* lse,
                           const void* dout, int32_t hq, int32_t hkv, int32_t d, float softmax_scale,
                           int32_t causal, void* dq, void* const* dk_parts, void* const* dv_parts,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * cp_attn_bwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture that may not call hipMalloc, tight
 * serving loops, harnesses that forbid allocation). The backward's only
 * scratch (two fp32 planes per query head and local row: 8 * hq * T_local
 * bytes) comes from a fixed device array of 32 MiB that every GPU the
 * library runs on holds until the process ends; the call makes no
 * allocation of any kind, and it never forks (everything runs on `stream`).
 * Calls that overlap on one GPU race on that array: order them (one stream,
 * or events). Errors: as cp_attn_bwd, and CP_ATTN_ERR_WORKSPACE (before any
 * launch) when 8 * hq * T_local exceeds 32 MiB, with the sizes in
 * cp_attn_last_error(). Other arguments and results: as cp_attn_bwd.
 */
cp_attn_status cp_attn_bwd_noalloc(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                                   const void* const* v_shards, const void* out, const float* lse, const void* dout,
                                   int32_t hq, int32_t hkv, int32_t d, float softmax_scale, int32_t causal,
                                   void* dq, void* const* dk_parts, void* const* dv_parts, void* stream);

/*
 * Data-loader helper: gather the rows that rank `shard` holds out of a global
 * packed tensor (rows in cu_seqlens_padded order) into that rank's local
 * layout (see the conventions above). row_bytes = heads * head_dim * element
 * size, a multiple of 16. `global` has cu_seqlens_padded[B] rows; `local` has
 * T_local rows (rows >= T_local are not touched). [I3] "Enablement" (2*CP
 * chunks) with the load-balanced pairing of chunks k and 2*CP-1-k.
 */
cp_attn_status cp_attn_shard_gather(const cp_attn_meta* m, int32_t shard, const void* global,
                                    void* local, size_t row_bytes, void* stream);

/*
 * One rank's share under all-gather context parallelism ([I3] "Implementation
 * Map": "all_gather" is one of the cp_comm_type values). Reading (the pages
 * name the type and nothing more): every rank first holds the gathered K/V of
 * the whole packed batch, computes its own query chunks against it, and its
 * contribution to the gradient of every gathered key row is what a
 * reduce-scatter across ranks would then sum. The attended pairs are the ring
 * share's, so these calls gather the shard views out of the gathered K/V (an
 * HBM-bound permutation into the workspace), run the ring-step kernels of
 * cp_attn_fwd / cp_attn_bwd, and the backward scatters the per-shard dK/dV
 * parts back to gathered rows (a permutation: each gathered row belongs to one
 * shard).
 *
 *  m                  metadata of this rank (cp_attn_rank_metadata)
 *  q, out, lse, dout, dq   this rank's local tensors, as for cp_attn_fwd/bwd
 *  k_full, v_full     gathered K / V, bf16 [cu_seqlens_padded[B], hkv, d] in
 *                     packed (cu_seqlens_padded) order, 16-byte aligned
 *  dk_full, dv_full   bf16 [cu_seqlens_padded[B], hkv, d] (overwritten: every
 *                     row [0, cu_seqlens_padded[B]) is written; rows of keys
 *                     no query of this rank reaches, and padding rows, are 0;
 *                     rows past cu_seqlens_padded[B] are not touched)
 *  workspace          device scratch of cp_attn_ag_workspace_bytes(m, hq, hkv,
 *                     d, pass) bytes (pass 0 forward, 1 backward), 256-byte
 *                     aligned: the shard views (and gradient parts) of t_alloc
 *                     rows each, then the ring steps' own workspace
 * Other arguments and errors as cp_attn_fwd / cp_attn_bwd. Never
 * synchronises; capturable in a HIP graph.
 */
size_t cp_attn_ag_workspace_bytes(const cp_attn_meta* m, int32_t hq, int32_t hkv, int32_t d, int32_t pass);
cp_attn_status cp_attn_ag_fwd(const cp_attn_meta* m, const void* q, const void* k_full, const void* v_full,
                              int32_t hq, int32_t hkv, int32_t d, float softmax_scale, int32_t causal, void* out,
                              float* lse, void* workspace, size_t ws_bytes, void* stream);
cp_attn_status cp_attn_ag_bwd(const cp_attn_meta* m, const void* q, const void* k_full, const void* v_full,
                              const void* out, const float* lse, const void* dout, int32_t hq, int32_t hkv, int32_t d,
                              float softmax_scale, int32_t causal, void* dq, void* dk_full, void* dv_full,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * The all-to-all of one a2a group of hierarchical (a2a + p2p) context
 * parallelism, played on one device. [I3] "Enablement" and "Implementation
 * Map": CP = a2a size x p2p size and every padded length divides by 2*CP;
 * [I1]: THD with the a2a and hierarchical communication types is what the
 * reference lacks. Reading: the a2a groups are runs of consecutive CP ranks
 * (CP rank c = p * a2a_size + a), so group p's chunks are exactly p2p rank
 * p's load-balanced chunk pair when each sequence is cut into 2 * (CP /
 * a2a_size) chunks. The row mapping is the same for every group.
 *
 *  m           metadata built with cp_size = CP (any rank): its device tables
 *              and its validation of the 2*CP divisibility are used
 *  a2a_size    A, dividing CP; p2p_rank: the group p (< CP / A)
 *  heads       heads per row (a multiple of A); head_bytes: bytes of one head
 *              (head_dim * element size), a multiple of 16
 * cp_attn_a2a_seq_to_head:
 *  in          HOST array of A device pointers: entry a = CP rank p*A + a's
 *              local tensor, [>= T_local, heads, head_bytes] (its layout per
 *              the conventions above; rows >= T_local are not read)
 *  out         HOST array of A device pointers: entry a' receives heads
 *              [a' heads/A, (a'+1) heads/A) of p2p rank p's local rows,
 *              [A * T_local, heads/A, head_bytes] (per sequence: CP chunks
 *              pA .. pA+A-1, then their mirrors, 2CP-1-(pA+A-1) .. 2CP-1-pA)
 * cp_attn_a2a_head_to_seq: the inverse (the gradients' way back), in/out
 *              with the roles above swapped.
 * T_local = cu_seqlens_padded[B] / CP. Never synchronises; capturable.
 */
cp_attn_status cp_attn_a2a_seq_to_head(const cp_attn_meta* m, int32_t a2a_size, int32_t p2p_rank, int32_t heads,
                                       int32_t head_bytes, const void* const* in, void* const* out, void* stream);
cp_attn_status cp_attn_a2a_head_to_seq(const cp_attn_meta* m, int32_t a2a_size, int32_t p2p_rank, int32_t heads,
                                       int32_t head_bytes, const void* const* in, void* const* out, void* stream);

/*
 * One rank share as a single HIP graph launch. [I2] "Describe the bug"
 * attributes the reference's lost time to gaps between many small launches
 * on the main stream, and "Expected behavior" asks for padding metadata that
 * stays valid under graph capture. The metadata is built once per batch
 * (cp_attn_rank_metadata synchronises once and is not capturable); then the
 * launches of cp_attn_fwd and/or cp_attn_bwd, with exactly these arguments,
 * are captured on a private stream into an instantiated graph, and every
 * cp_attn_graph_launch replays the whole share in one launch.
 *
 *  m, and the tensor / size / scale arguments: as cp_attn_fwd and cp_attn_bwd
 *                     (dout, dq, dk_parts, dv_parts, ws_bwd are ignored when
 *                     passes == 1; ws_fwd when passes == 2; lse and out are
 *                     the forward's outputs and the backward's inputs)
 *  passes             1 = forward, 2 = backward, 3 = forward then backward
 *  out_graph          receives the library-owned graph handle
 * The graph keeps the device pointers and sizes it was captured with (the
 * host pointer arrays are read during capture only): every buffer must stay
 * allocated, unmoved and of the same size while the graph is replayed, and
 * `m` must not be freed before the graph. Each replay reads the inputs'
 * contents at the time it runs. Errors found while capturing are returned as
 * by cp_attn_fwd / cp_attn_bwd and leave no graph.
 */
typedef struct cp_attn_graph cp_attn_graph;

cp_attn_status cp_attn_graph_capture(const cp_attn_meta* m, int32_t passes, const void* q,
                                     const void* const* k_shards, const void* const* v_shards, int32_t hq,
                                     int32_t hkv, int32_t d, float softmax_scale, int32_t causal, void* out,
                                     float* lse, const void* dout, void* dq, void* const* dk_parts,
                                     void* const* dv_parts, void* ws_fwd, size_t ws_fwd_bytes, void* ws_bwd,
                                     size_t ws_bwd_bytes, cp_attn_graph** out_graph);

/* Replay the captured share on `stream` (one graph launch; never synchronises). */
cp_attn_status cp_attn_graph_launch(const cp_attn_graph* g, void* stream);

/* Number of kernel launches the graph holds (host, no device work). */
int64_t cp_attn_graph_kernels(const cp_attn_graph* g);

/* Release the graph (waits for the device to finish its replays). NULL is a no-op. */
void cp_attn_graph_free(cp_attn_graph* g);

/*
 * Kernel timing (measurement tooling, not on the numerical path). While
 * enabled, every kernel launched by cp_attn_fwd / cp_attn_bwd is bracketed by
 * a pair of HIP events recorded on its launch stream (so the timing includes
 * nothing but that stream's work between the two records). Launches made
 * while their stream is being captured into a graph are not recorded.
 * Recording is not thread-safe: enable it only while a single thread calls
 * the library (a benchmarking thread); with recording off, calls from any
 * number of threads are unaffected.
 * cp_attn_timing_enable(1) clears earlier records and starts recording;
 * cp_attn_timing_enable(0) stops recording.
 * cp_attn_timing_read waits for the recorded events and fills up to `max`
 * entries: names (each in a `name_len`-byte slot of `names`, host buffer of
 * max * name_len bytes, NUL-terminated), the summed duration in milliseconds
 * and the launch count per kernel; returns the number of distinct kernels
 * (or -1 on a HIP error) and clears the records.
 */
cp_attn_status cp_attn_timing_enable(int32_t on);
int32_t cp_attn_timing_read(char* names, int32_t name_len, double* total_ms, int64_t* launches, int32_t max);

/*
 * Attainable bf16 matrix-unit rate (measurement tooling, not on the numerical
 * path): one launch of independent v_mfma_f32_32x32x16_bf16 chains on register
 * operands that rotate through pseudo-random bf16 values (so operand bits
 * toggle as with real data), two 256-thread blocks per compute unit of the
 * current device, `iters` products per chain (rounded up to a multiple of 8),
 * timed with HIP events on `stream` (the call waits for it). Reports the
 * launch's milliseconds and its dense bf16 TFLOP/s: the rate the matrix unit
 * sustains on data at the clock the device holds under its power limit. `sink`: device float, written only in a case that
 * cannot occur (keeps the products live). Errors: CP_ATTN_ERR_INVALID_ARG for
 * iters <= 0 or a NULL pointer, CP_ATTN_ERR_HIP for a failed launch.
 */
cp_attn_status cp_attn_mfma_probe(int32_t iters, float* sink, void* stream, double* ms, double* tflops);

/* Thread-local description of the last failure ("" if none). */
const char* cp_attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CP_ATTN_H_ */
