/*
 * cam.h -- C ABI of the per-GPU hot path of sequence/context-parallel attention
 * movement on MI355X (gfx950): the Ulysses all-to-all relayout, the
 * max/sum-aware LSE pack and the stable LSE-weighted combine.
 *
 * Sources (web pages, cited by title and section):
 *  [FV] FastVideo compare view "[perf] Probe H3 chunked all-to-all with direct
 *       output slices": ulysses_a2a.py (fused all-to-all: output identical to
 *       the collective's, with less traffic through local memory),
 *       benchmark_ulysses_a2a.py (all_to_all_4D(x, 2, 1) on the scatter
 *       operand [3, S/P, H, 128]; (1, 2) on the gather operand [1, S, H/P, 128]).
 *  [VA] vllm-ascend PR "[Performance][Attention] Fuse local SFA LSE formation
 *       into DCP pack": "What this PR does / why we need it?" and "How was this
 *       patch tested?".
 *  [CU] cuLA PR "feat(distributed): add packed hybrid runtime and THD planner":
 *       packed THD batches described by cu_seqlens, logical context-parallel
 *       ranks emulated in one process.
 *
 * Conventions common to every call
 *  - The P logical ranks of one exchange live in one GPU's memory; the
 *    all-to-all between them is the relayout itself (no peer traffic).
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    retains a pointer; all device pointers must stay valid until the enqueued
 *    work has finished on `stream`.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work: no host synchronisation, no device-to-host read, no allocation, so
 *    every call may be captured in a HIP graph.
 *  - Every argument is validated before anything is launched.  On failure the
 *    call returns a non-zero cam_status, records a message readable with
 *    cam_last_error() (thread-local), launches nothing and writes nothing.
 *  - Inputs and outputs must not overlap (CAM_ERR_OVERLAP).
 *  - Device pointers must be aligned to the element size; the kernels then
 *    pick the widest access (16, 8, 4 or 2 bytes) that the sizes, strides and
 *    pointer alignment allow.
 *  - No C++ exception crosses this boundary.  A failed launch returns
 *    CAM_ERR_HIP with the HIP error text in cam_last_error().
 */
#ifndef CAM_H
#define CAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cam_dtype {
    CAM_BF16 = 0, /* bfloat16 payload */
    CAM_FP16 = 1, /* IEEE binary16 payload */
    CAM_FP32 = 2, /* 4-byte words (relayouts only; used for index payloads) */
    /* Not dtypes: they widen the enumeration to every 32-bit code a caller
     * can pass, so that an unknown code is a well-defined value that the
     * validation rejects (CAM_ERR_UNSUPPORTED). */
    CAM_DTYPE_RANGE_MIN_ = INT32_MIN,
    CAM_DTYPE_RANGE_MAX_ = INT32_MAX
} cam_dtype;

typedef enum cam_status {
    CAM_OK = 0,
    CAM_ERR_NULL = 1,         /* a required pointer is NULL */
    CAM_ERR_SHAPE = 2,        /* a size is negative, or a size product overflows */
    CAM_ERR_DIVISIBILITY = 3, /* S, H or T not divisible by P where the layout needs it */
    CAM_ERR_ALIGNMENT = 4,    /* pointer or stride not a multiple of the element size */
    CAM_ERR_OVERLAP = 5,      /* an output overlaps an input */
    CAM_ERR_UNSUPPORTED = 6,  /* dtype, scatter_dim or P outside what the call supports */
    CAM_ERR_HIP = 7           /* the HIP runtime rejected the launch */
} cam_status;

/* Name of a status code (static string). */
const char* cam_status_string(cam_status s);

/* Detail of the last failed call on this thread ("" after a success). */
const char* cam_last_error(void);

/* ABI version of this header (incremented on any signature change). */
#define CAM_ABI_VERSION 1
int cam_abi_version(void);

/* Geometry of the latest kernel launched by this thread: workgroups, threads
 * per workgroup and dynamic LDS bytes (all zero before the first launch; a
 * call that launches nothing leaves the previous record).  For profilers and
 * benchmarks, which match a call to its kernel dispatches by grid size. */
cam_status cam_last_launch(uint64_t* workgroups, uint32_t* threads, uint64_t* lds_bytes);

/* ------------------------------------------------------------------------- */
/* Dense Ulysses relayout  ([FV] all_to_all_4D, benchmark_ulysses_a2a.py)      */
/* ------------------------------------------------------------------------- */
/*
 * Sequence-sharded side  seq[j][b][s][h][d]:  [P][B][S/P][H][D], rank j holds
 *   tokens [j*S/P, (j+1)*S/P) of each of the B planes (B = 3 carries Q, K, V).
 * Head-sharded side      head[r][b][t][h'][d]: [P][B][S][H/P][D], rank r holds
 *   heads [r*H/P, (r+1)*H/P) for all S tokens, tokens in source-rank order.
 *
 * ulysses_seq_to_head:  head[r][b][j*S/P + s][h'][d] = seq[j][b][s][r*H/P + h'][d]
 *   (all_to_all_4D scatter dim 2, gather dim 1: attention input Q, K, V).
 * ulysses_head_to_seq:  the inverse (scatter dim 1, gather dim 2: attention
 *   output O back to sequence shards).
 *
 * Elements are copied as bits (dt only sets the element size: 2 bytes for
 * CAM_BF16 / CAM_FP16, 4 for CAM_FP32).  Requires P >= 1, S % P == 0,
 * H % P == 0 (CAM_ERR_DIVISIBILITY).  Any of B, S, H, D may be 0 (no work).
 * `in` and `out` are device buffers of B*S*H*D elements each.
 * Limits (CAM_ERR_UNSUPPORTED beyond them): P and B below 2^32; one head block
 * of one row ((H/P)*D elements) and one (source rank, plane, destination
 * rank) slab below 2^31 access vectors; at most 2^32 tiles.
 */
cam_status ulysses_seq_to_head(const void* in, void* out, int64_t P, int64_t B, int64_t S,
                               int64_t H, int64_t D, cam_dtype dt, void* stream);
cam_status ulysses_head_to_seq(const void* in, void* out, int64_t P, int64_t B, int64_t S,
                               int64_t H, int64_t D, cam_dtype dt, void* stream);

/* ------------------------------------------------------------------------- */
/* Varlen (packed THD, cu_seqlens) relayout  ([CU] cu_seqlens shard offsets)   */
/* ------------------------------------------------------------------------- */
/*
 * A packed batch of nseq sequences: sequence i is global tokens
 * [cu_seqlens[i], cu_seqlens[i+1]) of length L_i, total T = cu_seqlens[nseq].
 * Each sequence is cut into P pieces; piece p is the in-sequence positions
 * [floor(p*L_i/P), floor((p+1)*L_i/P)) and lives on logical rank p.  Rank p
 * stores its pieces in sequence order: T_p tokens, slab [B][T_p][H][D] at token
 * offset R_p = T_0 + ... + T_{p-1} of a rank-major buffer (element offset
 * B*R_p*H*D).  With nseq = 1 and P | T this is exactly the dense layout.
 *
 * ulysses_varlen_plan (host only, no GPU call): from the host copy of
 *   cu_seqlens (nseq+1 int32, non-decreasing, cu_seqlens[0] = 0) fills
 *   rank_cu[p*(nseq+1) + i] = tokens of rank p before sequence i
 *   (rank_cu[p*(nseq+1) + nseq] = T_p) and rank_off[p] = R_p (rank_off[P] = T).
 *   Both arrays are caller-allocated host memory.
 *
 * ulysses_seq_to_head_varlen: rank-major ragged [B*T][H][D] -> head-sharded
 *   [P][B][T][H/P][D] (global packed token order).
 * ulysses_head_to_seq_varlen: the inverse.
 *   cu_seqlens, rank_cu, rank_off are DEVICE copies of the plan above and
 *   total_tokens = T is passed by the host (nothing is read back).  A plan that
 *   does not match cu_seqlens is not detected on the device; rows whose
 *   computed source or destination falls outside the buffers are skipped, so
 *   a malformed plan cannot make the kernel access out of bounds.
 *   Requires H % P == 0; T and nseq must fit int32 (CAM_ERR_SHAPE).  Limits
 *   (CAM_ERR_UNSUPPORTED beyond them): P and B below 2^32; one head block of
 *   one row and one (rank, plane) below 2^31 access vectors; at most 2^32
 *   tiles.
 */
cam_status ulysses_varlen_plan(const int32_t* cu_seqlens_host, int64_t nseq, int64_t P,
                               int32_t* rank_cu_host, int64_t* rank_off_host);
cam_status ulysses_seq_to_head_varlen(const void* in, void* out, const int32_t* cu_seqlens,
                                      const int32_t* rank_cu, const int64_t* rank_off,
                                      int64_t nseq, int64_t total_tokens, int64_t P, int64_t B,
                                      int64_t H, int64_t D, cam_dtype dt, void* stream);
cam_status ulysses_head_to_seq_varlen(const void* in, void* out, const int32_t* cu_seqlens,
                                      const int32_t* rank_cu, const int64_t* rank_off,
                                      int64_t nseq, int64_t total_tokens, int64_t P, int64_t B,
                                      int64_t H, int64_t D, cam_dtype dt, void* stream);

/* ------------------------------------------------------------------------- */
/* THD layout planner and planned relayout  ([CU] PR description: per-rank    */
/* work that grows with tokens and with causal position kept even; a short    */
/* sample stays on one rank; long sequences are dealt out in a direction that */
/* flips from rank to rank; several grids tried, the plain contiguous layout  */
/* kept as a candidate; equal aligned blocks per rank; a repeatable span list) */
/* ------------------------------------------------------------------------- */
typedef struct cam_thd_planner_config {
    int64_t block_size;          /* every length and min_split_tokens a multiple of it */
    int64_t min_split_tokens;    /* shorter samples are short (kept whole when they fit) */
    int64_t max_chunks_per_rank; /* planned candidates above it per rank are dropped */
    double token_weight;         /* cost of a token at position k:               */
    double causal_weight;        /*   token_weight + causal_weight * (k + 1)      */
    int64_t mode;                /* 0: best of the grids and the contiguous layout; 1: contiguous */
} cam_thd_planner_config;

/*
 * thd_plan (host only, no HIP call): plan the packed batch cu_seqlens[nseq+1]
 * over world_size ranks.  Rank r holds exactly floor((r+1)N/W) - floor(rN/W)
 * of the N aligned blocks.  Candidates: the contiguous layout, and for
 * g = 1..6 a grid that places the short samples whole (costliest first,
 * cheapest rank with room), deals each long sequence's W * 2^(g-1) chunks along
 * a snake whose direction alternates per round and per long sequence, then
 * moves the highest-position blocks of overfull ranks to the cheapest ranks
 * with room and lays shorts that fitted nowhere into the remaining room.  The
 * least maximum rank cost wins (ties: fewer spans, then the lower candidate).
 * Output, in packed token order: span_start[n+1] (first token of each span,
 * span_start[n] = T), span_rank[n], span_local[n] (first row in the rank's
 * slab, which lists the rank's spans in packed order), rank_off[W+1] (slab
 * token offsets), rank_cost[W] and *chosen (0 = contiguous, else the grid).
 * Tables are caller-owned host memory of max_spans (+1) entries; *n_spans is
 * set even when they are too small (CAM_ERR_SHAPE, nothing else written).
 * Errors: CAM_ERR_UNSUPPORTED (world_size < 1, non-positive sizes, weights
 * negative, non-finite or both zero), CAM_ERR_ALIGNMENT (a length or
 * min_split_tokens not a multiple of block_size), CAM_ERR_SHAPE (malformed
 * cu_seqlens, fewer blocks than ranks), CAM_ERR_NULL.
 */
cam_status thd_plan(const int32_t* cu_seqlens, int64_t nseq, int64_t world_size,
                    const cam_thd_planner_config* cfg, int64_t max_spans, int32_t* span_start,
                    int32_t* span_rank, int32_t* span_local, int64_t* rank_off, double* rank_cost,
                    int64_t* n_spans, int32_t* chosen);

/*
 * ulysses_seq_to_head_spans: the varlen relayout over a THD layout plan.  The
 *   sequence side is rank-major: rank p's slab [B][T_p][H][D] at token row
 *   B*rank_off[p], its rows being its spans in packed order; the head side is
 *   [P][B][T][H/P][D] in packed token order.  Token t of span s is row
 *   span_local[s] + t - span_start[s] of rank span_rank[s]'s slab.
 * ulysses_head_to_seq_spans: the inverse.
 *   span_start[n_spans+1], span_rank, span_local (int32) and rank_off[P+1]
 *   (int64) are DEVICE copies of thd_plan's tables for world_size = P;
 *   total_tokens = span_start[n_spans] is passed by the host.  Rows a
 *   malformed table would place outside the buffers are skipped.  H % P == 0.
 */
/*
 * thd_plan_first_positions (host only): first_pos[p * nseq + i] = the
 *   smallest position of sequence i held by rank p under the plan's spans
 *   (INT32_MAX if none), for the planned combine.  first_pos has world_size *
 *   nseq entries, caller-owned host memory.  CAM_ERR_SHAPE if a span lies
 *   outside the batch or the ranks.
 */
cam_status thd_plan_first_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t world_size,
                                    const int32_t* span_start, const int32_t* span_rank,
                                    int64_t n_spans, int32_t* first_pos);

cam_status ulysses_seq_to_head_spans(const void* in, void* out, const int32_t* span_start,
                                     const int32_t* span_rank, const int32_t* span_local,
                                     const int64_t* rank_off, int64_t n_spans, int64_t total_tokens,
                                     int64_t P, int64_t B, int64_t H, int64_t D, cam_dtype dt,
                                     void* stream);
cam_status ulysses_head_to_seq_spans(const void* in, void* out, const int32_t* span_start,
                                     const int32_t* span_rank, const int32_t* span_local,
                                     const int64_t* rank_off, int64_t n_spans, int64_t total_tokens,
                                     int64_t P, int64_t B, int64_t H, int64_t D, cam_dtype dt,
                                     void* stream);

/* ------------------------------------------------------------------------- */
/* Max/sum-aware LSE pack  ([VA] "What this PR does": the LSE is computed     */
/* inside the pack, so no separate fp32 LSE tensor is written beforehand)     */
/* ------------------------------------------------------------------------- */
/*
 * Inputs, for each source rank p < P (decode context parallel: rank p holds the
 * attention of every query over its share of the KV):
 *   out  [P][T][H][Dv] payload (CAM_BF16 / CAM_FP16), element strides o_sp,
 *        o_st, o_sh, Dv contiguous;
 *   smax, ssum  [P][T][H] fp32 softmax max and sum, element strides free.
 * LSE = smax + log(ssum) (natural log, fp32 result); a non-finite smax, a
 * non-finite ssum or ssum <= 0 (including -0.0 and NaN) gives -inf.
 *
 * Packed exchange layout: chunk (p, r) = what source p sends to destination r:
 *   scatter_dim = 1 (heads):  rows = T*(H/P), row q = t*(H/P) + h' carries
 *                             (t, head r*H/P + h');  requires H % P == 0;
 *   scatter_dim = 0 (tokens): rows = (T/P)*H, row q = t'*H + h carries
 *                             (token r*T/P + t', h); requires T % P == 0.
 *   chunk = O-region [rows][Dv] payload bits, padded to 16 bytes, then the
 *   L-region [rows] fp32, padded to 16 bytes.  Buffer = [P_src][P_dst][chunk],
 *   lse_pack_bytes() bytes.  Padding bytes are not written.
 * The O-region is a bit copy of `out`; the L-region is the LSE.
 *
 * lse_pack_bytes returns the packed buffer size in bytes, or -1 for invalid
 * arguments (the reason is in cam_last_error()).
 *
 * Limits (CAM_ERR_UNSUPPORTED beyond them): P < 65536; rows per chunk below
 * 2^31; one row, and one chunk's O-region, below 2^31 access vectors; P*P
 * chunks of tiles below 2^32 tiles.
 */
int64_t lse_pack_bytes(int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim,
                       cam_dtype dt);
cam_status lse_pack(const void* out, int64_t o_sp, int64_t o_st, int64_t o_sh,
                    const float* smax, int64_t m_sp, int64_t m_st, int64_t m_sh,
                    const float* ssum, int64_t s_sp, int64_t s_st, int64_t s_sh,
                    int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim, cam_dtype dt,
                    void* packed, void* stream);

/* ------------------------------------------------------------------------- */
/* Stable LSE-weighted combine  ([VA] "What this PR does": the PR keeps its    */
/* combine unchanged and feeds it -inf for invalid statistics; rows with no     */
/* valid partial)                                                               */
/* ------------------------------------------------------------------------- */
/*
 * Per output row, over the partials p < P in ascending order:
 *   V = {p : L_p finite};  M = max_{p in V} L_p;  w_p = exp(L_p - M);
 *   Z = sum w_p;  out = (sum_{p in V} w_p * O_p) / Z;  lse_out = M + log(Z).
 * If V is empty: out = +0.0 in every element and lse_out = -inf (no NaN).
 * The O row of a partial outside V is never read.  Arithmetic is fp32; the
 * output is rounded to the payload dtype (round to nearest even).
 *
 * lse_combine_packed: destination rank r combines the chunks (p, r) of every
 *   source p of a buffer written by lse_pack with the same P, T, H, Dv,
 *   scatter_dim, dt (the all-to-all is a strided view, no bytes move).  Output
 *   row r*rows + q: `out` is [P*rows][Dv] (= [P][T][H/P][Dv] for scatter_dim 1,
 *   [T][H][Dv] for scatter_dim 0); `lse_out` [P*rows] fp32 or NULL.
 *
 * lse_combine: generic strided form for P partials over rows (t, h):
 *   part_out (p, t, h, d) at element p*po_sp + t*po_st + h*po_sh + d;
 *   part_lse (p, t, h)    at element p*pl_sp + t*pl_st + h*pl_sh;
 *   out (t, h, d) at t*o_st + h*o_sh + d; lse_out (t, h) at t*lo_st + h*lo_sh
 *   (lse_out may be NULL).
 *
 * lse_combine_varlen: lse_combine for a packed THD batch whose P partials are
 *   the attention of each token over the P KV pieces of its own sequence
 *   (pieces as in the varlen relayout) under a causal mask: partial p of token
 *   t (position k of its sequence) is admitted only if piece p is non-empty and
 *   starts at or before k; otherwise neither its LSE nor its O row is read.
 *   cu_seqlens is a DEVICE array of nseq+1 int32; total_tokens = T.
 *
 * Limits of every combine entry point (lse_combine*, and their _seq, _planned
 * and _backward forms): 1 <= P <= 64 (a row's partials are reduced across
 * one wave; CAM_ERR_UNSUPPORTED above); T*H below 2^31 rows and one row
 * below 2^31 access vectors (CAM_ERR_UNSUPPORTED); strides non-negative; the
 * varlen and planned forms need nseq >= 1 and T < 2^31.
 */
cam_status lse_combine_packed(const void* packed, int64_t P, int64_t T, int64_t H, int64_t Dv,
                              int scatter_dim, cam_dtype dt, void* out, float* lse_out,
                              void* stream);
cam_status lse_combine(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                       const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                       int64_t P, int64_t T, int64_t H, int64_t D, cam_dtype dt, void* out,
                       int64_t o_st, int64_t o_sh, float* lse_out, int64_t lo_st, int64_t lo_sh,
                       void* stream);
cam_status lse_combine_varlen(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                              const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                              int64_t P, int64_t T, int64_t H, int64_t D, cam_dtype dt, void* out,
                              int64_t o_st, int64_t o_sh, float* lse_out, int64_t lo_st,
                              int64_t lo_sh, const int32_t* cu_seqlens, int64_t nseq,
                              void* stream);

/* ------------------------------------------------------------------------- */
/* Combine straight into the sequence-sharded layout ([FV] "direct output      */
/* slices": write the destination slices directly instead of a further pass)  */
/* ------------------------------------------------------------------------- */
/*
 * lse_combine_packed_seq: lse_combine_packed whose output rows go straight to
 *   token-major order, out [T][H][Dv] and lse_out [T][H] (nullable): the row of
 *   destination rank r for (t, head r*H/P + h') lands at (t, r*H/P + h').  This
 *   is the combine followed by ulysses_head_to_seq of its result, in one pass.
 *   For scatter_dim = 0 it writes what lse_combine_packed writes.
 *
 * lse_combine_varlen_seq: lse_combine_varlen whose combined token rows land in
 *   the rank-major (sequence-sharded) order of the varlen relayout: the token
 *   at local row l of rank p goes to row R_p + l of out [T][H][D] and lse_out
 *   [T][H] (both contiguous; lse_out nullable).  cu_seqlens, rank_cu and
 *   rank_off are the DEVICE copies of ulysses_varlen_plan's tables for the same
 *   P (the P partials are the P KV pieces, as in lse_combine_varlen).
 */
/*
 * lse_combine_planned: lse_combine_varlen for a batch laid out by a THD layout
 *   plan (context parallelism in which rank p holds the queries and keys of
 *   its spans): partial p of the token at position k of sequence i is the
 *   causal attention over the keys rank p holds of sequence i, admitted iff
 *   first_pos[p * nseq + i] <= k (thd_plan_first_positions; DEVICE copy, P
 *   = world_size); masked partials are not read.  For the per-sequence split
 *   it gives what lse_combine_varlen gives.
 */
cam_status lse_combine_planned(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                               const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                               int64_t P, int64_t T, int64_t H, int64_t D, cam_dtype dt, void* out,
                               int64_t o_st, int64_t o_sh, float* lse_out, int64_t lo_st, int64_t lo_sh,
                               const int32_t* cu_seqlens, const int32_t* first_pos, int64_t nseq,
                               void* stream);

cam_status lse_combine_packed_seq(const void* packed, int64_t P, int64_t T, int64_t H, int64_t Dv,
                                  int scatter_dim, cam_dtype dt, void* out, float* lse_out,
                                  void* stream);
cam_status lse_combine_varlen_seq(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                                  const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                                  int64_t P, int64_t T, int64_t H, int64_t D, cam_dtype dt, void* out,
                                  float* lse_out, const int32_t* cu_seqlens, const int32_t* rank_cu,
                                  const int64_t* rank_off, int64_t nseq, void* stream);

/* ------------------------------------------------------------------------- */
/* Online two-way merge for ring / context-parallel accumulation ([CU] ring    */
/* transport of the logical-CP emulation; [VA] stable combine semantics)       */
/* ------------------------------------------------------------------------- */
/*
 * lse_merge: per row (t, h) the accumulator (acc_out fp32 [T][H][D], acc_lse
 *   fp32 [T][H]) becomes the stable combine of itself and one partial
 *   (part_out [T][H][D] payload dt, part_lse fp32 [T][H]):
 *     M = max of the finite LSEs; w = exp(L - M) for each finite one;
 *     acc_out = (w_a*acc_out + w_b*part_out) / (w_a + w_b);
 *     acc_lse = M + log(w_a + w_b).
 *   An accumulator whose LSE is not finite is empty (its payload is ignored,
 *   so it may start uninitialised with acc_lse = -inf); if both are invalid the
 *   row becomes +0 with -inf LSE.  An invalid partial's row is never read.
 *   Merging the P partials of a row one hop at a time gives their one-shot
 *   combine (the combine is associative); the accumulator stays fp32 between
 *   hops.  out_final (nullable, payload dt [T][H][D]) also receives the
 *   rounded result, for the last hop.  All strides are in elements (D
 *   contiguous); D % 4 == 0; accumulator rows 16-byte and payload rows 8-byte
 *   aligned.  Updates in place; no buffer may overlap another.  T*H must be
 *   below 2^31 rows, D/4 below 2^31 and every stride non-negative
 *   (CAM_ERR_UNSUPPORTED).
 */
cam_status lse_merge(float* acc_out, int64_t a_st, int64_t a_sh, float* acc_lse, int64_t al_st,
                     int64_t al_sh, const void* part_out, int64_t p_st, int64_t p_sh,
                     const float* part_lse, int64_t pl_st, int64_t pl_sh, int64_t T, int64_t H,
                     int64_t D, cam_dtype dt, void* out_final, int64_t f_st, int64_t f_sh,
                     void* stream);

/* ------------------------------------------------------------------------- */
/* Training: gradient of the combine ([CU] forward and backward comparison of  */
/* context parallelism; [FV] benchmark training pair).  The gradient of a      */
/* relayout is the inverse relayout (ulysses_head_to_seq for            */
/* ulysses_seq_to_head and the other way round, the same for varlen).          */
/* ------------------------------------------------------------------------- */
/*
 * lse_combine_backward: the gradient of lse_combine.  For each row (t, h), with
 *   V the valid partials (finite LSE), w_p = exp(L_p - lse_out) their
 *   normalised weights (formed as in the forward), g the upstream gradient of
 *   out[t][h][:] and g_lse that of lse_out[t][h]:
 *     d_part_out[p][t][h][:] = w_p * g                        (p in V)
 *     d_part_lse[p][t][h]    = w_p * (<g, O_p> - sum_{q in V} w_q <g, O_q> + g_lse)
 *   and exact zeros for p outside V (an empty V gives zeros throughout).  The
 *   O row of a partial outside V is never read.  fp32 arithmetic; d_part_out
 *   rounded to the payload dtype (RNE), d_part_lse fp32.
 * Layouts (element strides, D contiguous): part_out, part_lse as in
 *   lse_combine; g_out (t, h, d) at go_st*t + go_sh*h + d, payload dt;
 *   g_lse (t, h) fp32 at gl_st*t + gl_sh*h, nullable (then zero);
 *   d_part_out (p, t, h, d) at dpo_sp*p + dpo_st*t + dpo_sh*h + d, payload dt;
 *   d_part_lse (p, t, h) at dpl_sp*p + dpl_st*t + dpl_sh*h, fp32.
 *   Every element of both gradients is written.  1 <= P <= 64; T*H < 2^31.
 *   Outputs may overlap neither an input nor each other.
 *
 * lse_combine_varlen_backward: the gradient of lse_combine_varlen (the causal
 *   piece rule decides V: a masked partial gets zero gradient and is not read).
 */
cam_status lse_combine_backward(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                                const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                                int64_t P, int64_t T, int64_t H, int64_t D, cam_dtype dt,
                                const void* g_out, int64_t go_st, int64_t go_sh, const float* g_lse,
                                int64_t gl_st, int64_t gl_sh, void* d_part_out, int64_t dpo_sp,
                                int64_t dpo_st, int64_t dpo_sh, float* d_part_lse, int64_t dpl_sp,
                                int64_t dpl_st, int64_t dpl_sh, void* stream);
cam_status lse_combine_varlen_backward(const void* part_out, int64_t po_sp, int64_t po_st,
                                       int64_t po_sh, const float* part_lse, int64_t pl_sp,
                                       int64_t pl_st, int64_t pl_sh, int64_t P, int64_t T, int64_t H,
                                       int64_t D, cam_dtype dt, const void* g_out, int64_t go_st,
                                       int64_t go_sh, const float* g_lse, int64_t gl_st, int64_t gl_sh,
                                       void* d_part_out, int64_t dpo_sp, int64_t dpo_st,
                                       int64_t dpo_sh, float* d_part_lse, int64_t dpl_sp,
                                       int64_t dpl_st, int64_t dpl_sh, const int32_t* cu_seqlens,
                                       int64_t nseq, void* stream);

/* lse_combine_planned_backward: the gradient of lse_combine_planned (layouts
 * and rules of lse_combine_backward, admission of lse_combine_planned). */
cam_status lse_combine_planned_backward(const void* part_out, int64_t po_sp, int64_t po_st,
                                        int64_t po_sh, const float* part_lse, int64_t pl_sp,
                                        int64_t pl_st, int64_t pl_sh, int64_t P, int64_t T, int64_t H,
                                        int64_t D, cam_dtype dt, const void* g_out, int64_t go_st,
                                        int64_t go_sh, const float* g_lse, int64_t gl_st,
                                        int64_t gl_sh, void* d_part_out, int64_t dpo_sp,
                                        int64_t dpo_st, int64_t dpo_sh, float* d_part_lse,
                                        int64_t dpl_sp, int64_t dpl_st, int64_t dpl_sh,
                                        const int32_t* cu_seqlens, const int32_t* first_pos,
                                        int64_t nseq, void* stream);

/* ------------------------------------------------------------------------- */
/* Q/K/V projection into the head-sharded layout  ([FV] "direct output        */
/* slices": the producer of the scatter operand writes the destination slices) */
/* ------------------------------------------------------------------------- */
/*
 * qkv_projection_head_sharded: out[r][b][t][h'][d] =
 *   sum_k x[t][k] * w[(b*H + r*H/P + h')*D + d][k], i.e. the projection x w^T
 *   written where ulysses_seq_to_head would put it, so that relayout's pass
 *   over Q/K/V is not needed.
 *   x [S][K]: the P ranks' sequence shards stacked in token order (rank j's
 *   rows are j*S/P .. (j+1)*S/P - 1); w [B*H*D][K]: the fused weight in a
 *   linear layer's layout (rows ordered b, h, d); out [P][B][S][H/P][D]; all
 *   contiguous, payload dt (bf16 or fp16) for all three.  fp32 accumulation
 *   on the matrix cores, rounded to dt (RNE).  Requires K a positive multiple
 *   of 64, B*H*D a multiple of 256, H % P == 0; x and w 16-byte aligned.
 */
cam_status qkv_projection_head_sharded(const void* x, const void* w, void* out, int64_t S, int64_t K,
                                       int64_t P, int64_t B, int64_t H, int64_t D, cam_dtype dt,
                                       void* stream);

/* ------------------------------------------------------------------------- */
/* Measurement helper                                                          */
/* ------------------------------------------------------------------------- */
/*
 * cam_ablation_seq_to_head_lds: what ulysses_seq_to_head computes (same
 *   arguments and layouts), by a different kernel kept only to measure the
 *   choice against it: each workgroup stages rows_per_tile whole
 *   sequence-side rows (all H heads) in LDS and writes every head block's rows
 *   as one contiguous run (the "LDS-staged transpose" of the head/sequence
 *   swap).  ulysses_seq_to_head does not call it.  16-byte accesses only: (H/P)*D*esize and both pointers must be
 *   multiples of 16 bytes (CAM_ERR_ALIGNMENT); rows_per_tile >= 1 with
 *   rows_per_tile*H*D*esize <= 64 KiB, and B below 2^32 (CAM_ERR_UNSUPPORTED).
 *   Other errors as ulysses_seq_to_head.
 */
cam_status cam_ablation_seq_to_head_lds(const void* in, void* out, int64_t P, int64_t B, int64_t S,
                                        int64_t H, int64_t D, cam_dtype dt, int64_t rows_per_tile,
                                        void* stream);

/*
 * cam_copy: plain 16-byte-vector device copy of `bytes` bytes (src and dst
 * 16-byte aligned, bytes % 16 == 0, no overlap) with the same launch shape as
 * the relayout kernels.  It is the achievable-copy ceiling measured beside
 * every relayout ([FV] profile_ulysses_mfu.py times a plain dst.copy_ next to
 * each all-to-all) and the known-size reference for hardware byte counters.
 */
cam_status cam_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CAM_H */
