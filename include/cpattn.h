/*
 * cpattn — one context-parallel rank's share of causal attention on MI355X (gfx950).
 *
 * C ABI of libcpattn.so.  Plain C types only: device buffers are passed as raw
 * device pointers, host tables as host pointers, the stream as an opaque
 * hipStream_t handle (void*, NULL = the null stream).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are token-major and contiguous: Q/O/dO/dQ are [T, Hq, D], K/V/dK/dV are
 *    [T, Hkv, D] (D fastest), log-sum-exp values are [T, Hq] fp32 in natural log.
 *    Positions and document ids are int32 [T].
 *  - Positions are GLOBAL token indices (the partition output); the causal rule is
 *    "key visible iff pos_k <= pos_q" (diagonal visible), plus "doc_k == doc_q" for
 *    packed documents.  Local numbering is storage only.
 *    Source: "上下文并行：一条序列跨卡，仍算同一个目标", section 01 (global j <= i);
 *    "Context Parallelism (CP)", section 5 (block-diagonal mask of packed documents).
 *  - Precondition for speed, not safety: inside each Q block and each KV segment,
 *    positions (and document ids) are non-decreasing — every partition output is.
 *    Tiles are classified empty / fully visible / partial from their first and last
 *    entries; a violated precondition gives wrong masks but never an out-of-bounds
 *    access.
 *  - Grouped queries: q head h reads kv head h / (Hq / Hkv).
 *  - The library allocates no device memory and keeps no state between calls,
 *    except the fixed per-device scratch array behind cpattn_bwd_noalloc (held from
 *    library load on).  All other device buffers belong to the caller; host arrays
 *    are read only during the call.  Work is enqueued asynchronously on `stream`; every argument the host
 *    can see is validated first, and on any error nothing is enqueued.
 *  - Outputs are overwritten, never accumulated across calls.
 *  - A row that sees no key at all gets O = 0 and LSE = -inf (never NaN).
 *  - Launch plans (work-group size, KV splits) follow the device's compute-unit
 *    count; the environment variable CPATTN_NUM_CUS (a positive integer) replaces it.
 *    A plan fixes the fp32 summation order, so results are bitwise repeatable for a
 *    given plan; different plans agree to rounding.  The order in which work-groups
 *    run does not change any result.
 *  - Status codes below; cpattn_strerror() names them.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------- */
#define CPATTN_OK 0
#define CPATTN_ERR_ARG 1          /* null pointer, negative / out-of-range size or rank */
#define CPATTN_ERR_ALIGN 2        /* length not divisible by 2*cp, cu_seqlens not monotone
                                     or not ending at total, pointer / row not 16-B aligned */
#define CPATTN_ERR_UNSUPPORTED 3  /* head dim, dtype, mask or head grouping not supported */
#define CPATTN_ERR_HIP 4          /* a HIP launch or runtime call failed */
#define CPATTN_ERR_WORKSPACE 5    /* workspace missing or smaller than required */

/* ---- enums ------------------------------------------------------------------- */
#define CPATTN_BF16 0             /* bfloat16 inputs, fp32 accumulation */
#define CPATTN_F32 1              /* float32 inputs, fp32 arithmetic throughout */

#define CPATTN_MASK_NONE 0        /* every key visible */
#define CPATTN_MASK_CAUSAL 1      /* pos_k <= pos_q */
#define CPATTN_MASK_CAUSAL_DOC 2  /* pos_k <= pos_q and doc_k == doc_q (packed documents) */

#define CPATTN_PART_ZIGZAG 0      /* one causal sequence cut into 2*cp chunks */
#define CPATTN_PART_THD 1         /* packed documents, zigzag inside every document */
#define CPATTN_PART_STRIPED 2     /* one causal sequence, rank r keeps tokens r, r+cp, r+2cp, ... */

/* Attention problem description shared by the attention calls. */
typedef struct {
  int32_t dtype;   /* CPATTN_BF16 or CPATTN_F32 (inputs Q, K, V, O, dO) */
  int32_t hq;      /* query heads (>= 1) */
  int32_t hkv;     /* key/value heads, hq % hkv == 0 */
  int32_t d;       /* head dim: 64 or 128 */
  float scale;     /* multiplies the fp32 scores; 0 means 1/sqrt(d) */
  int32_t mask;    /* CPATTN_MASK_* */
} cpattn_attn_desc;

/* A block of local queries (device pointers). */
typedef struct {
  const void* q;        /* [len, hq, d] in desc.dtype */
  const int32_t* pos;   /* [len] global positions */
  const int32_t* doc;   /* [len] document ids; may be NULL unless CPATTN_MASK_CAUSAL_DOC */
  int64_t len;          /* rows, >= 0 */
} cpattn_q_block;

/* A KV segment, e.g. one owner rank's keys/values (device pointers). */
typedef struct {
  const void* k;        /* [len, hkv, d] in desc.dtype */
  const void* v;        /* [len, hkv, d] */
  const int32_t* pos;   /* [len] global positions */
  const int32_t* doc;   /* [len] document ids; may be NULL unless CPATTN_MASK_CAUSAL_DOC */
  int64_t len;          /* rows, >= 0 */
} cpattn_kv_seg;

/* Human-readable name of a status code (static string, never NULL). */
const char* cpattn_strerror(int status);

/* Library version as 10000*major + 100*minor + patch. */
int cpattn_version(void);

/*
 * cpattn_partition — the rows one context-parallel rank holds, and their gather.
 *
 * Source: "04 · Megatron-LM 实现" (Megatron CP integration), section 1.1 (zigzag:
 * the sequence is viewed as 2*cp chunks, rank r keeps chunk r then chunk 2cp-1-r)
 * and section 1.2 with section 5 (packed THD: the same split inside every
 * document: for a document of length L at offset c, seg = L/(2cp), rows
 * c+[r*seg, (r+1)*seg) then c+[L-(r+1)*seg, L-r*seg); documents in order).
 * "推理系统基础设施（二）：Sequence Parallelism + Ring Attention", section 5, with
 * "Context Parallelism (CP)", sections 2.4 and 4 (striped: the interleaved
 * assignment [0, cp, 2cp, ...], [1, cp+1, ...], per token).
 *
 *  mode             CPATTN_PART_ZIGZAG (cu_seqlens ignored, one document [0,total)),
 *                   CPATTN_PART_THD or CPATTN_PART_STRIPED (cu_seqlens ignored).
 *  total            tokens of the full (packed) sequence; total % (2*cp) == 0
 *                   (striped: total % cp == 0).
 *  cp_size, cp_rank 1 <= cp_size, 0 <= cp_rank < cp_size.
 *  cu_seqlens_host  THD: host int32 [n_docs+1], 0 = cu[0] <= cu[1] <= ... = total,
 *                   every difference divisible by 2*cp (validated on the host).
 *  cu_seqlens_dev   THD: the same values in device memory (read by the kernel).
 *  n_docs           THD: number of documents (>= 1).
 *  idx_out          device int32 [total/cp]: global row index of each local row,
 *                   ascending; doubles as the rows' global positions.
 *  doc_out          device int32 [total/cp] document id of each local row, or NULL.
 *  n_gather         number of row tensors to gather (0..8).
 *  src, dst         host arrays of n_gather device pointers: src[g] is [total, row],
 *                   dst[g] is [total/cp, row]; dst[g][i] = src[g][idx_out[i]].
 *  row_bytes        host array of n_gather row sizes in bytes, multiples of 16;
 *                   src/dst pointers must be 16-byte aligned.
 * Errors: ARG, ALIGN (see above), HIP.  Output is bit-exact (integer work and
 * byte copies).
 */
int cpattn_partition(int32_t mode, int64_t total, int32_t cp_size, int32_t cp_rank,
                     const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                     int32_t n_docs, int32_t* idx_out, int32_t* doc_out, int32_t n_gather,
                     const void* const* src, void* const* dst, const int64_t* row_bytes,
                     void* stream);

/* Rotary embedding applied during a partition gather. */
typedef struct {
  uint32_t rotate_mask; /* bit g set: gathered tensor g is rotated; the others are copied */
  int32_t dtype;        /* element type of the rotated tensors: CPATTN_BF16 or CPATTN_F32 */
  int32_t d;            /* head dim: a multiple of 16, 16..256; a rotated row is
                           row_bytes / (element size * d) heads, each rotated alike */
  int32_t interleaved;  /* 0: pairs (x_i, x_{i+d/2}) ("rotate half"); 1: pairs (x_2i, x_2i+1) */
  float base;           /* theta_i = base^(-2i/d), i = 0 .. d/2-1; 0 means 10000 */
} cpattn_rope_desc;

/*
 * cpattn_partition_rope — cpattn_partition whose gather also applies the rotary
 * position embedding to the tensors rope->rotate_mask selects (typically Q and K).
 *
 * Source: "04 · Megatron-LM 实现", section 5: rotary embedding depends on absolute
 * positions, so the positions must be split exactly like the tokens (the zigzag
 * chunk pair; per packed document the front and mirrored slices of the frequency
 * table), and section 9's checklist: a token split and a rotary split that disagree
 * give a silently wrong loss.  "Context Parallelism (CP)", section 5: positions
 * restart at 0 in every packed document.
 *
 * Each head of a selected row at position p leaves with every pair (a, b) of its
 * elements replaced by (a cos t - b sin t, b cos t + a sin t), t = p * theta_i, where
 * p is the row's global index (zigzag, striped) or its index inside its document
 * (CPATTN_PART_THD).  The angle, its sine and cosine are computed in fp64, the
 * rotation in fp32, and the result is rounded once to the tensor's dtype (bf16:
 * round to nearest even).  Unselected tensors are copied bit for bit, as are the
 * index and document outputs.
 *
 *  rope             host pointer; every selected tensor's row_bytes must be a whole
 *                   number of heads.
 * Errors: those of cpattn_partition; ARG (rope NULL, rotate_mask naming a tensor
 * beyond n_gather, interleaved not 0/1, base negative or not finite); UNSUPPORTED
 * (dtype, d); ALIGN (a selected row not a whole number of heads).
 */
int cpattn_partition_rope(int32_t mode, int64_t total, int32_t cp_size, int32_t cp_rank,
                          const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                          int32_t n_docs, int32_t* idx_out, int32_t* doc_out, int32_t n_gather,
                          const void* const* src, void* const* dst, const int64_t* row_bytes,
                          const cpattn_rope_desc* rope, void* stream);

/*
 * cpattn_zigzag_edge_visible — whether an edge of a zigzag share's Q-KV task graph
 * holds any (query, key) pair that the causal mask keeps, so that edges without work
 * are never launched.
 *
 * Source: "Context Parallelism (CP)", section 2.1 (the task graph has an edge (i, j)
 * where KV block j holds keys visible to Q block i under the mask) and section 4
 * (zigzag: 2*cp equal chunks, rank r holds chunk r and chunk 2cp-1-r).  Positions are
 * the tokens' global indices, so within a chunk they are contiguous, and an edge has
 * work exactly when the segment's smallest key position is <= the block's largest
 * query position.
 *
 *  seq_len          tokens of the sequence: positive and a multiple of 2*cp_size.
 *  cp_size          ranks (>= 1).
 *  q_rank, kv_owner ranks holding the query block and the KV segment (0..cp_size-1).
 *  q_part, kv_part  which of that rank's chunks the block / segment holds:
 *                   0 = its front chunk (chunk rank), 1 = its back chunk
 *                   (chunk 2cp-1-rank), -1 = both (the rank's whole shard).
 *  visible          host output: 1 if the edge has work, else 0.
 * Host only (no GPU call).  Errors: ARG (sizes, ranks or parts out of range, NULL
 * output); ALIGN (seq_len not a multiple of 2*cp_size).
 */
int cpattn_zigzag_edge_visible(int64_t seq_len, int32_t cp_size, int32_t q_rank, int32_t q_part,
                               int32_t kv_owner, int32_t kv_part, int32_t* visible);

/*
 * cpattn_tile_fwd — TileAttention over a batch of independent (Q block, KV segment)
 * edges of the Q-KV task graph.
 *
 * Source: "Context Parallelism (CP)", section 2.1: each edge (i, j) is an
 * independent task producing the partial state A_ij = (O_ij, L_ij), where L_ij is
 * the per-row log-sum-exp of the masked, scaled scores Q_i K_j^T and O_ij is the
 * output normalised inside segment j only.
 *
 *  n_edges          number of edges (0 is a no-op); launched 20 edges at a time.
 *  q_blocks, segs   host arrays [n_edges]: the edge's queries and its KV segment.
 *  o_parts          host array [n_edges] of device fp32 [q.len, hq, d] outputs O_ij.
 *  lse_parts        host array [n_edges] of device fp32 [q.len, hq] outputs L_ij.
 *  workspace        device buffer (256-byte aligned) of workspace_bytes, or NULL.
 *                   With at least cpattn_tile_fwd_workspace_bytes() bytes, an edge
 *                   whose query tiles alone leave the GPU underfilled has its visible
 *                   KV tiles split over several work-groups whose partial states are
 *                   merged into O_ij (the same associative merge as cpattn_merge);
 *                   with less (or NULL) every query tile runs in one work-group.
 *                   Packed-document launches (CPATTN_MASK_CAUSAL_DOC, head groups a
 *                   multiple of 8) with many rounds of work-groups, or more than 1024
 *                   query tiles, use it instead for a plan built once by one
 *                   work-group: the order of their query tiles by work (up to 4096
 *                   query tiles; without a workspace 1024) and the KV tile table.
 *                   The planned launch runs the same work items and gives the same
 *                   results bit for bit.  Contents on entry are ignored; the results
 *                   do not depend on it beyond floating-point rounding.
 * Rows of a block that see nothing of the segment get (0, -inf).
 * Errors: ARG, UNSUPPORTED (d not 64/128, hq % hkv, dtype, mask), HIP.
 */
int cpattn_tile_fwd(const cpattn_attn_desc* desc, int32_t n_edges,
                    const cpattn_q_block* q_blocks, const cpattn_kv_seg* segs,
                    float* const* o_parts, float* const* lse_parts, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes that let cpattn_tile_fwd split the edges' KV ranges over more
 * work-groups when the edges alone cannot fill the GPU (0: no split planned, or
 * invalid arguments).  The plan depends on the arguments and the current device. */
size_t cpattn_tile_fwd_workspace_bytes(const cpattn_attn_desc* desc, int32_t n_edges,
                                       const cpattn_q_block* q_blocks, const cpattn_kv_seg* segs);

/*
 * cpattn_merge — the associative log-sum-exp merge of partial states.
 *
 * Source: "Context Parallelism (CP)", section 2.2: L_i = log sum_j exp(L_ij) and
 * O_i = sum_j exp(L_ij - L_i) O_ij; any order and grouping gives the same result
 * up to rounding.  Parts whose L is -inf contribute nothing; a row whose parts are
 * all -inf becomes (0, -inf).
 *
 *  n_parts          1..64.
 *  o_parts          host array [n_parts] of device fp32 [rows, hq, d].
 *  lse_parts        host array [n_parts] of device fp32 [rows, hq].
 *  out_dtype        CPATTN_BF16 (round to nearest even) or CPATTN_F32 for o_out.
 *  o_out            device [rows, hq, d]; lse_out device fp32 [rows, hq].
 * Errors: ARG, UNSUPPORTED (d not a multiple of 4 up to 256), HIP.
 */
int cpattn_merge(int32_t n_parts, const float* const* o_parts, const float* const* lse_parts,
                 int64_t rows, int32_t hq, int32_t d, int32_t out_dtype, void* o_out,
                 float* lse_out, void* stream);

/*
 * cpattn_merge_groups — several independent cpattn_merge calls in one launch (or as
 * few as the launch arguments allow), for example the merges of all query chunks of a
 * rank after a batch of tile edges.  Same source and arithmetic as cpattn_merge: each
 * group's result is bit-identical to cpattn_merge on that group alone.
 *
 *  n_groups         number of groups (0 is a no-op).
 *  n_parts          host array [n_groups], each 1..64.
 *  o_parts          host array [sum of n_parts] of device fp32 [rows[g], hq, d]: group
 *                   g's parts follow those of groups 0 .. g-1.
 *  lse_parts        host array [sum of n_parts] of device fp32 [rows[g], hq], same order.
 *  rows             host array [n_groups] (a group with 0 rows is skipped; its buffers
 *                   are not read and may be NULL).
 *  out_dtype        CPATTN_BF16 or CPATTN_F32 for every o_out[g].
 *  o_out, lse_out   host arrays [n_groups] of device [rows[g], hq, d] and fp32
 *                   [rows[g], hq] outputs.
 * Errors: ARG, ALIGN (16-byte aligned O buffers), UNSUPPORTED (as cpattn_merge), HIP.
 */
int cpattn_merge_groups(int32_t n_groups, const int32_t* n_parts, const float* const* o_parts,
                        const float* const* lse_parts, const int64_t* rows, int32_t hq, int32_t d,
                        int32_t out_dtype, void* const* o_out, float* const* lse_out, void* stream);

/*
 * cpattn_stream_fwd — the streaming online-softmax form over KV segments in
 * arrival order (the ring loop of one rank, with the other ranks' segments given
 * as local buffers).
 *
 * Source: "上下文并行：一条序列跨卡，仍算同一个目标", section 02 (per row:
 * m' = max(m, max_B S), c = e^{m-m'}, l' = c l + sum_B e^{S-m'},
 * a' = c a + sum_B e^{S-m'} V, O = a / l, lambda = m + log l) and
 * "推理系统基础设施（二）：Sequence Parallelism + Ring Attention", section 2
 * (Q stays, KV blocks arrive one by one, the running max/sum/output are updated).
 *
 *  q                the local query block.
 *  n_segs, segs     host array of KV segments in arrival order (1..2048).  A launch
 *                   streams up to 32 segments; a longer list runs as groups of 32, each
 *                   streamed into an fp32 partial state in the workspace, merged by
 *                   log-sum-exp at the end (needs cpattn_stream_fwd_workspace_bytes()
 *                   bytes, else CPATTN_ERR_WORKSPACE; no KV split then).
 *  o_out            device [q.len, hq, d] in desc.dtype (final output O).
 *  lse_out          device fp32 [q.len, hq] (lambda, natural log).
 *  workspace        as for cpattn_tile_fwd (cpattn_stream_fwd_workspace_bytes()): when
 *                   the query tiles cannot fill the GPU, each query tile's visible KV
 *                   tiles (in arrival order) are cut into consecutive runs, each run
 *                   keeps its own running (m, l, a) state, and the runs' partial states
 *                   are merged by log-sum-exp — the pool form of the same computation.
 * Errors: ARG, ALIGN, UNSUPPORTED, HIP.
 */
int cpattn_stream_fwd(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                      const cpattn_kv_seg* segs, void* o_out, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes for the KV-split plan of cpattn_stream_fwd (0: no split planned), or
 * for the per-group partial states of a list of more than 32 segments. */
size_t cpattn_stream_fwd_workspace_bytes(const cpattn_attn_desc* desc, const cpattn_q_block* q,
                                         int32_t n_segs, const cpattn_kv_seg* segs);

/*
 * cpattn_bwd — LSE-replay backward of one rank's share.
 *
 * Source: "上下文并行：一条序列跨卡，仍算同一个目标", sections 01-02: the local
 * probabilities are rebuilt from the full-row LSE and output, P_ij = exp(S_ij -
 * lambda_i); then dQ, dK, dV of every block follow from the softmax derivative,
 * dK_j = sum_i dS_ij Q_i / sqrt(d), dV_j = sum_i P_ij G_i, and the K/V gradient
 * contributions of all local queries are summed per owner (per segment here).
 *
 *  q, segs          as for cpattn_stream_fwd (bf16 only in this version; 1..2048
 *                   segments; beyond 32 segments the dQ pass runs unsplit, one launch
 *                   per group of 32 adding its part, and the dK/dV pass one launch per
 *                   group).
 *  o                device [q.len, hq, d] forward output (desc.dtype).
 *  lse              device fp32 [q.len, hq] forward log-sum-exp.
 *  dout             device [q.len, hq, d] upstream gradient G (desc.dtype).
 *  dq               device fp32 [q.len, hq, d] output.
 *  dk, dv           host arrays [n_segs] of device fp32 [segs[s].len, hkv, d] outputs:
 *                   the summed contribution of all local queries (and all query
 *                   heads of a group) to segment s's keys and values.
 *  workspace        256-byte aligned device buffer, at least q.len * hq * 4 bytes
 *                   (rounded up to 256); cpattn_bwd_workspace_bytes() bytes enable the
 *                   split dQ pass.  Contents on entry are ignored.
 * Computed as two passes without atomics — the calls below, in this order:
 * cpattn_bwd_dq_delta (which forms the per-row values into the start of the
 * workspace) with the rest of the workspace, then cpattn_bwd_dkdv.
 * Errors: ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
int cpattn_bwd(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
               const cpattn_kv_seg* segs, const void* o, const float* lse, const void* dout,
               float* dq, float* const* dk, float* const* dv, void* workspace,
               size_t workspace_bytes, void* stream);

/* Bytes of device workspace for cpattn_bwd (0 on invalid arguments): the per-row
 * rowsum(dO * O) values, plus room for the dQ pass to split its KV tiles over more
 * work-groups when the local queries alone cannot fill the GPU, or for its plan
 * (see cpattn_bwd_dq).  A workspace that
 * only holds the first part (q.len * hq * 4 bytes, rounded up to 256) is accepted
 * and runs the dQ pass unsplit. */
size_t cpattn_bwd_workspace_bytes(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                                  const cpattn_kv_seg* segs);

/*
 * The passes of cpattn_bwd as separate calls, for callers that schedule them
 * around communication: D once per backward, then per arriving KV segment the
 * dK/dV pass (whose result can go back to the segment's owner at once) and the dQ
 * pass.  Running cpattn_bwd_delta, cpattn_bwd_dq and cpattn_bwd_dkdv over the same
 * arguments gives exactly the outputs of cpattn_bwd, and so does cpattn_bwd_dq_delta
 * followed by cpattn_bwd_dkdv.  Same source as cpattn_bwd.
 */

/* cpattn_bwd_delta — D_i = sum_d G_i * O_i per (row, head), the term the softmax
 * derivative subtracts from dP (dS = P (dP - D)).
 *  rows             local query rows (>= 0); 0 is a no-op.
 *  o, dout          device [rows, hq, d] bf16 forward output and upstream gradient
 *                   (16-byte aligned).
 *  delta            device fp32 [rows, hq] output.
 * Errors: ARG, ALIGN, UNSUPPORTED (fp32 inputs), HIP. */
int cpattn_bwd_delta(const cpattn_attn_desc* desc, int64_t rows, const void* o, const void* dout,
                     float* delta, void* stream);

/* cpattn_bwd_dq — dQ_i = scale * sum_j dS_ij K_j over every visible key of the
 * segments, with P and dP rebuilt per key tile (query-major pass).
 *  q, n_segs, segs  as for cpattn_bwd.
 *  lse, delta       device fp32 [q.len, hq]: forward log-sum-exp and cpattn_bwd_delta.
 *  dout             device [q.len, hq, d] bf16 upstream gradient.
 *  dq               device fp32 [q.len, hq, d] output.
 *  workspace        NULL, or a 256-byte aligned device buffer; with
 *                   cpattn_bwd_dq_workspace_bytes() bytes the KV tiles of each query
 *                   tile are split over more work-groups when the queries alone cannot
 *                   fill the GPU (fp32 partial sums, added in a second launch), or
 *                   a packed-document launch is planned once as for cpattn_tile_fwd;
 *                   a smaller buffer runs unsplit and unplanned.  Contents on entry
 *                   are ignored.
 * Errors: ARG, ALIGN, UNSUPPORTED, HIP. */
int cpattn_bwd_dq(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                  const cpattn_kv_seg* segs, const float* lse, const float* delta, const void* dout,
                  float* dq, void* workspace, size_t workspace_bytes, void* stream);

/* cpattn_bwd_dq_delta — cpattn_bwd_dq that forms D_i = sum_d G_i * O_i itself from
 * the forward output and the dO rows it loads anyway, and stores it for
 * cpattn_bwd_dkdv: the values equal cpattn_bwd_delta's bit for bit (same products,
 * added in the same pairs), and dq equals what cpattn_bwd_dq gives with them.
 *  o                device [q.len, hq, d] bf16 forward output (16-byte aligned).
 *  delta            device fp32 [q.len, hq] output.
 *  the rest         as for cpattn_bwd_dq (lse, dout, dq, workspace, stream).
 * Errors: ARG, ALIGN, UNSUPPORTED, HIP. */
int cpattn_bwd_dq_delta(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                        const cpattn_kv_seg* segs, const void* o, const float* lse, const void* dout,
                        float* delta, float* dq, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes that let cpattn_bwd_dq split (0: no split planned or invalid arguments). */
size_t cpattn_bwd_dq_workspace_bytes(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                                     const cpattn_kv_seg* segs);

/* cpattn_bwd_dkdv — per segment s: dV_s = sum_i P_is^T G_i and dK_s = scale *
 * sum_i dS_is^T Q_i over all local query rows i (and all query heads of each kv
 * head's group): the contribution this rank returns to the owner of segment s.
 * One launch, key-major.
 *  q, n_segs, segs  as for cpattn_bwd.
 *  lse, delta, dout as for cpattn_bwd_dq.
 *  dk, dv           as for cpattn_bwd.
 * Errors: ARG, ALIGN, UNSUPPORTED, HIP. */
int cpattn_bwd_dkdv(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                    const cpattn_kv_seg* segs, const float* lse, const float* delta, const void* dout,
                    float* const* dk, float* const* dv, void* stream);

/*
 * cpattn_bwd_noalloc — cpattn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, rules, outputs and errors as cpattn_bwd, without the
 * workspace: the call uses a device array inside the library of
 * CPATTN_NOALLOC_SCRATCH_BYTES bytes, one per device, held from library load until
 * the process ends, and allocates nothing itself.
 *  - The array of the current device is used; `stream` must belong to that device.
 *  - Inputs whose per-row values (q.len * hq * 4 bytes, rounded up to 256) exceed
 *    the array return CPATTN_ERR_WORKSPACE; when the dQ pass's split plan does not
 *    fit beside them, the pass runs unsplit (results agree to rounding).
 *  - Every call on a device shares that device's array, which keeps the last call's
 *    contents: calls that overlap in time on one device (other streams, other host
 *    threads) race and must be serialised by the caller.
 */
#define CPATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int cpattn_bwd_noalloc(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                       const cpattn_kv_seg* segs, const void* o, const float* lse, const void* dout,
                       float* dq, float* const* dk, float* const* dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
