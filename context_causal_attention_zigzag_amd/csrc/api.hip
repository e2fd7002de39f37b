// C ABI of libcpattn.so: argument validation and kernel launches.
//
// Every check the host can make without touching device memory happens before any
// work is enqueued; on error the call returns a status and enqueues nothing.
// Calls are asynchronous on the given stream and keep no state between calls.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "../../include/cpattn.h"

#include "common.h"

using namespace cpattn;

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 30;
// Segments per call; a launch takes kMaxSegs of them, longer lists run as groups (at
// most 64: the parts of one merge launch).
constexpr int kMaxSegsTotal = 64 * kMaxSegs;

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

int seg_groups(int n_segs) { return (n_segs + kMaxSegs - 1) / kMaxSegs; }

// Workspace of a streaming forward over more than kMaxSegs segments: one fp32 partial
// state (O and LSE) per group of segments, merged at the end.
size_t grouped_stream_bytes(const cpattn_attn_desc* desc, int64_t q_len, int n_segs) {
  if (n_segs <= kMaxSegs) return 0;
  const size_t o = round256((size_t)q_len * desc->hq * desc->d * sizeof(float));
  const size_t l = round256((size_t)q_len * desc->hq * sizeof(float));
  return (size_t)seg_groups(n_segs) * (o + l);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_desc(const cpattn_attn_desc* d) {
  if (d == nullptr) return CPATTN_ERR_ARG;
  if (d->hq < 1 || d->hkv < 1) return CPATTN_ERR_ARG;
  if (!(std::isfinite(d->scale)) || d->scale < 0.0f) return CPATTN_ERR_ARG;
  if (d->dtype != CPATTN_BF16 && d->dtype != CPATTN_F32) return CPATTN_ERR_UNSUPPORTED;
  if (d->d != 64 && d->d != 128) return CPATTN_ERR_UNSUPPORTED;
  if (d->hq % d->hkv != 0) return CPATTN_ERR_UNSUPPORTED;
  if (d->mask < CPATTN_MASK_NONE || d->mask > CPATTN_MASK_CAUSAL_DOC) return CPATTN_ERR_UNSUPPORTED;
  return CPATTN_OK;
}

int check_qblock(const cpattn_attn_desc* d, const cpattn_q_block* q) {
  if (q == nullptr) return CPATTN_ERR_ARG;
  if (q->len < 0 || q->len > kMaxRows) return CPATTN_ERR_ARG;
  if (q->len == 0) return CPATTN_OK;
  if (q->q == nullptr || q->pos == nullptr) return CPATTN_ERR_ARG;
  if (d->mask == CPATTN_MASK_CAUSAL_DOC && q->doc == nullptr) return CPATTN_ERR_ARG;
  if (!aligned16(q->q)) return CPATTN_ERR_ALIGN;
  return CPATTN_OK;
}

int check_seg(const cpattn_attn_desc* d, const cpattn_kv_seg* s) {
  if (s->len < 0 || s->len > kMaxRows) return CPATTN_ERR_ARG;
  if (s->len == 0) return CPATTN_OK;
  if (s->k == nullptr || s->v == nullptr || s->pos == nullptr) return CPATTN_ERR_ARG;
  if (d->mask == CPATTN_MASK_CAUSAL_DOC && s->doc == nullptr) return CPATTN_ERR_ARG;
  if (!aligned16(s->k) || !aligned16(s->v)) return CPATTN_ERR_ALIGN;
  return CPATTN_OK;
}

float eff_scale(const cpattn_attn_desc* d) {
  return d->scale > 0.0f ? d->scale : 1.0f / std::sqrt((float)d->d);
}

int heads_per_wg(int group) { return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1); }

void fill_common(FwdArgs& a, const cpattn_attn_desc* d) {
  a.hq = d->hq;
  a.hkv = d->hkv;
  a.group = d->hq / d->hkv;
  a.heads_per_wg = heads_per_wg(a.group);
  a.mask = d->mask;
  a.scale_log2 = eff_scale(d) * kLog2e;
}

SegDesc to_seg(const cpattn_kv_seg& s) {
  SegDesc r{};
  r.k = s.k;
  r.v = s.v;
  r.pos = s.pos;
  r.doc = s.doc;
  r.len = (int32_t)s.len;
  return r;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CPATTN_OK : CPATTN_ERR_HIP; }

size_t bwd_delta_bytes(const cpattn_attn_desc* desc, int64_t q_len) {
  return ((size_t)q_len * (size_t)desc->hq * sizeof(float) + 255) & ~(size_t)255;
}

// Compute units of the current device (256 when no device is visible, for planning).
// Compute units the launch plans assume: the device's, unless CPATTN_NUM_CUS names a
// positive count (tests use a small count to reach the eight-wave plans on small shapes).
int device_cus() {
  if (const char* e = getenv("CPATTN_NUM_CUS")) {
    const int v = atoi(e);
    if (v > 0) return v;
  }
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

int check_tile_args(const cpattn_attn_desc* desc, int32_t n_edges, const cpattn_q_block* q_blocks,
                    const cpattn_kv_seg* segs) {
  int st = check_desc(desc);
  if (st != CPATTN_OK) return st;
  if (n_edges < 0) return CPATTN_ERR_ARG;
  if (n_edges == 0) return CPATTN_OK;
  if (q_blocks == nullptr || segs == nullptr) return CPATTN_ERR_ARG;
  for (int e = 0; e < n_edges; ++e) {
    if ((st = check_qblock(desc, &q_blocks[e])) != CPATTN_OK) return st;
    if ((st = check_seg(desc, &segs[e])) != CPATTN_OK) return st;
  }
  return CPATTN_OK;
}

// Fills one launch's worth of edges starting at *e; returns false when none are left.
bool next_edge_batch(FwdArgs& a, int32_t n_edges, const cpattn_q_block* q_blocks, const cpattn_kv_seg* segs,
                     float* const* o_parts, float* const* lse_parts, int& e) {
  a.n_jobs = 0;
  for (; e < n_edges && a.n_jobs < kMaxJobs; ++e) {
    if (q_blocks[e].len == 0) continue;
    const int j = a.n_jobs++;
    a.segs[j] = to_seg(segs[e]);
    JobDesc& jb = a.jobs[j];
    jb = JobDesc{};
    jb.q = q_blocks[e].q;
    jb.pos = q_blocks[e].pos;
    jb.doc = q_blocks[e].doc;
    jb.o = o_parts ? o_parts[e] : nullptr;
    jb.lse = lse_parts ? lse_parts[e] : nullptr;
    jb.len = (int32_t)q_blocks[e].len;
    jb.seg_begin = j;
    jb.seg_end = j + 1;
  }
  return a.n_jobs > 0;
}

void fill_stream_job(FwdArgs& a, const cpattn_q_block* q, int32_t n_segs, const cpattn_kv_seg* segs,
                     void* o_out, float* lse_out) {
  for (int s = 0; s < n_segs; ++s) a.segs[s] = to_seg(segs[s]);
  a.n_jobs = 1;
  JobDesc& jb = a.jobs[0];
  jb = JobDesc{};
  jb.q = q->q;
  jb.pos = q->pos;
  jb.doc = q->doc;
  jb.o = o_out;
  jb.lse = lse_out;
  jb.len = (int32_t)q->len;
  jb.seg_begin = 0;
  jb.seg_end = n_segs;
}

}  // namespace

extern "C" {

const char* cpattn_strerror(int status) {
  switch (status) {
    case CPATTN_OK: return "ok";
    case CPATTN_ERR_ARG: return "invalid argument (null pointer, negative or out-of-range size or rank)";
    case CPATTN_ERR_ALIGN: return "alignment error (length not divisible by 2*cp, bad cu_seqlens, or pointer/row not 16-byte aligned)";
    case CPATTN_ERR_UNSUPPORTED: return "unsupported configuration (head dim, dtype, mask or head grouping)";
    case CPATTN_ERR_HIP: return "HIP runtime or launch failure";
    case CPATTN_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int cpattn_version(void) { return 100; }

int cpattn_zigzag_edge_visible(int64_t seq_len, int32_t cp_size, int32_t q_rank, int32_t q_part,
                               int32_t kv_owner, int32_t kv_part, int32_t* visible) {
  if (visible == nullptr || cp_size < 1 || seq_len < 1) return CPATTN_ERR_ARG;
  if (q_rank < 0 || q_rank >= cp_size || kv_owner < 0 || kv_owner >= cp_size) return CPATTN_ERR_ARG;
  if (q_part < -1 || q_part > 1 || kv_part < -1 || kv_part > 1) return CPATTN_ERR_ARG;
  if (seq_len % (2 * (int64_t)cp_size) != 0) return CPATTN_ERR_ALIGN;
  const int64_t chunk = seq_len / (2 * (int64_t)cp_size);
  // the block's chunks end at (c + 1) * chunk - 1, the segment's start at c * chunk
  const int64_t q_front = q_rank, q_back = 2 * (int64_t)cp_size - 1 - q_rank;
  const int64_t k_front = kv_owner, k_back = 2 * (int64_t)cp_size - 1 - kv_owner;
  const int64_t q_chunk = q_part == 0 ? q_front : q_back;  // the later chunk when both
  const int64_t k_chunk = kv_part == 1 ? k_back : k_front;  // the earlier chunk when both
  const int64_t q_max = (q_chunk + 1) * chunk - 1, k_min = k_chunk * chunk;
  *visible = k_min <= q_max ? 1 : 0;
  return CPATTN_OK;
}

}  // extern "C"

namespace {

// Host checks of a partition call (before any rotation options).
int check_partition(int32_t mode, int64_t total, int32_t cp_size, int32_t cp_rank,
                    const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, int32_t n_docs,
                    int32_t* idx_out, int32_t n_gather, const void* const* src, void* const* dst,
                    const int64_t* row_bytes) {
  if (mode != CPATTN_PART_ZIGZAG && mode != CPATTN_PART_THD && mode != CPATTN_PART_STRIPED) return CPATTN_ERR_ARG;
  if (total < 0 || total > INT32_MAX || cp_size < 1 || cp_rank < 0 || cp_rank >= cp_size)
    return CPATTN_ERR_ARG;
  if (n_gather < 0 || n_gather > 8) return CPATTN_ERR_ARG;
  const int64_t unit = mode == CPATTN_PART_STRIPED ? (int64_t)cp_size : 2 * (int64_t)cp_size;
  if (total % unit != 0) return CPATTN_ERR_ALIGN;
  if (mode == CPATTN_PART_THD) {
    if (cu_seqlens_host == nullptr || cu_seqlens_dev == nullptr || n_docs < 1) return CPATTN_ERR_ARG;
    if (cu_seqlens_host[0] != 0 || cu_seqlens_host[n_docs] != total) return CPATTN_ERR_ALIGN;
    for (int k = 0; k < n_docs; ++k) {
      const int64_t len = (int64_t)cu_seqlens_host[k + 1] - cu_seqlens_host[k];
      if (len < 0 || len % (2 * (int64_t)cp_size) != 0) return CPATTN_ERR_ALIGN;
    }
  }
  if (total > 0 && idx_out == nullptr) return CPATTN_ERR_ARG;
  if (n_gather > 0 && (src == nullptr || dst == nullptr || row_bytes == nullptr)) return CPATTN_ERR_ARG;
  for (int g = 0; g < n_gather; ++g) {
    if (row_bytes[g] <= 0 || row_bytes[g] > ((int64_t)1 << 24)) return CPATTN_ERR_ARG;
    if (row_bytes[g] % 16 != 0) return CPATTN_ERR_ALIGN;
    if (total > 0 && (src[g] == nullptr || dst[g] == nullptr)) return CPATTN_ERR_ARG;
    if (!aligned16(src[g]) || !aligned16(dst[g])) return CPATTN_ERR_ALIGN;
  }
  return CPATTN_OK;
}

}  // namespace

extern "C" {

int cpattn_partition(int32_t mode, int64_t total, int32_t cp_size, int32_t cp_rank,
                     const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, int32_t n_docs,
                     int32_t* idx_out, int32_t* doc_out, int32_t n_gather, const void* const* src,
                     void* const* dst, const int64_t* row_bytes, void* stream) {
  const int st = check_partition(mode, total, cp_size, cp_rank, cu_seqlens_host, cu_seqlens_dev, n_docs, idx_out,
                                 n_gather, src, dst, row_bytes);
  if (st != CPATTN_OK || total == 0) return st;
  return hip_status(launch_partition(mode, total, cp_size, cp_rank, cu_seqlens_dev, n_docs, idx_out,
                                     doc_out, n_gather, src, dst, row_bytes, nullptr,
                                     reinterpret_cast<hipStream_t>(stream)));
}

int cpattn_partition_rope(int32_t mode, int64_t total, int32_t cp_size, int32_t cp_rank,
                          const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, int32_t n_docs,
                          int32_t* idx_out, int32_t* doc_out, int32_t n_gather, const void* const* src,
                          void* const* dst, const int64_t* row_bytes, const cpattn_rope_desc* rope,
                          void* stream) {
  int st = check_partition(mode, total, cp_size, cp_rank, cu_seqlens_host, cu_seqlens_dev, n_docs, idx_out,
                           n_gather, src, dst, row_bytes);
  if (st != CPATTN_OK) return st;
  if (rope == nullptr) return CPATTN_ERR_ARG;
  if (n_gather < 32 && (rope->rotate_mask >> n_gather) != 0) return CPATTN_ERR_ARG;
  if (rope->dtype != CPATTN_BF16 && rope->dtype != CPATTN_F32) return CPATTN_ERR_UNSUPPORTED;
  if (rope->d < 16 || rope->d > 256 || rope->d % 16 != 0) return CPATTN_ERR_UNSUPPORTED;
  if (rope->interleaved != 0 && rope->interleaved != 1) return CPATTN_ERR_ARG;
  if (!std::isfinite(rope->base) || rope->base < 0.0f) return CPATTN_ERR_ARG;
  const int64_t head_bytes = (int64_t)rope->d * (rope->dtype == CPATTN_F32 ? 4 : 2);
  for (int g = 0; g < n_gather; ++g) {
    if (!((rope->rotate_mask >> g) & 1u)) continue;
    if (row_bytes[g] % head_bytes != 0) return CPATTN_ERR_ALIGN;
    if (rope_table_entries(rope->d, rope->interleaved, row_bytes[g]) < 0) return CPATTN_ERR_UNSUPPORTED;
  }
  if (total == 0) return CPATTN_OK;
  RopeSpec spec{};
  spec.mask = rope->rotate_mask;
  spec.f32 = rope->dtype == CPATTN_F32;
  spec.d = rope->d;
  spec.interleaved = rope->interleaved;
  spec.log2_base = std::log2(rope->base > 0.0f ? (double)rope->base : 10000.0);
  return hip_status(launch_partition(mode, total, cp_size, cp_rank, cu_seqlens_dev, n_docs, idx_out,
                                     doc_out, n_gather, src, dst, row_bytes, &spec,
                                     reinterpret_cast<hipStream_t>(stream)));
}

size_t cpattn_tile_fwd_workspace_bytes(const cpattn_attn_desc* desc, int32_t n_edges,
                                       const cpattn_q_block* q_blocks, const cpattn_kv_seg* segs) {
  if (check_tile_args(desc, n_edges, q_blocks, segs) != CPATTN_OK) return 0;
  FwdArgs a{};
  fill_common(a, desc);
  const int cus = device_cus();
  size_t need = 0;
  int e = 0;
  while (next_edge_batch(a, n_edges, q_blocks, segs, nullptr, nullptr, e)) {
    const size_t b = plan_fwd(a, desc->d, desc->dtype, cus, true, 0);
    need = b > need ? b : need;
  }
  return need;
}

int cpattn_tile_fwd(const cpattn_attn_desc* desc, int32_t n_edges, const cpattn_q_block* q_blocks,
                    const cpattn_kv_seg* segs, float* const* o_parts, float* const* lse_parts,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_tile_args(desc, n_edges, q_blocks, segs);
  if (st != CPATTN_OK || n_edges == 0) return st;
  if (o_parts == nullptr || lse_parts == nullptr) return CPATTN_ERR_ARG;
  for (int e = 0; e < n_edges; ++e) {
    if (q_blocks[e].len > 0) {
      if (o_parts[e] == nullptr || lse_parts[e] == nullptr) return CPATTN_ERR_ARG;
      if (!aligned16(o_parts[e])) return CPATTN_ERR_ALIGN;
    }
  }
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return CPATTN_ERR_ALIGN;
  FwdArgs a{};
  fill_common(a, desc);
  const int cus = device_cus();
  int e = 0;
  while (next_edge_batch(a, n_edges, q_blocks, segs, o_parts, lse_parts, e)) {
    size_t need = plan_fwd(a, desc->d, desc->dtype, cus, workspace != nullptr, 0);
    if (need > workspace_bytes) need = plan_fwd(a, desc->d, desc->dtype, cus, false, 0);  // too small: no split
    if (need > 0) assign_fwd_workspace(a, desc->d, workspace);
    st = hip_status(launch_fwd(a, desc->d, desc->dtype, true, reinterpret_cast<hipStream_t>(stream)));
    if (st != CPATTN_OK) return st;
  }
  return CPATTN_OK;
}

int cpattn_merge(int32_t n_parts, const float* const* o_parts, const float* const* lse_parts,
                 int64_t rows, int32_t hq, int32_t d, int32_t out_dtype, void* o_out, float* lse_out,
                 void* stream) {
  if (n_parts < 1 || n_parts > 64 || rows < 0 || rows > kMaxRows || hq < 1) return CPATTN_ERR_ARG;
  if (d < 4 || d > 256 || d % 4 != 0) return CPATTN_ERR_UNSUPPORTED;
  if (out_dtype != CPATTN_BF16 && out_dtype != CPATTN_F32) return CPATTN_ERR_UNSUPPORTED;
  if (rows == 0) return CPATTN_OK;
  if (o_parts == nullptr || lse_parts == nullptr || o_out == nullptr || lse_out == nullptr)
    return CPATTN_ERR_ARG;
  for (int j = 0; j < n_parts; ++j) {
    if (o_parts[j] == nullptr || lse_parts[j] == nullptr) return CPATTN_ERR_ARG;
    if (!aligned16(o_parts[j])) return CPATTN_ERR_ALIGN;
  }
  if (!aligned16(o_out)) return CPATTN_ERR_ALIGN;
  return hip_status(launch_merge(n_parts, o_parts, lse_parts, rows, hq, d, out_dtype, o_out, lse_out,
                                 reinterpret_cast<hipStream_t>(stream)));
}

int cpattn_merge_groups(int32_t n_groups, const int32_t* n_parts, const float* const* o_parts,
                        const float* const* lse_parts, const int64_t* rows, int32_t hq, int32_t d,
                        int32_t out_dtype, void* const* o_out, float* const* lse_out, void* stream) {
  if (n_groups < 0 || hq < 1) return CPATTN_ERR_ARG;
  if (d < 4 || d > 256 || d % 4 != 0) return CPATTN_ERR_UNSUPPORTED;
  if (out_dtype != CPATTN_BF16 && out_dtype != CPATTN_F32) return CPATTN_ERR_UNSUPPORTED;
  if (n_groups == 0) return CPATTN_OK;
  if (n_parts == nullptr || rows == nullptr || o_out == nullptr || lse_out == nullptr) return CPATTN_ERR_ARG;
  for (int g = 0; g < n_groups; ++g)
    if (n_parts[g] < 1 || n_parts[g] > 64 || rows[g] < 0 || rows[g] > kMaxRows) return CPATTN_ERR_ARG;
  if (o_parts == nullptr || lse_parts == nullptr) return CPATTN_ERR_ARG;
  // the buffers of groups with rows are checked (a group of 0 rows reads none of them)
  int64_t j0 = 0;
  for (int g = 0; g < n_groups; j0 += n_parts[g], ++g) {
    if (rows[g] == 0) continue;
    for (int64_t j = j0; j < j0 + n_parts[g]; ++j) {
      if (o_parts[j] == nullptr || lse_parts[j] == nullptr) return CPATTN_ERR_ARG;
      if (!aligned16(o_parts[j])) return CPATTN_ERR_ALIGN;
    }
    if (o_out[g] == nullptr || lse_out[g] == nullptr) return CPATTN_ERR_ARG;
    if (!aligned16(o_out[g])) return CPATTN_ERR_ALIGN;
  }
  return hip_status(launch_merge_groups(n_groups, n_parts, o_parts, lse_parts, rows, hq, d, out_dtype, o_out,
                                        lse_out, reinterpret_cast<hipStream_t>(stream)));
}

size_t cpattn_stream_fwd_workspace_bytes(const cpattn_attn_desc* desc, const cpattn_q_block* q,
                                         int32_t n_segs, const cpattn_kv_seg* segs) {
  if (check_desc(desc) != CPATTN_OK || check_qblock(desc, q) != CPATTN_OK) return 0;
  if (n_segs < 1 || n_segs > kMaxSegsTotal || segs == nullptr || q->len == 0) return 0;
  for (int s = 0; s < n_segs; ++s)
    if (check_seg(desc, &segs[s]) != CPATTN_OK) return 0;
  if (n_segs > kMaxSegs) return grouped_stream_bytes(desc, q->len, n_segs);
  FwdArgs a{};
  fill_common(a, desc);
  fill_stream_job(a, q, n_segs, segs, nullptr, nullptr);
  return plan_fwd(a, desc->d, desc->dtype, device_cus(), true, 0);
}

int cpattn_stream_fwd(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                      const cpattn_kv_seg* segs, void* o_out, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != CPATTN_OK) return st;
  if ((st = check_qblock(desc, q)) != CPATTN_OK) return st;
  if (n_segs < 1 || n_segs > kMaxSegsTotal || segs == nullptr) return CPATTN_ERR_ARG;
  for (int s = 0; s < n_segs; ++s)
    if ((st = check_seg(desc, &segs[s])) != CPATTN_OK) return st;
  if (q->len == 0) return CPATTN_OK;
  if (o_out == nullptr || lse_out == nullptr) return CPATTN_ERR_ARG;
  if (!aligned16(o_out)) return CPATTN_ERR_ALIGN;
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return CPATTN_ERR_ALIGN;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (n_segs > kMaxSegs) {
    // groups of kMaxSegs segments, each streamed into its own fp32 partial state, then
    // the log-sum-exp merge of the groups (the same result up to rounding order)
    const size_t need = grouped_stream_bytes(desc, q->len, n_segs);
    if (workspace == nullptr || workspace_bytes < need) return CPATTN_ERR_WORKSPACE;
    const int ng = seg_groups(n_segs);
    const size_t ob = round256((size_t)q->len * desc->hq * desc->d * sizeof(float));
    const size_t lb = round256((size_t)q->len * desc->hq * sizeof(float));
    const float* o_parts[64];
    const float* l_parts[64];
    for (int g = 0; g < ng; ++g) {
      char* base = reinterpret_cast<char*>(workspace) + (size_t)g * (ob + lb);
      float* op = reinterpret_cast<float*>(base);
      float* lp = reinterpret_cast<float*>(base + ob);
      o_parts[g] = op;
      l_parts[g] = lp;
      const int s0 = g * kMaxSegs, cnt = min(kMaxSegs, n_segs - s0);
      FwdArgs a{};
      fill_common(a, desc);
      fill_stream_job(a, q, cnt, segs + s0, op, lp);
      plan_fwd(a, desc->d, desc->dtype, device_cus(), false, 0);
      const hipError_t e = launch_fwd(a, desc->d, desc->dtype, true, hs);
      if (e != hipSuccess) return CPATTN_ERR_HIP;
    }
    return hip_status(launch_merge(ng, o_parts, l_parts, q->len, desc->hq, desc->d, desc->dtype, o_out, lse_out,
                                   hs));
  }
  FwdArgs a{};
  fill_common(a, desc);
  fill_stream_job(a, q, n_segs, segs, o_out, lse_out);
  const int cus = device_cus();
  size_t need = plan_fwd(a, desc->d, desc->dtype, cus, workspace != nullptr, 0);
  if (need > workspace_bytes) need = plan_fwd(a, desc->d, desc->dtype, cus, false, 0);  // too small: no split
  if (need > 0) assign_fwd_workspace(a, desc->d, workspace);
  return hip_status(launch_fwd(a, desc->d, desc->dtype, false, hs));
}

}  // extern "C"

namespace {

// Checks shared by the backward calls (bf16 only): description, query block, segments.
int check_bwd_problem(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                      const cpattn_kv_seg* segs) {
  int st = check_desc(desc);
  if (st != CPATTN_OK) return st;
  if (desc->dtype != CPATTN_BF16) return CPATTN_ERR_UNSUPPORTED;
  if ((st = check_qblock(desc, q)) != CPATTN_OK) return st;
  if (n_segs < 1 || n_segs > kMaxSegsTotal || segs == nullptr) return CPATTN_ERR_ARG;
  for (int s = 0; s < n_segs; ++s)
    if ((st = check_seg(desc, &segs[s])) != CPATTN_OK) return st;
  return CPATTN_OK;
}

// Per-row inputs of the dQ and dK/dV passes (only read when there are local rows).
int check_bwd_rows(const cpattn_q_block* q, const float* lse, const float* delta, const void* dout) {
  if (q->len == 0) return CPATTN_OK;
  if (lse == nullptr || delta == nullptr || dout == nullptr) return CPATTN_ERR_ARG;
  return aligned16(dout) ? CPATTN_OK : CPATTN_ERR_ALIGN;
}

int check_bwd_dq(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                 const cpattn_kv_seg* segs, const float* lse, const float* delta, const void* dout,
                 const float* dq) {
  int st = check_bwd_problem(desc, q, n_segs, segs);
  if (st != CPATTN_OK) return st;
  if ((st = check_bwd_rows(q, lse, delta, dout)) != CPATTN_OK) return st;
  if (q->len > 0 && dq == nullptr) return CPATTN_ERR_ARG;
  if (q->len > 0 && !aligned16(dq)) return CPATTN_ERR_ALIGN;
  return CPATTN_OK;
}

int check_bwd_dkdv(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                   const cpattn_kv_seg* segs, const float* lse, const float* delta, const void* dout,
                   float* const* dk, float* const* dv) {
  int st = check_bwd_problem(desc, q, n_segs, segs);
  if (st != CPATTN_OK) return st;
  if ((st = check_bwd_rows(q, lse, delta, dout)) != CPATTN_OK) return st;
  if (dk == nullptr || dv == nullptr) return CPATTN_ERR_ARG;
  for (int s = 0; s < n_segs; ++s) {
    if (segs[s].len == 0) continue;
    if (dk[s] == nullptr || dv[s] == nullptr) return CPATTN_ERR_ARG;
    if (!aligned16(dk[s]) || !aligned16(dv[s])) return CPATTN_ERR_ALIGN;
  }
  return CPATTN_OK;
}

// The dQ pass as one query-major job over the segments; split over KV tiles into the
// workspace when it holds the plan's partial buffers.  More than kMaxSegs segments run
// as unsplit launches of kMaxSegs segments, each adding its part to dQ.
// o not null: the pass forms delta from O and dO and stores it instead of reading it
// (the first launch of a list of more than kMaxSegs segments; the others read it).
hipError_t run_bwd_dq(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                      const cpattn_kv_seg* segs, const float* lse, const float* delta, const void* dout,
                      float* dq, void* workspace, size_t workspace_bytes, hipStream_t stream,
                      const void* o = nullptr) {
  if (q->len == 0) return hipSuccess;
  float* dl = const_cast<float*>(delta);  // written only when o is set
  if (n_segs > kMaxSegs) {
    for (int s0 = 0; s0 < n_segs; s0 += kMaxSegs) {
      FwdArgs f{};
      fill_common(f, desc);
      fill_stream_job(f, q, min(kMaxSegs, n_segs - s0), segs + s0, dq, const_cast<float*>(lse));
      plan_fwd(f, desc->d, CPATTN_BF16, device_cus(), false, 0);
      const hipError_t e = launch_bwd_dq(f, dout, dl, eff_scale(desc), desc->d, s0 > 0, stream, s0 == 0 ? o : nullptr);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  FwdArgs f{};
  fill_common(f, desc);
  fill_stream_job(f, q, n_segs, segs, dq, const_cast<float*>(lse));
  const int cus = device_cus();
  size_t need = plan_fwd(f, desc->d, CPATTN_BF16, cus, true, 0);
  if (need > 0 && (workspace == nullptr || need > workspace_bytes))
    need = plan_fwd(f, desc->d, CPATTN_BF16, cus, false, 0);  // too small: no split
  if (need > 0) assign_fwd_workspace(f, desc->d, workspace);
  return launch_bwd_dq(f, dout, dl, eff_scale(desc), desc->d, false, stream, o);
}

hipError_t run_bwd_dkdv(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                        const cpattn_kv_seg* segs, const float* lse, const float* delta,
                        const void* dout, float* const* dk, float* const* dv, hipStream_t stream) {
  if (n_segs > kMaxSegs) {  // segments are independent here: one launch per group
    for (int s0 = 0; s0 < n_segs; s0 += kMaxSegs) {
      const hipError_t e = run_bwd_dkdv(desc, q, min(kMaxSegs, n_segs - s0), segs + s0, lse, delta, dout, dk + s0,
                                        dv + s0, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  BwdArgs a{};
  for (int s = 0; s < n_segs; ++s) {
    a.segs[s] = to_seg(segs[s]);
    a.dk[s] = dk[s];
    a.dv[s] = dv[s];
  }
  a.q = q->q;
  a.qpos = q->pos;
  a.qdoc = q->doc;
  a.lse = lse;
  a.dout = dout;
  a.delta = delta;
  a.q_len = (int32_t)q->len;
  a.n_segs = n_segs;
  a.hq = desc->hq;
  a.hkv = desc->hkv;
  a.group = desc->hq / desc->hkv;
  a.mask = desc->mask;
  a.scale = eff_scale(desc);
  a.scale_log2 = a.scale * kLog2e;
  return launch_bwd_dkdv(a, desc->d, stream);
}

size_t bwd_dq_split_bytes(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                          const cpattn_kv_seg* segs) {
  if (q->len == 0 || n_segs > kMaxSegs) return 0;
  FwdArgs f{};
  fill_common(f, desc);
  fill_stream_job(f, q, n_segs, segs, nullptr, nullptr);
  return plan_fwd(f, desc->d, CPATTN_BF16, device_cus(), true, 0);
}

}  // namespace

extern "C" {

int cpattn_bwd_delta(const cpattn_attn_desc* desc, int64_t rows, const void* o, const void* dout,
                     float* delta, void* stream) {
  int st = check_desc(desc);
  if (st != CPATTN_OK) return st;
  if (desc->dtype != CPATTN_BF16) return CPATTN_ERR_UNSUPPORTED;
  if (rows < 0 || rows > INT32_MAX) return CPATTN_ERR_ARG;
  if (rows == 0) return CPATTN_OK;
  if (o == nullptr || dout == nullptr || delta == nullptr) return CPATTN_ERR_ARG;
  if (!aligned16(o) || !aligned16(dout)) return CPATTN_ERR_ALIGN;
  return hip_status(launch_bwd_delta(o, dout, delta, rows * desc->hq, desc->d,
                                     reinterpret_cast<hipStream_t>(stream)));
}

size_t cpattn_bwd_dq_workspace_bytes(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                                     const cpattn_kv_seg* segs) {
  if (check_bwd_problem(desc, q, n_segs, segs) != CPATTN_OK) return 0;
  return bwd_dq_split_bytes(desc, q, n_segs, segs);
}

int cpattn_bwd_dq(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                  const cpattn_kv_seg* segs, const float* lse, const float* delta, const void* dout,
                  float* dq, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_bwd_dq(desc, q, n_segs, segs, lse, delta, dout, dq);
  if (st != CPATTN_OK) return st;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return CPATTN_ERR_ALIGN;
  return hip_status(run_bwd_dq(desc, q, n_segs, segs, lse, delta, dout, dq, workspace, workspace_bytes,
                               reinterpret_cast<hipStream_t>(stream)));
}

int cpattn_bwd_dq_delta(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                        const cpattn_kv_seg* segs, const void* o, const float* lse, const void* dout,
                        float* delta, float* dq, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_bwd_dq(desc, q, n_segs, segs, lse, delta, dout, dq);
  if (st != CPATTN_OK) return st;
  if (q->len > 0 && o == nullptr) return CPATTN_ERR_ARG;
  if (q->len > 0 && !aligned16(o)) return CPATTN_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return CPATTN_ERR_ALIGN;
  return hip_status(run_bwd_dq(desc, q, n_segs, segs, lse, delta, dout, dq, workspace, workspace_bytes,
                               reinterpret_cast<hipStream_t>(stream), o));
}

int cpattn_bwd_dkdv(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                    const cpattn_kv_seg* segs, const float* lse, const float* delta, const void* dout,
                    float* const* dk, float* const* dv, void* stream) {
  const int st = check_bwd_dkdv(desc, q, n_segs, segs, lse, delta, dout, dk, dv);
  if (st != CPATTN_OK) return st;
  return hip_status(run_bwd_dkdv(desc, q, n_segs, segs, lse, delta, dout, dk, dv,
                                 reinterpret_cast<hipStream_t>(stream)));
}

size_t cpattn_bwd_workspace_bytes(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                                  const cpattn_kv_seg* segs) {
  if (check_bwd_problem(desc, q, n_segs, segs) != CPATTN_OK) return 0;
  return bwd_delta_bytes(desc, q->len) + bwd_dq_split_bytes(desc, q, n_segs, segs);
}

int cpattn_bwd(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
               const cpattn_kv_seg* segs, const void* o, const float* lse, const void* dout, float* dq,
               float* const* dk, float* const* dv, void* workspace, size_t workspace_bytes,
               void* stream) {
  int st = check_bwd_problem(desc, q, n_segs, segs);
  if (st != CPATTN_OK) return st;
  const size_t delta_bytes = bwd_delta_bytes(desc, q->len);
  float* delta = reinterpret_cast<float*>(workspace);
  if (q->len > 0) {
    if (o == nullptr) return CPATTN_ERR_ARG;
    if (!aligned16(o)) return CPATTN_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < delta_bytes) return CPATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return CPATTN_ERR_ALIGN;
  }
  if ((st = check_bwd_dq(desc, q, n_segs, segs, lse, delta, dout, dq)) != CPATTN_OK) return st;
  if ((st = check_bwd_dkdv(desc, q, n_segs, segs, lse, delta, dout, dk, dv)) != CPATTN_OK) return st;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // the dQ pass forms delta itself (the same bits as the delta pass) and stores it for
  // the dK/dV pass: two launches instead of three
  char* rest = q->len > 0 ? reinterpret_cast<char*>(workspace) + delta_bytes : nullptr;
  hipError_t e = run_bwd_dq(desc, q, n_segs, segs, lse, delta, dout, dq, rest,
                            q->len > 0 ? workspace_bytes - delta_bytes : 0, hs, o);
  if (e == hipSuccess) e = run_bwd_dkdv(desc, q, n_segs, segs, lse, delta, dout, dk, dv, hs);
  return hip_status(e);
}

}  // extern "C"

// ---------------------------------------------------------------------------------
// The backward for callers that cannot allocate (graph capture, serving loops): its
// workspace is a file-scope device array.  In host code `scratch` names a host-side
// stand-in, not device memory; the device address comes from hipGetSymbolAddress,
// once per device (each device holds its own copy), and only that address is ever
// handed to kernels.
namespace {

static __device__ __align__(256) unsigned char scratch[CPATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on first use).
int current_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CPATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CPATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CPATTN_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return CPATTN_OK;
}

}  // namespace

extern "C" int cpattn_bwd_noalloc(const cpattn_attn_desc* desc, const cpattn_q_block* q, int32_t n_segs,
                                  const cpattn_kv_seg* segs, const void* o, const float* lse, const void* dout,
                                  float* dq, float* const* dk, float* const* dv, void* stream) {
  const int st = check_bwd_problem(desc, q, n_segs, segs);
  if (st != CPATTN_OK) return st;
  if (bwd_delta_bytes(desc, q->len) > (size_t)CPATTN_NOALLOC_SCRATCH_BYTES) return CPATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (q->len > 0) {
    const int sst = current_scratch(&ws);
    if (sst != CPATTN_OK) return sst;
  }
  // the per-row values are rewritten by every call before they are read, and every
  // split of the dQ pass writes its partial and its flag, so nothing needs clearing
  return cpattn_bwd(desc, q, n_segs, segs, o, lse, dout, dq, dk, dv, ws,
                    q->len > 0 ? (size_t)CPATTN_NOALLOC_SCRATCH_BYTES : 0, stream);
}
