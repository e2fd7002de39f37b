// Merge kernel: the associative log-sum-exp merge of partial attention states.
//
// "Context Parallelism (CP)", section 2.2: for one query row,
//   L = log sum_j exp(L_j),   O = sum_j exp(L_j - L) O_j,
// valid in any order and grouping.  Parts with L_j = -inf (no visible key) carry no
// weight; a row whose parts are all -inf becomes (0, -inf); a part whose L_j is NaN
// (a NaN among its inputs) makes the row NaN.
//
// Bandwidth-bound: each (row, head) pair is handled by d/4 threads that each own a
// 16-byte slice of the head vector, so the n partial outputs stream through in
// fully coalesced 16-byte loads and the result leaves in one store per thread.
#include "common.h"

namespace cpattn {

namespace {

constexpr int kMaxParts = 64;
constexpr int kMaxGroups = 8;
constexpr int kThreads = 256;

// One launch merges up to kMaxGroups groups of rows, each from its own parts (a run of
// the part arrays) into its own output; every block belongs to one group.
struct MergeArgs {
  const float* o[kMaxParts];
  const float* lse[kMaxParts];
  void* o_out[kMaxGroups];
  float* lse_out[kMaxGroups];
  int64_t pairs[kMaxGroups];            // rows * hq of each group
  int32_t block_begin[kMaxGroups + 1];  // first block of each group; the last entry ends the grid
  int32_t part_begin[kMaxGroups];
  int32_t n[kMaxGroups];
  int32_t n_groups;
  int32_t d;
};

// One thread's 4-float slice of the merge of n parts, in one pass over the parts with
// a running maximum (the same sums as the definition, rescaled as the maximum grows).
// Parts are taken kU at a time.  Eager (LAZY false): the LSE and O loads of a group are
// issued together, one memory round trip per group, and a part's O slice is loaded
// whatever its LSE and discarded when the LSE is -inf (its memory is in bounds but may
// never have been written) -- for edge partials, which are nearly all live.  LAZY: the
// group's LSEs first, then only the O slices of live parts, two round trips per group
// -- for KV-split partials, where the splits past a light query tile's visible keys
// are empty.  SUM: the plain sum of the parts whose LSE is not -inf.
template <bool SUM, int kU, bool LAZY, class L, class O>
__device__ __forceinline__ f32x4 merge_slice(int n, L lse_of, O o_of, float& lse_out) {
  float m = neg_inf(), s = 0.0f;
  bool nan_part = false;  // a NaN LSE: the merged state is NaN (fmaxf would drop it)
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < n; p0 += kU) {
    float lv[kU];
    f32x4 ov[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = min(p0 + u, n - 1);
      lv[u] = p0 + u < n ? lse_of(p) : neg_inf();
      if (!LAZY) ov[u] = o_of(p);
    }
    if (LAZY) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        ov[u] = lv[u] != neg_inf() ? o_of(min(p0 + u, n - 1)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (SUM) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (lv[u] != neg_inf()) acc += ov[u];
      continue;
    }
    float bm = lv[0];
#pragma unroll
    for (int u = 1; u < kU; ++u) bm = fmaxf(bm, lv[u]);
#pragma unroll
    for (int u = 0; u < kU; ++u) nan_part |= __builtin_isnan(lv[u]);
    const float m_new = fmaxf(m, bm);
    if (m_new == neg_inf()) continue;
    const float c = fast_exp2((m - m_new) * kLog2e);  // 0 while m is -inf
    s *= c;
    acc *= c;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool live = lv[u] != neg_inf();
      const float w = live ? fast_exp2((lv[u] - m_new) * kLog2e) : 0.0f;
      s += w;
      if (live) acc += w * ov[u];
    }
    m = m_new;
  }
  if (SUM) {
    lse_out = 0.0f;
    return acc;
  }
  if (nan_part) {
    lse_out = __builtin_nanf("");
    return f32x4{lse_out, lse_out, lse_out, lse_out};
  }
  if (!(s > 0.0f)) {
    lse_out = neg_inf();
    return f32x4{0.f, 0.f, 0.f, 0.f};
  }
  lse_out = m + fast_log2(s) * kLn2;
  return acc * (1.0f / s);
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_slice(void* o, int64_t off, f32x4 v) {
  if (OUT_BF16) {
    bf16x4 r;
    r[0] = (bf16)v[0];
    r[1] = (bf16)v[1];
    r[2] = (bf16)v[2];
    r[3] = (bf16)v[3];
    *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(o) + off) = r;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + off) = v;
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  // this block's group (uniform: a scalar walk over at most kMaxGroups entries)
  int g = 0;
  while (g + 1 < a.n_groups && a.block_begin[g + 1] <= (int)blockIdx.x) ++g;
  const int tpp = a.d >> 2;  // threads per (row, head) pair
  const int64_t gid = (int64_t)(blockIdx.x - a.block_begin[g]) * kThreads + threadIdx.x;
  const int64_t pair = gid / tpp;
  const int c = (int)(gid - pair * tpp);
  if (pair >= a.pairs[g]) return;
  const int64_t off = pair * a.d + 4 * c;
  const int p0 = a.part_begin[g];
  float lse;
  const f32x4 v = merge_slice<false, 4, false>(
      a.n[g], [&](int j) { return a.lse[p0 + j][pair]; },
      [&](int j) { return *reinterpret_cast<const f32x4*>(a.o[p0 + j] + off); }, lse);
  store_slice<OUT_BF16>(a.o_out[g], off, v);
  if (c == 0) a.lse_out[g][pair] = lse;
}

// Merge of the KV-split partial states of several forward jobs in one launch: job j
// has n parts at ws_o + p*len*hq*d / ws_lse + p*len*hq and writes (o, lse).
struct MergeJobsArgs {
  const float* ws_o[kMaxJobs];
  const float* ws_lse[kMaxJobs];
  void* o[kMaxJobs];
  float* lse[kMaxJobs];
  int64_t pairs[kMaxJobs];             // len * hq of each job
  int32_t block_begin[kMaxJobs + 1];   // first block of each job (every block in one job)
  int32_t n[kMaxJobs];
  int32_t n_jobs;
  int32_t d;
};

// SUM: plain sum of the parts whose flag (the LSE slot) is not -inf, for split
// gradient partials; otherwise the log-sum-exp merge.
template <bool OUT_BF16, bool SUM>
__global__ __launch_bounds__(kThreads) void merge_jobs_kernel(MergeJobsArgs a) {
  // this block's job (uniform: a scalar walk), so the job's pointers are scalar loads
  int j = 0;
  while (j + 1 < a.n_jobs && a.block_begin[j + 1] <= (int)blockIdx.x) ++j;
  const int tpp = a.d >> 2;
  const int64_t gid = (int64_t)(blockIdx.x - a.block_begin[j]) * kThreads + threadIdx.x;
  const int64_t pair = gid / tpp;
  const int c = (int)(gid - pair * tpp);
  const int64_t stride = a.pairs[j];  // len * hq
  if (pair >= stride) return;
  const int n = a.n[j];
  const float* lp = a.ws_lse[j] + pair;
  const float* op = a.ws_o[j] + pair * a.d + 4 * c;
  const int64_t ostride = stride * a.d;
  float lse;
  const f32x4 v = merge_slice<SUM, 8, true>(
      n, [&](int p) { return lp[p * stride]; },
      [&](int p) { return *reinterpret_cast<const f32x4*>(op + p * ostride); }, lse);
  const int64_t off = pair * a.d + 4 * c;
  if (SUM) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o[j]) + off) = v;
    return;
  }
  store_slice<OUT_BF16>(a.o[j], off, v);
  if (c == 0) a.lse[j][pair] = lse;
}

}  // namespace

hipError_t launch_merge_split_jobs(const FwdArgs& f, int d, int out_dtype, hipStream_t stream, bool sum) {
  MergeJobsArgs a{};
  int64_t blocks = 0;
  for (int j = 0; j < f.n_jobs; ++j) {
    const JobDesc& jb = f.jobs[j];
    if (jb.n_split <= 1) continue;
    const int k = a.n_jobs++;
    a.ws_o[k] = jb.ws_o;
    a.ws_lse[k] = jb.ws_lse;
    a.o[k] = jb.o;
    a.lse[k] = jb.lse;
    a.n[k] = jb.n_split;
    a.pairs[k] = (int64_t)jb.len * f.hq;
    a.block_begin[k] = (int32_t)blocks;
    blocks += (a.pairs[k] * (d / 4) + kThreads - 1) / kThreads;
  }
  a.block_begin[a.n_jobs] = (int32_t)blocks;
  a.d = d;
  if (blocks == 0) return hipSuccess;
  if (sum)
    hipLaunchKernelGGL((merge_jobs_kernel<false, true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else if (out_dtype == 0)
    hipLaunchKernelGGL((merge_jobs_kernel<true, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((merge_jobs_kernel<false, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge_groups(int n_groups, const int32_t* n_parts, const float* const* o_parts,
                               const float* const* lse_parts, const int64_t* rows, int hq, int d, int out_dtype,
                               void* const* o_out, float* const* lse_out, hipStream_t stream) {
  // groups go into launches in order, at most kMaxGroups groups and kMaxParts parts each
  int g0 = 0, p0 = 0;
  while (g0 < n_groups) {
    MergeArgs a{};
    int ng = 0, np = 0, blocks = 0;
    while (g0 + ng < n_groups && ng < kMaxGroups && np + n_parts[g0 + ng] <= kMaxParts) {
      const int g = g0 + ng;
      for (int j = 0; j < n_parts[g]; ++j) {
        a.o[np + j] = o_parts[p0 + np + j];
        a.lse[np + j] = lse_parts[p0 + np + j];
      }
      a.o_out[ng] = o_out[g];
      a.lse_out[ng] = lse_out[g];
      a.pairs[ng] = rows[g] * hq;
      a.part_begin[ng] = np;
      a.n[ng] = n_parts[g];
      a.block_begin[ng] = blocks;
      blocks += (int)((a.pairs[ng] * (d / 4) + kThreads - 1) / kThreads);
      np += n_parts[g];
      ++ng;
    }
    a.block_begin[ng] = blocks;
    a.n_groups = ng;
    a.d = d;
    if (blocks > 0) {
      if (out_dtype == 0)
        hipLaunchKernelGGL(merge_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
      else
        hipLaunchKernelGGL(merge_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    g0 += ng;
    p0 += np;
  }
  return hipSuccess;
}

hipError_t launch_merge(int n_parts, const float* const* o_parts, const float* const* lse_parts,
                        int64_t rows, int hq, int d, int out_dtype, void* o_out, float* lse_out,
                        hipStream_t stream) {
  const int32_t np = n_parts;
  void* oo = o_out;
  float* lo = lse_out;
  return launch_merge_groups(1, &np, o_parts, lse_parts, &rows, hq, d, out_dtype, &oo, &lo, stream);
}

}  // namespace cpattn
