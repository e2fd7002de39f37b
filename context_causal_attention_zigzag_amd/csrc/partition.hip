// Partition kernel: the rows one context-parallel rank holds, and their gather.
//
// "04 · Megatron-LM 实现" (Megatron CP integration), section 1.1: the sequence is
// viewed as 2*cp equal chunks; rank r keeps chunk r, then chunk 2cp-1-r.
// Same page, sections 1.2 and 5: packed documents are split the same way inside
// each document (front slice r, then the mirrored back slice).
//
// Every document contributes L/cp rows to every rank, so the local rows of
// document k start at cu[k]/cp: a local row finds its document with a binary
// search over cu/cp, then its global row with two affine cases.  The gather copies
// each selected row of every tensor in 16-byte vectors (HBM-bound).
#include "common.h"

namespace cpattn {

namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;
constexpr int kMaxGather = 8;

struct PartArgs {
  const void* src[kMaxGather];
  void* dst[kMaxGather];
  int32_t vpr[kMaxGather];  // 16-byte vectors per row of each tensor
  const int32_t* cu;        // device cu_seqlens (THD) or null (zigzag)
  int32_t* idx;
  int32_t* doc;
  int64_t total;
  int64_t local;            // total / cp
  int32_t n_docs;
  int32_t cp;
  int32_t rank;
  int32_t n_gather;
};

__device__ __forceinline__ void local_to_global(const PartArgs& a, int64_t t, int64_t& row,
                                                int32_t& docid) {
  int64_t start = 0, len = a.total;
  int lo = 0;
  if (a.cu != nullptr) {
    // largest k with cu[k]/cp <= t (cu[n_docs]/cp == local > t)
    int hi = a.n_docs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)a.cu[mid] / a.cp <= t) lo = mid; else hi = mid;
    }
    start = a.cu[lo];
    len = (int64_t)a.cu[lo + 1] - start;
  }
  const int64_t seg = len / (2 * a.cp);
  const int64_t u = t - start / a.cp;
  row = u < seg ? start + a.rank * seg + u
                : start + len - (int64_t)(a.rank + 1) * seg + (u - seg);
  docid = lo;
}

// grid.y selects the tensor (or, with no tensors, only the index output).  A block
// moves kVecPerThread * kThreads consecutive 16-byte vectors of the destination; thread
// k takes vectors k, k + kThreads, ..., so every load and store instruction of a wave
// covers 1 KiB of consecutive destination bytes (and of source bytes within a row).
__global__ __launch_bounds__(kThreads) void partition_kernel(PartArgs a) {
  const int g = blockIdx.y;
  const int vpr = a.n_gather > 0 ? a.vpr[g] : 1;
  const int64_t nvec = a.local * vpr;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kVecPerThread + threadIdx.x;
  if (a.n_gather == 0) {  // indices only: one row per vector
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      const int64_t t = base + (int64_t)i * kThreads;
      if (t >= nvec) break;
      int64_t row;
      int32_t d;
      local_to_global(a, t, row, d);
      a.idx[t] = (int32_t)row;
      if (a.doc) a.doc[t] = d;
    }
    return;
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src[g]);
  u32x4* dst = reinterpret_cast<u32x4*>(a.dst[g]);
  u32x4 buf[kVecPerThread];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v >= nvec) break;
    const int64_t t = v / vpr;
    const int c = (int)(v - t * vpr);
    int64_t row;
    int32_t d;
    local_to_global(a, t, row, d);
    if (g == 0 && c == 0) {
      a.idx[t] = (int32_t)row;
      if (a.doc) a.doc[t] = d;
    }
    buf[i] = __builtin_nontemporal_load(&src[row * vpr + c]);
  }
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) dst[v] = buf[i];
  }
}

}  // namespace

hipError_t launch_partition(int mode, int64_t total, int cp, int rank, const int32_t* cu_dev,
                            int n_docs, int32_t* idx, int32_t* doc, int n_gather,
                            const void* const* src, void* const* dst, const int64_t* row_bytes,
                            hipStream_t stream) {
  PartArgs a{};
  int64_t max_vec = 0;
  a.local = total / cp;
  for (int g = 0; g < n_gather; ++g) {
    a.src[g] = src[g];
    a.dst[g] = dst[g];
    a.vpr[g] = (int32_t)(row_bytes[g] / 16);
    max_vec = max_vec > a.local * a.vpr[g] ? max_vec : a.local * a.vpr[g];
  }
  if (n_gather == 0) max_vec = a.local;
  a.cu = mode == 1 ? cu_dev : nullptr;
  a.idx = idx;
  a.doc = doc;
  a.total = total;
  a.n_docs = mode == 1 ? n_docs : 1;
  a.cp = cp;
  a.rank = rank;
  a.n_gather = n_gather;
  if (a.local == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kThreads * kVecPerThread;
  const int64_t blocks = (max_vec + per_block - 1) / per_block;
  hipLaunchKernelGGL(partition_kernel, dim3((unsigned)blocks, n_gather > 0 ? n_gather : 1), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace cpattn
