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

constexpr int kRowsPerBlock = 64;
constexpr int kThreads = 256;
constexpr int kMaxGather = 8;

struct PartArgs {
  const void* src[kMaxGather];
  void* dst[kMaxGather];
  int64_t row_bytes[kMaxGather];
  const int32_t* cu;   // device cu_seqlens (THD) or null (zigzag)
  int32_t* idx;
  int32_t* doc;
  int64_t total;
  int64_t local;       // total / cp
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
    // largest k with cu[k]/cp <= t
    int hi = a.n_docs;  // cu[n_docs]/cp == local > t
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

__global__ __launch_bounds__(kThreads) void partition_kernel(PartArgs a) {
  __shared__ int64_t rows[kRowsPerBlock];
  const int64_t t0 = (int64_t)blockIdx.x * kRowsPerBlock;
  const int tid = threadIdx.x;
  if (tid < kRowsPerBlock) {
    const int64_t t = t0 + tid;
    if (t < a.local) {
      int64_t row;
      int32_t d;
      local_to_global(a, t, row, d);
      rows[tid] = row;
      a.idx[t] = (int32_t)row;
      if (a.doc) a.doc[t] = d;
    }
  }
  __syncthreads();
  const int nrows = (int)min((int64_t)kRowsPerBlock, a.local - t0);
  for (int g = 0; g < a.n_gather; ++g) {
    const int vpr = (int)(a.row_bytes[g] >> 4);  // 16-byte vectors per row
    const int nvec = vpr * nrows;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.src[g]);
    u32x4* dst = reinterpret_cast<u32x4*>(a.dst[g]);
    for (int i = tid; i < nvec; i += kThreads) {
      const int r = i / vpr;
      const int c = i - r * vpr;
      dst[(t0 + r) * vpr + c] = __builtin_nontemporal_load(&src[rows[r] * vpr + c]);
    }
  }
}

}  // namespace

hipError_t launch_partition(int mode, int64_t total, int cp, int rank, const int32_t* cu_dev,
                            int n_docs, int32_t* idx, int32_t* doc, int n_gather,
                            const void* const* src, void* const* dst, const int64_t* row_bytes,
                            hipStream_t stream) {
  PartArgs a{};
  for (int g = 0; g < n_gather; ++g) {
    a.src[g] = src[g];
    a.dst[g] = dst[g];
    a.row_bytes[g] = row_bytes[g];
  }
  a.cu = mode == 1 ? cu_dev : nullptr;
  a.idx = idx;
  a.doc = doc;
  a.total = total;
  a.local = total / cp;
  a.n_docs = mode == 1 ? n_docs : 1;
  a.cp = cp;
  a.rank = rank;
  a.n_gather = n_gather;
  if (a.local == 0) return hipSuccess;
  const int64_t blocks = (a.local + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(partition_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cpattn
