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
    // largest k with cu[k]/cp <= t, i.e. cu[k] <= (t+1)*cp - 1 (cu[n_docs]/cp == local > t)
    const int64_t lim = (t + 1) * a.cp - 1;
    int hi = a.n_docs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)a.cu[mid] <= lim) lo = mid; else hi = mid;
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
// moves kPerBlock consecutive 16-byte vectors of the destination; thread k takes
// vectors k, k + kThreads, ..., so every load and store instruction of a wave covers
// 1 KiB of consecutive destination bytes (and of source bytes within a row).  The
// block's local rows (at most kPerBlock + 1) are mapped to global rows once, into LDS,
// by one thread each; that thread also writes the index and document outputs when the
// row's first vector belongs to the block (tensor 0 only).
constexpr int kPerBlock = kThreads * kVecPerThread;

__global__ __launch_bounds__(kThreads) void partition_kernel(PartArgs a) {
  __shared__ int64_t rows[kPerBlock + 1];
  const int g = blockIdx.y;
  const int vpr = a.n_gather > 0 ? a.vpr[g] : 1;
  const int64_t nvec = a.local * vpr;
  const int64_t v0 = (int64_t)blockIdx.x * kPerBlock;
  if (v0 >= nvec) return;  // a smaller tensor than the grid is sized for
  const int64_t vlast = min(nvec, v0 + kPerBlock) - 1;
  const int64_t t0 = v0 / vpr;
  const int nrows = (int)(vlast / vpr - t0 + 1);
  for (int i = threadIdx.x; i < nrows; i += kThreads) {
    const int64_t t = t0 + i;
    int64_t row;
    int32_t d;
    local_to_global(a, t, row, d);
    rows[i] = row;
    if (g == 0 && t * vpr >= v0) {
      a.idx[t] = (int32_t)row;
      if (a.doc) a.doc[t] = d;
    }
  }
  if (a.n_gather == 0) return;
  __syncthreads();
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src[g]);
  u32x4* dst = reinterpret_cast<u32x4*>(a.dst[g]);
  // vector v lies in local row t0 + w / vpr, column w % vpr, with w = v - t0*vpr
  // (w < vpr + kPerBlock, so 32-bit arithmetic suffices)
  const uint32_t w0 = (uint32_t)(v0 - t0 * vpr) + threadIdx.x;
  u32x4 buf[kVecPerThread];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    if (v0 + threadIdx.x + (int64_t)i * kThreads > vlast) break;
    const uint32_t w = w0 + i * kThreads;
    const uint32_t lt = w / (uint32_t)vpr;
    const uint32_t c = w - lt * (uint32_t)vpr;
    buf[i] = __builtin_nontemporal_load(&src[rows[lt] * vpr + c]);
  }
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = v0 + threadIdx.x + (int64_t)i * kThreads;
    if (v <= vlast) dst[v] = buf[i];
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
  const int64_t blocks = (max_vec + kPerBlock - 1) / kPerBlock;
  hipLaunchKernelGGL(partition_kernel, dim3((unsigned)blocks, n_gather > 0 ? n_gather : 1), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace cpattn
