// Partition kernel: the rows one context-parallel rank holds, and their gather.
//
// "04 · Megatron-LM 实现" (Megatron CP integration), section 1.1: the sequence is
// viewed as 2*cp equal chunks; rank r keeps chunk r, then chunk 2cp-1-r.
// Same page, sections 1.2 and 5: packed documents are split the same way inside
// each document (front slice r, then the mirrored back slice).
// "推理系统基础设施（二）：Sequence Parallelism + Ring Attention", section 5: the
// striped split, rank r keeps tokens r, r + cp, r + 2cp, ...
//
// Every document contributes L/cp rows to every rank, so the local rows of
// document k start at cu[k]/cp: a local row finds its document with a binary
// search over cu/cp, then its global row with two affine cases.  The gather copies
// each selected row of every tensor in 16-byte vectors (HBM-bound).
//
// Rotary embedding in the gather (same Megatron page, section 5: positions follow
// the split; a packed document's positions restart at 0): a rotated tensor's rows
// leave rotated by the angles of the row's position, p * base^(-2i/d), computed in
// fp64 once per (row, frequency) of a block into an LDS table; the rotation itself
// is fp32, rounded to the tensor's dtype once.
#include "common.h"

namespace cpattn {

namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;
constexpr int kMaxGather = 8;
constexpr int kModeThd = 1, kModeStriped = 2;  // mode 0: zigzag

struct RopeArgs {
  uint32_t mask;      // bit g: tensor g is rotated
  int32_t f32;        // element type of the rotated tensors: 0 bf16, 1 fp32
  int32_t d;          // head dim (multiple of 16, at most 256)
  int32_t interleaved;
  double log2_base;   // log2 of the frequency base
};

struct PartArgs {
  const void* src[kMaxGather];
  void* dst[kMaxGather];
  int32_t vpr[kMaxGather];  // 16-byte vectors per row of each tensor
  const int32_t* cu;        // device cu_seqlens (THD) or null
  int32_t* idx;
  int32_t* doc;
  int64_t total;
  int64_t local;            // total / cp
  int32_t n_docs;
  int32_t cp;
  int32_t rank;
  int32_t n_gather;
  int32_t mode;
  RopeArgs rope;
};

// Global row, document and rotary position (inside the document for THD) of local row t.
__device__ __forceinline__ void local_to_global(const PartArgs& a, int64_t t, int64_t& row,
                                                int32_t& docid, int32_t& pos) {
  if (a.mode == kModeStriped) {
    row = a.rank + t * a.cp;
    docid = 0;
    pos = (int32_t)row;
    return;
  }
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
  pos = (int32_t)(row - start);
}

// Maps the local rows of a block to global rows (and rotary positions) in LDS, one
// thread per row; the thread also writes the index and document outputs when the
// row's first unit belongs to the block and the block serves tensor 0.
__device__ __forceinline__ int map_rows(const PartArgs& a, int g, int64_t u0, int64_t ulast, int64_t upr,
                                        int64_t* rows, int32_t* rpos) {
  const int64_t t0 = u0 / upr;
  const int nrows = (int)(ulast / upr - t0 + 1);
  for (int i = threadIdx.x; i < nrows; i += kThreads) {
    const int64_t t = t0 + i;
    int64_t row;
    int32_t d, p;
    local_to_global(a, t, row, d, p);
    rows[i] = row;
    if (rpos) rpos[i] = p;
    if (g == 0 && t * upr >= u0) {
      a.idx[t] = (int32_t)row;
      if (a.doc) a.doc[t] = d;
    }
  }
  return nrows;
}

// Plain gather.  grid.y selects the tensor (or, with no tensors, only the index
// output); rotated tensors are left to rope_kernel.  A block moves kPerBlock
// consecutive 16-byte vectors of the destination; thread k takes vectors k,
// k + kThreads, ..., so every load and store instruction of a wave covers 1 KiB of
// consecutive destination bytes (and of source bytes within a row).
constexpr int kPerBlock = kThreads * kVecPerThread;

__device__ __forceinline__ void plain_gather(const PartArgs& a, int g, int64_t* rows) {
  const int vpr = a.n_gather > 0 ? a.vpr[g] : 1;
  const int64_t nvec = a.local * vpr;
  const int64_t v0 = (int64_t)blockIdx.x * kPerBlock;
  if (v0 >= nvec) return;  // a smaller tensor than the grid is sized for
  const int64_t vlast = min(nvec, v0 + kPerBlock) - 1;
  const int64_t t0 = v0 / vpr;
  map_rows(a, g, v0, vlast, vpr, rows, nullptr);
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

__global__ __launch_bounds__(kThreads) void partition_kernel(PartArgs a) {
  __shared__ int64_t rows[kPerBlock + 1];
  plain_gather(a, blockIdx.y, rows);
}

// Rotated gather.  A block takes kPerBlock vectors too, as units that hold whole
// rotation pairs: a vector (interleaved pairs (2i, 2i+1)) or a vector of the first
// half of a head with its partner vector d/2 elements on (pairs (i, i + d/2)).  The
// cosine and sine table holds (rows of the block) x d/2 entries, at most 4096 + d
// (the host checks the bound).
constexpr int kRopeTab = 4096 + 256;

__device__ __forceinline__ void rope_pair(float a, float b, float c, float s, float& x, float& y) {
  x = fmaf(a, c, -b * s);
  y = fmaf(b, c, a * s);
}

template <bool F32, bool HALF>
__device__ __forceinline__ void rope_block(const PartArgs& a, int g, int64_t u0, int64_t ulast, int64_t t0,
                                           int upr, const int64_t* rows, const float* cs, const float* sn) {
  constexpr int kEpv = F32 ? 4 : 8;                            // elements per 16-byte vector
  constexpr int kPer = (HALF ? kPerBlock / 2 : kPerBlock) / kThreads;  // units per thread
  const int h2 = a.rope.d / 2;
  const int vph = a.rope.d / kEpv;
  const int vpr = a.vpr[g];
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src[g]);
  u32x4* dst = reinterpret_cast<u32x4*>(a.dst[g]);
  u32x4 lo[kPer], hi[kPer];
  int lt[kPer], v0[kPer], f0[kPer];
  // every load of the thread first, then the arithmetic and the stores
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t u = u0 + threadIdx.x + (int64_t)k * kThreads;
    lt[k] = -1;
    if (u > ulast) continue;
    const int64_t w = u - t0 * upr;
    lt[k] = (int)(w / upr);
    const int c = (int)(w - (int64_t)lt[k] * upr);
    if (HALF) {
      const int hh = c / (vph / 2), cc = c - hh * (vph / 2);
      v0[k] = hh * vph + cc;
      f0[k] = cc * kEpv;
    } else {
      const int hh = c / vph, cc = c - hh * vph;
      v0[k] = hh * vph + cc;
      f0[k] = cc * kEpv / 2;
    }
    const int64_t sb = rows[lt[k]] * vpr;
    lo[k] = __builtin_nontemporal_load(&src[sb + v0[k]]);
    if (HALF) hi[k] = __builtin_nontemporal_load(&src[sb + v0[k] + vph / 2]);
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (lt[k] < 0) continue;
    const float* cr = cs + lt[k] * h2 + f0[k];
    const float* sr = sn + lt[k] * h2 + f0[k];
    float x[kEpv], y[kEpv];
    if (F32) {
      const f32x4 xl = __builtin_bit_cast(f32x4, lo[k]);
#pragma unroll
      for (int e = 0; e < kEpv; ++e) x[e] = xl[e];
      if (HALF) {
        const f32x4 xh = __builtin_bit_cast(f32x4, hi[k]);
#pragma unroll
        for (int e = 0; e < kEpv; ++e) y[e] = xh[e];
      }
    } else {
      const bf16x8 xl = __builtin_bit_cast(bf16x8, lo[k]);
#pragma unroll
      for (int e = 0; e < kEpv; ++e) x[e] = (float)xl[e];
      if (HALF) {
        const bf16x8 xh = __builtin_bit_cast(bf16x8, hi[k]);
#pragma unroll
        for (int e = 0; e < kEpv; ++e) y[e] = (float)xh[e];
      }
    }
    float ox[kEpv], oy[kEpv];
    if (HALF) {
      // element e of the first-half vector pairs with element e of its partner
#pragma unroll
      for (int e = 0; e < kEpv; ++e) rope_pair(x[e], y[e], cr[e], sr[e], ox[e], oy[e]);
    } else {
#pragma unroll
      for (int e = 0; e < kEpv; e += 2) rope_pair(x[e], x[e + 1], cr[e / 2], sr[e / 2], ox[e], ox[e + 1]);
    }
    const int64_t db = (t0 + lt[k]) * vpr + v0[k];
    if (F32) {
      dst[db] = __builtin_bit_cast(u32x4, f32x4{ox[0], ox[1], ox[2], ox[3]});
      if (HALF) dst[db + vph / 2] = __builtin_bit_cast(u32x4, f32x4{oy[0], oy[1], oy[2], oy[3]});
    } else {
      bf16x8 bl, bh;
#pragma unroll
      for (int e = 0; e < kEpv; ++e) {
        bl[e] = (bf16)ox[e];
        if (HALF) bh[e] = (bf16)oy[e];
      }
      dst[db] = __builtin_bit_cast(u32x4, bl);
      if (HALF) dst[db + vph / 2] = __builtin_bit_cast(u32x4, bh);
    }
  }
}

__device__ __forceinline__ void rope_gather(const PartArgs& a, int g, int64_t* rows, int32_t* rpos, float* cs,
                                            float* sn) {
  const bool half = a.rope.interleaved == 0;
  const int vpr = a.vpr[g];
  const int upr = half ? vpr / 2 : vpr;  // units per row
  const int64_t per_block = half ? kPerBlock / 2 : kPerBlock;
  const int64_t nunit = a.local * upr;
  const int64_t u0 = (int64_t)blockIdx.x * per_block;
  if (u0 >= nunit) return;
  const int64_t ulast = min(nunit, u0 + per_block) - 1;
  const int nrows = map_rows(a, g, u0, ulast, upr, rows, rpos);
  __syncthreads();
  // cos / sin of every (row, frequency) of the block: the angle p * base^(-2f/d) and
  // its sine and cosine in fp64, stored as fp32
  const int h2 = a.rope.d / 2;
  for (int e = threadIdx.x; e < nrows * h2; e += kThreads) {
    const int r = e / h2, f = e - r * h2;
    const double theta = exp2(-(double)(2 * f) / a.rope.d * a.rope.log2_base);
    double sv, cv;
    sincos((double)rpos[r] * theta, &sv, &cv);
    cs[e] = (float)cv;
    sn[e] = (float)sv;
  }
  __syncthreads();
  const int64_t t0 = u0 / upr;
  if (a.rope.f32) {
    if (half)
      rope_block<true, true>(a, g, u0, ulast, t0, upr, rows, cs, sn);
    else
      rope_block<true, false>(a, g, u0, ulast, t0, upr, rows, cs, sn);
  } else {
    if (half)
      rope_block<false, true>(a, g, u0, ulast, t0, upr, rows, cs, sn);
    else
      rope_block<false, false>(a, g, u0, ulast, t0, upr, rows, cs, sn);
  }
}

// A gather with rotated tensors: one launch for every tensor, blockIdx.y choosing the
// tensor and with it the rotated or the plain path (uniform per block).
__global__ __launch_bounds__(kThreads) void rope_kernel(PartArgs a) {
  __shared__ int64_t rows[kPerBlock + 1];
  __shared__ int32_t rpos[kPerBlock + 1];
  __shared__ float cs[kRopeTab], sn[kRopeTab];
  const int g = blockIdx.y;
  if ((a.rope.mask >> g) & 1u)
    rope_gather(a, g, rows, rpos, cs, sn);
  else
    plain_gather(a, g, rows);
}

}  // namespace

hipError_t launch_partition(int mode, int64_t total, int cp, int rank, const int32_t* cu_dev,
                            int n_docs, int32_t* idx, int32_t* doc, int n_gather,
                            const void* const* src, void* const* dst, const int64_t* row_bytes,
                            const RopeSpec* rope, hipStream_t stream) {
  PartArgs a{};
  int64_t plain_blocks = 0, rope_blocks = 0;
  a.local = total / cp;
  if (rope != nullptr) {
    a.rope.mask = rope->mask;
    a.rope.f32 = rope->f32;
    a.rope.d = rope->d;
    a.rope.interleaved = rope->interleaved;
    a.rope.log2_base = rope->log2_base;
  }
  for (int g = 0; g < n_gather; ++g) {
    a.src[g] = src[g];
    a.dst[g] = dst[g];
    a.vpr[g] = (int32_t)(row_bytes[g] / 16);
    const int64_t nvec = a.local * a.vpr[g];  // a rotated tensor's units cover its vectors
    const int64_t b = (nvec + kPerBlock - 1) / kPerBlock;
    int64_t& blocks = ((a.rope.mask >> g) & 1u) ? rope_blocks : plain_blocks;
    blocks = blocks > b ? blocks : b;
  }
  if (n_gather == 0) plain_blocks = (a.local + kPerBlock - 1) / kPerBlock;
  a.cu = mode == kModeThd ? cu_dev : nullptr;
  a.idx = idx;
  a.doc = doc;
  a.total = total;
  a.n_docs = mode == kModeThd ? n_docs : 1;
  a.cp = cp;
  a.rank = rank;
  a.n_gather = n_gather;
  a.mode = mode;
  if (a.local == 0) return hipSuccess;
  const unsigned gy = n_gather > 0 ? n_gather : 1;
  if (rope_blocks > 0) {
    // rotated and plain tensors in one launch
    const int64_t blocks = rope_blocks > plain_blocks ? rope_blocks : plain_blocks;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks, gy), dim3(kThreads), 0, stream, a);
  } else if (plain_blocks > 0) {
    hipLaunchKernelGGL(partition_kernel, dim3((unsigned)plain_blocks, gy), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

int rope_table_entries(int d, int interleaved, int64_t row_bytes) {
  const int64_t vpr = row_bytes / 16;
  const int64_t upr = interleaved ? vpr : vpr / 2;
  const int64_t per_block = interleaved ? kPerBlock : kPerBlock / 2;
  const int64_t n = (per_block / upr + 2) * (d / 2);
  return n > kRopeTab ? -1 : (int)n;
}

}  // namespace cpattn
