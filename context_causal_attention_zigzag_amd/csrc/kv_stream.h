// KV-tile streaming shared by the forward kernel and the backward's dQ kernel:
// the double-buffered LDS image of a 64-key tile, its direct global->LDS fill plan,
// and the iterators that walk the visible tiles of a job (scan mode, or ballot-mask
// mode for KV splits).
#pragma once

#include "common.h"

namespace cpattn {
namespace kv {

constexpr int kBK = 64;         // keys per KV tile
constexpr int kThreads = 256;   // 4 waves
constexpr int kRowsPerWave = 32;
constexpr float kTau = 8.0f;    // lazy-rescale threshold (log2 units)
constexpr int kPosPad = 0x7fffffff;

struct TileRef {
  int seg;
  int tile;
};

// Double-buffered LDS image of one KV tile (kBK keys).  Row strides measured
// conflict-free on gfx950's 64-bank LDS: 16-byte row reads need a stride of 4
// (mod 16) dwords (D + 8 elements), transposing reads 16 (mod 64) dwords (D + 32).
template <int D, int KS, int VS>
struct KvSmem {
  static constexpr int kKS = KS;
  static constexpr int kVS = VS;
  bf16 k[2][kBK * kKS];
  bf16 v[2][kBK * kVS];
  int32_t kpos[2][kBK];
  int32_t kdoc[2][kBK];
};


// Next KV tile at or after (s, t) that the query range can see; seg = -1 if none.
__device__ __forceinline__ TileRef next_tile(const FwdArgs& a, int seg_end, int s, int t, int qmin,
                                             int qmax, int qdmin, int qdmax) {
  const int mask = a.mask;
  for (; s < seg_end; ++s, t = 0) {
    const int len = a.segs[s].len;
    const int32_t* pos = a.segs[s].pos;
    const int32_t* doc = a.segs[s].doc;
    const int nt = (len + kBK - 1) / kBK;
    for (; t < nt; ++t) {
      const int k0 = t * kBK;
      const int k1 = min(len, k0 + kBK) - 1;
      if (mask == kMaskNone) return {s, t};
      const int kmin = pos[k0];
      // positions ascend inside a segment: once a tile starts after the last query,
      // no later tile of that segment is visible either
      if (kmin > qmax) break;
      int kdmin = 0, kdmax = 0;
      if (mask == kMaskCausalDoc) {
        kdmin = doc[k0];
        kdmax = doc[k1];
      }
      if (classify(mask, qmin, qmax, qdmin, qdmax, kmin, pos[k1], kdmin, kdmax) != kTileEmpty) return {s, t};
    }
  }
  return {-1, 0};
}

// Iterator over the KV tiles one work-group processes.  Scan mode walks the job's
// segments with next_tile().  Mask mode (KV split across work-groups) first classifies
// every tile of the job lane-parallel into four 64-bit ballot masks over the job's
// tile sequence, then yields the visible tiles of rank [first, first + count).
struct TileIter {
  bool mask_mode;
  uint64_t v0, v1, v2, v3;
  uint64_t m;   // unvisited bits of the current word
  int w;        // current word
  int left;     // tiles still to yield
  int seg;      // segment of the last yielded tile
  __device__ __forceinline__ uint64_t word(int i) const {
    return i == 0 ? v0 : (i == 1 ? v1 : (i == 2 ? v2 : v3));
  }
};

__device__ __forceinline__ void iter_init_masks(TileIter& it, const FwdArgs& a, const JobDesc& job, int lane,
                                                int qmin, int qmax, int qdmin, int qdmax) {
  uint64_t v[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    bool vis = false;
    const int g = 64 * w + lane;
    if (64 * w < job.n_tiles) {
      for (int s = job.seg_begin; s < job.seg_end; ++s) {
        const int len = a.segs[s].len;
        const int t = g - a.segs[s].tile_off;
        if (t >= 0 && t * kBK < len) {
          const int k0 = t * kBK, k1 = min(len, k0 + kBK) - 1;
          const int32_t* pos = a.segs[s].pos;
          int kdmin = 0, kdmax = 0;
          if (a.mask == kMaskCausalDoc) {
            kdmin = a.segs[s].doc[k0];
            kdmax = a.segs[s].doc[k1];
          }
          vis = classify(a.mask, qmin, qmax, qdmin, qdmax, pos[k0], pos[k1], kdmin, kdmax) != kTileEmpty;
        }
      }
    }
    v[w] = __ballot(vis);
  }
  it.v0 = v[0];
  it.v1 = v[1];
  it.v2 = v[2];
  it.v3 = v[3];
}

__device__ __forceinline__ int iter_count(const TileIter& it) {
  return __popcll(it.v0) + __popcll(it.v1) + __popcll(it.v2) + __popcll(it.v3);
}

// Position the iterator before the visible tile of rank `first`, to yield `count`.
__device__ __forceinline__ void iter_seek(TileIter& it, int first, int count, int seg_begin) {
  int w = 0, rank = 0;
  while (w < 3 && rank + __popcll(it.word(w)) <= first) {
    rank += __popcll(it.word(w));
    ++w;
  }
  uint64_t m = it.word(w);
  for (; rank < first; ++rank) m &= m - 1;
  it.w = w;
  it.m = m;
  it.left = count;
  it.seg = seg_begin;
}

__device__ __forceinline__ TileRef iter_next(TileIter& it, const FwdArgs& a, const JobDesc& job, TileRef prev,
                                             int qmin, int qmax, int qdmin, int qdmax) {
  if (!it.mask_mode) {
    if (prev.seg < 0) return next_tile(a, job.seg_end, job.seg_begin, 0, qmin, qmax, qdmin, qdmax);
    return next_tile(a, job.seg_end, prev.seg, prev.tile + 1, qmin, qmax, qdmin, qdmax);
  }
  if (it.left == 0) return {-1, 0};
  while (it.m == 0) {
    ++it.w;
    it.m = it.word(it.w);
  }
  const int g = 64 * it.w + __builtin_ctzll(it.m);
  it.m &= it.m - 1;
  --it.left;
  while (it.seg + 1 < job.seg_end && a.segs[it.seg + 1].tile_off <= g) ++it.seg;
  return {it.seg, g - a.segs[it.seg].tile_off};
}

// Direct global->LDS fill of one KV tile.  The tile's LDS image is a sequence of
// 16-byte slots (row-major, kKS/8 or kVS/8 slots per key row, the last ones padding);
// fill instruction jj of the work-group writes slots 64*jj .. 64*jj+63, lane l slot
// 64*jj + l.  Each lane's (key row, column) per instruction is fixed for the kernel;
// padding slots load a valid dummy chunk and key rows past a ragged tile's end are
// clamped to its last key (those keys are masked).
template <int D, class Smem>
struct FillPlan {
  static constexpr int kKSlots = Smem::kKS / 8;
  static constexpr int kVSlots = Smem::kVS / 8;
  static constexpr int kKInst = kBK * kKSlots / kWave;
  static constexpr int kVInst = kBK * kVSlots / kWave;
  static constexpr int kKPer = (kKInst + 3) / 4;  // per wave (4 waves)
  static constexpr int kVPer = (kVInst + 3) / 4;
  static_assert(kBK * kKSlots % kWave == 0 && kBK * kVSlots % kWave == 0, "whole instructions");
  // per fill instruction: key row in the high half, element column in the low half
  uint32_t kslot[kKPer], vslot[kVPer];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int slot = kWave * (wave + 4 * j) + lane;
      const int c = slot % kKSlots;
      kslot[j] = (uint32_t)(slot / kKSlots) << 16 | (uint32_t)(c < D / 8 ? c * 8 : 0);
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int slot = kWave * (wave + 4 * j) + lane;
      const int c = slot % kVSlots;
      vslot[j] = (uint32_t)(slot / kVSlots) << 16 | (uint32_t)(c < D / 8 ? c * 8 : 0);
    }
  }
};

template <int D, class Smem>
__device__ __forceinline__ void fill_tile(Smem& sm, int buf, const SegDesc& sg, int tile, int kvh,
                                          int hkv, int mask, int wave, int lane, const FillPlan<D, Smem>& fp) {
  using FP = FillPlan<D, Smem>;
  const int k0 = tile * kBK;
  const int last = min(kBK, sg.len - k0) - 1;
  const uint32_t rs = (uint32_t)hkv * D;  // elements between consecutive keys
  const bf16* kb = reinterpret_cast<const bf16*>(sg.k) + ((int64_t)k0 * hkv + kvh) * D;
  const bf16* vb = reinterpret_cast<const bf16*>(sg.v) + ((int64_t)k0 * hkv + kvh) * D;
  char* kl = reinterpret_cast<char*>(sm.k[buf]);
  char* vl = reinterpret_cast<char*>(sm.v[buf]);
#pragma unroll
  for (int j = 0; j < FP::kKPer; ++j) {
    const int jj = wave + 4 * j;
    if (jj < FP::kKInst) {
      const uint32_t row = min(fp.kslot[j] >> 16, (uint32_t)last);
      global_to_lds16(kb + row * rs + (fp.kslot[j] & 0xffffu), kl + jj * kWave * 16);
    }
  }
#pragma unroll
  for (int j = 0; j < FP::kVPer; ++j) {
    const int jj = wave + 4 * j;
    if (jj < FP::kVInst) {
      const uint32_t row = min(fp.vslot[j] >> 16, (uint32_t)last);
      global_to_lds16(vb + row * rs + (fp.vslot[j] & 0xffffu), vl + jj * kWave * 16);
    }
  }
  if (wave == 0) global_to_lds4(sg.pos + k0 + min(lane, last), sm.kpos[buf]);
  if (wave == 1 && mask == kMaskCausalDoc) global_to_lds4(sg.doc + k0 + min(lane, last), sm.kdoc[buf]);
}

}  // namespace kv
}  // namespace cpattn
