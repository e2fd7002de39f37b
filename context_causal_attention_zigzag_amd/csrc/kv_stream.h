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

// Double-buffered LDS image of one KV tile (kBK keys).  Bank conflicts measured on
// gfx950's 64-bank LDS: 16-byte row reads are conflict-free at a stride of 4 (mod 16)
// dwords (D + 8 or D + 24 elements), transposing reads only at 16 (mod 64) dwords
// (D + 32); the kernels choose the stride per image (see their Smem types).
template <int D, int KS, int VS>
struct KvSmem {
  static constexpr int kKS = KS;
  static constexpr int kVS = VS;
  alignas(16) bf16 k[2][kBK * kKS];
  bf16 v[2][kBK * kVS];
  int32_t kpos[2][kBK];
  int32_t kdoc[2][kBK];
};


// Iterator over the KV tiles one work-group processes.  Positions (and documents) are
// non-decreasing inside a segment, so the tiles a query range can see are one
// contiguous range per segment: lane s of each wave finds segment s's range once by
// binary search (iter_init_lanes), together with a copy of the segment's descriptor,
// and the walk then touches no memory: it reads both back with readlane.  A KV split
// walks the visible tiles of rank [first, first + count) in the same order.
struct TileIter {
  // lane s: segment seg_begin + s
  int rlo, rhi;  // the work-group's visible tiles [rlo, rhi)
  int wlo, whi;  // the tiles this wave computes [wlo, whi)
  int flo, fhi;  // the whole tiles fully visible to every row of the wave [flo, fhi)
  uint32_t k_lo, k_hi, v_lo, v_hi, p_lo, p_hi, d_lo, d_hi;  // descriptor pointers
  int len;
  // walk state (wave-uniform)
  int seg0, tile0;  // first tile of the walk
  int left;         // tiles still to yield
};

// Scan ranges, per-lane segment table and per-wave visibility ranges in one pass.
// Lane s binary-searches segment seg_begin + s for six boundaries at once, each a
// monotone predicate over the tiles (positions and documents are non-decreasing):
//   hi / whi  first tile whose first key lies after the last query of the work-group /
//             of the wave (or in a later document): tiles from there on are invisible;
//   lo / wlo  first tile whose last key is in the first query document of the
//             work-group / of the wave or later (documents only): tiles before it are
//             invisible;
//   fhi       first whole tile whose last key lies after the wave's first query (or in
//             a later document than the wave's first) ...
//   flo       ... and the first tile whose first key is in the wave's query document:
//             tiles in [flo, fhi) are fully visible to every row of the wave (a wave
//             that spans several documents has none).
// [lo, hi) is the work-group's walk; [wlo, whi) the tiles the wave computes at all.
struct VisRanges {
  int lo, hi, wlo, whi, flo, fhi;
};

// Tile boundary table: for every KV tile m of segments [s0, s0 + n) the positions of its
// first and last key and their documents, in the second K/V buffer of the LDS image,
// which nothing writes before the walk's first barrier (every wave reaches it only after
// its boundary searches).  Segment s's tiles start at (s - s0) * stride.  One round of
// independent loads fills it, and the boundary searches then read LDS instead of
// chasing global memory one dependent load at a time.  stride 0: no table (more tiles
// than fit); the searches then read global memory.
struct TileTab {
  int s0;
  int stride;
};

template <class Sm>
struct TabLds {
  static constexpr int kCap = (sizeof(Sm::k) < sizeof(Sm::v) ? sizeof(Sm::k) : sizeof(Sm::v)) / 2 / 8;
  __device__ static int32_t* fpos(Sm& sm) { return reinterpret_cast<int32_t*>(sm.k[1]); }
  __device__ static int32_t* lpos(Sm& sm) { return reinterpret_cast<int32_t*>(sm.k[1]) + kCap; }
  __device__ static int32_t* fdoc(Sm& sm) { return reinterpret_cast<int32_t*>(sm.v[1]); }
  __device__ static int32_t* ldoc(Sm& sm) { return reinterpret_cast<int32_t*>(sm.v[1]) + kCap; }
};

// The launch's segment and job descriptors, one per lane: lane l of every wave holds
// segment l's and job l's fields, fetched by one round of independent loads at kernel
// start.  A thread that needs another entry's field reads it across lanes (ds_bpermute,
// no memory access).  Indexing the argument block with a per-thread index instead
// makes every field a dependent vector load: the prologue's searches and scans then
// waited on chains of three to five memory round trips.
struct LaneDescs {
  uint32_t sk_lo, sk_hi, sv_lo, sv_hi, sp_lo, sp_hi, sd_lo, sd_hi;  // segment: K, V, positions, documents
  int slen;
  uint32_t jp_lo, jp_hi, jd_lo, jd_hi;  // job: positions, documents
  int jlen, jsb, jns, jtps;             // job: rows, first segment, n_split, tiles_per_split
};

__device__ __forceinline__ LaneDescs load_lane_descs(const FwdArgs& a) {
  static_assert(kMaxSegs <= kWave && kMaxJobs <= kWave, "one descriptor per lane");
  const int l = threadIdx.x & (kWave - 1);
  LaneDescs d{};
  if (l < kMaxSegs) {  // entries past the launch's segments are zero
    const SegDesc& sg = a.segs[l];
    const uint64_t k = reinterpret_cast<uint64_t>(sg.k), v = reinterpret_cast<uint64_t>(sg.v);
    const uint64_t p = reinterpret_cast<uint64_t>(sg.pos), dc = reinterpret_cast<uint64_t>(sg.doc);
    d.sk_lo = (uint32_t)k;
    d.sk_hi = (uint32_t)(k >> 32);
    d.sv_lo = (uint32_t)v;
    d.sv_hi = (uint32_t)(v >> 32);
    d.sp_lo = (uint32_t)p;
    d.sp_hi = (uint32_t)(p >> 32);
    d.sd_lo = (uint32_t)dc;
    d.sd_hi = (uint32_t)(dc >> 32);
    d.slen = sg.len;
  }
  if (l < kMaxJobs) {
    const JobDesc& jb = a.jobs[l];
    const uint64_t p = reinterpret_cast<uint64_t>(jb.pos), dc = reinterpret_cast<uint64_t>(jb.doc);
    d.jp_lo = (uint32_t)p;
    d.jp_hi = (uint32_t)(p >> 32);
    d.jd_lo = (uint32_t)dc;
    d.jd_hi = (uint32_t)(dc >> 32);
    d.jlen = jb.len;
    d.jsb = jb.seg_begin;
    d.jns = jb.n_split;
    d.jtps = jb.tiles_per_split;
  }
  return d;
}

// Lane src's value.  Every lane of the wave must execute it, outside any condition:
// a read from a lane that is not active does not return that lane's value.
__device__ __forceinline__ int lane_val(int v, int src) { return __shfl(v, src); }

__device__ __forceinline__ const int32_t* lane_ptr(uint32_t lo, uint32_t hi, int src) {
  return reinterpret_cast<const int32_t*>((uint64_t)(uint32_t)__shfl((int)hi, src) << 32 |
                                          (uint32_t)__shfl((int)lo, src));
}

// Every thread of the work-group calls this with the same arguments.  All table entries
// of a thread are loaded before any is stored, so the table costs one round of loads.
template <int NT, class Sm>
__device__ __forceinline__ TileTab load_tile_table(Sm& sm, const FwdArgs& a, const LaneDescs& ld, int s0, int s1) {
  using T = TabLds<Sm>;
  int stride = 0;
  for (int s = s0; s < s1; ++s) stride = max(stride, (a.segs[s].len + kBK - 1) / kBK);
  if (stride == 0 || (s1 - s0) * stride > T::kCap) return {s0, 0};
  const bool docm = a.mask == kMaskCausalDoc;
  const int n = (s1 - s0) * stride;
  constexpr int kIt = (T::kCap + NT - 1) / NT;
  int fpv[kIt], lpv[kIt], fdv[kIt], ldv[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    if (it * NT < n) {  // uniform: every lane takes part in the cross-lane reads
      const int i = threadIdx.x + it * NT;
      const int sl = min(i / stride, s1 - s0 - 1), m = i - sl * stride;
      const int len = lane_val(ld.slen, s0 + sl);
      const int32_t* pos = lane_ptr(ld.sp_lo, ld.sp_hi, s0 + sl);
      const int32_t* dc = lane_ptr(ld.sd_lo, ld.sd_hi, s0 + sl);
      if (i < n && m * kBK < len) {
        const int f = m * kBK, l = min(len, f + kBK) - 1;
        fpv[it] = pos[f];
        lpv[it] = pos[l];
        if (docm) {
          fdv[it] = dc[f];
          ldv[it] = dc[l];
        }
      }
    }
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    if (it * NT < n) {
      const int i = threadIdx.x + it * NT;
      const int sl = min(i / stride, s1 - s0 - 1), m = i - sl * stride;
      const int len = lane_val(ld.slen, s0 + sl);
      if (i < n && m * kBK < len) {
        T::fpos(sm)[i] = fpv[it];
        T::lpos(sm)[i] = lpv[it];
        if (docm) {
          T::fdoc(sm)[i] = fdv[it];
          T::ldoc(sm)[i] = ldv[it];
        }
      }
    }
  }
  __syncthreads();
  return {s0, stride};
}

// The six boundaries of one segment (see iter_init_lanes) over accessors of its tiles'
// first / last key positions and documents (fp, lp, fd, ld; lp and ld of a full tile are
// its key kBK - 1).
template <class FP, class LP, class FD, class LD>
__device__ __forceinline__ VisRanges vis_search(int nt, int nf, bool docm, int qmax, int qdmin, int qdmax,
                                                bool wave_rows, int wqmin, int wqmax, int wqdmin, int wqdmax,
                                                FP fp, LP lp, FD fd, LD ld) {
  const int wnt = wave_rows ? nt : 0;
  const int wnf = wave_rows && (!docm || wqdmin == wqdmax) ? nf : 0;
  // [l, h) search intervals; the document-only searches start empty without documents
  int l0 = 0, h0 = nt, l1 = 0, h1 = docm ? nt : 0, l2 = 0, h2 = wnt, l3 = 0, h3 = docm ? wnt : 0;
  int l4 = 0, h4 = wnf, l5 = 0, h5 = docm ? wnf : 0;
  while (l0 < h0 || l1 < h1 || l2 < h2 || l3 < h3 || l4 < h4 || l5 < h5) {
    const int m0 = (l0 + h0) >> 1, m1 = (l1 + h1) >> 1, m2 = (l2 + h2) >> 1;
    const int m3 = (l3 + h3) >> 1, m4 = (l4 + h4) >> 1, m5 = (l5 + h5) >> 1;
    bool p0 = false, p1 = false, p2 = false, p3 = false, p4 = false, p5 = false;
    if (l0 < h0) p0 = fp(m0) > qmax || (docm && fd(m0) > qdmax);
    if (l1 < h1) p1 = ld(m1) >= qdmin;
    if (l2 < h2) p2 = fp(m2) > wqmax || (docm && fd(m2) > wqdmax);
    if (l3 < h3) p3 = ld(m3) >= wqdmin;
    if (l4 < h4) p4 = lp(m4) > wqmin || (docm && ld(m4) > wqdmin);
    if (l5 < h5) p5 = fd(m5) >= wqdmin;
    if (l0 < h0) { if (p0) h0 = m0; else l0 = m0 + 1; }
    if (l1 < h1) { if (p1) h1 = m1; else l1 = m1 + 1; }
    if (l2 < h2) { if (p2) h2 = m2; else l2 = m2 + 1; }
    if (l3 < h3) { if (p3) h3 = m3; else l3 = m3 + 1; }
    if (l4 < h4) { if (p4) h4 = m4; else l4 = m4 + 1; }
    if (l5 < h5) { if (p5) h5 = m5; else l5 = m5 + 1; }
  }
  return {l1, l0, l3, l2, l5, l4};
}

template <class Sm>
__device__ __forceinline__ void iter_init_lanes(TileIter& it, const FwdArgs& a, const LaneDescs& ld,
                                                const JobDesc& job, int lane, int qmax, int qdmin, int qdmax,
                                                bool wave_rows, int wqmin, int wqmax, int wqdmin, int wqdmax, Sm& sm,
                                                TileTab tt) {
  // lane s takes segment seg_begin + s of the job from the lane that holds it (every
  // lane reads: a cross-lane read does not see the value of a lane that is not active)
  const int src = min(job.seg_begin + lane, kMaxSegs - 1);
  const bool mine = lane < job.seg_end - job.seg_begin;
  const int slen = lane_val(ld.slen, src);
  const int len = mine ? slen : 0;
  const uint64_t kp = reinterpret_cast<uint64_t>(lane_ptr(ld.sk_lo, ld.sk_hi, src));
  const uint64_t vp = reinterpret_cast<uint64_t>(lane_ptr(ld.sv_lo, ld.sv_hi, src));
  const uint64_t pp = reinterpret_cast<uint64_t>(lane_ptr(ld.sp_lo, ld.sp_hi, src));
  const uint64_t dp = reinterpret_cast<uint64_t>(lane_ptr(ld.sd_lo, ld.sd_hi, src));
  VisRanges r = {0, 0, 0, 0, 0, 0};
  if (mine) {
    const int nt = (len + kBK - 1) / kBK, nf = len / kBK;
    const bool docm = a.mask == kMaskCausalDoc;
    const int wnt = wave_rows ? nt : 0;
    const int wnf = wave_rows && (!docm || wqdmin == wqdmax) ? nf : 0;
    r = {0, nt, 0, wnt, 0, wnf};
    if (a.mask != kMaskNone) {
      if (tt.stride > 0) {
        using T = TabLds<Sm>;
        const int b = (job.seg_begin + lane - tt.s0) * tt.stride;
        const int32_t* f = T::fpos(sm) + b;
        const int32_t* l = T::lpos(sm) + b;
        const int32_t* fdc = T::fdoc(sm) + b;
        const int32_t* ldc = T::ldoc(sm) + b;
        r = vis_search(nt, nf, docm, qmax, qdmin, qdmax, wave_rows, wqmin, wqmax, wqdmin, wqdmax,
                       [&](int m) { return f[m]; }, [&](int m) { return l[m]; },
                       [&](int m) { return fdc[m]; }, [&](int m) { return ldc[m]; });
      } else {
        const int32_t* pos = reinterpret_cast<const int32_t*>(pp);
        const int32_t* dc = reinterpret_cast<const int32_t*>(dp);
        r = vis_search(nt, nf, docm, qmax, qdmin, qdmax, wave_rows, wqmin, wqmax, wqdmin, wqdmax,
                       [&](int m) { return pos[m * kBK]; }, [&](int m) { return pos[min(len, m * kBK + kBK) - 1]; },
                       [&](int m) { return dc[m * kBK]; }, [&](int m) { return dc[min(len, m * kBK + kBK) - 1]; });
      }
    }
  }
  it.rlo = r.lo;
  it.rhi = r.hi;
  it.wlo = r.wlo;
  it.whi = r.whi;
  it.flo = r.flo;
  it.fhi = r.fhi;
  it.len = len;
  it.k_lo = (uint32_t)kp;
  it.k_hi = (uint32_t)(kp >> 32);
  it.v_lo = (uint32_t)vp;
  it.v_hi = (uint32_t)(vp >> 32);
  it.p_lo = (uint32_t)pp;
  it.p_hi = (uint32_t)(pp >> 32);
  it.d_lo = (uint32_t)dp;
  it.d_hi = (uint32_t)(dp >> 32);
}

// One visible tile with its segment's data resolved from the per-lane table
// (wave-uniform values; the pointers address the tile's first key).
struct KvTile {
  const bf16* k;
  const bf16* v;
  const int32_t* pos;
  const int32_t* doc;
  int last;    // index of the tile's last key (tile length - 1)
  bool full;   // every key visible to every row of the wave (and a whole tile)
  bool empty;  // no key visible to any row of the wave
};

__device__ __forceinline__ uint64_t lane_u64(uint32_t lo, uint32_t hi, int s) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, s) << 32 | (uint32_t)__builtin_amdgcn_readlane(lo, s);
}

__device__ __forceinline__ KvTile iter_tile(const TileIter& it, TileRef r, int seg_begin, int kvh, int hkv, int D) {
  const int s = r.seg - seg_begin;
  const int k0 = r.tile * kBK;
  const int64_t eoff = ((int64_t)k0 * hkv + kvh) * D;
  KvTile t;
  t.k = reinterpret_cast<const bf16*>(lane_u64(it.k_lo, it.k_hi, s)) + eoff;
  t.v = reinterpret_cast<const bf16*>(lane_u64(it.v_lo, it.v_hi, s)) + eoff;
  t.pos = reinterpret_cast<const int32_t*>(lane_u64(it.p_lo, it.p_hi, s)) + k0;
  t.doc = reinterpret_cast<const int32_t*>(lane_u64(it.d_lo, it.d_hi, s)) + k0;
  t.last = min(kBK, __builtin_amdgcn_readlane(it.len, s) - k0) - 1;
  t.full = r.tile >= __builtin_amdgcn_readlane(it.flo, s) && r.tile < __builtin_amdgcn_readlane(it.fhi, s);
  t.empty = r.tile < __builtin_amdgcn_readlane(it.wlo, s) || r.tile >= __builtin_amdgcn_readlane(it.whi, s);
  return t;
}

// Visibility of this lane's 16 raw scores of key half kb (keys 32 kb .. 32 kb + 31) of
// a partially visible tile (positions kp / documents kd in LDS, klen keys) for query
// position qpos / document qdoc: invisible scores become -inf.  Branch-free (the
// document image is read even when documents are off; its value is then ignored).
__device__ __forceinline__ void mask_half(f32x16& x, const int32_t* kp, const int32_t* kd, int klen, int qpos,
                                          int qdoc, int mask, int h, int kb) {
  const int qp = mask == kMaskNone ? 0x7fffffff : qpos;
  const bool docm = mask == kMaskCausalDoc;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int base = kb * 32 + 8 * g + 4 * h;
    const int4 kpv = *reinterpret_cast<const int4*>(kp + base);
    const int4 kdv = *reinterpret_cast<const int4*>(kd + base);
    const int kpa[4] = {kpv.x, kpv.y, kpv.z, kpv.w};
    const int kda[4] = {kdv.x, kdv.y, kdv.z, kdv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool vis = (base + e < klen) & (kpa[e] <= qp) & (!docm | (kda[e] == qdoc));
      x[g * 4 + e] = vis ? x[g * 4 + e] : neg_inf();
    }
  }
}

// Direct global->LDS fill of one KV tile into a KvSmem image, from a resolved tile.
// The image is a sequence of 16-byte slots (row-major, kKS / 8 or kVS / 8 slots per
// key row, the last ones padding); fill instruction jj of the work-group writes slots
// 64 jj .. 64 jj + 63, lane l slot 64 jj + l.  Per fill instruction each lane's source
// is a fixed offset from the tile's first key (key row * row stride + column; padding
// slots load a valid dummy chunk), clamped to that of key `last`'s last chunk: rows up
// to the tile's last key stay exact, rows after it (ragged tile) read the last chunk
// of key `last` (finite data; those keys are masked).
//
// Two forms of the per-lane offsets.  Full (kCompact false): the byte offsets, one
// register per fill instruction of the wave, computed once and hidden from the
// compiler, which otherwise recomputes their divisions at every tile to save the
// registers (about a dozen vector instructions per fill, in the forward kernel).
// Compact: 16-bit (row, column) entries, two per register, the offset formed at fill
// time -- for the dQ kernel, which holds them without recomputing and has no registers
// to spare (the full form made its 8K pass 3-5% slower).
template <int D, class Smem, int kWaves = 4, bool kCompact = false>
struct FillOffs {
  static constexpr int kKSlots = Smem::kKS / 8;
  static constexpr int kVSlots = Smem::kVS / 8;
  static constexpr int kKInst = kBK * kKSlots / kWave;
  static constexpr int kVInst = kBK * kVSlots / kWave;
  static constexpr int kKPer = (kKInst + kWaves - 1) / kWaves;  // per wave
  static constexpr int kVPer = (kVInst + kWaves - 1) / kWaves;
  static_assert(kBK * kKSlots % kWave == 0 && kBK * kVSlots % kWave == 0, "whole instructions");
  static_assert(D <= 256, "column offsets fit a byte");
  static constexpr int kKReg = kCompact ? (kKPer + 1) / 2 : kKPer;
  static constexpr int kVReg = kCompact ? (kVPer + 1) / 2 : kVPer;
  uint32_t ko[kKReg], vo[kVReg];

  // (row, column) of a slot: row in bits 8..13, element column in bits 0..7
  static __device__ __forceinline__ uint32_t entry(int slot, int slots) {
    const int c = slot % slots;
    return (uint32_t)min(slot / slots, kBK - 1) << 8 | (uint32_t)(c < D / 8 ? c * 8 : 0);
  }
  // element offset of an entry, rs: elements between consecutive keys
  static __device__ __forceinline__ uint32_t elems(uint32_t e, uint32_t rs) { return __umul24(e >> 8, rs) + (e & 0xffu); }
  __device__ __forceinline__ void init(int wave, int lane, uint32_t rs) {
    if (kCompact) {
#pragma unroll
      for (int j = 0; j < kKReg; ++j) ko[j] = 0;
#pragma unroll
      for (int j = 0; j < kVReg; ++j) vo[j] = 0;
#pragma unroll
      for (int j = 0; j < kKPer; ++j) ko[j >> 1] |= entry(kWave * (wave + kWaves * j) + lane, kKSlots) << (16 * (j & 1));
#pragma unroll
      for (int j = 0; j < kVPer; ++j) vo[j >> 1] |= entry(kWave * (wave + kWaves * j) + lane, kVSlots) << (16 * (j & 1));
    } else {
#pragma unroll
      for (int j = 0; j < kKReg; ++j) {
        ko[j] = elems(entry(kWave * (wave + kWaves * j) + lane, kKSlots), rs) * 2;
        asm volatile("" : "+v"(ko[j]));
      }
#pragma unroll
      for (int j = 0; j < kVReg; ++j) {
        vo[j] = elems(entry(kWave * (wave + kWaves * j) + lane, kVSlots), rs) * 2;
        asm volatile("" : "+v"(vo[j]));
      }
    }
  }
  // offset of fill j of the K (or V) image: elements (compact), bytes (full)
  __device__ __forceinline__ uint32_t koff(int j, uint32_t rs) const {
    return kCompact ? elems((ko[j >> 1] >> (16 * (j & 1))) & 0xffffu, rs) : ko[j];
  }
  __device__ __forceinline__ uint32_t voff(int j, uint32_t rs) const {
    return kCompact ? elems((vo[j >> 1] >> (16 * (j & 1))) & 0xffffu, rs) : vo[j];
  }
};

// Full form: every offset is clamped into a register of its own before the burst (an
// instruction that overwrites the address register of a fill still waiting for the
// memory pipeline stalls until that fill has read it, so a burst that reuses one
// register would be serialised).  Compact form: each fill's address is formed as it
// is issued.
template <int D, class Smem, int kWaves, bool kCompact>
__device__ __forceinline__ void fill_tile(Smem& sm, int buf, const KvTile& t, uint32_t rs, bool doc, int wave,
                                          int lane, const FillOffs<D, Smem, kWaves, kCompact>& fo) {
  using FO = FillOffs<D, Smem, kWaves, kCompact>;
  const uint32_t kl = lds_offset(sm.k[buf]), vl = lds_offset(sm.v[buf]);
  if constexpr (kCompact) {
    const uint32_t cap = (uint32_t)t.last * rs + D - 8;  // elements
#pragma unroll
    for (int j = 0; j < FO::kKPer; ++j) {
      const int jj = wave + kWaves * j;
      if (jj < FO::kKInst) fill16_untracked(t.k + min(fo.koff(j, rs), cap), kl + jj * kWave * 16);
    }
#pragma unroll
    for (int j = 0; j < FO::kVPer; ++j) {
      const int jj = wave + kWaves * j;
      if (jj < FO::kVInst) fill16_untracked(t.v + min(fo.voff(j, rs), cap), vl + jj * kWave * 16);
    }
  } else {
    __builtin_assume(wave >= 0 && wave < kWaves);
    const uint32_t cap = ((uint32_t)t.last * rs + D - 8) * 2;  // bytes
    const bf16* kb = uniform_ptr(t.k);
    const bf16* vb = uniform_ptr(t.v);
    uint32_t ko[FO::kKPer], vo[FO::kVPer];
#pragma unroll
    for (int j = 0; j < FO::kKPer; ++j) {
      ko[j] = min(fo.koff(j, rs), cap);
      asm volatile("" : "+v"(ko[j]));
    }
#pragma unroll
    for (int j = 0; j < FO::kVPer; ++j) {
      vo[j] = min(fo.voff(j, rs), cap);
      asm volatile("" : "+v"(vo[j]));
    }
#pragma unroll
    for (int j = 0; j < FO::kKPer; ++j) {
      const int jj = wave + kWaves * j;
      if (jj < FO::kKInst) fill16_off(kb, ko[j], kl + jj * kWave * 16);
    }
#pragma unroll
    for (int j = 0; j < FO::kVPer; ++j) {
      const int jj = wave + kWaves * j;
      if (jj < FO::kVInst) fill16_off(vb, vo[j], vl + jj * kWave * 16);
    }
#pragma unroll
    for (int j = 0; j < FO::kKPer; ++j) asm volatile("" ::"v"(ko[j]));
#pragma unroll
    for (int j = 0; j < FO::kVPer; ++j) asm volatile("" ::"v"(vo[j]));
  }
  if (wave == 0) fill4_untracked(t.pos + min(lane, t.last), lds_offset(sm.kpos[buf]));
  if (wave == 1 && doc) fill4_untracked(t.doc + min(lane, t.last), lds_offset(sm.kdoc[buf]));
}

// Walk every visible tile of the job.
__device__ __forceinline__ void iter_walk_all(TileIter& it, const JobDesc& job) {
  it.seg0 = job.seg_begin;
  it.tile0 = __builtin_amdgcn_readlane(it.rlo, 0);
  it.left = 0x7fffffff;
}

// Walk the visible tiles of rank [first, first + count) (in segment, then tile order);
// false when there are not more than `first` of them.
__device__ __forceinline__ bool iter_walk_split(TileIter& it, const JobDesc& job, int first, int count) {
  int before = 0;
  for (int s = job.seg_begin; s < job.seg_end; ++s) {
    const int lo = __builtin_amdgcn_readlane(it.rlo, s - job.seg_begin);
    const int n = max(0, __builtin_amdgcn_readlane(it.rhi, s - job.seg_begin) - lo);
    if (first < before + n) {
      it.seg0 = s;
      it.tile0 = lo + (first - before);
      it.left = count;
      return true;
    }
    before += n;
  }
  return false;
}

// Next tile after `prev` ({-1, 0}: the first), or {-1, 0} at the end of the walk.
__device__ __forceinline__ TileRef iter_next(TileIter& it, const JobDesc& job, TileRef prev) {
  if (it.left == 0) return {-1, 0};
  int s = prev.seg < 0 ? it.seg0 : prev.seg;
  int t = prev.seg < 0 ? it.tile0 : prev.tile + 1;
  while (s < job.seg_end) {
    if (t < __builtin_amdgcn_readlane(it.rhi, s - job.seg_begin)) {
      --it.left;
      return {s, t};
    }
    ++s;
    if (s < job.seg_end) t = __builtin_amdgcn_readlane(it.rlo, s - job.seg_begin);
  }
  return {-1, 0};
}

// ---------------------------------------------------------------------------
// Work-group -> work item (job, head group, query tile, KV split).
struct WorkItem {
  int job, hg, qt, split;
};

// Index order.  The dispatcher hands work-group b to XCD b % 8, and each XCD starts its
// work-groups in order as CUs free up.  Inside a job the head groups are outermost and
// the query tiles run latest first: in a causal zigzag share the later tiles see more
// keys, so every XCD starts its heaviest tiles first.  When the head groups divide by 8
// (no padding then), XCD x takes head groups [x*hpx, (x+1)*hpx) of every job, so a
// launch of several jobs of unequal weight (the edges of the tile form) gives every
// XCD the same share of each; otherwise each XCD takes one contiguous logical range
// (xcd_remap).  For a single job the two orders coincide.  job = -1: a padding
// work-group.
__device__ __forceinline__ WorkItem indexed_work_item(const FwdArgs& a, int qt_rows) {
  WorkItem w{-1, 0, 0, 0};
  const int n_hg = a.hq / a.heads_per_wg;
  if ((n_hg & 7) == 0) {
    const int hpx = n_hg >> 3;
    int i = blockIdx.x >> 3, j = 0, n_qt, nsplit;
    while (true) {
      n_qt = (a.jobs[j].len + qt_rows - 1) / qt_rows;
      nsplit = a.jobs[j].n_split;
      if (i < n_qt * nsplit * hpx) break;
      i -= n_qt * nsplit * hpx;
      ++j;
    }
    const int hl = i / (n_qt * nsplit);
    const int k = i - hl * (n_qt * nsplit);
    w.job = j;
    w.split = k % nsplit;
    w.qt = n_qt - 1 - k / nsplit;
    w.hg = (blockIdx.x & 7) * hpx + hl;
    return w;
  }
  const int logical = xcd_remap(blockIdx.x, a.padded_wgs);
  if (logical >= a.total_wgs) return w;
  int j = 0;
  while (j + 1 < a.n_jobs && a.jobs[j + 1].wg_begin <= logical) ++j;
  const JobDesc& job = a.jobs[j];
  const int n_qt = (job.len + qt_rows - 1) / qt_rows;
  const int nsplit = job.n_split;
  const int local = logical - job.wg_begin;
  w.job = j;
  w.split = local % nsplit;
  const int rest = local / nsplit;
  w.hg = rest / n_qt;
  w.qt = n_qt - 1 - (rest - w.hg * n_qt);
  return w;
}

// Ranked order, for packed documents: a query tile's work follows the lengths of the
// documents it falls in, not its index.
constexpr int kMaxRankedTiles = 1024;
// A ranked launch with more query tiles, or with many rounds of work-groups, is planned
// once by a single work-group (plan_ranked_kernel) when the workspace has room.
constexpr int kMaxPlanTiles = 4096;

// The launch ranks when the head groups split evenly over the 8 XCDs, no job has KV
// splits and the jobs hold 1..kMaxRankedTiles query tiles in all; then every logical
// work item is one (head group, job, query tile) and the grid needs no padding.
inline bool ranked_plan(const FwdArgs& a, int qt_rows, int cap = kMaxRankedTiles) {
  if (a.mask != kMaskCausalDoc || (a.hq / a.heads_per_wg) % 8 != 0) return false;
  int n_all = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    if (a.jobs[j].n_split != 1) return false;
    n_all += (a.jobs[j].len + qt_rows - 1) / qt_rows;
  }
  return n_all > 0 && n_all <= cap;
}

// Entries per array of the KV tile table in LDS: the kernels' smaller K/V image has a
// row stride of d + 8 elements (TabLds::kCap).
inline int tile_tab_cap(int d) { return 16 * (d + 8); }

// Layout of a ranked launch's plan: n_all ints of rank order (padded to 64), then the
// tile table's four arrays of n_tab entries (first / last key position, first / last
// key document of every KV tile of segments [0, s1)); n_tab = 0 when the table does
// not fit in LDS (the kernels then search global memory).
inline void plan_layout(const FwdArgs& a, int d, int qt_rows, int& n_all, int& n_tab) {
  n_all = 0;
  int s1 = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    n_all += (a.jobs[j].len + qt_rows - 1) / qt_rows;
    s1 = s1 > a.jobs[j].seg_end ? s1 : a.jobs[j].seg_end;
  }
  int stride = 0;
  for (int s = 0; s < s1; ++s) {
    const int nt = (a.segs[s].len + kBK - 1) / kBK;
    stride = stride > nt ? stride : nt;
  }
  n_tab = (stride > 0 && s1 * stride <= tile_tab_cap(d)) ? s1 * stride : 0;
}

inline size_t plan_bytes(int n_all, int n_tab) {
  return (size_t)(((n_all + 63) & ~63) + 4 * n_tab) * sizeof(int32_t);
}

// KV tiles the work-group of query rows [r0, r1) walks in one segment of nt tiles: from
// the first tile that reaches the rows' first document to the first tile past their
// last position or document (the boundaries the tile iterators find for the
// work-group), over accessors of the tiles' first key position / document and last
// key document.
template <class FP, class FD, class LD>
__device__ __forceinline__ int walk_tiles(int nt, int qmax, int qdmin, int qdmax, FP fp, FD fd, LD ld) {
  int l0 = 0, h0 = nt, l1 = 0, h1 = nt;
  while (l0 < h0 || l1 < h1) {
    const int m0 = (l0 + h0) >> 1, m1 = (l1 + h1) >> 1;
    if (l0 < h0) {
      if (fp(m0) > qmax || fd(m0) > qdmax) h0 = m0; else l0 = m0 + 1;
    }
    if (l1 < h1) {
      if (ld(m1) >= qdmin) h1 = m1; else l1 = m1 + 1;
    }
  }
  return max(0, l0 - l1);
}

// Visible KV tiles of query rows [.., qmax] (documents [qdmin, qdmax]) in one segment of
// nt tiles, the count the tile iterators walk: from the first tile that reaches the
// rows' first document (documents only) to the first tile past their last position or
// document.
template <class FP, class FD, class LD>
__device__ __forceinline__ int visible_tiles(int nt, bool docm, int qmax, int qdmin, int qdmax, FP fp, FD fd, LD ld) {
  if (docm) return walk_tiles(nt, qmax, qdmin, qdmax, fp, fd, ld);
  int l0 = 0, h0 = nt;
  while (l0 < h0) {
    const int m0 = (l0 + h0) >> 1;
    if (fp(m0) > qmax) h0 = m0; else l0 = m0 + 1;
  }
  return l0;
}

// (job, query tile, segment) triple k of the launch, jobs in order, segments inner
// (job -1: k is past the last triple).  A uniform loop over the jobs, so their
// descriptors come from scalar loads.
struct PairRef {
  int job, base, q, sidx;  // base: index of the job's first query tile over all jobs
};

__device__ __forceinline__ PairRef pair_at(const FwdArgs& a, int qt_rows, int k) {
  PairRef p{-1, 0, 0, 0};
  int acc = 0, base = 0, nseg = 1, kk = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    const int n_qt = (a.jobs[j].len + qt_rows - 1) / qt_rows;
    const int ns = a.jobs[j].seg_end - a.jobs[j].seg_begin;
    const int n = n_qt * ns;
    if (p.job < 0 && k >= acc && k < acc + n) {
      p.job = j;
      p.base = base;
      kk = k - acc;
      nseg = ns;
    }
    acc += n;
    base += n_qt;
  }
  p.q = kk / nseg;
  p.sidx = kk - p.q * nseg;
  return p;
}

// For every query tile t (over all jobs) the number of KV tiles its work-group walks,
// summed over the job's segments, in scratch[t]; returns the number of query tiles.
// Loads the tile table of every segment of the launch into tt.  Every thread calls
// this; scratch holds kMaxRankedTiles + 8 ints of LDS outside the table.  The first
// triple of each thread and its query tile's ends are loaded before the table, so the
// two rounds of loads overlap.
template <int NT, class Sm>
__device__ __forceinline__ int count_visible(const FwdArgs& a, const LaneDescs& ld, int qt_rows, int* scratch,
                                             Sm& sm, TileTab& tt) {
  const int tid = threadIdx.x;
  const bool docm = a.mask == kMaskCausalDoc;
  int n_all = 0, n_pairs = 0, s1 = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    const int n_qt = (a.jobs[j].len + qt_rows - 1) / qt_rows;
    n_all += n_qt;
    n_pairs += n_qt * (a.jobs[j].seg_end - a.jobs[j].seg_begin);
    s1 = max(s1, a.jobs[j].seg_end);
  }
  const int iters = (n_pairs + NT - 1) / NT;
  // values of this thread's triple k = tid + it * NT: query tile ends, segment
  int qmax = 0, qdmin = 0, qdmax = 0, seg = 0, slot = 0;
  auto prepare = [&](int it) {  // every lane calls this (cross-lane reads)
    const int k = tid + it * NT;
    const PairRef p = pair_at(a, qt_rows, k);
    const int jj = max(p.job, 0);
    const int len = lane_val(ld.jlen, jj);
    const int32_t* pos = lane_ptr(ld.jp_lo, ld.jp_hi, jj);
    const int32_t* dc = lane_ptr(ld.jd_lo, ld.jd_hi, jj);
    seg = min(lane_val(ld.jsb, jj) + p.sidx, kMaxSegs - 1);
    slot = p.base + p.q;
    if (p.job >= 0) {
      const int r0 = p.q * qt_rows, r1 = min(len, r0 + qt_rows);
      qmax = pos[r1 - 1];
      if (docm) {
        qdmin = dc[r0];
        qdmax = dc[r1 - 1];
      }
    }
  };
  if (iters > 0) prepare(0);
  for (int t = tid; t < n_all; t += NT) scratch[t] = 0;
  tt = load_tile_table<NT>(sm, a, ld, 0, s1);  // ends with a barrier
  for (int it = 0; it < iters; ++it) {
    if (it > 0) prepare(it);
    const int nt = (lane_val(ld.slen, seg) + kBK - 1) / kBK;
    const int32_t* spos = lane_ptr(ld.sp_lo, ld.sp_hi, seg);
    const int32_t* sdoc = lane_ptr(ld.sd_lo, ld.sd_hi, seg);
    const int slen = lane_val(ld.slen, seg);
    if (tid + it * NT < n_pairs) {
      int c;
      if (tt.stride > 0) {
        using T = TabLds<Sm>;
        const int b = (seg - tt.s0) * tt.stride;
        const int32_t* f = T::fpos(sm) + b;
        const int32_t* fdc = T::fdoc(sm) + b;
        const int32_t* ldc = T::ldoc(sm) + b;
        c = visible_tiles(nt, docm, qmax, qdmin, qdmax, [&](int m) { return f[m]; },
                          [&](int m) { return fdc[m]; }, [&](int m) { return ldc[m]; });
      } else {
        c = visible_tiles(nt, docm, qmax, qdmin, qdmax, [&](int m) { return spos[m * kBK]; },
                          [&](int m) { return sdoc[m * kBK]; },
                          [&](int m) { return sdoc[min(slen, m * kBK + kBK) - 1]; });
      }
      if (c) atomicAdd(&scratch[slot], c);
    }
  }
  __syncthreads();
  return n_all;
}

// Work-group b runs on XCD b % 8, which takes head groups [x*hpx, (x+1)*hpx) of every
// job, hpx = head groups / 8.  Every work-group counts, for every query tile of every
// job, the KV tiles that tile's work-group walks, ranks the (job, tile) pairs by that
// count (most first; ties: the later pair first) and takes the pair of rank (b / 8) /
// hpx, head group (b / 8) % hpx of its XCD's block: each XCD's list is then the
// longest-processing-time-first schedule of its share, its head groups inner.  Every
// thread of the work-group calls this; scratch holds kMaxRankedTiles + 8 ints of LDS
// that nothing else uses yet.
template <int NT, class Sm>
__device__ __forceinline__ WorkItem ranked_work_item(const FwdArgs& a, const LaneDescs& ld, int qt_rows,
                                                     int* scratch, Sm& sm, TileTab& tt) {
  const int b = blockIdx.x;
  const int hpx = (a.hq / a.heads_per_wg) >> 3;
  const int i = b >> 3;
  const int rank = i / hpx;
  WorkItem w;
  w.split = 0;
  w.hg = (b & 7) * hpx + (i - rank * hpx);
  const int tid = threadIdx.x;
  const int n_all = count_visible<NT, Sm>(a, ld, qt_rows, scratch, sm, tt);
  // rank of pair t = pairs with a larger count, plus pairs with the same count and a
  // larger index; every thread reads the counts four at a time (16-byte LDS reads, four
  // in flight), the list padded with -1 (no count is negative)
  const int n4 = (n_all + 3) & ~3;
  for (int t = n_all + tid; t < n4; t += NT) scratch[t] = -1;
  __syncthreads();
  const int4* s4 = reinterpret_cast<const int4*>(scratch);
  for (int t = tid; t < n_all; t += NT) {
    const int c = scratch[t];
    int r = 0;
#pragma unroll 4
    for (int p4 = 0; p4 < n4 / 4; ++p4) {
      const int4 v = s4[p4];
      const int p = 4 * p4;
      r += (v.x > c) | ((v.x == c) & (p > t));
      r += (v.y > c) | ((v.y == c) & (p + 1 > t));
      r += (v.z > c) | ((v.z == c) & (p + 2 > t));
      r += (v.w > c) | ((v.w == c) & (p + 3 > t));
    }
    if (r == rank) scratch[n4] = t;
  }
  __syncthreads();
  int t = __builtin_amdgcn_readfirstlane(scratch[n4]);
  __syncthreads();  // scratch free again
  int j = 0;
  while (t >= (a.jobs[j].len + qt_rows - 1) / qt_rows) {
    t -= (a.jobs[j].len + qt_rows - 1) / qt_rows;
    ++j;
  }
  w.job = j;
  w.qt = t;
  return w;
}

// The work item of a planned ranked launch: its pair from the plan's rank order (the
// same order ranked_work_item computes), and the tile table copied from the plan into
// LDS with coalesced loads, all of a thread's loads issued before any store.
template <int NT, class Sm>
__device__ __forceinline__ WorkItem planned_work_item(const FwdArgs& a, int qt_rows, Sm& sm, TileTab& tt) {
  using T = TabLds<Sm>;
  const int b = blockIdx.x;
  const int hpx = (a.hq / a.heads_per_wg) >> 3;
  const int i = b >> 3;
  const int rank = i / hpx;
  WorkItem w;
  w.split = 0;
  w.hg = (b & 7) * hpx + (i - rank * hpx);
  int n_all = 0, s1 = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    n_all += (a.jobs[j].len + qt_rows - 1) / qt_rows;
    s1 = max(s1, a.jobs[j].seg_end);
  }
  int t = a.plan[rank];
  int stride = 0;
  for (int s = 0; s < s1; ++s) stride = max(stride, (a.segs[s].len + kBK - 1) / kBK);
  const int n_tab = (stride > 0 && s1 * stride <= T::kCap) ? s1 * stride : 0;
  tt = {0, n_tab > 0 ? stride : 0};
  if (n_tab > 0) {
    const bool docm = a.mask == kMaskCausalDoc;
    const int32_t* tab = a.plan + ((n_all + 63) & ~63);
    constexpr int kIt = (T::kCap + NT - 1) / NT;
    int v[kIt][4];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int e = threadIdx.x + it * NT;
      if (it * NT < n_tab && e < n_tab) {
        v[it][0] = tab[e];
        v[it][1] = tab[n_tab + e];
        if (docm) {
          v[it][2] = tab[2 * n_tab + e];
          v[it][3] = tab[3 * n_tab + e];
        }
      }
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int e = threadIdx.x + it * NT;
      if (it * NT < n_tab && e < n_tab) {
        T::fpos(sm)[e] = v[it][0];
        T::lpos(sm)[e] = v[it][1];
        if (docm) {
          T::fdoc(sm)[e] = v[it][2];
          T::ldoc(sm)[e] = v[it][3];
        }
      }
    }
  }
  __syncthreads();
  t = __builtin_amdgcn_readfirstlane(t);
  int j = 0;
  while (t >= (a.jobs[j].len + qt_rows - 1) / qt_rows) {
    t -= (a.jobs[j].len + qt_rows - 1) / qt_rows;
    ++j;
  }
  w.job = j;
  w.qt = t;
  return w;
}

// The plan of a ranked launch, built once: one work-group counts every (job, query
// tile)'s visible KV tiles exactly as ranked_work_item does, sorts the pairs by
// (count, index), largest first (bitonic sort in LDS), and writes the order and the tile
// table to a.plan.  qt_rows as in the launch it plans.
template <int D>
struct PlanSmem {
  KvSmem<D, D + 8, D + 8> kv;  // the tile table lives in its second K/V images
  alignas(16) int32_t cnt[kMaxPlanTiles + 8];
  alignas(16) uint64_t key[kMaxPlanTiles];
};

constexpr int kPlanThreads = 1024;

template <int D>
__global__ __launch_bounds__(kPlanThreads) void plan_ranked_kernel(FwdArgs a, int qt_rows) {
  using Sm = KvSmem<D, D + 8, D + 8>;
  using T = TabLds<Sm>;
  __shared__ PlanSmem<D> ps;
  const int tid = threadIdx.x;
  const LaneDescs ld = load_lane_descs(a);
  TileTab tt{0, 0};
  const int n_all = count_visible<kPlanThreads, Sm>(a, ld, qt_rows, ps.cnt, ps.kv, tt);
  // the tile table, as the launch's work-groups would load it
  int s1 = 0;
  for (int j = 0; j < a.n_jobs; ++j) s1 = max(s1, a.jobs[j].seg_end);
  const int n_tab = tt.stride > 0 ? s1 * tt.stride : 0;
  int32_t* tab = a.plan + ((n_all + 63) & ~63);
  const bool docm = a.mask == kMaskCausalDoc;
  for (int e = tid; e < n_tab; e += kPlanThreads) {
    tab[e] = T::fpos(ps.kv)[e];
    tab[n_tab + e] = T::lpos(ps.kv)[e];
    if (docm) {
      tab[2 * n_tab + e] = T::fdoc(ps.kv)[e];
      tab[3 * n_tab + e] = T::ldoc(ps.kv)[e];
    }
  }
  // keys (count + 1, index): descending order is the rank order; padding keys are 0
  int n2 = 1;
  while (n2 < n_all) n2 <<= 1;
  for (int t = tid; t < n2; t += kPlanThreads)
    ps.key[t] = t < n_all ? ((uint64_t)(uint32_t)(ps.cnt[t] + 1) << 32 | (uint32_t)t) : 0ull;
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int t = tid; t < n2; t += kPlanThreads) {
        const int u = t ^ jj;
        if (u > t) {
          const uint64_t x = ps.key[t], y = ps.key[u];
          const bool desc = (t & k) == 0;
          if (desc ? x < y : x > y) {
            ps.key[t] = y;
            ps.key[u] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < n_all; r += kPlanThreads) a.plan[r] = (int32_t)(uint32_t)ps.key[r];
}

// Work items of a launch whose jobs are split over KV tiles, numbered densely over the
// splits that exist.  A query tile that sees V of its job's KV tiles needs
// ns = ceil(V / tiles_per_split) splits (at least one, which finds nothing when V = 0);
// the grid holds the plan's upper bound n_split per query tile.  Numbering only the
// splits that exist puts the surplus work-groups, which leave at once, after all the
// real ones in dispatch order: interleaved among them, they made the dispatcher place
// later real work-groups on compute units that were already full, while others held a
// single work-group (measured: the last ones started up to 50 us late at 8K).
// Order: as indexed_work_item (head-group blocks per XCD when the head groups divide
// by 8, else contiguous ranges), query tiles latest first, splits inner.
// Every thread calls this; it loads the tile table of every segment of the launch
// (returned in tt) and uses scratch, 2 * kMaxRankedTiles + 16 ints of LDS outside the
// table that nothing uses yet.  job = -1: surplus.

template <int NT, class Sm>
__device__ __forceinline__ WorkItem compact_work_item(const FwdArgs& a, const LaneDescs& ld, int qt_rows,
                                                      int* scratch, Sm& sm, TileTab& tt, int& ns_out) {
  const int tid = threadIdx.x;
  const int n_all = count_visible<NT, Sm>(a, ld, qt_rows, scratch, sm, tt);
  const int n_hg = a.hq / a.heads_per_wg;
  const int b = blockIdx.x;
  if (n_all <= kWave) {
    // one wave: lane t holds query tile t (over all jobs); the splits of its job's later
    // query tiles come from a segmented suffix scan across the lanes
    if (tid < kWave) {
      const int t = tid;
      const bool have = t < n_all;
      int jt = 0, tb = 0, acc = 0;
      for (int j = 0; j < a.n_jobs; ++j) {
        if (t >= acc) {
          jt = j;
          tb = acc;
        }
        acc += (a.jobs[j].len + qt_rows - 1) / qt_rows;
      }
      const int jlen = lane_val(ld.jlen, jt), jns = lane_val(ld.jns, jt), jtps = lane_val(ld.jtps, jt);
      const int te = have ? tb + (jlen + qt_rows - 1) / qt_rows - 1 : t;  // the job's last query tile
      int ns = 0;
      if (have) {
        const int v = scratch[t];
        ns = jns > 1 ? max(1, (v + jtps - 1) / jtps) : 1;
      }
      int suf = ns;  // splits of query tiles t .. te
#pragma unroll
      for (int dl = 1; dl < kWave; dl <<= 1) {
        const int o = __shfl_down(suf, dl);
        if (t + dl <= te) suf += o;
      }
      const int before = suf - ns;  // splits of the job's query tiles after t (numbered first)
      // the work-group's item: job totals from the lanes of the jobs' first query tiles
      int total = 0;
      {
        int tb_j = 0;
        for (int j = 0; j < a.n_jobs; ++j) {
          const int n_qt = (a.jobs[j].len + qt_rows - 1) / qt_rows;
          if (n_qt > 0) total += __builtin_amdgcn_readlane(suf, tb_j);
          tb_j += n_qt;
        }
      }
      int i = 0, hg_base = 0, hg_span = 1;
      bool live;
      if ((n_hg & 7) == 0) {
        const int hpx = n_hg >> 3;
        i = b >> 3;
        hg_base = (b & 7) * hpx;
        hg_span = hpx;
        live = true;
      } else {
        const int T = total * n_hg;
        const int per = (T + 7) >> 3;
        i = (b & 7) * per + (b >> 3);
        live = (b >> 3) < per && i < T;
        hg_span = n_hg;
      }
      int rj = -1, rq = 0, rs = 0, rhg = 0, rns = 1;
      if (live) {
        int tb_j = 0;
        for (int j = 0; j < a.n_jobs; ++j) {
          const int n_qt = (a.jobs[j].len + qt_rows - 1) / qt_rows;
          const int m = n_qt > 0 ? __builtin_amdgcn_readlane(suf, tb_j) : 0;
          if (i < m * hg_span) {
            const int hl = i / m;
            const int k = i - hl * m;
            const uint64_t hit = __ballot(have && jt == j && before <= k && k < before + ns);
            if (hit) {
              const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
              rj = j;
              rq = L - tb_j;
              rs = k - __builtin_amdgcn_readlane(before, L);
              rns = __builtin_amdgcn_readlane(ns, L);
              rhg = hg_base + hl;
            }
            break;
          }
          i -= m * hg_span;
          tb_j += n_qt;
        }
      }
      if (t == 0) {
        scratch[n_all] = rj;
        scratch[n_all + 1] = rq;
        scratch[n_all + 2] = rs;
        scratch[n_all + 3] = rhg;
        scratch[n_all + 4] = rns;
      }
    }
  } else if (tid < kWave) {
    // more query tiles than lanes: the same scan over chunks of one wave, the last chunk
    // first, each adding the suffix at the next chunk's first tile to the tiles whose
    // job continues there.  Split counts replace the visible counts in scratch; the
    // suffix sums go to sufs.
    int* sufs = scratch + n_all + 8;
    const int t_lane = tid;
    int carry = 0;
    for (int c = (n_all - 1) / kWave; c >= 0; --c) {
      const int t = c * kWave + t_lane;
      const bool have = t < n_all;
      const int end = min(n_all, (c + 1) * kWave) - 1;
      int jt = 0, tb = 0, acc = 0;
      for (int j = 0; j < a.n_jobs; ++j) {
        if (t >= acc) {
          jt = j;
          tb = acc;
        }
        acc += (a.jobs[j].len + qt_rows - 1) / qt_rows;
      }
      const int jlen = lane_val(ld.jlen, jt), jns = lane_val(ld.jns, jt), jtps = lane_val(ld.jtps, jt);
      const int te = have ? tb + (jlen + qt_rows - 1) / qt_rows - 1 : t;
      int ns = 0;
      if (have) {
        const int v = scratch[t];
        ns = jns > 1 ? max(1, (v + jtps - 1) / jtps) : 1;
      }
      const int tel = min(te, end);
      int suf = ns;
#pragma unroll
      for (int dl = 1; dl < kWave; dl <<= 1) {
        const int o = __shfl_down(suf, dl);
        if (t + dl <= tel) suf += o;
      }
      if (have && te > end) suf += carry;
      if (have) {
        scratch[t] = ns;
        sufs[t] = suf;
      }
      carry = __builtin_amdgcn_readlane(suf, 0);
    }
    int total = 0;
    {
      int tb_j = 0;
      for (int j = 0; j < a.n_jobs; ++j) {
        const int n_qt = (a.jobs[j].len + qt_rows - 1) / qt_rows;
        if (n_qt > 0) total += sufs[tb_j];
        tb_j += n_qt;
      }
    }
    int i = 0, hg_base = 0, hg_span = 1;
    bool live;
    if ((n_hg & 7) == 0) {
      const int hpx = n_hg >> 3;
      i = b >> 3;
      hg_base = (b & 7) * hpx;
      hg_span = hpx;
      live = true;
    } else {
      const int T = total * n_hg;
      const int per = (T + 7) >> 3;
      i = (b & 7) * per + (b >> 3);
      live = (b >> 3) < per && i < T;
      hg_span = n_hg;
    }
    int rj = -1, rq = 0, rs = 0, rhg = 0, rns = 1;
    if (live) {
      int tb_j = 0;
      for (int j = 0; j < a.n_jobs; ++j) {
        const int n_qt = (a.jobs[j].len + qt_rows - 1) / qt_rows;
        const int m = n_qt > 0 ? sufs[tb_j] : 0;
        if (i < m * hg_span) {
          const int hl = i / m;
          const int k = i - hl * m;
          for (int c0 = tb_j; c0 < tb_j + n_qt; c0 += kWave) {
            const int t = c0 + t_lane;
            const bool in = t < tb_j + n_qt;
            const int sv = in ? sufs[t] : 0, nv = in ? scratch[t] : 0;
            const uint64_t hit = __ballot(in && sv - nv <= k && k < sv);
            if (hit) {
              const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
              const int sl = __builtin_amdgcn_readlane(sv, L), nl = __builtin_amdgcn_readlane(nv, L);
              rj = j;
              rq = c0 + L - tb_j;
              rs = k - (sl - nl);
              rns = nl;
              rhg = hg_base + hl;
              break;
            }
          }
          break;
        }
        i -= m * hg_span;
        tb_j += n_qt;
      }
    }
    if (t_lane == 0) {
      scratch[n_all] = rj;
      scratch[n_all + 1] = rq;
      scratch[n_all + 2] = rs;
      scratch[n_all + 3] = rhg;
      scratch[n_all + 4] = rns;
    }
  }
  __syncthreads();
  WorkItem w;
  w.job = __builtin_amdgcn_readfirstlane(scratch[n_all]);
  w.qt = __builtin_amdgcn_readfirstlane(scratch[n_all + 1]);
  w.split = __builtin_amdgcn_readfirstlane(scratch[n_all + 2]);
  w.hg = __builtin_amdgcn_readfirstlane(scratch[n_all + 3]);
  ns_out = __builtin_amdgcn_readfirstlane(scratch[n_all + 4]);
  __syncthreads();  // scratch free again
  return w;
}

// A compact launch (no empty split) needs a document or causal mask, KV splits, and at
// most kMaxRankedTiles query tiles over all jobs.
inline bool compact_plan(const FwdArgs& a, int qt_rows) {
  if (a.mask == kMaskNone) return false;
  bool split = false;
  int n_all = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    split |= a.jobs[j].n_split > 1;
    n_all += (a.jobs[j].len + qt_rows - 1) / qt_rows;
  }
  return split && n_all <= kMaxRankedTiles;
}

}  // namespace kv
}  // namespace cpattn
