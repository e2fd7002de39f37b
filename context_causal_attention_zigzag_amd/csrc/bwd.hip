// LSE-replay backward of one rank's share.
//
// "上下文并行：一条序列跨卡，仍算同一个目标", sections 01-02: each KV block is
// replayed against the local queries; the block's probabilities are rebuilt from
// the saved full-row log-sum-exp, P_ij = exp(S_ij - lambda_i); the softmax
// derivative gives dS_ij = P_ij (dP_ij - D_i) with dP = G V^T and D_i = G_i . O_i;
// then dQ_i += dS_ij K_j / sqrt(d), dK_j += dS_ij Q_i / sqrt(d), dV_j += P_ij G_i,
// and the K/V gradients of every query are summed at the owner of the keys.
//
// Three launches, no atomics (gfx950, v_mfma_f32_32x32x16_bf16):
//  - delta: D_i = rowsum(dO * O) in fp32 into the workspace.
//  - dQ, query-major, built like the forward kernel: a wave keeps 32 query rows of Q
//    and dO in registers (B operands) and streams 64-key K/V tiles through LDS
//    (direct global->LDS fills, double-buffered).  S^T = K Q^T and dP^T = V dO^T put
//    one query row per lane, so P^T and dS^T come straight from the accumulators and
//    dS^T is at once the B operand of dQ^T += K^T dS^T; the K^T operand comes from
//    transposing LDS reads of the row-major K tile.  Underfilled launches split the
//    KV tiles over work-groups and sum the fp32 partials (one batched launch).
//  - dK/dV, key-major: one work-group of 4 waves per (KV segment, 128-key tile, kv
//    head); wave w keeps keys 32w..32w+31 (K and V rows) in registers as B operands
//    and owns their dK/dV accumulators, so the per-owner sums over all local queries
//    and all query heads of the group finish in registers and are stored once.  Q and
//    dO tiles are staged row-major in LDS: plain row reads give the A operands of
//    S = Q K^T and dP = dO V^T, transposing reads those of dV^T = dO^T P and
//    dK^T = Q^T dS, in the contraction order of the accumulator layout.
// The dQ pass recomputes S and dP (seven contractions instead of five); in return
// neither pass needs atomics and the dQ pass runs two waves per SIMD.
#include "common.h"
#include "kv_stream.h"

namespace cpattn {

namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 128;  // keys per dK/dV work-group (32 per wave)
constexpr int kBQ = 32;    // query rows per dK/dV step
constexpr int kPosPad = 0x7fffffff;

// ---------------------------------------------------------------------------
// D_i of one 8-element chunk of a row: O . dO in fp32, one fused multiply-add per
// element in order.  The delta kernel and the dQ pass that forms D itself share it, and
// both add a row's chunk values in the same pairs (distance half the chunk count, then
// halving), so the two give the same bits.
__device__ __forceinline__ float chunk_dot(const bf16x8& o, const bf16x8& g) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)o[e], (float)g[e], s);
  return s;
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(const bf16* __restrict__ o,
                                                              const bf16* __restrict__ dout,
                                                              float* __restrict__ delta, int64_t pairs) {
  constexpr int kTpp = D / 8;  // threads per (row, head): chunk c of the row each
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t pair = gid / kTpp;
  const int c = (int)(gid % kTpp);
  float s = 0.0f;
  if (pair < pairs) {
    const int64_t off = pair * D + c * 8;
    s = chunk_dot(*reinterpret_cast<const bf16x8*>(o + off), *reinterpret_cast<const bf16x8*>(dout + off));
  }
  // chunk c adds chunk c + w, w = kTpp / 2, ..., 1 (thread 0's sum is stored)
#pragma unroll
  for (int w = kTpp / 2; w >= 1; w >>= 1) s += __shfl_xor(s, w, kTpp);
  if (pair < pairs && c == 0) delta[pair] = s;
}

// ---------------------------------------------------------------------------
// dQ pass
template <int D>
// K is read both as rows and transposed, at row stride D + 24: its 16-byte row reads are
// conflict-free there, its transposing reads are not (44% of their LDS cycles in
// conflicts in a microbenchmark; only D + 32 serves them without conflicts, at 3.7x the
// cost of the row reads); V only as rows (D + 8).
using DqSmem = kv::KvSmem<D, D + 24, D + 8>;

struct DqExtra {
  const void* dout;
  float* delta;        // [q_len, hq]: read, or written when o is set
  float scale;         // softmax scale (factor of dS)
  int32_t accumulate;  // add to the output instead of overwriting it (unsplit jobs)
  const void* o;       // forward output: the pass forms D from O and dO (the first split stores it)
};

// One 64-key tile for one wave of the dQ pass, in four phases over the tile's key
// halves A (keys 0..31) and B (32..63):
//   S_A, dP_A;  S_B, dP_B beside dS_A;  dQ += K_A^T dS_A beside dS_B;  dQ += K_B^T dS_B,
// so that the matrix core has independent work while the wave computes
// dS = P (dP - D) scale with P = exp(S - LSE).  Operands are read two steps ahead.
template <int D>
__device__ __forceinline__ void dq_step(const bf16* __restrict__ ks, const bf16* __restrict__ vs,
                                        const int32_t* kpos, const int32_t* kdoc, int klen,
                                        const bf16x8 (&qf)[D / 16], const bf16x8 (&of)[D / 16],
                                        f32x16 (&dq)[D / 32], float lse2, float dl, int qpos, int qdoc,
                                        bool masked, int mask, float scale, float scale_log2, int lane) {
  using namespace kv;
  constexpr int kKS = DqSmem<D>::kKS, kVS = DqSmem<D>::kVS;
  constexpr int kSt = D / 16;   // stages of each middle phase
  constexpr int kE = 16 / kSt;  // dS values per stage
  static_assert(16 % kSt == 0 && kSt >= 4, "whole dS values per stage");
  const int r = lane & 31, h = lane >> 5;
  const bf16* ka = ks + r * kKS + h * 8;
  const bf16* va = vs + r * kVS + h * 8;
  const bf16* kl = ks + tr_lane_offset<4>(lane, kKS);
  auto row = [&](const bf16* base, int ds) { return *reinterpret_cast<const bf16x8*>(base + ds * 16); };
  // K^T operand of product k of a dQ phase: dims 32 (k / 2) .., key slice (k % 2) of the half
  auto ktr = [&](int half, int k) {
    const bf16* p = kl + (2 * half + (k & 1)) * 16 * kKS + (k >> 1) * 32;
    return concat(lds_read_tr4(p), lds_read_tr4(p + 8 * kKS));
  };
  bf16x8 dsf[4];  // dS^T as B operands of the four 16-key slices
  auto ds_val = [&](const f32x16& sv, const f32x16& pv, int i) {
    const float p = fast_exp2(fmaf(sv[i], scale_log2, -lse2));
    return (bf16)(p * (pv[i] - dl) * scale);
  };

  // S_A, dP_A
  f32x16 sa = {}, pa = {}, sb = {}, pb = {};
#pragma unroll
  for (int ds = 0; ds < kSt; ++ds) {
    sa = mfma32x32x16(row(ka, ds), qf[ds], sa);
    pa = mfma32x32x16(row(va, ds), of[ds], pa);
  }
  bf16x8 ko[2] = {row(ka + 32 * kKS, 0), row(ka + 32 * kKS, 1)};
  bf16x8 vo[2] = {row(va + 32 * kVS, 0), row(va + 32 * kVS, 1)};
  if (masked) mask_half(sa, kpos, kdoc, klen, qpos, qdoc, mask, h, 0);

  // S_B, dP_B beside dS_A
#pragma unroll
  for (int k = 0; k < kSt; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    sb = mfma32x32x16(ko[k & 1], qf[k], sb);
    pb = mfma32x32x16(vo[k & 1], of[k], pb);
    if (k + 2 < kSt) {
      ko[k & 1] = row(ka + 32 * kKS, k + 2);
      vo[k & 1] = row(va + 32 * kVS, k + 2);
    } else {
      ko[k & 1] = ktr(0, k + 2 - kSt);
    }
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int i = k * kE + e;
      dsf[i >> 3][i & 7] = ds_val(sa, pa, i);
    }
  }
  asm volatile("" ::"v"(dsf[0]), "v"(dsf[1]));
  __builtin_amdgcn_sched_barrier(0);
  if (masked) mask_half(sb, kpos, kdoc, klen, qpos, qdoc, mask, h, 1);

  // dQ += K_A^T dS_A beside dS_B
#pragma unroll
  for (int k = 0; k < kSt; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    dq[k >> 1] = mfma32x32x16(ko[k & 1], dsf[k & 1], dq[k >> 1]);
    ko[k & 1] = k + 2 < kSt ? ktr(0, k + 2) : ktr(1, k + 2 - kSt);
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int i = k * kE + e;
      dsf[2 + (i >> 3)][i & 7] = ds_val(sb, pb, i);
    }
  }
  asm volatile("" ::"v"(dsf[2]), "v"(dsf[3]));
  __builtin_amdgcn_sched_barrier(0);

  // dQ += K_B^T dS_B
#pragma unroll
  for (int k = 0; k < kSt; ++k) {
    dq[k >> 1] = mfma32x32x16(ko[k & 1], dsf[2 + (k & 1)], dq[k >> 1]);
    if (k + 2 < kSt) ko[k & 1] = ktr(1, k + 2);
  }
}

template <int D, int NW, bool RANKED>
__global__ __launch_bounds__(NW * kWave, NW == 8 ? 1 : 2) void bwd_dq_kernel(FwdArgs a, DqExtra x) {
  using namespace kv;
  __shared__ DqSmem<D> sm;
  // the work-list scratch sits in the first K image, below the tile table
  static_assert(sizeof(DqSmem<D>::k) / 2 >= (2 * kMaxRankedTiles + 16) * sizeof(int), "work-list scratch");
  const int hpw = a.heads_per_wg;
  const int qt_rows = NW * kRowsPerWave / hpw;
  const LaneDescs ld = load_lane_descs(a);
  TileTab tt{0, 0};
  WorkItem wi;
  int ns_mine = 1;      // splits that exist for this work item's query tile (compact launches)
  bool tt_all = false;  // the tile table covers every segment of the launch
  if constexpr (RANKED) {
    if (a.plan != nullptr)
      wi = planned_work_item<NW * kWave>(a, qt_rows, sm, tt);
    else
      wi = ranked_work_item<NW * kWave>(a, ld, qt_rows, reinterpret_cast<int*>(&sm), sm, tt);
  } else {
    if (a.compact) {
      wi = compact_work_item<NW * kWave>(a, ld, qt_rows, reinterpret_cast<int*>(&sm), sm, tt, ns_mine);
      tt_all = true;
    } else {
      wi = indexed_work_item(a, qt_rows);
    }
    if (wi.job < 0) return;
  }
  const JobDesc& job = a.jobs[wi.job];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsplit = job.n_split;
  const int split = wi.split, hg = wi.hg, qt = wi.qt;
  const int r0 = qt * qt_rows, r1 = min(job.len, r0 + qt_rows);
  const int head = hg * hpw + wave % hpw;
  const int kvh = (hg * hpw) / a.group;
  const int wr0 = r0 + (wave / hpw) * kRowsPerWave;
  const int wr1 = min(r1, wr0 + kRowsPerWave);
  const bool wave_rows = wr0 < wr1;
  const int myrow = wr0 + (lane & 31);
  const bool row_ok = myrow < wr1;
  const int mask = a.mask;

  const int qmax = job.pos[r1 - 1];
  int qdmin = 0, qdmax = 0, wqdmin = 0, wqdmax = 0;
  if (mask == kMaskCausalDoc) {
    qdmin = job.doc[r0];
    qdmax = job.doc[r1 - 1];
  }
  int wqmin = 0, wqmax = -1;
  if (wave_rows) {
    wqmin = job.pos[wr0];
    wqmax = job.pos[wr1 - 1];
    if (mask == kMaskCausalDoc) {
      wqdmin = job.doc[wr0];
      wqdmax = job.doc[wr1 - 1];
    }
  }

  bf16x8 qf[D / 16], of[D / 16], ov[D / 16];
  const bf16* obp = nullptr;  // the row's O (forming D)
  int qpos = kPosPad, qdoc = 0;
  float lse2 = __builtin_inff(), dl = 0.0f;
  {
    // rows past the end load the tile's first row (their results are never stored)
    const int64_t off = ((int64_t)(row_ok ? myrow : r0) * a.hq + head) * D + (lane >> 5) * 8;
    const bf16* qb = reinterpret_cast<const bf16*>(job.q) + off;
    const bf16* ob = reinterpret_cast<const bf16*>(x.dout) + off;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      qf[ds] = *reinterpret_cast<const bf16x8*>(qb + ds * 16);
      of[ds] = *reinterpret_cast<const bf16x8*>(ob + ds * 16);
    }
    if (row_ok) {
      qpos = job.pos[myrow];
      if (mask == kMaskCausalDoc) qdoc = job.doc[myrow];
      const float l = job.lse[(int64_t)myrow * a.hq + head];
      lse2 = l == neg_inf() ? __builtin_inff() : l * kLog2e;  // a row with no key: P = 0
      if (x.o == nullptr) dl = x.delta[(int64_t)myrow * a.hq + head];
    }
    if (x.o != nullptr) obp = reinterpret_cast<const bf16*>(x.o) + off;
  }
  // the row's O chunks for forming D: loaded beside the first tile fill, whose barrier
  // waits for them, so that no earlier wait of the set-up (loads complete in issue
  // order) includes them
  auto load_o = [&]() {
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) ov[ds] = *reinterpret_cast<const bf16x8*>(obp + ds * 16);
  };
  // D of the row from O and the dO operands held: this lane's chunks are 2 ds + h;
  // pairs as in the delta kernel (chunk distance D/16, then halving within the lane,
  // then the other half's sum), so the value equals its bits.  The first split stores
  // it.  Called at work-group-uniform points (the exchange between halves needs every lane).
  auto form_delta = [&]() {
    float p[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) p[ds] = chunk_dot(ov[ds], of[ds]);
#pragma unroll
    for (int w = D / 32; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) p[i] = p[i] + p[i + w];
    const float mine = p[0];
    const float d = mine + __shfl_xor(mine, 32);
    if (row_ok) {
      dl = d;
      if (split == 0 && (lane >> 5) == 0) x.delta[(int64_t)myrow * a.hq + head] = d;
    }
  };

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  float* flag_dst = nsplit > 1 ? job.ws_lse + (int64_t)split * job.len * a.hq : nullptr;
  // tiles of the walk, and per wave the skipped and the fully visible ones, from one
  // binary search per segment (kv_stream.h); the loop reads no segment table
  TileIter it;
  if (!RANKED && !tt_all && a.mask != kMaskNone)
    tt = load_tile_table<NW * kWave>(sm, a, ld, job.seg_begin, job.seg_end);
  iter_init_lanes(it, a, ld, job, lane, qmax, qdmin, qdmax, wave_rows, wqmin, wqmax, wqdmin, wqdmax, sm, tt);
  // compact launches run no work-group for the splits past a query tile's visible
  // tiles: the first split marks their partials empty for the sum
  if (nsplit > 1 && split == 0 && row_ok && (lane >> 5) == 0)
    for (int s = ns_mine; s < nsplit; ++s) job.ws_lse[((int64_t)s * job.len + myrow) * a.hq + head] = neg_inf();
  if (nsplit == 1) {
    iter_walk_all(it, job);
  } else if (!iter_walk_split(it, job, split * job.tiles_per_split, job.tiles_per_split)) {
    // nothing in this split: mark its partial empty (the first split still stores D)
    if (x.o != nullptr && split == 0) {
      load_o();
      form_delta();
    }
    if (row_ok && (lane >> 5) == 0) flag_dst[(int64_t)myrow * a.hq + head] = neg_inf();
    return;
  }

  using Sm = DqSmem<D>;
  const uint32_t rstride = (uint32_t)a.hkv * D;  // elements between consecutive keys
  FillOffs<D, Sm, NW, true> fo;
  fo.init(wave, lane, rstride);
  const bool doc = mask == kMaskCausalDoc;
  if (x.o != nullptr) load_o();
  TileRef cur = iter_next(it, job, TileRef{-1, 0});
  if (cur.seg < 0 && x.o != nullptr) form_delta();
  if (cur.seg >= 0) {
    KvTile tc = iter_tile(it, cur, job.seg_begin, kvh, a.hkv, D);
    fill_tile<D, Sm>(sm, 0, tc, rstride, doc, wave, lane, fo);
    fill_barrier();
    if (x.o != nullptr) form_delta();
    int buf = 0;
    while (true) {
      const TileRef nxt = iter_next(it, job, cur);
      KvTile tn = tc;
      if (nxt.seg >= 0) {
        tn = iter_tile(it, nxt, job.seg_begin, kvh, a.hkv, D);
        fill_tile<D, Sm>(sm, buf ^ 1, tn, rstride, doc, wave, lane, fo);
      }
      if (!tc.empty)
        dq_step<D>(sm.k[buf], sm.v[buf], sm.kpos[buf], sm.kdoc[buf], tc.last + 1, qf, of, dq, lse2, dl, qpos,
                   qdoc, !tc.full, mask, x.scale, a.scale_log2, lane);
      if (nxt.seg < 0) break;
      fill_barrier();
      buf ^= 1;
      cur = nxt;
      tc = tn;
    }
  }

  if (row_ok) {
    const int h = lane >> 5;
    const int64_t rowoff = ((int64_t)myrow * a.hq + head) * D;
    float* out = nsplit > 1 ? job.ws_o + (int64_t)split * job.len * a.hq * D : reinterpret_cast<float*>(job.o);
    const bool acc = x.accumulate != 0 && nsplit == 1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + h * 4;
        f32x4 val = {dq[db][4 * g], dq[db][4 * g + 1], dq[db][4 * g + 2], dq[db][4 * g + 3]};
        if (acc) val += *reinterpret_cast<const f32x4*>(out + rowoff + d0);
        *reinterpret_cast<f32x4*>(out + rowoff + d0) = val;
      }
    }
    if (nsplit > 1 && h == 0) flag_dst[(int64_t)myrow * a.hq + head] = 0.0f;
  }
}

// ---------------------------------------------------------------------------
// dK/dV pass
//
// Software pipeline over the query tiles a work-group visits; iteration i of a wave
// runs three independent pieces of work side by side:
//   the S / dP contractions of tile i+1,
//   the dV / dK contractions of tile i-1 (with its P / dS from iteration i-1),
//   the P / dS arithmetic of tile i (from its S / dP of iteration i-1),
// so the matrix cores and the vector ALU never wait on each other inside an iteration.
// Tiles i-1 .. i+1 are read while tiles i+2 (landed) and i+3 (filling, two iterations
// ahead) occupy the other LDS buffers: five tile buffers rotate.
constexpr int kQBufs = 5;

template <int D>
struct DkdvSmem {
  // Row stride (elements) of these tiles, read both as 16-byte rows and transposed:
  // D + 24 (304 bytes at D = 128) keeps the row reads conflict-free and leaves the
  // transposing reads with 44% of their LDS cycles in conflicts (microbenchmark with the
  // kernel's lane addressing); D + 32 would serve the transposing reads but make the row
  // reads 3.7x slower, so the cheaper side keeps the conflicts.
  static constexpr int kRS = D + 24;
  static constexpr int kSlots = kRS / 8;                                // 16-byte slots per row
  static constexpr int kTileInst = (kBQ * kSlots + kWave - 1) / kWave;  // fill instructions per tile
  // image of one tile: the rows, then slack that the last fill instruction's slots
  // past the last row write into
  static constexpr int kImage = kTileInst * kWave * 8;  // elements
  static constexpr int kBigPer = 2 * kTileInst / 4;      // Q and dO fill instructions per wave
  static constexpr int kFillPer = kBigPer + 1;            // + one 4-byte-per-lane fill
  static_assert(2 * kTileInst % 4 == 0, "whole fill instructions per wave");
  alignas(16) bf16 qs[kQBufs][kImage];
  alignas(16) bf16 dos[kQBufs][kImage];
};

// Per-row values of the query tiles: a separate LDS object from the tile images, so
// that reading them never waits on outstanding image fills.
struct RowSmem {
  alignas(16) float ld[kQBufs][2][kBQ];    // log-sum-exp, then delta, of the tile's rows
  alignas(16) int32_t pd[kQBufs][2][kBQ];  // positions, then document ids
};

// Per-lane sources of the Q / dO fill instructions: fill instruction jj of a tile
// writes the 64 16-byte slots 64*jj .. 64*jj+63 of the tile image, lane l slot
// 64*jj + l (row-major, kSlots per row, the last ones padding).  The byte offsets of a
// whole tile's sources are fixed for the kernel and computed once; only a ragged last
// tile recomputes them with its rows clamped.  The LDS images' base offsets are taken
// once too, so a fill costs the loop three instructions (m0, the wait state it needs,
// the load) instead of re-deriving pointers every step.
template <int D>
struct QFillPlan {
  using Sm = DkdvSmem<D>;
  uint32_t off[Sm::kBigPer];  // (row * rs + column) * 2 of a whole tile
  uint32_t lds_q, lds_o;      // LDS byte offsets of qs[0] and dos[0]

  __device__ __forceinline__ static uint32_t source(int wave, int lane, int j, uint32_t last, uint32_t rs) {
    const int jj = (wave + 4 * j) % Sm::kTileInst;
    const int s = kWave * jj + lane;
    const int c = s % Sm::kSlots;
    // slots past the last row (slack) and padding slots load a valid dummy chunk
    const uint32_t row = min((uint32_t)min(s / Sm::kSlots, kBQ - 1), last);
    return (row * rs + (uint32_t)(c < D / 8 ? c * 8 : 0)) * 2;
  }

  __device__ __forceinline__ void init(const Sm& sm, int wave, int lane, uint32_t rs) {
#pragma unroll
    for (int j = 0; j < Sm::kBigPer; ++j) off[j] = source(wave, lane, j, kBQ - 1, rs);
    lds_q = lds_offset(sm.qs[0]);
    lds_o = lds_offset(sm.dos[0]);
  }
};

struct QItem {
  int hh;  // head within the kv group (-1: none)
  int qt;  // query tile
};

struct QRange {
  int pmin, pmax, dmin, dmax;
};

// First / last position (and document) of query tile t, from the query block.
template <bool DOC>
__device__ __forceinline__ QRange qrange_global(const BwdArgs& a, int t) {
  const int q0 = t * kBQ, q1 = min(a.q_len, q0 + kBQ) - 1;
  return {a.qpos[q0], a.qpos[q1], DOC ? a.qdoc[q0] : 0, DOC ? a.qdoc[q1] : 0};
}

// The same for the tile whose row values sit in buffer `buf` (its first `nv` rows are
// real; the rows after them were marked invisible once the fill landed).
template <bool DOC>
__device__ __forceinline__ QRange qrange_lds(const RowSmem& sm, int buf, int nv) {
  return {sm.pd[buf][0][0], sm.pd[buf][0][nv - 1], DOC ? sm.pd[buf][1][0] : 0, DOC ? sm.pd[buf][1][nv - 1] : 0};
}

// The work-group's items are (head within the group, query tile) for every head and
// the query tiles [lo, hi) that the key range can see: positions (and documents) are
// non-decreasing along the query block, so those tiles are contiguous (a tile inside
// the range that nonetheless sees nothing is processed masked, with the same result).
__device__ __forceinline__ QItem next_qitem(QItem it, int group, int lo, int hi) {
  if (it.qt + 1 < hi) return {it.hh, it.qt + 1};
  if (it.hh + 1 < group) return {it.hh + 1, lo};
  return {-1, 0};
}

// Issues this wave's kBigPer direct global->LDS fill instructions of the Q / dO
// images of query tile `it` into buffer `buf`.  Rows past the end are clamped to the
// last row (their positions mark them invisible, see row_value).
template <int D, bool DOC>
__device__ __forceinline__ void fill_qtile(DkdvSmem<D>& sm, RowSmem& rsm, int buf, const BwdArgs& a,
                                           const QFillPlan<D>& fp, QItem it, int kvh, int wave, int lane) {
  using Sm = DkdvSmem<D>;
  const int head = kvh * a.group + it.hh;
  const int r0 = it.qt * kBQ;
  const uint32_t last = (uint32_t)(min(kBQ, a.q_len - r0) - 1);
  const uint32_t rs = (uint32_t)a.hq * D;
  const int64_t base = ((int64_t)r0 * a.hq + head) * D;
  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + base;
  const bf16* ob = reinterpret_cast<const bf16*>(a.dout) + base;
  const uint32_t ib = (uint32_t)buf * (Sm::kImage * 2);
  auto burst = [&](const uint32_t(&offs)[Sm::kBigPer]) {
#pragma unroll
    for (int j = 0; j < Sm::kBigPer; ++j) {
      const int jj = wave + 4 * j;
      const bool isq = jj < Sm::kTileInst;
      const uint32_t dst = (isq ? fp.lds_q : fp.lds_o) + ib + (uint32_t)(isq ? jj : jj - Sm::kTileInst) * (kWave * 16);
      fill16_off(isq ? qb : ob, offs[j], dst);
    }
  };
  if (last == kBQ - 1) {
    burst(fp.off);
  } else {
    // ragged last tile: rows past the end read the last row (their positions mark them
    // invisible); each offset in its own register before the burst
    uint32_t offs[Sm::kBigPer];
#pragma unroll
    for (int j = 0; j < Sm::kBigPer; ++j) offs[j] = QFillPlan<D>::source(wave, lane, j, last, rs);
    burst(offs);
#pragma unroll
    for (int j = 0; j < Sm::kBigPer; ++j) asm volatile("" ::"v"(offs[j]));
  }
  // per-row values: wave 1 positions (lanes 0..31) and document ids (32..63), the
  // others log-sum-exp (0..31) and delta (32..63) (identical data)
  const int q = r0 + (int)min((uint32_t)(lane & 31), last);
  const auto* qpos = uniform_ptr(a.qpos);
  const auto* qdoc = DOC ? uniform_ptr(a.qdoc) : qpos;
  const auto* lse = uniform_ptr(a.lse);
  const auto* del = uniform_ptr(a.delta);
  const void* src = wave == 1 ? static_cast<const void*>((lane < 32 ? qpos : qdoc) + q)
                              : static_cast<const void*>((lane < 32 ? lse : del) + (int64_t)q * a.hq + head);
  fill4_untracked(src, wave == 1 ? lds_offset(rsm.pd[buf]) : lds_offset(rsm.ld[buf]));
}

// Wave 1 marks the rows of tile `it` past the end invisible (position INT_MIN) once
// its position fill has landed.
__device__ __forceinline__ void seal_qtile(RowSmem& rsm, int buf, const BwdArgs& a, QItem it, int wave, int lane) {
  if (wave != 1) return;
  const int nvalid = a.q_len - it.qt * kBQ;
  if (nvalid < kBQ && lane < kBQ && lane >= nvalid) rsm.pd[buf][0][lane] = INT32_MIN;
}

// Waits for this wave's outstanding fills except the last `keep` tile's (every tile
// fill is kFillPer instructions per wave).
template <int D>
__device__ __forceinline__ void wait_fills(bool keep_one_tile) {
  static_assert(DkdvSmem<D>::kFillPer == 6 || DkdvSmem<D>::kFillPer == 4, "immediates below");
  if (keep_one_tile) {
    if (DkdvSmem<D>::kFillPer == 6)
      asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// S = Q K^T and dP = dO V^T for this wave's 32 keys: Q / dO rows from LDS as A
// operands, K / V in registers as B operands.  Accumulator layout: lane l holds key
// (l % 32) and queries 8(a/4) + 4(l/32) + a%4.
template <int D>
__device__ __forceinline__ void dkdv_sdp(const DkdvSmem<D>& sm, int buf, const bf16x8 (&kf)[D / 16],
                                         const bf16x8 (&vf)[D / 16], f32x16& s, f32x16& dp, int lane) {
  constexpr int kRS = DkdvSmem<D>::kRS;
  const int r = lane & 31, h = lane >> 5;
  const bf16* qrow = sm.qs[buf] + r * kRS + h * 8;
  const bf16* orow = sm.dos[buf] + r * kRS + h * 8;
  // all operands first: the reads overlap each other and the first contractions
  bf16x8 aq[D / 16], ao[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    aq[ds] = *reinterpret_cast<const bf16x8*>(qrow + ds * 16);
    ao[ds] = *reinterpret_cast<const bf16x8*>(orow + ds * 16);
  }
  s = f32x16{};
  dp = f32x16{};
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    s = mfma32x32x16(aq[ds], kf[ds], s);
    dp = mfma32x32x16(ao[ds], vf[ds], dp);
  }
}

// Row operands of the S / dP contraction step ds: the A operands (Q and dO rows of this
// lane's row r = lane % 32, dims 16 ds + 8 h .. +7).
struct RowOps {
  bf16x8 aq, ao;
};

template <int D>
__device__ __forceinline__ RowOps dkdv_rowops(const DkdvSmem<D>& sm, int buf, int ds, int lane) {
  constexpr int kRS = DkdvSmem<D>::kRS;
  const int off = (lane & 31) * kRS + (lane >> 5) * 8 + ds * 16;
  return {*reinterpret_cast<const bf16x8*>(sm.qs[buf] + off), *reinterpret_cast<const bf16x8*>(sm.dos[buf] + off)};
}

// P and dS/scale for accumulator group g (queries 8g + 4h .. +3): P rebuilt from the
// row's log-sum-exp, then the visibility test (key position <= query position, same
// document); kpos_eff is the key's position for masked tiles and INT_MIN + 1 for
// fully visible ones, INT_MAX for keys past the segment's end.
// Per-row values of the tile for this lane's 16 queries (4 groups of 4).
template <bool DOC>
struct RowVals {
  f32x4 l[4], dl[4];
  int4 qp[4], qd[DOC ? 4 : 1];
};

template <bool DOC>
__device__ __forceinline__ void load_rows(const RowSmem& sm, int buf, int h, RowVals<DOC>& rv) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int q0 = 8 * g + 4 * h;
    rv.l[g] = *reinterpret_cast<const f32x4*>(&sm.ld[buf][0][q0]);
    rv.dl[g] = *reinterpret_cast<const f32x4*>(&sm.ld[buf][1][q0]);
    rv.qp[g] = *reinterpret_cast<const int4*>(&sm.pd[buf][0][q0]);
    if (DOC) rv.qd[DOC ? g : 0] = *reinterpret_cast<const int4*>(&sm.pd[buf][1][q0]);
  }
}

template <int D, bool DOC>
__device__ __forceinline__ void dkdv_pds(const RowVals<DOC>& rv, const f32x16& s, const f32x16& dp, int g,
                                         int kpos_eff, int kdoc, float scale_log2, bf16x8 (&pf)[2],
                                         bf16x8 (&dsf)[2]) {
  const f32x4 l = rv.l[g];
  const f32x4 dl = rv.dl[g];
  const int4 qp = rv.qp[g];
  int4 qd = {0, 0, 0, 0};
  if (DOC) qd = rv.qd[DOC ? g : 0];
  const int qpa[4] = {qp.x, qp.y, qp.z, qp.w};
  const int qda[4] = {qd.x, qd.y, qd.z, qd.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * g + e;
    float p = fast_exp2(fmaf(s[i], scale_log2, -l[e] * kLog2e));
    bool vis = kpos_eff <= qpa[e];
    if (DOC) vis = vis && kdoc == qda[e];
    p = vis ? p : 0.0f;
    pf[i >> 3][i & 7] = (bf16)p;
    dsf[i >> 3][i & 7] = (bf16)(p * (dp[i] - dl[e]));
  }
}

// dV^T += dO^T P and dK^T += Q^T dS for the 32-dim block db and 16-query slice sl
// (pair j = 2 db + sl); the transposed operands come from transposing LDS reads in
// the accumulators' contraction order.
struct TrOps {
  bf16x8 ao, aq;
};

template <int D>
__device__ __forceinline__ TrOps dkdv_ops(const DkdvSmem<D>& sm, int buf, int j, int lane) {
  constexpr int kRS = DkdvSmem<D>::kRS;
  const int db = j >> 1, sl = j & 1;
  const int off = tr_lane_offset<4>(lane, kRS) + sl * 16 * kRS + db * 32;
  const bf16* qtr = sm.qs[buf] + off;
  const bf16* otr = sm.dos[buf] + off;
  return {concat(lds_read_tr4(otr), lds_read_tr4(otr + 8 * kRS)), concat(lds_read_tr4(qtr), lds_read_tr4(qtr + 8 * kRS))};
}

template <int D>
__device__ __forceinline__ void dkdv_mma(const TrOps& op, int j, const bf16x8 (&pf)[2], const bf16x8 (&dsf)[2],
                                         f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32]) {
  const int db = j >> 1, sl = j & 1;
  dv[db] = mfma32x32x16(op.ao, pf[sl], dv[db]);
  dk[db] = mfma32x32x16(op.aq, dsf[sl], dk[db]);
}

template <int D>
__device__ __forceinline__ void dkdv_acc_all(const DkdvSmem<D>& sm, int buf, const bf16x8 (&pf)[2],
                                             const bf16x8 (&dsf)[2], f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                             int lane) {
#pragma unroll
  for (int j = 0; j < D / 16; ++j) dkdv_mma<D>(dkdv_ops<D>(sm, buf, j, lane), j, pf, dsf, dk, dv);
}

template <int D, bool DOC>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using Sm = DkdvSmem<D>;
  __shared__ Sm sm;
  __shared__ RowSmem rs;
  int s = 0, kvh, jp;
  if (DOC && (a.hkv & 7) == 0) {
    // Packed documents: a key tile's work follows its documents, not its index, so
    // every XCD (b % 8) takes kv heads [x*hpx, (x+1)*hpx) of every segment, an equal
    // share of each segment's work: segment by segment, tile pairs in order, heads
    // inner.  The launch has no padding here.  (Zigzag shares keep contiguous ranges,
    // whose consecutive items share a segment and so its query rows in L2.)
    const int hpx = a.hkv >> 3;
    int i = blockIdx.x >> 3;
    while (true) {
      const int np = ((a.segs[s].len + kBKV - 1) / kBKV + 1) / 2;
      if (i < np * hpx) break;
      i -= np * hpx;
      ++s;
    }
    jp = i / hpx;
    kvh = (blockIdx.x & 7) * hpx + (i - jp * hpx);
  } else {
    const int logical = xcd_remap(blockIdx.x, a.padded_wgs);
    if (logical >= a.total_wgs) return;
    while (s + 1 < a.n_segs && a.seg_wg_begin[s + 1] <= logical) ++s;
    const int n_pair = ((a.segs[s].len + kBKV - 1) / kBKV + 1) / 2;
    const int local = logical - a.seg_wg_begin[s];
    kvh = local / n_pair;
    jp = local - kvh * n_pair;
  }
  const SegDesc& sg = a.segs[s];
  const int n_kt = (sg.len + kBKV - 1) / kBKV;
  // a work-group takes key tiles jp and n_kt - 1 - jp of its segment in turn: under
  // causal masking their visible query counts roughly add up to a constant (a zigzag
  // segment's early tiles see the most queries, its late ones the fewest), so the
  // work-groups carry even work
  for (int pass = 0; pass < 2; ++pass) {
  const int kt = pass == 0 ? jp : n_kt - 1 - jp;
  if (pass == 1) {
    if (kt <= jp) break;
    // every wave is done with its staged rows of the first tile (no fill is in flight:
    // the first pass waited for them before staging); its dK / dV stores may still be
    // in flight and drain under this pass's setup
    lds_barrier();
  }
  const int k0 = kt * kBKV, k1 = min(sg.len, k0 + kBKV);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int mask = a.mask;
  const bool docmask = DOC;
  const bf16* kb = reinterpret_cast<const bf16*>(sg.k);
  const bf16* vb = reinterpret_cast<const bf16*>(sg.v);

  // this wave's keys as B operands (lane: key 32*wave + r, dims 16*ds + 8*h .. +7)
  const int mykey = k0 + wave * 32 + r;
  const bool key_ok = mykey < k1;
  // effective key position of masked tiles (keys past the end are never visible)
  const int kpos_mask = key_ok ? (mask == kMaskNone ? INT32_MIN + 1 : sg.pos[mykey]) : INT32_MAX;
  const int kdoc = (key_ok && docmask) ? sg.doc[mykey] : 0;

  // key ranges of the work-group and of this wave (non-decreasing positions)
  const int kmin = sg.pos[k0], kmax = sg.pos[k1 - 1];
  int kdmin = 0, kdmax = 0;
  if (docmask) {
    kdmin = sg.doc[k0];
    kdmax = sg.doc[k1 - 1];
  }
  const int wk0 = k0 + wave * 32, wk1 = min(k1, wk0 + 32);
  const bool wave_keys = wk0 < wk1;
  int wkmin = 0, wkmax = 0, wkdmin = 0, wkdmax = 0;
  if (wave_keys) {
    wkmin = sg.pos[wk0];
    wkmax = sg.pos[wk1 - 1];
    if (docmask) {
      wkdmin = sg.doc[wk0];
      wkdmax = sg.doc[wk1 - 1];
    }
  }

  const int n_qt = (a.q_len + kBQ - 1) / kBQ;
  // the first query tiles' ranges go out before the K/V loads: completions count in
  // issue order, so the visible-range test below then waits for its own loads only
  QRange q_first = {0, -1, 0, 0};
  if (tid < n_qt) q_first = qrange_global<DOC>(a, tid);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 kf[D / 16], vf[D / 16];
  {
    // keys past the segment's end load the last key (their results are masked)
    const int64_t base = ((int64_t)min(mykey, k1 - 1) * a.hkv + kvh) * D + h * 8;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      kf[ds] = *reinterpret_cast<const bf16x8*>(kb + base + ds * 16);
      vf[ds] = *reinterpret_cast<const bf16x8*>(vb + base + ds * 16);
    }
  }
  __shared__ int vis_lo, vis_hi;
  if (tid == 0) {
    vis_lo = INT32_MAX;
    vis_hi = -1;
  }
  QFillPlan<D> fp;
  fp.init(sm, wave, lane, (uint32_t)a.hq * D);
  lds_barrier();
  // range of query tiles the work-group's keys can see (read from the query block:
  // any number of local rows)
  {
    int lo = INT32_MAX, hi = -1;
    for (int t = tid; t < n_qt; t += kThreads) {
      const QRange q = t == tid ? q_first : qrange_global<DOC>(a, t);
      if (classify(mask, q.pmin, q.pmax, q.dmin, q.dmax, kmin, kmax, kdmin, kdmax) != kTileEmpty) {
        lo = min(lo, t);
        hi = max(hi, t);
      }
    }
    if (hi >= 0) {
      atomicMin(&vis_lo, lo);
      atomicMax(&vis_hi, hi);
    }
  }
  lds_barrier();
  const int qlo = vis_lo, qhi = vis_hi + 1;

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  QItem cur = qhi > qlo ? QItem{0, qlo} : QItem{-1, 0};
  if (cur.hh >= 0) {
    // prologue: tiles 0, 1, 2 filled and landed, S / dP of tile 0
    QItem n1 = next_qitem(cur, a.group, qlo, qhi);
    QItem n2 = n1.hh >= 0 ? next_qitem(n1, a.group, qlo, qhi) : QItem{-1, 0};
    fill_qtile<D, DOC>(sm, rs, 0, a, fp, cur, kvh, wave, lane);
    if (n1.hh >= 0) fill_qtile<D, DOC>(sm, rs, 1, a, fp, n1, kvh, wave, lane);
    if (n2.hh >= 0) fill_qtile<D, DOC>(sm, rs, 2, a, fp, n2, kvh, wave, lane);
    QItem nf = n2.hh >= 0 ? next_qitem(n2, a.group, qlo, qhi) : QItem{-1, 0};
    // every load so far (fills and this wave's key values) has landed: the builtin
    // form lets the compiler know, so it adds no waits of its own inside the loop
    __builtin_amdgcn_s_waitcnt(0x0F70);
    seal_qtile(rs, 0, a, cur, wave, lane);
    if (n1.hh >= 0) seal_qtile(rs, 1, a, n1, wave, lane);
    if (n2.hh >= 0) seal_qtile(rs, 2, a, n2, wave, lane);
    lds_barrier();
    f32x16 sv, dpv;
    dkdv_sdp<D>(sm, 0, kf, vf, sv, dpv, lane);

    // Iteration i (tile i in buffer b0, i-1 in bp, i+1 in b1, i+2 in b2): one
    // straight-line body for every wave.  A wave whose keys see nothing of a tile runs
    // it masked (P = 0); the first iteration's "previous tile" dV/dK contractions run
    // on zeros over tile 0's (valid) image, and the last one's "next tile" S / dP on a
    // buffer whose results are not used.
    int b0 = 0, bp = 0;
    bf16x8 ppf[2] = {}, pdsf[2] = {};
    // operands of the first kNP dV / dK pairs of the coming iteration (its previous
    // tile); three at d = 128 (two and four measured slower), two at d = 64
    constexpr int kPairs = D / 16, kNP = kPairs >= 8 ? 3 : 2;
    TrOps to[kNP];
#pragma unroll
    for (int j = 0; j < kNP; ++j) to[j] = dkdv_ops<D>(sm, bp, j, lane);
    while (true) {
      const int b1 = b0 == kQBufs - 1 ? 0 : b0 + 1;
      const int b2 = b1 == kQBufs - 1 ? 0 : b1 + 1;
      const int b3 = b2 == kQBufs - 1 ? 0 : b2 + 1;
      // this iteration's LDS reads first (tile i's row values and range, the first
      // operands of tiles i+1 and i-1): their latency then overlaps the fill issue
      RowVals<DOC> rv;
      load_rows<DOC>(rs, b0, h, rv);
      RowOps ro[2] = {dkdv_rowops<D>(sm, b1, 0, lane), dkdv_rowops<D>(sm, b1, 1, lane)};
      const QRange q = qrange_lds<DOC>(rs, b0, min(kBQ, a.q_len - cur.qt * kBQ));
      // dV / dK of tile i-1, pairs 0 .. kNP-1: their operands were read in the last
      // iteration, so these contractions run while the wave waits for the reads above
      // and issues the fills
#pragma unroll
      for (int j = 0; j < kNP; ++j) {
        dkdv_mma<D>(to[j], j, ppf, pdsf, dk, dv);
        to[j] = j + kNP < kPairs ? dkdv_ops<D>(sm, bp, j + kNP, lane) : dkdv_ops<D>(sm, b0, j, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      // fill of tile i+3 (its buffers held tile i-2, released at the last barrier)
      const bool issued = nf.hh >= 0;
      if (issued) fill_qtile<D, DOC>(sm, rs, b3, a, fp, nf, kvh, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
      int kpos_eff = kpos_mask;
      {
        const int cls = classify(mask, q.pmin, q.pmax, q.dmin, q.dmax, wkmin, wkmax, wkdmin, wkdmax);
        // fully visible tiles skip the position test (ragged tiles never count as full)
        if (wave_keys && cls == kTileFull && wk1 - wk0 == 32 && a.q_len - cur.qt * kBQ >= kBQ)
          kpos_eff = INT32_MIN + 1;
      }
      // S / dP of tile i, computed last iteration
      f32x16 scur = sv, dpcur = dpv;
      asm volatile("" : "+v"(scur), "+v"(dpcur));
      bf16x8 pf[2], dsf[2];
      sv = f32x16{};
      dpv = f32x16{};
      // stage k: the contractions of pair k and the operand reads of pair k + 2 (stage
      // boundaries keep each read two stages ahead of its use)
#pragma unroll
      for (int k = 0; k < D / 16; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        // S / dP of tile i+1, contraction step k
        sv = mfma32x32x16(ro[k & 1].aq, kf[k], sv);
        dpv = mfma32x32x16(ro[k & 1].ao, vf[k], dpv);
        // dV / dK of tile i-1, pair k (pairs 0 .. kNP-1 ran in the opening); the last
        // stages read the next iteration's first pairs (tile i is its previous tile)
        if (k >= kNP) {
          dkdv_mma<D>(to[k % kNP], k, ppf, pdsf, dk, dv);
          // slot k % kNP holds pair k + kNP of this tile, or, once those are done, the
          // next iteration's pair k % kNP (slot j serves pair j in the opening)
          to[k % kNP] = k + kNP < kPairs ? dkdv_ops<D>(sm, bp, k + kNP, lane)
                                          : dkdv_ops<D>(sm, b0, k % kNP, lane);
        }
        if (k + 2 < D / 16) ro[k & 1] = dkdv_rowops<D>(sm, b1, k + 2, lane);
        // P / dS of tile i, a quarter per (D / 64) stages
        if ((k + 1) * 4 % (D / 16) == 0)
          dkdv_pds<D, DOC>(rv, scur, dpcur, (k + 1) * 4 / (D / 16) - 1, kpos_eff, kdoc, a.scale_log2, pf, dsf);
      }
      __builtin_amdgcn_sched_barrier(0);
      // keep the P / dS arithmetic in this iteration (it is consumed by the next one)
      asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(dsf[0]), "v"(dsf[1]));
      bp = b0;
      ppf[0] = pf[0];
      ppf[1] = pf[1];
      pdsf[0] = dsf[0];
      pdsf[1] = dsf[1];
      if (n1.hh < 0) break;
      // tile i+2 landed (tile i+3's fill may still be in flight)
      wait_fills<D>(issued);
      if (n2.hh >= 0) seal_qtile(rs, b2, a, n2, wave, lane);
      lds_barrier();
      cur = n1;
      n1 = n2;
      n2 = nf;
      if (nf.hh >= 0) nf = next_qitem(nf, a.group, qlo, qhi);
      b0 = b1;
    }
    dkdv_acc_all<D>(sm, bp, ppf, pdsf, dk, dv, lane);
  }

  // per-owner sums: this wave's 32 keys, all local queries and all heads of the group.
  // The accumulators give each lane 16-byte pieces of 32 different key rows; stored as
  // they are, every instruction would leave its cache lines partly written.  Each wave
  // therefore stages its rows in its own part of the (now idle) tile images and stores
  // whole 512-byte rows, two per instruction.  LDS operations of one wave complete in
  // order, so the dV rows may overwrite the dK rows as soon as their reads are issued.
  // every wave is done with the tile images, and no fill into them is in flight
  __builtin_amdgcn_s_waitcnt(0x0F70);
  lds_barrier();
  {
    constexpr int kRow = D + 4;  // staged row stride in floats (rows 16 bytes apart in the banks)
    static_assert(sizeof(Sm) >= 4 * 32 * kRow * sizeof(float), "staging space");
    float* stg = reinterpret_cast<float*>(&sm) + wave * 32 * kRow;
    const int nrows = max(0, min(32, k1 - (k0 + wave * 32)));
    const float sc = a.scale;
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * h;
          const f32x16& acc = mat == 0 ? dk[db] : dv[db];
          const float m = mat == 0 ? sc : 1.0f;
          *reinterpret_cast<f32x4*>(stg + r * kRow + d0) =
              f32x4{acc[4 * g] * m, acc[4 * g + 1] * m, acc[4 * g + 2] * m, acc[4 * g + 3] * m};
        }
      }
      __builtin_amdgcn_wave_barrier();
      float* outp = mat == 0 ? a.dk[s] : a.dv[s];
      constexpr int kPieces = D / 4;         // 16-byte pieces per row
      constexpr int kRowsPer = kWave / kPieces;  // rows per store instruction
#pragma unroll
      for (int j = 0; j < 32 / kRowsPer; ++j) {
        const int row = j * kRowsPer + lane / kPieces;
        const int col = (lane % kPieces) * 4;
        const f32x4 val = *reinterpret_cast<const f32x4*>(stg + row * kRow + col);
        if (row < nrows)
          *reinterpret_cast<f32x4*>(outp + ((int64_t)(k0 + wave * 32 + row) * a.hkv + kvh) * D + col) = val;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  }  // key tile pass
}

}  // namespace

hipError_t launch_bwd_delta(const void* o, const void* dout, float* delta, int64_t pairs, int d,
                            hipStream_t stream) {
  if (pairs == 0) return hipSuccess;
  const int64_t threads = pairs * (d / 8);
  const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
  if (d == 64)
    hipLaunchKernelGGL((bwd_delta_kernel<64>), grid, dim3(kThreads), 0, stream,
                       reinterpret_cast<const bf16*>(o), reinterpret_cast<const bf16*>(dout), delta, pairs);
  else
    hipLaunchKernelGGL((bwd_delta_kernel<128>), grid, dim3(kThreads), 0, stream,
                       reinterpret_cast<const bf16*>(o), reinterpret_cast<const bf16*>(dout), delta, pairs);
  return hipGetLastError();
}

template <int D, int NW>
void launch_dq(bool ranked, dim3 grid, dim3 block, hipStream_t stream, const FwdArgs& f, const DqExtra& x) {
  if (ranked)
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, true>), grid, block, 0, stream, f, x);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, false>), grid, block, 0, stream, f, x);
}

hipError_t launch_bwd_dq(const FwdArgs& args, const void* dout, float* delta, float scale, int d,
                         bool accumulate, hipStream_t stream, const void* o) {
  FwdArgs f = args;
  // work-groups as in the forward kernel (wave count chosen by the plan)
  const int nw = f.wg_waves == 8 ? 8 : 4;
  const int qt_rows = nw * kv::kRowsPerWave / f.heads_per_wg;
  int total = 0;
  for (int j = 0; j < f.n_jobs; ++j) {
    f.jobs[j].wg_begin = total;
    total += ((f.jobs[j].len + qt_rows - 1) / qt_rows) * (f.hq / f.heads_per_wg) * f.jobs[j].n_split;
  }
  if (total == 0) return hipSuccess;
  f.total_wgs = total;
  f.padded_wgs = (total + 7) & ~7;
  const DqExtra x{dout, delta, scale, accumulate ? 1 : 0, o};
  const dim3 grid(f.padded_wgs), block(nw * kWave);
  const bool ranked = kv::ranked_plan(f, qt_rows, f.plan != nullptr ? kv::kMaxPlanTiles : kv::kMaxRankedTiles);
  if (!ranked) f.plan = nullptr;
  f.compact = !ranked && kv::compact_plan(f, qt_rows) ? 1 : 0;
  if (f.plan != nullptr) {
    if (d == 64)
      hipLaunchKernelGGL((kv::plan_ranked_kernel<64>), dim3(1), dim3(kv::kPlanThreads), 0, stream, f, qt_rows);
    else
      hipLaunchKernelGGL((kv::plan_ranked_kernel<128>), dim3(1), dim3(kv::kPlanThreads), 0, stream, f, qt_rows);
    const hipError_t pe = hipGetLastError();
    if (pe != hipSuccess) return pe;
  }
  if (d == 64) {
    if (nw == 8)
      launch_dq<64, 8>(ranked, grid, block, stream, f, x);
    else
      launch_dq<64, 4>(ranked, grid, block, stream, f, x);
  } else {
    if (nw == 8)
      launch_dq<128, 8>(ranked, grid, block, stream, f, x);
    else
      launch_dq<128, 4>(ranked, grid, block, stream, f, x);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int j = 0; j < f.n_jobs; ++j)
    if (f.jobs[j].n_split > 1) return launch_merge_split_jobs(f, d, 1, stream, true);
  return hipSuccess;
}

hipError_t launch_bwd_dkdv(const BwdArgs& args, int d, hipStream_t stream) {
  BwdArgs a = args;
  int total = 0;
  for (int s = 0; s < a.n_segs; ++s) {
    a.seg_wg_begin[s] = total;
    total += ((a.segs[s].len + kBKV - 1) / kBKV + 1) / 2 * a.hkv;  // pairs of key tiles
  }
  a.seg_wg_begin[a.n_segs] = total;
  a.total_wgs = total;
  a.padded_wgs = (total + 7) & ~7;
  if (total == 0) return hipSuccess;
  const bool doc = a.mask == kMaskCausalDoc;
  const dim3 grid(a.padded_wgs), block(kThreads);
  if (d == 64 && doc)
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, true>), grid, block, 0, stream, a);
  else if (d == 64)
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, false>), grid, block, 0, stream, a);
  else if (doc)
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}



}  // namespace cpattn
