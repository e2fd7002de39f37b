// Forward attention kernels: TileAttention over task-graph edges and the
// streaming online-softmax form over KV segments in arrival order.
//
// Both forms run the same per-query-tile loop: for every KV tile (64 keys) that the
// query tile can see, the running row state (m, l, a) is updated as written in
// "上下文并行：一条序列跨卡，仍算同一个目标", section 02 (m' = max(m, max S),
// c = e^{m-m'}, l' = c l + sum e^{S-m'}, a' = c a + sum e^{S-m'} V), and at the end
// O = a / l and LSE = m + log l.  A job is either one edge of the Q-KV task graph
// ("Context Parallelism (CP)", section 2.1: output normalised inside its segment,
// fp32 O_ij and L_ij for a later merge) or one query block with its list of segments
// in ring arrival order (ring-attention page, section 2: final O in the input dtype).
//
// bf16 kernel (gfx950 matrix cores), per work-group of 4 waves, 32 query rows per wave,
// two work-groups per CU (two waves per SIMD: while one runs its softmax arithmetic
// or waits on LDS, the other keeps the matrix core busy):
//  - S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K from LDS is the A operand and the
//    wave's queries, held in registers for the whole loop, the B operand.  Each lane
//    then owns one query row (column of S^T), so row max / row sum are in-lane plus
//    one exchange between the two lane halves.
//  - P^T (bf16, converted in place from the accumulators) is directly the B operand
//    of O^T += V^T P^T.  V stays row-major in LDS; its transposed operand comes from
//    two transposing LDS reads (ds_read_b64_tr_b16) per product, addressed in the
//    contraction order the accumulator layout implies (common.h).
//  - The scale is applied to the fp32 scores (folded with log2 e into exp2).
//  - The running maximum is only moved when a new score exceeds it by more than
//    2^8 (probabilities stay <= 256, exact in fp32 and bf16 range), so the O rescale
//    is skipped on almost every tile.
//  - The tiles a work-group visits, and per wave the tiles it skips and those it sees
//    whole (no mask arithmetic), are found once per work-group by binary search over
//    each segment's key positions (kv_stream.h); the loop itself reads no segment
//    table and no key positions except for partially visible tiles.
//  - K/V tiles are double-buffered in LDS and filled by direct global->LDS loads
//    (no register staging): the next visible tile streams in while the current one
//    computes; one barrier per tile.
//
// fp32 kernel: a plain VALU kernel, one thread per (query row, head), used for fp32
// inputs (exact fp32 arithmetic, no bf16 rounding anywhere).
#include "common.h"
#include "kv_stream.h"

namespace cpattn {

namespace {

using namespace kv;

// K rows at stride D + 8 (row reads, conflict-free), V rows at D + 24 (transposing
// reads, 44% of their LDS cycles in conflicts; D + 32 would remove them but measured
// no faster and needs one more fill instruction per tile): 73 KiB with both
// double-buffered, two work-groups per CU.
template <int D>
using FwdSmem = KvSmem<D, D + 8, D + 24>;

// Work-group of the bf16 kernel: NW waves of 32 query rows share each K/V tile; 8
// waves (one work-group per CU, half the tile fills per query row) for launches whose
// query tiles fill the CUs, 4 (two work-groups per CU) with KV splits for small ones.
constexpr int wg_per_cu(int nw) { return nw == 8 ? 1 : 2; }

// V^T operand of O^T += V^T P^T for dims 32 db .. 32 db + 31 and key slice j (keys
// 16 j .. 16 j + 15 in the order of P^T's rows): two transposing reads of row-major V.
template <int D>
__device__ __forceinline__ bf16x8 v_op(const bf16* vl, int db, int j) {
  constexpr int kVS = FwdSmem<D>::kVS;
  const bf16* p = vl + j * 16 * kVS + db * 32;
  return concat(lds_read_tr4(p), lds_read_tr4(p + 8 * kVS));
}

// One KV tile for one wave: S^T, online-softmax update, O^T += V^T P^T, in four
// phases over the tile's two key halves A (keys 0..31) and B (32..63):
//   S_A;  S_B beside P_A;  O += V_A P_A beside P_B;  O += V_B P_B.
// Each middle phase pairs matrix-core work with independent vector work, so the wave
// keeps the matrix core busy while it exponentiates.  P of a half is computed against
// the running maximum of the earlier tiles (mu); a score above mu + 2^8 (rare after
// the first tile) sends the half through a rescale first: for half A before any of
// the tile's products (the maximum then covers the whole tile), for half B after
// the products of half A, which are still in the old scale and are rescaled with O.
// One code path for full and partial tiles (only the mask is conditional), so that
// the accumulators keep one register home across the loop.
template <int D>
__device__ __forceinline__ void tile_step(const bf16* __restrict__ ks, const bf16* __restrict__ vs,
                                          bool masked, const int32_t* kpos, const int32_t* kdoc, int klen,
                                          const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32],
                                          float& m, float& l, int qpos, int qdoc, int mask,
                                          float scale_log2, int lane) {
  constexpr int kKS = FwdSmem<D>::kKS;
  constexpr int kSt = D / 16;   // stages of each middle phase (= S steps = PV products per half)
  constexpr int kE = 16 / kSt;  // exponentials per stage
  static_assert(16 % kSt == 0 && kSt >= 4, "whole exponentials per stage");
  const int r = lane & 31, h = lane >> 5;
  const bf16* ka = ks + r * kKS + h * 8;
  const bf16* kb = ka + 32 * kKS;
  const bf16* vl = vs + tr_lane_offset<4>(lane, FwdSmem<D>::kVS);
  // product k of a PV phase: dims 32 (k / 2) .., key slice (k % 2) of the half
  auto vop = [&](int half, int k) { return v_op<D>(vl, k >> 1, 2 * half + (k & 1)); };
  auto kop = [&](const bf16* base, int ds) { return *reinterpret_cast<const bf16x8*>(base + ds * 16); };

  // S_A (raw scores; the softmax scale times log2 e is applied inside the exp argument)
  f32x16 sa = {}, sb = {};
#pragma unroll
  for (int ds = 0; ds < kSt; ++ds) sa = mfma32x32x16(kop(ka, ds), qf[ds], sa);
  // operands of the next phase's first two steps, two steps ahead from there on
  bf16x8 op[2] = {kop(kb, 0), kop(kb, 1)};
  if (masked) mask_half(sa, kpos, kdoc, klen, qpos, qdoc, mask, h, 0);
  float mu = (m == neg_inf()) ? 0.0f : m;

  // S_B beside P_A (at raised wave priority: the two middle phases feed the matrix core
  // while the other wave of the SIMD is in a phase without contractions)
  __builtin_amdgcn_s_setprio(1);
  bf16x8 pf[4];
  float rs = 0.0f, mta = neg_inf();
#pragma unroll
  for (int k = 0; k < kSt; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    sb = mfma32x32x16(op[k & 1], qf[k], sb);
    op[k & 1] = k + 2 < kSt ? kop(kb, k + 2) : vop(0, k + 2 - kSt);
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int i = k * kE + e;
      const float p = fast_exp2(fmaf(sa[i], scale_log2, -mu));
      rs += p;
      pf[i >> 3][i & 7] = (bf16)p;
      mta = fmaxf(mta, sa[i]);
    }
  }
  // keep P_A in its phase (it is used only after the branches below)
  asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(rs), "v"(mta));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  if (masked) mask_half(sb, kpos, kdoc, klen, qpos, qdoc, mask, h, 1);
  mta = half_max(mta) * scale_log2;  // -inf stays -inf (scale > 0)
  if (__any(mta > m + kTau)) {
    // the maximum moved in half A: rescale against the maximum of the whole tile (so
    // that half B cannot move it again), P_A again
    float mt = neg_inf();
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sb[i]);
    mt = fmaxf(mta, half_max(mt) * scale_log2);
    const float m_new = fmaxf(m, mt);
    const bool need = m_new > m + kTau;
    const float c = need ? fast_exp2(m - m_new) : 1.0f;
    if (need) m = m_new;
    mu = (m == neg_inf()) ? 0.0f : m;
    l *= c;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= c;
    rs = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(sa[i], scale_log2, -mu));
      rs += p;
      pf[i >> 3][i & 7] = (bf16)p;
    }
  }
  l += rs;

  // O += V_A P_A beside P_B
  __builtin_amdgcn_s_setprio(1);
  float mtb = neg_inf();
  rs = 0.0f;
#pragma unroll
  for (int k = 0; k < kSt; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    o[k >> 1] = mfma32x32x16(op[k & 1], pf[k & 1], o[k >> 1]);
    op[k & 1] = k + 2 < kSt ? vop(0, k + 2) : vop(1, k + 2 - kSt);
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int i = k * kE + e;
      const float p = fast_exp2(fmaf(sb[i], scale_log2, -mu));
      rs += p;
      pf[2 + (i >> 3)][i & 7] = (bf16)p;
      mtb = fmaxf(mtb, sb[i]);
    }
  }
  asm volatile("" ::"v"(pf[2]), "v"(pf[3]), "v"(rs), "v"(mtb));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  mtb = half_max(mtb) * scale_log2;
  if (__any(mtb > m + kTau)) {
    // the maximum moved in half B: O (with the products of half A, in the old scale)
    // and l follow, P_B again
    const float m_new = fmaxf(m, mtb);
    const bool need = m_new > m + kTau;
    const float c = need ? fast_exp2(m - m_new) : 1.0f;
    if (need) m = m_new;
    mu = (m == neg_inf()) ? 0.0f : m;
    l *= c;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= c;
    rs = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(sb[i], scale_log2, -mu));
      rs += p;
      pf[2 + (i >> 3)][i & 7] = (bf16)p;
    }
  }
  l += rs;

  // O += V_B P_B
#pragma unroll
  for (int k = 0; k < kSt; ++k) {
    o[k >> 1] = mfma32x32x16(op[k & 1], pf[2 + (k & 1)], o[k >> 1]);
    if (k + 2 < kSt) op[k & 1] = vop(1, k + 2);
  }
}

template <int D, bool PARTIAL_OUT, int NW, bool RANKED>
__global__ __launch_bounds__(NW * kWave, wg_per_cu(NW)) void fwd_bf16_kernel(FwdArgs a) {
  using Sm = FwdSmem<D>;
  __shared__ Sm sm;
  // the work-list scratch sits in the first K image, below the tile table
  static_assert(sizeof(Sm::k) / 2 >= (2 * kMaxRankedTiles + 16) * sizeof(int), "work-list scratch");
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
  const int h = lane >> 5;
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
  const bool doc = mask == kMaskCausalDoc;

  // work-group and wave query ranges (positions / documents are non-decreasing)
  const int qmax = job.pos[r1 - 1];
  int qdmin = 0, qdmax = 0, wqdmin = 0, wqdmax = 0;
  if (doc) {
    qdmin = job.doc[r0];
    qdmax = job.doc[r1 - 1];
  }
  int wqmin = 0, wqmax = -1;
  if (wave_rows) {
    wqmin = job.pos[wr0];
    wqmax = job.pos[wr1 - 1];
    if (doc) {
      wqdmin = job.doc[wr0];
      wqdmax = job.doc[wr1 - 1];
    }
  }

  bf16x8 qf[D / 16];
  int qpos = kPosPad, qdoc = 0;
  {
    const bf16* qb = reinterpret_cast<const bf16*>(job.q) + ((int64_t)myrow * a.hq + head) * D + h * 8;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) qf[ds] = row_ok ? *reinterpret_cast<const bf16x8*>(qb + ds * 16) : bf16x8{};
    if (row_ok) {
      qpos = job.pos[myrow];
      if (doc) qdoc = job.doc[myrow];
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m = neg_inf(), l = 0.0f;

  // destination: split partial (fp32, workspace), edge partial (fp32) or final output
  const bool out32 = PARTIAL_OUT || nsplit > 1;
  float* lse_dst = nsplit > 1 ? job.ws_lse + (int64_t)split * job.len * a.hq : job.lse;

  TileIter it;
  if (!RANKED && !tt_all && a.mask != kMaskNone)
    tt = load_tile_table<NW * kWave>(sm, a, ld, job.seg_begin, job.seg_end);
  iter_init_lanes(it, a, ld, job, lane, qmax, qdmin, qdmax, wave_rows, wqmin, wqmax, wqdmin, wqdmax, sm, tt);
  // compact launches run no work-group for the splits past a query tile's visible
  // tiles: the first split marks their partial states empty for the merge
  if (nsplit > 1 && split == 0 && row_ok && h == 0)
    for (int s = ns_mine; s < nsplit; ++s) job.ws_lse[((int64_t)s * job.len + myrow) * a.hq + head] = neg_inf();
  if (nsplit == 1) {
    iter_walk_all(it, job);
  } else if (!iter_walk_split(it, job, split * job.tiles_per_split, job.tiles_per_split)) {
    // nothing to do in this split: an empty partial state
    if (row_ok && h == 0) lse_dst[(int64_t)myrow * a.hq + head] = neg_inf();
    return;
  }

  const uint32_t rs = (uint32_t)a.hkv * D;  // elements between consecutive keys
  FillOffs<D, Sm, NW> fo;
  fo.init(wave, lane, rs);
  TileRef cur = iter_next(it, job, TileRef{-1, 0});
  if (cur.seg >= 0) {
    KvTile tc = iter_tile(it, cur, job.seg_begin, kvh, a.hkv, D);
    fill_tile<D, Sm>(sm, 0, tc, rs, doc, wave, lane, fo);
    fill_barrier();
    int buf = 0;
    while (true) {
      const TileRef nxt = iter_next(it, job, cur);
      KvTile tn = tc;
      // the other buffer was released by every wave at the previous barrier
      if (nxt.seg >= 0) {
        tn = iter_tile(it, nxt, job.seg_begin, kvh, a.hkv, D);
        fill_tile<D, Sm>(sm, buf ^ 1, tn, rs, doc, wave, lane, fo);
      }
      if (!tc.empty)
        tile_step<D>(sm.k[buf], sm.v[buf], !tc.full, sm.kpos[buf], sm.kdoc[buf], tc.last + 1, qf, o, m, l, qpos,
                     qdoc, mask, a.scale_log2, lane);
      if (nxt.seg < 0) break;
      fill_barrier();
      buf ^= 1;
      cur = nxt;
      tc = tn;
    }
  }

  // finalize: combine the two lane halves' partial sums, normalise, store.  A row that
  // saw a key has l >= 2^-8 (its largest score contributes at least that), so l == 0
  // means no visible key; a NaN input makes l NaN, which must reach O and the LSE.
  const float lt = half_sum(l);
  const bool live = !(lt == 0.0f);
  const float inv = live ? 1.0f / lt : 0.0f;
  const float lse = live ? (m + fast_log2(lt)) * kLn2 : neg_inf();
  if (row_ok) {
    const int64_t rowoff = ((int64_t)myrow * a.hq + head) * D;
    float* o32 = nsplit > 1 ? job.ws_o + (int64_t)split * job.len * a.hq * D : reinterpret_cast<float*>(job.o);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + h * 4;
        f32x4 v = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                   o[db][4 * g + 3] * inv};
        if (out32) {
          *reinterpret_cast<f32x4*>(o32 + rowoff + d0) = v;
        } else {
          bf16x4 b;
          b[0] = (bf16)v[0];
          b[1] = (bf16)v[1];
          b[2] = (bf16)v[2];
          b[3] = (bf16)v[3];
          *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(job.o) + rowoff + d0) = b;
        }
      }
    }
    if (h == 0) lse_dst[(int64_t)myrow * a.hq + head] = lse;
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: one thread per (query row, head), 64 rows of one head per block.
constexpr int kF32Rows = 64;
constexpr int kF32Keys = 32;

template <int D, bool PARTIAL_OUT>
__global__ __launch_bounds__(kF32Rows) void fwd_f32_kernel(FwdArgs a) {
  __shared__ float ks[kF32Keys][D + 1];
  __shared__ float vs[kF32Keys][D + 1];
  __shared__ int32_t kpos[kF32Keys];
  __shared__ int32_t kdoc[kF32Keys];
  const int logical = blockIdx.x;
  if (logical >= a.total_wgs) return;
  int j = 0;
  while (j + 1 < a.n_jobs && a.jobs[j + 1].wg_begin <= logical) ++j;
  const JobDesc& job = a.jobs[j];
  const int n_qt = (job.len + kF32Rows - 1) / kF32Rows;
  const int local = logical - job.wg_begin;
  const int head = local / n_qt;
  const int qt = local - head * n_qt;
  const int r0 = qt * kF32Rows, r1 = min(job.len, r0 + kF32Rows);
  const int tid = threadIdx.x;
  const int row = r0 + tid;
  const bool row_ok = row < r1;
  const int kvh = head / a.group;
  const int mask = a.mask;
  const float* qp = reinterpret_cast<const float*>(job.q) + ((int64_t)(row_ok ? row : r0) * a.hq + head) * D;
  float q[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    q[i] = row_ok ? qp[i] : 0.0f;
    acc[i] = 0.0f;
  }
  const int qpos = row_ok ? job.pos[row] : 0;
  const int qdoc = (row_ok && mask == kMaskCausalDoc) ? job.doc[row] : 0;
  const int qmin = job.pos[r0], qmax = job.pos[r1 - 1];
  const int qdmin = mask == kMaskCausalDoc ? job.doc[r0] : 0;
  const int qdmax = mask == kMaskCausalDoc ? job.doc[r1 - 1] : 0;
  const float scale = a.scale_log2 * kLn2;
  float m = neg_inf(), l = 0.0f;
  for (int s = job.seg_begin; s < job.seg_end; ++s) {
    const SegDesc& sg = a.segs[s];
    const float* kb = reinterpret_cast<const float*>(sg.k);
    const float* vb = reinterpret_cast<const float*>(sg.v);
    for (int k0 = 0; k0 < sg.len; k0 += kF32Keys) {
      const int klen = min(kF32Keys, sg.len - k0);
      const int kdmin = mask == kMaskCausalDoc ? sg.doc[k0] : 0;
      const int kdmax = mask == kMaskCausalDoc ? sg.doc[k0 + klen - 1] : 0;
      if (classify(mask, qmin, qmax, qdmin, qdmax, sg.pos[k0], sg.pos[k0 + klen - 1], kdmin, kdmax) ==
          kTileEmpty)
        continue;
      __syncthreads();
      for (int i = tid; i < klen * D; i += kF32Rows) {
        const int key = i / D, dd = i % D;
        ks[key][dd] = kb[((int64_t)(k0 + key) * a.hkv + kvh) * D + dd];
        vs[key][dd] = vb[((int64_t)(k0 + key) * a.hkv + kvh) * D + dd];
      }
      if (tid < klen) {
        kpos[tid] = sg.pos[k0 + tid];
        kdoc[tid] = mask == kMaskCausalDoc ? sg.doc[k0 + tid] : 0;
      }
      __syncthreads();
      for (int key = 0; key < klen; ++key) {
        bool vis = true;
        if (mask != kMaskNone) vis = kpos[key] <= qpos;
        if (mask == kMaskCausalDoc) vis = vis && kdoc[key] == qdoc;
        if (!vis) continue;
        float sc = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) sc = fmaf(q[i], ks[key][i], sc);
        sc *= scale;
        const float m_new = fmaxf(m, sc);
        const float c = expf(m - m_new);
        const float p = expf(sc - m_new);
        l = l * c + p;
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] = fmaf(p, vs[key][i], acc[i] * c);
        m = m_new;
      }
    }
  }
  if (!row_ok) return;
  const bool live = !(l == 0.0f);  // NaN inputs stay NaN
  const float inv = live ? 1.0f / l : 0.0f;
  const int64_t off = ((int64_t)row * a.hq + head) * D;
  float* out = reinterpret_cast<float*>(job.o) + off;  // fp32 in both modes
#pragma unroll
  for (int i = 0; i < D; ++i) out[i] = acc[i] * inv;
  job.lse[(int64_t)row * a.hq + head] = live ? m + logf(l) : neg_inf();
}

template <int D, bool PARTIAL_OUT, int NW>
void launch_fwd_bf16(bool ranked, dim3 grid, dim3 block, hipStream_t stream, const FwdArgs& a) {
  if (ranked)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, PARTIAL_OUT, NW, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, PARTIAL_OUT, NW, false>), grid, block, 0, stream, a);
}

template <int D>
hipError_t launch_fwd_d(FwdArgs& a, int dtype, bool partial_out, hipStream_t stream) {
  if (dtype == 0) {
    const int hpw = a.heads_per_wg;
    const int nw = a.wg_waves == 8 ? 8 : 4;
    const int qt_rows = nw * kRowsPerWave / hpw;
    int total = 0;
    for (int j = 0; j < a.n_jobs; ++j) {
      a.jobs[j].wg_begin = total;
      const int n_qt = (a.jobs[j].len + qt_rows - 1) / qt_rows;
      total += n_qt * (a.hq / hpw) * a.jobs[j].n_split;
    }
    a.total_wgs = total;
    a.padded_wgs = (total + 7) & ~7;
    if (total == 0) return hipSuccess;
    const dim3 grid(a.padded_wgs), block(nw * kWave);
    const bool ranked = ranked_plan(a, qt_rows, a.plan != nullptr ? kMaxPlanTiles : kMaxRankedTiles);
    if (!ranked) a.plan = nullptr;
    a.compact = !ranked && compact_plan(a, qt_rows) ? 1 : 0;
    if (a.plan != nullptr) {
      hipLaunchKernelGGL((plan_ranked_kernel<D>), dim3(1), dim3(kPlanThreads), 0, stream, a, qt_rows);
      const hipError_t pe = hipGetLastError();
      if (pe != hipSuccess) return pe;
    }
    if (nw == 8) {
      if (partial_out)
        launch_fwd_bf16<D, true, 8>(ranked, grid, block, stream, a);
      else
        launch_fwd_bf16<D, false, 8>(ranked, grid, block, stream, a);
    } else {
      if (partial_out)
        launch_fwd_bf16<D, true, 4>(ranked, grid, block, stream, a);
      else
        launch_fwd_bf16<D, false, 4>(ranked, grid, block, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // log-sum-exp merge of the KV splits of every split job, one launch
    bool any_split = false;
    for (int j = 0; j < a.n_jobs; ++j) any_split |= a.jobs[j].n_split > 1;
    if (any_split) {
      e = launch_merge_split_jobs(a, D, partial_out ? 1 : dtype, stream);
      if (e != hipSuccess) return e;
    }
  } else {
    int total = 0;
    for (int j = 0; j < a.n_jobs; ++j) {
      a.jobs[j].wg_begin = total;
      total += ((a.jobs[j].len + kF32Rows - 1) / kF32Rows) * a.hq;
    }
    a.total_wgs = total;
    a.padded_wgs = total;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3(total), dim3(kF32Rows), 0, stream, a);
  }
  return hipGetLastError();
}

constexpr int kMaxSplitTiles = 256;   // jobs longer than this carry enough work per query tile
// 1024 keys per split at least: each split writes an fp32 partial output of its query
// tile (4*d bytes per row) for 4*d flops per row and key, so shorter runs would turn
// the kernel into a writer of partial states
constexpr int kMinTilesPerSplit = 16;
constexpr int kMaxSplits = 64;        // parts the merge kernel takes

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// KV-split plan.  When the query tiles alone give fewer work-groups than the chip
// holds at once (wg_per_cu of the chosen size per compute unit), each job's visible KV
// tiles are cut into splits of tiles_per_split tiles, sized so that the busy
// work-groups fit one round: a query tile with V visible tiles takes ceil(V / u)
// work-groups, about V / u + 1/2, and under causal masking an average query tile sees
// about half of its job's tiles, so u = (sum of V) / (slots - query tiles / 2).  Jobs
// spanning more than 256 KV tiles are never split (they carry enough work per query
// tile).
size_t plan_fwd(FwdArgs& a, int d, int dtype, int num_cu, bool allow_split, int waves) {
  for (int j = 0; j < a.n_jobs; ++j) {
    JobDesc& jb = a.jobs[j];
    int off = 0;
    for (int s = jb.seg_begin; s < jb.seg_end; ++s) off += (a.segs[s].len + kBK - 1) / kBK;
    jb.n_tiles = off;
    jb.n_split = 1;
    jb.tiles_per_split = off;
    jb.ws_o = nullptr;
    jb.ws_lse = nullptr;
  }
  const int hpw = a.heads_per_wg;
  auto query_wgs = [&](int nw) {
    const int qt_rows = nw * kRowsPerWave / hpw;
    int64_t n = 0;
    for (int j = 0; j < a.n_jobs; ++j) n += (int64_t)((a.jobs[j].len + qt_rows - 1) / qt_rows) * (a.hq / hpw);
    return n;
  };
  if (waves == 0) waves = query_wgs(8) > num_cu ? 8 : 4;
  a.wg_waves = waves;
  a.plan_tiles = 0;
  a.plan = nullptr;
  if (dtype != 0 || !allow_split) return 0;
  const int64_t base = query_wgs(waves);
  const int64_t slots = (int64_t)wg_per_cu(waves) * num_cu;
  const int qt_rows = waves * kRowsPerWave / hpw;
  if (base == 0 || base >= slots) {
    // no KV split: a ranked launch is planned once when it runs more than two rounds of
    // work-groups (the per-work-group ranking then costs more than one plan) or holds
    // more query tiles than a work-group can rank
    if (base > 0 && kv::ranked_plan(a, qt_rows, kv::kMaxPlanTiles)) {
      int n_all = 0, n_tab = 0;
      kv::plan_layout(a, d, qt_rows, n_all, n_tab);
      if (base > 2 * slots || n_all > kv::kMaxRankedTiles) {
        a.plan_tiles = n_all;
        return align256(kv::plan_bytes(n_all, n_tab));
      }
    }
    return 0;
  }
  int64_t visible = 0;  // expected visible (query tile, KV tile) pairs over all work-groups
  for (int j = 0; j < a.n_jobs; ++j)
    visible += (int64_t)((a.jobs[j].len + qt_rows - 1) / qt_rows) * (a.hq / hpw) * a.jobs[j].n_tiles / 2;
  const int64_t room = slots - base / 2;
  const int64_t u_all = (visible + room - 1) / room;
  size_t bytes = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    JobDesc& jb = a.jobs[j];
    if (jb.n_tiles > kMaxSplitTiles || jb.n_tiles <= 2 * kMinTilesPerSplit) continue;
    int64_t u = u_all;
    if (u < kMinTilesPerSplit) u = kMinTilesPerSplit;
    int ns = (int)((jb.n_tiles + u - 1) / u);
    if (ns > kMaxSplits) {
      ns = kMaxSplits;
      u = (jb.n_tiles + ns - 1) / ns;
    }
    if (ns <= 1) continue;
    jb.n_split = ns;
    jb.tiles_per_split = (int)u;
    bytes += align256((size_t)ns * jb.len * a.hq * d * sizeof(float));
    bytes += align256((size_t)ns * jb.len * a.hq * sizeof(float));
  }
  return bytes;
}

void assign_fwd_workspace(FwdArgs& a, int d, void* ws) {
  char* p = reinterpret_cast<char*>(ws);
  for (int j = 0; j < a.n_jobs; ++j) {
    JobDesc& jb = a.jobs[j];
    if (jb.n_split <= 1) continue;
    jb.ws_o = reinterpret_cast<float*>(p);
    p += align256((size_t)jb.n_split * jb.len * a.hq * d * sizeof(float));
    jb.ws_lse = reinterpret_cast<float*>(p);
    p += align256((size_t)jb.n_split * jb.len * a.hq * sizeof(float));
  }
  if (a.plan_tiles > 0) a.plan = reinterpret_cast<int32_t*>(p);
}

hipError_t launch_fwd(const FwdArgs& args, int d, int dtype, bool partial_out, hipStream_t stream) {
  FwdArgs a = args;
  if (d == 64) return launch_fwd_d<64>(a, dtype, partial_out, stream);
  return launch_fwd_d<128>(a, dtype, partial_out, stream);
}

}  // namespace cpattn
