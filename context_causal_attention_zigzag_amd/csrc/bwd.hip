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
constexpr int kMaxQTiles = 2048;  // query tiles of the LDS range table (65536 local rows)

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(const bf16* __restrict__ o,
                                                              const bf16* __restrict__ dout,
                                                              float* __restrict__ delta, int64_t pairs) {
  constexpr int kTpp = D / 8;  // threads per (row, head), 8 elements each
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t pair = gid / kTpp;
  const int c = (int)(gid % kTpp);
  float s = 0.0f;
  if (pair < pairs) {
    const int64_t off = pair * D + c * 8;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + off);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int w = kTpp / 2; w >= 1; w >>= 1) s += __shfl_xor(s, w, kTpp);
  if (pair < pairs && c == 0) delta[pair] = s;
}

// ---------------------------------------------------------------------------
// dQ pass
template <int D>
using DqSmem = kv::KvSmem<D, D + 32, D + 8>;  // K: row reads and transposing reads; V: row reads

struct DqExtra {
  const void* dout;
  const float* delta;  // [q_len, hq]
  float scale;         // softmax scale (factor of dS)
};

// One 64-key tile for one wave of the dQ pass.
template <int D>
__device__ __forceinline__ void dq_step(const bf16* __restrict__ ks, const bf16* __restrict__ vs,
                                        const int32_t* kpos, const int32_t* kdoc, int klen,
                                        const bf16x8 (&qf)[D / 16], const bf16x8 (&of)[D / 16],
                                        f32x16 (&dq)[D / 32], float lse2, float dl, int qpos, int qdoc,
                                        bool masked, int mask, float scale, float scale_log2, int lane) {
  constexpr int kKS = DqSmem<D>::kKS, kVS = DqSmem<D>::kVS;
  const int r = lane & 31, h = lane >> 5;
  bf16x8 dsf[4];  // dS^T as B operands of the four 16-key slices
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + r) * kKS + ds * 16 + h * 8);
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(vs + (kb * 32 + r) * kVS + ds * 16 + h * 8);
      s = mfma32x32x16(ak, qf[ds], s);
      dp = mfma32x32x16(av, of[ds], dp);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int base = kb * 32 + 8 * g + 4 * h;
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[4 * g + e], scale_log2, -lse2));
      if (masked) {
        const int4 kp = *reinterpret_cast<const int4*>(kpos + base);
        const int4 kd = *reinterpret_cast<const int4*>(kdoc + base);
        const int kpa[4] = {kp.x, kp.y, kp.z, kp.w};
        const int kda[4] = {kd.x, kd.y, kd.z, kd.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bool vis = base + e < klen;
          if (mask != kMaskNone) vis = vis && kpa[e] <= qpos;
          if (mask == kMaskCausalDoc) vis = vis && kda[e] == qdoc;
          p[e] = vis ? p[e] : 0.0f;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 4 * g + e;
        dsf[kb * 2 + (a >> 3)][a & 7] = (bf16)(p[e] * (dp[a] - dl) * scale);
      }
    }
  }
  // dQ^T += K^T dS^T: K^T slices by transposing reads in the rows order of dS^T
  const bf16* kl = ks + tr_lane_offset<4>(lane, kKS);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16* p = kl + j * 16 * kKS + db * 32;
      const bf16x8 a = concat(lds_read_tr4(p), lds_read_tr4(p + 8 * kKS));
      dq[db] = mfma32x32x16(a, dsf[j], dq[db]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(FwdArgs a, DqExtra x) {
  using namespace kv;
  __shared__ DqSmem<D> sm;
  const int logical = xcd_remap(blockIdx.x, a.padded_wgs);
  if (logical >= a.total_wgs) return;
  int j = 0;
  while (j + 1 < a.n_jobs && a.jobs[j + 1].wg_begin <= logical) ++j;
  const JobDesc& job = a.jobs[j];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hpw = a.heads_per_wg;
  const int qt_rows = (kv::kThreads / kWave) * kRowsPerWave / hpw;
  const int n_qt = (job.len + qt_rows - 1) / qt_rows;
  const int nsplit = job.n_split;
  const int local = logical - job.wg_begin;
  const int split = local % nsplit;
  const int rest = local / nsplit;
  const int hg = rest / n_qt;
  const int qt = n_qt - 1 - (rest - hg * n_qt);
  const int r0 = qt * qt_rows, r1 = min(job.len, r0 + qt_rows);
  const int head = hg * hpw + wave % hpw;
  const int kvh = (hg * hpw) / a.group;
  const int wr0 = r0 + (wave / hpw) * kRowsPerWave;
  const int wr1 = min(r1, wr0 + kRowsPerWave);
  const bool wave_rows = wr0 < wr1;
  const int myrow = wr0 + (lane & 31);
  const bool row_ok = myrow < wr1;
  const int mask = a.mask;

  const int qmin = job.pos[r0], qmax = job.pos[r1 - 1];
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

  bf16x8 qf[D / 16], of[D / 16];
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
      dl = x.delta[(int64_t)myrow * a.hq + head];
    }
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  float* flag_dst = nsplit > 1 ? job.ws_lse + (int64_t)split * job.len * a.hq : nullptr;
  TileIter it;
  it.mask_mode = nsplit > 1;
  if (nsplit > 1) {
    iter_init_masks(it, a, job, lane, qmin, qmax, qdmin, qdmax);
    const int total = iter_count(it);
    const int first = split * job.tiles_per_split;
    if (first >= total) {  // nothing in this split: mark its partial empty
      if (row_ok && (lane >> 5) == 0) flag_dst[(int64_t)myrow * a.hq + head] = neg_inf();
      return;
    }
    iter_seek(it, first, min(total - first, job.tiles_per_split), job.seg_begin);
  }

  FillPlan<D, DqSmem<D>> fp;
  fp.init(wave, lane);
  TileRef cur = iter_next(it, a, job, TileRef{-1, 0}, qmin, qmax, qdmin, qdmax);
  if (cur.seg >= 0) {
    fill_tile<D, DqSmem<D>>(sm, 0, a.segs[cur.seg], cur.tile, kvh, a.hkv, mask, wave, lane, fp);
    fill_barrier();
    int buf = 0;
    while (true) {
      const TileRef nxt = iter_next(it, a, job, cur, qmin, qmax, qdmin, qdmax);
      if (nxt.seg >= 0) fill_tile<D, DqSmem<D>>(sm, buf ^ 1, a.segs[nxt.seg], nxt.tile, kvh, a.hkv, mask, wave, lane, fp);
      if (wave_rows) {
        const int klen = min(kBK, a.segs[cur.seg].len - cur.tile * kBK);
        const int32_t* kp = sm.kpos[buf];
        const int32_t* kd = sm.kdoc[buf];
        int wcls = classify(mask, wqmin, wqmax, wqdmin, wqdmax, kp[0], kp[klen - 1],
                            mask == kMaskCausalDoc ? kd[0] : 0, mask == kMaskCausalDoc ? kd[klen - 1] : 0);
        if (wcls == kTileFull && klen < kBK) wcls = kTilePartial;
        if (wcls != kTileEmpty)
          dq_step<D>(sm.k[buf], sm.v[buf], kp, kd, klen, qf, of, dq, lse2, dl, qpos, qdoc, wcls == kTilePartial,
                     mask, x.scale, a.scale_log2, lane);
      }
      if (nxt.seg < 0) break;
      fill_barrier();
      buf ^= 1;
      cur = nxt;
    }
  }

  if (row_ok) {
    const int h = lane >> 5;
    const int64_t rowoff = ((int64_t)myrow * a.hq + head) * D;
    float* out = nsplit > 1 ? job.ws_o + (int64_t)split * job.len * a.hq * D : reinterpret_cast<float*>(job.o);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + h * 4;
        *reinterpret_cast<f32x4*>(out + rowoff + d0) =
            f32x4{dq[db][4 * g], dq[db][4 * g + 1], dq[db][4 * g + 2], dq[db][4 * g + 3]};
      }
    }
    if (nsplit > 1 && h == 0) flag_dst[(int64_t)myrow * a.hq + head] = 0.0f;
  }
}

// ---------------------------------------------------------------------------
// dK/dV pass
template <int D>
struct BwdSmem {
  // Row stride for gfx950's 64-bank LDS: transposing reads are conflict-free at 16
  // (mod 64) dwords, 16-byte row reads at 4 (mod 16) dwords; Q and dO serve both,
  // with twice as many transposing reads.
  static constexpr int kRS = D + 32;
  bf16 qs[2][kBQ * kRS];
  bf16 dos[2][kBQ * kRS];
  float lse2[2][kBQ];
  float delta[2][kBQ];
  int32_t qpos[2][kBQ];
  int32_t qdoc[2][kBQ];
  // first/last position and document of every query tile
  int32_t qtab[4][kMaxQTiles];
};

template <int D>
struct QStageRegs {
  static constexpr int kChunks = kBQ * D / 8 / 128;  // 16-byte chunks per thread
  u32x4 x[kChunks];  // rows of Q (threads 0..127) or of dO (threads 128..255)
  float lse2, delta;
  int32_t pos, doc;
};

template <int D>
__device__ __forceinline__ void load_qstage(QStageRegs<D>& r, const BwdArgs& a, const bf16* base, int head,
                                            int r0, int tid) {
  constexpr int kCPR = D / 8;
  const int u = tid & 127;
#pragma unroll
  for (int i = 0; i < QStageRegs<D>::kChunks; ++i) {
    const int c = u + 128 * i;
    const int row = r0 + c / kCPR, dc = c % kCPR;
    r.x[i] = row < a.q_len ? *reinterpret_cast<const u32x4*>(base + ((int64_t)row * a.hq + head) * D + dc * 8)
                           : u32x4{0, 0, 0, 0};
  }
  if (tid < kBQ) {
    const int row = r0 + tid;
    if (row < a.q_len) {
      const float l = a.lse[(int64_t)row * a.hq + head];
      r.lse2 = l == neg_inf() ? __builtin_inff() : l * kLog2e;  // a row with no key adds nothing
      r.delta = a.delta[(int64_t)row * a.hq + head];
      r.pos = a.qpos[row];
      r.doc = a.mask == kMaskCausalDoc ? a.qdoc[row] : 0;
    } else {
      r.lse2 = __builtin_inff();
      r.delta = 0.0f;
      r.pos = -kPosPad - 1;  // sees nothing
      r.doc = 0;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_qstage(BwdSmem<D>& sm, int buf, const QStageRegs<D>& r, int tid) {
  constexpr int kCPR = D / 8, kRS = BwdSmem<D>::kRS;
  bf16* dst = (tid >> 7) ? sm.dos[buf] : sm.qs[buf];
  const int u = tid & 127;
#pragma unroll
  for (int i = 0; i < QStageRegs<D>::kChunks; ++i) {
    const int c = u + 128 * i;
    *reinterpret_cast<u32x4*>(&dst[(c / kCPR) * kRS + (c % kCPR) * 8]) = r.x[i];
  }
  if (tid < kBQ) {
    sm.lse2[buf][tid] = r.lse2;
    sm.delta[buf][tid] = r.delta;
    sm.qpos[buf][tid] = r.pos;
    sm.qdoc[buf][tid] = r.doc;
  }
}

struct QRef {
  int hh;  // head within the kv group
  int qt;  // query tile
};

struct QRange {
  int pmin, pmax, dmin, dmax;
};

template <int D>
__device__ __forceinline__ QRange qrange(const BwdSmem<D>& sm, int t) {
  return {sm.qtab[0][t], sm.qtab[1][t], sm.qtab[2][t], sm.qtab[3][t]};
}

// Next visible (head, query tile) at or after (hh, qt) for the key range [kmin, kmax].
template <int D>
__device__ __forceinline__ QRef next_qtile(const BwdSmem<D>& sm, const BwdArgs& a, int hh, int qt, int n_qt,
                                           int kmin, int kmax, int kdmin, int kdmax) {
  for (; hh < a.group; ++hh, qt = 0) {
    for (; qt < n_qt; ++qt) {
      const QRange q = qrange(sm, qt);
      if (classify(a.mask, q.pmin, q.pmax, q.dmin, q.dmax, kmin, kmax, kdmin, kdmax) != kTileEmpty)
        return {hh, qt};
    }
  }
  return {-1, 0};
}

// One (32-row query tile, this wave's 32 keys) block: S = Q K^T and dP = dO V^T from
// row-major LDS rows and register-resident K/V; P and dS in the accumulator layout;
// dV^T += dO^T P and dK^T += Q^T dS with the transposed operands read by transposing
// LDS reads in the accumulators' contraction order.
// `masked` (wave-uniform) selects the per-element mask; one inlined copy of the step
// keeps the register allocation of the kernel tractable.
template <int D>
__device__ __forceinline__ void dkdv_step(BwdSmem<D>& sm, int buf, const bf16x8 (&kf)[D / 16],
                                          const bf16x8 (&vf)[D / 16], f32x16 (&dk)[D / 32],
                                          f32x16 (&dv)[D / 32], int kpos, int kdoc, bool key_ok,
                                          bool masked, int mask, float scale, float scale_log2, int lane) {
  constexpr int kRS = BwdSmem<D>::kRS;
  const int r = lane & 31, h = lane >> 5;
  f32x16 s = {}, dp = {};
  const bf16* qrow = sm.qs[buf] + r * kRS + h * 8;
  const bf16* orow = sm.dos[buf] + r * kRS + h * 8;
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qrow + ds * 16);
    const bf16x8 ao = *reinterpret_cast<const bf16x8*>(orow + ds * 16);
    s = mfma32x32x16(aq, kf[ds], s);
    dp = mfma32x32x16(ao, vf[ds], dp);
  }
  bf16x8 pf[2], dsf[2];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int q0 = 8 * g + 4 * h;
    const f32x4 l2 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][q0]);
    const f32x4 dl = *reinterpret_cast<const f32x4*>(&sm.delta[buf][q0]);
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[4 * g + e], scale_log2, -l2[e]));
    if (masked) {
      const int4 qp = *reinterpret_cast<const int4*>(&sm.qpos[buf][q0]);
      const int4 qd = *reinterpret_cast<const int4*>(&sm.qdoc[buf][q0]);
      const int qpa[4] = {qp.x, qp.y, qp.z, qp.w};
      const int qda[4] = {qd.x, qd.y, qd.z, qd.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool vis = key_ok;
        if (mask != kMaskNone) vis = vis && kpos <= qpa[e];
        if (mask == kMaskCausalDoc) vis = vis && kdoc == qda[e];
        p[e] = vis ? p[e] : 0.0f;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int a = 4 * g + e;
      pf[a >> 3][a & 7] = (bf16)p[e];
      dsf[a >> 3][a & 7] = (bf16)(p[e] * (dp[a] - dl[e]) * scale);
    }
  }
  const bf16* qtr = sm.qs[buf] + tr_lane_offset<4>(lane, kRS);
  const bf16* otr = sm.dos[buf] + tr_lane_offset<4>(lane, kRS);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int off = sl * 16 * kRS + db * 32;
      const bf16x8 ao = concat(lds_read_tr4(otr + off), lds_read_tr4(otr + off + 8 * kRS));
      const bf16x8 aq = concat(lds_read_tr4(qtr + off), lds_read_tr4(qtr + off + 8 * kRS));
      dv[db] = mfma32x32x16(ao, pf[sl], dv[db]);
      dk[db] = mfma32x32x16(aq, dsf[sl], dk[db]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ BwdSmem<D> sm;
  const int logical = xcd_remap(blockIdx.x, a.padded_wgs);
  if (logical >= a.total_wgs) return;
  int s = 0;
  while (s + 1 < a.n_segs && a.seg_wg_begin[s + 1] <= logical) ++s;
  const SegDesc& sg = a.segs[s];
  const int n_kt = (sg.len + kBKV - 1) / kBKV;
  const int local = logical - a.seg_wg_begin[s];
  const int kvh = local / n_kt;
  const int kt = local - kvh * n_kt;
  const int k0 = kt * kBKV, k1 = min(sg.len, k0 + kBKV);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int mask = a.mask;
  const bf16* kb = reinterpret_cast<const bf16*>(sg.k);
  const bf16* vb = reinterpret_cast<const bf16*>(sg.v);
  const bf16* stage_base = wave >= 2 ? reinterpret_cast<const bf16*>(a.dout) : reinterpret_cast<const bf16*>(a.q);

  // this wave's keys as B operands (lane: key 32*wave + r, dims 16*ds + 8*h .. +7)
  const int mykey = k0 + wave * 32 + r;
  const bool key_ok = mykey < k1;
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
  const int kpos = key_ok ? sg.pos[mykey] : kPosPad;
  const int kdoc = (key_ok && mask == kMaskCausalDoc) ? sg.doc[mykey] : 0;

  // key ranges of the work-group and of this wave (non-decreasing positions)
  const int kmin = sg.pos[k0], kmax = sg.pos[k1 - 1];
  int kdmin = 0, kdmax = 0;
  if (mask == kMaskCausalDoc) {
    kdmin = sg.doc[k0];
    kdmax = sg.doc[k1 - 1];
  }
  const int wk0 = k0 + wave * 32, wk1 = min(k1, wk0 + 32);
  const bool wave_keys = wk0 < wk1;
  int wkmin = 0, wkmax = 0, wkdmin = 0, wkdmax = 0;
  if (wave_keys) {
    wkmin = sg.pos[wk0];
    wkmax = sg.pos[wk1 - 1];
    if (mask == kMaskCausalDoc) {
      wkdmin = sg.doc[wk0];
      wkdmax = sg.doc[wk1 - 1];
    }
  }

  // per-query-tile position ranges in LDS (n_qt <= kMaxQTiles is checked on the host)
  const int n_qt = (a.q_len + kBQ - 1) / kBQ;
  for (int t = tid; t < n_qt; t += kThreads) {
    const int q0 = t * kBQ, q1 = min(a.q_len, q0 + kBQ) - 1;
    sm.qtab[0][t] = a.qpos[q0];
    sm.qtab[1][t] = a.qpos[q1];
    sm.qtab[2][t] = mask == kMaskCausalDoc ? a.qdoc[q0] : 0;
    sm.qtab[3][t] = mask == kMaskCausalDoc ? a.qdoc[q1] : 0;
  }
  lds_barrier();

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  QRef cur = next_qtile(sm, a, 0, 0, n_qt, kmin, kmax, kdmin, kdmax);
  if (cur.hh >= 0) {
    QStageRegs<D> qr;
    load_qstage<D>(qr, a, stage_base, kvh * a.group + cur.hh, cur.qt * kBQ, tid);
    store_qstage<D>(sm, 0, qr, tid);
    lds_barrier();
    int buf = 0;
    while (true) {
      const QRef nxt = next_qtile(sm, a, cur.hh, cur.qt + 1, n_qt, kmin, kmax, kdmin, kdmax);
      if (nxt.hh >= 0) load_qstage<D>(qr, a, stage_base, kvh * a.group + nxt.hh, nxt.qt * kBQ, tid);
      const int r0 = cur.qt * kBQ, r1 = min(a.q_len, r0 + kBQ);
      if (wave_keys) {
        const QRange q = qrange(sm, cur.qt);
        int wcls = classify(mask, q.pmin, q.pmax, q.dmin, q.dmax, wkmin, wkmax, wkdmin, wkdmax);
        if (wcls == kTileFull && (wk1 - wk0 < 32 || r1 - r0 < kBQ)) wcls = kTilePartial;
        if (wcls != kTileEmpty)
          dkdv_step<D>(sm, buf, kf, vf, dk, dv, kpos, kdoc, key_ok, wcls == kTilePartial, mask, a.scale,
                       a.scale_log2, lane);
      }
      if (nxt.hh < 0) break;
      // the other buffer was released by every wave at the previous barrier
      store_qstage<D>(sm, buf ^ 1, qr, tid);
      lds_barrier();
      buf ^= 1;
      cur = nxt;
    }
  }

  // per-owner sums: this wave's 32 keys, all local queries and all heads of the group
  if (key_ok) {
    float* dkp = a.dk[s];
    float* dvp = a.dv[s];
    const int64_t rowoff = ((int64_t)mykey * a.hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * h;
        *reinterpret_cast<f32x4*>(dkp + rowoff + d0) =
            f32x4{dk[db][4 * g], dk[db][4 * g + 1], dk[db][4 * g + 2], dk[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(dvp + rowoff + d0) =
            f32x4{dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
      }
    }
  }
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

hipError_t launch_bwd_dq(const FwdArgs& args, const void* dout, const float* delta, float scale, int d,
                         hipStream_t stream) {
  FwdArgs f = args;
  // work-groups as in the forward kernel
  const int qt_rows = (kv::kThreads / kWave) * kv::kRowsPerWave / f.heads_per_wg;
  int total = 0;
  for (int j = 0; j < f.n_jobs; ++j) {
    f.jobs[j].wg_begin = total;
    total += ((f.jobs[j].len + qt_rows - 1) / qt_rows) * (f.hq / f.heads_per_wg) * f.jobs[j].n_split;
  }
  if (total == 0) return hipSuccess;
  f.total_wgs = total;
  f.padded_wgs = (total + 7) & ~7;
  const DqExtra x{dout, delta, scale};
  if (d == 64)
    hipLaunchKernelGGL((bwd_dq_kernel<64>), dim3(f.padded_wgs), dim3(kThreads), 0, stream, f, x);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<128>), dim3(f.padded_wgs), dim3(kThreads), 0, stream, f, x);
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
    total += ((a.segs[s].len + kBKV - 1) / kBKV) * a.hkv;
  }
  a.seg_wg_begin[a.n_segs] = total;
  a.total_wgs = total;
  a.padded_wgs = (total + 7) & ~7;
  if (total == 0) return hipSuccess;
  if (d == 64)
    hipLaunchKernelGGL((bwd_dkdv_kernel<64>), dim3(a.padded_wgs), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<128>), dim3(a.padded_wgs), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

int bwd_max_rows() { return kMaxQTiles * kBQ; }

}  // namespace cpattn
