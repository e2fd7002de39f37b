// LSE-replay backward of one rank's share.
//
// "上下文并行：一条序列跨卡，仍算同一个目标", sections 01-02: each KV block is
// replayed against the local queries; the block's probabilities are rebuilt from
// the saved full-row log-sum-exp, P_ij = exp(S_ij - lambda_i); the softmax
// derivative gives dS_ij = P_ij (dP_ij - D_i) with dP = G V^T and D_i = G_i . O_i;
// then dQ_i += dS_ij K_j / sqrt(d), dK_j += dS_ij Q_i / sqrt(d), dV_j += P_ij G_i,
// and the K/V gradients of every query are summed at the owner of the keys.
//
// Kernel layout (gfx950, v_mfma_f32_32x32x16_bf16):
//  - preprocess: D_i = rowsum(dO * O) in fp32 into the workspace, dQ zeroed.
//  - main: one work-group of 4 waves per (KV segment, 128-key tile, kv head); wave w
//    keeps keys 32w..32w+31 (K and V rows) in registers as B operands and owns their
//    dK/dV accumulators, so the per-owner sums over all local queries and all query
//    heads of the group finish in registers and are stored once (no atomics).
//    The work-group walks the visible 32-row query tiles: Q and dO are staged row-major
//    in LDS; they are the A operands of S = Q K^T and dP = dO V^T as plain row reads,
//    and of dV^T = dO^T P and dK^T = Q^T dS through transposing LDS reads addressed in
//    the contraction order of the accumulator layout, so P and dS feed the matrix
//    cores straight from the accumulators.  dS goes through LDS once more for
//    dQ = dS K (K^T slices read transposed from a row-major K tile), computed per
//    32-dim slice by each wave and added to the fp32 dQ with coalesced atomics.
//  - one LDS-only barrier per query tile; query tiles are staged two ahead so the
//    staging loads never wait behind the dQ atomics (see the main loop).
#include "common.h"

namespace cpattn {

namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 128;  // keys per work-group (32 per wave)
constexpr int kBQ = 32;    // query rows per step
constexpr int kPosPad = 0x7fffffff;
constexpr int kMaxQTiles = 2048;  // query tiles of the LDS range table (65536 local rows)

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const bf16* __restrict__ o,
                                                            const bf16* __restrict__ dout,
                                                            float* __restrict__ delta,
                                                            float* __restrict__ dq, int64_t pairs) {
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
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dq + off) = z;
    *reinterpret_cast<f32x4*>(dq + off + 4) = z;
  }
#pragma unroll
  for (int w = kTpp / 2; w >= 1; w >>= 1) s += __shfl_xor(s, w, kTpp);
  if (pair < pairs && c == 0) delta[pair] = s;
}

// ---------------------------------------------------------------------------
template <int D>
struct BwdSmem {
  // Row strides for gfx950's 64-bank LDS: transposing reads are conflict-free at 16
  // (mod 64) dwords, 16-byte row reads at 4 (mod 16) dwords.  Q and dO serve both
  // (twice as many transposing reads), K only transposing reads, dS only row reads.
  static constexpr int kRS = D + 32;    // Q / dO
  static constexpr int kKS = D + 32;    // K
  static constexpr int kSS = kBKV + 8;  // dS
  bf16 qs[2][kBQ * kRS];
  bf16 dos[2][kBQ * kRS];
  float lse2[2][kBQ];
  float delta[2][kBQ];
  int32_t qpos[2][kBQ];
  int32_t qdoc[2][kBQ];
  bf16 ds[2][kBQ * kSS];
  bf16 ks[kBKV * kKS];
  // first/last position and document of every query tile, so the per-tile
  // classification reads LDS instead of global memory (a vector load there would
  // wait behind the outstanding dQ atomics)
  int32_t qtab[4][kMaxQTiles];
};

template <int D>
struct QStageRegs {
  static constexpr int kChunks = kBQ * D / 8 / 128;  // 16-byte chunks per thread
  u32x4 x[kChunks];  // rows of Q (threads 0..127) or of dO (threads 128..255), raw
  float lse, delta;  // raw values of row r0 + (tid % 32), clamped to the last row
  int32_t pos, doc;
  int32_t r0;        // first row of the staged tile
};

// Every lane issues the same loads on every call (rows past the end are clamped):
// the number of vector-memory operations between these loads and their use is then
// the same on every path, so the wait at the LDS store leaves the younger dQ atomics
// in flight.  Nothing here touches the loaded values; store_qstage() zeroes the rows
// past the end and converts the LSE.
template <int D>
__device__ __forceinline__ void load_qstage(QStageRegs<D>& r, const BwdArgs& a, const bf16* base, int head,
                                            int r0, int tid) {
  constexpr int kCPR = D / 8;
  const int u = tid & 127;
  const int last = a.q_len - 1;
#pragma unroll
  for (int i = 0; i < QStageRegs<D>::kChunks; ++i) {
    const int c = u + 128 * i;
    const int row = min(r0 + c / kCPR, last), dc = c % kCPR;
    r.x[i] = *reinterpret_cast<const u32x4*>(base + ((int64_t)row * a.hq + head) * D + dc * 8);
  }
  const int64_t rr = min(r0 + (tid & (kBQ - 1)), last);
  r.lse = a.lse[rr * a.hq + head];
  r.delta = a.delta[rr * a.hq + head];
  r.pos = a.qpos[rr];
  r.doc = a.qdoc[rr];  // a valid array for every mask (the host passes positions when unused)
  r.r0 = r0;
}

template <int D>
__device__ __forceinline__ void store_qstage(BwdSmem<D>& sm, int buf, const QStageRegs<D>& r, int q_len,
                                             int mask, int tid) {
  constexpr int kCPR = D / 8, kRS = BwdSmem<D>::kRS;
  const int half = tid >> 7;
  const int u = tid & 127;
  bf16* dst = half ? sm.dos[buf] : sm.qs[buf];
#pragma unroll
  for (int i = 0; i < QStageRegs<D>::kChunks; ++i) {
    const int c = u + 128 * i;
    const bool ok = r.r0 + c / kCPR < q_len;
    const u32x4 x = r.x[i];
    *reinterpret_cast<u32x4*>(&dst[(c / kCPR) * kRS + (c % kCPR) * 8]) =
        u32x4{ok ? x[0] : 0u, ok ? x[1] : 0u, ok ? x[2] : 0u, ok ? x[3] : 0u};
  }
  if (tid < kBQ) {
    const bool ok = r.r0 + tid < q_len;
    // a row past the end, or one with no visible key, contributes nothing
    sm.lse2[buf][tid] = (ok && r.lse != neg_inf()) ? r.lse * kLog2e : __builtin_inff();
    sm.delta[buf][tid] = ok ? r.delta : 0.0f;
    sm.qpos[buf][tid] = ok ? r.pos : -kPosPad - 1;
    sm.qdoc[buf][tid] = mask == kMaskCausalDoc ? r.doc : 0;
  }
}

struct QRef {
  int hh;  // head within the kv group
  int qt;  // query tile
};

// Position / document range of query tile t (LDS table).
struct QRange {
  int pmin, pmax, dmin, dmax;
};

template <int D>
__device__ __forceinline__ QRange qrange(const BwdSmem<D>& sm, int t) {
  return {sm.qtab[0][t], sm.qtab[1][t], sm.qtab[2][t], sm.qtab[3][t]};
}

// Next visible (head, query tile) at or after (hh, qt) for the key range [kmin, kmax].
template <int D>
__device__ __forceinline__ QRef next_qtile(const BwdSmem<D>& sm, const BwdArgs& a, int hh, int qt,
                                           int n_qt, int kmin, int kmax, int kdmin, int kdmax) {
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
// LDS reads in the accumulators' contraction order; dS also goes to LDS for dQ.
template <int D, bool MASKED>
__device__ __forceinline__ void bwd_step(BwdSmem<D>& sm, int buf, const bf16x8 (&kf)[D / 16],
                                         const bf16x8 (&vf)[D / 16], f32x16 (&dk)[D / 32],
                                         f32x16 (&dv)[D / 32], int kpos, int kdoc, bool key_ok,
                                         int mask, float scale, float scale_log2, int wave, int lane) {
  constexpr int kRS = BwdSmem<D>::kRS, kSS = BwdSmem<D>::kSS;
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
  bf16* dsw = sm.ds[buf] + 4 * h * kSS + wave * 32 + r;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int q0 = 8 * g + 4 * h;
    const f32x4 l2 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][q0]);
    const f32x4 dl = *reinterpret_cast<const f32x4*>(&sm.delta[buf][q0]);
    int4 qp = {0, 0, 0, 0}, qd = {0, 0, 0, 0};
    if (MASKED) {
      qp = *reinterpret_cast<const int4*>(&sm.qpos[buf][q0]);
      if (mask == kMaskCausalDoc) qd = *reinterpret_cast<const int4*>(&sm.qdoc[buf][q0]);
    }
    const int qpa[4] = {qp.x, qp.y, qp.z, qp.w};
    const int qda[4] = {qd.x, qd.y, qd.z, qd.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int a = 4 * g + e;
      float p = fast_exp2(fmaf(s[a], scale_log2, -l2[e]));
      if (MASKED) {
        bool vis = key_ok;
        if (mask != kMaskNone) vis = vis && kpos <= qpa[e];
        if (mask == kMaskCausalDoc) vis = vis && kdoc == qda[e];
        p = vis ? p : 0.0f;
      }
      const float dsv = p * (dp[a] - dl[e]) * scale;
      pf[a >> 3][a & 7] = (bf16)p;
      const bf16 dsb = (bf16)dsv;
      dsf[a >> 3][a & 7] = dsb;
      dsw[(8 * g + e) * kSS] = dsb;
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
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdArgs a) {
  __shared__ BwdSmem<D> sm;
  constexpr int kSS = BwdSmem<D>::kSS, kKS = BwdSmem<D>::kKS;
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r = lane & 31, h = lane >> 5;
  const int mask = a.mask;
  const bf16* kb = reinterpret_cast<const bf16*>(sg.k);
  const bf16* vb = reinterpret_cast<const bf16*>(sg.v);
  // staging source of this wave: Q for waves 0-1, dO for waves 2-3 (a value select,
  // never a per-lane load of the argument block inside the loop)
  const bf16* qb = reinterpret_cast<const bf16*>(a.q);
  const bf16* ob = reinterpret_cast<const bf16*>(a.dout);
  const bf16* stage_base = wave >= 2 ? ob : qb;

  // this wave's keys as B operands (lane: key 32*wave + r, dims 16*ds + 8*h .. +7)
  const int mykey = k0 + wave * 32 + r;
  const bool key_ok = mykey < k1;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    if (key_ok) {
      const int64_t off = ((int64_t)mykey * a.hkv + kvh) * D + ds * 16 + h * 8;
      kf[ds] = *reinterpret_cast<const bf16x8*>(kb + off);
      vf[ds] = *reinterpret_cast<const bf16x8*>(vb + off);
    } else {
      kf[ds] = bf16x8{};
      vf[ds] = bf16x8{};
    }
  }
  const int kpos = key_ok ? sg.pos[mykey] : kPosPad;
  const int kdoc = (key_ok && mask == kMaskCausalDoc) ? sg.doc[mykey] : 0;

  // the work-group's K tile, row-major in LDS (operand of dQ = dS K)
  for (int c = tid; c < kBKV * (D / 8); c += kThreads) {
    const int key = c / (D / 8), dc = c % (D / 8);
    u32x4 x = {0, 0, 0, 0};
    if (k0 + key < k1) x = *reinterpret_cast<const u32x4*>(kb + ((int64_t)(k0 + key) * a.hkv + kvh) * D + dc * 8);
    *reinterpret_cast<u32x4*>(&sm.ks[key * kKS + dc * 8]) = x;
  }

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

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // dQ operand: K^T slice of this wave's 32 dims via transposing reads, natural key order
  const bf16* ktr = sm.ks + tr_lane_offset<8>(lane, kKS) + wave * 32;
  const int n_qt = (a.q_len + kBQ - 1) / kBQ;
  // n_qt <= kMaxQTiles is checked on the host
  for (int t = tid; t < n_qt; t += kThreads) {
    const int r0 = t * kBQ, r1 = min(a.q_len, r0 + kBQ) - 1;
    sm.qtab[0][t] = a.qpos[r0];
    sm.qtab[1][t] = a.qpos[r1];
    sm.qtab[2][t] = mask == kMaskCausalDoc ? a.qdoc[r0] : 0;
    sm.qtab[3][t] = mask == kMaskCausalDoc ? a.qdoc[r1] : 0;
  }
  lds_barrier();
  // Prefetch order matters: vmcnt is one in-order counter for loads, stores and
  // atomics.  Tiles 0 and 1 are staged before the loop; inside it, the staging loads
  // of tile t+2 are issued after the barrier of tile t and before tile t's dQ atomics,
  // and stored to LDS during tile t+1.  Every path from those loads to their use
  // crosses exactly the 16 atomics of one tile, so the wait before the LDS store
  // leaves them in flight instead of waiting for their round trip.
  QRef cur = next_qtile(sm, a, 0, 0, n_qt, kmin, kmax, kdmin, kdmax);
  if (cur.hh >= 0) {
    QStageRegs<D> qr;
    load_qstage<D>(qr, a, stage_base, kvh * a.group + cur.hh, cur.qt * kBQ, tid);
    store_qstage<D>(sm, 0, qr, a.q_len, mask, tid);
    QRef nxt = next_qtile(sm, a, cur.hh, cur.qt + 1, n_qt, kmin, kmax, kdmin, kdmax);
    if (nxt.hh >= 0) {
      load_qstage<D>(qr, a, stage_base, kvh * a.group + nxt.hh, nxt.qt * kBQ, tid);
      store_qstage<D>(sm, 1, qr, a.q_len, mask, tid);
    }
    lds_barrier();
    int buf = 0;
    bool staged_next = true;  // the next tile's stage is already in LDS
    while (true) {
      const int head = kvh * a.group + cur.hh;
      const int r0 = cur.qt * kBQ, r1 = min(a.q_len, r0 + kBQ);
      // wave-level class of (query tile, this wave's keys)
      int wcls = kTileEmpty;
      if (wave_keys) {
        const QRange q = qrange(sm, cur.qt);
        wcls = classify(mask, q.pmin, q.pmax, q.dmin, q.dmax, wkmin, wkmax, wkdmin, wkdmax);
        if (wcls == kTileFull && (wk1 - wk0 < 32 || r1 - r0 < kBQ)) wcls = kTilePartial;
      }
      if (wcls == kTileFull)
        bwd_step<D, false>(sm, buf, kf, vf, dk, dv, kpos, kdoc, key_ok, mask, a.scale, a.scale_log2, wave, lane);
      else if (wcls == kTilePartial)
        bwd_step<D, true>(sm, buf, kf, vf, dk, dv, kpos, kdoc, key_ok, mask, a.scale, a.scale_log2, wave, lane);
      else {
        bf16* dsw = sm.ds[buf] + wave * 32 + r;
#pragma unroll
        for (int q = 0; q < kBQ / 2; ++q) dsw[(2 * q + h) * kSS] = (bf16)0.0f;
      }
      // the other buffer's Q/dO stage was released by every wave at the previous barrier
      if (!staged_next && nxt.hh >= 0) store_qstage<D>(sm, buf ^ 1, qr, a.q_len, mask, tid);
      staged_next = false;
      lds_barrier();
      QRef nxt2 = {-1, 0};
      if (nxt.hh >= 0) nxt2 = next_qtile(sm, a, nxt.hh, nxt.qt + 1, n_qt, kmin, kmax, kdmin, kdmax);
      {
        const QRef ld = nxt2.hh >= 0 ? nxt2 : cur;  // always issue the loads (see load_qstage)
        load_qstage<D>(qr, a, stage_base, kvh * a.group + ld.hh, ld.qt * kBQ, tid);
      }
      // dQ[q][32*wave .. +31] += dS[q][:] K[:][...]  (scale already folded into dS)
      if (D == 128 || wave * 32 < D) {  // D = 64: two waves cover the dims
        f32x16 acc = {};
        const bf16* dsr = sm.ds[buf] + r * kSS + h * 8;
#pragma unroll
        for (int ks = 0; ks < kBKV / 16; ++ks) {
          const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dsr + ks * 16);
          const bf16* p = ktr + ks * 16 * kKS;
          const bf16x8 bk = concat(lds_read_tr4(p), lds_read_tr4(p + 4 * kKS));
          acc = mfma32x32x16(ad, bk, acc);
        }
        // always 16 atomics (rows past the end add 0 to row r0): a fixed count keeps
        // the staging waits precise (see load_qstage)
        float* dqp = a.dq + ((int64_t)r0 * a.hq + head) * D + wave * 32 + r;
        const int64_t rs = (int64_t)a.hq * D;
#pragma unroll
        for (int aa = 0; aa < 16; ++aa) {
          const int q = 8 * (aa >> 2) + 4 * h + (aa & 3);
          const bool ok = r0 + q < r1;
          unsafeAtomicAdd(dqp + (ok ? q : 0) * rs, ok ? acc[aa] : 0.0f);
        }
      }
      if (nxt.hh < 0) break;
      buf ^= 1;
      cur = nxt;
      nxt = nxt2;
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
        const f32x4 vk = {dk[db][4 * g], dk[db][4 * g + 1], dk[db][4 * g + 2], dk[db][4 * g + 3]};
        const f32x4 vv = {dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(dkp + rowoff + d0) = vk;
        *reinterpret_cast<f32x4*>(dvp + rowoff + d0) = vv;
      }
    }
  }
}

template <int D>
hipError_t launch_bwd_d(BwdArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.q_len * a.hq;
  if (pairs > 0) {
    const int64_t threads = pairs * (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, reinterpret_cast<const bf16*>(a.o),
                       reinterpret_cast<const bf16*>(a.dout), a.delta, a.dq, pairs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int total = 0;
  for (int s = 0; s < a.n_segs; ++s) {
    a.seg_wg_begin[s] = total;
    total += ((a.segs[s].len + kBKV - 1) / kBKV) * a.hkv;
  }
  a.seg_wg_begin[a.n_segs] = total;
  a.total_wgs = total;
  a.padded_wgs = (total + 7) & ~7;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_main_kernel<D>), dim3(a.padded_wgs), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int bwd_max_rows() { return kMaxQTiles * kBQ; }

hipError_t launch_bwd(const BwdArgs& args, int d, hipStream_t stream) {
  BwdArgs a = args;
  if (d == 64) return launch_bwd_d<64>(a, stream);
  return launch_bwd_d<128>(a, stream);
}

}  // namespace cpattn
