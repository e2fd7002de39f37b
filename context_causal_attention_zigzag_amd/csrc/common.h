// Device-side building blocks shared by the cpattn kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, one wave64):
//   A (32 x 16): lane l holds row (l % 32), contraction elements 8*(l / 32) .. +7
//   B (16 x 32): lane l holds column (l % 32), contraction elements 8*(l / 32) .. +7
//   C (32 x 32): lane l holds column (l % 32); accumulator a holds row
//                8*(a / 4) + 4*(l / 32) + (a % 4),  a = 0..15
// A C-layout matrix therefore already sits in B-operand form for a product that
// contracts over its rows, provided the other operand enumerates the contraction
// index in the same order: within each 16-row slice, lane half h and element e
// name row  perm16(h, e) = 8*(e / 4) + 4*h + (e % 4).  Operands staged in LDS for
// such products are stored with that permutation (swap of index bits 2 and 3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWave = 64;

// Mask kinds (values match the public CPATTN_MASK_* constants).
constexpr int kMaskNone = 0;
constexpr int kMaskCausal = 1;
constexpr int kMaskCausalDoc = 2;

// Tile classes for one (query tile, key tile) pair.
constexpr int kTileEmpty = 0;
constexpr int kTileFull = 1;
constexpr int kTilePartial = 2;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Transposing LDS read (ds_read_b64_tr_b16).  Lanes act in groups of 16: lane r of a
// group supplies the address of four consecutive 16-bit elements, and lane i of the
// group receives element (i % 4) of the quads supplied by lanes i/4, i/4+4, i/4+8 and
// i/4+12.  On a row-major [k][n] tile where lane r addresses row k0 + r/4, columns
// n0 + 4*(r%4) .. +3, lane i therefore receives column n0 + i, rows k0 .. k0+3 — four
// consecutive contraction elements of one operand column/row, as the matrix cores
// expect.  Offsets for that addressing: tr_lane_offset().
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Element offset, within a row-major tile of row stride `stride`, that lane `lane`
// addresses for lds_read_tr4 when the wave reads an operand whose lanes l % 32 own
// columns n0 + l % 32 and whose lane half h = lane / 32 owns the four contraction rows
// k0 + half_step*h .. +3: row half_step*h + (i / 4), column 16*(g % 2) + 4*(i % 4), with
// g = lane / 16, i = lane % 16.  half_step = 4 gives the contraction order of a C-layout
// B operand (two reads at k0 and k0 + 8 cover one 16-row slice), half_step = 8 the
// natural order (two reads at k0 and k0 + 4).
template <int kHalfStep>
__device__ __forceinline__ int tr_lane_offset(int lane, int stride) {
  const int g = lane >> 4, i = lane & 15;
  return (kHalfStep * (g >> 1) + (i >> 2)) * stride + 16 * (g & 1) + 4 * (i & 3);
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Work-group barrier that only orders LDS traffic: waits for this wave's outstanding
// LDS operations, then s_barrier.  Global stores and atomics stay in flight (a plain
// __syncthreads() would wait for every outstanding global access of the wave).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Barrier after direct global->LDS loads: waits for this wave's outstanding vector
// memory loads (which include the LDS fills) and LDS operations, then s_barrier.
__device__ __forceinline__ void fill_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct global->LDS copy of 16 bytes per lane: lane l's 16 bytes land at
// lds_base + 16*l (lds_base wave-uniform), as measured on gfx950.
__device__ __forceinline__ void global_to_lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}
// Same with 4 bytes per lane: lane l's dword lands at lds_base + 4*l.
__device__ __forceinline__ void global_to_lds4(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds_base), 4, 0, 0);
}

// Direct global->LDS loads issued as inline assembly (lane l's 16 bytes land at LDS
// byte offset lds_off + 16 l; the 4-byte form at lds_off + 4 l).  The compiler does
// not track them, so its wait insertion never makes an LDS read of another buffer
// wait for them; a kernel using them waits for its own fills (s_waitcnt vmcnt) before
// the barrier that publishes the data.  m0 is reserved for the compiler, which warns
// about the clobber; kernels using these keep no value of their own in m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void fill16_untracked(const void* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_off), "v"(g)
               : "memory", "m0");
}
// The same from base + off: base wave-uniform (scalar registers), off a per-lane byte
// offset.  Callers compute the offsets of a burst of fills into distinct registers
// before issuing any: an instruction that overwrites the address register of a fill
// still waiting for the memory pipeline to read it stalls until that read, which
// serialises a burst that reuses one register.
__device__ __forceinline__ void fill16_off(const void* base, uint32_t off, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_off), "v"(off), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void fill4_untracked(const void* g, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds_off), "v"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte offset of a __shared__ address (wave-uniform).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// A kernel-argument pointer held in scalar registers (a per-lane choice between two
// arguments is then made on their values, not on their addresses, which would fetch
// them with a vector load).
template <class T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>((uint64_t)hi << 32 | lo);
}

// Exchange between the two lane halves (v_permlane32_swap, a VALU instruction on
// gfx950).  lo_hi(x) yields, in every lane l, the values of lane l % 32 (first) and of
// lane l % 32 + 32 (second): combining the two gives the same result, in the same
// operation order, in both halves.
struct LoHi {
  float lo, hi;
};
__device__ __forceinline__ LoHi lo_hi(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0]: lanes 0..31 keep x, lanes 32..63 receive lanes 0..31; r[1]: lanes 0..31
  // receive lanes 32..63, lanes 32..63 keep x
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float half_max(float x) {
  const LoHi p = lo_hi(x);
  return fmaxf(p.lo, p.hi);
}
__device__ __forceinline__ float half_sum(float x) {
  const LoHi p = lo_hi(x);
  return p.lo + p.hi;
}
// Value held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  const LoHi p = lo_hi(x);
  return (threadIdx.x & 32) ? p.lo : p.hi;
}

// Swap of bits 2 and 3 inside each group of 16 (the contraction order of a C-layout
// B operand, see the header comment).
__device__ __forceinline__ int perm16(int k) {
  return (k & ~15) | ((k >> 2) & 1) << 3 | ((k >> 3) & 1) << 2 | (k & 3);
}

// Classification of a query tile [qmin, qmax] (document range [qdmin, qdmax])
// against a key tile [kmin, kmax] ([kdmin, kdmax]); positions and documents are
// non-decreasing inside tiles, so the extremes are the first and last entries.
__device__ __forceinline__ int classify(int mask, int qmin, int qmax, int qdmin, int qdmax,
                                        int kmin, int kmax, int kdmin, int kdmax) {
  if (mask == kMaskNone) return kTileFull;
  if (kmin > qmax) return kTileEmpty;
  if (mask == kMaskCausalDoc) {
    if (kdmax < qdmin || kdmin > qdmax) return kTileEmpty;
    if (kmax <= qmin && qdmin == qdmax && kdmin == kdmax && qdmin == kdmin) return kTileFull;
    return kTilePartial;
  }
  return kmax <= qmin ? kTileFull : kTilePartial;
}

// Work-group order remap: the dispatcher hands consecutive work-groups to the 8
// XCDs in turn, so logical work item (x * per + i) runs on XCD x; neighbours in
// logical order (same heads, adjacent query tiles) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int padded_n) {
  const int per = padded_n >> 3;
  return (b & 7) * per + (b >> 3);
}

// ---------------------------------------------------------------------------
// Kernel-argument tables (passed by value): at most kMaxSegs segments per launch; the
// host runs longer segment lists as several launches.
constexpr int kMaxSegs = 32;
constexpr int kMaxJobs = 20;

struct SegDesc {
  const void* k;
  const void* v;
  const int32_t* pos;
  const int32_t* doc;
  int32_t len;
};

struct JobDesc {
  const void* q;
  const int32_t* pos;
  const int32_t* doc;
  void* o;           // final output (input dtype) or fp32 partial output
  float* lse;        // [len, hq]
  float* ws_o;       // split partials [n_split][len][hq][d] (n_split > 1)
  float* ws_lse;     // split partial LSE [n_split][len][hq]
  int32_t len;
  int32_t seg_begin;
  int32_t seg_end;
  int32_t wg_begin;  // first logical work-group of this job
  int32_t n_split;   // KV splits per query tile (1: no split)
  int32_t tiles_per_split;
  int32_t n_tiles;   // KV tiles over all of the job's segments
  int32_t pad_;
};

struct FwdArgs {
  SegDesc segs[kMaxSegs];
  JobDesc jobs[kMaxJobs];
  int32_t n_jobs;
  int32_t hq;
  int32_t hkv;
  int32_t group;         // hq / hkv
  int32_t heads_per_wg;  // query heads sharing one work-group (divides group)
  int32_t mask;
  float scale_log2;      // softmax scale times log2(e)
  int32_t total_wgs;     // logical work-groups
  int32_t padded_wgs;    // grid size (multiple of 8)
  int32_t wg_waves;      // waves per work-group of the launch (32 query rows each)
  int32_t compact;       // KV splits numbered densely (no work-group for an empty split)
  int32_t plan_tiles;    // a ranked launch planned once: its query tiles over all jobs (else 0)
  int32_t* plan;         // that plan in the workspace (rank order, then the KV tile table)
};

struct BwdArgs {
  SegDesc segs[kMaxSegs];
  const void* q;
  const int32_t* qpos;
  const int32_t* qdoc;
  const float* lse;
  const void* dout;
  float* dk[kMaxSegs];
  float* dv[kMaxSegs];
  const float* delta;    // [q_len, hq]: rowsum(dO * O)
  int32_t q_len;
  int32_t n_segs;
  int32_t seg_wg_begin[kMaxSegs + 1];
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t mask;
  float scale;
  float scale_log2;
  int32_t total_wgs;
  int32_t padded_wgs;
};

// Rotary embedding applied by the partition gather (validated by the caller).
struct RopeSpec {
  uint32_t mask;     // bit g: gathered tensor g is rotated
  int f32;           // rotated tensors hold fp32 (else bf16)
  int d;             // head dim: multiple of 16, at most 256
  int interleaved;   // pairs (2i, 2i+1) instead of (i, i + d/2)
  double log2_base;  // log2 of the frequency base
};

// Host-side launchers (defined in the .hip files).
// mode: 0 zigzag, 1 packed documents (cu_dev), 2 striped.
hipError_t launch_partition(int mode, int64_t total, int cp, int rank, const int32_t* cu_dev,
                            int n_docs, int32_t* idx, int32_t* doc, int n_gather,
                            const void* const* src, void* const* dst, const int64_t* row_bytes,
                            const RopeSpec* rope, hipStream_t stream);
// Entries of the rotation table a block of the rotated gather needs for rows of
// row_bytes bytes, or -1 when they exceed its LDS table.
int rope_table_entries(int d, int interleaved, int64_t row_bytes);
hipError_t launch_fwd(const FwdArgs& a, int d, int dtype, bool partial_out, hipStream_t stream);
// Split plan for forward jobs: fills n_split / tiles_per_split / n_tiles of each job and
// the segments' tile offsets; returns the workspace bytes the plan needs.
// waves: work-group size of the kernel the plan is for (4 or 8), or 0 to let the
// forward choose (8 when the query tiles alone fill the CUs once, else 4).
size_t plan_fwd(FwdArgs& a, int d, int dtype, int num_cu, bool allow_split, int waves);
// Points the split jobs' partial buffers into a workspace of plan_fwd's size.
void assign_fwd_workspace(FwdArgs& a, int d, void* ws);
hipError_t launch_merge(int n_parts, const float* const* o_parts, const float* const* lse_parts,
                        int64_t rows, int hq, int d, int out_dtype, void* o_out, float* lse_out,
                        hipStream_t stream);
// Several independent merges (group g: n_parts[g] consecutive parts over rows[g] rows
// into o_out[g], lse_out[g]) in as few launches as the argument block allows.
hipError_t launch_merge_groups(int n_groups, const int32_t* n_parts, const float* const* o_parts,
                               const float* const* lse_parts, const int64_t* rows, int hq, int d, int out_dtype,
                               void* const* o_out, float* const* lse_out, hipStream_t stream);
// Backward passes: delta = rowsum(dO * O) over `pairs` (row, head) pairs; dQ
// (query-major, `dq` holds its job, split plan and partial buffers); dK/dV (key-major).
hipError_t launch_bwd_delta(const void* o, const void* dout, float* delta, int64_t pairs, int d,
                            hipStream_t stream);
// o not null: the dQ pass forms delta from O and dO itself and stores it (same bits as
// launch_bwd_delta) instead of reading it.
hipError_t launch_bwd_dq(const FwdArgs& dq, const void* dout, float* delta, float scale, int d,
                         bool accumulate, hipStream_t stream, const void* o = nullptr);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int d, hipStream_t stream);
// One launch merging the KV splits of every split job of a forward launch.
hipError_t launch_merge_split_jobs(const FwdArgs& f, int d, int out_dtype, hipStream_t stream,
                                   bool sum = false);

}  // namespace cpattn
