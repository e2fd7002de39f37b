// Host-side driver for the sanitizer build of the C ABI: every validation path, the
// workspace queries (launch plans, segment groups) and calls that reach a launch
// (which fail with CPATTN_ERR_HIP when no GPU is present).  Device pointers are fake
// and never dereferenced by host code.  Exits non-zero on the first unexpected code.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/cpattn.h"

static int fails = 0;
#define EXPECT(call, want)                                                               \
  do {                                                                                   \
    const int got_ = (call);                                                             \
    if (got_ != (want)) {                                                                \
      std::printf("line %d: %s returned %d, want %d\n", __LINE__, #call, got_, (want));  \
      ++fails;                                                                           \
    }                                                                                    \
  } while (0)
#define EXPECT_ANY(call, a, b)                                                           \
  do {                                                                                   \
    const int got_ = (call);                                                             \
    if (got_ != (a) && got_ != (b)) {                                                    \
      std::printf("line %d: %s returned %d\n", __LINE__, #call, got_);                   \
      ++fails;                                                                           \
    }                                                                                    \
  } while (0)

int main() {
  void* F = reinterpret_cast<void*>(0x100000);
  const int32_t* Fi = static_cast<const int32_t*>(F);
  int32_t* Fo = static_cast<int32_t*>(F);
  const void* src[8] = {F, F, F, F, F, F, F, F};
  void* dst[8] = {F, F, F, F, F, F, F, F};
  int64_t rb[8] = {256, 256, 512, 16, 32, 48, 64, 1 << 20};

  // zigzag edge check (host arithmetic only)
  int32_t vis = -1;
  EXPECT(cpattn_zigzag_edge_visible(8192, 4, 0, 0, 1, -1, &vis), CPATTN_OK);
  EXPECT(vis, 0);
  EXPECT(cpattn_zigzag_edge_visible(8192, 4, 0, 1, 3, 1, &vis), CPATTN_OK);
  EXPECT(vis, 1);
  EXPECT(cpattn_zigzag_edge_visible(INT64_MAX - 7, 4, 3, -1, 3, -1, &vis), CPATTN_OK);
  EXPECT(cpattn_zigzag_edge_visible(8192, 4, 4, 0, 0, 0, &vis), CPATTN_ERR_ARG);
  EXPECT(cpattn_zigzag_edge_visible(8190, 4, 0, 0, 0, 0, &vis), CPATTN_ERR_ALIGN);
  EXPECT(cpattn_zigzag_edge_visible(8192, 4, 0, 0, 0, 0, nullptr), CPATTN_ERR_ARG);

  // partition and its rotary form
  EXPECT(cpattn_partition(9, 64, 2, 0, nullptr, nullptr, 0, Fo, nullptr, 0, src, dst, rb, nullptr), CPATTN_ERR_ARG);
  EXPECT(cpattn_partition(CPATTN_PART_ZIGZAG, 100, 4, 0, nullptr, nullptr, 0, Fo, nullptr, 0, src, dst, rb, nullptr),
         CPATTN_ERR_ALIGN);
  EXPECT(cpattn_partition(CPATTN_PART_STRIPED, 10, 4, 0, nullptr, nullptr, 0, Fo, nullptr, 0, src, dst, rb, nullptr),
         CPATTN_ERR_ALIGN);
  const int32_t bad_cu[4] = {0, 40, 32, 64};
  EXPECT(cpattn_partition(CPATTN_PART_THD, 64, 2, 0, bad_cu, Fi, 3, Fo, nullptr, 0, src, dst, rb, nullptr),
         CPATTN_ERR_ALIGN);
  EXPECT(cpattn_partition(CPATTN_PART_ZIGZAG, 64, 2, 0, nullptr, nullptr, 0, Fo, nullptr, 9, src, dst, rb, nullptr),
         CPATTN_ERR_ARG);
  EXPECT(cpattn_partition(CPATTN_PART_ZIGZAG, 0, 2, 0, nullptr, nullptr, 0, nullptr, nullptr, 0, src, dst, rb,
                          nullptr),
         CPATTN_OK);
  EXPECT_ANY(cpattn_partition(CPATTN_PART_ZIGZAG, 64, 2, 0, nullptr, nullptr, 0, Fo, nullptr, 3, src, dst, rb,
                              nullptr),
             CPATTN_ERR_HIP, CPATTN_OK);
  cpattn_rope_desc rope = {3u, CPATTN_BF16, 128, 0, 10000.0f};
  EXPECT(cpattn_partition_rope(CPATTN_PART_ZIGZAG, 64, 2, 0, nullptr, nullptr, 0, Fo, nullptr, 2, src, dst, rb,
                               nullptr, nullptr),
         CPATTN_ERR_ARG);
  rope.d = 72;
  EXPECT(cpattn_partition_rope(CPATTN_PART_ZIGZAG, 64, 2, 0, nullptr, nullptr, 0, Fo, nullptr, 2, src, dst, rb, &rope,
                               nullptr),
         CPATTN_ERR_UNSUPPORTED);
  rope.d = 16;  // 256-byte rows of 16-wide bf16 heads: 8 heads
  EXPECT_ANY(cpattn_partition_rope(CPATTN_PART_ZIGZAG, 64, 2, 0, nullptr, nullptr, 0, Fo, nullptr, 2, src, dst, rb,
                                   &rope, nullptr),
             CPATTN_ERR_HIP, CPATTN_OK);
  rope.rotate_mask = 1u << 5;  // a 48-byte row: one and a half 16-wide bf16 heads
  EXPECT(cpattn_partition_rope(CPATTN_PART_ZIGZAG, 64, 2, 0, nullptr, nullptr, 0, Fo, nullptr, 8, src, dst, rb, &rope,
                               nullptr),
         CPATTN_ERR_ALIGN);
  rope.rotate_mask = 1u << 7 | 1u << 4;  // a 1 MiB row (2 rows per block) and a 32-byte row (514 rows)
  EXPECT_ANY(cpattn_partition_rope(CPATTN_PART_ZIGZAG, 64, 2, 0, nullptr, nullptr, 0, Fo, nullptr, 8, src, dst, rb,
                                   &rope, nullptr),
             CPATTN_ERR_HIP, CPATTN_OK);

  // attention problems
  cpattn_attn_desc d = {CPATTN_BF16, 8, 8, 128, 0.0f, CPATTN_MASK_CAUSAL};
  cpattn_q_block q = {F, Fi, nullptr, 2048};
  std::vector<cpattn_kv_seg> segs(2100, cpattn_kv_seg{F, F, Fi, nullptr, 512});
  std::vector<float*> outs(2100, static_cast<float*>(F));
  for (int n : {1, 4, 16, 32, 33, 64, 100, 2048}) {
    (void)cpattn_stream_fwd_workspace_bytes(&d, &q, n, segs.data());
    (void)cpattn_bwd_workspace_bytes(&d, &q, n, segs.data());
    (void)cpattn_bwd_dq_workspace_bytes(&d, &q, n, segs.data());
  }
  EXPECT(cpattn_stream_fwd(&d, &q, 2049, segs.data(), F, static_cast<float*>(F), nullptr, 0, nullptr), CPATTN_ERR_ARG);
  EXPECT(cpattn_stream_fwd(&d, &q, 100, segs.data(), F, static_cast<float*>(F), nullptr, 0, nullptr),
         CPATTN_ERR_WORKSPACE);
  EXPECT_ANY(cpattn_stream_fwd(&d, &q, 4, segs.data(), F, static_cast<float*>(F), nullptr, 0, nullptr), CPATTN_ERR_HIP,
             CPATTN_OK);
  std::vector<cpattn_q_block> qbs(25, q);
  qbs[23].q = nullptr;
  EXPECT(cpattn_tile_fwd(&d, 25, qbs.data(), segs.data(), outs.data(), outs.data(), nullptr, 0, nullptr),
         CPATTN_ERR_ARG);
  qbs[23].q = F;
  (void)cpattn_tile_fwd_workspace_bytes(&d, 25, qbs.data(), segs.data());
  EXPECT_ANY(cpattn_tile_fwd(&d, 25, qbs.data(), segs.data(), outs.data(), outs.data(), nullptr, 0, nullptr),
             CPATTN_ERR_HIP, CPATTN_OK);
  const float* cparts[70];
  for (auto& p : cparts) p = static_cast<const float*>(F);
  EXPECT(cpattn_merge(65, cparts, cparts, 16, 8, 128, CPATTN_BF16, F, static_cast<float*>(F), nullptr), CPATTN_ERR_ARG);
  EXPECT(cpattn_merge(4, cparts, cparts, 16, 8, 130, CPATTN_BF16, F, static_cast<float*>(F), nullptr),
         CPATTN_ERR_UNSUPPORTED);
  {
    // grouped merges: 12 groups of 6 parts (more than one launch's worth of groups and parts)
    std::vector<const float*> gp(72, static_cast<const float*>(F));
    std::vector<int32_t> gparts(12, 6);
    std::vector<int64_t> grows(12, 16);
    std::vector<void*> gout(12, F);
    std::vector<float*> glse(12, static_cast<float*>(F));
    EXPECT_ANY(cpattn_merge_groups(12, gparts.data(), gp.data(), gp.data(), grows.data(), 8, 128, CPATTN_BF16,
                                   gout.data(), glse.data(), nullptr),
               CPATTN_ERR_HIP, CPATTN_OK);
    gparts[5] = 0;
    EXPECT(cpattn_merge_groups(12, gparts.data(), gp.data(), gp.data(), grows.data(), 8, 128, CPATTN_BF16,
                               gout.data(), glse.data(), nullptr),
           CPATTN_ERR_ARG);
  }

  // backward
  float* Ff = static_cast<float*>(F);
  EXPECT(cpattn_bwd(&d, &q, 4, segs.data(), F, Ff, F, Ff, outs.data(), outs.data(), F, 100, nullptr),
         CPATTN_ERR_WORKSPACE);
  EXPECT_ANY(cpattn_bwd(&d, &q, 40, segs.data(), F, Ff, F, Ff, outs.data(), outs.data(), F, 1 << 20, nullptr),
             CPATTN_ERR_HIP, CPATTN_OK);
  EXPECT_ANY(cpattn_bwd_dkdv(&d, &q, 70, segs.data(), Ff, Ff, F, outs.data(), outs.data(), nullptr), CPATTN_ERR_HIP,
             CPATTN_OK);
  EXPECT(cpattn_bwd_dq_delta(&d, &q, 4, segs.data(), nullptr, Ff, F, Ff, Ff, nullptr, 0, nullptr), CPATTN_ERR_ARG);
  EXPECT_ANY(cpattn_bwd_dq_delta(&d, &q, 70, segs.data(), F, Ff, F, Ff, Ff, nullptr, 0, nullptr), CPATTN_ERR_HIP,
             CPATTN_OK);
  cpattn_attn_desc wide = {CPATTN_BF16, 64, 8, 128, 0.0f, CPATTN_MASK_CAUSAL};
  cpattn_q_block big = {F, Fi, nullptr, 300000};
  EXPECT(cpattn_bwd_noalloc(&wide, &big, 1, segs.data(), F, Ff, F, Ff, outs.data(), outs.data(), nullptr),
         CPATTN_ERR_WORKSPACE);
  for (int st = 0; st < 7; ++st) (void)cpattn_strerror(st);
  std::printf(fails ? "host driver: %d unexpected codes\n" : "host driver: ok\n", fails);
  return fails ? 1 : 0;
}
