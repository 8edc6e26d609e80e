// Host unit test of the library's planner (csrc/plan.h), built with g++ and the address and
// undefined-behaviour sanitizers by tests/test_host_plan.py.  No GPU and no HIP.
//
//  * The attention grid the host sizes equals, for every XCD, the queue the device's batch prep
//    builds: the device rule (rank of each user = longer users + equally long users of lower
//    index, or the identity above kLptMaxUsers users; snake deal of (user, head) groups over the
//    8 XCDs) is restated here as the device kernels compute it and compared with the planner, on
//    random batches on both sides of the user limit.
//  * Workspace regions are 256-byte aligned, disjoint and inside the reported total.
//  * Batch checks reject what the header says they reject.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <utility>
#include <vector>

#include "plan.h"

using namespace mtgr;

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

struct HostBatch {
  std::vector<int64_t> off;
  mtgr_batch b{};
  int64_t fake = 0;
  explicit HostBatch(const std::vector<int64_t>& lens) {
    off.assign(1, 0);
    for (int64_t n : lens) off.push_back(off.back() + n);
    b.num_users = (int32_t)lens.size();
    b.num_tokens = off.back();
    b.num_candidates = 0;
    b.offsets_host = off.data();
    b.offsets = &fake;                       // never dereferenced on the host
    b.group_ids = reinterpret_cast<const uint8_t*>(&fake);
    b.timestamps = reinterpret_cast<const float*>(&fake);
  }
};

// the device's user order, as its prep kernel computes it
static std::vector<int32_t> device_order(const std::vector<int64_t>& off) {
  const int32_t B = (int32_t)off.size() - 1;
  std::vector<int32_t> order(B);
  for (int32_t b = 0; b < B; ++b) {
    if (B > kLptMaxUsers) { order[b] = b; continue; }
    const int64_t n = off[b + 1] - off[b];
    int rank = 0;
    for (int32_t o = 0; o < B; ++o) {
      const int64_t no = off[o + 1] - off[o];
      rank += (no > n) || (no == n && o < b);
    }
    order[rank] = b;
  }
  return order;
}

// the device's per-XCD queues over that order
static void device_queues(const std::vector<int64_t>& off, const std::vector<int32_t>& order, int H, int q_tile,
                          int64_t out[kXcdCount]) {
  const int32_t B = (int32_t)off.size() - 1;
  const int64_t G = (int64_t)B * H;
  const int64_t R = (G + kXcdCount - 1) / kXcdCount;
  for (int x = 0; x < kXcdCount; ++x) {
    int64_t acc = 0;
    for (int64_t k = 0; k < R; ++k) {
      const int64_t g = k * kXcdCount + ((k & 1) ? (kXcdCount - 1 - x) : x);
      if (g < G) {
        const int32_t b = order[g / H];
        acc += (off[b + 1] - off[b] + q_tile - 1) / q_tile;
      }
    }
    out[x] = acc;
  }
}

static void test_grid_matches_device(std::mt19937_64& rng) {
  const int users[] = {1, 3, 8, 9, 100, 1000, kLptMaxUsers, kLptMaxUsers + 1, 20000};
  for (int B : users) {
    for (int lo_hi = 0; lo_hi < 2; ++lo_hi) {
      // small users (8..40 tokens) and a long-tailed mix (some of 3000 tokens)
      std::uniform_int_distribution<int> small(8, 40), mixed(0, 3000);
      std::vector<int64_t> lens(B);
      for (int i = 0; i < B; ++i) lens[i] = lo_hi == 0 ? small(rng) : (i % 10 == 3 ? 3000 : mixed(rng));
      HostBatch hb(lens);
      const std::vector<int32_t> order = device_order(hb.off);
      for (int H : {1, 4, 6}) {
        for (int qt : {kAttnFwdQTileBf16, kAttnQTileBf16, kAttnQTileF32}) {
          int64_t dev[kXcdCount], host[kXcdCount];
          device_queues(hb.off, order, H, qt, dev);
          plan::xcd_queue_tiles(&hb.b, H, qt, host);
          int64_t mx = 0, tot = 0;
          for (int x = 0; x < kXcdCount; ++x) {
            CHECK(dev[x] == host[x]);
            mx = std::max(mx, dev[x]);
            tot += dev[x];
          }
          CHECK(plan::xcd_grid_slots(&hb.b, H, qt) == mx);
          CHECK(tot == plan::total_tiles(&hb.b, qt) * H);
        }
      }
    }
  }
}

static void check_regions(std::vector<std::pair<size_t, size_t>> r, size_t total) {
  std::sort(r.begin(), r.end());
  for (size_t i = 0; i < r.size(); ++i) {
    CHECK(r[i].first % plan::kAlign == 0);
    CHECK(r[i].first + r[i].second <= total);
    if (i + 1 < r.size()) CHECK(r[i].first + r[i].second <= r[i + 1].first);
  }
}

static void test_plans() {
  for (int64_t T : {0LL, 1LL, 999LL, 20000LL, 630293LL}) {
    for (int dtype : {MTGR_F32, MTGR_BF16}) {
      plan::Sizes z;
      z.B = 37; z.T = T; z.C = T / 7; z.d = 768; z.h = 3072; z.hh = 384; z.dtype = dtype; z.H = 6;
      z.need_acts = z.need_xres = z.need_head = true;
      const plan::Plan p = plan::make_plan(z);
      const size_t es = plan::esize(dtype);
      const int64_t rounds = (z.B * z.H + kXcdCount - 1) / kXcdCount;
      check_regions({{p.flags, 16}, {p.seg, z.B * kUserSegBytes}, {p.order, z.B * 4}, {p.tile_off, (z.B + 1) * 4},
                     {p.cand_off, (z.B + 1) * 8}, {p.cand_idx, z.C * 8}, {p.xcd_off, kXcdCount * (rounds + 1) * 4},
                     {p.xcd_fwd, kXcdCount * (rounds + 1) * 4},
                     {p.xt, T * z.d * es}, {p.big, T * 4 * z.d * es}, {p.y, T * z.d * es}, {p.xres, T * z.d * 4},
                     {p.hin, z.C * z.d * es}, {p.hhid, z.C * z.hh * es}},
                    p.total);
      const plan::BwdPlan q = plan::make_bwd_plan(z);
      CHECK(q.ok);
      for (int gi = 0; gi < 3; ++gi) {
        CHECK(q.ks[gi] >= 1);
        CHECK(q.Tp[gi] >= T && q.Tp[gi] % (64 * q.ks[gi]) == 0 && q.Tp[gi] / 64 / q.ks[gi] >= 2);
      }
      check_regions({{q.xt, T * z.d * es}, {q.qkvu, T * 4 * z.d * es}, {q.y, T * z.d * es}, {q.vt, T * z.d * es},
                     {q.z, T * z.d * es}, {q.a, T * z.h * es}, {q.dhid, T * z.h * es}, {q.dz, T * z.d * es},
                     {q.dqkvu, T * 4 * z.d * es}, {q.wt, (size_t)z.h * z.d * es}, {0, q.prep.total}},
                    q.total);
    }
  }
}

static void test_batch_checks() {
  HostBatch ok({3, 0, 5});
  CHECK(plan::check_batch(&ok.b) == MTGR_OK);
  CHECK(plan::check_batch(nullptr) == MTGR_ERR_NULL_ARG);
  HostBatch bad({3, 5});
  bad.off[1] = 9;                            // offsets not monotone
  CHECK(plan::check_batch(&bad.b) == MTGR_ERR_BAD_BATCH);
  HostBatch tcount({4, 4});
  tcount.b.num_tokens = 7;                   // T != offsets[B]
  CHECK(plan::check_batch(&tcount.b) == MTGR_ERR_BAD_BATCH);
  HostBatch cand({4});
  cand.b.num_candidates = 5;                 // more candidates than tokens
  CHECK(plan::check_batch(&cand.b) == MTGR_ERR_BAD_BATCH);
  HostBatch empty({});
  CHECK(plan::check_batch(&empty.b) == MTGR_OK);
  CHECK(plan::check_attn_shape(768, 6, MTGR_BF16) == MTGR_OK);
  CHECK(plan::check_attn_shape(768, 5, MTGR_BF16) == MTGR_ERR_BAD_SHAPE);
  CHECK(plan::check_attn_shape(2048, 16, MTGR_BF16) == MTGR_ERR_BAD_SHAPE);
  HostBatch wide({349525});
  CHECK(plan::check_user_rows(&wide.b, 768, MTGR_BF16) == MTGR_OK);
  HostBatch wider({349526});
  CHECK(plan::check_user_rows(&wider.b, 768, MTGR_BF16) == MTGR_ERR_BAD_SHAPE);
}

int main() {
  std::mt19937_64 rng(20261203);
  test_grid_matches_device(rng);
  test_plans();
  test_batch_checks();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("planner checks passed\n");
  return 0;
}
