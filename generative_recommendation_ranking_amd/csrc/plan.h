// Host-side planning of libmtgr.so: batch and shape checks, workspace layout, and the placement
// of attention work on the XCDs.  Plain C++ with no HIP dependency, so the same code is compiled
// into the library and, on its own, into a host unit test (with the address and undefined-behaviour
// sanitizers).
//
// Placement of attention work.  A work item is (user, head, q-tile of 256, 128 or 64 rows).  Users are
// taken longest first (LPT) so the heaviest items start first; (user, head) groups g = p*H + h
// (p the user's position in that order) are dealt to the 8 XCDs in snake order, and every XCD runs
// its groups' q-tiles back to back so a group's tiles share one L2.  The device builds the same
// order and queues (prep.hip); the functions here are its host replica, which sizes the launch
// grid.  Both use one rule for the order: longest first with ties by index when B <= kLptMaxUsers,
// index order above it (the device's ranking is quadratic in B).
#pragma once

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/mtgr.h"

namespace mtgr {

constexpr int kXcdCount = 8;           // MI355X: 8 XCDs, workgroups dispatched round-robin by id
constexpr int kLptMaxUsers = 16384;    // above this many users the work order is the index order
constexpr int kAttnQTileBf16 = 128;    // query (key) rows per work item of the bf16 attention backward
constexpr int kAttnFwdQTileBf16 = 128; // query rows per work item of the bf16 attention forward
constexpr int kAttnQTileF32 = 64;      // (fp32 kernels)
constexpr size_t kUserSegBytes = 16;   // sizeof(UserSeg): four int32 segment lengths

// ---- sizes of helper kernels' partial-sum buffers (their launchers use the same functions) ----
// column-sum kernel: row blocks of the partial sums, [colsum_blocks(T, M)][M] floats
constexpr int kColsumRowBlocks = 2048;
inline int colsum_blocks(int64_t T, int M) {
  const int cg = (M + 511) / 512;
  return (int)std::max<int64_t>(1, std::min<int64_t>(kColsumRowBlocks / cg, (T + 63) / 64));
}
// Wavefronts of the GroupLN backward, each with one slot [2][4][d] of partial parameter gradients:
// one round of resident wavefronts on 256 CUs -- the fp32-input variant (prefetching, ~190 VGPRs)
// holds 2 per SIMD, the bf16 one (~120 VGPRs) 4
inline int groupln_bwd_waves(int64_t T, int x_kind) {
  const int64_t cap = x_kind == 0 ? 512 : 1024;
  return 4 * (int)std::max<int64_t>(1, std::min<int64_t>(cap, (T + 255) / 256));
}

namespace plan {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int esize(int dtype) { return dtype == MTGR_BF16 ? 2 : 4; }

// ---- batch and shape checks --------------------------------------------------------------------
inline mtgr_status check_batch(const mtgr_batch* b) {
  if (!b) return MTGR_ERR_NULL_ARG;
  if (b->num_users < 0 || b->num_tokens < 0 || b->num_candidates < 0) return MTGR_ERR_BAD_BATCH;
  if (b->num_users == 0) return (b->num_tokens == 0 && b->num_candidates == 0) ? MTGR_OK : MTGR_ERR_BAD_BATCH;
  if (!b->offsets_host || !b->offsets) return MTGR_ERR_NULL_ARG;
  if (b->num_tokens > 0 && (!b->group_ids || !b->timestamps)) return MTGR_ERR_NULL_ARG;
  const int64_t* o = b->offsets_host;
  if (o[0] != 0) return MTGR_ERR_BAD_BATCH;
  for (int32_t i = 0; i < b->num_users; ++i) {
    if (o[i + 1] < o[i]) return MTGR_ERR_BAD_BATCH;
    if (o[i + 1] - o[i] > (int64_t)(1 << 30)) return MTGR_ERR_BAD_BATCH;
  }
  if (o[b->num_users] != b->num_tokens) return MTGR_ERR_BAD_BATCH;
  if (b->num_candidates > b->num_tokens) return MTGR_ERR_BAD_BATCH;
  return MTGR_OK;
}

inline bool dh_ok(int dtype, int dh) {
  if (dtype == MTGR_BF16) return dh == 64 || dh == 128;
  return dh == 32 || dh == 64 || dh == 128;
}

inline mtgr_status check_attn_shape(int32_t d, int32_t H, int32_t dtype) {
  if (dtype != MTGR_F32 && dtype != MTGR_BF16) return MTGR_ERR_UNSUPPORTED;
  if (d <= 0 || H <= 0 || d % H != 0 || d > 1024) return MTGR_ERR_BAD_SHAPE;
  if (!dh_ok(dtype, d / H)) return MTGR_ERR_BAD_SHAPE;
  return MTGR_OK;
}

// The bf16 attention kernels reach one user's rows of a head through 32-bit buffer offsets; the
// widest rows they address are the QKVU rows (4d bf16 values, 8d bytes), so one user's rows must
// span less than 2^31 bytes: at d = 768, users of up to 349,525 tokens.
inline mtgr_status check_user_rows(const mtgr_batch* b, int32_t d, int32_t dtype) {
  if (dtype != MTGR_BF16) return MTGR_OK;
  int64_t longest = 0;
  for (int32_t i = 0; i < b->num_users; ++i)
    longest = std::max(longest, b->offsets_host[i + 1] - b->offsets_host[i]);
  return longest * 8 * (int64_t)d < ((int64_t)1 << 31) ? MTGR_OK : MTGR_ERR_BAD_SHAPE;
}

inline bool mask_mode_ok(int32_t m) { return m >= MTGR_MASK_DYNAMIC && m <= MTGR_MASK_FULL; }
inline bool norm_mode_ok(int32_t m) { return m == MTGR_NORM_GROUP || m == MTGR_NORM_SHARED; }

inline mtgr_status check_block(const mtgr_block_params* p) {
  if (!p) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_attn_shape(p->d_model, p->num_heads, p->dtype);
  if (st != MTGR_OK) return st;
  if (!mask_mode_ok(p->mask_mode) || !norm_mode_ok(p->norm_mode)) return MTGR_ERR_UNSUPPORTED;
  const int mult = p->dtype == MTGR_BF16 ? 64 : 8;
  if (p->d_model % mult != 0 || p->mlp_hidden <= 0 || p->mlp_hidden % mult != 0 ||
      p->mlp_hidden > 8192)
    return MTGR_ERR_BAD_SHAPE;
  if (p->dtype == MTGR_BF16 && (p->d_model < 128 || p->mlp_hidden < 128))
    return MTGR_ERR_BAD_SHAPE;   // the bf16 GEMM pipeline needs at least two 64-wide K slabs
  if (!(p->ln_eps >= 0.f) || !std::isfinite(p->ln_eps)) return MTGR_ERR_BAD_SHAPE;
  if (!p->gln1_gamma || !p->gln1_beta || !p->w_qkvu || !p->gln2_gamma || !p->gln2_beta ||
      !p->w_mlp1 || !p->w_mlp2)
    return MTGR_ERR_NULL_ARG;
  return MTGR_OK;
}

inline mtgr_status check_encoder(const mtgr_encoder_params* p) {
  if (!p || !p->layers) return MTGR_ERR_NULL_ARG;
  if (p->num_layers < 1) return MTGR_ERR_BAD_SHAPE;
  for (int32_t l = 0; l < p->num_layers; ++l) {
    mtgr_status st = check_block(&p->layers[l]);
    if (st != MTGR_OK) return st;
    if (p->layers[l].d_model != p->layers[0].d_model ||
        p->layers[l].num_heads != p->layers[0].num_heads ||
        p->layers[l].dtype != p->layers[0].dtype)
      return MTGR_ERR_BAD_SHAPE;
  }
  const int mult = p->layers[0].dtype == MTGR_BF16 ? 32 : 8;
  if (p->head_hidden <= 0 || p->head_hidden % mult != 0 || p->head_hidden > 8192)
    return MTGR_ERR_BAD_SHAPE;
  if (!p->w_head1 || !p->w_head2) return MTGR_ERR_NULL_ARG;
  return MTGR_OK;
}

// ---- attention work placement ------------------------------------------------------------------
inline int64_t user_len(const mtgr_batch* b, int32_t u) { return b->offsets_host[u + 1] - b->offsets_host[u]; }

// The order in which users' work is dealt: longest first, ties by index (B <= kLptMaxUsers), else
// index order.  The same rule as the device's batch prep.  `order` has room for B entries; the sort
// is in place (a total order, so std::sort needs no buffer of its own).
inline void user_order(const mtgr_batch* b, int32_t* order) {
  const int32_t B = b->num_users;
  for (int32_t i = 0; i < B; ++i) order[i] = i;
  if (B <= kLptMaxUsers)
    std::sort(order, order + B, [&](int32_t x, int32_t y) {
      const int64_t lx = user_len(b, x), ly = user_len(b, y);
      return lx > ly || (lx == ly && x < y);
    });
}

// XCD that group g = p*H + h goes to: round k = g / 8 takes groups 8k .. 8k+7, XCD x the group
// 8k + x in even rounds and 8k + 7 - x in odd ones.
inline int xcd_of_group(int64_t g) {
  const int64_t k = g / kXcdCount, r = g % kXcdCount;
  return (int)((k & 1) ? (kXcdCount - 1 - r) : r);
}

// q-tiles queued on each XCD.  `order_buf` (room for B entries, may be NULL above kLptMaxUsers
// users) holds the work order.
inline void xcd_queue_tiles(const mtgr_batch* b, int H, int q_tile, int64_t tiles[kXcdCount], int32_t* order_buf) {
  const int32_t B = b->num_users;
  if (B <= kLptMaxUsers) user_order(b, order_buf);
  for (int x = 0; x < kXcdCount; ++x) tiles[x] = 0;
  const int64_t G = (int64_t)B * H;
  for (int64_t g = 0; g < G; ++g) {
    const int32_t p = (int32_t)(g / H);
    const int32_t u = B <= kLptMaxUsers ? order_buf[p] : p;
    tiles[xcd_of_group(g)] += (user_len(b, u) + q_tile - 1) / q_tile;
  }
}
inline void xcd_queue_tiles(const mtgr_batch* b, int H, int q_tile, int64_t tiles[kXcdCount]) {
  std::vector<int32_t> order(b->num_users <= kLptMaxUsers ? b->num_users : 0);
  xcd_queue_tiles(b, H, q_tile, tiles, order.data());
}

// The attention grid, in workgroups per XCD: the longest XCD queue.
inline int64_t xcd_grid_slots(const mtgr_batch* b, int H, int q_tile, int32_t* order_buf) {
  int64_t tiles[kXcdCount];
  xcd_queue_tiles(b, H, q_tile, tiles, order_buf);
  return *std::max_element(tiles, tiles + kXcdCount);
}
inline int64_t xcd_grid_slots(const mtgr_batch* b, int H, int q_tile) {
  int64_t tiles[kXcdCount];
  xcd_queue_tiles(b, H, q_tile, tiles);
  return *std::max_element(tiles, tiles + kXcdCount);
}

inline int64_t total_tiles(const mtgr_batch* b, int q_tile) {
  int64_t t = 0;
  for (int32_t i = 0; i < b->num_users; ++i) t += (user_len(b, i) + q_tile - 1) / q_tile;
  return t;
}

// ---- workspace layout --------------------------------------------------------------------------
struct Sizes {
  int64_t B = 0, T = 0, C = 0;
  int d = 0, h = 0, hh = 0, dtype = MTGR_F32, H = 0;
  bool need_xres = false, need_head = false, need_acts = false;
};

inline Sizes sizes_for(const mtgr_batch* b, int d, int h, int hh, int dtype, int H) {
  Sizes z;
  z.H = H;
  z.B = b->num_users;
  z.T = b->num_tokens;
  z.C = b->num_candidates;
  z.d = d;
  z.h = h;
  z.hh = hh;
  z.dtype = dtype;
  return z;
}

// Byte offsets of the workspace regions (each 256-byte aligned), and the total.
struct Plan {
  size_t seg = 0, order = 0, tile_off = 0, cand_off = 0, cand_idx = 0, flags = 0, xcd_off = 0, xcd_fwd = 0;
  size_t xt = 0, big = 0, y = 0, xres = 0, hin = 0, hhid = 0;
  size_t total = 0;
};

inline Plan make_plan(const Sizes& z) {
  Plan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t es = esize(z.dtype);
  p.flags = take(4 * sizeof(int32_t));
  p.seg = take((size_t)z.B * kUserSegBytes);
  p.order = take((size_t)z.B * sizeof(int32_t));
  p.tile_off = take((size_t)(z.B + 1) * sizeof(int32_t));
  p.cand_off = take((size_t)(z.B + 1) * sizeof(int64_t));
  p.cand_idx = take((size_t)z.C * sizeof(int64_t));
  const int64_t rounds = (z.B * z.H + kXcdCount - 1) / kXcdCount;
  p.xcd_off = take((size_t)kXcdCount * (rounds + 1) * sizeof(int32_t));
  p.xcd_fwd = take((size_t)kXcdCount * (rounds + 1) * sizeof(int32_t));
  if (z.need_acts) {
    p.xt = take((size_t)z.T * z.d * es);
    p.big = take((size_t)z.T * std::max(4 * z.d, z.h) * es);
    p.y = take((size_t)z.T * z.d * es);
  }
  if (z.need_xres) p.xres = take((size_t)z.T * z.d * sizeof(float));
  if (z.need_head) {
    p.hin = take((size_t)z.C * z.d * es);
    p.hhid = take((size_t)z.C * z.hh * es);
  }
  p.total = off;
  return p;
}

// Workspace of the block backward after the prep buffers: the recomputed forward activations, the
// activation gradients, in fp32 transposed copies for the weight-gradient GEMMs (token axis last,
// padded to Tp with zeros, plus a ones row whose product gives the bias gradient), one transposed
// weight, and fp32 partial sums (split-K slices of the weight gradients, per-wavefront GroupLN slots).
struct BwdPlan {
  Plan prep;
  size_t xt = 0, qkvu = 0, y = 0, vt = 0, z = 0, a = 0, dout = 0, dhid = 0, dz = 0;
  size_t dqkvu = 0, ta = 0, tb = 0, wt = 0, part = 0, cs = 0, gpart = 0, total = 0;
  // per weight-gradient GEMM (0: W2, 1: W1, 2: W_qkvu): split count and padded token axis
  int ks[3] = {1, 1, 1};
  int64_t Tp[3] = {0, 0, 0};
  bool ok = true;   // every bf16 split within a 32-bit buffer range
};

constexpr int64_t kMaxBwdTokens = 4000000;
constexpr int64_t kGemmWorkgroups = 256;   // persistent GEMM grid: one workgroup per CU of an MI355X

inline int64_t tiles256(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 255) / 256); }

inline BwdPlan make_bwd_plan(const Sizes& z) {
  BwdPlan p;
  p.prep = make_plan(z);
  size_t off = p.prep.total;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t es = esize(z.dtype);
  const size_t T = (size_t)z.T, d = (size_t)z.d, h = (size_t)z.h;
  // Split count of each weight-gradient GEMM.  The persistent GEMM runs one workgroup per CU.  bf16
  // (k-major GEMM, no bias column): with at least 8 x 2048 tokens the split count is a multiple of
  // the XCD count (each split's tiles share one XCD's L2), chosen for whole rounds of each XCD's
  // workgroups, at most 64; below that 1..7 splits for whole rounds of the grid.  fp32 (transposed
  // operands with a ones row): 1..32 splits for whole rounds of the grid.  Each split is at least
  // 2048 tokens long, one split's rows stay within a 32-bit buffer range, ties go to fewer splits.
  const bool bf = z.dtype == MTGR_BF16;
  const int64_t Mg[3] = {(int64_t)d, (int64_t)h, 4 * (int64_t)d};
  const int64_t Kg[3] = {(int64_t)h, (int64_t)d, (int64_t)d};
  const int64_t per_xcd = kGemmWorkgroups / 8;
  int64_t tp_max = 0;
  size_t part_max = 0, cs_max = 0;
  for (int gi = 0; gi < 3; ++gi) {
    const int64_t tiles = tiles256(Mg[gi], Kg[gi] + (bf ? 0 : 8));
    const bool xcd_major = bf && z.T >= 8 * 2048;
    int best = 0;
    double best_eff = 0.0;
    for (int ks = xcd_major ? 8 : 1; ks <= (xcd_major ? 64 : bf ? 7 : 32) && (ks == 1 || z.T >= (int64_t)ks * 2048);
         ks += xcd_major ? 8 : 1) {
      const int64_t unit_k = 64 * (int64_t)ks;
      const int64_t tp_k = std::max((z.T + unit_k - 1) / unit_k * unit_k, 2 * unit_k);
      if (bf && (tp_k / ks) * std::max(Mg[gi], Kg[gi]) * 2 >= (int64_t(1) << 31)) continue;
      const int64_t work = xcd_major ? tiles * ks / 8 : tiles * ks;
      const int64_t slots = xcd_major ? per_xcd : kGemmWorkgroups;
      const int64_t rounds = (work + slots - 1) / slots;
      const double eff = (double)work / (double)(rounds * slots);
      if (eff > best_eff + 1e-9) { best_eff = eff; best = ks; }
    }
    p.ks[gi] = std::max(best, 1);
    if (best == 0) p.ok = false;
    const int64_t unit = 64 * (int64_t)p.ks[gi];
    p.Tp[gi] = std::max((z.T + unit - 1) / unit * unit, 2 * unit);
    tp_max = std::max(tp_max, p.Tp[gi]);
    part_max = std::max(part_max, (size_t)p.ks[gi] * Mg[gi] * (Kg[gi] + (bf ? 0 : 8)));
    if (bf) cs_max = std::max(cs_max, (size_t)colsum_blocks(z.T, (int)Mg[gi]) * Mg[gi]);
  }
  p.xt = take(T * d * es);
  p.qkvu = take(T * 4 * d * es);
  p.y = take(T * d * es);
  p.vt = take(T * d * es);
  p.z = take(T * d * es);
  p.a = take(T * h * es);
  p.dout = take(z.dtype == MTGR_BF16 ? T * d * es : 0);
  p.dhid = take(T * h * es);
  p.dz = take(T * d * es);
  p.dqkvu = take(T * 4 * d * es);
  // transposed copies for the fp32 weight-gradient GEMMs (the bf16 ones read activations in place)
  p.ta = take(bf ? 0 : std::max({d, h, 4 * d}) * (size_t)tp_max * es);
  p.tb = take(bf ? 0 : (std::max(d, h) + 8) * (size_t)tp_max * es);
  p.wt = take(std::max(h * d, 4 * d * d) * es);
  p.part = take(part_max * sizeof(float));
  p.cs = take(cs_max * sizeof(float));
  p.gpart = take((size_t)std::max(groupln_bwd_waves(z.T, 0), groupln_bwd_waves(z.T, 1)) * 8 * d * sizeof(float));
  p.total = off;
  return p;
}

}  // namespace plan
}  // namespace mtgr
