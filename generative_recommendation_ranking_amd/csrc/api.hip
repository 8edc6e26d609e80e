// C ABI of libmtgr.so: argument validation, workspace planning and launch sequencing for the
// MTGR HSTU encoder forward (marovi.ai MTGR page, 方法: GroupLN -> QKVU -> masked silu
// attention / N -> U gate -> GroupLN -> MLP + residual, L times; candidate head after the last
// block).  Every check runs on the host before the first launch.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/mtgr.h"
#include "kernels.h"

using namespace mtgr;
using namespace mtgr::plan;

// Fixed device scratch of mtgr_attention_fwd_noalloc: the batch-prep tables of one call.  Every GPU
// the library runs on holds its own copy until the process ends; host code reaches it only through
// the per-device address from hipGetSymbolAddress (the array's name is a host-side stand-in).
static constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

template <typename T>
inline T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

PrepBufs prep_bufs(void* ws, const Plan& p) {
  PrepBufs pb;
  pb.seg = at<UserSeg>(ws, p.seg);
  pb.order = at<int32_t>(ws, p.order);
  pb.tile_off = at<int32_t>(ws, p.tile_off);
  pb.cand_off = at<int64_t>(ws, p.cand_off);
  pb.cand_idx = at<int64_t>(ws, p.cand_idx);
  pb.flags = at<int32_t>(ws, p.flags);
  pb.xcd_off = at<int32_t>(ws, p.xcd_off);
  pb.xcd_fwd = at<int32_t>(ws, p.xcd_fwd);
  return pb;
}

inline int q_tile_for(int dtype) { return dtype == MTGR_BF16 ? kAttnQTileBf16 : kAttnQTileF32; }
inline int q_tile_fwd_for(int dtype) { return dtype == MTGR_BF16 ? kAttnFwdQTileBf16 : 0; }

mtgr_status hip_status(hipError_t e) { return e == hipSuccess ? MTGR_OK : MTGR_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

#define MTGR_TRY(expr)                           \
  do {                                           \
    hipError_t _e = (expr);                      \
    if (_e != hipSuccess) return MTGR_ERR_HIP;   \
  } while (0)

hipError_t linear(int64_t M, int N, int K, int dtype, int epi, const void* a, const void* w,
                  const void* bias, const float* resid, void* out, hipStream_t s) {
  if (dtype == MTGR_BF16)
    return launch_gemm_bf16(M, N, K, epi, static_cast<const bf16*>(a), static_cast<const bf16*>(w),
                            static_cast<const bf16*>(bias), resid, out, s);
  return launch_gemm_f32(M, N, K, epi, static_cast<const float*>(a), static_cast<const float*>(w),
                         static_cast<const float*>(bias), resid, static_cast<float*>(out), s);
}

// order_buf (room for min(B, kLptMaxUsers) entries, or NULL to use a vector) holds the host's work
// order while the grid is sized
hipError_t attention(const mtgr_batch* b, int d, int H, int dtype, int mask_mode,
                     const PrepBufs& pb, const void* qkvu, void* y, hipStream_t s,
                     void* vt = nullptr, int32_t* order_buf = nullptr) {
  if (dtype == MTGR_BF16)
    return launch_attention_bf16(b->num_users,
                                 order_buf ? xcd_grid_slots(b, H, kAttnFwdQTileBf16, order_buf)
                                           : xcd_grid_slots(b, H, kAttnFwdQTileBf16),
                                 d, H,
                                 mask_mode, b->offsets, pb.seg, pb.order, pb.xcd_fwd, b->timestamps,
                                 static_cast<const bf16*>(qkvu), static_cast<bf16*>(y),
                                 static_cast<bf16*>(vt), s);
  const int64_t tiles = total_tiles(b, kAttnQTileF32);
  return launch_attention_f32(b->num_users, tiles, d, H, mask_mode, b->offsets, pb.seg, pb.order,
                              pb.tile_off, b->timestamps, static_cast<const float*>(qkvu),
                              static_cast<float*>(y), static_cast<float*>(vt), s);
}

// Attention backward: dqkvu [T][4d] from qkvu, the ungated V~ and dy = dL/d(V~ (.) U).  bf16
// runs the MFMA kernels (g: [T][d] bf16 scratch for dy (.) U); fp32 the one-thread-per-row kernels.
hipError_t attention_bwd(const mtgr_batch* b, int d, int H, int dtype, int mask_mode, const PrepBufs& pb,
                         const void* qkvu, const void* vt, const void* dy, void* g, void* dqkvu,
                         hipStream_t s) {
  if (dtype == MTGR_BF16)
    return launch_attention_bwd_bf16(b->num_users, b->num_tokens, xcd_grid_slots(b, H, kAttnQTileBf16), d, H,
                                     mask_mode, b->offsets, pb.seg, pb.order, pb.xcd_off, b->timestamps,
                                     static_cast<const bf16*>(qkvu), static_cast<const bf16*>(vt),
                                     static_cast<const bf16*>(dy), static_cast<bf16*>(g),
                                     static_cast<bf16*>(dqkvu), s);
  return launch_attention_bwd_ref(b->num_users, total_tiles(b, kAttnQTileF32), kAttnQTileF32, d, H, mask_mode, 0,
                                  b->offsets, pb.seg, pb.order, pb.tile_off, b->timestamps, qkvu, vt, dy,
                                  dqkvu, s);
}

// One block: x_out = x_in + MLP(GLN2(attn(GLN1(x_in)) (.) U)); x_out may alias x_in.
hipError_t run_block(const mtgr_block_params* p, const mtgr_batch* b, const PrepBufs& pb,
                     const Plan& pl, void* ws, const float* x_in, float* x_out, hipStream_t s) {
  const int64_t T = b->num_tokens;
  const int d = p->d_model, h = p->mlp_hidden, dt = p->dtype;
  const int act = dt == MTGR_BF16 ? 1 : 0;
  void* xt = at<void>(ws, pl.xt);
  void* big = at<void>(ws, pl.big);
  void* y = at<void>(ws, pl.y);
  hipError_t e;
  const int shared = p->norm_mode == MTGR_NORM_SHARED;
  e = launch_groupln(T, d, 0, act, act, shared, x_in, b->group_ids, p->gln1_gamma, p->gln1_beta,
                     p->ln_eps, xt, s);
  if (e != hipSuccess) return e;
  e = linear(T, 4 * d, d, dt, MTGR_EPI_STORE, xt, p->w_qkvu, p->b_qkvu, nullptr, big, s);
  if (e != hipSuccess) return e;
  e = attention(b, d, p->num_heads, dt, p->mask_mode, pb, big, y, s);
  if (e != hipSuccess) return e;
  e = launch_groupln(T, d, act, act, act, shared, y, b->group_ids, p->gln2_gamma, p->gln2_beta,
                     p->ln_eps, xt, s);
  if (e != hipSuccess) return e;
  e = linear(T, h, d, dt, MTGR_EPI_SILU, xt, p->w_mlp1, p->b_mlp1, nullptr, big, s);
  if (e != hipSuccess) return e;
  return linear(T, d, h, dt, MTGR_EPI_RESIDUAL_F32, big, p->w_mlp2, p->b_mlp2, x_in, x_out, s);
}

// ---- backward ----------------------------------------------------------------------------------
// dW [M][K] (+ db [M]) = sum over tokens of dy^T x by split-K GEMMs and fixed-order reductions;
// dy [T][M] and x [T][K] token-major.  bf16: the k-major GEMM reads them in place and db is the
// column sum of dy.  fp32: transposed copies [M][Tp] and [K+8][Tp] (row K all ones, so that
// column K of the product is db) and the fp32 GEMM.
hipError_t weight_grad(const BwdPlan& pl, int gi, void* ws, int dtype, int64_t T, int M, int K, const void* dy,
                       const void* x, float* dw, float* db, hipStream_t s) {
  float* part = at<float>(ws, pl.part);
  hipError_t e;
  if (dtype == MTGR_BF16) {
    e = launch_gemm_bf16_kmajor_splitk(M, K, pl.Tp[gi], pl.ks[gi], T, static_cast<const bf16*>(dy), M,
                                       static_cast<const bf16*>(x), K, part, s);
    if (e == hipSuccess) e = launch_reduce_wb(M, K, K, pl.ks[gi], part, dw, nullptr, s);
    if (e == hipSuccess && db) e = launch_colsum_bf16(T, M, static_cast<const bf16*>(dy), at<float>(ws, pl.cs), db, s);
    return e;
  }
  const int Kx = K + 8;
  void* ta = at<void>(ws, pl.ta);
  void* tb = at<void>(ws, pl.tb);
  e = launch_transpose(T, M, pl.Tp[gi], 0, 0, dy, ta, s);
  if (e == hipSuccess) e = launch_transpose(T, K, pl.Tp[gi], 1, 0, x, tb, s);
  if (e == hipSuccess)
    e = launch_gemm_f32_splitk(M, Kx, (int)pl.Tp[gi], pl.ks[gi], static_cast<const float*>(ta),
                               static_cast<const float*>(tb), part, s);
  if (e != hipSuccess) return e;
  return launch_reduce_wb(M, K, Kx, pl.ks[gi], part, dw, db, s);
}

// GroupLN parameter gradients from the per-wavefront slots [waves][2][4][d].
hipError_t gln_param_grads(int64_t T, int d, int x_kind, const float* gpart, float* dgamma, float* dbeta,
                           hipStream_t s) {
  const int waves = T > 0 ? groupln_bwd_waves(T, x_kind) : 0;
  hipError_t e = launch_reduce(4 * (int64_t)d, waves, 8 * (int64_t)d, gpart, dgamma, s);
  if (e != hipSuccess) return e;
  return launch_reduce(4 * (int64_t)d, waves, 8 * (int64_t)d, gpart ? gpart + 4 * d : nullptr, dbeta, s);
}

hipError_t run_block_bwd(const mtgr_block_params* p, const mtgr_batch* b, const BwdPlan& pl,
                         void* ws, const float* x_in, const float* dx_out, float* dx_in,
                         const mtgr_block_grads* g, hipStream_t s) {
  const int64_t T = b->num_tokens;
  const int d = p->d_model, h = p->mlp_hidden, dt = p->dtype, H = p->num_heads;
  const int act = dt == MTGR_BF16 ? 1 : 0;
  const int shared = p->norm_mode == MTGR_NORM_SHARED;
  const PrepBufs pb = prep_bufs(ws, pl.prep);
  void* xt = at<void>(ws, pl.xt);
  void* qkvu = at<void>(ws, pl.qkvu);
  void* y = at<void>(ws, pl.y);
  void* vt = at<void>(ws, pl.vt);
  void* z = at<void>(ws, pl.z);
  void* a = at<void>(ws, pl.a);
  void* dhid = at<void>(ws, pl.dhid);
  void* dz = at<void>(ws, pl.dz);
  void* dqkvu = at<void>(ws, pl.dqkvu);
  void* wt = at<void>(ws, pl.wt);
  float* gpart = at<float>(ws, pl.gpart);
  const int q_tile = q_tile_for(dt);
  hipError_t e;
#define MTGR_BWD_TRY(expr)              \
  do {                                  \
    e = (expr);                         \
    if (e != hipSuccess) return e;      \
  } while (0)
  MTGR_BWD_TRY(launch_prep(b->num_users, b->num_candidates, b->offsets, b->group_ids, q_tile, q_tile_fwd_for(dt), H, pb, false, s));
  // forward, keeping what the backward needs: GLN1 output, QKVU, V~, the gated output, GLN2
  // output and the MLP pre-activation a (its SiLU replaces it in the SiLU backward)
  MTGR_BWD_TRY(launch_groupln(T, d, 0, act, act, shared, x_in, b->group_ids, p->gln1_gamma,
                              p->gln1_beta, p->ln_eps, xt, s));
  MTGR_BWD_TRY(linear(T, 4 * d, d, dt, MTGR_EPI_STORE, xt, p->w_qkvu, p->b_qkvu, nullptr, qkvu, s));
  MTGR_BWD_TRY(attention(b, d, H, dt, p->mask_mode, pb, qkvu, y, s, vt));
  MTGR_BWD_TRY(launch_groupln(T, d, act, act, act, shared, y, b->group_ids, p->gln2_gamma,
                              p->gln2_beta, p->ln_eps, z, s));
  MTGR_BWD_TRY(linear(T, h, d, dt, MTGR_EPI_STORE, z, p->w_mlp1, p->b_mlp1, nullptr, a, s));

  // MLP2 and the SiLU: dhid = dout W2, da = dhid (.) silu'(a) (in bf16 inside the GEMM's
  // epilogue), with hid = silu(a) replacing a; then dW2 = dout^T hid, db2 = sum dout
  const void* dout = dx_out;
  if (act) {   // bf16 copy of dout; db2 = its column sums, taken from the fp32 values on the way
    MTGR_BWD_TRY(launch_convert_colsum(T, d, dx_out, at<bf16>(ws, pl.dout), at<float>(ws, pl.cs), g->b_mlp2, s));
    dout = at<void>(ws, pl.dout);
  }
  MTGR_BWD_TRY(launch_transpose(d, h, d, 0, act, p->w_mlp2, wt, s));
  if (act) {   // bf16: the SiLU backward runs in the GEMM's epilogue
    MTGR_BWD_TRY(launch_gemm_bf16_silu_bwd(T, h, d, static_cast<const bf16*>(dout), static_cast<const bf16*>(wt),
                                           static_cast<bf16*>(a), static_cast<bf16*>(dhid), s));
  } else {
    MTGR_BWD_TRY(linear(T, h, d, dt, MTGR_EPI_STORE, dout, wt, nullptr, nullptr, dhid, s));
    MTGR_BWD_TRY(launch_silu_bwd(T * h, act, a, dhid, s));
  }
  MTGR_BWD_TRY(weight_grad(pl, 0, ws, dt, T, d, h, dout, a, g->w_mlp2, act ? nullptr : g->b_mlp2, s));
  // MLP1: dz = da W1, dW1 = da^T z, db1 = sum da
  MTGR_BWD_TRY(launch_transpose(h, d, h, 0, act, p->w_mlp1, wt, s));
  MTGR_BWD_TRY(linear(T, d, h, dt, MTGR_EPI_STORE, dhid, wt, nullptr, nullptr, dz, s));
  MTGR_BWD_TRY(weight_grad(pl, 1, ws, dt, T, h, d, dhid, z, g->w_mlp1, g->b_mlp1, s));
  // GLN2: dy (in place over dz) and the GLN2 parameter gradients
  MTGR_BWD_TRY(launch_groupln_bwd(T, d, act, act, shared, y, b->group_ids, p->gln2_gamma, p->ln_eps,
                                  dz, nullptr, dz, act, gpart, s));
  MTGR_BWD_TRY(gln_param_grads(T, d, act, gpart, g->gln2_gamma, g->gln2_beta, s));
  // gate and attention: dqkvu from qkvu, V~ and dy (G = dy (.) U goes to the free dout buffer)
  MTGR_BWD_TRY(attention_bwd(b, d, H, dt, p->mask_mode, pb, qkvu, vt, dz, at<void>(ws, pl.dout), dqkvu, s));
  // QKVU: dxt = dqkvu W_qkvu (over dz), dW_qkvu = dqkvu^T xt, db_qkvu = sum dqkvu
  MTGR_BWD_TRY(launch_transpose(4 * (int64_t)d, d, 4 * (int64_t)d, 0, act, p->w_qkvu, wt, s));
  MTGR_BWD_TRY(linear(T, d, 4 * d, dt, MTGR_EPI_STORE, dqkvu, wt, nullptr, nullptr, dz, s));
  MTGR_BWD_TRY(weight_grad(pl, 2, ws, dt, T, 4 * d, d, dqkvu, xt, g->w_qkvu, g->b_qkvu, s));
  // GLN1 plus the residual path: dx_in = dx_out + GLN1'(x_in)^T dxt
  MTGR_BWD_TRY(launch_groupln_bwd(T, d, 0, act, shared, x_in, b->group_ids, p->gln1_gamma, p->ln_eps,
                                  dz, dx_out, dx_in, 0, gpart, s));
  MTGR_BWD_TRY(gln_param_grads(T, d, 0, gpart, g->gln1_gamma, g->gln1_beta, s));
#undef MTGR_BWD_TRY
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t mtgr_abi_version(void) { return MTGR_ABI_VERSION; }

const char* mtgr_status_str(int32_t status) {
  switch (status) {
    case MTGR_OK: return "ok";
    case MTGR_ERR_NULL_ARG: return "a required pointer is NULL";
    case MTGR_ERR_BAD_SHAPE: return "unsupported or inconsistent shape";
    case MTGR_ERR_BAD_BATCH: return "malformed batch (offsets, token or candidate counts)";
    case MTGR_ERR_UNSUPPORTED: return "unsupported dtype or option";
    case MTGR_ERR_WORKSPACE: return "workspace missing or too small";
    case MTGR_ERR_HIP: return "HIP launch or copy failed";
    case MTGR_ERR_SCRATCH_LIMIT: return "batch needs more than the fixed scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

mtgr_status mtgr_encoder_workspace_size(const mtgr_encoder_params* p, const mtgr_batch* b,
                                        size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_encoder(p);
  if (st != MTGR_OK) return st;
  if ((st = check_batch(b)) != MTGR_OK) return st;
  if ((st = check_user_rows(b, p->layers[0].d_model, p->layers[0].dtype)) != MTGR_OK) return st;
  Sizes z = sizes_for(b, p->layers[0].d_model, 0, p->head_hidden, p->layers[0].dtype,
                      p->layers[0].num_heads);
  for (int32_t l = 0; l < p->num_layers; ++l) z.h = std::max(z.h, (int)p->layers[l].mlp_hidden);
  z.need_acts = z.need_xres = z.need_head = true;
  *bytes = make_plan(z).total;
  return MTGR_OK;
}

mtgr_status mtgr_block_workspace_size(const mtgr_block_params* p, const mtgr_batch* b,
                                      size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_block(p);
  if (st != MTGR_OK) return st;
  if ((st = check_batch(b)) != MTGR_OK) return st;
  if ((st = check_user_rows(b, p->d_model, p->dtype)) != MTGR_OK) return st;
  Sizes z = sizes_for(b, p->d_model, p->mlp_hidden, 0, p->dtype, p->num_heads);
  z.need_acts = true;
  *bytes = make_plan(z).total;
  return MTGR_OK;
}

mtgr_status mtgr_attention_workspace_size(const mtgr_batch* b, int32_t d, int32_t num_heads,
                                          size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_batch(b);
  if (st != MTGR_OK) return st;
  if (d <= 0 || num_heads <= 0 || d % num_heads != 0) return MTGR_ERR_BAD_SHAPE;
  Sizes z = sizes_for(b, d, 0, 0, MTGR_F32, num_heads);
  *bytes = make_plan(z).total;
  return MTGR_OK;
}

mtgr_status mtgr_block_bwd_workspace_size(const mtgr_block_params* p, const mtgr_batch* b,
                                          size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_block(p);
  if (st != MTGR_OK) return st;
  if ((st = check_batch(b)) != MTGR_OK) return st;
  if ((st = check_user_rows(b, p->d_model, p->dtype)) != MTGR_OK) return st;
  // a bound on the workspace; the bf16 weight-gradient GEMMs also need split counts that keep each
  // split's activation rows within a 32-bit buffer range
  if (b->num_tokens > kMaxBwdTokens) return MTGR_ERR_BAD_SHAPE;
  Sizes z = sizes_for(b, p->d_model, p->mlp_hidden, 0, p->dtype, p->num_heads);
  const BwdPlan pl = make_bwd_plan(z);
  if (!pl.ok) return MTGR_ERR_BAD_SHAPE;
  *bytes = pl.total;
  return MTGR_OK;
}

mtgr_status mtgr_block_bwd(const mtgr_block_params* p, const mtgr_batch* b, const float* x_in,
                           const float* dx_out, float* dx_in, const mtgr_block_grads* g, void* ws,
                           size_t ws_bytes, void* stream) {
  size_t need = 0;
  mtgr_status st = mtgr_block_bwd_workspace_size(p, b, &need);
  if (st != MTGR_OK) return st;
  if (!g || !g->gln1_gamma || !g->gln1_beta || !g->w_qkvu || !g->gln2_gamma || !g->gln2_beta ||
      !g->w_mlp1 || !g->w_mlp2)
    return MTGR_ERR_NULL_ARG;
  if (b->num_tokens > 0 && (!x_in || !dx_out || !dx_in)) return MTGR_ERR_NULL_ARG;
  if (!ws || ws_bytes < need) return MTGR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = p->d_model, h = p->mlp_hidden;
  if (b->num_users == 0 || b->num_tokens == 0) {
    // no tokens: every parameter gradient is an empty sum
    MTGR_TRY(launch_reduce_wb(d, h, h + 8, 0, nullptr, g->w_mlp2, g->b_mlp2, s));
    MTGR_TRY(launch_reduce_wb(h, d, d + 8, 0, nullptr, g->w_mlp1, g->b_mlp1, s));
    MTGR_TRY(launch_reduce_wb(4 * d, d, d + 8, 0, nullptr, g->w_qkvu, g->b_qkvu, s));
    MTGR_TRY(gln_param_grads(0, d, 0, nullptr, g->gln1_gamma, g->gln1_beta, s));
    MTGR_TRY(gln_param_grads(0, d, 0, nullptr, g->gln2_gamma, g->gln2_beta, s));
    return MTGR_OK;
  }
  Sizes z = sizes_for(b, d, h, 0, p->dtype, p->num_heads);
  const BwdPlan pl = make_bwd_plan(z);
  MTGR_TRY(run_block_bwd(p, b, pl, ws, x_in, dx_out, dx_in, g, s));
  return MTGR_OK;
}

mtgr_status mtgr_attention_bwd_workspace_size(const mtgr_batch* b, int32_t d, int32_t num_heads,
                                              int32_t dtype, size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_batch(b);
  if (st != MTGR_OK) return st;
  if ((st = check_attn_shape(d, num_heads, dtype)) != MTGR_OK) return st;
  if ((st = check_user_rows(b, d, dtype)) != MTGR_OK) return st;
  Sizes z = sizes_for(b, d, 0, 0, dtype, num_heads);
  *bytes = make_plan(z).total + align_up((size_t)b->num_tokens * d * esize(dtype));
  return MTGR_OK;
}

mtgr_status mtgr_attention_bwd(const mtgr_batch* b, int32_t d, int32_t num_heads, int32_t dtype,
                               int32_t mask_mode, const void* qkvu, const void* v_tilde,
                               const void* dy_gated, void* dqkvu, void* ws, size_t ws_bytes,
                               void* stream) {
  size_t need = 0;
  mtgr_status st = mtgr_attention_bwd_workspace_size(b, d, num_heads, dtype, &need);
  if (st != MTGR_OK) return st;
  if (!mask_mode_ok(mask_mode)) return MTGR_ERR_UNSUPPORTED;
  if (b->num_tokens > 0 && (!qkvu || !v_tilde || !dy_gated || !dqkvu)) return MTGR_ERR_NULL_ARG;
  if (!ws || ws_bytes < need) return MTGR_ERR_WORKSPACE;
  if (b->num_users == 0 || b->num_tokens == 0) return MTGR_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Sizes z = sizes_for(b, d, 0, 0, dtype, num_heads);
  const Plan pl = make_plan(z);
  const PrepBufs pb = prep_bufs(ws, pl);
  MTGR_TRY(launch_prep(b->num_users, b->num_candidates, b->offsets, b->group_ids, q_tile_for(dtype), q_tile_fwd_for(dtype), num_heads, pb,
                       false, s));
  MTGR_TRY(attention_bwd(b, d, num_heads, dtype, mask_mode, pb, qkvu, v_tilde, dy_gated, at<void>(ws, pl.total),
                         dqkvu, s));
  return MTGR_OK;
}

mtgr_status mtgr_encoder_fwd(const mtgr_encoder_params* p, const mtgr_batch* b, const float* x_in,
                             float* hidden_out, float* logits, void* ws, size_t ws_bytes,
                             void* stream) {
  size_t need = 0;
  mtgr_status st = mtgr_encoder_workspace_size(p, b, &need);
  if (st != MTGR_OK) return st;
  if (b->num_tokens > 0 && !x_in) return MTGR_ERR_NULL_ARG;
  if (b->num_candidates > 0 && !logits) return MTGR_ERR_NULL_ARG;
  if (!ws || ws_bytes < need) return MTGR_ERR_WORKSPACE;
  if (b->num_users == 0 || b->num_tokens == 0) return MTGR_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = p->layers[0].dtype;
  Sizes z = sizes_for(b, p->layers[0].d_model, 0, p->head_hidden, dt, p->layers[0].num_heads);
  for (int32_t l = 0; l < p->num_layers; ++l) z.h = std::max(z.h, (int)p->layers[l].mlp_hidden);
  z.need_acts = z.need_xres = z.need_head = true;
  const Plan pl = make_plan(z);
  const PrepBufs pb = prep_bufs(ws, pl);
  MTGR_TRY(launch_prep(b->num_users, b->num_candidates, b->offsets, b->group_ids, q_tile_for(dt), q_tile_fwd_for(dt), z.H, pb, true, s));
  float* xr = hidden_out ? hidden_out : at<float>(ws, pl.xres);
  for (int32_t l = 0; l < p->num_layers; ++l) {
    const float* src = (l == 0) ? x_in : xr;
    MTGR_TRY(run_block(&p->layers[l], b, pb, pl, ws, src, xr, s));
  }
  const int64_t C = b->num_candidates;
  if (C > 0) {
    const int d = z.d, hh = p->head_hidden;
    const int act = dt == MTGR_BF16 ? 1 : 0;
    void* hin = at<void>(ws, pl.hin);
    void* hhid = at<void>(ws, pl.hhid);
    MTGR_TRY(launch_gather_rows(C, b->num_tokens, d, xr, pb.cand_idx, act, hin, s));
    MTGR_TRY(linear(C, hh, d, dt, MTGR_EPI_SILU, hin, p->w_head1, p->b_head1, nullptr, hhid, s));
    MTGR_TRY(launch_head_out(C, hh, act, hhid, p->w_head2, p->b_head2, logits, s));
  }
  return MTGR_OK;
}

mtgr_status mtgr_block_fwd(const mtgr_block_params* p, const mtgr_batch* b, const float* x_in,
                           float* x_out, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  mtgr_status st = mtgr_block_workspace_size(p, b, &need);
  if (st != MTGR_OK) return st;
  if (b->num_tokens > 0 && (!x_in || !x_out)) return MTGR_ERR_NULL_ARG;
  if (!ws || ws_bytes < need) return MTGR_ERR_WORKSPACE;
  if (b->num_users == 0 || b->num_tokens == 0) return MTGR_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Sizes z = sizes_for(b, p->d_model, p->mlp_hidden, 0, p->dtype, p->num_heads);
  z.need_acts = true;
  const Plan pl = make_plan(z);
  const PrepBufs pb = prep_bufs(ws, pl);
  MTGR_TRY(launch_prep(b->num_users, b->num_candidates, b->offsets, b->group_ids, q_tile_for(p->dtype), q_tile_fwd_for(p->dtype), z.H, pb, false, s));
  MTGR_TRY(run_block(p, b, pb, pl, ws, x_in, x_out, s));
  return MTGR_OK;
}

mtgr_status mtgr_groupln_fwd(const mtgr_batch* b, int32_t d, int32_t in_dtype, int32_t out_dtype,
                             int32_t param_dtype, int32_t norm_mode, const void* gamma,
                             const void* beta, float eps, const void* x, void* y, void* stream) {
  mtgr_status st = check_batch(b);
  if (st != MTGR_OK) return st;
  if (d <= 0 || d % 8 != 0 || d > 1024) return MTGR_ERR_BAD_SHAPE;
  auto ok_dt = [](int32_t v) { return v == MTGR_F32 || v == MTGR_BF16; };
  if (!ok_dt(in_dtype) || !ok_dt(out_dtype) || !ok_dt(param_dtype)) return MTGR_ERR_UNSUPPORTED;
  if (in_dtype == MTGR_BF16 && out_dtype == MTGR_F32) return MTGR_ERR_UNSUPPORTED;
  if (!norm_mode_ok(norm_mode)) return MTGR_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return MTGR_ERR_BAD_SHAPE;
  if (b->num_tokens == 0) return MTGR_OK;
  if (!gamma || !beta || !x || !y) return MTGR_ERR_NULL_ARG;
  return hip_status(launch_groupln(b->num_tokens, d, in_dtype, out_dtype, param_dtype,
                                   norm_mode == MTGR_NORM_SHARED, x,
                                   b->group_ids, gamma, beta, eps, y,
                                   static_cast<hipStream_t>(stream)));
}

mtgr_status mtgr_linear_fwd(int64_t M, int32_t N, int32_t K, int32_t dtype, int32_t epilogue,
                            const void* a, const void* w, const void* bias, const float* resid,
                            void* out, void* stream) {
  if (dtype != MTGR_F32 && dtype != MTGR_BF16) return MTGR_ERR_UNSUPPORTED;
  if (epilogue < MTGR_EPI_STORE || epilogue > MTGR_EPI_RESIDUAL_F32) return MTGR_ERR_UNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0 || N > (1 << 20)) return MTGR_ERR_BAD_SHAPE;
  if (dtype == MTGR_BF16 && (K % 64 != 0 || K < 128 || N % 8 != 0)) return MTGR_ERR_BAD_SHAPE;
  if (dtype == MTGR_F32 && K % 4 != 0) return MTGR_ERR_BAD_SHAPE;
  if (M == 0) return MTGR_OK;
  if (!a || !w || !out) return MTGR_ERR_NULL_ARG;
  if (epilogue == MTGR_EPI_RESIDUAL_F32 && !resid) return MTGR_ERR_NULL_ARG;
  return hip_status(linear(M, N, K, dtype, epilogue, a, w, bias, resid, out,
                           static_cast<hipStream_t>(stream)));
}

mtgr_status mtgr_attention_fwd(const mtgr_batch* b, int32_t d, int32_t num_heads, int32_t dtype,
                               int32_t mask_mode, const void* qkvu, void* y_gated, void* ws,
                               size_t ws_bytes, void* stream) {
  size_t need = 0;
  mtgr_status st = mtgr_attention_workspace_size(b, d, num_heads, &need);
  if (st != MTGR_OK) return st;
  if ((st = check_attn_shape(d, num_heads, dtype)) != MTGR_OK) return st;
  if ((st = check_user_rows(b, d, dtype)) != MTGR_OK) return st;
  if (!mask_mode_ok(mask_mode)) return MTGR_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < need) return MTGR_ERR_WORKSPACE;
  if (b->num_users == 0 || b->num_tokens == 0) return MTGR_OK;
  if (!qkvu || !y_gated) return MTGR_ERR_NULL_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Sizes z = sizes_for(b, d, 0, 0, MTGR_F32, num_heads);
  const Plan pl = make_plan(z);
  const PrepBufs pb = prep_bufs(ws, pl);
  MTGR_TRY(launch_prep(b->num_users, b->num_candidates, b->offsets, b->group_ids, q_tile_for(dtype), q_tile_fwd_for(dtype), num_heads, pb, false, s));
  MTGR_TRY(attention(b, d, num_heads, dtype, mask_mode, pb, qkvu, y_gated, s));
  return MTGR_OK;
}

mtgr_status mtgr_attention_fwd_noalloc(const mtgr_batch* b, int32_t d, int32_t num_heads, int32_t dtype,
                                       int32_t mask_mode, const void* qkvu, void* y_gated, void* stream) {
  mtgr_status st = check_batch(b);
  if (st != MTGR_OK) return st;
  if (d <= 0 || num_heads <= 0 || d % num_heads != 0) return MTGR_ERR_BAD_SHAPE;
  if ((st = check_attn_shape(d, num_heads, dtype)) != MTGR_OK) return st;
  if ((st = check_user_rows(b, d, dtype)) != MTGR_OK) return st;
  if (!mask_mode_ok(mask_mode)) return MTGR_ERR_UNSUPPORTED;
  // the prep tables of this call (no candidate index: the attention does not read it)
  Sizes z = sizes_for(b, d, 0, 0, MTGR_F32, num_heads);
  z.C = 0;
  const Plan pl = make_plan(z);
  if (pl.total > kNoAllocScratchBytes) return MTGR_ERR_SCRATCH_LIMIT;
  if (b->num_users == 0 || b->num_tokens == 0) return MTGR_OK;
  if (!qkvu || !y_gated) return MTGR_ERR_NULL_ARG;
  void* ws = nullptr;
  MTGR_TRY(scratch_for_current_device(&ws));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PrepBufs pb = prep_bufs(ws, pl);
  // the host's work order for the grid size, in place of a heap vector
  int32_t order_buf[kLptMaxUsers];
  MTGR_TRY(launch_prep(b->num_users, 0, b->offsets, b->group_ids, q_tile_for(dtype), q_tile_fwd_for(dtype), num_heads,
                       pb, false, s));
  MTGR_TRY(attention(b, d, num_heads, dtype, mask_mode, pb, qkvu, y_gated, s, nullptr, order_buf));
  return MTGR_OK;
}

mtgr_status mtgr_validate_batch(const mtgr_batch* b, void* ws, size_t ws_bytes, void* stream,
                                int32_t* flags_out) {
  if (!flags_out) return MTGR_ERR_NULL_ARG;
  *flags_out = 0;
  mtgr_status st = check_batch(b);
  if (st != MTGR_OK) return st;
  Sizes z = sizes_for(b, 8, 0, 0, MTGR_F32, 0);
  const Plan pl = make_plan(z);
  if (!ws || ws_bytes < pl.total) return MTGR_ERR_WORKSPACE;
  if (b->num_users == 0) return MTGR_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* flags = at<int32_t>(ws, pl.flags);
  int32_t host[4] = {0, 0, 0, 0};
  MTGR_TRY(hipMemsetAsync(flags, 0, 4 * sizeof(int32_t), s));
  MTGR_TRY(launch_validate(b->num_users, b->offsets, b->group_ids, b->timestamps, flags, s));
  MTGR_TRY(hipMemcpyAsync(host, flags, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, s));
  MTGR_TRY(hipStreamSynchronize(s));
  int32_t f = host[0];
  if ((int64_t)host[1] != b->num_candidates) f |= 8;
  *flags_out = f;
  return MTGR_OK;
}

mtgr_status mtgr_debug_mask(const mtgr_batch* b, int32_t user, int32_t mask_mode,
                            uint8_t* mask_dev, void* ws, size_t ws_bytes, void* stream) {
  mtgr_status st = check_batch(b);
  if (st != MTGR_OK) return st;
  if (!mask_mode_ok(mask_mode)) return MTGR_ERR_UNSUPPORTED;
  if (user < 0 || user >= b->num_users) return MTGR_ERR_BAD_SHAPE;
  Sizes z = sizes_for(b, 8, 0, 0, MTGR_F32, 0);
  const Plan pl = make_plan(z);
  if (!ws || ws_bytes < pl.total) return MTGR_ERR_WORKSPACE;
  const int64_t n = b->offsets_host[user + 1] - b->offsets_host[user];
  if (n == 0) return MTGR_OK;
  if (!mask_dev) return MTGR_ERR_NULL_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PrepBufs pb = prep_bufs(ws, pl);
  MTGR_TRY(launch_prep(b->num_users, b->num_candidates, b->offsets, b->group_ids, kAttnQTileF32, 0, 0, pb, false, s));
  MTGR_TRY(launch_debug_mask(user, mask_mode, b->offsets, pb.seg, b->timestamps, n, mask_dev, s));
  return MTGR_OK;
}

}  // extern "C"
