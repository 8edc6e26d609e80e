// Batch preparation for the packed jagged batch (user-level aggregation of the MTGR pages:
// one sample per user, D = [U, S, R, [C,I]_1..K]; marovi.ai MTGR page, 方法, equation for D).
//
// From the per-user offsets and the per-token group ids this derives, on the device:
//   * the segment lengths N_U, N_S, N_R, K of every user (group ids are non-decreasing within a
//     user, so each boundary is one binary search);
//   * a longest-first user order (LPT) so the heaviest attention work items start first;
//   * the q-tile prefix over that order (one attention work item per (user, head, q-tile));
//   * candidate offsets and the packed-order list of candidate token rows for the head.
#include "kernels.h"

namespace mtgr {

namespace {

__device__ int64_t lower_bound_group(const uint8_t* g, int64_t lo, int64_t hi, int v) {
  while (lo < hi) {
    int64_t mid = lo + ((hi - lo) >> 1);
    if ((int)g[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ void k_prep_users(int32_t B, const int64_t* __restrict__ offsets,
                             const uint8_t* __restrict__ g, UserSeg* __restrict__ seg,
                             int32_t* __restrict__ order) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int64_t lo = offsets[b], hi = offsets[b + 1];
  int64_t e_u = lower_bound_group(g, lo, hi, 1);
  int64_t e_s = lower_bound_group(g, e_u, hi, 2);
  int64_t e_r = lower_bound_group(g, e_s, hi, 3);
  UserSeg sg;
  sg.n_u = (int32_t)(e_u - lo);
  sg.n_s = (int32_t)(e_s - e_u);
  sg.n_r = (int32_t)(e_r - e_s);
  sg.k = (int32_t)(hi - e_r);
  seg[b] = sg;
  if (B > kLptMaxUsers) {
    order[b] = b;
    return;
  }
  int64_t n = hi - lo;
  int rank = 0;
  for (int o = 0; o < B; ++o) {
    int64_t no = offsets[o + 1] - offsets[o];
    rank += (no > n) || (no == n && o < b);
  }
  order[rank] = b;
}

// Single-workgroup exclusive scans: q-tiles in LPT order, candidates in user order.
__global__ __launch_bounds__(1024) void k_prep_scan(int32_t B, int q_tile,
                                                    const int64_t* __restrict__ offsets,
                                                    const UserSeg* __restrict__ seg,
                                                    const int32_t* __restrict__ order,
                                                    int32_t* __restrict__ tile_off,
                                                    int64_t* __restrict__ cand_off) {
  __shared__ int64_t s_a[1024];
  __shared__ int64_t s_b[1024];
  __shared__ int64_t carry[2];
  const int tid = threadIdx.x;
  if (tid == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    int p = base + tid;
    int64_t va = 0, vb = 0;
    if (p < B) {
      int b = order[p];
      int64_t n = offsets[b + 1] - offsets[b];
      va = (n + q_tile - 1) / q_tile;
      vb = seg[p].k;
    }
    s_a[tid] = va;
    s_b[tid] = vb;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int64_t ta = (tid >= off) ? s_a[tid - off] : 0;
      int64_t tb = (tid >= off) ? s_b[tid - off] : 0;
      __syncthreads();
      s_a[tid] += ta;
      s_b[tid] += tb;
      __syncthreads();
    }
    if (p < B) {
      tile_off[p] = (int32_t)(carry[0] + s_a[tid] - va);
      cand_off[p] = carry[1] + s_b[tid] - vb;
    }
    __syncthreads();
    if (tid == 1023) { carry[0] += s_a[1023]; carry[1] += s_b[1023]; }
    __syncthreads();
  }
  if (tid == 0) {
    tile_off[B] = (int32_t)carry[0];
    cand_off[B] = carry[1];
  }
}

// XCD placement of attention work: groups g = (LPT position p, head h) = p*H + h are dealt to the
// 8 XCDs in snake order (round k = g / 8 holds groups 8k..8k+7; XCD x takes 8k + x in even rounds
// and 8k + 7 - x in odd ones).  xo[x][k] = q-tiles of XCD x's groups in rounds before k, so XCD x
// runs its groups one after another and all q-tiles of a group share that XCD's L2.
__global__ void k_prep_xcd(int32_t B, int H, int q_tile, const int64_t* __restrict__ offsets,
                           const int32_t* __restrict__ order, int32_t* __restrict__ xo) {
  const int x = threadIdx.x;
  if (x >= kXcdCount) return;
  const int64_t G = (int64_t)B * H;
  const int R = (int)((G + kXcdCount - 1) / kXcdCount);
  int32_t* row = xo + (int64_t)x * (R + 1);
  int32_t acc = 0;
  for (int k = 0; k < R; ++k) {
    row[k] = acc;
    const int64_t g = (int64_t)k * kXcdCount + ((k & 1) ? (kXcdCount - 1 - x) : x);
    if (g < G) {
      const int b = order[g / H];
      const int64_t n = offsets[b + 1] - offsets[b];
      acc += (int32_t)((n + q_tile - 1) / q_tile);
    }
  }
  row[R] = acc;
}

__global__ void k_prep_cand(int32_t B, int64_t C, const int64_t* __restrict__ offsets,
                            const UserSeg* __restrict__ seg, const int64_t* __restrict__ cand_off,
                            int64_t* __restrict__ cand_idx) {
  int b = blockIdx.x;
  if (b >= B) return;
  int64_t hi = offsets[b + 1];
  int kb = seg[b].k;
  int64_t first = hi - kb;
  int64_t dst = cand_off[b];
  for (int k = threadIdx.x; k < kb; k += blockDim.x)
    if (dst + k < C) cand_idx[dst + k] = first + k;  // C is the caller's count (validated apart)
}

// flags[0]: bit 1 group id out of range, bit 2 group order broken, bit 4 NaN R/C timestamp;
// flags[1]: number of candidate tokens.
__global__ void k_validate(int32_t B, const int64_t* __restrict__ offsets,
                           const uint8_t* __restrict__ g, const float* __restrict__ t,
                           int32_t* __restrict__ flags) {
  int b = blockIdx.x;
  if (b >= B) return;
  int64_t lo = offsets[b], hi = offsets[b + 1];
  int bad = 0, ncand = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    int gi = g[i];
    if (gi > 3) bad |= 1;
    if (i > lo && gi < (int)g[i - 1]) bad |= 2;
    if (gi >= 2 && t[i] != t[i]) bad |= 4;
    ncand += (gi == 3);
  }
  if (bad) atomicOr(&flags[0], bad);
  if (ncand) atomicAdd(&flags[1], ncand);
}

__global__ void k_debug_mask(int mode, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
                             const float* __restrict__ t, int32_t user, int64_t n,
                             uint8_t* __restrict__ mask) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * n) return;
  int i = (int)(idx / n), j = (int)(idx % n);
  UserSeg sg = seg[user];
  int n_static = sg.n_u + sg.n_s;
  int rc_end = n_static + sg.n_r;
  int64_t lo = offsets[user];
  mask[idx] = mtgr_visible_mode(mode, i, j, n_static, rc_end, t[lo + i], t[lo + j]) ? 1 : 0;
}

}  // namespace

hipError_t launch_prep(int32_t B, int64_t C, const int64_t* offsets, const uint8_t* group_ids,
                       int q_tile, int q_tile_fwd, int heads, const PrepBufs& pb, bool want_cand_idx,
                       hipStream_t s) {
  if (B <= 0) return hipSuccess;
  k_prep_users<<<(B + 255) / 256, 256, 0, s>>>(B, offsets, group_ids, pb.seg, pb.order);
  k_prep_scan<<<1, 1024, 0, s>>>(B, q_tile, offsets, pb.seg, pb.order, pb.tile_off, pb.cand_off);
  if (want_cand_idx) k_prep_cand<<<B, 256, 0, s>>>(B, C, offsets, pb.seg, pb.cand_off, pb.cand_idx);
  if (pb.xcd_off && heads > 0) k_prep_xcd<<<1, 64, 0, s>>>(B, heads, q_tile, offsets, pb.order, pb.xcd_off);
  if (pb.xcd_fwd && heads > 0 && q_tile_fwd > 0)
    k_prep_xcd<<<1, 64, 0, s>>>(B, heads, q_tile_fwd, offsets, pb.order, pb.xcd_fwd);
  return hipGetLastError();
}

hipError_t launch_validate(int32_t B, const int64_t* offsets, const uint8_t* group_ids,
                           const float* timestamps, int32_t* flags, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  k_validate<<<B, 256, 0, s>>>(B, offsets, group_ids, timestamps, flags);
  return hipGetLastError();
}

hipError_t launch_debug_mask(int32_t user, int mask_mode, const int64_t* offsets, const UserSeg* seg,
                             const float* timestamps, int64_t n_user, uint8_t* mask,
                             hipStream_t s) {
  int64_t total = n_user * n_user;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  k_debug_mask<<<(unsigned)blocks, 256, 0, s>>>(mask_mode, offsets, seg, timestamps, user, n_user, mask);
  return hipGetLastError();
}

}  // namespace mtgr
