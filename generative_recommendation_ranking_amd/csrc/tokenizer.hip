// Tokenizer front end on gfx950: field IDs -> encoder input x [T][d].
//
// Per token of group g (U, S, R, C), its F_g fields are embedded (one merged hash store for all
// tables of one width), concatenated, and projected to d_model by the MLP of its domain
// (chenhuiyu blog "MTGR", "Converting heterogeneous features into tokens"; fun-rec 7.3.2, the
// candidate-token equation; marovi.ai MTGR page, 方法, the tokens paragraph).  The IDs of the batch
// are deduplicated before the store lookup, so every distinct key is read once (marovi.ai MTGR
// page, 方法, training-framework paragraph).
//
// Launch sequence:
//   k_tok_users   per user, the token count of each group (group ids are non-decreasing within a
//                 user: three binary searches)
//   k_tok_scan    per group, the exclusive prefix of those counts over users: the position of a
//                 user's group-g tokens among all group-g tokens of the batch
//   k_tok_keys    merged key (table << 40 | id) of every used field, -1 elsewhere
//   dedup         distinct keys and the inverse index (hash_store.hip)
//   lookup        the store row of every distinct key, read once
//   k_tok_build   each token's concatenated field embeddings, written to its row of the
//                 group-sorted feature buffer (group g rows are contiguous, width F_g * e)
//   GEMMs         per group: hid = silu(feat W1_g^T + b1_g), y = hid W2_g^T + b2_g (fp32)
//   k_tok_scatter x[t] = y[pos(t)]; when x fits one 31-bit buffer range the second GEMM writes each
//                 row straight to its token instead (rowmap: sorted row -> token), and
//                 k_tok_zero_unplaced zeroes the tokens that got no sorted row
// Positions are computed from the device's own counts; every write is bounded by the group sizes
// the host was given, so inconsistent sizes give wrong rows, never out-of-range accesses.
#include <algorithm>

#include "kernels.h"

namespace mtgr {

namespace {

__device__ int64_t lower_bound_g(const uint8_t* g, int64_t lo, int64_t hi, int v) {
  while (lo < hi) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if ((int)g[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ void k_tok_users(int32_t B, const int64_t* __restrict__ offsets, const uint8_t* __restrict__ g,
                            int64_t* __restrict__ cnt) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int64_t lo = offsets[b], hi = offsets[b + 1];
  const int64_t e_u = lower_bound_g(g, lo, hi, 1);
  const int64_t e_s = lower_bound_g(g, e_u, hi, 2);
  const int64_t e_r = lower_bound_g(g, e_s, hi, 3);
  cnt[(int64_t)b * 4 + 0] = e_u - lo;
  cnt[(int64_t)b * 4 + 1] = e_s - e_u;
  cnt[(int64_t)b * 4 + 2] = e_r - e_s;
  cnt[(int64_t)b * 4 + 3] = hi - e_r;
}

// goff[g][b] = sum over users b' < b of cnt[b'][g]; one workgroup, tiles of 1024 users
__global__ __launch_bounds__(1024) void k_tok_scan(int32_t B, const int64_t* __restrict__ cnt,
                                                   int64_t* __restrict__ goff) {
  __shared__ int64_t buf[4][1024];
  __shared__ int64_t carry[4];
  const int tid = threadIdx.x;
  if (tid < 4) carry[tid] = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    const int b = base + tid;
    int64_t v[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      v[gi] = b < B ? cnt[(int64_t)b * 4 + gi] : 0;
      buf[gi][tid] = v[gi];
    }
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {        // inclusive Hillis-Steele scan per group
      int64_t add[4];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) add[gi] = tid >= o ? buf[gi][tid - o] : 0;
      __syncthreads();
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) buf[gi][tid] += add[gi];
      __syncthreads();
    }
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
      if (b < B) goff[(int64_t)gi * (B + 1) + b] = carry[gi] + buf[gi][tid] - v[gi];
    __syncthreads();
    if (tid < 4) carry[tid] += buf[tid][1023];
    __syncthreads();
  }
  if (tid < 4) goff[(int64_t)tid * (B + 1) + B] = carry[tid];
}

__global__ __launch_bounds__(256) void k_tok_keys(int64_t T, int fmax, const int64_t* __restrict__ ids,
                                                  const uint8_t* __restrict__ g, TokFields tf,
                                                  int64_t* __restrict__ keys) {
  const int64_t n = T * fmax;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / fmax;
    const int f = (int)(i - t * fmax);
    const int grp = g[t] & 3;
    int64_t key = -1;
    if (f < tf.nfields[grp]) {
      const int64_t id = ids[i];
      if (id >= 0 && id < (int64_t(1) << 40)) key = ((int64_t)tf.table[grp][f] << 40) | id;
    }
    keys[i] = key;
  }
}

// One 16-lane team per token: the token's sorted row and its F_g * e features, 16 bytes a lane.
__global__ __launch_bounds__(256) void k_tok_build(int64_t T, int32_t B, int fmax, int e,
                                                   const int64_t* __restrict__ offsets, const uint8_t* __restrict__ g,
                                                   const int64_t* __restrict__ cnt, const int64_t* __restrict__ goff,
                                                   TokGroups tg, const int64_t* __restrict__ inverse,
                                                   const bf16* __restrict__ uvals, int64_t* __restrict__ pos,
                                                   int32_t* __restrict__ rowmap, int32_t* __restrict__ flags) {
  const int lane16 = threadIdx.x & 15;
  const int64_t team = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int64_t teams = ((int64_t)gridDim.x * blockDim.x) >> 4;
  const int cpf = e * 2 / 16;                           // 16-byte chunks per field
  for (int64_t t = team; t < T; t += teams) {
    int lo = 0, hi = B;                                 // user of token t: last b with offsets[b] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= t) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int grp = g[t] & 3;
    int64_t first = offsets[b];
    for (int gi = 0; gi < grp; ++gi) first += cnt[(int64_t)b * 4 + gi];
    const int64_t p = goff[(int64_t)grp * (B + 1) + b] + (t - first);
    if (p < 0 || p >= tg.rows[grp]) {                  // sizes inconsistent with the host's
      if (lane16 == 0) { pos[t] = -1; atomicOr(flags, 1); }
      continue;
    }
    if (lane16 == 0) {
      pos[t] = tg.row0[grp] + p;
      if (rowmap) rowmap[tg.row0[grp] + p] = (int32_t)t;
    }
    const int nf = tg.nfields[grp];
    bf16* dst = tg.feat[grp] + p * (int64_t)(nf * e);
    for (int c = lane16; c < nf * cpf; c += 16) {
      const int f = c / cpf, w = c - f * cpf;
      const int64_t u = inverse[t * fmax + f];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (u >= 0) v = *reinterpret_cast<const uint4*>(uvals + u * e + w * 8);
      *reinterpret_cast<uint4*>(dst + f * e + w * 8) = v;
    }
  }
}

__global__ __launch_bounds__(256) void k_tok_scatter(int64_t T, int d, const int64_t* __restrict__ pos,
                                                     const float* __restrict__ y, float* __restrict__ x) {
  const int cpr = d / 4;
  const int64_t n = T * cpr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / cpr;
    const int c = (int)(i - t * cpr);
    const int64_t p = pos[t];
    const float4 v = p >= 0 ? *reinterpret_cast<const float4*>(y + p * d + c * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(x + t * d + c * 4) = v;
  }
}

__global__ void k_flags_reset(int32_t* flags) { *flags = 0; }

__global__ __launch_bounds__(256) void k_fill_i32(int64_t n, int32_t v, int32_t* __restrict__ p) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// x[t] = 0 for every token that has no sorted row (pos[t] < 0)
__global__ __launch_bounds__(256) void k_tok_zero_unplaced(int64_t T, int d, const int64_t* __restrict__ pos,
                                                           float* __restrict__ x) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T; t += (int64_t)gridDim.x * blockDim.x)
    if (pos[t] < 0)
      for (int c = 0; c < d; c += 4) *reinterpret_cast<float4*>(x + t * d + c) = make_float4(0.f, 0.f, 0.f, 0.f);
}

inline unsigned ew(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536)); }

}  // namespace

hipError_t launch_tok_prepare(int32_t B, int64_t T, int fmax, const int64_t* offsets, const uint8_t* group_ids,
                              const int64_t* ids, const TokFields& tf, int64_t* cnt, int64_t* goff, int64_t* keys,
                              int32_t* flags, hipStream_t s) {
  k_flags_reset<<<1, 1, 0, s>>>(flags);
  if (B > 0) {
    k_tok_users<<<(B + 255) / 256, 256, 0, s>>>(B, offsets, group_ids, cnt);
    k_tok_scan<<<1, 1024, 0, s>>>(B, cnt, goff);
  }
  if (T > 0) k_tok_keys<<<ew(T * fmax), 256, 0, s>>>(T, fmax, ids, group_ids, tf, keys);
  return hipGetLastError();
}

hipError_t launch_tok_build(int64_t T, int32_t B, int fmax, int e, const int64_t* offsets, const uint8_t* group_ids,
                            const int64_t* cnt, const int64_t* goff, const TokGroups& tg, const int64_t* inverse,
                            const bf16* uvals, int64_t* pos, int32_t* rowmap, int32_t* flags, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((T * 16 + 255) / 256, 65536);
  if (rowmap) {
    k_fill_i32<<<ew(T), 256, 0, s>>>(T, -1, rowmap);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  k_tok_build<<<(unsigned)blocks, 256, 0, s>>>(T, B, fmax, e, offsets, group_ids, cnt, goff, tg, inverse, uvals,
                                               pos, rowmap, flags);
  return hipGetLastError();
}

hipError_t launch_tok_zero_unplaced(int64_t T, int d, const int64_t* pos, float* x, hipStream_t s) {
  if (T == 0) return hipSuccess;
  k_tok_zero_unplaced<<<ew(T), 256, 0, s>>>(T, d, pos, x);
  return hipGetLastError();
}

hipError_t launch_tok_scatter(int64_t T, int d, const int64_t* pos, const float* y, float* x, hipStream_t s) {
  if (T == 0) return hipSuccess;
  k_tok_scatter<<<ew(T * (d / 4)), 256, 0, s>>>(T, d, pos, y, x);
  return hipGetLastError();
}

}  // namespace mtgr
