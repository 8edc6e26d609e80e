// Backward pass of one HSTU block on gfx950: the pieces that are not GEMMs (the GEMMs reuse the
// MFMA kernels of gemm.hip on transposed copies).  The block's update equations (marovi.ai MTGR
// page, 方法) differentiated by the chain rule:
//   MLP:        dH = dX' W2, dA = dH (.) silu'(A), dZ = dA W1         (A = Z W1^T + b1)
//   GroupLN:    dx = (dxh - mean(dxh) - xh mean(dxh (.) xh)) / s,  dxh = dz (.) gamma[g]
//   gate:       dV~ = dY (.) U,  dU = dY (.) V~
//   attention:  dS = M/N (.) silu'(S) (.) (dV~ V^T),  dQ = dS K,  dK = dS^T Q,  dV = (M/N (.) silu(S))^T dV~
// Parameter gradients are sums over tokens; every reduction here is deterministic (fixed
// partial-sum layout, fixed summation order).
#include <algorithm>

#include "kernels.h"

namespace mtgr {

namespace {

template <typename T>
__device__ __forceinline__ T cvt(float v) { return from_f32<T>(v); }

// ---- transposes -----------------------------------------------------------------------------
// dst[c][r] = src[r][c] for r < R, c < C; dst[c][r] = 0 for R <= r < Rp; with ones_row, an extra row dst[C][r] = (r < R) and rows C+1 .. C+7 zero.  dst
// row pitch Rp.  64 x 64 tiles through LDS.  The bf16 variant moves 16-byte row pieces (C and Rp
// multiples of 8): each thread reads 8 consecutive columns of one source row and writes 8
// consecutive rows of one destination row.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(int64_t R, int C, int64_t Rp, int ones_row,
                                                   const T* __restrict__ src, T* __restrict__ dst) {
  __shared__ float tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int crows = C + (ones_row ? 8 : 0);
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i;
    const int c = c0 + tx;
    float v = 0.f;
    if (r < R) {
      if (c < C) v = to_f32(src[r * C + c]);
      else if (ones_row && c == C) v = 1.f;
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i;
    const int64_t r = r0 + tx;
    if (c < crows && r < Rp) dst[(int64_t)c * Rp + r] = cvt<T>(tile[tx][i]);
  }
}

__global__ __launch_bounds__(256) void k_transpose_bf16x8(int64_t R, int C, int64_t Rp, int ones_row,
                                                          const bf16* __restrict__ src, bf16* __restrict__ dst) {
  __shared__ float tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  const int crows = C + (ones_row ? 8 : 0);
  // load: 64 rows x 8 chunks of 8 columns; thread -> (row lr, chunk lc), two rows per thread
  const int lc = threadIdx.x & 7, lr = threadIdx.x >> 3;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lr + 32 * k;
    const int64_t r = r0 + i;
    const int c = c0 + lc * 8;
    float v[8];
    if (r < R && c < C) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(src + r * C + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (r < R && ones_row && c + e == C) ? 1.f : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[i][lc * 8 + e] = v[e];
  }
  __syncthreads();
  // store: 64 destination rows (source columns) x 8 chunks of 8 source rows
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lr + 32 * k;      // destination row c0 + i
    const int c = c0 + i;
    const int64_t r = r0 + lc * 8;
    if (c < crows && r < Rp) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)tile[lc * 8 + e][i];
      *reinterpret_cast<bf16x8*>(dst + (int64_t)c * Rp + r) = o;
    }
  }
}

// ---- elementwise ----------------------------------------------------------------------------
// dh <- dh (.) silu'(a), silu'(z) = sigma(z) (1 + z (1 - sigma(z))), and a <- silu(a) = z sigma(z),
// the hidden activation that the weight gradient of the MLP's second layer reads; bf16: 8 elements
// per step
__global__ __launch_bounds__(256) void k_silu_bwd_bf16x8(int64_t n8, bf16* __restrict__ a, bf16* __restrict__ dh) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    bf16x8 z = *reinterpret_cast<const bf16x8*>(a + i * 8);
    bf16x8 g = *reinterpret_cast<const bf16x8*>(dh + i * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float zf = (float)z[e];
      const float sg = 1.0f / (1.0f + __expf(-zf));
      g[e] = (bf16)((float)g[e] * (sg * (1.0f + zf * (1.0f - sg))));
      z[e] = (bf16)(zf * sg);
    }
    *reinterpret_cast<bf16x8*>(dh + i * 8) = g;
    *reinterpret_cast<bf16x8*>(a + i * 8) = z;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_silu_bwd(int64_t n, T* __restrict__ a, T* __restrict__ dh) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float z = to_f32(a[i]);
    const float sg = 1.0f / (1.0f + __expf(-z));
    dh[i] = cvt<T>(to_f32(dh[i]) * sg * (1.0f + z * (1.0f - sg)));
    a[i] = cvt<T>(z * sg);
  }
}

// ---- column sums (bias gradients) ---------------------------------------------------------------
// Block (rb, cg) sums rows [rb * rpb, +rpb) of the 512 columns cg*512 .. +511: its 4 wavefronts take
// every 4th row each (one 16-byte chunk of 8 columns per lane, so a wavefront reads 1 KB of a row at
// once), then the 4 wavefront sums are added in wavefront order and written to part[rb][cols].
__global__ __launch_bounds__(256) void k_colsum_bf16(int64_t T, int M, int64_t rpb, const bf16* __restrict__ src,
                                                     float* __restrict__ part) {
  __shared__ float accw[4][512];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c0 = blockIdx.y * 512 + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.x * rpb, r1 = min(T, r0 + rpb);
  float acc[8] = {};
  if (c0 < M) {
    int64_t r = r0 + w;
    for (; r + 12 < r1; r += 16) {
      bf16x8 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const bf16x8*>(src + (r + 4 * u) * M + c0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)v[u][e];
    }
    for (; r < r1; r += 4) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + r * M + c0);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) accw[w][lane * 8 + e] = acc[e];
  __syncthreads();
  for (int c = threadIdx.x; c < 512; c += 256) {
    const int col = blockIdx.y * 512 + c;
    if (col < M) part[(int64_t)blockIdx.x * M + col] = ((accw[0][c] + accw[1][c]) + accw[2][c]) + accw[3][c];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_convert(int64_t n, const float* __restrict__ x, T* __restrict__ y) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    y[i] = cvt<T>(x[i]);
}

// ---- partial-sum reduction ------------------------------------------------------------------
// out[i] = sum_s part[s * stride + i] (i < n).  A block takes 64 columns; its 16 wavefronts sum the
// slots s = w, w + 16, ... in increasing order, and the 16 partial sums are added in wavefront
// order: a fixed summation order, so the result does not depend on scheduling.
constexpr int kReduceWaves = 16;
__global__ __launch_bounds__(64 * kReduceWaves) void k_reduce(int64_t n, int nsplit, int64_t stride,
                                                             const float* __restrict__ part, float* __restrict__ out) {
  __shared__ float accw[kReduceWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + lane;
  float acc = 0.f;
  if (i < n) {
#pragma unroll 8
    for (int s = w; s < nsplit; s += kReduceWaves) acc += part[s * stride + i];
  }
  accw[w][lane] = acc;
  __syncthreads();
  if (w == 0 && i < n) {
    float t = accw[0][lane];
#pragma unroll
    for (int k = 1; k < kReduceWaves; ++k) t += accw[k][lane];
    out[i] = t;
  }
}

// Sum the nsplit split-K partials of a weight gradient [M][Kx] into dW [M][K] and, when db is not
// NULL, db [M] = column K (Kx > K: the bias gradient, from the ones row appended to the transposed
// activations of the fp32 path), partials added in split order.
__global__ __launch_bounds__(256) void k_reduce_wb(int M, int K, int Kx, int nsplit, const float* __restrict__ part,
                                                   float* __restrict__ dw, float* __restrict__ db) {
  const int64_t n = (int64_t)M * (K + 1);
  const int64_t stride = (int64_t)M * Kx;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / (K + 1), k = i % (K + 1);
    if (k == K && !db) continue;
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) acc += part[s * stride + m * Kx + k];
    if (k < K) dw[m * K + k] = acc;
    else db[m] = acc;
  }
}

// The split-K slices without a bias column (Kx == K, db absent) are nsplit contiguous arrays of
// M*K values: four consecutive values per thread, the slices added in split order (the same order,
// so the same sums, as k_reduce_wb), eight slices' loads issued before their adds.
__global__ __launch_bounds__(256) void k_reduce_wb4(int64_t n4, int nsplit, int64_t stride4,
                                                    const f32x4* __restrict__ part, f32x4* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int sp = 0;
  for (; sp + 8 <= nsplit; sp += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(part + (int64_t)(sp + u) * stride4 + i);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[u][e];
  }
  for (; sp < nsplit; ++sp) {
    const f32x4 v = __builtin_nontemporal_load(part + (int64_t)sp * stride4 + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  dw[i] = acc;
}

// ---- GroupLN backward -------------------------------------------------------------------------
// One wavefront per token row, as in the forward; each wavefront takes a contiguous run of rows.
// dx = (dxh - mean(dxh) - xh mean(dxh xh)) / s; with resid, dx += resid (the residual path of the
// block input; dx may alias resid).  Parameter gradients: a wavefront sums dz (.) xh and dz for the
// current group in registers and adds them into its own slot [2][4][d] of `part` whenever the group
// changes (tokens come in group runs); only that wavefront touches the slot, in program order, and
// k_reduce sums the slots in a fixed order, so the result is deterministic.
// 8 consecutive values (16-byte aligned bf16, 32-byte aligned fp32) as one or two vector accesses
__device__ __forceinline__ void ld8(const bf16* p, float (&o)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
__device__ __forceinline__ void ld8(const float* p, float (&o)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[i + 4] = b[i]; }
}
__device__ __forceinline__ void st8(bf16* p, const float (&v)[8]) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ void st8(float* p, const float (&v)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[i + 4]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// PF: prefetch row+1 while row is reduced (wide fp32 rows); without it a wavefront holds one row
// and needs fewer registers, so more wavefronts share a SIMD (the bf16 variant).
template <typename Tx, typename Tdz, typename Tp, typename Tout, bool PF>
__global__ __launch_bounds__(256) void k_groupln_bwd(int64_t T, int d, int64_t rows_per_wave,
                                                     const Tx* __restrict__ x, const uint8_t* __restrict__ g,
                                                     const Tp* __restrict__ gamma, float eps, int gmask,
                                                     const Tdz* dz, const float* resid, Tout* dx,
                                                     float* __restrict__ part) {
  // the residual path exists for fp32-input rows only (GroupLN1); the bf16 variant takes none
  constexpr bool kResid = sizeof(Tx) == 4;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = d >> 3;
  float* slot = part + wave * 2 * 4 * d;            // [2][4][d]: dgamma, dbeta
  // each lane zeroes exactly the entries it later accumulates into (same thread, program order)
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch)
      for (int gi = 0; gi < 8; ++gi)
#pragma unroll
        for (int i = 0; i < 8; ++i) slot[gi * d + ch * 8 + i] = 0.f;
  }
  const int64_t r0 = wave * rows_per_wave;
  const int64_t r1 = min(T, r0 + rows_per_wave);
  float ag[2][8], ab[2][8];
  float gm[2][8];                                   // gamma of the current group, in registers
  int cur = -1;
  auto flush = [&]() {
    if (cur < 0) return;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          slot[cur * d + ch * 8 + i] += ag[c][i];
          slot[4 * d + cur * d + ch * 8 + i] += ab[c][i];
        }
    }
  };
  const float inv_d = 1.0f / (float)d;
  // With PF the loads of row+1 (x, dz and the residual) are issued before row is reduced, so a
  // wavefront always has a row in flight.  Nothing else is loaded per row: vector loads retire in
  // order, and a per-row gamma load issued after the prefetch would make every row wait for the
  // next one.  gamma is loaded when the group changes (tokens come in group runs).
  float v[2][8], dv[2][8], rs[2][8];
  float nv[2][8], ndv[2][8], nrs[2][8];
  auto load_row = [&](int64_t row, float (&a)[2][8], float (&b)[2][8], float (&c)[2][8]) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ch = lane + 64 * cc;
      if (ch < nch && row < r1) {
        ld8(x + row * d + ch * 8, a[cc]);
        ld8(dz + row * d + ch * 8, b[cc]);
        if (kResid && resid) {
          ld8(resid + row * d + ch * 8, c[cc]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) c[cc][i] = 0.f;
        }
      }
    }
  };
  if (PF && r0 < r1) load_row(r0, nv, ndv, nrs);
  for (int64_t row = r0; row < r1; ++row) {
    const int grp = g[row] & gmask;
    if constexpr (PF) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int i = 0; i < 8; ++i) { v[cc][i] = nv[cc][i]; dv[cc][i] = ndv[cc][i]; rs[cc][i] = nrs[cc][i]; }
    }
    if (grp != cur) {
      flush();
      cur = grp;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int ch = lane + 64 * cc;
        if (ch < nch) ld8(gamma + grp * d + ch * 8, gm[cc]);
#pragma unroll
        for (int i = 0; i < 8; ++i) { ag[cc][i] = 0.f; ab[cc][i] = 0.f; }
      }
    }
    if constexpr (PF) load_row(row + 1, nv, ndv, nrs);
    else load_row(row, v, dv, rs);
    float s1 = 0.f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
      if (lane + 64 * cc < nch)
#pragma unroll
        for (int i = 0; i < 8; ++i) s1 += v[cc][i];
    const float mean = wave_sum(s1) * inv_d;
    float q = 0.f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
      if (lane + 64 * cc < nch)
#pragma unroll
        for (int i = 0; i < 8; ++i) { const float e = v[cc][i] - mean; q += e * e; }
    const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_d + eps);
    float sa = 0.f, sb = 0.f;       // sum dxh, sum dxh * xh
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      if (lane + 64 * cc < nch) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xh = (v[cc][i] - mean) * rstd;
          const float dxh = dv[cc][i] * gm[cc][i];
          ag[cc][i] += dv[cc][i] * xh;
          ab[cc][i] += dv[cc][i];
          sa += dxh;
          sb += dxh * xh;
          v[cc][i] = xh;
          dv[cc][i] = dxh;
        }
      }
    }
    const float ma = wave_sum(sa) * inv_d, mb = wave_sum(sb) * inv_d;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ch = lane + 64 * cc;
      if (ch < nch) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (dv[cc][i] - ma - v[cc][i] * mb) * rstd + (kResid ? rs[cc][i] : 0.f);
        st8(dx + row * d + ch * 8, o);
      }
    }
  }
  flush();
}

// ---- masked SiLU attention backward (reference-style, one thread per row and head) ------------
// Query side: dQ_i = sum_j M_ij silu'(s_ij)/n (dv~_i . v_j) k_j, and dU_i = dy_i (.) v~_i.
// Key side:   dK_j = sum_i M_ij silu'(s_ij)/n (dv~_i . v_j) q_i, dV_j = sum_i M_ij silu(s_ij)/n dv~_i,
// with dv~_i = dy_i (.) u_i.  Work items: (user, q_tile-row tile) x head, one thread per row
// (blockDim.x = q_tile, the tiling of the prep's tile_off).
template <typename T, int DH>
__global__ __launch_bounds__(128) void k_attn_bwd_q(
    int32_t B, int d, int mode, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
    const int32_t* __restrict__ order, const int32_t* __restrict__ tile_off, const float* __restrict__ ts,
    const T* __restrict__ qkvu, const T* __restrict__ vt, const T* __restrict__ dy, T* __restrict__ dqkvu) {
  const int item = blockIdx.x, h = blockIdx.y;
  int lo = 0, hi = B;
  while (hi - lo > 1) { const int mid = (lo + hi) >> 1; if (tile_off[mid] <= item) lo = mid; else hi = mid; }
  const int b = order[lo];
  const int i = (item - tile_off[lo]) * (int)blockDim.x + threadIdx.x;
  const int64_t base = offsets[b];
  const int n = (int)(offsets[b + 1] - base);
  if (i >= n) return;
  const UserSeg sg = seg[b];
  const int ns = sg.n_u + sg.n_s, rc_end = ns + sg.n_r;
  const int64_t ld = 4 * (int64_t)d;
  const T* Qp = qkvu + base * ld + (int64_t)h * DH;
  const T* Kp = Qp + d;
  const T* Vp = Qp + 2 * d;
  const T* Up = Qp + 3 * d;
  const T* dYp = dy + base * (int64_t)d + (int64_t)h * DH;
  float q[DH], dvt[DH], acc[DH];
#pragma unroll
  for (int f = 0; f < DH; ++f) {
    q[f] = to_f32(Qp[i * ld + f]);
    dvt[f] = to_f32(dYp[i * (int64_t)d + f]) * to_f32(Up[i * ld + f]);
    acc[f] = 0.f;
  }
  const float inv_n = 1.0f / (float)n;
  const float ti = ts[base + i];
  for (int j = 0; j < n; ++j) {
    if (!mtgr_visible_mode(mode, i, j, ns, rc_end, ti, ts[base + j])) continue;
    float s = 0.f, da = 0.f;
#pragma unroll
    for (int f = 0; f < DH; ++f) {
      s = fmaf(q[f], to_f32(Kp[j * ld + f]), s);
      da = fmaf(dvt[f], to_f32(Vp[j * ld + f]), da);
    }
    const float sgm = 1.0f / (1.0f + __expf(-s));
    const float ds = da * sgm * (1.0f + s * (1.0f - sgm)) * inv_n;
#pragma unroll
    for (int f = 0; f < DH; ++f) acc[f] = fmaf(ds, to_f32(Kp[j * ld + f]), acc[f]);
  }
  T* dQ = dqkvu + (base + i) * ld + (int64_t)h * DH;
  T* dU = dQ + 3 * d;
  const T* Vt = vt + (base + i) * (int64_t)d + (int64_t)h * DH;
#pragma unroll
  for (int f = 0; f < DH; ++f) {
    dQ[f] = cvt<T>(acc[f]);
    dU[f] = cvt<T>(to_f32(dYp[i * (int64_t)d + f]) * to_f32(Vt[f]));
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(128) void k_attn_bwd_kv(
    int32_t B, int d, int mode, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
    const int32_t* __restrict__ order, const int32_t* __restrict__ tile_off, const float* __restrict__ ts,
    const T* __restrict__ qkvu, const T* __restrict__ dy, T* __restrict__ dqkvu) {
  const int item = blockIdx.x, h = blockIdx.y;
  int lo = 0, hi = B;
  while (hi - lo > 1) { const int mid = (lo + hi) >> 1; if (tile_off[mid] <= item) lo = mid; else hi = mid; }
  const int b = order[lo];
  const int j = (item - tile_off[lo]) * (int)blockDim.x + threadIdx.x;
  const int64_t base = offsets[b];
  const int n = (int)(offsets[b + 1] - base);
  if (j >= n) return;
  const UserSeg sg = seg[b];
  const int ns = sg.n_u + sg.n_s, rc_end = ns + sg.n_r;
  const int64_t ld = 4 * (int64_t)d;
  const T* Qp = qkvu + base * ld + (int64_t)h * DH;
  const T* Kp = Qp + d;
  const T* Vp = Qp + 2 * d;
  const T* Up = Qp + 3 * d;
  const T* dYp = dy + base * (int64_t)d + (int64_t)h * DH;
  float k[DH], v[DH], dk[DH], dv[DH];
#pragma unroll
  for (int f = 0; f < DH; ++f) {
    k[f] = to_f32(Kp[j * ld + f]);
    v[f] = to_f32(Vp[j * ld + f]);
    dk[f] = 0.f;
    dv[f] = 0.f;
  }
  const float inv_n = 1.0f / (float)n;
  const float tj = ts[base + j];
  for (int i = 0; i < n; ++i) {
    if (!mtgr_visible_mode(mode, i, j, ns, rc_end, ts[base + i], tj)) continue;
    float s = 0.f, da = 0.f;
#pragma unroll
    for (int f = 0; f < DH; ++f) {
      s = fmaf(to_f32(Qp[i * ld + f]), k[f], s);
      da = fmaf(to_f32(dYp[i * (int64_t)d + f]) * to_f32(Up[i * ld + f]), v[f], da);
    }
    const float sgm = 1.0f / (1.0f + __expf(-s));
    const float p = s * sgm * inv_n;
    const float ds = da * sgm * (1.0f + s * (1.0f - sgm)) * inv_n;
#pragma unroll
    for (int f = 0; f < DH; ++f) {
      dk[f] = fmaf(ds, to_f32(Qp[i * ld + f]), dk[f]);
      dv[f] = fmaf(p, to_f32(dYp[i * (int64_t)d + f]) * to_f32(Up[i * ld + f]), dv[f]);
    }
  }
  T* dK = dqkvu + (base + j) * ld + d + (int64_t)h * DH;
  T* dV = dK + d;
#pragma unroll
  for (int f = 0; f < DH; ++f) {
    dK[f] = cvt<T>(dk[f]);
    dV[f] = cvt<T>(dv[f]);
  }
}

// fp32 -> bf16 conversion of a [T][M] matrix fused with the column sums of the fp32 values, in the
// layout of k_colsum_bf16 (per-block partials, fixed-order reduction); part NULL: conversion only
__global__ __launch_bounds__(256) void k_convert_colsum(int64_t T, int M, int64_t rpb, const float* __restrict__ src,
                                                        bf16* __restrict__ dst, float* __restrict__ part) {
  __shared__ float accw[4][512];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c0 = blockIdx.y * 512 + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.x * rpb, r1 = min(T, r0 + rpb);
  float acc[8] = {};
  // one row: accumulate its 8 columns and store them rounded to bf16
  auto put = [&](int64_t r, const f32x4& a, const f32x4& b) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += a[e];
      acc[e + 4] += b[e];
      o[e] = (bf16)a[e];
      o[e + 4] = (bf16)b[e];
    }
    *reinterpret_cast<bf16x8*>(dst + r * M + c0) = o;
  };
  if (c0 < M) {
    // four rows' loads before their stores: vector memory operations retire in order, so a row's
    // loads issued after the previous row's store would wait for it.  The fp32 rows are read once
    // (non-temporal); the bf16 copy is read again by the weight-gradient GEMMs.
    int64_t r = r0 + w;
    for (; r + 12 < r1; r += 16) {
      f32x4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (r + 4 * u) * M + c0));
        b[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (r + 4 * u) * M + c0 + 4));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) put(r + 4 * u, a[u], b[u]);
    }
    for (; r < r1; r += 4)
      put(r, __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + r * M + c0)),
          __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + r * M + c0 + 4)));
  }
  if (!part) return;                                   // block-uniform
#pragma unroll
  for (int e = 0; e < 8; ++e) accw[w][lane * 8 + e] = acc[e];
  __syncthreads();
  for (int c = threadIdx.x; c < 512; c += 256) {
    const int col = blockIdx.y * 512 + c;
    if (col < M) part[(int64_t)blockIdx.x * M + col] = ((accw[0][c] + accw[1][c]) + accw[2][c]) + accw[3][c];
  }
}

inline unsigned ew_grid(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 16384); }

}  // namespace

hipError_t launch_transpose(int64_t R, int C, int64_t Rp, int ones_row, int kind, const void* src,
                            void* dst, hipStream_t s) {
  if (R == 0 && Rp == 0) return hipSuccess;
  const int crows = C + (ones_row ? 8 : 0);
  dim3 grid((unsigned)((crows + 63) / 64), (unsigned)((Rp + 63) / 64));
  if (kind == 1 && C % 8 == 0 && Rp % 8 == 0)
    k_transpose_bf16x8<<<grid, 256, 0, s>>>(R, C, Rp, ones_row, static_cast<const bf16*>(src),
                                             static_cast<bf16*>(dst));
  else if (kind == 1)
    k_transpose<bf16><<<grid, 256, 0, s>>>(R, C, Rp, ones_row, static_cast<const bf16*>(src), static_cast<bf16*>(dst));
  else
    k_transpose<float><<<grid, 256, 0, s>>>(R, C, Rp, ones_row, static_cast<const float*>(src), static_cast<float*>(dst));
  return hipGetLastError();
}

hipError_t launch_silu_bwd(int64_t n, int kind, void* a, void* dh, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (kind == 1 && n % 8 == 0)
    k_silu_bwd_bf16x8<<<ew_grid(n / 8), 256, 0, s>>>(n / 8, static_cast<bf16*>(a), static_cast<bf16*>(dh));
  else if (kind == 1) k_silu_bwd<bf16><<<ew_grid(n), 256, 0, s>>>(n, static_cast<bf16*>(a), static_cast<bf16*>(dh));
  else k_silu_bwd<float><<<ew_grid(n), 256, 0, s>>>(n, static_cast<float*>(a), static_cast<float*>(dh));
  return hipGetLastError();
}

hipError_t launch_convert_colsum(int64_t T, int M, const float* src, bf16* dst, float* part, float* out,
                                hipStream_t s) {
  if (T == 0 || M == 0) return hipSuccess;
  if (M % 8 != 0) return hipErrorInvalidValue;
  const int nrb = colsum_blocks(T, M);
  const int64_t rpb = (T + nrb - 1) / nrb;
  k_convert_colsum<<<dim3((unsigned)nrb, (unsigned)((M + 511) / 512)), 256, 0, s>>>(T, M, rpb, src, dst,
                                                                                   out ? part : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !out) return e;
  return launch_reduce(M, nrb, M, part, out, s);
}

hipError_t launch_colsum_bf16(int64_t T, int M, const bf16* src, float* part, float* out, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (M % 8 != 0) return hipErrorInvalidValue;
  const int nrb = colsum_blocks(T, M);
  const int64_t rpb = (T + nrb - 1) / nrb;
  k_colsum_bf16<<<dim3((unsigned)nrb, (unsigned)((M + 511) / 512)), 256, 0, s>>>(T, M, rpb, src, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce(M, nrb, M, part, out, s);
}

hipError_t launch_convert(int64_t n, int kind, const float* x, void* y, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (kind == 1) k_convert<bf16><<<ew_grid(n), 256, 0, s>>>(n, x, static_cast<bf16*>(y));
  else k_convert<float><<<ew_grid(n), 256, 0, s>>>(n, x, static_cast<float*>(y));
  return hipGetLastError();
}

hipError_t launch_reduce(int64_t n, int nsplit, int64_t stride, const float* part, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  k_reduce<<<(unsigned)((n + 63) / 64), 64 * kReduceWaves, 0, s>>>(n, nsplit, stride, part, out);
  return hipGetLastError();
}

hipError_t launch_reduce_wb(int M, int K, int Kx, int nsplit, const float* part, float* dw, float* db,
                            hipStream_t s) {
  const int64_t n = (int64_t)M * (K + 1);
  if (M == 0) return hipSuccess;
  const int64_t mk = (int64_t)M * K;
  if (!db && Kx == K && mk % 4 == 0 && nsplit > 0 &&
      reinterpret_cast<uintptr_t>(part) % 16 == 0 && reinterpret_cast<uintptr_t>(dw) % 16 == 0) {
    const int64_t n4 = mk / 4;
    k_reduce_wb4<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(n4, nsplit, n4, reinterpret_cast<const f32x4*>(part),
                                                               reinterpret_cast<f32x4*>(dw));
    return hipGetLastError();
  }
  k_reduce_wb<<<ew_grid(n), 256, 0, s>>>(M, K, Kx, nsplit, part, dw, db);
  return hipGetLastError();
}

hipError_t launch_groupln_bwd(int64_t T, int d, int x_kind, int act_kind, int shared, const void* x,
                              const uint8_t* g, const void* gamma, float eps, const void* dz,
                              const float* resid, void* dx, int out_kind, float* part, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int waves = groupln_bwd_waves(T, x_kind);
  const int64_t rpw = (T + waves - 1) / waves;
  const unsigned grid = (unsigned)(waves / 4);
  const int gm = shared ? 0 : 3;
  // (x, dz, gamma, dx) types: GLN2 uses (act, act, act, act); GLN1 uses (float, act, act, float)
  if (x_kind == 0 && act_kind == 0 && out_kind == 0)
    k_groupln_bwd<float, float, float, float, true><<<grid, 256, 0, s>>>(
        T, d, rpw, static_cast<const float*>(x), g, static_cast<const float*>(gamma), eps, gm,
        static_cast<const float*>(dz), resid, static_cast<float*>(dx), part);
  else if (x_kind == 1 && act_kind == 1 && out_kind == 1 && !resid)
    k_groupln_bwd<bf16, bf16, bf16, bf16, false><<<grid, 256, 0, s>>>(
        T, d, rpw, static_cast<const bf16*>(x), g, static_cast<const bf16*>(gamma), eps, gm,
        static_cast<const bf16*>(dz), resid, static_cast<bf16*>(dx), part);
  else if (x_kind == 0 && act_kind == 1 && out_kind == 0)
    k_groupln_bwd<float, bf16, bf16, float, true><<<grid, 256, 0, s>>>(
        T, d, rpw, static_cast<const float*>(x), g, static_cast<const bf16*>(gamma), eps, gm,
        static_cast<const bf16*>(dz), resid, static_cast<float*>(dx), part);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention_bwd_ref(int32_t B, int64_t total_tiles, int q_tile, int d, int H, int mask_mode, int kind,
                                    const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                    const int32_t* tile_off, const float* timestamps, const void* qkvu,
                                    const void* vt, const void* dy, void* dqkvu, hipStream_t s) {
  if (total_tiles == 0) return hipSuccess;
  if (q_tile != 64 && q_tile != 128) return hipErrorInvalidValue;
  const int dh = d / H;
  dim3 grid((unsigned)total_tiles, (unsigned)H);
#define MTGR_BWD(TT, DHV)                                                                          \
  do {                                                                                             \
    k_attn_bwd_q<TT, DHV><<<grid, q_tile, 0, s>>>(B, d, mask_mode, offsets, seg, order, tile_off,      \
                                              timestamps, static_cast<const TT*>(qkvu),            \
                                              static_cast<const TT*>(vt), static_cast<const TT*>(dy), \
                                              static_cast<TT*>(dqkvu));                            \
    k_attn_bwd_kv<TT, DHV><<<grid, q_tile, 0, s>>>(B, d, mask_mode, offsets, seg, order, tile_off,     \
                                               timestamps, static_cast<const TT*>(qkvu),           \
                                               static_cast<const TT*>(dy), static_cast<TT*>(dqkvu)); \
  } while (0)
  if (kind == 1) {
    if (dh == 128) MTGR_BWD(bf16, 128);
    else if (dh == 64) MTGR_BWD(bf16, 64);
    else if (dh == 32) MTGR_BWD(bf16, 32);
    else return hipErrorInvalidValue;
  } else {
    if (dh == 128) MTGR_BWD(float, 128);
    else if (dh == 64) MTGR_BWD(float, 64);
    else if (dh == 32) MTGR_BWD(float, 32);
    else return hipErrorInvalidValue;
  }
#undef MTGR_BWD
  return hipGetLastError();
}

}  // namespace mtgr
