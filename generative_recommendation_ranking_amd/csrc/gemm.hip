// Dense projections of the HSTU block on gfx950: the Q/K/V/U projection, the two MLP layers
// (with SiLU, and with the fp32 residual add), and the first layer of the candidate head
// (marovi.ai MTGR page, 方法, the block update equations).
//
//   out[M][N] = epi(a[M][K] . w[N][K]^T + bias[N])
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  A workgroup of 4 wavefronts owns
// a BM x BN output tile (2 x 2 wavefronts, each (BM/2) x (BN/2) = a grid of 32x32 MFMA tiles);
// the K loop stages BK-wide slabs of a and w through LDS (register-staged, double-buffered,
// rows padded by 16 bytes so the 16-byte fragment reads of 32 consecutive rows spread over the
// banks).  Both operands are K-contiguous, so every lane fetches its 8 consecutive k values of
// a fragment with one 16-byte LDS read.
//
// Workgroup order: MI355X dispatches consecutive workgroup ids round-robin to its 8 XCDs, each
// with a private L2.  Tiles are numbered so that every XCD walks its own M-tiles and, for each,
// all N-tiles back to back: each M-slab of `a` (the large, streamed operand) is then fetched
// from HBM into one L2 only, while the small weight matrix is shared through the MALL.
//
// fp32 path: a plain 64x64 register-tiled VALU kernel (used by the fp32 storage mode).
#include "../../include/mtgr.h"
#include "kernels.h"

namespace mtgr {

namespace {

constexpr int kXcd = 8;

template <int EPI, typename TOut>
__device__ __forceinline__ void store_out(TOut* out, const float* resid, int64_t idx, float v) {
  if constexpr (EPI == MTGR_EPI_SILU) {
    out[idx] = from_f32<TOut>(silu_f32(v));
  } else if constexpr (EPI == MTGR_EPI_RESIDUAL_F32) {
    out[idx] = from_f32<TOut>(v + resid[idx]);
  } else {
    out[idx] = from_f32<TOut>(v);
  }
}

template <int BM, int BN, int BK, int EPI, typename TOut>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16(int64_t M, int N, int K,
                                                      const bf16* __restrict__ A,
                                                      const bf16* __restrict__ W,
                                                      const bf16* __restrict__ bias,
                                                      const float* resid, TOut* out, int nN,
                                                      int64_t nM) {
  constexpr int NT = 256;
  constexpr int TM = BM / 2, TN = BN / 2;   // wavefront tile
  constexpr int FM = TM / 32, FN = TN / 32; // MFMA tiles per wavefront
  constexpr int LP = BK + 8;                // LDS row pitch (elements)
  constexpr int CPR = BK / 8;               // 16-byte chunks per slab row
  constexpr int CA = BM * CPR / NT;         // a chunks per thread
  constexpr int CB = BN * CPR / NT;         // w chunks per thread
  static_assert(CA * NT == BM * CPR && CB * NT == BN * CPR, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) bf16 As[2][BM][LP];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN][LP];

  // XCD-aware tile decode
  const int64_t bid = blockIdx.x;
  const int xcd = (int)(bid % kXcd);
  const int64_t slot = bid / kXcd;
  const int64_t m_tile = (slot / nN) * kXcd + xcd;
  const int n_tile = (int)(slot % nN);
  if (m_tile >= nM) return;
  const int64_t m0 = m_tile * BM;
  const int n0 = n_tile * BN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 ra[CA], rb[CB];
  const bf16x8 zero8 = {};

  auto load_slab = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / CPR, c = idx % CPR;
      const int64_t m = m0 + r;
      ra[i] = (m < M) ? *reinterpret_cast<const bf16x8*>(A + m * K + k0 + c * 8) : zero8;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / CPR, c = idx % CPR;
      const int n = n0 + r;
      rb[i] = (n < N) ? *reinterpret_cast<const bf16x8*>(W + (int64_t)n * K + k0 + c * 8) : zero8;
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / CPR, c = idx % CPR;
      *reinterpret_cast<bf16x8*>(&As[buf][r][c * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / CPR, c = idx % CPR;
      *reinterpret_cast<bf16x8*>(&Bs[buf][r][c * 8]) = rb[i];
    }
  };

  const int nk = K / BK;
  load_slab(0);
  store_slab(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_slab((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(&As[cur][wm * TM + i * 32 + l32][ks * 16 + hh * 8]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][wn * TN + j * 32 + l32][ks * 16 + hh * 8]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_slab(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element r of a 32x32 tile sits at row 8*(r/4) + 4*(lane/32) + r%4,
  // column lane%32.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * TN + j * 32 + l32;
    if (n >= N) continue;
    const float bv = bias ? (float)bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (m < M) store_out<EPI, TOut>(out, resid, m * N + n, acc[i][j][r] + bv);
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(int64_t M, int N, int K,
                                                  const float* __restrict__ A,
                                                  const float* __restrict__ W,
                                                  const float* __restrict__ bias,
                                                  const float* resid, float* out) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Ws[BK][BN + 4];
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    {
      const int r = tid / 4, c4 = (tid % 4) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = k0 + c4 + e;
        const int64_t m = m0 + r;
        const int n = n0 + r;
        As[c4 + e][r] = (m < M && k < K) ? A[m * K + k] : 0.f;
        Ws[c4 + e][r] = (n < N && k < K) ? W[(int64_t)n * K + k] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[k][ty * 4 + i]; w[i] = Ws[k][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float bv = bias ? bias[n] : 0.f;
      store_out<EPI, float>(out, resid, m * N + n, acc[i][j] + bv);
    }
  }
}

template <int BM, int BN, int EPI, typename TOut>
hipError_t run_bf16(int64_t M, int N, int K, const bf16* a, const bf16* w, const bf16* bias,
                    const float* resid, void* out, hipStream_t s) {
  constexpr int BK = 64;
  const int nN = (N + BN - 1) / BN;
  const int64_t nM = (M + BM - 1) / BM;
  const int64_t nMpad = (nM + kXcd - 1) / kXcd * kXcd;
  const int64_t blocks = nMpad * nN;
  k_gemm_bf16<BM, BN, BK, EPI, TOut><<<(unsigned)blocks, 256, 0, s>>>(
      M, N, K, a, w, bias, resid, static_cast<TOut*>(out), nN, nM);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(int64_t M, int N, int K, int epi, const bf16* a, const bf16* w,
                            const bf16* bias, const float* resid, void* out, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (epi) {
    case MTGR_EPI_STORE: return run_bf16<128, 128, MTGR_EPI_STORE, bf16>(M, N, K, a, w, bias, resid, out, s);
    case MTGR_EPI_SILU: return run_bf16<128, 128, MTGR_EPI_SILU, bf16>(M, N, K, a, w, bias, resid, out, s);
    case MTGR_EPI_RESIDUAL_F32:
      return run_bf16<128, 128, MTGR_EPI_RESIDUAL_F32, float>(M, N, K, a, w, bias, resid, out, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_f32(int64_t M, int N, int K, int epi, const float* a, const float* w,
                           const float* bias, const float* resid, float* out, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64));
  switch (epi) {
    case MTGR_EPI_STORE: k_gemm_f32<MTGR_EPI_STORE><<<grid, 256, 0, s>>>(M, N, K, a, w, bias, resid, out); break;
    case MTGR_EPI_SILU: k_gemm_f32<MTGR_EPI_SILU><<<grid, 256, 0, s>>>(M, N, K, a, w, bias, resid, out); break;
    case MTGR_EPI_RESIDUAL_F32:
      k_gemm_f32<MTGR_EPI_RESIDUAL_F32><<<grid, 256, 0, s>>>(M, N, K, a, w, bias, resid, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mtgr
