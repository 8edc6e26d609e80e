// Fused jagged masked-SiLU attention with the U gate, on gfx950.
//
// Per user b and head h (marovi.ai MTGR page, 方法, the V~ update equation, read token-wise):
//     y_i = u_i (.) (1/n_b) * sum_j M[i,j] * silu(q_i . k_j) * v_j
// with M the three-rule dynamic mask (fun-rec "MTGR: Hybrid Paradigm Modeling" 7.3.4) and n_b
// the user's total token count.  No softmax, no 1/sqrt(d_h), no running max.  Users never
// attend to each other (sequence packing, chenhuiyu blog "MTGR", training-system section).
//
// Work item = (user, head, 128-row q-tile); one 256-thread workgroup (4 wavefronts x 32 query
// rows).  Work items are ordered longest user first (LPT) by the prep kernels.
//
// Key range of a work item.  Tokens are ordered U, S, R, C.  Static keys [0, n_static) are
// visible to every row; R keys [n_static, rc_end) only to R/C rows, by timestamp; C keys only
// to themselves.  So a q-tile of static rows loops over [0, n_static) only, a tile with R/C rows
// over [0, rc_end); candidate keys never enter the MFMA loop (the candidate-candidate block is
// empty except its diagonal) and each candidate row's own term silu(q_i.k_i) v_i is added in
// the epilogue.  Key tiles that lie wholly inside the static range take no mask at all.  A
// wavefront skips a tile of pure R keys when none of them is earlier than its latest R/C row
// and the tile does not hold one of its own rows (the diagonal) -- correct for any R order.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, fp32 accumulate).  Scores are computed transposed,
// S^T = K Q^T (A = 32 keys x 16 features from LDS, B = this wavefront's Q fragments, held in
// registers for the whole work item), so that the accumulator of one lane holds one query and
// 16 keys.  After silu and masking those values are rounded to bf16 and used directly as the A
// operand of O = P V; V is stored transposed in LDS (feature-major, keys permuted so the 8 keys
// a lane needs are contiguous), and the B fragment is one 16-byte LDS read.
//
// LDS per workgroup: K 2 x 64 x (d_h+8) and V^T 2 x d_h x 72 bf16 (double-buffered,
// register-staged global->LDS copies), ~71 KB at d_h = 128, two workgroups per CU.
#include "kernels.h"

namespace mtgr {

namespace {

constexpr int BQ = kAttnQTileBf16;  // 128 query rows per work item
constexpr int BKV = 64;             // keys per tile

// Position of key k (0..63) of a tile inside a transposed V row: keys are grouped so that the
// 8 keys feeding slot 0..7 of lane-half hh in PV k-step ks sit at ks*16 + hh*8 + slot.
__device__ __forceinline__ int vt_pos(int k) {
  const int mt = k >> 5, G = (k >> 3) & 3, hk = (k >> 2) & 1, c = k & 3;
  return mt * 32 + (G >> 1) * 16 + hk * 8 + (G & 1) * 4 + c;
}

__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ int find_slot(const int32_t* __restrict__ tile_off, int B, int item) {
  int lo = 0, hi = B;  // largest p with tile_off[p] <= item
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

template <int DH>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(
    int32_t B, int d, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
    const int32_t* __restrict__ order, const int32_t* __restrict__ tile_off,
    const float* __restrict__ ts, const bf16* __restrict__ qkvu, bf16* __restrict__ y) {
  constexpr int KP = DH + 8;
  constexpr int VP = BKV + 8;
  constexpr int DCH = DH / 8;                    // 16-byte chunks per key row
  constexpr int CK = BKV * DCH / 256;            // K chunks per thread
  constexpr int VG = (BKV / 4) * DCH;            // V groups (4 keys x 8 features)
  constexpr int CV = (VG + 255) / 256;           // V groups per thread
  constexpr int NT = DH / 32;                    // output tiles of 32 features
  static_assert(CK * 256 == BKV * DCH, "K staging mismatch");

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BKV][KP];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][DH][VP];
  __shared__ __attribute__((aligned(16))) float Ts[2][BKV];

  const int item = blockIdx.x;
  const int h = blockIdx.y;
  const int slot = find_slot(tile_off, B, item);
  const int b = order[slot];
  const int qt = item - tile_off[slot];
  const int64_t base = offsets[b];
  const int n = (int)(offsets[b + 1] - base);
  const UserSeg sg = seg[b];
  const int ns = sg.n_u + sg.n_s;
  const int rc_end = ns + sg.n_r;
  const int q0 = qt * BQ;
  const int64_t ld = 4 * (int64_t)d;
  const bf16* Qp = qkvu + base * ld + (int64_t)h * DH;
  const bf16* Kp = Qp + d;
  const bf16* Vp = Qp + 2 * d;
  const bf16* Up = Qp + 3 * d;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wq0 = q0 + w * 32;
  const int qi = wq0 + l32;
  const bool q_valid = qi < n;
  const bf16x8 zero8 = {};

  bf16x8 qf[DH / 16];
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks)
    qf[ks] = q_valid ? *reinterpret_cast<const bf16x8*>(Qp + qi * ld + ks * 16 + hh * 8) : zero8;
  const bool q_rc = q_valid && qi >= ns;
  const float tq = q_rc ? ts[base + qi] : -INFINITY;

  const bool wave_rows = wq0 < n;
  const bool wave_rc = wave_rows && (wq0 + 32 > ns);
  const float wave_tmax = wave_max(tq);
  const int wr_lo = max(wq0, ns), wr_hi = min(min(wq0 + 32, rc_end), n);  // wavefront's R rows

  const bool blk_rc = (q0 + BQ > ns);
  const int kend = blk_rc ? rc_end : ns;
  const int nkt = (kend + BKV - 1) / BKV;

  f32x16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;

  bf16x8 rk[CK];
  bf16x8 rv[CV][4];
  float rt = INFINITY;

  auto stage_load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int idx = tid + i * 256;
      const int key = idx / DCH, c = idx % DCH;
      const int j = k0 + key;
      rk[i] = (j < kend) ? *reinterpret_cast<const bf16x8*>(Kp + j * ld + c * 8) : zero8;
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int idx = tid + i * 256;
      if (idx < VG) {
        const int kg = idx / DCH, c = idx % DCH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = k0 + kg * 4 + r;
          rv[i][r] = (j < kend) ? *reinterpret_cast<const bf16x8*>(Vp + j * ld + c * 8) : zero8;
        }
      }
    }
    if (tid < BKV) rt = (k0 + tid < kend) ? ts[base + k0 + tid] : INFINITY;
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int idx = tid + i * 256;
      const int key = idx / DCH, c = idx % DCH;
      *reinterpret_cast<bf16x8*>(&Ks[buf][key][c * 8]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int idx = tid + i * 256;
      if (idx < VG) {
        const int kg = idx / DCH, c = idx % DCH;
        const int p = vt_pos(kg * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16x4 v4;
          v4[0] = rv[i][0][e];
          v4[1] = rv[i][1][e];
          v4[2] = rv[i][2][e];
          v4[3] = rv[i][3][e];
          *reinterpret_cast<bf16x4*>(&Vt[buf][c * 8 + e][p]) = v4;
        }
      }
    }
    if (tid < BKV) Ts[buf][tid] = rt;
  };

  auto compute = [&](int buf, int k0) {
    const bool tile_static = (k0 + BKV <= ns);
    bool need = wave_rows && (k0 < ns || (wave_rc && k0 < rc_end));
    if (need && k0 >= ns) {
      // pure R tile: skip when no key is earlier than the wavefront's latest R/C row and the
      // wavefront's own R rows (the diagonal) are not in it
      const int j = k0 + lane;
      const float tk = (j < kend) ? Ts[buf][lane] : INFINITY;
      const float tmin = wave_min(tk);
      const bool diag = max(wr_lo, k0) < min(wr_hi, k0 + BKV);
      if (!diag && tmin >= wave_tmax) need = false;
    }
    if (!need) return;
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[buf][mt * 32 + l32][ks * 16 + hh * 8]);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[mt], 0, 0, 0);
      }
    }
    // s[mt][r]: key k0 + mt*32 + 8*(r/4) + 4*hh + r%4, query qi
    bf16x8 pa[4];
    if (tile_static) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pa[mt * 2 + (r >> 3)][r & 7] = (bf16)silu_fast(s[mt][r]);
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int kb = mt * 32 + 8 * g4 + 4 * hh;
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(&Ts[buf][kb]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = g4 * 4 + c;
            const int j = k0 + kb + c;
            const bool vis = (j < kend) && mtgr_visible(qi, j, ns, rc_end, tq, t4[c]);
            pa[mt * 2 + (r >> 3)][r & 7] = (bf16)(vis ? silu_fast(s[mt][r]) : 0.f);
          }
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&Vt[buf][t * 32 + l32][ks * 16 + hh * 8]);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], vf, o[t], 0, 0, 0);
      }
    }
  };

  stage_load(0);
  stage_store(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) stage_load((kt + 1) * BKV);
    compute(cur, kt * BKV);
    if (kt + 1 < nkt) stage_store(cur ^ 1);
    __syncthreads();
  }

  if (!wave_rows) return;

  // Candidate rows: their own term silu(q_i . k_i) v_i (the diagonal of the C block).
  const bool q_c = q_valid && qi >= rc_end;
  float part = 0.f;
  if (q_c) {
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Kp + qi * ld + ks * 16 + hh * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) part += (float)qf[ks][e] * (float)kf[e];
    }
  }
  const float s_self = part + __shfl_xor(part, 32, kWave);
  const float p_self = q_c ? (float)(bf16)silu_fast(s_self) : 0.f;
  const float inv_n = 1.0f / (float)n;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ql = 8 * (r >> 2) + 4 * hh + (r & 3);  // wavefront-local query of element r
    const int q = wq0 + ql;
    const float pw = __shfl(p_self, ql, kWave);
    if (q < n) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int f = t * 32 + l32;
        float acc = o[t][r];
        if (pw != 0.f) acc += pw * (float)Vp[q * ld + f];
        const float u = (float)Up[q * ld + f];
        y[(base + q) * (int64_t)d + (int64_t)h * DH + f] = (bf16)(acc * inv_n * u);
      }
    }
  }
}

// fp32 storage mode: the same rule set evaluated directly over every key of the user, one
// thread per query row, for exact comparison with the oracle.
template <int DH>
__global__ __launch_bounds__(64) void k_attn_f32(
    int32_t B, int d, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
    const int32_t* __restrict__ order, const int32_t* __restrict__ tile_off,
    const float* __restrict__ ts, const float* __restrict__ qkvu, float* __restrict__ y) {
  const int item = blockIdx.x;
  const int h = blockIdx.y;
  const int slot = find_slot(tile_off, B, item);
  const int b = order[slot];
  const int qt = item - tile_off[slot];
  const int64_t base = offsets[b];
  const int n = (int)(offsets[b + 1] - base);
  const UserSeg sg = seg[b];
  const int ns = sg.n_u + sg.n_s;
  const int rc_end = ns + sg.n_r;
  const int i = qt * kAttnQTileF32 + threadIdx.x;
  if (i >= n) return;
  const int64_t ld = 4 * (int64_t)d;
  const float* Qp = qkvu + base * ld + (int64_t)h * DH;
  const float* Kp = Qp + d;
  const float* Vp = Qp + 2 * d;
  const float* Up = Qp + 3 * d;
  float q[DH], acc[DH];
#pragma unroll
  for (int f = 0; f < DH; ++f) { q[f] = Qp[i * ld + f]; acc[f] = 0.f; }
  const float ti = ts[base + i];
  for (int j = 0; j < n; ++j) {
    if (!mtgr_visible(i, j, ns, rc_end, ti, ts[base + j])) continue;
    float s = 0.f;
#pragma unroll
    for (int f = 0; f < DH; ++f) s = fmaf(q[f], Kp[j * ld + f], s);
    const float p = silu_f32(s);
#pragma unroll
    for (int f = 0; f < DH; ++f) acc[f] = fmaf(p, Vp[j * ld + f], acc[f]);
  }
  const float inv_n = 1.0f / (float)n;
#pragma unroll
  for (int f = 0; f < DH; ++f)
    y[(base + i) * (int64_t)d + (int64_t)h * DH + f] = acc[f] * inv_n * Up[i * ld + f];
}

}  // namespace

hipError_t launch_attention_bf16(int32_t B, int64_t total_tiles, int d, int H,
                                 const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                 const int32_t* tile_off, const float* timestamps,
                                 const bf16* qkvu, bf16* y, hipStream_t s) {
  if (total_tiles == 0) return hipSuccess;
  const int dh = d / H;
  dim3 grid((unsigned)total_tiles, (unsigned)H);
  if (dh == 128)
    k_attn_bf16<128><<<grid, 256, 0, s>>>(B, d, offsets, seg, order, tile_off, timestamps, qkvu, y);
  else if (dh == 64)
    k_attn_bf16<64><<<grid, 256, 0, s>>>(B, d, offsets, seg, order, tile_off, timestamps, qkvu, y);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention_f32(int32_t B, int64_t total_tiles, int d, int H,
                                const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                const int32_t* tile_off, const float* timestamps,
                                const float* qkvu, float* y, hipStream_t s) {
  if (total_tiles == 0) return hipSuccess;
  const int dh = d / H;
  dim3 grid((unsigned)total_tiles, (unsigned)H);
  if (dh == 32)
    k_attn_f32<32><<<grid, 64, 0, s>>>(B, d, offsets, seg, order, tile_off, timestamps, qkvu, y);
  else if (dh == 64)
    k_attn_f32<64><<<grid, 64, 0, s>>>(B, d, offsets, seg, order, tile_off, timestamps, qkvu, y);
  else if (dh == 128)
    k_attn_f32<128><<<grid, 64, 0, s>>>(B, d, offsets, seg, order, tile_off, timestamps, qkvu, y);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mtgr
