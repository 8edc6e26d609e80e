// Backward of the fused jagged masked-SiLU attention with the U gate, bf16 storage, on gfx950.
//
// Per user and head, with S = Q K^T, P = M (.) silu(S) / n (no softmax; n = the user's token
// count; marovi.ai MTGR page, 方法, the V~ update equation; M the dynamic mask of fun-rec
// "MTGR: Hybrid Paradigm Modeling" 7.3.4), V~ = P V and y = V~ (.) U, the chain rule gives,
// with G = dy (.) U the gradient w.r.t. V~:
//   dU = dy (.) V~,  dV = P^T G,  dS = M (.) silu'(S) (.) (G V^T) / n,  dK = dS^T Q,  dQ = dS K.
// Three launches and no atomics -- every output element is written by one work item, so the
// result is the same bit for bit on every run:
//   k_gate_bwd      G (bf16 [T][d], workspace) and dU, elementwise.
//   k_attn_bwd_dkv  work item = (user, head, 128 keys), 4 wavefronts x 32 keys.  The K and V rows
//                   of a wavefront's keys stay in registers while 64-query tiles of Q and G stream
//                   through LDS (LDS-direct buffer loads, no staging registers).  S and dP = G V^T are computed with the key as the MFMA column,
//                   so that each lane holds one key and 16 queries; P and dS, rounded to bf16, are
//                   then directly the A operands of dV += P^T G and dK += dS^T Q.
//   k_attn_bwd_dq   work item = (user, head, 128 queries), the forward kernel's tiling: Q and G
//                   rows in registers, 64-key tiles of K and V through LDS (LDS-direct loads);
//                   S^T and dP^T with the query as the column, then dQ += dS K.
// Both take their work items from the forward's per-XCD queues (the tile counts agree: 128 keys
// or 128 queries per item).  Ranges and skipping follow the mask as in the forward: under the
// dynamic mask a candidate key is visible only to itself, so candidate keys take no MFMA path at
// all and the diagonal term of a candidate token (its dQ, dK and dV share) is added in the
// epilogues.  An R-key wavefront skips a query tile that holds no later R/C query and none of
// its own rows.
//
// Every LDS tile (Q and G in dK/dV, K and V in dQ) has pitch d_h, with the 16-byte chunk c of row
// r stored at chunk position c ^ swz(r); swz keeps the 16-lane row reads and the 32-lane
// transposing reads (ds_read_b64_tr_b16) free of bank conflicts (64 banks of 4 bytes).  Tiles are
// filled by LDS-direct buffer loads: one wavefront instruction writes 1 KB, lane l the 16 bytes at
// l*16, so lane l fetches the source chunk that belongs at that swizzled position.
#include "kernels.h"

#include <type_traits>

namespace mtgr {

namespace {

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kTile = 128;   // keys (dkv) or queries (dq) per work item: 4 wavefronts x 32

template <int DH>
__device__ __forceinline__ int swz(int r) {
  static_assert(DH == 64 || DH == 128, "head width");
  if constexpr (DH == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
// element offset of (row r, feature f) in a swizzled [rows][DH] tile
template <int DH>
__device__ __forceinline__ int sw_off(int r, int f) {
  return r * DH + ((((f >> 3) ^ swz<DH>(r))) << 3) + (f & 7);
}

__device__ __forceinline__ int find_slot(const int32_t* __restrict__ off, int cnt, int item) {
  int lo = 0, hi = cnt;  // largest p with off[p] <= item
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

// Work item of this workgroup in the per-XCD queues the prep kernels build (see the forward):
// user b, head h, tile index within the user.  False when the queue is exhausted.
__device__ __forceinline__ bool decode_item(int32_t B, int H, const int32_t* __restrict__ order,
                                            const int32_t* __restrict__ xcd_off, int& b, int& h,
                                            int& tile) {
  const int xcd = (int)(blockIdx.x % kXcdCount);
  const int pos = (int)(blockIdx.x / kXcdCount);
  const int R = (int)(((int64_t)B * H + kXcdCount - 1) / kXcdCount);
  const int32_t* xo = xcd_off + (int64_t)xcd * (R + 1);
  if (pos >= xo[R]) return false;
  const int round = find_slot(xo, R, pos);
  const int64_t grp = (int64_t)round * kXcdCount + ((round & 1) ? (kXcdCount - 1 - xcd) : xcd);
  b = order[grp / H];
  h = (int)(grp % H);
  tile = pos - xo[round];
  return true;
}

// 16 bytes per lane from a buffer resource straight into LDS: lane l writes lds + 16 l
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ float sigmoid_rcp(float s) { return __builtin_amdgcn_rcpf(1.0f + __expf(-s)); }

// B operand of a k-step over 16 tokens from a swizzled tile: slot e of lane-half hh is token
// kb + 4*hh + e%4 (+8 for e >= 4), kb = (ks/2)*32 + (ks%2)*16, feature t*32 + lane%32 -- the
// token order in which a 32x32 accumulator holds its rows, so a rounded score tile is an A
// operand as it stands.  ds_read_b64_tr_b16 hands lane i of a 16-lane group element i%4 of the
// 4-element rows addressed by lanes i/4 + 4e.
template <int DH>
__device__ __forceinline__ bf16x8 tr_frag(const bf16* tile, int ks, int t, int lane) {
  const int hh = lane >> 5;
  const int kb = (ks >> 1) * 32 + (ks & 1) * 16 + 4 * hh + (lane & 15) / 4;
  const int fc = t * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + sw_off<DH>(kb, fc)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + sw_off<DH>(kb + 8, fc)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---- G and dU ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gate_bwd(int64_t T, int d, const bf16* __restrict__ qkvu,
                                                  const bf16* __restrict__ vt, const bf16* __restrict__ dy,
                                                  bf16* __restrict__ g, bf16* __restrict__ dqkvu) {
  const int cpr = d >> 3;
  const int64_t n = T * cpr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / cpr;
    const int c = (int)(i - t * cpr);
    // dy, U and V~ are read once here and dU written once: non-temporal; G is read again by the
    // dK/dV and dQ passes and goes through the caches
    const bf16x8 y8 = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(dy + t * d + c * 8));
    const bf16x8 u8 = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(qkvu + t * 4 * d + 3 * d + c * 8));
    const bf16x8 v8 = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(vt + t * d + c * 8));
    bf16x8 g8, du8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      g8[e] = (bf16)((float)y8[e] * (float)u8[e]);
      du8[e] = (bf16)((float)y8[e] * (float)v8[e]);
    }
    *reinterpret_cast<bf16x8*>(g + t * d + c * 8) = g8;
    __builtin_nontemporal_store(du8, reinterpret_cast<bf16x8*>(dqkvu + t * 4 * d + 3 * d + c * 8));
  }
}

// ---- dK, dV -------------------------------------------------------------------------------------
template <int DH, int MODE>
__global__ __launch_bounds__(256, 1) void k_attn_bwd_dkv(
    int32_t B, int H, int d, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
    const int32_t* __restrict__ order, const int32_t* __restrict__ xcd_off, const float* __restrict__ ts,
    const bf16* __restrict__ qkvu, const bf16* __restrict__ gq, bf16* __restrict__ dqkvu) {
  constexpr int BQ = 64;                 // queries per LDS tile
  constexpr int CPR = DH / 8;            // 16-byte chunks per row
  constexpr int NT = DH / 32;            // 32-feature output tiles
  constexpr int KS = DH / 16;            // feature k-steps
  constexpr int OP = DH + 4;             // fp32 pitch of staged output rows
  constexpr size_t kLoopBytes = 4 * BQ * DH * sizeof(bf16) + 2 * BQ * sizeof(float);
  constexpr size_t kEpiBytes = 4 * 32 * OP * sizeof(float) + 2 * 4 * 32 * sizeof(float);
  __shared__ __attribute__((aligned(16))) char arena[kLoopBytes > kEpiBytes ? kLoopBytes : kEpiBytes];
  bf16 (*Qs)[BQ * DH] = reinterpret_cast<bf16 (*)[BQ * DH]>(arena);
  bf16 (*Gs)[BQ * DH] = reinterpret_cast<bf16 (*)[BQ * DH]>(arena + 2 * BQ * DH * sizeof(bf16));
  float (*Tq)[BQ] = reinterpret_cast<float (*)[BQ]>(arena + 4 * BQ * DH * sizeof(bf16));

  int b, h, tile;
  if (!decode_item(B, H, order, xcd_off, b, h, tile)) return;
  const int64_t base = offsets[b];
  const int n = (int)(offsets[b + 1] - base);
  const UserSeg sg = seg[b];
  const int ns = sg.n_u + sg.n_s;
  const int rc_end = ns + sg.n_r;
  const int k0 = tile * kTile;
  const int64_t ld = 4 * (int64_t)d;
  const bf16* Qp = qkvu + base * ld + (int64_t)h * DH;
  const bf16* Kp = Qp + d;
  const bf16* Vp = Qp + 2 * d;
  const bf16* Gp = gq + base * (int64_t)d + (int64_t)h * DH;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wk0 = k0 + w * 32;
  const int kj = wk0 + l32;
  const int kmend = MODE == kMaskDynamic ? rc_end : n;   // keys that take the MFMA path
  const bool k_m = kj < kmend;
  const bf16x8 zero8 = {};
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = k_m ? *reinterpret_cast<const bf16x8*>(Kp + kj * ld + ks * 16 + hh * 8) : zero8;
    vf[ks] = k_m ? *reinterpret_cast<const bf16x8*>(Vp + kj * ld + ks * 16 + hh * 8) : zero8;
  }
  // real-time keys carry their timestamp; every other key +inf (never "earlier" than a query)
  const bool k_r = MODE == kMaskDynamic && k_m && kj >= ns;
  const float tk = k_r ? ts[base + kj] : INFINITY;
  const bool wave_keys = wk0 < kmend;
  const bool wave_static = MODE == kMaskDynamic && wk0 < ns;
  const float wave_tmin = wave_min(tk);
  const int wr_lo = max(wk0, ns), wr_hi = min(wk0 + 32, rc_end);   // the wavefront's R keys

  // queries that can see a key of this tile: every query (static keys, full mask), queries at or
  // after k0 (causal), R/C queries (R keys); none for a tile of candidate keys only
  int qlo = 0;
  if (MODE == kMaskCausal) qlo = k0;
  if (MODE == kMaskDynamic) qlo = k0 < ns ? 0 : ns;
  const int qhi = (MODE == kMaskDynamic && k0 >= rc_end) ? 0 : n;
  const int qt0 = qlo / BQ;
  const int nqt = qhi > qlo ? (qhi + BQ - 1) / BQ - qt0 : 0;

  // The accumulators start as the result of an MFMA on zeros rather than as zeros written by
  // VALU moves: both inputs of their loop-carried value then come from MFMAs, so the register
  // allocator keeps them in accumulation registers for the whole key loop instead of moving all
  // 128 through the general registers on every query tile.
  f32x16 dk[NT], dv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zero8, zero8, f32x16{}, 0, 0, 0);
    dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zero8, zero8, f32x16{}, 0, 0, 0);
  }

  // Staging: LDS-direct buffer loads.  One wavefront instruction fills 1 KB of a tile, lane l the
  // 16 bytes at l*16: the chunk at swizzled position pos of row r, i.e. source chunk pos ^ swz(r).
  // Rows past n read as zero (the resources end at row n).  Timestamps go through a register.
  const uint32_t q_row = (uint32_t)(ld * 2), g_row = (uint32_t)d * 2;
  const __amdgpu_buffer_rsrc_t q_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Qp, (short)0, (int)((uint32_t)n * q_row), 0x00020000);
  const __amdgpu_buffer_rsrc_t g_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Gp, (short)0, (int)((uint32_t)n * g_row), 0x00020000);
  constexpr int NI = BQ * CPR / 64 / 4;  // 1 KB loads per wavefront per operand and tile
  static_assert(NI * 4 * 64 == BQ * CPR, "LDS-direct staging covers the tile");
  uint32_t q_vo[NI], g_vo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int p = (w * NI + i) * 64 + lane;
    const int r = p / CPR, c = (p % CPR) ^ swz<DH>(r);
    q_vo[i] = (uint32_t)r * q_row + c * 16;
    g_vo[i] = (uint32_t)r * g_row + c * 16;
  }
  float rt = -INFINITY;
  auto stage_load = [&](int q0, int buf) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      lds_dma16(q_rsrc, &Qs[buf][(w * NI + i) * 512], q_vo[i], (uint32_t)q0 * q_row);
      lds_dma16(g_rsrc, &Gs[buf][(w * NI + i) * 512], g_vo[i], (uint32_t)q0 * g_row);
    }
    if (MODE == kMaskDynamic && tid < BQ) {
      const int i = q0 + tid;   // R/C queries carry their timestamp, the rest -inf
      rt = (i >= ns && i < n) ? ts[base + i] : -INFINITY;
    }
  };
  // waits for this thread's loads (the tile and its timestamp) before the barrier that publishes it
  auto stage_store = [&](int buf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (MODE == kMaskDynamic && tid < BQ) Tq[buf][tid] = rt;
  };

  auto tile_needed = [&](int buf, int q0) {
    if (!wave_keys) return false;
    if (MODE == kMaskFull) return true;
    if (MODE == kMaskCausal) return q0 + BQ - 1 >= wk0;
    if (wave_static) return true;
    const float tmax = wave_max(Tq[buf][lane]);   // lane i: query q0 + i
    const bool diag = max(wr_lo, q0) < min(wr_hi, q0 + BQ);
    return diag || tmax > wave_tmin;
  };

  bf16x8 pa[4], da[4];
  auto compute_t = [&](auto masked_tag, int buf, int q0) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    // sc[r], dp[r] of one 32-query half: query q0 + mt*32 + 8*(r/4) + 4*hh + r%4, key kj.  Rows
    // and keys past the user's end were loaded as zeros: their score, silu and dP are 0 already.
    // The halves run one after the other, so only one half's score accumulators are live and the
    // first half's SiLU can overlap the second half's MFMAs.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = sw_off<DH>(mt * 32 + l32, ks * 16 + hh * 8);
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[buf][off]);
        const bf16x8 ga = *reinterpret_cast<const bf16x8*>(&Gs[buf][off]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vf[ks], dp, 0, 0, 0);
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 t4 = {};
        if (MODE == kMaskDynamic && kMasked) t4 = *reinterpret_cast<const f32x4*>(&Tq[buf][mt * 32 + 8 * g4 + 4 * hh]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = g4 * 4 + c;
          const int qi = q0 + mt * 32 + 8 * g4 + 4 * hh + c;
          const float s = sc[r];
          const float sgm = sigmoid_rcp(s);
          float p = s * sgm;
          float ds = dp[r] * sgm * (1.0f + s * (1.0f - sgm));
          if constexpr (kMasked) {
            // the rule of mtgr_visible with the key side folded into tk (finite only for R keys)
            const bool vis = MODE == kMaskCausal ? kj <= qi : (kj < ns) | (qi == kj) | (t4[c] > tk);
            p = vis ? p : 0.f;
            ds = vis ? ds : 0.f;
          }
          pa[mt * 2 + (r >> 3)][r & 7] = (bf16)p;
          da[mt * 2 + (r >> 3)][r & 7] = (bf16)ds;
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 gb = tr_frag<DH>(Gs[buf], ks, t, lane);
        dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], gb, dv[t], 0, 0, 0);
        const bf16x8 qb = tr_frag<DH>(Qs[buf], ks, t, lane);
        dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[ks], qb, dk[t], 0, 0, 0);
      }
    }
  };

  // tiles every pair of which is visible take the branch-free unmasked body
  auto compute = [&](int buf, int q0) {
    const bool unmasked = MODE == kMaskFull || (MODE == kMaskCausal ? q0 >= wk0 + 31 : wk0 + 32 <= ns);
    if (unmasked) compute_t(std::false_type{}, buf, q0);
    else compute_t(std::true_type{}, buf, q0);
  };

  if (nqt > 0) {
    stage_load(qt0 * BQ, 0);
    stage_store(0);
  }
  __syncthreads();
  for (int it = 0; it < nqt; ++it) {
    const int cur = it & 1;
    const int q0 = (qt0 + it) * BQ;
    const bool need = tile_needed(cur, q0);
    if (it + 1 < nqt) stage_load(q0 + BQ, cur ^ 1);
    if (need) compute(cur, q0);
    if (it + 1 < nqt) stage_store(cur ^ 1);
    __syncthreads();
  }

  if (wk0 >= n) return;

  // Candidate keys under the dynamic mask: their one visible pair is the diagonal (the key loop
  // gave them nothing), p = silu(q_j . k_j), ds = silu'(q_j . k_j) (g_j . v_j).
  float p_self = 0.f, ds_self = 0.f;
  if (MODE == kMaskDynamic) {
    const bool k_c = kj >= rc_end && kj < n;
    float sp = 0.f, dpp = 0.f;
    if (k_c) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(Qp + kj * ld + ks * 16 + hh * 8);
        const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(Kp + kj * ld + ks * 16 + hh * 8);
        const bf16x8 g8 = *reinterpret_cast<const bf16x8*>(Gp + kj * (int64_t)d + ks * 16 + hh * 8);
        const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(Vp + kj * ld + ks * 16 + hh * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sp += (float)q8[e] * (float)k8[e];
          dpp += (float)g8[e] * (float)v8[e];
        }
      }
    }
    sp += __shfl_xor(sp, 32, kWave);
    dpp += __shfl_xor(dpp, 32, kWave);
    if (k_c) {
      const float sgm = sigmoid_rcp(sp);
      p_self = sp * sgm;
      ds_self = dpp * sgm * (1.0f + sp * (1.0f - sgm));
    }
  }

  // dV then dK of this wavefront's keys through its private LDS region (the key loop ended with
  // a barrier), written as 16-byte row chunks.  Element r of tile t is key 8*(r/4)+4*hh+r%4,
  // feature t*32 + l32.
  float* Os = reinterpret_cast<float*>(arena) + w * 32 * OP;
  float* Ps = reinterpret_cast<float*>(arena) + 4 * 32 * OP + w * 32;
  float* Dsl = Ps + 4 * 32;
  if (hh == 0) { Ps[l32] = p_self; Dsl[l32] = ds_self; }
  const float inv_n = 1.0f / (float)n;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Os[(8 * (r >> 2) + 4 * hh + (r & 3)) * OP + t * 32 + l32] = pass == 0 ? dv[t][r] : dk[t][r];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int idx = lane; idx < 32 * CPR; idx += 64) {
      const int kl = idx / CPR, c = idx % CPR;
      const int j = wk0 + kl;
      if (j >= n) continue;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&Os[kl * OP + c * 8]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&Os[kl * OP + c * 8 + 4]);
      float acc[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) { acc[e] = a0[e]; acc[e + 4] = a1[e]; }
      if (MODE == kMaskDynamic && j >= rc_end) {
        const float coef = pass == 0 ? Ps[kl] : Dsl[kl];
        const bf16x8 src = pass == 0 ? *reinterpret_cast<const bf16x8*>(Gp + j * (int64_t)d + c * 8)
                                     : *reinterpret_cast<const bf16x8*>(Qp + j * ld + c * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += coef * (float)src[e];
      }
      bf16x8 o8;
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = (bf16)(acc[e] * inv_n);
      *reinterpret_cast<bf16x8*>(dqkvu + (base + j) * ld + (pass == 0 ? 2 * d : d) + (int64_t)h * DH + c * 8) = o8;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---- dQ -------------------------------------------------------------------------------------------
template <int DH, int MODE>
__global__ __launch_bounds__(256, 2) void k_attn_bwd_dq(
    int32_t B, int H, int d, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
    const int32_t* __restrict__ order, const int32_t* __restrict__ xcd_off, const float* __restrict__ ts,
    const bf16* __restrict__ qkvu, const bf16* __restrict__ gq, bf16* __restrict__ dqkvu) {
  constexpr int BKV = 64;                // keys per LDS tile
  constexpr int CPR = DH / 8;
  constexpr int NT = DH / 32;
  constexpr int KS = DH / 16;
  constexpr int OP = DH + 4;
  constexpr size_t kLoopBytes = 4 * BKV * DH * sizeof(bf16) + 2 * BKV * sizeof(float);
  constexpr size_t kEpiBytes = 4 * 32 * OP * sizeof(float) + 4 * 32 * sizeof(float);
  __shared__ __attribute__((aligned(16))) char arena[kLoopBytes > kEpiBytes ? kLoopBytes : kEpiBytes];
  bf16 (*Ks)[BKV * DH] = reinterpret_cast<bf16 (*)[BKV * DH]>(arena);
  bf16 (*Vs)[BKV * DH] = reinterpret_cast<bf16 (*)[BKV * DH]>(arena + 2 * BKV * DH * sizeof(bf16));
  float (*Ts)[BKV] = reinterpret_cast<float (*)[BKV]>(arena + 4 * BKV * DH * sizeof(bf16));

  int b, h, tile;
  if (!decode_item(B, H, order, xcd_off, b, h, tile)) return;
  const int64_t base = offsets[b];
  const int n = (int)(offsets[b + 1] - base);
  const UserSeg sg = seg[b];
  const int ns = sg.n_u + sg.n_s;
  const int rc_end = ns + sg.n_r;
  const int q0 = tile * kTile;
  const int64_t ld = 4 * (int64_t)d;
  const bf16* Qp = qkvu + base * ld + (int64_t)h * DH;
  const bf16* Kp = Qp + d;
  const bf16* Vp = Qp + 2 * d;
  const bf16* Gp = gq + base * (int64_t)d + (int64_t)h * DH;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wq0 = q0 + w * 32;
  const int qi = wq0 + l32;
  const bool q_valid = qi < n;
  const bf16x8 zero8 = {};
  bf16x8 qf[KS], gf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = q_valid ? *reinterpret_cast<const bf16x8*>(Qp + qi * ld + ks * 16 + hh * 8) : zero8;
    gf[ks] = q_valid ? *reinterpret_cast<const bf16x8*>(Gp + qi * (int64_t)d + ks * 16 + hh * 8) : zero8;
  }
  const bool q_rc = MODE == kMaskDynamic && q_valid && qi >= ns;
  const float tq = q_rc ? ts[base + qi] : -INFINITY;
  const bool wave_rows = wq0 < n;
  const bool wave_rc = wave_rows && (wq0 + 32 > ns);
  const float wave_tmax = wave_max(tq);
  const int wr_lo = max(wq0, ns), wr_hi = min(min(wq0 + 32, rc_end), n);  // wavefront's R rows
  const bool blk_rc = q0 + kTile > ns;
  // keys past kend are invisible to every row of this tile
  const int kend = MODE == kMaskFull ? n : MODE == kMaskCausal ? min(n, q0 + kTile) : blk_rc ? rc_end : ns;
  const int nkt = (kend + BKV - 1) / BKV;

  f32x16 dq[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[t][r] = 0.f;

  const uint32_t row_b = (uint32_t)(ld * 2);
  const int nbytes = (int)((uint32_t)kend * row_b);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Kp, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Vp, (short)0, nbytes, 0x00020000);
  // K and V tiles, both swizzled, through LDS-direct buffer loads
  constexpr int NI = BKV * CPR / 64 / 4;
  static_assert(NI * 4 * 64 == BKV * CPR, "LDS-direct staging covers the tile");
  uint32_t st_vo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int p = (w * NI + i) * 64 + lane;
    const int r = p / CPR, c = (p % CPR) ^ swz<DH>(r);
    st_vo[i] = (uint32_t)r * row_b + c * 16;
  }
  float rt = INFINITY;
  auto stage_load = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      lds_dma16(k_rsrc, &Ks[buf][(w * NI + i) * 512], st_vo[i], (uint32_t)k0 * row_b);
      lds_dma16(v_rsrc, &Vs[buf][(w * NI + i) * 512], st_vo[i], (uint32_t)k0 * row_b);
    }
    if (MODE == kMaskDynamic && tid < BKV) rt = (k0 + tid < kend) ? ts[base + k0 + tid] : INFINITY;
  };
  auto stage_store = [&](int buf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (MODE == kMaskDynamic && tid < BKV) Ts[buf][tid] = rt;
  };

  auto tile_needed = [&](int buf, int k0) {
    if (MODE == kMaskFull) return wave_rows;
    if (MODE == kMaskCausal) return wave_rows && k0 <= wq0 + 31;
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
    return need;
  };

  // S^T and dP^T one 32-key half at a time (only half the score accumulators live), then the
  // next tile's loads, then dQ += dS K: the loads stay in flight across the dQ MFMAs, and the
  // kernel fits two wavefronts per SIMD.
  bf16x8 da[4];
  auto scores_t = [&](auto masked_tag, int buf, int k0) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const int jb = k0 + 4 * hh;
    const int lim_static = ns - jb, lim_rc = rc_end - jb, self = qi - jb;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[buf][sw_off<DH>(mt * 32 + l32, ks * 16 + hh * 8)]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vs[buf][sw_off<DH>(mt * 32 + l32, ks * 16 + hh * 8)]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[ks], dp, 0, 0, 0);
      }
      // sc[r], dp[r]: key k0 + mt*32 + 8*(r/4) + 4*hh + r%4, query qi
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 t4 = {};
        if (MODE == kMaskDynamic && kMasked) t4 = *reinterpret_cast<const f32x4*>(&Ts[buf][mt * 32 + 8 * g4 + 4 * hh]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = g4 * 4 + c;
          const int dk = mt * 32 + 8 * g4 + c;
          const float s = sc[r];
          const float sgm = sigmoid_rcp(s);
          float ds = dp[r] * sgm * (1.0f + s * (1.0f - sgm));
          if constexpr (kMasked) {
            const bool vis = MODE == kMaskCausal
                                 ? dk <= self
                                 : (dk < lim_static) | (dk == self) | (q_rc & (dk < lim_rc) & (t4[c] < tq));
            ds = vis ? ds : 0.f;
          }
          da[mt * 2 + (r >> 3)][r & 7] = (bf16)ds;
        }
      }
    }
  };
  // tiles every pair of which is visible take the branch-free unmasked body
  auto scores = [&](int buf, int k0) {
    const bool unmasked = MODE == kMaskFull || (MODE == kMaskCausal ? k0 + BKV <= wq0 + 1 : k0 + BKV <= ns);
    if (unmasked) scores_t(std::false_type{}, buf, k0);
    else scores_t(std::true_type{}, buf, k0);
  };
  // The next tile's LDS-direct loads, then dQ += dS K over the current tile.  Both buffers live in
  // one array, so the compiler cannot tell them apart by name; restrict-qualified views of the
  // current K tile and of the next buffers tell it the loads do not write what the dQ reads read,
  // and it no longer waits for those loads before the reads (it did, on every tile).
  auto dq_phase = [&](const bf16* __restrict__ kcur, bf16* __restrict__ knxt, bf16* __restrict__ vnxt, bool need,
                      int k0) {
    if (k0 + BKV < kend) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        lds_dma16(k_rsrc, knxt + (w * NI + i) * 512, st_vo[i], (uint32_t)(k0 + BKV) * row_b);
        lds_dma16(v_rsrc, vnxt + (w * NI + i) * 512, st_vo[i], (uint32_t)(k0 + BKV) * row_b);
      }
      if (MODE == kMaskDynamic && tid < BKV) rt = (k0 + BKV + tid < kend) ? ts[base + k0 + BKV + tid] : INFINITY;
    }
    if (need) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 kb = tr_frag<DH>(kcur, ks, t, lane);
          dq[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[ks], kb, dq[t], 0, 0, 0);
        }
      }
    }
  };

  stage_load(0, 0);
  stage_store(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const int k0 = kt * BKV;
    const bool need = tile_needed(cur, k0);
    if (need) scores(cur, k0);
    dq_phase(Ks[cur], Ks[cur ^ 1], Vs[cur ^ 1], need, k0);
    if (kt + 1 < nkt) stage_store(cur ^ 1);
    __syncthreads();
  }

  if (!wave_rows) return;

  // Candidate rows under the dynamic mask: their own term ds_self k_i (the key loop stops short
  // of the candidate block).
  float ds_self = 0.f;
  if (MODE == kMaskDynamic) {
    const bool q_c = q_valid && qi >= rc_end;
    float sp = 0.f, dpp = 0.f;
    if (q_c) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(Kp + qi * ld + ks * 16 + hh * 8);
        const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(Vp + qi * ld + ks * 16 + hh * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sp += (float)qf[ks][e] * (float)k8[e];
          dpp += (float)gf[ks][e] * (float)v8[e];
        }
      }
    }
    sp += __shfl_xor(sp, 32, kWave);
    dpp += __shfl_xor(dpp, 32, kWave);
    if (q_c) {
      const float sgm = sigmoid_rcp(sp);
      ds_self = dpp * sgm * (1.0f + sp * (1.0f - sgm));
    }
  }

  float* Os = reinterpret_cast<float*>(arena) + w * 32 * OP;
  float* Ds = reinterpret_cast<float*>(arena) + 4 * 32 * OP + w * 32;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      Os[(8 * (r >> 2) + 4 * hh + (r & 3)) * OP + t * 32 + l32] = dq[t][r];
  if (hh == 0) Ds[l32] = ds_self;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float inv_n = 1.0f / (float)n;
  for (int idx = lane; idx < 32 * CPR; idx += 64) {
    const int ql = idx / CPR, c = idx % CPR;
    const int q = wq0 + ql;
    if (q >= n) continue;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(&Os[ql * OP + c * 8]);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(&Os[ql * OP + c * 8 + 4]);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) { acc[e] = a0[e]; acc[e + 4] = a1[e]; }
    const float dsq = Ds[ql];
    if (dsq != 0.f) {
      const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(Kp + q * ld + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += dsq * (float)k8[e];
    }
    bf16x8 o8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = (bf16)(acc[e] * inv_n);
    *reinterpret_cast<bf16x8*>(dqkvu + (base + q) * ld + (int64_t)h * DH + c * 8) = o8;
  }
}

template <int DH, int MODE>
hipError_t attn_bwd_mode(unsigned grid, int32_t B, int d, int H, const int64_t* offsets, const UserSeg* seg,
                         const int32_t* order, const int32_t* xcd_off, const float* ts, const bf16* qkvu,
                         const bf16* g, bf16* dqkvu, hipStream_t s) {
  k_attn_bwd_dkv<DH, MODE><<<grid, 256, 0, s>>>(B, H, d, offsets, seg, order, xcd_off, ts, qkvu, g, dqkvu);
  k_attn_bwd_dq<DH, MODE><<<grid, 256, 0, s>>>(B, H, d, offsets, seg, order, xcd_off, ts, qkvu, g, dqkvu);
  return hipGetLastError();
}

template <int DH>
hipError_t attn_bwd_dh(unsigned grid, int32_t B, int d, int H, int mask_mode, const int64_t* offsets,
                       const UserSeg* seg, const int32_t* order, const int32_t* xcd_off, const float* ts,
                       const bf16* qkvu, const bf16* g, bf16* dqkvu, hipStream_t s) {
  switch (mask_mode) {
    case kMaskDynamic:
      return attn_bwd_mode<DH, kMaskDynamic>(grid, B, d, H, offsets, seg, order, xcd_off, ts, qkvu, g, dqkvu, s);
    case kMaskCausal:
      return attn_bwd_mode<DH, kMaskCausal>(grid, B, d, H, offsets, seg, order, xcd_off, ts, qkvu, g, dqkvu, s);
    case kMaskFull:
      return attn_bwd_mode<DH, kMaskFull>(grid, B, d, H, offsets, seg, order, xcd_off, ts, qkvu, g, dqkvu, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attention_bwd_bf16(int32_t B, int64_t T, int64_t grid_slots, int d, int H, int mask_mode,
                                     const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                     const int32_t* xcd_off, const float* timestamps, const bf16* qkvu,
                                     const bf16* vt, const bf16* dy, bf16* g, bf16* dqkvu, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t chunks = T * (d / 8);
  // one 16-byte chunk per thread (the loop in the kernel only matters past 2^38 chunks): a thread
  // that looped over several would wait, at each chunk's loads, for its previous chunk's stores
  // (vector memory operations retire in order)
  k_gate_bwd<<<(unsigned)std::min<int64_t>((chunks + 255) / 256, int64_t(1) << 30), 256, 0, s>>>(T, d, qkvu, vt, dy, g, dqkvu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || grid_slots == 0) return e;
  const unsigned grid = (unsigned)(grid_slots * kXcdCount);
  const int dh = d / H;
  if (dh == 128) return attn_bwd_dh<128>(grid, B, d, H, mask_mode, offsets, seg, order, xcd_off, timestamps, qkvu, g, dqkvu, s);
  if (dh == 64) return attn_bwd_dh<64>(grid, B, d, H, mask_mode, offsets, seg, order, xcd_off, timestamps, qkvu, g, dqkvu, s);
  return hipErrorInvalidValue;
}

}  // namespace mtgr
