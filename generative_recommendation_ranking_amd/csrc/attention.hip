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
// operand of O = P V.  V stays row-major in LDS; each B fragment of P V is two transposing
// reads (ds_read_b64_tr_b16) that hand every lane the 8 keys of its feature column in the order
// the score accumulator holds them.
//
// LDS per workgroup: K 2 x 64 x (d_h+8) and V 2 x 64 x (d_h+32) bf16 (double-buffered,
// register-staged global->LDS copies), ~75 KB at d_h = 128, two workgroups per CU.
#include "kernels.h"

namespace mtgr {

namespace {

constexpr int BQ = kAttnQTileBf16;  // 128 query rows per work item
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
constexpr int BKV = 64;             // keys per tile

__device__ __forceinline__ int find_slot(const int32_t* __restrict__ tile_off, int B, int item) {
  int lo = 0, hi = B;  // largest p with tile_off[p] <= item
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

// MODE: kMaskDynamic (the three rules), kMaskCausal (j <= i) or kMaskFull (all keys of the user).
template <int DH, int MODE>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(
    int32_t B, int H, int d, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
    const int32_t* __restrict__ order, const int32_t* __restrict__ xcd_off,
    const float* __restrict__ ts, const bf16* __restrict__ qkvu, bf16* __restrict__ y,
    bf16* __restrict__ vt) {
  constexpr int KP = DH + 8;                     // K row pitch: 16-byte reads of 16 rows hit distinct banks
  // V row pitch: a transposing read by 32 lanes touches 4 rows x 2 column chunks of 32 bytes;
  // a pitch of 16 (mod 64) dwords puts those 8 chunks on disjoint banks.
  constexpr int VP = DH + 32;
  constexpr int DCH = DH / 8;                    // 16-byte chunks per key row
  constexpr int CH = BKV * DCH / 256;            // K (and V) chunks per thread per tile
  constexpr int NT = DH / 32;                    // output tiles of 32 features
  static_assert(CH * 256 == BKV * DCH && CH <= 4, "staging layout");

  // One LDS arena: K and V^T tiles (double-buffered) and the tile timestamps during the key loop;
  // reused afterwards to stage each wavefront's output rows for vectorised stores.
  constexpr int OP = DH + 4;                                   // fp32 pitch of staged output rows
  constexpr size_t kLoopBytes = (2 * BKV * KP + 2 * BKV * VP) * sizeof(bf16) + 2 * BKV * sizeof(float);
  constexpr size_t kEpiBytes = 4 * 32 * OP * sizeof(float) + 4 * 32 * sizeof(float);
  __shared__ __attribute__((aligned(16))) char arena[kLoopBytes > kEpiBytes ? kLoopBytes : kEpiBytes];
  bf16 (*Ks)[BKV][KP] = reinterpret_cast<bf16 (*)[BKV][KP]>(arena);
  bf16 (*Vs)[BKV][VP] = reinterpret_cast<bf16 (*)[BKV][VP]>(arena + 2 * BKV * KP * sizeof(bf16));
  float (*Ts)[BKV] = reinterpret_cast<float (*)[BKV]>(arena + (2 * BKV * KP + 2 * BKV * VP) * sizeof(bf16));

  // Work decode: workgroup ids go round-robin to the XCDs, so id % 8 is the XCD and id / 8 the
  // position in that XCD's queue; the queue lists its (user, head) groups' q-tiles back to back,
  // so all q-tiles of a group run on one XCD, together, and share its L2 while they sweep K/V.
  const int xcd = (int)(blockIdx.x % kXcdCount);
  const int pos = (int)(blockIdx.x / kXcdCount);
  const int R = (int)(((int64_t)B * H + kXcdCount - 1) / kXcdCount);
  const int32_t* xo = xcd_off + (int64_t)xcd * (R + 1);
  if (pos >= xo[R]) return;
  const int round = find_slot(xo, R, pos);
  const int64_t grp = (int64_t)round * kXcdCount + ((round & 1) ? (kXcdCount - 1 - xcd) : xcd);
  const int b = order[grp / H];
  const int h = (int)(grp % H);
  const int qt = pos - xo[round];
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
  const bool q_rc = MODE == kMaskDynamic && q_valid && qi >= ns;
  const float tq = q_rc ? ts[base + qi] : -INFINITY;

  const bool wave_rows = wq0 < n;
  const bool wave_rc = wave_rows && (wq0 + 32 > ns);
  const float wave_tmax = wave_max(tq);
  const int wr_lo = max(wq0, ns), wr_hi = min(min(wq0 + 32, rc_end), n);  // wavefront's R rows

  const bool blk_rc = (q0 + BQ > ns);
  // keys past kend are invisible to every row of this q-tile
  const int kend = MODE == kMaskFull ? n : MODE == kMaskCausal ? min(n, q0 + BQ) : blk_rc ? rc_end : ns;
  const int nkt = (kend + BKV - 1) / BKV;

  f32x16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;

  // Staging: every thread copies CH 16-byte chunks of the K tile and CH of the V tile (both kept
  // row-major in LDS), through buffer loads over this user's rows of head h sized to the first
  // kend keys, so keys at or past kend read as zero.  Per-lane byte offset in a VGPR, the tile
  // offset in an SGPR.
  bf16x8 stg[2 * CH];
  float rt = INFINITY;
  const uint32_t row_bytes = (uint32_t)(ld * 2);
  const int nbytes = (int)((uint32_t)kend * row_bytes);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Kp, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Vp, (short)0, nbytes, 0x00020000);
  const int st_key = tid / DCH, st_c = tid % DCH;             // chunk i: key st_key + i*(256/DCH)
  constexpr int KSTEP = 256 / DCH;
  const uint32_t st_off = (uint32_t)st_key * row_bytes + st_c * 16;

  auto stage_load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t so = (uint32_t)(k0 + i * KSTEP) * row_bytes;
      stg[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, st_off, so, 0));
      stg[CH + i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, st_off, so, 0));
    }
    if (MODE == kMaskDynamic && tid < BKV) rt = (k0 + tid < kend) ? ts[base + k0 + tid] : INFINITY;
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      *reinterpret_cast<bf16x8*>(&Ks[buf][st_key + i * KSTEP][st_c * 8]) = stg[i];
      *reinterpret_cast<bf16x8*>(&Vs[buf][st_key + i * KSTEP][st_c * 8]) = stg[CH + i];
    }
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
  bf16x8 pa[4];
  auto scores = [&](int buf, int k0) {
    f32x16 sc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[mt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[buf][mt * 32 + l32][ks * 16 + hh * 8]);
        sc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc[mt], 0, 0, 0);
      }
    }
    // sc[mt][r]: key k0 + mt*32 + 8*(r/4) + 4*hh + r%4, query qi
    // tiles every key of which is visible to every row of the wavefront skip the mask
    const bool unmasked = MODE == kMaskFull || (MODE == kMaskCausal ? k0 + BKV <= wq0 + 1 : k0 + BKV <= ns);
    if (unmasked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pa[mt * 2 + (r >> 3)][r & 7] = (bf16)silu_rcp(sc[mt][r]);
    } else {
      // Mask.  With jb = k0 + 4*hh this lane's keys are jb + dk, dk = mt*32 + 8*(r/4) + r%4 a
      // compile-time constant, so the visibility rule (the same as mtgr_visible) becomes three
      // integer compares against per-lane offsets plus one timestamp compare.  Keys at or past
      // kend were loaded as zeros: their score and silu are 0 already.
      const int jb = k0 + 4 * hh;
      const int lim_static = ns - jb, lim_rc = rc_end - jb, self = qi - jb;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(&Ts[buf][mt * 32 + 8 * g4 + 4 * hh]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = g4 * 4 + c;
            const int dk = mt * 32 + 8 * g4 + c;
            const float p = silu_rcp(sc[mt][r]);
            const bool vis = MODE == kMaskCausal
                                 ? dk <= self
                                 : (dk < lim_static) | (dk == self) | (q_rc & (dk < lim_rc) & (t4[c] < tq));
            pa[mt * 2 + (r >> 3)][r & 7] = (bf16)(vis ? p : 0.f);
          }
        }
      }
    }
  };
  auto accumulate = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // B fragment (keys x features) of PV k-step ks: slot jj of lane-half hh is key
        // kb + 4*hh + jj%4 (+8 for jj >= 4), kb = (ks/2)*32 + (ks%2)*16, feature t*32 + lane%32.
        // ds_read_b64_tr_b16 hands lane i of a 16-lane group element i%4 of the 4-element rows
        // addressed by lanes i/4 + 4e: point lane s at row kb + 4*hh + s/4, features
        // t*32 + 16*(group%2) + 4*(s%4), and each read returns 4 keys of one feature column.
        const int kb = (ks >> 1) * 32 + (ks & 1) * 16 + 4 * hh + (lane & 15) / 4;
        const int fc = t * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&Vs[buf][kb][fc]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&Vs[buf][kb + 8][fc]));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], vf, o[t], 0, 0, 0);
      }
    }
  };

  stage_load(0);
  stage_store(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const int k0 = kt * BKV;
    const bool need = tile_needed(cur, k0);
    if (need) scores(cur, k0);
    if (kt + 1 < nkt) stage_load(k0 + BKV);
    if (need) accumulate(cur);
    if (kt + 1 < nkt) stage_store(cur ^ 1);
    __syncthreads();
  }

  if (!wave_rows) return;

  // Candidate rows under the dynamic mask: their own term silu(q_i . k_i) v_i (the diagonal of
  // the C block, which the key loop stops short of).
  const bool q_c = MODE == kMaskDynamic && q_valid && qi >= rc_end;
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
  const float p_self = q_c ? (float)(bf16)silu_rcp(s_self) : 0.f;

  // Stage this wavefront's O rows (fp32) in LDS: element r of tile t is row 8*(r/4)+4*hh+r%4,
  // feature t*32 + l32.  The key loop ended with a barrier, so the arena is free.
  float* Os = reinterpret_cast<float*>(arena) + w * 32 * OP;
  float* Ps = reinterpret_cast<float*>(arena) + 4 * 32 * OP + w * 32;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      Os[(8 * (r >> 2) + 4 * hh + (r & 3)) * OP + t * 32 + l32] = o[t][r];
  if (hh == 0) Ps[l32] = p_self;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // y = (O + p_self v) / n (.) u, 8 features per lane step, 16-byte loads and stores.
  const float inv_n = 1.0f / (float)n;
  for (int idx = lane; idx < 32 * DCH; idx += 64) {
    const int ql = idx / DCH, c = idx % DCH;
    const int q = wq0 + ql;
    if (q >= n) continue;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(&Os[ql * OP + c * 8]);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(&Os[ql * OP + c * 8 + 4]);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) { acc[e] = a0[e]; acc[e + 4] = a1[e]; }
    const float ps = Ps[ql];
    if (ps != 0.f) {
      const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(Vp + q * ld + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += ps * (float)v8[e];
    }
    const bf16x8 u8 = *reinterpret_cast<const bf16x8*>(Up + q * ld + c * 8);
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (bf16)(acc[e] * inv_n * (float)u8[e]);
    if (vt) {   // the ungated V~ (kept for the backward pass)
      bf16x8 o2;
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = (bf16)(acc[e] * inv_n);
      *reinterpret_cast<bf16x8*>(vt + (base + q) * (int64_t)d + (int64_t)h * DH + c * 8) = o2;
    }
    *reinterpret_cast<bf16x8*>(y + (base + q) * (int64_t)d + (int64_t)h * DH + c * 8) = out;
  }
}

// fp32 storage mode: the same rule set (any mask mode) evaluated directly over every key of the user, one
// thread per query row, for exact comparison with the oracle.
template <int DH>
__global__ __launch_bounds__(64) void k_attn_f32(
    int32_t B, int d, int mode, const int64_t* __restrict__ offsets,
    const UserSeg* __restrict__ seg, const int32_t* __restrict__ order,
    const int32_t* __restrict__ tile_off, const float* __restrict__ ts,
    const float* __restrict__ qkvu, float* __restrict__ y, float* __restrict__ vt) {
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
    if (!mtgr_visible_mode(mode, i, j, ns, rc_end, ti, ts[base + j])) continue;
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
  if (vt) {   // the ungated V~ (kept for the backward pass)
#pragma unroll
    for (int f = 0; f < DH; ++f) vt[(base + i) * (int64_t)d + (int64_t)h * DH + f] = acc[f] * inv_n;
  }
}

}  // namespace

template <int MODE>
hipError_t attn_bf16_mode(unsigned grid, int32_t B, int d, int H, const int64_t* offsets,
                          const UserSeg* seg, const int32_t* order, const int32_t* xcd_off,
                          const float* timestamps, const bf16* qkvu, bf16* y, bf16* vt,
                          hipStream_t s) {
  const int dh = d / H;
  if (dh == 128)
    k_attn_bf16<128, MODE><<<grid, 256, 0, s>>>(B, H, d, offsets, seg, order, xcd_off, timestamps, qkvu, y, vt);
  else if (dh == 64)
    k_attn_bf16<64, MODE><<<grid, 256, 0, s>>>(B, H, d, offsets, seg, order, xcd_off, timestamps, qkvu, y, vt);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention_bf16(int32_t B, int64_t grid_slots, int d, int H, int mask_mode,
                                 const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                 const int32_t* xcd_off, const float* timestamps,
                                 const bf16* qkvu, bf16* y, bf16* vt, hipStream_t s) {
  if (grid_slots == 0) return hipSuccess;
  const unsigned grid = (unsigned)(grid_slots * kXcdCount);
  switch (mask_mode) {
    case kMaskDynamic:
      return attn_bf16_mode<kMaskDynamic>(grid, B, d, H, offsets, seg, order, xcd_off, timestamps, qkvu, y, vt, s);
    case kMaskCausal:
      return attn_bf16_mode<kMaskCausal>(grid, B, d, H, offsets, seg, order, xcd_off, timestamps, qkvu, y, vt, s);
    case kMaskFull:
      return attn_bf16_mode<kMaskFull>(grid, B, d, H, offsets, seg, order, xcd_off, timestamps, qkvu, y, vt, s);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_f32(int32_t B, int64_t total_tiles, int d, int H, int mask_mode,
                                const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                const int32_t* tile_off, const float* timestamps,
                                const float* qkvu, float* y, float* vt, hipStream_t s) {
  if (total_tiles == 0) return hipSuccess;
  const int dh = d / H;
  dim3 grid((unsigned)total_tiles, (unsigned)H);
  if (dh == 32)
    k_attn_f32<32><<<grid, 64, 0, s>>>(B, d, mask_mode, offsets, seg, order, tile_off, timestamps, qkvu, y, vt);
  else if (dh == 64)
    k_attn_f32<64><<<grid, 64, 0, s>>>(B, d, mask_mode, offsets, seg, order, tile_off, timestamps, qkvu, y, vt);
  else if (dh == 128)
    k_attn_f32<128><<<grid, 64, 0, s>>>(B, d, mask_mode, offsets, seg, order, tile_off, timestamps, qkvu, y, vt);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mtgr
