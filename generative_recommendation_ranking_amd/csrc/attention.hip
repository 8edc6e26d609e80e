// Fused jagged masked-SiLU attention with the U gate, on gfx950.
//
// Per user b and head h (marovi.ai MTGR page, 方法, the V~ update equation, read token-wise):
//     y_i = u_i (.) (1/n_b) * sum_j M[i,j] * silu(q_i . k_j) * v_j
// with M the three-rule dynamic mask (fun-rec "MTGR: Hybrid Paradigm Modeling" 7.3.4) and n_b
// the user's total token count.  No softmax, no 1/sqrt(d_h), no running max.  Users never
// attend to each other (sequence packing, chenhuiyu blog "MTGR", training-system section).
//
// Work item = (user, head, q-tile of 32 NW rows); one workgroup of NW wavefronts x 32 query rows.
// The forward runs NW = 4 (128 rows, two workgroups per CU, so two wavefronts per SIMD).  Work
// items are ordered longest user first (LPT) by the prep kernels.
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
// Staging: K, V and timestamp tiles go global -> LDS by LDS-direct buffer loads (no registers,
// no LDS write instructions), double-buffered: the loads of tile k+1 are issued before tile k is
// computed and waited for at the barrier that ends it.  Rows are unpadded and XOR-swizzled in
// 16-byte chunks.  LDS per workgroup: 4 x 64 x d_h bf16 + 512 B (65 KB at d_h = 128), reused
// afterwards for the fp32 staging of the output rows.
//
// Where the time goes (large workload, d_h = 128; MFMA work is within 2% of the algorithmic
// count).  A wavefront's 64-key tile costs 32 MFMAs (1024 cycles), ~176 vector instructions for
// SiLU (64 of them transcendental, 8 cycles each on gfx950) and 48 LDS fragment reads (32 KB);
// vector work and MFMAs of one wavefront barely overlap, across the two wavefronts of a SIMD
// about a quarter of the MFMA time does.  Measured per layer: register-staged copies 5.69 ms,
// LDS-direct 5.32 ms, fragments requested one (K) and two (V) steps ahead of their MFMAs 5.23 ms.  Tried and slower: SiLU interleaved between the MFMAs of one wavefront
// (5.63 ms); s_setprio raised over the MFMA phases (no change); an 8-wavefront ping-pong, where
// the two wavefronts of a SIMD alternate MFMA and vector phases between workgroup barriers over
// three LDS slots (co-issue doubled but barrier waits grew: 8% slower); 8 wavefronts over 256
// rows with plain double buffering (4% slower).
#include "kernels.h"

namespace mtgr {

namespace {

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
constexpr int BKV = 64;             // keys per tile

// LDS-direct buffer load: lane l's `bytes` (4 or 16) land at lds + l * bytes (lds wave-uniform).
// Kept in a device function of its own: written in a kernel's body, the builtin stops the host
// pass from emitting that kernel's launch stub.
__device__ __forceinline__ void lds_load(__amdgpu_buffer_rsrc_t r, void* lds, int bytes, uint32_t voff,
                                         uint32_t soff) {
  if (bytes == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ int find_slot(const int32_t* __restrict__ tile_off, int B, int item) {
  int lo = 0, hi = B;  // largest p with tile_off[p] <= item
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

// MODE: kMaskDynamic (the three rules), kMaskCausal (j <= i) or kMaskFull (all keys of the user).
// NW wavefronts of 32 query rows each.
template <int DH, int MODE, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_attn_bf16(
    int32_t B, int H, int d, const int64_t* __restrict__ offsets, const UserSeg* __restrict__ seg,
    const int32_t* __restrict__ order, const int32_t* __restrict__ xcd_off,
    const float* __restrict__ ts, const bf16* __restrict__ qkvu, bf16* __restrict__ y,
    bf16* __restrict__ vt) {
  constexpr int BQ = 32 * NW;                     // query rows per work item
  static_assert(BQ == kAttnFwdQTileBf16, "work items come from queues built with the forward's q-tile");
  static_assert(NW == 4, "the epilogue stages each wavefront's rows in one of the four tile buffers");
  constexpr int CPR = DH / 8;                    // 16-byte chunks per key row
  constexpr int RB = 1024 / (DH * 2);            // key rows per 1 KB LDS-direct block
  constexpr int NBW = BKV / RB / NW;             // blocks per wavefront, per operand and tile
  constexpr int TILE = BKV * DH;                 // bf16 elements of one K or V tile
  constexpr int NT = DH / 32;                    // output tiles of 32 features
  static_assert(NBW * RB * NW == BKV && NBW >= 1, "staging layout");
  static_assert(32 * DH * sizeof(float) <= TILE * sizeof(bf16), "a wavefront's output rows fit one tile buffer");

  // K and V tiles, double-buffered, as separate arrays so that reads of one buffer are not held
  // up behind the LDS-direct loads filling the other.  Rows are unpadded; the 16-byte chunk c of
  // row r sits at chunk position c ^ swk(r) (K) or c ^ swv(r) (V), which keeps the fragment reads
  // below free of bank conflicts (64 banks of 4 bytes).
  __shared__ __attribute__((aligned(1024))) bf16 Ks0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 Ks1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 Vs0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 Vs1[TILE];
  __shared__ __attribute__((aligned(256))) float Ts0[BKV];
  __shared__ __attribute__((aligned(256))) float Ts1[BKV];
  __shared__ float Ps_all[NW * 32];              // candidate rows' own-term weights, epilogue only
  // K fragment reads: 16 lanes take rows r..r+15 at one logical chunk
  auto swk = [](int r) { return DH == 128 ? (r & 15) : ((r >> 1) & 7); };
  // V transposing reads: 32 lanes take 4 rows x 4 chunks of one 64-byte column block
  auto swv = [](int r) { return DH == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };

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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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

  // Staging: LDS-direct buffer loads (global -> LDS without registers).  One wavefront
  // instruction fills a contiguous 1 KB block, lane l its 16 bytes at 16 l, i.e. row l / CPR,
  // chunk position l % CPR of the block's RB rows; the lane fetches the global chunk that the
  // swizzle puts there.  The buffers span this user's rows of head h up to kend, with the tile
  // offset in the SGPR offset: the range check covers both, so keys at or past kend land in LDS
  // as zeros.  Timestamps come the same way (one wavefront, 4 bytes a lane).
  const uint32_t row_bytes = (uint32_t)(ld * 2);
  const int nbytes = (int)((uint32_t)kend * row_bytes);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Kp, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Vp, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t t_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(ts + base), (short)0, kend * (int)sizeof(float), 0x00020000);
  uint32_t vo_k[NBW], vo_v[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int row = (w * NBW + i) * RB + lane / CPR, p = lane % CPR;
    vo_k[i] = (uint32_t)row * row_bytes + (uint32_t)((p ^ swk(row)) * 16);
    vo_v[i] = (uint32_t)row * row_bytes + (uint32_t)((p ^ swv(row)) * 16);
  }
  auto stage = [&](bf16* kd, bf16* vd, float* td, int k0) {
    const uint32_t so = (uint32_t)k0 * row_bytes;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      lds_load(k_rsrc, kd + (w * NBW + i) * 512, 16, vo_k[i], so);
      lds_load(v_rsrc, vd + (w * NBW + i) * 512, 16, vo_v[i], so);
    }
    if (MODE == kMaskDynamic && w == 0) lds_load(t_rsrc, td, 4, (uint32_t)lane * 4u, (uint32_t)k0 * 4u);
  };
  // every wavefront's LDS-direct loads have landed: its own wait, then the barrier
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
  };

  // fragment offsets (bytes within a tile).  K, k-step ks: row mt*32 + l32, logical chunk 2 ks + hh.
  uint32_t koff[DH / 16];
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks) koff[ks] = (uint32_t)((l32 * CPR + ((2 * ks + hh) ^ swk(l32))) * 16);
  // V, output tile t: the transposing read of lane s in a 16-lane group starts at row
  // rl = 4 hh + (s / 4) of an 8-row group and features t*32 + 16*(group % 2) + 4*(s % 4).
  uint32_t voff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int rl = 4 * hh + ((lane & 15) >> 2);
    const int c = 4 * t + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    voff[t] = (uint32_t)((rl * CPR + (c ^ swv(rl))) * 16 + 8 * (lane & 1));
  }

  auto tile_needed = [&](const float* Tb, int k0) {
    if (MODE == kMaskFull) return wave_rows;
    if (MODE == kMaskCausal) return wave_rows && k0 <= wq0 + 31;
    bool need = wave_rows && (k0 < ns || (wave_rc && k0 < rc_end));
    if (need && k0 >= ns) {
      // pure R tile: skip when no key is earlier than the wavefront's latest R/C row and the
      // wavefront's own R rows (the diagonal) are not in it
      const int j = k0 + lane;
      const float tk = (j < kend) ? Tb[lane] : INFINITY;
      const float tmin = wave_min(tk);
      const bool diag = max(wr_lo, k0) < min(wr_hi, k0 + BKV);
      if (!diag && tmin >= wave_tmax) need = false;
    }
    return need;
  };
  bf16x8 pa[4];
  auto scores = [&](const bf16* Kb, const float* Tb, int k0) {
    f32x16 sc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[mt][r] = 0.f;
    // the K fragments of k-step ks + 1 are requested before the MFMAs of k-step ks (the
    // scheduling barriers keep the compiler from sinking the reads back to their use)
    constexpr int NKS = DH / 16;
    bf16x8 kf[2][2];
    auto kread = [&](int ks, bf16x8* dst) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        dst[mt] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(Kb) + koff[ks] +
                                                   mt * 32 * DH * (int)sizeof(bf16));
    };
    kread(0, kf[0]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 1 < NKS) kread(ks + 1, kf[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks & 1][mt], qf[ks], sc[mt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // sc[mt][r]: key k0 + mt*32 + 8*(r/4) + 4*hh + r%4, query qi
    // tiles every key of which is visible to every row of the wavefront skip the mask
    const bool unmasked = MODE == kMaskFull || (MODE == kMaskCausal ? k0 + BKV <= wq0 + 1 : k0 + BKV <= ns);
    // silu(z) = z * rcp(1 + e^-z) (silu_rcp), computed 16 scores at a time with the steps of the
    // 16 chains issued side by side (exponentials, sums, reciprocals), not chain after chain
    auto silu16 = [&](int mt, float (&p)[16]) {
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __expf(-sc[mt][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_rcpf(1.0f + p[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = sc[mt][r] * p[r];
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);   // the products -z log2(e)
      __builtin_amdgcn_sched_group_barrier(0x400, 16, 0);   // 16 exponentials
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);   // 16 sums
      __builtin_amdgcn_sched_group_barrier(0x400, 16, 0);   // 16 reciprocals
    };
    if (unmasked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float p[16];
        silu16(mt, p);
#pragma unroll
        for (int r = 0; r < 16; ++r) pa[mt * 2 + (r >> 3)][r & 7] = (bf16)p[r];
      }
    } else {
      // Mask.  With jb = k0 + 4*hh this lane's keys are jb + dk, dk = mt*32 + 8*(r/4) + r%4 a
      // compile-time constant, so the visibility rule (the same as mtgr_visible) becomes three
      // integer compares against per-lane offsets plus one timestamp compare.  Keys at or past
      // kend were loaded as zeros: their score and silu are 0 already (their timestamps are 0 too,
      // but the per-lane limits already make them invisible).
      const int jb = k0 + 4 * hh;
      const int lim_static = ns - jb, lim_rc = rc_end - jb, self = qi - jb;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float ps[16];
        silu16(mt, ps);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(&Tb[mt * 32 + 8 * g4 + 4 * hh]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = g4 * 4 + c;
            const int dk = mt * 32 + 8 * g4 + c;
            const float p = ps[r];
            const bool vis = MODE == kMaskCausal
                                 ? dk <= self
                                 : (dk < lim_static) | (dk == self) | (q_rc & (dk < lim_rc) & (t4[c] < tq));
            pa[mt * 2 + (r >> 3)][r & 7] = (bf16)(vis ? p : 0.f);
          }
        }
      }
    }
  };
  auto accumulate = [&](const bf16* Vb) {
    // B fragment (keys x features) of P V k-step ks and output tile t: slot jj of lane-half hh is
    // key kb + 4*hh + jj%4 (+8 for jj >= 4), kb = (ks/2)*32 + (ks%2)*16, feature t*32 + lane%32.
    // ds_read_b64_tr_b16 hands lane i of a 16-lane group element i%4 of the 4-element rows
    // addressed by lanes i/4 + 4e: point lane s at row kb + 4*hh + s/4, features
    // t*32 + 16*(group%2) + 4*(s%4) (voff[t], swizzled), and each read returns 4 keys of one
    // feature column.  Fragments are requested two (ks, t) steps ahead of their MFMA.
    constexpr int NS = 4 * NT;
    auto vread = [&](int i) {
      const int ks = i / NT, t = i % NT;
      const char* vb = reinterpret_cast<const char*>(Vb) + voff[t] + ((ks >> 1) * 32 + (ks & 1) * 16) * DH * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vb);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + 8 * DH * 2));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vf[3];
    vf[0] = vread(0);
    vf[1] = vread(1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + 2 < NS) vf[(i + 2) % 3] = vread(i + 2);
      __builtin_amdgcn_sched_barrier(0);
      o[i % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i / NT], vf[i % 3], o[i % NT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Key loop, unrolled by two so that each half names its buffers at compile time: the next
  // tile's LDS-direct loads go out first and land while this tile is computed.
  auto step = [&](const bf16* Kb, const bf16* Vb, const float* Tb, bf16* Kn, bf16* Vn, float* Tn, int kt) {
    const int k0 = kt * BKV;
    if (kt + 1 < nkt) stage(Kn, Vn, Tn, k0 + BKV);
    if (tile_needed(Tb, k0)) {
      scores(Kb, Tb, k0);
      accumulate(Vb);
    }
    publish();
  };
  stage(Ks0, Vs0, Ts0, 0);
  publish();
  for (int kt = 0; kt < nkt; kt += 2) {
    step(Ks0, Vs0, Ts0, Ks1, Vs1, Ts1, kt);
    if (kt + 1 < nkt) step(Ks1, Vs1, Ts1, Ks0, Vs0, Ts0, kt + 1);
  }

  if (!wave_rows) return;

  // Every global load of the epilogue is issued before anything waits for one, so their
  // latencies overlap: the K rows of candidate queries (their own term silu(q_i . k_i) v_i, the
  // diagonal of the C block, which the key loop stops short of), and the U rows, plus the V rows of
  // candidate queries, of the output chunks this lane writes.
  // Buffer loads whose ranges cover exactly the rows wanted (U: the user's rows; K and V: its
  // candidate rows), so a lane with nothing to load passes an offset past the range and reads
  // zeros, with no branch (a branch per load made the compiler wait for each one).
  const bool q_c = MODE == kMaskDynamic && q_valid && qi >= rc_end;
  constexpr uint32_t kOut = 0x80000000u;         // past every range (rows span < 2^31 bytes)
  const int n_c = MODE == kMaskDynamic ? n - rc_end : 0;
  const __amdgpu_buffer_rsrc_t u_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Up, (short)0, (int)((uint32_t)n * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t kc_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Kp + (int64_t)rc_end * ld), (short)0, (int)((uint32_t)n_c * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t vc_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Vp + (int64_t)rc_end * ld), (short)0, (int)((uint32_t)n_c * row_bytes), 0x00020000);
  bf16x8 kr[DH / 16];
  const uint32_t k_off = q_c ? (uint32_t)(qi - rc_end) * row_bytes + hh * 16 : kOut;
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks)
    kr[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kc_rsrc, k_off, ks * 32, 0));
  constexpr int NE = 32 * CPR / 64;              // 16-byte output chunks per lane
  bf16x8 u8[NE], v8[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int idx = lane + 64 * e, ql = idx / CPR, c = idx % CPR, q = wq0 + ql;
    const uint32_t u_off = q < n ? (uint32_t)q * row_bytes + c * 16 : kOut;
    const uint32_t v_off = (MODE == kMaskDynamic && q < n && q >= rc_end) ? (uint32_t)(q - rc_end) * row_bytes + c * 16 : kOut;
    u8[e] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(u_rsrc, u_off, 0, 0));
    v8[e] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vc_rsrc, v_off, 0, 0));
  }

  // Stage this wavefront's O rows (fp32) in LDS, one tile buffer per wavefront (the key loop
  // ended with a barrier and no loads in flight, so they are free): element r of tile t is row
  // 8*(r/4)+4*hh+r%4, feature t*32 + l32, stored at column feature ^ (32 * ((row / 4) % 2)) of an
  // unpadded row so that the two lane halves write disjoint banks.
  float* Os = reinterpret_cast<float*>(w == 0 ? Ks0 : w == 1 ? Ks1 : w == 2 ? Vs0 : Vs1);
  float* Ps = Ps_all + w * 32;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      Os[(8 * (r >> 2) + 4 * hh + (r & 3)) * DH + ((t ^ hh) * 32 + l32)] = o[t][r];
  float part = 0.f;
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) part += (float)qf[ks][e] * (float)kr[ks][e];
  const float s_self = part + __shfl_xor(part, 32, kWave);
  const float p_self = q_c ? (float)(bf16)silu_rcp(s_self) : 0.f;
  if (hh == 0) Ps[l32] = p_self;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // y = (O + p_self v) / n (.) u, 8 features per lane step, 16-byte loads and stores.  Every
  // chunk's LDS reads are issued before the first one is used.
  const float inv_n = 1.0f / (float)n;
  f32x4 oa[NE][2];
  float pse[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int idx = lane + 64 * e, ql = idx / CPR, c = idx % CPR;
    const int col = (c * 8) ^ (32 * ((ql >> 2) & 1));
    oa[e][0] = *reinterpret_cast<const f32x4*>(&Os[ql * DH + col]);
    oa[e][1] = *reinterpret_cast<const f32x4*>(&Os[ql * DH + col + 4]);
    pse[e] = Ps[ql];
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int idx = lane + 64 * e, ql = idx / CPR, c = idx % CPR, q = wq0 + ql;
    if (q >= n) continue;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) { acc[i] = oa[e][0][i]; acc[i + 4] = oa[e][1][i]; }
    const float ps = pse[e];
    if (ps != 0.f) {   // a candidate row: its V row was loaded above
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += ps * (float)v8[e][i];
    }
    bf16x8 out;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (bf16)(acc[i] * inv_n * (float)u8[e][i]);
    if (vt) {   // the ungated V~ (kept for the backward pass)
      bf16x8 o2;
#pragma unroll
      for (int i = 0; i < 8; ++i) o2[i] = (bf16)(acc[i] * inv_n);
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
  constexpr int NW = kAttnFwdQTileBf16 / 32;
  if (dh == 128)
    k_attn_bf16<128, MODE, NW><<<grid, 64 * NW, 0, s>>>(B, H, d, offsets, seg, order, xcd_off, timestamps, qkvu, y, vt);
  else if (dh == 64)
    k_attn_bf16<64, MODE, NW><<<grid, 64 * NW, 0, s>>>(B, H, d, offsets, seg, order, xcd_off, timestamps, qkvu, y, vt);
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
