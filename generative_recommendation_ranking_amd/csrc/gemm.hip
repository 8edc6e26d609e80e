// Dense projections of the HSTU block on gfx950: the Q/K/V/U projection, the two MLP layers
// (with SiLU, and with the fp32 residual add), and the first layer of the candidate head
// (marovi.ai MTGR page, 方法, the block update equations).
//
//   out[M][N] = epi(a[M][K] . w[N][K]^T + bias[N])
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with fp32 accumulation, one persistent workgroup of 8
// wavefronts per CU walking 256 x 256 output tiles (wavefront tile 64 x 128); the K loop stages
// 64-wide slabs of a and w through two LDS buffers and keeps one software pipeline running across
// tile boundaries.  With both operands K-contiguous the slabs go from global memory straight into
// LDS (buffer loads with the LDS bit, XOR-swizzled rows) and every lane fetches the 8 consecutive
// k values of a fragment with one 16-byte LDS read; the k-major variant (weight gradients) stages
// through registers into padded rows and reads its fragments with transposing LDS reads.
//
// Where the time goes (large workload, Q/K/V/U projection 630,293 x 3072 x 768, about 2.9 ms):
// timing builds that skip one part each ran in 2.47 ms without the epilogue (2.55 ms without just
// its global stores), 2.32 ms without the weight DMA, 2.45 ms without the activation loads and
// 1.84 ms without both loads: the MFMA and LDS core runs at about 75% of peak, and the operand
// feed and the output stores are what the pipeline does not hide.  Tried without gain: a 2 x 2
// wavefront grid (128 x 128 per wavefront, one wavefront per SIMD: 10% slower), the slab DMA
// spread over the k-steps, workgroups started up to a few microseconds apart, the weights
// (instead of the activations) through registers, and each tile's slab 1 sent before the
// previous tile's epilogue with the staging moved out of the slab buffers.
//
// Workgroup order: MI355X dispatches consecutive workgroup ids round-robin to its 8 XCDs, each
// with a private L2.  Tiles are numbered so that every XCD walks its own M-tiles and, for each,
// all N-tiles back to back: each M-slab of `a` (the large, streamed operand) is then fetched
// from HBM into one L2 only, while the small weight matrix is shared through the MALL.
//
// fp32 path: a plain 64x64 register-tiled VALU kernel (used by the fp32 storage mode).
#include <algorithm>
#include <type_traits>

#include "../../include/mtgr.h"
#include "kernels.h"

namespace mtgr {

namespace {

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kXcd = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBiasLds = 4096;  // bias entries staged in LDS by the persistent bf16 GEMM
// one slab buffer of the DMA pipeline: 512 rows of 128 bytes plus a gap, 8 x 32 rows of 272 bytes
constexpr int kDmaBufBytes = 8 * 32 * 272;
static_assert(kDmaBufBytes >= 512 * 128, "DMA slab buffer");

// 16 bytes per lane from a buffer resource straight into LDS: lane l writes lds + 16 l; lanes
// past the resource's end write zeros
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// wait until at most N vector memory operations of this wavefront are outstanding
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

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

// Persistent variant: one workgroup per CU walks its share of output tiles and streams the
// K-slabs of consecutive tiles through one software pipeline, so the first loads of the next tile
// are in flight while the current tile finishes and stores its results.
//   * WM x WN wavefronts, 256 x 256 tile, BK = 64 (4 MFMA k-steps per slab), two LDS buffers.
//   * Global loads are buffer loads whose resource starts at the tile's first row and whose size
//     stops at M (N): rows past the end read as zero, and per-chunk offsets live in SGPRs.
//   * Per slab: the fragments of k-step ks+1 are read while the MFMAs of k-step ks run, and one
//     barrier per slab publishes the next slab and frees the buffer of the last one.
//   * K-contiguous operands: the next slab goes into the free buffer by DMA at the start of a
//     slab, the activation rows of most slabs through registers two slabs ahead (see the DMA
//     pipeline below).  k-major operands: the slab after next is fetched into registers after
//     k-step 1 and written to LDS one slab later.
// KMAJOR: both operands token-major (k-major) for weight gradients, out[m][n] = sum_t A[t][m] W[t][n] over the
// token axis K (t_rows real rows, the rest read as zero), A and W with row pitches lda and ldb;
// the slab is staged as [k][m] / [k][n] and the MFMA fragments come from transposing LDS reads.
// Split K with a split count that is a multiple of the XCD count: every tile of a split runs on
// one XCD, so the split's A and W slabs are fetched into that XCD's L2 once and shared by all of
// its row and column tiles.
template <int WM, int WN, int EPI, typename TOut, bool KMAJOR = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void k_gemm_bf16_persistent(
    int64_t M, int N, int K, const bf16* __restrict__ A, const bf16* __restrict__ W,
    const bf16* __restrict__ bias, const float* resid, TOut* out, int nN, int64_t nM, int nb,
    int ksplit, int64_t nMr, int64_t t_rows, int lda, int ldb, void* aux) {
  constexpr int BM = 256, BN = 256, BK = 64, NT = 64 * WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int LP = BK + 8, CPR = BK / 8;
  constexpr int CA = BM * CPR / NT, CB = BN * CPR / NT;   // 4 and 4 chunks per thread
  constexpr int RSTEP = NT / CPR;                          // rows covered by one chunk index

  // DMA: slabs of a and w go from global memory straight into LDS (K-contiguous operands only).
  // Buffer b then holds [BM rows of a][BN rows of w], 128-byte rows without padding, the 16-byte
  // chunk c of row r at position c ^ ((r >> 1) & 7), which keeps 16-byte fragment reads of 32
  // consecutive rows on distinct banks, followed by a gap that lets the epilogue stage 8 x 32
  // rows at its padded pitch in the buffer and its gap.
  constexpr bool DMA = !KMAJOR;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16 (*As)[BM][LP] = reinterpret_cast<bf16 (*)[BM][LP]>(smem);
  bf16 (*Bs)[BN][LP] = reinterpret_cast<bf16 (*)[BN][LP]>(smem + 2 * BM * LP * sizeof(bf16));
  // Bias table in LDS: the whole vector when N <= kBiasLds (staged once), else the current
  // tile's slice (staged at the start of each tile).  It seeds the accumulators.
  constexpr int kSlabBytes = DMA ? kDmaBufBytes : (BM + BN) * LP * (int)sizeof(bf16);
  bf16* Bias = reinterpret_cast<bf16*>(smem + 2 * kSlabBytes);
  constexpr int TP = BM + 32;   // k-major slabs [BK][BM + 32]: the same bytes as [BM][LP]; a pitch of 16
                                // (mod 64) dwords keeps the transposing reads conflict-free
  static_assert(BK * TP == BM * LP && BN == BM, "k-major slab layout");
  bf16 (*At)[BK][TP] = reinterpret_cast<bf16 (*)[BK][TP]>(smem);
  bf16 (*Bt)[BK][TP] = reinterpret_cast<bf16 (*)[BK][TP]>(smem + 2 * BM * LP * sizeof(bf16));
  const bool bias_whole = bias != nullptr && N <= kBiasLds;
  const bool bias_slice = bias != nullptr && N > kBiasLds;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hh = lane >> 5;

  // Tile sequence.  Workgroup ids reach the XCDs round-robin; XCD x owns M-tiles x, x+8, ...
  // and walks N in chunks of nb tiles (outer) and its M-tiles (inner), so while a chunk is being
  // processed only nb weight slices are live in that XCD's L2 and the activation slabs stream
  // through once per chunk.  nb is chosen by the host from an estimate of L2-miss traffic.
  const int xcd = (int)(blockIdx.x % kXcd);
  const int gx = (int)(gridDim.x / kXcd);
  const int64_t nMx = (nM + kXcd - 1) / kXcd;
  const int64_t nslots = nMx * nN;
  const int nchunk_full = nN / nb;                  // chunks of exactly nb tiles; the last may be short
  auto decode = [&](int64_t s, int64_t& m_tile, int& n_tile) {
    const int64_t per = nMx * nb;                   // slots per full chunk
    int64_t c = s / per;
    int64_t rem = s - c * per;
    int w = nb;
    if (c >= nchunk_full) { c = nchunk_full; rem = s - c * per; w = nN - nchunk_full * nb; }
    m_tile = (rem / w) * kXcd + xcd;
    n_tile = (int)(c * nb + rem % w);
  };
  auto valid_slot = [&](int64_t s) {
    if (s >= nslots) return false;
    int64_t m; int n; decode(s, m, n);
    return m < nM;
  };
  auto next_slot = [&](int64_t s) {  // next slot of this workgroup holding a real tile
    s += gx;
    while (s < nslots && !valid_slot(s)) s += gx;
    return s;
  };
  int64_t first = blockIdx.x / kXcd;
  if (!valid_slot(first)) first = next_slot(first);
  if (first >= nslots) return;

  // Split K: M-tile index mt in [0, nM) stands for a row tile r over the K range of split sp,
  // [sp * nk * BK, + nk * BK), written to out + sp * M * N (no bias then).  Split-major order (split
  // count a multiple of the XCD count): XCD x = mt % kXcd holds splits x, x + kXcd, ..., each with
  // all its row tiles; otherwise sp = mt / nMr, r = mt % nMr.
  const int nk = K / BK / ksplit;        // >= 2 (checked by the host)
  const bool split_major = KMAJOR && ksplit > 1 && ksplit % kXcd == 0;   // (k-major GEMMs only)
  auto split_row = [&](int64_t mt, int& sp, int64_t& r) {
    if (split_major) {
      const int64_t j = mt / kXcd;
      sp = (int)((j / nMr) * kXcd + mt % kXcd);
      r = j % nMr;
    } else {
      sp = (int)(mt / nMr);
      r = mt % nMr;
    }
  };
  const uint32_t vo = KMAJOR ? 0u : (uint32_t)((tid / CPR) * K * 2 + (tid % CPR) * 16);  // byte offset in slab
  // k-major: thread -> (token row tid/32 of 16, 16-byte chunk tid%32 of a 512-byte row segment)
  const uint32_t vo_a = KMAJOR ? (uint32_t)((tid >> 5) * lda * 2 + (tid & 31) * 16) : 0u;
  const uint32_t vo_b = KMAJOR ? (uint32_t)((tid >> 5) * ldb * 2 + (tid & 31) * 16) : 0u;

  struct TileRsrc {
    __amdgpu_buffer_rsrc_t a, w;
  };
  auto make_rsrc = [&](int64_t s) {
    int64_t mt; int ntile; decode(s, mt, ntile);
    int sp; int64_t rt;
    split_row(mt, sp, rt);
    const int ks_off = sp * nk * BK;
    const int64_t m0 = rt * BM;
    const int n0 = ntile * BN;
    const int64_t mrows = min((int64_t)BM, M - m0);
    const int nrows = min(BN, N - n0);
    TileRsrc r;
    if constexpr (KMAJOR) {
      // the split's token rows [ks_off, ks_off + nk*BK), clipped at t_rows; the resources start at
      // the tile's first column and end where the split's last real row ends, so padding rows read
      // as zero (columns past M or N read neighbouring data that only reaches dropped outputs)
      const int64_t rows = max((int64_t)0, min(t_rows, (int64_t)ks_off + (int64_t)nk * BK) - ks_off);
      const int64_t abytes = max((int64_t)0, (rows * lda - m0) * 2);
      const int64_t wbytes = max((int64_t)0, (rows * ldb - n0) * 2);
      r.a = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)ks_off * lda + m0), (short)0, (int)abytes, 0x00020000);
      r.w = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)ks_off * ldb + n0), (short)0, (int)wbytes, 0x00020000);
    } else {
      // the resources start at column ks_off of the first row; they end where row mrows (nrows)
      // would begin, so rows past the edge still read as zero
      r.a = __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * K + ks_off), (short)0,
                                              (int)((mrows * K - ks_off) * 2), 0x00020000);
      r.w = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)n0 * K + ks_off), (short)0,
                                              (int)(((int64_t)nrows * K - ks_off) * 2), 0x00020000);
    }
    return r;
  };
  bf16x8 ra[CA], rb[CB];
  auto issue_loads = [&](const TileRsrc& r, int kt) {
    if constexpr (KMAJOR) {
      static_assert(CA == BK / 16 && CB == BK / 16, "k-major staging: 16 token rows per pass");
#pragma unroll
      for (int i = 0; i < CA; ++i)
        ra[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               r.a, vo_a, (uint32_t)(kt * BK + i * 16) * (uint32_t)lda * 2u, 0));
#pragma unroll
      for (int i = 0; i < CB; ++i)
        rb[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               r.w, vo_b, (uint32_t)(kt * BK + i * 16) * (uint32_t)ldb * 2u, 0));
    } else {
      const int kb = kt * BK * 2;
#pragma unroll
      for (int i = 0; i < CA; ++i)
        ra[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r.a, vo, i * RSTEP * K * 2 + kb, 0));
#pragma unroll
      for (int i = 0; i < CB; ++i)
        rb[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r.w, vo, i * RSTEP * K * 2 + kb, 0));
    }
  };
  auto store_slab = [&](int buf) {
    if constexpr (KMAJOR) {
      const int row = tid >> 5, c8 = (tid & 31) * 8;
#pragma unroll
      for (int i = 0; i < CA; ++i) *reinterpret_cast<bf16x8*>(&At[buf][row + 16 * i][c8]) = ra[i];
#pragma unroll
      for (int i = 0; i < CB; ++i) *reinterpret_cast<bf16x8*>(&Bt[buf][row + 16 * i][c8]) = rb[i];
    } else {
#pragma unroll
      for (int i = 0; i < CA; ++i)
        *reinterpret_cast<bf16x8*>(&As[buf][tid / CPR + i * RSTEP][(tid % CPR) * 8]) = ra[i];
#pragma unroll
      for (int i = 0; i < CB; ++i)
        *reinterpret_cast<bf16x8*>(&Bs[buf][tid / CPR + i * RSTEP][(tid % CPR) * 8]) = rb[i];
    }
  };
  // Software pipeline over the K slabs of this workgroup's tiles, one after another: slab g is
  // in LDS buffer g%2 and the fragments of k-step ks+1 are read before the MFMAs of k-step ks.
  // Within slab g: after the MFMAs of k-step 1 the registers holding slab g+1 are written to the
  // other buffer and the loads of slab g+2 are issued (from the next tile once this tile's slabs
  // run out), so a load has a whole slab of MFMAs to arrive; after the MFMAs of k-step 2 one
  // barrier (LDS traffic only, global loads stay in flight) publishes slab g+1 and retires every
  // read of slab g's buffer before it is overwritten; during k-step 3 the first fragments of slab
  // g+1 are read, so the slab boundary exposes no LDS latency (at a tile boundary they are read
  // after the epilogue instead).  The loads run at most two slabs
  // ahead, so with at least two slabs per tile they only touch this tile or the next one.
  constexpr int KS = BK / 16;
  static_assert(KS == 4, "the schedule below assumes four k-steps per slab");
  bf16x8 fa[2][FM], fb[2][FN];
  // k-major fragments: the 16 k of k-step ks come from two transposing reads of 4 rows each,
  // rows kb + 4*hh + e%4 (+8 for e >= 4); A and B take the same k order, so the contraction holds
  auto tr_frag = [&](const bf16 (*tile)[TP], int ks, int col0) {
    const int kb = (ks >> 1) * 32 + (ks & 1) * 16 + 4 * hh + (lane & 15) / 4;
    const int fc = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&tile[kb][fc]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&tile[kb + 8][fc]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_frags = [&](int buf, int ks, int fslot) {
    if constexpr (KMAJOR) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[fslot][i] = tr_frag(At[buf], ks, wm * TM + i * 32);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[fslot][j] = tr_frag(Bt[buf], ks, wn * TN + j * 32);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[fslot][i] = *reinterpret_cast<const bf16x8*>(&As[buf][wm * TM + i * 32 + l32][ks * 16 + hh * 8]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[fslot][j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][wn * TN + j * 32 + l32][ks * 16 + hh * 8]);
    }
    // keep the reads ahead of the MFMAs that follow (the scheduler would otherwise sink them)
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  int64_t slot = first;
  int64_t next = next_slot(slot);
  TileRsrc r_cur = make_rsrc(slot);
  TileRsrc r_nxt = (next < nslots) ? make_rsrc(next) : r_cur;

  // prologue: the bias slice table, slab 0 into LDS buffer 0, slab 1 into registers
  if (bias_whole) {
    for (int i = tid; i < N; i += NT) Bias[i] = bias[i];
  }
  bool have_next = true;   // registers hold a slab still to be written to LDS
  if constexpr (!DMA) {
    issue_loads(r_cur, 0);
    store_slab(0);
    issue_loads(r_cur, 1);
    lds_barrier();
    read_frags(0, 0, 0);
  }

  int cur = 0;
  bool more_tiles = next < nslots;
  f32x16 acc[FM][FN];
  // The accumulators start at the bias of their columns (element r of MFMA tile j holds column
  // j*32 + 8(r/4) + 4hh + r%4 of the wavefront tile), so the epilogue never touches the bias.
  auto init_acc = [&] {
    if (!bias) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
      return;
    }
    int64_t mt_i; int nt_i; decode(slot, mt_i, nt_i);
    const int n0 = nt_i * BN;
    const bf16* btab = Bias;
    if (bias_slice) {
      // every wavefront passed a barrier after its last read of the previous slice
      for (int i = tid; i < BN; i += NT) Bias[i] = n0 + i < N ? bias[n0 + i] : (bf16)0.f;
      lds_barrier();
      btab = Bias - n0;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // columns past N are clamped to a valid entry; their results are dropped
        const int n = min(n0 + wn * TN + j * 32 + 8 * g + 4 * hh, N - 4);
        const bf16x4 b4 = *reinterpret_cast<const bf16x4*>(&btab[n]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j][4 * g + e] = (float)b4[e];
      }
  };
  auto mfmas = [&](int fs) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fs][j], fa[fs][i], acc[i][j], 0, 0, 0);
  };
  auto slab = [&](int kt) {
    const bool cont = kt + 1 < nk || more_tiles;
    read_frags(cur, 1, 1);
    mfmas(0);
    read_frags(cur, 2, 0);
    mfmas(1);
    if (have_next) store_slab(cur ^ 1);
    {
      // slab kt+2 of this tile, else slab kt+2-nk of the next tile
      const bool here = kt + 2 < nk;
      have_next = here || more_tiles;
      if (have_next) issue_loads(here ? r_cur : r_nxt, here ? kt + 2 : kt + 2 - nk);
    }
    read_frags(cur, 3, 1);
    mfmas(0);
    if (cont) {
      lds_barrier();
      // the next tile's first fragments are read after the epilogue, which needs the registers
      if (kt + 1 < nk) read_frags(cur ^ 1, 0, 0);
    }
    mfmas(1);
    if (cont) cur ^= 1;
  };

  // Epilogue.  An MFMA tile leaves each lane 4 consecutive columns of one row, so stores straight
  // from registers would write 16-byte pieces of 32 different rows per instruction; instead each
  // wavefront passes its results through a private region of the LDS slab buffer that the next
  // tile does not use yet, 32 rows at a time, and writes whole 256-byte row segments with 16-byte
  // stores (the residual rows of the fp32 variant are read the same way).  Vector memory
  // operations retire in order, so a wait for a load also waits for every store issued before it:
  // the bias is already in the accumulators, the residual chunks of a pass are requested one pass
  // ahead (before the previous pass's stores), and every lane issues the same fixed number of
  // stores whatever the tile's edges (the resource ends at the tile's last valid row; chunks past
  // column N get an offset beyond it and are dropped), so the compiler can also count past them
  // when it waits for the next tile's prefetched slab.
  constexpr uint32_t kDrop = 0x80000000u;   // > any valid byte offset (N <= 2^20, 256 rows)
  // the output rows are written once and not read again by this kernel: non-temporal stores keep
  // them from displacing the activation slabs that later column tiles re-read from L2
  constexpr int kStoreNT = 2;
  constexpr int SP = 272;                    // staging row pitch, bytes (16-byte aligned, 4-bank skew)
  // staged element type: the output type, except the SiLU-backward epilogue, which stages fp32
  // and finishes the product with silu'(a) on the way out
  using TS = std::conditional_t<EPI == kEpiSiluBwd, float, TOut>;
  constexpr int CPS = sizeof(TS) == 2 ? 4 : 2;     // MFMA column tiles per pass: 256 bytes of row
  constexpr int NPASS = FM * FN / CPS;
  constexpr int CW = 16 / (int)sizeof(TS);         // columns per 16-byte staged chunk
  static_assert(DMA ? WM * WN * 32 * SP <= kDmaBufBytes : (NT == 512 && 32 * SP <= BM * LP * (int)sizeof(bf16) / 4),
                "each wavefront stages 32 rows in a quarter of one operand buffer, or a share of one DMA buffer");
  // byte offset of this lane's first chunk inside a wavefront tile (row lane/16, 16-byte chunk
  // lane%16)
  const uint32_t lane_off =
      ((uint32_t)(wm * TM + (lane >> 4)) * (uint32_t)N + (uint32_t)(wn * TN + (lane & 15) * CW)) * (uint32_t)sizeof(TOut);
  auto epilogue = [&] {
    int64_t mt_e; int nt_e; decode(slot, mt_e, nt_e);
    int sp_e; int64_t rt_e;
    split_row(mt_e, sp_e, rt_e);
    TOut* outp = out + sp_e * M * N;
    const int64_t m0 = rt_e * BM;
    const int n0 = nt_e * BN;
    const uint32_t rows = (uint32_t)min((int64_t)BM, M - m0);
    const int nbytes = (int)(rows * (uint32_t)N * sizeof(TOut));
    // row scatter: the resource spans the whole destination [t_rows][N]; rows come from the map
    const __amdgpu_buffer_rsrc_t o_rsrc =
        EPI == kEpiRowScatter
            ? __builtin_amdgcn_make_buffer_rsrc((void*)outp, (short)0, (int)(t_rows * N * (int64_t)sizeof(TOut)), 0x00020000)
            : __builtin_amdgcn_make_buffer_rsrc((void*)(outp + m0 * N), (short)0, nbytes, 0x00020000);
    __amdgpu_buffer_rsrc_t r_rsrc = o_rsrc;
    if constexpr (EPI == MTGR_EPI_RESIDUAL_F32)
      r_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(resid + m0 * N), (short)0, nbytes, 0x00020000);
    if constexpr (EPI == kEpiSiluBwd)   // the pre-activation a, read and overwritten with silu(a)
      r_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<bf16*>(aux) + m0 * N), (short)0, nbytes, 0x00020000);
    // this wavefront's staging region in the buffer the last slab used: a quarter of its operand
    // buffer, or an eighth of the DMA buffer with its gap
    char* stage = DMA ? reinterpret_cast<char*>(smem) + (cur ^ 1) * kSlabBytes + wave * (32 * SP)
                      : (wave < 4 ? reinterpret_cast<char*>(&As[cur ^ 1][0][0])
                                  : reinterpret_cast<char*>(&Bs[cur ^ 1][0][0])) + (wave & 3) * (BM * LP * (int)sizeof(bf16) / 4);
    // fp32 residual chunks of pass pp (the same layout as the pass's stores), requested one pass
    // ahead: a pass's residual loads then precede the previous pass's stores, so waiting for them
    // does not wait for those stores
    auto load_resid = [&](int pp, f32x4 (&dst)[8]) {
      const int ip = pp / (FN / CPS), jp = (pp % (FN / CPS)) * CPS;
      const bool ok = n0 + wn * TN + jp * 32 + (lane & 15) * CW < N;
#pragma unroll
      for (int it = 0; it < 8; ++it)
        dst[it] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
            r_rsrc, ok ? lane_off : kDrop, (uint32_t)((ip * 32 + it * 4) * N + n0 + jp * 32) * (uint32_t)sizeof(TOut), 0));
    };
    f32x4 rq_next[8];
    if constexpr (EPI == MTGR_EPI_RESIDUAL_F32) load_resid(0, rq_next);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      // (one pass at a time: the accumulators of later passes stay where they are)
      __builtin_amdgcn_sched_barrier(0);
      const int i = p / (FN / CPS), j0 = (p % (FN / CPS)) * CPS;
      // Chunk it of this lane covers row i*32 + it*4 + lane/16 of the wavefront tile and columns
      // j0*32 + (lane%16)*CW .. +CW-1: a per-lane byte offset (one VGPR, or kDrop when the chunk
      // lies past column N) plus a wavefront-uniform offset in an SGPR.
      const bool col_ok = n0 + wn * TN + j0 * 32 + (lane & 15) * CW < N;
      const uint32_t vo_c = col_ok ? lane_off : kDrop;
      auto s_off = [&](int it) {
        return (uint32_t)((i * 32 + it * 4) * N + n0 + j0 * 32) * (uint32_t)sizeof(TOut);
      };
      // A VALU write to the data registers of a >8-byte buffer store needs a wait state after
      // the store; the compiler omits it when the store's SGPR offset field holds a register, but
      // gfx950 corrupts the stored data without it, so it is inserted here.
      auto store_chunk = [&](u32x4 c, int it) {
        __builtin_amdgcn_raw_buffer_store_b128(c, o_rsrc, vo_c, s_off(it), kStoreNT);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 1");
        __builtin_amdgcn_sched_barrier(0);
      };
      f32x4 rq[8];
      if constexpr (EPI == MTGR_EPI_RESIDUAL_F32) {
#pragma unroll
        for (int it = 0; it < 8; ++it) rq[it] = rq_next[it];
        if (p + 1 < NPASS) load_resid(p + 1, rq_next);
      }
      u32x2 za[8];
      if constexpr (EPI == kEpiSiluBwd) {
#pragma unroll
        for (int it = 0; it < 8; ++it) za[it] = __builtin_amdgcn_raw_buffer_load_b64(r_rsrc, vo_c, s_off(it), 0);
      }
      // row scatter: destination row of each chunk (-1: none), read before the pass's stores
      uint32_t vo_r[8];
      if constexpr (EPI == kEpiRowScatter) {
        const int32_t* rowmap = static_cast<const int32_t*>(aux);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int64_t gr = m0 + wm * TM + i * 32 + it * 4 + (lane >> 4);
          const int32_t dst = (gr < M) ? rowmap[gr] : -1;
          vo_r[it] = (dst >= 0 && col_ok)
                         ? ((uint32_t)dst * (uint32_t)N + (uint32_t)(n0 + wn * TN + j0 * 32 + (lane & 15) * CW)) * (uint32_t)sizeof(TOut)
                         : kDrop;
        }
      }
      // registers -> LDS: row l32, columns jj*32 + 8g + 4hh .. +3 of this pass
#pragma unroll
      for (int jj = 0; jj < CPS; ++jj) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cl = jj * 32 + 8 * g + 4 * hh;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j0 + jj][4 * g + e];
          if constexpr (EPI == MTGR_EPI_SILU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = silu_rcp(v[e]);
          }
          char* dst = stage + l32 * SP + cl * (int)sizeof(TS);
          if constexpr (sizeof(TS) == 4) {
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = v[e];
            *reinterpret_cast<f32x4*>(dst) = o;
          } else {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
            *reinterpret_cast<bf16x4*>(dst) = o;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // LDS -> global: 32 rows x 256 bytes = 512 chunks, 8 per lane, in two groups of four to
      // bound the registers in flight
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        if (it == 4) __builtin_amdgcn_sched_barrier(0);
        const int q = it * 64 + lane;
        u32x4 c = *reinterpret_cast<const u32x4*>(stage + (q / 16) * SP + (q % 16) * 16);
        if constexpr (EPI == MTGR_EPI_RESIDUAL_F32) {
          f32x4 f = __builtin_bit_cast(f32x4, c);
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] += rq[it][e];
          c = __builtin_bit_cast(u32x4, f);
        }
        if constexpr (EPI == kEpiSiluBwd) {
          // da = acc (.) silu'(a), silu'(z) = s (1 + z (1 - s)), s = sigmoid(z); a <- silu(a) = z s
          const f32x4 f = __builtin_bit_cast(f32x4, c);
          const bf16x4 z4 = __builtin_bit_cast(bf16x4, za[it]);
          bf16x4 d4, h4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = (float)z4[e];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
            d4[e] = (bf16)(f[e] * (sg * (1.0f + z * (1.0f - sg))));
            h4[e] = (bf16)(z * sg);
          }
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, d4), o_rsrc, vo_c, s_off(it), 0);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h4), r_rsrc, vo_c, s_off(it), 0);
        } else if constexpr (EPI == kEpiRowScatter) {
          __builtin_amdgcn_raw_buffer_store_b128(c, o_rsrc, vo_r[it], 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("s_nop 1");
          __builtin_amdgcn_sched_barrier(0);
        } else {
          store_chunk(c, it);
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // the next slab write reuses the staging buffer: every wavefront must be done with it
    lds_barrier();
  };

  // The tile loop is rotated so that each epilogue runs straight into the first slab of the next
  // tile with no control-flow merge between them (a merge would make the compiler's wait before
  // that slab's LDS write conservative again).
  if constexpr (!DMA) {
    init_acc();
    for (int kt = 0; kt < nk; ++kt) slab(kt);
    while (true) {
      epilogue();
      if (!more_tiles) break;
      slot = next;
      next = next_slot(slot);
      r_cur = r_nxt;
      if (next < nslots) r_nxt = make_rsrc(next);
      more_tiles = next < nslots;
      init_acc();
      read_frags(cur, 0, 0);
      slab(0);
      for (int kt = 1; kt < nk; ++kt) slab(kt);
    }
  } else {
    // DMA pipeline.  Phase kt runs from the barrier that published slab kt to the one that
    // publishes slab kt+1.  At its start the buffer of slab kt-1 is free (its last fragments were
    // read before that barrier; in a tile's first phase it is the epilogue's staging area, free
    // after the epilogue's barrier) and receives slab kt+1 by DMA, or in a tile's last phase the
    // next tile's slab 0, which then has the whole phase to land; the phase waits for it (vmcnt)
    // just before its closing barrier.  The buffers are passed to each phase as restrict views,
    // which tells the compiler that the reads of one buffer do not wait for the DMA into the other.
    bf16* const buf0 = reinterpret_cast<bf16*>(smem);
    auto abuf = [&](int b) { return buf0 + b * (kSlabBytes / (int)sizeof(bf16)); };
    auto bbuf = [&](int b) { return abuf(b) + BM * BK; };
    // wavefront w moves rows [RW w, RW (w + 1)) of both operands, 8 rows per instruction: lane l
    // takes row 8i + l/8 and LDS position l%8, i.e. global chunk (l%8) ^ swizzle(row), where the
    // swizzle of row RW w + 8i + j is 4(i&1) + j/2
    constexpr int RW = BM / (WM * WN);
    static_assert(BM == BN && RW % 16 == 0, "DMA row split");
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int j8 = lane >> 3, c8 = lane & 7;
    const uint32_t dvo0 = (uint32_t)(j8 * K * 2 + ((c8 ^ (j8 >> 1)) << 4));
    const uint32_t dvo1 = (uint32_t)(j8 * K * 2 + ((c8 ^ (4 + (j8 >> 1))) << 4));
    constexpr int NDI = RW / 8;   // DMA instructions per operand and wavefront
    auto dma_slab = [&](const TileRsrc& r, int kt, bf16* __restrict__ da, bf16* __restrict__ db, bool with_a) {
#pragma unroll
      for (int i = 0; i < NDI; ++i) {
        const int row = wu * RW + i * 8;
        const uint32_t so = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)(kt * BK * 2);
        if (with_a) lds_dma16(r.a, da + row * BK, (i & 1) ? dvo1 : dvo0, so);
        lds_dma16(r.w, db + row * BK, (i & 1) ? dvo1 : dvo0, so);
      }
    };
    // Activation slabs 2 .. nk-1 of a tile come through registers two phases ahead (register set
    // s & 1 holds slab s): thread t loads chunk t%8 of rows t/8 + 64i and writes it to its swizzled
    // position, (t/16) & 7 being the swizzle of those rows.
    bf16x8 rA[2][CA];
    const uint32_t a_vo = (uint32_t)((tid >> 3) * K * 2 + (tid & 7) * 16);
    const int s_row = tid >> 3, s_ch = ((tid & 7) ^ ((tid >> 4) & 7)) * 8;
    auto load_a = [&](auto set, int kt) {
      constexpr int S = decltype(set)::value;
#pragma unroll
      for (int i = 0; i < CA; ++i)
        rA[S][i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                  r_cur.a, a_vo, (uint32_t)(i * RSTEP * K * 2 + kt * BK * 2), 0));
    };
    auto store_a = [&](auto set, bf16* __restrict__ da) {
      constexpr int S = decltype(set)::value;
#pragma unroll
      for (int i = 0; i < CA; ++i) *reinterpret_cast<bf16x8*>(da + (s_row + i * RSTEP) * BK + s_ch) = rA[S][i];
    };
    // rows of a wavefront's fragments are 32-aligned plus l32, so their swizzle is (l32/2) & 7
    const int f_sw = (l32 >> 1) & 7;
    auto read_frags_d = [&](const bf16* pa, const bf16* pb, int ks, int fslot, bool fence = true) {
      const int ch = ((2 * ks + hh) ^ f_sw) * 8;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[fslot][i] = *reinterpret_cast<const bf16x8*>(pa + (wm * TM + i * 32 + l32) * BK + ch);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[fslot][j] = *reinterpret_cast<const bf16x8*>(pb + (wn * TN + j * 32 + l32) * BK + ch);
      if (fence) __builtin_amdgcn_sched_barrier(0);
    };
    // kind 0: first phase of a tile (its k-step 0 fragments are already in slot 0), 1: a middle
    // phase, 2: the last phase of a tile; P: the parity of kt (the register set it loads into)
    auto phase = [&](auto kind, auto par, int kt, const bf16* __restrict__ pa, const bf16* __restrict__ pb,
                     bf16* __restrict__ qa, bf16* __restrict__ qb) __attribute__((always_inline)) {
      constexpr int KIND = decltype(kind)::value, P = decltype(par)::value;
      const bool load_next = KIND != 2 && kt + 2 < nk;   // activation slab kt+2 into registers
      // Bracket b: the fragments of k-step b are read while the MFMAs of k-step b-1 run (k-step 3
      // of the previous slab for b = 0), each read issued right after one MFMA; bracket 0 also
      // issues the phase's global loads, one after each of its remaining MFMAs.
      auto bracket = [&](auto bc) {
        constexpr int B = decltype(bc)::value;
        constexpr int NV = B == 0 ? (KIND == 1 ? NDI : 2 * NDI) + (KIND == 2 ? 0 : CA) : 0;
        constexpr int NM = (KIND == 0 && B == 0) ? 0 : FM * FN;
        constexpr int NR = (KIND == 0 && B == 0) ? 0 : FM + FN;
        if constexpr (NR > 0) read_frags_d(pa, pb, B, B & 1, false);
        if constexpr (NM > 0) mfmas((B + 1) & 1);
        if constexpr (B == 0) {
          // slab kt+1 by DMA (its activation rows too in a tile's first phase), or the next
          // tile's slab 0 in its last phase
          if constexpr (KIND != 2) dma_slab(r_cur, kt + 1, qa, qb, KIND == 0);
          if constexpr (KIND == 2) {
            if (more_tiles) dma_slab(r_nxt, 0, qa, qb, true);
          }
          if (load_next) load_a(std::integral_constant<int, P>{}, kt + 2);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // one MFMA
          if (m < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);           // one LDS read
          if (m >= NM - NV) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);     // one global load
        }
        if constexpr (NV > NM) __builtin_amdgcn_sched_group_barrier(0x010, NV - NM, 0);
        __builtin_amdgcn_sched_barrier(0);
      };
      bracket(std::integral_constant<int, 0>{});
      bracket(std::integral_constant<int, 1>{});
      bracket(std::integral_constant<int, 2>{});
      bracket(std::integral_constant<int, 3>{});
      if (KIND != 2 || more_tiles) {
        __builtin_amdgcn_sched_barrier(0);   // the phase's MFMAs issue before the wait
        // everything but the activation loads just issued: this phase's DMA and, in a middle
        // phase, the registers of slab kt+1, which then go to LDS
        if (load_next) wait_vm<CA>();
        else wait_vm<0>();
        if constexpr (KIND == 1) store_a(std::integral_constant<int, P ^ 1>{}, qa);
        lds_barrier();
      }
    };
    // the buffer addresses are formed anew in every phase (an opaque copy of `cur`), which keeps
    // the compiler from holding both buffers' fragment addresses in registers across the loop
    auto phase_at = [&](auto kind, auto par, int kt) __attribute__((always_inline)) {
      int c = __builtin_amdgcn_readfirstlane(cur);
      asm volatile("" : "+s"(c));
      phase(kind, par, kt, abuf(c), bbuf(c), abuf(c ^ 1), bbuf(c ^ 1));
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    auto run_tile = [&]() __attribute__((always_inline)) {
      phase_at(I0{}, I0{}, 0);
      cur ^= 1;
      // middle phases 1 .. nk-2 in pairs (odd kt, then even), so each names its register sets
      // at compile time
      int kt = 1;
      for (; kt + 2 < nk; kt += 2) {
        phase_at(I1{}, I1{}, kt);
        cur ^= 1;
        phase_at(I1{}, I0{}, kt + 1);
        cur ^= 1;
      }
      if (kt + 1 < nk) {
        phase_at(I1{}, I1{}, kt);
        cur ^= 1;
      }
      phase_at(I2{}, I0{}, nk - 1);
      if (more_tiles) cur ^= 1;
      mfmas(1);   // k-step 3 of the last slab
    };
    // prologue: slab 0 by DMA into buffer 0
    dma_slab(r_cur, 0, abuf(0), bbuf(0), true);
    wait_vm<0>();
    lds_barrier();
    init_acc();
    read_frags_d(abuf(0), bbuf(0), 0, 0);
    run_tile();
    while (true) {
      epilogue();
      if (!more_tiles) break;
      slot = next;
      next = next_slot(slot);
      r_cur = r_nxt;
      if (next < nslots) r_nxt = make_rsrc(next);
      more_tiles = next < nslots;
      init_acc();
      read_frags_d(abuf(cur), bbuf(cur), 0, 0);
      run_tile();
    }
  }
}

// grid.z > 1 splits K: block z sums over k in [z*K/gz, (z+1)*K/gz) (K a multiple of gz) and
// writes its partial (EPI_STORE only) to out + z*M*N.
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
  const int kc = K / (int)gridDim.z;
  const int kbeg = (int)blockIdx.z * kc, kfin = kbeg + kc;
  out += (int64_t)blockIdx.z * M * N;
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kfin; k0 += BK) {
    {
      const int r = tid / 4, c4 = (tid % 4) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = k0 + c4 + e;
        const int64_t m = m0 + r;
        const int n = n0 + r;
        As[c4 + e][r] = (m < M && k < kfin) ? A[m * K + k] : 0.f;
        Ws[c4 + e][r] = (n < N && k < kfin) ? W[(int64_t)n * K + k] : 0.f;
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

struct KMajorArgs {
  int64_t t_rows = 0;
  int lda = 0, ldb = 0;
};

template <int WM, int WN, int EPI, typename TOut, bool KMAJOR = false>
hipError_t run_bf16_persistent(int64_t M, int N, int K, const bf16* a, const bf16* w,
                               const bf16* bias, const float* resid, void* out, hipStream_t s,
                               int ksplit = 1, KMajorArgs km = KMajorArgs(), void* aux = nullptr) {
  constexpr size_t lds = (!KMAJOR ? 2 * (size_t)kDmaBufBytes : 2 * (size_t)(256 + 256) * (64 + 8) * sizeof(bf16)) +
                         kBiasLds * sizeof(bf16);
  auto kern = k_gemm_bf16_persistent<WM, WN, EPI, TOut, KMAJOR>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int nN = (N + 255) / 256;
  const int64_t nMr = (M + 255) / 256;
  const int64_t nM = nMr * ksplit;
  const int64_t tiles_pad = (nM + kXcd - 1) / kXcd * kXcd * nN;
  const int64_t grid = std::min<int64_t>(tiles_pad, (int64_t)cus / kXcd * kXcd);
  // N-chunk width: estimated bytes missing a 4 MB XCD L2, activations re-read once per chunk
  // versus weights re-read once per round of concurrently running M-tiles when they do not fit.
  const double a_bytes = (double)M * K * 2, slice = 256.0 * (K / ksplit) * 2, l2 = 4.0 * 1024 * 1024;
  const double wg_per_xcd = (double)grid / kXcd;
  // (split-major split K: all of a split's column tiles at once, they share its slabs)
  int nb = nN;
  double best = 1e300;
  for (int c = 1; c <= nN && !(KMAJOR && ksplit > 1 && ksplit % kXcd == 0); ++c) {
    const double chunks = (double)((nN + c - 1) / c);
    const bool fits = c * slice <= 0.6 * l2;
    const double rounds = (double)((nM + kXcd - 1) / kXcd) * c / std::max(1.0, wg_per_xcd);
    const double w_traffic = fits ? kXcd * nN * slice : kXcd * rounds * c * slice * chunks;
    const double t = a_bytes * chunks + w_traffic;
    if (t < best * 0.98) { best = t; nb = c; }
  }
  kern<<<(unsigned)grid, 64 * WM * WN, lds, s>>>(M, N, K, a, w, bias, resid, static_cast<TOut*>(out), nN, nM, nb,
                                                  ksplit, nMr, km.t_rows, km.lda, km.ldb, aux);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(int64_t M, int N, int K, int epi, const bf16* a, const bf16* w,
                            const bf16* bias, const float* resid, void* out, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (epi) {
    case MTGR_EPI_STORE: return run_bf16_persistent<4, 2, MTGR_EPI_STORE, bf16>(M, N, K, a, w, bias, resid, out, s);
    case MTGR_EPI_SILU: return run_bf16_persistent<4, 2, MTGR_EPI_SILU, bf16>(M, N, K, a, w, bias, resid, out, s);
    case MTGR_EPI_RESIDUAL_F32:
      return run_bf16_persistent<4, 2, MTGR_EPI_RESIDUAL_F32, float>(M, N, K, a, w, bias, resid, out, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_bf16_silu_bwd(int64_t M, int N, int K, const bf16* a, const bf16* w, bf16* act,
                                     bf16* out, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K % 64 != 0 || K < 128 || N % 8 != 0) return hipErrorInvalidValue;
  return run_bf16_persistent<4, 2, kEpiSiluBwd, bf16>(M, N, K, a, w, nullptr, nullptr, out, s, 1, KMajorArgs(), act);
}

hipError_t launch_gemm_bf16_f32out_rows(int64_t M, int N, int K, const bf16* a, const bf16* w, const bf16* bias,
                                        const int32_t* rowmap, int64_t out_rows, float* out, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K % 64 != 0 || K < 128 || N % 8 != 0) return hipErrorInvalidValue;
  if (out_rows * N * 4 >= (int64_t(1) << 31)) return hipErrorInvalidValue;   // one 31-bit buffer range
  KMajorArgs km;
  km.t_rows = out_rows;
  return run_bf16_persistent<4, 2, kEpiRowScatter, float>(M, N, K, a, w, bias, nullptr, out, s, 1, km,
                                                          const_cast<int32_t*>(rowmap));
}

hipError_t launch_gemm_bf16_kmajor_splitk(int M, int N, int64_t Kp, int ksplit, int64_t T, const bf16* a, int lda,
                                          const bf16* w, int ldb, float* part, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (ksplit < 1 || Kp % (64 * ksplit) != 0 || Kp / 64 / ksplit < 2 || T > Kp || lda < M || ldb < N ||
      ldb % 8 != 0 || lda % 8 != 0)
    return hipErrorInvalidValue;
  // a split's rows must stay within a 32-bit buffer range
  if ((Kp / ksplit) * (int64_t)std::max(lda, ldb) * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  KMajorArgs km;
  km.t_rows = T;
  km.lda = lda;
  km.ldb = ldb;
  return run_bf16_persistent<4, 2, MTGR_EPI_STORE, float, true>(M, N, (int)Kp, a, w, nullptr, nullptr, part, s, ksplit, km);
}

hipError_t launch_gemm_bf16_f32out(int64_t M, int N, int K, const bf16* a, const bf16* w, const bf16* bias,
                                   float* out, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K % 64 != 0 || K < 128 || N % 8 != 0) return hipErrorInvalidValue;
  return run_bf16_persistent<4, 2, MTGR_EPI_STORE, float>(M, N, K, a, w, bias, nullptr, out, s);
}

hipError_t launch_gemm_f32_splitk(int64_t M, int N, int K, int ksplit, const float* a, const float* w,
                                  float* part, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (ksplit < 1 || K % ksplit != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)ksplit);
  k_gemm_f32<MTGR_EPI_STORE><<<grid, 256, 0, s>>>(M, N, K, a, w, nullptr, nullptr, part);
  return hipGetLastError();
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
