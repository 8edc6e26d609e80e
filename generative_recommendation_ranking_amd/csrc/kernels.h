// Internal launchers of libmtgr.so (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "plan.h"

namespace mtgr {

static_assert(sizeof(UserSeg) == kUserSegBytes, "the planner sizes the segment table");

// ---- batch prep (prep.hip) ----------------------------------------------------------------
// Segment counts per user, LPT user order (longest users first), q-tile offsets in that order,
// candidate offsets per user and the packed-order candidate token index list.
struct PrepBufs {
  UserSeg* seg;        // [B]
  int32_t* order;      // [B]   users sorted by token count, descending (ties by index)
  int32_t* tile_off;   // [B+1] exclusive prefix of ceil(n_b / q_tile) in `order`
  int64_t* cand_off;   // [B+1] exclusive prefix of K_b in user order
  int64_t* cand_idx;   // [C]   token row of each candidate, packed order
  int32_t* flags;      // [4]   validation flags / counters
  int32_t* xcd_off;    // [8][R+1] per-XCD q-tile prefix over (user, head) groups, R = ceil(B*H/8)
  int32_t* xcd_fwd;    // [8][R+1] the same for the forward's q-tile size (may be NULL)
};
// q_tile sizes tile_off and xcd_off; q_tile_fwd > 0 also builds xcd_fwd
hipError_t launch_prep(int32_t B, int64_t C, const int64_t* offsets, const uint8_t* group_ids,
                       int q_tile, int q_tile_fwd, int heads, const PrepBufs& pb, bool want_cand_idx,
                       hipStream_t s);
hipError_t launch_validate(int32_t B, const int64_t* offsets, const uint8_t* group_ids,
                           const float* timestamps, int32_t* flags, hipStream_t s);
hipError_t launch_debug_mask(int32_t user, int mask_mode, const int64_t* offsets, const UserSeg* seg,
                             const float* timestamps, int64_t n_user, uint8_t* mask,
                             hipStream_t s);

// ---- GroupLN (groupln.hip) ---------------------------------------------------------------
// in_kind/out_kind/param_kind: 0 = float, 1 = bf16; shared != 0: every row takes gamma[0]/beta[0]
hipError_t launch_groupln(int64_t T, int d, int in_kind, int out_kind, int param_kind, int shared,
                          const void* x, const uint8_t* group_ids, const void* gamma,
                          const void* beta, float eps, void* y, hipStream_t s);

// ---- GEMMs (gemm.hip) ----------------------------------------------------------------------
// out[M][N] = epi(a[M][K] w[N][K]^T + bias); epi as MTGR_EPI_*.
hipError_t launch_gemm_bf16(int64_t M, int N, int K, int epi, const bf16* a, const bf16* w,
                            const bf16* bias, const float* resid, void* out, hipStream_t s);
hipError_t launch_gemm_f32(int64_t M, int N, int K, int epi, const float* a, const float* w,
                           const float* bias, const float* resid, float* out, hipStream_t s);

// ---- attention (attention.hip) -------------------------------------------------------------
// grid_slots = max over XCDs of that XCD's q-tile count (the host replica of k_prep_xcd); the bf16
// forward takes its work from queues built with kAttnFwdQTileBf16.
// vt (may be NULL) receives the ungated V~ for the backward pass.
// mask_mode: kMaskDynamic / kMaskCausal / kMaskFull
hipError_t launch_attention_bf16(int32_t B, int64_t grid_slots, int d, int H, int mask_mode,
                                 const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                 const int32_t* xcd_off, const float* timestamps,
                                 const bf16* qkvu, bf16* y, bf16* vt, hipStream_t s);
hipError_t launch_attention_f32(int32_t B, int64_t total_tiles, int d, int H, int mask_mode,
                                const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                const int32_t* tile_off, const float* timestamps,
                                const float* qkvu, float* y, float* vt, hipStream_t s);

// ---- backward pieces (backward.hip) -------------------------------------------------------------
// kind / *_kind: 0 = float, 1 = bf16
// dst[c][r] = src[r][c] (r < R, c < C), zero for R <= r < Rp; ones_row adds row C = (r < R) and
// rows C+1..C+7 = 0.  dst row pitch Rp.
hipError_t launch_transpose(int64_t R, int C, int64_t Rp, int ones_row, int kind, const void* src,
                            void* dst, hipStream_t s);
// dh <- dh (.) silu'(a); then a <- silu(a) (the MLP's hidden activation, for its weight gradient)
hipError_t launch_silu_bwd(int64_t n, int kind, void* a, void* dh, hipStream_t s);
hipError_t launch_convert(int64_t n, int kind, const float* x, void* y, hipStream_t s);
// out[i] = sum over s < nsplit of part[s*stride + i]
hipError_t launch_reduce(int64_t n, int nsplit, int64_t stride, const float* part, float* out, hipStream_t s);
// sum of nsplit partials [nsplit][M][Kx] -> dw [M][K] and db [M] = column K (db may be NULL)
hipError_t launch_reduce_wb(int M, int K, int Kx, int nsplit, const float* part, float* dw, float* db,
                            hipStream_t s);
// GroupLN backward: dx = GLN'(x)^T dz (+ resid); per-wavefront partials of (dgamma, dbeta)
// [groupln_bwd_waves(T)][2][4][d] (plan.h)
hipError_t launch_groupln_bwd(int64_t T, int d, int x_kind, int act_kind, int shared, const void* x,
                              const uint8_t* g, const void* gamma, float eps, const void* dz,
                              const float* resid, void* dx, int out_kind, float* part, hipStream_t s);
// masked SiLU attention backward, one thread per (row, head): dqkvu [T][4d] from qkvu, the ungated
// V~ and dy (gradient w.r.t. the gated output); work items (user, q_tile rows) in prep order
// (tile_off built with the same q_tile, 64 or 128)
hipError_t launch_attention_bwd_ref(int32_t B, int64_t total_tiles, int q_tile, int d, int H, int mask_mode, int kind,
                                    const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                    const int32_t* tile_off, const float* timestamps, const void* qkvu,
                                    const void* vt, const void* dy, void* dqkvu, hipStream_t s);
// bf16 attention backward on MFMA (attention_bwd.hip): G = dy (.) U into g [T][d] (workspace),
// dU = dy (.) vt, then dK/dV (key tiles) and dQ (query tiles); work items from the forward's
// per-XCD queues (xcd_off built with q_tile 128), grid_slots as for launch_attention_bf16
hipError_t launch_attention_bwd_bf16(int32_t B, int64_t T, int64_t grid_slots, int d, int H, int mask_mode,
                                     const int64_t* offsets, const UserSeg* seg, const int32_t* order,
                                     const int32_t* xcd_off, const float* timestamps, const bf16* qkvu,
                                     const bf16* vt, const bf16* dy, bf16* g, bf16* dqkvu, hipStream_t s);
// the backward of the MLP's SiLU fused into the GEMM that produces its input gradient: with
// g = a[M][K] w[N][K]^T (fp32), out = bf16(g (.) silu'(act)) and act <- bf16(silu(act)) in place
// (act: the pre-activation [M][N], bf16)
constexpr int kEpiSiluBwd = 16;   // internal epilogue id (not one of the public MTGR_EPI_*)
// out[rowmap[m]][n] = a[m][K] w[n][K]^T + bias (fp32), row m dropped where rowmap[m] < 0; out has
// out_rows rows (out_rows * N * 4 < 2^31)
constexpr int kEpiRowScatter = 17;
hipError_t launch_gemm_bf16_f32out_rows(int64_t M, int N, int K, const bf16* a, const bf16* w, const bf16* bias,
                                        const int32_t* rowmap, int64_t out_rows, float* out, hipStream_t s);
hipError_t launch_gemm_bf16_silu_bwd(int64_t M, int N, int K, const bf16* a, const bf16* w, bf16* act,
                                     bf16* out, hipStream_t s);
// k-major split-K GEMM for weight gradients without transposed copies: part[s][m][n] =
// sum over token rows t of split s of a[t][m] w[t][n] (a: [T][lda], w: [T][ldb], token axis padded
// to Kp with zero rows; Kp a multiple of 64 * ksplit, at least two 64-row slabs per split); a split
// count that is a multiple of 8 keeps each split on one XCD
hipError_t launch_gemm_bf16_kmajor_splitk(int M, int N, int64_t Kp, int ksplit, int64_t T, const bf16* a, int lda,
                                          const bf16* w, int ldb, float* part, hipStream_t s);
// column sums of a bf16 [T][M] matrix (M % 8 == 0): per-block partials part[colsum_blocks(T, M)][M],
// then out[m] = their sum in block order (deterministic); part holds colsum_blocks(T, M) * M floats (plan.h)
hipError_t launch_colsum_bf16(int64_t T, int M, const bf16* src, float* part, float* out, hipStream_t s);
// dst = bf16(src) for an fp32 [T][M] matrix and, when out is not NULL, out[m] = the column sums of
// src (fp32, the same partial layout and order as launch_colsum_bf16)
hipError_t launch_convert_colsum(int64_t T, int M, const float* src, bf16* dst, float* part, float* out,
                                 hipStream_t s);
hipError_t launch_gemm_f32_splitk(int64_t M, int N, int K, int ksplit, const float* a, const float* w,
                                  float* part, hipStream_t s);

// ---- hash embedding store and dedup (hash_store.hip) ------------------------------------------
constexpr size_t kHashHeaderBytes = 256;
inline size_t hash_align(size_t v) { return (v + 255) / 256 * 256; }
// index_mem: header + index_cap slots of 16 bytes (index_cap a power of two >= 8); arena_mem:
// header, free stack [rows] int32, last use [rows] int32, values [rows][row_bytes] (may be NULL
// for a key-only index, as the dedup scratch)
struct HashDesc {
  void* index_mem;
  int64_t index_cap;
  void* arena_mem;
  int32_t rows;
  int32_t row_bytes;
};
hipError_t launch_hash_init(const HashDesc& h, bool index, bool arena, hipStream_t s);
// res: [n] int64 scratch
hipError_t launch_hash_insert(const HashDesc& h, int64_t n, const int64_t* keys, const void* init, int32_t step,
                              int32_t* rows_out, int64_t* res, hipStream_t s);
// n_dev (may be NULL): a device count; keys past min(n, *n_dev) are skipped
hipError_t launch_hash_lookup(const HashDesc& h, int64_t n, const int64_t* keys, int32_t step, void* out,
                              int32_t* rows_out, hipStream_t s, const int64_t* n_dev = nullptr);
hipError_t launch_hash_evict(const HashDesc& h, int64_t n, const int64_t* keys, hipStream_t s);
hipError_t launch_hash_evict_older(const HashDesc& h, int32_t threshold, hipStream_t s);
hipError_t launch_hash_rebuild(const HashDesc& src, const HashDesc& dst, hipStream_t s);
// distinct keys in claim order into uniq, per-occurrence index into inverse, count into *count
hipError_t launch_dedup(int64_t n, const int64_t* keys, const HashDesc& scratch, int64_t* res, int64_t* uniq,
                        int64_t* inverse, unsigned long long* count, hipStream_t s);

// ---- tokenizer front end (tokenizer.hip) --------------------------------------------------------
constexpr int kTokMaxFields = 8;
struct TokFields {                 // fields of each group and the table each one reads
  int nfields[4];
  int table[4][kTokMaxFields];
};
struct TokGroups {                 // group-sorted feature buffers
  int nfields[4];
  int64_t rows[4];                 // tokens of each group (as the host was told)
  int64_t row0[4];                 // first row of each group in the [T][d] group-sorted outputs
  bf16* feat[4];                   // [rows][nfields * e]
};
// per-user group counts cnt [B][4], their per-group exclusive prefix goff [4][B+1], merged keys
// [T][fmax] (-1 for unused fields), flags reset
hipError_t launch_tok_prepare(int32_t B, int64_t T, int fmax, const int64_t* offsets, const uint8_t* group_ids,
                              const int64_t* ids, const TokFields& tf, int64_t* cnt, int64_t* goff, int64_t* keys,
                              int32_t* flags, hipStream_t s);
hipError_t launch_tok_build(int64_t T, int32_t B, int fmax, int e, const int64_t* offsets, const uint8_t* group_ids,
                            const int64_t* cnt, const int64_t* goff, const TokGroups& tg, const int64_t* inverse,
                            const bf16* uvals, int64_t* pos, int32_t* rowmap, int32_t* flags, hipStream_t s);
hipError_t launch_tok_scatter(int64_t T, int d, const int64_t* pos, const float* y, float* x, hipStream_t s);
hipError_t launch_tok_zero_unplaced(int64_t T, int d, const int64_t* pos, float* x, hipStream_t s);
// out (float [M][N]) = a[M][K] w[N][K]^T + bias (bf16 operands)
hipError_t launch_gemm_bf16_f32out(int64_t M, int N, int K, const bf16* a, const bf16* w, const bf16* bias,
                                   float* out, hipStream_t s);

// ---- head (head.hip) -----------------------------------------------------------------------
// rows[c] = (out_kind) x[cand_idx[c]]  (fp32 hidden state -> head input dtype)
hipError_t launch_gather_rows(int64_t C, int64_t T, int d, const float* x,
                              const int64_t* cand_idx, int out_kind, void* rows, hipStream_t s);
// logits[c][o] = sum_k hid[c][k] w2[o][k] + b2[o]  (o in {0,1})
hipError_t launch_head_out(int64_t C, int hh, int kind, const void* hid, const void* w2,
                           const void* b2, float* logits, hipStream_t s);

}  // namespace mtgr
