// Device-side helpers shared by the gfx950 kernels of libmtgr.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtgr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// Reductions over the 64 lanes of a wavefront (called with every lane active), on DPP row
// operations instead of LDS permutes: the butterfly within each quad, the two halves of each row
// of 16 (mirrors), then rows 0+1 and 2+3 (lane 15 broadcast into rows 1 and 3) and the two halves
// (lane 31 into rows 2 and 3); lane 63 then holds the result, read back as a scalar.  Lanes a
// broadcast does not reach combine with the identity.  The order is fixed: deterministic.
template <int CTRL, int ROW_MASK> __device__ __forceinline__ float dpp_mov(float v, float identity) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, identity), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xF, false));
}
template <typename Op> __device__ __forceinline__ float wave_reduce(float v, float identity, Op op) {
  v = op(v, dpp_mov<0xB1, 0xF>(v, identity));     // quad_perm [1,0,3,2]
  v = op(v, dpp_mov<0x4E, 0xF>(v, identity));     // quad_perm [2,3,0,1]
  v = op(v, dpp_mov<0x141, 0xF>(v, identity));    // row_half_mirror
  v = op(v, dpp_mov<0x140, 0xF>(v, identity));    // row_mirror
  v = op(v, dpp_mov<0x142, 0xA>(v, identity));    // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_mov<0x143, 0xC>(v, identity));    // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, 0.f, [](float a, float b) { return a + b; });
}
// Sum over each half of the wavefront (lanes 0-31 and 32-63), every lane getting its own half's
// sum: the same steps as wave_reduce up to the broadcast of lane 15 into rows 1 and 3, after which
// lanes 31 and 63 hold the two halves' sums.
__device__ __forceinline__ float half_wave_sum(float v) {
  v += dpp_mov<0xB1, 0xF>(v, 0.f);
  v += dpp_mov<0x4E, 0xF>(v, 0.f);
  v += dpp_mov<0x141, 0xF>(v, 0.f);
  v += dpp_mov<0x140, 0xF>(v, 0.f);
  v += dpp_mov<0x142, 0xA>(v, 0.f);
  const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  return (threadIdx.x & 32) ? hi : lo;
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min(float v) {
  return wave_reduce(v, INFINITY, [](float a, float b) { return fminf(a, b); });
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).  __expf maps to the hardware exp2 with a
// log2(e) pre-scale; for z < -88 the exponential overflows to +inf and the quotient is -0,
// which is the correctly rounded limit.
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }
// Same function with the hardware reciprocal (about 1 ulp) in place of the IEEE division; used
// where the result is rounded to bf16 anyway.  rcp(+inf) = 0 gives the same -0 limit.
__device__ __forceinline__ float silu_rcp(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Visibility of key j to query i inside one user whose tokens are ordered U, S, R, C, with
// n_static = N_U + N_S and rc_end = N_U + N_S + N_R.  Rules of the dynamic mask (fun-rec
// "MTGR: Hybrid Paradigm Modeling" 7.3.4 Rules 1-3; marovi.ai MTGR page, 方法): static keys
// are visible to every query; every token sees itself; a real-time key is visible to a
// real-time or candidate query with a strictly later timestamp; candidate keys are visible
// to nobody else.  Used by every attention kernel and by the debug mask dump.
__device__ __forceinline__ bool mtgr_visible(int i, int j, int n_static, int rc_end, float ti,
                                             float tj) {
  // non-short-circuit form: evaluates to a few compares and a select, no branches
  return (j < n_static) | (i == j) | ((i >= n_static) & (j < rc_end) & (tj < ti));
}

// Mask modes (values of MTGR_MASK_*).  Dynamic is the method's mask; causal (key j visible iff
// j <= i in sequence order) and full (every key of the user) are the ablation baselines: the
// causal mask is what the dynamic rules replace (fun-rec 7.3.4; marovi.ai MTGR page, 方法).
enum { kMaskDynamic = 0, kMaskCausal = 1, kMaskFull = 2 };

__device__ __forceinline__ bool mtgr_visible_mode(int mode, int i, int j, int n_static, int rc_end,
                                                  float ti, float tj) {
  if (mode == kMaskCausal) return j <= i;
  if (mode == kMaskFull) return true;
  return mtgr_visible(i, j, n_static, rc_end, ti, tj);
}

// Per-user segment record written by the batch-prep kernel.
struct UserSeg {
  int32_t n_u, n_s, n_r, k;
};

}  // namespace mtgr
