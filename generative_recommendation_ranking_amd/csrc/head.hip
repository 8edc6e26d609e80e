// Candidate readout head (chenhuiyu blog "MTGR", section on turning features into tokens: the
// hidden state at each candidate position goes through an MLP that emits CTR and CTCVR logits;
// fun-rec "MTGR: Hybrid Paradigm Modeling" 7.3.1: scoring happens at candidate positions only).
//
//   logits[c] = W_h2 silu(W_h1 x[cand_idx[c]] + b_h1) + b_h2,   columns (CTR, CTCVR).
//
// The first layer runs on the GEMM kernels after a gather of the candidate rows (converted to
// the head's storage dtype); the 2-wide output layer is one wavefront per candidate.
#include "kernels.h"

namespace mtgr {

namespace {

template <typename TOut>
__global__ __launch_bounds__(256) void k_gather(int64_t C, int64_t T, int d,
                                                const float* __restrict__ x,
                                                const int64_t* __restrict__ idx,
                                                TOut* __restrict__ rows) {
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= C) return;
  const int64_t r = idx[c];
  TOut* dst = rows + c * d;
  if (r < 0 || r >= T) {  // only with a candidate count that disagrees with the group ids
    for (int f = lane; f < d; f += 64) dst[f] = from_f32<TOut>(0.f);
    return;
  }
  const float* src = x + r * d;
  for (int f = lane; f < d; f += 64) dst[f] = from_f32<TOut>(src[f]);
}

template <typename T>
__global__ __launch_bounds__(256) void k_head_out(int64_t C, int hh, const T* __restrict__ hid,
                                                  const T* __restrict__ w2,
                                                  const T* __restrict__ b2,
                                                  float* __restrict__ logits) {
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= C) return;
  const T* hr = hid + c * hh;
  float a0 = 0.f, a1 = 0.f;
  for (int k = lane; k < hh; k += 64) {
    const float hv = to_f32(hr[k]);
    a0 = fmaf(hv, to_f32(w2[k]), a0);
    a1 = fmaf(hv, to_f32(w2[hh + k]), a1);
  }
  a0 = wave_sum(a0);
  a1 = wave_sum(a1);
  if (lane == 0) {
    logits[c * 2 + 0] = a0 + (b2 ? to_f32(b2[0]) : 0.f);
    logits[c * 2 + 1] = a1 + (b2 ? to_f32(b2[1]) : 0.f);
  }
}

}  // namespace

hipError_t launch_gather_rows(int64_t C, int64_t T, int d, const float* x,
                              const int64_t* cand_idx, int out_kind, void* rows, hipStream_t s) {
  if (C == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((C + 3) / 4);
  if (out_kind == 0)
    k_gather<float><<<blocks, 256, 0, s>>>(C, T, d, x, cand_idx, static_cast<float*>(rows));
  else
    k_gather<bf16><<<blocks, 256, 0, s>>>(C, T, d, x, cand_idx, static_cast<bf16*>(rows));
  return hipGetLastError();
}

hipError_t launch_head_out(int64_t C, int hh, int kind, const void* hid, const void* w2,
                           const void* b2, float* logits, hipStream_t s) {
  if (C == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((C + 3) / 4);
  if (kind == 0)
    k_head_out<float><<<blocks, 256, 0, s>>>(C, hh, static_cast<const float*>(hid),
                                             static_cast<const float*>(w2),
                                             static_cast<const float*>(b2), logits);
  else
    k_head_out<bf16><<<blocks, 256, 0, s>>>(C, hh, static_cast<const bf16*>(hid),
                                            static_cast<const bf16*>(w2),
                                            static_cast<const bf16*>(b2), logits);
  return hipGetLastError();
}

}  // namespace mtgr
