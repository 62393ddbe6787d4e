// Fused top-k router for gfx950: softmax -> top-k -> renormalise, plus the expert histogram
// the permutation starts from, in one pass over the logits.
//
// Method (page "BioNeMo Uses Grouped Kernels and MXFP8", Figure 1: a router sends each token to
// k of the experts and their outputs are combined with the routing weights):
//   idx[t, :]  = the k largest logits of token t in descending order, equal logits -> lower
//                expert id first (softmax is increasing, so these are the k largest
//                probabilities);
//   prob[t, j] = exp(l_j - l_max) / sum over the k selected of exp(l_i - l_max), which is the
//                softmax over all E experts renormalised over the k (the full denominator
//                cancels).
//
// Block b routes tokens [256 b, 256 b + 256), one thread per token -- exactly the chunk of the
// permutation's histogram -- and writes the chunk's expert counts in the layout the scan reads,
// so the permutation's own histogram pass is skipped.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <bool kF32>
__device__ __forceinline__ float logit_at(const void* lg, int64_t o) {
  if constexpr (kF32) return reinterpret_cast<const float*>(lg)[o];
  else return bf16_to_f32(reinterpret_cast<const uint16_t*>(lg)[o]);
}

template <bool kF32>
__global__ __launch_bounds__(kPermTokens) void router_kernel(const void* __restrict__ logits, int64_t T, int E,
                                                               int k, int32_t* __restrict__ idx,
                                                               float* __restrict__ prob,
                                                               int32_t* __restrict__ block_counts,
                                                               int32_t* __restrict__ block_bad) {
  __shared__ int cnt[kMaxExperts];
  if (block_counts) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
  }
  const int64_t t = (int64_t)blockIdx.x * kPermTokens + threadIdx.x;
  if (t < T) {
    // sorted top-k by insertion, ordered by (logit descending, expert id ascending): the carried
    // entry (the new logit, then whatever it displaces) takes a slot that is empty (id -1, which
    // accepts anything, -inf included) or holds a smaller logit, or an equal logit of a higher
    // id -- a displaced entry can have a lower id than an equal one further down
    float v[kMaxTopK];
    int id[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) { v[j] = 0.f; id[j] = -1; }
    const int64_t row = t * E;
    for (int e = 0; e < E; ++e) {
      float cv = logit_at<kF32>(logits, row + e);
      int ci = e;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        const bool take = j < k && ci >= 0 && (id[j] < 0 || cv > v[j] || (cv == v[j] && ci < id[j]));
        const float tv = v[j];
        const int ti = id[j];
        v[j] = take ? cv : tv;
        id[j] = take ? ci : ti;
        cv = take ? tv : cv;
        ci = take ? ti : ci;
      }
    }
    float s = 0.f, w[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      w[j] = j < k ? __expf(v[j] - v[0]) : 0.f;
      s += w[j];
    }
    const float inv = 1.0f / s;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) continue;
      idx[t * k + j] = id[j];
      prob[t * k + j] = w[j] * inv;
      if (block_counts) atomicAdd(&cnt[id[j]], 1);
    }
  }
  if (block_counts) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) block_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
    if (threadIdx.x == 0) block_bad[blockIdx.x] = 0;
  }
}

}  // namespace

hipError_t launch_router(const void* logits, bool f32, int64_t T, int E, int k, int32_t* idx, float* prob,
                         int32_t* block_counts, hipStream_t st) {
  const int nb = perm_blocks(T);
  int32_t* block_bad = block_counts ? block_counts + (int64_t)nb * E : nullptr;
  if (f32) router_kernel<true><<<nb, kPermTokens, 0, st>>>(logits, T, E, k, idx, prob, block_counts, block_bad);
  else router_kernel<false><<<nb, kPermTokens, 0, st>>>(logits, T, E, k, idx, prob, block_counts, block_bad);
  return hipGetLastError();
}

}  // namespace moe
