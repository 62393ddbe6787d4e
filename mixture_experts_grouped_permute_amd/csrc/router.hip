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
// Block b routes tokens [64 b, 64 b + 64), four lanes per token -- exactly the chunk of the
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

// Insert (cv, ci) into the sorted list (v, id) of kK slots, ordered by (logit descending, expert
// id ascending): the carried entry (the new logit, then whatever it displaces) takes a slot that
// is empty (id -1, which accepts anything, -inf included) or holds a smaller logit, or an equal
// logit of a higher id -- a displaced entry can have a lower id than an equal one further down.
template <int kK>
__device__ __forceinline__ void topk_insert(float (&v)[kK], int (&id)[kK], float cv, int ci, int k) {
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    const bool take = j < k && ci >= 0 && (id[j] < 0 || cv > v[j] || (cv == v[j] && ci < id[j]));
    const float tv = v[j];
    const int ti = id[j];
    v[j] = take ? cv : tv;
    id[j] = take ? ci : ti;
    cv = take ? tv : cv;
    ci = take ? ti : ci;
  }
}

// Four lanes per token: lane s keeps the top-k of experts s, s + 4, s + 8, ...; lane 0 of the
// four then merges the other three lists into its own and writes the token.
template <bool kF32, int kK>
__global__ __launch_bounds__(4 * kPermTokens) void router_kernel(const void* __restrict__ logits, int64_t T, int E,
                                                                   int k, int32_t* __restrict__ idx,
                                                                   float* __restrict__ prob,
                                                                   int32_t* __restrict__ block_counts,
                                                                   int32_t* __restrict__ block_bad) {
  __shared__ int cnt[kMaxExperts];
  if (block_counts) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
  }
  const int sub = threadIdx.x & 3;
  const int64_t t = (int64_t)blockIdx.x * kPermTokens + (threadIdx.x >> 2);
  const bool live = t < T;
  float v[kK];
  int id[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) { v[j] = 0.f; id[j] = -1; }
  if (live) {
    const int64_t row = t * E;
    for (int e = sub; e < E; e += 4) topk_insert<kK>(v, id, logit_at<kF32>(logits, row + e), e, k);
  }
  // merge: lanes 1..3 of each group of four hand their lists to lane 0
#pragma unroll
  for (int s = 1; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      const float ov = __shfl_down(v[j], s, 64);
      const int oi = __shfl_down(id[j], s, 64);
      if (sub == 0) topk_insert<kK>(v, id, ov, oi, k);
    }
  if (live && sub == 0) {
    float s = 0.f, w[kK];
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      w[j] = j < k ? __expf(v[j] - v[0]) : 0.f;
      s += w[j];
    }
    const float inv = 1.0f / s;
#pragma unroll
    for (int j = 0; j < kK; ++j) {
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

template <bool kF32>
hipError_t launch_router_k(const void* logits, int64_t T, int E, int k, int32_t* idx, float* prob,
                           int32_t* block_counts, int32_t* block_bad, int nb, hipStream_t st) {
  const dim3 grid(nb), block(4 * kPermTokens);
  if (k <= 2) router_kernel<kF32, 2><<<grid, block, 0, st>>>(logits, T, E, k, idx, prob, block_counts, block_bad);
  else if (k <= 4) router_kernel<kF32, 4><<<grid, block, 0, st>>>(logits, T, E, k, idx, prob, block_counts, block_bad);
  else if (k <= 8) router_kernel<kF32, 8><<<grid, block, 0, st>>>(logits, T, E, k, idx, prob, block_counts, block_bad);
  else router_kernel<kF32, 16><<<grid, block, 0, st>>>(logits, T, E, k, idx, prob, block_counts, block_bad);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const void* logits, bool f32, int64_t T, int E, int k, int32_t* idx, float* prob,
                         int32_t* block_counts, hipStream_t st) {
  const int nb = perm_blocks(T);
  int32_t* block_bad = block_counts ? block_counts + (int64_t)nb * E : nullptr;
  return f32 ? launch_router_k<true>(logits, T, E, k, idx, prob, block_counts, block_bad, nb, st)
             : launch_router_k<false>(logits, T, E, k, idx, prob, block_counts, block_bad, nb, st);
}

}  // namespace moe
