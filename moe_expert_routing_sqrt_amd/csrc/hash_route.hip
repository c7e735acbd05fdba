// Hash router on gfx950 (mastering-deepseek-v4 "MoE + Expert-Parallel Overlap
// (Exp08)", Implemented: a hash router emulates the early layers -- a token's
// experts depend on its token id, not on the gate).
//
// The pages do not give the hash.  It is the published counter-based generator
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11), keyed by (seed, 0) with
// counter (token id as uint32, block, 0, 0).  The four 64-bit words of a block
// are used in order; word u picks expert floor(u * E / 2^64) (the high half of
// a 64x64-bit product); an expert already chosen for the token is skipped.
// After kMaxBlocks blocks any slot still empty takes the smallest unused
// experts in increasing order, so the work per token is bounded.  Groups play
// no part.  Gate weights are 1/k, or with logits the renormalised affinities
// of the chosen experts (w_j = s_j / (((s_0 + s_1) + s_2) + ...)), computed by
// the same operation sequence as the top-k router (affinity.h).
//
// One thread per token; a work-group of 256 threads covers four 64-token route
// blocks and writes their rows of the per-block expert histogram.
#pragma clang fp contract(off)

#include "affinity.h"
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSub = kThreads / MOE_ROUTE_BLOCK;  // route blocks per work-group
constexpr int kMaxBlocks = 256;
constexpr int kMaxK = 16;

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ inline void philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                     uint64_t k0, uint64_t k1, uint64_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

struct HashArgs {
  const int32_t* ids;
  int64_t T;
  int E, k;
  uint64_t seed;
  const float* logits;  // [T, E] or nullptr
  int32_t* idx;
  float* w;
  int32_t* block_counts;
};

__global__ __launch_bounds__(kThreads) void hash_route_kernel(const HashArgs p) {
  __shared__ int s_cnt[kSub][kMaxExperts];
  const int tid = threadIdx.x;
  const int sub = tid / MOE_ROUTE_BLOCK;
  for (int e = tid % MOE_ROUTE_BLOCK; e < p.E; e += MOE_ROUTE_BLOCK) s_cnt[sub][e] = 0;
  __syncthreads();

  const int64_t t = (int64_t)blockIdx.x * kThreads + tid;
  if (t < p.T) {
    const uint64_t v = static_cast<uint32_t>(p.ids[t]);
    int chosen[kMaxK];
    int n = 0;
    // a candidate joins the list unless it is already there (indices stay
    // compile-time, so the list lives in registers)
    auto offer = [&](int e) {
      bool dup = false;
#pragma unroll
      for (int i = 0; i < kMaxK; ++i) dup = dup || (i < n && chosen[i] == e);
      if (!dup) {
#pragma unroll
        for (int i = 0; i < kMaxK; ++i)
          if (i == n) chosen[i] = e;
        ++n;
      }
    };
    for (int b = 0; b < kMaxBlocks && n < p.k; ++b) {
      uint64_t u[4];
      philox4x64_10(v, static_cast<uint64_t>(b), 0, 0, p.seed, 0, u);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (n < p.k) offer(static_cast<int>(__umul64hi(u[q], static_cast<uint64_t>(p.E))));
    }
    for (int e = 0; e < p.E && n < p.k; ++e) offer(e);

    if (p.logits == nullptr) {
      const float wu = 1.0f / static_cast<float>(p.k);
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < p.k) {
          p.idx[t * p.k + j] = chosen[j];
          p.w[t * p.k + j] = wu;
        }
    } else {
      float s[kMaxK];
      float S = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < p.k) {
          s[j] = aff::affinity_spec(p.logits[t * p.E + chosen[j]]);
          S = j == 0 ? s[j] : S + s[j];
        }
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < p.k) {
          p.idx[t * p.k + j] = chosen[j];
          p.w[t * p.k + j] = s[j] / S;
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < p.k) atomicAdd(&s_cnt[sub][chosen[j]], 1);
  }
  __syncthreads();
  const int64_t rb = (int64_t)blockIdx.x * kSub + sub;  // this thread's route block
  if (rb * MOE_ROUTE_BLOCK < p.T)
    for (int e = tid % MOE_ROUTE_BLOCK; e < p.E; e += MOE_ROUTE_BLOCK)
      p.block_counts[rb * p.E + e] = s_cnt[sub][e];
}

}  // namespace

hipError_t launch_hash_route(const int32_t* ids, int64_t T, int E, int k, uint64_t seed,
                             const float* logits, int32_t* idx, float* w, int32_t* block_counts,
                             hipStream_t s) {
  HashArgs a{ids, T, E, k, seed, logits, idx, w, block_counts};
  const unsigned grid = static_cast<unsigned>((T + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(hash_route_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
