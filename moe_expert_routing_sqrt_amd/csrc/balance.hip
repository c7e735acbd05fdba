// Per-expert bias update for auxiliary-loss-free load balancing
// (mastering-deepseek-v4 "MoE + Expert-Parallel Overlap (Exp08)", Implemented
// and Measured):
//     load[e] = sum_r counts[r][e]
//     bias[e] += gamma * sign(sum(load)/E - load[e])
// One work-group: the n_rows x E count matrix (moe_route's per-block counts, a
// few hundred KB at most) is summed column-wise by parts x experts threads,
// the total by a block reduction in 64-bit integers, and the sign is taken
// from the exact integer comparison sum(load) vs E * load[e].
#pragma clang fp contract(off)

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                               int64_t n_rows, int E, float gamma,
                                                               float* __restrict__ bias,
                                                               int32_t* __restrict__ load) {
  __shared__ long long s_part[kThreads];
  __shared__ long long s_total;
  const int tid = threadIdx.x;
  const int parts = max(1, kThreads / E);
  const int e = tid % E, part = tid / E;
  const bool active = part < parts;
  long long sum = 0;
  if (active)
    for (int64_t r = part; r < n_rows; r += parts) sum += counts[r * E + e];
  s_part[tid] = active ? sum : 0;
  __syncthreads();
  // column sums: part 0 of each expert collects the other parts
  long long col = 0;
  if (part == 0)
    for (int q = 0; q < parts; ++q) col += s_part[q * E + e];
  __syncthreads();
  s_part[tid] = part == 0 ? col : 0;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {  // total over experts
    if (tid < o) s_part[tid] += s_part[tid + o];
    __syncthreads();
  }
  if (tid == 0) s_total = s_part[0];
  __syncthreads();
  if (part == 0) {
    const long long lhs = s_total, rhs = (long long)E * col;  // sign(mean - load) = sign(total - E*load)
    if (lhs > rhs) bias[e] = bias[e] + gamma;
    else if (lhs < rhs) bias[e] = bias[e] - gamma;
    if (load != nullptr) load[e] = static_cast<int32_t>(col);
  }
}

}  // namespace

hipError_t launch_bias_update(int64_t n_rows, int E, const int32_t* counts, float gamma, float* bias,
                              int32_t* load, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(kThreads), 0, s, counts, n_rows, E, gamma, bias,
                     load);
  return hipGetLastError();
}

}  // namespace moe
