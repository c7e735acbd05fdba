// Combine on gfx950: out[t] = ysh[t] + sum_j w[t,j] * yp[dest[t,j]]
// (w = nullptr: unit weights, which is also the backward of dispatch)
// (deepmox ch.5 "The network becomes part of the forward pass": the forward
// chunk ends by combining the expert outputs; zenaique "Why all to all
// dominates": combine brings FFN outputs back to the token's owner).
//
// A gather, not a scatter: each work-group owns a few tokens and pulls their k
// expert rows in 16-byte chunks, so every output element is written once,
// without atomics, and the fp32 sum runs in slot order (deterministic).  Every
// byte is touched once, so accesses are nontemporal.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerWg = 4;
constexpr int kMaxK = 16;
constexpr int kVec = 8;  // elements per chunk

struct CombArgs {
  int64_t T;
  int k, d;
  const int32_t* dest;
  const float* w;
  const void* yp;
  const void* ysh;
  void* out;
};

template <typename TY>
__device__ __forceinline__ void load8(const TY* p, float (&f)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&f)[8]) {
  const uint4 v = ld_stream(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
    f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&f)[8]) {
  const uint4 a = ld_stream(p), b = ld_stream(p + 4);
  f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
  f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
}

template <typename TO>
__device__ __forceinline__ void store8(TO* p, const float (&f)[8]);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float (&f)[8]) {
  st_stream(p, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                          pack_bf16x2(f[6], f[7])));
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&f)[8]) {
  st_stream(p, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])));
  st_stream(p + 4, make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7])));
}

template <typename TY, typename TO, bool ACC>
__global__ __launch_bounds__(kThreads) void combine_kernel(const CombArgs p) {
  __shared__ int s_dest[kTokPerWg * kMaxK];
  __shared__ float s_w[kTokPerWg * kMaxK];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerWg;
  const int ntok = static_cast<int>(min((int64_t)kTokPerWg, p.T - t0));
  for (int q = tid; q < ntok * p.k; q += kThreads) {
    const int tt = q / p.k, j = q % p.k;
    s_dest[tt * kMaxK + j] = p.dest[(t0 + tt) * p.k + j];
    s_w[tt * kMaxK + j] = p.w == nullptr ? 1.0f : p.w[(t0 + tt) * p.k + j];
  }
  __syncthreads();
  const int nch = p.d / kVec;
  const TY* yp = static_cast<const TY*>(p.yp);
  const TY* ysh = static_cast<const TY*>(p.ysh);
  TO* out = static_cast<TO*>(p.out);
  for (int q = tid; q < ntok * nch; q += kThreads) {
    const int tt = q / nch, c = q % nch;
    const int64_t t = t0 + tt;
    float acc[8];
    if constexpr (ACC) {
      load8<TO>(out + t * p.d + c * kVec, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    if (ysh != nullptr) {
      float f[8];
      load8<TY>(ysh + t * p.d + c * kVec, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
    for (int j = 0; j < p.k; ++j) {
      const int r = s_dest[tt * kMaxK + j];
      if (r < 0) continue;
      const float wj = s_w[tt * kMaxK + j];
      float f[8];
      load8<TY>(yp + (int64_t)r * p.d + c * kVec, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, f[i], acc[i]);
    }
    store8<TO>(out + t * p.d + c * kVec, acc);
  }
}

template <typename TY, typename TO, bool ACC>
hipError_t launch_t(const CombArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.T + kTokPerWg - 1) / kTokPerWg);
  hipLaunchKernelGGL((combine_kernel<TY, TO, ACC>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(int64_t T, int k, int d, const int32_t* dest, const float* w,
                          const void* yp, int y_dtype, const void* ysh, void* out,
                          int out_dtype, int accumulate, hipStream_t s) {
  CombArgs a{T, k, d, dest, w, yp, ysh, out};
  if (y_dtype == MOE_BF16) {
    if (out_dtype == MOE_BF16) return launch_t<uint16_t, uint16_t, false>(a, s);
    return accumulate ? launch_t<uint16_t, float, true>(a, s) : launch_t<uint16_t, float, false>(a, s);
  }
  if (out_dtype == MOE_BF16) return launch_t<float, uint16_t, false>(a, s);
  return accumulate ? launch_t<float, float, true>(a, s) : launch_t<float, float, false>(a, s);
}

}  // namespace moe
