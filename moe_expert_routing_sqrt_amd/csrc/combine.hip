// Combine on gfx950: out[t] = ysh[t] + sum_j w[t,j] * yp[dest[t,j]]
// (w = nullptr: unit weights, which is also the backward of dispatch)
// (deepmox ch.5 "The network becomes part of the forward pass": the forward
// chunk ends by combining the expert outputs; zenaique "Why all to all
// dominates": combine brings FFN outputs back to the token's owner).
//
// A gather, not a scatter: each work-group owns a few tokens and pulls their k
// expert rows in 16-byte chunks, so every output element is written once,
// without atomics, and the fp32 sum runs in slot order (deterministic).  Every
// byte is touched once.  Measured on MI355X (V3 rows): nontemporal loads with
// ordinary stores beat the other three combinations (0.426 ms against
// 0.456-0.478), and 2 tokens per 256-thread work-group beat 4 and 8.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerWg = 2;
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

// 8 consecutive values in their stored form: one 16-byte chunk of bf16, or
// two of f32
template <typename TY>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  u32x4 v;
};
template <>
struct Raw8<float> {
  u32x4 a, b;
};

__device__ __forceinline__ Raw8<uint16_t> load_raw8(const uint16_t* p) {
  return {__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))};
}
__device__ __forceinline__ Raw8<float> load_raw8(const float* p) {
  return {__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)),
          __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4))};
}

// an empty asm that takes the registers as operands: the compiler must have
// the load complete here, which puts one wait after a batch of loads
__device__ __forceinline__ void landed(Raw8<uint16_t>& r) { asm volatile("" : "+v"(r.v)); }
__device__ __forceinline__ void landed(Raw8<float>& r) { asm volatile("" : "+v"(r.a), "+v"(r.b)); }

__device__ __forceinline__ void to_f32(const Raw8<uint16_t>& r, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(static_cast<uint16_t>(r.v[i] & 0xFFFFu));
    f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(r.v[i] >> 16));
  }
}
__device__ __forceinline__ void to_f32(const Raw8<float>& r, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = __uint_as_float(r.a[i]);
    f[4 + i] = __uint_as_float(r.b[i]);
  }
}

template <typename TO>
__device__ __forceinline__ void store8(TO* p, const float (&f)[8]);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float (&f)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                            pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&f)[8]) {
  reinterpret_cast<uint4*>(p)[0] =
      make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  reinterpret_cast<uint4*>(p)[1] =
      make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7]));
}

// KU: compile-time bound on k.  A token's local slots are listed first in LDS
// (in slot order, so the sum keeps the slot order); a lane issues the row loads
// of all of them, and of the shared-expert row and the accumulated output,
// before it waits once and sums.
template <typename TY, typename TO, bool ACC, int KU>
__global__ __launch_bounds__(kThreads) void combine_kernel(const CombArgs p) {
  __shared__ __align__(16) int s_dest[kTokPerWg * kMaxK];
  __shared__ __align__(16) float s_w[kTokPerWg * kMaxK];
  __shared__ int s_nv[kTokPerWg];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerWg;
  const int ntok = static_cast<int>(min((int64_t)kTokPerWg, p.T - t0));
  static_assert(kTokPerWg * kMaxK <= kWave, "the slot table is built by one wave");
  if (tid < kWave) {
    // lane tid = slot j of token tt; a ballot compacts each token's local slots
    const int tt = tid / p.k, j = tid - tt * p.k;
    const bool in = tt < ntok;
    const int r = in ? p.dest[(t0 + tt) * p.k + j] : -1;
    const uint64_t valid = __ballot(r >= 0);
    const uint64_t first = 1ull << (tt * p.k);  // tt * k < 64 whenever `in`
    if (r >= 0) {
      const int pos = __popcll(valid & ((1ull << tid) - first));
      s_dest[tt * kMaxK + pos] = r;
      s_w[tt * kMaxK + pos] = p.w == nullptr ? 1.0f : p.w[(t0 + tt) * p.k + j];
    }
    if (in && j == 0) s_nv[tt] = __popcll((valid >> (tt * p.k)) & ((1ull << p.k) - 1ull));
  }
  __syncthreads();
  const int nch = p.d / kVec;
  const TY* yp = static_cast<const TY*>(p.yp);
  const TY* ysh = static_cast<const TY*>(p.ysh);
  TO* out = static_cast<TO*>(p.out);
  for (int q = tid; q < ntok * nch; q += kThreads) {
    const int tt = q / nch, c = q - tt * nch;
    const int64_t e0 = (t0 + tt) * p.d + c * kVec;
    const int nv = s_nv[tt];
    int rj[KU];
    float wj[KU];  // entries at and past nv are stale and never used
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      rj[j] = s_dest[tt * kMaxK + j];
      wj[j] = s_w[tt * kMaxK + j];
    }
    Raw8<TY> raw[KU];
#pragma unroll
    for (int j = 0; j < KU; ++j)
      if (j < nv) raw[j] = load_raw8(yp + (int64_t)rj[j] * p.d + c * kVec);
    Raw8<TY> rsh;
    if (ysh != nullptr) rsh = load_raw8(ysh + e0);
    Raw8<TO> rout;
    if constexpr (ACC) rout = load_raw8(out + e0);
#pragma unroll
    for (int j = 0; j < KU; ++j) landed(raw[j]);
    landed(rsh);
    if constexpr (ACC) landed(rout);

    float acc[8];
    if constexpr (ACC) {
      to_f32(rout, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    if (ysh != nullptr) {
      float f[8];
      to_f32(rsh, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      if (j >= nv) break;
      float f[8];
      to_f32(raw[j], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj[j], f[i], acc[i]);
    }
    store8<TO>(out + e0, acc);
  }
}

template <typename TY, typename TO, bool ACC>
hipError_t launch_t(const CombArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.T + kTokPerWg - 1) / kTokPerWg);
  if (a.k <= 8)
    hipLaunchKernelGGL((combine_kernel<TY, TO, ACC, 8>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<TY, TO, ACC, kMaxK>), dim3(grid), dim3(kThreads), 0, s, a);
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
