// Weight preparation kernels (run once per weight load, not per step).
//
//  gate_prepare     fp32 W_g [d, E] -> three bf16 planes [3, E, d] with
//                   hi + mid + lo == W exactly: hi = bf16(w), mid = bf16(w - hi),
//                   lo = bf16(w - hi - mid).  Each residual is exact in fp32
//                   and fits the next plane's 8 significant bits, so the gate
//                   product can run on bf16 matrix cores with exact products
//                   (the router stays out of low precision: deepnotes "The
//                   iteration loop").
//  quantize_blocks  fp32 [n, R, C] -> e4m3 codes with one fp32 scale per
//                   128 x 128 block (the fp8 workload's weight format).
//  quantize_rows    bf16 [rows, C] -> e4m3 codes with one fp32 scale per
//                   1 x 128 tile of a row (the shared expert's input in the fp8
//                   workload; routed rows are quantised inside dispatch).
#pragma clang fp contract(off)

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// split != nullptr: block 0 also writes the split gate product's ticket set
// (zeros) and its group offsets {0, T, ..., S*T} after it.
__global__ __launch_bounds__(256) void gate_prepare_kernel(int d, int E, const float* __restrict__ w,
                                                           uint16_t* __restrict__ out, int* split, int S,
                                                           int64_t T) {
  if (split != nullptr && blockIdx.x == 0) {
    for (int j = threadIdx.x; j < kTicketInts; j += 256) split[j] = 0;
    if (threadIdx.x <= S) split[kTicketInts + threadIdx.x] = static_cast<int>(threadIdx.x * T);
  }
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over E*d, d fastest
  if (i >= (int64_t)E * d) return;
  const int e = static_cast<int>(i / d), kk = static_cast<int>(i % d);
  const float v = w[(int64_t)kk * E + e];
  const uint16_t hi = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(hi);
  const uint16_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  const uint16_t lo = f32_to_bf16(r2);
  const int64_t plane = (int64_t)E * d;
  out[i] = hi;
  out[plane + i] = mid;
  out[2 * plane + i] = lo;
}

// The same split, 64 x 64 tiles through LDS (d % 64 == 0, E % 64 == 0): the
// tile is read as 64 rows of W_g (64 experts, contiguous) and written as 64
// plane rows (64 columns of d, contiguous), both in whole cache lines.
__global__ __launch_bounds__(256) void gate_prepare_tiled_kernel(int d, int E, const float* __restrict__ w,
                                                                 uint16_t* __restrict__ out, int* split, int S,
                                                                 int64_t T) {
  __shared__ float tile[64][65];
  if (split != nullptr && blockIdx.x == 0 && blockIdx.y == 0) {
    for (int j = threadIdx.x; j < kTicketInts; j += 256) split[j] = 0;
    if (threadIdx.x <= S) split[kTicketInts + threadIdx.x] = static_cast<int>(threadIdx.x * T);
  }
  const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int t = threadIdx.x;
  {
    const int c = (t % 16) * 4;  // 4 experts per thread
#pragma unroll
    for (int r = t / 16; r < 64; r += 16) {
      const float4 v = *reinterpret_cast<const float4*>(w + (int64_t)(k0 + r) * E + e0 + c);
      tile[r][c] = v.x;
      tile[r][c + 1] = v.y;
      tile[r][c + 2] = v.z;
      tile[r][c + 3] = v.w;
    }
  }
  __syncthreads();
  const int e = t / 4, kc = (t % 4) * 16;  // 16 columns of d per thread
  uint16_t hi[16], mid[16], lo[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float v = tile[kc + j][e];
    hi[j] = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi[j]);
    mid[j] = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid[j]);
    lo[j] = f32_to_bf16(r2);
  }
  const int64_t plane = (int64_t)E * d;
  const int64_t base = (int64_t)(e0 + e) * d + k0 + kc;
  auto put = [&](uint16_t* dst, const uint16_t* v) {
    uint4 a, b;
    a.x = v[0] | (uint32_t)v[1] << 16; a.y = v[2] | (uint32_t)v[3] << 16;
    a.z = v[4] | (uint32_t)v[5] << 16; a.w = v[6] | (uint32_t)v[7] << 16;
    b.x = v[8] | (uint32_t)v[9] << 16; b.y = v[10] | (uint32_t)v[11] << 16;
    b.z = v[12] | (uint32_t)v[13] << 16; b.w = v[14] | (uint32_t)v[15] << 16;
    reinterpret_cast<uint4*>(dst)[0] = a;
    reinterpret_cast<uint4*>(dst)[1] = b;
  };
  put(out + base, hi);
  put(out + plane + base, mid);
  put(out + 2 * plane + base, lo);
}

constexpr int kBlk = MOE_FP8_TILE;

__global__ __launch_bounds__(256) void quantize_blocks_kernel(int rows, int cols,
                                                              const float* __restrict__ w,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ scale) {
  __shared__ float s_red[4];
  const int rb = rows / kBlk, cb = cols / kBlk;
  const int64_t blk = blockIdx.x;
  const int64_t mat = blk / ((int64_t)rb * cb);
  const int br = static_cast<int>((blk / cb) % rb), bc = static_cast<int>(blk % cb);
  const float* base = w + mat * rows * (int64_t)cols + (int64_t)br * kBlk * cols + bc * kBlk;
  uint8_t* qbase = q + mat * rows * (int64_t)cols + (int64_t)br * kBlk * cols + bc * kBlk;
  const int tid = threadIdx.x;
  float amax = 0.0f;
  for (int i = tid; i < kBlk * kBlk / 4; i += 256) {
    const int r = i / (kBlk / 4), c4 = i % (kBlk / 4);
    const float4 v = reinterpret_cast<const float4*>(base + (int64_t)r * cols)[c4];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  if ((tid & 63) == 0) s_red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float sc = e4m3_tile_scale(amax);
  if (tid == 0) scale[blk] = sc;
  for (int i = tid; i < kBlk * kBlk / 4; i += 256) {
    const int r = i / (kBlk / 4), c4 = i % (kBlk / 4);
    const float4 v = reinterpret_cast<const float4*>(base + (int64_t)r * cols)[c4];
    const uint32_t packed = f32_to_e4m3(v.x / sc) | (f32_to_e4m3(v.y / sc) << 8) |
                            (f32_to_e4m3(v.z / sc) << 16) | (f32_to_e4m3(v.w / sc) << 24);
    reinterpret_cast<uint32_t*>(qbase + (int64_t)r * cols)[c4] = packed;
  }
}

// 8 lanes per 128-wide tile, 16 elements each (two 16-byte loads, one
// 16-byte store of codes); a wave covers 8 rows of one tile column and a
// work-group 32 rows, so a work-group's block-major scales are 32
// consecutive floats.
__global__ __launch_bounds__(256) void quantize_rows_kernel(int64_t rows, int cols,
                                                            const uint16_t* __restrict__ x,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  if (row >= rows) return;  // whole 8-lane groups
  const int blk = blockIdx.y;
  const int sub = threadIdx.x & 7;
  const int64_t col = (int64_t)blk * kBlk + sub * 16;
  const uint4* src = reinterpret_cast<const uint4*>(x + row * cols + col);
  const uint4 v0 = src[0], v1 = src[1];
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  float f[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
    f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  const float sc = e4m3_tile_scale(amax);
  uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i >> 2] |= f32_to_e4m3(f[i] / sc) << (8 * (i & 3));
  *reinterpret_cast<uint4*>(q + row * cols + col) = make_uint4(o[0], o[1], o[2], o[3]);
  // scales block-major: [cols/128][rows]
  if (sub == 0) scale[(int64_t)blk * rows + row] = sc;
}

}  // namespace

hipError_t launch_quantize_rows(int64_t rows, int cols, const uint16_t* x, uint8_t* q, float* scale,
                                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols / kBlk > 65535) return hipErrorInvalidValue;  // tile columns are the grid's y
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((rows + 31) / 32), (unsigned)(cols / kBlk)), dim3(256),
                     0, s, rows, cols, x, q, scale);
  return hipGetLastError();
}

hipError_t launch_gate_prepare(int d, int E, const float* w_gate, uint16_t* w_prep,
                               hipStream_t s, int* split, int S, int64_t T) {
  const int64_t n = (int64_t)E * d;
  if (split != nullptr && (S < 1 || S > kMaxGateSplits)) return hipErrorInvalidValue;
  if (d % 64 == 0 && E % 64 == 0 && (reinterpret_cast<uintptr_t>(w_gate) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(w_prep) & 31) == 0) {
    hipLaunchKernelGGL(gate_prepare_tiled_kernel, dim3((unsigned)(d / 64), (unsigned)(E / 64)), dim3(256), 0, s,
                       d, E, w_gate, w_prep, split, S, T);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gate_prepare_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, d, E,
                     w_gate, w_prep, split, S, T);
  return hipGetLastError();
}

hipError_t launch_quantize_blocks(int64_t n, int rows, int cols, const float* w, uint8_t* q,
                                  float* scale, hipStream_t s) {
  const int64_t nb = n * (rows / kBlk) * (cols / kBlk);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_blocks_kernel, dim3((unsigned)nb), dim3(256), 0, s, rows, cols, w, q,
                     scale);
  return hipGetLastError();
}

}  // namespace moe
