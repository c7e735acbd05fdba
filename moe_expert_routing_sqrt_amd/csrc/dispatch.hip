// Dispatch on gfx950: per-expert counts, exclusive scan and the stable
// permutation that packs token rows into an expert-contiguous buffer
// (deepmox ch.5 "The network becomes part of the forward pass": the forward
// chunk dispatches tokens to the experts; zenaique "Why all to all dominates":
// dispatch ships each token row to the holders of its k experts).
//
// Determinism without atomics on the output order: moe_route already counted
// pairs per (64-token block, expert).  A scan kernel turns those counts into
// per-expert offsets and a base row for every (block, expert).  The permute
// kernel then gives pair (t, j) with expert e the row
//     base[block(t)][e] + #{ t' < t in the same block : e in idx[t'] },
// the within-block rank read off an LDS presence bitmap (one 64-bit word per
// expert; bit i = token i of the block chose e) with a popcount.  Rows within an
// expert therefore follow token order, exactly as the sequential definition.
//
// The copy reads each token row once and writes it to its k rows with 16-byte
// vector accesses; for the fp8 workload each 1 x 128 tile is quantised on the
// way (scale = amax/448, code = e4m3(x/scale)), once per token, and the codes
// are stored to every copy.  The scales go once per token into a token-major
// table (block-major over tokens, coalesced); a second pass gathers them into
// the block-major packed layout, xp_scale[b][r] = table[b][src[r]], so that the
// packed scales are written contiguously instead of as one scattered 4-byte
// store per (copy, block).
#pragma clang fp contract(off)

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

// base[b][e] = offsets[e] + pairs of expert e in blocks before b
__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(
    const int32_t* __restrict__ block_counts, int nblk, int E, int e_begin, int n,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ base) {
  __shared__ int s_part[kScanThreads];   // partial sums per (part, expert)
  __shared__ int s_tot[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int parts = max(1, kScanThreads / n);
  const int bpp = (nblk + parts - 1) / parts;
  const int e = tid % n, part = tid / n;
  const bool active = part < parts && tid < parts * n;
  const int b0 = part * bpp, b1 = min(nblk, b0 + bpp);

  // (the block loops are unrolled so that a thread's loads are in flight
  // together rather than one round trip per block)
  int sum = 0;
  if (active) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) sum += block_counts[(int64_t)b * E + e_begin + e];
    s_part[part * n + e] = sum;
  }
  __syncthreads();
  // per expert: exclusive scan over parts (one thread per expert)
  if (tid < n) {
    int run = 0;
    for (int q = 0; q < parts; ++q) {
      const int v = s_part[q * n + tid];
      s_part[q * n + tid] = run;
      run += v;
    }
    s_tot[tid] = run;
    counts[tid] = run;
  }
  __syncthreads();
  // exclusive scan over experts (wave 0, chunk per lane)
  if (tid < kWave) {
    const int per = (n + kWave - 1) / kWave;
    const int g0 = tid * per;
    int csum = 0;
    for (int g = g0; g < g0 + per && g < n; ++g) csum += s_tot[g];
    int incl = csum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (tid >= o) incl += v;
    }
    int run = incl - csum;
    for (int g = g0; g < g0 + per && g < n; ++g) {
      const int c = s_tot[g];
      s_tot[g] = run;
      offsets[g] = run;
      run += c;
    }
    if (tid == kWave - 1) offsets[n] = incl;
  }
  __syncthreads();
  if (active) {
    int run = s_tot[e] + s_part[part * n + e];
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      base[(int64_t)b * n + e] = run;
      run += block_counts[(int64_t)b * E + e_begin + e];
    }
  }
}

constexpr int kPermThreads = 256;
constexpr int kTokPerWg = 16;  // a 64-token route block is split over 4 work-groups
constexpr int kMaxK = 16;

struct PermArgs {
  const int32_t* idx;
  const int32_t* base;
  int64_t T;
  int k, e_begin, e_end, n;
  const void* x;
  int d;
  int32_t* dest;
  int32_t* src;
  void* xp;
  float* tok_scale;  // [d/128][T]: e4m3 scale of token t's block b at tok_scale[b * T + t]
};

// ROW_BYTES_ELEM: bytes per input element (2 bf16, 4 f32); FP8: quantise bf16 -> e4m3
template <int ELEM, bool FP8>
__global__ __launch_bounds__(kPermThreads) void dispatch_permute_kernel(const PermArgs p) {
  __shared__ unsigned long long s_pres[256];
  __shared__ int s_dest[kTokPerWg * kMaxK];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerWg;
  const int64_t bstart = t0 / MOE_ROUTE_BLOCK * MOE_ROUTE_BLOCK;
  const int blk = static_cast<int>(t0 / MOE_ROUTE_BLOCK);
  const int64_t t_end = min(p.T, t0 + kTokPerWg);
  if (t0 >= p.T) return;

  for (int e = tid; e < p.n; e += kPermThreads) s_pres[e] = 0ull;
  __syncthreads();
  // presence bits of the block's tokens up to this work-group's last token
  const int npairs_pre = static_cast<int>(t_end - bstart) * p.k;
  for (int q = tid; q < npairs_pre; q += kPermThreads) {
    const int i = q / p.k;
    const int e = p.idx[(bstart + i) * p.k + q % p.k];
    if (e >= p.e_begin && e < p.e_end) atomicOr(&s_pres[e - p.e_begin], 1ull << i);
  }
  __syncthreads();
  const int ntok = static_cast<int>(t_end - t0);
  for (int q = tid; q < ntok * p.k; q += kPermThreads) {
    const int tt = q / p.k, j = q % p.k;
    const int64_t t = t0 + tt;
    const int e = p.idx[t * p.k + j];
    int r = -1;
    if (e >= p.e_begin && e < p.e_end) {
      const int le = e - p.e_begin;
      const int i = static_cast<int>(t - bstart);
      const unsigned long long below = i == 0 ? 0ull : (s_pres[le] & ((1ull << i) - 1ull));
      r = p.base[(int64_t)blk * p.n + le] + __popcll(below);
      p.src[r] = static_cast<int32_t>(t);
    }
    p.dest[t * p.k + j] = r;
    s_dest[tt * kMaxK + j] = r;
  }
  __syncthreads();

  // row copies: 16-byte chunks, token-major over this work-group's tokens
  constexpr int kVec = 16 / ELEM;  // elements per chunk
  const int nch = p.d / kVec;
  const int k = p.k;
  if constexpr (!FP8) {
    for (int q = tid; q < ntok * nch; q += kPermThreads) {
      const int tt = q / nch, c = q % nch;
      const uint4 v = reinterpret_cast<const uint4*>(static_cast<const char*>(p.x) + (t0 + tt) * (int64_t)p.d * ELEM)[c];
      for (int j = 0; j < k; ++j) {
        const int r = s_dest[tt * kMaxK + j];
        if (r >= 0) st_stream(static_cast<char*>(p.xp) + ((int64_t)r * p.d * ELEM + (int64_t)c * 16), v);
      }
    }
  } else {
    // e4m3: a lane takes 16 bf16 (two 16-byte chunks) and writes their 16
    // codes as one 16-byte store; a 128-column tile is 8 consecutive lanes
    const int npair = p.d / 16;
    for (int q = tid; q < ntok * npair; q += kPermThreads) {
      const int tt = q / npair, c2 = q % npair;
      const int64_t t = t0 + tt;
      const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + t * (int64_t)p.d);
      const uint4 v0 = xr[2 * c2], v1 = xr[2 * c2 + 1];
      float f[16];
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
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
      const float scale = e4m3_tile_scale(amax);
      uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i >> 2] |= f32_to_e4m3(f[i] / scale) << (8 * (i & 3));
      const uint4 out = make_uint4(o[0], o[1], o[2], o[3]);
      if ((c2 & 7) == 0) p.tok_scale[(int64_t)(c2 >> 3) * p.T + t] = scale;
      for (int j = 0; j < k; ++j) {
        const int r = s_dest[tt * kMaxK + j];
        if (r >= 0) st_stream(static_cast<uint8_t*>(p.xp) + (int64_t)r * p.d + (int64_t)c2 * 16, out);
      }
    }
  }
}

// xp_scale[b][r] = tok_scale[b][src[r]] for the packed rows r < offsets[n]
// (block b = blockIdx.y; rows past them are left as they are)
__global__ __launch_bounds__(256) void scale_gather_kernel(const int32_t* __restrict__ src,
                                                           const int32_t* __restrict__ n_rows,
                                                           const float* __restrict__ tok_scale, int64_t T,
                                                           int64_t P, float* __restrict__ xp_scale) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= *n_rows) return;
  const int64_t b = blockIdx.y;
  xp_scale[b * P + r] = tok_scale[b * T + src[r]];
}

}  // namespace

hipError_t launch_dispatch(const int32_t* idx, const int32_t* block_counts, int64_t T, int k,
                           int E, int e_begin, int e_end, const void* x, int x_dtype,
                           int out_dtype, int d, int32_t* counts, int32_t* offsets,
                           int32_t* dest, int32_t* src, void* xp, float* xp_scale, int32_t* base,
                           float* tok_scale, hipStream_t s) {
  const int n = e_end - e_begin;
  const int nblk = static_cast<int>((T + MOE_ROUTE_BLOCK - 1) / MOE_ROUTE_BLOCK);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, block_counts, nblk, E,
                     e_begin, n, counts, offsets, base);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  PermArgs a{idx, base, T, k, e_begin, e_end, n, x, d, dest, src, xp, tok_scale};
  const unsigned grid = static_cast<unsigned>((T + kTokPerWg - 1) / kTokPerWg);
  if (out_dtype == MOE_E4M3) {
    hipLaunchKernelGGL((dispatch_permute_kernel<2, true>), dim3(grid), dim3(kPermThreads), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t P = T * k;
    const dim3 g(static_cast<unsigned>((P + 255) / 256), static_cast<unsigned>(d / MOE_FP8_TILE));
    hipLaunchKernelGGL(scale_gather_kernel, g, dim3(256), 0, s, src, offsets + n, tok_scale, T, P, xp_scale);
  } else if (x_dtype == MOE_BF16)
    hipLaunchKernelGGL((dispatch_permute_kernel<2, false>), dim3(grid), dim3(kPermThreads), 0, s, a);
  else
    hipLaunchKernelGGL((dispatch_permute_kernel<4, false>), dim3(grid), dim3(kPermThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
