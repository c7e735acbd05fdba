// Grouped GEMM on the vector ALUs (fp32 FMA), for fp32 workloads and for
// shapes the matrix-core tiles do not cover.  Same grouped tile map as the MFMA
// kernels; 64 x 64 output tile, 256 threads with 4 x 4 outputs each, K staged
// through LDS 16 at a time.  Stages:
//   GATE  logits = x . (hi + mid + lo)   (three bf16 planes summed exactly)
//   UP    h = silu(x W1^T) * (x W3^T)    (SwiGLU, mastering-deepseek-v4 Exp08)
//   DOWN  y = h W2^T
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

enum { ST_GATE = 0, ST_UP = 1, ST_DOWN = 2 };

struct SimtArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t b_group_stride;
  void* C;
  int64_t ldc;
  const int* offsets;
  int n_exp;
  int64_t rows_total;
  int K;
  int n_out;   // output columns
  int n_tiles;
  int d_ff;    // UP: first W3 row; GATE: plane stride / K
};

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

template <typename T, int ST>
__global__ __launch_bounds__(256) void gemm_simt_kernel(const SimtArgs p) {
  constexpr int BM = 64, BN = 64, BKs = 16;
  __shared__ float sA[BKs][BM + 1];
  __shared__ float sB[BKs][BN + 1];
  __shared__ float sB2[BKs][BN + 1];
  __shared__ int s_pre[kMapInts];

  TileInfo ti;
  if (!map_tile(p.offsets, p.n_exp, p.rows_total, BM, p.n_tiles, s_pre, ti)) return;

  const T* A = static_cast<const T*>(p.A);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = ti.n_tile * BN;
  float acc[4][4] = {}, acc2[4][4] = {};

  for (int k0 = 0; k0 < p.K; k0 += BKs) {
    for (int e = tid; e < BM * BKs; e += 256) {
      const int r = e / BKs, kk = e % BKs;
      float v = 0.0f;
      if (r < ti.rows && k0 + kk < p.K) v = ld(A, (ti.row0 + r) * p.lda + k0 + kk);
      sA[kk][r] = v;
    }
    for (int e = tid; e < BN * BKs; e += 256) {
      const int n = e / BKs, kk = e % BKs, gn = n0 + n;
      float v = 0.0f, v2 = 0.0f;
      if (gn < p.n_out && k0 + kk < p.K) {
        if constexpr (ST == ST_GATE) {
          const uint16_t* B = static_cast<const uint16_t*>(p.B);
          const int64_t plane = (int64_t)p.n_out * p.K;
          const int64_t o = (int64_t)gn * p.K + k0 + kk;
          v = (bf16_to_f32(B[o]) + bf16_to_f32(B[o + plane])) + bf16_to_f32(B[o + 2 * plane]);
        } else {
          const T* B = static_cast<const T*>(p.B) + (int64_t)ti.group * p.b_group_stride;
          v = ld(B, (int64_t)gn * p.K + k0 + kk);
          if constexpr (ST == ST_UP) v2 = ld(B, (int64_t)(p.d_ff + gn) * p.K + k0 + kk);
        }
      }
      sB[kk][n] = v;
      if constexpr (ST == ST_UP) sB2[kk][n] = v2;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKs; ++kk) {
      float a[4], b[4], b2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = sB[kk][tx * 4 + j];
        if constexpr (ST == ST_UP) b2[j] = sB2[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
          if constexpr (ST == ST_UP) acc2[i][j] = __builtin_fmaf(a[i], b2[j], acc2[i][j]);
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= ti.rows) continue;
    const int64_t grow = ti.row0 + r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= p.n_out) continue;
      if constexpr (ST == ST_GATE) {
        static_cast<float*>(p.C)[grow * p.ldc + col] = acc[i][j];
      } else if constexpr (ST == ST_UP) {
        const float g = acc[i][j];
        st(static_cast<T*>(p.C), grow * p.ldc + col, g / (1.0f + __expf(-g)) * acc2[i][j]);
      } else {
        st(static_cast<T*>(p.C), grow * p.ldc + col, acc[i][j]);
      }
    }
  }
}

template <typename T, int ST>
hipError_t launch(const SimtArgs& a, int64_t max_rows, hipStream_t s) {
  const int64_t mt = max_row_tiles(max_rows, a.offsets == nullptr ? 1 : a.n_exp, 64);
  const int64_t grid = (mt * a.n_tiles + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_simt_kernel<T, ST>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_gemm_simt(const void* x, int x_dtype, const uint16_t* w_prep,
                                 float* logits, int64_t T, int d, int E, hipStream_t s) {
  SimtArgs a{};
  a.A = x;
  a.lda = d;
  a.B = w_prep;
  a.C = logits;
  a.ldc = E;
  a.offsets = nullptr;
  a.n_exp = 1;
  a.rows_total = T;
  a.K = d;
  a.n_out = E;
  a.n_tiles = (E + 63) / 64;
  if (x_dtype == MOE_F32) return launch<float, ST_GATE>(a, T, s);
  return launch<uint16_t, ST_GATE>(a, T, s);
}

hipError_t launch_ffn_simt(int stage, int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                           int d_ff, int dtype, const void* in, const void* w, void* out,
                           hipStream_t s) {
  SimtArgs a{};
  a.A = in;
  a.B = w;
  a.C = out;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.d_ff = d_ff;
  if (stage == MOE_FFN_UP) {
    a.lda = d;
    a.b_group_stride = (int64_t)2 * d_ff * d;
    a.ldc = d_ff;
    a.K = d;
    a.n_out = d_ff;
  } else {
    a.lda = d_ff;
    a.b_group_stride = (int64_t)d * d_ff;
    a.ldc = d;
    a.K = d_ff;
    a.n_out = d;
  }
  a.n_tiles = (a.n_out + 63) / 64;
  if (dtype == MOE_F32) {
    return stage == MOE_FFN_UP ? launch<float, ST_UP>(a, max_rows, s)
                               : launch<float, ST_DOWN>(a, max_rows, s);
  }
  return stage == MOE_FFN_UP ? launch<uint16_t, ST_UP>(a, max_rows, s)
                             : launch<uint16_t, ST_DOWN>(a, max_rows, s);
}

}  // namespace moe
