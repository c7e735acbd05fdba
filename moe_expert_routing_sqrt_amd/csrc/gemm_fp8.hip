// Grouped e4m3 GEMM on gfx950 matrix cores for the fp8 workload: activations
// with one fp32 scale per 1 x 128 tile of a row, weights with one fp32 scale
// per 128 x 128 block, fp32 accumulation.
//
//   C[m][n] = sum_kb  sa[m][kb] * sb[n/128][kb] * sum_{k in kb} qa[m][k] * qb[n][k]
//
// The matrix cores' own block scales are powers of two per 32 elements, which
// cannot express fp32 scales, so each 128-wide K block is accumulated on its
// own (two v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales into a partial
// accumulator) and promoted on the vector ALUs: acc += partial * sa * sb.
//
// Tile: 128 tokens x 256 features x 128 (one scale block) per K step, 512
// threads = 8 wave64s (2 x 4), each owning 64 x 64.  Two waves per SIMD let
// one wave's promotion overlap the other's MFMAs.  A K step is 128 bytes per
// row, the same LDS row format as the bf16 kernel: 16-byte chunks swizzled by
// (row >> 1) & 7, three-stage DMA ring, one barrier per step, each wave
// waiting only for its own DMA of the stage it reads.  Row scales of A travel
// with the stage (4-byte DMA), block scales of B are scalar loads.
//
// Epilogues
//   SWIGLU  h = silu(gate) * up in fp32, then quantised per 1 x 128 tile of h
//           (a tile's 128 h columns are one quantisation tile: the row amax is
//           reduced across lanes and across the four feature waves in LDS);
//           writes e4m3 codes and the fp32 scale.
//   STORE   bf16 output (the down projection).
#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 256, BKB = 128;  // K step = 128 fp8 bytes = one scale block
constexpr int kThreads = 512;
constexpr int WAVES_M = 2, WAVES_N = 4;
constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // 64 x 64 per wave
constexpr int RM = TM / 32, RN = TN / 32;             // 2 x 2 accumulators of 32 x 32
constexpr int NW = kThreads / 64;
constexpr int ADMA = BM / 8 / NW;   // 1 KB blocks per wave per step
constexpr int BDMA = BN / 8 / NW;
constexpr int DMA_PER_STEP = ADMA + BDMA + 1;  // + one 4-byte DMA of row scales

enum { MODE_SWIGLU = 0, MODE_STORE = 1 };

struct Fp8Args {
  const uint8_t* A;       // [rows, K] codes
  const float* A_scale;   // [K/128][rows_total]: a 128-wide block's scales contiguous over rows
  int64_t lda;            // bytes per row (= K)
  const uint8_t* B;       // [groups][N_rows][K] codes
  const float* B_scale;   // [groups][N_rows/128][K/128]
  int64_t b_group_stride; // bytes
  int64_t bs_group_stride;// floats
  void* C;
  float* C_scale;         // SWIGLU: [d_ff/128][rows_total]
  int64_t ldc;
  const int* offsets;
  int n_exp;
  int64_t rows_total;
  int K;
  int n_tiles;
  int d_ff;               // SWIGLU: first up row
};

typedef int i32x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8v as_i32x8(uint4 lo, uint4 hi) {
  i32x8v r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(const Fp8Args p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  __shared__ uint4 sA0[BM * 8], sA1[BM * 8], sA2[BM * 8];
  __shared__ uint4 sB0[BN * 8], sB1[BN * 8], sB2[BN * 8];
  __shared__ float sS0[BM], sS1[BM], sS2[BM];
  __shared__ float s_amax[WAVES_N][BM];
  __shared__ int s_pre[kMapInts];

  TileInfo ti;
  if (!map_tile(p.offsets, p.n_exp, p.rows_total, BM, p.n_tiles, s_pre, ti)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // DMA addressing (see the bf16 kernel): block j = wave + 8i covers rows
  // 8j..8j+7; for those rows (r >> 1) & 7 = 4*(wave & 1) + (lane >> 4).
  const int lrow = lane >> 3;
  const int lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  const uint8_t* a_src[ADMA];
  const uint8_t* b_src[BDMA];
#pragma unroll
  for (int i = 0; i < ADMA; ++i) {
    const int r = (wave + NW * i) * 8 + lrow;
    const int rc = r < ti.rows ? r : ti.rows - 1;
    a_src[i] = p.A + (int64_t)(ti.row0 + rc) * p.lda + lch * 16;
  }
  const uint8_t* bg = p.B + (int64_t)ti.group * p.b_group_stride + lch * 16;
#pragma unroll
  for (int i = 0; i < BDMA; ++i) {
    const int r = (wave + NW * i) * 8 + lrow;
    int grow;
    if constexpr (MODE == MODE_SWIGLU) {
      const int part = r / TN, within = r % TN;
      const int h0 = ti.n_tile * (BN / 2) + part * (TN / 2);
      grow = within < TN / 2 ? h0 + within : p.d_ff + h0 + (within - TN / 2);
    } else {
      grow = ti.n_tile * BN + r;
    }
    b_src[i] = bg + (int64_t)grow * p.K;
  }
  // row scales: lanes 0..15 of wave w fetch rows 16w..16w+15
  const int nkb = p.K / BKB;
  const int srow = 16 * wave + (lane & 15);
  const float* s_src = p.A_scale + (ti.row0 + (srow < ti.rows ? srow : ti.rows - 1));
  // block scales of B for this wave's two 32-column blocks
  const float* bs = p.B_scale + (int64_t)ti.group * p.bs_group_stride;
  int sb_row[RN];
  if constexpr (MODE == MODE_SWIGLU) {
    sb_row[0] = ti.n_tile;                       // gate features of this tile
    sb_row[1] = p.d_ff / BKB + ti.n_tile;        // the matching up features
  } else {
    sb_row[0] = sb_row[1] = (ti.n_tile * BN + wn * TN) / BKB;
  }

  const int nsteps = nkb;

  auto issue_part = [&](int kt, uint4* sa, uint4* sb, float* ss, int q0, int q1) {
    const int k0 = kt * BKB;
    const uint32_t la = lds_addr(sa), lb = lds_addr(sb);
#pragma unroll
    for (int q = 0; q < ADMA + BDMA + 1; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < ADMA) {
        dma16(a_src[q] + k0, la + (wave + NW * q) * 1024);
      } else if (q < ADMA + BDMA) {
        dma16(b_src[q - ADMA] + k0, lb + (wave + NW * (q - ADMA)) * 1024);
      } else {
        if (lane < 16) dma4(s_src + (int64_t)kt * p.rows_total, lds_addr(ss) + 64 * wave);
      }
    }
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int unit_scale = 0x7F7F7F7F;  // e8m0 127 = 2^0 in every byte

  auto compute = [&](const uint4* sa, const uint4* sb, const float* ss, int kt, int kn, uint4* na,
                     uint4* nb, float* ns) {
    // block scales of this step (scalar loads, used after the MFMAs)
    float sbv[RN];
#pragma unroll
    for (int j = 0; j < RN; ++j) sbv[j] = bs[(int64_t)sb_row[j] * nkb + kt];
    i32x8v fa[2][RM], fb[2][RN];
    auto read = [&](int buf, int h) {
      const int c0 = 4 * h + 2 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        const int r = wm * TM + i * 32 + (lane & 31);
        fa[buf][i] = as_i32x8(sa[swz(r, c0)], sa[swz(r, c0 + 1)]);
      }
#pragma unroll
      for (int j = 0; j < RN; ++j) {
        const int r = wn * TN + j * 32 + (lane & 31);
        fb[buf][j] = as_i32x8(sb[swz(r, c0)], sb[swz(r, c0 + 1)]);
      }
    };
    f32x16 part[RM][RN];
    read(0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 0) read(1, 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) {
          f32x16 c;
          if (h == 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) c[v] = 0.0f;
          } else {
            c = part[i][j];
          }
          part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[h][i], fb[h][j], c, 0, 0, 0, unit_scale, 0, unit_scale);
        }
      if (kn >= 0) {
        if (h == 0) issue_part(kn, na, nb, ns, 0, 4);
        else issue_part(kn, na, nb, ns, 4, ADMA + BDMA + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // promotion: acc += partial * sa[row] * sb[block]
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sa4 =
            *reinterpret_cast<const float4*>(ss + wm * TM + i * 32 + 8 * g + 4 * (lane >> 5));
        const float sav[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int j = 0; j < RN; ++j) {
            const int v = 4 * g + q;
            acc[i][j][v] = __builtin_fmaf(part[i][j][v], sav[q] * sbv[j], acc[i][j][v]);
          }
        }
      }
    }
  };

  auto step = [&](int kt, uint4* sa, uint4* sb, float* ss, uint4* na, uint4* nb, float* ns) {
    if (kt + 1 < nsteps) wait_vmcnt<DMA_PER_STEP>(); else wait_vmcnt<0>();
    barrier_only();
    compute(sa, sb, ss, kt, kt + 2 < nsteps ? kt + 2 : -1, na, nb, ns);
  };

  issue_part(0, sA0, sB0, sS0, 0, ADMA + BDMA + 1);
  if (nsteps > 1) issue_part(1, sA1, sB1, sS1, 0, ADMA + BDMA + 1);
  for (int kt = 0; kt < nsteps; kt += 3) {
    step(kt, sA0, sB0, sS0, sA2, sB2, sS2);
    if (kt + 1 < nsteps) step(kt + 1, sA1, sB1, sS1, sA0, sB0, sS0);
    if (kt + 2 < nsteps) step(kt + 2, sA2, sB2, sS2, sA1, sB1, sS1);
  }

  if constexpr (MODE == MODE_SWIGLU) {
    // h in fp32, then one e4m3 tile per row over the tile's 128 h columns
    float hv[RM][16];
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float g = acc[i][0][v];
        const float u = acc[i][1][v];
        hv[i][v] = g / (1.0f + __expf(-g)) * u;
        float m = fabsf(hv[i][v]);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        const int lr = wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if ((lane & 31) == 0) s_amax[wn][lr] = m;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (lr >= ti.rows) continue;
        float amax = s_amax[0][lr];
#pragma unroll
        for (int w = 1; w < WAVES_N; ++w) amax = fmaxf(amax, s_amax[w][lr]);
        const float sc = e4m3_tile_scale(amax);
        const int64_t grow = ti.row0 + lr;
        const int col = ti.n_tile * (BN / 2) + wn * (TN / 2) + (lane & 31);
        static_cast<uint8_t*>(p.C)[grow * p.ldc + col] = static_cast<uint8_t>(f32_to_e4m3(hv[i][v] / sc));
        if (wn == 0 && (lane & 31) == 0) p.C_scale[(int64_t)ti.n_tile * p.rows_total + grow] = sc;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (lr >= ti.rows) continue;
        uint16_t* out = static_cast<uint16_t*>(p.C) + (ti.row0 + lr) * p.ldc;
#pragma unroll
        for (int j = 0; j < RN; ++j)
          out[ti.n_tile * BN + wn * TN + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][v]);
      }
    }
  }
#endif
}

template <int MODE>
hipError_t launch(const Fp8Args& a, int64_t max_rows, hipStream_t s) {
  const int64_t mt = max_row_tiles(max_rows, a.offsets == nullptr ? 1 : a.n_exp, BM);
  const int64_t grid = (mt * a.n_tiles + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_fp8_kernel<MODE>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up_fp8(int n_exp, const int32_t* offsets, int64_t max_rows, int d, int d_ff,
                             const uint8_t* xp, const float* xp_scale, const uint8_t* w13,
                             const float* w13_scale, uint8_t* h, float* h_scale, hipStream_t s) {
  Fp8Args a{};
  a.A = xp;
  a.A_scale = xp_scale;
  a.lda = d;
  a.B = w13;
  a.B_scale = w13_scale;
  a.b_group_stride = (int64_t)2 * d_ff * d;
  a.bs_group_stride = (int64_t)(2 * d_ff / BKB) * (d / BKB);
  a.C = h;
  a.C_scale = h_scale;
  a.ldc = d_ff;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.K = d;
  a.n_tiles = d_ff / (BN / 2);
  a.d_ff = d_ff;
  return launch<MODE_SWIGLU>(a, max_rows, s);
}

hipError_t launch_ffn_down_fp8(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                               int d_ff, const uint8_t* h, const float* h_scale,
                               const uint8_t* w2, const float* w2_scale, uint16_t* yp,
                               hipStream_t s) {
  Fp8Args a{};
  a.A = h;
  a.A_scale = h_scale;
  a.lda = d_ff;
  a.B = w2;
  a.B_scale = w2_scale;
  a.b_group_stride = (int64_t)d * d_ff;
  a.bs_group_stride = (int64_t)(d / BKB) * (d_ff / BKB);
  a.C = yp;
  a.ldc = d;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.K = d_ff;
  a.n_tiles = d / BN;
  return launch<MODE_STORE>(a, max_rows, s);
}

}  // namespace moe
