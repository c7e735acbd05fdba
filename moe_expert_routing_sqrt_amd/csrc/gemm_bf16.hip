// Grouped bf16 GEMM on gfx950 matrix cores: the expert FFN products and the
// fp32-accurate gate product.
//
//   C[m][n] = sum_k A[m][k] * B[n][k]       (A: activations, B: weights [out, in])
//
// Work-group tile BM x BN x 64 (K), 256 threads = 4 wave64s laid out
// WAVES_M x WAVES_N; each wave owns a (BM/WAVES_M) x (BN/WAVES_N) block of
// 32x32 accumulators fed by v_mfma_f32_32x32x16_bf16 (fp32 accumulate).
// Operands stage through LDS in 128-byte rows (64 bf16 of K) whose 16-byte
// chunks are XOR-swizzled by row, so the 32 rows a wave reads for one MFMA
// operand spread over all banks.  Global loads for step k+1 are issued before
// the MFMAs of step k (register prefetch, one LDS buffer, two barriers/step).
//
// Epilogues
//   SWIGLU  (up projection of the SwiGLU expert, mastering-deepseek-v4 Exp08,
//           Implemented):  the BN weight rows of a tile are BN/2 gate rows
//           (W1) and the matching BN/2 up rows (W3); each wave holds the gate
//           and up accumulators of the same features, so
//           h = silu(gate) * up is formed in registers and stored as bf16.
//   STORE   (down projection): bf16 store.
//   GATE3   (router gate): B is three bf16 planes whose sum is the fp32 gate
//           weight exactly; the K loop runs over the three planes into one
//           fp32 accumulator, stored as fp32 logits.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int BK = 64;
constexpr int kThreads = 256;

enum { MODE_SWIGLU = 0, MODE_STORE = 1, MODE_GATE3 = 2 };

struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t b_group_stride;  // elements between consecutive groups' weights
  int64_t b_plane_stride;  // GATE3: elements between planes
  void* C;
  int64_t ldc;
  const int* offsets;      // [n_exp + 1] or nullptr (one group of rows_total rows)
  int n_exp;
  int64_t rows_total;
  int K;                   // reduction length (per plane)
  int n_tiles;
  int d_ff;                // SWIGLU: first up-projection row of w13
};

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ (r & 7)); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int BM, int BN, int WAVES_M, int MODE>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_kernel(const GemmArgs p) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int RM = TM / 32, RN = TN / 32;
  constexpr int AC = BM * 8 / kThreads;  // 16-byte chunks per thread per K step
  constexpr int BC = BN * 8 / kThreads;
  constexpr int PLANES = MODE == MODE_GATE3 ? 3 : 1;
  static_assert(RM >= 1 && RN >= 1 && AC >= 1 && BC >= 1, "tile too small");
  static_assert(MODE != MODE_SWIGLU || RN % 2 == 0, "gate/up blocks come in pairs");

  __shared__ uint4 sA[BM * 8];
  __shared__ uint4 sB[BN * 8];
  __shared__ int s_pre[kMaxExperts + 1];

  TileInfo ti;
  if (!map_tile(p.offsets, p.n_exp, p.rows_total, BM, p.n_tiles, s_pre, ti)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int r0 = tid >> 3;  // first tile row this thread loads
  const int ch = tid & 7;   // 16-byte chunk within the 128-byte K slice

  // global source rows of this thread's chunks (row r0 + 32*c)
  const uint16_t* a_src = p.A + (int64_t)ti.row0 * p.lda + ch * 8;
  const uint16_t* b_src[BC];
  const uint16_t* bg = p.B + (int64_t)ti.group * p.b_group_stride + ch * 8;
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    const int r = r0 + 32 * c;
    int grow;
    if constexpr (MODE == MODE_SWIGLU) {
      const int part = r / TN, within = r % TN;
      const int h0 = ti.n_tile * (BN / 2) + part * (TN / 2);
      grow = within < TN / 2 ? h0 + within : p.d_ff + h0 + (within - TN / 2);
    } else {
      grow = ti.n_tile * BN + r;
    }
    b_src[c] = bg + (int64_t)grow * p.K;
  }

  uint4 ra[AC], rb[BC];
  const int nkp = p.K / BK;
  const int nsteps = PLANES * nkp;

  auto gload = [&](int kt) {
    const int plane = PLANES == 1 ? 0 : kt / nkp;
    const int k0 = (kt - plane * nkp) * BK;
#pragma unroll
    for (int c = 0; c < AC; ++c) {
      const int r = r0 + 32 * c;
      if (r < ti.rows)
        ra[c] = *reinterpret_cast<const uint4*>(a_src + (int64_t)(32 * c) * p.lda + k0);
      else
        ra[c] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < BC; ++c)
      rb[c] = *reinterpret_cast<const uint4*>(b_src[c] + (int64_t)plane * p.b_plane_stride + k0);
  };
  auto sstore = [&]() {
#pragma unroll
    for (int c = 0; c < AC; ++c) sA[swz(r0 + 32 * c, ch)] = ra[c];
#pragma unroll
    for (int c = 0; c < BC; ++c) sB[swz(r0 + 32 * c, ch)] = rb[c];
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < nsteps; ++kt) {
    if (kt + 1 < nsteps) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int kc = 2 * s + (lane >> 5);
      bf16x8 af[RM], bfr[RN];
#pragma unroll
      for (int i = 0; i < RM; ++i) af[i] = as_bf16x8(sA[swz(wm * TM + i * 32 + (lane & 31), kc)]);
#pragma unroll
      for (int j = 0; j < RN; ++j) bfr[j] = as_bf16x8(sB[swz(wn * TN + j * 32 + (lane & 31), kc)]);
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nsteps) {
      sstore();
      __syncthreads();
    }
  }

  // epilogue: accumulator (i, j) register v holds row 8*(v/4) + 4*(lane/32) + v%4
  // and column lane%32 of its 32x32 block
#pragma unroll
  for (int i = 0; i < RM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int lr = wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (lr >= ti.rows) continue;
      const int64_t grow = ti.row0 + lr;
      if constexpr (MODE == MODE_SWIGLU) {
        uint16_t* out = static_cast<uint16_t*>(p.C) + grow * p.ldc;
#pragma unroll
        for (int jj = 0; jj < RN / 2; ++jj) {
          const float g = acc[i][jj][v];
          const float u = acc[i][jj + RN / 2][v];
          const float hval = g / (1.0f + __expf(-g)) * u;
          const int col = ti.n_tile * (BN / 2) + wn * (TN / 2) + jj * 32 + (lane & 31);
          out[col] = f32_to_bf16(hval);
        }
      } else if constexpr (MODE == MODE_STORE) {
        uint16_t* out = static_cast<uint16_t*>(p.C) + grow * p.ldc;
#pragma unroll
        for (int j = 0; j < RN; ++j)
          out[ti.n_tile * BN + wn * TN + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][v]);
      } else {
        float* out = static_cast<float*>(p.C) + grow * p.ldc;
#pragma unroll
        for (int j = 0; j < RN; ++j) out[ti.n_tile * BN + wn * TN + j * 32 + (lane & 31)] = acc[i][j][v];
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int MODE>
hipError_t launch(const GemmArgs& a, int64_t max_rows, hipStream_t s) {
  const int64_t mt = max_row_tiles(max_rows, a.offsets == nullptr ? 1 : a.n_exp, BM);
  const int64_t grid = (mt * a.n_tiles + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WAVES_M, MODE>), dim3((unsigned)grid), dim3(kThreads),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace

bool gate_gemm_bf16_supported(int d, int E) { return d % BK == 0 && E % 64 == 0; }

hipError_t launch_gate_gemm_bf16(const uint16_t* x, const uint16_t* w_prep, float* logits,
                                 int64_t T, int d, int E, hipStream_t s) {
  GemmArgs a{};
  a.A = x;
  a.lda = d;
  a.B = w_prep;
  a.b_group_stride = 0;
  a.b_plane_stride = (int64_t)E * d;
  a.C = logits;
  a.ldc = E;
  a.offsets = nullptr;
  a.n_exp = 1;
  a.rows_total = T;
  a.K = d;
  if (E % 128 == 0) {
    a.n_tiles = E / 128;
    return launch<128, 128, 2, MODE_GATE3>(a, T, s);
  }
  a.n_tiles = E / 64;
  return launch<64, 64, 2, MODE_GATE3>(a, T, s);
}

hipError_t launch_ffn_up_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                              int d_ff, const uint16_t* xp, const uint16_t* w13, uint16_t* h,
                              hipStream_t s) {
  GemmArgs a{};
  a.A = xp;
  a.lda = d;
  a.B = w13;
  a.b_group_stride = (int64_t)2 * d_ff * d;
  a.C = h;
  a.ldc = d_ff;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.K = d;
  a.n_tiles = d_ff / 128;
  a.d_ff = d_ff;
  return launch<128, 256, 2, MODE_SWIGLU>(a, max_rows, s);
}

hipError_t launch_ffn_down_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                                int d_ff, const uint16_t* h, const uint16_t* w2, uint16_t* yp,
                                hipStream_t s) {
  GemmArgs a{};
  a.A = h;
  a.lda = d_ff;
  a.B = w2;
  a.b_group_stride = (int64_t)d * d_ff;
  a.C = yp;
  a.ldc = d;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.K = d_ff;
  a.n_tiles = d / 256;
  return launch<128, 256, 2, MODE_STORE>(a, max_rows, s);
}

}  // namespace moe
