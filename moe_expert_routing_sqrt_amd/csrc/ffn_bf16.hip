// Grouped bf16 expert products on gfx950 matrix cores (the routed experts and
// the shared expert of the SwiGLU MoE layer):
//
//   up   (SWIGLU): h[r][f] = silu(x_r . W1[f]) * (x_r . W3[f])
//   down (STORE) : y[r][n] = h_r . W2[n]
//
// with rows r grouped by expert (offsets on the device) and weights in [out, in]
// layout, so K is contiguous for both operands.
//
// Work-group tile 256 rows x 256 weight rows x 64 (K), 512 threads = 8 wave64s
// laid out 4 x 2, each owning 2 x 4 blocks of 32x32 fp32 accumulators (64 rows x
// 128 weight rows) fed by v_mfma_f32_32x32x16_bf16; two waves share each SIMD,
// so one wave's memory stalls are covered by the other's MFMAs.  256 x 256 tiles halve the operand
// bytes per FLOP of a 128 x 128 tile; a step moves 64 KB into LDS for 8.4 MFLOP.
//
// Pipeline (two LDS stages of 64 KB, 128-byte rows, XOR-swizzled chunks):
//   * a K step is four slices of 16; in the shadow of each MFMA a wave issues
//     at most one fragment read for the next slice and at most one
//     direct-to-LDS DMA (global_load_lds_dwordx4), so neither piles up behind
//     a batch;
//   * the barrier of step k sits before its last slice: by then every wave
//     holds all of step k's fragments, so stage k can be refilled, and the
//     last slice's MFMAs cover both the reads of step k+1's first slice and
//     the first half of step k+2's DMA; the second half goes out in the first
//     slice of step k+1.
//
// Ragged groups: a tile covers up to 256 rows of one expert.  Wave row wm owns
// the 32-row blocks at rows 32*wm and 128 + 32*wm, so the two waves sharing a
// SIMD (wm and wm + 2) hold blocks in every 64-row band of the tile.  A block
// past the tile's valid rows is skipped (no MFMAs, no fragment reads), and a
// wave with no valid block skips its activation DMA too (it still moves its
// share of the weight tile and joins every barrier).  The busiest SIMD then
// runs ceil(rows / 64) of its four blocks, so a ragged tile costs its rows
// rounded up to 64.
//
// SwiGLU is fused (mastering-deepseek-v4 Exp08, "Implemented"): a tile's 256
// weight rows are 128 gate rows (W1) and the matching 128 up rows (W3), and
// each wave holds the gate and up accumulators of the same 64 features.
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int BM = 256;          // activation rows per tile
constexpr int BN = 256;          // weight rows per tile
constexpr int BK = 64;           // K per step (128-byte LDS rows)
constexpr int NW = 8;            // waves
constexpr int WAVES_M = 4;
constexpr int WAVES_N = NW / WAVES_M;
constexpr int kThreads = NW * 64;
constexpr int TM = BM / WAVES_M;  // 64
constexpr int TN = BN / WAVES_N;  // 128
constexpr int RM = TM / 32, RN = TN / 32;
constexpr int HB = BM / RM;       // row distance between a wave's blocks (128)
constexpr int ADMA = BM / (8 * NW);  // 1 KB DMA blocks of 8 rows, per wave per step
constexpr int BDMA = BN / (8 * NW);
constexpr int NDMA = ADMA + BDMA;
constexpr int NS = BK / 16;       // MFMA K slices per step
constexpr int NQ = RM * RN;       // MFMAs per slice
constexpr int NR = RM + RN;       // fragment reads per slice
constexpr int DHALF = NDMA / 2;   // DMA issued in the last slice of the step before
static_assert(NR <= NQ, "one fragment read per MFMA slot");
static_assert(RM == 2, "a wave's blocks sit in the two halves of the tile");
static_assert(NW % 2 == 0, "a wave's DMA blocks share the swizzle parity");

enum { MODE_SWIGLU = 0, MODE_STORE = 1, MODE_SWIGLU_SAVE = 2 };  // SAVE: also [a | u]

struct FfnArgs {
  const uint16_t* A;       // packed rows [rows, K]
  int64_t lda;
  const uint16_t* B;       // weights of group 0 [*, K]
  int64_t b_group_stride;  // elements between consecutive groups' weights
  uint16_t* C;             // output [rows, ldc]
  int64_t ldc;
  const int* offsets;      // [n_exp + 1] on the device, or nullptr (one group)
  int n_exp;
  int64_t rows_total;
  int K;
  int n_tiles;             // column tiles per group
  int d_ff;                // SWIGLU: first up-projection row of w13
  uint16_t* C2;            // SWIGLU_SAVE: [a | u] output [rows, 2*d_ff]
};

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void ffn_gemm_kernel(const FfnArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr bool SWI = MODE != MODE_STORE;
  constexpr int OUT_COLS = SWI ? BN / 2 : BN;
  constexpr int ROW_BYTES = OUT_COLS * 2;
  constexpr int PITCH = ROW_BYTES + 16;  // output staging row pitch
  constexpr int AU_PITCH = BN * 2 + 16;  // SWIGLU_SAVE: staging of [a | u]
  constexpr int STAGE = (BM + BN) * 8;   // uint4 per stage
  constexpr int RING = 2 * STAGE;
  constexpr int OUT_U4 = BM * (MODE == MODE_SWIGLU_SAVE ? AU_PITCH : PITCH) / 16;
  __shared__ uint4 smem[RING > OUT_U4 ? RING : OUT_U4];
  __shared__ int s_pre[kMaxExperts + 1];
  uint4* const sA0 = smem;
  uint4* const sB0 = smem + BM * 8;
  uint4* const sA1 = smem + STAGE;
  uint4* const sB1 = smem + STAGE + BM * 8;

  TileInfo ti;
  if (!map_tile(p.offsets, p.n_exp, p.rows_total, BM, p.n_tiles, s_pre, ti)) return;
  ti.group = __builtin_amdgcn_readfirstlane(ti.group);
  ti.n_tile = __builtin_amdgcn_readfirstlane(ti.n_tile);
  ti.row0 = __builtin_amdgcn_readfirstlane(ti.row0);
  ti.rows = __builtin_amdgcn_readfirstlane(ti.rows);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  // valid 32-row blocks of this wave: block i covers rows i*HB + 32*wm + [0, 32)
  const int nb = __builtin_amdgcn_readfirstlane((ti.rows > 32 * wm) + (ti.rows > HB + 32 * wm));

  // Direct-to-LDS loads: one instruction moves 64 lanes x 16 B into 1 KB of
  // LDS at lane*16, i.e. 8 rows of 128 B.  The LDS slot of a lane is fixed, so
  // the swizzle is applied to the global address: the lane filling physical
  // chunk pc of row r fetches logical chunk pc ^ ((r >> 1) & 7).  This wave
  // fills blocks j = wave + 8i (rows 8j..8j+7), for which (r >> 1) & 7 =
  // 4*(wave & 1) + (lane >> 4).
  const int lrow = lane >> 3;
  const int lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  const uint16_t* a_src[ADMA];
  const uint16_t* b_src[BDMA];
#pragma unroll
  for (int i = 0; i < ADMA; ++i) {
    const int r = (wave + NW * i) * 8 + lrow;
    const int rc = r < ti.rows ? r : ti.rows - 1;  // padding rows read a valid row
    a_src[i] = p.A + (int64_t)(ti.row0 + rc) * p.lda + lch * 8;
  }
  const uint16_t* bg = p.B + (int64_t)ti.group * p.b_group_stride + lch * 8;
#pragma unroll
  for (int i = 0; i < BDMA; ++i) {
    const int r = (wave + NW * i) * 8 + lrow;
    int grow;
    if constexpr (SWI) {
      // tile rows [part*TN, part*TN + TN/2) are gate rows, the next TN/2 the
      // matching up rows, for features n_tile*BN/2 + part*TN/2 + [0, TN/2)
      const int part = r / TN, within = r % TN;
      const int h0 = ti.n_tile * (BN / 2) + part * (TN / 2);
      grow = within < TN / 2 ? h0 + within : p.d_ff + h0 + (within - TN / 2);
    } else {
      grow = ti.n_tile * BN + r;
    }
    b_src[i] = bg + (int64_t)grow * p.K;
  }
  const int nsteps = p.K / BK;

  // DMA part q of step kt into stage (sa, sb).  Activation blocks wholly past
  // the valid rows are skipped after the first two steps (the in-loop waits are
  // for zero outstanding loads, so per-wave counts may differ; the prologue
  // wait counts every part).
  auto dma_one = [&](int kt, uint4* sa, uint4* sb, int q) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    if (q < ADMA) {
      if (kt < 2 || (wave + NW * q) * 8 < ti.rows)
        dma16(a_src[q] + k0, lds_addr(sa) + (wave + NW * q) * 1024);
    } else {
      dma16(b_src[q - ADMA] + k0, lds_addr(sb) + (wave + NW * (q - ADMA)) * 1024);
    }
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragments live in two register buffers, selected by slice parity.
  // Fragment f of a slice, in order of first use: a0, b0..b(RN-1), a1..a(RM-1).
  bf16x8 fa[2][RM], fb[2][RN];
  auto read_frag = [&](const uint4* sa, const uint4* sb, int buf, int s, int f)
                       __attribute__((always_inline)) {
    const int kc = 2 * s + (lane >> 5);
    if (f == 0) {
      fa[buf][0] = as_bf16x8(sa[swz(32 * wm + (lane & 31), kc)]);
    } else if (f <= RN) {
      fb[buf][f - 1] = as_bf16x8(sb[swz(wn * TN + (f - 1) * 32 + (lane & 31), kc)]);
    } else {
      fa[buf][f - RN] = as_bf16x8(sa[swz((f - RN) * HB + 32 * wm + (lane & 31), kc)]);
    }
  };
  // MFMAs of slice s over the first NB row blocks; reads of slice rs of
  // (rsa, rsb) into the other buffer (rsa == nullptr: none); DMA parts
  // [d0, d1) of step kd (kd < 0: none).  With one block there are five reads
  // for four MFMA slots: the first slot takes two.
  auto slice = [&](auto nbc, int s, const uint4* rsa, const uint4* rsb, int rs, int kd, uint4* da,
                   uint4* db, int d0, int d1) __attribute__((always_inline)) {
    constexpr int NB = decltype(nbc)::value;
    constexpr int NQB = NB * RN, NRB = NB + RN;
    constexpr int XR = NRB > NQB ? NRB - NQB : 0;  // reads doubled up in slot 0
    const int buf = s & 1;
    const int nd = d1 - d0;
#pragma unroll
    for (int q = 0; q < NQB; ++q) {
      const int i = q / RN, j = q % RN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
      if (rsa != nullptr) {
#pragma unroll
        for (int f = 0; f < NRB; ++f)
          if ((f < XR ? 0 : f - XR) == q) read_frag(rsa, rsb, buf ^ 1, rs, f);
      }
      if (kd >= 0) {
#pragma unroll
        for (int t = 0; t < NDMA; ++t)
          if (t < nd && (t * NQB) / nd == q) dma_one(kd, da, db, d0 + t);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep this interleaving
    }
  };
  // Step kt computes from stage (sa, sb); (na, nb) holds step kt+1.
  auto step = [&](auto nbc, int kt, uint4* sa, uint4* sb, uint4* na, uint4* nb)
                  __attribute__((always_inline)) {
    const bool more = kt + 1 < nsteps;
    // second half of step kt+1's DMA (the prologue issued all of step 1's)
    slice(nbc, 0, sa, sb, 1, (kt >= 1 && more) ? kt + 1 : -1, na, nb, DHALF, NDMA);
#pragma unroll
    for (int s = 1; s + 1 < NS; ++s) slice(nbc, s, sa, sb, s + 1, -1, nullptr, nullptr, 0, 0);
    if (more) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): step kt's fragments are in registers
      wait_vmcnt<0>();                     // this wave's DMA of step kt+1 has landed
      barrier_only();                      // everyone's has; stage (sa, sb) is free
    }
    // last slice: reads of step kt+1's first slice, first half of step kt+2's DMA
    slice(nbc, NS - 1, more ? na : nullptr, nb, 0, kt + 2 < nsteps ? kt + 2 : -1, sa, sb, 0, DHALF);
  };
  // A wave without valid rows keeps the same DMA parts and barriers.
  auto idle_step = [&](int kt, uint4* sa, uint4* sb, uint4* na, uint4* nb) __attribute__((always_inline)) {
    const bool more = kt + 1 < nsteps;
    if (kt >= 1 && more) {
#pragma unroll
      for (int q = DHALF; q < NDMA; ++q) dma_one(kt + 1, na, nb, q);
    }
    if (more) {
      wait_vmcnt<0>();
      barrier_only();
    }
    if (kt + 2 < nsteps) {
#pragma unroll
      for (int q = 0; q < DHALF; ++q) dma_one(kt + 2, sa, sb, q);
    }
  };

#pragma unroll
  for (int q = 0; q < NDMA; ++q) dma_one(0, sA0, sB0, q);
  if (nsteps > 1) {
#pragma unroll
    for (int q = 0; q < NDMA; ++q) dma_one(1, sA1, sB1, q);
    wait_vmcnt<NDMA>();  // step 0 landed; step 1 may be in flight
  } else {
    wait_vmcnt<0>();
  }
  barrier_only();
  if (nb == RM) {
    using NBC = std::integral_constant<int, RM>;
#pragma unroll
    for (int f = 0; f < NR; ++f) read_frag(sA0, sB0, 0, 0, f);
    for (int kt = 0; kt < nsteps; kt += 2) {
      step(NBC{}, kt, sA0, sB0, sA1, sB1);
      if (kt + 1 < nsteps) step(NBC{}, kt + 1, sA1, sB1, sA0, sB0);
    }
  } else if (nb == 1) {
    using NBC = std::integral_constant<int, 1>;
#pragma unroll
    for (int f = 0; f <= RN; ++f) read_frag(sA0, sB0, 0, 0, f);
    for (int kt = 0; kt < nsteps; kt += 2) {
      step(NBC{}, kt, sA0, sB0, sA1, sB1);
      if (kt + 1 < nsteps) step(NBC{}, kt + 1, sA1, sB1, sA0, sB0);
    }
  } else {
    for (int kt = 0; kt < nsteps; kt += 2) {
      idle_step(kt, sA0, sB0, sA1, sB1);
      if (kt + 1 < nsteps) idle_step(kt + 1, sA1, sB1, sA0, sB0);
    }
  }

  // Epilogue.  Accumulator (i, j) register v holds row 8*(v/4) + 4*(lane/32) +
  // v%4 and column lane%32 of its 32x32 block, so each lane owns one column.
  // The tile is staged in LDS (row pitch padded by 16 bytes) and leaves as
  // 16-byte row chunks.  All DMA has landed (the last in-loop wait was for
  // zero outstanding); the barrier ends every wave's reads of the last stage.
  // Registers v and v+1 (v even) are consecutive rows of one column: each pair
  // is rounded by one packed conversion and leaves as two 2-byte LDS writes.
  // silu(g) = g / (1 + e^-g) takes the hardware reciprocal (1 ulp, far below
  // the bf16 rounding of h).
  char* const stage = reinterpret_cast<char*>(smem);
  auto put2 = [&](int lr, int col, int pitch, uint32_t pk) __attribute__((always_inline)) {
    uint16_t* r0 = reinterpret_cast<uint16_t*>(stage + lr * pitch);
    uint16_t* r1 = reinterpret_cast<uint16_t*>(stage + (lr + 1) * pitch);
    r0[col] = static_cast<uint16_t>(pk);
    r1[col] = static_cast<uint16_t>(pk >> 16);
  };
  auto silu_mul = [](float g, float u) __attribute__((always_inline)) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
  };
  barrier_only();
  if (nb > 0) {
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int lr = i * HB + 32 * wm + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if constexpr (SWI) {
#pragma unroll
          for (int jj = 0; jj < RN / 2; ++jj) {
            const f32x16& g = acc[i][jj];
            const f32x16& u = acc[i][jj + RN / 2];
            put2(lr, wn * (TN / 2) + jj * 32 + (lane & 31), PITCH,
                 pack_bf16x2(silu_mul(g[v], u[v]), silu_mul(g[v + 1], u[v + 1])));
          }
        } else {
#pragma unroll
          for (int j = 0; j < RN; ++j)
            put2(lr, wn * TN + j * 32 + (lane & 31), PITCH, pack_bf16x2(acc[i][j][v], acc[i][j][v + 1]));
        }
      }
    }
  }
  __syncthreads();
  constexpr int OCH = ROW_BYTES / 16;
  const int64_t col0 = (int64_t)ti.n_tile * OUT_COLS;
  for (int q = tid; q < ti.rows * OCH; q += kThreads) {
    const int r = q / OCH, c = q % OCH;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + r * PITCH + c * 16);
    char* dst = reinterpret_cast<char*>(p.C + (ti.row0 + r) * p.ldc + col0) + c * 16;
    *reinterpret_cast<uint4*>(dst) = v;
  }
  if constexpr (MODE == MODE_SWIGLU_SAVE) {
    // the pre-activations for the backward: a (gate) at columns
    // [n_tile*BN/2, +BN/2) and u (up) at d_ff + the same, bf16
    __syncthreads();  // every read of the h staging is done
    if (nb > 0) {
#pragma unroll
      for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int lr = i * HB + 32 * wm + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
          for (int jj = 0; jj < RN / 2; ++jj) {
            const int c = wn * (TN / 2) + jj * 32 + (lane & 31);
            put2(lr, c, AU_PITCH, pack_bf16x2(acc[i][jj][v], acc[i][jj][v + 1]));
            put2(lr, BN / 2 + c, AU_PITCH, pack_bf16x2(acc[i][jj + RN / 2][v], acc[i][jj + RN / 2][v + 1]));
          }
        }
      }
    }
    __syncthreads();
    constexpr int HCH = BN / 2 * 2 / 16;  // 16-byte chunks per half row
    const int64_t ld2 = 2 * (int64_t)p.d_ff;
    for (int q = tid; q < ti.rows * 2 * HCH; q += kThreads) {
      const int r = q / (2 * HCH), c = q % (2 * HCH);
      const int half = c / HCH, cc = c % HCH;
      const uint4 v = *reinterpret_cast<const uint4*>(stage + r * AU_PITCH + c * 16);
      uint16_t* dst = p.C2 + (ti.row0 + r) * ld2 + half * p.d_ff + col0 + cc * 8;
      *reinterpret_cast<uint4*>(dst) = v;
    }
  }
#endif
}

template <int MODE>
hipError_t launch(const FfnArgs& a, int64_t max_rows, hipStream_t s) {
  const int64_t mt = max_row_tiles(max_rows, a.offsets == nullptr ? 1 : a.n_exp, BM);
  const int64_t grid = (mt * a.n_tiles + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_gemm_kernel<MODE>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                              int d_ff, const uint16_t* xp, const uint16_t* w13, uint16_t* h,
                              hipStream_t s, uint16_t* au) {
  FfnArgs a{};
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
  a.n_tiles = d_ff / (BN / 2);
  a.d_ff = d_ff;
  a.C2 = au;
  if (au != nullptr) return launch<MODE_SWIGLU_SAVE>(a, max_rows, s);
  return launch<MODE_SWIGLU>(a, max_rows, s);
}

hipError_t launch_ffn_store_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int K, int N,
                                 const uint16_t* A, const uint16_t* B, uint16_t* C, hipStream_t s) {
  FfnArgs a{};
  a.A = A;
  a.lda = K;
  a.B = B;
  a.b_group_stride = (int64_t)N * K;
  a.C = C;
  a.ldc = N;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.K = K;
  a.n_tiles = N / BN;
  return launch<MODE_STORE>(a, max_rows, s);
}

hipError_t launch_ffn_down_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                                int d_ff, const uint16_t* h, const uint16_t* w2, uint16_t* yp,
                                hipStream_t s) {
  return launch_ffn_store_bf16(n_exp, offsets, max_rows, d_ff, d, h, w2, yp, s);
}

}  // namespace moe
