// Grouped bf16 products of the expert FFN backward on gfx950 matrix cores
// (deepmox ch.5: the backward splits into the gradient for the input and the
// gradient for the weights).  With the weights stored [out, in]:
//
//   DGRAD  C[r][n] = sum_k A[r][k] * W[k][n]   rows r of a group, W its weight
//          (d_h = d_y W2 with W2 [d, d_ff]; d_x = d_au W13 with W13 [2 d_ff, d])
//   WGRAD  C[m][n] = sum_r A[r][m] * B[r][n]   over the group's rows r
//          (dW2 = d_y^T h, dW13 = d_au^T x), fp32 output per group
//
// Same skeleton as the forward kernel (ffn_bf16.hip): 256 x 256 x 64 tiles,
// 8 wave64s (two per SIMD) of 64 x 128 accumulators, two 64 KB LDS stages
// filled by direct-to-LDS DMA, the step barrier before the last K slice,
// fragment reads and DMA interleaved one per MFMA slot.
//
// K-major operands (W in DGRAD; both in WGRAD) are staged as they lie in
// memory: 64 rows of K, each 512 bytes of contiguous M or N (one DMA
// instruction moves two rows).  The 16-byte chunks of row k are XORed with
// 4*(k & 3).  An MFMA operand wants 8 consecutive K for one column per lane;
// gfx950's transposing LDS read (ds_read_b64_tr_b16) delivers it: within each
// group of 16 lanes, source lane a points at 4 columns of row k0 + a/4, and
// lane i receives column i of those four rows.  Two such reads (k0 and k0+4)
// form the 8-value fragment; with the chunk XOR, the 32 lanes that read
// together touch 16 distinct chunks, so all 64 banks once.
//
// WGRAD's K is the group's row count: the last step is partial, and rows past
// the group (or past the buffer) are fetched from a zero row.
#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe {

__device__ uint4 g_zero_row[32];  // 512 zero bytes: K-major rows past a group's end

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NW = 8, WAVES_M = 4, WAVES_N = 2;
constexpr int kThreads = NW * 64;
constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // 64 x 128 per wave
constexpr int RM = TM / 32, RN = TN / 32;
constexpr int NS = BK / 16, NQ = RM * RN;
constexpr int KROW_BYTES = 512;          // K-major LDS row: 256 bf16
constexpr int DPW = 4;                   // DMA instructions per operand per wave per step
constexpr int NDMA = 2 * DPW;
constexpr int DHALF = NDMA / 2;

enum { MODE_DGRAD = 0, MODE_WGRAD = 1 };

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i16 lds_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
}

struct BwdArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  int64_t b_group_stride;  // DGRAD: elements between groups' weights
  void* C;
  int64_t ldc;
  int64_t c_group_stride;  // WGRAD: elements between groups' outputs
  const int* offsets;
  int n_exp;
  int64_t rows_total;
  int K;                   // DGRAD: reduction length
  int m_tiles, n_tiles;    // WGRAD: tiles per group (DGRAD: n_tiles only)
};

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void ffn_bwd_kernel(const BwdArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int STAGE = 2 * 32 * 1024 / 16;  // uint4: A 32 KB + B 32 KB
  constexpr int OUT_PITCH = BN * 2 + 16;      // DGRAD bf16 staging row
  constexpr int OUT_U4 = MODE == MODE_DGRAD ? BM * OUT_PITCH / 16 : 0;
  constexpr int RING = 2 * STAGE;
  __shared__ uint4 smem[RING > OUT_U4 ? RING : OUT_U4];
  __shared__ int s_pre[kMapInts];
  char* const base = reinterpret_cast<char*>(smem);
  char* const sA0 = base;
  char* const sB0 = base + 32 * 1024;
  char* const sA1 = base + 64 * 1024;
  char* const sB1 = base + 96 * 1024;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // ---- tile of this work-group
  int group, m_tile, n_tile, row0, rows;  // rows: DGRAD valid rows of the tile / WGRAD K
  if constexpr (MODE == MODE_DGRAD) {
    TileInfo ti;
    if (!map_tile(p.offsets, p.n_exp, p.rows_total, BM, p.n_tiles, s_pre, ti)) return;
    group = ti.group;
    m_tile = ti.m_tile;
    n_tile = ti.n_tile;
    row0 = ti.row0;
    rows = ti.rows;
  } else {
    const int per = p.m_tiles * p.n_tiles;
    const int total = p.n_exp * per;
    const int rr = (total + kXcds - 1) / kXcds * kXcds;
    const int w = blockIdx.x;
    if (w >= rr) return;
    const int L = (w % kXcds) * (rr / kXcds) + w / kXcds;  // XCD-contiguous slices
    if (L >= total) return;
    group = L / per;
    const int rem = L % per;
    m_tile = rem / p.n_tiles;
    n_tile = rem % p.n_tiles;
    row0 = p.offsets == nullptr ? 0 : p.offsets[group];
    rows = p.offsets == nullptr ? static_cast<int>(p.rows_total) : p.offsets[group + 1] - row0;
  }
  group = __builtin_amdgcn_readfirstlane(group);
  m_tile = __builtin_amdgcn_readfirstlane(m_tile);
  n_tile = __builtin_amdgcn_readfirstlane(n_tile);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  // DGRAD: a wave whose 64 rows lie past the valid rows skips its MFMAs
  const bool act = MODE == MODE_WGRAD || wm * TM < rows;
  const int nsteps = MODE == MODE_DGRAD ? p.K / BK : (rows + BK - 1) / BK;

  // ---- DMA sources.  Row-major operand (DGRAD A): blocks of 8 rows x 128 B,
  // chunk swizzle (r >> 1) & 7 applied to the global address.  K-major
  // operand: blocks of 2 rows x 512 B; lane l fills row 2b + l/32, physical
  // chunk l%32, logical chunk (l%32) ^ (4*(k&3)).
  const char* a_src[DPW];
  const char* b_src[DPW];
  int a_row[DPW];  // K-major A: K row of the lane within the step (WGRAD)
  const int kr_lane = lane >> 5;                       // row within a K-major block
  const int kr_chunk = (lane & 31) ^ (4 * ((2 * (wave & 1) + kr_lane) & 3));
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int blk = wave + NW * i;
    if constexpr (MODE == MODE_DGRAD) {
      const int r = blk * 8 + (lane >> 3);
      const int rc = r < rows ? r : rows - 1;
      const int lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
      a_src[i] = reinterpret_cast<const char*>(p.A + (int64_t)(row0 + rc) * p.lda + lch * 8);
      // W rows k = 2*blk + kr_lane of the step, columns of the n tile
      b_src[i] = reinterpret_cast<const char*>(p.B + (int64_t)group * p.b_group_stride +
                                               (int64_t)(2 * blk + kr_lane) * p.ldb + n_tile * BN +
                                               kr_chunk * 8);
      a_row[i] = 0;
    } else {
      a_row[i] = 2 * blk + kr_lane;
      a_src[i] = reinterpret_cast<const char*>(p.A + (int64_t)m_tile * BM + kr_chunk * 8);
      b_src[i] = reinterpret_cast<const char*>(p.B + (int64_t)n_tile * BN + kr_chunk * 8);
    }
  }
  const char* zrow = reinterpret_cast<const char*>(g_zero_row) + kr_chunk * 16;

  // DMA part q (< DPW: A, else B) of step kt into stage (sa, sb)
  auto dma_one = [&](int kt, char* sa, char* sb, int q) __attribute__((always_inline)) {
    const int i = q < DPW ? q : q - DPW;
    const int blk = wave + NW * i;
    if constexpr (MODE == MODE_DGRAD) {
      if (q < DPW) {
        if (kt < 2 || blk * 8 < rows)
          dma16(a_src[i] + (int64_t)kt * BK * 2, lds_addr(sa) + blk * 1024);
      } else {
        dma16(b_src[i] + (int64_t)kt * BK * p.ldb * 2, lds_addr(sb) + blk * 1024);
      }
    } else {
      const int k = kt * BK + a_row[i];  // row within the group
      const bool in = k < rows;
      if (q < DPW) {
        const char* g = in ? a_src[i] + (int64_t)(row0 + k) * p.lda * 2 : zrow;
        dma16(g, lds_addr(sa) + blk * 1024);
      } else {
        const char* g = in ? b_src[i] + (int64_t)(row0 + k) * p.ldb * 2 : zrow;
        dma16(g, lds_addr(sb) + blk * 1024);
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

  // ---- fragments.  Row-major tile: one 16-byte read at swz(row, chunk).
  // K-major tile: two transposing reads of 4 K each.
  const int tr_a = lane & 15;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (tr_a & 3);  // column within a 32-block
  const int tr_row = tr_a >> 2;                                // row within 4
  auto kmajor_frag = [&](const char* s, int col0, int s16) __attribute__((always_inline)) {
    const int n = col0 + tr_col;
    const int k0 = 16 * s16 + 8 * (lane >> 5) + tr_row;
    const int c = n >> 3;
    const int within = (n & 7) * 2;
    const v4i16 lo = lds_tr16(s + k0 * KROW_BYTES + ((c ^ (4 * (k0 & 3))) << 4) + within);
    const int k1 = k0 + 4;
    const v4i16 hi = lds_tr16(s + k1 * KROW_BYTES + ((c ^ (4 * (k1 & 3))) << 4) + within);
    const v4i16 v[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, v);
  };
  bf16x8 fa[2][RM], fb[2][RN];
  auto read_frag = [&](const char* sa, const char* sb, int buf, int s16, int f) __attribute__((always_inline)) {
    // order of first use: a0, b0 .. b(RN-1), a1 .. a(RM-1)
    const bool is_a = f == 0 || f > RN;
    const int idx = f == 0 ? 0 : (f <= RN ? f - 1 : f - RN);
    if (is_a) {
      if constexpr (MODE == MODE_DGRAD) {
        const uint4* s = reinterpret_cast<const uint4*>(sa);
        fa[buf][idx] = as_bf16x8(s[swz(wm * TM + idx * 32 + (lane & 31), 2 * s16 + (lane >> 5))]);
      } else {
        fa[buf][idx] = kmajor_frag(sa, wm * TM + idx * 32, s16);
      }
    } else {
      fb[buf][idx] = kmajor_frag(sb, wn * TN + idx * 32, s16);
    }
  };
  constexpr int NR = RM + RN;
  static_assert(NR <= NQ, "one read per MFMA slot");
  auto slice = [&](int s, const char* rsa, const char* rsb, int rs, int kd, char* da, char* db, int d0,
                   int d1) __attribute__((always_inline)) {
    const int buf = s & 1;
    const int nd = d1 - d0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = q / RN, j = q % RN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
      if (rsa != nullptr && q < NR) read_frag(rsa, rsb, buf ^ 1, rs, q);
      if (kd >= 0) {
#pragma unroll
        for (int t = 0; t < NDMA; ++t)
          if (t < nd && (t * NQ) / nd == q) dma_one(kd, da, db, d0 + t);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](int kt, char* sa, char* sb, char* na, char* nb) __attribute__((always_inline)) {
    const bool more = kt + 1 < nsteps;
    slice(0, sa, sb, 1, (kt >= 1 && more) ? kt + 1 : -1, na, nb, DHALF, NDMA);
#pragma unroll
    for (int s = 1; s + 1 < NS; ++s) slice(s, sa, sb, s + 1, -1, nullptr, nullptr, 0, 0);
    if (more) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      wait_vmcnt<0>();
      barrier_only();
    }
    slice(NS - 1, more ? na : nullptr, nb, 0, kt + 2 < nsteps ? kt + 2 : -1, sa, sb, 0, DHALF);
  };
  auto idle_step = [&](int kt, char* sa, char* sb, char* na, char* nb) __attribute__((always_inline)) {
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

  if (nsteps > 0) {
#pragma unroll
    for (int q = 0; q < NDMA; ++q) dma_one(0, sA0, sB0, q);
    if (nsteps > 1) {
#pragma unroll
      for (int q = 0; q < NDMA; ++q) dma_one(1, sA1, sB1, q);
      wait_vmcnt<NDMA>();
    } else {
      wait_vmcnt<0>();
    }
    barrier_only();
    if (act) {
#pragma unroll
      for (int f = 0; f < NR; ++f) read_frag(sA0, sB0, 0, 0, f);
      for (int kt = 0; kt < nsteps; kt += 2) {
        step(kt, sA0, sB0, sA1, sB1);
        if (kt + 1 < nsteps) step(kt + 1, sA1, sB1, sA0, sB0);
      }
    } else {
      for (int kt = 0; kt < nsteps; kt += 2) {
        idle_step(kt, sA0, sB0, sA1, sB1);
        if (kt + 1 < nsteps) idle_step(kt + 1, sA1, sB1, sA0, sB0);
      }
    }
  }

  // ---- epilogue.  Accumulator (i, j) register v holds row 8*(v/4) +
  // 4*(lane/32) + v%4 and column lane%32 of its 32x32 block.
  if constexpr (MODE == MODE_DGRAD) {
    barrier_only();
    if (act) {
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          uint16_t* row = reinterpret_cast<uint16_t*>(base + lr * OUT_PITCH);
#pragma unroll
          for (int j = 0; j < RN; ++j) row[wn * TN + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][v]);
        }
    }
    __syncthreads();
    constexpr int OCH = BN * 2 / 16;
    uint16_t* C = static_cast<uint16_t*>(p.C);
    for (int q = tid; q < rows * OCH; q += kThreads) {
      const int r = q / OCH, c = q % OCH;
      const uint4 v = *reinterpret_cast<const uint4*>(base + r * OUT_PITCH + c * 16);
      *reinterpret_cast<uint4*>(C + (int64_t)(row0 + r) * p.ldc + (int64_t)n_tile * BN + c * 8) = v;
    }
  } else {
    // fp32 weight gradient: for a fixed register, the 32 lanes of a half-wave
    // write 128 contiguous bytes of one row, so direct stores stay coalesced
    float* C = static_cast<float*>(p.C) + (int64_t)group * p.c_group_stride;
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m_tile * BM + wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
        for (int j = 0; j < RN; ++j)
          C[(int64_t)m * p.ldc + n_tile * BN + wn * TN + j * 32 + (lane & 31)] = acc[i][j][v];
      }
  }
#endif
}

template <int MODE>
hipError_t launch(const BwdArgs& a, int64_t tiles, hipStream_t s) {
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_bwd_kernel<MODE>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool ffn_bwd_bf16_supported(int d, int d_ff) { return d % 256 == 0 && d_ff % 256 == 0; }

// C [rows, N] bf16 = A [rows, K] x W_g [K, N]  (rows grouped by offsets)
hipError_t launch_ffn_dgrad_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int K, int N,
                                 const uint16_t* A, const uint16_t* W, uint16_t* C, hipStream_t s) {
  BwdArgs a{};
  a.A = A;
  a.lda = K;
  a.B = W;
  a.ldb = N;
  a.b_group_stride = (int64_t)K * N;
  a.C = C;
  a.ldc = N;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.K = K;
  a.n_tiles = N / BN;
  const int64_t mt = max_row_tiles(max_rows, offsets == nullptr ? 1 : n_exp, BM);
  return launch<MODE_DGRAD>(a, mt * a.n_tiles, s);
}

// C_g [M, N] fp32 = sum over the group's rows r of A[r][m] * B[r][n]
hipError_t launch_ffn_wgrad_bf16(int n_exp, const int32_t* offsets, int64_t rows_total, int M, int N,
                                 const uint16_t* A, const uint16_t* B, float* C, hipStream_t s) {
  BwdArgs a{};
  a.A = A;
  a.lda = M;
  a.B = B;
  a.ldb = N;
  a.C = C;
  a.ldc = N;
  a.c_group_stride = (int64_t)M * N;
  a.offsets = offsets;
  a.n_exp = offsets == nullptr ? 1 : n_exp;
  a.rows_total = rows_total;
  a.m_tiles = M / BM;
  a.n_tiles = N / BN;
  return launch<MODE_WGRAD>(a, (int64_t)a.n_exp * a.m_tiles * a.n_tiles, s);
}

}  // namespace moe
