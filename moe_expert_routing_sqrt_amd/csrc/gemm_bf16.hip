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
// operand spread over all banks.  Tiles reach LDS by direct-to-LDS DMA
// (global_load_lds_dwordx4, no register staging) through a three-stage ring:
// the loads for step k+2 are in flight while step k computes, with one
// barrier per step.
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Work-group barrier without the memory fence __syncthreads() carries: the
// fence would wait for every outstanding global load, including the LDS DMA of
// later pipeline stages.  Callers wait for exactly what they need first.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// N 16-byte LDS reads in one asm block that also waits for them: the LDS reads
// are then invisible to the compiler's memory-counter bookkeeping, which would
// otherwise treat every in-flight DMA of later stages as a possible writer of
// the stage being read and wait for all of them.  The wait inside the block
// means no output register is handed back while its load is still in flight.
template <int N>
__device__ __forceinline__ void lds_read(uint4 (&v)[N], const uint32_t (&a)[N]) {
  if constexpr (N == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(a[0]), "v"(a[1]) : "memory");
  } else if constexpr (N == 3) {
    asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]) : "v"(a[0]), "v"(a[1]), "v"(a[2]) : "memory");
  } else if constexpr (N == 4) {
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
                 "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
  } else if constexpr (N == 6) {
    asm volatile("ds_read_b128 %0, %6\n\tds_read_b128 %1, %7\n\tds_read_b128 %2, %8\n\t"
                 "ds_read_b128 %3, %9\n\tds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]) : "memory");
  } else {
    static_assert(N == 2, "unsupported fragment count");
  }
}

template <int BM, int BN, int WAVES_M, int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(const GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int RM = TM / 32, RN = TN / 32;
  constexpr int ADMA = BM / 32;  // 1 KB (8-row) LDS blocks per wave per K step
  constexpr int BDMA = BN / 32;
  constexpr int DMA_PER_STEP = ADMA + BDMA;
  constexpr int PLANES = MODE == MODE_GATE3 ? 3 : 1;
  static_assert(RM >= 1 && RN >= 1 && ADMA >= 1 && BDMA >= 1, "tile too small");
  static_assert(MODE != MODE_SWIGLU || RN % 2 == 0, "gate/up blocks come in pairs");

  // three pipeline stages, each its own LDS object so the compiler can tell the
  // DMA into one stage from the reads of another
  __shared__ uint4 sA0[BM * 8], sA1[BM * 8], sA2[BM * 8];
  __shared__ uint4 sB0[BN * 8], sB1[BN * 8], sB2[BN * 8];
  __shared__ int s_pre[kMaxExperts + 1];

  TileInfo ti;
  if (!map_tile(p.offsets, p.n_exp, p.rows_total, BM, p.n_tiles, s_pre, ti)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // Direct-to-LDS loads: one instruction moves 64 lanes x 16 B into 1 KB of
  // LDS at lane*16, i.e. 8 rows of 128 B.  The LDS layout is row-major with the
  // 16-byte chunks of a row XOR-swizzled by (row & 7); since the LDS slot of a
  // lane is fixed, the swizzle is applied to the global address instead: the
  // lane filling physical chunk pc of row r fetches logical chunk pc ^ (r & 7).
  const int lrow = lane >> 3;                  // row within the 8-row block
  const int lch = (lane & 7) ^ (lrow & 7);     // logical chunk this lane fetches
  const uint16_t* a_src[ADMA];
  const uint16_t* b_src[BDMA];
#pragma unroll
  for (int i = 0; i < ADMA; ++i) {
    const int r = (wave + 4 * i) * 8 + lrow;
    const int rc = r < ti.rows ? r : ti.rows - 1;  // padding rows: any valid row
    a_src[i] = p.A + (int64_t)(ti.row0 + rc) * p.lda + lch * 8;
  }
  const uint16_t* bg = p.B + (int64_t)ti.group * p.b_group_stride + lch * 8;
#pragma unroll
  for (int i = 0; i < BDMA; ++i) {
    const int r = (wave + 4 * i) * 8 + lrow;
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

  const int nkp = p.K / BK;
  const int nsteps = PLANES * nkp;

  auto issue = [&](int kt, uint4* sa, uint4* sb) {
    const int plane = PLANES == 1 ? 0 : kt / nkp;
    const int k0 = (kt - plane * nkp) * BK;
#pragma unroll
    for (int i = 0; i < ADMA; ++i)
      __builtin_amdgcn_global_load_lds(a_src[i] + k0, (lds_ptr_t)(sa + (wave + 4 * i) * 64), 16, 0, 0);
    const int64_t boff = (int64_t)plane * p.b_plane_stride + k0;
#pragma unroll
    for (int i = 0; i < BDMA; ++i)
      __builtin_amdgcn_global_load_lds(b_src[i] + boff, (lds_ptr_t)(sb + (wave + 4 * i) * 64), 16, 0, 0);
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragment addresses: row r of an operand tile is 128 bytes, chunk c of it
  // sits at (c ^ (r & 7)) * 16; rows used by a lane are lane%32 plus multiples
  // of 8, so the swizzle term depends on the lane only.
  constexpr int NF = RM + RN;
  uint32_t frag_off[NF];
#pragma unroll
  for (int i = 0; i < RM; ++i) frag_off[i] = (wm * TM + i * 32 + (lane & 31)) * 128;
#pragma unroll
  for (int j = 0; j < RN; ++j) frag_off[RM + j] = (wn * TN + j * 32 + (lane & 31)) * 128;
  const int sw = lane & 7, khalf = lane >> 5;

  auto compute = [&](const uint4* sa, const uint4* sb) {
    const uint32_t a_base = lds_addr(sa), b_base = lds_addr(sb);
    uint4 fr[2][NF];
    auto read = [&](uint4 (&f)[NF], int s) {
      const uint32_t co = ((2 * s + khalf) ^ sw) * 16;
      uint32_t ad[NF];
#pragma unroll
      for (int i = 0; i < RM; ++i) ad[i] = a_base + frag_off[i] + co;
#pragma unroll
      for (int j = 0; j < RN; ++j) ad[RM + j] = b_base + frag_off[RM + j] + co;
      lds_read<NF>(f, ad);
    };
    read(fr[0], 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[s & 1][i]),
                                                               as_bf16x8(fr[s & 1][RM + j]),
                                                               acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < BK / 16) read(fr[(s + 1) & 1], s + 1);
    }
  };

  // Step kt consumes stage kt % 3.  Before reading it, this wave waits for its
  // own DMA of step kt (the DMA of step kt+1 may stay in flight), then the
  // barrier makes every wave's part visible and guarantees that all waves are
  // done with the stage the next DMA (step kt+2) overwrites.
  auto step = [&](int kt, uint4* sa, uint4* sb, uint4* na, uint4* nb) {
    if (kt + 1 < nsteps) wait_vmcnt<DMA_PER_STEP>(); else wait_vmcnt<0>();
    barrier_only();
    if (kt + 2 < nsteps) issue(kt + 2, na, nb);
    compute(sa, sb);
  };

  issue(0, sA0, sB0);
  if (nsteps > 1) issue(1, sA1, sB1);
  for (int kt = 0; kt < nsteps; kt += 3) {
    step(kt, sA0, sB0, sA2, sB2);
    if (kt + 1 < nsteps) step(kt + 1, sA1, sB1, sA0, sB0);
    if (kt + 2 < nsteps) step(kt + 2, sA2, sB2, sA1, sB1);
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
#endif
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
