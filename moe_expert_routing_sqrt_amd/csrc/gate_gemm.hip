// Router gate product on gfx950 matrix cores, fp32-accurate:
//
//   logits[t][e] = sum_k x[t][k] * W_g[k][e]
//
// x is bf16 (exact); the fp32 gate weight is split into three bf16 planes whose
// sum is exact (prepared by every route call), and the K loop runs over the
// three planes into one fp32 accumulator, plane fastest: the three steps that
// share a 64-column slice of x follow each other, so the slice comes from HBM
// once and from L2 for the other two planes (plane-major order streamed x
// three times: 11% slower at V3).
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
// Split over the reduction: the 3 * d / 64 plane-and-column steps divide into
// S equal ranges, one per grid row (blockIdx.y), each writing its own fp32
// partial product [T, E] (the route selection sums them in order), so that a
// product with few output tiles still fills the chip.
//
#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int PLANES = 3;

struct GateArgs {
  const uint16_t* A;       // x [T, d] bf16
  int64_t lda;
  const uint16_t* B;       // three planes [E, d] bf16
  int64_t b_plane_stride;  // elements between planes
  float* C;                // logits [T, E]
  int64_t ldc;
  int64_t rows_total;      // T
  int K;                   // d
  int n_tiles;             // E / BN
  int ksteps;              // steps of each split (grid row y takes [y * ksteps, (y + 1) * ksteps))
  int64_t c_split_stride;  // elements between the splits' partial products
};

template <int BM, int BN, int WAVES_M>
__global__ __launch_bounds__(kThreads, 1) void gate_gemm_kernel(const GateArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int RM = TM / 32, RN = TN / 32;
  constexpr int ADMA = BM / 32;  // 1 KB (8-row) LDS blocks per wave per K step
  constexpr int BDMA = BN / 32;
  constexpr int DMA_PER_STEP = ADMA + BDMA;
  static_assert(RM >= 1 && RN >= 1 && ADMA >= 1 && BDMA >= 1, "tile too small");

  // three pipeline stages of (A tile, B tile); after the K loop the same LDS
  // stages the output tile so it leaves in 16-byte row chunks
  constexpr int STAGE = (BM + BN) * 8;  // uint4 per stage
  __shared__ uint4 smem[3 * STAGE];
  __shared__ int s_pre[kMapInts];
  uint4* const sA0 = smem;
  uint4* const sB0 = smem + BM * 8;
  uint4* const sA1 = smem + STAGE;
  uint4* const sB1 = smem + STAGE + BM * 8;
  uint4* const sA2 = smem + 2 * STAGE;
  uint4* const sB2 = smem + 2 * STAGE + BM * 8;

  TileInfo ti;
  if (!map_tile(nullptr, 1, p.rows_total, BM, p.n_tiles, s_pre, ti)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // Direct-to-LDS loads: one instruction moves 64 lanes x 16 B into 1 KB of
  // LDS at lane*16, i.e. 8 rows of 128 B.  The LDS slot of a lane is fixed, so
  // the swizzle is applied to the global address instead: the lane filling
  // physical chunk pc of row r fetches logical chunk pc ^ ((r >> 1) & 7).
  // Block j covers rows 8j..8j+7 and this wave only fills blocks j = wave + 4i,
  // so (r >> 1) & 7 = 4*(wave & 1) + (lane >> 4) for every row it fills.
  const int lrow = lane >> 3;  // row within the 8-row block
  const int lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);  // logical chunk fetched
  const uint16_t* a_src[ADMA];
  const uint16_t* b_src[BDMA];
#pragma unroll
  for (int i = 0; i < ADMA; ++i) {
    const int r = (wave + 4 * i) * 8 + lrow;
    const int rc = r < ti.rows ? r : ti.rows - 1;  // padding rows: any valid row
    a_src[i] = p.A + (int64_t)(ti.row0 + rc) * p.lda + lch * 8;
  }
#pragma unroll
  for (int i = 0; i < BDMA; ++i) {
    const int r = (wave + 4 * i) * 8 + lrow;
    b_src[i] = p.B + (int64_t)(ti.n_tile * BN + r) * p.K + lch * 8;
  }

  const int split = blockIdx.y;
  const int kbase = split * p.ksteps;  // this split's first plane-and-column step
  const int nsteps = p.ksteps;
  float* const C = p.C + (int64_t)split * p.c_split_stride;

  // DMA of one K step, split into parts so they can be spread between MFMA
  // groups (issuing all at once stalls the wave on address back-pressure).
  constexpr int NDMA = ADMA + BDMA;
  auto issue_part = [&](int kt, uint4* sa, uint4* sb, int q0, int q1) {
    const int kg = kbase + kt;
    const int kin = kg / PLANES;
    const int plane = kg - kin * PLANES;
    const int k0 = kin * BK;
    const uint32_t la = lds_addr(sa), lb = lds_addr(sb);
    const int64_t boff = (int64_t)plane * p.b_plane_stride + k0;
#pragma unroll
    for (int q = 0; q < NDMA; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < ADMA) dma16(a_src[q] + k0, la + (wave + 4 * q) * 1024);
      else dma16(b_src[q - ADMA] + boff, lb + (wave + 4 * (q - ADMA)) * 1024);
    }
  };
  auto issue = [&](int kt, uint4* sa, uint4* sb) { issue_part(kt, sa, sb, 0, NDMA); };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragment reads: row r of an operand tile is 128 bytes and chunk c of it
  // sits at (c ^ (r & 7)) * 16.  Slice s+1 is read while the MFMAs of slice s
  // run.
  auto compute = [&](const uint4* sa, const uint4* sb, int kn, uint4* na, uint4* nb) {
    bf16x8 fa[2][RM], fb[2][RN];
    auto read = [&](int buf, int s) {
      const int kc = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < RM; ++i) fa[buf][i] = as_bf16x8(sa[swz(wm * TM + i * 32 + (lane & 31), kc)]);
#pragma unroll
      for (int j = 0; j < RN; ++j) fb[buf][j] = as_bf16x8(sb[swz(wn * TN + j * 32 + (lane & 31), kc)]);
    };
    constexpr int NS = BK / 16;
    read(0, 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + 1 < NS) read((s + 1) & 1, s + 1);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads of slice s+1 ahead of these MFMAs
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][i], fb[s & 1][j], acc[i][j], 0, 0, 0);
      // a share of the next stage's DMA goes out while these MFMAs run
      if (kn >= 0 && s < NS - 1) {
        constexpr int per = (NDMA + NS - 2) / (NS - 1);
        issue_part(kn, na, nb, s * per, (s + 1) * per);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step kt consumes stage kt % 3.  Before reading it, this wave waits for its
  // own DMA of step kt (the DMA of step kt+1 may stay in flight), then the
  // barrier makes every wave's part visible and guarantees that all waves are
  // done with the stage the next DMA (step kt+2) overwrites.
  auto step = [&](int kt, uint4* sa, uint4* sb, uint4* na, uint4* nb) {
    if (kt + 1 < nsteps) wait_vmcnt<DMA_PER_STEP>(); else wait_vmcnt<0>();
    barrier_only();
    compute(sa, sb, kt + 2 < nsteps ? kt + 2 : -1, na, nb);
  };

  issue(0, sA0, sB0);
  if (nsteps > 1) issue(1, sA1, sB1);
  for (int kt = 0; kt < nsteps; kt += 3) {
    step(kt, sA0, sB0, sA2, sB2);
    if (kt + 1 < nsteps) step(kt + 1, sA1, sB1, sA0, sB0);
    if (kt + 2 < nsteps) step(kt + 2, sA2, sB2, sA1, sB1);
  }

  // Epilogue.  Accumulator (i, j) register v holds row 8*(v/4) + 4*(lane/32) +
  // v%4 and column lane%32 of its 32x32 block: each lane owns one column, so
  // direct stores would be 2-byte scatters.  The tile is written to LDS first
  // (row pitch padded by 16 bytes), then streamed out as 16-byte row chunks.
  constexpr int ROW_BYTES = BN * 4;
  constexpr int PITCH = ROW_BYTES + 16;
  static_assert(BM * PITCH <= 3 * STAGE * 16, "output tile must fit the LDS ring");
  char* const stage = reinterpret_cast<char*>(smem);
  barrier_only();  // every wave is done with the last stage (its DMA was waited for)
#pragma unroll
  for (int i = 0; i < RM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int lr = wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      float* row = reinterpret_cast<float*>(stage + lr * PITCH);
#pragma unroll
      for (int j = 0; j < RN; ++j) row[wn * TN + j * 32 + (lane & 31)] = acc[i][j][v];
    }
  }
  __syncthreads();
  constexpr int CPR = ROW_BYTES / 16;  // 16-byte chunks per row
  const int64_t col0 = (int64_t)ti.n_tile * BN;
  for (int q = tid; q < ti.rows * CPR; q += kThreads) {
    const int r = q / CPR, c = q % CPR;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + r * PITCH + c * 16);
    char* dst = reinterpret_cast<char*>(C + (ti.row0 + r) * p.ldc + col0) + c * 16;
    *reinterpret_cast<uint4*>(dst) = v;
  }
#endif
}

template <int BM, int BN, int WAVES_M>
hipError_t launch(const GateArgs& a, int S, hipStream_t s) {
  const int64_t mt = (a.rows_total + BM - 1) / BM;
  const int64_t grid = (mt * a.n_tiles + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gate_gemm_kernel<BM, BN, WAVES_M>), dim3((unsigned)grid, (unsigned)S), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

// the tile of a product with E output columns: 128 x 128 when E % 128 == 0,
// else 64 x 64
int tile_of(int E) { return E % 128 == 0 ? 128 : 64; }

}  // namespace

bool gate_gemm_bf16_supported(int d, int E) { return d % BK == 0 && E % 64 == 0; }

// The most splits (up to kMaxGateSplits) that keep the launch within 256
// work-groups (one per CU of an MI355X; a fixed figure, so that the workspace
// size does not depend on the device), each with a whole number of at least
// two steps.
int gate_gemm_split_count(int64_t T, int d, int E) {
  if (!gate_gemm_bf16_supported(d, E)) return 0;
  constexpr int64_t kTargetTiles = 256;
  const int tile = tile_of(E);
  const int steps = PLANES * (d / BK);
  const int64_t tiles1 = (T + tile - 1) / tile * (E / tile);
  int best = 1;
  for (int S = 2; S <= kMaxGateSplits; ++S) {
    if (tiles1 * S > kTargetTiles) break;
    if (steps % S == 0 && steps / S >= 2) best = S;
  }
  return best;
}

hipError_t launch_gate_gemm_bf16(const uint16_t* x, const uint16_t* w_prep, float* logits,
                                 int64_t T, int d, int E, int S, hipStream_t s) {
  const int steps = PLANES * (d / BK);
  if (S < 1 || steps % S != 0) return hipErrorInvalidValue;
  GateArgs a{};
  a.ksteps = steps / S;
  a.c_split_stride = T * E;
  a.A = x;
  a.lda = d;
  a.B = w_prep;
  a.b_plane_stride = (int64_t)E * d;
  a.C = logits;
  a.ldc = E;
  a.rows_total = T;
  a.K = d;
  if (tile_of(E) == 128) {
    a.n_tiles = E / 128;
    return launch<128, 128, 2>(a, S, s);
  }
  a.n_tiles = E / 64;
  return launch<64, 64, 2>(a, S, s);
}

}  // namespace moe
