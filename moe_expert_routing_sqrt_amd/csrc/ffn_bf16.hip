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
// so one wave's memory stalls are covered by the other's MFMAs.  256 x 256
// tiles halve the operand bytes per FLOP of a 128 x 128 tile; a step moves
// 64 KB into LDS for 8.4 MFLOP.
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
// Persistent work-groups: one per CU.  Logical tiles (the grouped tile map of
// common.h) are split into one contiguous range per XCD, and the work-groups
// of XCD x take tiles of range x in order from an atomic ticket counter, so
// the tiles running together on an XCD are neighbours that share weights and
// activations in its L2, and a CU that finishes a cheap ragged tile early
// simply takes the next one.  A work-group holds its next ticket one tile
// ahead; the DMA stream runs on across tiles (the last two K steps of a tile
// fetch the first two of the next), so a new tile starts without a prologue,
// and the tile map is built once per work-group.  The epilogue stages each
// wave's output through a private 2 KB LDS slot, 8 rows at a time, so it never
// touches the stages that already hold the next tile.  The ticket counters
// are a caller-owned set (common.h: zero at launch, cleared by the last
// work-group to retire).
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
#include <algorithm>
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

// epilogue staging, per wave: 8 rows of up to TN bf16 columns
constexpr int ST_PITCH = TN * 2 + 16;   // bytes; 17 chunks of 16, so rows start on different banks
constexpr int ST_BYTES = 8 * ST_PITCH;

constexpr int kCtrStride = kTicketStride;

// SAVE: also [a | u]; ACC_F32: C (fp32) += A B^T, one group; GATE: the router's
// gate product split over K (below)
enum { MODE_SWIGLU = 0, MODE_STORE = 1, MODE_SWIGLU_SAVE = 2, MODE_ACC_F32 = 3, MODE_GATE = 4 };

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
  int K;                   // multiple of 2*BK, at least 4*BK
  int n_tiles;             // column tiles per group
  int d_ff;                // SWIGLU: first up-projection row of w13
  uint16_t* C2;            // SWIGLU_SAVE: [a | u] output [rows, 2*d_ff]
  float* Cf;               // ACC_F32: fp32 output [rows, ldc], accumulated into
  int* tickets;            // this launch's ticket counter set (kTicketInts, zero)
  // an extra group after the n_exp groups of the offsets, with its own
  // buffers (the shared expert of the layer); x_rows = 0: none
  const uint16_t* Ax;      // [x_rows, K] activation rows
  const uint16_t* Bx;      // its weights [*, K]
  uint16_t* Cx;            // [x_rows, ldc] output
  int64_t x_rows;
  // GATE: K' = 3 * K / BK steps over the three bf16 planes of the gate weight
  // (B, B + plane_bytes, B + 2 * plane_bytes, each [n_tiles * BN, K]), plane
  // fastest; group g of the offsets holds the same T rows of A and takes steps
  // [g * ksteps, (g + 1) * ksteps), writing its fp32 partial product to rows
  // offsets[g] .. of Cf
  int ksteps;
  int64_t plane_bytes;
};

__device__ __forceinline__ void uniform_tile(TileInfo& t) {
  t.group = __builtin_amdgcn_readfirstlane(t.group);
  t.m_tile = __builtin_amdgcn_readfirstlane(t.m_tile);
  t.n_tile = __builtin_amdgcn_readfirstlane(t.n_tile);
  t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
  t.rows = __builtin_amdgcn_readfirstlane(t.rows);
}

// LDS writes of this wave are visible to its own later LDS reads
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void ffn_gemm_kernel(const FfnArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr bool SWI = MODE == MODE_SWIGLU || MODE == MODE_SWIGLU_SAVE;
  constexpr int STAGE = (BM + BN) * 8;   // uint4 per stage
  __shared__ uint4 smem[2 * STAGE];
  __shared__ uint4 s_stage[NW * ST_BYTES / 16];
  __shared__ int s_map[kMapInts];
  __shared__ int s_tick;
  // [A stage 0 | A stage 1 | B stage 0 | B stage 1]: a fragment read is a
  // per-lane base plus an immediate offset below 64 KB
  uint4* const sA0 = smem;
  uint4* const sA1 = smem + BM * 8;
  uint4* const sB0 = smem + 2 * BM * 8;
  uint4* const sB1 = smem + 2 * BM * 8 + BN * 8;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int xcd = blockIdx.x % kXcds;
  int* const tickets = p.tickets;

  constexpr bool GATE = MODE == MODE_GATE;
  const int n_grp = tile_map_build(p.offsets, p.n_exp, p.rows_total, BM, s_map, p.x_rows);
  const int total = s_map[n_grp] * p.n_tiles;
  const int ch = xcd_chunk(total);
  int tick_reg = 0;  // thread 0: the counter value fetched for the next tile
  if (tid == 0) s_tick = xcd_tile(atomicAdd(&tickets[xcd * kCtrStride], 1), xcd, ch);
  __syncthreads();
  const int l_first = __builtin_amdgcn_readfirstlane(s_tick);

  if (l_first < total) {
    const int nsteps = GATE ? p.ksteps : p.K / BK;
    TileInfo ti, tn;
    // the extra group's rows are counted from its own first row
    const int x_row0 = p.x_rows > 0 ? tile_map_offsets(s_map)[p.n_exp] : 0;
    auto localize = [&](TileInfo& t) __attribute__((always_inline)) {
      if (p.x_rows > 0 && t.group == p.n_exp) t.row0 -= x_row0;
    };
    tile_map_decode(l_first, n_grp, BM, p.n_tiles, s_map, 0, ti);
    uniform_tile(ti);
    localize(ti);
    bool nx = false;  // a next tile exists (known from step nsteps-2 on)

    // Direct-to-LDS loads: one instruction moves 64 lanes x 16 B into 1 KB of
    // LDS at lane*16, i.e. 8 rows of 128 B.  The LDS slot of a lane is fixed, so
    // the swizzle is applied to the global address: the lane filling physical
    // chunk pc of row r fetches logical chunk pc ^ ((r >> 1) & 7).  This wave
    // fills blocks j = wave + 8i (rows 8j..8j+7), for which (r >> 1) & 7 =
    // 4*(wave & 1) + (lane >> 4).
    const int lrow = lane >> 3;
    const int lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    // DMA sources: per-lane byte offsets that are the same for every tile,
    // added to wave-uniform bases (the tile's first row; its group's weight
    // tile).  Rows past the tile's valid rows: an 8-row block wholly past them
    // is not loaded (a wave-uniform branch, no instruction issued); in the
    // block that straddles the end, the lanes of invalid rows read the tile's
    // first row instead.  Every address stays inside the tile's rows (LDS-DMA
    // lanes switched off by EXEC were measured to still fetch), and the
    // padding rows' LDS values only reach padding outputs.
    uint32_t a_off[ADMA], b_off[BDMA];
    int a_row[ADMA];  // tile row this lane loads for part i
#pragma unroll
    for (int i = 0; i < ADMA; ++i) {
      a_row[i] = (wave + NW * i) * 8 + lrow;
      a_off[i] = static_cast<uint32_t>((a_row[i] * p.lda + lch * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < BDMA; ++i) {
      const int r = (wave + NW * i) * 8 + lrow;
      int wrow;  // weight row relative to the tile's base
      if constexpr (SWI) {
        // tile rows [part*TN, part*TN + TN/2) are gate rows, the next TN/2 the
        // matching up rows, for features n_tile*BN/2 + part*TN/2 + [0, TN/2)
        const int part = r / TN, within = r % TN;
        wrow = within < TN / 2 ? part * (TN / 2) + within : p.d_ff + part * (TN / 2) + (within - TN / 2);
      } else {
        wrow = r;
      }
      b_off[i] = static_cast<uint32_t>(((int64_t)wrow * p.K + lch * 8) * 2);
    }
    struct Src {
      const char* a;  // activation row of the tile's first row
      const char* b;  // the tile's first weight row
      int rows;
      int k0;         // GATE: the tile's first step of K'
    };
    auto src_of = [&](const TileInfo& t) __attribute__((always_inline)) {
      Src x;
      const int64_t w0 = (int64_t)t.n_tile * (SWI ? BN / 2 : BN);
      const bool ext = p.x_rows > 0 && t.group == p.n_exp;  // the extra group: its own buffers
      x.a = reinterpret_cast<const char*>((ext ? p.Ax : p.A) + (int64_t)t.row0 * p.lda);
      x.b = reinterpret_cast<const char*>(ext ? p.Bx + w0 * p.K
                                              : p.B + (int64_t)t.group * p.b_group_stride + w0 * p.K);
      x.rows = t.rows;
      x.k0 = 0;
      if constexpr (GATE) {
        // every group holds the same rows of A: count them from its first
        x.a = reinterpret_cast<const char*>(p.A + (int64_t)(t.row0 - tile_map_offsets(s_map)[t.group]) * p.lda);
        x.b = reinterpret_cast<const char*>(p.B + w0 * p.K);
        x.k0 = t.group * p.ksteps;
      }
      return x;
    };
    Src cur = src_of(ti), nxt = cur;

    // DMA part q of K step kk of the current tile (or of the next one) into
    // stage (sa, sb).
    auto dma_one = [&](int kk, bool next, uint4* sa, uint4* sb, int q) __attribute__((always_inline)) {
      const Src& x = next ? nxt : cur;
      int64_t kb = kk * BK * 2;  // byte offset of the step along K
      int64_t kbb = kb;
      if constexpr (GATE) {
        // step kg of K': 64 columns kin of x times plane kg - 3 kin
        const int kg = x.k0 + kk;
        const int kin = kg / 3;
        kb = (int64_t)kin * (BK * 2);
        kbb = (int64_t)(kg - 3 * kin) * p.plane_bytes + kb;
      }
      if (q < ADMA) {
        if ((wave + NW * q) * 8 < x.rows)
          dma16_s(x.a + kb, a_row[q] < x.rows ? a_off[q] : static_cast<uint32_t>(lch * 16),
                  lds_addr(sa) + (wave + NW * q) * 1024);
      } else {
        dma16_s(x.b + kbb, b_off[q - ADMA], lds_addr(sb) + (wave + NW * (q - ADMA)) * 1024);
      }
    };
    // Step nsteps-2, after its barrier: take the next ticket and address
    // that tile.
    auto retarget = [&]() __attribute__((always_inline)) {
      const int l_next = __builtin_amdgcn_readfirstlane(s_tick);
      nx = l_next < total;
      if (nx) {
        tile_map_decode(l_next, n_grp, BM, p.n_tiles, s_map, ti.group, tn);
        uniform_tile(tn);
        localize(tn);
        nxt = src_of(tn);
      }
    };
    // Step 0, after its barrier: thread 0 asks for the following ticket (its
    // reply is waited for with the DMA at step 1's barrier, then published).
    // (the counter's index carries an opaque zero, so the compiler keeps a
    // plain one-lane atomic instead of a wave-combined one that reads its
    // result back at once)
    int zero = lane >> 6;
    asm volatile("" : "+v"(zero));
    auto ask_ticket = [&]() __attribute__((always_inline)) {
      if (tid == 0) tick_reg = atomicAdd(&tickets[xcd * kCtrStride + zero], 1);
    };
    auto publish_ticket = [&]() __attribute__((always_inline)) {
      if (tid == 0) s_tick = xcd_tile(tick_reg, xcd, ch);
    };

    f32x16 acc[RM][RN];
    bf16x8 fa[2][RM], fb[2][RN];
    // Fragment rows start on multiples of 32, so the swizzle term (r >> 1) & 7
    // of row r = base + (lane & 31) depends on the lane only: a read is a
    // per-lane offset (one per slice) plus a constant row base.
    // The wave's row base is folded into the per-lane offsets (one per slice
    // and operand), so the fragments of a slice differ by constants only.
    int a_lane[NS], b_lane[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int off = (lane & 31) * 8 + ((2 * s + (lane >> 5)) ^ (((lane & 31) >> 1) & 7));
      a_lane[s] = 32 * wm * 8 + off;
      b_lane[s] = wn * TN * 8 + off;
    }
    auto read_frag = [&](const uint4* sa, const uint4* sb, int buf, int s, int f)
                         __attribute__((always_inline)) {
      if (f == 0) {
        fa[buf][0] = as_bf16x8(sa[a_lane[s]]);
      } else if (f <= RN) {
        fb[buf][f - 1] = as_bf16x8(sb[b_lane[s] + (f - 1) * 32 * 8]);
      } else {
        fa[buf][f - RN] = as_bf16x8(sa[a_lane[s] + (f - RN) * HB * 8]);
      }
    };
    // MFMAs of slice s over the first NB row blocks; reads of slice rs of
    // (rsa, rsb) into the other buffer (rs < 0: none); DMA parts
    // [d0, d1) of step kd (kd < 0: none).  With one block there are five reads
    // for four MFMA slots: the first slot takes two.
    auto slice = [&](auto nbc, int s, const uint4* rsa, const uint4* rsb, int rs, int kd, bool next,
                     uint4* da, uint4* db, int d0, int d1) __attribute__((always_inline)) {
      constexpr int NB = decltype(nbc)::value;
      constexpr int NQB = NB * RN, NRB = NB + RN;
      constexpr int XR = NRB > NQB ? NRB - NQB : 0;  // reads doubled up in slot 0
      const int buf = s & 1;
      const int nd = d1 - d0;
#pragma unroll
      for (int q = 0; q < NQB; ++q) {
        const int i = q / RN, j = q % RN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
        if (rs >= 0) {
#pragma unroll
          for (int f = 0; f < NRB; ++f)
            if ((f < XR ? 0 : f - XR) == q) read_frag(rsa, rsb, buf ^ 1, rs, f);
        }
        if (kd >= 0) {
#pragma unroll
          for (int t = 0; t < NDMA; ++t)
            if (t < nd && (t * NQB) / nd == q) dma_one(kd, next, da, db, d0 + t);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep this interleaving
      }
    };
    // K steps.  Step kt's second DMA half is that of step kt+1, its first
    // half that of step kt+2; in the last two steps of a tile these are the
    // first two steps of the next tile (stage parity carries over because
    // nsteps is even).  Step kt computes from stage (sa, sb); (na, nb_) holds
    // step kt+1.  The main loop runs steps 0 .. nsteps-3; the tail runs the
    // last two, where the next tile is taken.
    auto step = [&](auto nbc, int kt, uint4* sa, uint4* sb, uint4* na, uint4* nb_)
                    __attribute__((always_inline)) {
      slice(nbc, 0, sa, sb, 1, kt + 1, false, na, nb_, DHALF, NDMA);
#pragma unroll
      for (int s = 1; s + 1 < NS; ++s) slice(nbc, s, sa, sb, s + 1, -1, false, nullptr, nullptr, 0, 0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): step kt's fragments are in registers
      wait_vmcnt<0>();                     // this wave's DMA of step kt+1 has landed
      if (kt == 1) publish_ticket();
      barrier_only();                      // everyone's has; stage (sa, sb) is free
      if (kt == 0) ask_ticket();
      // last slice: reads of step kt+1's first slice, first DMA half of step kt+2
      slice(nbc, NS - 1, na, nb_, 0, kt + 2, false, sa, sb, 0, DHALF);
    };
    // the last two steps: stages 0 and 1
    auto tail = [&](auto nbc) __attribute__((always_inline)) {
      // step nsteps-2: this tile's step nsteps-1, then the next tile's step 0
      slice(nbc, 0, sA0, sB0, 1, nsteps - 1, false, sA1, sB1, DHALF, NDMA);
#pragma unroll
      for (int s = 1; s + 1 < NS; ++s) slice(nbc, s, sA0, sB0, s + 1, -1, false, nullptr, nullptr, 0, 0);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      wait_vmcnt<0>();
      barrier_only();
      retarget();
      slice(nbc, NS - 1, sA1, sB1, 0, nx ? 0 : -1, true, sA0, sB0, 0, DHALF);
      // step nsteps-1: the next tile's step 0 (second half) and step 1 (first half)
      slice(nbc, 0, sA1, sB1, 1, nx ? 0 : -1, true, sA0, sB0, DHALF, NDMA);
#pragma unroll
      for (int s = 1; s + 1 < NS; ++s) slice(nbc, s, sA1, sB1, s + 1, -1, false, nullptr, nullptr, 0, 0);
      if (nx) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        wait_vmcnt<0>();  // the next tile's step 0 has landed
        barrier_only();
      }
      slice(nbc, NS - 1, sA0, sB0, -1, nx ? 1 : -1, true, sA1, sB1, 0, DHALF);
    };
    // A wave without valid rows keeps the same DMA parts and barriers.
    auto idle_dma = [&](int kd, bool next, uint4* da, uint4* db, int d0, int d1) __attribute__((always_inline)) {
      if (kd >= 0) {
#pragma unroll
        for (int q = 0; q < NDMA; ++q)
          if (q >= d0 && q < d1) dma_one(kd, next, da, db, q);
      }
    };
    auto idle_step = [&](int kt, uint4* sa, uint4* sb, uint4* na, uint4* nb_) __attribute__((always_inline)) {
      idle_dma(kt + 1, false, na, nb_, DHALF, NDMA);
      wait_vmcnt<0>();
      if (kt == 1) publish_ticket();
      barrier_only();
      if (kt == 0) ask_ticket();
      idle_dma(kt + 2, false, sa, sb, 0, DHALF);
    };
    auto idle_tail = [&]() __attribute__((always_inline)) {
      idle_dma(nsteps - 1, false, sA1, sB1, DHALF, NDMA);
      wait_vmcnt<0>();
      barrier_only();
      retarget();
      idle_dma(nx ? 0 : -1, true, sA0, sB0, 0, DHALF);
      idle_dma(nx ? 0 : -1, true, sA0, sB0, DHALF, NDMA);
      if (nx) {
        wait_vmcnt<0>();
        barrier_only();
      }
      idle_dma(nx ? 1 : -1, true, sA1, sB1, 0, DHALF);
    };

    // Epilogue of tile ti, by each wave for its own rows.  Accumulator (i, j)
    // register v holds row 8*(v/4) + 4*(lane/32) + v%4 and column lane%32 of
    // its 32x32 block; a pass takes the 8 rows of one v/4 and leaves as
    // 16-byte row chunks through this wave's staging slot.  Registers v and
    // v+1 (v even) are consecutive rows of one column: each pair is rounded by
    // one packed conversion.  silu(g) = g / (1 + e^-g) takes the hardware
    // reciprocal (1 ulp, far below the bf16 rounding of h).
    char* const st = reinterpret_cast<char*>(s_stage) + wave * ST_BYTES;
    auto put2 = [&](int lr, int col, uint32_t pk) __attribute__((always_inline)) {
      reinterpret_cast<uint16_t*>(st + lr * ST_PITCH)[col] = static_cast<uint16_t>(pk);
      reinterpret_cast<uint16_t*>(st + (lr + 1) * ST_PITCH)[col] = static_cast<uint16_t>(pk >> 16);
    };
    // (the epilogue's addresses derive from an opaque copy of the lane index,
    // so the compiler computes them per tile instead of holding them in
    // registers through the K loop)
    auto silu_mul = [](float g, float u) __attribute__((always_inline)) {
      return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
    };
    auto epilogue = [&](int nb) __attribute__((always_inline)) {
      int lane = tid & 63;
      asm volatile("" : "+v"(lane));
      constexpr int OUT_COLS = SWI ? BN / 2 : BN;
      const int64_t col0 = (int64_t)ti.n_tile * OUT_COLS;
      const int lr0 = 4 * (lane >> 5);
      uint16_t* const cb = p.x_rows > 0 && ti.group == p.n_exp ? p.Cx : p.C;  // output buffer of the tile
      if constexpr (MODE == MODE_ACC_F32 || GATE) {
        // fp32 read-modify-write (GATE: store) straight from the registers:
        // for a fixed register the 32 lanes of a half-wave cover 128
        // contiguous bytes
#pragma unroll
        for (int i = 0; i < RM; ++i) {
          if (i >= nb) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = i * HB + 32 * wm + 8 * (v >> 2) + lr0 + (v & 3);
            if (r >= ti.rows) continue;
            float* row = p.Cf + ((int64_t)ti.row0 + r) * p.ldc + col0 + wn * TN + (lane & 31);
#pragma unroll
            for (int j = 0; j < RN; ++j) {
              if constexpr (GATE) row[j * 32] = acc[i][j][v];
              else row[j * 32] += acc[i][j][v];
            }
          }
        }
        return;
      }
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        if (i >= nb) continue;
#pragma unroll
        for (int quad = 0; quad < 4; ++quad) {
          const int rb = i * HB + 32 * wm + 8 * quad;  // tile row of the pass's first row
          if (rb >= ti.rows) continue;
          const int64_t grow0 = (int64_t)ti.row0 + rb;
#pragma unroll
          for (int v = 4 * quad; v < 4 * quad + 4; v += 2) {
            const int lr = lr0 + (v & 3);
            if constexpr (SWI) {
#pragma unroll
              for (int jj = 0; jj < RN / 2; ++jj) {
                const f32x16& g = acc[i][jj];
                const f32x16& u = acc[i][jj + RN / 2];
                put2(lr, jj * 32 + (lane & 31), pack_bf16x2(silu_mul(g[v], u[v]), silu_mul(g[v + 1], u[v + 1])));
              }
            } else {
#pragma unroll
              for (int j = 0; j < RN; ++j)
                put2(lr, j * 32 + (lane & 31), pack_bf16x2(acc[i][j][v], acc[i][j][v + 1]));
            }
          }
          wave_lds_fence();
          if constexpr (SWI) {
            // 8 rows x 128 B: one chunk per lane
            const int r = lane >> 3, c = lane & 7;
            if (rb + r < ti.rows) {
              const uint4 val = *reinterpret_cast<const uint4*>(st + r * ST_PITCH + c * 16);
              *reinterpret_cast<uint4*>(cb + (grow0 + r) * p.ldc + col0 + wn * (TN / 2) + c * 8) = val;
            }
          } else {
            // 8 rows x 256 B: two chunks per lane
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int q = lane + 64 * h;
              const int r = q >> 4, c = q & 15;
              if (rb + r < ti.rows) {
                const uint4 val = *reinterpret_cast<const uint4*>(st + r * ST_PITCH + c * 16);
                *reinterpret_cast<uint4*>(cb + (grow0 + r) * p.ldc + col0 + wn * TN + c * 8) = val;
              }
            }
          }
          if constexpr (MODE == MODE_SWIGLU_SAVE) {
            // the pre-activations for the backward: a (gate) at column
            // col0 + f and u (up) at d_ff + col0 + f, bf16
            wave_lds_fence();  // the h chunks have been read
#pragma unroll
            for (int v = 4 * quad; v < 4 * quad + 4; v += 2) {
              const int lr = lr0 + (v & 3);
#pragma unroll
              for (int jj = 0; jj < RN / 2; ++jj) {
                const int c = jj * 32 + (lane & 31);
                put2(lr, c, pack_bf16x2(acc[i][jj][v], acc[i][jj][v + 1]));
                put2(lr, TN / 2 + c, pack_bf16x2(acc[i][jj + RN / 2][v], acc[i][jj + RN / 2][v + 1]));
              }
            }
            wave_lds_fence();
            const int64_t ld2 = 2 * (int64_t)p.d_ff;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int q = lane + 64 * h;
              const int r = q >> 4, c = q & 15;
              const int half = c >> 3, cc = c & 7;
              if (rb + r < ti.rows) {
                const uint4 val = *reinterpret_cast<const uint4*>(st + r * ST_PITCH + c * 16);
                *reinterpret_cast<uint4*>(p.C2 + (grow0 + r) * ld2 + half * p.d_ff + col0 +
                                          wn * (TN / 2) + cc * 8) = val;
              }
            }
          }
          wave_lds_fence();  // the chunks have been read before the next pass overwrites the slot
        }
      }
    };

    // prologue of the first tile: what a tile's predecessor sends in its last
    // two steps (all of step 0, the first half of step 1)
#pragma unroll
    for (int q = 0; q < NDMA; ++q) dma_one(0, false, sA0, sB0, q);
#pragma unroll
    for (int q = 0; q < DHALF; ++q) dma_one(1, false, sA1, sB1, q);
    wait_vmcnt<0>();
    barrier_only();

    for (;;) {
      // valid 32-row blocks of this wave: block i covers rows i*HB + 32*wm + [0, 32)
      const int nb = __builtin_amdgcn_readfirstlane((ti.rows > 32 * wm) + (ti.rows > HB + 32 * wm));
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      if (nb == RM) {
        using NBC = std::integral_constant<int, RM>;
#pragma unroll
        for (int f = 0; f < NR; ++f) read_frag(sA0, sB0, 0, 0, f);
        for (int kt = 0; kt < nsteps - 2; kt += 2) {
          step(NBC{}, kt, sA0, sB0, sA1, sB1);
          step(NBC{}, kt + 1, sA1, sB1, sA0, sB0);
        }
        tail(NBC{});
      } else if (nb == 1) {
        using NBC = std::integral_constant<int, 1>;
#pragma unroll
        for (int f = 0; f <= RN; ++f) read_frag(sA0, sB0, 0, 0, f);
        for (int kt = 0; kt < nsteps - 2; kt += 2) {
          step(NBC{}, kt, sA0, sB0, sA1, sB1);
          step(NBC{}, kt + 1, sA1, sB1, sA0, sB0);
        }
        tail(NBC{});
      } else {
        for (int kt = 0; kt < nsteps - 2; kt += 2) {
          idle_step(kt, sA0, sB0, sA1, sB1);
          idle_step(kt + 1, sA1, sB1, sA0, sB0);
        }
        idle_tail();
      }
      epilogue(nb);
      if (!nx) break;
      ti = tn;
      cur = nxt;
      nx = false;
    }
  }
  // retire: the last work-group out clears this launch's counters
  if (tid == 0) {
    if (atomicAdd(&tickets[kXcds * kCtrStride], 1) == (int)gridDim.x - 1) {
#pragma unroll
      for (int x = 0; x <= kXcds; ++x) atomicExch(&tickets[x * kCtrStride], 0);
    }
  }
#endif
}

template <int MODE>
hipError_t launch(FfnArgs& a, int64_t max_rows, hipStream_t s) {
  if (MODE == MODE_GATE) {
    if (a.ksteps % 2 != 0 || a.ksteps < 4 || a.K % BK != 0) return hipErrorInvalidValue;
  } else if (a.K % (2 * BK) != 0 || a.K < 4 * BK) {
    return hipErrorInvalidValue;
  }
  // 32-bit per-lane DMA offsets: a tile's rows and a group's weights
  constexpr bool swi = MODE == MODE_SWIGLU || MODE == MODE_SWIGLU_SAVE;
  const int64_t b_rows = swi ? 2 * (int64_t)a.d_ff : (int64_t)a.n_tiles * BN;
  if ((int64_t)BM * a.lda * 2 >= (1LL << 31) || b_rows * a.K * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  const int64_t mt = max_row_tiles(max_rows, a.offsets == nullptr ? 1 : a.n_exp, BM, a.x_rows);
  const int64_t tiles = mt * a.n_tiles;
  if (tiles <= 0) return hipSuccess;
  // one work-group per CU the stream may use (the LDS holds one), a multiple
  // of the XCD count
  const int64_t grid = (std::min<int64_t>(tiles, stream_cu_count(s)) + kXcds - 1) / kXcds * kXcds;
  if (a.tickets == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL((ffn_gemm_kernel<MODE>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                              int d_ff, const uint16_t* xp, const uint16_t* w13, uint16_t* h,
                              int* tickets, hipStream_t s, uint16_t* au, const moe_ffn_extra* extra) {
  FfnArgs a{};
  a.tickets = tickets;
  if (extra != nullptr && extra->rows > 0) {
    if (offsets == nullptr || au != nullptr) return hipErrorInvalidValue;
    a.Ax = static_cast<const uint16_t*>(extra->x);
    a.Bx = static_cast<const uint16_t*>(extra->w13);
    a.Cx = static_cast<uint16_t*>(extra->h);
    a.x_rows = extra->rows;
  }
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
                                 const uint16_t* A, const uint16_t* B, uint16_t* C, int* tickets,
                                 hipStream_t s) {
  FfnArgs a{};
  a.tickets = tickets;
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

hipError_t launch_gemm_acc_f32(int64_t rows, int K, int N, const uint16_t* A, const uint16_t* B, float* C,
                               int* tickets, hipStream_t s) {
  FfnArgs a{};
  a.tickets = tickets;
  a.A = A;
  a.lda = K;
  a.B = B;
  a.Cf = C;
  a.ldc = N;
  a.offsets = nullptr;
  a.n_exp = 1;
  a.rows_total = rows;
  a.K = K;
  a.n_tiles = N / BN;
  return launch<MODE_ACC_F32>(a, rows, s);
}

// The router gate product as S split-K partial products on this kernel (GATE
// mode): parts[g] = x * (planes over steps [g*K'/S, (g+1)*K'/S))^T, fp32,
// [S, T, E].  offsets = {0, T, 2T, ..., S*T} on the device.
bool gate_split_supported(int d, int E) { return E % BN == 0 && d % BK == 0; }

// The most splits that keep the launch at one tile per CU of an MI355X (256;
// a fixed figure, so that the workspace size does not depend on the device),
// with an even step count of at least 4 per split.
int gate_split_count(int64_t T, int d, int E) {
  if (!gate_split_supported(d, E)) return 0;
  constexpr int64_t kTargetTiles = 256;
  const int steps = 3 * (d / BK);
  const int64_t tiles1 = (T + BM - 1) / BM * (E / BN);
  int best = 0;
  for (int S = 1; S <= kMaxGateSplits; ++S) {
    if (steps % (2 * S) != 0 || steps / S < 4) continue;
    if (S > 1 && tiles1 * S > kTargetTiles) break;
    best = S;
  }
  return best;
}

hipError_t launch_gate_split_bf16(const uint16_t* x, const uint16_t* planes, float* parts, int64_t T,
                                  int d, int E, int S, const int32_t* offsets, int* tickets,
                                  hipStream_t s) {
  if (S < 1 || 3 * (d / BK) % S != 0) return hipErrorInvalidValue;
  FfnArgs a{};
  a.tickets = tickets;
  a.A = x;
  a.lda = d;
  a.B = planes;
  a.Cf = parts;
  a.ldc = E;
  a.offsets = offsets;
  a.n_exp = S;
  a.rows_total = S * T;
  a.K = d;
  a.n_tiles = E / BN;
  a.ksteps = 3 * (d / BK) / S;
  a.plane_bytes = (int64_t)E * d * 2;
  return launch<MODE_GATE>(a, S * T, s);
}

hipError_t launch_ffn_down_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                                int d_ff, const uint16_t* h, const uint16_t* w2, uint16_t* yp,
                                int* tickets, hipStream_t s, const moe_ffn_extra* extra) {
  if (extra == nullptr || extra->rows == 0)
    return launch_ffn_store_bf16(n_exp, offsets, max_rows, d_ff, d, h, w2, yp, tickets, s);
  if (offsets == nullptr) return hipErrorInvalidValue;
  FfnArgs a{};
  a.tickets = tickets;
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
  a.n_tiles = d / BN;
  a.Ax = static_cast<const uint16_t*>(extra->h);
  a.Bx = static_cast<const uint16_t*>(extra->w2);
  a.Cx = static_cast<uint16_t*>(extra->y);
  a.x_rows = extra->rows;
  return launch<MODE_STORE>(a, max_rows, s);
}

}  // namespace moe
