// Grouped e4m3 expert products on gfx950 matrix cores, persistent form (the
// fp8 workload's routed and shared experts when K is a multiple of 256 and at
// least 512; gemm_fp8.hip covers the other widths):
//
//   up   (SWIGLU): h = silu(x W1^T) * (x W3^T), requantised to e4m3 per 1 x 128
//   down (STORE) : y = h W2^T, bf16
//
// with activations carrying one fp32 scale per 1 x 128 tile of a row and
// weights one fp32 scale per 128 x 128 block, fp32 accumulation:
//
//   C[m][n] = sum_kb  sa[m][kb] * sb[n/128][kb] * P_kb[m][n],
//   P_kb    = sum_{k in block kb} qa[m][k] * qb[n][k]   (exact in fp32).
//
// Promotion without a second accumulator: the accumulator holds C divided by
// the current block's scale product S_kb = sa[m][kb] * sb[n/128][kb].  Before
// block kb's MFMAs each element is multiplied by S_{kb-1} / S_kb, after which
// the MFMAs add P_kb straight into it; the epilogue multiplies by the last
// block's S.  That is one vector multiply per accumulator element per block
// (the same count as an explicit FMA promotion of a partial sum) and no
// partial-sum registers.
//
// Tile 256 rows x 256 weight rows (the 1 x 128 quantisation tile of h, 128
// features = 256 gate/up weight rows, lies in one work-group).  8 waves as
// 4 x 2, each 64 x 128 (2 x 4 blocks of 32x32).  A K step is 128 bytes per row
// (one scale block; two v_mfma_scale_f32_32x32x64_f8f6f4 slices with unit
// matrix-core scales) and moves 64 KB for 16.8 MFLOP: a 128-row tile would
// need half again as many bytes per FLOP, more than the per-CU load path
// delivers at the fp8 rate.  An fp8 fragment is 8 VGPRs, so the 64 x 128 wave
// tile fits two waves per SIMD only with one set of fragments: each read of
// the next slice goes out in the MFMA slot right after the last use of the
// fragment it replaces.  The rest follows the bf16 kernel (ffn_bf16.hip): two
// 64 KB stages of swizzled 128-byte rows filled by direct-to-LDS DMA,
// persistent work-groups taking ticketed tiles with the DMA stream running on
// across tiles, a wave's row blocks in both halves of the tile.  The
// activation row scales travel by 4-byte DMA into a ring of four slots; the
// weight block scales are scalar loads.
//
// Epilogues
//   SWIGLU  g, u = the accumulators times their scales, h = silu(g) * u; the
//           1 x 128 quantisation tile of h spans the two feature waves of a
//           row, so each wave reduces its half of the row amax and the
//           halves meet in LDS; codes = e4m3(h / scale), scale = amax / 448.
//   STORE   bf16 output through each wave's staging slot.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int BM = 256;          // activation rows per tile
constexpr int BN = 256;          // weight rows per tile
constexpr int BKB = 128;         // K per step: 128 e4m3 bytes = one scale block
constexpr int NW = 8;
constexpr int WAVES_M = 4;
constexpr int WAVES_N = NW / WAVES_M;
constexpr int kThreads = NW * 64;
constexpr int TM = BM / WAVES_M;  // 64
constexpr int TN = BN / WAVES_N;  // 128
constexpr int RM = TM / 32, RN = TN / 32;
constexpr int HB = BM / RM;       // 128: row distance between a wave's blocks
constexpr int ADMA = BM / (8 * NW);
constexpr int BDMA = BN / (8 * NW);
constexpr int NDMA = ADMA + BDMA;
constexpr int DHALF = NDMA / 2;
constexpr int NS = 2;             // K = 64 slices per step
constexpr int SC_SLOTS = 4;       // activation-scale ring
static_assert(RM == 2 && RN == 4, "tile layout");

constexpr int ST_PITCH = TN * 2 + 16;  // STORE staging: 8 rows of 128 bf16
constexpr int ST_BYTES = 8 * ST_PITCH;
constexpr int H_PITCH = TN / 2 + 16;   // SWIGLU staging: 8 rows of 64 codes
constexpr int H_BYTES = 8 * H_PITCH;

constexpr int kCtrStride = kTicketStride;

enum { MODE_SWIGLU = 0, MODE_STORE = 1 };

struct Fp8Args {
  const uint8_t* A;         // [rows, K] codes
  const float* A_scale;     // [K/128][scale_ld]: one 128-wide block's scales contiguous over rows
  int64_t lda;              // bytes per row (= K)
  const uint8_t* B;         // [groups][N_rows][K] codes
  const float* B_scale;     // [groups][N_rows/128][K/128]
  int64_t b_group_stride;   // bytes
  int64_t bs_group_stride;  // floats
  void* C;
  float* C_scale;           // SWIGLU: [d_ff/128][scale_ld]
  int64_t scale_ld;         // rows of the scale matrices (the buffers' row capacity)
  int64_t ldc;              // elements
  const int* offsets;
  int n_exp;
  int64_t rows_total;
  int K;
  int n_tiles;
  int d_ff;                 // SWIGLU: first up row of w13
  int* tickets;             // this launch's ticket counter set (kTicketInts, zero)
};

typedef int i32x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8v as_i32x8(uint4 lo, uint4 hi) {
  i32x8v r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

__device__ __forceinline__ void uniform_tile(TileInfo& t) {
  t.group = __builtin_amdgcn_readfirstlane(t.group);
  t.m_tile = __builtin_amdgcn_readfirstlane(t.m_tile);
  t.n_tile = __builtin_amdgcn_readfirstlane(t.n_tile);
  t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
  t.rows = __builtin_amdgcn_readfirstlane(t.rows);
}

__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float uniform_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// MFMA slot of a slice (row block outer, weight block inner) after which
// fragment f of the next slice is read (f = 0: a0, 1..RN: b, RN + 1: a1),
// with nb row blocks in use: the slot of the last use of the fragment it
// replaces, so one set of fragment registers is live at a time.  With one
// block, a0 goes a slot early, as b(RN-1) takes the last one.
__host__ __device__ constexpr int read_slot(int nb, int f) {
  return nb == RM ? (f == 0 ? RN - 1 : f <= RN ? RN + f - 1 : 2 * RN - 1)
                  : (f == 0 ? RN - 2 : f - 1);
}
static_assert(read_slot(RM, 0) == 3 && read_slot(RM, 1) == 4 && read_slot(RM, RN) == 7 &&
              read_slot(RM, RN + 1) == 7 && read_slot(1, 0) == 2 && read_slot(1, RN) == 3,
              "read schedule");

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void ffn_fp8_kernel(const Fp8Args p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr bool SWI = MODE == MODE_SWIGLU;
  constexpr int NJB = SWI ? 2 : 1;  // weight scale blocks of a wave's columns (SWIGLU: gate, up)
  constexpr int NJW = RN / NJB;     // accumulator columns per weight scale block
  constexpr int STAGE = (BM + BN) * 8;
  constexpr int STG_U4 = NW * (SWI ? H_BYTES : ST_BYTES) / 16;
  __shared__ uint4 smem[2 * STAGE];
  __shared__ float s_sc[SC_SLOTS][BM];          // activation row scales per step
  __shared__ float s_sc_junk[64];               // scale loads of the waves past BM/64
  __shared__ float s_fac[NW][NJB][TM];          // per-wave row factors
  __shared__ uint4 s_stage[STG_U4];
  __shared__ float s_amax[SWI ? WAVES_N : 1][SWI ? BM : 1];
  __shared__ int s_map[kMapInts];
  __shared__ int s_tick;
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

  const int n_grp = tile_map_build(p.offsets, p.n_exp, p.rows_total, BM, s_map);
  const int total = s_map[n_grp] * p.n_tiles;
  const int ch = xcd_chunk(total);
  int tick_reg = 0;
  if (tid == 0) s_tick = xcd_tile(atomicAdd(&tickets[xcd * kCtrStride], 1), xcd, ch);
  __syncthreads();
  const int l_first = __builtin_amdgcn_readfirstlane(s_tick);

  if (l_first < total) {
    const int nsteps = p.K / BKB;
    TileInfo ti, tn;
    tile_map_decode(l_first, n_grp, BM, p.n_tiles, s_map, 0, ti);
    uniform_tile(ti);
    bool nx = false;
    int sc_base = 0;  // scale-ring slot of the tile's step 0 (steps run on across tiles)

    // DMA sources: tile-invariant per-lane offsets on wave-uniform bases;
    // lanes of rows past the tile's valid ones read its first row.
    const int lrow = lane >> 3;
    const int lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    uint32_t a_off[ADMA], b_off[BDMA];
    int a_row[ADMA];
#pragma unroll
    for (int i = 0; i < ADMA; ++i) {
      a_row[i] = (wave + NW * i) * 8 + lrow;
      a_off[i] = static_cast<uint32_t>(a_row[i] * p.lda + lch * 16);
    }
#pragma unroll
    for (int i = 0; i < BDMA; ++i) {
      const int r = (wave + NW * i) * 8 + lrow;
      int wrow;
      if constexpr (SWI) {
        const int part = r / TN, within = r % TN;
        wrow = within < TN / 2 ? part * (TN / 2) + within : p.d_ff + part * (TN / 2) + (within - TN / 2);
      } else {
        wrow = r;
      }
      b_off[i] = static_cast<uint32_t>((int64_t)wrow * p.K + lch * 16);
    }
    const int nkb = p.K / BKB;
    struct Src {
      const char* a;    // activation row of the tile's first row
      const char* b;    // the tile's first weight row
      const float* as;  // activation scales of the tile's first row
      const float* bs;  // weight block scales of the tile's group
      int rows, n_tile;
    };
    auto src_of = [&](const TileInfo& t) __attribute__((always_inline)) {
      Src x;
      x.a = reinterpret_cast<const char*>(p.A + (int64_t)t.row0 * p.lda);
      const int64_t w0 = (int64_t)t.n_tile * (SWI ? BN / 2 : BN);
      x.b = reinterpret_cast<const char*>(p.B + (int64_t)t.group * p.b_group_stride + w0 * p.K);
      x.as = p.A_scale + t.row0;
      x.bs = p.B_scale + (int64_t)t.group * p.bs_group_stride;
      x.rows = t.rows;
      x.n_tile = t.n_tile;
      return x;
    };
    Src cur = src_of(ti), nxt = cur;

    // weight scale block rows of this wave's columns: SWIGLU gate / up blocks
    // of the tile's features; STORE the 128-row block of its 128 columns
    auto sb_blk = [&](const Src& x, int jb) __attribute__((always_inline)) {
      if constexpr (SWI) return jb == 0 ? x.n_tile : p.d_ff / BKB + x.n_tile;
      return (x.n_tile * BN + wn * TN) / 128;
    };
    auto sb_load = [&](const Src& x, int jb, int kk) __attribute__((always_inline)) {
      return x.bs[(int64_t)sb_blk(x, jb) * nkb + kk];
    };

    // DMA part q of step kk (of the current tile, or the next) into stage
    // (sa, sb); waves 0..3 also bring that step's 256 row scales into ring
    // slot `slot`.
    // (No branches here: a branch per MFMA slot lets the compiler sink the
    // MFMAs past them and hold several slices' fragments at once.  Every
    // activation block is loaded, rows past the valid ones reading the
    // tile's first row; every wave issues the scale load, waves past the
    // BM/64 that cover the tile writing a scratch slot instead.)
    auto dma_one = [&](int kk, bool next, uint4* sa, uint4* sb, int q, int slot) __attribute__((always_inline)) {
      const Src& x = next ? nxt : cur;
      const int kb = kk * BKB;
      if (q < ADMA) {
        dma16_s(x.a + kb, a_row[q] < x.rows ? a_off[q] : static_cast<uint32_t>(lch * 16),
                lds_addr(sa) + (wave + NW * q) * 1024);
        if (q == 0) {
          const int r = 64 * (wave % (BM / 64)) + lane;
          const int rr = r < x.rows ? r : 0;
          const uint32_t dst = wave < BM / 64 ? lds_addr(&s_sc[slot][0]) + 64 * 4 * wave : lds_addr(&s_sc_junk[0]);
          dma4(x.as + (int64_t)kk * p.scale_ld + rr, dst);
        }
      } else {
        dma16_s(x.b + kb, b_off[q - ADMA], lds_addr(sb) + (wave + NW * (q - ADMA)) * 1024);
      }
    };
    auto retarget = [&]() __attribute__((always_inline)) {
      const int l_next = __builtin_amdgcn_readfirstlane(s_tick);
      nx = l_next < total;
      if (nx) {
        tile_map_decode(l_next, n_grp, BM, p.n_tiles, s_map, ti.group, tn);
        uniform_tile(tn);
        nxt = src_of(tn);
      }
    };
    int zero = lane >> 6;
    asm volatile("" : "+v"(zero));
    auto ask_ticket = [&]() __attribute__((always_inline)) {
      if (tid == 0) tick_reg = atomicAdd(&tickets[xcd * kCtrStride + zero], 1);
    };
    auto publish_ticket = [&]() __attribute__((always_inline)) {
      if (tid == 0) s_tick = xcd_tile(tick_reg, xcd, ch);
    };
    auto slot_of = [&](int kk) __attribute__((always_inline)) { return (sc_base + kk) & (SC_SLOTS - 1); };

    f32x16 acc[RM][RN];
    i32x8v fa[2][RM], fb[2][RN];  // by slice parity

    // fragment addressing: slice h covers K bytes [64h, 64h + 64); lanes
    // 0-31 the first 32 of them, lanes 32-63 the next; a fragment is two
    // 16-byte chunks c0 ^ x and (c0 + 1) ^ x of its row, x = ((row >> 1) & 7)
    // depends on the lane only (rows start on multiples of 32)
    int a_l0[NS], a_l1[NS], b_l0[NS], b_l1[NS];
#pragma unroll
    for (int h = 0; h < NS; ++h) {
      const int x = ((lane & 31) >> 1) & 7;
      const int c0 = (4 * h + 2 * (lane >> 5)) ^ x;
      const int c1 = c0 ^ 1;
      a_l0[h] = (32 * wm + (lane & 31)) * 8 + c0;
      a_l1[h] = (32 * wm + (lane & 31)) * 8 + c1;
      b_l0[h] = (wn * TN + (lane & 31)) * 8 + c0;
      b_l1[h] = (wn * TN + (lane & 31)) * 8 + c1;
    }
    // fragment f of slice h into buffer buf: f = 0: a0, 1..RN: b, then a1
    auto read_frag = [&](const uint4* sa, const uint4* sb, int buf, int h, int f) __attribute__((always_inline)) {
      if (f == 0) {
        fa[buf][0] = as_i32x8(sa[a_l0[h]], sa[a_l1[h]]);
      } else if (f <= RN) {
        const int j = f - 1;
        fb[buf][j] = as_i32x8(sb[b_l0[h] + j * 32 * 8], sb[b_l1[h] + j * 32 * 8]);
      } else {
        const int i = f - RN;
        fa[buf][i] = as_i32x8(sa[a_l0[h] + i * HB * 8], sa[a_l1[h] + i * HB * 8]);
      }
    };

    // row factors: lane l of the wave owns row (l / 32) * HB + 32 * wm + l % 32
    // of the tile; s_fac[wave][jb][l] = value * fb[jb] for that row, read back
    // four consecutive rows at a time in the accumulator's row order
    const int my_row = (lane >> 5) * HB + 32 * wm + (lane & 31);
    auto put_factors = [&](float rowv, const float (&fbj)[NJB]) __attribute__((always_inline)) {
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) s_fac[wave][jb][lane] = rowv * fbj[jb];
    };
    auto get_factors = [&](int i, int jb, float (&f)[16]) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = *reinterpret_cast<const float4*>(&s_fac[wave][jb][i * 32 + 8 * g + 4 * (lane >> 5)]);
        f[4 * g] = v.x; f[4 * g + 1] = v.y; f[4 * g + 2] = v.z; f[4 * g + 3] = v.w;
      }
    };
    // weight block scales of the current and the next step (wave-uniform)
    float sbc[NJB], sbn[NJB];

    // MFMAs of slice h over the first NB row blocks (buffer h); rescale:
    // multiply each block by its row factors (from s_fac) just before its
    // first MFMA.  Reads of slice rs of (ra, rb) into the other buffer
    // (rs < 0: none) at the slots read_slot gives, DMA parts [d0, d1) of
    // step kd (kd < 0: none) spread over the slots.
    auto slice = [&](auto nbc, int h, bool rescale, const uint4* ra, const uint4* rb, int rs, int kd,
                     bool next, uint4* da, uint4* db, int d0, int d1, int dslot) __attribute__((always_inline)) {
      constexpr int NB = decltype(nbc)::value;
      constexpr int NQB = NB * RN, NRB = NB + RN;
      const int nd = d1 - d0;
      float f[16];
#pragma unroll
      for (int q = 0; q < NQB; ++q) {
        const int i = q / RN, j = q % RN;
        if (rescale) {
          if (j % NJW == 0) get_factors(i, j / NJW, f);
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] *= f[v];
        }
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[h][i], fb[h][j], acc[i][j], 0, 0, 0,
                                                                     0x7F7F7F7F, 0, 0x7F7F7F7F);
        // (an opaque use pins each MFMA to its slot: without it the compiler
        // gathers them, and the fragments of several slices stay live)
        asm volatile("" : "+v"(acc[i][j]));
        if (rs >= 0) {
#pragma unroll
          for (int fr = 0; fr < NRB; ++fr)
            if (read_slot(NB, fr) == q) read_frag(ra, rb, h ^ 1, rs, fr);
        }
        if (kd >= 0) {
#pragma unroll
          for (int t = 0; t < NDMA; ++t)
            if (t < nd && (t * NQB) / nd == q) dma_one(kd, next, da, db, d0 + t, dslot);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // (sbc: step kt's weight scales; sbn: step kt+1's, fetched at step kt's start)
    auto make_ratio = [&](int kt) __attribute__((always_inline)) {
      float fbj[NJB];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) fbj[jb] = uniform_f(sbc[jb] * __builtin_amdgcn_rcpf(sbn[jb]));
      const float a_cur = s_sc[slot_of(kt)][my_row];
      const float a_nxt = s_sc[slot_of(kt + 1)][my_row];
      put_factors(a_cur * __builtin_amdgcn_rcpf(a_nxt), fbj);
    };

    // Step kt of the main loop (kt + 2 < nsteps): slice 0 (rescaled for kt >
    // 0), barrier, slice 1 with the next step's first reads and DMA two steps
    // ahead.
    auto step = [&](auto nbc, int kt, uint4* sa, uint4* sb, uint4* na, uint4* nb_) __attribute__((always_inline)) {
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sbn[jb] = sb_load(cur, jb, kt + 1);
      slice(nbc, 0, kt > 0, sa, sb, 1, kt + 1, false, na, nb_, DHALF, NDMA, slot_of(kt + 1));
      __builtin_amdgcn_s_waitcnt(0xC07F);
      wait_vmcnt<0>();
      if (kt == 1) publish_ticket();
      barrier_only();
      if (kt == 0) ask_ticket();
      make_ratio(kt);
      slice(nbc, 1, false, na, nb_, 0, kt + 2, false, sa, sb, 0, DHALF, slot_of(kt + 2));
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sbc[jb] = sbn[jb];
    };
    // the last two steps (stages 0 and 1): the next tile is taken and its
    // first two steps are fetched
    auto tail = [&](auto nbc) __attribute__((always_inline)) {
      const int k0 = nsteps - 2, k1 = nsteps - 1;
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sbn[jb] = sb_load(cur, jb, k1);
      slice(nbc, 0, k0 > 0, sA0, sB0, 1, k1, false, sA1, sB1, DHALF, NDMA, slot_of(k1));
      __builtin_amdgcn_s_waitcnt(0xC07F);
      wait_vmcnt<0>();
      barrier_only();
      retarget();
      make_ratio(k0);
      slice(nbc, 1, false, sA1, sB1, 0, nx ? 0 : -1, true, sA0, sB0, 0, DHALF, slot_of(nsteps));
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sbc[jb] = sbn[jb];
      slice(nbc, 0, true, sA1, sB1, 1, nx ? 0 : -1, true, sA0, sB0, DHALF, NDMA, slot_of(nsteps));
      if (nx) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        wait_vmcnt<0>();
        barrier_only();
      }
      slice(nbc, 1, false, sA1, sB1, -1, nx ? 1 : -1, true, sA1, sB1, 0, DHALF, slot_of(nsteps + 1));
    };
    auto idle_dma = [&](int kd, bool next, uint4* da, uint4* db, int d0, int d1, int dslot) __attribute__((always_inline)) {
      if (kd >= 0) {
#pragma unroll
        for (int q = 0; q < NDMA; ++q)
          if (q >= d0 && q < d1) dma_one(kd, next, da, db, q, dslot);
      }
    };
    auto idle_step = [&](int kt, uint4* sa, uint4* sb, uint4* na, uint4* nb_) __attribute__((always_inline)) {
      idle_dma(kt + 1, false, na, nb_, DHALF, NDMA, slot_of(kt + 1));
      wait_vmcnt<0>();
      if (kt == 1) publish_ticket();
      barrier_only();
      if (kt == 0) ask_ticket();
      idle_dma(kt + 2, false, sa, sb, 0, DHALF, slot_of(kt + 2));
    };
    auto idle_tail = [&]() __attribute__((always_inline)) {
      idle_dma(nsteps - 1, false, sA1, sB1, DHALF, NDMA, slot_of(nsteps - 1));
      wait_vmcnt<0>();
      barrier_only();
      retarget();
      idle_dma(nx ? 0 : -1, true, sA0, sB0, 0, DHALF, slot_of(nsteps));
      idle_dma(nx ? 0 : -1, true, sA0, sB0, DHALF, NDMA, slot_of(nsteps));
      if (nx) {
        wait_vmcnt<0>();
        barrier_only();
      }
      idle_dma(nx ? 1 : -1, true, sA1, sB1, 0, DHALF, slot_of(nsteps + 1));
    };

    // Epilogue: the accumulators times the last step's scales.  Each wave
    // handles its own rows; SWIGLU needs one work-group barrier (the row
    // amax of a quantisation tile spans both feature waves), which every
    // wave joins, idle or not.
    char* const st = reinterpret_cast<char*>(s_stage) + wave * (SWI ? H_BYTES : ST_BYTES);
    auto silu_mul = [](float g, float u) __attribute__((always_inline)) {
      return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
    };
    auto epilogue = [&](int nb) __attribute__((always_inline)) {
      int ln = tid & 63;
      asm volatile("" : "+v"(ln));
      const int lr0 = 4 * (ln >> 5);
      const int last = nsteps - 1;
      // final factors: sa_last[row] * sb_last[jb]
      {
        float fbj[NJB];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) fbj[jb] = sbc[jb];
        put_factors(s_sc[slot_of(last)][my_row], fbj);
      }
      wave_lds_fence();
      float f[16];
      if (nb > 0) {
#pragma unroll
        for (int i = 0; i < RM; ++i) {
          if (i >= nb) continue;
#pragma unroll
          for (int j = 0; j < RN; ++j) {
            if (j % NJW == 0) get_factors(i, j / NJW, f);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] *= f[v];
          }
        }
      }
      if constexpr (SWI) {
        // h into the gate registers; this wave's half of each row's amax
#pragma unroll
        for (int i = 0; i < RM; ++i) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float m = 0.0f;
#pragma unroll
            for (int jj = 0; jj < RN / 2; ++jj) {
              const float hv = silu_mul(acc[i][jj][v], acc[i][jj + RN / 2][v]);
              acc[i][jj][v] = hv;
              m = fmaxf(m, fabsf(hv));
            }
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
            const int lr = i * HB + 32 * wm + 8 * (v >> 2) + lr0 + (v & 3);
            if ((ln & 31) == 0 && i < nb) s_amax[wn][lr] = m;
          }
        }
        barrier_only();
        const int64_t col0 = (int64_t)ti.n_tile * (BN / 2) + wn * (TN / 2);
#pragma unroll
        for (int i = 0; i < RM; ++i) {
          if (i >= nb) continue;
#pragma unroll
          for (int quad = 0; quad < 4; ++quad) {
            const int rb = i * HB + 32 * wm + 8 * quad;
            if (rb >= ti.rows) continue;
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
              const int v = 4 * quad + vv;
              const int lr = rb + lr0 + vv;
              float amax = s_amax[0][lr];
#pragma unroll
              for (int w = 1; w < WAVES_N; ++w) amax = fmaxf(amax, s_amax[w][lr]);
              const float sc = e4m3_tile_scale(amax);
#pragma unroll
              for (int jj = 0; jj < RN / 2; ++jj)
                reinterpret_cast<uint8_t*>(st + (lr0 + vv) * H_PITCH)[jj * 32 + (ln & 31)] =
                    static_cast<uint8_t>(f32_to_e4m3(acc[i][jj][v] / sc));
              if (wn == 0 && (ln & 31) == 0 && lr < ti.rows)
                p.C_scale[(int64_t)ti.n_tile * p.scale_ld + ti.row0 + lr] = sc;
            }
            wave_lds_fence();
            // 8 rows x 64 codes: 8 bytes per lane
            const int r = ln >> 3, c = ln & 7;
            if (rb + r < ti.rows) {
              const uint2 val = *reinterpret_cast<const uint2*>(st + r * H_PITCH + c * 8);
              *reinterpret_cast<uint2*>(static_cast<uint8_t*>(p.C) + ((int64_t)ti.row0 + rb + r) * p.ldc +
                                        col0 + c * 8) = val;
            }
            wave_lds_fence();
          }
        }
      } else {
        const int64_t col0 = (int64_t)ti.n_tile * BN + wn * TN;
        auto put2 = [&](int lr, int col, uint32_t pk) __attribute__((always_inline)) {
          reinterpret_cast<uint16_t*>(st + lr * ST_PITCH)[col] = static_cast<uint16_t>(pk);
          reinterpret_cast<uint16_t*>(st + (lr + 1) * ST_PITCH)[col] = static_cast<uint16_t>(pk >> 16);
        };
#pragma unroll
        for (int i = 0; i < RM; ++i) {
          if (i >= nb) continue;
#pragma unroll
          for (int quad = 0; quad < 4; ++quad) {
            const int rb = i * HB + 32 * wm + 8 * quad;
            if (rb >= ti.rows) continue;
#pragma unroll
            for (int v = 4 * quad; v < 4 * quad + 4; v += 2) {
              const int lr = lr0 + (v & 3);
#pragma unroll
              for (int j = 0; j < RN; ++j)
                put2(lr, j * 32 + (ln & 31), pack_bf16x2(acc[i][j][v], acc[i][j][v + 1]));
            }
            wave_lds_fence();
            // 8 rows x 128 bf16: two 16-byte chunks per lane
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int q = ln + 64 * hh;
              const int r = q >> 4, c = q & 15;
              if (rb + r < ti.rows) {
                const uint4 val = *reinterpret_cast<const uint4*>(st + r * ST_PITCH + c * 16);
                *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.C) + ((int64_t)ti.row0 + rb + r) * p.ldc +
                                          col0 + c * 8) = val;
              }
            }
            wave_lds_fence();
          }
        }
      }
    };

    // prologue of the first tile: all of step 0, the first half of step 1
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) sbc[jb] = sb_load(cur, jb, 0);
#pragma unroll
    for (int q = 0; q < NDMA; ++q) dma_one(0, false, sA0, sB0, q, slot_of(0));
#pragma unroll
    for (int q = 0; q < DHALF; ++q) dma_one(1, false, sA1, sB1, q, slot_of(1));
    wait_vmcnt<0>();
    barrier_only();

    for (;;) {
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
        for (int fr = 0; fr < RM + RN; ++fr) read_frag(sA0, sB0, 0, 0, fr);
        for (int kt = 0; kt < nsteps - 2; kt += 2) {
          step(NBC{}, kt, sA0, sB0, sA1, sB1);
          step(NBC{}, kt + 1, sA1, sB1, sA0, sB0);
        }
        tail(NBC{});
      } else if (nb == 1) {
        using NBC = std::integral_constant<int, 1>;
#pragma unroll
        for (int fr = 0; fr <= RN; ++fr) read_frag(sA0, sB0, 0, 0, fr);
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
      sc_base = (sc_base + nsteps) & (SC_SLOTS - 1);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) sbc[jb] = sb_load(cur, jb, 0);
    }
  }
  if (tid == 0) {
    if (atomicAdd(&tickets[kXcds * kCtrStride], 1) == (int)gridDim.x - 1) {
#pragma unroll
      for (int x = 0; x <= kXcds; ++x) atomicExch(&tickets[x * kCtrStride], 0);
    }
  }
#endif
}

template <int MODE>
hipError_t launch(Fp8Args& a, int64_t max_rows, hipStream_t s) {
  if (!ffn_fp8p_supported_k(a.K)) return hipErrorInvalidValue;
  const int64_t b_rows = MODE == MODE_STORE ? (int64_t)a.n_tiles * BN : 2 * (int64_t)a.d_ff;
  if ((int64_t)BM * a.lda >= (1LL << 31) || b_rows * a.K >= (1LL << 31)) return hipErrorInvalidValue;
  const int64_t mt = max_row_tiles(max_rows, a.offsets == nullptr ? 1 : a.n_exp, BM);
  const int64_t tiles = mt * a.n_tiles;
  if (tiles <= 0) return hipSuccess;
  const int64_t grid = (std::min<int64_t>(tiles, stream_cu_count(s)) + kXcds - 1) / kXcds * kXcds;
  if (a.tickets == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL((ffn_fp8_kernel<MODE>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool ffn_fp8p_supported_k(int K) { return K % (2 * BKB) == 0 && K >= 4 * BKB; }

hipError_t launch_ffn_up_fp8p(int n_exp, const int32_t* offsets, int64_t max_rows, int d, int d_ff,
                              const uint8_t* xp, const float* xp_scale, const uint8_t* w13,
                              const float* w13_scale, uint8_t* h, float* h_scale, int* tickets,
                              hipStream_t s) {
  Fp8Args a{};
  a.tickets = tickets;
  a.A = xp;
  a.A_scale = xp_scale;
  a.lda = d;
  a.B = w13;
  a.B_scale = w13_scale;
  a.b_group_stride = (int64_t)2 * d_ff * d;
  a.bs_group_stride = (int64_t)(2 * d_ff / BKB) * (d / BKB);
  a.C = h;
  a.C_scale = h_scale;
  a.scale_ld = max_rows;
  a.ldc = d_ff;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.K = d;
  a.n_tiles = d_ff / (BN / 2);
  a.d_ff = d_ff;
  return launch<MODE_SWIGLU>(a, max_rows, s);
}

hipError_t launch_ffn_down_fp8p(int n_exp, const int32_t* offsets, int64_t max_rows, int d, int d_ff,
                                const uint8_t* h, const float* h_scale, const uint8_t* w2,
                                const float* w2_scale, uint16_t* yp, int* tickets, hipStream_t s) {
  Fp8Args a{};
  a.tickets = tickets;
  a.A = h;
  a.A_scale = h_scale;
  a.lda = d_ff;
  a.B = w2;
  a.B_scale = w2_scale;
  a.b_group_stride = (int64_t)d * d_ff;
  a.bs_group_stride = (int64_t)(d / BKB) * (d_ff / BKB);
  a.C = yp;
  a.scale_ld = max_rows;
  a.ldc = d;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = max_rows;
  a.K = d_ff;
  a.n_tiles = d / BN;
  return launch<MODE_STORE>(a, max_rows, s);
}

}  // namespace moe
