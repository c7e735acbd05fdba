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
#include <algorithm>
#include <type_traits>

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
constexpr int HB = BM / RM;  // DGRAD: row distance between a wave's two 32-row blocks
constexpr int NS = BK / 16, NQ = RM * RN;
constexpr int KROW_BYTES = 512;          // K-major LDS row: 256 bf16
constexpr int DPW = 4;                   // DMA instructions per operand per wave per step
constexpr int NDMA = 2 * DPW;
constexpr int DHALF = NDMA / 2;

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
  const int* offsets;      // [n_exp + 1] on the device, or nullptr: WGRAD groups of
  int n_exp;               // split_rows consecutive rows (the last one shorter)
  int64_t rows_total;
  int split_rows;
  int K;                   // DGRAD: reduction length
  int m_tiles, n_tiles;    // WGRAD: tiles per group (DGRAD: n_tiles only)
};

__global__ __launch_bounds__(kThreads, 1) void ffn_dgrad_kernel(const BwdArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int STAGE = 2 * 32 * 1024 / 16;  // uint4: A 32 KB + B 32 KB
  constexpr int OUT_PITCH = BN * 2 + 16;      // bf16 staging row
  constexpr int OUT_U4 = BM * OUT_PITCH / 16;
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
  TileInfo ti;
  if (!map_tile(p.offsets, p.n_exp, p.rows_total, BM, p.n_tiles, s_pre, ti)) return;
  const int group = __builtin_amdgcn_readfirstlane(ti.group);
  const int n_tile = __builtin_amdgcn_readfirstlane(ti.n_tile);
  const int row0 = __builtin_amdgcn_readfirstlane(ti.row0);
  const int rows = __builtin_amdgcn_readfirstlane(ti.rows);  // valid rows of the tile
  // valid 32-row blocks of this wave: block i covers rows i*HB + 32*wm + [0, 32),
  // so the two waves sharing a SIMD (wm and wm + 2) hold blocks in every 64-row
  // band and a ragged tile costs its rows rounded up to 64; a block past the
  // valid rows skips its MFMAs and fragment reads
  const int nb = __builtin_amdgcn_readfirstlane((rows > 32 * wm) + (rows > HB + 32 * wm));
  const int nsteps = p.K / BK;

  // ---- DMA sources.  Row-major A: blocks of 8 rows x 128 B, chunk swizzle
  // (r >> 1) & 7 applied to the global address; rows past the valid ones
  // read the last valid row.  K-major W: blocks of 2 rows x 512 B; lane l
  // fills row 2b + l/32, physical chunk l%32, logical chunk (l%32) ^ (4*(k&3)).
  const char* a_src[DPW];
  const char* b_src[DPW];
  const int kr_lane = lane >> 5;                       // row within a K-major block
  const int kr_chunk = (lane & 31) ^ (4 * ((2 * (wave & 1) + kr_lane) & 3));
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int blk = wave + NW * i;
    const int r = blk * 8 + (lane >> 3);
    const int rc = r < rows ? r : rows - 1;
    const int lch = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    a_src[i] = reinterpret_cast<const char*>(p.A + (int64_t)(row0 + rc) * p.lda + lch * 8);
    // W rows k = 2*blk + kr_lane of the step, columns of the n tile
    b_src[i] = reinterpret_cast<const char*>(p.B + (int64_t)group * p.b_group_stride +
                                             (int64_t)(2 * blk + kr_lane) * p.ldb + n_tile * BN + kr_chunk * 8);
  }

  // DMA part q (< DPW: A, else B) of step kt into stage (sa, sb)
  auto dma_one = [&](int kt, char* sa, char* sb, int q) __attribute__((always_inline)) {
    const int i = q < DPW ? q : q - DPW;
    const int blk = wave + NW * i;
    if (q < DPW) {
      if (kt < 2 || blk * 8 < rows)
        dma16(a_src[i] + (int64_t)kt * BK * 2, lds_addr(sa) + blk * 1024);
    } else {
      dma16(b_src[i] + (int64_t)kt * BK * p.ldb * 2, lds_addr(sb) + blk * 1024);
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
      const uint4* s = reinterpret_cast<const uint4*>(sa);
      fa[buf][idx] = as_bf16x8(s[swz(idx * HB + 32 * wm + (lane & 31), 2 * s16 + (lane >> 5))]);
    } else {
      fb[buf][idx] = kmajor_frag(sb, wn * TN + idx * 32, s16);
    }
  };
  static_assert(RM + RN <= NQ, "one read per MFMA slot");
  // MFMAs of slice s over the first NB row blocks; with one block there are
  // five reads for four MFMA slots: the first slot takes two
  auto slice = [&](auto nbc, int s, const char* rsa, const char* rsb, int rs, int kd, char* da, char* db, int d0,
                   int d1) __attribute__((always_inline)) {
    constexpr int NB = decltype(nbc)::value;
    constexpr int NQB = NB * RN, NRB = NB + RN;
    constexpr int XR = NRB > NQB ? NRB - NQB : 0;
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
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](auto nbc, int kt, char* sa, char* sb, char* na, char* nb_) __attribute__((always_inline)) {
    const bool more = kt + 1 < nsteps;
    slice(nbc, 0, sa, sb, 1, (kt >= 1 && more) ? kt + 1 : -1, na, nb_, DHALF, NDMA);
#pragma unroll
    for (int s = 1; s + 1 < NS; ++s) slice(nbc, s, sa, sb, s + 1, -1, nullptr, nullptr, 0, 0);
    if (more) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      wait_vmcnt<0>();
      barrier_only();
    }
    slice(nbc, NS - 1, more ? na : nullptr, nb_, 0, kt + 2 < nsteps ? kt + 2 : -1, sa, sb, 0, DHALF);
  };
  auto idle_step = [&](int kt, char* sa, char* sb, char* na, char* nb_) __attribute__((always_inline)) {
    const bool more = kt + 1 < nsteps;
    if (kt >= 1 && more) {
#pragma unroll
      for (int q = DHALF; q < NDMA; ++q) dma_one(kt + 1, na, nb_, q);
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
    if (nb == RM) {
      using NBC = std::integral_constant<int, RM>;
#pragma unroll
      for (int f = 0; f < RM + RN; ++f) read_frag(sA0, sB0, 0, 0, f);
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
  }

  // ---- epilogue.  Accumulator (i, j) register v holds row 8*(v/4) +
  // 4*(lane/32) + v%4 and column lane%32 of its 32x32 block.
  barrier_only();
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    if (i >= nb) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int lr = i * HB + 32 * wm + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
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
#endif
}

// WGRAD, persistent: one work-group per CU walks a static list of tiles
// (those of its XCD's contiguous range, every (grid / 8)-th), and its K steps
// form one stream across tiles: the DMA two steps ahead and the fragment reads
// one slice ahead run on into the next tile, so a tile (an expert's ~8 steps
// on V3) starts without a pipeline fill.  Between tiles the accumulators are
// stored straight from registers and cleared.  A tile of an expert with no
// rows runs one step over the zero row and stores zeros.  Past the end of
// the stream the DMA and fragment reads keep going, on the zero row and on
// stale LDS, so no MFMA slot holds a branch.
struct WgradCursor {
  const char* a;  // A bytes of the step's first K row, the tile's columns
  const char* b;  // the same for B
  int valid, group, m_tile, n_tile, rows, ns, s, lim;  // lim: valid K rows from the step's first
};

__global__ __launch_bounds__(kThreads, 1) void ffn_wgrad_kernel(const BwdArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  // stages as [A0 | A1 | B0 | B1] (32 KB each): every fragment read is a
  // per-lane base plus an immediate offset below 64 KB
  __shared__ uint4 smem[4 * 32 * 1024 / 16];
  char* const base = reinterpret_cast<char*>(smem);
  char* const sA0 = base;
  char* const sA1 = base + 32 * 1024;
  char* const sB0 = base + 64 * 1024;
  char* const sB1 = base + 96 * 1024;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // this work-group's tiles: L = begin + j + i * gpx within [begin, end)
  const int per = p.m_tiles * p.n_tiles;
  const int total = p.n_exp * per;
  const int gpx = static_cast<int>(gridDim.x) / kXcds;
  const int xcd = blockIdx.x % kXcds, j0 = blockIdx.x / kXcds;
  const int per_x = (total + kXcds - 1) / kXcds;
  const int l_end = min(total, (xcd + 1) * per_x);
  int l_next = xcd * per_x + j0;  // next tile of the list to open
  const int64_t a_step = (int64_t)BK * p.lda * 2, b_step = (int64_t)BK * p.ldb * 2;
  auto open_tile = [&](WgradCursor& c) __attribute__((always_inline)) {
    const int L = l_next;
    l_next += gpx;
    c.valid = L < l_end;
    if (!c.valid) {
      c.lim = 0;
      return;
    }
    c.group = L / per;
    const int rem = L % per;
    c.m_tile = rem / p.n_tiles;
    c.n_tile = rem % p.n_tiles;
    int row0;
    if (p.offsets == nullptr) {
      row0 = c.group * p.split_rows;
      c.rows = static_cast<int>(min((int64_t)p.split_rows, p.rows_total - row0));
    } else {
      row0 = __builtin_amdgcn_readfirstlane(p.offsets[c.group]);
      c.rows = __builtin_amdgcn_readfirstlane(p.offsets[c.group + 1]) - row0;
    }
    c.ns = max(1, (c.rows + BK - 1) / BK);
    c.s = 0;
    c.lim = c.rows;
    c.a = reinterpret_cast<const char*>(p.A + (int64_t)row0 * p.lda + (int64_t)c.m_tile * BM);
    c.b = reinterpret_cast<const char*>(p.B + (int64_t)row0 * p.ldb + (int64_t)c.n_tile * BN);
  };
  auto advance = [&](WgradCursor& c) __attribute__((always_inline)) {
    if (!c.valid) return;
    if (++c.s == c.ns) {
      open_tile(c);
    } else {
      c.lim -= BK;
      c.a += a_step;
      c.b += b_step;
    }
  };

  // DMA: K-major operand blocks of 2 rows x 512 B; lane l fills K row
  // 2 * blk + l / 32 of the step, physical chunk l % 32, logical chunk
  // (l % 32) ^ (4 * (k & 3)).  Rows past the group read the zero row.
  int k_row[DPW];
  uint32_t a_off[DPW], b_off[DPW];
  const int kr_lane = lane >> 5;
  const int kr_chunk = (lane & 31) ^ (4 * ((2 * (wave & 1) + kr_lane) & 3));
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    k_row[i] = 2 * (wave + NW * i) + kr_lane;
    a_off[i] = static_cast<uint32_t>(k_row[i] * p.lda * 2 + kr_chunk * 16);
    b_off[i] = static_cast<uint32_t>(k_row[i] * p.ldb * 2 + kr_chunk * 16);
  }
  const char* zrow = reinterpret_cast<const char*>(g_zero_row) + kr_chunk * 16;
  auto dma_one = [&](const WgradCursor& c, char* sa, char* sb, int q) __attribute__((always_inline)) {
    const int i = q < DPW ? q : q - DPW;
    const int blk = wave + NW * i;
    const bool in = k_row[i] < c.lim;
    if (q < DPW) dma16(in ? c.a + a_off[i] : zrow, lds_addr(sa) + blk * 1024);
    else dma16(in ? c.b + b_off[i] : zrow, lds_addr(sb) + blk * 1024);
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragment of 32 columns from col0 for K16 slice s16 of a K-major stage:
  // lane reads (transposing) 4 columns of K row k0 = 16 s16 + 8 (lane / 32)
  // + r, r = (lane % 16) / 4, and of row k0 + 4; the chunk XOR 4 (k & 3) is
  // 4 r for both, so a fragment is a per-lane offset plus immediates
  const int tr_a = lane & 15;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (tr_a & 3);
  const int tr_row = tr_a >> 2;
  auto frag_off = [&](int col0) __attribute__((always_inline)) {
    const int n = col0 + tr_col;
    const int k0 = 8 * (lane >> 5) + tr_row;
    return k0 * KROW_BYTES + (((n >> 3) ^ (4 * tr_row)) << 4) + (n & 7) * 2;
  };
  int fo_a[RM], fo_b[RN];
#pragma unroll
  for (int i = 0; i < RM; ++i) fo_a[i] = frag_off(wm * TM + i * 32);
#pragma unroll
  for (int j = 0; j < RN; ++j) fo_b[j] = frag_off(wn * TN + j * 32);
  auto kmajor_frag = [&](const char* st, int off, int s16) __attribute__((always_inline)) {
    const char* q = st + off + s16 * 16 * KROW_BYTES;
    const v4i16 lo = lds_tr16(q);
    const v4i16 hi = lds_tr16(q + 4 * KROW_BYTES);
    const v4i16 v[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, v);
  };
  bf16x8 fa[2][RM], fb[2][RN];
  auto read_frag = [&](const char* sa, const char* sb, int buf, int s16, int f) __attribute__((always_inline)) {
    // order of first use: a0, b0 .. b(RN-1), a1 .. a(RM-1)
    const bool is_a = f == 0 || f > RN;
    const int idx = f == 0 ? 0 : (f <= RN ? f - 1 : f - RN);
    if (is_a) fa[buf][idx] = kmajor_frag(sa, fo_a[idx], s16);
    else fb[buf][idx] = kmajor_frag(sb, fo_b[idx], s16);
  };
  constexpr int NR = RM + RN;
  // MFMAs of slice s (buffer s & 1); reads of slice rs of (rsa, rsb) into the
  // other buffer; DMA parts [d0, d1) of cursor dc (dc == nullptr: none)
  auto slice = [&](int s, const char* rsa, const char* rsb, int rs, const WgradCursor* dc, char* da, char* db,
                   int d0, int d1) __attribute__((always_inline)) {
    const int buf = s & 1;
    const int nd = d1 - d0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = q / RN, j = q % RN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
      asm volatile("" : "+v"(acc[i][j]));  // keeps the MFMA in its slot
      if (q < NR) read_frag(rsa, rsb, buf ^ 1, rs, q);
      if (dc != nullptr) {
#pragma unroll
        for (int t = 0; t < NDMA; ++t)
          if (t < nd && (t * NQ) / nd == q) dma_one(*dc, da, db, d0 + t);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // fp32 tile store (nontemporal: nothing here reads it again), then clear
  auto epilogue = [&](const WgradCursor& c) __attribute__((always_inline)) {
    float* C = static_cast<float*>(p.C) + (int64_t)c.group * p.c_group_stride;
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = c.m_tile * BM + wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
#pragma unroll
        for (int j = 0; j < RN; ++j) {
          __builtin_nontemporal_store(acc[i][j][v],
                                      &C[(int64_t)m * p.ldc + c.n_tile * BN + wn * TN + j * 32 + (lane & 31)]);
          acc[i][j][v] = 0.0f;
        }
      }
  };

  // cur: the step being multiplied; c1, c2: the next two steps of the stream
  WgradCursor cur, c1, c2;
  open_tile(cur);
  if (cur.valid) {
    c1 = cur;
    advance(c1);
    c2 = c1;
    advance(c2);
#pragma unroll
    for (int q = 0; q < NDMA; ++q) dma_one(cur, sA0, sB0, q);
#pragma unroll
    for (int q = 0; q < NDMA; ++q) dma_one(c1, sA1, sB1, q);
    wait_vmcnt<NDMA>();
    barrier_only();
#pragma unroll
    for (int f = 0; f < NR; ++f) read_frag(sA0, sB0, 0, 0, f);
    // one step of the stream from stage (sa, sb), next stage (na, nb); first:
    // the stream's first step (its successor's DMA went out whole)
    auto step = [&](bool first, char* sa, char* sb, char* na, char* nb) __attribute__((always_inline)) {
      slice(0, sa, sb, 1, first ? nullptr : &c1, na, nb, DHALF, NDMA);
#pragma unroll
      for (int s = 1; s + 1 < NS; ++s) slice(s, sa, sb, s + 1, nullptr, nullptr, nullptr, 0, 0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      wait_vmcnt<0>();
      barrier_only();
      slice(NS - 1, na, nb, 0, &c2, sa, sb, 0, DHALF);
      if (cur.s == cur.ns - 1) epilogue(cur);
      cur = c1;
      c1 = c2;
      advance(c2);
    };
    step(true, sA0, sB0, sA1, sB1);
    while (cur.valid) {
      step(false, sA1, sB1, sA0, sB0);
      if (!cur.valid) break;
      step(false, sA0, sB0, sA1, sB1);
    }
    wait_vmcnt<0>();  // the zero-row DMA issued past the stream's end
  }
#endif
}

hipError_t launch_dgrad(const BwdArgs& a, int64_t tiles, hipStream_t s) {
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(ffn_dgrad_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
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
  return launch_dgrad(a, mt * a.n_tiles, s);
}

// C_g [M, N] fp32 = sum over the group's rows r of A[r][m] * B[r][n]
hipError_t launch_ffn_wgrad_bf16(int n_exp, const int32_t* offsets, int64_t rows_total, int M, int N,
                                 const uint16_t* A, const uint16_t* B, float* C, hipStream_t s, int split_rows) {
  if (offsets == nullptr) {
    // groups of split_rows consecutive rows (all rows when split_rows <= 0)
    const int64_t sr = split_rows > 0 && split_rows < rows_total ? split_rows : std::max<int64_t>(rows_total, 1);
    if (sr >= (1LL << 31)) return hipErrorInvalidValue;
    split_rows = static_cast<int>(sr);
    n_exp = static_cast<int>(std::max<int64_t>((rows_total + sr - 1) / sr, 1));
  }
  BwdArgs a{};
  a.A = A;
  a.lda = M;
  a.B = B;
  a.ldb = N;
  a.C = C;
  a.ldc = N;
  a.c_group_stride = (int64_t)M * N;
  a.offsets = offsets;
  a.n_exp = n_exp;
  a.rows_total = rows_total;
  a.split_rows = split_rows;
  a.m_tiles = M / BM;
  a.n_tiles = N / BN;
  const int64_t tiles = (int64_t)a.n_exp * a.m_tiles * a.n_tiles;
  if (tiles <= 0) return hipSuccess;
  // tile numbers and the 32-bit per-lane DMA offsets (64 K rows of A and B)
  if (tiles >= (1LL << 31) || (int64_t)BK * std::max(M, N) * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  const int64_t grid = (std::min<int64_t>(tiles, stream_cu_count(s)) + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(ffn_wgrad_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
