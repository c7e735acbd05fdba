// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;  // per moe_expert_ffn call
constexpr int kXcds = 8;           // MI355X: 8 accelerator complex dies, 32 CUs each

// Ticket counters of one persistent grouped-GEMM launch: one tile counter per
// XCD and a retire counter, each on its own 64-byte line, in caller-owned
// device memory.  They must be zero when the launch starts; the last
// work-group to retire sets them back to zero, so a set can serve the next
// launch on the same stream.  Launches that may run at the same time need
// distinct sets.
constexpr int kTicketStride = 16;  // ints between counters
constexpr int kTicketInts = (kXcds + 1) * kTicketStride;
constexpr size_t kTicketBytes = kTicketInts * sizeof(int);

// the router gate product runs as at most this many split-K partial products
constexpr int kMaxGateSplits = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// round to nearest, ties to even (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two values rounded to nearest even in one v_cvt_pk_bf16_f32 (lo in bits
// 0-15); the same bits as f32_to_bf16 for finite inputs
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---------------------------------------------------------------- e4m3 (OCP E4M3FN)

// Nearest e4m3 value, ties to the even code, saturating at +-448.  The sign
// bit follows the input's sign (small negatives give -0, code 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x43E00000u) {                     // |v| > 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {              // |v| < 2^-6: subnormal step 2^-9
    float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
    code = static_cast<uint32_t>(q);         // 0..8 (8 = 2^-6, the first normal)
  } else {
    int e = static_cast<int>(a >> 23) - 127;  // -6..8
    uint32_t frac = a & 0x7FFFFFu;
    uint32_t q = frac >> 20;
    uint32_t rem = frac & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1u;
    code = (static_cast<uint32_t>(e + 7) << 3) + q;  // a carry moves to the next binade
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0 ? static_cast<float>(m) * 0.001953125f
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// fp32 scale of an e4m3 tile from its largest magnitude
__device__ __forceinline__ float e4m3_tile_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}

// ---------------------------------------------------------------- streaming accesses
// 16-byte loads/stores marked nontemporal: data read or written once per pass
// streams through the caches instead of displacing reused lines.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, static_cast<u32x4*>(p));
}

// ---------------------------------------------------------------- grouped tile map
//
// A grouped GEMM launch covers n_exp row groups (experts): group i owns rows
// [offsets[i], offsets[i+1]).  Each group is cut into ceil(rows/BM) row tiles;
// each row tile meets n_tiles column tiles.  Logical tiles are numbered group by
// group; inside a group the row tiles form bands of kBandRows, and inside a
// band the numbering is column-tile-major with the band's row tiles innermost.
// The 32 tiles an XCD runs at once then cover about 4 row tiles x 8 column
// tiles: each activation tile is shared by ~8 running tiles and each weight
// tile by ~4 (a routed expert of at most 4 row tiles is one band).
// Work-group w is remapped so that each XCD (w % 8) walks one contiguous slice
// of the logical tiles: the tiles that share weights and activations then sit in
// one XCD's L2.  Offsets live on the device; the map is rebuilt by every
// work-group from them (a few hundred ints), so no host sync and no planning
// kernel are needed.

constexpr int kBandRows = 4;  // row tiles per band of the tile order

struct TileInfo {
  int group;    // expert within the call
  int m_tile;   // row tile within the group
  int n_tile;   // column tile
  int row0;     // first row of the tile
  int rows;     // valid rows in the tile (1..BM)
};

// s_pre: LDS scratch of kMapInts ints: the groups' row-tile prefix (up to
// kMaxExperts + 2 ints: the groups of the offsets and one extra group), then
// a copy of the row offsets at s_pre + kMapStride.
constexpr int kMapStride = kMaxExperts + 2;
constexpr int kMapInts = 2 * kMapStride;

__device__ __forceinline__ const int* tile_map_offsets(const int* s_pre) { return s_pre + kMapStride; }

// Builds the map in s_pre (ends with a work-group barrier); returns the number
// of groups (1 when offsets is nullptr: one group of rows_total rows).  With
// extra_rows > 0 (and offsets given) one more group of that many rows follows
// the n_exp groups: its rows are numbered on from offsets[n_exp].  Must be
// called by all threads.
__device__ __forceinline__ int tile_map_build(const int* __restrict__ offsets, int n_exp,
                                              int64_t rows_total, int BM, int* s_pre,
                                              int64_t extra_rows = 0) {
  const int tid = threadIdx.x;
  int* const s_off = s_pre + kMapStride;
  if (offsets == nullptr) {
    n_exp = 1;
    if (tid == 0) {
      s_pre[0] = 0;
      s_pre[1] = static_cast<int>((rows_total + BM - 1) / BM);
      s_off[0] = 0;
      s_off[1] = static_cast<int>(rows_total);
    }
  } else {
    // one global round trip: every thread copies offsets into LDS, then wave 0
    // scans per-lane chunks of consecutive groups
    for (int g = tid; g <= n_exp; g += blockDim.x) s_off[g] = offsets[g];
    __syncthreads();
    if (tid < kWave) {
      const int per = (n_exp + kWave - 1) / kWave;
      const int g0 = tid * per;
      int sum = 0;
      for (int g = g0; g < g0 + per && g < n_exp; ++g) sum += (s_off[g + 1] - s_off[g] + BM - 1) / BM;
      int incl = sum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        int v = __shfl_up(incl, o, kWave);
        if (tid >= o) incl += v;
      }
      int run = incl - sum;
      if (tid == 0) s_pre[0] = 0;
      for (int g = g0; g < g0 + per && g < n_exp; ++g) {
        run += (s_off[g + 1] - s_off[g] + BM - 1) / BM;
        s_pre[g + 1] = run;
      }
    }
  }
  __syncthreads();
  if (offsets != nullptr && extra_rows > 0) {
    if (tid == 0) {
      s_off[n_exp + 1] = s_off[n_exp] + static_cast<int>(extra_rows);
      s_pre[n_exp + 1] = s_pre[n_exp] + static_cast<int>((extra_rows + BM - 1) / BM);
    }
    __syncthreads();
    return n_exp + 1;
  }
  return n_exp;
}

// Logical tile L (< s_pre[n_grp] * n_tiles) of a built map.  g_lo is a group
// with s_pre[g_lo] * n_tiles <= L (0 when nothing better is known).
__device__ __forceinline__ void tile_map_decode(int L, int n_grp, int BM, int n_tiles,
                                                const int* s_pre, int g_lo, TileInfo& ti) {
  const int* const s_off = s_pre + kMapStride;
  int g = g_lo;
  if (s_pre[g + 1] * n_tiles <= L) {
    int lo = g + 1, hi = n_grp;  // invariant: s_pre[lo]*nt <= L < s_pre[hi]*nt
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] * n_tiles <= L) lo = mid; else hi = mid;
    }
    g = lo;
  }
  const int mt = s_pre[g + 1] - s_pre[g];
  const int i = L - s_pre[g] * n_tiles;
  ti.group = g;
  const int band = i / (kBandRows * n_tiles);
  const int bm = min(kBandRows, mt - band * kBandRows);  // row tiles in this band
  const int ib = i - band * kBandRows * n_tiles;
  ti.n_tile = ib / bm;
  ti.m_tile = band * kBandRows + ib % bm;
  ti.row0 = s_off[g] + ti.m_tile * BM;
  ti.rows = min(BM, s_off[g + 1] - ti.row0);
}

// The tile of work-group blockIdx.x, for one-tile-per-work-group launches.
// Returns false for a work-group with no tile (uniform across the work-group).
// Must be called by all threads.
__device__ __forceinline__ bool map_tile(const int* __restrict__ offsets, int n_exp,
                                         int64_t rows_total, int BM, int n_tiles, int* s_pre,
                                         TileInfo& ti) {
  const int n_grp = tile_map_build(offsets, n_exp, rows_total, BM, s_pre);
  const int total = s_pre[n_grp] * n_tiles;
  const int rr = (total + kXcds - 1) / kXcds * kXcds;
  const int w = blockIdx.x;
  if (w >= rr) return false;
  const int L = (w % kXcds) * (rr / kXcds) + w / kXcds;
  if (L >= total) return false;
  tile_map_decode(L, n_grp, BM, n_tiles, s_pre, 0, ti);
  return true;
}

// Persistent launches deal the logical tiles to the XCDs in chunks of ch
// tiles, round robin: the i-th ticket of XCD x is tile
// ((i / ch) * kXcds + x) * ch + i % ch.  A chunk is one XCD's worth of
// concurrently running tiles (its work-groups: 32 on a whole MI355X, fewer on
// a stream whose CU mask keeps some CUs for other work), which share weight
// and activation tiles in its L2; dealing whole chunks round robin spreads
// every part of the tile order (e.g. a trailing dense group) over all XCDs.
// A launch of fewer tiles uses ch = ceil(total / kXcds), one chunk per XCD.
__device__ __forceinline__ int xcd_chunk(int total) {
  return max(1, min(static_cast<int>(gridDim.x) / kXcds, (total + kXcds - 1) / kXcds));
}
__device__ __forceinline__ int xcd_tile(int i, int xcd, int ch) {
  return ((i / ch) * kXcds + xcd) * ch + i % ch;
}

// upper bound on the row tiles of a grouped launch (plus an extra group of
// extra_rows rows)
inline int64_t max_row_tiles(int64_t max_rows, int n_exp, int BM, int64_t extra_rows = 0) {
  return (max_rows + BM - 1) / BM + (n_exp > 1 ? n_exp : 0) + (extra_rows + BM - 1) / BM;
}

}  // namespace moe
