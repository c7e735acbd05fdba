// Routing on gfx950: affinities, bias-adjusted node-limited top-k, gate
// weights and the per-block expert histogram (mastering-deepseek-v4 "MoE +
// Expert-Parallel Overlap (Exp08)", Implemented: Sqrt(Softplus) affinities,
// top-k gating, per-expert bias; zenaique "MoE node-limited routing": a
// token's experts span at most M nodes).
//
// One wave64 per token.  Lane l holds experts [l*EPL, (l+1)*EPL) (EPL =
// ceil(E/64)), so a group of E/G consecutive experts is an aligned run of
// lanes and group reductions are xor-butterflies inside the run.  Orderings use
// 64-bit keys (ordered fp32 bits << 32 | ~index): the largest key is the
// largest value, ties to the lower index.
//
// Every floating-point value is produced by one fixed operation sequence with
// no contraction (this file is compiled with -ffp-contract=off, correctly
// rounded divide and sqrt, and fp32 denormals kept), so the result is a
// deterministic function of the fp32 logits:
//   s = sqrt(softplus(l)) by the fixed fp64 sequence in affinity.h, rounded
//       once to fp32 (non-decreasing in l, like the exact function)
//   b = s + bias
//   group score = its group_topk largest b added largest first;
//   keep the M best groups (ties to the lower group), choose the k best b in
//   them (ties to the lower expert), w_j = s_j / (((s_0 + s_1) + s_2) + ...).
#pragma clang fp contract(off)

#include "affinity.h"
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

using aff::affinity_spec;

__device__ __forceinline__ uint64_t make_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(idx));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = static_cast<uint32_t>(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_index(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// ---------------------------------------------------------------- lane exchanges
// A max over aligned groups of 2^s lanes is built stage by stage: once every
// lane of each 2^(s-1)-lane group holds its group's max, any exchange that
// pairs each such group with its partner group finishes the next stage.
// Inside a 16-lane row the exchanges are DPP moves (quad permutes, then the
// 8- and 16-lane mirrors); across rows they are gfx950's row swaps (16 and
// 32 lanes).  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(v), CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(v >> 32), CTRL, 0xF, 0xF, false);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// max of v and the value of the lane 16 (ROW32: 32) lanes away
template <bool ROW32>
__device__ __forceinline__ uint64_t row_swap_max_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  uint32_t l0, l1, h0, h1;
  if constexpr (ROW32) {
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    l0 = l[0]; l1 = l[1]; h0 = h[0]; h1 = h[1];
  } else {
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    l0 = l[0]; l1 = l[1]; h0 = h[0]; h1 = h[1];
  }
  // one of the two halves is the lane's own value, the other its partner's
  return umax64((static_cast<uint64_t>(h0) << 32) | l0, (static_cast<uint64_t>(h1) << 32) | l1);
}

// max over aligned groups of `width` lanes (a power of two, 1..64), in every lane
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v, int width) {
  if (width >= 2) v = umax64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
  if (width >= 4) v = umax64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
  if (width >= 8) v = umax64(v, dpp_u64<0x141>(v));  // row_half_mirror
  if (width >= 16) v = umax64(v, dpp_u64<0x140>(v)); // row_mirror
  if (width >= 32) v = row_swap_max_u64<false>(v);
  if (width >= 64) v = row_swap_max_u64<true>(v);
  return v;
}

__device__ __forceinline__ float lane_value(float v, int lane_uniform) {
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), __builtin_amdgcn_readfirstlane(lane_uniform)));
}

constexpr int kTokPerBlock = MOE_ROUTE_BLOCK;
constexpr int kWavesPerWg = 16;
constexpr int kRankGroups = 16;  // up to this many groups: top-M by rank

struct RouteArgs {
  const float* logits;     // nparts partial products [nparts][T, E], summed in order
  int64_t part_stride;     // elements between parts
  int nparts;
  float* logits_out;       // [T, E]: the summed logits, or nullptr
  const float* bias;
  const float* offset;
  int32_t* idx;
  float* w;
  int32_t* block_counts;
  int64_t T;
  int E, G, M, k, gk;
};

template <int EPL>
__global__ __launch_bounds__(kWavesPerWg * kWave) void route_select_kernel(const RouteArgs p) {
  __shared__ int s_cnt[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < p.E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();

  const int E = p.E;
  const int gsz = E / p.G;
  const int lpg = gsz / EPL;          // lanes per group (power of two)
  const int e0 = lane * EPL;
  const bool lane_ok = e0 < E;
  const int my_group = lane_ok ? e0 / gsz : 0;
  float bias_l[EPL], off_l[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    bias_l[i] = lane_ok ? p.bias[e0 + i] : 0.0f;
    off_l[i] = (lane_ok && p.offset != nullptr) ? p.offset[e0 + i] : 0.0f;
  }

  const int64_t t_begin = (int64_t)blockIdx.x * kTokPerBlock;
  for (int tt = wave; tt < kTokPerBlock; tt += kWavesPerWg) {
    const int64_t t = t_begin + tt;
    if (t >= p.T) break;
    float s[EPL], b[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float l = 0.0f;
      if (lane_ok) {
        l = p.logits[t * E + e0 + i];
        for (int q = 1; q < p.nparts; ++q) l = l + p.logits[q * p.part_stride + t * E + e0 + i];
        if (p.logits_out != nullptr) p.logits_out[t * E + e0 + i] = l;
      }
      if (p.offset != nullptr) l = l + off_l[i];
      s[i] = affinity_spec(l);
      float bb = s[i] + bias_l[i];
      b[i] = bb == 0.0f ? 0.0f : bb;  // one zero: +0
    }

    // The lane's EPL (key, s) pairs sorted by key, largest first: every
    // round below takes the largest key not yet taken, which is then the head
    // of the lane's list, and only the winning lane moves its list on.
    uint64_t key[EPL];
    float ks[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      key[i] = lane_ok ? make_key(b[i], e0 + i) : 0;
      ks[i] = s[i];
    }
#pragma unroll
    for (int a = 0; a + 1 < EPL; ++a) {
#pragma unroll
      for (int c = 0; c + 1 < EPL - a; ++c) {
        const bool sw = key[c + 1] > key[c];
        const uint64_t k0 = sw ? key[c + 1] : key[c], k1 = sw ? key[c] : key[c + 1];
        const float s0 = sw ? ks[c + 1] : ks[c], s1 = sw ? ks[c] : ks[c + 1];
        key[c] = k0;
        key[c + 1] = k1;
        ks[c] = s0;
        ks[c + 1] = s1;
      }
    }
    // drops the head of a list in the lanes where `win` holds
    auto pop = [&](uint64_t (&kl)[EPL], float* sl, bool win) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const uint64_t nk = i + 1 < EPL ? kl[i + 1] : 0;
        kl[i] = win ? nk : kl[i];
        if (sl != nullptr) {
          const float ns = i + 1 < EPL ? sl[i + 1] : 0.0f;
          sl[i] = win ? ns : sl[i];
        }
      }
    };

    // group score: the gk largest b of the group, added largest first
    float gscore = 0.0f;
    {
      uint64_t gl[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) gl[i] = key[i];
      for (int r = 0; r < p.gk; ++r) {
        const uint64_t m = group_max_u64(gl[0], lpg);
        const float v = key_value(m);
        gscore = r == 0 ? v : gscore + v;
        pop(gl, nullptr, gl[0] == m && m != 0);
      }
    }

    // keep the M best groups: with few groups, a group is kept when fewer
    // than M groups have a larger key (each group's key read from its first
    // lane); otherwise M rounds of a wave-wide max
    uint64_t gkey = lane_ok ? make_key(gscore, my_group) : 0;
    bool gsel = false;
    if (p.G <= kRankGroups) {
      int rank = 0;
      for (int g = 0; g < p.G; ++g) {
        const int src = g * lpg;
        const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(gkey), src);
        const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(gkey >> 32), src);
        rank += ((static_cast<uint64_t>(hi) << 32) | lo) > gkey ? 1 : 0;
      }
      gsel = lane_ok && rank < p.M;
    } else {
      for (int r = 0; r < p.M; ++r) {
        const uint64_t m = group_max_u64(gkey, kWave);
        if (lane_ok && gkey == m) {
          gsel = true;
          gkey = 0;
        }
      }
    }

    // k best experts inside the kept groups
    float S = 0.0f, my_s = 0.0f;
    int my_idx = 0;
    for (int j = 0; j < p.k; ++j) {
      const uint64_t cand = gsel ? key[0] : 0;
      const uint64_t m = group_max_u64(cand, kWave);
      const int win = key_index(m);
      const float s_win = lane_value(ks[0], win / EPL);
      pop(key, ks, cand == m);
      S = j == 0 ? s_win : S + s_win;
      if (lane == j) {
        my_idx = win;
        my_s = s_win;
      }
    }
    if (lane < p.k) {
      p.idx[t * p.k + lane] = my_idx;
      p.w[t * p.k + lane] = my_s / S;
      if (my_idx >= 0 && my_idx < E) atomicAdd(&s_cnt[my_idx], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) p.block_counts[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

template <int EPL>
hipError_t launch_sel(const RouteArgs& a, hipStream_t s) {
  const int64_t nblk = (a.T + kTokPerBlock - 1) / kTokPerBlock;
  hipLaunchKernelGGL(route_select_kernel<EPL>, dim3((unsigned)nblk), dim3(kWavesPerWg * kWave), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace

bool route_select_supported(int E, int G, int k, int gk) {
  if (E > 256 || (E > 64 && E % 64 != 0)) return false;
  const int epl = (E + 63) / 64;
  const int gsz = E / G;
  if (gsz % epl != 0) return false;
  const int lpg = gsz / epl;
  if ((lpg & (lpg - 1)) != 0) return false;
  return gk <= 4 && k <= 16;
}

hipError_t launch_route_select(const float* logits, int nparts, float* logits_out, const float* bias,
                               const float* offset, int32_t* idx, float* w, int32_t* block_counts,
                               int64_t T, int E, int G, int M, int k, int gk, hipStream_t s) {
  RouteArgs a{logits, T * E, nparts, logits_out, bias, offset, idx, w, block_counts, T, E, G, M, k, gk};
  switch ((E + 63) / 64) {
    case 1: return launch_sel<1>(a, s);
    case 2: return launch_sel<2>(a, s);
    case 3: return launch_sel<3>(a, s);
    default: return launch_sel<4>(a, s);
  }
}

}  // namespace moe
