// Elementwise and small kernels of the MoE layer backward (deepmox ch.5: the
// backward carries its own communication and splits into input and weight
// gradients).  Derivatives of the forward with the expert selection fixed:
//
//   combine : d_yp[dest[t,j]] = w[t,j] g[t];  d_w[t,j] = <g[t], yp[dest[t,j]]>
//   SwiGLU  : h = silu(a) u;  da = d_h u sig(a) (1 + a (1 - sig(a))),  du = d_h silu(a)
//   gate    : w_j = s_j / S, s = sqrt(softplus(l)):
//             ds_j = (d_w_j - sum_i w_i d_w_i) / S,  dl_j = ds_j sig(l_j) / (2 s_j)
//   gate products: dx += dL W_g^T, dW_g = x^T dL   (fp32, vector ALUs)
#pragma clang fp contract(off)

#include "affinity.h"
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&f)[8]);
template <>
__device__ __forceinline__ void load8f<uint16_t>(const uint16_t* p, float (&f)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
    f[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
  }
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float (&f)[8]) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
  f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
  f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
}

__device__ __forceinline__ void store8bf(uint16_t* p, const float (&f)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                            pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------- combine backward
// One work-group per token: every thread covers chunks of 8 columns, keeps one
// partial dot product per slot, and the slot sums are reduced in a fixed order
// (lane butterfly, then the four waves in order), so d_w is deterministic.
struct CombBwdArgs {
  int64_t T;
  int k, d;
  const int32_t* dest;
  const float* w;
  const void* yp;    // [rows, d] bf16 or f32
  const void* g;     // [T, d] bf16 or f32
  uint16_t* d_yp;    // [rows, d] bf16
  float* d_w;        // [T, k]
};

template <typename TY, typename TG>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const CombBwdArgs p) {
  __shared__ float s_part[4][kMaxK];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int dest[kMaxK];
  float wt[kMaxK];
  float part[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    dest[j] = j < p.k ? p.dest[t * p.k + j] : -1;
    wt[j] = j < p.k ? p.w[t * p.k + j] : 0.0f;
    part[j] = 0.0f;
  }
  const TG* g = static_cast<const TG*>(p.g) + t * p.d;
  const TY* yp = static_cast<const TY*>(p.yp);
  const int nch = p.d / 8;
  for (int c = tid; c < nch; c += 256) {
    float gf[8];
    load8f<TG>(g + c * 8, gf);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (dest[j] < 0) continue;
      float yf[8], o[8];
      load8f<TY>(yp + (int64_t)dest[j] * p.d + c * 8, yf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        part[j] = __builtin_fmaf(gf[i], yf[i], part[j]);
        o[i] = wt[j] * gf[i];
      }
      store8bf(p.d_yp + (int64_t)dest[j] * p.d + c * 8, o);
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    float v = part[j];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    if (lane == 0) s_part[wave][j] = v;
  }
  __syncthreads();
  if (tid < p.k) {
    const float s = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
    p.d_w[t * p.k + tid] = dest[tid] < 0 ? 0.0f : s;
  }
}

// ---------------------------------------------------------------- SwiGLU backward
// au = [a | u] per row (the up-projection recomputed without the epilogue);
// dh holds d_h on entry and h on exit.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const int32_t* rows_dev, int64_t max_rows,
                                                         int d_ff, const uint16_t* au, uint16_t* dh,
                                                         uint16_t* d_au) {
  const int nch = d_ff / 8;
  const int64_t rows = rows_dev == nullptr ? max_rows : *rows_dev;
  const int64_t total = rows * nch;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int64_t r = q / nch;
    const int c = static_cast<int>(q % nch);
    float a[8], u[8], g[8], da[8], du[8], h[8];
    load8f<uint16_t>(au + r * 2 * d_ff + c * 8, a);
    load8f<uint16_t>(au + r * 2 * d_ff + d_ff + c * 8, u);
    load8f<uint16_t>(dh + r * d_ff + c * 8, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sg = sigmoid(a[i]);
      const float silu = a[i] * sg;
      h[i] = silu * u[i];
      du[i] = g[i] * silu;
      da[i] = g[i] * u[i] * (sg * (1.0f + a[i] * (1.0f - sg)));
    }
    store8bf(d_au + r * 2 * d_ff + c * 8, da);
    store8bf(d_au + r * 2 * d_ff + d_ff + c * 8, du);
    store8bf(dh + r * d_ff + c * 8, h);
  }
}

// ---------------------------------------------------------------- gate backward
// One wave per token: lanes j < k derive dl_j from the token's logits and slot
// gradients; every lane then writes its share of the dense dL row once.
__global__ __launch_bounds__(256) void gate_bwd_kernel(int64_t T, int E, int k, const float* logits,
                                                       const float* offset, const int32_t* idx,
                                                       const float* d_w, float* dL) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int e = -1;
  float l = 0.0f, s = 0.0f, dw = 0.0f;
  if (lane < k) {
    e = idx[t * k + lane];
    l = logits[t * E + e];
    if (offset != nullptr) l = l + offset[e];  // as the forward routed
    s = aff::affinity_spec(l);
    dw = d_w[t * k + lane];
  }
  // S and sum_i w_i dw_i in slot order
  float S = 0.0f;
  for (int j = 0; j < k; ++j) S = j == 0 ? __shfl(s, j, kWave) : S + __shfl(s, j, kWave);
  float dot = 0.0f;
  for (int j = 0; j < k; ++j) dot += (__shfl(s, j, kWave) / S) * __shfl(dw, j, kWave);
  float dl = 0.0f;
  if (lane < k && s > 0.0f) dl = ((dw - dot) / S) * sigmoid(l) / (2.0f * s);
  // gather the k (expert, dl) pairs into every lane before the divergent loop
  int ej[kMaxK];
  float dj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ej[j] = __shfl(e, j < k ? j : 0, kWave);
    dj[j] = __shfl(dl, j < k ? j : 0, kWave);
  }
  for (int c = lane; c < E; c += kWave) {
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k && ej[j] == c) v = dj[j];
    dL[t * E + c] = v;
  }
}

// ---------------------------------------------------------------- fp32 products
// C[m][n] (+)= sum_k A(m, k) B(n, k) with A(m, k) = A[m*sam + k*sak] (bf16 or
// fp32) and B(n, k) = B[n*sbn + k*sbk] (fp32): 64 x 64 tiles, 4 x 4 per thread,
// K staged 16 at a time; operand loads follow whichever index is contiguous.
struct F32Args {
  const void* A;
  int64_t sam, sak;
  const float* B;
  int64_t sbn, sbk;
  float* C;
  int64_t ldc;
  int M, N, K;
  int accumulate;
  int64_t split_stride;  // split-K: part z writes C + z * split_stride over its K range
  int k_per_split;
};

template <typename TA>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const F32Args p) {
  constexpr int BT = 64, BKs = 16;
  __shared__ float sA[BKs][BT + 1];
  __shared__ float sB[BKs][BT + 1];
  const TA* A = static_cast<const TA*>(p.A);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * BT, n0 = blockIdx.x * BT;
  const int kb = blockIdx.z * p.k_per_split;
  const int ke = min(p.K, kb + p.k_per_split);
  float acc[4][4] = {};
  for (int k0 = kb; k0 < ke; k0 += BKs) {
    for (int e = tid; e < BT * BKs; e += 256) {
      // contiguous index innermost across threads
      int r, kk;
      if (p.sam == 1) { r = e % BT; kk = e / BT; } else { kk = e % BKs; r = e / BKs; }
      float v = 0.0f;
      if (m0 + r < p.M && k0 + kk < ke) {
        const int64_t off = (int64_t)(m0 + r) * p.sam + (int64_t)(k0 + kk) * p.sak;
        if constexpr (sizeof(TA) == 2) v = bf16_to_f32(A[off]); else v = A[off];
      }
      sA[kk][r] = v;
    }
    for (int e = tid; e < BT * BKs; e += 256) {
      int r, kk;
      if (p.sbn == 1) { r = e % BT; kk = e / BT; } else { kk = e % BKs; r = e / BKs; }
      float v = 0.0f;
      if (n0 + r < p.N && k0 + kk < ke) v = p.B[(int64_t)(n0 + r) * p.sbn + (int64_t)(k0 + kk) * p.sbk];
      sB[kk][r] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKs; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= p.N) continue;
      float* c = p.C + blockIdx.z * p.split_stride + (int64_t)m * p.ldc + n;
      *c = p.accumulate ? *c + acc[i][j] : acc[i][j];
    }
  }
}

// sum of the split-K parts in part order: out[i] = ((p0 + p1) + p2) + ...
__global__ __launch_bounds__(256) void split_sum_kernel(const float* parts, int nparts, int64_t n, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float v = parts[i];
    for (int z = 1; z < nparts; ++z) v += parts[z * n + i];
    out[i] = v;
  }
}

// ---------------------------------------------------------------- matrix-core gate products
// fp32 operands as three bf16 planes, a = hi + mid + lo, each plane the bf16
// rounding of what the planes before it leave (24 significant bits in all).
__device__ __forceinline__ void planes3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  lo = f32_to_bf16(r1 - bf16_to_f32(mid));
}

// dL [T, E] -> a6 [T, 6E] = [hi | hi | mid | hi | lo | mid] and p3 [T, ld3] =
// [hi | mid | lo | zero padding]; one thread per (row, column < E + ld3 - 3E)
__global__ __launch_bounds__(256) void dl_planes_kernel(const float* __restrict__ dl, int64_t T, int E, int ld3,
                                                        uint16_t* __restrict__ a6, uint16_t* __restrict__ p3,
                                                        int* __restrict__ tickets) {
  const int cols = E + (ld3 - 3 * E);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x < kTicketInts / kTicketStride)
    tickets[threadIdx.x * kTicketStride] = 0;  // the ticket counters of the next product
  if (i >= T * cols) return;
  const int64_t t = i / cols;
  const int c = static_cast<int>(i % cols);
  if (c >= E) {
    p3[t * ld3 + 3 * E + (c - E)] = 0;
    return;
  }
  uint16_t hi, mid, lo;
  planes3(dl[t * E + c], hi, mid, lo);
  uint16_t* a = a6 + t * 6 * E + c;
  a[0] = hi;
  a[E] = hi;
  a[2 * E] = mid;
  a[3 * E] = hi;
  a[4 * E] = lo;
  a[5 * E] = mid;
  uint16_t* q = p3 + t * ld3 + c;
  q[0] = hi;
  q[E] = mid;
  q[2 * E] = lo;
}

// W_g [d, E] -> w6 [d, 6E] = [hi | mid | hi | lo | hi | mid], matching a6
// block by block: hi.hi, hi.mid, mid.hi, hi.lo, lo.hi, mid.mid (the plane
// products above 2^-24 of the product)
__global__ __launch_bounds__(256) void w_planes_kernel(const float* __restrict__ w, int d, int E,
                                                       uint16_t* __restrict__ w6) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d * E) return;
  const int64_t c = i / E;
  const int e = static_cast<int>(i % E);
  uint16_t hi, mid, lo;
  planes3(w[i], hi, mid, lo);
  uint16_t* o = w6 + c * 6 * E + e;
  o[0] = hi;
  o[E] = mid;
  o[2 * E] = hi;
  o[3 * E] = lo;
  o[4 * E] = hi;
  o[5 * E] = mid;
}

// dW_g[c][e] = sum over row splits z (in order) of ((hi + mid) + lo) partials
__global__ __launch_bounds__(256) void plane_sum_kernel(const float* __restrict__ part, int splits, int d, int E,
                                                        int ld3, float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d * E) return;
  const int64_t c = i / E;
  const int e = static_cast<int>(i % E);
  const int64_t zs = (int64_t)d * ld3;
  float v = 0.0f;
  for (int z = 0; z < splits; ++z) {
    const float* q = part + z * zs + c * ld3 + e;
    v += (q[0] + q[E]) + q[2 * E];
  }
  dw[i] = v;
}

hipError_t launch_f32(const F32Args& a, int a_dtype, hipStream_t s, int splits = 1) {
  const dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, splits);
  if (a_dtype == MOE_BF16) hipLaunchKernelGGL(gemm_f32_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(gemm_f32_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_bwd(int64_t T, int k, int d, const int32_t* dest, const float* w, const void* yp,
                              int y_dtype, const void* g, int g_dtype, uint16_t* d_yp, float* d_w,
                              hipStream_t s) {
  CombBwdArgs a{T, k, d, dest, w, yp, g, d_yp, d_w};
  const dim3 grid(static_cast<unsigned>(T));
  if (y_dtype == MOE_BF16) {
    if (g_dtype == MOE_BF16) hipLaunchKernelGGL((combine_bwd_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_bwd_kernel<uint16_t, float>), grid, dim3(256), 0, s, a);
  } else {
    if (g_dtype == MOE_BF16) hipLaunchKernelGGL((combine_bwd_kernel<float, uint16_t>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_bwd_kernel<float, float>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const int32_t* rows_dev, int64_t max_rows, int d_ff, const uint16_t* au,
                             uint16_t* dh, uint16_t* d_au, hipStream_t s) {
  const int64_t work = max_rows * (d_ff / 8);
  const int64_t blocks = (work + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 256 * 64 ? blocks : 256 * 64);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid), dim3(256), 0, s, rows_dev, max_rows, d_ff, au, dh, d_au);
  return hipGetLastError();
}

int gate_bwd_splits(int64_t T) {
  int s = static_cast<int>(T / 1024);
  return s < 1 ? 1 : (s > 16 ? 16 : s);
}

namespace {

// matrix-core path: bf16 x, d a multiple of 256, E a multiple of 64
bool gate_bwd_mfma(int d, int E, int x_dtype) { return x_dtype == MOE_BF16 && d % 256 == 0 && E % 64 == 0; }

struct GateMfmaWs {
  int ld3, splits, split_rows;
  size_t a6, w6, p3, part, tick, total;  // byte offsets into the workspace
};

GateMfmaWs gate_mfma_ws(int64_t T, int d, int E) {
  GateMfmaWs w{};
  w.ld3 = (3 * E + 255) / 256 * 256;
  int64_t sp = T / 2048;
  w.splits = static_cast<int>(sp < 1 ? 1 : (sp > 16 ? 16 : sp));
  w.split_rows = static_cast<int>(((T + w.splits - 1) / w.splits + 63) / 64 * 64);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  w.a6 = 0;
  w.w6 = up(w.a6 + (size_t)T * 6 * E * 2);
  w.p3 = up(w.w6 + (size_t)d * 6 * E * 2);
  w.part = up(w.p3 + (size_t)T * w.ld3 * 2);
  w.tick = up(w.part + (size_t)w.splits * d * w.ld3 * 4);
  w.total = w.tick + kTicketBytes;
  return w;
}

}  // namespace

size_t gate_bwd_workspace_bytes(int64_t T, int d, int E) {
  const int s = gate_bwd_splits(T);
  const size_t simt = s > 1 ? (size_t)s * d * E * sizeof(float) : 0;
  // the larger of the two paths' needs: the path depends on x's dtype
  const size_t mfma = d % 256 == 0 && E % 64 == 0 ? gate_mfma_ws(T, d, E).total : 0;
  return simt > mfma ? simt : mfma;
}

hipError_t launch_gate_bwd(int64_t T, int d, int E, int k, const void* x, int x_dtype, const float* w_gate,
                           const float* logits, const float* offset, const int32_t* idx, const float* d_w,
                           float* dL, float* dx, float* dw_gate, float* ws, hipStream_t s) {
  hipLaunchKernelGGL(gate_bwd_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, s, T, E, k,
                     logits, offset, idx, d_w, dL);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (gate_bwd_mfma(d, E, x_dtype)) {
    const GateMfmaWs w = gate_mfma_ws(T, d, E);
    char* base = reinterpret_cast<char*>(ws);
    uint16_t* a6 = reinterpret_cast<uint16_t*>(base + w.a6);
    uint16_t* w6 = reinterpret_cast<uint16_t*>(base + w.w6);
    uint16_t* p3 = reinterpret_cast<uint16_t*>(base + w.p3);
    float* part = reinterpret_cast<float*>(base + w.part);
    int* tick = reinterpret_cast<int*>(base + w.tick);
    const int64_t n1 = T * (E + (w.ld3 - 3 * E));
    // (the first work-group also clears the ticket counters of the dx product)
    hipLaunchKernelGGL(dl_planes_kernel, dim3(static_cast<unsigned>((n1 + 255) / 256)), dim3(256), 0, s, dL, T, E,
                       w.ld3, a6, p3, tick);
    const int64_t n2 = (int64_t)d * E;
    hipLaunchKernelGGL(w_planes_kernel, dim3(static_cast<unsigned>((n2 + 255) / 256)), dim3(256), 0, s, w_gate, d,
                       E, w6);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dx[t][c] += sum over K' = 6E of a6[t][k'] w6[c][k']
    if ((e = launch_gemm_acc_f32(T, 6 * E, d, a6, w6, dx, tick, s)) != hipSuccess) return e;
    // partials[z][c][k] = sum over split z's rows t of x[t][c] p3[t][k]
    if ((e = launch_ffn_wgrad_bf16(0, nullptr, T, d, w.ld3, static_cast<const uint16_t*>(x), p3, part, s,
                                   w.split_rows)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(plane_sum_kernel, dim3(static_cast<unsigned>((n2 + 255) / 256)), dim3(256), 0, s, part,
                       static_cast<int>((T + w.split_rows - 1) / w.split_rows), d, E, w.ld3, dw_gate);
    return hipGetLastError();
  }
  // dx[t][c] += sum_e dL[t][e] W_g[c][e]
  F32Args a{dL, E, 1, w_gate, E, 1, dx, d, static_cast<int>(T), d, E, 1, 0, E};
  if ((e = launch_f32(a, MOE_F32, s)) != hipSuccess) return e;
  // dW_g[c][e] = sum_t x[t][c] dL[t][e]: K = T split into gate_bwd_splits(T)
  // parts of the workspace, summed in part order (deterministic)
  const int splits = gate_bwd_splits(T);
  const int kps = static_cast<int>((T + splits - 1) / splits + 15) / 16 * 16;
  F32Args b{x, 1, d, dL, 1, E, splits > 1 ? ws : dw_gate, E, d, E, static_cast<int>(T), 0,
            (int64_t)d * E, kps};
  if ((e = launch_f32(b, x_dtype, s, splits)) != hipSuccess || splits == 1) return e;
  const int64_t n = (int64_t)d * E;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     ws, splits, n, dw_gate);
  return hipGetLastError();
}

}  // namespace moe
