// C ABI of the MoE layer forward (declared in include/moe.h): host-side
// argument checks, then kernel launches on the caller's stream.  Nothing here
// allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "common.h"
#include "launch.h"
#include "moe.h"

using namespace moe;

// Workspace of moe_dispatch_noalloc, held by the library: one copy per device,
// at that device's own address, for the life of the process.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the device symbol); it uses the device address hipGetSymbolAddress returns.
static constexpr size_t kScratchBytes = size_t{8} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static_assert(kScratchBytes == MOE_DISPATCH_NOALLOC_SCRATCH, "the header states the scratch size");

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];  // device address of `scratch`, per device (under the mutex)

// The current device's address of `scratch`, looked up once per device with
// that device current.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kScratchDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

hipStream_t as_stream(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

int check_shape(const moe_shape* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->d <= 0 || s->E <= 0 || s->G <= 0 || s->M <= 0 || s->k <= 0 ||
      s->group_topk <= 0 || s->d_ff <= 0)
    return MOE_ERR_INVALID_ARG;
  if (s->E % s->G != 0 || s->M > s->G) return MOE_ERR_INVALID_ARG;
  const int gsz = s->E / s->G;
  if (s->group_topk > gsz || s->k > s->M * gsz) return MOE_ERR_INVALID_ARG;
  if (s->T > (int64_t)INT32_MAX / s->k) return MOE_ERR_UNSUPPORTED;  // row ids are int32
  return MOE_OK;
}

bool is_dtype(int t) { return t == MOE_F32 || t == MOE_BF16 || t == MOE_E4M3; }

size_t align256(size_t n) { return (n + 255) / 256 * 256; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

// ticket counter sets at the start of a workspace (one per persistent launch
// of a call), 256-byte aligned
constexpr size_t kTicketSetBytes = (kTicketBytes + 255) / 256 * 256;
int* ticket_set(void* ws, int i) {
  return reinterpret_cast<int*>(static_cast<char*>(ws) + static_cast<size_t>(i) * kTicketSetBytes);
}

}  // namespace

namespace moe {
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// CUs the stream's work may use: the population of its CU mask (a stream made
// with hipExtStreamCreateWithCUMask, e.g. to leave CUs to communication
// kernels on another stream), else the device's.  Persistent launches size
// their grid by it, so that no work-group waits for a CU the mask keeps from
// the launch.
int stream_cu_count(hipStream_t s) {
  const int n = device_cu_count();
  if (s == nullptr) return n;
  constexpr int kMaxWords = 64;
  uint32_t mask[kMaxWords] = {};
  const int words = (n + 31) / 32;
  if (words > kMaxWords) return n;
  if (hipExtStreamGetCUMask(s, static_cast<uint32_t>(words), mask) != hipSuccess) {
    (void)hipGetLastError();  // the query's own failure is not the launch's
    return n;
  }
  int c = 0;
  for (int w = 0; w < words; ++w) c += __builtin_popcount(mask[w]);
  return c > 0 && c <= n ? c : n;
}
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "needs more than the library's static scratch buffer";
    default: return "unknown status";
  }
}

// route workspace: the gate weight's three bf16 planes [3, E, d], then (when
// the caller passes no logits buffer) the logits [T, E] fp32
static size_t route_planes_bytes(const moe_shape* s) {
  return align256(static_cast<size_t>(3) * s->E * s->d * sizeof(uint16_t));
}
// route workspace: the planes; for the gate product on the expert GEMM
// kernel (bf16 x, E % 256 == 0) its ticket set and offsets; the S partial
// products of a split gate product when S > 1; else the logits when the
// caller keeps none
static size_t route_split_bytes() { return align256((kTicketInts + kMaxGateSplits + 1) * sizeof(int)); }
// splits of the gate product on the expert GEMM kernel (0: not that path)
static int route_gate_splits(const moe_shape* s, int x_dtype) {
  return x_dtype == MOE_BF16 ? gate_split_count(s->T, s->d, s->E) : 0;
}
// splits of the gate product on either matrix-core path (0: vector ALUs)
static int route_splits(const moe_shape* s, int x_dtype) {
  const int S = route_gate_splits(s, x_dtype);
  if (S >= 1 || x_dtype != MOE_BF16) return S;
  return gate_gemm_split_count(s->T, s->d, s->E);
}
static size_t route_ws_bytes(const moe_shape* s, bool logits_in_ws, int x_dtype) {
  const size_t logits_bytes = align256(static_cast<size_t>(s->T) * s->E * sizeof(float));
  size_t b = route_planes_bytes(s);
  if (route_gate_splits(s, x_dtype) >= 1) b += route_split_bytes();
  const int S = route_splits(s, x_dtype);
  if (S > 1) return b + S * logits_bytes;
  return b + (logits_in_ws ? logits_bytes : 0);
}

int moe_route(const moe_shape* shape, const void* x, int x_dtype, const float* w_gate,
              const float* bias, const float* logit_offset, float* logits, int32_t* topk_idx,
              float* topk_w, int32_t* block_counts, int flags, void* ws, size_t ws_bytes,
              moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const bool logits_in = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  if ((flags & ~MOE_ROUTE_LOGITS_IN) != 0) return MOE_ERR_INVALID_ARG;
  if (bias == nullptr || topk_idx == nullptr || topk_w == nullptr || block_counts == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (logits_in && logits == nullptr) return MOE_ERR_INVALID_ARG;
  if (!logits_in) {
    if (x == nullptr || w_gate == nullptr) return MOE_ERR_INVALID_ARG;
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  }
  if (!route_select_supported(shape->E, shape->G, shape->k, shape->group_topk))
    return MOE_ERR_UNSUPPORTED;
  if (!logits_in) {
    if (ws == nullptr || ws_bytes < route_ws_bytes(shape, logits == nullptr, x_dtype) || !aligned256(ws))
      return MOE_ERR_WORKSPACE;
  }
  if (shape->T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  const float* parts = logits;  // what the selection reads
  int nparts = 1;
  float* logits_out = nullptr;
  if (!logits_in) {
    char* w = static_cast<char*>(ws);
    uint16_t* planes = reinterpret_cast<uint16_t*>(w);
    w += route_planes_bytes(shape);
    const int Sg = route_gate_splits(shape, x_dtype);
    const int S = route_splits(shape, x_dtype);
    int* split = nullptr;
    if (Sg >= 1) {
      split = reinterpret_cast<int*>(w);
      w += route_split_bytes();
    }
    float* out = logits != nullptr ? logits : reinterpret_cast<float*>(w);
    hipError_t e = launch_gate_prepare(shape->d, shape->E, w_gate, planes, s, split, Sg, shape->T);
    if (e != hipSuccess) return MOE_ERR_HIP;
    // S > 1: partial products in the workspace, summed (and written to the
    // caller's logits) by the selection
    float* const dst = S > 1 ? reinterpret_cast<float*>(w) : out;
    if (S >= 1) {
      const uint16_t* xb = static_cast<const uint16_t*>(x);
      e = Sg >= 1 ? launch_gate_split_bf16(xb, planes, dst, shape->T, shape->d, shape->E, S, split + kTicketInts,
                                           split, s)
                  : launch_gate_gemm_bf16(xb, planes, dst, shape->T, shape->d, shape->E, S, s);
      parts = dst;
      nparts = S;
      if (S > 1) logits_out = logits;
    } else {
      e = launch_gate_gemm_simt(x, x_dtype, planes, out, shape->T, shape->d, shape->E, s);
      parts = out;
    }
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(launch_route_select(parts, nparts, logits_out, bias, logit_offset, topk_idx, topk_w,
                                        block_counts, shape->T, shape->E, shape->G, shape->M, shape->k,
                                        shape->group_topk, s));
}

// dispatch workspace: per-(block, expert) base rows, then (for the e4m3
// output) the token-major scale table [d/128][T] at a 256-byte aligned offset
static size_t dispatch_base_bytes(const moe_shape* shape, int32_t e_begin, int32_t e_end) {
  const int64_t nblk = (shape->T + MOE_ROUTE_BLOCK - 1) / MOE_ROUTE_BLOCK;
  return static_cast<size_t>(nblk) * static_cast<size_t>(e_end - e_begin) * sizeof(int32_t);
}
static size_t dispatch_scale_offset(const moe_shape* shape, int32_t e_begin, int32_t e_end) {
  return (dispatch_base_bytes(shape, e_begin, e_end) + 255) / 256 * 256;
}

static size_t dispatch_ws_bytes(const moe_shape* shape, int32_t e_begin, int32_t e_end, int out_dtype) {
  if (check_shape(shape) != MOE_OK || e_begin < 0 || e_end < e_begin || e_end > shape->E) return 0;
  if (out_dtype != MOE_E4M3 || shape->d % MOE_FP8_TILE != 0) return dispatch_base_bytes(shape, e_begin, e_end);
  return dispatch_scale_offset(shape, e_begin, e_end) +
         static_cast<size_t>(shape->d / MOE_FP8_TILE) * static_cast<size_t>(shape->T) * sizeof(float);
}

// Argument checks of moe_dispatch before any workspace is looked at.
static int dispatch_check(const moe_shape* shape, const int32_t* topk_idx, const int32_t* block_counts,
                          int32_t e_begin, int32_t e_end, const void* x, int x_dtype, int out_dtype,
                          int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src, void* xp,
                          float* xp_scale) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (e_begin < 0 || e_end <= e_begin || e_end > shape->E) return MOE_ERR_INVALID_ARG;
  if (topk_idx == nullptr || block_counts == nullptr || x == nullptr || counts == nullptr ||
      offsets == nullptr || dest == nullptr || src == nullptr || xp == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!is_dtype(out_dtype)) return MOE_ERR_INVALID_ARG;
  if (out_dtype == MOE_E4M3) {
    if (x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (xp_scale == nullptr) return MOE_ERR_INVALID_ARG;
    if (shape->d % MOE_FP8_TILE != 0) return MOE_ERR_UNSUPPORTED;
  } else if (out_dtype != x_dtype) {
    return MOE_ERR_UNSUPPORTED;
  }
  const int elem = x_dtype == MOE_F32 ? 4 : 2;
  if ((shape->d * elem) % 16 != 0) return MOE_ERR_UNSUPPORTED;  // 16-byte row chunks
  if (e_end - e_begin > 256 || shape->k > 16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static int dispatch_launch(const moe_shape* shape, const int32_t* topk_idx, const int32_t* block_counts,
                           int32_t e_begin, int32_t e_end, const void* x, int x_dtype, int out_dtype,
                           int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src, void* xp,
                           float* xp_scale, void* ws, moe_stream_t stream) {
  float* tok_scale = out_dtype == MOE_E4M3
                         ? reinterpret_cast<float*>(static_cast<char*>(ws) + dispatch_scale_offset(shape, e_begin, e_end))
                         : nullptr;
  return hip_status(launch_dispatch(topk_idx, block_counts, shape->T, shape->k, shape->E, e_begin,
                                    e_end, x, x_dtype, out_dtype, shape->d, counts, offsets, dest,
                                    src, xp, xp_scale, static_cast<int32_t*>(ws), tok_scale,
                                    as_stream(stream)));
}

int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, const int32_t* block_counts,
                 int32_t e_begin, int32_t e_end, const void* x, int x_dtype, int out_dtype,
                 int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src, void* xp,
                 float* xp_scale, void* ws, size_t ws_bytes, moe_stream_t stream) {
  const int st = dispatch_check(shape, topk_idx, block_counts, e_begin, e_end, x, x_dtype, out_dtype, counts,
                                offsets, dest, src, xp, xp_scale);
  if (st != MOE_OK) return st;
  if (ws == nullptr || ws_bytes < dispatch_ws_bytes(shape, e_begin, e_end, out_dtype) || !aligned256(ws))
    return MOE_ERR_WORKSPACE;
  if (shape->T == 0) return MOE_OK;
  return dispatch_launch(shape, topk_idx, block_counts, e_begin, e_end, x, x_dtype, out_dtype, counts, offsets,
                         dest, src, xp, xp_scale, ws, stream);
}

int moe_dispatch_noalloc(const moe_shape* shape, const int32_t* topk_idx, const int32_t* block_counts,
                         int32_t e_begin, int32_t e_end, const void* x, int x_dtype, int out_dtype,
                         int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src, void* xp,
                         float* xp_scale, moe_stream_t stream) {
  const int st = dispatch_check(shape, topk_idx, block_counts, e_begin, e_end, x, x_dtype, out_dtype, counts,
                                offsets, dest, src, xp, xp_scale);
  if (st != MOE_OK) return st;
  if (dispatch_ws_bytes(shape, e_begin, e_end, out_dtype) > kScratchBytes) return MOE_ERR_SCRATCH;
  if (shape->T == 0) return MOE_OK;
  void* ws = nullptr;
  const int sa = scratch_address(&ws);
  if (sa != MOE_OK) return sa;
  return dispatch_launch(shape, topk_idx, block_counts, e_begin, e_end, x, x_dtype, out_dtype, counts, offsets,
                         dest, src, xp, xp_scale, ws, stream);
}

int moe_expert_ffn(int32_t n_exp, const int32_t* offsets, int64_t max_rows, int32_t d,
                   int32_t d_ff, int dtype, const void* xp, const float* xp_scale,
                   const void* w13, const float* w13_scale, const void* w2,
                   const float* w2_scale, void* h, float* h_scale, void* yp, int stages,
                   const moe_ffn_extra* extra, void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (n_exp <= 0 || n_exp > kMaxExperts || offsets == nullptr || max_rows < 0 || d <= 0 ||
      d_ff <= 0 || h == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!is_dtype(dtype)) return MOE_ERR_INVALID_ARG;
  if (stages < 1 || stages > MOE_FFN_ALL) return MOE_ERR_INVALID_ARG;
  const bool up = (stages & MOE_FFN_UP) != 0, down = (stages & MOE_FFN_DOWN) != 0;
  if (up && (xp == nullptr || w13 == nullptr)) return MOE_ERR_INVALID_ARG;
  if (down && (w2 == nullptr || yp == nullptr)) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_E4M3) {
    if (h_scale == nullptr || (up && (xp_scale == nullptr || w13_scale == nullptr)) ||
        (down && w2_scale == nullptr))
      return MOE_ERR_INVALID_ARG;
    if (d % 256 != 0 || d_ff % 128 != 0) return MOE_ERR_UNSUPPORTED;
  }
  if (extra != nullptr && extra->rows < 0) return MOE_ERR_INVALID_ARG;
  const bool has_x = extra != nullptr && extra->rows > 0;
  if (has_x) {
    if (extra->h == nullptr || (up && (extra->x == nullptr || extra->w13 == nullptr)) ||
        (down && (extra->w2 == nullptr || extra->y == nullptr)))
      return MOE_ERR_INVALID_ARG;
    if (dtype == MOE_E4M3 && (extra->h_scale == nullptr || (up && (extra->x_scale == nullptr ||
                                                                    extra->w13_scale == nullptr)) ||
                              (down && extra->w2_scale == nullptr)))
      return MOE_ERR_INVALID_ARG;
  }
  if (ws == nullptr || ws_bytes < 2 * kTicketSetBytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  if (max_rows == 0 && !has_x) return MOE_OK;
  hipStream_t s = as_stream(stream);
  const bool mfma = dtype == MOE_BF16 && d % 256 == 0 && d_ff % 128 == 0 && d_ff >= 256;
  int* const tick_up = ticket_set(ws, 0);
  int* const tick_down = ticket_set(ws, 1);
  // The bf16 matrix-core products take the extra group into their launches;
  // every other path runs it after the routed groups as one group of its own
  // (no offsets), reusing the ticket sets in stream order.  (The e4m3
  // persistent kernel has no registers left for a second set of buffers.)
  const moe_ffn_extra* merged_up = mfma && has_x ? extra : nullptr;
  const moe_ffn_extra* merged_down = merged_up;
  auto up_launch = [&](int n, const int32_t* off, int64_t rows, const void* x_, const float* xs_, const void* w13_,
                       const float* w13s_, void* h_, float* hs_) -> hipError_t {
    if (dtype == MOE_E4M3 && ffn_fp8p_supported_k(d))
      return launch_ffn_up_fp8p(n, off, rows, d, d_ff, static_cast<const uint8_t*>(x_), xs_,
                                static_cast<const uint8_t*>(w13_), w13s_, static_cast<uint8_t*>(h_), hs_, tick_up, s);
    if (dtype == MOE_E4M3)
      return launch_ffn_up_fp8(n, off, rows, d, d_ff, static_cast<const uint8_t*>(x_), xs_,
                               static_cast<const uint8_t*>(w13_), w13s_, static_cast<uint8_t*>(h_), hs_, s);
    if (mfma)
      return launch_ffn_up_bf16(n, off, rows, d, d_ff, static_cast<const uint16_t*>(x_),
                                static_cast<const uint16_t*>(w13_), static_cast<uint16_t*>(h_), tick_up, s, nullptr,
                                off != nullptr ? merged_up : nullptr);
    return launch_ffn_simt(MOE_FFN_UP, n, off, rows, d, d_ff, dtype, x_, w13_, h_, s);
  };
  auto down_launch = [&](int n, const int32_t* off, int64_t rows, const void* h_, const float* hs_, const void* w2_,
                         const float* w2s_, void* y_) -> hipError_t {
    if (dtype == MOE_E4M3 && ffn_fp8p_supported_k(d_ff))
      return launch_ffn_down_fp8p(n, off, rows, d, d_ff, static_cast<const uint8_t*>(h_), hs_,
                                  static_cast<const uint8_t*>(w2_), w2s_, static_cast<uint16_t*>(y_), tick_down, s);
    if (dtype == MOE_E4M3)
      return launch_ffn_down_fp8(n, off, rows, d, d_ff, static_cast<const uint8_t*>(h_), hs_,
                                 static_cast<const uint8_t*>(w2_), w2s_, static_cast<uint16_t*>(y_), s);
    if (mfma)
      return launch_ffn_down_bf16(n, off, rows, d, d_ff, static_cast<const uint16_t*>(h_),
                                  static_cast<const uint16_t*>(w2_), static_cast<uint16_t*>(y_), tick_down, s,
                                  off != nullptr ? merged_down : nullptr);
    return launch_ffn_simt(MOE_FFN_DOWN, n, off, rows, d, d_ff, dtype, h_, w2_, y_, s);
  };
  if (up) {
    if ((max_rows > 0 || merged_up != nullptr) &&
        up_launch(n_exp, offsets, max_rows, xp, xp_scale, w13, w13_scale, h, h_scale) != hipSuccess)
      return MOE_ERR_HIP;
    if (has_x && merged_up == nullptr && up_launch(1, nullptr, extra->rows, extra->x, extra->x_scale, extra->w13, extra->w13_scale,
                              extra->h, extra->h_scale) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (down) {
    if ((max_rows > 0 || merged_down != nullptr) &&
        down_launch(n_exp, offsets, max_rows, h, h_scale, w2, w2_scale, yp) != hipSuccess)
      return MOE_ERR_HIP;
    if (has_x && merged_down == nullptr && down_launch(1, nullptr, extra->rows, extra->h, extra->h_scale, extra->w2, extra->w2_scale,
                                extra->y) != hipSuccess)
      return MOE_ERR_HIP;
  }
  return MOE_OK;
}

int moe_combine(const moe_shape* shape, const int32_t* dest, const float* topk_w, const void* yp,
                int y_dtype, const void* ysh, void* out, int out_dtype, int accumulate,
                moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (dest == nullptr || topk_w == nullptr || yp == nullptr || out == nullptr)
    return MOE_ERR_INVALID_ARG;
  if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
    return MOE_ERR_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return MOE_ERR_INVALID_ARG;
  if (accumulate && out_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (shape->d % 8 != 0 || shape->k > 16) return MOE_ERR_UNSUPPORTED;
  if (shape->T == 0) return MOE_OK;
  return hip_status(launch_combine(shape->T, shape->k, shape->d, dest, topk_w, yp, y_dtype, ysh, out,
                                   out_dtype, accumulate, as_stream(stream)));
}

int moe_quantize_rows_e4m3(int64_t rows, int32_t cols, const void* x, uint8_t* q, float* scale,
                           moe_stream_t stream) {
  if (rows < 0 || cols <= 0 || x == nullptr || q == nullptr || scale == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (cols % MOE_FP8_TILE != 0) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_rows(rows, cols, static_cast<const uint16_t*>(x), q, scale,
                                         as_stream(stream)));
}

int moe_quantize_blocks_e4m3(int64_t n, int32_t rows, int32_t cols, const float* w, uint8_t* q,
                             float* scale, moe_stream_t stream) {
  if (n < 0 || rows <= 0 || cols <= 0 || w == nullptr || q == nullptr || scale == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (rows % MOE_FP8_TILE != 0 || cols % MOE_FP8_TILE != 0) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_blocks(n, rows, cols, w, q, scale, as_stream(stream)));
}

int moe_combine_backward(const moe_shape* shape, const int32_t* dest, const float* topk_w, const void* yp,
                         int y_dtype, const void* grad_out, int g_dtype, void* d_yp, float* d_topk_w,
                         moe_stream_t stream) {
  if (shape == nullptr || shape->T < 0 || shape->k < 1 || shape->d < 1) return MOE_ERR_INVALID_ARG;
  if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (g_dtype != MOE_F32 && g_dtype != MOE_BF16))
    return MOE_ERR_INVALID_ARG;
  if (shape->k > 16 || shape->d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (shape->T == 0) return MOE_OK;
  if (dest == nullptr || topk_w == nullptr || yp == nullptr || grad_out == nullptr || d_yp == nullptr ||
      d_topk_w == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine_bwd(shape->T, shape->k, shape->d, dest, topk_w, yp, y_dtype, grad_out,
                                       g_dtype, static_cast<uint16_t*>(d_yp), d_topk_w, as_stream(stream)));
}

int moe_expert_ffn_train(int32_t n_exp, const int32_t* offsets, int64_t max_rows, int32_t d, int32_t d_ff,
                         int dtype, const void* xp, const void* w13, const void* w2, void* h, void* au, void* yp,
                         void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (n_exp < 1 || n_exp > kMaxExperts || max_rows < 0 || d < 1 || d_ff < 1) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || !ffn_bwd_bf16_supported(d, d_ff)) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && n_exp != 1) return MOE_ERR_INVALID_ARG;
  if (xp == nullptr || w13 == nullptr || w2 == nullptr || h == nullptr || au == nullptr || yp == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < 2 * kTicketSetBytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  if (max_rows == 0) return MOE_OK;
  const hipStream_t s = as_stream(stream);
  hipError_t e = launch_ffn_up_bf16(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint16_t*>(xp),
                                    static_cast<const uint16_t*>(w13), static_cast<uint16_t*>(h), ticket_set(ws, 0),
                                    s, static_cast<uint16_t*>(au));
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_ffn_down_bf16(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint16_t*>(h),
                                         static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(yp),
                                         ticket_set(ws, 1), s));
}

int moe_expert_ffn_backward(int32_t n_exp, const int32_t* offsets, int64_t max_rows, int32_t d, int32_t d_ff,
                            int dtype, const void* xp, const void* w13, const void* w2, const void* d_yp,
                            void* au, void* h, void* d_au, void* d_xp, float* dw13, float* dw2, int flags,
                            void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (n_exp < 1 || n_exp > kMaxExperts || max_rows < 0 || d < 1 || d_ff < 1) return MOE_ERR_INVALID_ARG;
  if ((flags & ~MOE_BWD_AU_SAVED) != 0) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || !ffn_bwd_bf16_supported(d, d_ff)) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && n_exp != 1) return MOE_ERR_INVALID_ARG;
  if (xp == nullptr || w13 == nullptr || w2 == nullptr || d_yp == nullptr || au == nullptr || h == nullptr ||
      d_au == nullptr || d_xp == nullptr || dw13 == nullptr || dw2 == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < kTicketSetBytes || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  const hipStream_t s = as_stream(stream);
  const auto* X = static_cast<const uint16_t*>(xp);
  const auto* W13 = static_cast<const uint16_t*>(w13);
  const auto* W2 = static_cast<const uint16_t*>(w2);
  const auto* DY = static_cast<const uint16_t*>(d_yp);
  auto* AU = static_cast<uint16_t*>(au);
  auto* H = static_cast<uint16_t*>(h);
  auto* DAU = static_cast<uint16_t*>(d_au);
  hipError_t e;
  // [a | u] (kept by moe_expert_ffn_train, else recomputed), d_h = d_y W2,
  // then SwiGLU's derivative (h on the side)
  if (!(flags & MOE_BWD_AU_SAVED) &&
      (e = launch_ffn_store_bf16(n_exp, offsets, max_rows, d, 2 * d_ff, X, W13, AU, ticket_set(ws, 0), s)) !=
          hipSuccess)
    return hip_status(e);
  if ((e = launch_ffn_dgrad_bf16(n_exp, offsets, max_rows, d, d_ff, DY, W2, H, s)) != hipSuccess)
    return hip_status(e);
  if ((e = launch_swiglu_bwd(offsets == nullptr ? nullptr : offsets + n_exp, max_rows, d_ff, AU, H, DAU, s)) !=
      hipSuccess)
    return hip_status(e);
  // d_x = [da | du] W13, dW2 = d_y^T h, dW13 = [da | du]^T x
  if ((e = launch_ffn_dgrad_bf16(n_exp, offsets, max_rows, 2 * d_ff, d, DAU, W13, static_cast<uint16_t*>(d_xp),
                                 s)) != hipSuccess)
    return hip_status(e);
  if ((e = launch_ffn_wgrad_bf16(n_exp, offsets, max_rows, d, d_ff, DY, H, dw2, s)) != hipSuccess)
    return hip_status(e);
  return hip_status(launch_ffn_wgrad_bf16(n_exp, offsets, max_rows, 2 * d_ff, d, DAU, X, dw13, s));
}

int moe_dispatch_backward(const moe_shape* shape, const int32_t* dest, const void* d_xp, int xp_dtype,
                          const void* d_extra, float* dx, int accumulate, moe_stream_t stream) {
  if (shape == nullptr || shape->T < 0 || shape->k < 1 || shape->d < 1) return MOE_ERR_INVALID_ARG;
  if ((xp_dtype != MOE_F32 && xp_dtype != MOE_BF16) || (accumulate != 0 && accumulate != 1))
    return MOE_ERR_INVALID_ARG;
  if (shape->k > 16 || shape->d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (shape->T == 0) return MOE_OK;
  if (dest == nullptr || d_xp == nullptr || dx == nullptr) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(shape->T, shape->k, shape->d, dest, nullptr, d_xp, xp_dtype, d_extra, dx,
                                   MOE_F32, accumulate, as_stream(stream)));
}

int moe_route_backward(const moe_shape* shape, const void* x, int x_dtype, const float* w_gate,
                       const float* logit_offset, const float* logits, const int32_t* topk_idx,
                       const float* d_topk_w, float* dlogits, float* dx, float* dw_gate, void* ws,
                       size_t ws_bytes, moe_stream_t stream) {
  if (shape == nullptr || shape->T < 0 || shape->E < 1 || shape->k < 1 || shape->k > shape->E || shape->d < 1)
    return MOE_ERR_INVALID_ARG;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (shape->k > 16 || shape->E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (shape->T == 0) return MOE_OK;
  if (x == nullptr || w_gate == nullptr || logits == nullptr || topk_idx == nullptr || d_topk_w == nullptr ||
      dlogits == nullptr || dx == nullptr || dw_gate == nullptr)
    return MOE_ERR_INVALID_ARG;
  const size_t need = gate_bwd_workspace_bytes(shape->T, shape->d, shape->E);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned256(ws))) return MOE_ERR_WORKSPACE;
  return hip_status(launch_gate_bwd(shape->T, shape->d, shape->E, shape->k, x, x_dtype, w_gate, logits,
                                    logit_offset, topk_idx, d_topk_w, dlogits, dx, dw_gate,
                                    static_cast<float*>(ws), as_stream(stream)));
}

int moe_route_hash(const moe_shape* shape, const int32_t* token_ids, uint64_t seed,
                   const float* logits, int32_t* topk_idx, float* topk_w, int32_t* block_counts,
                   moe_stream_t stream) {
  if (shape == nullptr) return MOE_ERR_INVALID_ARG;
  if (shape->T < 0 || shape->E < 1 || shape->k < 1 || shape->k > shape->E) return MOE_ERR_INVALID_ARG;
  if (shape->E > kMaxExperts || shape->k > 16) return MOE_ERR_UNSUPPORTED;
  if (shape->T == 0) return MOE_OK;
  if (token_ids == nullptr || topk_idx == nullptr || topk_w == nullptr || block_counts == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_hash_route(token_ids, shape->T, shape->E, shape->k, seed, logits, topk_idx,
                                      topk_w, block_counts, as_stream(stream)));
}

int moe_bias_update(int64_t n_rows, int32_t E, const int32_t* counts, float gamma, float* bias,
                    int32_t* load, moe_stream_t stream) {
  if (n_rows < 0 || E < 1 || E > kMaxExperts || !std::isfinite(gamma)) return MOE_ERR_INVALID_ARG;
  if (n_rows == 0) return MOE_OK;
  if (counts == nullptr || bias == nullptr) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(n_rows, E, counts, gamma, bias, load, as_stream(stream)));
}

size_t moe_workspace_size(int op, const moe_shape* shape, int dtype) {
  switch (op) {
    case MOE_OP_ROUTE:
      if (check_shape(shape) != MOE_OK) return 0;
      return route_ws_bytes(shape, true, dtype);
    case MOE_OP_DISPATCH:
      if (check_shape(shape) != MOE_OK) return 0;
      return dispatch_ws_bytes(shape, 0, shape->E, dtype);
    case MOE_OP_EXPERT_FFN:
      return 2 * kTicketSetBytes;
    case MOE_OP_COMBINE:
      return 0;
    case MOE_OP_ROUTE_BACKWARD:
      if (shape == nullptr || shape->T <= 0 || shape->d < 1 || shape->E < 1) return 0;
      return gate_bwd_workspace_bytes(shape->T, shape->d, shape->E);
    case MOE_OP_EXPERT_FFN_BACKWARD:
      return kTicketSetBytes;
    default:
      return 0;
  }
}

}  // extern "C"
