// C ABI of the MoE layer forward (declared in include/moe.h): host-side
// argument checks, then kernel launches on the caller's stream.  Nothing here
// allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>

#include "common.h"
#include "launch.h"
#include "moe.h"

using namespace moe;

namespace {

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
    default: return "unknown status";
  }
}

int moe_gate_prepare(int32_t d, int32_t E, const float* w_gate, void* w_prep, moe_stream_t stream) {
  if (d <= 0 || E <= 0 || w_gate == nullptr || w_prep == nullptr) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_gate_prepare(d, E, w_gate, static_cast<uint16_t*>(w_prep), as_stream(stream)));
}

int moe_route(const moe_shape* shape, const void* x, int x_dtype, const void* w_prep,
              const float* bias, const float* logit_offset, float* logits, int32_t* topk_idx,
              float* topk_w, int32_t* block_counts, int flags, moe_stream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const bool logits_in = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  if ((flags & ~MOE_ROUTE_LOGITS_IN) != 0) return MOE_ERR_INVALID_ARG;
  if (bias == nullptr || logits == nullptr || topk_idx == nullptr || topk_w == nullptr ||
      block_counts == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!logits_in) {
    if (x == nullptr || w_prep == nullptr) return MOE_ERR_INVALID_ARG;
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  }
  if (!route_select_supported(shape->E, shape->G, shape->k, shape->group_topk))
    return MOE_ERR_UNSUPPORTED;
  if (shape->T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  if (!logits_in) {
    hipError_t e;
    if (x_dtype == MOE_BF16 && gate_gemm_bf16_supported(shape->d, shape->E))
      e = launch_gate_gemm_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_prep),
                                logits, shape->T, shape->d, shape->E, s);
    else
      e = launch_gate_gemm_simt(x, x_dtype, static_cast<const uint16_t*>(w_prep), logits, shape->T,
                                shape->d, shape->E, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(launch_route_select(logits, bias, logit_offset, topk_idx, topk_w, block_counts,
                                        shape->T, shape->E, shape->G, shape->M, shape->k,
                                        shape->group_topk, s));
}

// dispatch workspace: per-(block, expert) base rows, then (when d % 128 == 0,
// for the e4m3 output) the token-major scale table [d/128][T] at a 256-byte
// aligned offset
static size_t dispatch_base_bytes(const moe_shape* shape, int32_t e_begin, int32_t e_end) {
  const int64_t nblk = (shape->T + MOE_ROUTE_BLOCK - 1) / MOE_ROUTE_BLOCK;
  return static_cast<size_t>(nblk) * static_cast<size_t>(e_end - e_begin) * sizeof(int32_t);
}
static size_t dispatch_scale_offset(const moe_shape* shape, int32_t e_begin, int32_t e_end) {
  return (dispatch_base_bytes(shape, e_begin, e_end) + 255) / 256 * 256;
}

size_t moe_dispatch_workspace_size(const moe_shape* shape, int32_t e_begin, int32_t e_end) {
  if (check_shape(shape) != MOE_OK || e_begin < 0 || e_end < e_begin || e_end > shape->E) return 0;
  if (shape->d % MOE_FP8_TILE != 0) return dispatch_base_bytes(shape, e_begin, e_end);
  return dispatch_scale_offset(shape, e_begin, e_end) +
         static_cast<size_t>(shape->d / MOE_FP8_TILE) * static_cast<size_t>(shape->T) * sizeof(float);
}

int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, const int32_t* block_counts,
                 int32_t e_begin, int32_t e_end, const void* x, int x_dtype, int out_dtype,
                 int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src, void* xp,
                 float* xp_scale, void* ws, size_t ws_bytes, moe_stream_t stream) {
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
  if (ws == nullptr || ws_bytes < moe_dispatch_workspace_size(shape, e_begin, e_end))
    return MOE_ERR_WORKSPACE;
  if (shape->T == 0) return MOE_OK;
  float* tok_scale = out_dtype == MOE_E4M3
                         ? reinterpret_cast<float*>(static_cast<char*>(ws) + dispatch_scale_offset(shape, e_begin, e_end))
                         : nullptr;
  return hip_status(launch_dispatch(topk_idx, block_counts, shape->T, shape->k, shape->E, e_begin,
                                    e_end, x, x_dtype, out_dtype, shape->d, counts, offsets, dest,
                                    src, xp, xp_scale, static_cast<int32_t*>(ws), tok_scale,
                                    as_stream(stream)));
}

int moe_expert_ffn(int32_t n_exp, const int32_t* offsets, int64_t max_rows, int32_t d,
                   int32_t d_ff, int dtype, const void* xp, const float* xp_scale,
                   const void* w13, const float* w13_scale, const void* w2,
                   const float* w2_scale, void* h, float* h_scale, void* yp, int stages,
                   moe_stream_t stream) {
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
  if (max_rows == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  const bool mfma = dtype == MOE_BF16 && d % 256 == 0 && d_ff % 128 == 0 && d_ff >= 256;
  if (up) {
    hipError_t e;
    if (dtype == MOE_E4M3 && ffn_fp8p_supported_k(d))
      e = launch_ffn_up_fp8p(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint8_t*>(xp),
                             xp_scale, static_cast<const uint8_t*>(w13), w13_scale,
                             static_cast<uint8_t*>(h), h_scale, s);
    else if (dtype == MOE_E4M3)
      e = launch_ffn_up_fp8(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint8_t*>(xp),
                            xp_scale, static_cast<const uint8_t*>(w13), w13_scale,
                            static_cast<uint8_t*>(h), h_scale, s);
    else if (mfma)
      e = launch_ffn_up_bf16(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint16_t*>(xp),
                             static_cast<const uint16_t*>(w13), static_cast<uint16_t*>(h), s);
    else
      e = launch_ffn_simt(MOE_FFN_UP, n_exp, offsets, max_rows, d, d_ff, dtype, xp, w13, h, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (down) {
    hipError_t e;
    if (dtype == MOE_E4M3 && ffn_fp8p_supported_k(d_ff))
      e = launch_ffn_down_fp8p(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint8_t*>(h),
                               h_scale, static_cast<const uint8_t*>(w2), w2_scale,
                               static_cast<uint16_t*>(yp), s);
    else if (dtype == MOE_E4M3)
      e = launch_ffn_down_fp8(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint8_t*>(h),
                              h_scale, static_cast<const uint8_t*>(w2), w2_scale,
                              static_cast<uint16_t*>(yp), s);
    else if (mfma)
      e = launch_ffn_down_bf16(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint16_t*>(h),
                               static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(yp), s);
    else
      e = launch_ffn_simt(MOE_FFN_DOWN, n_exp, offsets, max_rows, d, d_ff, dtype, h, w2, yp, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
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
                         moe_stream_t stream) {
  if (n_exp < 1 || n_exp > kMaxExperts || max_rows < 0 || d < 1 || d_ff < 1) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || !ffn_bwd_bf16_supported(d, d_ff)) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && n_exp != 1) return MOE_ERR_INVALID_ARG;
  if (xp == nullptr || w13 == nullptr || w2 == nullptr || h == nullptr || au == nullptr || yp == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (max_rows == 0) return MOE_OK;
  const hipStream_t s = as_stream(stream);
  hipError_t e = launch_ffn_up_bf16(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint16_t*>(xp),
                                    static_cast<const uint16_t*>(w13), static_cast<uint16_t*>(h), s,
                                    static_cast<uint16_t*>(au));
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_ffn_down_bf16(n_exp, offsets, max_rows, d, d_ff, static_cast<const uint16_t*>(h),
                                         static_cast<const uint16_t*>(w2), static_cast<uint16_t*>(yp), s));
}

int moe_expert_ffn_backward(int32_t n_exp, const int32_t* offsets, int64_t max_rows, int32_t d, int32_t d_ff,
                            int dtype, const void* xp, const void* w13, const void* w2, const void* d_yp,
                            void* au, void* h, void* d_au, void* d_xp, float* dw13, float* dw2, int flags,
                            moe_stream_t stream) {
  if (n_exp < 1 || n_exp > kMaxExperts || max_rows < 0 || d < 1 || d_ff < 1) return MOE_ERR_INVALID_ARG;
  if ((flags & ~MOE_BWD_AU_SAVED) != 0) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || !ffn_bwd_bf16_supported(d, d_ff)) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && n_exp != 1) return MOE_ERR_INVALID_ARG;
  if (xp == nullptr || w13 == nullptr || w2 == nullptr || d_yp == nullptr || au == nullptr || h == nullptr ||
      d_au == nullptr || d_xp == nullptr || dw13 == nullptr || dw2 == nullptr)
    return MOE_ERR_INVALID_ARG;
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
      (e = launch_ffn_store_bf16(n_exp, offsets, max_rows, d, 2 * d_ff, X, W13, AU, s)) != hipSuccess)
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

size_t moe_route_backward_workspace_size(const moe_shape* shape) {
  if (shape == nullptr || shape->T <= 0 || shape->d < 1 || shape->E < 1) return 0;
  return gate_bwd_workspace_bytes(shape->T, shape->d, shape->E);
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
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return MOE_ERR_WORKSPACE;
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

}  // extern "C"
