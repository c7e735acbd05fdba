// Host-side launchers of the gfx950 kernels (internal to the library; the C
// ABI in moe.h checks arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// compute units of the current device (cached per device; 256 if the query fails)
int device_cu_count();
// CUs a launch on stream s may use (its CU mask, else the device's)
int stream_cu_count(hipStream_t s);

// gate logits
// S split products over the reduction: partial products [S, T, E] at logits
// (S = 1: the logits themselves); gate_gemm_split_count: the S a launch takes
hipError_t launch_gate_gemm_bf16(const uint16_t* x, const uint16_t* w_prep, float* logits,
                                 int64_t T, int d, int E, int S, hipStream_t s);
int gate_gemm_split_count(int64_t T, int d, int E);
hipError_t launch_gate_gemm_simt(const void* x, int x_dtype, const uint16_t* w_prep,
                                 float* logits, int64_t T, int d, int E, hipStream_t s);
bool gate_gemm_bf16_supported(int d, int E);
// the gate product as S split-K partial products [S, T, E] fp32 on the expert
// GEMM kernel (E % 256 == 0, d % 64 == 0); gate_split_count: the S a launch
// takes (0: not supported)
bool gate_split_supported(int d, int E);
int gate_split_count(int64_t T, int d, int E);
hipError_t launch_gate_split_bf16(const uint16_t* x, const uint16_t* planes, float* parts, int64_t T,
                                  int d, int E, int S, const int32_t* offsets, int* tickets,
                                  hipStream_t s);

// selection + block histogram
// logits: nparts partial products [nparts][T, E] summed in order (1: the
// logits themselves); logits_out: where the sums go, or nullptr
hipError_t launch_route_select(const float* logits, int nparts, float* logits_out, const float* bias,
                               const float* offset, int32_t* idx, float* w, int32_t* block_counts,
                               int64_t T, int E, int G, int M, int k, int gk, hipStream_t s);
bool route_select_supported(int E, int G, int k, int gk);

// dispatch
hipError_t launch_dispatch(const int32_t* idx, const int32_t* block_counts, int64_t T, int k,
                           int E, int e_begin, int e_end, const void* x, int x_dtype,
                           int out_dtype, int d, int32_t* counts, int32_t* offsets,
                           int32_t* dest, int32_t* src, void* xp, float* xp_scale, int32_t* base,
                           float* tok_scale, hipStream_t s);

// grouped expert FFN.  `tickets`: a zeroed ticket counter set (kTicketInts
// ints, common.h) that no concurrently running launch shares
// `extra`: one more group after the n_exp groups of the offsets, with its own
// buffers (bf16: x, w13, h for the up-projection; h, w2, y for the down),
// computed in the same launch; NULL or rows = 0: none
hipError_t launch_ffn_up_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                              int d_ff, const uint16_t* xp, const uint16_t* w13, uint16_t* h,
                              int* tickets, hipStream_t s, uint16_t* au = nullptr,
                              const moe_ffn_extra* extra = nullptr);
hipError_t launch_ffn_down_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                                int d_ff, const uint16_t* h, const uint16_t* w2, uint16_t* yp,
                                int* tickets, hipStream_t s, const moe_ffn_extra* extra = nullptr);
// C [rows, N] = A [rows, K] x B_g^T with B_g [N, K] per group (plain bf16 store)
hipError_t launch_ffn_store_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int K, int N,
                                 const uint16_t* A, const uint16_t* B, uint16_t* C, int* tickets,
                                 hipStream_t s);
// backward products (ffn_bwd_bf16.hip)
bool ffn_bwd_bf16_supported(int d, int d_ff);
hipError_t launch_ffn_dgrad_bf16(int n_exp, const int32_t* offsets, int64_t max_rows, int K, int N,
                                 const uint16_t* A, const uint16_t* W, uint16_t* C, hipStream_t s);
// (offsets == nullptr: groups of split_rows consecutive rows, one group when split_rows <= 0)
hipError_t launch_ffn_wgrad_bf16(int n_exp, const int32_t* offsets, int64_t rows_total, int M, int N,
                                 const uint16_t* A, const uint16_t* B, float* C, hipStream_t s,
                                 int split_rows = 0);
// C [rows, N] fp32 += A [rows, K] B [N, K]^T, bf16 operands (K % 128 == 0, K >= 256, N % 256 == 0)
hipError_t launch_gemm_acc_f32(int64_t rows, int K, int N, const uint16_t* A, const uint16_t* B, float* C,
                               int* tickets, hipStream_t s);
hipError_t launch_ffn_simt(int stage, int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                           int d_ff, int dtype, const void* in, const void* w, void* out,
                           hipStream_t s);
hipError_t launch_ffn_up_fp8(int n_exp, const int32_t* offsets, int64_t max_rows, int d, int d_ff,
                             const uint8_t* xp, const float* xp_scale, const uint8_t* w13,
                             const float* w13_scale, uint8_t* h, float* h_scale, hipStream_t s);
hipError_t launch_ffn_down_fp8(int n_exp, const int32_t* offsets, int64_t max_rows, int d,
                               int d_ff, const uint8_t* h, const float* h_scale,
                               const uint8_t* w2, const float* w2_scale, uint16_t* yp,
                               hipStream_t s);
// persistent form (gemm_fp8p.hip) for K % 256 == 0 and K >= 512
bool ffn_fp8p_supported_k(int K);
hipError_t launch_ffn_up_fp8p(int n_exp, const int32_t* offsets, int64_t max_rows, int d, int d_ff,
                              const uint8_t* xp, const float* xp_scale, const uint8_t* w13,
                              const float* w13_scale, uint8_t* h, float* h_scale, int* tickets,
                              hipStream_t s);
hipError_t launch_ffn_down_fp8p(int n_exp, const int32_t* offsets, int64_t max_rows, int d, int d_ff,
                                const uint8_t* h, const float* h_scale, const uint8_t* w2,
                                const float* w2_scale, uint16_t* yp, int* tickets, hipStream_t s);

// combine
hipError_t launch_combine(int64_t T, int k, int d, const int32_t* dest, const float* w,
                          const void* yp, int y_dtype, const void* ysh, void* out,
                          int out_dtype, int accumulate, hipStream_t s);

// weight preparation
// split: the split gate product's ticket set and offsets (kTicketInts + S + 1
// ints, reset by this launch), or nullptr
hipError_t launch_gate_prepare(int d, int E, const float* w_gate, uint16_t* w_prep,
                               hipStream_t s, int* split = nullptr, int S = 0, int64_t T = 0);
hipError_t launch_quantize_rows(int64_t rows, int cols, const uint16_t* x, uint8_t* q, float* scale,
                                hipStream_t s);
hipError_t launch_quantize_blocks(int64_t n, int rows, int cols, const float* w, uint8_t* q,
                                  float* scale, hipStream_t s);

// hash router
hipError_t launch_hash_route(const int32_t* ids, int64_t T, int E, int k, uint64_t seed,
                             const float* logits, int32_t* idx, float* w, int32_t* block_counts,
                             hipStream_t s);

// backward (backward.hip)
hipError_t launch_combine_bwd(int64_t T, int k, int d, const int32_t* dest, const float* w, const void* yp,
                              int y_dtype, const void* g, int g_dtype, uint16_t* d_yp, float* d_w,
                              hipStream_t s);
hipError_t launch_swiglu_bwd(const int32_t* rows_dev, int64_t max_rows, int d_ff, const uint16_t* au,
                             uint16_t* dh, uint16_t* d_au, hipStream_t s);
int gate_bwd_splits(int64_t T);
size_t gate_bwd_workspace_bytes(int64_t T, int d, int E);
hipError_t launch_gate_bwd(int64_t T, int d, int E, int k, const void* x, int x_dtype, const float* w_gate,
                           const float* logits, const float* offset, const int32_t* idx, const float* d_w,
                           float* dL, float* dx, float* dw_gate, float* ws, hipStream_t s);

// load balancing
hipError_t launch_bias_update(int64_t n_rows, int E, const int32_t* counts, float gamma, float* bias,
                              int32_t* load, hipStream_t s);

}  // namespace moe
