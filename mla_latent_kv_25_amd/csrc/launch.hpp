// Internal launch interface between the C-ABI layer (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

// Plain-value copy of mla_cache passed by value to kernels.
struct CacheArgs {
  void* rows;
  float* scales;
  const int32_t* block_table;
  int64_t t_cap;
  int32_t dtype;
  int32_t page_size;
  int32_t max_pages;
  int32_t num_pages;
};

// Workspace layout of mla_decode_attn / mla_combine (byte offsets).
struct DecodeLayout {
  int64_t n_pieces;   // num_splits + B - 1
  size_t off_cu;      // int64 [B + 1] prefix sums of seq_lens
  size_t off_fmt;     // int32: partial-output format (0 float32, 2 scaled float16)
  size_t off_lse;     // float [n_pieces, n_h]
  size_t off_sc;      // float [n_pieces, n_h]: row scales of float16 partials
  size_t off_o;       // float or float16 [n_pieces, n_h, d_c]
  size_t off_q8;      // MFMA shape only: the query in operand form [B, n_h, 1152 bytes]
  size_t off_fh;      // MFMA shape only: float [B, n_h], 2^-e of each head's query scaling
  size_t bytes;
};
DecodeLayout decode_layout(const mla_dims& d, int B, int G);

// GEMM workspace layouts.
struct AbsorbQLayout { size_t off_cq, off_qc, off_part, part_floats, bytes; };
AbsorbQLayout absorb_q_layout(const mla_dims& d, int B);
struct AbsorbOutLayout { size_t off_o, off_part, part_floats, bytes; };
AbsorbOutLayout absorb_out_layout(const mla_dims& d, int B);
AbsorbOutLayout absorb_out_pre_layout(const mla_dims& d, int B);

hipError_t launch_rope(const mla_dims& d, int B, const int32_t* seq_lens, float* q_pe, float* kv_new,
                       const CacheArgs* cache, hipStream_t st);
hipError_t launch_prefill_tables(int B, int C, int max_pages, const int32_t* p0, const int32_t* bt_in,
                                 int32_t* seq_lens_out, int32_t* bt_out, hipStream_t st);
hipError_t launch_cache_store(const mla_dims& d, const CacheArgs& c, int B, const int32_t* n_rows,
                              int max_rows, const float* src, int64_t src_stride, hipStream_t st);

// Returns hipErrorNotSupported (nothing launched) when no kernel covers the dims/dtype.
hipError_t launch_decode(const mla_dims& d, int B, const float* q_lat, const float* q_pe,
                         const CacheArgs& c, const int32_t* seq_lens, int G, float sm_scale,
                         void* ws, hipStream_t st);
bool decode_supported(const mla_dims& d, int cache_dtype, int page_size);
hipError_t launch_combine(const mla_dims& d, int B, int G, const void* ws, float* o_lat, float* lse,
                          hipStream_t st);

hipError_t launch_absorb_q(const mla_dims& d, int B, int wdtype, const void* h, const void* W_dq,
                           const void* W_uq, const void* W_qr, const void* W_uk, const void* W_dkv,
                           const void* W_kr, void* ws, float* q_lat, float* q_pe, float* kv_new,
                           hipStream_t st);
hipError_t launch_absorb_out(const mla_dims& d, int B, int wdtype, const float* o_lat, const void* W_uv,
                             const void* W_o, void* ws, float* u, hipStream_t st);

// Pre-combined absorption (W~^Q, W~^O): building the matrices and the two products that use them.
hipError_t launch_precombine(const mla_dims& d, int wdt, const void* W_uq, const void* W_uk, const void* W_uv,
                             const void* W_o, void* Wq_pre, void* Wo_pre, hipStream_t st);
hipError_t launch_absorb_q_pre(const mla_dims& d, int B, int wdt, const void* h, const void* W_dq,
                               const void* Wq_pre, const void* W_qr, const void* W_dkv, const void* W_kr, void* ws,
                               float* q_lat, float* q_pe, float* kv_new, hipStream_t st);
hipError_t launch_absorb_out_pre(const mla_dims& d, int B, int wdt, const float* o_lat, const void* Wo_pre, void* ws,
                                 float* u, hipStream_t st);

// Naive-form prefill (k_naive.hip, k_gemm.hip): workspace of gathered rows [B, max_ctx, d_c + d_r]
// bf16, K^C [B * max_ctx, n_h d_h] bf16 and V [B * max_ctx, n_h d_h] bf16 (d_h = 128, d_c = 512, d_r = 64).
struct NaiveLayout { size_t off_ctx, off_kc, off_v, bytes; };
NaiveLayout naive_layout(int n_h, int B, int max_ctx);
hipError_t launch_gather_rows(const CacheArgs& c, int B, int C, const int32_t* p0, int max_ctx, void* ctx,
                              hipStream_t st);
hipError_t launch_mha_prefill(int B, int C, int max_ctx, int n_h, const int32_t* p0, const float* q_c,
                              const float* q_pe, const void* ws, float qscale, void* o, hipStream_t st);
hipError_t launch_absorb_q_naive(const mla_dims& d, int B, const void* h, const void* W_dq, const void* W_uq,
                                 const void* W_qr, const void* W_dkv, const void* W_kr, void* ws, float* q_c,
                                 float* q_pe, float* kv_new, hipStream_t st);
hipError_t launch_materialize_kv(const mla_dims& d, int R, const void* ctx, const void* W_uk, const void* W_uv,
                                 void* kc, void* vv, hipStream_t st);
AbsorbOutLayout output_proj_layout(const mla_dims& d, int N);
hipError_t launch_output_proj(const mla_dims& d, int N, const void* o, bool o_bf16, const void* W_o, void* ws,
                              float* u, hipStream_t st);
bool naive_supported(const mla_dims& d);

// Combine fused with the W^UV product (k_decode.hip): o [B, n_h d_h] bf16 from the decode
// workspace's pieces; V2 head shape (d_c = 512, d_h = 128), bf16 W^UV.
bool combine_uv_supported(const mla_dims& d, int G);
hipError_t launch_combine_uv(const mla_dims& d, int B, int G, const void* ws, const void* W_uv, void* o, float* lse,
                             hipStream_t st);

int device_cu_count();

// Read-only streaming ceiling (k_stream.hip).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace mla
