// C ABI of libmla: host-side validation, workspace sizing and dispatch. Every entry point checks
// its arguments before enqueueing anything; no entry point allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/mla.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mla_status ok() {
  g_err[0] = 0;
  return MLA_OK;
}

mla_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  if (e == hipErrorNotSupported) return fail(MLA_E_UNSUPPORTED, "%s: no kernel for these dims/dtype", what);
  return fail(MLA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_wdtype(int32_t t) { return t == MLA_F32 || t == MLA_F16 || t == MLA_BF16; }
bool valid_cdtype(int32_t t) {
  return t == MLA_F32 || t == MLA_F16 || t == MLA_BF16 || t == MLA_FP8_E4M3 || t == MLA_FP6_E2M3;
}

// Kernels use 16-byte vector accesses on tensors and workspaces (16-byte alignment required);
// int32 / float arrays read element by element (lengths, block tables, scales) need 4 bytes.
template <typename... P>
bool misaligned(const P*... ptrs) {
  return ((((uintptr_t)(const void*)ptrs) & 15u) || ...);
}
template <typename... P>
bool misaligned4(const P*... ptrs) {
  return ((((uintptr_t)(const void*)ptrs) & 3u) || ...);
}

mla_status check_dims(const mla_dims* d, const char* fn) {
  if (!d) return fail(MLA_E_ARG, "%s: dims is NULL", fn);
  if (d->d <= 0 || d->n_h <= 0 || d->d_h <= 0 || d->d_c <= 0 || d->d_cq <= 0 || d->d_r <= 0)
    return fail(MLA_E_ARG, "%s: every dimension must be > 0", fn);
  if (d->d_r % 8 != 0 || d->d_c % 8 != 0) return fail(MLA_E_ARG, "%s: d_c and d_r must be multiples of 8", fn);
  if (!(d->rope_base > 1.0) || !std::isfinite(d->rope_base)) return fail(MLA_E_ARG, "%s: rope_base must be > 1", fn);
  if (!std::isfinite(d->sm_scale)) return fail(MLA_E_ARG, "%s: sm_scale must be finite", fn);
  if (!std::isfinite(d->yarn_factor)) return fail(MLA_E_ARG, "%s: yarn_factor must be finite", fn);
  if (d->yarn_factor > 1.f) {
    if (d->yarn_orig_len < 1) return fail(MLA_E_ARG, "%s: yarn_orig_len must be >= 1", fn);
    if (!(d->yarn_alpha >= 0.f) || !(d->yarn_beta > d->yarn_alpha) || !std::isfinite(d->yarn_beta))
      return fail(MLA_E_ARG, "%s: YaRN ramp needs 0 <= yarn_alpha < yarn_beta", fn);
  }
  return MLA_OK;
}

mla_status check_cache(const mla_cache* c, const char* fn, mla::CacheArgs* out) {
  if (!c) return fail(MLA_E_ARG, "%s: cache is NULL", fn);
  if (!c->rows) return fail(MLA_E_ARG, "%s: cache rows is NULL", fn);
  if (!valid_cdtype(c->dtype)) return fail(MLA_E_ARG, "%s: bad cache dtype %d", fn, c->dtype);
  if (misaligned(c->rows) || misaligned4(c->scales, c->block_table))
    return fail(MLA_E_ARG, "%s: cache pointers must be 16-byte aligned", fn);
  if ((c->dtype == MLA_FP8_E4M3 || c->dtype == MLA_FP6_E2M3) != (c->scales != nullptr))
    return fail(MLA_E_ARG, "%s: scales must be given exactly for the fp8 and fp6 caches", fn);
  if (c->page_size < 0) return fail(MLA_E_ARG, "%s: page_size < 0", fn);
  if (c->page_size == 0) {
    if (c->t_cap < 1) return fail(MLA_E_ARG, "%s: contiguous cache needs t_cap >= 1", fn);
  } else {
    if (!c->block_table) return fail(MLA_E_ARG, "%s: paged cache needs a block table", fn);
    if (c->max_pages < 1 || c->num_pages < 1) return fail(MLA_E_ARG, "%s: paged cache needs max_pages, num_pages >= 1", fn);
    if (c->t_cap != (int64_t)c->max_pages * c->page_size)
      return fail(MLA_E_ARG, "%s: paged cache t_cap must equal max_pages * page_size", fn);
  }
  out->rows = c->rows;
  out->scales = c->scales;
  out->block_table = c->block_table;
  out->t_cap = c->t_cap;
  out->dtype = c->dtype;
  out->page_size = c->page_size;
  out->max_pages = c->max_pages;
  out->num_pages = c->num_pages;
  return MLA_OK;
}

float resolve_scale(const mla_dims* d) {
  if (d->sm_scale > 0.f) return d->sm_scale;
  double t = 1.0;  // YaRN attention temperature on the default scale
  if (d->yarn_factor > 1.f) {
    const double m = 0.1 * std::log((double)d->yarn_factor) + 1.0;
    t = m * m;
  }
  return (float)(t / std::sqrt((double)(d->d_h + d->d_r)));
}

}  // namespace

namespace mla {
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}
}  // namespace mla

// ------------------------------------------------------------------------------------------------
// Scratch of mla_absorb_out_noalloc: a file-scope device array (each GPU the library runs on holds
// its own copy, at its own address, until the process ends). In host code `scratch` is only a
// stand-in symbol, never a device address: its address on the current device is looked up once per
// device with hipGetSymbolAddress and only that pointer is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (resolved on the first call on that device).
mla_status scratch_on_current_device(void** out, const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_E_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_E_UNSUPPORTED, "%s: device ordinal %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLA_E_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}
}  // namespace

// Default range count: one per CU at the DeepSeek-V2 shape (the MFMA kernels hold a CU each);
// two per CU otherwise, so that the latency-bound generic kernel has two workgroups per CU.
static int resolve_splits(const mla_dims* d, int32_t num_splits) {
  if (num_splits > 0) return num_splits;
  const bool v2 = d->n_h == 128 && d->d_c == 512 && d->d_r == 64;
  const int n = mla::device_cu_count() * (v2 ? 1 : 2);
  return n < 1024 ? n : 1024;
}

extern "C" {

const char* mla_version(void) { return "mla_latent_kv_25_amd 0.1 (gfx950)"; }
const char* mla_last_error(void) { return g_err; }

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_E_ARG: return "MLA_E_ARG";
    case MLA_E_UNSUPPORTED: return "MLA_E_UNSUPPORTED";
    case MLA_E_WORKSPACE: return "MLA_E_WORKSPACE";
    case MLA_E_HIP: return "MLA_E_HIP";
  }
  return "MLA_E_?";
}

size_t mla_absorb_q_workspace_bytes(const mla_dims* dims, int32_t B) {
  if (!dims || B <= 0) return 0;
  return mla::absorb_q_layout(*dims, B).bytes;
}

mla_status mla_absorb_q(const mla_dims* dims, int32_t B, int32_t wdtype, const void* h, const void* W_dq,
                        const void* W_uq, const void* W_qr, const void* W_uk, const void* W_dkv, const void* W_kr,
                        void* workspace, size_t ws_bytes, float* q_lat, float* q_pe, float* kv_new,
                        hipStream_t stream) {
  const char* fn = "mla_absorb_q";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (B == 0) return ok();
  if (!h || !W_dq || !W_uq || !W_qr || !W_uk || !W_dkv || !W_kr || !q_lat || !q_pe || !kv_new)
    return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(h, W_dq, W_uq, W_qr, W_uk, W_dkv, W_kr, q_lat, q_pe, kv_new, workspace))
    return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  if (!workspace || ws_bytes < mla_absorb_q_workspace_bytes(dims, B))
    return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, mla_absorb_q_workspace_bytes(dims, B));
  return hip_status(mla::launch_absorb_q(*dims, B, wdtype, h, W_dq, W_uq, W_qr, W_uk, W_dkv, W_kr, workspace, q_lat,
                                         q_pe, kv_new, stream),
                    fn);
}

mla_status mla_rope(const mla_dims* dims, int32_t B, const int32_t* seq_lens, float* q_pe, float* kv_new,
                    const mla_cache* cache, hipStream_t stream) {
  const char* fn = "mla_rope";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (B == 0) return ok();
  if (!seq_lens || !q_pe || !kv_new) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(q_pe, kv_new) || misaligned4(seq_lens)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  mla::CacheArgs c{};
  if (cache) {
    s = check_cache(cache, fn, &c);
    if (s) return s;
  }
  return hip_status(mla::launch_rope(*dims, B, seq_lens, q_pe, kv_new, cache ? &c : nullptr, stream), fn);
}

size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t B, int32_t num_splits) {
  if (!dims || B <= 0 || num_splits < 0) return 0;
  return mla::decode_layout(*dims, B, resolve_splits(dims, num_splits)).bytes;
}

mla_status mla_decode_attn(const mla_dims* dims, int32_t B, const float* q_lat, const float* q_pe,
                           const mla_cache* cache, const int32_t* seq_lens, int32_t num_splits, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
  const char* fn = "mla_decode_attn";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (num_splits < 0 || num_splits > 1024) return fail(MLA_E_ARG, "%s: num_splits must be in [0, 1024]", fn);
  mla::CacheArgs c{};
  s = check_cache(cache, fn, &c);
  if (s) return s;
  if (B == 0) return ok();
  if (!q_lat || !q_pe || !seq_lens) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(q_lat, q_pe, workspace) || misaligned4(seq_lens)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  if (!mla::decode_supported(*dims, c.dtype, c.page_size))
    return fail(MLA_E_UNSUPPORTED, "%s: no decode kernel for n_h=%d d_c=%d d_r=%d with cache dtype %d", fn,
                dims->n_h, dims->d_c, dims->d_r, c.dtype);
  const int G = resolve_splits(dims, num_splits);
  const size_t need = mla::decode_layout(*dims, B, G).bytes;
  if (!workspace || ws_bytes < need) return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  return hip_status(mla::launch_decode(*dims, B, q_lat, q_pe, c, seq_lens, G, resolve_scale(dims), workspace, stream),
                    fn);
}

mla_status mla_combine(const mla_dims* dims, int32_t B, int32_t num_splits, const int32_t* seq_lens,
                       const void* workspace, size_t ws_bytes, float* o_lat, float* lse, hipStream_t stream) {
  const char* fn = "mla_combine";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (num_splits < 0 || num_splits > 1024) return fail(MLA_E_ARG, "%s: num_splits must be in [0, 1024]", fn);
  if (B == 0) return ok();
  if (!seq_lens || !o_lat) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(o_lat, workspace) || misaligned4(seq_lens, lse)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  const int G = resolve_splits(dims, num_splits);
  const size_t need = mla::decode_layout(*dims, B, G).bytes;
  if (!workspace || ws_bytes < need) return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  return hip_status(mla::launch_combine(*dims, B, G, workspace, o_lat, lse, stream), fn);
}

size_t mla_absorb_out_workspace_bytes(const mla_dims* dims, int32_t B) {
  if (!dims || B <= 0) return 0;
  return mla::absorb_out_layout(*dims, B).bytes;
}

mla_status mla_absorb_out(const mla_dims* dims, int32_t B, int32_t wdtype, const float* o_lat, const void* W_uv,
                          const void* W_o, void* workspace, size_t ws_bytes, float* u, hipStream_t stream) {
  const char* fn = "mla_absorb_out";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (B == 0) return ok();
  if (!o_lat || !W_uv || !W_o || !u) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(o_lat, W_uv, W_o, u, workspace)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  if (!workspace || ws_bytes < mla_absorb_out_workspace_bytes(dims, B))
    return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, mla_absorb_out_workspace_bytes(dims, B));
  return hip_status(mla::launch_absorb_out(*dims, B, wdtype, o_lat, W_uv, W_o, workspace, u, stream), fn);
}

mla_status mla_combine_absorb_out(const mla_dims* dims, int32_t B, int32_t wdtype, int32_t num_splits,
                                  const void* dec_workspace, size_t dec_ws_bytes, const void* W_uv, const void* W_o,
                                  void* workspace, size_t ws_bytes, float* u, float* lse, hipStream_t stream) {
  const char* fn = "mla_combine_absorb_out";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (num_splits < 0 || num_splits > 1024) return fail(MLA_E_ARG, "%s: num_splits must be in [0, 1024]", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  const int G = resolve_splits(dims, num_splits);
  if (wdtype != MLA_BF16 || !mla::naive_supported(*dims) || !mla::combine_uv_supported(*dims, G))
    return fail(MLA_E_UNSUPPORTED, "%s: needs bf16 weights, d_h=128, d_c=512, d_r=64 (use mla_combine + "
                "mla_absorb_out)", fn);
  if (B == 0) return ok();
  if (!dec_workspace || !W_uv || !W_o || !u) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(dec_workspace, W_uv, W_o, u, workspace) || misaligned4(lse))
    return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  const size_t need_d = mla::decode_layout(*dims, B, G).bytes;
  if (dec_ws_bytes < need_d) return fail(MLA_E_WORKSPACE, "%s: decode workspace needs %zu bytes", fn, need_d);
  const size_t need = mla_absorb_out_workspace_bytes(dims, B);
  if (!workspace || ws_bytes < need) return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  const mla::AbsorbOutLayout L = mla::absorb_out_layout(*dims, B);
  void* o = (char*)workspace + L.off_o;  // bf16 per-head outputs
  hipError_t e = mla::launch_combine_uv(*dims, B, G, dec_workspace, W_uv, o, lse, stream);
  if (e == hipSuccess) e = mla::launch_output_proj(*dims, B, o, true, W_o, (char*)workspace + L.off_part, u, stream);
  return hip_status(e, fn);
}

mla_status mla_absorb_out_noalloc(const mla_dims* dims, int32_t B, int32_t wdtype, const float* o_lat,
                                  const void* W_uv, const void* W_o, float* u, hipStream_t stream) {
  const char* fn = "mla_absorb_out_noalloc";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (B == 0) return ok();
  if (!o_lat || !W_uv || !W_o || !u) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(o_lat, W_uv, W_o, u)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  const size_t need = mla_absorb_out_workspace_bytes(dims, B);
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_E_WORKSPACE, "%s: B=%d needs %zu bytes of scratch, more than the %zu the library holds", fn, B,
                need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  s = scratch_on_current_device(&ws, fn);
  if (s) return s;
  return hip_status(mla::launch_absorb_out(*dims, B, wdtype, o_lat, W_uv, W_o, ws, u, stream), fn);
}

mla_status mla_precombine(const mla_dims* dims, int32_t wdtype, const void* W_uq, const void* W_uk,
                          const void* W_uv, const void* W_o, void* Wq_pre, void* Wo_pre, hipStream_t stream) {
  const char* fn = "mla_precombine";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (!Wq_pre && !Wo_pre) return ok();
  if (Wq_pre && (!W_uq || !W_uk)) return fail(MLA_E_ARG, "%s: Wq_pre needs W_uq and W_uk", fn);
  if (Wo_pre && (!W_uv || !W_o)) return fail(MLA_E_ARG, "%s: Wo_pre needs W_uv and W_o", fn);
  if (misaligned(W_uq, W_uk, W_uv, W_o, Wq_pre, Wo_pre)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  return hip_status(mla::launch_precombine(*dims, wdtype, W_uq, W_uk, W_uv, W_o, Wq_pre, Wo_pre, stream), fn);
}

mla_status mla_absorb_q_pre(const mla_dims* dims, int32_t B, int32_t wdtype, const void* h, const void* W_dq,
                            const void* Wq_pre, const void* W_qr, const void* W_dkv, const void* W_kr,
                            void* workspace, size_t ws_bytes, float* q_lat, float* q_pe, float* kv_new,
                            hipStream_t stream) {
  const char* fn = "mla_absorb_q_pre";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (B == 0) return ok();
  if (!h || !W_dq || !Wq_pre || !W_qr || !W_dkv || !W_kr || !q_lat || !q_pe || !kv_new)
    return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(h, W_dq, Wq_pre, W_qr, W_dkv, W_kr, q_lat, q_pe, kv_new, workspace))
    return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  if (!workspace || ws_bytes < mla_absorb_q_workspace_bytes(dims, B))
    return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, mla_absorb_q_workspace_bytes(dims, B));
  return hip_status(mla::launch_absorb_q_pre(*dims, B, wdtype, h, W_dq, Wq_pre, W_qr, W_dkv, W_kr, workspace, q_lat,
                                             q_pe, kv_new, stream),
                    fn);
}

size_t mla_absorb_out_pre_workspace_bytes(const mla_dims* dims, int32_t B) {
  if (!dims || B <= 0) return 0;
  return mla::absorb_out_pre_layout(*dims, B).bytes;
}

mla_status mla_absorb_out_pre(const mla_dims* dims, int32_t B, int32_t wdtype, const float* o_lat,
                              const void* Wo_pre, void* workspace, size_t ws_bytes, float* u, hipStream_t stream) {
  const char* fn = "mla_absorb_out_pre";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (B == 0) return ok();
  if (!o_lat || !Wo_pre || !u) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(o_lat, Wo_pre, u, workspace)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  const size_t need = mla_absorb_out_pre_workspace_bytes(dims, B);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  return hip_status(mla::launch_absorb_out_pre(*dims, B, wdtype, o_lat, Wo_pre, workspace, u, stream), fn);
}

mla_status mla_prefill_tables(const mla_cache* cache, int32_t B, int32_t C, const int32_t* p0,
                              int32_t* seq_lens_out, int32_t* block_table_out, hipStream_t stream) {
  const char* fn = "mla_prefill_tables";
  if (!cache) return fail(MLA_E_ARG, "%s: cache is NULL", fn);
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (C < 1) return fail(MLA_E_ARG, "%s: chunk length C must be >= 1", fn);
  if ((int64_t)B * C > (int64_t)INT32_MAX / 2) return fail(MLA_E_ARG, "%s: B * C too large", fn);
  if (cache->page_size <= 0 || !cache->block_table || cache->max_pages <= 0)
    return fail(MLA_E_ARG, "%s: the cache must be paged (page_size > 0, block table, max_pages > 0)", fn);
  if (B == 0) return ok();
  if (!p0 || !seq_lens_out || !block_table_out) return fail(MLA_E_ARG, "%s: NULL pointer", fn);
  if (misaligned4(p0, seq_lens_out, block_table_out, cache->block_table))
    return fail(MLA_E_ARG, "%s: pointers must be 4-byte aligned", fn);
  return hip_status(mla::launch_prefill_tables(B, C, cache->max_pages, p0, cache->block_table, seq_lens_out,
                                               block_table_out, stream), fn);
}

mla_status mla_absorb_q_naive(const mla_dims* dims, int32_t B, int32_t wdtype, const void* h, const void* W_dq,
                              const void* W_uq, const void* W_qr, const void* W_dkv, const void* W_kr,
                              void* workspace, size_t ws_bytes, float* q_c, float* q_pe, float* kv_new,
                              hipStream_t stream) {
  const char* fn = "mla_absorb_q_naive";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (wdtype != MLA_BF16 || !mla::naive_supported(*dims))
    return fail(MLA_E_UNSUPPORTED, "%s: the naive form needs bf16 weights, d_h=128, d_c=512, d_r=64", fn);
  if (B == 0) return ok();
  if (!h || !W_dq || !W_uq || !W_qr || !W_dkv || !W_kr || !q_c || !q_pe || !kv_new)
    return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(h, W_dq, W_uq, W_qr, W_dkv, W_kr, q_c, q_pe, kv_new, workspace))
    return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  if (!workspace || ws_bytes < mla_absorb_q_workspace_bytes(dims, B))
    return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, mla_absorb_q_workspace_bytes(dims, B));
  return hip_status(mla::launch_absorb_q_naive(*dims, B, h, W_dq, W_uq, W_qr, W_dkv, W_kr, workspace, q_c, q_pe,
                                               kv_new, stream),
                    fn);
}

size_t mla_prefill_naive_workspace_bytes(const mla_dims* dims, int32_t B, int32_t max_ctx) {
  if (!dims || B <= 0 || max_ctx <= 0 || dims->n_h <= 0) return 0;
  return mla::naive_layout(dims->n_h, B, max_ctx).bytes;
}

mla_status mla_prefill_naive_attn(const mla_dims* dims, int32_t B, int32_t C, int32_t wdtype, const float* q_c,
                                  const float* q_pe, const mla_cache* cache, const int32_t* p0, int32_t max_ctx,
                                  const void* W_uk, const void* W_uv, void* workspace, size_t ws_bytes, void* o,
                                  hipStream_t stream) {
  const char* fn = "mla_prefill_naive_attn";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  mla::CacheArgs c{};
  s = check_cache(cache, fn, &c);
  if (s) return s;
  if (B < 0) return fail(MLA_E_ARG, "%s: B < 0", fn);
  if (C < 1) return fail(MLA_E_ARG, "%s: chunk length C must be >= 1", fn);
  if (max_ctx < C) return fail(MLA_E_ARG, "%s: max_ctx must be >= C", fn);
  if ((int64_t)max_ctx > c.t_cap) return fail(MLA_E_ARG, "%s: max_ctx exceeds the cache capacity", fn);
  if ((int64_t)B * C > (int64_t)INT32_MAX / 2 || (int64_t)B * max_ctx > (int64_t)INT32_MAX / 2 ||
      (int64_t)((C + 127) / 128) * dims->n_h * B > (int64_t)INT32_MAX - 8)
    return fail(MLA_E_ARG, "%s: B * C, B * max_ctx or the attention grid too large", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (wdtype != MLA_BF16 || c.dtype != MLA_BF16 || !mla::naive_supported(*dims))
    return fail(MLA_E_UNSUPPORTED, "%s: the naive form needs bf16 weights and cache, d_h=128, d_c=512, d_r=64", fn);
  if (B == 0) return ok();
  if (!q_c || !q_pe || !p0 || !W_uk || !W_uv || !o) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(q_c, q_pe, W_uk, W_uv, o, workspace) || misaligned4(p0))
    return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  const size_t need = mla_prefill_naive_workspace_bytes(dims, B, max_ctx);
  if (!workspace || ws_bytes < need) return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  const mla::NaiveLayout L = mla::naive_layout(dims->n_h, B, max_ctx);
  char* ws = (char*)workspace;
  hipError_t e = mla::launch_gather_rows(c, B, C, p0, max_ctx, ws + L.off_ctx, stream);
  if (e == hipSuccess)
    e = mla::launch_materialize_kv(*dims, B * max_ctx, ws + L.off_ctx, W_uk, W_uv, ws + L.off_kc, ws + L.off_v, stream);
  if (e == hipSuccess)
    e = mla::launch_mha_prefill(B, C, max_ctx, dims->n_h, p0, q_c, q_pe, workspace,
                                resolve_scale(dims) * 1.4426950408889634f, o, stream);
  return hip_status(e, fn);
}

size_t mla_output_proj_workspace_bytes(const mla_dims* dims, int32_t N) {
  if (!dims || N <= 0) return 0;
  return mla::output_proj_layout(*dims, N).bytes;
}

mla_status mla_output_proj(const mla_dims* dims, int32_t N, int32_t wdtype, int32_t odtype, const void* o,
                           const void* W_o, void* workspace, size_t ws_bytes, float* u, hipStream_t stream) {
  const char* fn = "mla_output_proj";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  if (N < 0) return fail(MLA_E_ARG, "%s: N < 0", fn);
  if (!valid_wdtype(wdtype)) return fail(MLA_E_ARG, "%s: weight dtype must be F32, F16 or BF16", fn);
  if (odtype != MLA_F32 && odtype != MLA_BF16) return fail(MLA_E_ARG, "%s: o must be F32 or BF16", fn);
  if (wdtype != MLA_BF16 || !mla::naive_supported(*dims))
    return fail(MLA_E_UNSUPPORTED, "%s: needs bf16 weights and the MFMA GEMM shapes", fn);
  if (N == 0) return ok();
  if (!o || !W_o || !u) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(o, W_o, u, workspace)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  const size_t need = mla_output_proj_workspace_bytes(dims, N);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(MLA_E_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  return hip_status(mla::launch_output_proj(*dims, N, o, odtype == MLA_BF16, W_o, workspace, u, stream), fn);
}

mla_status mla_cache_store(const mla_dims* dims, const mla_cache* cache, int32_t B, const int32_t* n_rows,
                           int32_t max_rows, const float* src, int64_t src_stride, hipStream_t stream) {
  const char* fn = "mla_cache_store";
  mla_status s = check_dims(dims, fn);
  if (s) return s;
  mla::CacheArgs c{};
  s = check_cache(cache, fn, &c);
  if (s) return s;
  if (B < 0 || max_rows < 0) return fail(MLA_E_ARG, "%s: B and max_rows must be >= 0", fn);
  if (B == 0 || max_rows == 0) return ok();
  if (!n_rows || !src) return fail(MLA_E_ARG, "%s: NULL tensor pointer", fn);
  if (misaligned(src) || misaligned4(n_rows)) return fail(MLA_E_ARG, "%s: pointers must be 16-byte aligned", fn);
  if (src_stride < max_rows) return fail(MLA_E_ARG, "%s: src_stride < max_rows", fn);
  if (max_rows > c.t_cap) return fail(MLA_E_ARG, "%s: max_rows exceeds the cache capacity", fn);
  return hip_status(mla::launch_cache_store(*dims, c, B, n_rows, max_rows, src, src_stride, stream), fn);
}

mla_status mla_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const char* fn = "mla_stream_read";
  if (!src || !sink) return fail(MLA_E_ARG, "%s: NULL pointer", fn);
  if (bytes == 0 || bytes % 16) return fail(MLA_E_ARG, "%s: bytes must be a positive multiple of 16", fn);
  if (misaligned(src) || misaligned4(sink)) return fail(MLA_E_ARG, "%s: src must be 16-byte aligned, sink 4-byte", fn);
  return hip_status(mla::launch_stream_read(src, bytes, sink, stream), fn);
}

}  // extern "C"
