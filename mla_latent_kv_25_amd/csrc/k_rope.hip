// Decoupled rotary embedding + cache append, and the prefix cache fill.
//
// "DeepSeek-V2 from Scratch" section 3.1: RoPE is a position-dependent rotation; sections 4.1-4.2:
// every head has its own rotary query q^R_i, all heads share one rotary key k^R; section 4.5: k^R
// is stored already rotated next to the latent c^KV. Pairs (x[2m], x[2m+1]) turn by
// pos * base^(-2m/d_r); angles are formed and evaluated in float64 so that positions up to 2^17
// keep full float32 accuracy in the rotated values. The DeepSeek-V2 review page ("4. Pre-Training")
// extends the context of k^R with YaRN; with a factor s > 1 each pair's frequency is blended
// between theta / s and theta by the published ramp over its turns in the original context.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

// Row address of cached token j of sequence b (element index, not bytes).
__device__ __forceinline__ int64_t cache_row_index(const CacheArgs& c, int b, int64_t j) {
  if (c.page_size == 0) return (int64_t)b * c.t_cap + j;
  int32_t page = c.block_table[(int64_t)b * c.max_pages + j / c.page_size];
  return (int64_t)page * c.page_size + (j % c.page_size);
}

// Four e2m3 codes of consecutive elements -> the 3 bytes of their 24 bits in the row's little-endian
// 6-bit stream (code j at bits 6j .. 6j + 5; rows hold a multiple of 4 codes).
__device__ __forceinline__ void store_e2m3x4(uint8_t* row, int g, const float* v, float scale) {
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) bits |= f32_to_e2m3(v[k] / scale) << (6 * k);
  row[3 * g] = (uint8_t)bits;
  row[3 * g + 1] = (uint8_t)(bits >> 8);
  row[3 * g + 2] = (uint8_t)(bits >> 16);
}

// Store one row held by a 256-thread block in `vals` (LDS, float32, `rw` values).
// fp8: scale = amax / 448 (1 for an all-zero row), code = e4m3(x / scale).
// fp6: scale = amax / 7.5 (1 for an all-zero row), code = e2m3(x / scale), packed 6 bits each.
__device__ void store_row_block(const CacheArgs& c, int64_t ridx, const float* vals, int rw,
                                float* red) {
  const int tid = threadIdx.x;
  if (c.dtype == MLA_FP8_E4M3 || c.dtype == MLA_FP6_E2M3) {
    float a = 0.f;
    for (int e = tid; e < rw; e += blockDim.x) a = fmaxf(a, fabsf(vals[e]));
    a = wave_max(a);
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    float amax = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);
    if (c.dtype == MLA_FP6_E2M3) {
      const float scale = amax == 0.f ? 1.f : amax / 7.5f;
      uint8_t* dst = (uint8_t*)c.rows + ridx * (rw / 4 * 3);
      for (int g = tid; g < rw / 4; g += blockDim.x) store_e2m3x4(dst, g, vals + 4 * g, scale);
      if (tid == 0) c.scales[ridx] = scale;
      return;
    }
    float scale = amax == 0.f ? 1.f : amax / 448.0f;
    uint8_t* dst = (uint8_t*)c.rows + ridx * rw;
    for (int e = tid; e < rw; e += blockDim.x) dst[e] = (uint8_t)f32_to_e4m3(vals[e] / scale);
    if (tid == 0) c.scales[ridx] = scale;
    return;
  }
  for (int e = tid; e < rw; e += blockDim.x) {
    float v = vals[e];
    if (c.dtype == MLA_F32) ((float*)c.rows)[ridx * rw + e] = v;
    else if (c.dtype == MLA_BF16) ((uint16_t*)c.rows)[ridx * rw + e] = f32_to_bf16_bits(v);
    else ((uint16_t*)c.rows)[ridx * rw + e] = f32_to_f16_bits(v);
  }
}

// Grid (B, 1 + head blocks): blockIdx.y == 0 rotates k^R and appends the row; block y > 0
// rotates the queries of heads [(y-1) * RH, y * RH). Each block forms the cos/sin table itself.
constexpr int RH = 32;
// Rotary frequency of pair m: base^(-2m/d_r), or its YaRN blend when s > 1 (the pair's turns
// over the original context, r = L theta / 2pi, pick theta / s below alpha, theta above beta and a
// linear mix in between).
struct RopeFreq {
  double base, s, L, alpha, beta;
  __device__ double operator()(int m, int d_r) const {
    const double theta = pow(base, -2.0 * (double)m / (double)d_r);
    if (!(s > 1.0)) return theta;
    const double r = L * theta * 0.15915494309189533577;  // 1 / (2 pi)
    const double g = r < alpha ? 0.0 : (r > beta ? 1.0 : (r - alpha) / (beta - alpha));
    return (1.0 - g) * theta / s + g * theta;
  }
};

__global__ __launch_bounds__(256) void k_rope_append(int n_h, int d_c, int d_r, RopeFreq freq,
                                                      const int32_t* __restrict__ seq_lens,
                                                      float* __restrict__ q_pe, float* __restrict__ kv_new,
                                                      CacheArgs cache, int write_cache) {
  extern __shared__ float sm[];
  const int rw = d_c + d_r;
  const int half = d_r / 2;
  float* cs = sm;                 // [half] cos
  float* sn = sm + half;          // [half] sin
  float* row = sm + 2 * half;     // [rw] the row to store
  float* red = row + rw;          // [4]
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int pos = seq_lens[b] - 1;
  // a zero-length sequence (outside the contract) has no current token: nothing is rotated and no
  // row is stored (pos = -1 would address the row before the sequence's first one)
  if (pos < 0) return;
  for (int m = tid; m < half; m += blockDim.x) {
    double ang = (double)pos * freq(m, d_r);
    double s, c;
    sincos(ang, &s, &c);
    cs[m] = (float)c;
    sn[m] = (float)s;
  }
  __syncthreads();
  if (blockIdx.y > 0) {
    // rotary queries of this block's heads; one thread per (head, pair), pairs read as float2
    const int h0 = (blockIdx.y - 1) * RH;
    const int nh = (n_h - h0) < RH ? (n_h - h0) : RH;
    float2* q = (float2*)(q_pe + ((int64_t)b * n_h + h0) * d_r);
    for (int i = tid; i < nh * half; i += blockDim.x) {
      const int m = i % half;
      const float2 x = q[i];
      q[i] = float2{x.x * cs[m] - x.y * sn[m], x.x * sn[m] + x.y * cs[m]};
    }
    return;
  }
  // shared rotary key (after the latent in the row)
  float* kv = kv_new + (int64_t)b * rw;
  for (int m = tid; m < half; m += blockDim.x) {
    float x0 = kv[d_c + 2 * m], x1 = kv[d_c + 2 * m + 1];
    float y0 = x0 * cs[m] - x1 * sn[m];
    float y1 = x0 * sn[m] + x1 * cs[m];
    kv[d_c + 2 * m] = y0;
    kv[d_c + 2 * m + 1] = y1;
    row[d_c + 2 * m] = y0;
    row[d_c + 2 * m + 1] = y1;
  }
  for (int e = tid; e < d_c; e += blockDim.x) row[e] = kv[e];
  __syncthreads();
  if (write_cache) store_row_block(cache, cache_row_index(cache, b, pos), row, rw, red);
}

// Prefix fill: one wave per row. Rows of sequence b: j < n_rows[b] <= max_rows.
__global__ __launch_bounds__(256) void k_cache_store(int rw, CacheArgs cache,
                                                      const int32_t* __restrict__ n_rows,
                                                      const float* __restrict__ src, int64_t src_stride) {
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + wave;
  if (j >= n_rows[b]) return;
  const float* s = src + ((int64_t)b * src_stride + j) * rw;
  const int64_t ridx = cache_row_index(cache, b, j);
  if (cache.dtype == MLA_FP6_E2M3) {
    float a = 0.f;
    for (int e = lane; e < rw; e += 64) a = fmaxf(a, fabsf(s[e]));
    a = wave_max(a);
    const float scale = a == 0.f ? 1.f : a / 7.5f;
    uint8_t* dst = (uint8_t*)cache.rows + ridx * (rw / 4 * 3);
    for (int g = lane; g < rw / 4; g += 64) store_e2m3x4(dst, g, s + 4 * g, scale);
    if (lane == 0) cache.scales[ridx] = scale;
    return;
  }
  if (cache.dtype == MLA_FP8_E4M3) {
    float a = 0.f;
    for (int e = lane; e < rw; e += 64) a = fmaxf(a, fabsf(s[e]));
    a = wave_max(a);
    float scale = a == 0.f ? 1.f : a / 448.0f;
    uint8_t* dst = (uint8_t*)cache.rows + ridx * rw;
    for (int e = lane; e < rw; e += 64) dst[e] = (uint8_t)f32_to_e4m3(s[e] / scale);
    if (lane == 0) cache.scales[ridx] = scale;
    return;
  }
  for (int e = lane; e < rw; e += 64) {
    float v = s[e];
    if (cache.dtype == MLA_F32) ((float*)cache.rows)[ridx * rw + e] = v;
    else if (cache.dtype == MLA_BF16) ((uint16_t*)cache.rows)[ridx * rw + e] = f32_to_bf16_bits(v);
    else ((uint16_t*)cache.rows)[ridx * rw + e] = f32_to_f16_bits(v);
  }
}

// Chunked prefill as causal pseudo-sequences: pseudo-sequence b * C + t is token t of sequence
// b's chunk; it attends to rows 0 .. p0[b] + t and shares sequence b's pages (block-table row
// copied). One block per pseudo-sequence.
__global__ __launch_bounds__(256) void k_prefill_tables(int C, int max_pages, const int32_t* __restrict__ p0,
                                                         const int32_t* __restrict__ bt_in,
                                                         int32_t* __restrict__ seq_lens_out,
                                                         int32_t* __restrict__ bt_out) {
  const int ps = blockIdx.x;
  const int b = ps / C, t = ps - b * C;
  if (threadIdx.x == 0) seq_lens_out[ps] = p0[b] + t + 1;
  for (int j = threadIdx.x; j < max_pages; j += blockDim.x)
    bt_out[(int64_t)ps * max_pages + j] = bt_in[(int64_t)b * max_pages + j];
}

hipError_t launch_prefill_tables(int B, int C, int max_pages, const int32_t* p0, const int32_t* bt_in,
                                 int32_t* seq_lens_out, int32_t* bt_out, hipStream_t st) {
  hipLaunchKernelGGL(k_prefill_tables, dim3((unsigned)(B * C)), dim3(256), 0, st, C, max_pages, p0, bt_in,
                     seq_lens_out, bt_out);
  return hipGetLastError();
}

hipError_t launch_rope(const mla_dims& d, int B, const int32_t* seq_lens, float* q_pe, float* kv_new,
                       const CacheArgs* cache, hipStream_t st) {
  CacheArgs c = cache ? *cache : CacheArgs{};
  size_t smem = (size_t)(d.d_r + d.d_c + d.d_r + 4) * sizeof(float);
  const RopeFreq freq{d.rope_base, d.yarn_factor > 1.f ? (double)d.yarn_factor : 1.0, (double)d.yarn_orig_len,
                      (double)d.yarn_alpha, (double)d.yarn_beta};
  hipLaunchKernelGGL(k_rope_append, dim3(B, 1 + (d.n_h + RH - 1) / RH), dim3(256), smem, st, d.n_h, d.d_c, d.d_r, freq,
                     seq_lens, q_pe, kv_new, c, cache ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_cache_store(const mla_dims& d, const CacheArgs& c, int B, const int32_t* n_rows,
                              int max_rows, const float* src, int64_t src_stride, hipStream_t st) {
  dim3 grid((max_rows + 3) / 4, B);
  hipLaunchKernelGGL(k_cache_store, grid, dim3(256), 0, st, d.d_c + d.d_r, c, n_rows, src, src_stride);
  return hipGetLastError();
}

}  // namespace mla
