// Projection GEMMs of the decode step: query pathway with W^UK absorbed, the current token's
// KV projection, and the two-step output (W^UV, then W^O).
//
// "DeepSeek-V2 from Scratch" section 4.1 (c^Q = W^DQ h; q^C = W^UQ c^Q; raw q^R = W^QR c^Q),
// section 2.1 (c^KV = W^DKV h), section 4.2 (raw k^R = W^KR h), section 5.1 (absorbed query
// q~_i = (W^UK_i)^T q^C_i), section 5.2 (o_i = W^UV_i o_lat_i) and section 6 (u = W^O [o]).
//
// All are "skinny" products Y[n][m] = sum_k W(m, k) X[n][k] with n over the batch (tens of rows)
// and W read exactly once from HBM, so they are bound by weight bandwidth. bf16 weights run on
// MFMA: W is the A operand, loaded from global memory directly in MFMA layout; float32
// activations are split into hi + lo bf16 parts (x = hi + lo holds 16 significand bits), costing
// a second MFMA that is free under the bandwidth bound and keeping the activation error near
// float32 instead of bf16. float32 / float16 weights run on a tiled float32 VALU kernel.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

// ------------------------------------------------------------------ workspace layouts
static size_t al256h(size_t x) { return (x + 255) & ~(size_t)255; }

namespace gm {
constexpr int SPLIT_K1 = 8;   // split-K of the first projection (K = d, few outputs)
constexpr int SPLIT_K5 = 4;   // split-K of the output projection (K = n_h d_h)
constexpr int MAXB = 128;     // batch rows per MFMA launch
}

AbsorbQLayout absorb_q_layout(const mla_dims& d, int B) {
  AbsorbQLayout L;
  L.off_cq = 0;
  L.off_qc = al256h((size_t)B * d.d_cq * 4);
  L.off_part = L.off_qc + al256h((size_t)B * d.n_h * d.d_h * 4);
  L.part_floats = (size_t)gm::SPLIT_K1 * B * (d.d_cq + d.d_c + d.d_r);
  L.bytes = L.off_part + al256h(L.part_floats * 4);
  return L;
}
AbsorbOutLayout absorb_out_layout(const mla_dims& d, int B) {
  AbsorbOutLayout L;
  L.off_o = 0;
  L.off_part = al256h((size_t)B * d.n_h * d.d_h * 4);
  L.part_floats = (size_t)gm::SPLIT_K5 * B * d.d;
  L.bytes = L.off_part + al256h(L.part_floats * 4);
  return L;
}

// ------------------------------------------------------------------ segment table
// Up to 3 weight matrices stacked along M that share the same activation X (e.g. W^DQ, W^DKV,
// W^KR all multiply h). Segment s owns rows [m0[s], m0[s+1]) of the stacked output.
struct Seg {
  const void* W[3];
  float* Y[3];
  int64_t ldy[3];
  int m0[4];
  int nseg;
};

__device__ __forceinline__ int seg_of(const Seg& s, int m) {
  int k = 0;
  while (k + 1 < s.nseg && m >= s.m0[k + 1]) ++k;
  return k;
}

// ================================================================================================
// MFMA bf16 skinny GEMM. Workgroup = 4 waves = one 64-row tile of the stacked output over one
// K slice; the 4 waves split that slice and are summed through LDS. Each wave keeps
// 2 (m-blocks of 32) x NB (n-blocks of 32) accumulators. The reduction over k is permuted per
// 64-wide group so that each lane reads 64 contiguous bytes of its weight row and 128 contiguous
// bytes (float32) of its activation row: lane half g of a group owns k in [32g, 32g + 32), split
// into the four 8-wide MFMA k-slots of the group's four steps. Both operands use the same
// permutation, so the products pair the same k.
//   XF32 = true: X is float32, split hi/lo (2 MFMAs per step); false: X is bf16.
//   split_k > 1: the workgroup writes its sum to part[ky][n][m] for a later ordered reduction;
//   otherwise it writes Y directly.
template <int NB, bool XF32>
__global__ __launch_bounds__(256) void k_gemm_mfma(Seg seg, int N, int K, const void* __restrict__ Xv,
                                                   int64_t ldx, int split_k, float* __restrict__ part,
                                                   int Mtot, int64_t zW, int64_t zX, int64_t zY) {
  __shared__ float red[4][64 * 32 * NB];  // per-wave partial tiles [m 64][n 32*NB]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int mt = blockIdx.x;                 // 64-row tile of the stacked output
  const int ky = blockIdx.y;                 // K slice
  const int z = blockIdx.z;                  // batched (per-head) problems
  const int m_base = mt * 64;
  const int s = seg_of(seg, m_base);
  const int lda = K;
  const uint16_t* W = (const uint16_t*)seg.W[s] + (int64_t)z * zW + (int64_t)(m_base - seg.m0[s]) * lda;

  // k groups of 64 assigned to (slice, wave)
  const int KG = K / 64;
  const int part_id = ky * 4 + w, nparts = split_k * 4;
  const int g0 = (int)((int64_t)KG * part_id / nparts), g1 = (int)((int64_t)KG * (part_id + 1) / nparts);

  f32x16 acc[2][NB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  for (int kg = g0; kg < g1; ++kg) {
    const int kb = kg * 64 + 32 * g;
    // A fragments: rows l32 and 32 + l32, 32 contiguous k each (4 x 16 bytes)
    u32x4 a[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4* src = (const u32x4*)(W + (int64_t)(32 * i + l32) * lda + kb);
#pragma unroll
      for (int st = 0; st < 4; ++st) a[i][st] = src[st];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = 32 * j + l32;
      const bool nv = n < N;
      bf16x8 bh[4], bl[4];
      if constexpr (XF32) {
        const float* xs = (const float*)Xv + (int64_t)z * zX + (int64_t)(nv ? n : 0) * ldx + kb;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          f32x4 x0 = nv ? *(const f32x4*)(xs + 8 * st) : f32x4{};
          f32x4 x1 = nv ? *(const f32x4*)(xs + 8 * st + 4) : f32x4{};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            __bf16 h0 = (__bf16)x0[e], h1 = (__bf16)x1[e];
            bh[st][e] = h0; bh[st][4 + e] = h1;
            bl[st][e] = (__bf16)(x0[e] - (float)h0);
            bl[st][4 + e] = (__bf16)(x1[e] - (float)h1);
          }
        }
      } else {
        const uint16_t* xs = (const uint16_t*)Xv + (int64_t)z * zX + (int64_t)(nv ? n : 0) * ldx + kb;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          u32x4 v = nv ? *(const u32x4*)(xs + 8 * st) : u32x4{};
          bh[st] = __builtin_bit_cast(bf16x8, v);
        }
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          bf16x8 av = __builtin_bit_cast(bf16x8, a[i][st]);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh[st], acc[i][j], 0, 0, 0);
          if constexpr (XF32) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl[st], acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  // accumulator layout: lane holds column n = 32j + l32, rows m = 32i + 8(r/4) + 4g + r%4
  float* my = red[w];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        const int n = 32 * j + l32;
        my[m * (32 * NB) + n] = acc[i][j][r];
      }
  __syncthreads();
  for (int e = tid; e < 64 * 32 * NB; e += 256) {
    const int m = e / (32 * NB), n = e % (32 * NB);
    if (n >= N) continue;
    const float v = red[0][e] + red[1][e] + red[2][e] + red[3][e];
    const int mg = m_base + m;
    if (split_k > 1) {
      part[((int64_t)ky * N + n) * Mtot + mg] = v;
    } else {
      float* Y = seg.Y[s] + (int64_t)z * zY;
      Y[(int64_t)n * seg.ldy[s] + (mg - seg.m0[s])] = v;
    }
  }
}

// Ordered split-K reduction: Y[n][m] = sum_{ky} part[ky][n][m], scattered to the segments.
__global__ __launch_bounds__(256) void k_splitk_reduce(Seg seg, int N, int Mtot, int split_k,
                                                       const float* __restrict__ part) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)N * Mtot) return;
  const int n = (int)(e / Mtot), m = (int)(e % Mtot);
  float v = 0.f;
  for (int k = 0; k < split_k; ++k) v += part[(int64_t)k * N * Mtot + e];
  const int s = seg_of(seg, m);
  seg.Y[s][(int64_t)n * seg.ldy[s] + (m - seg.m0[s])] = v;
}

// ================================================================================================
// Absorbed query: q_lat[b][i][c] = sum_e W^UK[i d_h + e][c] q^C[b][i d_h + e]. The reduction
// runs down the columns of W^UK, so a 128(e) x 128(c) tile is staged in LDS and read with the
// transposing LDS load (4 consecutive e of one column per lane). Workgroup = (head, 128 columns);
// wave w owns 32 columns; MFMA D[c][b] = sum_e A[c][e] X^T[e][b].
namespace absq {
constexpr int DH = 128, TC = 128, PITCH = 136;  // bf16 elements per LDS row (padded)
}
template <int NB>
__global__ __launch_bounds__(256) void k_absorb_uk(int n_h, int d_c, int N, const uint16_t* __restrict__ W_uk,
                                                   const float* __restrict__ qC, float* __restrict__ q_lat) {
  using namespace absq;
  __shared__ __attribute__((aligned(16))) uint16_t tile[DH * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int i = blockIdx.y;              // head
  const int c0 = blockIdx.x * TC;        // column tile
  // stage W^UK[i*128 .. +128][c0 .. c0+128] (row-major, 16-byte pieces)
  for (int f = tid; f < DH * TC / 8; f += 256) {
    const int e = f / (TC / 8), cc = (f % (TC / 8)) * 8;
    *(u32x4*)(tile + e * PITCH + cc) = *(const u32x4*)(W_uk + ((int64_t)i * DH + e) * d_c + c0 + cc);
  }
  __syncthreads();
  const int j16 = lane & 15, h2 = (lane >> 4) & 1;
  f32x16 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks) {
    // A[c][e]: lane column c = 32w + l32; e-slots 8g..8g+7 of this step via two transposed reads
    const int e0 = 16 * ks + 8 * g + (j16 >> 2);
    const int cc = 32 * w + 16 * h2 + 4 * (j16 & 3);
    const u32x2 x0 = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(MLA_LDS void*)(tile + e0 * PITCH + cc)));
    const u32x2 x1 = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(MLA_LDS void*)(tile + (e0 + 4) * PITCH + cc)));
    const u32x4 av = {x0.x, x0.y, x1.x, x1.y};
    const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = 32 * j + l32;
      const bool nv = n < N;
      // B[e][n] = q^C[n][i*128 + e], e = 16ks + 8g + 0..7: first 4 from rows e0.., i.e. the slot
      // order of the transposed read: slots 0-3 -> e = 16ks + 8g + 0..3, slots 4-7 -> +4..7.
      const float* xs = qC + (int64_t)(nv ? n : 0) * n_h * DH + (int64_t)i * DH + 16 * ks + 8 * g;
      f32x4 v0 = nv ? *(const f32x4*)xs : f32x4{};
      f32x4 v1 = nv ? *(const f32x4*)(xs + 4) : f32x4{};
      bf16x8 bh, bl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __bf16 h0 = (__bf16)v0[e], h1 = (__bf16)v1[e];
        bh[e] = h0; bh[4 + e] = h1;
        bl[e] = (__bf16)(v0[e] - (float)h0);
        bl[4 + e] = (__bf16)(v1[e] - (float)h1);
      }
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc[j], 0, 0, 0);
    }
  }
  // D[c][n]: lane holds n = 32j + l32, rows c = 8(r/4) + 4g + r%4 of this wave's 32 columns
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = 32 * j + l32;
    if (n >= N) continue;
    float* dst = q_lat + ((int64_t)n * n_h + i) * d_c + c0 + 32 * w;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v;
      v[0] = acc[j][4 * r4]; v[1] = acc[j][4 * r4 + 1]; v[2] = acc[j][4 * r4 + 2]; v[3] = acc[j][4 * r4 + 3];
      *(f32x4*)(dst + 8 * r4 + 4 * g) = v;
    }
  }
}

// ================================================================================================
// float32 VALU GEMM for float32 / float16 / bf16 weights of any shape:
//   Y[n][m] = sum_k A(m, k) X[n][k],  A(m, k) = TRANS ? W[k*lda + m] : W[m*lda + k].
// Tile 64 (m) x 16 (n) per 256 threads, k in steps of 32 through LDS.
template <int ADT, int XDT, bool TRANS>
__global__ __launch_bounds__(256) void k_gemm_valu(int M, int N, int K, const void* __restrict__ Wv,
                                                   int64_t lda, int64_t zW, const void* __restrict__ Xv,
                                                   int64_t ldx, int64_t zX, float* __restrict__ Y,
                                                   int64_t ldy, int64_t zY) {
  __shared__ float Ws[64][33];
  __shared__ float Xs[16][33];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 16, z = blockIdx.z;
  const typename Elem<ADT>::T* W = (const typename Elem<ADT>::T*)Wv + (int64_t)z * zW;
  const typename Elem<XDT>::T* X = (const typename Elem<XDT>::T*)Xv + (int64_t)z * zX;
  const int mi = tid & 63, nq = tid >> 6;  // thread: row mi, columns nq*4 .. nq*4+3
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 32) {
    for (int e = tid; e < 64 * 32; e += 256) {
      int mm, kk;
      if (TRANS) { mm = e & 63; kk = e >> 6; } else { kk = e & 31; mm = e >> 5; }
      const int m = m0 + mm, k = k0 + kk;
      float v = 0.f;
      if (m < M && k < K) v = Elem<ADT>::ld(W, TRANS ? (int64_t)k * lda + m : (int64_t)m * lda + k);
      Ws[mm][kk] = v;
    }
    for (int e = tid; e < 16 * 32; e += 256) {
      const int nn = e >> 5, kk = e & 31;
      const int n = n0 + nn, k = k0 + kk;
      Xs[nn][kk] = (n < N && k < K) ? Elem<XDT>::ld(X, (int64_t)n * ldx + k) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float a = Ws[mi][kk];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += a * Xs[nq * 4 + q][kk];
    }
    __syncthreads();
  }
  const int m = m0 + mi;
  if (m >= M) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = n0 + nq * 4 + q;
    if (n < N) Y[(int64_t)z * zY + (int64_t)n * ldy + m] = acc[q];
  }
}

// ------------------------------------------------------------------ dispatch helpers
template <int ADT, int XDT, bool TRANS>
static void valu(hipStream_t st, int M, int N, int K, const void* W, int64_t lda, int64_t zW, const void* X,
                 int64_t ldx, int64_t zX, float* Y, int64_t ldy, int64_t zY, int Z) {
  dim3 grid((M + 63) / 64, (N + 15) / 16, Z);
  hipLaunchKernelGGL((k_gemm_valu<ADT, XDT, TRANS>), grid, dim3(256), 0, st, M, N, K, W, lda, zW, X, ldx, zX, Y,
                     ldy, zY);
}

// Y[n][m] = sum_k A(m,k) X[n][k] with runtime weight dtype; X is float32 or the weight dtype.
static void valu_any(int wdt, bool x_is_w, bool trans, hipStream_t st, int M, int N, int K, const void* W,
                     int64_t lda, int64_t zW, const void* X, int64_t ldx, int64_t zX, float* Y, int64_t ldy,
                     int64_t zY, int Z) {
#define MLA_VALU_CASE(ADT)                                                                           \
  if (wdt == ADT) {                                                                                  \
    if (x_is_w) {                                                                                    \
      if (trans) valu<ADT, ADT, true>(st, M, N, K, W, lda, zW, X, ldx, zX, Y, ldy, zY, Z);           \
      else valu<ADT, ADT, false>(st, M, N, K, W, lda, zW, X, ldx, zX, Y, ldy, zY, Z);                \
    } else {                                                                                         \
      if (trans) valu<ADT, MLA_F32, true>(st, M, N, K, W, lda, zW, X, ldx, zX, Y, ldy, zY, Z);       \
      else valu<ADT, MLA_F32, false>(st, M, N, K, W, lda, zW, X, ldx, zX, Y, ldy, zY, Z);            \
    }                                                                                                \
    return;                                                                                          \
  }
  MLA_VALU_CASE(MLA_F32)
  MLA_VALU_CASE(MLA_F16)
  MLA_VALU_CASE(MLA_BF16)
#undef MLA_VALU_CASE
}

static bool mfma_dims_ok(const mla_dims& d) {
  return d.d % 256 == 0 && d.d_cq % 256 == 0 && d.d_cq % 64 == 0 && d.d_c % 128 == 0 && d.d_r % 64 == 0 &&
         d.d_h == absq::DH && (d.n_h * d.d_h) % 256 == 0;
}

template <bool XF32>
static void mfma_gemm(hipStream_t st, const Seg& sg, int N, int K, const void* X, int64_t ldx, int split_k,
                      float* part, int Z, int64_t zW, int64_t zX, int64_t zY) {
  const int Mtot = sg.m0[sg.nseg];
  dim3 grid(Mtot / 64, split_k, Z);
  if (N <= 32)
    hipLaunchKernelGGL((k_gemm_mfma<1, XF32>), grid, dim3(256), 0, st, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
  else if (N <= 64)
    hipLaunchKernelGGL((k_gemm_mfma<2, XF32>), grid, dim3(256), 0, st, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
  else if (N <= 96)
    hipLaunchKernelGGL((k_gemm_mfma<3, XF32>), grid, dim3(256), 0, st, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
  else
    hipLaunchKernelGGL((k_gemm_mfma<4, XF32>), grid, dim3(256), 0, st, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
  if (split_k > 1) {
    const int64_t tot = (int64_t)N * Mtot;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, sg, N, Mtot, split_k, part);
  }
}

hipError_t launch_absorb_q(const mla_dims& d, int B, int wdt, const void* h, const void* W_dq, const void* W_uq,
                           const void* W_qr, const void* W_uk, const void* W_dkv, const void* W_kr, void* ws,
                           float* q_lat, float* q_pe, float* kv_new, hipStream_t st) {
  AbsorbQLayout L = absorb_q_layout(d, B);
  float* cq = (float*)((char*)ws + L.off_cq);
  float* qc = (float*)((char*)ws + L.off_qc);
  float* part = (float*)((char*)ws + L.off_part);
  const int rw = d.d_c + d.d_r;
  const int nhdh = d.n_h * d.d_h;
  if (wdt == MLA_BF16 && mfma_dims_ok(d)) {
    for (int b0 = 0; b0 < B; b0 += gm::MAXB) {
      const int nb = B - b0 < gm::MAXB ? B - b0 : gm::MAXB;
      // stage 1: [c^Q | c^KV | k^R raw] = [W^DQ; W^DKV; W^KR] h
      Seg s1{};
      s1.W[0] = W_dq; s1.W[1] = W_dkv; s1.W[2] = W_kr;
      s1.Y[0] = cq + (int64_t)b0 * d.d_cq; s1.ldy[0] = d.d_cq;
      s1.Y[1] = kv_new + (int64_t)b0 * rw; s1.ldy[1] = rw;
      s1.Y[2] = kv_new + (int64_t)b0 * rw + d.d_c; s1.ldy[2] = rw;
      s1.m0[0] = 0; s1.m0[1] = d.d_cq; s1.m0[2] = d.d_cq + d.d_c; s1.m0[3] = d.d_cq + rw; s1.nseg = 3;
      mfma_gemm<false>(st, s1, nb, d.d, (const uint16_t*)h + (int64_t)b0 * d.d, d.d, gm::SPLIT_K1, part, 1, 0, 0, 0);
      // stage 2: [q^C | q^R raw] = [W^UQ; W^QR] c^Q
      Seg s2{};
      s2.W[0] = W_uq; s2.W[1] = W_qr;
      s2.Y[0] = qc + (int64_t)b0 * nhdh; s2.ldy[0] = nhdh;
      s2.Y[1] = q_pe + (int64_t)b0 * d.n_h * d.d_r; s2.ldy[1] = (int64_t)d.n_h * d.d_r;
      s2.m0[0] = 0; s2.m0[1] = nhdh; s2.m0[2] = nhdh + d.n_h * d.d_r; s2.nseg = 2;
      mfma_gemm<true>(st, s2, nb, d.d_cq, cq + (int64_t)b0 * d.d_cq, d.d_cq, 1, nullptr, 1, 0, 0, 0);
      // stage 3: q_lat_i = (W^UK_i)^T q^C_i
      dim3 g3(d.d_c / absq::TC, d.n_h);
      const float* qcb = qc + (int64_t)b0 * nhdh;
      float* qlb = q_lat + (int64_t)b0 * d.n_h * d.d_c;
      if (nb <= 32) hipLaunchKernelGGL(k_absorb_uk<1>, g3, dim3(256), 0, st, d.n_h, d.d_c, nb, (const uint16_t*)W_uk, qcb, qlb);
      else if (nb <= 64) hipLaunchKernelGGL(k_absorb_uk<2>, g3, dim3(256), 0, st, d.n_h, d.d_c, nb, (const uint16_t*)W_uk, qcb, qlb);
      else if (nb <= 96) hipLaunchKernelGGL(k_absorb_uk<3>, g3, dim3(256), 0, st, d.n_h, d.d_c, nb, (const uint16_t*)W_uk, qcb, qlb);
      else hipLaunchKernelGGL(k_absorb_uk<4>, g3, dim3(256), 0, st, d.n_h, d.d_c, nb, (const uint16_t*)W_uk, qcb, qlb);
    }
    return hipGetLastError();
  }
  // VALU path (any dims, float32/float16/bf16 weights)
  valu_any(wdt, true, false, st, d.d_cq, B, d.d, W_dq, d.d, 0, h, d.d, 0, cq, d.d_cq, 0, 1);
  valu_any(wdt, true, false, st, d.d_c, B, d.d, W_dkv, d.d, 0, h, d.d, 0, kv_new, rw, 0, 1);
  valu_any(wdt, true, false, st, d.d_r, B, d.d, W_kr, d.d, 0, h, d.d, 0, kv_new + d.d_c, rw, 0, 1);
  valu_any(wdt, false, false, st, nhdh, B, d.d_cq, W_uq, d.d_cq, 0, cq, d.d_cq, 0, qc, nhdh, 0, 1);
  valu_any(wdt, false, false, st, d.n_h * d.d_r, B, d.d_cq, W_qr, d.d_cq, 0, cq, d.d_cq, 0, q_pe,
           (int64_t)d.n_h * d.d_r, 0, 1);
  // per head: q_lat[n][i][c] = sum_e W_uk[i*d_h + e][c] qC[n][i*d_h + e]  (transposed access)
  valu_any(wdt, false, true, st, d.d_c, B, d.d_h, W_uk, d.d_c, (int64_t)d.d_h * d.d_c, qc, nhdh, d.d_h, q_lat,
           (int64_t)d.n_h * d.d_c, d.d_c, d.n_h);
  return hipGetLastError();
}

hipError_t launch_absorb_out(const mla_dims& d, int B, int wdt, const float* o_lat, const void* W_uv,
                             const void* W_o, void* ws, float* u, hipStream_t st) {
  AbsorbOutLayout L = absorb_out_layout(d, B);
  float* o = (float*)((char*)ws + L.off_o);
  float* part = (float*)((char*)ws + L.off_part);
  const int nhdh = d.n_h * d.d_h;
  if (wdt == MLA_BF16 && mfma_dims_ok(d)) {
    for (int b0 = 0; b0 < B; b0 += gm::MAXB) {
      const int nb = B - b0 < gm::MAXB ? B - b0 : gm::MAXB;
      // o_i = W^UV_i o_lat_i, batched over heads (z): rows of W^UV_i are outputs
      Seg s4{};
      s4.W[0] = W_uv; s4.Y[0] = o + (int64_t)b0 * nhdh; s4.ldy[0] = nhdh;
      s4.m0[0] = 0; s4.m0[1] = d.d_h; s4.nseg = 1;
      mfma_gemm<true>(st, s4, nb, d.d_c, o_lat + (int64_t)b0 * d.n_h * d.d_c, (int64_t)d.n_h * d.d_c, 1, nullptr,
                      d.n_h, (int64_t)d.d_h * d.d_c, d.d_c, d.d_h);
      // u = W^O [o_1; ...; o_nh]
      Seg s5{};
      s5.W[0] = W_o; s5.Y[0] = u + (int64_t)b0 * d.d; s5.ldy[0] = d.d;
      s5.m0[0] = 0; s5.m0[1] = d.d; s5.nseg = 1;
      mfma_gemm<true>(st, s5, nb, nhdh, o + (int64_t)b0 * nhdh, nhdh, gm::SPLIT_K5, part, 1, 0, 0, 0);
    }
    return hipGetLastError();
  }
  valu_any(wdt, false, false, st, d.d_h, B, d.d_c, W_uv, d.d_c, (int64_t)d.d_h * d.d_c, o_lat,
           (int64_t)d.n_h * d.d_c, d.d_c, o, nhdh, d.d_h, d.n_h);
  valu_any(wdt, false, false, st, d.d, B, nhdh, W_o, nhdh, 0, o, nhdh, 0, u, d.d, 0, 1);
  return hipGetLastError();
}

}  // namespace mla
