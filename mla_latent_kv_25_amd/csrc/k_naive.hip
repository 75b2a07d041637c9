// Naive-form (MHA-form) attention for a prefill chunk: the keys and values of every context token are
// materialised per head ("DeepSeek-V2 from Scratch" section 2.2: k^C_{j,i} = W^UK_i c_j and
// v_{j,i} = W^UV_i c_j; section 4.2: k_{j,i} = [k^C_{j,i} ; k^R_j]) and each chunk token attends to its
// causal prefix with the un-absorbed query q_{t,i} = [q^C_{t,i} ; q^R_{t,i}] (section 4.4). The absorbed
// path computes the same outputs ("DeepSeek-V2 from Scratch" section 5: absorption is exact) at 278,528
// flop per (query, key) pair against 81,920 here, but here every context token's K and V are built
// first (33.5 Mflop per token): for long chunks this form needs fewer flops.
//
//   k_gather_rows: the context rows of each sequence out of its pages, into [B, max_ctx, 576]
//                  (rows past a sequence's context zero-filled, so that the keys and values built from
//                  them are finite zeros);
//   K^C and V:     one product (k_gemm.hip, bf16 output) of the gathered latents with [W^UK ; W^UV];
//   k_mha_prefill: per (query block, head, sequence) workgroup, flash-style attention on MFMA.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

// ------------------------------------------------------------------------------------ gather
// One thread per 16-byte chunk of a row (72 per row): row j of sequence b comes from page
// block_table[b][j / page_size], slot j % page_size (paged cache), or row b t_cap + j (contiguous).
// A sequence's rows are 0 .. min(p0[b] + C, max_ctx) - 1; the rest of its max_ctx rows are zeros.
__global__ __launch_bounds__(256) void k_gather_rows(CacheArgs c, int B, int C, const int32_t* __restrict__ p0,
                                                     int max_ctx, uint8_t* __restrict__ ctx) {
  constexpr int RB = 576 * 2, CH = RB / 16;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)B * max_ctx * CH;
  if (e >= total) return;
  const int ch = (int)(e % CH);
  const int64_t r = e / CH;
  const int b = (int)(r / max_ctx), j = (int)(r % max_ctx);
  const int L = p0[b] + C;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (j < L) {
    const int64_t row = c.page_size > 0
                            ? (int64_t)c.block_table[(int64_t)b * c.max_pages + j / c.page_size] * c.page_size +
                                  j % c.page_size
                            : (int64_t)b * c.t_cap + j;
    v = *(const u32x4*)((const uint8_t*)c.rows + row * RB + ch * 16);
  }
  *(u32x4*)(ctx + r * RB + ch * 16) = v;
}

// ------------------------------------------------------------------------------------ attention
// Workgroup = 4 waves over QB = 64 NQB queries of one (sequence b, head i); wave w owns queries
// 16 NQB w .. + 16 NQB. The keys come in 32-key tiles shared by the four waves through a 3-slot LDS
// ring (global -> LDS copies; each wave issues 6 of the 24 1-KB copies of a tile, one barrier per
// tile). A tile holds the keys' rows [k^C (128) | k^R (64)] (25 chunks per row, an odd stride, so the
// row reads of 16 lanes hit 16 distinct bank groups) and their value rows (18 chunks per row, which
// makes the transposing reads conflict-free).
//   scores: S^T[16 keys x 16 queries] blocks on MFMA 16x16x32 (key rows as A, the queries of the
//     lane's column as B, 6 k-steps over 192 dims, the scale folded into the query); lane (g, n) gets
//     query n's scores of keys 4g..4g+3 and 16+4g..16+4g+3, which are the eight values the PV product
//     needs from that lane as its B operand (the reduction runs over the tile's keys in that order);
//   softmax: online, per query, in float32 (base 2);
//   PV: O^T[16 value columns x 16 queries] += V^T P^T per 16 columns, V^T by transposing 16-bit reads.
// Causal: query t (position p0[b] + t) sees keys 0 .. p0[b] + t.
namespace nv {
constexpr int DH = 128, DR = 64, DC = 512;  // d_h, d_r, d_c (the DeepSeek-V2 shape; any head count)
constexpr int TT = 32;                 // keys per tile
constexpr int KCHP = 25;               // LDS stride of a key row in 16-byte chunks (24 used)
constexpr int VCHP = 18;               // LDS stride of a value row in chunks (16 used)
constexpr int KB = TT * KCHP * 16;     // 12800
constexpr int VOFF = KB;               // value rows after the key rows
constexpr int SLOT = 24 * 1024;        // tile slot: 24 copies of 1 KB (1376 chunks used)
constexpr int NSLOT = 3;
constexpr int NCP = 6;                 // copies per wave per tile
}

template <int NQB>
__global__ __launch_bounds__(256, NQB == 1 ? 2 : 1) void k_mha_prefill(int C, int max_ctx, int n_h, const int32_t* __restrict__ p0,
                                                        const float* __restrict__ q_c, const float* __restrict__ q_pe,
                                                        const uint16_t* __restrict__ ctx, const uint16_t* __restrict__ kc,
                                                        const uint16_t* __restrict__ vv, float qscale,
                                                        float* __restrict__ o) {
  using namespace nv;
  __shared__ __attribute__((aligned(16))) uint8_t lds[NSLOT * SLOT];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int qb = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int NHD = n_h * DH;
  const int P0 = p0[b] > 0 ? p0[b] : 0;
  const int tq0 = 64 * NQB * qb;                              // first query of the workgroup
  const int tqe = C < tq0 + 64 * NQB ? C : tq0 + 64 * NQB;    // one past its last
  // keys 0 .. P0 + tqe - 1 (held to the gathered rows: a context beyond max_ctx is a caller error)
  const int nkeys = P0 + tqe < max_ctx ? P0 + tqe : max_ctx;
  const int ntiles = (nkeys + TT - 1) / TT;
  const int64_t rowbase = (int64_t)b * max_ctx;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MLA_LDS void*)lds;

  // copy plan: LDS chunk q = 64 (4 k + w) + lane of a slot (k = 0 .. 5): key chunk q < 800 (row q / 25,
  // column q % 25: 0..15 from k^C, 16..23 from k^R, 24 a duplicate), value chunk 800 <= q < 1376
  // (row, column of q - 800 in rows of 18: 0..15 from v, 16..17 duplicates), q >= 1376 unused
  // (a duplicate); kind 0: k^C / v of the head, 1: k^R
  uint32_t plan[NCP];
#pragma unroll
  for (int k = 0; k < NCP; ++k) {
    const int q = 64 * (4 * k + w) + lane;
    int row, src;  // src: byte offset inside the source row (bit 15 set: value rows)
    if (q < TT * KCHP) {
      row = q / KCHP;
      const int cc = q % KCHP;
      src = cc < 16 ? cc * 16 : (cc < 24 ? (1 << 14) | ((cc - 16) * 16) : 0);
    } else if (q < TT * KCHP + TT * VCHP) {
      const int qq = q - TT * KCHP;
      row = qq / VCHP;
      const int cc = qq % VCHP;
      src = (1 << 15) | ((cc < 16 ? cc : 0) * 16);
    } else {
      row = 0;
      src = 0;
    }
    plan[k] = ((uint32_t)row << 16) | (uint32_t)src;
  }
  auto issue = [&](int it) __attribute__((always_inline)) {
    const int j0 = TT * it;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((it % NSLOT) * SLOT + w * 1024));
#pragma unroll
    for (int k = 0; k < NCP; ++k) {
      int j = j0 + (int)(plan[k] >> 16);
      j = j < nkeys ? j : nkeys - 1;
      const uint32_t src = plan[k] & 0xffffu;
      const int64_t r = rowbase + j;
      const uint8_t* p;
      if (src & (1u << 15)) p = (const uint8_t*)(vv + r * NHD + (int64_t)i * DH) + (src & 0x7fffu);
      else if (src & (1u << 14)) p = (const uint8_t*)(ctx + r * 576 + DC) + (src & 0x3fffu);
      else p = (const uint8_t*)(kc + r * NHD + (int64_t)i * DH) + src;
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(p), "s"(dst + (uint32_t)(k * 4096)) : "memory", "m0");
    }
  };

  if (ntiles > 0) issue(0);
  // queries of the wave: query block qq (16 queries), lane column n: t = tq0 + 16 (NQB w + qq) + n;
  // dims 32 ks + 8 g .. + 7 of [q^C (128) | q^R (64)], times qscale, as bf16 B fragments
  bf16x8 qf[NQB][6];
  int tpos[NQB];
#pragma unroll
  for (int qq = 0; qq < NQB; ++qq) {
    const int t = tq0 + 16 * (NQB * w + qq) + n;
    tpos[qq] = t < C ? P0 + t : -1;
    const int tc = t < C ? t : C - 1;
    const int64_t tok = (int64_t)b * C + tc;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      const float* src = d0 < DH ? q_c + tok * NHD + (int64_t)i * DH + d0 : q_pe + (tok * n_h + i) * DR + (d0 - DH);
      const f32x4 a = *(const f32x4*)src * qscale, c4 = *(const f32x4*)(src + 4) * qscale;
      qf[qq][ks] = bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                          (__bf16)c4[0], (__bf16)c4[1], (__bf16)c4[2], (__bf16)c4[3]};
    }
  }
  if (ntiles > 1) issue(1);

  float m_run[NQB], l_run[NQB];
  f32x4 O[NQB][8];
#pragma unroll
  for (int qq = 0; qq < NQB; ++qq) {
    m_run[qq] = -__builtin_inff();
    l_run[qq] = 0.f;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) O[qq][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int it = 0; it < ntiles; ++it) {
    // tile it landed (tile it + 1 may be in flight); every wave is done with tile it - 1
    if (it + 1 < ntiles) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NCP) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (it + 2 < ntiles) issue(it + 2);  // into the slot tile it - 1 used
    const uint8_t* tile = lds + (it % NSLOT) * SLOT;
    const int j0 = TT * it;
    // key fragments (shared by the query blocks): rows n and 16 + n, chunk 4 ks + g
    bf16x8 ka[2][6];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) ka[kb][ks] = *(const bf16x8*)(tile + ((16 * kb + n) * KCHP + 4 * ks + g) * 16);
    // value fragments: rows 4g + n/4 and 16 + 4g + n/4, columns 16 cb + 4 (n % 4)
    const uint8_t* va = tile + VOFF + (4 * g + (n >> 2)) * VCHP * 16 + (n & 3) * 8;
    bf16x8 vf[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(uintptr_t)(uint32_t)(uintptr_t)(MLA_LDS void*)(va + 32 * cb));
      const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (MLA_LDS s16x4*)(uintptr_t)(uint32_t)(uintptr_t)(MLA_LDS void*)(va + 16 * VCHP * 16 + 32 * cb));
      vf[cb] = __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, x0).x, __builtin_bit_cast(u32x2, x0).y,
                                                __builtin_bit_cast(u32x2, x1).x, __builtin_bit_cast(u32x2, x1).y});
    }
#pragma unroll
    for (int qq = 0; qq < NQB; ++qq) {
      f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0][ks], qf[qq][ks], S0, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1][ks], qf[qq][ks], S1, 0, 0, 0);
      }
      // causal mask: key j0 + 4g + r (S0) / j0 + 16 + 4g + r (S1) is seen iff it is <= the query's position
      const int lim = tpos[qq] - j0;
      float tm = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        S0[r] = 4 * g + r <= lim ? S0[r] : -__builtin_inff();
        S1[r] = 16 + 4 * g + r <= lim ? S1[r] : -__builtin_inff();
        tm = fmaxf(tm, fmaxf(S0[r], S1[r]));
      }
      tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
      tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
      const float m_new = fmaxf(m_run[qq], tm);
      // a query that sees no key of this tile keeps its state (and a query past the chunk sees none)
      const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qq] - m_use);
      float rs = 0.f;
      bf16x8 pf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e0 = __builtin_amdgcn_exp2f(S0[r] - m_use), e1 = __builtin_amdgcn_exp2f(S1[r] - m_use);
        rs += e0 + e1;
        pf[r] = (__bf16)e0;
        pf[4 + r] = (__bf16)e1;
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run[qq] = l_run[qq] * alpha + rs;
      m_run[qq] = m_new;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
        O[qq][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[cb], pf, O[qq][cb] * alpha, 0, 0, 0);
    }
  }
  // o[b * C + t][i * 128 + 16 cb + 4 g .. + 3] = O / l
#pragma unroll
  for (int qq = 0; qq < NQB; ++qq) {
    const int t = tq0 + 16 * (NQB * w + qq) + n;
    if (t >= C) continue;
    const float inv = 1.f / l_run[qq];
    float* dst = o + ((int64_t)b * C + t) * NHD + (int64_t)i * DH + 4 * g;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) *(f32x4*)(dst + 16 * cb) = O[qq][cb] * inv;
  }
}

// ------------------------------------------------------------------------------------ launch
NaiveLayout naive_layout(int n_h, int B, int max_ctx) {
  NaiveLayout L;
  const size_t rows = (size_t)B * max_ctx, nhd = (size_t)n_h * nv::DH;
  L.off_ctx = 0;
  L.off_kc = (rows * 576 * 2 + 255) & ~(size_t)255;
  L.off_v = L.off_kc + ((rows * nhd * 2 + 255) & ~(size_t)255);
  L.bytes = L.off_v + rows * nhd * 2;
  return L;
}

hipError_t launch_gather_rows(const CacheArgs& c, int B, int C, const int32_t* p0, int max_ctx, void* ctx,
                              hipStream_t st) {
  const int64_t total = (int64_t)B * max_ctx * 72;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, c, B, C, p0, max_ctx,
                     (uint8_t*)ctx);
  return hipGetLastError();
}

hipError_t launch_mha_prefill(int B, int C, int max_ctx, int n_h, const int32_t* p0, const float* q_c,
                              const float* q_pe, const void* ws, float qscale, float* o, hipStream_t st) {
  const NaiveLayout L = naive_layout(n_h, B, max_ctx);
  const uint16_t* ctx = (const uint16_t*)((const char*)ws + L.off_ctx);
  const uint16_t* kc = (const uint16_t*)((const char*)ws + L.off_kc);
  const uint16_t* vv = (const uint16_t*)((const char*)ws + L.off_v);
  if (C > 64) {
    hipLaunchKernelGGL(k_mha_prefill<2>, dim3((unsigned)((C + 127) / 128), n_h, B), dim3(256), 0, st, C, max_ctx, n_h,
                       p0, q_c, q_pe, ctx, kc, vv, qscale, o);
  } else {
    hipLaunchKernelGGL(k_mha_prefill<1>, dim3((unsigned)((C + 63) / 64), n_h, B), dim3(256), 0, st, C, max_ctx, n_h,
                       p0, q_c, q_pe, ctx, kc, vv, qscale, o);
  }
  return hipGetLastError();
}

}  // namespace mla
