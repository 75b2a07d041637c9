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
//   k_mha_prefill: per (128-query block, head, sequence) workgroup, flash-style attention on MFMA.
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
// Workgroup = 4 waves over 128 queries of one (sequence b, head i); wave w owns queries
// tq0 + 32 w .. + 31, two waves per SIMD (two workgroups per CU). The keys come in 32-key tiles
// shared by the four waves through a 3-slot LDS ring (global -> LDS copies; each wave issues 6 of
// the 24 1-KB copies of a tile, one barrier per tile). A tile holds the keys' rows
// [k^C (128) | k^R (64)] (25 chunks per row: an odd stride spreads the row reads of consecutive
// lanes over the banks) and their value rows (18 chunks per row, for the transposing reads).
//   scores: S^T[32 keys x 32 queries] on MFMA 32x32x16 (key rows as A, the wave's queries as B,
//     12 k-steps over 192 dims, the scale folded into the bf16 query); lane (g, n) gets query n's
//     scores of keys 8 (r / 4) + 4 g + r % 4, r = 0..15: values r = 0..7 and 8..15 are that lane's
//     B operand for the two 16-key steps of the PV product (the reduction runs over the keys in
//     that order);
//   softmax: online, per query, in float32 (base 2); a lane's 16 scores reduce as a tree, the two
//     lane halves meet through a cross-half swap (maximum per tile, sum once at the end); the
//     rescale of O is skipped when no query of the wave raised its maximum;
//   PV: O^T[32 value columns x 32 queries] += V^T P^T per 32 columns, V^T by transposing 16-bit
//     reads (rows 16 kk + 4 g .. + 3 and 16 kk + 8 + 4 g .. + 3 for lane half g).
// Causal: query t (position p0[b] + t) sees keys 0 .. p0[b] + t.
// v of lane l and of lane l ^ 32, through v_permlane32_swap: of the two results, one holds the
// lane's own value and the other its partner's, so a symmetric combination of both is the same in
// the two lanes. (The results are copied out element by element: a bit_cast applied straight to
// an element of the returned pair was compiled as if both elements were the first.)
__device__ __forceinline__ void swap_pair(float v, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float halves_max(float v) {
  float a, b;
  swap_pair(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float halves_sum(float v) {
  float a, b;
  swap_pair(v, a, b);
  return a + b;
}

namespace nv {
constexpr int DH = 128, DR = 64, DC = 512;  // d_h, d_r, d_c (the DeepSeek-V2 shape; any head count)
constexpr int QB = 128;                // queries per workgroup
constexpr int TT = 32;                 // keys per tile
constexpr int KCHP = 25;               // LDS stride of a key row in 16-byte chunks (24 used)
constexpr int VCHP = 18;               // LDS stride of a value row in chunks (16 used)
constexpr int KB = TT * KCHP * 16;     // 12800
constexpr int VOFF = KB;               // value rows after the key rows
constexpr int SLOT = 24 * 1024;        // tile slot: 24 copies of 1 KB (1376 chunks used)
constexpr int NSLOT = 3;
constexpr int NCP = 6;                 // copies per wave per tile
}

__global__ __launch_bounds__(256, 2) void k_mha_prefill(int B, int C, int max_ctx, int n_h, const int32_t* __restrict__ p0,
                                                        const float* __restrict__ q_c, const float* __restrict__ q_pe,
                                                        const uint16_t* __restrict__ ctx, const uint16_t* __restrict__ kc,
                                                        const uint16_t* __restrict__ vv, float qscale,
                                                        uint16_t* __restrict__ o) {
  using namespace nv;
  __shared__ __attribute__((aligned(16))) uint8_t lds[NSLOT * SLOT];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
  // block t = (b * n_h + i) * nqb + qb: consecutive t go to one XCD (workgroups are dealt
  // round-robin to the 8 XCDs), so the query blocks of one (sequence, head), which walk the same
  // keys at about the same pace, and neighbouring heads, which share k^R, read them through one L2
  const int nqb = (C + QB - 1) / QB;
  const int tb = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
  if (tb >= nqb * n_h * B) return;  // padding workgroup (uniform)
  const int qb = tb % nqb, i = (tb / nqb) % n_h, b = tb / (nqb * n_h);
  const int NHD = n_h * DH;
  const int P0 = p0[b] > 0 ? p0[b] : 0;
  const int tq0 = QB * qb;                                    // first query of the workgroup
  const int tqe = C < tq0 + QB ? C : tq0 + QB;                // one past its last
  // keys 0 .. P0 + tqe - 1 (held to the gathered rows: a context beyond max_ctx is a caller error)
  const int nkeys = P0 + tqe < max_ctx ? P0 + tqe : max_ctx;
  const int ntiles = (nkeys + TT - 1) / TT;
  const int64_t rowbase = (int64_t)b * max_ctx;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MLA_LDS void*)lds;

  // copy plan: LDS chunk q = 64 (4 k + w) + lane of a slot (k = 0 .. 5): key chunk q < 800 (row q / 25,
  // column q % 25: 0..15 from k^C, 16..23 from k^R, 24 a duplicate), value chunk 800 <= q < 1376
  // (row, column of q - 800 in rows of 18: 0..15 from v, 16..17 duplicates), q >= 1376 unused
  // (a duplicate); kind 0: k^C / v of the head, 1: k^R
  // The lane's source for copy k: row rk[k] of the tile, from the key row base gb[k] (k^C or v of
  // head i, or the shared k^R) at a row stride of gs[k] bytes; gp[k] walks it tile by tile.
  const uint8_t* gp[NCP];
  uint32_t gs[NCP];
  int rk[NCP];
#pragma unroll
  for (int k = 0; k < NCP; ++k) {
    const int q = 64 * (4 * k + w) + lane;
    int row, cc;
    const uint8_t* base;
    uint32_t stride;
    if (q < TT * KCHP) {
      row = q / KCHP;
      cc = q % KCHP;
      if (cc < 16) {
        base = (const uint8_t*)(kc + rowbase * NHD + (int64_t)i * DH) + cc * 16;
        stride = (uint32_t)NHD * 2;
      } else {
        base = (const uint8_t*)(ctx + rowbase * 576 + DC) + (cc < 24 ? cc - 16 : 0) * 16;
        stride = 576 * 2;
      }
    } else {
      const int qq = q < TT * KCHP + TT * VCHP ? q - TT * KCHP : 0;
      row = qq / VCHP;
      cc = qq % VCHP;
      base = (const uint8_t*)(vv + rowbase * NHD + (int64_t)i * DH) + (cc < 16 ? cc : 0) * 16;
      stride = (uint32_t)NHD * 2;
    }
    rk[k] = row;
    gs[k] = stride;
    gp[k] = base + (int64_t)row * stride;
  }
  // copies of tile it (issued in order it = 0, 1, 2, ...): whole tiles advance the row pointers;
  // the last, partial tile holds its rows to the last key
  auto issue = [&](int it) __attribute__((always_inline)) {
    const int j0 = TT * it;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((it % NSLOT) * SLOT + w * 1024));
    const bool whole = j0 + TT <= nkeys;
#pragma unroll
    for (int k = 0; k < NCP; ++k) {
      const uint8_t* p = gp[k];
      if (!whole) {
        const int j = j0 + rk[k] < nkeys ? j0 + rk[k] : nkeys - 1;
        p -= (int64_t)rk[k] * gs[k];
        p += (int64_t)(j - j0) * gs[k];
      }
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(p), "s"(dst + (uint32_t)(k * 4096)) : "memory", "m0");
      gp[k] += (int64_t)TT * gs[k];
    }
  };

  if (ntiles > 0) issue(0);
  // the wave's queries: lane column n: t = tq0 + 32 w + n; B fragment ks holds dims
  // 16 ks + 8 g .. + 7 of [q^C (128) | q^R (64)], times qscale, in bf16
  const int t = tq0 + 32 * w + n;
  const int tpos = t < C ? P0 + t : -1;
  bf16x8 qf[12];
  {
    const int tc = t < C ? t : C - 1;
    const int64_t tok = (int64_t)b * C + tc;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      const int d0 = 16 * ks + 8 * g;
      const float* src = d0 < DH ? q_c + tok * NHD + (int64_t)i * DH + d0 : q_pe + (tok * n_h + i) * DR + (d0 - DH);
      const f32x4 a = *(const f32x4*)src * qscale, c4 = *(const f32x4*)(src + 4) * qscale;
      qf[ks] = bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                      (__bf16)c4[0], (__bf16)c4[1], (__bf16)c4[2], (__bf16)c4[3]};
    }
  }
  if (ntiles > 1) issue(1);
  // first query position of the wave: tiles wholly at or below it need no mask
  const int wpos0 = tq0 + 32 * w < C ? P0 + tq0 + 32 * w : -1;

  // lane part of the value-row read address inside a tile slot
  const int va_lane = VOFF + (4 * g + ((lane & 15) >> 2)) * VCHP * 16 + (16 * (n >> 4) + 4 * (lane & 3)) * 2;

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x16 O[4];
#pragma unroll
  for (int vb = 0; vb < 4; ++vb) O[vb] = f32x16{};

  for (int it = 0; it < ntiles; ++it) {
    // tile it landed (tile it + 1 may be in flight); every wave is done with tile it - 1
    if (it + 1 < ntiles) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NCP) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (it + 2 < ntiles) issue(it + 2);  // into the slot tile it - 1 used
    const uint8_t* tile = lds + (it % NSLOT) * SLOT;
    const int j0 = TT * it;
    // scores: key row n, chunk 2 ks + g
    f32x16 S = {};
    const uint8_t* krow = tile + (n * KCHP + g) * 16;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks)
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow + 32 * ks), qf[ks], S, 0, 0, 0);
    // key fragments requested four ahead of their MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // causal mask (tiles that reach past the wave's first query position)
    if (j0 + TT - 1 > wpos0) {
      const int lim = tpos - j0;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = 8 * (r >> 2) + 4 * g + (r & 3) <= lim ? S[r] : -__builtin_inff();
    }
    // the tile's maximum per query: a tree over the lane's 16 scores, then the other lane half
    // (lane l and l ^ 32 hold the same query) through a cross-half swap
    float mx[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) mx[r] = fmaxf(S[r], S[r + 8]);
#pragma unroll
    for (int h = 4; h >= 1; h >>= 1)
#pragma unroll
      for (int r = 0; r < h; ++r) mx[r] = fmaxf(mx[r], mx[r + h]);
    const float tm = halves_max(mx[0]);
    const float m_new = fmaxf(m_run, tm);
    // a query that sees no key of this tile keeps its state (and a query past the chunk sees none)
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    // probabilities; each lane half keeps the sum over its own 16 keys (the halves are added once,
    // at the end: both use the same maximum, hence the same rescale factors)
    float ev[16];
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ev[r] = __builtin_amdgcn_exp2f(S[r] - m_use);
      pf[r >> 3][r & 7] = (__bf16)ev[r];
    }
#pragma unroll
    for (int h = 8; h >= 1; h >>= 1)
#pragma unroll
      for (int r = 0; r < h; ++r) ev[r] += ev[r + h];
    const float rs = ev[0];
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) O[vb] *= alpha;
    }
    l_run += rs;
    m_run = m_new;
    // PV: value rows 16 kk + 4 g + (j16 / 4) (+ 8), columns 32 vb + 16 (n / 16) + 4 (j16 % 4); one
    // LDS-space base per tile, the rest constant offsets of the reads
    const MLA_LDS uint8_t* va = (const MLA_LDS uint8_t*)lds + (it % NSLOT) * SLOT + va_lane;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        const MLA_LDS uint8_t* pa = va + 16 * kk * VCHP * 16 + 64 * vb;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)pa);
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(pa + 8 * VCHP * 16));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, x0).x, __builtin_bit_cast(u32x2, x0).y,
                                                           __builtin_bit_cast(u32x2, x1).x, __builtin_bit_cast(u32x2, x1).y});
        O[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], O[vb], 0, 0, 0);
      }
  }
  // o[b * C + t][i * 128 + 32 vb + 8 (r / 4) + 4 g + r % 4] = O / l, rounded to bf16
  l_run = halves_sum(l_run);
  if (t < C) {
    const float inv = 1.f / l_run;
    uint16_t* dst = o + ((int64_t)b * C + t) * NHD + (int64_t)i * DH + 4 * g;
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(u32x2*)(dst + 32 * vb + 8 * r4) = u32x2{pack_bf16x2(O[vb][4 * r4] * inv, O[vb][4 * r4 + 1] * inv),
                                                  pack_bf16x2(O[vb][4 * r4 + 2] * inv, O[vb][4 * r4 + 3] * inv)};
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
                              const float* q_pe, const void* ws, float qscale, void* o, hipStream_t st) {
  const NaiveLayout L = naive_layout(n_h, B, max_ctx);
  const uint16_t* ctx = (const uint16_t*)((const char*)ws + L.off_ctx);
  const uint16_t* kc = (const uint16_t*)((const char*)ws + L.off_kc);
  const uint16_t* vv = (const uint16_t*)((const char*)ws + L.off_v);
  // one-dimensional grid of (sequence, head, query block) tiles, padded to a multiple of 8
  const int64_t tiles = (int64_t)((C + nv::QB - 1) / nv::QB) * n_h * B;
  hipLaunchKernelGGL(k_mha_prefill, dim3((unsigned)((tiles + 7) & ~(int64_t)7)), dim3(256), 0, st, B, C, max_ctx,
                     n_h, p0, q_c, q_pe, ctx, kc, vv, qscale, (uint16_t*)o);
  return hipGetLastError();
}

}  // namespace mla
