// Projection GEMMs of the decode step: query pathway with W^UK absorbed, the current token's
// KV projection, and the two-step output (W^UV, then W^O).
//
// "DeepSeek-V2 from Scratch" section 4.1 (c^Q = W^DQ h; q^C = W^UQ c^Q; raw q^R = W^QR c^Q),
// section 2.1 (c^KV = W^DKV h), section 4.2 (raw k^R = W^KR h), section 5.1 (absorbed query
// q~_i = (W^UK_i)^T q^C_i), section 5.2 (o_i = W^UV_i o_lat_i) and section 6 (u = W^O [o]).
//
// All are "skinny" products Y[n][m] = sum_k W(m, k) X[n][k] with n over the batch (tens of rows)
// and W read exactly once from HBM, so they are bound by weight bandwidth. bf16 weights run on
// MFMA: W (the A operand) streams through a ring of LDS stages fed by direct global->LDS copies,
// several stages ahead of the math; float32 activations are split into hi + lo bf16 parts
// (x = hi + lo holds 16 significand bits), costing a second MFMA that is free under the
// bandwidth bound and keeping the activation error near float32 instead of bf16. float32 /
// float16 weights run on a tiled float32 VALU kernel.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

// ------------------------------------------------------------------ workspace layouts
static size_t al256h(size_t x) { return (x + 255) & ~(size_t)255; }

namespace gm {
constexpr int MAXB = 128;      // columns per tile (batch rows) of the widest MFMA tile
constexpr int MT = 128;        // output rows per workgroup (4 waves x 32)
constexpr int KC = 64;         // k per pipeline stage
constexpr int TARGET_WG = 256; // workgroups aimed for when choosing the K split
}

// K split of a launch with `mtiles` row tiles, S stages of KC and Z batched problems: enough
// workgroups to cover the chip once, never more slices than stages.
static int split_for(int mtiles, int S, int Z) {
  int sk = gm::TARGET_WG / (mtiles * Z);
  if (sk < 1) sk = 1;
  if (sk > S) sk = S;
  return sk;
}
static int cdiv(int a, int b) { return (a + b - 1) / b; }

// column tiles of an N-column product (128 columns each)
static int col_tiles(int N) { return cdiv(N, gm::MAXB); }
struct QSplits { int sk1; };
static QSplits q_splits(const mla_dims& d, int B) {
  // the first projection runs on 64-row tiles (more workgroups, so a smaller K split)
  return {split_for(cdiv(d.d_cq + d.d_c + d.d_r, 64) * col_tiles(B), d.d / gm::KC, 1)};
}
struct OSplits { int sk4, sk5; };
// W^O runs on 256-row tiles when the batch is at most 64 rows
static bool o_wide(int B) { return B <= 64; }
static OSplits o_splits(const mla_dims& d, int B) {
  // W^UV: one workgroup per (head, 64 rows); a K split would add a reduction pass
  return {1, split_for(cdiv(d.d, o_wide(B) ? 2 * gm::MT : gm::MT) * col_tiles(B), d.n_h * d.d_h / gm::KC, 1)};
}

// Wide products (N >= cgm::MIN_N: chunked prefill) run on the compute-shaped kernel k_cgemm:
// 256 (or, for products of at most 128 rows, 128) rows x 128 columns per workgroup, two
// workgroups per CU. Its K split only tops a small tile count up to about two workgroups per CU.
namespace cgm {
constexpr int MIN_N = 256;   // columns from which a product takes the compute-shaped kernel
constexpr int BN = 128;      // columns per workgroup
constexpr int BK = 32;       // k per stage
}
static int cg_bm(int Mtot) { return Mtot <= 128 ? 128 : 256; }
// 256 x 256 tiles (one workgroup per CU) for long-K products with many rows: half the operand
// traffic per MFMA of the 256 x 128 tile
static bool cg_big(int Mtot, int K) { return Mtot >= 2048 && K >= 8192; }
static int cg_split(int Mtot, int N, int K, int Z) {
  const bool big = cg_big(Mtot, K);
  const int slots = big ? 256 : 512;   // resident workgroups
  const int tiles = cdiv(Mtot, cg_bm(Mtot)) * cdiv(N, big ? 2 * cgm::BN : cgm::BN) * Z;
  if (tiles >= 3 * slots / 4) return 1;
  int sk = (slots + tiles / 2) / tiles;
  const int smax = K / 512 > 1 ? K / 512 : 1;   // at least 16 stages per slice
  return sk < 1 ? 1 : (sk > smax ? smax : sk);
}

AbsorbQLayout absorb_q_layout(const mla_dims& d, int B) {
  AbsorbQLayout L;
  const int sk1 = q_splits(d, B).sk1;
  L.off_cq = 0;
  L.off_qc = al256h((size_t)B * d.d_cq * 4);
  L.off_part = L.off_qc + al256h((size_t)B * d.n_h * d.d_h * 4);
  L.part_floats = sk1 > 1 ? (size_t)sk1 * B * (d.d_cq + d.d_c + d.d_r) : 0;
  if (B >= cgm::MIN_N) {
    const int m1 = d.d_cq + d.d_c + d.d_r, c1 = cg_split(m1, B, d.d, 1);
    const size_t pc = c1 > 1 ? (size_t)c1 * B * m1 : 0;
    if (pc > L.part_floats) L.part_floats = pc;
  }
  L.bytes = L.off_part + al256h(L.part_floats * 4);
  return L;
}
AbsorbOutLayout absorb_out_layout(const mla_dims& d, int B) {
  AbsorbOutLayout L;
  const OSplits sp = o_splits(d, B);
  L.off_o = 0;
  L.off_part = al256h((size_t)B * d.n_h * d.d_h * 4);
  const size_t p4 = sp.sk4 > 1 ? (size_t)sp.sk4 * d.n_h * B * d.d_h : 0;
  size_t p5 = sp.sk5 > 1 ? (size_t)sp.sk5 * B * d.d : 0;
  if (B >= cgm::MIN_N) {
    const int c4 = cg_split(d.d_h, B, d.d_c, d.n_h), c5 = cg_split(d.d, B, d.n_h * d.d_h, 1);
    if (c5 > 1 && (size_t)c5 * B * d.d > p5) p5 = (size_t)c5 * B * d.d;
    if (c4 > 1 && (size_t)c4 * d.n_h * B * d.d_h > p5) p5 = (size_t)c4 * d.n_h * B * d.d_h;
  }
  L.part_floats = p4 > p5 ? p4 : p5;
  L.bytes = L.off_part + al256h(L.part_floats * 4);
  return L;
}

// u = Wo_pre [o_lat] in one product (pre-combined form): only the K-split partials
static OSplits o_pre_splits(const mla_dims& d, int B) {
  return {1, split_for(cdiv(d.d, o_wide(B) ? 2 * gm::MT : gm::MT) * col_tiles(B), d.n_h * d.d_c / gm::KC, 1)};
}
AbsorbOutLayout absorb_out_pre_layout(const mla_dims& d, int B) {
  AbsorbOutLayout L;
  const int sk = o_pre_splits(d, B).sk5;
  L.off_o = 0;
  L.off_part = 0;
  L.part_floats = sk > 1 ? (size_t)sk * B * d.d : 0;
  if (B >= cgm::MIN_N) {
    const int c5 = cg_split(d.d, B, d.n_h * d.d_c, 1);
    if (c5 > 1 && (size_t)c5 * B * d.d > L.part_floats) L.part_floats = (size_t)c5 * B * d.d;
  }
  L.bytes = al256h(L.part_floats * 4);
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

// 16-byte global -> LDS copy per lane: uniform 64-bit base in SGPRs + 32-bit lane offset; the LDS
// destination is the wave-uniform `lds_addr` + 16 * lane. Written as asm so the compiler does not
// wait for every outstanding copy before each LDS read; the kernel counts them itself.
__device__ __forceinline__ void g2l16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
// The same copy, non-temporal: for weights, read once per product, so that their stream does not
// evict the activations every workgroup re-reads from L2.
__device__ __forceinline__ void g2l16_nt(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
// The same copy from a per-lane 64-bit address (rows of different stacked products in one tile).
__device__ __forceinline__ void g2l16_v_nt(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(src), "s"(lds_addr) : "memory", "m0");
}
// At most N copies of this wave still in flight, this wave's LDS reads done, then barrier.
template <int N>
__device__ __forceinline__ void wait_copies_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// ================================================================================================
// Weight-streaming MFMA GEMM: Y[n][m] = sum_k W(m, k) X[n][k], W bf16 row-major (lda = K).
// Workgroup = 32*MB output rows x 32*NB columns (a column tile; N beyond it takes more tiles),
// over one K slice, one wave per SIMD. The
// slice streams through an NS-deep ring of LDS stages (64 k each: the W tile and the matching X
// columns) filled by direct global->LDS copies, up to NS-1 stages ahead of the MFMAs. LDS rows
// are XOR-swizzled in 16-byte chunks so the MFMA fragment reads are conflict-free.
// Wave w runs k-step w of every stage for all rows (MB m-blocks) and all N columns; the four
// partial tiles are summed through LDS at the end. The reduction index is permuted inside each
// 64-k stage: in k-step st, lane half g supplies k = 32g + 8st + 0..7 for both operands (the same
// real k on both sides of every product).
// Software pipeline per stage j: the copies of stage j + NS - 1 are issued one after each of the
// first MFMAs; four MFMAs before the end, the wave waits for stage j + 1, joins the barrier and
// requests the next fragments, so the LDS latency and the barrier hide under the last MFMAs.
// The MFMAs are volatile asm (the copies must stay between them): each starts with 2 wait states
// for a VALU-written operand, and the accumulators are read only after the loop's closing nops.
//   XF32: X is float32, split on the fly into bf16 hi + lo (2 MFMAs, ~16 significand bits);
//         otherwise X is bf16.
//   split_k > 1: partial sums go to part[(ky * Z + z) * N + n][m] for the ordered reduction.
template <int NB, bool XF32, int MB>
struct WCfg {
  static constexpr int WB = 32 * MB * gm::KC * 2;                // W bytes per stage
  static constexpr int XROW = gm::KC * (XF32 ? 4 : 2);            // X bytes per row per stage
  static constexpr int XB = NB * 32 * XROW;                       // X bytes per stage
  static constexpr int SB = WB + XB;
  static constexpr int NS = (163840 / SB) < 6 ? (163840 / SB) : 6;
  static constexpr int DW = WB / 4096;                            // copies per thread per stage
  static constexpr int DX = XB / 4096;
  static constexpr int DT = DW + DX;
  static constexpr int NM = MB * NB * (XF32 ? 2 : 1);             // MFMAs per wave per stage
};

template <int N>
__device__ __forceinline__ void wait_ahead(int ahead) {
  switch (ahead) {
    case 0: wait_copies_barrier<0>(); break;
    case 1: wait_copies_barrier<N>(); break;
    case 2: wait_copies_barrier<2 * N>(); break;
    case 3: wait_copies_barrier<3 * N>(); break;
    default: wait_copies_barrier<4 * N>(); break;
  }
}

// Eight float32 values (v0, then v1) as bf16 hi + lo parts (x = hi + lo to ~16 significand bits).
// Pairs are rounded to bf16 in one conversion; a bf16 widens back to float by placing its bits in
// the high half, so lo = x - hi is exact before its own rounding.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <int NB, bool XF32, int MB>
__global__ __launch_bounds__(256, 1) void k_wgemm(Seg seg, int N, int ntiles, int K, const void* __restrict__ Xv,
                                                  int64_t ldx, int split_k, float* __restrict__ part,
                                                  int Mtot, int64_t zW, int64_t zX, int64_t zY) {
  using C = WCfg<NB, XF32, MB>;
  constexpr int MT = 32 * MB, KC = gm::KC, NS = C::NS, DT = C::DT, NM = C::NM;
  static_assert(NS >= 3 && (NS - 1) * DT <= 63, "ring depth / vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NS * C::SB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // One column tile: blockIdx.x is the row tile. Several: workgroups are dealt round-robin to
  // the 8 XCDs, so blockIdx.x is mapped to tile t = (x % 8) * (gridDim.x / 8) + x / 8 (gridDim.x
  // is a multiple of 8) and t = row tile * ntiles + column tile; each XCD then runs consecutive
  // column tiles of the same row tile, which read that W slice from its L2 rather than HBM.
  int mt = blockIdx.x, nt = 0;
  if (ntiles > 1) {
    const int t = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
    if (t >= ((Mtot + MT - 1) / MT) * ntiles) return;   // padding workgroup (uniform)
    mt = t / ntiles;
    nt = t - mt * ntiles;
  }
  const int ky = blockIdx.y, z = blockIdx.z, Z = gridDim.z;
  const int n0 = nt * 32 * NB;                         // first column of this tile
  const int NL = (N - n0) < 32 * NB ? (N - n0) : 32 * NB;
  const int m_base = mt * MT;
  const int S = K / KC;
  const int st0 = (int)((int64_t)S * ky / split_k), st1 = (int)((int64_t)S * (ky + 1) / split_k);
  const int ns = st1 - st0;
  constexpr int ESX = XF32 ? 4 : 2;
  const uint8_t* Xb = (const uint8_t*)Xv + ((int64_t)z * zX + (int64_t)n0 * ldx) * ESX;

  // Copy plan: thread tid fills 16-byte LDS slots p = 256 i + tid. W slot p: row p / 8, physical
  // chunk p % 8, which holds logical chunk (p % 8) ^ ((row / 2) % 8); each W lane addresses its row
  // in its own segment (a tile may straddle two stacked products), rows past the last one re-read
  // it. X slot (bf16): same with 8 chunks per row; X slot (float32): 16 chunks per row, logical
  // chunk (p % 16) ^ (row % 16).
  // Rows past the segment / past N re-read the last valid row (their results are dropped).
  uint32_t ofs[DT];
  const uint8_t* wrow[C::DW];
  {
    const int wc = (tid & 7) ^ ((tid >> 4) & 7);
#pragma unroll
    for (int i = 0; i < C::DW; ++i) {
      int m = m_base + i * 32 + (tid >> 3);
      if (m > Mtot - 1) m = Mtot - 1;
      const int sg = seg_of(seg, m);
      wrow[i] = (const uint8_t*)seg.W[sg] + ((int64_t)z * zW + (int64_t)(m - seg.m0[sg]) * K) * 2 + (wc << 4);
      ofs[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < C::DX; ++i) {
      const int p = i * 256 + tid;
      int row, c;
      if constexpr (XF32) { row = p >> 4; c = (p & 15) ^ (row & 15); }
      else { row = p >> 3; c = (p & 7) ^ ((row >> 1) & 7); }
      if (row > NL - 1) row = NL - 1;
      ofs[C::DW + i] = (uint32_t)((int64_t)row * ldx * ESX) + (uint32_t)(c << 4);
    }
  }
  // copy i (0 .. DT-1) of stage j: W pieces first, then X pieces
  auto copy = [&](int j, int i) __attribute__((always_inline)) {
    const int kst = (st0 + j) * KC;
    uint8_t* buf = lds + (j % NS) * C::SB;
    if (i < C::DW) {
      const uint32_t wl = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLA_LDS void*)(buf + w * 1024));
      g2l16_v_nt(wrow[i] + (int64_t)kst * 2, wl + i * 4096);
    } else {
      const uint32_t xl = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLA_LDS void*)(buf + C::WB + w * 1024));
      g2l16(Xb + (int64_t)kst * ESX, ofs[i], xl + (i - C::DW) * 4096);
    }
  };

  // Fragment offsets inside a stage (k-step w):
  //   A (m-block mb): row 32 mb + l32, logical chunk 4g + w;  B (bf16): row 32 jb + l32, same
  //   chunk;  B (float32): row 32 jb + l32, logical chunks 8g + 2w and 8g + 2w + 1.
  const int key8 = (l32 >> 1) & 7;
  const uint32_t aoff = (uint32_t)(l32 * 128 + (((4 * g + w) ^ key8) << 4));
  const uint32_t boff = (uint32_t)(C::WB + l32 * 128 + (((4 * g + w) ^ key8) << 4));
  const uint32_t bofx0 = (uint32_t)(C::WB + l32 * 256 + (((8 * g + 2 * w) ^ (l32 & 15)) << 4));
  const uint32_t bofx1 = (uint32_t)(C::WB + l32 * 256 + (((8 * g + 2 * w + 1) ^ (l32 & 15)) << 4));

  // raw fragments of one stage, straight from LDS
  struct Frag {
    bf16x8 a[MB];
    f32x4 x0[XF32 ? NB : 1], x1[XF32 ? NB : 1];
    bf16x8 b[XF32 ? 1 : NB];
  };
  auto load_frag = [&](int j, Frag& f) __attribute__((always_inline)) {
    const uint8_t* buf = lds + (j % NS) * C::SB;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) f.a[mb] = *(const bf16x8*)(buf + aoff + mb * 32 * 128);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      if constexpr (XF32) {
        f.x0[jb] = *(const f32x4*)(buf + bofx0 + jb * 32 * 256);
        f.x1[jb] = *(const f32x4*)(buf + bofx1 + jb * 32 * 256);
      } else {
        f.b[jb] = *(const bf16x8*)(buf + boff + jb * 32 * 128);
      }
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = f32x16{};

  for (int j = 0; j < NS - 1 && j < ns; ++j)
#pragma unroll
    for (int i = 0; i < DT; ++i) copy(j, i);
  {
    const int ahead = (ns - 1) < (NS - 2) ? (ns - 1) : (NS - 2);
    wait_ahead<DT>(ahead);
  }
  Frag cur;
  load_frag(0, cur);
  constexpr int QB = NM > 4 ? NM - 4 : 0;  // MFMA slot before which the next stage is requested
  for (int j = 0; j < ns; ++j) {
    const bool more = j + 1 < ns;
    const bool refill = j + NS - 1 < ns;
    Frag nxt;
    bf16x8 bh, bl;
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      // MFMA order: (jb, half, mb); one accumulator is never used by two consecutive MFMAs
      const int jb = q / (XF32 ? 2 * MB : MB), half = XF32 ? (q / MB) & 1 : 0, mb = q % MB;
      if (q == QB) {
        if (refill)
#pragma unroll
          for (int i = (QB < DT ? QB : DT); i < DT; ++i) copy(j + NS - 1, i);
        if (more) {
          const int ahead = (ns - 2 - j) < (NS - 2) ? (ns - 2 - j) : (NS - 2);
          wait_ahead<DT>(ahead);
          load_frag(j + 1, nxt);
        }
      }
      if constexpr (XF32) {
        if (q % (2 * MB) == 0) {
          split_hi_lo(cur.x0[jb], cur.x1[jb], bh, bl);
        }
        mfma_acc(acc[mb][jb], cur.a[mb], half ? bl : bh);
      } else {
        mfma_acc(acc[mb][jb], cur.a[mb], cur.b[jb]);
      }
      if (refill && q < QB && q < DT) copy(j + NS - 1, q);
    }
    cur = nxt;
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");  // last MFMA results readable

  // Sum of the four waves' tiles, one m-block at a time through two alternating LDS regions
  // (wave-major, fixed order w = 0..3). Accumulator element r of lane (g, l32) is column
  // n = 32 jb + l32, row 32 mb + 8(r/4) + 4g + r%4: four consecutive rows per r/4.
  __syncthreads();  // every wave is done with the last stage
  constexpr int RB = 4 * NB * 4 * 64;  // float4 slots per region (waves x blocks x r4 x lanes)
  f32x4* red = (f32x4*)lds;
  // a tile inside one segment looks it up once (uniform values); otherwise row by row
  const int sg_lo = seg_of(seg, m_base);
  const bool one_seg = sg_lo == seg_of(seg, (m_base + MT < Mtot ? m_base + MT : Mtot) - 1);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    f32x4* reg = red + (mb & 1) * RB;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        reg[((w * NB + jb) * 4 + r4) * 64 + lane] =
            f32x4{acc[mb][jb][4 * r4], acc[mb][jb][4 * r4 + 1], acc[mb][jb][4 * r4 + 2], acc[mb][jb][4 * r4 + 3]};
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int idx = q * 256 + tid;           // (jb, r4, lane) of one output float4
      const int ln = idx & 63, r4 = (idx >> 6) & 3, jb = idx >> 8;
      const int n = 32 * jb + (ln & 31);
      const int mloc = 32 * mb + 8 * r4 + 4 * (ln >> 5);
      f32x4 v = reg[(jb * 4 + r4) * 64 + ln];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        const f32x4 x = reg[((ww * NB + jb) * 4 + r4) * 64 + ln];
        v[0] += x[0]; v[1] += x[1]; v[2] += x[2]; v[3] += x[3];
      }
      if (n >= NL || m_base + mloc >= Mtot) continue;
      if (split_k > 1) {
        *(f32x4*)(part + ((int64_t)(ky * Z + z) * N + n0 + n) * Mtot + m_base + mloc) = v;
      } else {
        const int m = m_base + mloc;
        const int sg = one_seg ? sg_lo : seg_of(seg, m);  // segment boundaries are multiples of 4
        *(f32x4*)(seg.Y[sg] + (int64_t)z * zY + (int64_t)(n0 + n) * seg.ldy[sg] + (m - seg.m0[sg])) = v;
      }
    }
  }
}

// ================================================================================================
// Compute-shaped MFMA GEMM for wide products (chunked prefill: N = chunk tokens, hundreds to
// thousands): Y[n][m] = sum_k W(m, k) X[n][k], W bf16 row-major (lda = K) in stacked segments, X
// float32 (split on the fly into bf16 hi + lo, 2 MFMAs) or bf16. Unlike the weight-streaming kernel
// above, both operands are tiles: a workgroup owns BM = 64 WMB rows x BN = 64 WNB columns, its four
// waves a 2 x 2 grid of (32 WMB) x (32 WNB) sub-tiles, so every operand fragment read from LDS feeds
// WNB (rows) or WMB (columns) MFMAs. Stages of 32 k go through an NS-deep LDS ring (global -> LDS
// copies, NS - 1 stages ahead of the math, one barrier per stage). LDS rows are XOR-swizzled in
// 16-byte chunks (W and bf16 X: 4 chunks per row, key (row / 4) % 4; float32 X: 8 chunks, key
// (row / 2) % 8), which makes the 16 lanes of each quarter-wave fragment read hit 16 distinct bank
// groups. Tiles may straddle segments (each copy lane and each stored row finds its own segment).
//   split_k > 1: partial sums go to part[(ky * Z + z) * N + n][m] for k_splitk_reduce.
template <bool XF32, int WMB, int WNB, int NS>
struct CgCfg {
  static constexpr int BM = 64 * WMB, BN = 64 * WNB;
  static constexpr int WB = BM * cgm::BK * 2;                   // W bytes per stage
  static constexpr int XB = BN * cgm::BK * (XF32 ? 4 : 2);        // X bytes per stage
  static constexpr int SB = WB + XB;
  static constexpr int DW = WB / 4096, DX = XB / 4096;          // copies per thread per stage
  static constexpr int DT = DW + DX;
};

__device__ __forceinline__ void g2l16_v(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_addr) : "memory", "m0");
}

template <bool XF32, int WMB, int WNB, int NS, bool OB16 = false>
__global__ __launch_bounds__(256, WMB * WNB > 8 ? 1 : (OB16 && !XF32 ? 3 : 2)) void k_cgemm(Seg seg, int N, int ntn, int gm, int K, const void* __restrict__ Xv,
                                                  int64_t ldx, int split_k, float* __restrict__ part, int Mtot,
                                                  int64_t zW, int64_t zX, int64_t zY) {
  using C = CgCfg<XF32, WMB, WNB, NS>;
  constexpr int BM = C::BM, BN = C::BN, BK = cgm::BK, DW = C::DW, DX = C::DX, DT = C::DT;
  constexpr int ESX = XF32 ? 4 : 2;
  static_assert((NS - 1) * DT <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NS * C::SB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = w & 1, wn = w >> 1;
  // consecutive tiles t go to one XCD (workgroups are dealt round-robin to the 8 XCDs)
  const int ntm = (Mtot + BM - 1) / BM;
  const int t = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
  if (t >= ntm * ntn) return;  // padding workgroup (uniform)
  // bands of gm row tiles, column tile by column tile inside a band: the tiles in flight on one XCD
  // then share a few W row tiles and a few X column tiles in its L2 (gm = 1: row tile by row tile)
  const int band = t / (gm * ntn), gmb = (ntm - band * gm) < gm ? (ntm - band * gm) : gm;
  const int idx = t - band * gm * ntn;
  const int nt = idx / gmb, mt = band * gm + (idx - nt * gmb);
  const int ky = blockIdx.y, z = blockIdx.z, Z = gridDim.z;
  const int m_base = mt * BM, n_base = nt * BN;
  const int S = K / BK;
  const int st0 = (int)((int64_t)S * ky / split_k), st1 = (int)((int64_t)S * (ky + 1) / split_k);
  const int ns = st1 - st0;

  // copy plan. W: slot p = 256 i + tid is row p / 4, physical chunk p % 4 (logical chunk
  // (p % 4) ^ ((row / 4) % 4)); rows past the product re-read its last row.
  const uint8_t* wsrc[DW];
#pragma unroll
  for (int i = 0; i < DW; ++i) {
    const int p = 256 * i + tid, row = p >> 2, lc = (p & 3) ^ ((row >> 2) & 3);
    int m = m_base + row;
    m = m < Mtot ? m : Mtot - 1;
    const int sg = seg_of(seg, m);
    wsrc[i] = (const uint8_t*)seg.W[sg] + ((int64_t)z * zW + (int64_t)(m - seg.m0[sg]) * K + (int64_t)st0 * BK + 8 * lc) * 2;
  }
  // X: float32 rows of 8 chunks (key (row / 2) % 8) or bf16 rows of 4 chunks (key (row / 4) % 4)
  const uint8_t* xsrc[DX];
#pragma unroll
  for (int i = 0; i < DX; ++i) {
    const int p = 256 * i + tid;
    int row, lc;
    if constexpr (XF32) { row = p >> 3; lc = (p & 7) ^ ((row >> 1) & 7); }
    else { row = p >> 2; lc = (p & 3) ^ ((row >> 2) & 3); }
    int n = n_base + row;
    n = n < N ? n : N - 1;
    xsrc[i] = (const uint8_t*)Xv + ((int64_t)z * zX + (int64_t)n * ldx + (int64_t)st0 * BK) * ESX + 16 * lc;
  }
  auto issue = [&](int j) __attribute__((always_inline)) {
    uint8_t* buf = lds + (j % NS) * C::SB;
    const uint32_t wl = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLA_LDS void*)(buf + w * 1024));
    const uint32_t xl = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLA_LDS void*)(buf + C::WB + w * 1024));
#pragma unroll
    for (int i = 0; i < DW; ++i) g2l16_v(wsrc[i] + (int64_t)j * BK * 2, wl + i * 4096);
#pragma unroll
    for (int i = 0; i < DX; ++i) g2l16_v(xsrc[i] + (int64_t)j * BK * ESX, xl + i * 4096);
  };

  // fragment offsets: A (m-block mb): row 32 WMB wm + 32 mb + l32, logical chunk 2 ks + g;
  // B (n-block nb): row 32 WNB wn + 32 nb + l32, float32: logical chunks 4 ks + 2 g and + 1; bf16: 2 ks + g
  auto a_off = [&](int mb, int ks) -> uint32_t {
    const int row = 32 * WMB * wm + 32 * mb + l32;
    return (uint32_t)(row * 64 + (((2 * ks + g) ^ ((row >> 2) & 3)) << 4));
  };
  auto b_off = [&](int nb, int ks, int h) -> uint32_t {
    const int row = 32 * WNB * wn + 32 * nb + l32;
    if constexpr (XF32) return (uint32_t)(C::WB + row * 128 + (((4 * ks + 2 * g + h) ^ ((row >> 1) & 7)) << 4));
    else return (uint32_t)(C::WB + row * 64 + (((2 * ks + g) ^ ((row >> 2) & 3)) << 4));
  };

  f32x16 acc[WMB][WNB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) acc[mb][nb] = f32x16{};

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < ns) issue(j);
  for (int j = 0; j < ns; ++j) {
    // stage j landed (later stages may still be in flight); every wave is done with stage j - 1
    const int ahead = (ns - 1 - j) < (NS - 2) ? (ns - 1 - j) : (NS - 2);
    if (ahead >= 2) wait_copies_barrier<2 * DT>();
    else if (ahead == 1) wait_copies_barrier<DT>();
    else wait_copies_barrier<0>();
    if (j + NS - 1 < ns) issue(j + NS - 1);   // into the buffer stage j - 1 used
    const uint8_t* buf = lds + (j % NS) * C::SB;
    // every fragment of the stage is requested at once, in the order of use (LDS reads complete in
    // order, so the first MFMAs wait only for their own operands)
    bf16x8 a[BK / 16][WMB];
    f32x4 xr[BK / 16][WNB][XF32 ? 2 : 1];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) a[ks][mb] = *(const bf16x8*)(buf + a_off(mb, ks));
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int h = 0; h < (XF32 ? 2 : 1); ++h) xr[ks][nb][h] = *(const f32x4*)(buf + b_off(nb, ks, h));
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        if constexpr (XF32) {
          bf16x8 bh, bl;
          split_hi_lo(xr[ks][nb][0], xr[ks][nb][1], bh, bl);
#pragma unroll
          for (int mb = 0; mb < WMB; ++mb) {
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][mb], bh, acc[mb][nb], 0, 0, 0);
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][mb], bl, acc[mb][nb], 0, 0, 0);
          }
        } else {
          const bf16x8 b = __builtin_bit_cast(bf16x8, xr[ks][nb][0]);
#pragma unroll
          for (int mb = 0; mb < WMB; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][mb], b, acc[mb][nb], 0, 0, 0);
        }
      }
    }
  }

  // accumulator element r of lane (g, l32): column 32 WNB wn + 32 nb + l32, row 32 WMB wm + 32 mb +
  // 8 (r / 4) + 4 g + r % 4 (four consecutive rows per r / 4; segment boundaries are multiples of 4)
  // A tile inside one segment (the usual case) looks its segment up once, with scalar values; a
  // tile across a boundary finds each row's segment.
  const int m_last = (m_base + BM < Mtot ? m_base + BM : Mtot) - 1;
  const int sg_lo = seg_of(seg, m_base);
  const bool one_seg = split_k == 1 && sg_lo == seg_of(seg, m_last);
  auto store = [&](const f32x4& v, int n, int m, int sg) __attribute__((always_inline)) {
    if constexpr (OB16) {
      // bf16 output (round to nearest even): Y holds uint16 elements, ldy in elements
      uint16_t* y = (uint16_t*)seg.Y[sg] + (int64_t)z * zY + (int64_t)n * seg.ldy[sg] + (m - seg.m0[sg]);
      *(u32x2*)y = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else {
      *(f32x4*)(seg.Y[sg] + (int64_t)z * zY + (int64_t)n * seg.ldy[sg] + (m - seg.m0[sg])) = v;
    }
  };
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb) {
    const int n = n_base + 32 * WNB * wn + 32 * nb + l32;
    if (n >= N) continue;
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int m = m_base + 32 * WMB * wm + 32 * mb + 8 * r4 + 4 * g;
        if (m >= Mtot) continue;
        const f32x4 v = {acc[mb][nb][4 * r4], acc[mb][nb][4 * r4 + 1], acc[mb][nb][4 * r4 + 2], acc[mb][nb][4 * r4 + 3]};
        if (split_k > 1) *(f32x4*)(part + ((int64_t)(ky * Z + z) * N + n) * Mtot + m) = v;
        else if (one_seg) store(v, n, m, sg_lo);
        else store(v, n, m, seg_of(seg, m));
      }
  }
}

// Ordered split-K reduction: Y[n][m] = sum_{ky} part[ky][n][m] (4 consecutive m per thread),
// scattered to the segments; blockIdx.y = batched problem z. The partials of up to 16 slices are
// requested together and then added in slice order.
__global__ __launch_bounds__(256) void k_splitk_reduce(Seg seg, int N, int Mtot, int split_k,
                                                       const float* __restrict__ part, int64_t zY) {
  const int z = blockIdx.y, Z = gridDim.y;
  const int M4 = Mtot / 4;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)N * M4) return;
  const int n = (int)(e / M4), m = (int)(e % M4) * 4;
  const int64_t slice = (int64_t)Z * N * Mtot;
  const float* src = part + ((int64_t)z * N + n) * Mtot + m;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < split_k; k0 += 16) {
    f32x4 x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      x[k] = k0 + k < split_k ? *(const f32x4*)(src + (int64_t)(k0 + k) * slice) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      v[0] += x[k][0]; v[1] += x[k][1]; v[2] += x[k][2]; v[3] += x[k][3];
    }
  }
  const int s = seg_of(seg, m);
  *(f32x4*)(seg.Y[s] + (int64_t)z * zY + (int64_t)n * seg.ldy[s] + (m - seg.m0[s])) = v;
}

// ================================================================================================
// Absorbed query: q_lat[b][i][c] = sum_e W^UK[i d_h + e][c] q^C[b][i d_h + e]. The reduction
// runs down the columns of W^UK, so a 128(e) x 128(c) tile is staged in LDS and read with the
// transposing LDS load (4 consecutive e of one column per lane). Workgroup = (head, 128 columns);
// wave w owns 32 columns; MFMA D[c][b] = sum_e A[c][e] X^T[e][b].
namespace absq {
constexpr int DH = 128, TC = 128, PITCH = 136;  // bf16 elements per W^UK row in LDS (padded)
constexpr int XP = DH + 4;                      // floats per q^C row in LDS (padded)
}
// One round trip per workgroup: the W^UK tile and this head's q^C rows (all N of them) are
// requested together, stored to LDS, then the 8 k-steps run from LDS.
template <int NB>
__global__ __launch_bounds__(256) void k_absorb_uk(int n_h, int d_c, int N, const uint16_t* __restrict__ W_uk,
                                                   const float* __restrict__ qC, float* __restrict__ q_lat) {
  using namespace absq;
  __shared__ __attribute__((aligned(16))) uint16_t tile[DH * PITCH];
  __shared__ __attribute__((aligned(16))) float xs[NB * 32 * XP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // tile t = (head i * batch chunks + chunk zc) * column tiles + column tile; consecutive t go to
  // one XCD (workgroups are dealt round-robin to the 8 XCDs), so a head's column tiles and batch
  // chunks, which share its q^C rows and W^UK tiles, read them through one L2
  const int nct = d_c / TC, nzc = (N + 32 * NB - 1) / (32 * NB);
  const int t = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
  if (t >= nct * nzc * n_h) return;  // padding workgroup (uniform)
  const int i = t / (nct * nzc);         // head
  const int c0 = (t % nct) * TC;         // column tile
  // batch rows [32 NB zc, 32 NB (zc + 1)) (one launch covers any N)
  const int nz = 32 * NB * ((t / nct) % nzc);
  N -= nz;
  qC += (int64_t)nz * n_h * DH;
  q_lat += (int64_t)nz * n_h * d_c;
  {
    // W^UK[i*128 .. +128][c0 .. c0+128]: 2048 16-byte pieces, 8 per thread;
    // q^C[n][i*128 .. +128] for n < 32 NB: 32 NB * 32 pieces, 4 NB per thread
    u32x4 wv[8];
    f32x4 xv[4 * NB];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int f = k * 256 + tid, e = f >> 4, cc = (f & 15) * 8;
      wv[k] = __builtin_nontemporal_load((const u32x4*)(W_uk + ((int64_t)i * DH + e) * d_c + c0 + cc));
    }
#pragma unroll
    for (int k = 0; k < 4 * NB; ++k) {
      const int f = k * 256 + tid, n = f >> 5, ee = (f & 31) * 4;
      xv[k] = n < N ? *(const f32x4*)(qC + (int64_t)n * n_h * DH + (int64_t)i * DH + ee) : f32x4{};
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int f = k * 256 + tid, e = f >> 4, cc = (f & 15) * 8;
      *(u32x4*)(tile + e * PITCH + cc) = wv[k];
    }
#pragma unroll
    for (int k = 0; k < 4 * NB; ++k) {
      const int f = k * 256 + tid, n = f >> 5, ee = (f & 31) * 4;
      *(f32x4*)(xs + n * XP + ee) = xv[k];
    }
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
      // B[e][n] = q^C[n][i*128 + e], e = 16ks + 8g + 0..7: slots 0-3 come from the first
      // transposed read (rows e0..), slots 4-7 from the second (rows e0 + 4..).
      const float* xr = xs + (32 * j + l32) * XP + 16 * ks + 8 * g;
      const f32x4 v0 = *(const f32x4*)xr, v1 = *(const f32x4*)(xr + 4);
      bf16x8 bh, bl;
      split_hi_lo(v0, v1, bh, bl);
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
// Tile 64 (m) x 16 (n) per 256 threads, k in steps of 32 through LDS. The shapes it serves are
// small (tens of workgroups), so each step's compute is far shorter than a load round trip: the
// elements of the next PD steps are kept in flight in registers (one round trip per 256 k).
// Barrier for LDS hand-offs only (waits for this wave's LDS operations, not its global loads).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Up to 3 products sharing X, K and lda launched as one grid (segment s owns the 64-row tiles
// [t0[s], t0[s+1]) of blockIdx.x): the running model's first projections are too small to fill
// the chip one at a time.
struct VSeg {
  int n;
  int t0[4];
  const void* W[3];
  float* Y[3];
  int64_t ldy[3];
  int M[3];
};

template <int ADT, int XDT, bool TRANS>
__global__ __launch_bounds__(256) void k_gemm_valu(VSeg sg, int N, int K, int64_t lda, int64_t zW,
                                                   const void* __restrict__ Xv, int64_t ldx, int64_t zX,
                                                   int64_t zY) {
  __shared__ float Ws[64][33];
  __shared__ float Xs[16][33];
  const int tid = threadIdx.x;
  const int mt = blockIdx.x;
  const int s = sg.n > 2 && mt >= sg.t0[2] ? 2 : (sg.n > 1 && mt >= sg.t0[1] ? 1 : 0);
  const int M = sg.M[s];
  const int64_t ldy = sg.ldy[s];
  float* __restrict__ Y = sg.Y[s];
  const int m0 = (mt - sg.t0[s]) * 64, n0 = blockIdx.y * 16, z = blockIdx.z;
  const typename Elem<ADT>::T* W = (const typename Elem<ADT>::T*)sg.W[s] + (int64_t)z * zW;
  const typename Elem<XDT>::T* X = (const typename Elem<XDT>::T*)Xv + (int64_t)z * zX;
  const int mi = tid & 63, nq = tid >> 6;  // thread: row mi, columns nq*4 .. nq*4+3
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  // the elements of k-chunks k0 .. k0 + 32 PD - 32 are fetched into registers (slot p holds
  // chunk k0 + 32p) while earlier chunks are used from LDS; barriers wait for LDS only, so those
  // loads stay in flight. Loads use clamped (always valid) indices and keep the stored bits:
  // a conditional load, or a conversion at the load, makes the compiler wait for it at once.
  constexpr int PD = 8;
  typename Elem<ADT>::T wr[PD][8];
  typename Elem<XDT>::T xr[PD][2];
  auto w_el = [&](int q, int& mm, int& kk) __attribute__((always_inline)) {
    const int e = tid + 256 * q;
    if (TRANS) { mm = e & 63; kk = e >> 6; } else { kk = e & 31; mm = e >> 5; }
  };
  auto fetch = [&](int p, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      int mm, kk;
      w_el(q, mm, kk);
      const int m = min(m0 + mm, M - 1), k = min(k0 + kk, K - 1);
      wr[p][q] = W[TRANS ? (int64_t)k * lda + m : (int64_t)m * lda + k];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q;
      const int n = min(n0 + (e >> 5), N - 1), k = min(k0 + (e & 31), K - 1);
      xr[p][q] = X[(int64_t)n * ldx + k];
    }
  };
#pragma unroll
  for (int p = 0; p < PD; ++p)
    if (32 * p < K) fetch(p, 32 * p);
  for (int kb = 0; kb < K; kb += 32 * PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int k0 = kb + 32 * p;
      if (k0 >= K) break;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        int mm, kk;
        w_el(q, mm, kk);
        Ws[mm][kk] = (m0 + mm < M && k0 + kk < K) ? Elem<ADT>::cvt(wr[p][q]) : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = tid + 256 * q;
        Xs[e >> 5][e & 31] = (n0 + (e >> 5) < N && k0 + (e & 31) < K) ? Elem<XDT>::cvt(xr[p][q]) : 0.f;
      }
      lds_sync();
      if (k0 + 32 * PD < K) fetch(p, k0 + 32 * PD);
#pragma unroll 8
      for (int kk = 0; kk < 32; ++kk) {
        const float a = Ws[mi][kk];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += a * Xs[nq * 4 + q][kk];
      }
      lds_sync();
    }
  }
  const int m = m0 + mi;
  if (m >= M) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = n0 + nq * 4 + q;
    if (n < N) Y[(int64_t)z * zY + (int64_t)n * ldy + m] = acc[q];
  }
}

// ================================================================================================
// Small products at decode batch sizes (N <= 64), any weight type, on float32 MFMA:
//   Y[n][m] = sum_k A(m, k) X[n][k],  A(m, k) = TRANS ? W[k*lda + m] : W[m*lda + k].
// The running model's projections are a few hundred rows by a few hundred k: too little work to
// fill the chip, so their time is latency. A workgroup owns a 16 (m) x 16 (n) output tile and its
// four waves split K in 32-k chunks (wave w: chunks w, w + 4, ...); one LDS reduction at the end.
// v_mfma_f32_16x16x4_f32 multiplies the widened weights and float32 activations exactly, as the
// VALU kernel does. Lane (g, r) supplies row m0 + r of A and row n0 + r of X for k = 32c + 8g + e
// in the e-th MFMA of chunk c (the same k on both sides), so each lane reads 8 consecutive k
// (one vector load when aligned; TRANS weights: the 16 lanes of a group read 16 consecutive m).
// Stacked segments as in VSeg, with tile starts in units of 16 rows.
template <int DT>
__device__ __forceinline__ void load8(const typename Elem<DT>::T* p, bool vec, int valid, float (&v)[8]) {
  if (vec && valid >= 8) {
    if constexpr (DT == MLA_F32) {
      const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
    } else {
      const u32x4 a = *(const u32x4*)p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = Elem<DT>::cvt((uint16_t)(a[e] & 0xffffu));
        v[2 * e + 1] = Elem<DT>::cvt((uint16_t)(a[e] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < valid ? Elem<DT>::ld(p, e) : 0.f;
  }
}

template <int ADT, int XDT, bool TRANS>
__global__ __launch_bounds__(256) void k_gemm_tiny(VSeg sg, int N, int K, int64_t lda, int64_t zW,
                                                  const void* __restrict__ Xv, int64_t ldx, int64_t zX, int64_t zY,
                                                  int wvec, int xvec) {
  __shared__ f32x4 red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int mt = blockIdx.x;
  const int s = sg.n > 2 && mt >= sg.t0[2] ? 2 : (sg.n > 1 && mt >= sg.t0[1] ? 1 : 0);
  const int M = sg.M[s];
  const int m0 = (mt - sg.t0[s]) * 16, n0 = blockIdx.y * 16, z = blockIdx.z;
  const typename Elem<ADT>::T* W = (const typename Elem<ADT>::T*)sg.W[s] + (int64_t)z * zW;
  const typename Elem<XDT>::T* X = (const typename Elem<XDT>::T*)Xv + (int64_t)z * zX;
  const int m = min(m0 + r, M - 1), n = min(n0 + r, N - 1);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nchunk = (K + 31) / 32;
  for (int c = w; c < nchunk; c += 4) {
    const int kb = 32 * c + 8 * g;
    const int valid = K - kb < 8 ? (K - kb > 0 ? K - kb : 0) : 8;
    float a[8], x[8];
    if constexpr (TRANS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = e < valid ? Elem<ADT>::ld(W, (int64_t)(kb + e) * lda + m) : 0.f;
    } else {
      load8<ADT>(W + (int64_t)m * lda + kb, wvec != 0, valid, a);
    }
    load8<XDT>(X + (int64_t)n * ldx + kb, xvec != 0, valid, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], x[e], acc, 0, 0, 0);
  }
  red[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 v = red[0][lane];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) v += red[ww][lane];
    // lane (g, r): column n0 + r, rows m0 + 4g .. + 3
    if (n0 + r < N) {
      float* Y = sg.Y[s] + (int64_t)z * zY + (int64_t)(n0 + r) * sg.ldy[s];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m0 + 4 * g + i < M) Y[m0 + 4 * g + i] = v[i];
    }
  }
}

// ------------------------------------------------------------------ dispatch helpers
static VSeg vseg1(int M, const void* W, float* Y, int64_t ldy) {
  VSeg sg{};
  sg.n = 1;
  sg.t0[0] = 0;
  sg.t0[1] = (M + 63) / 64;
  sg.W[0] = W;
  sg.Y[0] = Y;
  sg.ldy[0] = ldy;
  sg.M[0] = M;
  return sg;
}

// decode batch sizes take the small-product MFMA kernel (16-row tiles), wider N the VALU tiles
constexpr int TINY_N = 64;
template <int ADT, int XDT, bool TRANS>
static void valu_seg(hipStream_t st, const VSeg& sg, int N, int K, int64_t lda, int64_t zW, const void* X,
                     int64_t ldx, int64_t zX, int64_t zY, int Z) {
  if (N <= TINY_N) {
    VSeg t = sg;
    t.t0[0] = 0;
    for (int i = 0; i < sg.n; ++i) t.t0[i + 1] = t.t0[i] + (sg.M[i] + 15) / 16;
    // 16-byte vector loads of 8 consecutive k: row strides and bases must keep them aligned
    auto al = [](const void* ptr, int64_t ld, int64_t zs, int es) {
      return (int)(((uintptr_t)ptr % 16) == 0 && (ld * es) % 16 == 0 && (zs * es) % 16 == 0);
    };
    constexpr int EA = ADT == MLA_F32 ? 4 : 2, EX = XDT == MLA_F32 ? 4 : 2;
    int wv = !TRANS;
    for (int i = 0; i < sg.n; ++i) wv &= al(sg.W[i], lda, zW, EA);
    const int xv = al(X, ldx, zX, EX);
    dim3 grid(t.t0[t.n], (N + 15) / 16, Z);
    hipLaunchKernelGGL((k_gemm_tiny<ADT, XDT, TRANS>), grid, dim3(256), 0, st, t, N, K, lda, zW, X, ldx, zX, zY,
                       wv, xv);
    return;
  }
  dim3 grid(sg.t0[sg.n], (N + 15) / 16, Z);
  hipLaunchKernelGGL((k_gemm_valu<ADT, XDT, TRANS>), grid, dim3(256), 0, st, sg, N, K, lda, zW, X, ldx, zX, zY);
}
template <int ADT, int XDT, bool TRANS>
static void valu(hipStream_t st, int M, int N, int K, const void* W, int64_t lda, int64_t zW, const void* X,
                 int64_t ldx, int64_t zX, float* Y, int64_t ldy, int64_t zY, int Z) {
  valu_seg<ADT, XDT, TRANS>(st, vseg1(M, W, Y, ldy), N, K, lda, zW, X, ldx, zX, zY, Z);
}
// Three products Y_s[n][m] = sum_k W_s[m][k] X[n][k] (W_s row-major with lda = K; X in the weight
// dtype) in one launch.
static void valu_stacked(int wdt, hipStream_t st, int N, int K, const void* X, int64_t ldx, const void* W0,
                         int M0, float* Y0, int64_t ldy0, const void* W1, int M1, float* Y1, int64_t ldy1,
                         const void* W2, int M2, float* Y2, int64_t ldy2) {
  VSeg sg{};
  sg.n = 3;
  sg.t0[0] = 0;
  sg.t0[1] = (M0 + 63) / 64;
  sg.t0[2] = sg.t0[1] + (M1 + 63) / 64;
  sg.t0[3] = sg.t0[2] + (M2 + 63) / 64;
  sg.W[0] = W0; sg.W[1] = W1; sg.W[2] = W2;
  sg.Y[0] = Y0; sg.Y[1] = Y1; sg.Y[2] = Y2;
  sg.ldy[0] = ldy0; sg.ldy[1] = ldy1; sg.ldy[2] = ldy2;
  sg.M[0] = M0; sg.M[1] = M1; sg.M[2] = M2;
  if (wdt == MLA_F32) valu_seg<MLA_F32, MLA_F32, false>(st, sg, N, K, K, 0, X, ldx, 0, 0, 1);
  else if (wdt == MLA_F16) valu_seg<MLA_F16, MLA_F16, false>(st, sg, N, K, K, 0, X, ldx, 0, 0, 1);
  else valu_seg<MLA_BF16, MLA_BF16, false>(st, sg, N, K, K, 0, X, ldx, 0, 0, 1);
}

// Two products Y_s[n][m] = sum_k W_s[m][k] X[n][k] sharing a float32 X (W_s row-major, lda = K) in
// one launch.
static void valu_pair_f32x(int wdt, hipStream_t st, int N, int K, const float* X, int64_t ldx, const void* W0,
                           int M0, float* Y0, int64_t ldy0, const void* W1, int M1, float* Y1, int64_t ldy1) {
  VSeg sg{};
  sg.n = 2;
  sg.t0[0] = 0;
  sg.t0[1] = (M0 + 63) / 64;
  sg.t0[2] = sg.t0[1] + (M1 + 63) / 64;
  sg.W[0] = W0; sg.W[1] = W1;
  sg.Y[0] = Y0; sg.Y[1] = Y1;
  sg.ldy[0] = ldy0; sg.ldy[1] = ldy1;
  sg.M[0] = M0; sg.M[1] = M1;
  if (wdt == MLA_F32) valu_seg<MLA_F32, MLA_F32, false>(st, sg, N, K, K, 0, X, ldx, 0, 0, 1);
  else if (wdt == MLA_F16) valu_seg<MLA_F16, MLA_F32, false>(st, sg, N, K, K, 0, X, ldx, 0, 0, 1);
  else valu_seg<MLA_BF16, MLA_F32, false>(st, sg, N, K, K, 0, X, ldx, 0, 0, 1);
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

// Y[n][m] = sum_k W[m][k] X[n][k] (W row-major, lda = ldx = K, X float32) with K cut into S
// slices: the slices run as S batched problems into part[S][N][M] (float32; at least S*N*M floats),
// then k_splitk_reduce adds them in slice order into Y (deterministic). For products whose few
// 64-row tiles would otherwise each run the whole K serially. Falls back to one launch when K does
// not split into slices of at least 32.
static void valu_splitk(int wdt, hipStream_t st, int M, int N, int K, const void* W, const float* X, float* Y,
                        int64_t ldy, int S, float* part) {
  if (N <= TINY_N || S < 2 || K % S != 0 || K / S < 32 || M % 4 != 0 || part == nullptr) {
    valu_any(wdt, false, false, st, M, N, K, W, K, 0, X, K, 0, Y, ldy, 0, 1);
    return;
  }
  const int Ks = K / S;
  valu_any(wdt, false, false, st, M, N, Ks, W, K, Ks, X, K, Ks, part, M, (int64_t)N * M, S);
  Seg sg{};
  sg.Y[0] = Y; sg.ldy[0] = ldy;
  sg.m0[0] = 0; sg.m0[1] = M; sg.nseg = 1;
  const int64_t n4 = (int64_t)N * (M / 4);
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((n4 + 255) / 256), 1), dim3(256), 0, st, sg, N, M, S,
                     (const float*)part, (int64_t)0);
}

static bool mfma_dims_ok(const mla_dims& d) {
  return d.d % 256 == 0 && d.d_cq % 256 == 0 && d.d_cq % 64 == 0 && d.d_c % 128 == 0 && d.d_r % 64 == 0 &&
         d.d_h == absq::DH && (d.n_h * d.d_h) % 256 == 0;
}

template <int NB, bool XF32, int MB>
static void wgemm_nb(hipStream_t st, dim3 grid, const Seg& sg, int N, int K, const void* X, int64_t ldx,
                     int split_k, float* part, int Mtot, int64_t zW, int64_t zX, int64_t zY) {
  const int ntiles = cdiv(N, 32 * NB);
  const int tiles = cdiv(Mtot, 32 * MB) * ntiles;
  if (ntiles > 1) grid.x = (unsigned)((tiles + 7) & ~7);
  hipLaunchKernelGGL((k_wgemm<NB, XF32, MB>), grid, dim3(256), 0, st, sg, N, ntiles, K, X, ldx, split_k, part, Mtot,
                     zW, zX, zY);
}

// Y = W X over stacked segments (segment boundaries on multiples of 4; a tile may straddle them).
// Row tiles of 32*mb rows: mb = 8 halves the X traffic per W byte (N <= 64 only), mb = 2 doubles
// the workgroup count of short problems, mb = 3 gives the V2 shape's W^UQ/W^QR product one 96-row
// tile per CU (256); otherwise 128 rows. N above 128 runs as 128-column tiles in the same launch.
static int tile_mb(int mb, int N) { return (mb == 8 && N > 64) ? 4 : mb; }
template <bool XF32>
static void mfma_gemm(hipStream_t st, const Seg& sg, int N, int K, const void* X, int64_t ldx, int split_k,
                      float* part, int Z, int64_t zW, int64_t zX, int64_t zY, int mb = 4) {
  const int Mtot = sg.m0[sg.nseg];
  if (N >= cgm::MIN_N) {
    // wide product: compute-shaped tiles, with their own K split (the caller's is for the skinny shape)
    const bool big = cg_big(Mtot, K);
    const int bm = cg_bm(Mtot), ntn = cdiv(N, big ? 2 * cgm::BN : cgm::BN);
    // a K split needs the caller's partial buffer (the layouts size it for the products that pass one)
    const int sk = part != nullptr ? cg_split(Mtot, N, K, Z) : 1;
    dim3 g2((unsigned)((cdiv(Mtot, bm) * ntn + 7) & ~7), sk, Z);
    // bands of 4 row tiles: the tiles in flight on one XCD share W and X stages in its L2
    if (big) hipLaunchKernelGGL((k_cgemm<XF32, 4, 4, 3>), g2, dim3(256), 0, st, sg, N, ntn, 4, K, X, ldx, sk, part, Mtot, zW, zX, zY);
    else if (bm == 128) hipLaunchKernelGGL((k_cgemm<XF32, 2, 2, 2>), g2, dim3(256), 0, st, sg, N, ntn, 4, K, X, ldx, sk, part, Mtot, zW, zX, zY);
    else hipLaunchKernelGGL((k_cgemm<XF32, 4, 2, 2>), g2, dim3(256), 0, st, sg, N, ntn, 4, K, X, ldx, sk, part, Mtot, zW, zX, zY);
    if (sk > 1) {
      const int64_t tot = (int64_t)N * (Mtot / 4);
      hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((tot + 255) / 256), Z), dim3(256), 0, st, sg, N, Mtot,
                         sk, part, zY);
    }
    return;
  }
  mb = tile_mb(mb, N);
  dim3 grid(cdiv(Mtot, 32 * mb), split_k, Z);
  if (mb == 8) {
    if (N <= 32) wgemm_nb<1, XF32, 8>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
    else wgemm_nb<2, XF32, 8>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
  } else if (mb == 3) {
    if (N <= 32) wgemm_nb<1, XF32, 3>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
    else if (N <= 64) wgemm_nb<2, XF32, 3>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
    else wgemm_nb<4, XF32, 3>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
  } else if (mb == 2) {
    if (N <= 32) wgemm_nb<1, XF32, 2>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
    else if (N <= 64) wgemm_nb<2, XF32, 2>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
    else wgemm_nb<4, XF32, 2>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
  } else {
    if (N <= 32) wgemm_nb<1, XF32, 4>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
    else if (N <= 64) wgemm_nb<2, XF32, 4>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
    else wgemm_nb<4, XF32, 4>(st, grid, sg, N, K, X, ldx, split_k, part, Mtot, zW, zX, zY);
  }
  if (split_k > 1) {
    const int64_t tot = (int64_t)N * (Mtot / 4);
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((tot + 255) / 256), Z), dim3(256), 0, st, sg, N, Mtot,
                       split_k, part, zY);
  }
}

// A wide product (N >= cgm::MIN_N) written as bf16, without a K split (the K-split partials are
// float32): the prefill's W^UV product, whose output feeds W^O.
template <bool XF32>
static void wide_gemm_bf16_out(hipStream_t st, const Seg& sg, int N, int K, const void* X, int64_t ldx, int Z,
                               int64_t zW, int64_t zX, int64_t zY) {
  const int Mtot = sg.m0[sg.nseg];
  const int bm = cg_bm(Mtot), ntn = cdiv(N, cgm::BN);
  dim3 g2((unsigned)((cdiv(Mtot, bm) * ntn + 7) & ~7), 1, Z);
  if (bm == 128) hipLaunchKernelGGL((k_cgemm<XF32, 2, 2, 2, true>), g2, dim3(256), 0, st, sg, N, ntn, 4, K, X, ldx, 1, (float*)nullptr, Mtot, zW, zX, zY);
  else hipLaunchKernelGGL((k_cgemm<XF32, 4, 2, 2, true>), g2, dim3(256), 0, st, sg, N, ntn, 4, K, X, ldx, 1, (float*)nullptr, Mtot, zW, zX, zY);
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
    // stage 1: [c^Q | c^KV | k^R raw] = [W^DQ; W^DKV; W^KR] h
    Seg s1{};
    s1.W[0] = W_dq; s1.W[1] = W_dkv; s1.W[2] = W_kr;
    s1.Y[0] = cq; s1.ldy[0] = d.d_cq;
    s1.Y[1] = kv_new; s1.ldy[1] = rw;
    s1.Y[2] = kv_new + d.d_c; s1.ldy[2] = rw;
    s1.m0[0] = 0; s1.m0[1] = d.d_cq; s1.m0[2] = d.d_cq + d.d_c; s1.m0[3] = d.d_cq + rw; s1.nseg = 3;
    mfma_gemm<false>(st, s1, B, d.d, h, d.d, q_splits(d, B).sk1, part, 1, 0, 0, 0, 2);
    // stage 2: [q^C | q^R raw] = [W^UQ; W^QR] c^Q
    Seg s2{};
    s2.W[0] = W_uq; s2.W[1] = W_qr;
    s2.Y[0] = qc; s2.ldy[0] = nhdh;
    s2.Y[1] = q_pe; s2.ldy[1] = (int64_t)d.n_h * d.d_r;
    s2.m0[0] = 0; s2.m0[1] = nhdh; s2.m0[2] = nhdh + d.n_h * d.d_r; s2.nseg = 2;
    mfma_gemm<true>(st, s2, B, d.d_cq, cq, d.d_cq, 1, nullptr, 1, 0, 0, 0, 3);
    // stage 3: q_lat_i = (W^UK_i)^T q^C_i, batch rows in chunks of 32 NB (one-dimensional grid of
    // (head, chunk, column tile) tiles, padded to a multiple of 8). Chunks of at most 64 rows keep
    // the workgroup at 69 KB of LDS, two per CU, so that one's loads overlap the other's stores.
    const int nb_uk = B <= 32 ? 1 : 2;
    dim3 g3((unsigned)(((d.d_c / absq::TC) * d.n_h * cdiv(B, 32 * nb_uk) + 7) & ~7));
    const uint16_t* wuk = (const uint16_t*)W_uk;
    if (B <= 32) hipLaunchKernelGGL(k_absorb_uk<1>, g3, dim3(256), 0, st, d.n_h, d.d_c, B, wuk, qc, q_lat);
    else hipLaunchKernelGGL(k_absorb_uk<2>, g3, dim3(256), 0, st, d.n_h, d.d_c, B, wuk, qc, q_lat);
    return hipGetLastError();
  }
  // VALU path (any dims, float32/float16/bf16 weights); W^DQ, W^DKV and W^KR share h: one launch
  valu_stacked(wdt, st, B, d.d, h, d.d, W_dq, d.d_cq, cq, d.d_cq, W_dkv, d.d_c, kv_new, rw, W_kr, d.d_r,
               kv_new + d.d_c, rw);
  valu_pair_f32x(wdt, st, B, d.d_cq, cq, d.d_cq, W_uq, nhdh, qc, nhdh, W_qr, d.n_h * d.d_r, q_pe,
                 (int64_t)d.n_h * d.d_r);
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
  if (wdt == MLA_BF16 && mfma_dims_ok(d) && B >= cgm::MIN_N) {
    // wide batches (chunked prefill): o_i = W^UV_i o_lat_i rounded to bf16, then W^O on the bf16
    // per-head outputs (one MFMA per step instead of the float32 hi + lo pair)
    Seg s4{};
    s4.W[0] = W_uv; s4.Y[0] = o; s4.ldy[0] = nhdh;
    s4.m0[0] = 0; s4.m0[1] = d.d_h; s4.nseg = 1;
    wide_gemm_bf16_out<true>(st, s4, B, d.d_c, o_lat, (int64_t)d.n_h * d.d_c, d.n_h, (int64_t)d.d_h * d.d_c, d.d_c,
                             d.d_h);
    Seg s5{};
    s5.W[0] = W_o; s5.Y[0] = u; s5.ldy[0] = d.d;
    s5.m0[0] = 0; s5.m0[1] = d.d; s5.nseg = 1;
    mfma_gemm<false>(st, s5, B, nhdh, o, nhdh, o_splits(d, B).sk5, part, 1, 0, 0, 0, 4);
    return hipGetLastError();
  }
  if (wdt == MLA_BF16 && mfma_dims_ok(d)) {
    // o_i = W^UV_i o_lat_i, batched over heads (z): rows of W^UV_i are outputs
    Seg s4{};
    s4.W[0] = W_uv; s4.Y[0] = o; s4.ldy[0] = nhdh;
    s4.m0[0] = 0; s4.m0[1] = d.d_h; s4.nseg = 1;
    const OSplits sp = o_splits(d, B);
    mfma_gemm<true>(st, s4, B, d.d_c, o_lat, (int64_t)d.n_h * d.d_c, sp.sk4, part, d.n_h, (int64_t)d.d_h * d.d_c,
                    d.d_c, d.d_h, 2);
    // u = W^O [o_1; ...; o_nh]
    Seg s5{};
    s5.W[0] = W_o; s5.Y[0] = u; s5.ldy[0] = d.d;
    s5.m0[0] = 0; s5.m0[1] = d.d; s5.nseg = 1;
    mfma_gemm<true>(st, s5, B, nhdh, o, nhdh, sp.sk5, part, 1, 0, 0, 0, o_wide(B) ? 8 : 4);
    return hipGetLastError();
  }
  valu_any(wdt, false, false, st, d.d_h, B, d.d_c, W_uv, d.d_c, (int64_t)d.d_h * d.d_c, o_lat,
           (int64_t)d.n_h * d.d_c, d.d_c, o, nhdh, d.d_h, d.n_h);
  // W^O: the layout's partial area holds sk5 * B * d floats
  const int sk5 = o_splits(d, B).sk5;
  valu_splitk(wdt, st, d.d, B, nhdh, W_o, o, u, d.d, sk5, sk5 > 1 ? part : nullptr);
  return hipGetLastError();
}

// ================================================================================================
// Naive-form prefill pieces (k_naive.hip holds the attention): the query pathway without the W^UK
// absorption, the keys and values of every context token, and W^O on the per-head outputs.

// [c^Q | c^KV | k^R raw] = [W^DQ; W^DKV; W^KR] h, then [q^C | q^R raw] = [W^UQ; W^QR] c^Q, with q^C
// written to the caller's buffer (the absorbed form goes on to W^UK instead).
hipError_t launch_absorb_q_naive(const mla_dims& d, int B, const void* h, const void* W_dq, const void* W_uq,
                                 const void* W_qr, const void* W_dkv, const void* W_kr, void* ws, float* q_c,
                                 float* q_pe, float* kv_new, hipStream_t st) {
  AbsorbQLayout L = absorb_q_layout(d, B);
  float* cq = (float*)((char*)ws + L.off_cq);
  float* part = (float*)((char*)ws + L.off_part);
  const int rw = d.d_c + d.d_r;
  const int nhdh = d.n_h * d.d_h;
  Seg s1{};
  s1.W[0] = W_dq; s1.W[1] = W_dkv; s1.W[2] = W_kr;
  s1.Y[0] = cq; s1.ldy[0] = d.d_cq;
  s1.Y[1] = kv_new; s1.ldy[1] = rw;
  s1.Y[2] = kv_new + d.d_c; s1.ldy[2] = rw;
  s1.m0[0] = 0; s1.m0[1] = d.d_cq; s1.m0[2] = d.d_cq + d.d_c; s1.m0[3] = d.d_cq + rw; s1.nseg = 3;
  mfma_gemm<false>(st, s1, B, d.d, h, d.d, q_splits(d, B).sk1, part, 1, 0, 0, 0, 2);
  Seg s2{};
  s2.W[0] = W_uq; s2.W[1] = W_qr;
  s2.Y[0] = q_c; s2.ldy[0] = nhdh;
  s2.Y[1] = q_pe; s2.ldy[1] = (int64_t)d.n_h * d.d_r;
  s2.m0[0] = 0; s2.m0[1] = nhdh; s2.m0[2] = nhdh + d.n_h * d.d_r; s2.nseg = 2;
  mfma_gemm<true>(st, s2, B, d.d_cq, cq, d.d_cq, 1, nullptr, 1, 0, 0, 0, 3);
  return hipGetLastError();
}

// K^C[r][i d_h + e] = sum_c W^UK[i d_h + e][c] ctx[r][c] and V[r][...] likewise with W^UV, for the
// R gathered rows (576 elements each, latent first): one product of [W^UK; W^UV] with bf16 output.
hipError_t launch_materialize_kv(const mla_dims& d, int R, const void* ctx, const void* W_uk, const void* W_uv,
                                 void* kc, void* vv, hipStream_t st) {
  const int nhdh = d.n_h * d.d_h;
  Seg sg{};
  sg.W[0] = W_uk; sg.W[1] = W_uv;
  sg.Y[0] = (float*)kc; sg.ldy[0] = nhdh;
  sg.Y[1] = (float*)vv; sg.ldy[1] = nhdh;
  sg.m0[0] = 0; sg.m0[1] = nhdh; sg.m0[2] = 2 * nhdh; sg.nseg = 2;
  // 256 x 128 tiles, a 2-stage ring, three workgroups per CU (K = d_c is only 16 stages of 32: more
  // workgroups in flight hide more of each tile's load latency and epilogue than a deeper ring);
  // bands of 8 row tiles, so that the ~96 tiles in flight per XCD share [W^UK; W^UV] rows and
  // latent rows in its L2 instead of streaming every row tile's worth of latents from memory again
  const int Mtot = 2 * nhdh, ntn = cdiv(R, cgm::BN);
  dim3 g2((unsigned)((cdiv(Mtot, 256) * ntn + 7) & ~7), 1, 1);
  hipLaunchKernelGGL((k_cgemm<false, 4, 2, 2, true>), g2, dim3(256), 0, st, sg, R, ntn, 8, d.d_c, ctx,
                     (int64_t)(d.d_c + d.d_r), 1, (float*)nullptr, Mtot, (int64_t)0, (int64_t)0, (int64_t)0);
  return hipGetLastError();
}

// dims the naive-form path has kernels for: the MFMA GEMM shapes and the attention kernel's d_h, d_c, d_r
bool naive_supported(const mla_dims& d) {
  return mfma_dims_ok(d) && d.d_h == 128 && d.d_c == 512 && d.d_r == 64;
}

// u = W^O o for per-head outputs o [N, n_h d_h] (float32, or bf16); the workspace holds only K-split partials
AbsorbOutLayout output_proj_layout(const mla_dims& d, int N) {
  AbsorbOutLayout L;
  const int sk5 = o_splits(d, N).sk5;
  L.off_o = 0;
  L.off_part = 0;
  L.part_floats = sk5 > 1 ? (size_t)sk5 * N * d.d : 0;
  if (N >= cgm::MIN_N) {
    const int c5 = cg_split(d.d, N, d.n_h * d.d_h, 1);
    if (c5 > 1 && (size_t)c5 * N * d.d > L.part_floats) L.part_floats = (size_t)c5 * N * d.d;
  }
  L.bytes = al256h(L.part_floats * 4);
  return L;
}
hipError_t launch_output_proj(const mla_dims& d, int N, const void* o, bool o_bf16, const void* W_o, void* ws,
                              float* u, hipStream_t st) {
  float* part = (float*)ws;
  const int nhdh = d.n_h * d.d_h;
  Seg s5{};
  s5.W[0] = W_o; s5.Y[0] = u; s5.ldy[0] = d.d;
  s5.m0[0] = 0; s5.m0[1] = d.d; s5.nseg = 1;
  // bf16 o: 128-row tiles (a 6-stage ring at this stage size) and the K split that fills the chip
  // with them (at most o_splits' split, which sizes the partial area)
  if (o_bf16)
    mfma_gemm<false>(st, s5, N, nhdh, o, nhdh, split_for(cdiv(d.d, gm::MT) * col_tiles(N), nhdh / gm::KC, 1), part,
                     1, 0, 0, 0, 4);
  else mfma_gemm<true>(st, s5, N, nhdh, o, nhdh, o_splits(d, N).sk5, part, 1, 0, 0, 0, o_wide(N) ? 8 : 4);
  return hipGetLastError();
}

// ================================================================================================
// Pre-combined absorbed matrices ("DeepSeek-V2 from Scratch" section 5.1: W~^Q_i = (W^UK_i)^T W^UQ_i;
// section 5.2: W~^O_i = W^O_i W^UV_i), built once from the factors:
//   C_z(r, c) = sum_{e < K} A_z(r, e) B_z(e, c),  A_z(r, e) = A[z*azs + r*ars + e*aks],
//   B_z(e, c) = B[z*bzs + e*bks + c],  C_z(r, c) = C[z*czs + r*crs + c],
// float32 accumulation, one rounding to the weight type on the store. A plain LDS-tiled VALU
// kernel: 64 x 64 outputs per workgroup (4 x 4 per thread), K in chunks of 16. It runs once per
// set of weights, outside the decode step.
template <int DT>
__global__ __launch_bounds__(256) void k_precombine(int R, int Cc, int K, const void* __restrict__ Av, int64_t azs,
                                                    int64_t ars, int64_t aks, const void* __restrict__ Bv,
                                                    int64_t bzs, int64_t bks, void* __restrict__ Cv, int64_t czs,
                                                    int64_t crs) {
  using E = Elem<DT>;
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tid = threadIdx.x, z = blockIdx.z;
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const typename E::T* A = (const typename E::T*)Av + (int64_t)z * azs;
  const typename E::T* Bp = (const typename E::T*)Bv + (int64_t)z * bzs;
  const int tr = tid >> 4, tc = tid & 15;  // rows tr + 16 i, columns tc + 16 j
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = tid; e < 16 * 64; e += 256) {
      const int kk = e >> 6, rr = e & 63;
      const int r = r0 + rr, k = k0 + kk;
      As[kk][rr] = (r < R && k < K) ? E::ld(A, (int64_t)r * ars + (int64_t)k * aks) : 0.f;
      const int c = c0 + rr;
      Bs[kk][rr] = (c < Cc && k < K) ? E::ld(Bp, (int64_t)k * bks + c) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][tr + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[kk][tc + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * bb[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + tr + 16 * i, c = c0 + tc + 16 * j;
      if (r >= R || c >= Cc) continue;
      const int64_t o = (int64_t)z * czs + (int64_t)r * crs + c;
      if constexpr (DT == MLA_F32) ((float*)Cv)[o] = acc[i][j];
      else if constexpr (DT == MLA_F16) ((uint16_t*)Cv)[o] = f32_to_f16_bits(acc[i][j]);
      else ((uint16_t*)Cv)[o] = f32_to_bf16_bits(acc[i][j]);
    }
}

template <int DT>
static void precombine_dt(const mla_dims& d, const void* W_uq, const void* W_uk, const void* W_uv, const void* W_o,
                          void* Wq_pre, void* Wo_pre, hipStream_t st) {
  if (Wq_pre) {  // rows i*d_c + c, columns k: sum_e W_uk[i*d_h + e][c] W_uq[i*d_h + e][k]
    dim3 g(cdiv(d.d_c, 64), cdiv(d.d_cq, 64), d.n_h);
    hipLaunchKernelGGL(k_precombine<DT>, g, dim3(256), 0, st, d.d_c, d.d_cq, d.d_h, W_uk, (int64_t)d.d_h * d.d_c,
                       (int64_t)1, (int64_t)d.d_c, W_uq, (int64_t)d.d_h * d.d_cq, (int64_t)d.d_cq, Wq_pre,
                       (int64_t)d.d_c * d.d_cq, (int64_t)d.d_cq);
  }
  if (Wo_pre) {  // rows m, columns i*d_c + c: sum_e W_o[m][i*d_h + e] W_uv[i*d_h + e][c]
    dim3 g(cdiv(d.d, 64), cdiv(d.d_c, 64), d.n_h);
    hipLaunchKernelGGL(k_precombine<DT>, g, dim3(256), 0, st, d.d, d.d_c, d.d_h, W_o, (int64_t)d.d_h,
                       (int64_t)d.n_h * d.d_h, (int64_t)1, W_uv, (int64_t)d.d_h * d.d_c, (int64_t)d.d_c, Wo_pre,
                       (int64_t)d.d_c, (int64_t)d.n_h * d.d_c);
  }
}

hipError_t launch_precombine(const mla_dims& d, int wdt, const void* W_uq, const void* W_uk, const void* W_uv,
                             const void* W_o, void* Wq_pre, void* Wo_pre, hipStream_t st) {
  if (wdt == MLA_F32) precombine_dt<MLA_F32>(d, W_uq, W_uk, W_uv, W_o, Wq_pre, Wo_pre, st);
  else if (wdt == MLA_F16) precombine_dt<MLA_F16>(d, W_uq, W_uk, W_uv, W_o, Wq_pre, Wo_pre, st);
  else precombine_dt<MLA_BF16>(d, W_uq, W_uk, W_uv, W_o, Wq_pre, Wo_pre, st);
  return hipGetLastError();
}

// MFMA shapes of the pre-combined products: stage 1 as in the two-step form, then
// [W~^Q; W^QR] c^Q (segment boundary n_h*d_c) and W~^O [o_lat] (K = n_h*d_c).
static bool mfma_pre_dims_ok(const mla_dims& d) {
  return d.d % 256 == 0 && d.d_cq % 256 == 0 && d.d_c % 128 == 0 && d.d_r % 64 == 0 && (d.n_h * d.d_c) % 256 == 0 &&
         (d.n_h * d.d_r) % 64 == 0;
}

hipError_t launch_absorb_q_pre(const mla_dims& d, int B, int wdt, const void* h, const void* W_dq,
                               const void* Wq_pre, const void* W_qr, const void* W_dkv, const void* W_kr, void* ws,
                               float* q_lat, float* q_pe, float* kv_new, hipStream_t st) {
  AbsorbQLayout L = absorb_q_layout(d, B);
  float* cq = (float*)((char*)ws + L.off_cq);
  float* part = (float*)((char*)ws + L.off_part);
  const int rw = d.d_c + d.d_r;
  const int nhdc = d.n_h * d.d_c;
  if (wdt == MLA_BF16 && mfma_pre_dims_ok(d)) {
    // stage 1: [c^Q | c^KV | k^R raw] = [W^DQ; W^DKV; W^KR] h (as in the two-step form)
    Seg s1{};
    s1.W[0] = W_dq; s1.W[1] = W_dkv; s1.W[2] = W_kr;
    s1.Y[0] = cq; s1.ldy[0] = d.d_cq;
    s1.Y[1] = kv_new; s1.ldy[1] = rw;
    s1.Y[2] = kv_new + d.d_c; s1.ldy[2] = rw;
    s1.m0[0] = 0; s1.m0[1] = d.d_cq; s1.m0[2] = d.d_cq + d.d_c; s1.m0[3] = d.d_cq + rw; s1.nseg = 3;
    mfma_gemm<false>(st, s1, B, d.d, h, d.d, q_splits(d, B).sk1, part, 1, 0, 0, 0, 2);
    // stage 2: [q~ | q^R raw] = [W~^Q; W^QR] c^Q, one product
    Seg s2{};
    s2.W[0] = Wq_pre; s2.W[1] = W_qr;
    s2.Y[0] = q_lat; s2.ldy[0] = nhdc;
    s2.Y[1] = q_pe; s2.ldy[1] = (int64_t)d.n_h * d.d_r;
    s2.m0[0] = 0; s2.m0[1] = nhdc; s2.m0[2] = nhdc + d.n_h * d.d_r; s2.nseg = 2;
    mfma_gemm<true>(st, s2, B, d.d_cq, cq, d.d_cq, 1, nullptr, 1, 0, 0, 0, 3);
    return hipGetLastError();
  }
  valu_stacked(wdt, st, B, d.d, h, d.d, W_dq, d.d_cq, cq, d.d_cq, W_dkv, d.d_c, kv_new, rw, W_kr, d.d_r,
               kv_new + d.d_c, rw);
  valu_pair_f32x(wdt, st, B, d.d_cq, cq, d.d_cq, Wq_pre, nhdc, q_lat, nhdc, W_qr, d.n_h * d.d_r, q_pe,
                 (int64_t)d.n_h * d.d_r);
  return hipGetLastError();
}

hipError_t launch_absorb_out_pre(const mla_dims& d, int B, int wdt, const float* o_lat, const void* Wo_pre, void* ws,
                                 float* u, hipStream_t st) {
  const int nhdc = d.n_h * d.d_c;
  if (wdt == MLA_BF16 && mfma_pre_dims_ok(d)) {
    Seg s{};
    s.W[0] = Wo_pre; s.Y[0] = u; s.ldy[0] = d.d;
    s.m0[0] = 0; s.m0[1] = d.d; s.nseg = 1;
    mfma_gemm<true>(st, s, B, nhdc, o_lat, nhdc, o_pre_splits(d, B).sk5, (float*)ws, 1, 0, 0, 0,
                    o_wide(B) ? 8 : 4);
    return hipGetLastError();
  }
  // the layout holds sk * B * d partial floats
  const int sk = o_pre_splits(d, B).sk5;
  valu_splitk(wdt, st, d.d, B, nhdc, Wo_pre, o_lat, u, d.d, sk, sk > 1 ? (float*)ws : nullptr);
  return hipGetLastError();
}

}  // namespace mla
