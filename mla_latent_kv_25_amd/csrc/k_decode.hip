// Latent-space decode attention and the split-sequence combine.
//
// "DeepSeek-V2 from Scratch" section 4.4: the score of head i against cached token j is
// q^C_i.k^C_{j,i} + q^R_i.k^R_j over sqrt(d_h + d_h^R); section 5.1: the content part equals
// q~_i.c_j with q~_i = (W^UK_i)^T q^C_i; section 5.3 steps 2-3: dot the absorbed query with every
// cached latent and sum the latents under the softmax weights. Each cached row is
// [c_j (d_c) | k^R_j (d_r)], so with q = [q~_i | q^R_i] the whole score is one dot product over
// the row, and the weighted sum runs over the first d_c entries of the same rows.
//
// Work split: the batch's tokens (concatenated sequence by sequence) are cut into G equal ranges;
// range p is one workgroup. A range may cover the end of one sequence and the start of the next;
// each (range, sequence) piece writes a normalised partial o and its log-sum-exp into slot p + b
// of the workspace (slots are unique: ranges and sequences both advance with the token order).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(const mla_dims& d, int B, int G) {
  DecodeLayout L;
  L.n_pieces = (int64_t)G + B - 1;
  L.off_cu = 0;
  L.off_fmt = al256((size_t)(B + 1) * 8);
  L.off_lse = L.off_fmt + 256;
  L.off_sc = al256(L.off_lse + (size_t)L.n_pieces * d.n_h * 4);
  L.off_o = al256(L.off_sc + (size_t)L.n_pieces * d.n_h * 4);
  L.bytes = L.off_o + (size_t)L.n_pieces * d.n_h * d.d_c * 4;  // sized for float32 partials
  // MFMA shape: the query in the MFMA kernels' operand form (1152 bytes per head: bf16, or two
  // e4m3 parts per element) and the fp8 form's per-head power-of-two factor
  L.off_q8 = L.off_fh = 0;
  if (d.n_h == 128 && d.d_c == 512 && d.d_r == 64) {
    L.off_q8 = al256(L.bytes);
    L.off_fh = al256(L.off_q8 + (size_t)B * d.n_h * 1152);
    L.bytes = L.off_fh + (size_t)B * d.n_h * 4;
  }
  return L;
}

__device__ __forceinline__ int64_t row_index(const CacheArgs& c, int b, int64_t j) {
  if (c.page_size == 0) return (int64_t)b * c.t_cap + j;
  int32_t page = c.block_table[(int64_t)b * c.max_pages + j / c.page_size];
  return (int64_t)page * c.page_size + (j % c.page_size);
}

// ------------------------------------------------------------------------------------------------
// Range planning on the device, inside the decode kernels (no separate launch): every wave of a
// workgroup locates its range from seq_lens with wave-wide scans; workgroup 0 also writes the
// prefix sums cu[b] = sum_{b' < b} seq_lens[b'] and the partial-output format word that
// mla_combine reads.
__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t x = __shfl_up(v, o, 64);
    if (lane >= o) v += x;
  }
  return v;
}
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Range p: token interval [start, end) of the concatenated batch, the first sequence b whose
// interval [s0, s1) reaches past `start`. Uniform across the wave (kept in scalar registers).
struct RangeStart {
  int64_t start, end, s0, s1;
  int b;
};
__device__ __forceinline__ RangeStart locate_range(const int32_t* __restrict__ seq_lens, int B, int G, int p,
                                                   int lane) {
  // the first 64 lengths are loaded once and serve both the total and the scan below
  const int64_t v_first = lane < B ? (int64_t)seq_lens[lane] : 0;
  int64_t acc = v_first;
  for (int i = lane + 64; i < B; i += 64) acc += seq_lens[i];
  const int64_t total = wave_sum_i64(acc);
  RangeStart r;
  r.start = range_start(p, total, G);
  r.end = range_start(p + 1, total, G);
  r.b = 0;
  r.s0 = r.s1 = 0;
  int64_t base = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int i = c0 + lane;
    const int64_t v = c0 == 0 ? v_first : (i < B ? (int64_t)seq_lens[i] : 0);
    const int64_t inc = wave_incl_scan_i64(v, lane);
    const uint64_t hit = __ballot(base + inc > r.start);
    if (hit) {
      const int f = __builtin_ctzll(hit);
      r.b = c0 + f;
      r.s1 = base + __shfl(inc, f, 64);
      r.s0 = r.s1 - __shfl(v, f, 64);
      break;
    }
    base += __shfl(inc, 63, 64);
  }
  r.start = uniform_i64(r.start);
  r.end = uniform_i64(r.end);
  r.s0 = uniform_i64(r.s0);
  r.s1 = uniform_i64(r.s1);
  r.b = __builtin_amdgcn_readfirstlane(r.b);
  return r;
}

// cu[0..B] and the format word, by one wave of workgroup 0.
__device__ __forceinline__ void write_prefix(const int32_t* __restrict__ seq_lens, int B, int fmt,
                                             int64_t* __restrict__ cu, int32_t* __restrict__ fmt_out, int lane) {
  int64_t base = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int i = c0 + lane;
    const int64_t v = i < B ? (int64_t)seq_lens[i] : 0;
    const int64_t inc = wave_incl_scan_i64(v, lane);
    if (i < B) cu[i + 1] = base + inc;
    base += __shfl(inc, 63, 64);
  }
  if (lane == 0) {
    cu[0] = 0;
    *fmt_out = fmt;
  }
}

// Range assignment: workgroups are dispatched round-robin over the 8 XCDs; consecutive ranges
// (usually the same sequence, sharing its query in L2) are mapped onto the same XCD.
__device__ __forceinline__ int range_for_block(int bid, int G) {
  if (G % 8 == 0) return (bid & 7) * (G >> 3) + (bid >> 3);
  return bid;
}


// ================================================================================================
// MFMA kernels for the DeepSeek-V2 shape: n_h = 128, d_c = 512, d_r = 64 (row = 576). One
// workgroup = 4 waves; all heads share each latent tile, staged once in LDS. Per 32-token tile:
//   S^T[32 tok x 32 heads] = K[32 x 576] Q^T for wave w's heads [32w, 32w + 32)
//       (K rows read from LDS; Q in registers, scale folded in)
//   softmax in float32 (base 2) against a fixed per-head reference
//   O^T[128 columns of wave w x 128 heads] += V^T P^T (32 MFMA 32x32x16 bf16, V^T via
//       transposing LDS reads, P of all heads through LDS)
// Softmax reference: per head, the maximum of the segment's first tile. Later probabilities are
// exp2(s - m_ref), so the accumulators are never rescaled; a score more than HEAD (64) above
// m_ref makes the workgroup run the segment once more with a reference at (or just above) the
// segment's true maximum (exact; at most one re-run).
// This section holds the shared pieces; the bf16 kernel (rows as bf16 in LDS) and the fp8 kernel
// (rows as e4m3 codes in LDS) follow.
namespace v2 {
constexpr int NH = 128, DC = 512, DR = 64, RW = 576;
constexpr int TT = 32;                     // tokens per tile
constexpr int ROWB = RW * 2;               // bytes of one bf16 row in LDS
constexpr int CHUNKS = RW / 8;             // 16-byte chunks per row (72)
constexpr int TILE_CHUNKS = TT * CHUNKS;   // 2304
constexpr int TILEB = TT * ROWB;           // 36864
constexpr int LOADS = TILE_CHUNKS / 256;   // chunks staged per thread per tile (9)
constexpr int KSTEPS = RW / 16;            // 36
constexpr int CB = DC / 32;                // 16 output column blocks
}  // namespace v2

// LDS position of chunk c of tile row t: XOR of the low 3 chunk-index bits with a per-row key
// (stays inside the aligned group of 8 chunks, so rows of 72 chunks never overflow). The key is
// (t>>1) with its bits permuted so that (a) 16 consecutive rows read at one chunk index hit 16
// distinct 16-byte bank groups (score reads) and (b) the 8 rows x 4 chunks of one transposing
// V read spread evenly over the 64 banks (2 bank cycles per 512-byte read, the minimum).
__device__ __forceinline__ int swz_key(int t) {
  const int g = t >> 1;
  return ((g & 1) << 2) | (((g >> 2) & 1) << 1) | ((g >> 1) & 1);
}
__device__ __forceinline__ int swz(int t, int c) { return c ^ swz_key(t); }

// 16-byte global -> LDS copy per lane (LDS destination: wave-uniform `lds_addr` + 16 * lane).
// Written as asm so the compiler does not add its conservative "wait for every LDS DMA" before
// each LDS read: the kernel tracks these loads itself (vm_wait_barrier). The instruction has no
// VGPR result; only M0 (not used by any other instruction of these kernels) is changed. Cached
// rows are read once: the copies are non-temporal (nt), so the stream does not evict what the
// workgroups share through L2 (the query).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(src), "s"(lds_addr) : "memory", "m0");
}

// Same copy with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding, then barrier.
// The memory clobber keeps the compiler from moving LDS reads above it.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Cached-row locator for one sequence: contiguous [B, t_cap, row] or pages of 2^ps_shift rows.
// Within one 32-token tile at most two pages occur (page size >= 32); their ids are read once
// per tile with uniform (scalar) loads.
template <bool PAGED>
struct Rows {
  int64_t base_row;       // contiguous: b * t_cap
  const int32_t* bt;      // paged: block table row of sequence b
  int ps_shift;
  int32_t pg0, pg1;
  int64_t tile_page0;
  __device__ __forceinline__ void init(const CacheArgs& c, int b) {
    if constexpr (PAGED) {
      bt = c.block_table + (int64_t)__builtin_amdgcn_readfirstlane(b) * c.max_pages;
      ps_shift = __builtin_ctz((unsigned)c.page_size);
    } else {
      base_row = (int64_t)b * c.t_cap;
    }
  }
  __device__ __forceinline__ void tile(int64_t t0, int64_t t_last) {
    if constexpr (PAGED) {
      // uniform page indices -> scalar loads (counted by lgkmcnt, so they never wait on the
      // in-flight tile copies that vmcnt tracks)
      tile_page0 = t0 >> ps_shift;
      const int i0 = __builtin_amdgcn_readfirstlane((int)tile_page0);
      const int i1 = __builtin_amdgcn_readfirstlane((int)(t_last >> ps_shift));
      // the block table is read-only for the whole kernel: constant address space -> s_load
      const __attribute__((address_space(4))) int32_t* btc = (const __attribute__((address_space(4))) int32_t*)bt;
      pg0 = btc[i0];
      pg1 = btc[i1];
    }
  }
  // Byte address of row tt0 + tr (tr < 32) of the tile that starts at tt0 (row width rb bytes).
  __device__ __forceinline__ const uint8_t* tile_row(const uint8_t* base, int64_t tt0, int tr, int rb) const {
    if constexpr (PAGED) {
      const int64_t tok = tt0 + tr;
      return base + row(tok) * rb;
    } else {
      return base + (base_row + tt0) * rb + (uint32_t)(tr * rb);
    }
  }
  __device__ __forceinline__ int64_t row(int64_t tok) const {
    if constexpr (PAGED) {
      const int32_t pg = (tok >> ps_shift) == tile_page0 ? pg0 : pg1;
      return ((int64_t)pg << ps_shift) + (tok & ((1 << ps_shift) - 1));
    } else {
      return base_row + tok;
    }
  }
};

// Scores of one tile: S^T[32 tok x 32 heads] = sum over 36 k-steps of K-tile rows x Q^T.
// The chain is written with explicit MFMA instructions so that S lives in VGPRs: the 256
// accumulators of O^T take all AGPRs, and letting the compiler place S in AGPRs too evicts the
// query fragments. Volatile asm statements keep their program order relative to memory
// operations, so the LDS reads are issued LA k-steps ahead of the MFMA that consumes them.
// MFMA -> MFMA accumulation into the same registers needs no wait states; the 24 wait states
// after the last step cover the MFMA-result -> VALU-read dependency and sit in the same asm
// statement so no reader can be scheduled between them.
__device__ __forceinline__ f32x16 tile_scores(const uint8_t* tile, const uint32_t (&kq)[4],
                                              const bf16x8 (&qf)[v2::KSTEPS]) {
  constexpr int KS = v2::KSTEPS, LA = 4;
  bf16x8 a[KS];
#pragma unroll
  for (int j = 0; j < LA; ++j) a[j] = *(const bf16x8*)(tile + kq[j & 3] + 128 * (j >> 2));
  f32x16 s;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(a[0]), "v"(qf[0]));
  a[LA] = *(const bf16x8*)(tile + kq[LA & 3] + 128 * (LA >> 2));
#pragma unroll
  for (int ks = 1; ks < KS - 1; ++ks) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a[ks]), "v"(qf[ks]));
    if (ks + LA < KS) a[ks + LA] = *(const bf16x8*)(tile + kq[(ks + LA) & 3] + 128 * ((ks + LA) >> 2));
  }
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(s) : "v"(a[KS - 1]), "v"(qf[KS - 1]));
  return s;
}

// ================================================================================================
// The query of every (sequence, head) in the MFMA kernels' operand form, once per call instead
// of once per workgroup. Layout: [B][wave block w = head / 32][36 loads][64 lanes][16 bytes], so
// that load j of lane (g = lane / 32, head 32w + lane % 32) is one coalesced 1 KB wave load.
//   bf16 kernel: load ks holds bf16(q * qscale) for dims 16ks + 8g .. +7 (the B fragment of k-step ks).
//   fp8 kernel: x = q * qscale * 2^e_h with the head's largest |x| in [128, 256), split into e4m3
//     parts x = hi + lo (hi = RNE(x), lo = RNE(x - hi)); loads 4kb + p (p = 0, 1) hold hi and
//     4kb + 2 + p lo of dims 64kb + 32g + 16p .. +15 (the B fragments of k block kb); 2^-e_h goes
//     to fh.
// One workgroup per (sequence, 8 heads): 128-byte runs of its rows of the layout, 16 bytes per
// thread and store (16 workgroups per sequence, so that small batches still spread over the chip).
template <bool FP8>
__global__ __launch_bounds__(256) void k_qprep(const float* __restrict__ q_lat, const float* __restrict__ q_pe,
                                               float qscale, uint8_t* __restrict__ qop, float* __restrict__ fh) {
  using namespace v2;
  constexpr int HB = 8;                              // heads per workgroup
  const int tid = threadIdx.x;
  const int64_t head0 = (int64_t)blockIdx.x * HB;    // first (sequence, head) row
  const int bw = (int)(head0 >> 5), l0 = (int)(head0 & 31);
  uint8_t* const blk = qop + (int64_t)bw * 36 * 1024;
  // 8 consecutive elements d0.. of head row hr (d0 % 8 == 0, never straddling q_lat / q_pe)
  auto load8 = [&](int64_t hr, int d0, f32x4& a, f32x4& c) __attribute__((always_inline)) {
    const float* src = d0 < DC ? q_lat + hr * DC + d0 : q_pe + hr * DR + (d0 - DC);
    a = *(const f32x4*)src;
    c = *(const f32x4*)(src + 4);
  };
  if constexpr (!FP8) {
    for (int u = tid; u < 36 * 2 * HB; u += 256) {    // unit = (k-step, g, head)
      const int ks = u / (2 * HB), g = (u / HB) & 1, l = u % HB;
      f32x4 a, c;
      load8(head0 + l, 16 * ks + 8 * g, a, c);
      a *= qscale;
      c *= qscale;
      *(u32x4*)(blk + ((ks * 64 + g * 32 + l0 + l) << 4)) =
          u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
    }
  } else {
    __shared__ float qsh[HB];
    {
      // head l = tid / 32, 32 threads per head over its 72 groups of 8 elements
      const int l = tid >> 5, part = tid & 31;
      float mx = 0.f;
      for (int q = part; q < RW / 8; q += 32) {
        f32x4 a, c;
        load8(head0 + l, 8 * q, a, c);
        mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(fabsf(a[0]), fabsf(a[1])), fmaxf(fabsf(a[2]), fabsf(a[3]))),
                             fmaxf(fmaxf(fabsf(c[0]), fabsf(c[1])), fmaxf(fabsf(c[2]), fabsf(c[3])))));
      }
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      mx *= qscale;
      int e = 0;
      if (mx > 0.f) (void)frexpf(mx, &e);  // mx = m 2^e, m in [0.5, 1)
      if (part == 0) {
        qsh[l] = ldexpf(qscale, 8 - e);
        fh[head0 + l] = ldexpf(1.f, e - 8);
      }
    }
    __syncthreads();
    // unit pair (kb, p, g, head): 16 elements, whose hi bytes go to load 4kb + p and lo to 4kb + 2 + p
    for (int u = tid; u < 18 * 2 * HB; u += 256) {
      const int kp = u / (2 * HB), g = (u / HB) & 1, l = u % HB, kb = kp >> 1, p = kp & 1;
      const float qs = qsh[l];
      const int d0 = 64 * kb + 32 * g + 16 * p;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 a, c;
        load8(head0 + l, d0 + 8 * h, a, c);
        const f32x4 xs[2] = {a * qs, c * qs};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 x = xs[q];
          int hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
          hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hw, true);
          const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
          const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
          int lw = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - h01[0], x[1] - h01[1], 0, false);
          lw = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - h23[0], x[3] - h23[1], lw, true);
          hi[2 * h + q] = (uint32_t)hw;
          lo[2 * h + q] = (uint32_t)lw;
        }
      }
      const int ln = g * 32 + l0 + l;
      *(u32x4*)(blk + (((4 * kb + p) * 64 + ln) << 4)) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *(u32x4*)(blk + (((4 * kb + 2 + p) * 64 + ln) << 4)) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  }
}

// ================================================================================================
// MFMA kernel for bf16 caches at the DeepSeek-V2 shape: 36 MFMA 32x32x16 per tile for the
// scores (K rows via ds_read_b128), V^T via ds_read_b64_tr_b16. Tiles go straight from HBM into
// LDS (global->LDS copies), and the memory traffic is spread over the math:
// per iteration `it` (tiles it+1.. it+3 in flight),
//   scores of tile it (36 MFMAs) with the nine copies of tile it+3 slotted between them, so the
//   four waves do not all queue 36 KB of copies at the same instant,
//   softmax of tile it; P published to LDS; barrier,
//   O^T[128 columns of wave w x 128 heads] += V^T P^T (32 MFMAs, P of all heads from LDS).
// The softmax keeps per-lane (half-head) maxima and sums: no cross-lane traffic per tile; the
// two halves of a head are joined once per segment.
namespace v3 {
constexpr int NBUF = 4;
constexpr int EARLY = 1;  // tiles whose copies are issued before the query loads
}

// Scores of one tile (as tile_scores) with between(ks) run after MFMA ks; the calls sit between
// the volatile MFMA statements in program order (used to issue tile copies under the math).
template <typename F>
__device__ __forceinline__ f32x16 tile_scores_copy(const uint8_t* tile, const uint32_t (&kq)[4],
                                                   const bf16x8 (&qf)[v2::KSTEPS], F&& between) {
  constexpr int KS = v2::KSTEPS, LA = 4;
  bf16x8 a[KS];
#pragma unroll
  for (int j = 0; j < LA; ++j) a[j] = *(const bf16x8*)(tile + kq[j & 3] + 128 * (j >> 2));
  f32x16 s;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(a[0]), "v"(qf[0]));
  between(0);
  a[LA] = *(const bf16x8*)(tile + kq[LA & 3] + 128 * (LA >> 2));
#pragma unroll
  for (int ks = 1; ks < KS - 1; ++ks) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a[ks]), "v"(qf[ks]));
    between(ks);
    if (ks + LA < KS) a[ks + LA] = *(const bf16x8*)(tile + kq[(ks + LA) & 3] + 128 * ((ks + LA) >> 2));
  }
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(s) : "v"(a[KS - 1]), "v"(qf[KS - 1]));
  return s;
}

template <bool PAGED>
__global__ __launch_bounds__(256, 1) void k_decode_v3(const uint8_t* __restrict__ qop, CacheArgs cache,
                                                      const int32_t* __restrict__ seq_lens, int B, int G,
                                                      int64_t* __restrict__ cu_out, int32_t* __restrict__ fmt_out,
                                                      float* __restrict__ lse_part,
                                                      float* __restrict__ sc_part,
                                                      uint16_t* __restrict__ o_part) {
  using namespace v2;
  constexpr int NBUF = v3::NBUF;
  constexpr float HEAD = 64.f;
  constexpr int FILL_STEPS = 20;  // softmax steps
  constexpr int PB = NH * TT * 2;  // bytes of P of one tile, [head][token]
  __shared__ __attribute__((aligned(16))) uint8_t lds[NBUF * TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_p[2 * PB];  // P of two consecutive tiles
  // scratch of the pass / segment end, on the tile ring (idle there: every copy has landed and
  // every wave is past its last tile read at the barriers that precede each use)
  int* const redo_flag = (int*)lds;
  float* const lds_l = (float*)(lds + 16);
  float (*const lds_m)[NH] = (float (*)[NH])(lds + 16 + NH * 4);
  // staging of the float16 partial rows (per wave NH rows of 256 bytes + 16 bytes of padding,
  // which spreads the row-wise writes over all banks), also on the idle tile ring
  constexpr int OTR = 272;
  static_assert(4096 + 4 * NH * OTR <= NBUF * TILEB, "partial staging exceeds the tile ring");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int p = range_for_block(blockIdx.x, G);
  if (blockIdx.x == 0 && w == 1) write_prefix(seq_lens, B, 2, cu_out, fmt_out, lane);
  const RangeStart rp = locate_range(seq_lens, B, G, p, lane);
  int64_t start = rp.start;
  const int64_t end = rp.end;
  if (start >= end) return;
  int b = rp.b;
  int64_t s0 = rp.s0, s1 = rp.s1;
  const int head = 32 * w + l32;
  uint8_t* const otr = lds + 4096 + w * (NH * OTR);

  uint32_t kq[4];
  {
    const int kx = swz_key(l32);
#pragma unroll
    for (int j = 0; j < 4; ++j) kq[j] = l32 * ROWB + (((2 * j + g) ^ kx) << 4);
  }
  uint32_t vq[2][2][2];
  {
    const int j16 = lane & 15, h2 = (lane >> 4) & 1;
    const int cst = 2 * h2 + ((j16 & 3) >> 1);
    const int sub = (j16 & 1) * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) {
        const int t = 16 * kk + 4 * g + (j16 >> 2) + 8 * ab;
        const int key = swz_key(t);
#pragma unroll
        for (int par = 0; par < 2; ++par) vq[kk][ab][par] = t * ROWB + sub + (((4 * par + cst) ^ key) << 4);
      }
  }
  // byte offset of the lane's i-th 16-byte chunk in a tile, one register each: unpacking two
  // 16-bit offsets per register cost two VALU instructions per copy inside the score chain
  uint32_t doff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int f = i * 256 + tid, t = f / CHUNKS;
    doff[i] = (uint32_t)(t * ROWB + (swz(t, f - t * CHUNKS) << 4));
  }

  while (start < end) {
    if (s1 <= start) {  // an empty sequence: move on
      ++b;
      s0 = s1;
      s1 = s0 + seq_lens[b];
      continue;
    }
    const int64_t seg_end = end < s1 ? end : s1;
    const int64_t t0 = start - s0, t1 = seg_end - s0;
    const int64_t slot = (int64_t)p + b;
    Rows<PAGED> rows;
    rows.init(cache, b);
    const int64_t n = t1 - t0;
    const int ntiles = (int)((n + TT - 1) / TT);
    const uint8_t* rows_b = (const uint8_t*)cache.rows;

    // ---- tile copies: plan(it) fixes the uniform sources of tile it, copy(cp, i) issues the
    // lane's i-th 16-byte chunk (rows past the segment re-read its last row)
    struct CopyPlan {
      const uint8_t* b0;
      const uint8_t* b1;
      uint32_t split, dst;
      int last;
    };
    auto plan_tile = [&](int it) -> CopyPlan {
      CopyPlan cp;
      const int64_t tt0 = t0 + (int64_t)it * TT;
      cp.last = (int)((t1 - 1 - tt0) < (TT - 1) ? (t1 - 1 - tt0) : (TT - 1));
      cp.dst = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(MLA_LDS void*)(lds + (it % NBUF) * TILEB + w * 1024));
      if constexpr (!PAGED) {
        cp.b0 = rows_b + (rows.base_row + tt0) * ROWB;
        cp.b1 = cp.b0;
        cp.split = 0xffffffffu;
      } else {
        rows.tile(tt0, tt0 + cp.last);
        const int ps = 1 << rows.ps_shift;
        const int s_in = (int)(tt0 & (ps - 1));
        cp.split = (uint32_t)(ps - s_in) * ROWB;
        cp.b0 = rows_b + ((int64_t)rows.pg0 * ps + s_in) * ROWB;
        cp.b1 = rows_b + (int64_t)rows.pg1 * ps * ROWB - (int64_t)cp.split;
      }
      return cp;
    };
    // `partial`: the tile may end before its 32nd row (only a segment's last tile does); callers
    // pass a constant so that full tiles carry no branch
    auto copy = [&](const CopyPlan& cp, int i, bool partial) __attribute__((always_inline)) {
      uint32_t off = doff[i];
      if (partial && cp.last < TT - 1) {
        const int t = (int)(off / ROWB);
        if (t > cp.last) off -= (uint32_t)(t - cp.last) * ROWB;
      }
      if constexpr (!PAGED) dma16_s(cp.b0, off, cp.dst + i * 4096);
      else dma16((off < cp.split ? cp.b0 : cp.b1) + off, cp.dst + i * 4096);
    };
    auto issue_all = [&](int it) {
      const CopyPlan cp = plan_tile(it);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) copy(cp, i, true);
    };
    auto prime = [&]() {
#pragma unroll 1
      for (int it = 0; it < 3 && it < ntiles; ++it) issue_all(it);
    };
    // The first tiles go out ahead of the query loads (the query waits then also cover them);
    // the rest of the prime follows once the query is in registers, so that it does not queue
    // in front of the query.
    constexpr int EARLY = v3::EARLY;
#pragma unroll 1
    for (int it = 0; it < EARLY && it < ntiles; ++it) issue_all(it);

    // ---- absorbed query of this wave's 32 heads, as bf16 B-operand fragments (scale folded in;
    // k_qprep's layout: one coalesced 1 KB load per k-step)
    bf16x8 qf[KSTEPS];
    {
      const bf16x8* src = (const bf16x8*)(qop + ((int64_t)b * 4 + w) * 36 * 1024) + lane;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = src[64 * ks];
      // every fragment in registers before the remaining copies are issued (keeps the waits for
      // the query loads in front of those copies)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) asm volatile("" : "+v"(qf[ks]));
    }
#pragma unroll 1
    for (int it = EARLY; it < 3 && it < ntiles; ++it) issue_all(it);
    auto valid_of = [&](int it) -> int {
      const int64_t r = n - (int64_t)it * TT;
      return r < TT ? (int)r : TT;
    };

    f32x16 O[CB];
    float m_ref = -__builtin_inff(), m_seg = -__builtin_inff(), l_lane = 0.f;
    bool have_ref = false;

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) O[cb] = f32x16{};
      l_lane = 0.f;
      bool over = false;
      if (pass > 0) prime();

      // softmax of one tile in FILL_STEPS steps; register r of s holds token 8(r/4) + 4g + r%4
      f32x16 S;
      float mx = 0.f, rs = 0.f;
      int valid = TT;
      uint8_t* pw = lds_p;  // where fill() puts P
      auto mask_tail = [&]() __attribute__((always_inline)) {
        if (valid < TT) {
          // token 8(r/4) + 4g + r%4 is valid iff 8(r/4) + r%4 < valid - 4g (constants per r,
          // so no per-register index is kept live)
          const int vg = valid - 4 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r) S[r] = (8 * (r >> 2) + (r & 3)) < vg ? S[r] : -__builtin_inff();
        }
      };
      // Softmax step ks of the tile in S (tail already masked). `first`: the segment's first
      // tile, which fixes m_ref (pass 0); inside the tile loop m_ref is set and the steps are
      // branch-free, so they interleave with the PV MFMAs.
      auto fill = [&](int ks, bool first) __attribute__((always_inline)) {
        if (ks == 0) {
          mx = fmaxf(fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3])), fmaxf(fmaxf(S[4], S[5]), fmaxf(S[6], S[7])));
          mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(S[8], S[9]), fmaxf(S[10], S[11])),
                               fmaxf(fmaxf(S[12], S[13]), fmaxf(S[14], S[15]))));
        } else if (ks == 1) {
          if (first && !have_ref) {  // first tile of the segment: the head's maximum over both halves
            m_ref = fmaxf(mx, __shfl_xor(mx, 32, 64));
            have_ref = true;
          }
          m_seg = fmaxf(m_seg, mx);
          over |= mx > m_ref + HEAD;
          rs = 0.f;
        } else if (ks < 18) {
          const int r = ks - 2;
          // keeps the step behind the MFMA issued before it (the MFMAs are volatile asm)
          if (!first) asm volatile("" : "+v"(S[r]));
          // no clamp: a score past m_ref + HEAD sets `over`, and the whole pass is redone
          const float e = __builtin_amdgcn_exp2f(S[r] - m_ref);
          rs += e;
          S[r] = e;
        } else if (ks == 18) {  // P of this tile straight to lds_p, [head][token], swizzled
          l_lane += rs;
          *(bf16x8*)(pw + head * 64 + ((g ^ ((head >> 2) & 3)) << 4)) =
              bf16x8{(__bf16)S[0], (__bf16)S[1], (__bf16)S[2], (__bf16)S[3],
                     (__bf16)S[4], (__bf16)S[5], (__bf16)S[6], (__bf16)S[7]};
        } else if (ks == 19) {
          *(bf16x8*)(pw + head * 64 + (((2 + g) ^ ((head >> 2) & 3)) << 4)) =
              bf16x8{(__bf16)S[8], (__bf16)S[9], (__bf16)S[10], (__bf16)S[11],
                     (__bf16)S[12], (__bf16)S[13], (__bf16)S[14], (__bf16)S[15]};
        }
      };

      // PV of tile `tile` (P from `pr`) with between(j) after MFMA j (0..31)
      auto pv = [&](const uint8_t* tile, const uint8_t* pr, auto&& between) __attribute__((always_inline)) {
        uint32_t vb[2][2][2];
        const uint32_t tb = (uint32_t)(uintptr_t)(MLA_LDS void*)tile + 256u * w;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int par = 0; par < 2; ++par) {
              vb[kk][ab][par] = tb + vq[kk][ab][par];
              asm volatile("" : "+v"(vb[kk][ab][par]));
            }
        auto ldv = [&](int kk, int cb) __attribute__((always_inline)) -> u32x4 {
          const uint32_t ia = vb[kk][0][cb & 1] + 128u * (cb >> 1);
          const uint32_t ib = vb[kk][1][cb & 1] + 128u * (cb >> 1);
          const u32x2 x0 = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(uintptr_t)ia));
          const u32x2 x1 = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(uintptr_t)ib));
          return u32x4{x0.x, x0.y, x1.x, x1.y};
        };
        auto ldp = [&](int kk, int hb) __attribute__((always_inline)) -> bf16x8 {
          const int hr = 32 * hb + l32;
          return *(const bf16x8*)(pr + hr * 64 + (((2 * kk + g) ^ ((hr >> 2) & 3)) << 4));
        };
        u32x4 av[4];
        bf16x8 pbc, pbn;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) av[cb] = ldv(0, cb);
        pbc = ldp(0, 0);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            const bool last_group = kk == 1 && hb == 3;
            if (!last_group) pbn = ldp(hb == 3 ? kk + 1 : kk, hb == 3 ? 0 : hb + 1);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
              if (last_group && cb == 3) {
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                             : "+a"(O[4 * cb + hb]) : "v"(av[cb]), "v"(pbc));
              } else {
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+a"(O[4 * cb + hb]) : "v"(av[cb]), "v"(pbc));
              }
              between(16 * kk + 4 * hb + cb);
              if (kk == 0 && hb == 3) av[cb] = ldv(1, cb);
            }
            pbc = pbn;
          }
        }
      };

      // Software pipeline over the tiles of the segment. Iteration it computes the scores of tile
      // it + 1, issuing the copies of tile it + 3 (into the buffer of tile it - 1) between its
      // MFMAs, then PV of tile it with the softmax of tile it + 1 between the PV MFMAs. P
      // alternates between the two halves of lds_p; one barrier per tile orders it all.
      auto tile_buf = [&](int it) -> const uint8_t* { return lds + (it % NBUF) * TILEB; };
      if (ntiles > 2) vm_wait_barrier<2 * LOADS>();
      else if (ntiles > 1) vm_wait_barrier<LOADS>();
      else vm_wait_barrier<0>();
      S = tile_scores(lds, kq, qf);
      valid = valid_of(0);
      mask_tail();
      pw = lds_p;
#pragma unroll
      for (int ks = 0; ks < FILL_STEPS; ++ks) fill(ks, true);
      for (int it = 0; it < ntiles; ++it) {
        // P(it) visible, tile it + 1 resident (tile it + 2 may be in flight), every wave past PV(it - 1)
        if (it + 2 < ntiles) vm_wait_barrier<LOADS>();
        else vm_wait_barrier<0>();
        const uint8_t* pr = lds_p + (it & 1) * PB;
        if (it + 1 < ntiles) {
          const uint8_t* tn = tile_buf(it + 1);
          if (it + 3 < ntiles) {
            const CopyPlan cp = plan_tile(it + 3);
            if (cp.last < TT - 1) {
              S = tile_scores_copy(tn, kq, qf, [&](int ks) __attribute__((always_inline)) {
                if (ks % 4 == 1 && ks / 4 < LOADS) copy(cp, ks / 4, true);
              });
            } else {
              S = tile_scores_copy(tn, kq, qf, [&](int ks) __attribute__((always_inline)) {
                if (ks % 4 == 1 && ks / 4 < LOADS) copy(cp, ks / 4, false);
              });
            }
          } else {
            S = tile_scores(tn, kq, qf);
          }
        }
        // after the last tile the softmax runs on no valid token: every score is masked, so it
        // adds nothing and only writes zeros into the P buffer nobody reads any more
        valid = it + 1 < ntiles ? valid_of(it + 1) : 0;
        mask_tail();
        pw = lds_p + ((it + 1) & 1) * PB;
        pv(tile_buf(it), pr, [&](int j) __attribute__((always_inline)) {
          if (j < FILL_STEPS) fill(j, false);
        });
      }
      // does any head of the workgroup need the second pass?
      __syncthreads();
      if (tid == 0) *redo_flag = 0;
      __syncthreads();
      if (__builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) *redo_flag = 1;
      __syncthreads();
      const int redo = *redo_flag;
      __syncthreads();
      if (!redo) break;
      m_ref = fmaxf(m_seg, __shfl_xor(m_seg, 32, 64));  // exact maximum of the segment per head
    }

    // ---- normalised partial (float16 rows scaled by 2^-e, 2^e to the scale array) and lse
    const float l_run = l_lane + __shfl_xor(l_lane, 32, 64);
    if (g == 0) lds_l[head] = l_run;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      float m = 0.f;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(O[4 * cb + hb][r]));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (g == 0) lds_m[w][32 * hb + l32] = m;
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int hr = 32 * hb + l32;
      const float inv_l = 1.f / lds_l[hr];
      const float mx2 = fmaxf(fmaxf(lds_m[0][hr], lds_m[1][hr]), fmaxf(lds_m[2][hr], lds_m[3][hr])) * inv_l;
      int e = 0;
      if (mx2 > 0.f) (void)frexpf(mx2, &e);
      const float f = ldexpf(inv_l, -e);
      // this wave's 128 columns of head hr, staged in LDS as one 256-byte row (stride OTR)
      uint8_t* dst = otr + hr * OTR;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x16& o = O[4 * cb + hb];
          const u32x2 v = {pack_f16x2(o[4 * r4 + 0] * f, o[4 * r4 + 1] * f),
                           pack_f16x2(o[4 * r4 + 2] * f, o[4 * r4 + 3] * f)};
          *(u32x2*)(dst + 64 * cb + 16 * r4 + 8 * g) = v;
        }
      if (w == 0 && g == 0) sc_part[slot * NH + hr] = ldexpf(1.f, e);
    }
    // rows back out of LDS as whole 256-byte runs: 16 lanes per row, 4 rows per store (this
    // wave's own staging area, so no barrier; LDS operations of one wave complete in order)
    {
      uint16_t* dst = o_part + slot * NH * DC + 128 * w;
      const int rsub = lane >> 4, ch = lane & 15;
#pragma unroll 8
      for (int j = 0; j < NH / 4; ++j) {
        const int r = 4 * j + rsub;
        const u32x4 v = *(const u32x4*)(otr + r * OTR + 16 * ch);
        *(u32x4*)(dst + (int64_t)r * DC + 8 * ch) = v;
      }
    }
    if (g == 0) lse_part[slot * NH + head] = (m_ref + __log2f(l_run)) * 0.69314718055994530942f;
    __syncthreads();  // lds_l / lds_m and the staging rows are reused by the next segment

    start = seg_end;
    if (start < end) {
      ++b;
      s0 = s1;
      s1 = s0 + seq_lens[b];
    }
  }
}

// ================================================================================================
// MFMA kernel for fp8 e4m3 caches at the DeepSeek-V2 shape. Rows stay fp8 in LDS, so a tile is
// half the bytes of a bf16 tile both in HBM and in LDS. Work split, pipeline (one barrier per
// tile, P double-buffered, copies slotted between the score MFMAs), softmax reference and
// epilogue are those of the bf16 kernel above; what differs:
//   scores: fp8 MFMA 32x32x64 straight on the codes. The query of each head is scaled by a power
//     of two 2^e_h (its largest element lands in [128, 256)) and split into two e4m3 parts
//     q = q_hi + q_lo (about 8 significant bits, like bf16); S = K q_hi + K q_lo is two MFMAs per
//     64-wide k block, and the true score is S * scale_token * 2^-e_h.
//   PV: V^T fragments come from transposing 8-bit LDS reads (8 tokens of one column per lane),
//     widened to bf16 in registers; the token scale is folded into P (P = p * scale_token).
//   tiles: 32 rows of 576 bytes plus the 32 token scales, copied straight into LDS; a 7-buffer
//     ring keeps up to 5 tiles in flight.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

namespace f8 {
constexpr int RB = 576;                    // bytes of one fp8 row
constexpr int CH = RB / 16;                // 16-byte chunks per row (36)
constexpr int ROWSB = v2::TT * RB;         // 18432
constexpr int SCB = 512;                   // two 256-byte token-scale slots
constexpr int TILEB = ROWSB + SCB;         // 18944
constexpr int NBUF = 7;
constexpr int AHEAD = NBUF - 2;            // tiles in flight besides the two being computed on
constexpr int LOADS = 5;                   // copy instructions per wave per tile
constexpr int KB = RB / 64;                // 64-wide k blocks (9)
constexpr int PB = v2::NH * v2::TT * 2;    // bytes of P of one tile
constexpr int LDS_BYTES = NBUF * TILEB + 2 * PB;
}  // namespace f8

// The same kernel over fp6 e2m3 caches: rows of 576 codes packed 6 bits each (432 bytes) are
// copied into a ring of packed slots, and each tile is converted once, exactly, into the e4m3 tile
// layout above (every e2m3 value is an e4m3 value) in one of two e4m3 buffers; the scores, softmax
// and PV then run as for an fp8 cache. A packed slot holds the 32 rows, 512 bytes that absorb the
// copy lanes past the last row, and the two token-scale slots.
namespace f6 {
constexpr int RB = 432;                    // bytes of one packed row
constexpr int CH = RB / 16;                // 16-byte chunks per row (27)
constexpr int ROWSB = v2::TT * RB;         // 13824 (864 chunks: 13.5 copies of 1 KB)
constexpr int SCO = ROWSB + 512;           // token-scale slots
constexpr int SLOTB = SCO + 512;           // 14848
constexpr int NBUF = 7;
constexpr int LOADS = 4;                   // copy instructions per wave per tile
constexpr int EB = v2::TT * f8::RB;        // one e4m3 tile (18432)
constexpr int LDS_BYTES = NBUF * SLOTB + 2 * EB + 2 * f8::PB;
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
}  // namespace f6

// 16-byte chunk c of fp8 tile row t sits at chunk position (c & ~3) | ((c & 3) ^ key8(t)) (rows of
// 36 chunks, so the XOR stays inside the aligned group of 4). With rows 576 bytes apart, row t
// starts at bank group 4t mod 16; the key separates rows t, t+4, t+8, t+12, so the 16 rows of a
// 16-lane score read and the 8 rows x 2 chunks of a 32-lane transposing read hit distinct groups.
__device__ __forceinline__ int key8(int t) { return (t >> 2) & 3; }

// 4-byte global -> LDS copy per lane (LDS destination: wave-uniform `lds_addr` + 4 * lane).
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt"
               :: "v"(src), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

// Scores of one fp8 tile: S^T[32 tok x 32 heads] over the 9 k blocks, two MFMAs per block (q_hi,
// q_lo). K fragment of block kb: 32 bytes of row l32 at k = 32g.. (chunks 4kb + 2g, 4kb + 2g + 1),
// read LA blocks ahead. between(j) runs after MFMA j (0..17). The leading s_nop covers a VALU
// write of the query registers right before; the trailing ones the MFMA-result -> VALU-read wait.
template <typename F>
__device__ __forceinline__ f32x16 tile_scores8(const uint8_t* tile, const uint32_t (&kq)[2],
                                               const i32x8 (&qh)[f8::KB], const i32x8 (&ql)[f8::KB],
                                               F&& between) {
  constexpr int KB = f8::KB, LA = 2;
  i32x8 a[KB];
  auto lda = [&](int kb) __attribute__((always_inline)) -> i32x8 {
    const u32x4 x = *(const u32x4*)(tile + kq[0] + 64 * kb);
    const u32x4 y = *(const u32x4*)(tile + kq[1] + 64 * kb);
    return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  };
#pragma unroll
  for (int j = 0; j < LA; ++j) a[j] = lda(j);
  f32x16 s;
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=v"(s) : "v"(a[0]), "v"(qh[0]));
  between(0);
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(a[0]), "v"(ql[0]));
  between(1);
  a[LA] = lda(LA);
#pragma unroll
  for (int kb = 1; kb < KB; ++kb) {
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(a[kb]), "v"(qh[kb]));
    between(2 * kb);
    if (kb == KB - 1) {
      asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+v"(s) : "v"(a[kb]), "v"(ql[kb]));
    } else {
      asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(a[kb]), "v"(ql[kb]));
    }
    between(2 * kb + 1);
    if (kb + LA < KB) a[kb + LA] = lda(kb + LA);
  }
  return s;
}

// 8 e4m3 codes -> 8 bf16 (exact); the hardware pair conversion takes the codes of one 16-bit half
__device__ __forceinline__ bf16x8 widen8(u32x2 r) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// LDS-only barrier: waits for this wave's LDS operations (not for its in-flight global->LDS copies)
__device__ __forceinline__ void lds_sync_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool PAGED, bool FP6>
__global__ __launch_bounds__(256, 1) void k_decode_fp8(const uint8_t* __restrict__ qop,
                                                      const float* __restrict__ fh_in, CacheArgs cache,
                                                      const int32_t* __restrict__ seq_lens, int B, int G,
                                                      int64_t* __restrict__ cu_out, int32_t* __restrict__ fmt_out,
                                                      float* __restrict__ lse_part,
                                                      float* __restrict__ sc_part,
                                                      uint16_t* __restrict__ o_part) {
  using namespace v2;
  using f8::RB;        // e4m3 row bytes in LDS
  using f8::KB;
  // HRB: bytes of one cached row in HBM (and in the copy slots); SLOTB: one copy slot; SCO: offset
  // of its token-scale slots
  constexpr int HRB = FP6 ? f6::RB : f8::RB, HCH = FP6 ? f6::CH : f8::CH;
  constexpr int SLOTB = FP6 ? f6::SLOTB : f8::TILEB, SCO = FP6 ? f6::SCO : f8::ROWSB;
  constexpr int NBUF = FP6 ? f6::NBUF : f8::NBUF, AHEAD = NBUF - 2, LOADS8 = FP6 ? f6::LOADS : f8::LOADS;
  constexpr int PB = f8::PB;
  constexpr int LDS_BYTES = FP6 ? f6::LDS_BYTES : f8::LDS_BYTES;
  constexpr float HEAD = 64.f;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  uint8_t* const ebase = lds + NBUF * SLOTB;              // fp6: the two converted e4m3 tiles
  uint8_t* const lds_p = ebase + (FP6 ? 2 * f6::EB : 0);  // P of two consecutive tiles
  int* const redo_flag = (int*)lds;
  float* const lds_l = (float*)(lds + 16);
  float (*const lds_m)[NH] = (float (*)[NH])(lds + 16 + NH * 4);
  constexpr int OTR = 272;
  static_assert(4096 + 4 * NH * OTR <= LDS_BYTES, "partial staging exceeds the tile ring");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int g = lane >> 5, l32 = lane & 31;
  const int p = range_for_block(blockIdx.x, G);
  if (blockIdx.x == 0 && w == 1) write_prefix(seq_lens, B, 2, cu_out, fmt_out, lane);
  const RangeStart rp = locate_range(seq_lens, B, G, p, lane);
  int64_t start = rp.start;
  const int64_t end = rp.end;
  if (start >= end) return;
  int b = rp.b;
  int64_t s0 = rp.s0, s1 = rp.s1;
  const int head = 32 * w + l32;
  uint8_t* const otr = lds + 4096 + w * (NH * OTR);

  // K fragments: chunks 4kb + 2g + h of row l32 -> kq[h] + 64 kb
  uint32_t kq[2];
  {
    const int kx = key8(l32);
#pragma unroll
    for (int h = 0; h < 2; ++h) kq[h] = l32 * RB + (((2 * g + h) ^ kx) << 4);
  }
  // V^T fragments (transposing 8-bit reads): in each 16-lane group, lanes 2r and 2r+1 address row
  // 16kk + 8(r/4) + 4g + r%4 at columns 128w + 32cb + 16h2 + 8(lane & 1), and lane c of the group
  // receives column c of the 8 rows in row order: slot j = token 16kk + 8(j/4) + 4g + j%4, the
  // token order of P's B operand. Chunk 8w + 4(cb/2) + 2(cb%2) + h2 -> vq[kk][cb%2] + 64(cb/2).
  uint32_t vq[2][2];
  {
    const int j16 = lane & 15, h2 = (lane >> 4) & 1, r = j16 >> 1;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int t = 16 * kk + 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
      for (int par = 0; par < 2; ++par)
        vq[kk][par] = t * RB + (((2 * par + h2) ^ key8(t)) << 4) + 8 * (j16 & 1);
    }
  }
  // Copies: wave w moves row chunks R = w + 4i (i < 4) and, for w < 2, R = 16 + w; waves 2 and 3
  // copy the 32 token scales (each into its own slot, so that every wave issues 5 copies per
  // tile). Row chunk R, lane L fills LDS chunk 64R + L = row t, position pos: source chunk
  // (pos & ~3) | ((pos & 3) ^ key8(t)) of row t. One offset per register (unpacking two 16-bit
  // offsets per register cost two VALU instructions per copy inside the score chain).
  // fp6: the packed rows are copied as they are (LDS chunk 64R + L from source chunk 64R + L):
  // wave w moves R = w + 4i (i < 3) and, for w < 2, R = 12 + w; waves 2 and 3 copy the scales, so
  // every wave issues 4 copies. The 32 lanes of R = 13 past the 864 chunks of the rows re-read the
  // last chunk into the slot's 512-byte pad.
  uint32_t doff[LOADS8];
#pragma unroll
  for (int i = 0; i < LOADS8; ++i) {
    doff[i] = 0u;
    if constexpr (FP6) {
      const int R = i < 3 ? w + 4 * i : 12 + w;
      if (R < 14) {
        const int f = 64 * R + lane;
        doff[i] = (uint32_t)((f < 864 ? f : 863) << 4);
      }
    } else {
      const int R = i < 4 ? w + 4 * i : 16 + w;
      if (R < 18) {
        const int f = 64 * R + lane, t = f / f8::CH, pos = f - t * f8::CH;
        doff[i] = (uint32_t)(t * RB + (((pos & ~3) | ((pos & 3) ^ key8(t))) << 4));
      }
    }
  }

  while (start < end) {
    if (s1 <= start) {  // an empty sequence: move on
      ++b;
      s0 = s1;
      s1 = s0 + seq_lens[b];
      continue;
    }
    const int64_t seg_end = end < s1 ? end : s1;
    const int64_t t0 = start - s0, t1 = seg_end - s0;
    const int64_t slot = (int64_t)p + b;
    Rows<PAGED> rows;
    rows.init(cache, b);
    const int64_t n = t1 - t0;
    const int ntiles = (int)((n + TT - 1) / TT);
    const uint8_t* rows_b = (const uint8_t*)cache.rows;

    struct CopyPlan {
      const uint8_t* b0;
      const uint8_t* b1;
      const float* sc0;
      int64_t tt0;
      uint32_t split, dst;
      int last;
    };
    auto plan_tile = [&](int it) -> CopyPlan {
      CopyPlan cp;
      const int64_t tt0 = t0 + (int64_t)it * TT;
      cp.tt0 = tt0;
      cp.last = (int)((t1 - 1 - tt0) < (TT - 1) ? (t1 - 1 - tt0) : (TT - 1));
      cp.dst = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(MLA_LDS void*)(lds + (it % NBUF) * SLOTB));
      if constexpr (!PAGED) {
        cp.b0 = rows_b + (rows.base_row + tt0) * HRB;
        cp.b1 = cp.b0;
        cp.sc0 = cache.scales + rows.base_row + tt0;
        cp.split = 0xffffffffu;
      } else {
        rows.tile(tt0, tt0 + cp.last);
        const int ps = 1 << rows.ps_shift;
        const int s_in = (int)(tt0 & (ps - 1));
        cp.split = (uint32_t)(ps - s_in) * HRB;
        cp.b0 = rows_b + ((int64_t)rows.pg0 * ps + s_in) * HRB;
        cp.b1 = rows_b + (int64_t)rows.pg1 * ps * HRB - (int64_t)cp.split;
        cp.sc0 = cache.scales;
      }
      return cp;
    };
    // copy i of this wave for the planned tile; `partial` as in the bf16 kernel (a chunk of a row
    // past the segment's last row re-reads the same chunk of the last row)
    constexpr int NROWCP = FP6 ? 3 : 4;  // row copies every wave issues; waves 0 and 1 add one more
    auto copy = [&](const CopyPlan& cp, int i, bool partial) __attribute__((always_inline)) {
      if (i < NROWCP || wu < 2) {
        uint32_t off = doff[i];
        if (partial && cp.last < TT - 1) {
          const int t = (int)(off / HRB);
          if (t > cp.last) off -= (uint32_t)(t - cp.last) * HRB;
        }
        const uint32_t dst = cp.dst + 1024u * (uint32_t)(i < NROWCP ? wu + 4 * i : 4 * NROWCP + wu);
        if constexpr (!PAGED) dma16_s(cp.b0, off, dst);
        else dma16((off < cp.split ? cp.b0 : cp.b1) + off, dst);
      } else {
        const int tk = l32 < cp.last ? l32 : cp.last;
        const uint32_t dst = cp.dst + (uint32_t)SCO + 256u * (uint32_t)(wu - 2);
        if constexpr (!PAGED) dma4_s(cp.sc0, 4u * (uint32_t)tk, dst);
        else dma4(cp.sc0 + rows.row(cp.tt0 + tk), dst);
      }
    };
    auto issue_all = [&](int it) {
      const CopyPlan cp = plan_tile(it);
#pragma unroll
      for (int i = 0; i < LOADS8; ++i) copy(cp, i, true);
    };
    constexpr int EARLY = 2;
#pragma unroll 1
    for (int it = 0; it < EARLY && it < ntiles; ++it) issue_all(it);

    // ---- absorbed query of this wave's 32 heads as two e4m3 parts (k_qprep's layout: the
    // B-operand bytes of lane half g, k = 32g..32g+31 of each 64-wide block)
    i32x8 qh[KB], ql[KB];
    float fh;  // 2^-e_h
    {
      const u32x4* src = (const u32x4*)(qop + ((int64_t)b * 4 + w) * 36 * 1024) + lane;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 x0 = src[64 * (4 * kb)], x1 = src[64 * (4 * kb + 1)];
        const u32x4 y0 = src[64 * (4 * kb + 2)], y1 = src[64 * (4 * kb + 3)];
        qh[kb] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        ql[kb] = i32x8{(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
      }
      fh = fh_in[(int64_t)b * NH + head];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+v"(qh[kb]), "+v"(ql[kb]));
      asm volatile("" : "+v"(fh));
    }
    auto prime = [&](int from) {
#pragma unroll 1
      for (int it = from; it < AHEAD + 1 && it < ntiles; ++it) issue_all(it);
    };
    prime(EARLY);
    auto valid_of = [&](int it) -> int {
      const int64_t r = n - (int64_t)it * TT;
      return r < TT ? (int)r : TT;
    };
    // wait until tile `need` has landed, given that tiles up to `issued` have been requested
    auto wait_tile = [&](int need, int issued) __attribute__((always_inline)) {
      const int k = issued - need;  // tiles that may stay in flight
      if (k >= 5) vm_wait_barrier<5 * LOADS8>();
      else if (k == 4) vm_wait_barrier<4 * LOADS8>();
      else if (k == 3) vm_wait_barrier<3 * LOADS8>();
      else if (k == 2) vm_wait_barrier<2 * LOADS8>();
      else if (k == 1) vm_wait_barrier<LOADS8>();
      else vm_wait_barrier<0>();
    };

    f32x16 O[CB];
    // m_ref: the reference maximum (true score units, base 2); x_max: the largest exponent
    // s - m_ref this lane met in the pass (the segment's maximum is m_ref + x_max)
    float m_ref = -__builtin_inff(), x_max = -__builtin_inff(), l_lane = 0.f;
    bool have_ref = false;

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) O[cb] = f32x16{};
      l_lane = 0.f;
      bool over = false;
      if (pass > 0) prime(0);

      // Softmax of one tile; register r of S holds token 8(r/4) + 4g + r%4 of the tile. With
      // c_r = scale_token * 2^-e_h, the score is S_r c_r; the probability against the reference
      // is e_r = 2^(S_r c_r - m_ref) and P carries e_r c_r (= p * scale_token * 2^-e_h: the output
      // accumulates 2^-e_h O, and the normaliser l 2^-e_h undoes it). Steps 0-15 handle one
      // register each; 16 and 17 publish P.
      // The token scales of register group q (tokens 8q + 4g ..+3) are read from the tile's scale
      // slot one group ahead, into cg[q & 1] (group 0 during the scores).
      f32x16 S;
      f32x4 cg[2];
      const float* sct = (const float*)(lds + SCO);  // scale slot of the tile being softmaxed
      float rs = 0.f;
      int valid = TT;
      uint8_t* pw = lds_p;
      auto load_group = [&](int q) __attribute__((always_inline)) {
        cg[q & 1] = *(const f32x4*)(sct + 8 * q + 4 * g);
      };
      auto mask_tail = [&]() __attribute__((always_inline)) {
        if (valid < TT) {
          const int vg = valid - 4 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r) S[r] = (8 * (r >> 2) + (r & 3)) < vg ? S[r] : -__builtin_inff();
        }
      };
      // the segment's first tile fixes m_ref (pass 0): the head's maximum over both halves
      auto set_ref = [&]() __attribute__((always_inline)) {
        if (!have_ref) {
          float mx = -__builtin_inff();
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[r] * sct[8 * (r >> 2) + 4 * g + (r & 3)] * fh);
          m_ref = fmaxf(mx, __shfl_xor(mx, 32, 64));
          have_ref = true;
        }
      };
      auto fill = [&](int ks, bool first) __attribute__((always_inline)) {
        if (ks < 16) {
          const int r = ks;
          if ((r & 3) == 0 && r < 12) load_group((r >> 2) + 1);
          if (!first) asm volatile("" : "+v"(S[r]));
          const float c = cg[(r >> 2) & 1][r & 3] * fh;
          const float x = fmaf(S[r], c, -m_ref);
          x_max = fmaxf(x_max, x);
          const float e = __builtin_amdgcn_exp2f(x);
          rs = r == 0 ? e : rs + e;
          S[r] = e * c;
        } else if (ks == 16) {
          l_lane += rs;
          *(bf16x8*)(pw + head * 64 + ((g ^ ((head >> 2) & 3)) << 4)) =
              bf16x8{(__bf16)S[0], (__bf16)S[1], (__bf16)S[2], (__bf16)S[3],
                     (__bf16)S[4], (__bf16)S[5], (__bf16)S[6], (__bf16)S[7]};
        } else if (ks == 17) {
          *(bf16x8*)(pw + head * 64 + (((2 + g) ^ ((head >> 2) & 3)) << 4)) =
              bf16x8{(__bf16)S[8], (__bf16)S[9], (__bf16)S[10], (__bf16)S[11],
                     (__bf16)S[12], (__bf16)S[13], (__bf16)S[14], (__bf16)S[15]};
        }
      };
      constexpr int FILL8 = 18;

      // V^T fragments of one tile: transposing 8-bit reads, widened to bf16
      auto vbase = [&](const uint8_t* tile, uint32_t (&vb)[2][2]) __attribute__((always_inline)) {
        const uint32_t tb = (uint32_t)(uintptr_t)(MLA_LDS void*)tile + 128u * w;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            vb[kk][par] = tb + vq[kk][par];
            asm volatile("" : "+v"(vb[kk][par]));
          }
      };
      auto ldv = [&](const uint32_t (&vb)[2][2], int kk, int cb) __attribute__((always_inline)) -> u32x2 {
        const uint32_t ia = vb[kk][cb & 1] + 64u * (cb >> 1);
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)(uintptr_t)ia));
      };
      // P fragment (B operand) of heads 32hb.. for k step kk
      auto ldp = [&](const uint8_t* pr, int kk, int hb) __attribute__((always_inline)) -> bf16x8 {
        const int hr = 32 * hb + l32;
        return *(const bf16x8*)(pr + hr * 64 + (((2 * kk + g) ^ ((hr >> 2) & 3)) << 4));
      };
      // PV of tile `tile` (P from `pr`); av: the kk = 0 fragments, already widened; p0: the first
      // P fragment. between(j) runs after MFMA j (0..31). The first MFMA that reads a freshly
      // widened fragment starts with the 2 wait states a VALU write -> MFMA read needs.
      auto pv = [&](const uint8_t* tile, const uint8_t* pr, bf16x8 (&av)[4], const bf16x8& p0, auto&& between)
                    __attribute__((always_inline)) {
        uint32_t vb[2][2];
        vbase(tile, vb);
        u32x2 rv[4];
        bf16x8 pbc = p0, pbn;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            const bool last_group = kk == 1 && hb == 3;
            if (!last_group) pbn = ldp(pr, hb == 3 ? kk + 1 : kk, hb == 3 ? 0 : hb + 1);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
              if (last_group && cb == 3) {
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                             : "+a"(O[4 * cb + hb]) : "v"(av[cb]), "v"(pbc));
              } else if (hb == 0) {
                asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+a"(O[4 * cb + hb]) : "v"(av[cb]), "v"(pbc));
              } else {
                asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+a"(O[4 * cb + hb]) : "v"(av[cb]), "v"(pbc));
              }
              between(16 * kk + 4 * hb + cb);
              if (kk == 0 && hb == 1) rv[cb] = ldv(vb, 1, cb);
              if (kk == 0 && hb == 3) av[cb] = widen8(rv[cb]);
            }
            pbc = pbn;
          }
        }
      };
      // Scores of tile tn (`copies` runs after MFMA j as well). Spread over its MFMAs, what the
      // next steps need first is fetched well ahead of use: the kk = 0 V fragments of tile tv
      // (read, then widened one per MFMA), the first P fragment of PV (from pr), and the
      // coefficients c_r of tile tn.
      auto scores = [&](const uint8_t* tn, const uint8_t* sn, const uint8_t* tv, const uint8_t* pr, bf16x8 (&av)[4],
                        bf16x8& p0, auto&& copies) __attribute__((always_inline)) {
        sct = (const float*)sn;
        uint32_t vb[2][2];
        vbase(tv, vb);
        u32x2 rv[4];
        // after score MFMA j: V reads at JV, JV + 1; P fragment at JP; widening at JW..JW+3;
        // the first scale group at JS
        constexpr int JV = 5, JP = 12, JW = 9, JS = 14;
        S = tile_scores8(tn, kq, qh, ql, [&](int j) __attribute__((always_inline)) {
          copies(j);
          if (j == JV) { rv[0] = ldv(vb, 0, 0); rv[1] = ldv(vb, 0, 1); }
          if (j == JV + 1) { rv[2] = ldv(vb, 0, 2); rv[3] = ldv(vb, 0, 3); }
          if (j == JP) p0 = ldp(pr, 0, 0);
          if (j >= JW && j < JW + 4) {
            av[j - JW] = widen8(rv[j - JW]);
            asm volatile("" : "+v"(av[j - JW]));
          }
          if (j == JS) load_group(0);
        });
      };

      // e4m3 rows of tile j (fp8: its copy slot; fp6: converted buffer j & 1) and its token scales
      auto tile_buf = [&](int it) -> const uint8_t* {
        if constexpr (FP6) return ebase + (it & 1) * f6::EB;
        else return lds + (it % NBUF) * SLOTB;
      };
      auto scale_buf = [&](int it) -> const uint8_t* { return lds + (it % NBUF) * SLOTB + SCO; };
      // fp6: the packed rows of tile j -> the e4m3 layout of buffer j & 1 (exact: every e2m3 value
      // is an e4m3 value); group = 32 codes of one row (24 packed bytes -> two 16-byte chunks).
      // Every wave must be past the last reads of that buffer (PV of tile j - 2) and every copy of
      // tile j must have landed: the callers run it right after the barrier that ensures both.
      auto convert = [&](int j) __attribute__((always_inline)) {
        if constexpr (FP6) {
          typedef int i32x6 __attribute__((ext_vector_type(6)));
          typedef float f32x32 __attribute__((ext_vector_type(32)));
          const uint8_t* ps = lds + (j % NBUF) * SLOTB;
          uint8_t* eb = ebase + (j & 1) * f6::EB;
          for (int gi = tid; gi < TT * 18; gi += 256) {
            const int t = gi / 18, kb = gi - 18 * t;
            const uint8_t* src = ps + t * f6::RB + kb * 24;
            const u32x2 a0 = *(const u32x2*)src, a1 = *(const u32x2*)(src + 8), a2 = *(const u32x2*)(src + 16);
            const i32x6 x = {(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y};
            const f32x32 f = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(x, 1.0f);
            uint32_t wd[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              int hw = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * q], f[4 * q + 1], 0, false);
              hw = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * q + 2], f[4 * q + 3], hw, true);
              wd[q] = (uint32_t)hw;
            }
            const int kx = key8(t);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int cc = 2 * kb + h;
              *(u32x4*)(eb + t * RB + (((cc & ~3) | ((cc & 3) ^ kx)) << 4)) =
                  u32x4{wd[4 * h], wd[4 * h + 1], wd[4 * h + 2], wd[4 * h + 3]};
            }
          }
          lds_sync_barrier();
        }
      };
      bf16x8 av[4], p0;
      wait_tile(0, (AHEAD < ntiles - 1 ? AHEAD : ntiles - 1));
      convert(0);
      scores(tile_buf(0), scale_buf(0), tile_buf(0), lds_p, av, p0, [](int) {});
      valid = valid_of(0);
      mask_tail();
      if (pass == 0) set_ref();
      pw = lds_p;
#pragma unroll
      for (int ks = 0; ks < FILL8; ++ks) fill(ks, true);
      for (int it = 0; it < ntiles; ++it) {
        // P(it) visible, tile it + 1 resident, every wave past PV(it - 1)
        {
          const int issued = it + AHEAD < ntiles - 1 ? it + AHEAD : ntiles - 1;
          wait_tile(it + 1 < ntiles ? it + 1 : issued, issued);
        }
        const uint8_t* pr = lds_p + (it & 1) * PB;
        const uint8_t* tv = tile_buf(it);
        if (it + 1 < ntiles) {
          convert(it + 1);
          const uint8_t* tn = tile_buf(it + 1);
          const uint8_t* sn = scale_buf(it + 1);
          if (it + AHEAD + 1 < ntiles) {
            const CopyPlan cp = plan_tile(it + AHEAD + 1);
            if (cp.last < TT - 1) {
              scores(tn, sn, tv, pr, av, p0, [&](int j) __attribute__((always_inline)) {
                if (j % 3 == 1 && j / 3 < LOADS8) copy(cp, j / 3, true);
              });
            } else {
              scores(tn, sn, tv, pr, av, p0, [&](int j) __attribute__((always_inline)) {
                if (j % 3 == 1 && j / 3 < LOADS8) copy(cp, j / 3, false);
              });
            }
          } else {
            scores(tn, sn, tv, pr, av, p0, [](int) {});
          }
        } else {
          uint32_t vb[2][2];
          vbase(tv, vb);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) av[cb] = widen8(ldv(vb, 0, cb));
          p0 = ldp(pr, 0, 0);
        }
        valid = it + 1 < ntiles ? valid_of(it + 1) : 0;
        mask_tail();
        pw = lds_p + ((it + 1) & 1) * PB;
        pv(tv, pr, av, p0, [&](int j) __attribute__((always_inline)) {
          if (j < FILL8) fill(j, false);
        });
      }
      over = x_max > HEAD;
      __syncthreads();
      if (tid == 0) *redo_flag = 0;
      __syncthreads();
      if (__builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) *redo_flag = 1;
      __syncthreads();
      const int redo = *redo_flag;
      __syncthreads();
      if (!redo) break;
      // the segment's exact maximum per head (x_max >= 0: the first tile holds the reference)
      m_ref += fmaxf(x_max, __shfl_xor(x_max, 32, 64));
      x_max = -__builtin_inff();
    }

    // ---- normalised partial (float16 rows scaled by 2^-e, 2^e to the scale array) and lse
    const float l_run = l_lane + __shfl_xor(l_lane, 32, 64);
    if (g == 0) lds_l[head] = l_run * fh;  // O holds 2^-e_h times the weighted sum
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      float m = 0.f;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(O[4 * cb + hb][r]));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (g == 0) lds_m[w][32 * hb + l32] = m;
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int hr = 32 * hb + l32;
      const float inv_l = 1.f / lds_l[hr];
      const float mx2 = fmaxf(fmaxf(lds_m[0][hr], lds_m[1][hr]), fmaxf(lds_m[2][hr], lds_m[3][hr])) * inv_l;
      int e = 0;
      if (mx2 > 0.f) (void)frexpf(mx2, &e);
      const float f = ldexpf(inv_l, -e);
      uint8_t* dst = otr + hr * OTR;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x16& o = O[4 * cb + hb];
          const u32x2 v = {pack_f16x2(o[4 * r4 + 0] * f, o[4 * r4 + 1] * f),
                           pack_f16x2(o[4 * r4 + 2] * f, o[4 * r4 + 3] * f)};
          *(u32x2*)(dst + 64 * cb + 16 * r4 + 8 * g) = v;
        }
      if (w == 0 && g == 0) sc_part[slot * NH + hr] = ldexpf(1.f, e);
    }
    {
      uint16_t* dst = o_part + slot * NH * DC + 128 * w;
      const int rsub = lane >> 4, ch = lane & 15;
#pragma unroll 8
      for (int j = 0; j < NH / 4; ++j) {
        const int r = 4 * j + rsub;
        const u32x4 v = *(const u32x4*)(otr + r * OTR + 16 * ch);
        *(u32x4*)(dst + (int64_t)r * DC + 8 * ch) = v;
      }
    }
    if (g == 0) lse_part[slot * NH + head] = (m_ref + __log2f(l_run)) * 0.69314718055994530942f;
    __syncthreads();

    start = seg_end;
    if (start < end) {
      ++b;
      s0 = s1;
      s1 = s0 + seq_lens[b];
    }
  }
}

// ================================================================================================
// Generic kernel (any cache dtype, small dims): float32 arithmetic throughout. Used for the
// running model and float32 caches. Limits: n_h*(d_c+d_r) <= 16384, d_c+d_r <= 512, n_h <= 64,
// n_h*d_c <= 4096. Tiles of 32 tokens: wave w fetches rows w, w+4, ... of the next tile into
// registers while the current tile is processed from LDS (rows padded to an odd stride, so the
// per-token score reads hit distinct banks).
// Barrier for LDS hand-offs only: waits for this wave's LDS operations, not for its global loads
// (__syncthreads() also waits for every outstanding global load, which would drain the next
// tile's prefetch at each barrier).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

namespace gen {
constexpr int TT = 32;
constexpr int OPT = 16;  // outputs per thread
}

// Raw stored bits of one element, and their value (fp8: times the row's scale). Loads keep the raw
// bits so that no conversion waits on a load before the next ones are issued.
// fp6 rows are rw * 6 / 8 bytes: code e sits at bits 6e .. 6e + 5 of the row's little-endian
// stream, i.e. in byte 6e / 8 and (for a shift above 2) the next byte, which is then inside the row.
template <int CDT>
__device__ __forceinline__ uint32_t cache_bits(const CacheArgs& c, int64_t ridx, int rw, int e) {
  if constexpr (CDT == MLA_F32) return ((const uint32_t*)c.rows)[ridx * rw + e];
  else if constexpr (CDT == MLA_F16 || CDT == MLA_BF16) return ((const uint16_t*)c.rows)[ridx * rw + e];
  else if constexpr (CDT == MLA_FP6_E2M3) {
    const uint8_t* row = (const uint8_t*)c.rows + ridx * (rw / 4 * 3);
    const int bit = 6 * e, byte = bit >> 3, sh = bit & 7;
    const int nxt = sh > 2 ? byte + 1 : byte;
    return (((uint32_t)row[byte] | ((uint32_t)row[nxt] << 8)) >> sh) & 63u;
  }
  else return ((const uint8_t*)c.rows)[ridx * rw + e];
}
template <int CDT>
__device__ __forceinline__ float bits_value(uint32_t x, float sc) {
  if constexpr (CDT == MLA_F32) return __builtin_bit_cast(float, x);
  else if constexpr (CDT == MLA_F16) return f16_bits_to_f32((uint16_t)x);
  else if constexpr (CDT == MLA_BF16) return bf16_bits_to_f32((uint16_t)x);
  else if constexpr (CDT == MLA_FP6_E2M3) return e2m3_to_f32(x) * sc;
  else return e4m3_to_f32(x) * sc;
}


template <int CDT, int EPL, bool PAGED>
__global__ __launch_bounds__(256) void k_decode_generic(int n_h, int d_c, int d_r,
                                                        const float* __restrict__ q_lat,
                                                        const float* __restrict__ q_pe, CacheArgs cache,
                                                        const int32_t* __restrict__ seq_lens, int B, int G,
                                                        int64_t* __restrict__ cu_out, int32_t* __restrict__ fmt_out,
                                                        float qscale, float* __restrict__ lse_part,
                                                        float* __restrict__ o_part) {
  using namespace gen;
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int rw = d_c + d_r;
  // padded row stride of the tile in LDS: a multiple of 4 floats whose quarter is odd (rw is a
  // multiple of 8), so 16 consecutive rows read at one offset hit 16 distinct 16-byte bank groups
  const int rwp = rw + 4;
  float* qs = sm;                       // [n_h][rw]
  float* ts = qs + n_h * rw;            // [TT][rwp]
  float* ss = ts + TT * rwp;            // [n_h][TT]
  float* mrun = ss + n_h * TT;          // [n_h]
  float* lrun = mrun + n_h;             // [n_h]
  float* alf = lrun + n_h;              // [n_h]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int p = range_for_block(blockIdx.x, G);
  if (blockIdx.x == 0 && w == 1) write_prefix(seq_lens, B, 0, cu_out, fmt_out, lane);
  const RangeStart rp = locate_range(seq_lens, B, G, p, lane);
  int64_t start = rp.start;
  const int64_t end = rp.end;
  if (start >= end) return;
  int b = rp.b;
  int64_t s0 = rp.s0, s1 = rp.s1;
  const int nout = n_h * d_c;

  while (start < end) {
    if (s1 <= start) {
      ++b;
      s0 = s1;
      s1 = s0 + seq_lens[b];
      continue;
    }
    const int64_t seg_end = end < s1 ? end : s1;
    const int64_t t0 = start - s0, t1 = seg_end - s0;
    const int64_t slot = (int64_t)p + b;
    for (int i = tid; i < n_h * rw; i += 256) {
      int h = i / rw, e = i % rw;
      qs[i] = (e < d_c ? q_lat[((int64_t)b * n_h + h) * d_c + e] : q_pe[((int64_t)b * n_h + h) * d_r + e - d_c]) * qscale;
    }
    for (int h = tid; h < n_h; h += 256) { mrun[h] = -__builtin_inff(); lrun[h] = 0.f; }
    constexpr int OPT4 = OPT / 4;
    const int nout4 = nout / 4;
    f32x4 O[OPT4];
#pragma unroll
    for (int k = 0; k < OPT4; ++k) O[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // rows of one tile in registers: row w + 4m, elements lane + 64j (rows past the segment
    // re-read its last row; their scores are masked)
    // EPL = element groups of 64 per row (rw <= 64 * EPL)
    constexpr int RPW = TT / 4;
    uint32_t v[RPW][EPL];
    float vsc[RPW];
    auto fetch = [&](int64_t tb) __attribute__((always_inline)) {
      const int vt = (int)((t1 - tb) < TT ? (t1 - tb) : TT);
      int64_t ridx[RPW];
#pragma unroll
      for (int m = 0; m < RPW; ++m) {
        const int64_t j = tb + (w + 4 * m < vt ? w + 4 * m : vt - 1);
        if constexpr (PAGED) ridx[m] = row_index(cache, b, j);
        else ridx[m] = (int64_t)b * cache.t_cap + j;
      }
      // every load is issued (indices past the row clamp to its last element), none behind a branch
#pragma unroll
      for (int m = 0; m < RPW; ++m) {
        if constexpr (CDT == MLA_FP8_E4M3 || CDT == MLA_FP6_E2M3) vsc[m] = cache.scales[ridx[m]];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const int e = lane + 64 * j;
          v[m][j] = cache_bits<CDT>(cache, ridx[m], rw, e < rw ? e : rw - 1);
        }
      }
    };
    fetch(t0);
    lds_barrier();
    for (int64_t tb = t0; tb < t1; tb += TT) {
      const int valid = (int)((t1 - tb) < TT ? (t1 - tb) : TT);
#pragma unroll
      for (int m = 0; m < RPW; ++m)
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const int e = lane + 64 * j;
          if (e < rw)
            ts[(w + 4 * m) * rwp + e] =
                bits_value<CDT>(v[m][j], (CDT == MLA_FP8_E4M3 || CDT == MLA_FP6_E2M3) ? vsc[m] : 1.f);
        }
      lds_barrier();
      if (tb + TT < t1) fetch(tb + TT);  // in flight while this tile is processed
      // scores: one (head, token) pair per thread, four independent partial sums
      for (int i = tid; i < n_h * TT; i += 256) {
        const int h = i / TT, t = i % TT;
        const f32x4* qv = (const f32x4*)(qs + h * rw);
        const f32x4* xv = (const f32x4*)(ts + t * rwp);
        f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int e4 = 0; e4 < rw / 4; ++e4) {
          const f32x4 q = qv[e4], x = xv[e4];
          a4[0] += q[0] * x[0]; a4[1] += q[1] * x[1]; a4[2] += q[2] * x[2]; a4[3] += q[3] * x[3];
        }
        ss[i] = t < valid ? (a4[0] + a4[1]) + (a4[2] + a4[3]) : -__builtin_inff();
      }
      lds_barrier();
      // online softmax: each half-wave takes one head (32 lanes = the tile's 32 tokens), so a
      // round covers 8 heads with 5-step reductions
      for (int h0 = 0; h0 < n_h; h0 += 8) {
        const int h = h0 + 2 * w + (lane >> 5), t = lane & 31;
        if (h < n_h) {
          const float v = ss[h * TT + t];
          float mx = v;
#pragma unroll
          for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
          const float m_old = mrun[h];
          const float m_new = fmaxf(m_old, mx);
          const float e = exp2f(v - m_new);
          float sum = e;
#pragma unroll
          for (int o = 16; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 32);
          ss[h * TT + t] = e;
          if (t == 0) {
            const float a = exp2f(m_old - m_new);
            alf[h] = a;
            lrun[h] = lrun[h] * a + sum;
            mrun[h] = m_new;
          }
        }
      }
      lds_barrier();
      // values: four consecutive columns of one head per thread and group
#pragma unroll
      for (int k = 0; k < OPT4; ++k) {
        const int i4 = tid + 256 * k;
        if (i4 < nout4) {
          const int h = (4 * i4) / d_c, c = 4 * i4 - h * d_c;
          const float a = alf[h];
          f32x4 acc = {O[k][0] * a, O[k][1] * a, O[k][2] * a, O[k][3] * a};
#pragma unroll 4
          for (int t = 0; t < valid; ++t) {
            const float pt = ss[h * TT + t];
            const f32x4 x = *(const f32x4*)(ts + t * rwp + c);
            acc[0] += pt * x[0]; acc[1] += pt * x[1]; acc[2] += pt * x[2]; acc[3] += pt * x[3];
          }
          O[k] = acc;
        }
      }
      lds_barrier();
    }
#pragma unroll
    for (int k = 0; k < OPT4; ++k) {
      const int i4 = tid + 256 * k;
      if (i4 < nout4) {
        const float inv = 1.f / lrun[(4 * i4) / d_c];
        *(f32x4*)(o_part + slot * nout + 4 * i4) = f32x4{O[k][0] * inv, O[k][1] * inv, O[k][2] * inv, O[k][3] * inv};
      }
    }
    for (int h = tid; h < n_h; h += 256)
      lse_part[slot * n_h + h] = (mrun[h] + __log2f(lrun[h])) * 0.69314718055994530942f;
    __syncthreads();
    start = seg_end;
    if (start < end) {
      ++b;
      s0 = s1;
      s1 = s0 + seq_lens[b];
    }
  }
}

// ================================================================================================
// MFMA kernel for a few heads (n_h <= 16; the running model has 8) over 16-bit caches (fp16 or
// bf16 rows of 32*KS elements, d_c = 16*CB). Same equations as above ("DeepSeek-V2 from Scratch"
// section 5.3: scores of the absorbed query against the cached latent rows, softmax, latent-weighted
// sum); with so few heads a tile is little math, so the kernel is organised around the stream of
// rows instead of around the accumulators:
//   - a workgroup of two waves owns a range of tokens; each wave takes every other 32-token tile of
//     the range's segments and keeps its own online softmax, so waves never wait for each other
//     inside the loop (one merge per segment at the end);
//   - each wave copies its tiles straight into its own ring of LDS slots (global->LDS copies, rows
//     padded to an odd number of 16-byte chunks), three tiles in flight;
//   - scores: S^T[16 tok x 16 heads] blocks with MFMA 16x16x32 (rows of the tile as A, the query
//     of the lane's head as B, heads past n_h zero); the accumulator layout gives lane (g, n) the
//     scores of head n for tokens 4g..4g+3 and 16+4g..16+4g+3, which are exactly the eight values
//     the PV product needs from that lane as its B operand (the reduction runs over the tile's
//     tokens in that order), so P never leaves the registers;
//   - PV: O^T[16 columns x 16 heads] += V^T P^T per 16 latent columns, V^T gathered with the
//     transposing 16-bit LDS read (rows 4g.. and 16+4g.. of the lane's column).
// The query is scaled by a power of two per head (its largest element just below 2^14) before it is
// rounded to the 16-bit type, so fp16 neither overflows nor loses precision to small magnitudes;
// the scores are scaled back exactly. Partial outputs are float32 (format 0).
namespace smh {
constexpr int NW = 2;       // waves per workgroup
constexpr int TT = 32;      // tokens per tile
constexpr int NSLOT = 3;    // tile slots per wave
}
template <int KS>
struct SmCfg {
  static constexpr int CH = 4 * KS;                          // 16-byte chunks per cached row
  static constexpr int CHP = CH + 1;                         // padded LDS row stride in chunks (odd)
  static constexpr int NCP = (smh::TT * CHP + 63) / 64;      // copy instructions per tile (1 KB each)
  static constexpr int SLOTB = NCP * 1024;                   // bytes of one tile slot
  static constexpr int RB = CH * 16;                         // bytes of one cached row
};

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int CDT, int KS, int CB, bool PAGED>
__global__ __launch_bounds__(128) void k_decode_small(int n_h, const float* __restrict__ q_lat,
                                                      const float* __restrict__ q_pe, CacheArgs cache,
                                                      const int32_t* __restrict__ seq_lens, int B, int G,
                                                      int64_t* __restrict__ cu_out, int32_t* __restrict__ fmt_out,
                                                      float qscale, float* __restrict__ lse_part,
                                                      float* __restrict__ o_part) {
  using Cfg = SmCfg<KS>;
  using namespace smh;
  constexpr int DC = 16 * CB, DR = 32 * KS - DC, CHP = Cfg::CHP, NCP = Cfg::NCP, SLOTB = Cfg::SLOTB, RB = Cfg::RB;
  static_assert(DR > 0 && DC % 8 == 0, "row split");
  static_assert(NCP - 1 + (NSLOT - 1) * NCP <= 63, "vmcnt range");
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef typename std::conditional<CDT == MLA_F16, h8, bf16x8>::type op8;
  __shared__ __attribute__((aligned(16))) uint8_t lds[NW * NSLOT * SLOTB];
  __shared__ float mw[NW][16], lw[NW][16];
  // the wave index is uniform: kept in a scalar register, so the tile addresses are too
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int p = range_for_block(blockIdx.x, G);
  if (blockIdx.x == 0 && w == 1) write_prefix(seq_lens, B, 0, cu_out, fmt_out, lane);
  const RangeStart rp = locate_range(seq_lens, B, G, p, lane);
  int64_t start = rp.start;
  const int64_t end = rp.end;
  if (start >= end) return;
  int b = rp.b;
  int64_t s0 = rp.s0, s1 = rp.s1;
  uint8_t* const slots = lds + w * NSLOT * SLOTB;
  const uint32_t slots_lds = (uint32_t)(uintptr_t)(MLA_LDS void*)slots;
  const uint8_t* rows_b = (const uint8_t*)cache.rows;

  // copy plan: LDS chunk q = 64 i + lane of a slot holds chunk q % CHP of tile row q / CHP (the pad
  // chunk and the rows past the tile take a harmless duplicate)
  uint32_t plan[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int q = 64 * i + lane, r = q / CHP, c = q % CHP;
    plan[i] = (uint32_t)((r < TT ? r : TT - 1) << 8) | (uint32_t)(c < Cfg::CH ? c : 0);
  }

  while (start < end) {
    if (s1 <= start) {
      ++b;
      s0 = s1;
      s1 = s0 + seq_lens[b];
      continue;
    }
    const int64_t seg_end = end < s1 ? end : s1;
    const int64_t t0 = start - s0, t1 = seg_end - s0;
    const int64_t slot = (int64_t)p + b;
    const int ntiles = (int)((t1 - t0 + TT - 1) / TT);
    const int nk = ntiles > w ? (ntiles - w + NW - 1) / NW : 0;   // this wave's tiles: w, w + NW, ...
    Rows<PAGED> rows;
    rows.init(cache, b);

    // the copies of this wave's k-th tile into slot k % NSLOT (rows past the segment repeat its last row)
    auto issue = [&](int k) __attribute__((always_inline)) {
      const int64_t tt0 = t0 + (int64_t)(w + NW * k) * TT;
      const int last = (int)((t1 - 1 - tt0) < (TT - 1) ? (t1 - 1 - tt0) : (TT - 1));
      const uint32_t dst = __builtin_amdgcn_readfirstlane(slots_lds + (uint32_t)((k % NSLOT) * SLOTB));
      if constexpr (PAGED) rows.tile(tt0, tt0 + last);
      // every earlier LDS read of the slot has completed before it is overwritten
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < NCP; ++i) {
        int r = (int)(plan[i] >> 8);
        r = r < last ? r : last;
        const uint32_t cb16 = (plan[i] & 0xffu) << 4;
        if constexpr (PAGED) {
          dma16(rows_b + rows.row(tt0 + r) * RB + cb16, dst + i * 1024);
        } else {
          dma16_s(rows_b + (rows.base_row + tt0) * RB, (uint32_t)(r * RB) + cb16, dst + i * 1024);
        }
      }
    };

    if (nk > 0) issue(0);
    // query of head n (zero past n_h), dims 32 ks + 8 g .. + 7, times qscale, as 16-bit B fragments
    // scaled by 2^(14 - e_h) (e_h: exponent of the head's largest element)
    f32x4 qv[KS][2];
    float qmax = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      if (n < n_h) {
        const float* src = d0 < DC ? q_lat + ((int64_t)b * n_h + n) * DC + d0 : q_pe + ((int64_t)b * n_h + n) * DR + (d0 - DC);
        qv[ks][0] = *(const f32x4*)src * qscale;
        qv[ks][1] = *(const f32x4*)(src + 4) * qscale;
      } else {
        qv[ks][0] = qv[ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) qmax = fmaxf(qmax, fmaxf(fabsf(qv[ks][0][j]), fabsf(qv[ks][1][j])));
    }
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
    int qe = 0;
    if (qmax > 0.f) (void)frexpf(qmax, &qe);
    const float up = ldexpf(1.f, 14 - qe), down = ldexpf(1.f, qe - 14);
    op8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (j < 4 ? qv[ks][0][j] : qv[ks][1][j - 4]) * up;
        if constexpr (CDT == MLA_F16) qf[ks][j] = (_Float16)x;
        else qf[ks][j] = (__bf16)x;
      }
#pragma unroll
    for (int k = 1; k < NSLOT; ++k)
      if (k < nk) issue(k);

    float m_run = -__builtin_inff(), l_run = 0.f;
    f32x4 O[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) O[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < nk; ++k) {
      // tile k landed (the copies of at most NSLOT - 1 later tiles still in flight)
      const int later = (nk - 1 - k) < (NSLOT - 1) ? (nk - 1 - k) : (NSLOT - 1);
      if (later >= 2) vm_wait<2 * NCP>();
      else if (later == 1) vm_wait<NCP>();
      else vm_wait<0>();
      const uint8_t* tile = slots + (k % NSLOT) * SLOTB;
      const int64_t tt0 = t0 + (int64_t)(w + NW * k) * TT;
      const int valid = (int)((t1 - tt0) < TT ? (t1 - tt0) : TT);
      // scores of tokens 0..15 (S0) and 16..31 (S1): lane (g, n) gets head n, tokens 4g + r
      f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const op8 a0 = *(const op8*)(tile + (n * CHP + 4 * ks + g) * 16);
        const op8 a1 = *(const op8*)(tile + ((16 + n) * CHP + 4 * ks + g) * 16);
        if constexpr (CDT == MLA_F16) {
          S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qf[ks], S0, 0, 0, 0);
          S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qf[ks], S1, 0, 0, 0);
        } else {
          S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], S0, 0, 0, 0);
          S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], S1, 0, 0, 0);
        }
      }
      float tm = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        S0[r] = 4 * g + r < valid ? S0[r] * down : -__builtin_inff();
        S1[r] = 16 + 4 * g + r < valid ? S1[r] * down : -__builtin_inff();
        tm = fmaxf(tm, fmaxf(S0[r], S1[r]));
      }
      tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
      tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
      const float m_new = fmaxf(m_run, tm);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float rs = 0.f;
      op8 pf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e0 = __builtin_amdgcn_exp2f(S0[r] - m_new), e1 = __builtin_amdgcn_exp2f(S1[r] - m_new);
        rs += e0 + e1;
        if constexpr (CDT == MLA_F16) { pf[r] = (_Float16)e0; pf[4 + r] = (_Float16)e1; }
        else { pf[r] = (__bf16)e0; pf[4 + r] = (__bf16)e1; }
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run = l_run * alpha + rs;
      m_run = m_new;
      // V^T of the lane's column 16 cb + n: rows 4g + 0..3 and 16 + 4g + 0..3 (transposing reads:
      // lane j of each 16-lane group supplies row j / 4, columns 4 (j % 4) .. + 3 of the block)
      const uint8_t* va = tile + (4 * g + (n >> 2)) * CHP * 16 + (n & 3) * 8;
      const uint8_t* vb = va + 16 * CHP * 16;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(uintptr_t)(uint32_t)(uintptr_t)(MLA_LDS void*)(va + 32 * cb));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(uintptr_t)(uint32_t)(uintptr_t)(MLA_LDS void*)(vb + 32 * cb));
        const op8 av = __builtin_bit_cast(op8, u32x4{__builtin_bit_cast(u32x2, x0).x, __builtin_bit_cast(u32x2, x0).y,
                                                     __builtin_bit_cast(u32x2, x1).x, __builtin_bit_cast(u32x2, x1).y});
        const f32x4 o = O[cb] * alpha;
        if constexpr (CDT == MLA_F16) O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pf, o, 0, 0, 0);
        else O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pf, o, 0, 0, 0);
      }
      if (k + NSLOT < nk) issue(k + NSLOT);
    }

    // merge the waves: O of wave w (head n, columns 16 cb + 4 g + r) to its own slots, then every
    // thread combines four consecutive columns of one head
    __syncthreads();  // both waves are past their last tile reads
    float* ow = (float*)slots;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) *(f32x4*)(ow + n * DC + 16 * cb + 4 * g) = O[cb];
    if (g == 0) {
      mw[w][n] = m_run;
      lw[w][n] = l_run;
    }
    __syncthreads();
    for (int i4 = tid; i4 < n_h * DC / 4; i4 += 64 * NW) {
      const int h = (4 * i4) / DC, c = 4 * i4 - h * DC;
      float M = -__builtin_inff();
#pragma unroll
      for (int v = 0; v < NW; ++v) M = fmaxf(M, mw[v][h]);
      float L = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const float wt = __builtin_amdgcn_exp2f(mw[v][h] - M);
        L += wt * lw[v][h];
        acc += *(const f32x4*)((const float*)(lds + v * NSLOT * SLOTB) + h * DC + c) * wt;
      }
      *(f32x4*)(o_part + (slot * n_h + h) * DC + c) = acc * (1.f / L);
      if (c == 0) lse_part[slot * n_h + h] = (M + __log2f(L)) * 0.69314718055994530942f;
    }
    __syncthreads();  // the slots are reused by the next segment

    start = seg_end;
    if (start < end) {
      ++b;
      s0 = s1;
      s1 = s0 + seq_lens[b];
    }
  }
}

// ================================================================================================
// Combine: per sequence, merge the pieces of the ranges that cover it. One block = one sequence
// and CH heads; the piece list and the per-(piece, head) weights exp(lse_s - M) / sum are built
// once in LDS, then every output element is a weighted sum over the pieces (fixed order).
// Partial outputs are float32 (generic kernel, format 0) or float16 rows with a power-of-two
// scale per (piece, head) (MFMA kernel, format 2), as the format word says; the scale is folded
// into the piece weights.
namespace cmb {
constexpr int CH = 8;        // most heads per block
}

__device__ __forceinline__ f32x4 load4(const float* p, int64_t i) { return ((const f32x4*)p)[i]; }
__device__ __forceinline__ f32x4 load4(const _Float16* p, int64_t i) {
  typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_convertvector(((const f16x4_t*)p)[i], f32x4);
}

// Weighted sum over the pieces. With ng = nh * d_c / 4 output groups of 4 elements:
//  - ng >= 256: every thread owns up to 4 groups per round and issues the loads of 4 pieces
//    before accumulating them;
//  - ng < 256 (few heads per block, many pieces): psplit = 256 / ng threads share a group, thread
//    part q takes pieces q, q + psplit, ..., and the parts are added through LDS in order q.
// Either way the order of the sum is fixed for a given launch shape (deterministic).
// The block covers columns [c0, c0 + dcc) of heads h0 .. h0 + nh - 1 (dcc < d_c only with nh = 1).
template <typename PT>
__device__ __forceinline__ void combine_sum(const PT* __restrict__ o_part, int n_h, int d_c, int h0, int nh,
                                            int c0, int dcc, int np, const int* slots,
                                            const float* wts, int ws, float* dst, f32x4* red) {
  const int tid = threadIdx.x;
  const int nv4 = nh * dcc / 4;
  const int d_c_ = dcc;  // row width seen by the group -> head mapping below
  const PT* src = o_part + (int64_t)h0 * d_c + c0;
  const int64_t pstride = (int64_t)n_h * d_c / 4;  // 4-element groups per piece slot
  f32x4* dst4 = (f32x4*)dst;
  if (nv4 < 256) {
    const int psplit = 256 / nv4;
    const int grp = tid % nv4, part = tid / nv4;
    const float* wcol = wts + grp * 4 / d_c_;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (part < psplit) {
      int i = part;
      for (; i + 3 * psplit < np; i += 4 * psplit) {
        f32x4 x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = load4(src, (int64_t)slots[i + k * psplit] * pstride + grp);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float wk = wcol[(i + k * psplit) * ws];
          acc[0] += wk * x[k][0]; acc[1] += wk * x[k][1]; acc[2] += wk * x[k][2]; acc[3] += wk * x[k][3];
        }
      }
      for (; i < np; i += psplit) {
        const f32x4 x = load4(src, (int64_t)slots[i] * pstride + grp);
        const float wk = wcol[i * ws];
        acc[0] += wk * x[0]; acc[1] += wk * x[1]; acc[2] += wk * x[2]; acc[3] += wk * x[3];
      }
      red[tid] = acc;
    }
    __syncthreads();
    if (part == 0) {
      for (int q = 1; q < psplit; ++q) {
        const f32x4 y = red[q * nv4 + grp];
        acc[0] += y[0]; acc[1] += y[1]; acc[2] += y[2]; acc[3] += y[3];
      }
      dst4[grp] = acc;
    }
    return;
  }
  for (int e0 = 0; e0 < nv4; e0 += 1024) {
    int idx[4];
    f32x4 acc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      idx[v] = e0 + tid + 256 * v;
      acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int i = 0;
    for (; i + 4 <= np; i += 4) {
      f32x4 x[4][4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          x[k][v] = idx[v] < nv4 ? load4(src, (int64_t)slots[i + k] * pstride + idx[v]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float wk = wts[(i + k) * ws + (idx[v] < nv4 ? idx[v] : 0) * 4 / d_c_];
          acc[v][0] += wk * x[k][v][0]; acc[v][1] += wk * x[k][v][1];
          acc[v][2] += wk * x[k][v][2]; acc[v][3] += wk * x[k][v][3];
        }
    }
    for (; i < np; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (idx[v] >= nv4) continue;
        const f32x4 x = load4(src, (int64_t)slots[i] * pstride + idx[v]);
        const float wk = wts[i * ws + idx[v] * 4 / d_c_];
        acc[v][0] += wk * x[0]; acc[v][1] += wk * x[1]; acc[v][2] += wk * x[2]; acc[v][3] += wk * x[3];
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (idx[v] < nv4) dst4[idx[v]] = acc[v];
  }
}

// Dynamic LDS: slots[G] (piece slot of each range of the sequence, in range order), then lse and
// scale of every (piece, head) and finally the weights, ch floats per piece each. A sequence is
// covered by at most G ranges, so G entries always suffice.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_combine(int n_h, int d_c, int ch, int dcc, const int64_t* __restrict__ cu, int B, int G,
                                                 const int32_t* __restrict__ fmt,
                                                 const float* __restrict__ lse_part,
                                                 const float* __restrict__ sc_part,
                                                 const void* __restrict__ o_part, float* __restrict__ o_lat,
                                                 float* __restrict__ lse_out) {
  extern __shared__ float dyn[];
  __shared__ f32x4 red[256];
  __shared__ int sh_np;
  int* slots = (int*)dyn;
  float* lse_s = dyn + G;
  float* sc_s = lse_s + (int64_t)G * ch;
  float* wts = lse_s;  // the weights overwrite the lse values in place
  const int b = blockIdx.y;
  const int h0 = blockIdx.x * ch;
  const int nh = (n_h - h0) < ch ? (n_h - h0) : ch;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t total = cu[B];
  const int64_t s0 = cu[b], s1 = cu[b + 1];
  const int c0 = blockIdx.z * dcc;
  const bool f16 = *fmt == 2;
  float* dst = o_lat + ((int64_t)b * n_h + h0) * d_c + c0;
  if (s1 <= s0) {  // empty sequence (outside the contract): defined output
    for (int e = tid; e < nh * dcc; e += 256) dst[(e / dcc) * d_c + e % dcc] = 0.f;
    if (lse_out && tid < nh && blockIdx.z == 0) lse_out[(int64_t)b * n_h + h0 + tid] = -__builtin_inff();
    return;
  }
  if (w == 0) {  // piece list, in range order: one candidate range per lane, compacted by ballot
    const int64_t plo = range_of(s0, total, G), phi = range_of(s1 - 1, total, G);
    int np = 0;
    for (int64_t p0 = plo; p0 <= phi && np < G; p0 += 64) {
      const int64_t p = p0 + lane;
      const bool keep = p <= phi && range_start(p, total, G) != range_start(p + 1, total, G);
      const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
      const int pos = np + (int)__builtin_popcountll(m & ((1ull << lane) - 1));
      if (keep && pos < G) slots[pos] = (int)(p + b);
      np += (int)__builtin_popcountll(m);
    }
    if (lane == 0) sh_np = np < G ? np : G;
  }
  __syncthreads();
  const int np = sh_np;
  // Fast path for float16 partials and a block of 4096 outputs (two 8-element groups per
  // thread): the rows of the first PF pieces are requested before the weights are built, so that
  // their latency overlaps the lse loads.
  constexpr int PF = 4;
  const bool fast = f16 && nh * dcc == 4096;
  const _Float16* srcp = (const _Float16*)o_part + (int64_t)h0 * d_c + c0;
  const int64_t pst = (int64_t)n_h * d_c;
  // every (piece, head) lse and scale, loaded by the whole block in one pass; then the weights
  auto build_weights = [&]() __attribute__((always_inline)) {
    for (int e = tid; e < np * nh; e += 256) {
      const int i = e / nh, hh = e - i * nh;
      const int64_t r = (int64_t)slots[i] * n_h + h0 + hh;
      lse_s[i * ch + hh] = lse_part[r];
      sc_s[i * ch + hh] = f16 ? sc_part[r] : 1.f;
    }
    __syncthreads();
    // weights: wave w handles heads w, w+4, ...
    for (int hh = w; hh < nh; hh += 4) {
      float M = -__builtin_inff();
      for (int i = lane; i < np; i += 64) M = fmaxf(M, lse_s[i * ch + hh]);
      M = wave_max(M);
      float sum = 0.f;
      for (int i = lane; i < np; i += 64) sum += __expf(lse_s[i * ch + hh] - M);
      sum = wave_sum(sum);
      const float inv = 1.f / sum;
      for (int i = lane; i < np; i += 64) wts[i * ch + hh] = __expf(lse_s[i * ch + hh] - M) * inv * sc_s[i * ch + hh];
      if (lse_out && lane == 0 && blockIdx.z == 0) lse_out[(int64_t)b * n_h + h0 + hh] = M + __logf(sum);
    }
    __syncthreads();
  };
  if (fast) {  // same order of the sum as combine_sum: piece by piece
    const int npf = np < PF ? np : PF;
    int off[2], hhv[2];
    f16x8 xp[PF][2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int e = 8 * (tid + 256 * v);
      hhv[v] = e / dcc;
      off[v] = hhv[v] * d_c + (e - hhv[v] * dcc);
    }
#pragma unroll
    for (int k = 0; k < PF; ++k)
      if (k < npf) {
        const int64_t sb = (int64_t)slots[k] * pst;
#pragma unroll
        for (int v = 0; v < 2; ++v) xp[k][v] = *(const f16x8*)(srcp + sb + off[v]);
      }
    build_weights();
    f32x4 acc[2][2] = {};
    auto add = [&](int k, int v, const f16x8& x) __attribute__((always_inline)) {
      const float wk = wts[k * ch + hhv[v]];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[v][0][j] += wk * (float)x[j];
        acc[v][1][j] += wk * (float)x[4 + j];
      }
    };
#pragma unroll
    for (int k = 0; k < PF; ++k)
      if (k < npf) {
#pragma unroll
        for (int v = 0; v < 2; ++v) add(k, v, xp[k][v]);
      }
    for (int k = PF; k < np; ++k) {
      const int64_t sb = (int64_t)slots[k] * pst;
#pragma unroll
      for (int v = 0; v < 2; ++v) add(k, v, *(const f16x8*)(srcp + sb + off[v]));
    }
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      *(f32x4*)(dst + off[v]) = acc[v][0];
      *(f32x4*)(dst + off[v] + 4) = acc[v][1];
    }
    return;
  }
  build_weights();
  if (f16) combine_sum((const _Float16*)o_part, n_h, d_c, h0, nh, c0, dcc, np, slots, wts, ch, dst, red);
  else combine_sum((const float*)o_part, n_h, d_c, h0, nh, c0, dcc, np, slots, wts, ch, dst, red);
}

// ================================================================================================
// Combine fused with the per-head value up-projection ("DeepSeek-V2 from Scratch" section 4.4 for
// the softmax regrouped over pieces, section 5.2 for o_i = W^UV_i o_lat_i): workgroup = (head i,
// 32 sequences). It merges the pieces of its sequences for head i alone (o_lat_i never goes to
// HBM) and multiplies by W^UV_i on MFMA, writing o [B, n_h d_h] float32 for the W^O product.
//   phase 0: every wave requests its 32 rows of W^UV_i as A fragments (32 k-steps of 16, kept in
//            registers), so the weight read overlaps the combine;
//   phase 1: lane j of wave 0 lists the pieces of sequence j;
//   phase 2: 8 threads per sequence request the pieces' rows, lse and scales together, form the
//            weights (as k_combine) and sum the rows (piece by piece) into LDS as bf16 hi/lo;
//   phase 3: D[e][b] = sum_c W^UV_i[e][c] o_lat_i[b][c] on 32x32x16 bf16 MFMA, hi then lo part,
//            written as bf16 (the W^O product then runs one MFMA per step on half the bytes).
namespace cuv {
constexpr int DC = 512, DH = 128, SB = 32;   // d_c, d_h, sequences per workgroup
constexpr int PITCH = DC + 8;                // bf16 elements per o_lat row in LDS
constexpr int MAXP = 1024 + SB;              // pieces of SB sequences: at most G + SB - 1
}
__global__ __launch_bounds__(256, 1) void k_combine_uv(int n_h, int B, int G, int ntiles, const int64_t* __restrict__ cu,
                                                       const int32_t* __restrict__ fmt,
                                                       const float* __restrict__ lse_part,
                                                       const float* __restrict__ sc_part, const void* __restrict__ o_part,
                                                       const uint16_t* __restrict__ W_uv, uint16_t* __restrict__ o,
                                                       float* __restrict__ lse_out) {
  using namespace cuv;
  __shared__ __attribute__((aligned(16))) uint16_t hi[SB * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t lo[SB * PITCH];
  __shared__ int slots[MAXP];
  __shared__ int pbeg[SB + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // tile t = head * nslices + slice; consecutive tiles (the slices of one head, sharing W^UV_i)
  // go to one XCD (workgroups are dealt round-robin to the 8 XCDs)
  const int t = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
  if (t >= ntiles) return;
  const int nsl = (B + SB - 1) / SB;
  const int i = t / nsl, sl = t - i * nsl;
  const int b0 = sl * SB;
  const int l32 = lane & 31, g = lane >> 5;

  // phase 0: A fragments of rows 32 w + l32 of W^UV_i, k = 16 ks + 8 g .. + 7
  bf16x8 a[DC / 16];
  const uint16_t* wrow = W_uv + ((int64_t)i * DH + 32 * w + l32) * DC + 8 * g;
#pragma unroll
  for (int ks = 0; ks < DC / 16; ++ks) a[ks] = *(const bf16x8*)(wrow + 16 * ks);

  // phase 1: the piece list of each sequence (lane j of wave 0 owns sequence b0 + j)
  const bool f16 = *fmt == 2;
  const int64_t total = cu[B];
  if (w == 0) {
    int np = 0;
    int64_t plo = 0, phi = -1;
    const int b = b0 + lane;
    if (lane < SB && b < B) {
      const int64_t s0 = cu[b], s1 = cu[b + 1];
      if (s1 > s0) {
        plo = range_of(s0, total, G);
        phi = range_of(s1 - 1, total, G);
        for (int64_t p = plo; p <= phi; ++p) np += range_start(p, total, G) != range_start(p + 1, total, G);
      }
    }
    // exclusive prefix of np over the 32 sequences
    int incl = np;
#pragma unroll
    for (int o2 = 1; o2 < 32; o2 <<= 1) {
      const int x = __shfl_up(incl, o2, 64);
      if ((lane & 31) >= o2) incl += x;
    }
    const int beg = incl - np;
    if (lane < SB) pbeg[lane] = beg < MAXP ? beg : MAXP;
    if (lane == SB - 1) pbeg[SB] = incl < MAXP ? incl : MAXP;
    if (lane < SB) {
      int k = beg;
      for (int64_t p = plo; p <= phi; ++p)
        if (range_start(p, total, G) != range_start(p + 1, total, G) && k < MAXP) slots[k++] = (int)(p + b);
    }
  }
  __syncthreads();

  // phase 2: thread (j = tid / 8, u = tid % 8) sums columns 64 k + 8 u .. + 7 (k = 0..7) of
  // sequence b0 + j's pieces with their softmax weights exp(lse - M) / sum * scale (every thread
  // of the sequence forms them itself); a sequence past the batch or with no pieces gives zeros.
  // Up to PF pieces (every sequence at the decode batch sizes): their rows, lse and scales are all
  // requested at once; more pieces take a two-pass loop.
  {
    constexpr int PF = 6;
    const int j = tid >> 3, u = tid & 7;
    const int q0 = pbeg[j], np = pbeg[j + 1] - q0;
    f32x4 acc[8][2];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k][0] = acc[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t pst = (int64_t)n_h * DC;
    const _Float16* ph = (const _Float16*)o_part + (int64_t)i * DC + 8 * u;
    const float* pf32 = (const float*)o_part + (int64_t)i * DC + 8 * u;
    auto add16 = [&](float wk, const f16x8 (&x)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[k][0][e] += wk * (float)x[k][e];
          acc[k][1][e] += wk * (float)x[k][4 + e];
        }
    };
    auto add_row = [&](float wk, int slot) __attribute__((always_inline)) {
      if (f16) {
        f16x8 x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = *(const f16x8*)(ph + (int64_t)slot * pst + 64 * k);
        add16(wk, x);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float* src = pf32 + (int64_t)slot * pst + 64 * k;
          acc[k][0] += wk * *(const f32x4*)src;
          acc[k][1] += wk * *(const f32x4*)(src + 4);
        }
      }
    };
    float M = -__builtin_inff(), sum = 0.f;
    if (f16 && np <= PF) {
      f16x8 x[PF][8];
      float lv[PF], sv[PF];
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        const int slot = q < np ? slots[q0 + q] : 0;
        lv[q] = q < np ? lse_part[(int64_t)slot * n_h + i] : -__builtin_inff();
        sv[q] = q < np ? sc_part[(int64_t)slot * n_h + i] : 0.f;
        if (q < np) {
#pragma unroll
          for (int k = 0; k < 8; ++k) x[q][k] = *(const f16x8*)(ph + (int64_t)slot * pst + 64 * k);
        }
      }
#pragma unroll
      for (int q = 0; q < PF; ++q) M = fmaxf(M, lv[q]);
#pragma unroll
      for (int q = 0; q < PF; ++q)
        if (q < np) sum += __expf(lv[q] - M);
      const float inv = 1.f / sum;
#pragma unroll
      for (int q = 0; q < PF; ++q)
        if (q < np) add16(__expf(lv[q] - M) * inv * sv[q], x[q]);
    } else {
      for (int q = 0; q < np; ++q) M = fmaxf(M, lse_part[(int64_t)slots[q0 + q] * n_h + i]);
      for (int q = 0; q < np; ++q) sum += __expf(lse_part[(int64_t)slots[q0 + q] * n_h + i] - M);
      const float inv = 1.f / sum;
      for (int q = 0; q < np; ++q) {
        const int64_t r = (int64_t)slots[q0 + q] * n_h + i;
        add_row(__expf(lse_part[r] - M) * inv * (f16 ? sc_part[r] : 1.f), slots[q0 + q]);
      }
    }
    if (lse_out && u == 0 && b0 + j < B) lse_out[(int64_t)(b0 + j) * n_h + i] = np > 0 ? M + __logf(sum) : -__builtin_inff();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      bf16x8 bh, bl;
      split_hi_lo(acc[k][0], acc[k][1], bh, bl);
      const int off = j * PITCH + 64 * k + 8 * u;
      *(bf16x8*)(hi + off) = bh;
      *(bf16x8*)(lo + off) = bl;
    }
  }
  __syncthreads();

  // phase 3: D[e = 32 w + row][b = l32], B operand column l32, k = 16 ks + 8 g .. + 7
  f32x16 D = {};
  const int boff = l32 * PITCH + 8 * g;
#pragma unroll
  for (int ks = 0; ks < DC / 16; ++ks) {
    const bf16x8 bh = *(const bf16x8*)(hi + boff + 16 * ks);
    const bf16x8 bl = *(const bf16x8*)(lo + boff + 16 * ks);
    D = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bh, D, 0, 0, 0);
    D = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bl, D, 0, 0, 0);
  }
  // element r of lane (g, l32): row 8 (r / 4) + 4 g + r % 4, column l32
  const int b = b0 + l32;
  if (b < B) {
    uint16_t* dst = o + (int64_t)b * n_h * DH + (int64_t)i * DH + 32 * w + 4 * g;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *(u32x2*)(dst + 8 * r4) = u32x2{pack_bf16x2(D[4 * r4], D[4 * r4 + 1]), pack_bf16x2(D[4 * r4 + 2], D[4 * r4 + 3])};
  }
}

// ================================================================================================
static bool is_v2(const mla_dims& d) { return d.n_h == v2::NH && d.d_c == v2::DC && d.d_r == v2::DR; }
static bool v2_page_ok(int ps) { return ps == 0 || (ps >= 32 && (ps & (ps - 1)) == 0); }

// the few-head MFMA kernel: the running model's row split (d_c = 128, d_r = 32) over 16-bit caches
static bool small_shape(const mla_dims& d, int cdt, int page_size) {
  return d.n_h <= 16 && d.d_c == 128 && d.d_r == 32 && (cdt == MLA_F16 || cdt == MLA_BF16) && v2_page_ok(page_size);
}

bool decode_supported(const mla_dims& d, int cdt, int page_size) {
  if (is_v2(d) && (cdt == MLA_BF16 || cdt == MLA_FP8_E4M3 || cdt == MLA_FP6_E2M3)) return v2_page_ok(page_size);
  if (small_shape(d, cdt, page_size)) return true;
  const int rw = d.d_c + d.d_r;
  return d.n_h * rw <= 16384 && rw <= 512 && d.n_h <= 64 && d.n_h * d.d_c <= 256 * gen::OPT;
}

hipError_t launch_decode(const mla_dims& d, int B, const float* q_lat, const float* q_pe,
                         const CacheArgs& c, const int32_t* seq_lens, int G, float sm_scale,
                         void* ws, hipStream_t st) {
  if (!decode_supported(d, c.dtype, c.page_size)) return hipErrorNotSupported;
  DecodeLayout L = decode_layout(d, B, G);
  char* base = (char*)ws;
  int64_t* cu = (int64_t*)(base + L.off_cu);
  int32_t* fmt = (int32_t*)(base + L.off_fmt);
  float* lse_part = (float*)(base + L.off_lse);
  float* o_part = (float*)(base + L.off_o);
  const bool mfma = is_v2(d) && (c.dtype == MLA_BF16 || c.dtype == MLA_FP8_E4M3 || c.dtype == MLA_FP6_E2M3);
  const float qscale = sm_scale * 1.44269504088896340736f;  // log2(e)
  if (mfma) {
    const bool paged = c.page_size > 0;
#define MLA_FP8(PG, F6) \
    hipLaunchKernelGGL((k_decode_fp8<PG, F6>), dim3(G), dim3(256), 0, st, qop, fhv, c, seq_lens, B, G, cu, fmt, \
                       lse_part, (float*)(base + L.off_sc), (uint16_t*)o_part)
#define MLA_V3(PG) \
    hipLaunchKernelGGL((k_decode_v3<PG>), dim3(G), dim3(256), 0, st, qop, c, seq_lens, B, G, cu, fmt, \
                       lse_part, (float*)(base + L.off_sc), (uint16_t*)o_part)
    uint8_t* qop = (uint8_t*)(base + L.off_q8);
    float* fhv = (float*)(base + L.off_fh);
    if (c.dtype == MLA_BF16) {
      hipLaunchKernelGGL(k_qprep<false>, dim3(B * 16), dim3(256), 0, st, q_lat, q_pe, qscale, qop, fhv);
      if (paged) MLA_V3(true); else MLA_V3(false);
    } else {
      hipLaunchKernelGGL(k_qprep<true>, dim3(B * 16), dim3(256), 0, st, q_lat, q_pe, qscale, qop, fhv);
      if (c.dtype == MLA_FP6_E2M3) {
        if (paged) MLA_FP8(true, true); else MLA_FP8(false, true);
      } else {
        if (paged) MLA_FP8(true, false); else MLA_FP8(false, false);
      }
    }
#undef MLA_FP8
#undef MLA_V3
  } else if (small_shape(d, c.dtype, c.page_size)) {
    const bool paged = c.page_size > 0;
#define MLA_SMALL(CDT, PG)                                                                                    \
    hipLaunchKernelGGL((k_decode_small<CDT, 5, 8, PG>), dim3(G), dim3(64 * smh::NW), 0, st, d.n_h, q_lat, q_pe, c, \
                       seq_lens, B, G, cu, fmt, qscale, lse_part, o_part)
    if (c.dtype == MLA_F16) { if (paged) MLA_SMALL(MLA_F16, true); else MLA_SMALL(MLA_F16, false); }
    else { if (paged) MLA_SMALL(MLA_BF16, true); else MLA_SMALL(MLA_BF16, false); }
#undef MLA_SMALL
  } else {
    const int rw = d.d_c + d.d_r;
    size_t smem = (size_t)(d.n_h * rw + gen::TT * (rw + 4) + d.n_h * gen::TT + 3 * d.n_h) * 4;
    const bool paged = c.page_size > 0;
    const bool narrow = rw <= 192;  // running-model rows (160 elements)
#define MLA_GEN(CDT, EPL, PG)                                                                              \
  hipLaunchKernelGGL((k_decode_generic<CDT, EPL, PG>), dim3(G), dim3(256), smem, st, d.n_h, d.d_c, d.d_r, q_lat, q_pe, \
                     c, seq_lens, B, G, cu, fmt, qscale, lse_part, o_part)
#define MLA_GEN_DT(CDT)                                    \
  if (narrow) { if (paged) MLA_GEN(CDT, 3, true); else MLA_GEN(CDT, 3, false); } \
  else { if (paged) MLA_GEN(CDT, 8, true); else MLA_GEN(CDT, 8, false); }
    switch (c.dtype) {
      case MLA_F32: MLA_GEN_DT(MLA_F32); break;
      case MLA_F16: MLA_GEN_DT(MLA_F16); break;
      case MLA_BF16: MLA_GEN_DT(MLA_BF16); break;
      case MLA_FP6_E2M3: MLA_GEN_DT(MLA_FP6_E2M3); break;
      default: MLA_GEN_DT(MLA_FP8_E4M3); break;
    }
#undef MLA_GEN_DT
#undef MLA_GEN
  }
  return hipGetLastError();
}

hipError_t launch_combine(const mla_dims& d, int B, int G, const void* ws, float* o_lat, float* lse,
                          hipStream_t st) {
  DecodeLayout L = decode_layout(d, B, G);
  const char* base = (const char*)ws;
  // heads per block: up to CH, fewer when the batch is small, so that about 1024 blocks run
  int ch = (int)(((int64_t)B * d.n_h) / 1024);
  ch = ch < 1 ? 1 : (ch > cmb::CH ? cmb::CH : ch);
  while (ch > 1 && (size_t)G * (4 + 8 * (size_t)ch) > 60 * 1024) --ch;  // dynamic LDS below 60 KB
  // with one head per block and still few blocks, the columns are split too (chunks of >= 64)
  int nchunk = 1;
  if (ch == 1) {
    const int64_t nb = (int64_t)B * d.n_h;
    while (nb * nchunk * 2 <= 1024 && d.d_c % (nchunk * 2 * 4) == 0 && d.d_c / (nchunk * 2) >= 64) nchunk *= 2;
  }
  dim3 grid((unsigned)((d.n_h + ch - 1) / ch), B, nchunk);
  const size_t smem = (size_t)G * (4 + 8 * (size_t)ch);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), smem, st, d.n_h, d.d_c, ch, d.d_c / nchunk, (const int64_t*)(base + L.off_cu), B, G,
                     (const int32_t*)(base + L.off_fmt), (const float*)(base + L.off_lse),
                     (const float*)(base + L.off_sc), (const void*)(base + L.off_o), o_lat, lse);
  return hipGetLastError();
}

bool combine_uv_supported(const mla_dims& d, int G) {
  return d.d_c == cuv::DC && d.d_h == cuv::DH && G + cuv::SB - 1 <= cuv::MAXP;
}

hipError_t launch_combine_uv(const mla_dims& d, int B, int G, const void* ws, const void* W_uv, void* o, float* lse,
                             hipStream_t st) {
  if (!combine_uv_supported(d, G)) return hipErrorNotSupported;
  DecodeLayout L = decode_layout(d, B, G);
  const char* base = (const char*)ws;
  const int ntiles = d.n_h * ((B + cuv::SB - 1) / cuv::SB);
  hipLaunchKernelGGL(k_combine_uv, dim3((unsigned)((ntiles + 7) & ~7)), dim3(256), 0, st, d.n_h, B, G, ntiles,
                     (const int64_t*)(base + L.off_cu), (const int32_t*)(base + L.off_fmt),
                     (const float*)(base + L.off_lse), (const float*)(base + L.off_sc), (const void*)(base + L.off_o),
                     (const uint16_t*)W_uv, (uint16_t*)o, lse);
  return hipGetLastError();
}

}  // namespace mla
