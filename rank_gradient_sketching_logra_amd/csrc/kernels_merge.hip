// Merge of the low-rank update into the weights: W <- round(W - s U A).
//
// Sources: "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches" (paperpeel.com) §2.1 (W <- W - alpha eta U A) and §2.2 (merged
// directly into the weights, no adapter; the rollout side regenerates A from
// its seed and applies the received alpha eta U).  "Randomized Gradient
// Compression" blog, "How it works": bf16 weights updated in place with
// stochastic rounding, the update rebuilt a block of rows at a time and never
// held whole.
//
// bf16 W runs on v_mfma_f32_32x32x16_bf16 with the product transposed:
// for a 32-row band of W, instance e of a wave computes
// C[m][n] = sum over ranks of sigma[rank][col(m, e)] * U[row n][rank], with
// U split into bf16 hi + lo (two MFMAs per 16-rank step) and sigma exact in
// bf16.  Lane l holds C[m][n = l & 31] for m = 8(j>>2) + 4(l>>5) + (j&3),
// j = 0..15, and the columns are assigned so that those sixteen values are
// sixteen consecutive columns of one W row.  Interior tiles of W pass
// through LDS: each 32-row band is loaded with direct global->LDS copies of
// whole row segments (the lane-to-chunk order permuted so that the LDS tile
// is swizzled and the matrix-side reads do not collide in banks), updated in
// place in LDS, and written back with whole-row stores.  Every element's sum
// runs over rank steps in ascending order, hi then lo, whatever the row or
// block position, so a merge of a row block equals the same rows of a
// whole-matrix merge; the sixteen stochastic-rounding draws of a lane's
// elements come from two Philox4x32 blocks when k is a multiple of 16.
#include "device_common.h"
#include "kernels.h"

#include <atomic>

namespace logra {

namespace {

// Two bf16 bit patterns, the operand and result type of v_cvt_sr_bf16_f32.
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// Sixteen bf16 of W row `row` from column c (two 16-byte words); zero
// outside the matrix.
__device__ __forceinline__ void load_w16(const uint16_t* __restrict__ W, int64_t ldw,
                                         int64_t d, int64_t k, int64_t row, int64_t c,
                                         u32x4& w0, u32x4& w1) {
  if (row < d && c + 16 <= k) {
    const u32x4* p = reinterpret_cast<const u32x4*>(W + row * ldw + c);
    w0 = p[0];
    w1 = p[1];
    return;
  }
  uint32_t e[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) e[i] = (row < d && c + i < k) ? W[row * ldw + c + i] : 0u;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    w0[p] = e[2 * p] | (e[2 * p + 1] << 16);
    w1[p] = e[8 + 2 * p] | (e[8 + 2 * p + 1] << 16);
  }
}

// Whether any of sixteen values is NaN: their sum is NaN whenever one of
// them is (and also for +inf beside -inf, which only costs a pass that finds
// nothing).  Timed faster than unordered compares of pairs.
__device__ __forceinline__ bool any_nan16(const float (&v)[16]) {
  float sum = v[0];
#pragma unroll
  for (int t = 1; t < 16; ++t) sum += v[t];
  return __builtin_isnan(sum);
}

// Sixteen updated bf16 of one lane: W values w (two words), products
// acc[0..15] of consecutive columns, element index e0 of the first (for the
// stochastic-rounding draws).  aligned: e0 is a multiple of 16, so the
// sixteen draws are exactly two generator blocks, element t taking bits
// [16 (t & 1), +16) of word (t & 7) >> 1 of block t >> 3.  PRE (aligned
// only): the two blocks were generated earlier by the caller, in pre.
template <bool STOCH, bool PRE = false>
__device__ __forceinline__ void update16(const u32x4& w0, const u32x4& w1, const f32x16& acc,
                                         float sc, KeyWords srk, uint64_t e0, bool aligned,
                                         u32x4& o0, u32x4& o1, const u32x4* pre = nullptr) {
  uint32_t out[8];
  auto value = [&](int t) __attribute__((always_inline)) {
    const uint32_t word = (t < 8) ? w0[t >> 1] : w1[(t - 8) >> 1];
    const uint32_t wbits = (t & 1) ? (word >> 16) : (word & 0xFFFFu);
    return __builtin_fmaf(-sc, acc[t], bf16_bits_to_f32(wbits));
  };
  auto put = [&](int t, uint32_t o) __attribute__((always_inline)) {
    if (t & 1)
      out[t >> 1] = (out[t >> 1] & 0xFFFFu) | (o << 16);
    else
      out[t >> 1] = (out[t >> 1] & 0xFFFF0000u) | o;
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = 0u;
  if constexpr (!STOCH) {
    // The hardware conversion keeps a NaN's (quieted) payload; a NaN is
    // returned as the quiet NaN of its sign, as in the stochastic path.
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = value(t);
#pragma unroll
    for (int t = 0; t < 16; ++t) put(t, (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[t]));
    if (any_nan16(v)) {
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (__builtin_isnan(v[t])) put(t, f32_to_bf16_rne(v[t]));
    }
  } else if (aligned) {
    // v_cvt_sr_bf16_f32 adds the high 16 bits of its second operand to the
    // discarded half of the fp32 pattern and truncates: the rule above for
    // every non-NaN value (infinity stays infinity, overflow lands on it).  So
    // an odd element takes its generator word as it is (its draw is the high
    // half) and an even one the word shifted up by 16; the two results of a
    // pair fill the halves of one output word.  NaN is the one case the
    // instruction rounds differently: when any of the sixteen values is NaN,
    // the NaN elements take the quiet NaN of their sign.
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = value(t);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t pw[4];
      if constexpr (PRE) {
#pragma unroll
        for (int q = 0; q < 4; ++q) pw[q] = pre[h][q];
      } else {
        const Philox4x32 p = sr_block(srk, (e0 >> 3) + h);
#pragma unroll
        for (int q = 0; q < 4; ++q) pw[q] = p.w[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // both halves are written, so pk may start as any value
        s16x2 pk = __builtin_bit_cast(s16x2, pw[q] << 16);
        pk = __builtin_amdgcn_cvt_sr_bf16_f32(pk, v[8 * h + 2 * q], pw[q] << 16, false);
        pk = __builtin_amdgcn_cvt_sr_bf16_f32(pk, v[8 * h + 2 * q + 1], pw[q], true);
        out[4 * h + q] = __builtin_bit_cast(uint32_t, pk);
      }
    }
    if (any_nan16(v)) {
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (__builtin_isnan(v[t])) put(t, f32_to_bf16_rne(v[t]));
    }
  } else {
    // Elements e0 .. e0 + 15 lie in blocks g0, g0 + 1 and, when e0 is not a
    // multiple of 8, g0 + 2; each block rounds the elements it covers.
    const uint64_t g0 = e0 >> 3;
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const Philox4x32 p = sr_block(srk, g0 + (uint64_t)b);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint64_t ee = e0 + (uint64_t)t;
        if ((ee >> 3) - g0 == (uint64_t)b) put(t, f32_to_bf16_sr(value(t), sr_draw(p, ee)));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  o0 = u32x4{out[0], out[1], out[2], out[3]};
  o1 = u32x4{out[4], out[5], out[6], out[7]};
}

// s_waitcnt with only the vector-memory counter constrained.
template <int N>
__device__ __forceinline__ void merge_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Direct global->LDS copy of one 16-byte chunk per lane.
__device__ __forceinline__ void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
// The same with the non-temporal hint (cache policy NT), for W: each of its
// lines is read once and written once, so it should not displace the packed
// update that the column blocks of a run share in L2.
__device__ __forceinline__ void dma16_nt(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 2);
}

// LDS accesses of the streamed tiles are written as statements the compiler
// cannot order against the direct loads still in flight (it would otherwise
// wait for all of them before any LDS access): reads complete inside the
// statement; writes are complete once lgkmcnt reaches zero.  Outputs are
// early-clobber so that no destination shares a register with an address.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
// N 16-byte reads at a + 1024 i.
template <int N>
__device__ __forceinline__ void lds_read_slabs(uint32_t a, u32x4 (&x)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "slab count");
  if constexpr (N == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x[0]) : "v"(a) : "memory");
  } else if constexpr (N == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(x[0]), "=&v"(x[1]) : "v"(a) : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]) : "v"(a) : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7])
        : "v"(a)
        : "memory");
  }
}
// The same N reads, issued only; the registers are valid after
// lds_wait_slabs() (the outputs stay tied to the wait, so they are neither
// read nor reused before it).
template <int N>
__device__ __forceinline__ void lds_issue_slabs(uint32_t a, u32x4 (&x)[N]) {
  static_assert(N == 4, "slab count");
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]) : "v"(a) : "memory");
}
template <int N>
__device__ __forceinline__ void lds_wait_slabs(u32x4 (&x)[N]) {
  static_assert(N == 4, "slab count");
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]) : : "memory");
}
// 16-byte reads at two or four arbitrary addresses.
__device__ __forceinline__ void lds_read_at(const uint32_t (&a)[2], u32x4 (&x)[2]) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x[0]), "=&v"(x[1]) : "v"(a[0]), "v"(a[1]) : "memory");
}
__device__ __forceinline__ void lds_read_at(const uint32_t (&a)[4], u32x4 (&x)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}
__device__ __forceinline__ void lds_write16(uint32_t a, const u32x4& v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier without the memory fence of __syncthreads (which waits
// for every outstanding global access, the loads in flight included).
__device__ __forceinline__ void merge_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A block = 8 waves (two per SIMD) x E 32-column instances.  The work of a
// launch is a list of units (matrix, column block of BC = 256 E columns,
// 32-row band), ordered by matrix, then column block, then band; block b
// takes units [b U / G, (b + 1) U / G) of the U units over G blocks, so the
// blocks carry equal shares.  Its range splits into segments of one column
// block each; for each, the signs of A for the block's columns are generated
// into LDS as bits and expanded into per-lane A operands, then each band
// computes C = sigma^T U^T (KS 16-rank steps), updates and rounds.  Interior
// bands of column-interior blocks stream through LDS (a ring of W tiles and
// U slabs, the next bands' loads in flight while one computes); the others
// take guarded register loads and stores.
constexpr int kMergeWaves = 8;
constexpr int kMergeRunSlack = 110;

struct MergeGroupArgs {
  KeyArg key[kMaxGroup];
  KeyArg sr_key[kMaxGroup];
  uint16_t* W[kMaxGroup];
  const void* U[kMaxGroup];               // fp32 [d x r], or packed operands
  const uint16_t* A[kMaxGroup];           // explicit projection in operand form, or null
  int64_t d[kMaxGroup];
  int64_t k[kMaxGroup];
  int64_t ldw[kMaxGroup];
  int64_t row0[kMaxGroup];
  int64_t unit_begin[kMaxGroup + 1];      // first unit of each matrix
  // runs: block-per-run schedule instead of equal shares -- matrix i has
  // blocks [block_begin[i], block_begin[i + 1]).  With pack[i] > 1 block j
  // of it takes every band of column blocks [j pack, (j + 1) pack); else
  // block (cb, g) of it (cb fastest) takes bands [g nb / m, (g + 1) nb / m)
  // of column block cb, m = nruns[i] runs of nearly equal length.
  int runs;
  int nruns[kMaxGroup];
  int pack[kMaxGroup];
  int64_t block_begin[kMaxGroup + 1];
  int64_t nblocks;  // blocks with work; the grid is padded to a multiple of 8
  int n;
  int64_t r;
  float scale_cr;
  const float* scale_dev;
};

// PACKED: U arrives already split in operand order (see the packed update
// layout); the band's U slabs are then copied into the ring as they are,
// with no split pass and no split buffer.
// EXPLICIT (with PACKED): the A operands come from an explicit projection
// packed in the merge's operand order (bf16 hi and lo, see
// pack_merge_projection_kernel) instead of sign bits; each rank step then
// takes three MFMAs (A hi x U hi, A hi x U lo, A lo x U hi).
template <int KS, int E, bool STOCH, bool PACKED, bool EXPLICIT = false>
__global__ __launch_bounds__(kMergeWaves * 64, 1) void merge_bf16_kernel(MergeGroupArgs g) {
  constexpr int NWV = kMergeWaves;
  constexpr int BC = 32 * NWV * E;        // columns per block
  constexpr int NWd = BC / 32;            // sign words per rank
  constexpr int CH = BC / 8;              // 16-byte chunks per tile row
  constexpr int WT = 32 * BC / 8;         // 16-byte chunks per W tile (32 rows)
  constexpr int UT = 32 * KS * 4;         // 16-byte chunks per U band (operand order)
  constexpr int SLOT = WT + UT;           // one band: W tile, then U (fp32 or packed)
  // bands in the LDS ring: three when they fit in the 160 KiB, else two
  constexpr int NR = (3 * SLOT + (PACKED ? 0 : UT)) * 16 <= 160 * 1024 ? 3 : 2;
  // LDS: a ring of NR bands, then (fp32 U) the band's U as bf16 hi/lo
  // operands (KS hi slabs, KS lo slabs).  The sign bits live in the ring
  // until the A operands are built.
  __shared__ __align__(16) u32x4 lds[NR * SLOT + (PACKED ? 0 : UT)];
  // With many rank steps (the MFMA chain long against the rounding), the
  // stochastic-rounding draws of a band are generated inside the chain and
  // parked here until the rounding: two generator blocks per instance.
  constexpr bool kDrawsInChain = STOCH && PACKED && !EXPLICIT && KS >= 8;
  __shared__ __align__(16) u32x4 draws[kDrawsInChain ? NWV * 2 * E * 64 : 1];
  // With fewer rank steps the draws stay in registers: they are generated
  // after the chain's MFMAs are issued, in the same scheduling region, so
  // the generator's vector work issues while the matrix cores run.
  constexpr bool kDrawsInRegs = STOCH && PACKED && !EXPLICIT && !kDrawsInChain;
  static_assert(16 * KS * NWd <= 4 * WT, "sign bits must fit in one W tile");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t r = g.r;
  const float scale_cr = g.scale_cr;
  const float* __restrict__ scale_dev = g.scale_dev;

  // Logical block index: blocks are dispatched round-robin over the 8 XCDs,
  // so logical blocks x nxb .. (x + 1) nxb - 1 run on XCD x.  The column
  // blocks of one band run (consecutive logical blocks) then share that
  // XCD's L2 copy of the run's packed U instead of each fetching it.
  const int64_t nxb = gridDim.x >> 3;
  const int64_t lb = (int64_t)(blockIdx.x & 7) * nxb + (int64_t)(blockIdx.x >> 3);
  if (lb >= g.nblocks) return;  // padding (uniform per block, before any barrier)

  int64_t pos, pos_end;
  if (g.runs) {
    int it = 0;
    while (lb >= g.block_begin[it + 1]) ++it;
    const int64_t nb = (g.d[it] + 31) / 32;
    const int64_t ncb = (g.unit_begin[it + 1] - g.unit_begin[it]) / nb;
    const int64_t local = lb - g.block_begin[it];
    if (g.pack[it] > 1) {
      const int64_t cb0 = local * g.pack[it];
      const int64_t cb1 = cb0 + g.pack[it] < ncb ? cb0 + g.pack[it] : ncb;
      pos = g.unit_begin[it] + cb0 * nb;
      pos_end = g.unit_begin[it] + cb1 * nb;
    } else {
      const int64_t m = g.nruns[it];
      const int64_t cb = local % ncb, bg = local / ncb;
      pos = g.unit_begin[it] + cb * nb + bg * nb / m;
      pos_end = g.unit_begin[it] + cb * nb + (bg + 1) * nb / m;
    }
  } else {
    const int64_t total = g.unit_begin[g.n];
    pos = lb * total / g.nblocks;
    pos_end = (lb + 1) * total / g.nblocks;
  }
  for (bool first = true; pos < pos_end; first = false) {
    // The lane index is opaque per segment, so that nothing derived from it
    // is hoisted out of the segment loop and held in registers throughout.
    int lane_o = tid & 63;
    asm volatile("" : "+v"(lane_o));
    const int lane = lane_o;
    const int n = lane & 31;     // W row within the band (B and C layouts)
    const int hw = lane >> 5;
    // The segment: one column block of one matrix, bands [band_begin, band_end).
    int item = 0;
    while (pos >= g.unit_begin[item + 1]) ++item;
    const KeyArg key = g.key[item];
    const KeyArg sr_key = g.sr_key[item];
    uint16_t* __restrict__ W = g.W[item];
    const float* __restrict__ U = static_cast<const float*>(g.U[item]);
    const uint16_t* __restrict__ Up = static_cast<const uint16_t*>(g.U[item]);
    const int64_t d = g.d[item], k = g.k[item], ldw = g.ldw[item], row0 = g.row0[item];
    const int64_t nbands = (d + 31) / 32;
    const int64_t cb = (pos - g.unit_begin[item]) / nbands;
    const int64_t cblk = cb * BC;
    const int64_t band_begin = pos - g.unit_begin[item] - cb * nbands;
    const int64_t seg_end = g.unit_begin[item] + (cb + 1) * nbands < pos_end
                                ? g.unit_begin[item] + (cb + 1) * nbands
                                : pos_end;
    const int64_t band_end = band_begin + (seg_end - pos);
    pos = seg_end;
    if (!first) __syncthreads();  // the previous segment's LDS reads are done

    // Sign bits of ranks [0, 16 KS) for the block's columns: word w of rank j
    // holds columns cblk + 32w + (0..31), bit set meaning -1.
    uint32_t* sbits = reinterpret_cast<uint32_t*>(lds);
    if constexpr (!EXPLICIT) {
      const KeyWords kw{key.k0, key.k1};
      constexpr int NP = (BC + 255) / 256;  // Philox blocks per rank
      for (int task = tid; task < 16 * KS * NP; task += NWV * 64) {
        const int j = task / NP;
        const int pb = task - j * NP;
        const int64_t c256 = (cblk >> 8) + pb;
        uint32_t words[8];
        if (j < r && c256 * 256 < k) {
          const Philox4 p = sigma_block(kw, (uint64_t)j, (uint64_t)c256);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            words[2 * w] = (uint32_t)p.w[w];
            words[2 * w + 1] = (uint32_t)(p.w[w] >> 32);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 8; ++w) words[w] = 0u;
        }
        if constexpr (BC >= 256) {
#pragma unroll
          for (int w = 0; w < 8; ++w) sbits[j * NWd + 8 * pb + w] = words[w];
        } else {
          const int off = (int)((cblk & 255) >> 5);  // 128-column block: half of the 256 bits
#pragma unroll
          for (int w = 0; w < NWd; ++w) sbits[j * NWd + w] = words[off + w];
        }
      }
    }
    __syncthreads();

    // A operands: instance e holds, for MFMA row m = l & 31, column
    // 32(E wave + e) + 16((m >> 2) & 1) + 4(m >> 3) + (m & 3) of the block and
    // ranks 16s + 8(l >> 5) + i, i = 0..7.  Ranks >= r read as +1; their U
    // terms are zero.  At 256 ranks the E KS operands would not fit in the
    // register file beside the rest, so they are held as sign bits instead,
    // four operands per word (operand q of a word: the signs of ranks 2p and
    // 2p + 1 at bits 15 - 4q - p and 31 - 4q - p), and expanded at each use.
    constexpr bool SBITS = !EXPLICIT && KS == 16;
    constexpr int NAW = SBITS ? (E * KS + 3) / 4 : 1;
    u32x4 afrag[E][SBITS ? 1 : KS];
    u32x4 alo[E][EXPLICIT ? KS : 1];
    uint32_t awords[NAW];
    if constexpr (EXPLICIT) {
      const uint16_t* __restrict__ Ap = g.A[item];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const uint16_t* p = Ap + (((((cb * NWV + wave) * E + e) * KS + s) * 2) * 512) + lane * 8;
          afrag[e][s] = *reinterpret_cast<const u32x4*>(p);
          alo[e][s] = *reinterpret_cast<const u32x4*>(p + 512);
        }
    } else {
      const int m = lane & 31;
      const int cm = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
#pragma unroll
      for (int w = 0; w < NAW; ++w) awords[w] = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int cl = 32 * (E * wave + e) + cm;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          // An opaque base per step, so that the step's eight reads are not
          // hoisted with every other step's and held at once.
          int base = (16 * s + 8 * hw) * NWd + (cl >> 5);
          if constexpr (SBITS) asm volatile("" : "+v"(base));
          uint32_t byte = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) byte |= ((sbits[base + i * NWd] >> (cl & 31)) & 1u) << i;
          if constexpr (SBITS) {
            const int o = e * KS + s, q = o & 3;
            uint32_t w = 0;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp)
              w |= (((byte >> (2 * pp)) & 1u) << (15 - 4 * q - pp)) |
                   (((byte >> (2 * pp + 1)) & 1u) << (31 - 4 * q - pp));
            awords[o >> 2] |= w;
          } else {
            afrag[e][s] = u32x4{
                0x3F803F80u | ((byte << 15) & 0x8000u) | ((byte << 30) & 0x80000000u),
                0x3F803F80u | ((byte << 13) & 0x8000u) | ((byte << 28) & 0x80000000u),
                0x3F803F80u | ((byte << 11) & 0x8000u) | ((byte << 26) & 0x80000000u),
                0x3F803F80u | ((byte << 9) & 0x8000u) | ((byte << 24) & 0x80000000u)};
          }
          if constexpr (KS > 8) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // The A operand of instance e, rank step s.
    auto aop = [&](int e, int s) __attribute__((always_inline)) {
      if constexpr (SBITS) {
        const int o = e * KS + s;
        return expand_sign_pairs(awords[o >> 2] << (4 * (o & 3)));
      } else {
        return afrag[e][s];
      }
    };
    __syncthreads();  // the sign bits are dead; the ring may be loaded

    float sc = scale_cr;
    if (scale_dev != nullptr) sc *= *scale_dev;
    const KeyWords srk{sr_key.k0, sr_key.k1};
    const int64_t cw = cblk + 32 * E * wave;   // this wave's first column
    const bool col_interior = cblk + BC <= k;
    const bool u_dma = PACKED || (r & 3) == 0;
    const bool r_full = (r & 15) == 0;
    // Every lane's sixteen columns start at a multiple of 16, so with k a
    // multiple of 16 each lane's draws are one whole generator block.
    const bool sr_aligned = (k & 15) == 0;

    // C of one band: acc[e] over all rank steps, B operands from bfrag(s).
    auto mfma_band = [&](f32x16 (&acc)[E], auto&& bfrag) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[e][i] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 bh, bl;
        bfrag(s, bh, bl);
#pragma unroll
        for (int e = 0; e < E; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop(e, s)), as_bf16x8(bh),
                                                           acc[e], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < E; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop(e, s)), as_bf16x8(bl),
                                                           acc[e], 0, 0, 0);
        if constexpr (EXPLICIT) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(alo[e][s]), as_bf16x8(bh),
                                                             acc[e], 0, 0, 0);
        }
        // With many rank steps, keep each step's operand loads next to their
        // use: hoisting them all would exceed the register file.
        if constexpr (KS > 8) __builtin_amdgcn_sched_barrier(0);
      }
    };

    constexpr int kPackedGroup = KS < 4 ? KS : (KS == 16 && E == 2) ? 2 : 4;
    // C of one band from packed U slabs in LDS (slab 2s the hi term, 2s + 1
    // the lo term of step s, 1 KiB apart): the slabs of G steps are read in
    // one group and waited for once, so a band takes KS / G LDS round trips.
    // after_group(i) runs after the MFMAs of group i, in the same scheduling
    // region, so independent vector work placed there issues while the
    // matrix cores are busy.
    auto mfma_band_packed = [&](f32x16 (&acc)[E], const u32x4* ut, auto&& after_group)
                                __attribute__((always_inline)) {
      constexpr int G = kPackedGroup;
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[e][i] = 0.f;
      // With several groups, group g + 1's slabs are read while group g's
      // MFMAs run (two register sets).
      constexpr bool kAhead = KS / G >= 2 && 2 * G == 4;
      u32x4 x[2 * G];
      if constexpr (kAhead) lds_read_slabs<2 * G>(lds_u32(ut + lane), x);
#pragma unroll
      for (int s0 = 0; s0 < KS; s0 += G) {
        u32x4 xn[2 * G];
        const bool more = kAhead && s0 + G < KS;  // a constant once unrolled
        if constexpr (kAhead) {
          if (more) lds_issue_slabs<2 * G>(lds_u32(ut + (2 * (s0 + G)) * 64 + lane), xn);
          __builtin_amdgcn_sched_barrier(0);  // the reads go out before this group's MFMAs
        } else {
          lds_read_slabs<2 * G>(lds_u32(ut + (2 * s0) * 64 + lane), x);
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const int s = s0 + i;
#pragma unroll
          for (int e = 0; e < E; ++e)
            acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop(e, s)), as_bf16x8(x[2 * i]),
                                                             acc[e], 0, 0, 0);
#pragma unroll
          for (int e = 0; e < E; ++e)
            acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aop(e, s)),
                                                             as_bf16x8(x[2 * i + 1]), acc[e], 0, 0, 0);
          if constexpr (EXPLICIT) {
#pragma unroll
            for (int e = 0; e < E; ++e)
              acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(alo[e][s]),
                                                               as_bf16x8(x[2 * i]), acc[e], 0, 0, 0);
          }
        }
        after_group(s0 / G);
        if constexpr (kAhead) {
          if (more) {
            __builtin_amdgcn_sched_barrier(0);  // and are waited for after them
            lds_wait_slabs<2 * G>(xn);
#pragma unroll
            for (int i = 0; i < 2 * G; ++i) x[i] = xn[i];
          }
        }
        if constexpr (KS > 8) __builtin_amdgcn_sched_barrier(0);
      }
    };

    u32x4* bs = lds + NR * SLOT;   // split U: KS hi slabs then KS lo slabs (fp32 U only)
    // Four fp32 U values of rank slab li (step s = li >> 1, half q = li & 1)
    // into the hi and lo operands of step s in bs; ranks >= r count as zero.
    auto split_to_bs = [&](int li, const float (&xin)[4], int rr) __attribute__((always_inline)) {
      const int s = li >> 1, q = li & 1;
      const int j0 = 16 * s + 8 * hw + 4 * q;
      float h[4], l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = xin[i];
        if (!r_full && j0 + i >= rr) x = 0.f;
        h[i] = (float)(__bf16)x;
        l[i] = x - h[i];
      }
      const uint32_t hi0 = bf16_pair(h[0], h[1]), hi1 = bf16_pair(h[2], h[3]);
      const uint32_t lo0 = bf16_pair(l[0], l[1]), lo1 = bf16_pair(l[2], l[3]);
      const uint32_t ah = lds_u32(bs + s * 64 + lane) + 8 * q;
      const uint32_t al = lds_u32(bs + (KS + s) * 64 + lane) + 8 * q;
      asm volatile("ds_write_b64 %0, %1\n\tds_write_b64 %2, %3"
                   :
                   : "v"(ah), "v"(hi0 | ((uint64_t)hi1 << 32)), "v"(al),
                     "v"(lo0 | ((uint64_t)lo1 << 32))
                   : "memory");
    };
    // The band's hi and lo B operands of step s from bs.
    auto bfrag_lds = [&](int s, u32x4& bh, u32x4& bl) __attribute__((always_inline)) {
      u32x4 hl[1];
      lds_read_slabs<1>(lds_u32(bs + s * 64 + lane), hl);
      bh = hl[0];
      lds_read_slabs<1>(lds_u32(bs + (KS + s) * 64 + lane), hl);
      bl = hl[0];
    };

    // Guarded path for one band (row or column edge): W by guarded register
    // loads and stores; fp32 U split through bs as in the streamed path,
    // packed U read straight from memory (its rows are padded to the band).
    auto edge_band = [&](int64_t band) __attribute__((always_inline)) {
      const int64_t row = band * 32 + n;
      f32x16 acc[E];
      if constexpr (PACKED) {
        const uint16_t* ub = Up + band * KS * 1024 + lane * 8;
        mfma_band(acc, [&](int s, u32x4& bh, u32x4& bl) __attribute__((always_inline)) {
          bh = *reinterpret_cast<const u32x4*>(ub + s * 1024);
          bl = *reinterpret_cast<const u32x4*>(ub + s * 1024 + 512);
        });
      } else {
        merge_barrier();  // no wave still reads bs
        {
          // An opaque copy of r: the rank bounds are not hoisted out of the loop.
          int rr = (int)r;
          asm volatile("" : "+s"(rr));
          for (int li = wave; li < 2 * KS; li += NWV) {
            const int j0 = 16 * (li >> 1) + 8 * hw + 4 * (li & 1);
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              x[i] = (row < d && j0 + i < rr) ? U[row * r + j0 + i] : 0.f;
            split_to_bs(li, x, rr);
          }
        }
        lds_wait();
        merge_barrier();  // the band's operands are split
        mfma_band(acc, bfrag_lds);
      }
      if (row >= d) return;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int64_t c = cw + 32 * e + 16 * hw;
        if (c >= k) continue;
        u32x4 w0, w1, o0, o1;
        load_w16(W, ldw, d, k, row, c, w0, w1);
        update16<STOCH>(w0, w1, acc[e], sc, srk,
                        (uint64_t)(row0 + row) * (uint64_t)k + (uint64_t)c, sr_aligned, o0, o1);
        if (c + 16 <= k) {
          u32x4* dst = reinterpret_cast<u32x4*>(W + row * ldw + c);
          dst[0] = o0;
          dst[1] = o1;
        } else {
          for (int t = 0; t < 16 && c + t < k; ++t) {
            const uint32_t word = (t < 8) ? o0[t >> 1] : o1[(t - 8) >> 1];
            W[row * ldw + c + t] = (uint16_t)((t & 1) ? (word >> 16) : (word & 0xFFFFu));
          }
        }
      }
    };

    // Interior bands: [band_begin, fast_end) when the block is column-interior
    // and U rows are 16-byte aligned; the rest take the guarded path.
    int64_t fast_end = band_begin;
    if (col_interior && u_dma) {
      fast_end = band_end;
      if (fast_end * 32 > d) --fast_end;  // the partial last band of W
    }

    if (fast_end > band_begin) {
      // Loads of band b into ring slot b % NR: W rows as whole 16E-chunk
      // segments (lane L of a load covers row a = a0 + L / CH, LDS position
      // L % CH, global chunk (L % CH) ^ (a & (CH - 1))), then U in operand
      // order (load (s, q) gives lane L row L & 31, ranks 16s + 8(L>>5) + 4q
      // .. +3).  Two bands are in flight while one computes.
      constexpr int RPL = 64 / CH;              // W rows per 1 KiB load
      constexpr int WL = 32 / RPL / NWV;        // W loads (and stores) per wave per band
      constexpr int UL = (2 * KS + NWV - 1) / NWV;  // U loads per wave per band
      constexpr int LB = WL + UL;               // loads per wave per band
      static_assert(WL * RPL * NWV == 32, "W loads must cover the band");
      auto slot_of = [&](int64_t band) __attribute__((always_inline)) {
        return lds + (int)((band - band_begin) % NR) * SLOT;
      };
      auto issue = [&](int64_t band) __attribute__((always_inline)) {
        u32x4* wt = slot_of(band);
        u32x4* ut = wt + WT;
#pragma unroll
        for (int t = 0; t < WL; ++t) {
          const int a = (wave * WL + t) * RPL + lane / CH;
          const int pos = lane % CH;
          const int chunk = pos ^ (a & (CH - 1));
          dma16_nt(W + (band * 32 + a) * ldw + cblk + 8 * chunk, wt + (wave * WL + t) * 64);
        }
#pragma unroll
        for (int t = 0; t < UL; ++t) {
          int li = wave + NWV * t;
          if (li > 2 * KS - 1) li = 2 * KS - 1;   // repeat a load: same bytes, same place
          if constexpr (PACKED) {
            // slab li = 2s + (lo term) of the band, stored contiguously
            dma16(Up + (band * 2 * KS + li) * 512 + lane * 8, ut + li * 64);
          } else {
            const int s = li >> 1, q = li & 1;
            int64_t j = 16 * s + 8 * hw + 4 * q;
            if (j + 4 > r) j = r - 4;              // ranks past r: any in-bounds chunk, zeroed later
            const int64_t row = band * 32 + n;
            dma16(U + row * r + j, ut + li * 64);
          }
        }
      };
      // Wait until this wave's loads of band b have landed, given how many
      // vector-memory operations it issued after them (see the loop).
      auto wait_band = [&](int64_t band) __attribute__((always_inline)) {
        const int64_t i = band - band_begin;
        if constexpr (NR == 3) {
          const bool more1 = band + 1 < fast_end;
          if (i == 0) {
            if (more1) merge_wait_vmcnt<LB>(); else merge_wait_vmcnt<0>();
          } else if (i == 1) {
            if (more1) merge_wait_vmcnt<LB + WL>(); else merge_wait_vmcnt<WL>();
          } else {
            if (more1) merge_wait_vmcnt<2 * WL + LB>(); else merge_wait_vmcnt<2 * WL>();
          }
        } else {
          if (i == 0) merge_wait_vmcnt<0>(); else merge_wait_vmcnt<WL>();
        }
      };
#pragma unroll
      for (int t = 0; t < NR - 1; ++t)
        if (band_begin + t < fast_end) issue(band_begin + t);
      for (int64_t band = band_begin; band < fast_end; ++band) {
        // Issue order per wave: loads(b0) .. loads(b0 + NR - 2), then per band
        // j: loads(j + NR - 1), stores(j).
        wait_band(band);
        merge_barrier();  // every wave's loads of this band have landed, and the
                          // slot of band - 1 is no longer read
        if (band + NR - 1 < fast_end) issue(band + NR - 1);
        u32x4* wt = slot_of(band);
        const u32x4* ut = wt + WT;
        // Split U once per band: wave w converts fp32 slabs w, w + NWV, ...
        // (step s, half q) into halves of the hi and lo operands of step s.
        if constexpr (!PACKED) {
          int rr = (int)r;  // opaque: the rank bounds are not hoisted
          asm volatile("" : "+s"(rr));
          for (int li = wave; li < 2 * KS; li += NWV) {
            u32x4 xv[1];
            lds_read_slabs<1>(lds_u32(ut + li * 64 + lane), xv);
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t bits = xv[0][i];
              x[i] = __builtin_bit_cast(float, bits);
            }
            split_to_bs(li, x, rr);
          }
          lds_wait();
          merge_barrier();  // the band's operands are split
        }
        // This lane's W chunks: columns 32e + 16hw .. +15 of row n are chunks
        // cc, cc + 1 with cc = 4(E wave + e) + 2hw.
        uint32_t wa[2 * E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int cc = 4 * (E * wave + e) + 2 * hw;
          wa[2 * e] = lds_u32(wt + n * CH + (cc ^ (n & (CH - 1))));
          wa[2 * e + 1] = lds_u32(wt + n * CH + ((cc + 1) ^ (n & (CH - 1))));
        }
        const int64_t row = band * 32 + n;
        // The draws (aligned k) are generated one block after each of the
        // first 2E groups of the chain; they depend only on the element
        // index, not on the products.
        static_assert(!kDrawsInChain || KS / kPackedGroup >= 2 * E, "one draw block per group");
        // The W values are read before the chain, or, with the draws in it,
        // after it (the draws take their registers meanwhile).
        u32x4 wx[2 * E];
        if constexpr (!kDrawsInChain) lds_read_at(wa, wx);
        f32x16 acc[E];
        u32x4 pre[E][2];
        if constexpr (PACKED) {
          mfma_band_packed(acc, ut, [&](int grp) __attribute__((always_inline)) {
            if constexpr (kDrawsInRegs) {
              if (grp == 0) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                  const uint64_t e0 =
                      (uint64_t)(row0 + row) * (uint64_t)k + (uint64_t)(cw + 32 * e + 16 * hw);
#pragma unroll
                  for (int h = 0; h < 2; ++h) {
                    const Philox4x32 p = sr_block(srk, (e0 >> 3) + h);
                    pre[e][h] = u32x4{p.w[0], p.w[1], p.w[2], p.w[3]};
                  }
                }
              }
            }
            if constexpr (kDrawsInChain) {
              if (grp < 2 * E) {
                const int e = grp >> 1, h = grp & 1;
                const uint64_t e0 =
                    (uint64_t)(row0 + row) * (uint64_t)k + (uint64_t)(cw + 32 * e + 16 * hw);
                const Philox4x32 p = sr_block(srk, (e0 >> 3) + h);
                lds_write16(lds_u32(draws + (wave * 2 * E + grp) * 64 + lane),
                            u32x4{p.w[0], p.w[1], p.w[2], p.w[3]});
              }
            }
          });
        } else {
          mfma_band(acc, bfrag_lds);
        }
        if constexpr (kDrawsInChain) {
          lds_read_at(wa, wx);
          u32x4 dv[2 * E];
          lds_read_slabs<2 * E>(lds_u32(draws + (wave * 2 * E) * 64 + lane), dv);
#pragma unroll
          for (int b = 0; b < 2 * E; ++b) pre[b >> 1][b & 1] = dv[b];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          u32x4 o0, o1;
          const uint64_t e0 = (uint64_t)(row0 + row) * (uint64_t)k + (uint64_t)(cw + 32 * e + 16 * hw);
          if ((kDrawsInChain || kDrawsInRegs) && sr_aligned)
            update16<STOCH, kDrawsInChain || kDrawsInRegs>(wx[2 * e], wx[2 * e + 1], acc[e], sc, srk, e0,
                                                           true, o0, o1, pre[e]);
          else
            update16<STOCH>(wx[2 * e], wx[2 * e + 1], acc[e], sc, srk, e0, sr_aligned, o0, o1);
          lds_write16(wa[2 * e], o0);
          lds_write16(wa[2 * e + 1], o1);
        }
        lds_wait();
        merge_barrier();  // the whole tile is updated
        // Whole-row stores, in the load's lane order, non-temporal as the loads.
        u32x4 ov[WL];
        lds_read_slabs<WL>(lds_u32(wt + (wave * WL) * 64 + lane), ov);
#pragma unroll
        for (int t = 0; t < WL; ++t) {
          const int a = (wave * WL + t) * RPL + lane / CH;
          const int pos = lane % CH;
          const int chunk = pos ^ (a & (CH - 1));
          __builtin_nontemporal_store(ov[t], reinterpret_cast<u32x4*>(W + (band * 32 + a) * ldw + cblk + 8 * chunk));
        }
      }
      merge_wait_vmcnt<0>();
    }
    for (int64_t band = fast_end; band < band_end; ++band) edge_band(band);
  }  // segments
}

// fp32 W: a block owns 16 rows x one 256-column Philox block; signs in LDS
// as bits; fp64 sums; the update is rounded once to fp32.
__global__ __launch_bounds__(256) void merge_f32_kernel(KeyArg key, int64_t d, int64_t k,
                                                        int64_t r, float* __restrict__ W,
                                                        int64_t ldw, const float* __restrict__ U,
                                                        double scale_cr,
                                                        const float* __restrict__ scale_dev) {
  __shared__ uint32_t bits[kMaxRank][8];
  const int64_t b = blockIdx.x;
  const int64_t i0 = (int64_t)blockIdx.y * 16;
  const int tid = threadIdx.x;
  for (int64_t j = tid; j < r; j += 256) {
    const Philox4 p = sigma_block(KeyWords{key.k0, key.k1}, (uint64_t)j, (uint64_t)b);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      bits[j][2 * w] = (uint32_t)p.w[w];
      bits[j][2 * w + 1] = (uint32_t)(p.w[w] >> 32);
    }
  }
  __syncthreads();
  double sc = scale_cr;
  if (scale_dev != nullptr) sc *= (double)*scale_dev;
  const int64_t l = b * 256 + tid;
  if (l >= k) return;
  for (int64_t i = i0; i < i0 + 16 && i < d; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < r; ++j) {
      const double u = (double)U[i * r + j];
      acc += ((bits[j][tid >> 5] >> (tid & 31)) & 1u) ? -u : u;
    }
    W[i * ldw + l] = (float)((double)W[i * ldw + l] - sc * acc);
  }
}

}  // namespace

// Compute units of the current device (queried once per device; concurrent
// first calls may both query, and store the same value).
int64_t compute_units() {
  static std::atomic<int64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int64_t v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    v = n;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

hipError_t launch_merge_grouped(const MergeItem* items, int n, int64_t r, double scale,
                                const float* scale_dev, bool stochastic, bool packed,
                                hipStream_t s) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  const double cr = 1.0 / std::sqrt((double)r);
  const int ks = merge_rank_steps(r);
  const bool explicit_a = items[0].A != nullptr;  // all or none (checked by the caller)
  // 32-column instances per wave (must match the kernel instantiated below)
  const int e = (ks <= 4 || (ks == 16 && !explicit_a)) ? 2 : 1;
  const int64_t bc = 32 * kMergeWaves * e;
  MergeGroupArgs g{};
  g.n = n;
  g.r = r;
  if (explicit_a && !packed) return hipErrorInvalidValue;
  g.scale_cr = (float)(explicit_a ? scale : scale * cr);
  g.scale_dev = scale_dev;
  g.unit_begin[0] = 0;
  for (int i = 0; i < n; ++i) {
    g.key[i] = items[i].key;
    g.sr_key[i] = items[i].sr_key;
    g.W[i] = static_cast<uint16_t*>(items[i].W);
    g.U[i] = items[i].U;
    g.A[i] = static_cast<const uint16_t*>(items[i].A);
    g.d[i] = items[i].d;
    g.k[i] = items[i].k;
    g.ldw[i] = items[i].ldw;
    g.row0[i] = items[i].row0;
    const int64_t ncb = (items[i].k + bc - 1) / bc;
    const int64_t nb = (items[i].d + 31) / 32;
    g.unit_begin[i + 1] = g.unit_begin[i] + ncb * nb;
  }
  // At most one block per compute unit (a second round of blocks would
  // double the time of the units it holds).  Equal shares balance the load
  // but may split a column block's run of bands over two blocks (each
  // then builds the block's A operands and fills its ring), and the blocks
  // running at one time hold different bands, so each fetches its own
  // packed U.  Runs avoid both: the column blocks of one band range are
  // consecutive logical blocks on one XCD, so they read the range's U from
  // that XCD's L2.  Each matrix takes m runs of nearly equal length per
  // column block, or, when its column blocks are short, several whole
  // column blocks per block; the run length L starts at the equal share
  // and grows until the runs fit the compute units.  The runs are taken
  // when the longest is within kMergeRunSlack percent of the equal share.
  const int64_t cus = compute_units();
  const int64_t total = g.unit_begin[n];
  if (total == 0) return hipSuccess;
  int64_t blocks = total < cus ? total : cus;
  const int64_t share = (total + blocks - 1) / blocks;
  g.runs = 0;
  for (int64_t L = share; L <= 2 * share; ++L) {
    int64_t nblk = 0, worst = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t nb = (items[i].d + 31) / 32;
      const int64_t ncb = nb > 0 ? (g.unit_begin[i + 1] - g.unit_begin[i]) / nb : 0;
      if (2 * nb <= L) {
        const int64_t c = std::min<int64_t>(std::max<int64_t>(L / nb, 1), std::max<int64_t>(ncb, 1));
        g.pack[i] = (int)c;
        g.nruns[i] = 1;
        nblk += (ncb + c - 1) / c;
        worst = std::max(worst, c * nb);
      } else {
        const int64_t m = (nb + L - 1) / L;
        g.pack[i] = 1;
        g.nruns[i] = (int)m;
        nblk += ncb * m;
        worst = std::max(worst, (nb + m - 1) / m);
      }
    }
    if (nblk <= cus) {
      if (worst * 100 <= share * kMergeRunSlack) {
        g.runs = 1;
        g.block_begin[0] = 0;
        for (int i = 0; i < n; ++i) {
          const int64_t nb = (items[i].d + 31) / 32;
          const int64_t ncb = nb > 0 ? (g.unit_begin[i + 1] - g.unit_begin[i]) / nb : 0;
          g.block_begin[i + 1] = g.block_begin[i] +
                                 (g.pack[i] > 1 ? (ncb + g.pack[i] - 1) / g.pack[i] : ncb * g.nruns[i]);
        }
        blocks = g.block_begin[n];
      }
      break;
    }
  }
  g.nblocks = blocks;
  const dim3 grid((unsigned)((blocks + 7) / 8 * 8));
#define LOGRA_MERGE_LAUNCH_P(KS, E, P)                                                      \
  if (stochastic)                                                                           \
    hipLaunchKernelGGL((merge_bf16_kernel<KS, E, true, P>), grid, dim3(kMergeWaves * 64), 0, \
                       s, g);                                                               \
  else                                                                                      \
    hipLaunchKernelGGL((merge_bf16_kernel<KS, E, false, P>), grid, dim3(kMergeWaves * 64), 0, \
                       s, g);
#define LOGRA_MERGE_LAUNCH_X(KS, E)                                                            \
  if (stochastic)                                                                          \
    hipLaunchKernelGGL((merge_bf16_kernel<KS, E, true, true, true>), grid,                \
                       dim3(kMergeWaves * 64), 0, s, g);                                  \
  else                                                                                     \
    hipLaunchKernelGGL((merge_bf16_kernel<KS, E, false, true, true>), grid,               \
                       dim3(kMergeWaves * 64), 0, s, g);
#define LOGRA_MERGE_LAUNCH(KS, E)        \
  if (explicit_a) {                      \
    LOGRA_MERGE_LAUNCH_X(KS, E)          \
  } else if (packed) {                   \
    LOGRA_MERGE_LAUNCH_P(KS, E, true)    \
  } else {                               \
    LOGRA_MERGE_LAUNCH_P(KS, E, false)   \
  }
  switch (ks) {
    case 1: LOGRA_MERGE_LAUNCH(1, 2) break;
    case 2: LOGRA_MERGE_LAUNCH(2, 2) break;
    case 4: LOGRA_MERGE_LAUNCH(4, 2) break;
    case 8: LOGRA_MERGE_LAUNCH(8, 1) break;
    case 16:
      if (explicit_a) {
        LOGRA_MERGE_LAUNCH_X(16, 1)
      } else if (packed) {
        LOGRA_MERGE_LAUNCH_P(16, 2, true)
      } else {
        LOGRA_MERGE_LAUNCH_P(16, 2, false)
      }
      break;
    default: return hipErrorInvalidValue;
  }
#undef LOGRA_MERGE_LAUNCH
#undef LOGRA_MERGE_LAUNCH_P
#undef LOGRA_MERGE_LAUNCH_X
  return hipGetLastError();
}

hipError_t launch_merge(KeyArg key, int64_t d, int64_t k, int64_t r, void* W, bool bf16,
                        int64_t ldw, const float* U, double scale, const float* scale_dev,
                        bool stochastic, KeyArg sr_key, int64_t row0, hipStream_t s) {
  if (!bf16) {
    const double cr = 1.0 / std::sqrt((double)r);
    const dim3 grid((unsigned)((k + 255) / 256), (unsigned)((d + 15) / 16));
    hipLaunchKernelGGL(merge_f32_kernel, grid, dim3(256), 0, s, key, d, k, r,
                       static_cast<float*>(W), ldw, U, scale * cr, scale_dev);
    return hipGetLastError();
  }
  const MergeItem it{key, sr_key, W, d, k, ldw, U, row0};
  return launch_merge_grouped(&it, 1, r, scale, scale_dev, stochastic, false, s);
}

// Packed update: U [d x r] fp32 (times a scale, 1 for a plain update) as the
// merge's B operands.  For 32-row band
// g and 16-rank step s (steps padded to KS = 1, 2, 4, 8 or 16), a 1 KiB hi
// slab then a 1 KiB lo slab, lane l holding rows 32g + (l & 31), ranks
// 16s + 8(l >> 5) + i (i = 0..7) as bf16 hi = RNE(u), lo = RNE(u - hi);
// rows >= d and ranks >= r are zero.
int merge_rank_steps(int64_t r) {
  const int64_t ksteps = (r + 15) / 16;
  return ksteps <= 1 ? 1 : ksteps <= 2 ? 2 : ksteps <= 4 ? 4 : ksteps <= 8 ? 8 : 16;
}
size_t packed_update_bytes(int64_t d, int64_t r) {
  return (size_t)((d + 31) / 32) * (size_t)merge_rank_steps(r) * 2048;
}

namespace {
__global__ __launch_bounds__(256) void pack_update_kernel(int64_t d, int64_t r, int ks, float scale,
                                                          const float* __restrict__ scale_dev,
                                                          const float* __restrict__ U,
                                                          uint16_t* __restrict__ P) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (band, step, lane)
  const int lane = (int)(t & 63);
  const int64_t bs = t >> 6;
  const int64_t nb = (d + 31) / 32;
  if (bs >= nb * ks) return;
  const int64_t band = bs / ks;
  const int s = (int)(bs - band * ks);
  const int64_t row = band * 32 + (lane & 31);
  const int64_t j0 = 16 * s + 8 * (lane >> 5);
  const float sc = scale_dev != nullptr ? scale * *scale_dev : scale;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (row < d && j0 + i < r) ? sc * U[row * r + j0 + i] : 0.f;
  u32x4 hv, lv;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float h0 = (float)(__bf16)x[2 * p], h1 = (float)(__bf16)x[2 * p + 1];
    hv[p] = bf16_pair(h0, h1);
    lv[p] = bf16_pair(x[2 * p] - h0, x[2 * p + 1] - h1);
  }
  uint16_t* dst = P + bs * 1024 + lane * 8;
  *reinterpret_cast<u32x4*>(dst) = hv;
  *reinterpret_cast<u32x4*>(dst + 512) = lv;
}
}  // namespace

// An explicit projection A [r x k] (fp32 row-major) in the merge's A-operand
// order: for column block cb (BC = 256 E columns, E = 2 when the merge takes
// at most four 16-rank steps, else 1), wave w, instance e and rank step s, a
// 1 KiB hi slab then a 1 KiB lo slab, lane l holding column
// BC cb + 32(E w + e) + 16((m >> 2) & 1) + 4(m >> 3) + (m & 3) (m = l & 31)
// and ranks 16s + 8(l >> 5) .. +7; ranks >= r and columns >= k are zero.
size_t merge_projection_packed_bytes(int64_t r, int64_t k) {
  const int ks = merge_rank_steps(r);
  const int e = ks <= 4 ? 2 : 1;
  const int64_t bc = 32 * kMergeWaves * e;
  return (size_t)((k + bc - 1) / bc) * kMergeWaves * e * ks * 2048;
}

namespace {
__global__ __launch_bounds__(256) void pack_merge_projection_kernel(int64_t r, int64_t k, int ks,
                                                                    int ee,
                                                                    const float* __restrict__ A,
                                                                    uint16_t* __restrict__ P) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lane = (int)(t & 63);
  const int64_t unit = t >> 6;  // (((cb * waves + w) * E + e) * KS + s)
  const int64_t bc = 32 * kMergeWaves * ee;
  const int64_t ncb = (k + bc - 1) / bc;
  if (unit >= ncb * kMergeWaves * ee * ks) return;
  const int s = (int)(unit % ks);
  const int64_t u1 = unit / ks;
  const int e = (int)(u1 % ee);
  const int64_t u2 = u1 / ee;
  const int w = (int)(u2 % kMergeWaves);
  const int64_t cb = u2 / kMergeWaves;
  const int m = lane & 31;
  const int64_t col = cb * bc + 32 * (ee * w + e) + 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
  const int64_t j0 = 16 * s + 8 * (lane >> 5);
  uint32_t hv[4], lv[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float x[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t j = j0 + 2 * p + q;
      x[q] = (j < r && col < k) ? A[j * k + col] : 0.f;
    }
    const float h0 = (float)(__bf16)x[0], h1 = (float)(__bf16)x[1];
    hv[p] = bf16_pair(h0, h1);
    lv[p] = bf16_pair(x[0] - h0, x[1] - h1);
  }
  uint16_t* dst = P + unit * 1024 + lane * 8;
  *reinterpret_cast<u32x4*>(dst) = u32x4{hv[0], hv[1], hv[2], hv[3]};
  *reinterpret_cast<u32x4*>(dst + 512) = u32x4{lv[0], lv[1], lv[2], lv[3]};
}
}  // namespace

hipError_t launch_pack_merge_projection(int64_t r, int64_t k, const float* A, void* packed,
                                        hipStream_t s) {
  const int ks = merge_rank_steps(r);
  const int ee = ks <= 4 ? 2 : 1;
  const int64_t bc = 32 * kMergeWaves * ee;
  const int64_t threads = (k + bc - 1) / bc * kMergeWaves * ee * ks * 64;
  hipLaunchKernelGGL(pack_merge_projection_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, s, r, k, ks, ee, A, static_cast<uint16_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_pack_update(int64_t d, int64_t r, const float* U, float scale,
                              const float* scale_dev, void* packed, hipStream_t s) {
  const int ks = merge_rank_steps(r);
  const int64_t threads = (d + 31) / 32 * ks * 64;
  hipLaunchKernelGGL(pack_update_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     d, r, ks, scale, scale_dev, U, static_cast<uint16_t*>(packed));
  return hipGetLastError();
}

}  // namespace logra
