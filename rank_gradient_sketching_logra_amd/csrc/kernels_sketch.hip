// Projection regeneration, input projection and sketch accumulation.
//
// Sources: "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches" (paperpeel.com) §2.1 -- the sketch S = G A^T is accumulated per
// microbatch in fp32 by projecting the inputs of the weight-gradient product
// before multiplying by the backward derivatives; §2.2 -- A is regenerated
// from its seed.  "Randomized Gradient Compression" blog, "How it works" --
// the same contraction written C += D^T (X P).
//
// bf16 inputs run on v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  Operand
// layout of that instruction for lane l (half h = l >> 5, i = 0..7):
//   A[m][k]: m = l & 31, k = 8h + i       B[k][n]: k = 8h + i, n = l & 31
//   C[m][n] (16 floats): n = l & 31, m = 8*(reg >> 2) + 4h + (reg & 3)
// Both operands of every product use the same (lane, i) -> k map, so the
// contraction index may be assigned to any token or column as long as A and
// B agree.  fp32 inputs take plain VALU kernels with fp64 accumulation.
#include "device_common.h"
#include "kernels.h"

#include <algorithm>
#include <atomic>
#include <vector>

namespace logra {

namespace {

__device__ __forceinline__ uint64_t pick_word(const Philox4& p, int i) {
  const uint64_t a = (i & 1) ? p.w[1] : p.w[0];
  const uint64_t b = (i & 1) ? p.w[3] : p.w[2];
  return (i & 2) ? b : a;
}

// Four consecutive bf16 of row `row` from column `col` as two words; zero
// outside [0, nrows) x [0, ncols).  col is a multiple of 4 and rows start
// 16-byte aligned, so the whole run is one 8-byte load.
__device__ __forceinline__ void load_bf16x4(const uint16_t* __restrict__ base, int64_t ld,
                                            int64_t row, int64_t col, int64_t nrows,
                                            int64_t ncols, uint32_t& w0, uint32_t& w1) {
  w0 = 0u;
  w1 = 0u;
  if (row >= nrows || col >= ncols) return;
  // X is device memory: read through the global address space, so the loads
  // count on the vector-memory counter only (a flat load also counts on the
  // LDS counter, and every wait for an LDS access would then wait for it).
  typedef __attribute__((address_space(1))) const uint16_t gu16;
  typedef __attribute__((address_space(1))) const u32x2 gu2;
  gu16* p = (gu16*)base + row * ld + col;
  if (col + 4 <= ncols) {
    const u32x2 v = *(gu2*)p;
    w0 = v[0];
    w1 = v[1];
    return;
  }
  uint32_t e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = (col + i < ncols) ? p[i] : 0u;
  w0 = e[0] | (e[1] << 16);
  w1 = e[2] | (e[3] << 16);
}

// X operand of one projection MFMA in the paired column order: for lane
// group g = lane >> 4 and the 32 columns from c32, element 2p holds column
// c32 + 15 - 4g - p and element 2p + 1 column c32 + 31 - 4g - p.  Their
// signs are bits 15 - 4g - p and 31 - 4g - p of the columns' 32-bit Philox
// half-word w, which expand_sign_pairs(w << 4g) places in the same elements.
// Any order of the 32 columns within one MFMA gives the same sum over them
// up to rounding; this one makes the sign expansion two operations per pair.
__device__ __forceinline__ u32x4 load_x_paired(const uint16_t* __restrict__ base, int64_t ld,
                                               int64_t row, int64_t c32, int g, int64_t nrows,
                                               int64_t ncols) {
  uint32_t l0, l1, h0, h1;
  const int64_t c = c32 + 12 - 4 * g;  // runs c .. c+3 and c+16 .. c+19
  load_bf16x4(base, ld, row, c, nrows, ncols, l0, l1);
  load_bf16x4(base, ld, row, c + 16, nrows, ncols, h0, h1);
  u32x4 v;
  v[0] = __builtin_amdgcn_perm(h1, l1, 0x07060302u);  // columns c+3, c+19
  v[1] = __builtin_amdgcn_perm(h1, l1, 0x05040100u);  // c+2, c+18
  v[2] = __builtin_amdgcn_perm(h0, l0, 0x07060302u);  // c+1, c+17
  v[3] = __builtin_amdgcn_perm(h0, l0, 0x05040100u);  // c, c+16
  return v;
}

// Eight consecutive columns of one row of X as one 16-byte load, for ncols a
// multiple of 8 and rows 16-byte aligned (each group of eight columns lies
// wholly inside or outside the matrix; a group outside, or a row past nrows,
// reads sixteen zero bytes).
__device__ const u32x4 kZeroX8 = {0u, 0u, 0u, 0u};
__device__ __forceinline__ u32x4 load_x8(const uint16_t* __restrict__ base, int64_t ld,
                                         int64_t row, int64_t col, int64_t nrows,
                                         int64_t ncols) {
  typedef __attribute__((address_space(1))) const uint16_t gu16;
  typedef __attribute__((address_space(1))) const u32x4 gu4;
  const bool ok = row < nrows && col < ncols;
  return *(ok ? (gu4*)((gu16*)base + row * ld + col) : (gu4*)&kZeroX8);
}
// Bits 0, 2, .., 30 of x in bits 0 .. 15.
__device__ __forceinline__ uint32_t even_bits(uint32_t x) {
  x &= 0x55555555u;
  x = (x | (x >> 1)) & 0x33333333u;
  x = (x | (x >> 2)) & 0x0F0F0F0Fu;
  x = (x | (x >> 4)) & 0x00FF00FFu;
  return (x | (x >> 8)) & 0x0000FFFFu;
}
// The sign word of 32 columns (bit j: column j) rearranged for operands in
// the consecutive column order: bit 15 - i takes column 2i and bit 31 - i
// column 2i + 1, so that expand_sign_pairs(w << 4g) gives the signs of
// columns 8g .. 8g + 7 in element order, matching one 16-byte load of X.
__device__ __forceinline__ uint32_t sign_word_consecutive(uint32_t w) {
  return __builtin_bitreverse32(even_bits(w >> 1) | (even_bits(w) << 16));
}

// Eight consecutive bf16 of row `row` starting at column `col`; zero outside
// [0, nrows) x [0, ncols).  Rows start 16-byte aligned (checked on the host).
__device__ __forceinline__ u32x4 load_bf16x8(const uint16_t* __restrict__ base, int64_t ld,
                                             int64_t row, int64_t col, int64_t nrows,
                                             int64_t ncols) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row >= nrows || col >= ncols) return v;
  const uint16_t* p = base + row * ld + col;
  if (col + 8 <= ncols) return *reinterpret_cast<const u32x4*>(p);
  uint32_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = (col + i < ncols) ? p[i] : 0u;
  v[0] = e[0] | (e[1] << 16);
  v[1] = e[2] | (e[3] << 16);
  v[2] = e[4] | (e[5] << 16);
  v[3] = e[6] | (e[7] << 16);
  return v;
}

// Block index -> logical tile so that consecutive logical tiles run on the
// same XCD (blocks are dispatched round-robin over the 8 XCDs).  gridDim.x
// is a multiple of 8.
__device__ __forceinline__ int64_t xcd_logical_block() {
  const int64_t per = gridDim.x >> 3;
  return (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
}

// ------------------------------------------------------------- regen A

__global__ void regen_A_kernel(KeyArg key, int64_t r, int64_t k, int int8_out, float cr,
                               void* __restrict__ A) {
  const int64_t kq = (k + 3) >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= r * kq) return;
  const int64_t j = idx / kq;
  const int64_t l0 = (idx - j * kq) * 4;
  const Philox4 p = sigma_block(KeyWords{key.k0, key.k1}, (uint64_t)j, (uint64_t)(l0 >> 8));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t l = l0 + q;
    if (l >= k) break;
    const uint32_t bit = (uint32_t)(pick_word(p, (int)((l & 255) >> 6)) >> (l & 63)) & 1u;
    if (int8_out)
      static_cast<int8_t*>(A)[j * k + l] = bit ? (int8_t)-1 : (int8_t)1;
    else
      static_cast<float*>(A)[j * k + l] = bit ? -cr : cr;
  }
}

// Gaussian projection variant: A[j][l] = fl32(z / sqrt(r)), z from
// gaussian_block; one thread per row and 4-column group.
__global__ void regen_A_gaussian_kernel(KeyArg key, int64_t r, int64_t k, float* __restrict__ A) {
  const int64_t ng = (k + 3) >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= r * ng) return;
  const int64_t j = idx / ng;
  const int64_t c = idx - j * ng;
  double z[4];
  gaussian_block(KeyWords{key.k0, key.k1}, (uint64_t)j, (uint64_t)c, z);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t l = 4 * c + q;
    if (l < k) A[j * k + l] = (float)(z[q] / sqrt((double)r));
  }
}

// An explicit projection A [r x k] (fp32, row-major) as the projection
// kernel's B operands: for 256-column block b, 32-column step s (8 per
// block) and 16-rank block nb (NB16 of them), a 1 KiB hi slab then a 1 KiB lo
// slab, lane l holding rank 16nb + (l & 15), columns 256b + 32s + 8(l >> 4)
// .. +7 as bf16 hi = RNE(a), lo = RNE(a - hi); ranks >= r and columns >= k
// are zero.  One thread per (b, s, nb, lane).
__global__ __launch_bounds__(256) void pack_projection_kernel(int64_t r, int64_t k, int nb16,
                                                              const float* __restrict__ A,
                                                              uint16_t* __restrict__ P) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lane = (int)(t & 63);
  const int64_t unit = t >> 6;                 // (b * 8 + s) * nb16 + nb
  const int64_t nblk = (k + 255) >> 8;
  if (unit >= nblk * 8 * nb16) return;
  const int nb = (int)(unit % nb16);
  const int64_t bs = unit / nb16;
  const int64_t j = 16 * nb + (lane & 15);
  const int64_t c0 = 32 * bs + 8 * (lane >> 4);  // 256 b + 32 s + 8 (l >> 4)
  uint32_t hv[4], lv[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float x[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t c = c0 + 2 * p + q;
      x[q] = (j < r && c < k) ? A[j * k + c] : 0.f;
    }
    const __bf16 h0 = (__bf16)x[0], h1 = (__bf16)x[1];
    const __bf16 l0 = (__bf16)(x[0] - (float)h0), l1 = (__bf16)(x[1] - (float)h1);
    hv[p] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    lv[p] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  }
  uint16_t* dst = P + (unit * 2) * 512 + lane * 8;
  *reinterpret_cast<u32x4*>(dst) = u32x4{hv[0], hv[1], hv[2], hv[3]};
  *reinterpret_cast<u32x4*>(dst + 512) = u32x4{lv[0], lv[1], lv[2], lv[3]};
}

// ------------------------------------------------------------- project

// bf16 X: one block = 16 tokens (one 16-token step of the packed form) x
// all ranks.  Its eight waves take the 256-column blocks of k round-robin,
// each with the loads of its next block in flight while it computes the
// current one, then add their partial tiles in a fixed order.  The product is
// v_mfma_f32_16x16x32_bf16: A lane l holds token t0 + (l & 15) and eight of
// the columns 32s .. 32s + 31 of the 256-column block (s = 0..7) in the
// paired order of load_x_paired (the explicit-projection path: columns
// 32s + 8(l >> 4) .. +7); B lane l holds the signs of rank 16nb + (l & 15)
// for the same columns, expanded from the Philox words of the lane that
// generated that rank; C lane l holds rank
// 16nb + (l & 15) of tokens t0 + 4(l >> 4) + j in register j.  NB16 =
// 16-rank blocks computed (>= r / 16).
constexpr int kProjTokens = 16;
constexpr int kProjWaves = 8;
constexpr int kProjTableMax = 1024;  // projections in one table launch

// EXPLICIT: the B operands come from an explicit projection packed as bf16
// hi/lo operands (see pack_projection_kernel) instead of sign bits: two MFMAs
// (hi, lo) per operand, no sign generation; cr is then 1.
template <int NB16, bool EXPLICIT>
__global__ __launch_bounds__(kProjWaves * 64) void project_bf16_kernel(
    KeyArg key, int64_t T, int64_t k, int64_t r, const uint16_t* __restrict__ X, int64_t ldx,
    float cr, float* __restrict__ XAt, uint16_t* __restrict__ planes, int nrb, int nsteps,
    const uint16_t* __restrict__ Ap) {
  constexpr int NQ = (NB16 + 3) / 4;  // 64-rank groups, one Philox block per lane each
  constexpr int RP = NB16 * 16;
  __shared__ float red[kProjTokens][RP + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g4 = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kProjTokens;
  const int64_t trow = t0 + (lane & 15);
  const KeyWords kw{key.k0, key.k1};

  f32x4 acc[NB16];
#pragma unroll
  for (int nb = 0; nb < NB16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t nblk = (k + 255) >> 8;
  u32x4 a[8];
  auto load = [&](int64_t b, u32x4 (&dst)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      dst[s] = EXPLICIT ? load_bf16x8(X, ldx, trow, b * 256 + 32 * s + 8 * g4, T, k)
                        : load_x_paired(X, ldx, trow, b * 256 + 32 * s, g4, T, k);
  };
  if (wave < nblk) load(wave, a);
  for (int64_t b = wave; b < nblk; b += kProjWaves) {
    u32x4 an[8];
    if (b + kProjWaves < nblk) load(b + kProjWaves, an);
    if constexpr (EXPLICIT) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int nb = 0; nb < NB16; ++nb) {
          const uint16_t* ap = Ap + (((b * 8 + s) * NB16 + nb) * 2) * 512 + lane * 8;
          const u32x4 bh = *reinterpret_cast<const u32x4*>(ap);
          const u32x4 bl = *reinterpret_cast<const u32x4*>(ap + 512);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[s]), as_bf16x8(bh), acc[nb],
                                                            0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[s]), as_bf16x8(bl), acc[nb],
                                                            0, 0, 0);
        }
      }
    } else {
      uint32_t bits[NQ][8];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int64_t j = lane + 64 * q;
        const Philox4 p = sigma_block(kw, (uint64_t)j, (uint64_t)b);
        const bool live = j < r;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          bits[q][2 * w] = live ? (uint32_t)p.w[w] : 0u;
          bits[q][2 * w + 1] = live ? (uint32_t)(p.w[w] >> 32) : 0u;
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int nb = 0; nb < NB16; ++nb) {
          const int src = 16 * (nb & 3) + (lane & 15);
          const uint32_t wv = (uint32_t)__shfl((int)bits[nb >> 2][s], src, 64);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(a[s]), as_bf16x8(expand_sign_pairs(wv << (4 * g4))), acc[nb], 0, 0, 0);
        }
      }
    }
    if (b + kProjWaves < nblk) {
#pragma unroll
      for (int s = 0; s < 8; ++s) a[s] = an[s];
    }
  }

  // Fixed-order reduction over the eight waves: (((w0 + w1) + w2) + ...) + w7.
  for (int w = 0; w < kProjWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = 4 * g4 + j;
          const int n = nb * 16 + (lane & 15);
          red[m][n] = (w == 0) ? acc[nb][j] : red[m][n] + acc[nb][j];
        }
    }
    __syncthreads();
  }
  if (XAt) {
    for (int idx = threadIdx.x; idx < kProjTokens * r; idx += kProjWaves * 64) {
      const int m = idx / (int)r;
      const int j = idx - m * (int)r;
      const int64_t t = t0 + m;
      if (t < T) XAt[t * r + j] = red[m][j] * cr;
    }
  }
  if (planes && blockIdx.x < nsteps) {
    // This block's 16-token step in the accumulate's operand order: wave b
    // writes 32-rank block b, lane l holding tokens 8(l>>5) + i of rank
    // 32b + (l & 31) as hi and lo bf16 terms.  Rows past T are zero (X reads
    // past T are zero); ranks past r are written as zero.
    for (int b = wave; b < nrb; b += kProjWaves) {
      const int j = 32 * b + (lane & 31);
      float hv[8], lv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = j < r ? red[8 * (lane >> 5) + i][j] * cr : 0.f;
        hv[i] = (float)(__bf16)v;
        lv[i] = v - hv[i];
      }
      u32x4 vh, vl;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        vh[p] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[2 * p]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[2 * p + 1]) << 16);
        vl[p] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lv[2 * p]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lv[2 * p + 1]) << 16);
      }
      uint16_t* dst = planes + ((int64_t)blockIdx.x * nrb + b) * 1024 + lane * 8;
      __builtin_nontemporal_store(vh, reinterpret_cast<u32x4*>(dst));
      __builtin_nontemporal_store(vl, reinterpret_cast<u32x4*>(dst + 512));
    }
  }
}

}  // namespace

// Projections that read one input X, up to this many to an entry (at most
// 64 ranks; one above).
constexpr int kProjFuse = 3;

// One entry of a table-driven projection (device memory): np projections of
// the same input X, each with its own A and outputs; entry n holds only
// item_begin = the total number of work items.
struct ProjTableEntry {
  const uint16_t* X;              // bf16 [T x k], leading dimension ldx
  float* XAt[kProjFuse];          // fp32 [T x r] or null
  uint16_t* planes[kProjFuse];    // packed projected input or null
  uint64_t k0[kProjFuse], k1[kProjFuse];  // key words of each projection's A
  int64_t ldx, k, item_begin;
  int np;
};

namespace {

constexpr int kPtWaves = 4;  // waves per block of the table projection

// Persistent projection over a device-resident table of projections (e.g.
// every projection of every layer for one microbatch).  The work items are
// (entry, TS consecutive 16-token steps) in table order, an entry being up to
// NPF projections of one input (q, k and v of a layer; gate and up), so X is
// read once for all of them; each wave takes one item at a
// time and computes it whole -- all k columns, all ranks -- so no two waves
// share a result and nothing is exchanged between waves.  An item holds two
// token steps, which share each expanded sign operand (the generation, the
// lane exchange and the expansion are VALU work that does not depend on the
// tokens).  Wave w of block b
// starts at item 4b + w and then takes the next unclaimed item from a
// counter, so items are handed out in order and the fast waves take more.
// Per item: for each 256-column block in order, the next block's X loads in
// flight, the signs of the lane's rank (one Philox block per 64 ranks)
// expanded in the paired column order (X16: the inputs as 16-byte loads of
// eight consecutive columns, the sign words rearranged to match), eight
// 16x16x32 MFMA steps per token step; the sums
// run over the column blocks in ascending order in one accumulator.  The
// tile then goes through the wave's own LDS rows to the fp32 output and/or
// the accumulate's packed operand form, as in project_bf16_kernel.  The
// column blocks' partial sums are added in another order than in
// project_bf16_kernel, so the two differ in the last bits; each is
// deterministic.
// Token steps per work item of the table projection.
constexpr int kProjTableSteps = 2;

template <int NB16, bool X16>
__global__ __launch_bounds__(kPtWaves * 64)
__attribute__((amdgpu_waves_per_eu(2))) void project_table_kernel(
    const ProjTableEntry* __restrict__ tab, unsigned* __restrict__ next, int n, int64_t T,
    int64_t r, float cr, int nrb) {
  constexpr int NQ = (NB16 + 3) / 4;
  constexpr int RP = NB16 * 16;
  constexpr int NPF = NB16 <= 4 ? kProjFuse : 1;  // projections an entry may hold
  constexpr int TS = kProjTableSteps;
  __shared__ int64_t begin_s[kProjTableMax + 1];
  __shared__ float red[kPtWaves][kProjTokens][RP + 1];
  for (int i = threadIdx.x; i <= n; i += blockDim.x) begin_s[i] = tab[i].item_begin;
  __syncthreads();  // the only block-wide barrier: waves run independently below
  const int64_t total = begin_s[n];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t grid_waves = (int64_t)gridDim.x * kPtWaves;
  int64_t item = (int64_t)blockIdx.x * kPtWaves + wave;
  while (item < total) {
    // The lane index is opaque per item, so that lane-derived addresses are
    // not hoisted out of the item loop and held in registers throughout.
    int lane_o = threadIdx.x & 63;
    asm volatile("" : "+v"(lane_o));
    const int lane = lane_o;
    const int g4 = lane >> 4;
    float (*rw)[RP + 1] = red[wave];
    // Claim the wave's following item now; the value is needed only when
    // this one is done.  The address is opaque per lane so that the atomic is
    // not turned into a wave-wide form that waits for its result at once.
    unsigned claim = 0;
    if (lane == 0) {
      int lane_o = lane;
      asm volatile("" : "+v"(lane_o));
      claim = atomicAdd(next + lane_o, 1u);
    }
    int lo = 0, hi = n - 1;  // the entry holding the item
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (begin_s[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const ProjTableEntry& e = tab[lo];
    const uint16_t* __restrict__ X = e.X;
    const int64_t ldx = e.ldx, k = e.k;
    const int np = e.np;
    const int64_t st0 = (item - begin_s[lo]) * TS;  // the item's first token step
    const int64_t trow = st0 * kProjTokens + (lane & 15);

    f32x4 acc[TS][NPF][NB16];
#pragma unroll
    for (int h = 0; h < TS; ++h)
#pragma unroll
      for (int pj = 0; pj < NPF; ++pj)
#pragma unroll
        for (int nb = 0; nb < NB16; ++nb) acc[h][pj][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t nblk = (k + 255) >> 8;
    // Rows at or beyond T load as zeros (a last step past T is never stored).
    auto load = [&](int64_t b, u32x4 (&dst)[TS][8]) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < TS; ++h)
#pragma unroll
        for (int s = 0; s < 8; ++s)
          dst[h][s] = X16 ? load_x8(X, ldx, trow + h * kProjTokens, b * 256 + 32 * s + 8 * g4, T, k)
                          : load_x_paired(X, ldx, trow + h * kProjTokens, b * 256 + 32 * s, g4, T, k);
    };
    // With one token step per item the next block's X loads would be in
    // flight during this block's work; with two the block's own loads are
    // issued first and are in flight while the first projection's signs are
    // generated (registers for a second set are not there).
    constexpr bool kAhead = TS == 1;
    u32x4 a[TS][8];
    if constexpr (kAhead) load(0, a);
    for (int64_t b = 0; b < nblk; ++b) {
      u32x4 an[TS][8];
      if constexpr (kAhead) {
        if (b + 1 < nblk) load(b + 1, an);
      } else {
        load(b, a);
      }
#pragma unroll
      for (int pj = 0; pj < NPF; ++pj) {
        if (pj >= np) break;  // uniform per wave
        const KeyWords kw{e.k0[pj], e.k1[pj]};
        // One 64-rank quarter at a time: its signs, then its MFMAs (each
        // accumulator still takes the eight column steps in order).
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int64_t j = lane + 64 * q;
          const Philox4 p = sigma_block(kw, (uint64_t)j, (uint64_t)b);
          const bool live = j < r;
          uint32_t bits[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            bits[2 * w] = live ? (uint32_t)p.w[w] : 0u;
            bits[2 * w + 1] = live ? (uint32_t)(p.w[w] >> 32) : 0u;
          }
          if constexpr (X16) {
#pragma unroll
            for (int w = 0; w < 8; ++w) bits[w] = sign_word_consecutive(bits[w]);
          }
#pragma unroll
          for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int nb = 4 * q; nb < 4 * q + 4 && nb < NB16; ++nb) {
              const int src = 16 * (nb & 3) + (lane & 15);
              const uint32_t wv = (uint32_t)__shfl((int)bits[s], src, 64);
              const bf16x8 sg = as_bf16x8(expand_sign_pairs(wv << (4 * g4)));
#pragma unroll
              for (int h = 0; h < TS; ++h)
                acc[h][pj][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(a[h][s]), sg, acc[h][pj][nb], 0, 0, 0);
            }
          }
        }
      }
      if (kAhead && b + 1 < nblk) {
#pragma unroll
        for (int h = 0; h < TS; ++h)
#pragma unroll
          for (int s = 0; s < 8; ++s) a[h][s] = an[h][s];
      }
    }

    // Each projection's tile through the wave's own LDS rows (a wave's LDS
    // accesses take effect in program order, so no barrier is needed), one
    // token step at a time.
#pragma unroll
    for (int h = 0; h < TS; ++h) {
    const int64_t st = st0 + h;
    const int64_t t0 = st * kProjTokens;
    if (t0 >= T) break;  // uniform per wave
#pragma unroll
    for (int pj = 0; pj < NPF; ++pj) {
    if (pj >= np) break;  // uniform per wave
#pragma unroll
    for (int nb = 0; nb < NB16; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) rw[4 * g4 + j][nb * 16 + (lane & 15)] = acc[h][pj][nb][j];
    asm volatile("" ::: "memory");
    if (e.XAt[pj]) {
      float* __restrict__ XAt = e.XAt[pj];
      for (int idx = lane; idx < kProjTokens * r; idx += 64) {
        const int m = idx / (int)r;
        const int j = idx - m * (int)r;
        const int64_t t = t0 + m;
        if (t < T) __builtin_nontemporal_store(rw[m][j] * cr, XAt + t * r + j);
      }
    }
    if (e.planes[pj]) {
      for (int b = 0; b < nrb; ++b) {
        const int j = 32 * b + (lane & 31);
        float hv[8], lv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = j < r ? rw[8 * (lane >> 5) + i][j] * cr : 0.f;
          hv[i] = (float)(__bf16)v;
          lv[i] = v - hv[i];
        }
        u32x4 vh, vl;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          vh[p] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[2 * p]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[2 * p + 1]) << 16);
          vl[p] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lv[2 * p]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lv[2 * p + 1]) << 16);
        }
        // non-temporal: the planes are read by a later launch, not from L2
        uint16_t* dst = e.planes[pj] + (st * nrb + b) * 1024 + lane * 8;
        __builtin_nontemporal_store(vh, reinterpret_cast<u32x4*>(dst));
        __builtin_nontemporal_store(vl, reinterpret_cast<u32x4*>(dst + 512));
      }
    }
    asm volatile("" ::: "memory");  // this tile's LDS reads before the next tile's writes
    }
    }
    item = grid_waves + (int64_t)__builtin_amdgcn_readfirstlane(claim);
  }
}

// Block-wide projection for more than 64 ranks (one projection per entry).
// A work item is (entry, 256 consecutive tokens); the eight waves of the
// block take two 16-token steps each, so the signs of every 256-column block
// are generated once per 256 tokens and shared by the block, instead of once
// per two steps as in project_table_kernel, where their generation and
// expansion outweighed the matrix work.  The chunks c = (column block b,
// 32-column step s) run in order with one block barrier each; iteration c
//   generates column block b + 1's sign words when s = 0 (one Philox4x32-10
//   per thread: the low or high half of sigma_block for one rank),
//   expands chunk c + 1's words into MFMA operands (two per thread),
//   loads the inputs of chunk c + 3 (a ring of four chunks in registers),
//   and runs chunk c's MFMAs with the operands from LDS,
// in double-buffered LDS areas, each written one barrier or more after its
// last read.  Every accumulator takes the same MFMAs with the same operands
// in the same order as in project_table_kernel ((b, s) ascending), so the
// outputs are identical.
constexpr int kPbWaves = 8;
constexpr int kPbSteps = 2;                                        // token steps per wave
constexpr int kPbTokens = kPbWaves * kPbSteps * kProjTokens;       // tokens per item
constexpr int kPbAhead = 3;                                        // chunks of inputs in flight

template <int NB16>
__global__ __launch_bounds__(kPbWaves * 64, 1) void project_blocked_kernel(
    const ProjTableEntry* __restrict__ tab, unsigned* __restrict__ next, int n, int64_t T,
    int64_t r, float cr, int nrb) {
  static_assert(NB16 >= 5 && NB16 <= 16, "more than 64 ranks, at most 256");
  constexpr int RP = NB16 * 16;
  constexpr int TS = kPbSteps;
  constexpr int XR = kPbAhead + 1;  // input ring slots
  static_assert(8 % XR == 0, "chunk c sits in slot s % XR, s = c mod 8: XR must divide 8");
  // sign words [buffer][rank][word]; operands [buffer][rank block][lane]
  constexpr int kWordsBytes = 2 * RP * 8 * 4;
  constexpr int kOpsBytes = 2 * NB16 * 64 * 16;
  constexpr int kRedBytes = kPbWaves * kProjTokens * (RP + 1) * 4;  // the epilogue's rows
  constexpr int kLds = kWordsBytes + kOpsBytes > kRedBytes ? kWordsBytes + kOpsBytes : kRedBytes;
  __shared__ __align__(16) unsigned char lds[kLds];
  __shared__ int64_t begin_s[kProjTableMax + 1];
  __shared__ unsigned claim_s;
  uint32_t (*words)[RP][8] = reinterpret_cast<uint32_t (*)[RP][8]>(lds);
  u32x4 (*ops)[NB16][64] = reinterpret_cast<u32x4 (*)[NB16][64]>(lds + kWordsBytes);
  for (int i = threadIdx.x; i <= n; i += blockDim.x) begin_s[i] = tab[i].item_begin;
  __syncthreads();
  const int64_t total = begin_s[n];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t item = blockIdx.x;
  while (item < total) {  // uniform per block
    int lane_o = threadIdx.x & 63;
    asm volatile("" : "+v"(lane_o));
    const int lane = lane_o;
    const int g4 = lane >> 4;
    if (threadIdx.x == 0) claim_s = atomicAdd(next, 1u);  // read after the item's last barrier
    int lo = 0, hi = n - 1;  // the entry holding the item
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (begin_s[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const ProjTableEntry& e = tab[lo];
    const uint16_t* __restrict__ X = e.X;
    const int64_t ldx = e.ldx, k = e.k;
    const uint32_t s0 = (uint32_t)e.k0[0], s1 = (uint32_t)(e.k0[0] >> 32);
    const uint32_t mid = (uint32_t)e.k1[0], stp = (uint32_t)(e.k1[0] >> 32);
    const int64_t st0 = (item - begin_s[lo]) * (kPbWaves * TS) + wave * TS;  // the wave's first step
    const int64_t trow = st0 * kProjTokens + (lane & 15);
    const int64_t nblk = (k + 255) >> 8;
    const int64_t nch = nblk * 8;
    // Column block b's sign words: thread t computes half t & 1 of
    // sigma_block for rank t >> 1 (words 0..3 the low half, 4..7 the high).
    auto gen = [&](int64_t b) __attribute__((always_inline)) {
      const int j = (int)(threadIdx.x >> 1), half = (int)(threadIdx.x & 1);
      if (j < RP) {
        const Philox4x32 p =
            philox4x32_10((uint32_t)(2 * b + half), (uint32_t)j | 0x80000000u, mid, stp, s0, s1);
        const bool live = j < r;
#pragma unroll
        for (int i = 0; i < 4; ++i) words[b & 1][j][4 * half + i] = live ? p.w[i] : 0u;
      }
    };
    // Chunk c's operands: rank blocks 2w and 2w + 1 of wave w, the lane's rank
    // 16 nb + (l & 15) holding the step's 32 columns in the consecutive order
    // (lane group g: columns 8g .. 8g + 7), as the X operand holds them.
    auto expand = [&](int64_t c) __attribute__((always_inline)) {
      const int64_t b = c >> 3;
      const int s = (int)(c & 7);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int nb = 2 * wave + i;
        if (nb < NB16) {  // uniform
          const uint32_t wv = words[b & 1][16 * nb + (lane & 15)][s];
          ops[c & 1][nb][lane] = expand_sign_pairs(sign_word_consecutive(wv) << (4 * g4));
        }
      }
    };
    auto load_chunk = [&](int64_t c, u32x4 (&x)[TS]) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < TS; ++h)
        x[h] = load_x8(X, ldx, trow + h * kProjTokens, (c >> 3) * 256 + 32 * (c & 7) + 8 * g4, T, k);
    };
    f32x4 acc[TS][NB16];
#pragma unroll
    for (int h = 0; h < TS; ++h)
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb) acc[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Loaded words of chunk c in slot c % XR.  Every wave loads and computes
    // every chunk with no branch around the loads (loads in branches are
    // waited for in full): a wave past T loads zeros and its sums are never
    // stored, and loads past the last chunk repeat it and are not used.
    u32x4 xr[XR][TS];
#pragma unroll
    for (int c = 0; c < kPbAhead; ++c) load_chunk(c < nch ? c : nch - 1, xr[c]);
    gen(0);
    __syncthreads();
    expand(0);
    __syncthreads();
    for (int64_t b = 0; b < nblk; ++b) {
      // the step is a constant in each copy of the body, and so is every
      // ring slot
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int64_t c = 8 * b + s;
        if (s == 0 && b + 1 < nblk) gen(b + 1);
        if (c + 1 < nch) expand(c + 1);
        load_chunk(c + kPbAhead < nch ? c + kPbAhead : nch - 1, xr[(s + kPbAhead) % XR]);
#pragma unroll
        for (int nb = 0; nb < NB16; ++nb) {
          const u32x4 op = ops[c & 1][nb][lane];
#pragma unroll
          for (int h = 0; h < TS; ++h)
            acc[h][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xr[s % XR][h]),
                                                                 as_bf16x8(op), acc[h][nb], 0, 0, 0);
        }
        __syncthreads();
      }
    }
    // Each wave's tile through its own LDS rows, as in project_table_kernel.
    float (*rw)[RP + 1] = reinterpret_cast<float (*)[RP + 1]>(lds) + wave * kProjTokens;
#pragma unroll
    for (int h = 0; h < TS; ++h) {
      const int64_t st = st0 + h;
      const int64_t t0 = st * kProjTokens;
      if (t0 >= T) break;  // uniform per wave
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) rw[4 * g4 + j][nb * 16 + (lane & 15)] = acc[h][nb][j];
      asm volatile("" ::: "memory");
      if (e.XAt[0]) {
        float* __restrict__ XAt = e.XAt[0];
        for (int idx = lane; idx < kProjTokens * r; idx += 64) {
          const int m = idx / (int)r;
          const int j = idx - m * (int)r;
          const int64_t t = t0 + m;
          if (t < T) __builtin_nontemporal_store(rw[m][j] * cr, XAt + t * r + j);
        }
      }
      if (e.planes[0]) {
        for (int bb = 0; bb < nrb; ++bb) {
          const int j = 32 * bb + (lane & 31);
          float hv[8], lv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float v = j < r ? rw[8 * (lane >> 5) + i][j] * cr : 0.f;
            hv[i] = (float)(__bf16)v;
            lv[i] = v - hv[i];
          }
          u32x4 vh, vl;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            vh[p] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[2 * p]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[2 * p + 1]) << 16);
            vl[p] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lv[2 * p]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lv[2 * p + 1]) << 16);
          }
          uint16_t* dst = e.planes[0] + (st * nrb + bb) * 1024 + lane * 8;
          __builtin_nontemporal_store(vh, reinterpret_cast<u32x4*>(dst));
          __builtin_nontemporal_store(vl, reinterpret_cast<u32x4*>(dst + 512));
        }
      }
      asm volatile("" ::: "memory");  // this step's LDS reads before the next step's writes
    }
    __syncthreads();  // the rows are read; the next item's words may be written
    item = (int64_t)gridDim.x + (int64_t)claim_s;
    __syncthreads();  // every thread has read claim_s before the next item rewrites it
  }
}

// fp32 X: one thread per (token, rank); fp64 sum of signed inputs.
__global__ void project_f32_kernel(KeyArg key, int64_t T, int64_t k, int64_t r,
                                   const float* __restrict__ X, int64_t ldx, double cr,
                                   float* __restrict__ XAt) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * r) return;
  const int64_t t = idx / r;
  const int64_t j = idx - t * r;
  const KeyWords kw{key.k0, key.k1};
  double acc = 0.0;
  for (int64_t b = 0; b * 256 < k; ++b) {
    const Philox4 p = sigma_block(kw, (uint64_t)j, (uint64_t)b);
    for (int w = 0; w < 4; ++w) {
      const uint64_t word = pick_word(p, w);
      for (int bit = 0; bit < 64; ++bit) {
        const int64_t l = b * 256 + w * 64 + bit;
        if (l >= k) break;
        const double x = (double)X[t * ldx + l];
        acc += ((word >> bit) & 1ull) ? -x : x;
      }
    }
  }
  XAt[t * r + j] = (float)(acc * cr);
}

// ---------------------------------------------------------- accumulate

// Packed projected input.  XAt is split into two bf16 terms, hi = RNE(x) and
// lo = RNE(x - hi), laid out in MFMA B-operand order for
// v_mfma_f32_32x32x16_bf16: for 16-token step s and 32-rank block b, two
// 1 KiB operands (hi then lo) in which lane l holds tokens 16s + 8(l>>5) + i
// (i = 0..7) of rank 32b + (l & 31).  One wave reads one operand with one
// fully contiguous 16-byte-per-lane load.  Tokens >= T and ranks >= r are 0.
constexpr int kAccStep = 16;        // tokens per MFMA step
constexpr int kAccCols = 256;       // columns of D per block: 32 lanes x 8
constexpr int kAccWaves = 8;        // waves per block: rank blocks x token classes
constexpr int kAccBAhead = 2;       // 256 ranks: steps the B operands are loaded ahead

struct AccGroupArgs {
  const void* D[kMaxGroup];
  const float* XAt[kMaxGroup];
  float* S[kMaxGroup];
  uint16_t* planes[kMaxGroup];  // packed XAt of each item (workspace)
  int pack[kMaxGroup];          // 0: item shares an earlier item's XAt and planes
  int64_t d[kMaxGroup];
  int64_t ldd[kMaxGroup];
  int64_t nq[kMaxGroup];        // 256-column blocks of each item
  int64_t tile_begin[kMaxGroup + 1];
  int n;
  int64_t T, r;
  int nsteps;   // ceil(T / 16)
  int nrb;      // 32-rank blocks packed: ceil(r / 32) rounded up to 1, 2, 4 or 8
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// One wave per (step, rank block) of one item.
__global__ __launch_bounds__(256) void acc_pack_kernel(AccGroupArgs g) {
  const int item = blockIdx.y;
  if (!g.pack[item]) return;
  const int64_t chunk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (chunk >= (int64_t)g.nsteps * g.nrb) return;
  const int lane = threadIdx.x & 63;
  const int64_t s = chunk / g.nrb;
  const int64_t b = chunk - s * g.nrb;
  const int64_t j = 32 * b + (lane & 31);
  const int64_t t0 = kAccStep * s + 8 * (lane >> 5);
  const float* __restrict__ x = g.XAt[item];
  float h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = (t0 + i < g.T && j < g.r) ? x[(t0 + i) * g.r + j] : 0.f;
    const __bf16 hb = (__bf16)v;
    h[i] = (float)hb;
    l[i] = v - h[i];
  }
  u32x4 vh, vl;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    vh[p] = pack_bf16x2(h[2 * p], h[2 * p + 1]);
    vl[p] = pack_bf16x2(l[2 * p], l[2 * p + 1]);
  }
  uint16_t* dst = g.planes[item] + chunk * 1024 + lane * 8;
  __builtin_nontemporal_store(vh, reinterpret_cast<u32x4*>(dst));
  __builtin_nontemporal_store(vl, reinterpret_cast<u32x4*>(dst + 512));
}

// Eight bf16 of row t of D from column col; zero outside the matrix.
__device__ __forceinline__ u32x4 load_drow(const uint16_t* __restrict__ D, int64_t ldd,
                                           int64_t t, int64_t T, int64_t col, int64_t d,
                                           bool full) {
  if (t >= T || col >= d) return u32x4{0u, 0u, 0u, 0u};
  const uint16_t* p = D + t * ldd + col;
  if (full) return *reinterpret_cast<const u32x4*>(p);
  uint32_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = (col + i < d) ? p[i] : 0u;
  return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
               e[6] | (e[7] << 16)};
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their
// maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0) with the other counters unconstrained.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Transpose of a lane's 8 x 8 block of bf16 (row[i] = eight columns of token
// i), one operand: the eight tokens of column e, as one MFMA operand.  Each
// output word takes one 16-bit half from each of two rows (one byte permute).
__device__ __forceinline__ u32x4 transpose8x8_e(const u32x4 (&row)[8], int e) {
  const int q = e >> 1;
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  u32x4 a;
#pragma unroll
  for (int p = 0; p < 4; ++p) a[p] = __builtin_amdgcn_perm(row[2 * p + 1][q], row[2 * p][q], sel);
  return a;
}
// The whole transpose: a[e] for e = 0..7.
__device__ __forceinline__ void transpose8x8(const u32x4 (&row)[8], u32x4 (&a)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = transpose8x8_e(row, e);
}

// 32-bit LDS address of a shared-memory object.
template <typename Tp>
__device__ __forceinline__ uint32_t lds_addr(Tp* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) Tp*)p;
}

// LDS reads that complete inside the statement: the compiler never sees an
// LDS read it could order against pending direct global->LDS loads, and the
// results exist only once the data has arrived.  The outputs are
// early-clobber: a destination sharing a register with the address would be
// overwritten by the first read's data while later reads still use it.
//
// One step's operands: eight 1 KiB row slabs at ad and two 1 KiB B operands
// (hi, lo) at ab; lane l's 16 bytes at byte 16 l of each slab.
__device__ __forceinline__ void acc_read_step(uint32_t ad, uint32_t ab, u32x4 (&row)[8],
                                              u32x4& bh, u32x4& bl) {
  asm volatile(
      "ds_read_b128 %0, %10\n\t"
      "ds_read_b128 %1, %10 offset:1024\n\t"
      "ds_read_b128 %2, %10 offset:2048\n\t"
      "ds_read_b128 %3, %10 offset:3072\n\t"
      "ds_read_b128 %4, %10 offset:4096\n\t"
      "ds_read_b128 %5, %10 offset:5120\n\t"
      "ds_read_b128 %6, %10 offset:6144\n\t"
      "ds_read_b128 %7, %10 offset:7168\n\t"
      "ds_read_b128 %8, %11\n\t"
      "ds_read_b128 %9, %11 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(row[0]), "=&v"(row[1]), "=&v"(row[2]), "=&v"(row[3]), "=&v"(row[4]),
        "=&v"(row[5]), "=&v"(row[6]), "=&v"(row[7]), "=&v"(bh), "=&v"(bl)
      : "v"(ad), "v"(ab)
      : "memory");
}
// The same ten reads, issued only: the destinations are not valid until
// acc_read_wait() (which names them, so nothing reads them before it).
__device__ __forceinline__ void acc_read_issue(uint32_t ad, uint32_t ab, u32x4 (&row)[8],
                                               u32x4& bh, u32x4& bl) {
  asm volatile(
      "ds_read_b128 %0, %10\n\t"
      "ds_read_b128 %1, %10 offset:1024\n\t"
      "ds_read_b128 %2, %10 offset:2048\n\t"
      "ds_read_b128 %3, %10 offset:3072\n\t"
      "ds_read_b128 %4, %10 offset:4096\n\t"
      "ds_read_b128 %5, %10 offset:5120\n\t"
      "ds_read_b128 %6, %10 offset:6144\n\t"
      "ds_read_b128 %7, %10 offset:7168\n\t"
      "ds_read_b128 %8, %11\n\t"
      "ds_read_b128 %9, %11 offset:1024"
      : "=&v"(row[0]), "=&v"(row[1]), "=&v"(row[2]), "=&v"(row[3]), "=&v"(row[4]),
        "=&v"(row[5]), "=&v"(row[6]), "=&v"(row[7]), "=&v"(bh), "=&v"(bl)
      : "v"(ad), "v"(ab)
      : "memory");
}
__device__ __forceinline__ void acc_read_wait(u32x4 (&row)[8], u32x4& bh, u32x4& bl) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(row[0]), "+v"(row[1]), "+v"(row[2]), "+v"(row[3]), "+v"(row[4]),
                 "+v"(row[5]), "+v"(row[6]), "+v"(row[7]), "+v"(bh), "+v"(bl)
               :
               : "memory");
}

// The eight row slabs only, issued; valid after acc_read_rows_wait().
__device__ __forceinline__ void acc_read_rows_issue(uint32_t ad, u32x4 (&row)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168"
      : "=&v"(row[0]), "=&v"(row[1]), "=&v"(row[2]), "=&v"(row[3]), "=&v"(row[4]),
        "=&v"(row[5]), "=&v"(row[6]), "=&v"(row[7])
      : "v"(ad)
      : "memory");
}
__device__ __forceinline__ void acc_read_rows_wait(u32x4 (&row)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(row[0]), "+v"(row[1]), "+v"(row[2]), "+v"(row[3]), "+v"(row[4]),
                 "+v"(row[5]), "+v"(row[6]), "+v"(row[7])
               :
               : "memory");
}

// The two B operands only.
__device__ __forceinline__ void acc_read_b(uint32_t ab, u32x4& bh, u32x4& bl) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %2 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(bh), "=&v"(bl)
      : "v"(ab)
      : "memory");
}

// Workgroup barrier with no memory fence.  The ring's ordering is explicit:
// loads into LDS are waited for by count before it, and every LDS read has
// completed inside its own statement, so the fence __syncthreads() adds
// (which waits for every outstanding global load) is not needed.  The empty
// statements keep the compiler from moving memory operations across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global->LDS loads of N 1 KiB row slabs at dst: rows prow,
// prow + ldd, ...; lane l's 16 bytes land at byte 16 l of each.  D is read
// once, so its loads carry the non-temporal hint (cache policy NT) and do not
// displace the packed input, which the column tiles of a matrix share in L2.
template <int N>
__device__ __forceinline__ void acc_issue_rows(u32x4* dst, const uint16_t* prow, int64_t ldd) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_global_load_lds(prow + i * ldd, dst + i * 64, 16, 0, 2);
}

// Direct global->LDS load of one 1 KiB slab from p to dst.
__device__ __forceinline__ void acc_issue_slab(u32x4* dst, const uint16_t* p) {
  __builtin_amdgcn_global_load_lds(p, dst, 16, 0, 0);
}
// The same with the non-temporal hint, for slabs of D.
__device__ __forceinline__ void acc_issue_slab_nt(u32x4* dst, const uint16_t* p) {
  __builtin_amdgcn_global_load_lds(p, dst, 16, 0, 2);
}

// acc[e] += A_e B over one 16-token step, hi term then lo term.
__device__ __forceinline__ void acc_mfma_step(f32x16 (&acc)[8], const u32x4 (&a)[8], u32x4 bh,
                                              u32x4 bl) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[e]), as_bf16x8(bh), acc[e], 0,
                                                     0, 0);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[e]), as_bf16x8(bl), acc[e], 0,
                                                     0, 0);
}

// Shape of the accumulate block for RB 32-rank blocks (RB = 1, 2, 4, 8: all
// ranks in one block, so D is read once).  The eight waves are RBW rank
// slots times NQ token classes; class u takes the 16-token steps s = u
// (mod NQ).  A ring slot holds, per class, the step's eight row slabs and
// the B operands of its RB rank blocks.
template <int RB>
struct AccShape {
  static constexpr int RBW = RB < 2 ? 2 : RB;           // waves per token class
  static constexpr int NQ = kAccWaves / RBW;            // token classes: 4, 4, 2, 1
  static constexpr int NS = 8 / RBW;                    // row slabs each wave loads per step
  static constexpr int kClass = 8 + 2 * RB;             // 1 KiB slabs per class in a slot
  static constexpr int kSlot = NQ * kClass;             // 1 KiB slabs per slot
  static constexpr int R = RB <= 2 ? 3 : (RB == 4 ? 4 : 6);  // ring slots
  static constexpr int kSmemKiB = R * kSlot > 128 ? R * kSlot : 128;  // exchange needs 128
};

// bf16 D.  A block covers 256 columns of D (rows of S) and all ranks (RB
// 32-rank blocks) over all T tokens.  Its eight waves (two per SIMD, so one
// wave's matrix work overlaps the other's loads and transposes) are RBW rank
// slots times NQ token classes: wave w takes rank block w % RBW (idle for
// compute when that is >= RB) and the 16-token steps s = u (mod NQ) of class
// u = w / RBW, so the block streams consecutive tokens.  Lane l covers D rows
// 16s + 8(l>>5) + i (i = 0..7), columns c0 + 8(l&31) .. +7, so 32 lanes read
// 512 contiguous bytes of a row.  A ring of R steps in LDS is filled by
// direct global->LDS loads: a slot holds, for each class, the step's eight
// row slabs (loaded 8 / RBW each by the class's waves and read by all of
// them) and the B operands of the rank blocks (each wave loads its own), so
// R - 1 steps are in flight while one computes.  The lane's 8 x 8 block is
// transposed in registers: for e = 0..7, operand A_e holds the eight tokens
// of column c0 + 8(l&31) + e, which is MFMA row m = l & 31 of instance e; the
// B operand holds the same tokens for rank n = l & 31, so each 32x32x16 MFMA
// adds 16 tokens.  Instance e gives C[m][n] = S[c0 + 8m + e][32b + n], lane l
// holding n = l & 31 and m = 8(j>>2) + 4(l>>5) + (j&3) in register j.  Each
// wave sums its class's steps in ascending order (hi term then lo term per
// step); the class sums meet through LDS as (Q0 + Q1) + (Q2 + Q3) (NQ = 4)
// or H0 + H1 (NQ = 2), and the result is added to S -- through an LDS tile
// in whole rows for NQ = 4, straight from the accumulators (128-byte row
// segments) otherwise.  The order depends on T and r alone, so grouped and
// single calls give the same bits.  Blocks that reach past column d take
// guarded register loads; rows past T (last step only) are loaded from row
// T - 1 and zeroed.
}  // namespace

// One matrix of a table-driven accumulate (device memory); entry n holds only
// tile_begin = the total tile count.
struct AccTableEntry {
  const void* D;
  const uint16_t* planes;
  float* S;
  int64_t d, ldd, tile_begin;
};

namespace {

// One tile of the accumulate: 256 columns of one matrix, all ranks, all tokens.
struct AccTile {
  const uint16_t* D;       // bf16 [T x d], leading dimension ldd
  const uint16_t* planes;  // packed projected input
  float* S;                // [d x r]
  int64_t d, ldd, q, T, r;
  int nsteps, nrb;
};

// loop_done() runs once the tile's loads have all landed, before the class
// sums meet and S is updated.
template <int RB, typename LoopDone>
__device__ __forceinline__ void acc_tile(const AccTile& tile, u32x4* smem, LoopDone&& loop_done) {
  using Sh = AccShape<RB>;
  constexpr int R = Sh::R, NQ = Sh::NQ, NS = Sh::NS, RBW = Sh::RBW;
  constexpr int kClass = Sh::kClass, kSlot = Sh::kSlot;

  const int64_t q = tile.q;
  const uint16_t* __restrict__ D = tile.D;
  const int64_t ldd = tile.ldd;
  const int64_t d = tile.d;
  const int64_t T = tile.T;

  // The lane index is opaque per tile, so that a loop over tiles does not
  // hoist every lane-derived address out of it and hold them throughout.
  int lane_o = threadIdx.x & 63;
  asm volatile("" : "+v"(lane_o));
  const int lane = lane_o;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = wave % RBW;            // rank block of this wave
  const int qt = wave / RBW;            // token class
  const bool has_rb = rb < RB;          // uniform per wave
  const int hw = lane >> 5;
  const int nsteps = tile.nsteps;
  const int Q = (nsteps + NQ - 1) / NQ;  // iterations: steps NQ k + qt, k < Q

  const int64_t c0 = q * kAccCols;
  const int64_t col = c0 + 8 * (lane & 31);
  const bool interior = c0 + kAccCols <= d;  // uniform per block
  const bool col_full = col + 8 <= d;
  const uint16_t* __restrict__ planes = tile.planes + (int64_t)rb * 1024 + lane * 8;
  const int64_t bstride = (int64_t)tile.nrb * 1024;

  f32x16 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[e][i] = 0.f;

  // Loads of iteration k (step NQ k + qt) into slot k % R: this wave's B
  // operands (hi, lo of its rank block) and, for an interior block, its NS
  // of the step's eight row slabs.  Iterations past the last step re-read it
  // (already cached) so that every iteration issues the same number of
  // loads; rows past T read row T - 1.
  auto issue = [&](int k) {
    const int st = NQ * k + qt;
    const int sc = st < nsteps ? st : nsteps - 1;
    u32x4* qs = smem + ((k % R) * kSlot + qt * kClass) * 64;
    if (has_rb) {
      const uint16_t* pb = planes + (int64_t)sc * bstride;
      acc_issue_slab(qs + (8 + 2 * rb) * 64, pb);
      acc_issue_slab(qs + (9 + 2 * rb) * 64, pb + 512);
    }
    if (!interior) return;
    const int64_t t0 = (int64_t)kAccStep * sc + 8 * hw + NS * rb;
    if ((int64_t)kAccStep * (sc + 1) <= T) {
      acc_issue_rows<NS>(qs + NS * rb * 64, D + t0 * ldd + col, ldd);
    } else {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int64_t t = t0 + i < T ? t0 + i : T - 1;
        acc_issue_slab_nt(qs + (NS * rb + i) * 64, D + t * ldd + col);
      }
    }
  };

  if (interior && RB <= 2) {
#pragma unroll
    for (int k = 0; k < R - 1; ++k) issue(k);
    for (int k = 0; k < Q; ++k) {
      // Iteration k has landed once only the loads of iterations
      // k+1 .. k+R-2 remain (2 + NS per iteration, NS without a rank block).
      if (has_rb) wait_vmcnt<(R - 2) * (2 + NS)>();
      else wait_vmcnt<(R - 2) * NS>();
      ring_barrier();  // the other waves' rows of iteration k have landed and
                       // every wave is done with iteration k - 1's slot
      issue(k + R - 1);
      const int s = NQ * k + qt;
      if (has_rb && s < nsteps) {
        const u32x4* qs = smem + ((k % R) * kSlot + qt * kClass) * 64;
        u32x4 row[8], a[8], bh, bl;
        acc_read_step(lds_addr(qs + lane), lds_addr(qs + (8 + 2 * rb) * 64 + lane), row, bh, bl);
        if ((int64_t)kAccStep * (s + 1) > T) {
          const int64_t t0 = (int64_t)kAccStep * s + 8 * hw;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (t0 + i >= T) row[i] = u32x4{0u, 0u, 0u, 0u};
        }
        transpose8x8(row, a);
        acc_mfma_step(acc, a, bh, bl);
      }
    }
  } else if (RB == 8 && interior) {
    if constexpr (RB == 8) {
      // Eight rank blocks: a wave's B operands (its rank block's packed
      // input, which no other wave reads) are loaded straight into registers
      // P steps ahead, and only the D rows, which all eight waves read, pass
      // through the LDS ring (P + 2 slots of eight slabs).  Iteration k
      // issues B(k + P) and then D(k + P + 2) into the slot D(k) left.
      // Loads complete in issue order, so once no more than the loads issued
      // after iteration k - P's B loads remain (its D load and three per
      // later iteration), B(k) and D(k + 1) (issued in iteration k - P - 1)
      // have landed.  Iteration k's operands A (the transposed rows) are in
      // registers before it starts; its hi-term MFMAs run while the LDS reads
      // of step k + 1 are in flight.
      constexpr int P = kAccBAhead, NB = P + 1, RD = P + 2;
      typedef __attribute__((address_space(1))) const u32x4 gb4;
      typedef __attribute__((address_space(1))) const uint16_t gb16;
      // Only a ragged last step has rows past T.  The empty volatile asm
      // keeps this a branch: flattened into selects it costs every step
      // some forty vector instructions.
      auto clip = [&](u32x4 (&row)[8], int s) __attribute__((always_inline)) {
        if (__builtin_expect((int64_t)kAccStep * (s + 1) > T, 0)) {
          asm volatile("");
          const int64_t t0 = (int64_t)kAccStep * s + 8 * hw;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (t0 + i >= T) row[i] = u32x4{0u, 0u, 0u, 0u};
        }
      };
      u32x4 bh[NB], bl[NB], a[8];
      auto load_b = [&](int st, u32x4& h, u32x4& l) __attribute__((always_inline)) {
        const int sc = st < nsteps ? st : nsteps - 1;
        const gb4* p = (const gb4*)((const gb16*)planes + (int64_t)sc * bstride);
        h = p[0];
        l = p[64];
      };
      auto issue_d = [&](int st) __attribute__((always_inline)) {
        const int sc = st < nsteps ? st : nsteps - 1;
        const int64_t t0 = (int64_t)kAccStep * sc + 8 * hw + rb;
        const int64_t t = t0 < T ? t0 : T - 1;
        acc_issue_slab_nt(smem + ((st % RD) * 8 + rb) * 64, D + t * ldd + col);
      };
#pragma unroll
      for (int j = 0; j < RD - P; ++j) issue_d(j);
#pragma unroll
      for (int j = 0; j < P; ++j) {
        load_b(j, bh[j], bl[j]);
        issue_d(j + RD - P);
      }
      wait_vmcnt<RD - P - 1 + 3 * P>();  // D(0) has landed
      ring_barrier();
      {
        u32x4 row[8];
        acc_read_rows_issue(lds_addr(smem + lane), row);
        acc_read_rows_wait(row);
        clip(row, 0);
        transpose8x8(row, a);
      }
      auto iter = [&](int k, auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        wait_vmcnt<1 + 3 * (P - 1)>();
        ring_barrier();  // every wave's D(k + 1) has landed and every wave
                         // has read D(k)'s slot
        load_b(k + P, bh[(u + P) % NB], bl[(u + P) % NB]);
        issue_d(k + RD);
        u32x4 rn[8];
        acc_read_rows_issue(lds_addr(smem + ((k + 1) % RD) * 8 * 64 + lane), rn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[e]), as_bf16x8(bh[u]),
                                                           acc[e], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        acc_read_rows_wait(rn);
        clip(rn, k + 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[e]), as_bf16x8(bl[u]),
                                                           acc[e], 0, 0, 0);
          a[e] = transpose8x8_e(rn, e);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      static_assert(NB == 3, "the unrolled ring below has three entries");
      int k = 0;
      for (; k + NB <= Q; k += NB) {
        iter(k, I0{});
        iter(k + 1, I1{});
        iter(k + 2, I2{});
      }
      if (k < Q) iter(k, I0{});
      if (k + 1 < Q) iter(k + 1, I1{});
    }
  } else if (interior) {
    // Four rank blocks (each wave computes every step of its class) are
    // software-pipelined: iteration k's operands are in registers (a, bh,
    // bl) before it starts; its hi-term MFMAs run while the LDS reads of
    // iteration k + 1 are in flight.  Own loads in flight at the top of
    // iteration k: iterations k+1 .. k+R-1 (2 + NS each, NS without a rank
    // block); k + 1 has landed once (R - 2) iterations' loads remain.
    constexpr int kWaitRb = (R - 2) * (2 + NS), kWaitNoRb = (R - 2) * NS;
    // zero the rows of a step's block past T (last step only)
    auto clip = [&](u32x4 (&row)[8], int s) __attribute__((always_inline)) {
      if ((int64_t)kAccStep * (s + 1) > T) {
        const int64_t t0 = (int64_t)kAccStep * s + 8 * hw;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (t0 + i >= T) row[i] = u32x4{0u, 0u, 0u, 0u};
      }
    };
    u32x4 a[8], bh, bl;
#pragma unroll
    for (int k = 0; k < R - 1; ++k) issue(k);
    if (has_rb) wait_vmcnt<kWaitRb>();
    else wait_vmcnt<kWaitNoRb>();
    ring_barrier();
    issue(R - 1);
    if (has_rb) {
      u32x4 row[8];
      acc_read_step(lds_addr(smem + qt * kClass * 64 + lane),
                    lds_addr(smem + (qt * kClass + 8 + 2 * rb) * 64 + lane), row, bh, bl);
      clip(row, qt);
      transpose8x8(row, a);
    }
    for (int k = 0; k < Q; ++k) {
      if (has_rb) wait_vmcnt<kWaitRb>();
      else wait_vmcnt<kWaitNoRb>();
      ring_barrier();  // every wave's loads of iteration k + 1 have landed and
                       // every wave has read iteration k's slot
      issue(k + R);
      if (!has_rb) continue;
      const bool live = NQ * k + qt < nsteps;  // uniform per wave
      const u32x4* qs = smem + (((k + 1) % R) * kSlot + qt * kClass) * 64;
      u32x4 rn[8], bhn, bln;
      acc_read_issue(lds_addr(qs + lane), lds_addr(qs + (8 + 2 * rb) * 64 + lane), rn, bhn, bln);
      __builtin_amdgcn_sched_barrier(0);
      if (live) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[e]), as_bf16x8(bh), acc[e],
                                                           0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      acc_read_wait(rn, bhn, bln);
      clip(rn, NQ * (k + 1) + qt);
      if (live) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[e]), as_bf16x8(bl), acc[e], 0,
                                                           0, 0);
      }
      transpose8x8(rn, a);
      bh = bhn;
      bl = bln;
    }
  } else {
    // Block reaching past column d: the same barriers and B loads; rows by
    // guarded register loads.
#pragma unroll
    for (int k = 0; k < R - 1; ++k) issue(k);
    for (int k = 0; k < Q; ++k) {
      wait_vmcnt<0>();
      ring_barrier();
      issue(k + R - 1);
      const int s = NQ * k + qt;
      if (has_rb && s < nsteps) {
        const u32x4* qs = smem + ((k % R) * kSlot + qt * kClass) * 64;
        const int64_t t0 = (int64_t)kAccStep * s + 8 * hw;
        u32x4 row[8], a[8], bh, bl;
#pragma unroll
        for (int i = 0; i < 8; ++i) row[i] = load_drow(D, ldd, t0 + i, T, col, d, col_full);
        acc_read_b(lds_addr(qs + (8 + 2 * rb) * 64 + lane), bh, bl);
        transpose8x8(row, a);
        acc_mfma_step(acc, a, bh, bl);
      }
    }
  }
  wait_vmcnt<0>();  // no load may still target LDS past this point
  loop_done();

  // S through the global address space: flat accesses also count on the LDS
  // counter, so every wait for an LDS access below would wait for them too
  // (with flat stores, each row's store would wait for the one before).
  typedef __attribute__((address_space(1))) float gf32;
  gf32* __restrict__ S = (gf32*)tile.S;
  const int64_t r = tile.r;
  // Class sums in accumulator order: element (e, j) of lane l at
  // [slot][(4e + j / 4) 64 + l] as float4, one 32 KiB slot per wave.
  f32x4* xr = reinterpret_cast<f32x4*>(smem);
  auto put = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        xr[(slot * 32 + 4 * e + v) * 64 + lane] =
            f32x4{acc[e][4 * v], acc[e][4 * v + 1], acc[e][4 * v + 2], acc[e][4 * v + 3]};
  };
  auto add_e = [&](int slot, int e) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x4 x = xr[(slot * 32 + 4 * e + v) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[e][4 * v + i] += x[i];
    }
  };
  auto add = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) add_e(slot, e);
  };

  if constexpr (NQ == 4) {
    // This thread's share of the block's S tile (256 rows x 32 RB ranks):
    // rank lane of rows row0 + 8k, so a wave reads whole row segments.  The
    // loads are issued now and complete while the class sums meet.
    constexpr int TJ = 32 * RB;
    constexpr int kRowsPerThread = kAccCols / kAccWaves;
    const int64_t row0 = c0 + wave;
    const int64_t j = lane;
    const bool jok = lane < TJ && j < r;
    const int64_t jc = j < r ? j : r - 1;  // in-bounds address for idle lanes
    int64_t rstride = kAccWaves * r;
    float sv[kRowsPerThread];
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
      const int64_t row = row0 + kAccWaves * k < d ? row0 + kAccWaves * k : d - 1;
      sv[k] = S[row * r + jc];
    }
    // Keep the addresses from being held live across the exchange below.
    asm volatile("" : "+s"(rstride));
    ring_barrier();  // every wave is done with the ring

    // Q0 + Q1 and Q2 + Q3 (slots rb + 2 (qt >> 1)).
    if (has_rb && (qt & 1)) put(rb + 2 * (qt >> 1));
    wait_lgkmcnt0();
    ring_barrier();
    if (has_rb && !(qt & 1)) add(rb + 2 * (qt >> 1));
    wait_lgkmcnt0();
    ring_barrier();
    // (Q0 + Q1) + (Q2 + Q3).
    if (has_rb && qt == 2) put(rb);
    wait_lgkmcnt0();
    ring_barrier();
    // The tile in LDS after the first 64 KiB, rows of TJ + 1 floats.
    float* yt = reinterpret_cast<float*>(smem + 2 * 32 * 64);
    constexpr int YS = TJ + 1;
    if (has_rb && qt == 0) {
      add(rb);
      const int n = lane & 31;
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 8 * v + 4 * hw + i;
            yt[(8 * m + e) * YS + 32 * rb + n] = acc[e][4 * v + i];
          }
    }
    wait_lgkmcnt0();
    ring_barrier();
    wait_vmcnt<0>();  // the S loads (long complete): no waits between the stores below
    if (jok) {
      gf32* p = S + row0 * r + j;
#pragma unroll
      for (int k = 0; k < kRowsPerThread; ++k) {
        if (row0 + kAccWaves * k < d) *p = sv[k] + yt[(wave + kAccWaves * k) * YS + lane];
        p += rstride;
      }
    }
  } else {
    if constexpr (NQ == 2) {
      // H0 + H1: class 1 hands its sums to class 0 (four 32 KiB slots),
      // which adds them instance by instance below.
      ring_barrier();  // every wave is done with the ring
      if (qt == 1) put(rb);
      wait_lgkmcnt0();
      ring_barrier();
      if (qt != 0) return;
    }
    // S += the wave's 256 x 32 tile straight from the accumulators: for
    // instance e and register 4v + i, the 32 lanes of a half hold 32
    // consecutive ranks of row c0 + 8(8v + 4(l>>5) + i) + e.  The next
    // instance's S values are loaded before this one's are stored.
    const int j = 32 * rb + (lane & 31);
    if (j >= r) return;
    // The block's rows of S start at a wave-uniform base; lane offsets are
    // 32-bit (256 rows x r <= 65536 floats).
    gf32* __restrict__ Sb = S + c0 * r;
    const uint32_t ur = (uint32_t)r;
    const int nrows = d - c0 < kAccCols ? (int)(d - c0) : kAccCols;
    float cur[16], nxt[16];
    auto load = [&](int e, float (&dst)[16]) __attribute__((always_inline)) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * (8 * v + 4 * hw + i) + e;
          dst[4 * v + i] = row < nrows ? Sb[(uint32_t)row * ur + (uint32_t)j] : 0.f;
        }
    };
    load(0, cur);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < 7) load(e + 1, nxt);
      if constexpr (NQ == 2) add_e(rb, e);  // class 1's sums, instance e
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * (8 * v + 4 * hw + i) + e;
          if (row < nrows) Sb[(uint32_t)row * ur + (uint32_t)j] = cur[4 * v + i] + acc[e][4 * v + i];
        }
      if (e < 7) {
#pragma unroll
        for (int x = 0; x < 16; ++x) cur[x] = nxt[x];
      }
    }
  }
}

template <int RB>
__global__ __launch_bounds__(512, 1) void acc_bf16_kernel(AccGroupArgs g) {
  __shared__ __align__(16) u32x4 smem[AccShape<RB>::kSmemKiB * 64];
  const int64_t logical = xcd_logical_block();
  if (logical >= g.tile_begin[g.n]) return;
  int item = 0;
  while (logical >= g.tile_begin[item + 1]) ++item;
  const AccTile tile{static_cast<const uint16_t*>(g.D[item]), g.planes[item], g.S[item], g.d[item],
                     g.ldd[item], logical - g.tile_begin[item], g.T, g.r, g.nsteps, g.nrb};
  acc_tile<RB>(tile, smem, [] {});
}

// Persistent form over a device-resident table of many matrices (e.g. every
// projection of every layer for one microbatch): the grid is a whole number
// of blocks per XCD, at most one block per compute unit.  The table's tile
// list (matrix by matrix, column block by column block) is cut into eight
// contiguous ranges, one per XCD (blocks are dispatched round-robin over the
// XCDs), and the blocks of an XCD take its range's tiles in order from a
// counter of their own.  The column tiles of one matrix so run close together
// in time on one XCD and read its packed input from that XCD's L2, and the
// compute units left idle by one layer's tiles and the ramp of separate
// launches are shared across the whole table.  Each tile is still computed
// whole by one block, so the results are bit-identical to the per-layer
// launches; which block runs a tile changes nothing.
template <int RB>
__global__ __launch_bounds__(512, 1) void acc_bf16_table_kernel(const AccTableEntry* __restrict__ tab,
                                                                unsigned* __restrict__ next, int n,
                                                                int64_t T, int64_t r, int nsteps,
                                                                int nrb) {
  __shared__ __align__(16) u32x4 smem[AccShape<RB>::kSmemKiB * 64];
  __shared__ unsigned claimed[2];
  const int64_t total = tab[n].tile_begin;
  const int xcd = (int)(blockIdx.x & 7);
  const int64_t per = gridDim.x >> 3;  // blocks per XCD
  const int64_t begin = total * xcd / 8, end = total * (xcd + 1) / 8;
  int64_t t = begin + (blockIdx.x >> 3);
  for (int it = 0; t < end; ++it) {
    // Claim the block's following tile now; the index is needed only when
    // this tile is done, so the atomic's latency is hidden behind it.
    // The address is made opaque per lane (lane_o is 0 here): with a uniform
    // address the compiler turns the atomic into a wave-wide form whose
    // result is broadcast, and waits for it, right away.
    unsigned c = 0;
    if (threadIdx.x == 0) {
      int lane_o = (int)threadIdx.x;
      asm volatile("" : "+v"(lane_o));
      c = atomicAdd(next + xcd + lane_o, 1u);
    }
    int lo = 0, hi = n - 1;  // the entry holding tile t: tile_begin[lo] <= t < tile_begin[lo + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tab[mid].tile_begin <= t) lo = mid; else hi = mid - 1;
    }
    const AccTableEntry& e = tab[lo];
    const AccTile tile{static_cast<const uint16_t*>(e.D), e.planes, e.S, e.d, e.ldd,
                       t - e.tile_begin, T, r, nsteps, nrb};
    // The claim is stored once the tile's loads have landed (the atomic has
    // returned by then, so its wait costs nothing).  Slot it & 1 is written
    // again two tiles on, after a barrier every thread reaches only once it
    // has read the slot here.
    acc_tile<RB>(tile, smem, [&] {
      if (threadIdx.x == 0) claimed[it & 1] = c;
    });
    // Every wave is done with the LDS before the next tile's loads land.  The
    // tile's S stores need not have completed: the next tile touches other
    // rows of S, and its waits by count only grow more conservative while
    // stores are outstanding.
    wait_lgkmcnt0();
    ring_barrier();
    t = begin + per + (int64_t)claimed[it & 1];
  }
}

// fp32 D: one thread per (row of S, rank); fp64 sum over tokens.
__global__ void acc_f32_kernel(AccGroupArgs g) {
  const int item = blockIdx.y;
  const int64_t d = g.d[item], r = g.r;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= d * r) return;
  const int64_t c = idx / r;
  const int64_t j = idx - c * r;
  const float* __restrict__ D = static_cast<const float*>(g.D[item]);
  const float* __restrict__ x = g.XAt[item];
  double acc = 0.0;
  for (int64_t t = 0; t < g.T; ++t) acc += (double)D[t * g.ldd[item] + c] * (double)x[t * r + j];
  float* S = g.S[item];
  S[c * r + j] = (float)((double)S[c * r + j] + acc);
}

}  // namespace

// ------------------------------------------------------------ launchers

int64_t acc_rank_pad(int64_t r) {
  const int64_t nrb = (r + 31) / 32;
  return 32 * (nrb <= 2 ? nrb : nrb <= 4 ? 4 : (nrb + 7) / 8 * 8);
}
int64_t acc_token_pad(int64_t T) { return (T + kAccStep - 1) / kAccStep * kAccStep; }
static int64_t acc_col_blocks(int64_t d) { return (d + kAccCols - 1) / kAccCols; }
static size_t round256(size_t x) { return (x + 255) / 256 * 256; }
size_t acc_ws_bytes_per_item(int64_t T, int64_t /*d*/, int64_t r) {
  return round256((size_t)(acc_rank_pad(r) * acc_token_pad(T) * 4));
}

hipError_t launch_regen_A(KeyArg key, int64_t r, int64_t k, bool int8_out, void* A,
                          hipStream_t s) {
  const int64_t n = r * ((k + 3) / 4);
  const float cr = (float)(1.0 / std::sqrt((double)r));
  hipLaunchKernelGGL(regen_A_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, key, r,
                     k, int8_out ? 1 : 0, cr, A);
  return hipGetLastError();
}

// 16-rank blocks the projection kernel computes for rank r.
int proj_nb16(int64_t r) {
  const int64_t nb16 = (r + 15) / 16;
  return nb16 <= 1 ? 1 : nb16 <= 2 ? 2 : nb16 <= 4 ? 4 : nb16 <= 6 ? 6 : nb16 <= 8 ? 8
       : nb16 <= 12 ? 12 : 16;
}

size_t projection_packed_bytes(int64_t r, int64_t k) {
  return (size_t)((k + 255) / 256) * 8 * (size_t)proj_nb16(r) * 2048;
}

hipError_t launch_regen_A_gaussian(KeyArg key, int64_t r, int64_t k, float* A, hipStream_t s) {
  const int64_t n = r * ((k + 3) / 4);
  hipLaunchKernelGGL(regen_A_gaussian_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     key, r, k, A);
  return hipGetLastError();
}

hipError_t launch_pack_projection(int64_t r, int64_t k, const float* A, void* packed,
                                  hipStream_t s) {
  const int nb16 = proj_nb16(r);
  const int64_t threads = (k + 255) / 256 * 8 * nb16 * 64;
  hipLaunchKernelGGL(pack_projection_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, r, k, nb16, A, static_cast<uint16_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_project(KeyArg key, int64_t T, int64_t k, int64_t r, const void* X,
                          bool bf16, int64_t ldx, float* XAt, uint16_t* planes, hipStream_t s,
                          const void* A_packed) {
  const double crd = 1.0 / std::sqrt((double)r);
  const int nrb = (int)(acc_rank_pad(r) / 32);
  const int nsteps = (int)(acc_token_pad(T) / kAccStep);
  if (!bf16) {
    if (planes || A_packed) return hipErrorInvalidValue;
    const int64_t n = T * r;
    hipLaunchKernelGGL(project_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       key, T, k, r, static_cast<const float*>(X), ldx, crd, XAt);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((T + kProjTokens - 1) / kProjTokens));
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  const uint16_t* Ap = static_cast<const uint16_t*>(A_packed);
  const float cr = A_packed ? 1.0f : (float)crd;
  switch (proj_nb16(r)) {
#define LOGRA_PROJ_CASE(NB)                                                                     \
  case NB:                                                                                      \
    if (Ap)                                                                                     \
      hipLaunchKernelGGL((project_bf16_kernel<NB, true>), grid, dim3(kProjWaves * 64), 0, s, key, \
                         T, k, r, Xb, ldx, cr, XAt, planes, nrb, nsteps, Ap);                   \
    else                                                                                        \
      hipLaunchKernelGGL((project_bf16_kernel<NB, false>), grid, dim3(kProjWaves * 64), 0, s,    \
                         key, T, k, r, Xb, ldx, cr, XAt, planes, nrb, nsteps, Ap);              \
    break;
    LOGRA_PROJ_CASE(1)
    LOGRA_PROJ_CASE(2)
    LOGRA_PROJ_CASE(4)
    LOGRA_PROJ_CASE(6)
    LOGRA_PROJ_CASE(8)
    LOGRA_PROJ_CASE(12)
    LOGRA_PROJ_CASE(16)
#undef LOGRA_PROJ_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int proj_table_max() { return kProjTableMax; }

// Workspace: the n + 1 table entries, then one more entry's room holding the
// item counter.
size_t proj_table_ws_bytes(int n) { return round256((size_t)(n + 2) * sizeof(ProjTableEntry)); }

template <int NB, bool X16 = false>
static hipError_t launch_project_table_nb(const ProjTableEntry* t, unsigned* next, int n,
                                          int64_t T, int64_t r, float cr, int nrb,
                                          hipStream_t s) {
  // resident blocks per compute unit, from the occupancy query (once; concurrent
  // first calls store the same value)
  static std::atomic<int> cached_per_cu{0};
  int per_cu = cached_per_cu.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int b = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, project_table_kernel<NB, X16>,
                                                                kPtWaves * 64, 0);
    if (e != hipSuccess) return e;
    per_cu = b > 0 ? b : 1;
    cached_per_cu.store(per_cu, std::memory_order_relaxed);
  }
  const dim3 grid((unsigned)(per_cu * compute_units()));
  hipLaunchKernelGGL((project_table_kernel<NB, X16>), grid, dim3(kPtWaves * 64), 0, s, t, next, n,
                     T, r, cr, nrb);
  return hipGetLastError();
}

hipError_t launch_project_table(int64_t T, int64_t r, const ProjItem* items, int n, void* ws,
                                hipStream_t s) {
  if (n < 1 || n > kProjTableMax) return hipErrorInvalidValue;
  std::vector<ProjTableEntry> tab((size_t)n + 2, ProjTableEntry{});
  // Above 64 ranks a block takes 256 tokens of one projection at a time
  // (project_blocked_kernel); otherwise a wave takes two token steps.
  bool blocked = proj_nb16(r) > 4;
  for (int i = 0; i < n && blocked; ++i) blocked = items[i].k % 8 == 0;  // its 16-byte loads need it
  const int64_t per_tokens = blocked ? (int64_t)kPbTokens : (int64_t)kProjTokens * kProjTableSteps;
  const int64_t per = (T + per_tokens - 1) / per_tokens;  // items per entry
  // Consecutive projections of one input (same X, k and leading dimension)
  // share an entry, up to kProjFuse of them at <= 64 ranks: X is read once for
  // all.  Each projection's sums are formed as they would be alone, so the
  // outputs do not depend on the grouping.
  const int fuse = proj_nb16(r) <= 4 ? kProjFuse : 1;
  int ne = 0;
  for (int i = 0; i < n; ++i) {
    ProjTableEntry* cur = ne > 0 ? &tab[ne - 1] : nullptr;
    if (cur && cur->np < fuse && cur->X == items[i].X && cur->k == items[i].k &&
        cur->ldx == items[i].ldx) {
      cur->XAt[cur->np] = items[i].XAt;
      cur->planes[cur->np] = items[i].planes;
      cur->k0[cur->np] = items[i].key.k0;
      cur->k1[cur->np] = items[i].key.k1;
      ++cur->np;
      continue;
    }
    ProjTableEntry& t = tab[ne];
    t.X = static_cast<const uint16_t*>(items[i].X);
    t.XAt[0] = items[i].XAt;
    t.planes[0] = items[i].planes;
    t.k0[0] = items[i].key.k0;
    t.k1[0] = items[i].key.k1;
    t.ldx = items[i].ldx;
    t.k = items[i].k;
    t.item_begin = per * ne;
    t.np = 1;
    ++ne;
  }
  // Entries with the widest inputs first: work is claimed in table order, so
  // the launch ends on the shortest items and its tail is short.
  std::stable_sort(tab.begin(), tab.begin() + ne,
                   [](const ProjTableEntry& a, const ProjTableEntry& b) { return a.k > b.k; });
  for (int i = 0; i < ne; ++i) tab[i].item_begin = per * i;
  tab[ne].item_begin = per * ne;
  n = ne;
  // From pageable memory the copy is staged before the call returns.
  hipError_t e = hipMemcpyAsync(ws, tab.data(), tab.size() * sizeof(ProjTableEntry),
                                hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  const ProjTableEntry* t = static_cast<const ProjTableEntry*>(ws);
  unsigned* next = reinterpret_cast<unsigned*>(static_cast<ProjTableEntry*>(ws) + n + 1);
  const float cr = (float)(1.0 / std::sqrt((double)r));
  const int nrb = (int)(acc_rank_pad(r) / 32);
  if (blocked) {
    const dim3 grid((unsigned)compute_units());  // one block per compute unit (its LDS)
    switch (proj_nb16(r)) {
#define LOGRA_PROJ_BLOCKED(NB)                                                                  \
  case NB:                                                                                      \
    hipLaunchKernelGGL(project_blocked_kernel<NB>, grid, dim3(kPbWaves * 64), 0, s, t, next, n, T, \
                       r, cr, nrb);                                                             \
    return hipGetLastError();
      LOGRA_PROJ_BLOCKED(6)
      LOGRA_PROJ_BLOCKED(8)
      LOGRA_PROJ_BLOCKED(12)
      LOGRA_PROJ_BLOCKED(16)
#undef LOGRA_PROJ_BLOCKED
      default: return hipErrorInvalidValue;
    }
  }
  // Up to 64 ranks, when every k is a multiple of 8, the inputs are loaded 16
  // bytes at a time (eight consecutive columns) and the sign words rearranged
  // to match, as in the block form.
  bool x16 = true;
  for (int i = 0; i < n && x16; ++i) x16 = items[i].k % 8 == 0;
  if (x16) {
    switch (proj_nb16(r)) {
      case 1: return launch_project_table_nb<1, true>(t, next, n, T, r, cr, nrb, s);
      case 2: return launch_project_table_nb<2, true>(t, next, n, T, r, cr, nrb, s);
      case 4: return launch_project_table_nb<4, true>(t, next, n, T, r, cr, nrb, s);
      default: break;
    }
  }
  switch (proj_nb16(r)) {
    case 1: return launch_project_table_nb<1>(t, next, n, T, r, cr, nrb, s);
    case 2: return launch_project_table_nb<2>(t, next, n, T, r, cr, nrb, s);
    case 4: return launch_project_table_nb<4>(t, next, n, T, r, cr, nrb, s);
    case 6: return launch_project_table_nb<6>(t, next, n, T, r, cr, nrb, s);
    case 8: return launch_project_table_nb<8>(t, next, n, T, r, cr, nrb, s);
    case 12: return launch_project_table_nb<12>(t, next, n, T, r, cr, nrb, s);
    case 16: return launch_project_table_nb<16>(t, next, n, T, r, cr, nrb, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_accumulate(int64_t T, int64_t r, bool bf16, const AccItem* items, int n,
                             bool packed, hipStream_t s) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  AccGroupArgs g{};
  g.n = n;
  g.T = T;
  g.r = r;
  g.nsteps = (int)(acc_token_pad(T) / kAccStep);
  g.nrb = (int)(acc_rank_pad(r) / 32);
  for (int i = 0; i < n; ++i) {
    g.D[i] = items[i].D;
    g.XAt[i] = items[i].XAt;
    g.S[i] = items[i].S;
    g.d[i] = items[i].d;
    g.ldd[i] = items[i].ldd;
    g.nq[i] = acc_col_blocks(items[i].d);
    g.planes[i] = static_cast<uint16_t*>(items[i].ws);
    g.pack[i] = packed ? 0 : 1;
    // Items that read the same projected input share one packed copy: it is
    // packed once, into the first such item's space.
    for (int j = 0; j < i && !packed; ++j)
      if (items[j].XAt == items[i].XAt) {
        g.planes[i] = g.planes[j];
        g.pack[i] = 0;
        break;
      }
  }
  if (!bf16) {
    int64_t maxdr = 0;
    for (int i = 0; i < n; ++i) maxdr = std::max(maxdr, g.d[i] * r);
    hipLaunchKernelGGL(acc_f32_kernel, dim3((unsigned)((maxdr + 255) / 256), (unsigned)n),
                       dim3(256), 0, s, g);
    return hipGetLastError();
  }
  if (!packed) {
    const int64_t chunks = (int64_t)g.nsteps * g.nrb;
    hipLaunchKernelGGL(acc_pack_kernel, dim3((unsigned)((chunks + 3) / 4), (unsigned)n),
                       dim3(256), 0, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  g.tile_begin[0] = 0;
  for (int i = 0; i < n; ++i) g.tile_begin[i + 1] = g.tile_begin[i] + g.nq[i];
  const int64_t tiles = g.tile_begin[n];
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  switch (g.nrb) {
    case 1: hipLaunchKernelGGL(acc_bf16_kernel<1>, grid, dim3(kAccWaves * 64), 0, s, g); break;
    case 2: hipLaunchKernelGGL(acc_bf16_kernel<2>, grid, dim3(kAccWaves * 64), 0, s, g); break;
    case 4: hipLaunchKernelGGL(acc_bf16_kernel<4>, grid, dim3(kAccWaves * 64), 0, s, g); break;
    case 8: hipLaunchKernelGGL(acc_bf16_kernel<8>, grid, dim3(kAccWaves * 64), 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Workspace: the n + 1 table entries, then one more entry's room holding the
// eight per-XCD tile counters.
static_assert(sizeof(AccTableEntry) >= 8 * sizeof(unsigned), "counters fit one entry");
size_t acc_table_ws_bytes(int n) { return round256((size_t)(n + 2) * sizeof(AccTableEntry)); }

hipError_t launch_accumulate_table(int64_t T, int64_t r, const AccItem* items, int n, void* ws,
                                   hipStream_t s) {
  if (n < 1) return hipErrorInvalidValue;
  // The table and the zeroed counters (entry n + 1) go over in one copy.
  std::vector<AccTableEntry> tab((size_t)n + 2, AccTableEntry{nullptr, nullptr, nullptr, 0, 0, 0});
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    tab[i] = AccTableEntry{items[i].D, static_cast<const uint16_t*>(items[i].ws), items[i].S,
                           items[i].d, items[i].ldd, tiles};
    tiles += acc_col_blocks(items[i].d);
  }
  tab[n] = AccTableEntry{nullptr, nullptr, nullptr, 0, 0, tiles};
  // From pageable memory the copy is staged before the call returns, so the
  // table may go out of scope right after.
  hipError_t e = hipMemcpyAsync(ws, tab.data(), tab.size() * sizeof(AccTableEntry),
                                hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  const int nrb = (int)(acc_rank_pad(r) / 32);
  const int nsteps = (int)(acc_token_pad(T) / kAccStep);
  // Blocks per XCD: enough for every tile of the largest range, at most the
  // XCD's share of the compute units.
  const int64_t cus_per_xcd = compute_units() / 8 > 0 ? compute_units() / 8 : 1;
  const int64_t range = (tiles + 7) / 8;
  const dim3 grid((unsigned)(8 * (range < cus_per_xcd ? range : cus_per_xcd)));
  const AccTableEntry* t = static_cast<const AccTableEntry*>(ws);
  unsigned* next = reinterpret_cast<unsigned*>(static_cast<AccTableEntry*>(ws) + n + 1);
  switch (nrb) {
    case 1: hipLaunchKernelGGL(acc_bf16_table_kernel<1>, grid, dim3(kAccWaves * 64), 0, s, t, next, n, T, r, nsteps, nrb); break;
    case 2: hipLaunchKernelGGL(acc_bf16_table_kernel<2>, grid, dim3(kAccWaves * 64), 0, s, t, next, n, T, r, nsteps, nrb); break;
    case 4: hipLaunchKernelGGL(acc_bf16_table_kernel<4>, grid, dim3(kAccWaves * 64), 0, s, t, next, n, T, r, nsteps, nrb); break;
    case 8: hipLaunchKernelGGL(acc_bf16_table_kernel<8>, grid, dim3(kAccWaves * 64), 0, s, t, next, n, T, r, nsteps, nrb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace logra
