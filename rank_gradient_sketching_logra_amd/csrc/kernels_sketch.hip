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

namespace logra {

namespace {

__device__ __forceinline__ uint64_t pick_word(const Philox4& p, int i) {
  const uint64_t a = (i & 1) ? p.w[1] : p.w[0];
  const uint64_t b = (i & 1) ? p.w[3] : p.w[2];
  return (i & 2) ? b : a;
}

// Eight bf16 values +-1 from the low 8 bits of b (bit i set -> element i is -1).
__device__ __forceinline__ u32x4 expand_signs(uint32_t b) {
  u32x4 v;
  v[0] = 0x3F803F80u | ((b << 15) & 0x8000u) | ((b << 30) & 0x80000000u);
  v[1] = 0x3F803F80u | ((b << 13) & 0x8000u) | ((b << 28) & 0x80000000u);
  v[2] = 0x3F803F80u | ((b << 11) & 0x8000u) | ((b << 26) & 0x80000000u);
  v[3] = 0x3F803F80u | ((b << 9) & 0x8000u) | ((b << 24) & 0x80000000u);
  return v;
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

// ------------------------------------------------------------- project

// bf16 X: one block = 32 tokens x all ranks; the four waves take the
// 256-column blocks of k round-robin, then add their partial tiles in a
// fixed order.  NBT = padded rank / 32.
template <int NBT>
__global__ __launch_bounds__(256) void project_bf16_kernel(KeyArg key, int64_t T, int64_t k,
                                                           int64_t r,
                                                           const uint16_t* __restrict__ X,
                                                           int64_t ldx, float cr,
                                                           float* __restrict__ XAt) {
  constexpr int NQ = (NBT + 1) / 2;
  constexpr int RP = NBT * 32;
  __shared__ __align__(16) float red[32][RP + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int64_t trow = t0 + (lane & 31);
  const KeyWords kw{key.k0, key.k1};

  f32x16 acc[NBT];
#pragma unroll
  for (int nb = 0; nb < NBT; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[nb][e] = 0.f;

  const int64_t nblk = (k + 255) >> 8;
  for (int64_t b = wave; b < nblk; b += 4) {
    uint32_t bits[NQ][8];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t j = lane + 64 * q;
      Philox4 p = sigma_block(kw, (uint64_t)j, (uint64_t)b);
      const bool live = j < r;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        bits[q][2 * w] = live ? (uint32_t)p.w[w] : 0u;
        bits[q][2 * w + 1] = live ? (uint32_t)(p.w[w] >> 32) : 0u;
      }
    }
    u32x4 a[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
      a[s] = load_bf16x8(X, ldx, trow, b * 256 + 16 * s + 8 * half, T, k);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb) {
        const int src = (nb & 1) * 32 + (lane & 31);
        const uint32_t wv = (uint32_t)__shfl((int)bits[nb >> 1][s >> 1], src, 64);
        const uint32_t byte = (wv >> (16 * (s & 1) + 8 * half)) & 0xFFu;
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[s]),
                                                          as_bf16x8(expand_signs(byte)),
                                                          acc[nb], 0, 0, 0);
      }
    }
  }

  // Fixed-order reduction over the four waves: ((w0 + w1) + w2) + w3.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb)
#pragma unroll
        for (int reg = 0; reg < 16; ++reg) {
          const int m = 8 * (reg >> 2) + 4 * half + (reg & 3);
          const int n = nb * 32 + (lane & 31);
          red[m][n] = (w == 0) ? acc[nb][reg] : red[m][n] + acc[nb][reg];
        }
    }
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < 32 * r; idx += 256) {
    const int m = idx / (int)r;
    const int j = idx - m * (int)r;
    const int64_t t = t0 + m;
    if (t < T) XAt[t * r + j] = red[m][j] * cr;
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
// v_mfma_f32_16x16x32_bf16: for 32-token step s and 16-rank block b, two
// 1 KiB operands (hi then lo) in which lane l holds tokens 32s + 8(l>>4) + i
// (i = 0..7) of rank 16b + (l & 15).  One wave reads one operand with one
// fully contiguous 16-byte-per-lane load.  Tokens >= T and ranks >= r are 0.
constexpr int kAccStep = 32;       // tokens per MFMA step
constexpr int kAccCols = 128;      // columns of D per block: 16 lanes x 8
constexpr int kAccSlices = 4;      // token slices per block, one per wave
constexpr int kAccGroupRB = 4;     // 16-rank blocks per rank group (64 ranks)

struct AccGroupArgs {
  const void* D[kMaxGroup];
  const float* XAt[kMaxGroup];
  float* S[kMaxGroup];
  uint16_t* planes[kMaxGroup];
  int64_t d[kMaxGroup];
  int64_t ldd[kMaxGroup];
  int64_t tile_begin[kMaxGroup + 1];
  int n;
  int64_t T, r;
  int nsteps;   // ceil(T / 32)
  int nrb;      // 16-rank blocks packed: ceil(r / 16), rounded up to a
                // multiple of 4 when there is more than one rank group
  int ngroups;  // nrb / RB rank groups (RB = min(nrb, 4))
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// One wave per (step, rank block) of one item.
__global__ __launch_bounds__(256) void acc_pack_kernel(AccGroupArgs g) {
  const int item = blockIdx.y;
  const int64_t chunk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (chunk >= (int64_t)g.nsteps * g.nrb) return;
  const int lane = threadIdx.x & 63;
  const int64_t s = chunk / g.nrb;
  const int64_t b = chunk - s * g.nrb;
  const int64_t j = 16 * b + (lane & 15);
  const int64_t t0 = kAccStep * s + 8 * (lane >> 4);
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
  *reinterpret_cast<u32x4*>(dst) = vh;
  *reinterpret_cast<u32x4*>(dst + 512) = vl;
}

// Eight bf16 of row t of D from column col; zero outside the matrix.
__device__ __forceinline__ u32x4 load_drow(const uint16_t* __restrict__ D, int64_t ldd,
                                           int64_t t, int64_t T, int64_t col, int64_t d,
                                           bool full) {
  if (t >= T) return u32x4{0u, 0u, 0u, 0u};
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

// Transpose a lane's 8 x 8 block of bf16 (row[i] = eight columns of token
// i): a[e] = the eight tokens of column e, as one MFMA operand.
__device__ __forceinline__ void transpose8x8(const u32x4 (&row)[8], u32x4 (&a)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = e >> 1;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t x0 = row[2 * p][q], x1 = row[2 * p + 1][q];
      a[e][p] = (e & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
    }
  }
}

// acc[e][b] += A_e B_b over one 32-token step, hi term then lo term.
template <int RB>
__device__ __forceinline__ void acc_mfma_step(f32x4 (&acc)[8][RB], const u32x4 (&a)[8],
                                              const u32x4 (&bh)[RB], const u32x4 (&bl)[RB]) {
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc[e][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[e]), as_bf16x8(bh[b]),
                                                          acc[e][b], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc[e][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[e]), as_bf16x8(bl[b]),
                                                          acc[e][b], 0, 0, 0);
  }
}

// Direct global->LDS loads of one step into a wave's stage: eight 1 KiB row
// loads (rows prow, prow + ldd, ...) and the 2 RB B operands at pb.  Lane
// l's 16 bytes land at byte 16 l of each 1 KiB slab.
template <int RB>
__device__ __forceinline__ void acc_issue_step(u32x4 (*slabs)[64], const uint16_t* prow,
                                               int64_t ldd, const uint16_t* pb) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_global_load_lds(prow + i * ldd, &slabs[i][0], 16, 0, 0);
#pragma unroll
  for (int h = 0; h < 2 * RB; ++h)
    __builtin_amdgcn_global_load_lds(pb + h * 512, &slabs[8 + h][0], 16, 0, 0);
}

// bf16 D.  A block owns 128 columns of D (rows of S) and one group of up to
// 64 ranks; its four waves take four contiguous slices of the 32-token steps.
// Lane l covers D rows 32s + 8(l>>4) + i (i = 0..7), columns c0 + 8(l&15) ..
// +7 -- sixteen lanes cover 256 contiguous bytes of a row.  Each wave stages
// one step at a time in a private 16 KiB LDS area filled by direct
// global->LDS loads (eight 1 KiB row loads, lane l's 16 bytes at offset
// 16 l, and the step's B operands, i.e. the packed XAt above).  A step is
// read back into registers completely before the next step's loads are
// issued, so the next step is in flight while this one computes, without
// holding registers.  The lane's 8 x 8 block is transposed in registers:
// for e = 0..7, operand A_e holds the eight tokens of column c0 + 8(l&15) +
// e, which is MFMA row m = l & 15 of instance e; the B operand has the same
// token for each (lane, element), so each 16x16x32 MFMA adds 32 tokens.
// Instance e, rank block b gives C[m][n] = S[c0 + 8m + e][16b + n], lane l
// holding m = 4(l>>4) + i, n = l & 15.  Each wave sums its slice in
// ascending step order (hi term then lo term per step), the slices are
// combined as w0 + (w1 + (w2 + w3)) through LDS and the total is added to S.
// The slicing depends on T alone, so the result bits do not depend on
// grouping.  A strip that reaches past column d of D, and the last step
// when T is not a multiple of 32, take guarded loads instead.
template <int RB>
__global__ __launch_bounds__(256, 2) void acc_bf16_kernel(AccGroupArgs g) {
  constexpr int kStage = 8 + 2 * RB;  // 1 KiB slabs per wave: rows, then B hi/lo
  __shared__ __align__(16) u32x4 stage[4][kStage][64];  // 64 KiB at RB = 4
  static_assert(sizeof(stage) >= sizeof(float) * RB * 32 * 64, "reduction fits in the stage");
  float* red = reinterpret_cast<float*>(&stage[0][0][0]);

  const int64_t logical = xcd_logical_block();
  if (logical >= g.tile_begin[g.n]) return;
  int item = 0;
  while (logical >= g.tile_begin[item + 1]) ++item;
  const int64_t local = logical - g.tile_begin[item];
  const int rg = (int)(local % g.ngroups);
  const int64_t c0 = (local / g.ngroups) * kAccCols;
  const uint16_t* __restrict__ D = static_cast<const uint16_t*>(g.D[item]);
  const int64_t ldd = g.ldd[item];
  const int64_t d = g.d[item];
  const int64_t T = g.T;
  const int rb0 = rg * RB;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int grp = lane >> 4;
  const int per = (g.nsteps + kAccSlices - 1) / kAccSlices;
  const int s_begin = wave * per;
  const int s_end = (s_begin + per) < g.nsteps ? (s_begin + per) : g.nsteps;

  const int64_t col = c0 + 8 * n;
  const bool col_full = col + 8 <= d;
  const uint16_t* __restrict__ planes = g.planes[item] + (int64_t)rb0 * 1024;

  f32x4 acc[8][RB];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[e][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Steps whose 32 rows all lie inside D: [s_begin, s_full).
  const int s_full = (int)((int64_t)s_end * kAccStep <= T ? s_end : T / kAccStep);
  int s_rest = s_begin;
  if (s_begin < s_full && c0 + kAccCols <= d) {
    // Interior strip: every lane's 16 bytes lie inside a row of D.
    const int64_t rstride = (int64_t)kAccStep * ldd;
    const int64_t bstride = (int64_t)g.nrb * 1024;
    const uint16_t* prow = D + ((int64_t)kAccStep * s_begin + 8 * grp) * ldd + col;
    const uint16_t* pb = planes + (int64_t)s_begin * bstride + lane * 8;
    acc_issue_step<RB>(stage[wave], prow, ldd, pb);
    for (int s = s_begin; s < s_full; ++s) {
      wait_vmcnt<0>();  // step s has landed in the stage
      u32x4 row[8], a[8], bh[RB], bl[RB];
#pragma unroll
      for (int i = 0; i < 8; ++i) row[i] = stage[wave][i][lane];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        bh[b] = stage[wave][8 + 2 * b][lane];
        bl[b] = stage[wave][9 + 2 * b][lane];
      }
      wait_lgkmcnt0();  // the stage has been read; it may be refilled
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < s_full) {
        prow += rstride;
        pb += bstride;
        acc_issue_step<RB>(stage[wave], prow, ldd, pb);
      }
      __builtin_amdgcn_sched_barrier(0);
      transpose8x8(row, a);
      acc_mfma_step<RB>(acc, a, bh, bl);
    }
    s_rest = s_full;
  }
  if (s_rest < s_end) {
    // Edge strips and the partial last step: guarded loads, no prefetch.
    for (int s = s_rest; s < s_end; ++s) {
      const int64_t t0 = (int64_t)kAccStep * s + 8 * grp;
      u32x4 row[8], a[8], bh[RB], bl[RB];
#pragma unroll
      for (int i = 0; i < 8; ++i) row[i] = load_drow(D, ldd, t0 + i, T, col, d, col_full);
      const uint16_t* pb = planes + (int64_t)s * g.nrb * 1024 + lane * 8;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        bh[b] = *reinterpret_cast<const u32x4*>(pb + 1024 * b);
        bl[b] = *reinterpret_cast<const u32x4*>(pb + 1024 * b + 512);
      }
      transpose8x8(row, a);
      acc_mfma_step<RB>(acc, a, bh, bl);
    }
  }
  __syncthreads();  // every wave is done with its stage

  // Fixed-order combination of the four slices, w0 + (w1 + (w2 + w3)), in
  // the accumulator layout (element (e, b, i) of lane l at [(e RB + b) 4 + i][l]).
  for (int w = kAccSlices - 1; w >= 1; --w) {
    if (wave == w) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* p = &red[((e * RB + b) * 4 + i) * 64 + lane];
            *p = (w == kAccSlices - 1) ? acc[e][b][i] : acc[e][b][i] + *p;
          }
    }
    __syncthreads();
  }
  // Wave 0 forms the total and stores it as a row-major tile [c][j] in the
  // second half of the stage.
  constexpr int TJ = 16 * RB;               // ranks per tile row
  constexpr int PER = kAccCols * TJ / 256;  // tile elements per thread
  float* tile = red + RB * 32 * 64;
  static_assert(sizeof(stage) >= 2 * sizeof(float) * RB * 32 * 64, "tile fits in the stage");
  if (wave == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cl = 8 * (4 * grp + i) + e;
          tile[cl * TJ + 16 * b + n] = acc[e][b][i] + red[((e * RB + b) * 4 + i) * 64 + lane];
        }
  }
  __syncthreads();
  // S += tile over the block's rows c0 .. c0 + 127 and ranks 16 rb0 ..
  // + 16 RB, consecutive threads on consecutive ranks of a row.
  const int64_t r = g.r;
  float* __restrict__ S = g.S[item];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = threadIdx.x + 256 * m;
    const int64_t c = c0 + idx / TJ;
    const int64_t j = 16 * rb0 + idx % TJ;
    if (c < d && j < r) S[c * r + j] += tile[idx];
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
  const int64_t nrb = (r + 15) / 16;
  return 16 * (nrb <= kAccGroupRB ? nrb : (nrb + kAccGroupRB - 1) / kAccGroupRB * kAccGroupRB);
}
int64_t acc_token_pad(int64_t T) { return (T + kAccStep - 1) / kAccStep * kAccStep; }
size_t acc_ws_bytes_per_item(int64_t T, int64_t r) {
  return (size_t)(2 * acc_rank_pad(r) * acc_token_pad(T) * sizeof(uint16_t));
}

hipError_t launch_regen_A(KeyArg key, int64_t r, int64_t k, bool int8_out, void* A,
                          hipStream_t s) {
  const int64_t n = r * ((k + 3) / 4);
  const float cr = (float)(1.0 / std::sqrt((double)r));
  hipLaunchKernelGGL(regen_A_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, key, r,
                     k, int8_out ? 1 : 0, cr, A);
  return hipGetLastError();
}

hipError_t launch_project(KeyArg key, int64_t T, int64_t k, int64_t r, const void* X,
                          bool bf16, int64_t ldx, float* XAt, hipStream_t s) {
  const double crd = 1.0 / std::sqrt((double)r);
  if (!bf16) {
    const int64_t n = T * r;
    hipLaunchKernelGGL(project_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       key, T, k, r, static_cast<const float*>(X), ldx, crd, XAt);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((T + 31) / 32));
  const float cr = (float)crd;
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  switch ((r + 31) / 32) {
#define LOGRA_PROJ_CASE(NB)                                                                   \
  case NB:                                                                                    \
    hipLaunchKernelGGL(project_bf16_kernel<NB>, grid, dim3(256), 0, s, key, T, k, r, Xb, ldx, \
                       cr, XAt);                                                              \
    break;
    LOGRA_PROJ_CASE(1)
    LOGRA_PROJ_CASE(2)
    LOGRA_PROJ_CASE(3)
    LOGRA_PROJ_CASE(4)
    LOGRA_PROJ_CASE(5)
    LOGRA_PROJ_CASE(6)
    LOGRA_PROJ_CASE(7)
    LOGRA_PROJ_CASE(8)
#undef LOGRA_PROJ_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_accumulate(int64_t T, int64_t r, bool bf16, const AccItem* items, int n,
                             hipStream_t s) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  AccGroupArgs g{};
  g.n = n;
  g.T = T;
  g.r = r;
  g.nsteps = (int)(acc_token_pad(T) / kAccStep);
  g.nrb = (int)(acc_rank_pad(r) / 16);
  const int rb = g.nrb < kAccGroupRB ? g.nrb : kAccGroupRB;
  g.ngroups = g.nrb / rb;
  for (int i = 0; i < n; ++i) {
    g.D[i] = items[i].D;
    g.XAt[i] = items[i].XAt;
    g.S[i] = items[i].S;
    g.planes[i] = static_cast<uint16_t*>(items[i].ws);
    g.d[i] = items[i].d;
    g.ldd[i] = items[i].ldd;
  }
  if (!bf16) {
    int64_t maxdr = 0;
    for (int i = 0; i < n; ++i) maxdr = std::max(maxdr, g.d[i] * r);
    hipLaunchKernelGGL(acc_f32_kernel, dim3((unsigned)((maxdr + 255) / 256), (unsigned)n),
                       dim3(256), 0, s, g);
    return hipGetLastError();
  }
  {
    const int64_t chunks = (int64_t)g.nsteps * g.nrb;
    hipLaunchKernelGGL(acc_pack_kernel, dim3((unsigned)((chunks + 3) / 4), (unsigned)n),
                       dim3(256), 0, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  g.tile_begin[0] = 0;
  for (int i = 0; i < n; ++i)
    g.tile_begin[i + 1] = g.tile_begin[i] + (g.d[i] + kAccCols - 1) / kAccCols * g.ngroups;
  const int64_t tiles = g.tile_begin[n];
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  switch (rb) {
    case 1: hipLaunchKernelGGL(acc_bf16_kernel<1>, grid, dim3(256), 0, s, g); break;
    case 2: hipLaunchKernelGGL(acc_bf16_kernel<2>, grid, dim3(256), 0, s, g); break;
    case 3: hipLaunchKernelGGL(acc_bf16_kernel<3>, grid, dim3(256), 0, s, g); break;
    case 4: hipLaunchKernelGGL(acc_bf16_kernel<4>, grid, dim3(256), 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace logra
