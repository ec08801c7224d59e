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
constexpr int kAccStep = 32;        // tokens per MFMA step
constexpr int kAccCols = 128;       // columns of D per wave: 16 lanes x 8
constexpr int kAccWaves = 4;        // waves per block: 2 strips x 2 token halves
constexpr int kAccBlockCols = 2 * kAccCols;
constexpr int kAccGroupRB = 4;      // 16-rank blocks per rank group (64 ranks)
constexpr int kAccRing = 3;         // steps in flight per block (LDS ring depth)

struct AccGroupArgs {
  const void* D[kMaxGroup];
  const float* XAt[kMaxGroup];
  float* S[kMaxGroup];
  uint16_t* planes[kMaxGroup];  // packed XAt of each item (workspace)
  int64_t d[kMaxGroup];
  int64_t ldd[kMaxGroup];
  int64_t nq[kMaxGroup];        // 256-column blocks of each item
  int64_t tile_begin[kMaxGroup + 1];
  int n;
  int64_t T, r;
  int nsteps;   // ceil(T / 32)
  int nrb;      // 16-rank blocks packed: ceil(r / 16), rounded up to a
                // multiple of 4 when there is more than one rank group
  int rb;       // 16-rank blocks per rank group: min(nrb, 4)
  int ngroups;  // nrb / rb rank groups
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

// 32-bit LDS address of a shared-memory object.
template <typename Tp>
__device__ __forceinline__ uint32_t lds_addr(Tp* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) Tp*)p;
}

// LDS reads of consecutive 1 KiB slabs (lane l's 16 bytes at byte 16 l of
// each) that complete inside the statement: the compiler never sees an LDS
// read it could order against pending direct global->LDS loads, and the
// results exist only once the data has arrived.  The outputs are
// early-clobber: a destination sharing a register with the address would be
// overwritten by the first read's data while later reads still use it.
__device__ __forceinline__ void lds_read8(uint32_t a, u32x4 (&r)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
      : "v"(a)
      : "memory");
}
__device__ __forceinline__ void lds_read2(uint32_t a, u32x4& x, u32x4& y) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %2 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x), "=&v"(y)
      : "v"(a)
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

// Rows (8 slabs at ad) and B operands (2 RB slabs at ab: hi, lo per rank
// block) of one step.
template <int RB>
__device__ __forceinline__ void acc_read_step(uint32_t ad, uint32_t ab, u32x4 (&row)[8],
                                              u32x4 (&bh)[RB], u32x4 (&bl)[RB]) {
  if constexpr (RB == 4) {
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %16 offset:1024\n\t"
        "ds_read_b128 %2, %16 offset:2048\n\t"
        "ds_read_b128 %3, %16 offset:3072\n\t"
        "ds_read_b128 %4, %16 offset:4096\n\t"
        "ds_read_b128 %5, %16 offset:5120\n\t"
        "ds_read_b128 %6, %16 offset:6144\n\t"
        "ds_read_b128 %7, %16 offset:7168\n\t"
        "ds_read_b128 %8, %17\n\t"
        "ds_read_b128 %9, %17 offset:1024\n\t"
        "ds_read_b128 %10, %17 offset:2048\n\t"
        "ds_read_b128 %11, %17 offset:3072\n\t"
        "ds_read_b128 %12, %17 offset:4096\n\t"
        "ds_read_b128 %13, %17 offset:5120\n\t"
        "ds_read_b128 %14, %17 offset:6144\n\t"
        "ds_read_b128 %15, %17 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(row[0]), "=&v"(row[1]), "=&v"(row[2]), "=&v"(row[3]), "=&v"(row[4]), "=&v"(row[5]),
          "=&v"(row[6]), "=&v"(row[7]), "=&v"(bh[0]), "=&v"(bl[0]), "=&v"(bh[1]), "=&v"(bl[1]),
          "=&v"(bh[2]), "=&v"(bl[2]), "=&v"(bh[3]), "=&v"(bl[3])
        : "v"(ad), "v"(ab)
        : "memory");
  } else {
    lds_read8(ad, row);
#pragma unroll
    for (int b = 0; b < RB; ++b) lds_read2(ab + 2048 * b, bh[b], bl[b]);
  }
}

// acc[e][b] += A_e B_b over one 32-token step for rank block b only.
template <int RB>
__device__ __forceinline__ void acc_mfma_rb(f32x4 (&acc)[8][RB], const u32x4 (&a)[8], int b,
                                            u32x4 bh, u32x4 bl) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    acc[e][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[e]), as_bf16x8(bh),
                                                        acc[e][b], 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    acc[e][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[e]), as_bf16x8(bl),
                                                        acc[e][b], 0, 0, 0);
}

// Direct global->LDS loads of a wave's eight 1 KiB row slabs of one step:
// rows prow, prow + ldd, ...; lane l's 16 bytes land at byte 16 l.
__device__ __forceinline__ void acc_issue_rows(u32x4 (*slabs)[64], const uint16_t* prow,
                                               int64_t ldd) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_global_load_lds(prow + i * ldd, &slabs[i][0], 16, 0, 0);
}

// Direct global->LDS load of row slab i (row pointer prow) of a wave.
__device__ __forceinline__ void acc_issue_rows_one(u32x4 (*slabs)[64], int i,
                                                   const uint16_t* prow) {
  __builtin_amdgcn_global_load_lds(prow, &slabs[i][0], 16, 0, 0);
}

// Direct global->LDS loads of one wave's share of a half's B operands for
// one step: the 1 KiB operands j = strip, strip + 2, ... of the 2 RB at pb.
template <int RB>
__device__ __forceinline__ void acc_issue_b(u32x4 (*bs)[64], const uint16_t* pb, int strip) {
#pragma unroll
  for (int j0 = 0; j0 < 2 * RB; j0 += 2)
    __builtin_amdgcn_global_load_lds(pb + (j0 + strip) * 512, &bs[j0 + strip][0], 16, 0, 0);
}

// bf16 D.  A block covers 256 columns of D (rows of S) and one group of up
// to 64 ranks over all T tokens.  Its four waves are two 128-column strips
// times two token halves: wave w takes the strip of columns
// c0 = 256 q + 128 (w & 1) onwards and, for w >> 1 = 0 (1), the steps
// [0, h) ([h, nsteps)) with h = ceil(nsteps / 2).  Lane l covers D rows
// 32s + 8(l>>4) + i (i = 0..7), columns c0 + 8(l&15) .. +7, so sixteen lanes
// read 256 contiguous bytes of a row.  A three-step ring in LDS is filled by
// direct global->LDS loads: every wave streams its own rows, and each half's
// B operands (the packed XAt above) are loaded once per step by that half's
// two waves and shared by both strips.  Two steps are in flight while a
// third computes.  The lane's 8 x 8 block is transposed in registers: for
// e = 0..7, operand A_e holds the eight tokens of column c0 + 8(l&15) + e,
// which is MFMA row m = l & 15 of instance e; the B operand has the same
// token for each (lane, element), so each 16x16x32 MFMA adds 32 tokens.
// Instance e, rank block b gives C[m][n] = S[c0 + 8m + e][16b + n], lane l
// holding m = 4(l>>4) + i, n = l & 15.  Each wave sums its half's steps in
// ascending order (hi term then lo term per step); the second half's sum R
// passes through LDS to the first half's wave, which forms L + R, and the
// block adds that to S through an LDS tile so that S is read and written
// in whole rows.  The order depends on T alone, so grouped and single calls
// give the same bits.  Strips that reach past column d take guarded loads;
// rows past T (last step only) are loaded from row T - 1 and zeroed.
template <int RB>
__global__ __launch_bounds__(256, 1) void acc_bf16_kernel(AccGroupArgs g) {
  constexpr int R = kAccRing;
  constexpr int NB = 2 * RB;                  // B operands per step and half
  constexpr int kRing = R * kAccWaves * 8;    // 1 KiB row slabs
  __shared__ __align__(16) u32x4 smem[(kRing + R * 2 * NB) * 64];  // 144 KiB at RB = 4
  u32x4 (*dring)[kAccWaves][8][64] = reinterpret_cast<u32x4 (*)[kAccWaves][8][64]>(smem);
  u32x4 (*bring)[2][NB][64] = reinterpret_cast<u32x4 (*)[2][NB][64]>(smem + kRing * 64);

  const int64_t logical = xcd_logical_block();
  if (logical >= g.tile_begin[g.n]) return;
  int item = 0;
  while (logical >= g.tile_begin[item + 1]) ++item;
  const int64_t local = logical - g.tile_begin[item];
  const int rg = (int)(local % g.ngroups);  // rank groups of a column block are adjacent
  const int64_t q = local / g.ngroups;
  const uint16_t* __restrict__ D = static_cast<const uint16_t*>(g.D[item]);
  const int64_t ldd = g.ldd[item];
  const int64_t d = g.d[item];
  const int64_t T = g.T;
  const int rb0 = rg * RB;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = wave & 1;
  const int half = wave >> 1;
  const int n = lane & 15;
  const int grp = lane >> 4;
  const int nsteps = g.nsteps;
  const int h = (nsteps + 1) >> 1;
  const int s_begin = half ? h : 0;
  const int s_end = half ? nsteps : h;

  const int64_t c0 = q * kAccBlockCols + kAccCols * strip;  // this wave's strip
  const int64_t col = c0 + 8 * n;
  const bool active = c0 < d;                  // uniform per wave
  const bool interior = c0 + kAccCols <= d;    // uniform per wave
  const bool col_full = col + 8 <= d;
  const uint16_t* __restrict__ planes = g.planes[item] + (int64_t)rb0 * 1024 + lane * 8;
  const int64_t bstride = (int64_t)g.nrb * 1024;

  f32x4 acc[8][RB];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[e][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads of iteration k (step s_begin + k) into ring slot k % R: this
  // wave's share of its half's B operands and, for an interior strip, its
  // eight row slabs.  Iterations past the half re-read its last step
  // (already cached) so that every iteration issues the same number of
  // loads; rows past T read row T - 1.
  auto issue = [&](int k, bool rows) {
    const int st = s_begin + k;
    const int sc = st < s_end ? st : s_end - 1;
    const int slot = k % R;
    acc_issue_b<RB>(bring[slot][half], planes + (int64_t)sc * bstride, strip);
    if (!rows) return;
    const int64_t t0 = (int64_t)kAccStep * sc + 8 * grp;
    if ((int64_t)kAccStep * (sc + 1) <= T) {
      acc_issue_rows(dring[slot][wave], D + t0 * ldd + col, ldd);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = t0 + i < T ? t0 + i : T - 1;
        acc_issue_rows_one(dring[slot][wave], i, D + t * ldd + col);
      }
    }
  };

  if (interior) {
#pragma unroll
    for (int k = 0; k < R - 1; ++k) issue(k, true);
    for (int k = 0; k < h; ++k) {
      // Iteration k has landed once only the loads of iteration k + 1 (eight
      // row slabs and RB B operands) remain.
      static_assert(R == 3, "the wait count assumes a three-step ring");
      wait_vmcnt<8 + RB>();
      ring_barrier();  // both waves' shares of the half's B operands have landed
      const int slot = k % R;
      const int s = s_begin + k;
      u32x4 row[8], a[8], bh[RB], bl[RB];
      acc_read_step<RB>(lds_addr(&dring[slot][wave][0][lane]),
                        lds_addr(&bring[slot][half][0][lane]), row, bh, bl);
      if ((int64_t)kAccStep * (s + 1) > T) {
        const int64_t t0 = (int64_t)kAccStep * s + 8 * grp;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (t0 + i >= T) row[i] = u32x4{0u, 0u, 0u, 0u};
      }
      // Refill the slot every wave finished reading before this barrier.
      issue(k + R - 1, true);
      if (s < s_end) {
        transpose8x8(row, a);
        acc_mfma_step<RB>(acc, a, bh, bl);
      }
    }
  } else {
    // Edge or empty strip: the same barriers and B shares; rows by guarded
    // loads when the strip starts inside D.
#pragma unroll
    for (int k = 0; k < R - 1; ++k) issue(k, false);
    for (int k = 0; k < h; ++k) {
      wait_vmcnt<0>();
      ring_barrier();
      const int slot = k % R;
      const int s = s_begin + k;
      if (active && s < s_end) {
        const int64_t t0 = (int64_t)kAccStep * s + 8 * grp;
        u32x4 row[8], a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) row[i] = load_drow(D, ldd, t0 + i, T, col, d, col_full);
        transpose8x8(row, a);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          u32x4 bh, bl;
          lds_read2(lds_addr(&bring[slot][half][2 * b][lane]), bh, bl);
          acc_mfma_rb<RB>(acc, a, b, bh, bl);
        }
      }
      issue(k + R - 1, false);
    }
  }
  wait_vmcnt<0>();  // no load may still target LDS past this point

  // This thread's share of the block's S tile (256 rows x 16 RB ranks): rank
  // j0 + lane of rows row0 + wave + 4k, so a wave reads whole row segments.
  // The loads are issued now and complete while L + R is formed.
  constexpr int TJ = 16 * RB;
  constexpr int kRowsPerThread = kAccBlockCols / kAccWaves;
  float* __restrict__ S = g.S[item];
  const int64_t r = g.r;
  const int64_t row0 = q * kAccBlockCols + wave;
  const int64_t j = 16 * (int64_t)rb0 + lane;
  const bool jok = lane < TJ && j < r;
  int64_t rstride = 4 * r;
  const int64_t jc = j < r ? j : r - 1;  // in-bounds address for idle lanes
  float sv[kRowsPerThread];
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int64_t row = row0 + 4 * k < d ? row0 + 4 * k : d - 1;
    sv[k] = S[row * r + jc];
  }
  // Keep the addresses from being held live across the exchange below.
  asm volatile("" : "+s"(rstride));
  ring_barrier();  // every wave is done with the ring

  // R of each strip, in accumulator order: element (e, b) of lane l at
  // [strip][(e RB + b) 64 + l].  Then the L + R tile, rows of TJ + 1 floats.
  f32x4* xr = reinterpret_cast<f32x4*>(smem);
  float* yt = reinterpret_cast<float*>(smem + 2 * 8 * RB * 64);
  constexpr int YS = TJ + 1;
  if (half == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int b = 0; b < RB; ++b) xr[(strip * 8 * RB + e * RB + b) * 64 + lane] = acc[e][b];
  }
  wait_lgkmcnt0();
  ring_barrier();
  if (half == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const f32x4 rr = xr[(strip * 8 * RB + e * RB + b) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * grp + i;
          yt[(kAccCols * strip + 8 * m + e) * YS + 16 * b + n] = acc[e][b][i] + rr[i];
        }
      }
  }
  wait_lgkmcnt0();
  ring_barrier();
  wait_vmcnt<0>();  // the S loads (long complete): no waits between the stores below
  if (jok) {
    float* p = S + row0 * r + j;
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
      if (row0 + 4 * k < d) *p = sv[k] + yt[(wave + 4 * k) * YS + lane];
      p += rstride;
    }
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
static int64_t acc_col_blocks(int64_t d) { return (d + kAccBlockCols - 1) / kAccBlockCols; }
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
  g.rb = g.nrb < kAccGroupRB ? g.nrb : kAccGroupRB;
  g.ngroups = g.nrb / g.rb;
  for (int i = 0; i < n; ++i) {
    g.D[i] = items[i].D;
    g.XAt[i] = items[i].XAt;
    g.S[i] = items[i].S;
    g.d[i] = items[i].d;
    g.ldd[i] = items[i].ldd;
    g.nq[i] = acc_col_blocks(items[i].d);
    g.planes[i] = static_cast<uint16_t*>(items[i].ws);
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
  for (int i = 0; i < n; ++i) g.tile_begin[i + 1] = g.tile_begin[i] + g.nq[i] * g.ngroups;
  const int64_t tiles = g.tile_begin[n];
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  switch (g.rb) {
    case 1: hipLaunchKernelGGL(acc_bf16_kernel<1>, grid, dim3(256), 0, s, g); break;
    case 2: hipLaunchKernelGGL(acc_bf16_kernel<2>, grid, dim3(256), 0, s, g); break;
    case 3: hipLaunchKernelGGL(acc_bf16_kernel<3>, grid, dim3(256), 0, s, g); break;
    case 4: hipLaunchKernelGGL(acc_bf16_kernel<4>, grid, dim3(256), 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace logra
