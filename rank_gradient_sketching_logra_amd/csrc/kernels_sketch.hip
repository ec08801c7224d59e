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

// Packed projected input: two bf16 planes (hi, lo) of XAt^T, [RP x TP] each,
// zero-padded to whole 32-rank blocks and 256-token chunks, so one 16-byte
// load is one MFMA B operand (8 consecutive tokens of one rank).
constexpr int kTokPad = 256;

struct AccGroupArgs {
  const void* D[kMaxGroup];
  const float* XAt[kMaxGroup];
  float* S[kMaxGroup];
  uint16_t* planes[kMaxGroup];
  int64_t d[kMaxGroup];
  int64_t ldd[kMaxGroup];
  int64_t tile_begin[kMaxGroup + 1];
  int n;
  int64_t T, TP, r, RP;
};

__global__ void acc_pack_kernel(AccGroupArgs g) {
  const int item = blockIdx.y;
  const int64_t ntg = g.TP >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= ntg * g.RP) return;
  const int64_t tg = idx / g.RP;
  const int64_t j = idx - tg * g.RP;
  const float* __restrict__ x = g.XAt[item];
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = tg * 8 + i;
    const float v = (t < g.T && j < g.r) ? x[t * g.r + j] : 0.f;
    split_hi_lo(v, h[i], l[i]);
  }
  uint16_t* hi = g.planes[item] + j * g.TP + tg * 8;
  uint16_t* lo = hi + g.RP * g.TP;
  u32x4 vh, vl;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    vh[p] = h[2 * p] | (h[2 * p + 1] << 16);
    vl[p] = l[2 * p] | (l[2 * p + 1] << 16);
  }
  *reinterpret_cast<u32x4*>(hi) = vh;
  *reinterpret_cast<u32x4*>(lo) = vl;
}

// bf16 D.  One block = MC = 32*WM columns of D (rows of S) x all ranks x all
// tokens; waves form a WM x (4/WM) grid over (column block, rank blocks).
// D is staged through LDS in row-major chunks of TC tokens (prefetched one
// chunk ahead in registers); the MFMA A operand (8 tokens of one column) is
// read from LDS as 16-bit values.  The B operand (8 tokens of one rank) is
// one 16-byte load from the packed planes.  Each output element accumulates
// over tokens in ascending 16-token steps, hi term then lo term, whatever
// the tiling -- so single and grouped calls give identical bits.
template <int WM, int NBW, int TC>
__global__ __launch_bounds__(256) void acc_bf16_kernel(AccGroupArgs g) {
  constexpr int WN = 4 / WM;
  constexpr int MC = 32 * WM;
  constexpr int PITCH = MC + 4;            // 16-bit elements per LDS row
  constexpr int VPR = MC / 8;              // 16-byte vectors per chunk row
  constexpr int NV = TC * VPR / 256;       // vectors per thread per chunk
  static_assert(NV >= 1 && TC * VPR % 256 == 0, "chunk must split evenly");
  __shared__ __align__(16) uint16_t Ds[TC * PITCH];

  const int64_t logical = xcd_logical_block();
  if (logical >= g.tile_begin[g.n]) return;
  int item = 0;
  while (logical >= g.tile_begin[item + 1]) ++item;
  const int64_t c0 = (logical - g.tile_begin[item]) * MC;
  const uint16_t* __restrict__ D = static_cast<const uint16_t*>(g.D[item]);
  const int64_t ldd = g.ldd[item];
  const int64_t d = g.d[item];
  const uint16_t* __restrict__ planes = g.planes[item];
  const int64_t T = g.T, TP = g.TP, RP = g.RP;
  const int NBT = (int)(RP >> 5);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int half = lane >> 5;

  u32x4 pre[NV];
  auto load_chunk = [&](int64_t tbase) {
#pragma unroll
    for (int p = 0; p < NV; ++p) {
      const int v = tid + 256 * p;
      const int row = v / VPR;
      const int cv = v - row * VPR;
      pre[p] = load_bf16x8(D, ldd, tbase + row, c0 + cv * 8, T, d);
    }
  };

  f32x16 acc[NBW];
#pragma unroll
  for (int q = 0; q < NBW; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[q][e] = 0.f;

  const int64_t nch = (T + TC - 1) / TC;
  load_chunk(0);
  for (int64_t ch = 0; ch < nch; ++ch) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NV; ++p) {
      const int v = tid + 256 * p;
      const int row = v / VPR;
      const int cv = v - row * VPR;
      uint32_t* dst = reinterpret_cast<uint32_t*>(&Ds[row * PITCH + cv * 8]);
      dst[0] = pre[p][0];
      dst[1] = pre[p][1];
      dst[2] = pre[p][2];
      dst[3] = pre[p][3];
    }
    __syncthreads();
    const int64_t tbase = ch * TC;
    if (ch + 1 < nch) load_chunk(tbase + TC);

#pragma unroll
    for (int s = 0; s < TC / 16; ++s) {
      u32x4 a;
      const uint16_t* col = &Ds[(16 * s + 8 * half) * PITCH + 32 * wm + (lane & 31)];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        a[ii] = (uint32_t)col[(2 * ii) * PITCH] | ((uint32_t)col[(2 * ii + 1) * PITCH] << 16);
#pragma unroll
      for (int q = 0; q < NBW; ++q) {
        const int nb = wn + WN * q;
        if (nb < NBT) {
          const uint16_t* ph =
              planes + (int64_t)(nb * 32 + (lane & 31)) * TP + tbase + 16 * s + 8 * half;
          const u32x4 bh = *reinterpret_cast<const u32x4*>(ph);
          const u32x4 bl = *reinterpret_cast<const u32x4*>(ph + RP * TP);
          acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bh), acc[q],
                                                           0, 0, 0);
          acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bl), acc[q],
                                                           0, 0, 0);
        }
      }
    }
  }

  float* __restrict__ S = g.S[item];
  const int64_t r = g.r;
#pragma unroll
  for (int q = 0; q < NBW; ++q) {
    const int nb = wn + WN * q;
    if (nb >= NBT) continue;
    const int64_t j = nb * 32 + (lane & 31);
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) {
      const int64_t c = c0 + 32 * wm + 8 * (reg >> 2) + 4 * half + (reg & 3);
      if (c < d && j < r) S[c * r + j] += acc[q][reg];
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

int64_t acc_rank_pad(int64_t r) { return (r + 31) / 32 * 32; }
int64_t acc_token_pad(int64_t T) { return (T + kTokPad - 1) / kTokPad * kTokPad; }
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
  g.TP = acc_token_pad(T);
  g.RP = acc_rank_pad(r);
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
  // Pack XAt into hi/lo planes.
  {
    const int64_t m = (g.TP / 8) * g.RP;
    hipLaunchKernelGGL(acc_pack_kernel, dim3((unsigned)((m + 255) / 256), (unsigned)n),
                       dim3(256), 0, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nbt = (int)(g.RP / 32);
  const int wm = (nbt == 1) ? 4 : 2;
  const int mc = 32 * wm;
  g.tile_begin[0] = 0;
  for (int i = 0; i < n; ++i) g.tile_begin[i + 1] = g.tile_begin[i] + (g.d[i] + mc - 1) / mc;
  const int64_t tiles = g.tile_begin[n];
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  if (nbt == 1) {
    hipLaunchKernelGGL((acc_bf16_kernel<4, 1, 128>), grid, dim3(256), 0, s, g);
  } else {
    switch ((nbt + 1) / 2) {
      case 1:
        hipLaunchKernelGGL((acc_bf16_kernel<2, 1, 128>), grid, dim3(256), 0, s, g);
        break;
      case 2:
        hipLaunchKernelGGL((acc_bf16_kernel<2, 2, 128>), grid, dim3(256), 0, s, g);
        break;
      case 3:
        hipLaunchKernelGGL((acc_bf16_kernel<2, 3, 64>), grid, dim3(256), 0, s, g);
        break;
      case 4:
        hipLaunchKernelGGL((acc_bf16_kernel<2, 4, 64>), grid, dim3(256), 0, s, g);
        break;
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace logra
