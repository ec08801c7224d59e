// Reconstruction-cosine diagnostic: how much of a dense gradient G [d x k]
// the sketch keeps, cos(G, (G A^T) A) ("LoGRA: Scaling LLM Reinforcement
// Learning with Low-Rank Gradient Sketches", paperpeel.com, App. D.3
// "Reconstruction heatmaps").
//
// With S = G A^T [d x r], two identities avoid forming (G A^T) A:
//   <G, S A>_F = sum_i sum_l S_il (G A^T)_il = ||S||_F^2,
//   ||S A||_F^2 = sum_i S_i (A A^T) S_i^T,
// and A A^T = c_r^2 (k - 2 popcount(sigma_j xor sigma_l)) is exact from the
// sign bits.  S comes from the projection kernel; the sums run in fp64 in a
// fixed order (per-block trees, then one block), so the result is
// reproducible.
#include "device_common.h"
#include "kernels.h"

namespace logra {

namespace {

constexpr int kCosRows = 32;  // rows of G and S per block

// Sign words of A: bits[j nw + w], bit b set meaning sigma[j][64 w + b] = -1;
// zero past column k.
__global__ __launch_bounds__(256) void sign_words_kernel(KeyArg key, int64_t r, int64_t k,
                                                         int64_t nw, uint64_t* __restrict__ bits) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= r * nw) return;
  const int64_t j = idx / nw;
  const int64_t w = idx - j * nw;
  const Philox4 p = sigma_block(KeyWords{key.k0, key.k1}, (uint64_t)j, (uint64_t)(w >> 2));
  const int q = (int)(w & 3);
  uint64_t v = q == 0 ? p.w[0] : q == 1 ? p.w[1] : q == 2 ? p.w[2] : p.w[3];
  const int64_t left = k - 64 * w;
  if (left < 64) v &= (1ull << left) - 1ull;
  bits[idx] = v;
}

// M = A A^T [r x r] in fp64: c^2 (k - 2 popcount(bits_j xor bits_l)), c the
// fp32 c_r the projection applies.
__global__ __launch_bounds__(256) void sign_gram_kernel(int64_t r, int64_t k, int64_t nw, double c2,
                                                        const uint64_t* __restrict__ bits,
                                                        double* __restrict__ M) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= r * r) return;
  const int64_t j = idx / r;
  const int64_t l = idx - j * r;
  int64_t pop = 0;
  for (int64_t w = 0; w < nw; ++w) pop += __popcll(bits[j * nw + w] ^ bits[l * nw + w]);
  M[idx] = c2 * (double)(k - 2 * pop);
}

// M = A A^T [r x r] in fp64 from an explicit fp32 A [r x k]: one block per
// 16 x 16 tile of M, the two 16-row slices of A staged through LDS 64
// columns at a time; each thread sums one entry in column order.
__global__ __launch_bounds__(256) void explicit_gram_kernel(int64_t r, int64_t k,
                                                            const float* __restrict__ A,
                                                            double* __restrict__ M) {
  __shared__ float sa[16][65], sb[16][65];
  const int tj = threadIdx.x >> 4, tl = threadIdx.x & 15;
  const int64_t j0 = (int64_t)blockIdx.y * 16, l0 = (int64_t)blockIdx.x * 16;
  double acc = 0.0;
  for (int64_t c0 = 0; c0 < k; c0 += 64) {
    for (int idx = threadIdx.x; idx < 16 * 64; idx += 256) {
      const int row = idx >> 6, col = idx & 63;
      const int64_t c = c0 + col;
      sa[row][col] = (j0 + row < r && c < k) ? A[(j0 + row) * k + c] : 0.f;
      sb[row][col] = (l0 + row < r && c < k) ? A[(l0 + row) * k + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int col = 0; col < 64; ++col) acc += (double)sa[tj][col] * (double)sb[tl][col];
    __syncthreads();
  }
  if (j0 + tj < r && l0 + tl < r) M[(j0 + tj) * r + l0 + tl] = acc;
}

// Fixed-tree sum over the block's 256 threads (every thread gets the total).
__device__ double cos_block_sum(double x, double* red) {
  __syncthreads();
  red[threadIdx.x] = x;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  return red[0];
}

// Per block of 32 rows: sum G^2, sum S^2 and sum_i S_i M S_i^T, written to
// part[b], part[nb + b], part[2 nb + b].  Thread j < r forms t_ij = (M S_i^T)_j
// for the block's rows, streaming M once per block.
template <bool BF16>
__global__ __launch_bounds__(256) void cos_rows_kernel(int64_t d, int64_t k, int64_t r,
                                                       const void* __restrict__ G, int64_t ldg,
                                                       const float* __restrict__ S,
                                                       const double* __restrict__ M,
                                                       double* __restrict__ part) {
  __shared__ double sS[kCosRows][kMaxRank];
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * kCosRows;
  const int nrows = d - row0 < kCosRows ? (int)(d - row0) : kCosRows;
  // ||G||^2 of the block's rows: 16-byte loads (rows are 16-byte aligned),
  // then the tail of each row element by element.
  constexpr int V = BF16 ? 8 : 4;  // elements per 16 bytes
  const int64_t kv = k / V;
  double g2 = 0.0;
  for (int i = 0; i < nrows; ++i) {
    const int64_t base = (row0 + i) * ldg;
    for (int64_t c = tid; c < kv; c += 256) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(
          static_cast<const char*>(G) + (base + c * V) * (BF16 ? 2 : 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (BF16) {
          const double lo = (double)bf16_bits_to_f32(w[q] & 0xFFFFu);
          const double hi = (double)bf16_bits_to_f32(w[q] >> 16);
          g2 += lo * lo + hi * hi;
        } else {
          const double x = (double)__uint_as_float(w[q]);
          g2 += x * x;
        }
      }
    }
    for (int64_t c = kv * V + tid; c < k; c += 256) {
      const double x = BF16 ? (double)bf16_bits_to_f32(static_cast<const uint16_t*>(G)[base + c])
                            : (double)static_cast<const float*>(G)[base + c];
      g2 += x * x;
    }
  }
  double s2 = 0.0;
  for (int idx = tid; idx < kCosRows * kMaxRank; idx += 256) {
    const int i = idx / kMaxRank, j = idx - i * kMaxRank;
    const double x = (i < nrows && j < r) ? (double)S[(row0 + i) * r + j] : 0.0;
    sS[i][j] = x;
    s2 += x * x;
  }
  __syncthreads();
  double q = 0.0;
  if (tid < r) {
    double t[kCosRows];
#pragma unroll
    for (int i = 0; i < kCosRows; ++i) t[i] = 0.0;
    for (int64_t l = 0; l < r; ++l) {
      const double m = M[l * r + tid];  // M is symmetric: row l, coalesced over threads
#pragma unroll
      for (int i = 0; i < kCosRows; ++i) t[i] += m * sS[i][l];
    }
#pragma unroll
    for (int i = 0; i < kCosRows; ++i) q += sS[i][tid] * t[i];
  }
  const double G2 = cos_block_sum(g2, red);
  const double S2 = cos_block_sum(s2, red);
  const double Q = cos_block_sum(q, red);
  if (tid == 0) {
    part[blockIdx.x] = G2;
    part[gridDim.x + blockIdx.x] = S2;
    part[2 * gridDim.x + blockIdx.x] = Q;
  }
}

// out = {cos, ||G||^2, ||S||^2, ||S A||^2}.
__global__ __launch_bounds__(256) void cos_final_kernel(int64_t nb, const double* __restrict__ part,
                                                        double* __restrict__ out) {
  __shared__ double red[256];
  double a = 0.0, b = 0.0, c = 0.0;
  for (int64_t i = threadIdx.x; i < nb; i += 256) {
    a += part[i];
    b += part[nb + i];
    c += part[2 * nb + i];
  }
  const double G2 = cos_block_sum(a, red);
  const double S2 = cos_block_sum(b, red);
  const double Q = cos_block_sum(c, red);
  if (threadIdx.x == 0) {
    out[0] = (G2 > 0.0 && Q > 0.0) ? S2 / (sqrt(G2) * sqrt(Q)) : 0.0;
    out[1] = G2;
    out[2] = S2;
    out[3] = Q;
  }
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct CosWs {
  float* S;
  uint64_t* bits;
  double* M;
  double* part;
};

CosWs cos_ws_layout(void* ws, int64_t d, int64_t k, int64_t r) {
  char* p = static_cast<char*>(ws);
  CosWs w;
  w.S = reinterpret_cast<float*>(p);
  p += round256((size_t)(d * r) * 4);
  w.bits = reinterpret_cast<uint64_t*>(p);
  p += round256((size_t)(r * ((k + 63) / 64)) * 8);
  w.M = reinterpret_cast<double*>(p);
  p += round256((size_t)(r * r) * 8);
  w.part = reinterpret_cast<double*>(p);
  return w;
}

}  // namespace

size_t reconstruction_cosine_ws_bytes(int64_t d, int64_t k, int64_t r) {
  const int64_t nb = (d + kCosRows - 1) / kCosRows;
  return round256((size_t)(d * r) * 4) + round256((size_t)(r * ((k + 63) / 64)) * 8) +
         round256((size_t)(r * r) * 8) + round256((size_t)(3 * nb) * 8);
}

hipError_t launch_reconstruction_cosine(KeyArg key, int64_t d, int64_t k, int64_t r, const void* G,
                                        bool bf16, int64_t ldg, double* out, void* ws,
                                        hipStream_t s, const float* A, const void* A_packed) {
  const CosWs w = cos_ws_layout(ws, d, k, r);
  hipError_t e = launch_project(key, d, k, r, G, bf16, ldg, w.S, nullptr, s, A_packed);
  if (e != hipSuccess) return e;
  if (A != nullptr) {
    const dim3 g((unsigned)((r + 15) / 16), (unsigned)((r + 15) / 16));
    hipLaunchKernelGGL(explicit_gram_kernel, g, dim3(256), 0, s, r, k, A, w.M);
  } else {
    const int64_t nw = (k + 63) / 64;
    hipLaunchKernelGGL(sign_words_kernel, dim3((unsigned)((r * nw + 255) / 256)), dim3(256), 0, s,
                       key, r, k, nw, w.bits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const double c = (double)(float)(1.0 / std::sqrt((double)r));
    hipLaunchKernelGGL(sign_gram_kernel, dim3((unsigned)((r * r + 255) / 256)), dim3(256), 0, s, r,
                       k, nw, c * c, w.bits, w.M);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nb = (d + kCosRows - 1) / kCosRows;
  if (bf16)
    hipLaunchKernelGGL(cos_rows_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, d, k, r, G, ldg,
                       w.S, w.M, w.part);
  else
    hipLaunchKernelGGL(cos_rows_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, d, k, r, G, ldg,
                       w.S, w.M, w.part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cos_final_kernel, dim3(1), dim3(256), 0, s, nb, w.part, out);
  return hipGetLastError();
}

}  // namespace logra
