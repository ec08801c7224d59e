// RowAdam scaling of the sketch, predicted-KL coefficient q and step rule.
//
// Sources: paperlayer.ai summary of the LoGRA paper, "B. RowAdam" (row-wise
// running squared magnitude, Frobenius norm restored, d statistics that
// persist across projection refreshes); "LoGRA: Scaling LLM Reinforcement
// Learning with Low-Rank Gradient Sketches" (paperpeel.com) App. D.1 Table 4
// (beta2, no first moment, relative epsilon), §2.3 and App. A.1 (q as the
// softmax-weighted variance of the logit change rates), App. A.2 (alpha).
//
// All reductions are fixed-order trees (no atomics), so results are
// bit-reproducible.  RowAdam reduces in fp64; q accumulates per thread in
// fp32 and combines partial results in fp64.
#include "device_common.h"
#include "kernels.h"

#include <atomic>
#include <cmath>
#include <vector>

namespace logra {

namespace {

// ------------------------------------------------------------- RowAdam

constexpr int kRowsPerBlock = 16;

struct RowAdamWs {
  double* m;        // [d] row energy sum_j S_ij^2
  double* vh;       // [d] bias-corrected second moment
  double* partial;  // [2 * nblocks]: per block (sum m, sum vh)
  double* scalars;  // [4]: eps*rho, norm ratio, -, -
};

// One sketch of a grouped RowAdam (device table; entry n holds only the
// totals rb_begin and ap_begin).
struct RowAdamEntry {
  const float* S;
  float* v;
  uint16_t* P;
  int64_t d, rb_begin, ap_begin;
  RowAdamWs ws;
};

__device__ __forceinline__ double wave_sum(double x) {
  // Butterfly over the 64 lanes (fixed pattern, every lane gets the total).
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// One block's 16 rows (block index blk of the matrix): energies, the
// second-moment update, and the block's partial sums.
__device__ __forceinline__ void rowadam_rows_block(int64_t blk, int64_t d, int64_t r,
                                                   const float* __restrict__ S,
                                                   float* __restrict__ v, double beta,
                                                   double bias_corr, const RowAdamWs& ws) {
  __shared__ double sm[kRowsPerBlock], svh[kRowsPerBlock];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t base = blk * kRowsPerBlock;
  for (int q = wave; q < kRowsPerBlock; q += 4) {
    const int64_t i = base + q;
    double m = 0.0, vh = 0.0;
    if (i < d) {
      double acc = 0.0;
      for (int64_t j = lane; j < r; j += 64) {
        const double x = (double)S[i * r + j];
        acc += x * x;
      }
      m = wave_sum(acc);
      const double vn = beta * (double)v[i] + (1.0 - beta) * m;
      vh = vn / bias_corr;
      if (lane == 0) {
        v[i] = (float)vn;
        ws.m[i] = m;
        ws.vh[i] = vh;
      }
    }
    if (lane == 0) {
      sm[q] = m;
      svh[q] = vh;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, b = 0.0;
    for (int q = 0; q < kRowsPerBlock; ++q) {
      a += sm[q];
      b += svh[q];
    }
    ws.partial[2 * blk] = a;
    ws.partial[2 * blk + 1] = b;
  }
}

__global__ __launch_bounds__(256) void rowadam_rows_kernel(int64_t d, int64_t r,
                                                           const float* __restrict__ S,
                                                           float* __restrict__ v, double beta,
                                                           double bias_corr, RowAdamWs ws) {
  rowadam_rows_block(blockIdx.x, d, r, S, v, beta, bias_corr, ws);
}

// Sum of one value per thread over the block's 256 threads: a fixed tree,
// every thread gets the total.
__device__ double block_sum256(double x, double* red) {
  __syncthreads();  // red may still be read by an earlier call
  red[threadIdx.x] = x;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  return red[0];
}

// One block: rho, then ||Ut||_F^2 = sum_i m_i / (sqrt(vh_i) + eps rho)^2 and
// the norm-restoring ratio ||S||_F / ||Ut||_F.
__device__ __forceinline__ void rowadam_norm_block(int64_t d, int64_t nblocks, double eps,
                                                   const RowAdamWs& ws) {
  __shared__ double red[256];
  // Per-block partial sums, thread t taking blocks t, t + 256, ...
  double a = 0.0, b = 0.0;
  for (int64_t q = threadIdx.x; q < nblocks; q += 256) {
    a += ws.partial[2 * q];
    b += ws.partial[2 * q + 1];
  }
  const double sum_m = block_sum256(a, red);   // ||S||_F^2
  const double sum_vh = block_sum256(b, red);  // sum vh
  const double erho = eps * sqrt(sum_vh / (double)d);
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256) {
    const double den = sqrt(ws.vh[i]) + erho;
    if (den > 0.0) acc += ws.m[i] / (den * den);
  }
  const double nu2 = block_sum256(acc, red);
  if (threadIdx.x == 0) {
    ws.scalars[0] = erho;
    ws.scalars[1] = nu2 > 0.0 ? sqrt(sum_m / nu2) : 0.0;
  }
}

__global__ __launch_bounds__(256) void rowadam_norm_kernel(int64_t d, int64_t nblocks,
                                                           double eps, RowAdamWs ws) {
  rowadam_norm_block(d, nblocks, eps, ws);
}

// Scaling pass: U = S * ratio / (sqrt(vh_i) + eps rho), row by row.
__global__ __launch_bounds__(256) void rowadam_apply_kernel(int64_t d, int64_t r,
                                                            const float* S, float* U,
                                                            RowAdamWs ws) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= d * r) return;
  const int64_t i = idx / r;
  const double den = sqrt(ws.vh[i]) + ws.scalars[0];
  const double f = den > 0.0 ? ws.scalars[1] / den : 0.0;
  U[idx] = (float)((double)S[idx] * f);
}

// The scaling pass writing the merge's packed update instead of fp32 U (the
// same fp32 values, split into bf16 hi and lo terms in operand order): one
// thread per (32-row band, 16-rank step, lane).
__device__ __forceinline__ void rowadam_apply_packed_thread(int64_t t, int64_t d, int64_t r, int ks,
                                                            const float* S, uint16_t* P,
                                                            const RowAdamWs& ws) {
  const int lane = (int)(t & 63);
  const int64_t bs = t >> 6;
  const int64_t nb = (d + 31) / 32;
  if (bs >= nb * ks) return;
  const int64_t band = bs / ks;
  const int s = (int)(bs - band * ks);
  const int64_t i = band * 32 + (lane & 31);
  const int64_t j0 = 16 * s + 8 * (lane >> 5);
  double f = 0.0;
  if (i < d) {
    const double den = sqrt(ws.vh[i]) + ws.scalars[0];
    f = den > 0.0 ? ws.scalars[1] / den : 0.0;
  }
  float x[8];
  if (i < d && j0 + 8 <= r && (r & 3) == 0) {
    // the row's eight values as two 16-byte loads (rows of S are 16-byte
    // aligned when r is a multiple of 4); S is read once here
    typedef __attribute__((address_space(1))) const f32x4 gf4;
    const gf4* ps = (const gf4*)(S + i * r + j0);
    const f32x4 a = __builtin_nontemporal_load(ps), b = __builtin_nontemporal_load(ps + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[q] = (float)((double)a[q] * f);
      x[4 + q] = (float)((double)b[q] * f);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      x[q] = (i < d && j0 + q < r) ? (float)((double)S[i * r + j0 + q] * f) : 0.f;
  }
  uint32_t hv[4], lv[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const __bf16 h0 = (__bf16)x[2 * p], h1 = (__bf16)x[2 * p + 1];
    const __bf16 l0 = (__bf16)(x[2 * p] - (float)h0), l1 = (__bf16)(x[2 * p + 1] - (float)h1);
    hv[p] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
            ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    lv[p] = (uint32_t)__builtin_bit_cast(uint16_t, l0) |
            ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  }
  // one 16-byte store per term, non-temporal: the merge reads them in a later launch
  u32x4* dst = reinterpret_cast<u32x4*>(P + bs * 1024 + lane * 8);
  __builtin_nontemporal_store(u32x4{hv[0], hv[1], hv[2], hv[3]}, dst);
  __builtin_nontemporal_store(u32x4{lv[0], lv[1], lv[2], lv[3]}, dst + 64);
}

__global__ __launch_bounds__(256) void rowadam_apply_packed_kernel(int64_t d, int64_t r, int ks,
                                                                   const float* S,
                                                                   uint16_t* P, RowAdamWs ws) {
  rowadam_apply_packed_thread((int64_t)blockIdx.x * 256 + threadIdx.x, d, r, ks, S, P, ws);
}

// Grouped RowAdam over many sketches (device table): entry e's row blocks are
// blocks [rb_begin, rb_begin of e + 1) of the rows launch, its norm is block
// e of the norm launch, and its (band, step) units of the packed scaling pass
// are [ap_begin, ap_begin of e + 1).  Each sketch's arithmetic is that of
// the single call, so the results are bit-identical.
__device__ __forceinline__ int rowadam_entry(const RowAdamEntry* __restrict__ tab, int n,
                                             int64_t x, bool by_rows) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((by_rows ? tab[mid].rb_begin : tab[mid].ap_begin) <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void rowadam_rows_grouped_kernel(const RowAdamEntry* __restrict__ tab,
                                                                   int n, int64_t r, double beta,
                                                                   double bias_corr) {
  const int e = rowadam_entry(tab, n, blockIdx.x, true);
  const RowAdamEntry& t = tab[e];
  rowadam_rows_block((int64_t)blockIdx.x - t.rb_begin, t.d, r, t.S, t.v, beta, bias_corr, t.ws);
}

__global__ __launch_bounds__(256) void rowadam_norm_grouped_kernel(const RowAdamEntry* __restrict__ tab,
                                                                   double eps) {
  const RowAdamEntry& t = tab[blockIdx.x];
  rowadam_norm_block(t.d, (t.d + kRowsPerBlock - 1) / kRowsPerBlock, eps, t.ws);
}

__global__ __launch_bounds__(256) void rowadam_apply_packed_grouped_kernel(
    const RowAdamEntry* __restrict__ tab, int n, int64_t total, int64_t r, int ks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t unit = t >> 6;
  if (unit >= total) return;
  const int e = rowadam_entry(tab, n, unit, false);
  const RowAdamEntry& x = tab[e];
  rowadam_apply_packed_thread(t - x.ap_begin * 64, x.d, r, ks, x.S, x.P, x.ws);
}

// -------------------------------------------------------- predicted KL q

// Softmax-weighted moments of zdot over part of one context, relative to
// the part's largest logit m = max z/tau: w = sum exp(l - m), the weighted
// mean of zdot - c, and M2 = sum exp(l - m) (zdot - c - mean)^2, with c a
// zdot value of the part (each thread's first).  They are updated one value
// at a time (Welford) and merged pairwise (Chan, Golub and LeVeque), so the
// variance never comes from a difference of large sums, and the shift keeps
// an offset common to the context out of the fp32 means: neither a common
// offset of zdot nor a few outlying entries cost precision.
struct Moments {
  float m, w, mean, M2, c;
};

__device__ __forceinline__ Moments combine(Moments a, Moments b) {
  if (b.w == 0.f && b.m == -INFINITY) return a;
  if (a.w == 0.f && a.m == -INFINITY) return b;
  const float m = fmaxf(a.m, b.m);
  const float fa = __expf(a.m - m), fb = __expf(b.m - m);
  const float wa = a.w * fa, wb = b.w * fb;
  const float w = wa + wb;  // >= 1: the part holding the larger maximum has weight >= 1
  const float delta = (b.mean - a.mean) + (b.c - a.c);
  return Moments{m, w, a.mean + delta * (wb / w),
                 a.M2 * fa + b.M2 * fb + delta * delta * (wa * (wb / w)), a.c};
}

constexpr int kKlqThreads = 256;
constexpr int kKlqChunks = 16;  // chunks of V per context

template <bool BF16>
__device__ __forceinline__ float load_val(const void* p, int64_t i) {
  if (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

template <bool BF16>
__global__ __launch_bounds__(kKlqThreads) void klq_partial_kernel(int64_t V, const void* z,
                                                                  const void* zd, float inv_tau,
                                                                  double* __restrict__ part) {
  __shared__ Moments red[kKlqThreads];
  const int64_t s = blockIdx.y;
  const int64_t chunk = (V + kKlqChunks - 1) / kKlqChunks;
  const int64_t lo = blockIdx.x * chunk;
  const int64_t hi = lo + chunk < V ? lo + chunk : V;
  const int64_t row = s * V;
  const int64_t first = lo + (int64_t)threadIdx.x * 8;
  const float c = first < hi ? load_val<BF16>(zd, row + first) : 0.f;
  Moments mo{-INFINITY, 0.f, 0.f, 0.f, c};
  for (int64_t v0 = lo + (int64_t)threadIdx.x * 8; v0 < hi; v0 += (int64_t)kKlqThreads * 8) {
    float l[8], y[8];
    float gm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = v0 + e < hi;
      l[e] = ok ? load_val<BF16>(z, row + v0 + e) * inv_tau : -INFINITY;
      y[e] = ok ? load_val<BF16>(zd, row + v0 + e) - c : 0.f;
      gm = fmaxf(gm, l[e]);
    }
    // Eight masked entries (logit -inf, weight 0) add nothing; skipped, they
    // cannot turn into exp(-inf - (-inf)) = NaN before the first finite one.
    if (gm == -INFINITY) continue;
    if (gm > mo.m) {
      const float f = __expf(mo.m - gm);  // the mean is unchanged by a common factor
      mo.w *= f;
      mo.M2 *= f;
      mo.m = gm;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __expf(l[e] - mo.m);
      if (p > 0.f) {  // masked entries (and weights below the fp32 range) add nothing
        const float w = mo.w + p;
        const float dy = y[e] - mo.mean;
        mo.mean += dy * (p / w);
        mo.M2 += p * dy * (y[e] - mo.mean);
        mo.w = w;
      }
    }
  }
  red[threadIdx.x] = mo;
  __syncthreads();
  for (int w = kKlqThreads / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = combine(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double* o = part + (s * kKlqChunks + blockIdx.x) * 4;
    o[0] = red[0].m;
    o[1] = red[0].w;
    o[2] = (double)red[0].mean + (double)red[0].c;  // the mean of zdot itself
    o[3] = red[0].M2;
  }
}

// Combine the chunk partials of each context in order (fp64), form the
// centred variance, and sum over contexts in a fixed tree.
__global__ __launch_bounds__(256) void klq_final_kernel(int64_t P, const double* __restrict__ part,
                                                        double scale, float* __restrict__ q) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int64_t s = threadIdx.x; s < P; s += 256) {
    // The chunks' moments merged in order, as in combine() but in fp64.
    double m = -INFINITY, w = 0.0, mean = 0.0, M2 = 0.0;
    for (int c = 0; c < kKlqChunks; ++c) {
      const double* o = part + (s * kKlqChunks + c) * 4;
      if (o[1] == 0.0 && o[0] == -INFINITY) continue;
      const double mm = o[0] > m ? o[0] : m;
      const double fa = exp(m - mm), fb = exp(o[0] - mm);
      const double wa = w * fa, wb = o[1] * fb;
      const double wn = wa + wb;
      const double delta = o[2] - mean;
      mean += delta * (wb / wn);
      M2 = M2 * fa + o[3] * fb + delta * delta * (wa * (wb / wn));
      w = wn;
      m = mm;
    }
    acc += M2 / w;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) q[0] = (float)(red[0] * scale);
}

__global__ void step_alpha_kernel(const float* q, float delta, float amax, float* alpha) {
  const float qq = *q;
  float a;
  if (!(qq >= 0.f)) a = __int_as_float(0x7FC00000);
  else if (qq == 0.f) a = amax;
  else a = fminf(amax, sqrtf(delta / qq));
  *alpha = a;
}

// -------------------------------------------------- exact KL of a step

// Per context s (one block): KL(p || p') with p = softmax(z/tau) and p' =
// softmax((z + alpha zdot)/tau), logits linear in alpha.  With c = alpha/tau
// and mu = E_p[zdot], KL = log E_p[exp(c (zdot - mu))] (the normalisers and
// the linear term cancel), evaluated as log1p(E_p[expm1(c (zdot - mu))]) so
// that a small step keeps its digits.  Three passes over the row in fp64:
// max of z/tau, then the weights' sum and first moment, then the expm1
// moment; fixed-tree block sums.
__device__ double kl_block_sum(double x, double* red) {
  __syncthreads();
  red[threadIdx.x] = x;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  return red[0];
}
__device__ double kl_block_max(double x, double* red) {
  __syncthreads();
  red[threadIdx.x] = x;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  return red[0];
}

template <bool BF16>
__global__ __launch_bounds__(256) void exact_kl_rows_kernel(int64_t V, const void* z, const void* zd,
                                                            double inv_tau, double c,
                                                            double* __restrict__ kl) {
  __shared__ double red[256];
  const int64_t row = (int64_t)blockIdx.x * V;
  double m = -INFINITY;
  for (int64_t v = threadIdx.x; v < V; v += 256) m = fmax(m, (double)load_val<BF16>(z, row + v) * inv_tau);
  m = kl_block_max(m, red);
  double w = 0.0, wy = 0.0;
  for (int64_t v = threadIdx.x; v < V; v += 256) {
    const double e = exp((double)load_val<BF16>(z, row + v) * inv_tau - m);
    w += e;
    wy += e * (double)load_val<BF16>(zd, row + v);
  }
  const double W = kl_block_sum(w, red);
  const double mu = kl_block_sum(wy, red) / W;
  double g = 0.0;
  for (int64_t v = threadIdx.x; v < V; v += 256) {
    const double e = exp((double)load_val<BF16>(z, row + v) * inv_tau - m);
    g += e * expm1(c * ((double)load_val<BF16>(zd, row + v) - mu));
  }
  const double G = kl_block_sum(g, red);
  if (threadIdx.x == 0) kl[blockIdx.x] = log1p(G / W);
}

// Mean over contexts in a fixed tree.
__global__ __launch_bounds__(256) void exact_kl_mean_kernel(int64_t P, const double* __restrict__ kl,
                                                            double* __restrict__ out) {
  __shared__ double red[256];
  double a = 0.0;
  for (int64_t i = threadIdx.x; i < P; i += 256) a += kl[i];
  const double t = kl_block_sum(a, red);
  if (threadIdx.x == 0) *out = t / (double)P;
}

RowAdamWs rowadam_ws_layout(void* ws, int64_t d) {
  const int64_t nb = (d + kRowsPerBlock - 1) / kRowsPerBlock;
  double* p = static_cast<double*>(ws);
  RowAdamWs w;
  w.m = p;
  w.vh = p + d;
  w.partial = p + 2 * d;
  w.scalars = p + 2 * d + 2 * nb;
  return w;
}

}  // namespace

size_t rowadam_ws_bytes(int64_t d) {
  const int64_t nb = (d + kRowsPerBlock - 1) / kRowsPerBlock;
  return (size_t)(2 * d + 2 * nb + 4) * sizeof(double);
}

hipError_t launch_rowadam(int64_t d, int64_t r, const float* S, float* v, int64_t t,
                          double beta, double eps, float* U, void* U_packed, void* ws,
                          hipStream_t s) {
  const RowAdamWs w = rowadam_ws_layout(ws, d);
  const int64_t nb = (d + kRowsPerBlock - 1) / kRowsPerBlock;
  const double b = beta;
  const double bias = 1.0 - std::pow(b, (double)t);
  hipLaunchKernelGGL(rowadam_rows_kernel, dim3((unsigned)nb), dim3(256), 0, s, d, r, S, v, b,
                     bias, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rowadam_norm_kernel, dim3(1), dim3(256), 0, s, d, nb, eps, w);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (U != nullptr) {
    const int64_t n = d * r;
    hipLaunchKernelGGL(rowadam_apply_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       d, r, S, U, w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (U_packed != nullptr) {
    const int ks = merge_rank_steps(r);
    const int64_t threads = (d + 31) / 32 * ks * 64;
    hipLaunchKernelGGL(rowadam_apply_packed_kernel, dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, d, r, ks, S, static_cast<uint16_t*>(U_packed), w);
    e = hipGetLastError();
  }
  return e;
}

size_t rowadam_grouped_ws_bytes(int n, int64_t total_rows) {
  // the table, then per sketch its m, vh, partial sums and scalars (at most
  // total_rows / 16 + n row blocks in all)
  const size_t tab = ((size_t)(n + 1) * sizeof(RowAdamEntry) + 255) / 256 * 256;
  const int64_t nb = total_rows / kRowsPerBlock + n;
  return tab + (size_t)(2 * total_rows + 2 * nb + 4 * n) * sizeof(double);
}

hipError_t launch_rowadam_packed_grouped(const RowAdamItem* items, int n, int64_t r, int64_t t,
                                         double beta, double eps, void* ws, hipStream_t s) {
  if (n < 1) return hipErrorInvalidValue;
  std::vector<RowAdamEntry> tab((size_t)n + 1, RowAdamEntry{});
  const size_t tab_bytes = ((size_t)(n + 1) * sizeof(RowAdamEntry) + 255) / 256 * 256;
  double* area = reinterpret_cast<double*>(static_cast<char*>(ws) + tab_bytes);
  const int ks = merge_rank_steps(r);
  int64_t rb = 0, ap = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t d = items[i].d;
    const int64_t nb = (d + kRowsPerBlock - 1) / kRowsPerBlock;
    RowAdamEntry& e = tab[i];
    e.S = items[i].S;
    e.v = items[i].v;
    e.P = static_cast<uint16_t*>(items[i].P);
    e.d = d;
    e.rb_begin = rb;
    e.ap_begin = ap;
    e.ws = rowadam_ws_layout(area, d);
    area += 2 * d + 2 * nb + 4;
    rb += nb;
    ap += (d + 31) / 32 * ks;
  }
  tab[n].rb_begin = rb;
  tab[n].ap_begin = ap;
  // From pageable memory the copy is staged before the call returns.
  hipError_t e = hipMemcpyAsync(ws, tab.data(), tab.size() * sizeof(RowAdamEntry),
                                hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  const RowAdamEntry* dtab = static_cast<const RowAdamEntry*>(ws);
  const double bias = 1.0 - std::pow(beta, (double)t);
  hipLaunchKernelGGL(rowadam_rows_grouped_kernel, dim3((unsigned)rb), dim3(256), 0, s, dtab, n, r,
                     beta, bias);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(rowadam_norm_grouped_kernel, dim3((unsigned)n), dim3(256), 0, s, dtab, eps);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(rowadam_apply_packed_grouped_kernel, dim3((unsigned)((ap * 64 + 255) / 256)),
                     dim3(256), 0, s, dtab, n, ap, r, ks);
  return hipGetLastError();
}

size_t klq_ws_bytes(int64_t P, int64_t V) {
  (void)V;
  return (size_t)(P * kKlqChunks * 4) * sizeof(double);
}

hipError_t launch_predicted_kl_q(int64_t P, int64_t V, const void* z, const void* zd,
                                 bool bf16, float tau, float* q, void* ws, hipStream_t s) {
  double* part = static_cast<double*>(ws);
  const dim3 grid(kKlqChunks, (unsigned)P);
  const float inv_tau = (float)(1.0 / (double)tau);
  if (bf16)
    hipLaunchKernelGGL(klq_partial_kernel<true>, grid, dim3(kKlqThreads), 0, s, V, z, zd,
                       inv_tau, part);
  else
    hipLaunchKernelGGL(klq_partial_kernel<false>, grid, dim3(kKlqThreads), 0, s, V, z, zd,
                       inv_tau, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const double scale = 1.0 / (2.0 * (double)P * (double)tau * (double)tau);
  hipLaunchKernelGGL(klq_final_kernel, dim3(1), dim3(256), 0, s, P, part, scale, q);
  return hipGetLastError();
}

// Scratch of the allocation-free q: the per-chunk partial moments of up to
// kNoAllocMaxContexts contexts.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` is only a stand-in for
// the symbol: the device address comes from hipGetSymbolAddress, per device.
constexpr int64_t kNoAllocMaxContexts = 4096;
static __device__ __align__(256) double scratch[kNoAllocMaxContexts * kKlqChunks * 4];

int64_t noalloc_max_contexts() { return kNoAllocMaxContexts; }

// The current device's address of `scratch`, looked up once per device (a
// concurrent first call on the same device looks it up too and stores the
// same address).
static hipError_t scratch_address(void** out) {
  static std::atomic<void*> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_predicted_kl_q_noalloc(int64_t P, int64_t V, const void* z, const void* zd,
                                         bool bf16, float tau, float* q, hipStream_t s) {
  if (P < 1 || P > kNoAllocMaxContexts) return hipErrorInvalidValue;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  // Every partial the final pass reads is written by this call's first pass
  // (P x kKlqChunks entries), so nothing needs clearing.
  return launch_predicted_kl_q(P, V, z, zd, bf16, tau, q, ws, s);
}

size_t exact_kl_ws_bytes(int64_t P) { return (size_t)P * sizeof(double); }

hipError_t launch_exact_kl(int64_t P, int64_t V, const void* z, const void* zd, bool bf16,
                           double alpha, double tau, double* out, void* ws, hipStream_t s) {
  double* kl = static_cast<double*>(ws);
  const double inv_tau = 1.0 / tau;
  const double c = alpha / tau;
  if (bf16)
    hipLaunchKernelGGL(exact_kl_rows_kernel<true>, dim3((unsigned)P), dim3(256), 0, s, V, z, zd,
                       inv_tau, c, kl);
  else
    hipLaunchKernelGGL(exact_kl_rows_kernel<false>, dim3((unsigned)P), dim3(256), 0, s, V, z, zd,
                       inv_tau, c, kl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(exact_kl_mean_kernel, dim3(1), dim3(256), 0, s, P, kl, out);
  return hipGetLastError();
}

hipError_t launch_step_alpha(const float* q, float delta, float amax, float* alpha,
                             hipStream_t s) {
  hipLaunchKernelGGL(step_alpha_kernel, dim3(1), dim3(1), 0, s, q, delta, amax, alpha);
  return hipGetLastError();
}

}  // namespace logra
