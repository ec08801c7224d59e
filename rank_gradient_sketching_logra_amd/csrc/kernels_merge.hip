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
// bf16 W runs on v_mfma_f32_16x16x32_bf16 with the product transposed: for
// a 16-row band of W, instance e of a wave computes C[m][n] = sum over ranks
// of sigma[rank][col(m, e)] * U[row n][rank], with U split into bf16 hi + lo
// (two MFMAs per rank step) and sigma exact in bf16.  Lane l holds
// C[m = 4(l>>4) + i][n = l & 15], and the columns are assigned so that lane
// l owns 16 consecutive columns of one W row per 64-column group: W is read,
// updated and written straight from registers with 16-byte accesses, and the
// 16 stochastic-rounding draws of those elements come from one Philox block
// when k is a multiple of 16.  Every element's sum runs over rank steps in
// ascending order, hi then lo, whatever the row or block position, so a merge
// of a row block equals the same rows of a whole-matrix merge.
#include "device_common.h"
#include "kernels.h"

namespace logra {

namespace {

constexpr int kMergeBand = 16;  // rows per band: one MFMA n-block

__device__ __forceinline__ uint64_t pick_word_m(const Philox4& p, int i) {
  const uint64_t a = (i & 1) ? p.w[1] : p.w[0];
  const uint64_t b = (i & 1) ? p.w[3] : p.w[2];
  return (i & 2) ? b : a;
}

__device__ __forceinline__ uint32_t sr_draw(const Philox4& p, uint64_t e) {
  return (uint32_t)(pick_word_m(p, (int)((e & 15) >> 2)) >> (16 * (e & 3))) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// Eight consecutive fp32 of U row `row` from rank j0, split into bf16 hi/lo
// B operands; zero for rows >= d or ranks >= r.
__device__ __forceinline__ void load_u8(const float* __restrict__ U, int64_t d, int64_t r,
                                        int64_t row, int64_t j0, bool r_vec, u32x4& hi,
                                        u32x4& lo) {
  float x[8];
  if (row < d && r_vec && j0 + 8 <= r) {
    const f32x4* p = reinterpret_cast<const f32x4*>(U + row * r + j0);
    const f32x4 x0 = p[0], x1 = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = x0[e];
      x[4 + e] = x1[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (row < d && j0 + e < r) ? U[row * r + j0 + e] : 0.f;
  }
  float h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (float)(__bf16)x[e];
    l[e] = x[e] - h[e];
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    hi[p] = bf16_pair(h[2 * p], h[2 * p + 1]);
    lo[p] = bf16_pair(l[2 * p], l[2 * p + 1]);
  }
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

// A block = 4 waves x NG 64-column groups: columns [cb * 256 NG, +256 NG),
// row bands [band_begin, band_end) shared by the four waves.  KS = 32-rank
// steps.  The signs of A for the block's columns are generated once into LDS
// as bits; each wave expands its A operands into registers, then streams its
// bands: U band as B operands, W straight into registers, 2 KS MFMAs per
// instance, update, round, store -- with the next band's loads in flight
// when PREFETCH.
template <int KS, int NG, bool PREFETCH>
__global__ __launch_bounds__(256, KS >= 8 ? 1 : 2) void merge_bf16_kernel(
    KeyArg key, int64_t d, int64_t k, int64_t r, uint16_t* __restrict__ W, int64_t ldw,
    const float* __restrict__ U, float scale_cr, const float* __restrict__ scale_dev,
    int stochastic, KeyArg sr_key, int64_t row0, int64_t ncb, int64_t bands_per_block) {
  constexpr int BC = 256 * NG;  // columns per block
  constexpr int NW = BC / 32;   // sign words per rank
  constexpr int NI = 4 * NG;    // MFMA instances per wave and band
  __shared__ uint32_t sbits[KS * 32 * NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t cb = blockIdx.x % ncb;
  const int64_t bg = blockIdx.x / ncb;
  const int64_t cblk = cb * BC;
  const int64_t nbands = (d + kMergeBand - 1) / kMergeBand;
  const int64_t band_begin = bg * bands_per_block;
  const int64_t band_end =
      band_begin + bands_per_block < nbands ? band_begin + bands_per_block : nbands;
  if (band_begin >= band_end) return;

  // Sign bits of ranks [0, 32 KS) for the block's columns: word w of rank j
  // holds columns cblk + 32w + (0..31), bit set meaning -1.
  {
    const KeyWords kw{key.k0, key.k1};
    for (int task = tid; task < KS * 32 * NG; task += 256) {
      const int j = task / NG;
      const int pb = task - j * NG;
      const int64_t cbase = cblk + 256 * pb;
      uint32_t* dst = &sbits[j * NW + 8 * pb];
      if (j < r && cbase < k) {
        const Philox4 p = sigma_block(kw, (uint64_t)j, (uint64_t)(cbase >> 8));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          dst[2 * w] = (uint32_t)p.w[w];
          dst[2 * w + 1] = (uint32_t)(p.w[w] >> 32);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 8; ++w) dst[w] = 0u;
      }
    }
  }
  __syncthreads();

  // A operands: instance e = 4G + jj holds, for MFMA row m = l & 15, column
  // 64(NG wave + G) + 16(m >> 2) + 4jj + (m & 3) of the block and ranks
  // 32s + 8(l >> 4) + i, i = 0..7.  Ranks >= r read as +1; their U terms
  // are zero.
  const int m = lane & 15;
  const int kg = lane >> 4;
  u32x4 afrag[NI][KS];
#pragma unroll
  for (int e = 0; e < NI; ++e) {
    const int G = e >> 2, jj = e & 3;
    const int cl = 64 * (NG * wave + G) + 16 * (m >> 2) + 4 * jj + (m & 3);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint32_t byte = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        byte |= ((sbits[(32 * s + 8 * kg + i) * NW + (cl >> 5)] >> (cl & 31)) & 1u) << i;
      afrag[e][s] = u32x4{
          0x3F803F80u | ((byte << 15) & 0x8000u) | ((byte << 30) & 0x80000000u),
          0x3F803F80u | ((byte << 13) & 0x8000u) | ((byte << 28) & 0x80000000u),
          0x3F803F80u | ((byte << 11) & 0x8000u) | ((byte << 26) & 0x80000000u),
          0x3F803F80u | ((byte << 9) & 0x8000u) | ((byte << 24) & 0x80000000u)};
    }
  }

  float sc = scale_cr;
  if (scale_dev != nullptr) sc *= *scale_dev;
  const KeyWords srk{sr_key.k0, sr_key.k1};
  const bool r_vec = (r & 3) == 0;
  const int n = lane & 15;  // W row within the band (B and C layouts)
  const int q = lane >> 4;  // 16-column slot within a 64-column group
  const int64_t cwave = cblk + 64 * NG * wave;

  u32x4 wv[NG][2], uh[KS], ul[KS];
  u32x4 wn[NG][2], nh[KS], nl[KS];
  auto load_band = [&](int64_t band, u32x4(&w)[NG][2], u32x4(&h)[KS], u32x4(&l)[KS]) {
    const int64_t row = band * kMergeBand + n;
#pragma unroll
    for (int s = 0; s < KS; ++s) load_u8(U, d, r, row, 32 * s + 8 * kg, r_vec, h[s], l[s]);
#pragma unroll
    for (int G = 0; G < NG; ++G)
      load_w16(W, ldw, d, k, row, cwave + 64 * G + 16 * q, w[G][0], w[G][1]);
  };

  load_band(band_begin, wv, uh, ul);
  for (int64_t band = band_begin; band < band_end; ++band) {
    const bool more = band + 1 < band_end;
    if (PREFETCH && more) load_band(band + 1, wn, nh, nl);
    const int64_t row = band * kMergeBand + n;
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      f32x4 acc[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(afrag[4 * G + jj][s]), as_bf16x8(uh[s]), acc[jj], 0, 0, 0);
          acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(afrag[4 * G + jj][s]), as_bf16x8(ul[s]), acc[jj], 0, 0, 0);
        }
      }
      const int64_t c = cwave + 64 * G + 16 * q;
      if (row >= d || c >= k) continue;
      // Element t of the lane's 16 columns is C[m = 4q + (t & 3)] of
      // instance jj = t >> 2: acc[t >> 2][t & 3].
      const uint64_t e0 = (uint64_t)(row0 + row) * (uint64_t)k + (uint64_t)c;
      Philox4 p0, p1;
      if (stochastic) {
        p0 = sr_block(srk, e0 >> 4);
        p1 = (((e0 + 15) >> 4) != (e0 >> 4)) ? sr_block(srk, (e0 + 15) >> 4) : p0;
      }
      uint32_t out[8];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint32_t word = wv[G][t >> 3][(t & 7) >> 1];
        const uint32_t wbits = (t & 1) ? (word >> 16) : (word & 0xFFFFu);
        const float x = __builtin_fmaf(-sc, acc[t >> 2][t & 3], bf16_bits_to_f32(wbits));
        uint32_t o;
        if (stochastic) {
          const uint64_t ee = e0 + t;
          const uint32_t u = ((ee >> 4) == (e0 >> 4)) ? sr_draw(p0, ee) : sr_draw(p1, ee);
          o = f32_to_bf16_sr(x, u);
        } else {
          o = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
        }
        if (t & 1)
          out[t >> 1] |= o << 16;
        else
          out[t >> 1] = o;
      }
      if (c + 16 <= k) {
        u32x4* dst = reinterpret_cast<u32x4*>(W + row * ldw + c);
        dst[0] = u32x4{out[0], out[1], out[2], out[3]};
        dst[1] = u32x4{out[4], out[5], out[6], out[7]};
      } else {
        for (int t = 0; t < 16 && c + t < k; ++t)
          W[row * ldw + c + t] = (uint16_t)((out[t >> 1] >> (16 * (t & 1))) & 0xFFFFu);
      }
    }
    if (more) {
      if (PREFETCH) {
#pragma unroll
        for (int G = 0; G < NG; ++G) {
          wv[G][0] = wn[G][0];
          wv[G][1] = wn[G][1];
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          uh[s] = nh[s];
          ul[s] = nl[s];
        }
      } else {
        load_band(band + 1, wv, uh, ul);
      }
    }
  }
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

hipError_t launch_merge(KeyArg key, int64_t d, int64_t k, int64_t r, void* W, bool bf16,
                        int64_t ldw, const float* U, double scale, const float* scale_dev,
                        bool stochastic, KeyArg sr_key, int64_t row0, hipStream_t s) {
  const double cr = 1.0 / std::sqrt((double)r);
  if (!bf16) {
    const dim3 grid((unsigned)((k + 255) / 256), (unsigned)((d + 15) / 16));
    hipLaunchKernelGGL(merge_f32_kernel, grid, dim3(256), 0, s, key, d, k, r,
                       static_cast<float*>(W), ldw, U, scale * cr, scale_dev);
    return hipGetLastError();
  }
  const int64_t ksteps = (r + 31) / 32;
  const int ks = ksteps <= 1 ? 1 : ksteps <= 2 ? 2 : ksteps <= 4 ? 4 : 8;
  const int ng = ks <= 2 ? 2 : 1;
  const int64_t bc = 256 * ng;
  const int64_t ncb = (k + bc - 1) / bc;
  const int64_t nbands = (d + kMergeBand - 1) / kMergeBand;
  // Enough blocks to fill the chip several times over, each with a few bands
  // to amortise the sign setup.
  int64_t per = (nbands * ncb + 2047) / 2048;
  if (per < 4) per = 4;
  if (per > nbands) per = nbands;
  const int64_t groups = (nbands + per - 1) / per;
  const dim3 grid((unsigned)(ncb * groups));
  uint16_t* Wb = static_cast<uint16_t*>(W);
  const float scf = (float)(scale * cr);
  const int st = stochastic ? 1 : 0;
#define LOGRA_MERGE_LAUNCH(KS, NG, PF)                                                      \
  hipLaunchKernelGGL((merge_bf16_kernel<KS, NG, PF>), grid, dim3(256), 0, s, key, d, k, r, \
                     Wb, ldw, U, scf, scale_dev, st, sr_key, row0, ncb, per)
  switch (ks) {
    case 1: LOGRA_MERGE_LAUNCH(1, 2, true); break;
    case 2: LOGRA_MERGE_LAUNCH(2, 2, true); break;
    case 4: LOGRA_MERGE_LAUNCH(4, 1, true); break;
    case 8: LOGRA_MERGE_LAUNCH(8, 1, false); break;
    default: return hipErrorInvalidValue;
  }
#undef LOGRA_MERGE_LAUNCH
  return hipGetLastError();
}

}  // namespace logra
