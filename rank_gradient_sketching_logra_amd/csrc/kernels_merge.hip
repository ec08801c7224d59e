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
// bf16 W: a block owns one column block of NK columns and a range of 64-row
// tiles.  It regenerates the signs of A for its columns once, into LDS as
// bf16 +-1 (column-major, so one 16-byte read is one MFMA B operand), then
// per row tile computes the U*sigma tile on v_mfma_f32_32x32x16_bf16 with U
// split into bf16 hi + lo, stages the scaled tile in LDS and streams W with
// coalesced 16-byte accesses, 16 consecutive elements per thread (one
// Philox block of stochastic-rounding draws when k is a multiple of 16).
#include "device_common.h"
#include "kernels.h"

namespace logra {

namespace {

constexpr int kMergeRows = 64;  // rows per tile (two 32-row MFMA blocks)

__device__ __forceinline__ uint64_t pick_word_m(const Philox4& p, int i) {
  const uint64_t a = (i & 1) ? p.w[1] : p.w[0];
  const uint64_t b = (i & 1) ? p.w[3] : p.w[2];
  return (i & 2) ? b : a;
}

__device__ __forceinline__ uint32_t sr_draw(const Philox4& p, uint64_t e) {
  return (uint32_t)(pick_word_m(p, (int)((e & 15) >> 2)) >> (16 * (e & 3))) & 0xFFFFu;
}

// NKB = 32-column blocks per column block (NK = 32 * NKB); KS = RP / 16
// rank steps of the MFMA.
template <int NKB, int KS>
__global__ __launch_bounds__(256) void merge_bf16_kernel(
    KeyArg key, int64_t d, int64_t k, int64_t r, uint16_t* __restrict__ W, int64_t ldw,
    const float* __restrict__ U, float scale_cr, const float* __restrict__ scale_dev,
    int stochastic, KeyArg sr_key, int64_t row0, int64_t ncb, int64_t tiles_per_block) {
  constexpr int NK = 32 * NKB;
  constexpr int RP = 16 * KS;
  constexpr int SPITCH = RP + 8;           // bf16 per LDS column of sigma
  constexpr int CPITCH = NK + 4;           // floats per LDS row of the C tile
  constexpr int NBW = NKB / 2;             // N blocks per wave
  constexpr int GROUPS = kMergeRows * NK / 16 / 256;  // 16-element groups per thread
  static_assert(NKB % 2 == 0 && GROUPS >= 1, "tile shape");
  __shared__ __align__(16) uint16_t sigT[NK * SPITCH];
  __shared__ __align__(16) float Cs[kMergeRows * CPITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int mb = wave & 1;
  const int nb0 = (wave >> 1) * NBW;
  const int64_t cb = blockIdx.x % ncb;
  const int64_t gi = blockIdx.x / ncb;
  const int64_t lb = cb * NK;
  const int64_t ntiles = (d + kMergeRows - 1) / kMergeRows;
  const int64_t rt_begin = gi * tiles_per_block;
  const int64_t rt_end = rt_begin + tiles_per_block < ntiles ? rt_begin + tiles_per_block : ntiles;
  if (rt_begin >= rt_end) return;

  // Signs of A for columns [lb, lb + NK): sigT[l][j].
  if (tid < RP) {
    const int j = tid;
    const Philox4 p = sigma_block(KeyWords{key.k0, key.k1}, (uint64_t)j, (uint64_t)(lb >> 8));
    const int o = (int)(lb & 255);
    for (int l = 0; l < NK; ++l) {
      const int bitpos = o + l;
      const uint32_t bit = (uint32_t)(pick_word_m(p, bitpos >> 6) >> (bitpos & 63)) & 1u;
      const bool live = (j < r) && (lb + l < k);
      sigT[l * SPITCH + j] = live ? (uint16_t)(bit ? 0xBF80u : 0x3F80u) : (uint16_t)0;
    }
  }
  __syncthreads();

  u32x4 bfrag[KS][NBW];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int q = 0; q < NBW; ++q)
      bfrag[s][q] = *reinterpret_cast<const u32x4*>(
          &sigT[((nb0 + q) * 32 + (lane & 31)) * SPITCH + 16 * s + 8 * half]);

  float sc = scale_cr;
  if (scale_dev != nullptr) sc *= *scale_dev;
  const KeyWords srk{sr_key.k0, sr_key.k1};
  const bool r_vec = (r & 3) == 0;

  for (int64_t rt = rt_begin; rt < rt_end; ++rt) {
    const int64_t i0 = rt * kMergeRows;

    // Issue this tile's W loads early.
    u32x4 wv[GROUPS][2];
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      const int v = tid + 256 * g;
      const int row = v / (NK / 16);
      const int cg = v - row * (NK / 16);
      const int64_t i = i0 + row;
      const int64_t l = lb + 16 * cg;
      if (i < d && l + 16 <= k) {
        const u32x4* p = reinterpret_cast<const u32x4*>(W + i * ldw + l);
        wv[g][0] = p[0];
        wv[g][1] = p[1];
      } else {
        for (int h = 0; h < 2; ++h)
          for (int e = 0; e < 4; ++e) {
            uint32_t lo = 0, hi = 0;
            const int64_t c = l + 8 * h + 2 * e;
            if (i < d && c < k) lo = W[i * ldw + c];
            if (i < d && c + 1 < k) hi = W[i * ldw + c + 1];
            wv[g][h][e] = lo | (hi << 16);
          }
      }
    }

    // U rows of this wave's 32-row block as bf16 hi/lo A operands.
    const int64_t ui = i0 + 32 * mb + (lane & 31);
    u32x4 ah[KS], al[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int64_t j0 = 16 * s + 8 * half;
      float x[8];
      if (ui < d && r_vec && j0 + 8 <= r) {
        const f32x4* p = reinterpret_cast<const f32x4*>(U + ui * r + j0);
        const f32x4 x0 = p[0], x1 = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = x0[e];
          x[4 + e] = x1[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (ui < d && j0 + e < r) ? U[ui * r + j0 + e] : 0.f;
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t h0, l0, h1, l1;
        split_hi_lo(x[2 * p], h0, l0);
        split_hi_lo(x[2 * p + 1], h1, l1);
        ah[s][p] = h0 | (h1 << 16);
        al[s][p] = l0 | (l1 << 16);
      }
    }

#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah[s]), as_bf16x8(bfrag[s][q]),
                                                      acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al[s]), as_bf16x8(bfrag[s][q]),
                                                      acc, 0, 0, 0);
      }
      const int n = (nb0 + q) * 32 + (lane & 31);
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int m = 32 * mb + 8 * (reg >> 2) + 4 * half + (reg & 3);
        Cs[m * CPITCH + n] = acc[reg] * sc;
      }
    }
    __syncthreads();

#pragma unroll
    for (int g = 0; g < GROUPS; ++g) {
      const int v = tid + 256 * g;
      const int row = v / (NK / 16);
      const int cg = v - row * (NK / 16);
      const int64_t i = i0 + row;
      const int64_t l = lb + 16 * cg;
      if (i >= d || l >= k) continue;
      const f32x4* cp = reinterpret_cast<const f32x4*>(&Cs[row * CPITCH + 16 * cg]);
      float c[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 t4 = cp[q4];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[4 * q4 + e] = t4[e];
      }
      uint32_t out[8];
      const uint64_t e0 = (uint64_t)(row0 + i) * (uint64_t)k + (uint64_t)l;
      Philox4 p0, p1;
      if (stochastic) {
        p0 = sr_block(srk, e0 >> 4);
        if (((e0 + 15) >> 4) != (e0 >> 4)) p1 = sr_block(srk, (e0 + 15) >> 4);
        else p1 = p0;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t wbits = (wv[g][e >> 3][(e & 7) >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const float x = bf16_bits_to_f32(wbits) - c[e];
        uint32_t o;
        if (stochastic) {
          const uint64_t ee = e0 + e;
          const uint32_t u = ((ee >> 4) == (e0 >> 4)) ? sr_draw(p0, ee) : sr_draw(p1, ee);
          o = f32_to_bf16_sr(x, u);
        } else {
          o = f32_to_bf16_rne(x);
        }
        if (e & 1) out[e >> 1] |= o << 16;
        else out[e >> 1] = o;
      }
      if (l + 16 <= k) {
        u32x4* dst = reinterpret_cast<u32x4*>(W + i * ldw + l);
        u32x4 o0, o1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o0[e] = out[e];
          o1[e] = out[4 + e];
        }
        dst[0] = o0;
        dst[1] = o1;
      } else {
        for (int e = 0; e < 16 && l + e < k; ++e)
          W[i * ldw + l + e] = (uint16_t)((out[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      }
    }
    __syncthreads();
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
  const int64_t rp16 = (r + 15) / 16;  // rank steps of 16
  const int64_t ks = rp16 <= 2 ? 2 : rp16 <= 4 ? 4 : rp16 <= 8 ? 8 : 16;
  const int64_t nk = ks >= 16 ? 64 : 128;
  const int64_t ncb = (k + nk - 1) / nk;
  const int64_t ntiles = (d + kMergeRows - 1) / kMergeRows;
  int64_t groups = (1024 + ncb - 1) / ncb;
  if (groups > ntiles) groups = ntiles;
  if (groups < 1) groups = 1;
  const int64_t per = (ntiles + groups - 1) / groups;
  groups = (ntiles + per - 1) / per;
  const dim3 grid((unsigned)(ncb * groups));
  uint16_t* Wb = static_cast<uint16_t*>(W);
  const float scf = (float)(scale * cr);
  const int st = stochastic ? 1 : 0;
#define LOGRA_MERGE_LAUNCH(NKB, KS)                                                           \
  hipLaunchKernelGGL((merge_bf16_kernel<NKB, KS>), grid, dim3(256), 0, s, key, d, k, r, Wb, \
                     ldw, U, scf, scale_dev, st, sr_key, row0, ncb, per)
  switch (ks) {
    case 2: LOGRA_MERGE_LAUNCH(4, 2); break;
    case 4: LOGRA_MERGE_LAUNCH(4, 4); break;
    case 8: LOGRA_MERGE_LAUNCH(4, 8); break;
    case 16: LOGRA_MERGE_LAUNCH(2, 16); break;
    default: return hipErrorInvalidValue;
  }
#undef LOGRA_MERGE_LAUNCH
  return hipGetLastError();
}

}  // namespace logra
