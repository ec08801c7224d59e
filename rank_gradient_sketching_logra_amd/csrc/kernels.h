// Internal launcher interface between the C ABI layer and the HIP kernels.
// Launchers assume validated arguments (checked in logra_abi.cpp) and only
// enqueue work on `stream`; they return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace logra {

struct KeyArg {
  uint64_t k0, k1;
};

constexpr int kMaxGroup = 16;
constexpr int kMaxRank = 256;

struct AccItem {
  const void* D;   // [T x d] bf16 or fp32
  const float* XAt;
  float* S;
  int64_t d;
  int64_t ldd;
  void* ws;        // workspace of this item: packed projected input
};

// Rank padded to 1, 2, 4 or 8 whole 32-rank blocks, tokens to 16-token
// steps; size of the packed projected input of one accumulate item (a
// multiple of 256 bytes).
int64_t acc_rank_pad(int64_t r);
int64_t acc_token_pad(int64_t T);
size_t acc_ws_bytes_per_item(int64_t T, int64_t d, int64_t r);

hipError_t launch_regen_A(KeyArg key, int64_t r, int64_t k, bool int8_out, void* A,
                          hipStream_t s);
// XAt may be null when planes is given (bf16 X only); planes, when not
// null, receives the packed projected input the accumulate reads.  A_packed,
// when not null, is an explicit projection in the kernel's operand form (bf16
// X only) used instead of the key's signs.
hipError_t launch_project(KeyArg key, int64_t T, int64_t k, int64_t r, const void* X,
                          bool bf16, int64_t ldx, float* XAt, uint16_t* planes, hipStream_t s,
                          const void* A_packed = nullptr);
// Gaussian projection variant A [r x k] fp32; explicit projections packed for
// the projection kernel (projection_packed_bytes of them).
hipError_t launch_regen_A_gaussian(KeyArg key, int64_t r, int64_t k, float* A, hipStream_t s);
size_t projection_packed_bytes(int64_t r, int64_t k);
hipError_t launch_pack_projection(int64_t r, int64_t k, const float* A, void* packed,
                                  hipStream_t s);
// packed: items' ws already hold the packed projected input (XAt unused).
hipError_t launch_accumulate(int64_t T, int64_t r, bool bf16, const AccItem* items, int n,
                             bool packed, hipStream_t s);
// Packed accumulate over any number of matrices in one persistent launch:
// the matrix table (acc_table_ws_bytes(n) of device workspace) is copied in
// from the host on the stream.
size_t acc_table_ws_bytes(int n);
hipError_t launch_accumulate_table(int64_t T, int64_t r, const AccItem* items, int n, void* ws,
                                   hipStream_t s);
// Table-driven bf16 projection: any number (<= proj_table_max()) of
// projections sharing T and r in one persistent launch; the table
// (proj_table_ws_bytes(n) of device workspace) is copied in from the host on
// the stream.  Each item writes XAt and/or planes (either may be null).
struct ProjItem {
  const void* X;   // [T x k] bf16
  int64_t ldx, k;
  KeyArg key;
  float* XAt;
  uint16_t* planes;
};
int proj_table_max();
size_t proj_table_ws_bytes(int n);
hipError_t launch_project_table(int64_t T, int64_t r, const ProjItem* items, int n, void* ws,
                                hipStream_t s);
// Compute units of the current device.
int64_t compute_units();

// Streaming probe: read `bytes` of src (one 16-byte word per block into dst's
// 256 slots) or copy them to dst; blocks_per_cu blocks of 256 threads per
// compute unit.
hipError_t launch_probe(bool copy, const void* src, void* dst, int64_t bytes, int blocks_per_cu,
                        hipStream_t s);

// cos(G, (G A^T) A) and its parts {cos, ||G||^2, ||G A^T||^2, ||G A^T A||^2}
// written to out (4 doubles on the device).
size_t reconstruction_cosine_ws_bytes(int64_t d, int64_t k, int64_t r);
// With A (fp32 [r x k]) and A_packed (its projection operands) given, the
// explicit projection is used instead of the key's signs (bf16 G only).
hipError_t launch_reconstruction_cosine(KeyArg key, int64_t d, int64_t k, int64_t r, const void* G,
                                        bool bf16, int64_t ldg, double* out, void* ws,
                                        hipStream_t s, const float* A = nullptr,
                                        const void* A_packed = nullptr);

size_t rowadam_ws_bytes(int64_t d);
// One sketch of a grouped RowAdam writing packed updates.
struct RowAdamItem {
  const float* S;
  float* v;
  void* P;
  int64_t d;
};
size_t rowadam_grouped_ws_bytes(int n, int64_t total_rows);
hipError_t launch_rowadam_packed_grouped(const RowAdamItem* items, int n, int64_t r, int64_t t,
                                         double beta, double eps, void* ws, hipStream_t s);
// U (fp32) and/or U_packed (the merge's packed update) may be null.
hipError_t launch_rowadam(int64_t d, int64_t r, const float* S, float* v, int64_t t,
                          double beta, double eps, float* U, void* U_packed, void* ws,
                          hipStream_t s);

// Mean over P contexts of KL(softmax(z/tau) || softmax((z + alpha zdot)/tau)), fp64, to *out.
size_t exact_kl_ws_bytes(int64_t P);
hipError_t launch_exact_kl(int64_t P, int64_t V, const void* z, const void* zd, bool bf16,
                           double alpha, double tau, double* out, void* ws, hipStream_t s);

size_t klq_ws_bytes(int64_t P, int64_t V);
// The same q with the partials in the library's per-GPU scratch array (no
// workspace, no allocation); at most noalloc_max_contexts() contexts.
int64_t noalloc_max_contexts();
hipError_t launch_predicted_kl_q_noalloc(int64_t P, int64_t V, const void* z, const void* zd,
                                         bool bf16, float tau, float* q, hipStream_t s);
hipError_t launch_predicted_kl_q(int64_t P, int64_t V, const void* z, const void* zd,
                                 bool bf16, float tau, float* q, void* ws, hipStream_t s);
hipError_t launch_step_alpha(const float* q, float delta, float amax, float* alpha,
                             hipStream_t s);

struct MergeItem {
  KeyArg key;      // sign key of the matrix
  KeyArg sr_key;   // stochastic-rounding key of the matrix
  void* W;         // [d x k] bf16, leading dimension ldw
  int64_t d, k, ldw;
  const void* U;   // [d x r] fp32, or the packed update (packed launches)
  int64_t row0;
  const void* A = nullptr;  // explicit projection in merge operand order (packed launches), or null
};
// Several bf16 merges sharing r, the scale and the rounding mode in one launch.
hipError_t launch_merge_grouped(const MergeItem* items, int n, int64_t r, double scale,
                                const float* scale_dev, bool stochastic, bool packed,
                                hipStream_t s);
// 16-rank steps of the merge (1, 2, 4, 8 or 16) and the packed update's size.
int merge_rank_steps(int64_t r);
size_t packed_update_bytes(int64_t d, int64_t r);
// packed = split(fl32(s U)), s = scale * (*scale_dev if given).
size_t merge_projection_packed_bytes(int64_t r, int64_t k);
hipError_t launch_pack_merge_projection(int64_t r, int64_t k, const float* A, void* packed,
                                        hipStream_t s);
hipError_t launch_pack_update(int64_t d, int64_t r, const float* U, float scale,
                              const float* scale_dev, void* packed, hipStream_t s);
hipError_t launch_merge(KeyArg key, int64_t d, int64_t k, int64_t r, void* W, bool bf16,
                        int64_t ldw, const float* U, double scale, const float* scale_dev,
                        bool stochastic, KeyArg sr_key, int64_t row0, hipStream_t s);

}  // namespace logra
