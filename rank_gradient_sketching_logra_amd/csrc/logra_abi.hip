// C ABI entry points: host-side validation, then launches on the caller's
// stream.  Nothing is launched when validation fails.  See include/logra.h
// for the contract of every call.
#include <algorithm>
#include <cmath>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <new>

#include "../../include/logra.h"
#include "kernels.h"

namespace {

// The calling thread's last error message.  A fixed buffer: recording an
// error allocates nothing, so it cannot itself fail inside the guard below.
thread_local char g_last_error[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return LOGRA_OK;
}

// Every int-returning entry point runs its body inside LOGRA_TRY ...
// LOGRA_CATCH, so no C++ exception (std::bad_alloc from a descriptor table,
// say) crosses the C ABI: it becomes LOGRA_ERR_HOST with a message.
#define LOGRA_TRY try {
#define LOGRA_CATCH(name)                                                                  \
  }                                                                                        \
  catch (const std::bad_alloc&) {                                                          \
    return fail(LOGRA_ERR_HOST, "%s: out of host memory", name);                           \
  }                                                                                        \
  catch (const std::exception& ex) {                                                       \
    return fail(LOGRA_ERR_HOST, "%s: host-side exception: %s", name, ex.what());          \
  }                                                                                        \
  catch (...) {                                                                            \
    return fail(LOGRA_ERR_HOST, "%s: unknown host-side exception", name);                  \
  }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LOGRA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [p, p + n).
struct Range {
  uintptr_t lo, hi;
};
Range range(const void* p, size_t n) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + n};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

size_t elem_size(logra_dtype t) { return t == LOGRA_F32 ? 4 : t == LOGRA_BF16 ? 2 : 1; }

// Extent in bytes of a [rows x cols] matrix with leading dimension ld.
size_t extent(int64_t rows, int64_t cols, int64_t ld, size_t es) {
  return (size_t)((rows - 1) * ld + cols) * es;
}

bool bad_rank(int64_t r) { return r < 1 || r > LOGRA_MAX_RANK; }

// Bounds that keep every byte count the validation forms (extents, T * r * 4,
// d * k * 2, ...) far inside int64_t / size_t: a dimension or leading
// dimension is at most 2^40 elements and one matrix at most 2^50 elements.
constexpr int64_t kMaxDim = int64_t(1) << 40;
constexpr int64_t kMaxElems = int64_t(1) << 50;
bool bad_dim(int64_t x) { return x < 1 || x > kMaxDim; }

logra::KeyArg key_words(uint64_t seed, const logra_key* key) {
  return logra::KeyArg{seed, ((uint64_t)key->step << 32) | (uint64_t)key->matrix_id};
}

// A matrix operand (X, D or W): dtype, alignment of base and rows.
int check_matrix(const char* name, const void* p, logra_dtype t, int64_t ld, int64_t rows, int64_t cols) {
  if (t != LOGRA_F32 && t != LOGRA_BF16) return fail(LOGRA_ERR_DTYPE, "%s: dtype must be F32 or BF16", name);
  if (ld < cols) return fail(LOGRA_ERR_SHAPE, "%s: leading dimension %lld < %lld", name, (long long)ld, (long long)cols);
  if (bad_dim(rows) || bad_dim(cols) || ld > kMaxDim || rows > kMaxElems / ld)
    return fail(LOGRA_ERR_SHAPE, "%s: %lld x %lld (leading dimension %lld) is out of range", name, (long long)rows,
                (long long)cols, (long long)ld);
  if (!aligned16(p)) return fail(LOGRA_ERR_ALIGN, "%s: base pointer not 16-byte aligned", name);
  if ((ld * (int64_t)elem_size(t)) % 16 != 0)
    return fail(LOGRA_ERR_ALIGN, "%s: rows not 16-byte aligned (leading dimension %lld)", name, (long long)ld);
  return LOGRA_OK;
}

}  // namespace

extern "C" {

LOGRA_API const char* logra_version(void) { return "logra-mi355x 0.1.0 (gfx950)"; }

LOGRA_API const char* logra_last_error(void) { return g_last_error; }

LOGRA_API int64_t logra_sketch_bytes(int64_t d, int64_t r) {
  if (d < 0 || r < 0) return -1;
  return 4 * d * r;
}

LOGRA_API int logra_regen_A(const logra_key* key, int64_t r, int64_t k, logra_dtype out,
                            void* A, logra_stream stream) {
  LOGRA_TRY
  if (!key || !A) return fail(LOGRA_ERR_NULL, "regen_A: NULL key or output");
  if (bad_rank(r) || bad_dim(k)) return fail(LOGRA_ERR_SHAPE, "regen_A: need 1 <= r <= %d and k >= 1", LOGRA_MAX_RANK);
  if (out != LOGRA_I8 && out != LOGRA_F32) return fail(LOGRA_ERR_DTYPE, "regen_A: output must be I8 or F32");
  return hip_status(logra::launch_regen_A(key_words(key->seed, key), r, k, out == LOGRA_I8, A,
                                          static_cast<hipStream_t>(stream)),
                    "regen_A launch");
  LOGRA_CATCH("regen_A")
}

LOGRA_API int logra_project_input(const logra_key* key, int64_t T, int64_t k, int64_t r,
                                  const void* X, logra_dtype x_dtype, int64_t ldx, float* XAt,
                                  logra_stream stream) {
  LOGRA_TRY
  if (!key || !X || !XAt) return fail(LOGRA_ERR_NULL, "project_input: NULL pointer");
  if (bad_dim(T) || bad_dim(k) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "project_input: need T, k >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  int st = check_matrix("project_input X", X, x_dtype, ldx, T, k);
  if (st) return st;
  if (!aligned16(XAt)) return fail(LOGRA_ERR_ALIGN, "project_input: XAt not 16-byte aligned");
  if (overlap(range(X, extent(T, k, ldx, elem_size(x_dtype))), range(XAt, (size_t)(T * r) * 4)))
    return fail(LOGRA_ERR_ALIAS, "project_input: XAt overlaps X");
  return hip_status(logra::launch_project(key_words(key->seed, key), T, k, r, X, x_dtype == LOGRA_BF16,
                                          ldx, XAt, nullptr, static_cast<hipStream_t>(stream)),
                    "project_input launch");
  LOGRA_CATCH("project_input")
}

LOGRA_API int logra_regen_A_gaussian(const logra_key* key, int64_t r, int64_t k, float* A,
                                     logra_stream stream) {
  LOGRA_TRY
  if (!key || !A) return fail(LOGRA_ERR_NULL, "regen_A_gaussian: NULL pointer");
  if (bad_dim(k) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "regen_A_gaussian: need k >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  if (!aligned16(A)) return fail(LOGRA_ERR_ALIGN, "regen_A_gaussian: A not 16-byte aligned");
  return hip_status(logra::launch_regen_A_gaussian(key_words(key->seed, key), r, k, A,
                                                   static_cast<hipStream_t>(stream)),
                    "regen_A_gaussian launch");
  LOGRA_CATCH("regen_A_gaussian")
}

LOGRA_API size_t logra_projection_packed_bytes(int64_t r, int64_t k) {
  if (bad_dim(k) || bad_rank(r)) return 0;
  return logra::projection_packed_bytes(r, k);
}

LOGRA_API int logra_pack_projection(int64_t r, int64_t k, const float* A, void* A_packed,
                                    size_t packed_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!A || !A_packed) return fail(LOGRA_ERR_NULL, "pack_projection: NULL pointer");
  if (bad_dim(k) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "pack_projection: need k >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  const size_t need = logra::projection_packed_bytes(r, k);
  if (packed_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "pack_projection: %zu bytes needed", need);
  if (!aligned16(A_packed)) return fail(LOGRA_ERR_ALIGN, "pack_projection: output not 16-byte aligned");
  if (overlap(range(A, (size_t)(r * k) * 4), range(A_packed, need)))
    return fail(LOGRA_ERR_ALIAS, "pack_projection: A overlaps the packed output");
  return hip_status(logra::launch_pack_projection(r, k, A, A_packed, static_cast<hipStream_t>(stream)),
                    "pack_projection launch");
  LOGRA_CATCH("pack_projection")
}

LOGRA_API int logra_project_input_explicit(int64_t T, int64_t k, int64_t r, const void* X,
                                           logra_dtype x_dtype, int64_t ldx, const void* A_packed,
                                           size_t packed_bytes, float* XAt, void* planes,
                                           size_t planes_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!X || !A_packed || (!XAt && !planes)) return fail(LOGRA_ERR_NULL, "project_input_explicit: NULL pointer");
  if (bad_dim(T) || bad_dim(k) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "project_input_explicit: need T, k >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  if (x_dtype != LOGRA_BF16) return fail(LOGRA_ERR_DTYPE, "project_input_explicit: X must be bf16");
  int st = check_matrix("project_input_explicit X", X, x_dtype, ldx, T, k);
  if (st) return st;
  const size_t aneed = logra::projection_packed_bytes(r, k);
  if (packed_bytes < aneed) return fail(LOGRA_ERR_WORKSPACE, "project_input_explicit: the packed projection needs %zu bytes", aneed);
  const size_t pneed = planes ? logra::acc_ws_bytes_per_item(T, 1, r) : 0;
  if (planes && planes_bytes < pneed) return fail(LOGRA_ERR_WORKSPACE, "project_input_explicit: %zu bytes of packed output needed", pneed);
  if (!aligned16(A_packed) || (planes && !aligned16(planes)) || (XAt && !aligned16(XAt)))
    return fail(LOGRA_ERR_ALIGN, "project_input_explicit: operands must be 16-byte aligned");
  const Range rx = range(X, extent(T, k, ldx, elem_size(x_dtype))), ra = range(A_packed, aneed);
  const Range rp = planes ? range(planes, pneed) : Range{0, 0};
  const Range ro = XAt ? range(XAt, (size_t)(T * r) * 4) : Range{0, 0};
  if (overlap(rx, rp) || overlap(rx, ro) || overlap(rp, ro) || overlap(ra, rp) || overlap(ra, ro))
    return fail(LOGRA_ERR_ALIAS, "project_input_explicit: outputs overlap an input or each other");
  return hip_status(logra::launch_project(logra::KeyArg{0, 0}, T, k, r, X, true, ldx, XAt,
                                          static_cast<uint16_t*>(planes), static_cast<hipStream_t>(stream),
                                          A_packed),
                    "project_input_explicit launch");
  LOGRA_CATCH("project_input_explicit")
}

LOGRA_API int logra_reconstruction_cosine_explicit(int64_t d, int64_t k, int64_t r, const void* G,
                                                   logra_dtype g_dtype, int64_t ldg, const float* A,
                                                   const void* A_packed, size_t packed_bytes,
                                                   double* out_dev, void* ws, size_t ws_bytes,
                                                   logra_stream stream) {
  LOGRA_TRY
  if (!G || !A || !A_packed || !out_dev) return fail(LOGRA_ERR_NULL, "reconstruction_cosine_explicit: NULL pointer");
  if (bad_dim(d) || bad_dim(k) || bad_rank(r))
    return fail(LOGRA_ERR_SHAPE, "reconstruction_cosine_explicit: need d, k >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  if (g_dtype != LOGRA_BF16) return fail(LOGRA_ERR_DTYPE, "reconstruction_cosine_explicit: G must be bf16");
  int st = check_matrix("reconstruction_cosine_explicit G", G, g_dtype, ldg, d, k);
  if (st) return st;
  const size_t aneed = logra::projection_packed_bytes(r, k);
  if (packed_bytes < aneed) return fail(LOGRA_ERR_WORKSPACE, "reconstruction_cosine_explicit: the packed projection needs %zu bytes", aneed);
  const size_t need = logra::reconstruction_cosine_ws_bytes(d, k, r);
  if (!ws || ws_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "reconstruction_cosine_explicit: workspace of %zu bytes needed", need);
  if (!aligned16(ws) || !aligned16(A_packed) || (reinterpret_cast<uintptr_t>(out_dev) & 7u) != 0)
    return fail(LOGRA_ERR_ALIGN, "reconstruction_cosine_explicit: workspace and packed projection 16-byte, output 8-byte aligned");
  const Range rg = range(G, extent(d, k, ldg, 2)), rw = range(ws, need), ro = range(out_dev, 32);
  if (overlap(rg, rw) || overlap(rg, ro) || overlap(rw, ro) || overlap(rw, range(A, (size_t)(r * k) * 4)) ||
      overlap(rw, range(A_packed, aneed)))
    return fail(LOGRA_ERR_ALIAS, "reconstruction_cosine_explicit: operands overlap");
  return hip_status(logra::launch_reconstruction_cosine(logra::KeyArg{0, 0}, d, k, r, G, true, ldg, out_dev, ws,
                                                        static_cast<hipStream_t>(stream), A, A_packed),
                    "reconstruction_cosine_explicit launch");
  LOGRA_CATCH("reconstruction_cosine_explicit")
}

LOGRA_API size_t logra_reconstruction_cosine_ws_bytes(int64_t d, int64_t k, int64_t r) {
  if (bad_dim(d) || bad_dim(k) || bad_rank(r)) return 0;
  return logra::reconstruction_cosine_ws_bytes(d, k, r);
}

LOGRA_API int logra_reconstruction_cosine(const logra_key* key, int64_t d, int64_t k, int64_t r,
                                          const void* G, logra_dtype g_dtype, int64_t ldg,
                                          double* out_dev, void* ws, size_t ws_bytes,
                                          logra_stream stream) {
  LOGRA_TRY
  if (!key || !G || !out_dev) return fail(LOGRA_ERR_NULL, "reconstruction_cosine: NULL pointer");
  if (bad_dim(d) || bad_dim(k) || bad_rank(r))
    return fail(LOGRA_ERR_SHAPE, "reconstruction_cosine: need d, k >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  int st = check_matrix("reconstruction_cosine G", G, g_dtype, ldg, d, k);
  if (st) return st;
  const size_t need = logra::reconstruction_cosine_ws_bytes(d, k, r);
  if (!ws || ws_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "reconstruction_cosine: workspace of %zu bytes needed", need);
  if (!aligned16(ws) || (reinterpret_cast<uintptr_t>(out_dev) & 7u) != 0)
    return fail(LOGRA_ERR_ALIGN, "reconstruction_cosine: workspace 16-byte and output 8-byte aligned");
  const Range rg = range(G, extent(d, k, ldg, elem_size(g_dtype))), rw = range(ws, need), ro = range(out_dev, 32);
  if (overlap(rg, rw) || overlap(rg, ro) || overlap(rw, ro))
    return fail(LOGRA_ERR_ALIAS, "reconstruction_cosine: G, output and workspace must not overlap");
  return hip_status(logra::launch_reconstruction_cosine(key_words(key->seed, key), d, k, r, G,
                                                        g_dtype == LOGRA_BF16, ldg, out_dev, ws,
                                                        static_cast<hipStream_t>(stream)),
                    "reconstruction_cosine launch");
  LOGRA_CATCH("reconstruction_cosine")
}

LOGRA_API size_t logra_packed_input_bytes(int64_t T, int64_t r) {
  if (bad_dim(T) || bad_rank(r)) return 0;
  return logra::acc_ws_bytes_per_item(T, 1, r);
}

LOGRA_API int logra_project_input_packed(const logra_key* key, int64_t T, int64_t k, int64_t r,
                                         const void* X, logra_dtype x_dtype, int64_t ldx,
                                         float* XAt, void* planes, size_t planes_bytes,
                                         logra_stream stream) {
  LOGRA_TRY
  if (!key || !X || !planes) return fail(LOGRA_ERR_NULL, "project_input_packed: NULL pointer");
  if (bad_dim(T) || bad_dim(k) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "project_input_packed: need T, k >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  if (x_dtype != LOGRA_BF16) return fail(LOGRA_ERR_DTYPE, "project_input_packed: X must be bf16");
  int st = check_matrix("project_input_packed X", X, x_dtype, ldx, T, k);
  if (st) return st;
  const size_t need = logra::acc_ws_bytes_per_item(T, 1, r);
  if (planes_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "project_input_packed: %zu bytes of packed output needed", need);
  if (!aligned16(planes) || (XAt && !aligned16(XAt))) return fail(LOGRA_ERR_ALIGN, "project_input_packed: outputs must be 16-byte aligned");
  const Range rx = range(X, extent(T, k, ldx, elem_size(x_dtype)));
  const Range rp = range(planes, need);
  if (overlap(rx, rp) || (XAt && (overlap(rx, range(XAt, (size_t)(T * r) * 4)) || overlap(rp, range(XAt, (size_t)(T * r) * 4)))))
    return fail(LOGRA_ERR_ALIAS, "project_input_packed: outputs overlap X or each other");
  return hip_status(logra::launch_project(key_words(key->seed, key), T, k, r, X, true, ldx, XAt,
                                          static_cast<uint16_t*>(planes), static_cast<hipStream_t>(stream)),
                    "project_input_packed launch");
  LOGRA_CATCH("project_input_packed")
}

LOGRA_API size_t logra_project_input_table_ws_bytes(int n) {
  if (n < 1 || n > LOGRA_MAX_PROJECT_TABLE) return 0;
  return logra::proj_table_ws_bytes(n);
}

LOGRA_API int logra_project_input_table(int64_t T, int64_t r, const logra_project_desc* descs,
                                        int n, void* ws, size_t ws_bytes, logra_stream stream) {
  LOGRA_TRY
  static_assert(LOGRA_MAX_PROJECT_TABLE <= 1024, "the kernel's table limit");
  if (!descs || !ws) return fail(LOGRA_ERR_NULL, "project_input_table: NULL pointer");
  if (n < 1 || n > LOGRA_MAX_PROJECT_TABLE) return fail(LOGRA_ERR_SHAPE, "project_input_table: need 1 <= n <= %d", LOGRA_MAX_PROJECT_TABLE);
  if (bad_dim(T) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "project_input_table: need T >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  const size_t tneed = logra::proj_table_ws_bytes(n);
  if (ws_bytes < tneed) return fail(LOGRA_ERR_WORKSPACE, "project_input_table: workspace of %zu bytes needed", tneed);
  if (!aligned16(ws)) return fail(LOGRA_ERR_ALIGN, "project_input_table: workspace not 16-byte aligned");
  const size_t pneed = logra::acc_ws_bytes_per_item(T, 1, r);
  const size_t xat_bytes = (size_t)(T * r) * 4;
  std::vector<logra::ProjItem> items((size_t)n);
  std::vector<Range> xs((size_t)n), outs;
  outs.reserve(2 * (size_t)n + 1);
  outs.push_back(range(ws, tneed));
  for (int i = 0; i < n; ++i) {
    const logra_project_desc& e = descs[i];
    if (!e.X) return fail(LOGRA_ERR_NULL, "project_input_table: NULL X in descriptor %d", i);
    if (!e.XAt && !e.planes) return fail(LOGRA_ERR_NULL, "project_input_table: descriptor %d has no output", i);
    if (bad_dim(e.k)) return fail(LOGRA_ERR_SHAPE, "project_input_table: k must be >= 1");
    if (e.planes && e.planes_bytes < pneed)
      return fail(LOGRA_ERR_WORKSPACE, "project_input_table: descriptor %d: the packed input needs %zu bytes", i, pneed);
    int st = check_matrix("project_input_table X", e.X, LOGRA_BF16, e.ldx, T, e.k);
    if (st) return st;
    if ((e.XAt && !aligned16(e.XAt)) || (e.planes && !aligned16(e.planes)))
      return fail(LOGRA_ERR_ALIGN, "project_input_table: outputs must be 16-byte aligned");
    xs[i] = range(e.X, extent(T, e.k, e.ldx, 2));
    if (e.XAt) outs.push_back(range(e.XAt, xat_bytes));
    if (e.planes) outs.push_back(range(e.planes, pneed));
    items[i] = logra::ProjItem{e.X, e.ldx, e.k, key_words(e.key.seed, &e.key), e.XAt,
                               static_cast<uint16_t*>(e.planes)};
  }
  // Outputs (and the workspace) against each other, sorted by address, then
  // against every input; inputs may be shared.
  std::sort(outs.begin(), outs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < outs.size(); ++i)
    if (overlap(outs[i - 1], outs[i])) return fail(LOGRA_ERR_ALIAS, "project_input_table: two outputs (or an output and the workspace) overlap");
  for (const Range& o : outs)
    for (int j = 0; j < n; ++j)
      if (overlap(o, xs[j])) return fail(LOGRA_ERR_ALIAS, "project_input_table: an output or the workspace overlaps the X of descriptor %d", j);
  return hip_status(logra::launch_project_table(T, r, items.data(), n, ws, static_cast<hipStream_t>(stream)),
                    "project_input_table launch");
  LOGRA_CATCH("project_input_table")
}

LOGRA_API size_t logra_sketch_accumulate_ws_bytes(int64_t T, int64_t d, int64_t r) {
  if (bad_dim(T) || bad_dim(d) || bad_rank(r)) return 0;
  return logra::acc_ws_bytes_per_item(T, d, r);
}

static int check_acc_item(const char* name, int64_t T, int64_t r, logra_dtype dt, const void* D,
                          int64_t d, int64_t ldd, const float* XAt, const float* S, void* ws,
                          size_t ws_bytes) {
  if (!D || !XAt || !S) return fail(LOGRA_ERR_NULL, "%s: NULL pointer", name);
  if (bad_dim(d)) return fail(LOGRA_ERR_SHAPE, "%s: d must be >= 1", name);
  int st = check_matrix(name, D, dt, ldd, T, d);
  if (st) return st;
  if (!aligned16(XAt) || !aligned16(S)) return fail(LOGRA_ERR_ALIGN, "%s: XAt and S must be 16-byte aligned", name);
  const Range rs = range(S, (size_t)(d * r) * 4);
  if (overlap(rs, range(D, extent(T, d, ldd, elem_size(dt)))) || overlap(rs, range(XAt, (size_t)(T * r) * 4)))
    return fail(LOGRA_ERR_ALIAS, "%s: S overlaps D or XAt", name);
  if (dt == LOGRA_BF16) {
    const size_t need = logra::acc_ws_bytes_per_item(T, d, r);
    if (!ws || ws_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", name, need);
    if (!aligned16(ws)) return fail(LOGRA_ERR_ALIGN, "%s: workspace not 16-byte aligned", name);
    const Range rw = range(ws, need);
    if (overlap(rw, rs) || overlap(rw, range(D, extent(T, d, ldd, elem_size(dt)))) ||
        overlap(rw, range(XAt, (size_t)(T * r) * 4)))
      return fail(LOGRA_ERR_ALIAS, "%s: workspace overlaps an operand", name);
  }
  return LOGRA_OK;
}

LOGRA_API int logra_sketch_accumulate(int64_t T, int64_t d, int64_t r, const void* D,
                                      logra_dtype d_dtype, int64_t ldd, const float* XAt,
                                      float* S, void* ws, size_t ws_bytes, logra_stream stream) {
  LOGRA_TRY
  if (bad_dim(T) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate: need T >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  int st = check_acc_item("sketch_accumulate", T, r, d_dtype, D, d, ldd, XAt, S, ws, ws_bytes);
  if (st) return st;
  logra::AccItem it{D, XAt, S, d, ldd, ws};
  return hip_status(logra::launch_accumulate(T, r, d_dtype == LOGRA_BF16, &it, 1, false,
                                             static_cast<hipStream_t>(stream)),
                    "sketch_accumulate launch");
  LOGRA_CATCH("sketch_accumulate")
}

LOGRA_API int logra_sketch_accumulate_grouped(int64_t T, int64_t r, logra_dtype d_dtype,
                                              const logra_acc_desc* descs, int n, void* ws,
                                              size_t ws_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!descs) return fail(LOGRA_ERR_NULL, "sketch_accumulate_grouped: NULL descriptors");
  if (n < 1 || n > LOGRA_MAX_GROUP) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate_grouped: need 1 <= n <= %d", LOGRA_MAX_GROUP);
  if (bad_dim(T) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate_grouped: need T >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  logra::AccItem items[LOGRA_MAX_GROUP];
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const size_t per = descs[i].d >= 1 ? logra::acc_ws_bytes_per_item(T, descs[i].d, r) : 0;
    void* wsi = (d_dtype == LOGRA_BF16 && ws) ? static_cast<char*>(ws) + off : nullptr;
    if (d_dtype == LOGRA_BF16 && (!ws || ws_bytes < off + per))
      return fail(LOGRA_ERR_WORKSPACE, "sketch_accumulate_grouped: workspace of at least %zu bytes needed", off + per);
    int st = check_acc_item("sketch_accumulate_grouped", T, r, d_dtype, descs[i].D, descs[i].d, descs[i].ldd,
                            descs[i].XAt, descs[i].S, wsi, per);
    if (st) return st;
    for (int j = 0; j < i; ++j)
      if (overlap(range(descs[i].S, (size_t)(descs[i].d * r) * 4), range(descs[j].S, (size_t)(descs[j].d * r) * 4)))
        return fail(LOGRA_ERR_ALIAS, "sketch_accumulate_grouped: sketches %d and %d overlap", j, i);
    items[i] = logra::AccItem{descs[i].D, descs[i].XAt, descs[i].S, descs[i].d, descs[i].ldd, wsi};
    if (d_dtype == LOGRA_BF16) off += per;
  }
  return hip_status(logra::launch_accumulate(T, r, d_dtype == LOGRA_BF16, items, n, false,
                                             static_cast<hipStream_t>(stream)),
                    "sketch_accumulate_grouped launch");
  LOGRA_CATCH("sketch_accumulate_grouped")
}

LOGRA_API int logra_sketch_accumulate_grouped_packed(int64_t T, int64_t r,
                                                     const logra_acc_packed_desc* descs, int n,
                                                     logra_stream stream) {
  LOGRA_TRY
  if (!descs) return fail(LOGRA_ERR_NULL, "sketch_accumulate_grouped_packed: NULL descriptors");
  if (n < 1 || n > LOGRA_MAX_GROUP) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate_grouped_packed: need 1 <= n <= %d", LOGRA_MAX_GROUP);
  if (bad_dim(T) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate_grouped_packed: need T >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  const size_t need = logra::acc_ws_bytes_per_item(T, 1, r);
  logra::AccItem items[LOGRA_MAX_GROUP];
  for (int i = 0; i < n; ++i) {
    const logra_acc_packed_desc& e = descs[i];
    if (!e.D || !e.planes || !e.S) return fail(LOGRA_ERR_NULL, "sketch_accumulate_grouped_packed: NULL pointer in descriptor %d", i);
    if (bad_dim(e.d)) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate_grouped_packed: d must be >= 1");
    if (e.planes_bytes < need)
      return fail(LOGRA_ERR_WORKSPACE, "sketch_accumulate_grouped_packed: descriptor %d: the packed input needs %zu bytes", i, need);
    int st = check_matrix("sketch_accumulate_grouped_packed D", e.D, LOGRA_BF16, e.ldd, T, e.d);
    if (st) return st;
    if (!aligned16(e.planes) || !aligned16(e.S)) return fail(LOGRA_ERR_ALIGN, "sketch_accumulate_grouped_packed: planes and S must be 16-byte aligned");
    const Range rs = range(e.S, (size_t)(e.d * r) * 4);
    if (overlap(rs, range(e.D, extent(T, e.d, e.ldd, 2))) || overlap(rs, range(e.planes, need)))
      return fail(LOGRA_ERR_ALIAS, "sketch_accumulate_grouped_packed: S overlaps D or the packed input");
    for (int j = 0; j < i; ++j)
      if (overlap(rs, range(descs[j].S, (size_t)(descs[j].d * r) * 4)) || overlap(rs, range(descs[j].planes, need)))
        return fail(LOGRA_ERR_ALIAS, "sketch_accumulate_grouped_packed: sketch %d overlaps an operand of %d", i, j);
    items[i] = logra::AccItem{e.D, nullptr, e.S, e.d, e.ldd, const_cast<uint16_t*>(e.planes)};
  }
  return hip_status(logra::launch_accumulate(T, r, true, items, n, true, static_cast<hipStream_t>(stream)),
                    "sketch_accumulate_grouped_packed launch");
  LOGRA_CATCH("sketch_accumulate_grouped_packed")
}

LOGRA_API size_t logra_sketch_accumulate_table_ws_bytes(int n) {
  if (n < 1) return 0;
  return logra::acc_table_ws_bytes(n);
}

LOGRA_API int logra_sketch_accumulate_table(int64_t T, int64_t r, const logra_acc_packed_desc* descs,
                                            int n, void* ws, size_t ws_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!descs || !ws) return fail(LOGRA_ERR_NULL, "sketch_accumulate_table: NULL pointer");
  if (n < 1) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate_table: need n >= 1");
  if (bad_dim(T) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate_table: need T >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  const size_t tneed = logra::acc_table_ws_bytes(n);
  if (ws_bytes < tneed) return fail(LOGRA_ERR_WORKSPACE, "sketch_accumulate_table: workspace of %zu bytes needed", tneed);
  if (!aligned16(ws)) return fail(LOGRA_ERR_ALIGN, "sketch_accumulate_table: workspace not 16-byte aligned");
  const size_t need = logra::acc_ws_bytes_per_item(T, 1, r);
  const Range rws = range(ws, tneed);
  std::vector<logra::AccItem> items((size_t)n);
  std::vector<Range> rs((size_t)n);
  for (int i = 0; i < n; ++i) {
    const logra_acc_packed_desc& e = descs[i];
    if (!e.D || !e.planes || !e.S) return fail(LOGRA_ERR_NULL, "sketch_accumulate_table: NULL pointer in descriptor %d", i);
    if (bad_dim(e.d)) return fail(LOGRA_ERR_SHAPE, "sketch_accumulate_table: d must be >= 1");
    if (e.planes_bytes < need)
      return fail(LOGRA_ERR_WORKSPACE, "sketch_accumulate_table: descriptor %d: the packed input needs %zu bytes", i, need);
    int st = check_matrix("sketch_accumulate_table D", e.D, LOGRA_BF16, e.ldd, T, e.d);
    if (st) return st;
    if (!aligned16(e.planes) || !aligned16(e.S)) return fail(LOGRA_ERR_ALIGN, "sketch_accumulate_table: planes and S must be 16-byte aligned");
    rs[i] = range(e.S, (size_t)(e.d * r) * 4);
    if (overlap(rs[i], range(e.D, extent(T, e.d, e.ldd, 2))) || overlap(rs[i], range(e.planes, need)) ||
        overlap(rws, rs[i]) || overlap(rws, range(e.D, extent(T, e.d, e.ldd, 2))) || overlap(rws, range(e.planes, need)))
      return fail(LOGRA_ERR_ALIAS, "sketch_accumulate_table: S or the workspace overlaps an operand of descriptor %d", i);
    items[i] = logra::AccItem{e.D, nullptr, e.S, e.d, e.ldd, const_cast<uint16_t*>(e.planes)};
  }
  // Every sketch against every other matrix's operands (sorted by address, so
  // the pairwise check stays cheap for whole-model tables).
  std::vector<int> order((size_t)n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int a, int b) { return rs[a].lo < rs[b].lo; });
  for (int i = 1; i < n; ++i)
    if (overlap(rs[order[i - 1]], rs[order[i]])) return fail(LOGRA_ERR_ALIAS, "sketch_accumulate_table: two sketches overlap");
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j)
      if (i != j && (overlap(rs[i], range(descs[j].D, extent(T, descs[j].d, descs[j].ldd, 2))) ||
                     overlap(rs[i], range(descs[j].planes, need))))
        return fail(LOGRA_ERR_ALIAS, "sketch_accumulate_table: sketch %d overlaps an operand of %d", i, j);
  return hip_status(logra::launch_accumulate_table(T, r, items.data(), n, ws, static_cast<hipStream_t>(stream)),
                    "sketch_accumulate_table launch");
  LOGRA_CATCH("sketch_accumulate_table")
}

LOGRA_API size_t logra_rowadam_ws_bytes(int64_t d) {
  if (bad_dim(d)) return 0;
  return logra::rowadam_ws_bytes(d);
}

namespace {
// RowAdam with U written as fp32 (U) or as the packed update (P, P_bytes).
int rowadam_impl(const char* name, int64_t d, int64_t r, const float* S, float* v, int64_t t,
                 double beta, double eps, float* U, void* P, size_t P_bytes, void* ws,
                 size_t ws_bytes, logra_stream stream) {
  if (!S || !v || (!U && !P)) return fail(LOGRA_ERR_NULL, "%s: NULL pointer", name);
  if (bad_dim(d) || bad_dim(r) || d > kMaxElems / r) return fail(LOGRA_ERR_SHAPE, "%s: d x r out of range", name);
  if (P && bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "%s: need r <= %d", name, LOGRA_MAX_RANK);
  if (t < 1) return fail(LOGRA_ERR_DOMAIN, "%s: t counts updates from 1", name);
  if (!(beta >= 0.0 && beta < 1.0)) return fail(LOGRA_ERR_DOMAIN, "%s: beta must be in [0, 1)", name);
  if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(LOGRA_ERR_DOMAIN, "%s: eps must be finite and >= 0", name);
  const size_t need = logra::rowadam_ws_bytes(d);
  if (!ws || ws_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", name, need);
  const size_t pneed = P ? logra::packed_update_bytes(d, r) : 0;
  if (P && P_bytes < pneed) return fail(LOGRA_ERR_WORKSPACE, "%s: the packed update needs %zu bytes", name, pneed);
  if (!aligned16(S) || (U && !aligned16(U)) || (P && !aligned16(P)) || !aligned16(v) || !aligned16(ws))
    return fail(LOGRA_ERR_ALIGN, "%s: S, U, v and workspace must be 16-byte aligned", name);
  const Range rs = range(S, (size_t)(d * r) * 4);
  const Range ru = U ? range(U, (size_t)(d * r) * 4) : Range{0, 0};
  const Range rp = P ? range(P, pneed) : Range{0, 0};
  if (U && overlap(rs, ru) && rs.lo != ru.lo) return fail(LOGRA_ERR_ALIAS, "%s: U partially overlaps S", name);
  if (P && (overlap(rp, rs) || overlap(rp, ru))) return fail(LOGRA_ERR_ALIAS, "%s: the packed update overlaps S or U", name);
  const Range rv = range(v, (size_t)d * 4), rw = range(ws, need);
  if (overlap(rv, rs) || overlap(rv, ru) || overlap(rw, rs) || overlap(rw, ru) || overlap(rw, rv) ||
      overlap(rv, rp) || overlap(rw, rp))
    return fail(LOGRA_ERR_ALIAS, "%s: v or workspace overlaps an operand", name);
  return hip_status(logra::launch_rowadam(d, r, S, v, t, beta, eps, U, P, ws, static_cast<hipStream_t>(stream)),
                    "rowadam launch");
}
}  // namespace

LOGRA_API int logra_rowadam(int64_t d, int64_t r, const float* S, float* v, int64_t t,
                            double beta, double eps, float* U, void* ws, size_t ws_bytes,
                            logra_stream stream) {
  LOGRA_TRY
  if (!U) return fail(LOGRA_ERR_NULL, "rowadam: NULL pointer");
  return rowadam_impl("rowadam", d, r, S, v, t, beta, eps, U, nullptr, 0, ws, ws_bytes, stream);
  LOGRA_CATCH("rowadam")
}

LOGRA_API int logra_rowadam_packed(int64_t d, int64_t r, const float* S, float* v, int64_t t,
                                   double beta, double eps, void* U_packed, size_t packed_bytes,
                                   void* ws, size_t ws_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!U_packed) return fail(LOGRA_ERR_NULL, "rowadam_packed: NULL pointer");
  return rowadam_impl("rowadam_packed", d, r, S, v, t, beta, eps, nullptr, U_packed, packed_bytes, ws,
                      ws_bytes, stream);
  LOGRA_CATCH("rowadam_packed")
}

LOGRA_API size_t logra_rowadam_grouped_ws_bytes(int n, int64_t total_rows) {
  if (n < 1 || n > LOGRA_MAX_ROWADAM_GROUP || total_rows < n || total_rows > kMaxElems) return 0;
  return logra::rowadam_grouped_ws_bytes(n, total_rows);
}

LOGRA_API int logra_rowadam_packed_grouped(int64_t r, const logra_rowadam_desc* descs, int n,
                                           int64_t t, double beta, double eps, void* ws,
                                           size_t ws_bytes, logra_stream stream) {
  LOGRA_TRY
  static const char* name = "rowadam_packed_grouped";
  if (!descs || !ws) return fail(LOGRA_ERR_NULL, "%s: NULL pointer", name);
  if (n < 1 || n > LOGRA_MAX_ROWADAM_GROUP) return fail(LOGRA_ERR_SHAPE, "%s: need 1 <= n <= %d", name, LOGRA_MAX_ROWADAM_GROUP);
  if (r < 1 || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "%s: need 1 <= r <= %d", name, LOGRA_MAX_RANK);
  if (t < 1) return fail(LOGRA_ERR_DOMAIN, "%s: t counts updates from 1", name);
  if (!(beta >= 0.0 && beta < 1.0)) return fail(LOGRA_ERR_DOMAIN, "%s: beta must be in [0, 1)", name);
  if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(LOGRA_ERR_DOMAIN, "%s: eps must be finite and >= 0", name);
  if (!aligned16(ws)) return fail(LOGRA_ERR_ALIGN, "%s: workspace not 16-byte aligned", name);
  int64_t rows = 0;
  std::vector<logra::RowAdamItem> items((size_t)n);
  std::vector<Range> ins((size_t)n), outs;
  outs.reserve(2 * (size_t)n + 1);
  for (int i = 0; i < n; ++i) {
    const logra_rowadam_desc& e = descs[i];
    if (!e.S || !e.v || !e.U_packed) return fail(LOGRA_ERR_NULL, "%s: NULL pointer in descriptor %d", name, i);
    if (bad_dim(e.d)) return fail(LOGRA_ERR_SHAPE, "%s: descriptor %d needs d >= 1", name, i);
    const size_t pneed = logra::packed_update_bytes(e.d, r);
    if (e.packed_bytes < pneed) return fail(LOGRA_ERR_WORKSPACE, "%s: descriptor %d: the packed update needs %zu bytes", name, i, pneed);
    if (!aligned16(e.S) || !aligned16(e.v) || !aligned16(e.U_packed))
      return fail(LOGRA_ERR_ALIGN, "%s: descriptor %d: S, v and the packed update must be 16-byte aligned", name, i);
    ins[i] = range(e.S, (size_t)(e.d * r) * 4);
    outs.push_back(range(e.v, (size_t)e.d * 4));
    outs.push_back(range(e.U_packed, pneed));
    items[i] = logra::RowAdamItem{e.S, e.v, e.U_packed, e.d};
    rows += e.d;
  }
  const size_t need = logra::rowadam_grouped_ws_bytes(n, rows);
  if (ws_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", name, need);
  outs.push_back(range(ws, need));
  std::sort(outs.begin(), outs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < outs.size(); ++i)
    if (overlap(outs[i - 1], outs[i])) return fail(LOGRA_ERR_ALIAS, "%s: two outputs (or an output and the workspace) overlap", name);
  // Every output against every sketch: with the sketches sorted by start and
  // the running maximum of their ends, an output [lo, hi) meets a sketch iff
  // some sketch starting before hi ends after lo.
  std::vector<Range> sin = ins;
  std::sort(sin.begin(), sin.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  std::vector<uintptr_t> maxhi(sin.size());
  for (size_t q = 0; q < sin.size(); ++q) maxhi[q] = q ? std::max(maxhi[q - 1], sin[q].hi) : sin[q].hi;
  for (const Range& o : outs) {
    const size_t m = (size_t)(std::lower_bound(sin.begin(), sin.end(), o.hi,
                                               [](const Range& a, uintptr_t x) { return a.lo < x; }) -
                              sin.begin());
    if (m > 0 && maxhi[m - 1] > o.lo)
      return fail(LOGRA_ERR_ALIAS, "%s: an output or the workspace overlaps a sketch", name);
  }
  return hip_status(logra::launch_rowadam_packed_grouped(items.data(), n, r, t, beta, eps, ws,
                                                         static_cast<hipStream_t>(stream)),
                    "rowadam_packed_grouped launch");
  LOGRA_CATCH("rowadam_packed_grouped")
}

LOGRA_API size_t logra_packed_update_bytes(int64_t d, int64_t r) {
  if (bad_dim(d) || bad_rank(r)) return 0;
  return logra::packed_update_bytes(d, r);
}

LOGRA_API int logra_pack_update(int64_t d, int64_t r, const float* U, void* U_packed,
                                size_t packed_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!U || !U_packed) return fail(LOGRA_ERR_NULL, "pack_update: NULL pointer");
  if (bad_dim(d) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "pack_update: need d >= 1, 1 <= r <= %d", LOGRA_MAX_RANK);
  const size_t need = logra::packed_update_bytes(d, r);
  if (packed_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "pack_update: the packed update needs %zu bytes", need);
  if (!aligned16(U_packed)) return fail(LOGRA_ERR_ALIGN, "pack_update: the packed update must be 16-byte aligned");
  if (overlap(range(U, (size_t)(d * r) * 4), range(U_packed, need)))
    return fail(LOGRA_ERR_ALIAS, "pack_update: U overlaps the packed update");
  return hip_status(logra::launch_pack_update(d, r, U, 1.0f, nullptr, U_packed, static_cast<hipStream_t>(stream)),
                    "pack_update launch");
  LOGRA_CATCH("pack_update")
}

LOGRA_API size_t logra_predicted_kl_q_ws_bytes(int64_t P, int64_t V) {
  if (bad_dim(P) || bad_dim(V)) return 0;
  return logra::klq_ws_bytes(P, V);
}

LOGRA_API int logra_predicted_kl_q(int64_t P, int64_t V, const void* z, const void* zdot,
                                   logra_dtype dtype, float tau, float* q_dev, void* ws,
                                   size_t ws_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!z || !zdot || !q_dev) return fail(LOGRA_ERR_NULL, "predicted_kl_q: NULL pointer");
  if (bad_dim(P) || bad_dim(V)) return fail(LOGRA_ERR_SHAPE, "predicted_kl_q: need P, V >= 1");
  if (P > 65535) return fail(LOGRA_ERR_SHAPE, "predicted_kl_q: at most 65535 contexts per call");
  if (dtype != LOGRA_F32 && dtype != LOGRA_BF16) return fail(LOGRA_ERR_DTYPE, "predicted_kl_q: dtype must be F32 or BF16");
  if (!(tau > 0.f) || !std::isfinite(tau)) return fail(LOGRA_ERR_DOMAIN, "predicted_kl_q: tau must be finite and > 0");
  const size_t need = logra::klq_ws_bytes(P, V);
  if (!ws || ws_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "predicted_kl_q: workspace of %zu bytes needed", need);
  if (!aligned16(z) || !aligned16(zdot) || !aligned16(ws)) return fail(LOGRA_ERR_ALIGN, "predicted_kl_q: z, zdot and workspace must be 16-byte aligned");
  return hip_status(logra::launch_predicted_kl_q(P, V, z, zdot, dtype == LOGRA_BF16, tau, q_dev, ws,
                                                 static_cast<hipStream_t>(stream)),
                    "predicted_kl_q launch");
  LOGRA_CATCH("predicted_kl_q")
}

LOGRA_API int logra_predicted_kl_q_noalloc(int64_t P, int64_t V, const void* z, const void* zdot,
                                           logra_dtype dtype, float tau, float* q_dev,
                                           logra_stream stream) {
  LOGRA_TRY
  static_assert(LOGRA_NOALLOC_MAX_CONTEXTS == 4096, "the scratch array's size");
  if (!z || !zdot || !q_dev) return fail(LOGRA_ERR_NULL, "predicted_kl_q_noalloc: NULL pointer");
  if (bad_dim(P) || bad_dim(V)) return fail(LOGRA_ERR_SHAPE, "predicted_kl_q_noalloc: need P, V >= 1");
  if (P > logra::noalloc_max_contexts())
    return fail(LOGRA_ERR_SHAPE, "predicted_kl_q_noalloc: at most %d contexts per call", LOGRA_NOALLOC_MAX_CONTEXTS);
  if (dtype != LOGRA_F32 && dtype != LOGRA_BF16) return fail(LOGRA_ERR_DTYPE, "predicted_kl_q_noalloc: dtype must be F32 or BF16");
  if (!(tau > 0.f) || !std::isfinite(tau)) return fail(LOGRA_ERR_DOMAIN, "predicted_kl_q_noalloc: tau must be finite and > 0");
  if (!aligned16(z) || !aligned16(zdot)) return fail(LOGRA_ERR_ALIGN, "predicted_kl_q_noalloc: z and zdot must be 16-byte aligned");
  return hip_status(logra::launch_predicted_kl_q_noalloc(P, V, z, zdot, dtype == LOGRA_BF16, tau, q_dev,
                                                         static_cast<hipStream_t>(stream)),
                    "predicted_kl_q_noalloc launch");
  LOGRA_CATCH("predicted_kl_q_noalloc")
}

LOGRA_API size_t logra_exact_kl_ws_bytes(int64_t P) {
  if (bad_dim(P)) return 0;
  return logra::exact_kl_ws_bytes(P);
}

LOGRA_API int logra_exact_kl(int64_t P, int64_t V, const void* z, const void* zdot,
                             logra_dtype dtype, double alpha, double tau, double* out_dev,
                             void* ws, size_t ws_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!z || !zdot || !out_dev) return fail(LOGRA_ERR_NULL, "exact_kl: NULL pointer");
  if (bad_dim(P) || bad_dim(V)) return fail(LOGRA_ERR_SHAPE, "exact_kl: need P, V >= 1");
  if (P > 2147483647) return fail(LOGRA_ERR_SHAPE, "exact_kl: too many contexts");
  if (dtype != LOGRA_F32 && dtype != LOGRA_BF16) return fail(LOGRA_ERR_DTYPE, "exact_kl: dtype must be F32 or BF16");
  if (!(tau > 0.0) || !std::isfinite(tau)) return fail(LOGRA_ERR_DOMAIN, "exact_kl: tau must be finite and > 0");
  if (!std::isfinite(alpha)) return fail(LOGRA_ERR_DOMAIN, "exact_kl: alpha must be finite");
  const size_t need = logra::exact_kl_ws_bytes(P);
  if (!ws || ws_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "exact_kl: workspace of %zu bytes needed", need);
  if (!aligned16(ws) || (reinterpret_cast<uintptr_t>(out_dev) & 7u) != 0)
    return fail(LOGRA_ERR_ALIGN, "exact_kl: workspace 16-byte and output 8-byte aligned");
  return hip_status(logra::launch_exact_kl(P, V, z, zdot, dtype == LOGRA_BF16, alpha, tau, out_dev, ws,
                                           static_cast<hipStream_t>(stream)),
                    "exact_kl launch");
  LOGRA_CATCH("exact_kl")
}

LOGRA_API int logra_step_alpha(double q, double delta, double alpha_max, double* alpha) {
  LOGRA_TRY
  if (!alpha) return fail(LOGRA_ERR_NULL, "step_alpha: NULL output");
  if (!(delta > 0.0) || !(alpha_max > 0.0)) return fail(LOGRA_ERR_DOMAIN, "step_alpha: delta and alpha_max must be > 0");
  if (std::isnan(q) || q < 0.0) return fail(LOGRA_ERR_DOMAIN, "step_alpha: q must be >= 0");
  *alpha = q == 0.0 ? alpha_max : std::fmin(alpha_max, std::sqrt(delta / q));
  return ok();
  LOGRA_CATCH("step_alpha")
}

LOGRA_API int logra_kl_budget(int64_t u, int64_t H, double delta_max, double delta_min,
                              double* delta_u) {
  LOGRA_TRY
  if (!delta_u) return fail(LOGRA_ERR_NULL, "kl_budget: NULL output");
  if (u < 1 || H < 2) return fail(LOGRA_ERR_DOMAIN, "kl_budget: need u >= 1 and H >= 2");
  if (!std::isfinite(delta_max) || !std::isfinite(delta_min) || delta_min < 0.0 || delta_max < delta_min)
    return fail(LOGRA_ERR_DOMAIN, "kl_budget: need 0 <= delta_min <= delta_max, finite");
  if (u >= H) {
    *delta_u = delta_min;
    return ok();
  }
  const double pi = 3.14159265358979323846;
  *delta_u = delta_min + 0.5 * (delta_max - delta_min) *
                             (1.0 + std::cos(pi * (double)(u - 1) / (double)(H - 1)));
  return ok();
  LOGRA_CATCH("kl_budget")
}

LOGRA_API int logra_mismatch_update(logra_mismatch_state* state, double measurement, double weight) {
  LOGRA_TRY
  if (!state) return fail(LOGRA_ERR_NULL, "mismatch_update: NULL state");
  if (!(weight > 0.0 && weight <= 1.0)) return fail(LOGRA_ERR_DOMAIN, "mismatch_update: weight must be in (0, 1]");
  if (std::isinf(measurement)) return fail(LOGRA_ERR_DOMAIN, "mismatch_update: infinite measurement");
  if (std::isnan(measurement)) return ok();  // no valid measurement this update
  const double k = state->valid ? weight * measurement + (1.0 - weight) * state->kappa : measurement;
  state->kappa = k > 0.0 ? k : 0.0;
  state->valid = 1;
  return ok();
  LOGRA_CATCH("mismatch_update")
}

LOGRA_API int logra_effective_budget(double delta_u, const logra_mismatch_state* state,
                                     double* delta_eff) {
  LOGRA_TRY
  if (!state || !delta_eff) return fail(LOGRA_ERR_NULL, "effective_budget: NULL pointer");
  if (!(delta_u >= 0.0) || !std::isfinite(delta_u)) return fail(LOGRA_ERR_DOMAIN, "effective_budget: delta_u must be finite and >= 0");
  if (!state->valid) {
    *delta_eff = delta_u;
    return ok();
  }
  const double sub = delta_u - state->kappa;
  const double floor = 0.5 * delta_u;
  *delta_eff = sub > floor ? sub : floor;
  return ok();
  LOGRA_CATCH("effective_budget")
}

LOGRA_API int logra_step_alpha_dev(const float* q_dev, float delta, float alpha_max,
                                   float* alpha_dev, logra_stream stream) {
  LOGRA_TRY
  if (!q_dev || !alpha_dev) return fail(LOGRA_ERR_NULL, "step_alpha_dev: NULL pointer");
  if (!(delta > 0.f) || !(alpha_max > 0.f)) return fail(LOGRA_ERR_DOMAIN, "step_alpha_dev: delta and alpha_max must be > 0");
  return hip_status(logra::launch_step_alpha(q_dev, delta, alpha_max, alpha_dev, static_cast<hipStream_t>(stream)),
                    "step_alpha_dev launch");
  LOGRA_CATCH("step_alpha_dev")
}

namespace {
// One matrix of a grouped merge, U as fp32 or packed.
struct MergeOperands {
  const logra_key* key;
  void* W;
  int64_t d, k, ldw;
  const void* U;
  int64_t row0;
  const void* A = nullptr;  // explicit projection (merge operand order), or null
  size_t U_bytes = 0;       // bytes available at a packed U (unused for fp32 U)
  size_t A_bytes = 0;       // bytes available at A
};
int merge_grouped_impl(const char* name, int64_t r, const MergeOperands* ops, int n, double scale,
                       const float* scale_dev, logra_round mode, uint64_t sr_seed, bool packed,
                       logra_stream stream) {
  if (n < 1 || n > LOGRA_MAX_GROUP) return fail(LOGRA_ERR_SHAPE, "%s: need 1 <= n <= %d", name, LOGRA_MAX_GROUP);
  if (bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "%s: need 1 <= r <= %d", name, LOGRA_MAX_RANK);
  if (mode != LOGRA_ROUND_NEAREST && mode != LOGRA_ROUND_STOCHASTIC) return fail(LOGRA_ERR_DOMAIN, "%s: unknown rounding mode", name);
  if (!std::isfinite(scale)) return fail(LOGRA_ERR_DOMAIN, "%s: scale must be finite", name);
  auto u_range = [&](const MergeOperands& e) {
    return range(e.U, packed ? logra::packed_update_bytes(e.d, r) : (size_t)(e.d * r) * 4);
  };
  logra::MergeItem items[LOGRA_MAX_GROUP];
  for (int i = 0; i < n; ++i) {
    const MergeOperands& e = ops[i];
    if (!e.W || !e.U) return fail(LOGRA_ERR_NULL, "%s: NULL pointer in descriptor %d", name, i);
    if (bad_dim(e.d) || bad_dim(e.k) || e.row0 < 0 || e.row0 > kMaxElems) return fail(LOGRA_ERR_SHAPE, "%s: need d, k >= 1 and row0 >= 0", name);
    int st = check_matrix("merge_grouped W", e.W, LOGRA_BF16, e.ldw, e.d, e.k);
    if (st) return st;
    if (!aligned16(e.U)) return fail(LOGRA_ERR_ALIGN, "%s: U not 16-byte aligned", name);
    if (packed && e.U_bytes < logra::packed_update_bytes(e.d, r))
      return fail(LOGRA_ERR_WORKSPACE, "%s: descriptor %d: the packed update needs %zu bytes", name, i,
                  logra::packed_update_bytes(e.d, r));
    const Range rw = range(e.W, extent(e.d, e.k, e.ldw, 2));
    if (scale_dev && overlap(rw, range(scale_dev, 4))) return fail(LOGRA_ERR_ALIAS, "%s: W overlaps the device scale", name);
    for (int j = 0; j <= i; ++j) {
      if (overlap(rw, u_range(ops[j])) ||
          (j < i && overlap(rw, range(ops[j].W, extent(ops[j].d, ops[j].k, ops[j].ldw, 2)))))
        return fail(LOGRA_ERR_ALIAS, "%s: W of descriptor %d overlaps an operand of %d", name, i, j);
      if (j < i && overlap(u_range(e), range(ops[j].W, extent(ops[j].d, ops[j].k, ops[j].ldw, 2))))
        return fail(LOGRA_ERR_ALIAS, "%s: U of descriptor %d overlaps W of %d", name, i, j);
    }
    if ((e.A != nullptr) != (ops[0].A != nullptr))
      return fail(LOGRA_ERR_NULL, "%s: explicit projections for all descriptors or none", name);
    if (e.A) {
      if (e.A_bytes < logra::merge_projection_packed_bytes(r, e.k))
        return fail(LOGRA_ERR_WORKSPACE, "%s: descriptor %d: the packed projection needs %zu bytes", name, i,
                    logra::merge_projection_packed_bytes(r, e.k));
      const Range ra = range(e.A, logra::merge_projection_packed_bytes(r, e.k));
      if (!aligned16(e.A)) return fail(LOGRA_ERR_ALIGN, "%s: projection %d not 16-byte aligned", name, i);
      for (int j = 0; j <= i; ++j)
        if (overlap(ra, range(ops[j].W, extent(ops[j].d, ops[j].k, ops[j].ldw, 2))))
          return fail(LOGRA_ERR_ALIAS, "%s: projection %d overlaps a W", name, i);
    }
    items[i] = logra::MergeItem{key_words(e.key->seed, e.key), key_words(sr_seed, e.key), e.W, e.d, e.k,
                                e.ldw, e.U, e.row0, e.A};
  }
  return hip_status(logra::launch_merge_grouped(items, n, r, scale, scale_dev, mode == LOGRA_ROUND_STOCHASTIC,
                                                packed, static_cast<hipStream_t>(stream)),
                    "merge_grouped launch");
}
}  // namespace

LOGRA_API int logra_merge_grouped(int64_t r, const logra_merge_desc* descs, int n, double scale,
                                  const float* scale_dev, logra_round mode, uint64_t sr_seed,
                                  logra_stream stream) {
  LOGRA_TRY
  if (!descs) return fail(LOGRA_ERR_NULL, "merge_grouped: NULL descriptors");
  if (n < 1 || n > LOGRA_MAX_GROUP) return fail(LOGRA_ERR_SHAPE, "merge_grouped: need 1 <= n <= %d", LOGRA_MAX_GROUP);
  MergeOperands ops[LOGRA_MAX_GROUP];
  for (int i = 0; i < n; ++i)
    ops[i] = MergeOperands{&descs[i].key, descs[i].W, descs[i].d, descs[i].k, descs[i].ldw, descs[i].U,
                           descs[i].row0};
  return merge_grouped_impl("merge_grouped", r, ops, n, scale, scale_dev, mode, sr_seed, false, stream);
  LOGRA_CATCH("merge_grouped")
}

LOGRA_API int logra_merge_grouped_packed(int64_t r, const logra_merge_packed_desc* descs, int n,
                                         double scale, const float* scale_dev, logra_round mode,
                                         uint64_t sr_seed, logra_stream stream) {
  LOGRA_TRY
  if (!descs) return fail(LOGRA_ERR_NULL, "merge_grouped_packed: NULL descriptors");
  if (n < 1 || n > LOGRA_MAX_GROUP)
    return fail(LOGRA_ERR_SHAPE, "merge_grouped_packed: need 1 <= n <= %d", LOGRA_MAX_GROUP);
  MergeOperands ops[LOGRA_MAX_GROUP];
  for (int i = 0; i < n; ++i)
    ops[i] = MergeOperands{&descs[i].key, descs[i].W, descs[i].d, descs[i].k, descs[i].ldw,
                           descs[i].U_packed, descs[i].row0, nullptr, descs[i].packed_bytes};
  return merge_grouped_impl("merge_grouped_packed", r, ops, n, scale, scale_dev, mode, sr_seed, true,
                            stream);
  LOGRA_CATCH("merge_grouped_packed")
}

LOGRA_API size_t logra_merge_projection_packed_bytes(int64_t r, int64_t k) {
  if (bad_dim(k) || bad_rank(r)) return 0;
  return logra::merge_projection_packed_bytes(r, k);
}

LOGRA_API int logra_pack_merge_projection(int64_t r, int64_t k, const float* A, void* A_packed,
                                          size_t packed_bytes, logra_stream stream) {
  LOGRA_TRY
  if (!A || !A_packed) return fail(LOGRA_ERR_NULL, "pack_merge_projection: NULL pointer");
  if (bad_dim(k) || bad_rank(r)) return fail(LOGRA_ERR_SHAPE, "pack_merge_projection: need k >= 1 and 1 <= r <= %d", LOGRA_MAX_RANK);
  const size_t need = logra::merge_projection_packed_bytes(r, k);
  if (packed_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "pack_merge_projection: %zu bytes needed", need);
  if (!aligned16(A_packed)) return fail(LOGRA_ERR_ALIGN, "pack_merge_projection: output not 16-byte aligned");
  if (overlap(range(A, (size_t)(r * k) * 4), range(A_packed, need)))
    return fail(LOGRA_ERR_ALIAS, "pack_merge_projection: A overlaps the packed output");
  return hip_status(logra::launch_pack_merge_projection(r, k, A, A_packed, static_cast<hipStream_t>(stream)),
                    "pack_merge_projection launch");
  LOGRA_CATCH("pack_merge_projection")
}

LOGRA_API int logra_merge_grouped_explicit(int64_t r, const logra_merge_explicit_desc* descs, int n,
                                           double scale, const float* scale_dev, logra_round mode,
                                           uint64_t sr_seed, logra_stream stream) {
  LOGRA_TRY
  if (!descs) return fail(LOGRA_ERR_NULL, "merge_grouped_explicit: NULL descriptors");
  if (n < 1 || n > LOGRA_MAX_GROUP)
    return fail(LOGRA_ERR_SHAPE, "merge_grouped_explicit: need 1 <= n <= %d", LOGRA_MAX_GROUP);
  MergeOperands ops[LOGRA_MAX_GROUP];
  for (int i = 0; i < n; ++i) {
    if (!descs[i].A_packed) return fail(LOGRA_ERR_NULL, "merge_grouped_explicit: NULL projection in descriptor %d", i);
    ops[i] = MergeOperands{&descs[i].key, descs[i].W, descs[i].d, descs[i].k, descs[i].ldw,
                           descs[i].U_packed, descs[i].row0, descs[i].A_packed, descs[i].packed_bytes,
                           descs[i].A_packed_bytes};
  }
  return merge_grouped_impl("merge_grouped_explicit", r, ops, n, scale, scale_dev, mode, sr_seed, true,
                            stream);
  LOGRA_CATCH("merge_grouped_explicit")
}

LOGRA_API int logra_sync_pack(const logra_key* key, int64_t d, int64_t k, int64_t r,
                              const float* U, double scale, const float* scale_dev,
                              logra_round mode, uint64_t sr_seed, int64_t row0,
                              logra_sync_header* header, void* payload, size_t payload_bytes,
                              logra_stream stream) {
  LOGRA_TRY
  if (!key || !U || !header || !payload) return fail(LOGRA_ERR_NULL, "sync_pack: NULL pointer");
  if (bad_dim(d) || bad_dim(k) || bad_rank(r) || row0 < 0 || row0 > kMaxElems)
    return fail(LOGRA_ERR_SHAPE, "sync_pack: need d, k >= 1, 1 <= r <= %d, row0 >= 0", LOGRA_MAX_RANK);
  if (mode != LOGRA_ROUND_NEAREST && mode != LOGRA_ROUND_STOCHASTIC) return fail(LOGRA_ERR_DOMAIN, "sync_pack: unknown rounding mode");
  if (!std::isfinite(scale)) return fail(LOGRA_ERR_DOMAIN, "sync_pack: scale must be finite");
  const size_t need = logra::packed_update_bytes(d, r);
  if (payload_bytes < need) return fail(LOGRA_ERR_WORKSPACE, "sync_pack: the payload needs %zu bytes", need);
  if (!aligned16(payload)) return fail(LOGRA_ERR_ALIGN, "sync_pack: payload must be 16-byte aligned");
  if (overlap(range(U, (size_t)(d * r) * 4), range(payload, need)))
    return fail(LOGRA_ERR_ALIAS, "sync_pack: U overlaps the payload");
  header->magic = LOGRA_SYNC_MAGIC;
  header->version = LOGRA_SYNC_VERSION;
  header->key = *key;
  header->d = d;
  header->k = k;
  header->r = r;
  header->mode = (int32_t)mode;
  header->reserved = 0;
  header->sr_seed = sr_seed;
  header->row0 = row0;
  header->payload_bytes = need;
  return hip_status(logra::launch_pack_update(d, r, U, (float)scale, scale_dev, payload,
                                              static_cast<hipStream_t>(stream)),
                    "sync_pack launch");
  LOGRA_CATCH("sync_pack")
}

LOGRA_API int logra_sync_apply(const logra_sync_desc* descs, int n, logra_stream stream) {
  LOGRA_TRY
  if (!descs) return fail(LOGRA_ERR_NULL, "sync_apply: NULL descriptors");
  if (n < 1 || n > LOGRA_MAX_GROUP) return fail(LOGRA_ERR_SHAPE, "sync_apply: need 1 <= n <= %d", LOGRA_MAX_GROUP);
  MergeOperands ops[LOGRA_MAX_GROUP];
  for (int i = 0; i < n; ++i) {
    const logra_sync_header* h = descs[i].header;
    if (!h || !descs[i].payload || !descs[i].W) return fail(LOGRA_ERR_NULL, "sync_apply: NULL pointer in descriptor %d", i);
    if (h->magic != LOGRA_SYNC_MAGIC || h->version != LOGRA_SYNC_VERSION)
      return fail(LOGRA_ERR_DOMAIN, "sync_apply: descriptor %d has no valid header", i);
    if (bad_dim(h->d) || bad_dim(h->k) || bad_rank(h->r) || h->payload_bytes != logra::packed_update_bytes(h->d, h->r))
      return fail(LOGRA_ERR_DOMAIN, "sync_apply: header %d sizes are inconsistent", i);
    if (h->r != descs[0].header->r || h->mode != descs[0].header->mode || h->sr_seed != descs[0].header->sr_seed)
      return fail(LOGRA_ERR_SHAPE, "sync_apply: descriptors must share r, mode and sr_seed");
    ops[i] = MergeOperands{&h->key, descs[i].W, h->d, h->k, descs[i].ldw, descs[i].payload, h->row0, nullptr,
                           (size_t)h->payload_bytes};
  }
  const logra_sync_header* h0 = descs[0].header;
  return merge_grouped_impl("sync_apply", h0->r, ops, n, 1.0, nullptr, (logra_round)h0->mode, h0->sr_seed,
                            true, stream);
  LOGRA_CATCH("sync_apply")
}

LOGRA_API int logra_merge(const logra_key* key, int64_t d, int64_t k, int64_t r, void* W,
                          logra_dtype w_dtype, int64_t ldw, const float* U, double scale,
                          const float* scale_dev, logra_round mode, uint64_t sr_seed,
                          int64_t row0, logra_stream stream) {
  LOGRA_TRY
  if (!key || !W || !U) return fail(LOGRA_ERR_NULL, "merge: NULL pointer");
  if (bad_dim(d) || bad_dim(k) || bad_rank(r) || row0 < 0 || row0 > kMaxElems) return fail(LOGRA_ERR_SHAPE, "merge: need d, k >= 1, 1 <= r <= %d, row0 >= 0", LOGRA_MAX_RANK);
  int st = check_matrix("merge W", W, w_dtype, ldw, d, k);
  if (st) return st;
  if (mode != LOGRA_ROUND_NEAREST && mode != LOGRA_ROUND_STOCHASTIC) return fail(LOGRA_ERR_DOMAIN, "merge: unknown rounding mode");
  if (w_dtype == LOGRA_F32 && mode == LOGRA_ROUND_STOCHASTIC)
    return fail(LOGRA_ERR_DTYPE, "merge: stochastic rounding is defined for bf16 weights only");
  if (!std::isfinite(scale)) return fail(LOGRA_ERR_DOMAIN, "merge: scale must be finite");
  if (!aligned16(U)) return fail(LOGRA_ERR_ALIGN, "merge: U not 16-byte aligned");
  const Range rw = range(W, extent(d, k, ldw, elem_size(w_dtype)));
  if (overlap(rw, range(U, (size_t)(d * r) * 4))) return fail(LOGRA_ERR_ALIAS, "merge: W overlaps U");
  if (scale_dev && overlap(rw, range(scale_dev, 4))) return fail(LOGRA_ERR_ALIAS, "merge: W overlaps the device scale");
  return hip_status(logra::launch_merge(key_words(key->seed, key), d, k, r, W, w_dtype == LOGRA_BF16, ldw, U,
                                        scale, scale_dev, mode == LOGRA_ROUND_STOCHASTIC,
                                        key_words(sr_seed, key), row0, static_cast<hipStream_t>(stream)),
                    "merge launch");
  LOGRA_CATCH("merge")
}

LOGRA_API int logra_bandwidth_probe(logra_probe mode, const void* src, void* dst, size_t bytes,
                                    int blocks_per_cu, logra_stream stream) {
  LOGRA_TRY
  if (!src || !dst) return fail(LOGRA_ERR_NULL, "bandwidth_probe: NULL pointer");
  if (mode != LOGRA_PROBE_READ && mode != LOGRA_PROBE_COPY) return fail(LOGRA_ERR_DOMAIN, "bandwidth_probe: unknown mode");
  if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 50))
    return fail(LOGRA_ERR_SHAPE, "bandwidth_probe: bytes must be a positive multiple of 16, at most 2^50");
  if (blocks_per_cu < 1 || blocks_per_cu > 32) return fail(LOGRA_ERR_SHAPE, "bandwidth_probe: need 1 <= blocks_per_cu <= 32");
  if (!aligned16(src) || !aligned16(dst)) return fail(LOGRA_ERR_ALIGN, "bandwidth_probe: src and dst must be 16-byte aligned");
  const size_t dbytes = mode == LOGRA_PROBE_COPY ? bytes : 4096;
  if (overlap(range(src, bytes), range(dst, dbytes))) return fail(LOGRA_ERR_ALIAS, "bandwidth_probe: src and dst overlap");
  return hip_status(logra::launch_probe(mode == LOGRA_PROBE_COPY, src, dst, (int64_t)bytes, blocks_per_cu,
                                        static_cast<hipStream_t>(stream)),
                    "bandwidth_probe launch");
  LOGRA_CATCH("bandwidth_probe")
}

}  // extern "C"
