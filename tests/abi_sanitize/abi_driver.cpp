// Host-side check of the C ABI of liblogra under AddressSanitizer and
// UndefinedBehaviorSanitizer.
//
// Built host-only (no device code) together with the library's sources, then
// run on a machine with no GPU visible: every call below either fails
// validation (the expected status is checked) or reaches the HIP runtime,
// which reports that no device is available.  No kernel can run.  What the
// sanitizers watch is the host code: argument validation, overlap checks,
// descriptor tables and the error path.  The global operator new is replaced
// by one that can be told to throw std::bad_alloc, to check that the entry
// points turn host exceptions into LOGRA_ERR_HOST instead of letting them
// cross the C ABI.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "logra.h"

namespace {
long g_throw_in = -1;  // allocations left before operator new throws; -1: never
int g_failures = 0;
int g_checks = 0;

void check(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, logra_last_error());
  }
}
#define EXPECT_STATUS(call, want)                                                     \
  do {                                                                                \
    const int st_ = (call);                                                           \
    check(st_ == (want), #call " -> " #want, __LINE__);                               \
    if (st_ != (want)) std::fprintf(stderr, "  got status %d\n", st_);                \
  } while (0)
#define EXPECT_NOT_OK(call) check((call) != LOGRA_OK, #call " fails", __LINE__)

// Fake device addresses, 16-byte aligned, far apart: validation never
// dereferences device pointers.
char* const A = reinterpret_cast<char*>(uintptr_t(0x10000000));
char* const B = reinterpret_cast<char*>(uintptr_t(0x20000000));
char* const C = reinterpret_cast<char*>(uintptr_t(0x30000000));
char* const D = reinterpret_cast<char*>(uintptr_t(0x40000000));
char* const E = reinterpret_cast<char*>(uintptr_t(0x50000000));
const int64_t kHuge = int64_t(1) << 62;
}  // namespace

void* operator new(std::size_t n) {
  if (g_throw_in == 0) {
    g_throw_in = -1;
    throw std::bad_alloc();
  }
  if (g_throw_in > 0) --g_throw_in;
  if (void* p = std::malloc(n ? n : 1)) return p;
  throw std::bad_alloc();
}
void* operator new[](std::size_t n) { return ::operator new(n); }
void operator delete(void* p) noexcept { std::free(p); }
void operator delete[](void* p) noexcept { std::free(p); }
void operator delete(void* p, std::size_t) noexcept { std::free(p); }
void operator delete[](void* p, std::size_t) noexcept { std::free(p); }
// The non-throwing forms too, so every allocation and release pairs malloc with free.
void* operator new(std::size_t n, const std::nothrow_t&) noexcept { return std::malloc(n ? n : 1); }
void* operator new[](std::size_t n, const std::nothrow_t&) noexcept { return std::malloc(n ? n : 1); }
void operator delete(void* p, const std::nothrow_t&) noexcept { std::free(p); }
void operator delete[](void* p, const std::nothrow_t&) noexcept { std::free(p); }

static void sizes_and_scalars() {
  check(logra_sketch_bytes(4096, 64) == (int64_t(1) << 20), "sketch bytes 1 MiB", __LINE__);
  check(logra_sketch_bytes(-1, 1) == -1, "negative size", __LINE__);
  check(logra_packed_input_bytes(kHuge, 64) == 0, "huge T", __LINE__);
  check(logra_packed_update_bytes(kHuge, 64) == 0, "huge d", __LINE__);
  check(logra_projection_packed_bytes(64, kHuge) == 0, "huge k", __LINE__);
  check(logra_merge_projection_packed_bytes(64, kHuge) == 0, "huge k (merge)", __LINE__);
  check(logra_reconstruction_cosine_ws_bytes(kHuge, kHuge, 8) == 0, "huge cosine", __LINE__);
  check(logra_rowadam_grouped_ws_bytes(4, kHuge) == 0, "huge rows", __LINE__);
  check(logra_predicted_kl_q_ws_bytes(kHuge, kHuge) == 0, "huge contexts", __LINE__);
  double a = 0;
  EXPECT_STATUS(logra_step_alpha(8e-3, 2e-3, 4.0, &a), LOGRA_OK);
  check(a == 0.5, "alpha = 1/2 at q = 4 delta", __LINE__);
  EXPECT_STATUS(logra_step_alpha(-1.0, 2e-3, 4.0, &a), LOGRA_ERR_DOMAIN);
  EXPECT_STATUS(logra_step_alpha(1.0, 2e-3, 4.0, nullptr), LOGRA_ERR_NULL);
  EXPECT_STATUS(logra_kl_budget(1, 1, 1.0, 0.5, &a), LOGRA_ERR_DOMAIN);
  EXPECT_STATUS(logra_kl_budget(3, 300, 2e-4, 2e-5, &a), LOGRA_OK);
  logra_mismatch_state ms{};
  EXPECT_STATUS(logra_mismatch_update(&ms, 1e-5, 0.3), LOGRA_OK);
  EXPECT_STATUS(logra_mismatch_update(&ms, 1.0 / 0.0, 0.3), LOGRA_ERR_DOMAIN);
  EXPECT_STATUS(logra_effective_budget(1e-4, &ms, &a), LOGRA_OK);
  // a long message is cut to the buffer, not written past it
  std::vector<logra_project_desc> many(2000);
  EXPECT_STATUS(logra_project_input_table(64, 64, many.data(), 2000, A, 1 << 30, nullptr), LOGRA_ERR_SHAPE);
  check(std::strlen(logra_last_error()) < 512, "message length", __LINE__);
}

static void out_of_range_sizes() {
  const logra_key key{1, 2, 3};
  // extents that would overflow 64-bit arithmetic are rejected as shapes
  EXPECT_STATUS(logra_project_input(&key, kHuge, 64, 8, A, LOGRA_BF16, 64, reinterpret_cast<float*>(B), nullptr),
                LOGRA_ERR_SHAPE);
  EXPECT_STATUS(logra_project_input(&key, 1 << 20, 1 << 20, 8, A, LOGRA_BF16, kHuge, reinterpret_cast<float*>(B),
                                    nullptr),
                LOGRA_ERR_SHAPE);
  EXPECT_STATUS(logra_merge(&key, kHuge, kHuge, 8, A, LOGRA_BF16, kHuge, reinterpret_cast<float*>(B), 1.0, nullptr,
                            LOGRA_ROUND_NEAREST, 0, 0, nullptr),
                LOGRA_ERR_SHAPE);
  EXPECT_STATUS(logra_merge(&key, 64, 64, 8, A, LOGRA_BF16, 64, reinterpret_cast<float*>(B), 1.0, nullptr,
                            LOGRA_ROUND_NEAREST, 0, kHuge, nullptr),
                LOGRA_ERR_SHAPE);
  std::vector<char> ws(1 << 12);
  EXPECT_STATUS(logra_rowadam(kHuge, kHuge, reinterpret_cast<float*>(A), reinterpret_cast<float*>(B), 1, 0.9, 1e-8,
                              reinterpret_cast<float*>(C), D, 1 << 20, nullptr),
                LOGRA_ERR_SHAPE);
  EXPECT_STATUS(logra_sketch_accumulate(kHuge, 64, 64, A, LOGRA_BF16, 64, reinterpret_cast<float*>(B),
                                        reinterpret_cast<float*>(C), D, 1 << 20, nullptr),
                LOGRA_ERR_SHAPE);
  logra_acc_packed_desc pd{A, reinterpret_cast<const uint16_t*>(B), reinterpret_cast<float*>(C), kHuge, kHuge,
                           size_t(1) << 40};
  EXPECT_STATUS(logra_sketch_accumulate_table(4096, 64, &pd, 1, D, 1 << 20, nullptr), LOGRA_ERR_SHAPE);
  EXPECT_STATUS(logra_predicted_kl_q(kHuge, kHuge, A, B, LOGRA_BF16, 1.0f, reinterpret_cast<float*>(C), D, 1 << 20,
                                     nullptr),
                LOGRA_ERR_SHAPE);
  EXPECT_STATUS(logra_regen_A(&key, 8, kHuge, LOGRA_I8, A, nullptr), LOGRA_ERR_SHAPE);
  EXPECT_STATUS(logra_sync_pack(&key, kHuge, 64, 8, reinterpret_cast<float*>(A), 1.0, nullptr, LOGRA_ROUND_NEAREST,
                                0, 0, nullptr, B, 1 << 20, nullptr),
                LOGRA_ERR_NULL);
}

static void tables_and_validation() {
  const logra_key key{1, 2, 3};
  const int64_t T = 128, r = 64;
  const size_t pin = logra_packed_input_bytes(T, r);
  // accumulate table: valid descriptors, an overlap, a short packed input
  std::vector<logra_acc_packed_desc> acc;
  for (int i = 0; i < 40; ++i)
    acc.push_back(logra_acc_packed_desc{A + (size_t)i * 0x100000, reinterpret_cast<const uint16_t*>(B),
                                        reinterpret_cast<float*>(C + (size_t)i * 0x10000), 64, 64, pin});
  const size_t aws = logra_sketch_accumulate_table_ws_bytes(40);
  EXPECT_NOT_OK(logra_sketch_accumulate_table(T, r, acc.data(), 40, E, aws, nullptr));  // no device: HIP error
  acc[7].S = acc[8].S;
  EXPECT_STATUS(logra_sketch_accumulate_table(T, r, acc.data(), 40, E, aws, nullptr), LOGRA_ERR_ALIAS);
  acc[7].S = reinterpret_cast<float*>(C + 7 * 0x10000);
  acc[39].planes_bytes = pin - 16;
  EXPECT_STATUS(logra_sketch_accumulate_table(T, r, acc.data(), 40, E, aws, nullptr), LOGRA_ERR_WORKSPACE);
  EXPECT_STATUS(logra_sketch_accumulate_grouped_packed(T, r, acc.data() + 39, 1, nullptr), LOGRA_ERR_WORKSPACE);
  // projection table: shared inputs, then an output inside an input
  std::vector<logra_project_desc> pr;
  for (int i = 0; i < 30; ++i)
    pr.push_back(logra_project_desc{key, A + (size_t)(i / 3) * 0x100000, 256, 256, nullptr,
                                    B + (size_t)i * 0x100000, pin});
  const size_t pws = logra_project_input_table_ws_bytes(30);
  EXPECT_NOT_OK(logra_project_input_table(T, r, pr.data(), 30, E, pws, nullptr));
  pr[4].planes = A + 0x100000 + 64;
  EXPECT_STATUS(logra_project_input_table(T, r, pr.data(), 30, E, pws, nullptr), LOGRA_ERR_ALIAS);
  pr[4].planes = B + 4 * 0x100000;
  // grouped RowAdam: valid, then an output inside a sketch
  const size_t pup = logra_packed_update_bytes(64, r);
  std::vector<logra_rowadam_desc> ra;
  for (int i = 0; i < 20; ++i)
    ra.push_back(logra_rowadam_desc{reinterpret_cast<const float*>(A + (size_t)i * 0x10000),
                                    reinterpret_cast<float*>(B + (size_t)i * 0x1000), C + (size_t)i * 0x10000, pup,
                                    64});
  const size_t rws = logra_rowadam_grouped_ws_bytes(20, 20 * 64);
  EXPECT_NOT_OK(logra_rowadam_packed_grouped(r, ra.data(), 20, 1, 0.95, 1e-8, E, rws, nullptr));
  ra[3].U_packed = A + 0x10000 + 256;
  EXPECT_STATUS(logra_rowadam_packed_grouped(r, ra.data(), 20, 1, 0.95, 1e-8, E, rws, nullptr), LOGRA_ERR_ALIAS);
  // merges: packed update sizes, explicit projection sizes, sync headers
  logra_merge_packed_desc mp{key, A, 64, 64, 64, B, 0, pup};
  EXPECT_NOT_OK(logra_merge_grouped_packed(r, &mp, 1, 1.0, nullptr, LOGRA_ROUND_STOCHASTIC, 2, nullptr));
  mp.packed_bytes = pup - 1;
  EXPECT_STATUS(logra_merge_grouped_packed(r, &mp, 1, 1.0, nullptr, LOGRA_ROUND_NEAREST, 0, nullptr),
                LOGRA_ERR_WORKSPACE);
  logra_merge_explicit_desc me{key, A, 64, 64, 64, B, C, 0, pup, 16};
  EXPECT_STATUS(logra_merge_grouped_explicit(r, &me, 1, 1.0, nullptr, LOGRA_ROUND_NEAREST, 0, nullptr),
                LOGRA_ERR_WORKSPACE);
  logra_sync_header h{};
  EXPECT_NOT_OK(logra_sync_pack(&key, 64, 64, r, reinterpret_cast<const float*>(A), 1e-3, nullptr,
                                LOGRA_ROUND_NEAREST, 0, 0, &h, B, pup, nullptr));
  check(h.magic == LOGRA_SYNC_MAGIC && h.payload_bytes == pup, "header filled", __LINE__);
  logra_sync_desc sd{&h, B, A, 64};
  EXPECT_NOT_OK(logra_sync_apply(&sd, 1, nullptr));
  h.payload_bytes = 16;
  EXPECT_STATUS(logra_sync_apply(&sd, 1, nullptr), LOGRA_ERR_DOMAIN);
}

static void exceptions_stay_inside() {
  // The first host allocation inside each call throws std::bad_alloc; the call must
  // return LOGRA_ERR_HOST with a message instead of letting it escape.
  const logra_key key{1, 2, 3};
  const size_t pin = logra_packed_input_bytes(128, 64);
  logra_acc_packed_desc acc{A, reinterpret_cast<const uint16_t*>(B), reinterpret_cast<float*>(C), 64, 64, pin};
  g_throw_in = 0;
  EXPECT_STATUS(logra_sketch_accumulate_table(128, 64, &acc, 1, E, logra_sketch_accumulate_table_ws_bytes(1), nullptr),
                LOGRA_ERR_HOST);
  check(std::strstr(logra_last_error(), "out of host memory") != nullptr, "bad_alloc message", __LINE__);
  logra_project_desc pd{key, A, 256, 256, nullptr, B, pin};
  g_throw_in = 0;
  EXPECT_STATUS(logra_project_input_table(128, 64, &pd, 1, E, logra_project_input_table_ws_bytes(1), nullptr),
                LOGRA_ERR_HOST);
  logra_rowadam_desc rd{reinterpret_cast<const float*>(A), reinterpret_cast<float*>(B), C,
                        logra_packed_update_bytes(64, 64), 64};
  g_throw_in = 0;
  EXPECT_STATUS(logra_rowadam_packed_grouped(64, &rd, 1, 1, 0.95, 1e-8, E, logra_rowadam_grouped_ws_bytes(1, 64),
                                             nullptr),
                LOGRA_ERR_HOST);
  g_throw_in = -1;
  // later calls work normally
  double a = 0;
  EXPECT_STATUS(logra_step_alpha(8e-3, 2e-3, 4.0, &a), LOGRA_OK);
  check(logra_last_error()[0] == '\0', "error cleared by a successful call", __LINE__);
}

int main() {
  std::printf("%s\n", logra_version());
  sizes_and_scalars();
  out_of_range_sizes();
  tables_and_validation();
  exceptions_stay_inside();
  std::printf("%d checks, %d failed\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
