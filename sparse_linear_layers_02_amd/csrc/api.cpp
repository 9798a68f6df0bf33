// Host side of the C ABI declared in include/sbn.h: argument validation,
// workspace sizing, dispatch to the HIP launchers and error reporting.
// Validation runs entirely on the host before any HIP call, so a rejected
// call launches nothing and touches no output.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "sbn_internal.h"

using namespace sbn;

namespace {

thread_local char g_last_error[512] = "";

sbn_status fail(sbn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

sbn_status ok() {
  g_last_error[0] = '\0';
  return SBN_OK;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("SBN_DEBUG_SYNC");
    return e && e[0] == '1';
  }();
  return on;
}

// SBN_CHECK_FINITE=1: entry points scan their floating-point inputs for
// NaN / Inf first (read on every call, so a process can switch it).  Skipped
// while the stream is being captured: the scan reads a flag back to the host.
sbn_status check_finite(const char* fn, const char* what, const void* x, int64_t rows, int64_t cols, int64_t ld,
                        int elem_bytes, hipStream_t st) {
  const char* env = std::getenv("SBN_CHECK_FINITE");
  if (!(env && env[0] == '1')) return SBN_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return SBN_OK;
  bool found = false;
  const hipError_t e = scan_nonfinite(x, rows, cols, ld, elem_bytes, st, &found);
  if (e != hipSuccess) return fail(SBN_ERR_HIP, "%s: finite check of %s: %s", fn, what, hipGetErrorString(e));
  if (found) return fail(SBN_ERR_VALUE, "%s: %s holds a NaN or Inf (SBN_CHECK_FINITE)", fn, what);
  return SBN_OK;
}

thread_local bool g_injected = false;

sbn_status hip_result(hipError_t e, hipStream_t st, const char* what) {
  if (g_injected) {
    g_injected = false;
    return fail(SBN_ERR_HIP, "%s: launch failed (injected by SBN_TEST_INJECT_LAUNCH_FAILURE)", what);
  }
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(SBN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t K_MAX = int64_t(1) << 18;
constexpr int64_t NUMEL_MAX = int64_t(1) << 37;   // elements of W, Xq, dX, dW
constexpr int64_t ROWS_MAX = int64_t(1) << 40;    // any T or R (so that R*K, T*K fit in int64)
constexpr int64_t SPAN_MAX = int64_t(1) << 40;    // rows times a leading dimension (Y, X, W, dY)

// a * b < limit for 1 <= a, b, decided without forming the product
bool prod_below(int64_t a, int64_t b, int64_t limit) { return a <= (limit - 1) / b; }

sbn_status check_nm(int n, int m) {
  if (!(m == 4 || m == 8) || n < 1 || n > m)
    return fail(SBN_ERR_UNSUPPORTED_NM, "unsupported N:M ratio %d:%d (m in {4,8}, 1 <= n <= m)", n, m);
  return SBN_OK;
}

sbn_status check_k(int64_t K) {
  if (K < 64 || K % 64 != 0 || K > K_MAX)
    return fail(SBN_ERR_SHAPE, "K = %lld must be a positive multiple of 64 and <= 2^18", (long long)K);
  return SBN_OK;
}

sbn_status check_rows(const char* name, int64_t v) {
  if (v < 1) return fail(SBN_ERR_SHAPE, "%s = %lld must be >= 1", name, (long long)v);
  if (v > ROWS_MAX) return fail(SBN_ERR_SHAPE, "%s = %lld exceeds 2^40", name, (long long)v);
  return SBN_OK;
}

// rows x K elements (rows and K already checked): below NUMEL_MAX
sbn_status check_numel(const char* fn, const char* what, int64_t rows, int64_t K) {
  if (!prod_below(rows, K, NUMEL_MAX)) return fail(SBN_ERR_SHAPE, "%s: %s has 2^37 elements or more", fn, what);
  return SBN_OK;
}

// a leading dimension of `len` elements per row, for `rows` rows (rows already checked)
sbn_status check_ld(const char* name, int64_t ld, int64_t len, int64_t rows = 1) {
  if (ld < len) return fail(SBN_ERR_SHAPE, "%s = %lld is smaller than the row length %lld", name, (long long)ld, (long long)len);
  if (ld % 8 != 0) return fail(SBN_ERR_ALIGN, "%s = %lld is not a multiple of 8", name, (long long)ld);
  if (!prod_below(rows, ld, SPAN_MAX))
    return fail(SBN_ERR_SHAPE, "%s = %lld times %lld rows reaches 2^40 elements", name, (long long)ld, (long long)rows);
  return SBN_OK;
}

#define SBN_TRY(expr)                 \
  do {                                \
    const sbn_status s_ = (expr);     \
    if (s_ != SBN_OK) return s_;      \
  } while (0)

#define SBN_NONNULL(p)                                                        \
  do {                                                                        \
    if (!(p)) return fail(SBN_ERR_NULL, "%s: argument '%s' is NULL", fn, #p); \
  } while (0)

#define SBN_ALIGNED(p)                                                                         \
  do {                                                                                         \
    if ((p) && !aligned16(p)) return fail(SBN_ERR_ALIGN, "%s: '%s' is not 16-byte aligned", fn, #p); \
  } while (0)

size_t packed_codes(int64_t R, int64_t K, int n, int m) {
  return (size_t)round_up(R * K * n / (4 * m), 16);
}
size_t packed_meta(int64_t R, int64_t K, int n, int m) {
  return n == m ? 0 : (size_t)round_up(R * K / 8, 16);
}

sbn_status check_matmul_args(const char* fn, const int8_t* Xq, const float* s_x, int64_t T,
                             int64_t K, const uint8_t* codes, const uint8_t* meta,
                             const float* s_w, int64_t R, int n, int m, void* Y, sbn_dtype ydt,
                             int64_t ldy) {
  SBN_NONNULL(Xq);
  SBN_NONNULL(s_x);
  SBN_NONNULL(codes);
  SBN_NONNULL(s_w);
  SBN_NONNULL(Y);
  SBN_TRY(check_nm(n, m));
  if (n < m) SBN_NONNULL(meta);
  SBN_TRY(check_rows("T", T));
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  SBN_TRY(check_numel(fn, "Xq (T*K)", T, K));
  SBN_TRY(check_ld("ldy", ldy, R, T));
  if (ydt != SBN_F32 && ydt != SBN_BF16 && ydt != SBN_I32_ACC)
    return fail(SBN_ERR_DTYPE, "%s: unknown output dtype %d", fn, (int)ydt);
  SBN_ALIGNED(Xq);
  SBN_ALIGNED(codes);
  SBN_ALIGNED(meta);
  SBN_ALIGNED(Y);
  return SBN_OK;
}

// ---------------------------------------------------------------- kernel timing
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
std::atomic<int> g_prof_on{0};
char g_prof_only[64] = "";          // empty: every kernel
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;
std::map<std::string, std::pair<long long, double>> g_prof_totals;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  // timing-only events: no system-scope fence, so recording them does not add
  // an L2 write-back and invalidate to the bracketed kernel's interval
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// drain recorded events into the totals (caller holds the lock)
hipError_t prof_collect() {
  hipError_t err = hipSuccess;
  for (ProfRec& r : g_prof_recs) {
    if (r.stop) {
      hipError_t e = hipEventSynchronize(r.stop);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
      if (e != hipSuccess) err = e;
      auto& t = g_prof_totals[r.name];
      t.first += 1;
      t.second += ms;
      g_prof_pool.push_back(r.stop);
    }
    if (r.start) g_prof_pool.push_back(r.start);
  }
  g_prof_recs.clear();
  return err;
}

}  // namespace

namespace sbn {

bool inject_launch_failure() {
  static const bool on = [] {
    const char* e = std::getenv("SBN_TEST_INJECT_LAUNCH_FAILURE");
    return e && e[0] == '1';
  }();
  return on;
}

void note_injected_failure() { g_injected = true; }

int prof_begin(hipStream_t st, const char* name) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_only[0] && strcmp(g_prof_only, name) != 0) return -1;
  ProfRec r{name, prof_event(), nullptr};
  if (!r.start) return -1;
  (void)hipEventRecord(r.start, st);
  g_prof_recs.push_back(r);
  return (int)g_prof_recs.size() - 1;
}

void prof_end(int slot, hipStream_t st) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (slot >= (int)g_prof_recs.size()) return;
  hipEvent_t e = prof_event();
  if (!e) return;
  (void)hipEventRecord(e, st);
  g_prof_recs[slot].stop = e;
}

}  // namespace sbn

extern "C" {

sbn_status sbn_profile_enable(int on, const char* kernel) {
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    snprintf(g_prof_only, sizeof(g_prof_only), "%s", kernel ? kernel : "");
  }
  g_prof_on.store(on ? 1 : 0);
  return ok();
}

sbn_status sbn_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipError_t e = prof_collect();
  g_prof_totals.clear();
  if (e != hipSuccess) return fail(SBN_ERR_HIP, "sbn_profile_reset: %s", hipGetErrorString(e));
  return ok();
}

sbn_status sbn_profile_dump(char* buf, size_t buf_bytes) {
  const char* fn = "sbn_profile_dump";
  SBN_NONNULL(buf);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipError_t e = prof_collect();
  std::string out;
  for (auto& kv : g_prof_totals) {
    char line[160];
    snprintf(line, sizeof(line), "%s %lld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  if (buf_bytes) {
    const size_t nb = out.size() < buf_bytes - 1 ? out.size() : buf_bytes - 1;
    memcpy(buf, out.data(), nb);
    buf[nb] = '\0';
  }
  if (e != hipSuccess) return fail(SBN_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

int sbn_abi_version(void) { return SBN_ABI_VERSION; }

const char* sbn_status_string(sbn_status s) {
  switch (s) {
    case SBN_OK: return "ok";
    case SBN_ERR_NULL: return "null pointer argument";
    case SBN_ERR_SHAPE: return "invalid shape";
    case SBN_ERR_UNSUPPORTED_NM: return "unsupported N:M ratio";
    case SBN_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case SBN_ERR_WORKSPACE: return "workspace too small";
    case SBN_ERR_DTYPE: return "unsupported dtype";
    case SBN_ERR_HIP: return "HIP runtime error";
    case SBN_ERR_FLAGS: return "flag not accepted by this call";
    case SBN_ERR_VALUE: return "scalar argument out of range";
  }
  return "unknown status";
}

const char* sbn_last_error(void) { return g_last_error; }

sbn_status sbn_packed_bytes(int64_t R, int64_t K, int n, int m, size_t* codes_bytes,
                            size_t* meta_bytes) {
  const char* fn = "sbn_packed_bytes";
  SBN_NONNULL(codes_bytes);
  SBN_NONNULL(meta_bytes);
  SBN_TRY(check_nm(n, m));
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  *codes_bytes = packed_codes(R, K, n, m);
  *meta_bytes = packed_meta(R, K, n, m);
  return ok();
}

sbn_status sbn_workspace_bytes(sbn_op op, int64_t T, int64_t R, int64_t K, int n, int m,
                               size_t* bytes) {
  const char* fn = "sbn_workspace_bytes";
  SBN_NONNULL(bytes);
  switch (op) {
    case SBN_OP_ACT_QUANT:
    case SBN_OP_GEMV:
      *bytes = 0;
      return ok();
    case SBN_OP_PACK:
      SBN_TRY(check_nm(n, m));
      SBN_TRY(check_rows("R", R));
      SBN_TRY(check_k(K));
      SBN_TRY(check_numel(fn, "W (R*K)", R, K));
      *bytes = pack_plan(R, K).bytes;
      return ok();
    case SBN_OP_GEMM:
      SBN_TRY(check_nm(n, m));
      SBN_TRY(check_rows("T", T));
      SBN_TRY(check_rows("R", R));
      SBN_TRY(check_k(K));
      SBN_TRY(check_numel(fn, "W (R*K)", R, K));
      SBN_TRY(check_numel(fn, "Xq (T*K)", T, K));
      *bytes = gemm_ws_bytes(T, R, K, n, m);
      return ok();
    case SBN_OP_GEMM_PREPARED:
      SBN_TRY(check_rows("T", T));
      SBN_TRY(check_k(K));
      SBN_TRY(check_nm(n, m));
      SBN_TRY(check_numel(fn, "Xq (T*K)", T, K));
      *bytes = gemm_x_bytes(T, K, n, m);
      return ok();
    case SBN_OP_FORWARD:
      SBN_TRY(check_nm(n, m));
      SBN_TRY(check_rows("T", T));
      SBN_TRY(check_rows("R", R));
      SBN_TRY(check_k(K));
      SBN_TRY(check_numel(fn, "W (R*K)", R, K));
      SBN_TRY(check_numel(fn, "Xq (T*K)", T, K));
      *bytes = align256(pack_plan(R, K).bytes) + gemm_ws_bytes(T, R, K, n, m);
      return ok();
    case SBN_OP_BACKWARD:
      SBN_TRY(check_nm(n, m));
      SBN_TRY(check_rows("T", T));
      SBN_TRY(check_rows("R", R));
      SBN_TRY(check_k(K));
      SBN_TRY(check_numel(fn, "W (R*K)", R, K));
      SBN_TRY(check_numel(fn, "Xq (T*K)", T, K));
      SBN_TRY(check_numel(fn, "dY (T*R)", T, R));
      *bytes = bwd_ws_bytes(T, R, K, n, m);
      return ok();
  }
  return fail(SBN_ERR_SHAPE, "%s: unknown op %d", fn, (int)op);
}

static sbn_status pack_common(const char* fn, const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                              uint32_t flags, uint8_t* codes, uint8_t* meta, float* s_w, void* ws,
                              size_t ws_bytes, const float* G, int64_t ldg, float lr, void* stream) {
  SBN_NONNULL(W);
  SBN_NONNULL(codes);
  SBN_NONNULL(s_w);
  SBN_NONNULL(ws);
  SBN_TRY(check_nm(n, m));
  if (n < m) SBN_NONNULL(meta);
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  SBN_TRY(check_ld("ldw", ldw, K, R));
  if (flags & ~(uint32_t)SBN_MASK_FROM_TERNARY)
    return fail(SBN_ERR_FLAGS, "%s: flags 0x%x: only SBN_MASK_FROM_TERNARY is accepted", fn, (unsigned)flags);
  SBN_ALIGNED(W);
  SBN_ALIGNED(codes);
  if (n < m) SBN_ALIGNED(meta);
  SBN_ALIGNED(ws);
  const size_t need = pack_plan(R, K).bytes;
  if (ws_bytes < need)
    return fail(SBN_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  SBN_TRY(check_finite(fn, "W", W, R, K, ldw, 2, st));
  if (G) SBN_TRY(check_finite(fn, "G", G, R, K, ldg, 4, st));
  return hip_result(launch_pack(W, R, K, ldw, n, m, codes, meta, s_w, ws, flags, G, ldg, lr, st), st, fn);
}

sbn_status sbn_mask_ternarize_pack(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n,
                                   int m, uint8_t* codes, uint8_t* meta, float* s_w, void* ws,
                                   size_t ws_bytes, void* stream) {
  return pack_common("sbn_mask_ternarize_pack", W, R, K, ldw, n, m, 0u, codes, meta, s_w, ws, ws_bytes,
                     nullptr, 0, 0.0f, stream);
}

sbn_status sbn_mask_ternarize_pack_ex(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                                      uint32_t flags, uint8_t* codes, uint8_t* meta, float* s_w, void* ws,
                                      size_t ws_bytes, void* stream) {
  return pack_common("sbn_mask_ternarize_pack_ex", W, R, K, ldw, n, m, flags, codes, meta, s_w, ws, ws_bytes,
                     nullptr, 0, 0.0f, stream);
}

sbn_status sbn_mask_ternarize_pack_noalloc(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                                           uint8_t* codes, uint8_t* meta, float* s_w, void* stream) {
  const char* fn = "sbn_mask_ternarize_pack_noalloc";
  SBN_NONNULL(W);
  SBN_NONNULL(codes);
  SBN_NONNULL(s_w);
  SBN_TRY(check_nm(n, m));
  if (n < m) SBN_NONNULL(meta);
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  SBN_TRY(check_ld("ldw", ldw, K, R));
  SBN_ALIGNED(W);
  SBN_ALIGNED(codes);
  if (n < m) SBN_ALIGNED(meta);
  const size_t need = pack_plan(R, K).bytes;
  if (need > noalloc_scratch_bytes())
    return fail(SBN_ERR_WORKSPACE,
                "%s: R*K = %lld needs %zu bytes of scratch, above the library's fixed %zu (R*K up to 2^28); "
                "use sbn_mask_ternarize_pack with a workspace",
                fn, (long long)(R * K), need, noalloc_scratch_bytes());
  void* scr = nullptr;
  const hipError_t e = noalloc_scratch(&scr);
  if (e != hipSuccess) return fail(SBN_ERR_HIP, "%s: scratch address: %s", fn, hipGetErrorString(e));
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_pack(W, R, K, ldw, n, m, codes, meta, s_w, scr, 0u, nullptr, 0, 0.0f, st), st, fn);
}

sbn_status sbn_sgd_update_pack(uint16_t* W, int64_t R, int64_t K, int64_t ldw, const float* G, int64_t ldg,
                               float lr, int n, int m, uint32_t flags, uint8_t* codes, uint8_t* meta,
                               float* s_w, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "sbn_sgd_update_pack";
  SBN_NONNULL(G);
  SBN_ALIGNED(G);
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_ld("ldg", ldg, K, R));
  if (!std::isfinite(lr)) return fail(SBN_ERR_VALUE, "%s: lr must be finite", fn);
  return pack_common(fn, W, R, K, ldw, n, m, flags, codes, meta, s_w, ws, ws_bytes, G, ldg, lr, stream);
}

sbn_status sbn_act_quant(const uint16_t* X, int64_t T, int64_t K, int64_t ldx, int8_t* Xq,
                         float* s_x, void* stream) {
  const char* fn = "sbn_act_quant";
  SBN_NONNULL(X);
  SBN_NONNULL(Xq);
  SBN_NONNULL(s_x);
  SBN_TRY(check_rows("T", T));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "Xq (T*K)", T, K));
  SBN_TRY(check_ld("ldx", ldx, K, T));
  SBN_ALIGNED(X);
  SBN_ALIGNED(Xq);
  hipStream_t st = (hipStream_t)stream;
  SBN_TRY(check_finite(fn, "X", X, T, K, ldx, 2, st));
  return hip_result(launch_act_quant(X, T, K, ldx, Xq, s_x, st), st, fn);
}

sbn_status sbn_sparse_ternary_gemm(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                   const uint8_t* codes, const uint8_t* meta, const float* s_w,
                                   int64_t R, int n, int m, void* Y, sbn_dtype ydt, int64_t ldy,
                                   void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "sbn_sparse_ternary_gemm";
  SBN_TRY(check_matmul_args(fn, Xq, s_x, T, K, codes, meta, s_w, R, n, m, Y, ydt, ldy));
  SBN_NONNULL(ws);
  SBN_ALIGNED(ws);
  const size_t need = gemm_ws_bytes(T, R, K, n, m);
  if (ws_bytes < need)
    return fail(SBN_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemm(Xq, s_x, T, K, codes, n == m ? nullptr : meta, s_w, R, n, m, Y,
                                ydt, ldy, ws, st),
                    st, fn);
}

sbn_status sbn_gemm_weight_bytes(int64_t R, int64_t K, int n, int m, size_t* bytes) {
  const char* fn = "sbn_gemm_weight_bytes";
  SBN_NONNULL(bytes);
  SBN_TRY(check_nm(n, m));
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  *bytes = gemm_weight_bytes(R, K, n, m);
  return ok();
}

sbn_status sbn_prepare_gemm_weight(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, int n, int m,
                                   uint8_t* prepared, void* stream) {
  const char* fn = "sbn_prepare_gemm_weight";
  SBN_NONNULL(codes);
  SBN_NONNULL(prepared);
  SBN_TRY(check_nm(n, m));
  if (n < m) SBN_NONNULL(meta);
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  SBN_ALIGNED(codes);
  if (n < m) SBN_ALIGNED(meta);
  SBN_ALIGNED(prepared);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_prepare_gemm_weight(codes, n == m ? nullptr : meta, R, K, n, m, prepared, st), st, fn);
}

sbn_status sbn_sparse_ternary_gemm_prepared(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                            const uint8_t* prepared, const float* s_w, int64_t R, int n, int m,
                                            void* Y, sbn_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes,
                                            void* stream) {
  const char* fn = "sbn_sparse_ternary_gemm_prepared";
  SBN_NONNULL(prepared);
  // the packed-weight checks with the prepared operand standing in for both planes
  SBN_TRY(check_matmul_args(fn, Xq, s_x, T, K, prepared, prepared, s_w, R, n, m, Y, ydt, ldy));
  const size_t need = gemm_x_bytes(T, K, n, m);
  if (need > 0) {
    SBN_NONNULL(ws);
    SBN_ALIGNED(ws);
    if (ws_bytes < need)
      return fail(SBN_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  }
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemm_prepared(Xq, s_x, T, K, prepared, s_w, R, n, m, Y, ydt, ldy, ws, st), st, fn);
}

sbn_status sbn_forward(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, const uint16_t* X, int64_t T,
                       int64_t ldx, int n, int m, uint32_t flags, uint8_t* codes, uint8_t* meta, float* s_w,
                       int8_t* Xq, float* s_x, void* Y, sbn_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes,
                       void* stream) {
  const char* fn = "sbn_forward";
  SBN_NONNULL(W);
  SBN_NONNULL(X);
  SBN_NONNULL(ws);
  SBN_TRY(check_matmul_args(fn, Xq, s_x, T, K, codes, meta, s_w, R, n, m, Y, ydt, ldy));
  SBN_TRY(check_ld("ldw", ldw, K, R));
  SBN_TRY(check_ld("ldx", ldx, K, T));
  if (flags & ~(uint32_t)SBN_MASK_FROM_TERNARY)
    return fail(SBN_ERR_FLAGS, "%s: flags 0x%x: only SBN_MASK_FROM_TERNARY is accepted", fn, (unsigned)flags);
  SBN_ALIGNED(W);
  SBN_ALIGNED(X);
  SBN_ALIGNED(ws);
  const size_t pack_b = align256(pack_plan(R, K).bytes);
  const size_t need = pack_b + gemm_ws_bytes(T, R, K, n, m);
  if (ws_bytes < need)
    return fail(SBN_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  SBN_TRY(check_finite(fn, "W", W, R, K, ldw, 2, st));
  SBN_TRY(check_finite(fn, "X", X, T, K, ldx, 2, st));
  uint8_t* mp = n == m ? nullptr : meta;
  hipError_t e;
  if (forward_writes_operand(T, R, K, n, m, flags)) {
    // three launches: pass 2 also writes the GEMM's weight operand (into the
    // GEMM part of ws, laid out as a prepared weight), and the GEMM reads it
    uint8_t* op = (uint8_t*)ws + pack_b;
    e = launch_pack_quant_operand(W, R, K, ldw, codes, mp, s_w, ws, X, T, ldx, Xq, s_x, op,
                                  (uint32_t*)(op + gemm_operand_idx_offset(R, K, n, m)), st);
    if (e == hipSuccess) e = launch_gemm_prepared(Xq, s_x, T, K, op, s_w, R, n, m, Y, ydt, ldy, nullptr, st);
  } else {
    e = launch_pack_quant(W, R, K, ldw, n, m, codes, mp, s_w, ws, flags, X, T, ldx, Xq, s_x, st);
    if (e == hipSuccess)
      e = launch_gemm(Xq, s_x, T, K, codes, mp, s_w, R, n, m, Y, ydt, ldy, (uint8_t*)ws + pack_b, st);
  }
  return hip_result(e, st, fn);
}

sbn_status sbn_sparse_ternary_gemv(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                   const uint8_t* codes, const uint8_t* meta, const float* s_w,
                                   int64_t R, int n, int m, void* Y, sbn_dtype ydt, int64_t ldy,
                                   void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "sbn_sparse_ternary_gemv";
  (void)ws;
  (void)ws_bytes;
  SBN_TRY(check_matmul_args(fn, Xq, s_x, T, K, codes, meta, s_w, R, n, m, Y, ydt, ldy));
  if (T > 16) return fail(SBN_ERR_SHAPE, "%s: T = %lld exceeds 16; use the GEMM", fn, (long long)T);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemv(Xq, s_x, T, K, codes, n == m ? nullptr : meta, s_w, R, n, m, Y,
                                ydt, ldy, st),
                    st, fn);
}

sbn_status sbn_sparse_ternary_gemv_batched(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                           const uint8_t* const* codes, const uint8_t* const* meta,
                                           const float* const* s_w, int64_t R, int n, int m,
                                           void* const* Y, sbn_dtype ydt, int64_t ldy, int64_t count,
                                           void* stream) {
  const char* fn = "sbn_sparse_ternary_gemv_batched";
  SBN_NONNULL(codes);
  SBN_NONNULL(s_w);
  SBN_NONNULL(Y);
  if (count < 1 || count > SBN_GEMV_MAX_BATCH)
    return fail(SBN_ERR_SHAPE, "%s: count = %lld must be in [1, %d]", fn, (long long)count, SBN_GEMV_MAX_BATCH);
  SBN_TRY(check_nm(n, m));
  if (n < m) SBN_NONNULL(meta);
  const uint8_t* metas[SBN_GEMV_MAX_BATCH];
  for (int64_t b = 0; b < count; ++b) {
    metas[b] = n < m ? meta[b] : nullptr;
    const sbn_status st_b = check_matmul_args(fn, Xq, s_x, T, K, codes[b], metas[b], s_w[b], R, n, m, Y[b], ydt, ldy);
    if (st_b != SBN_OK) {
      char msg[512];
      snprintf(msg, sizeof(msg), "%s (weight %lld)", sbn_last_error(), (long long)b);
      return fail(st_b, "%s", msg);
    }
  }
  if (T > 16) return fail(SBN_ERR_SHAPE, "%s: T = %lld exceeds 16; use the GEMM", fn, (long long)T);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemv_batched(Xq, s_x, T, K, codes, metas, s_w, R, n, m, Y, ydt, ldy, (int)count, st),
                    st, fn);
}

static sbn_status backward_common(const char* fn, const uint16_t* dY, int64_t T, int64_t R, const int8_t* Xq,
                                  const float* s_x, int64_t K, const uint8_t* codes, const uint8_t* meta,
                                  const float* s_w, int n, int m, void* dX, sbn_dtype dxdt, float* dW,
                                  uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  SBN_NONNULL(dY);
  SBN_NONNULL(Xq);
  SBN_NONNULL(s_x);
  SBN_NONNULL(codes);
  SBN_NONNULL(s_w);
  SBN_NONNULL(ws);
  SBN_TRY(check_nm(n, m));
  if (n < m) SBN_NONNULL(meta);
  SBN_TRY(check_rows("T", T));
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  if (R % 8 != 0) return fail(SBN_ERR_SHAPE, "%s: R = %lld must be a multiple of 8", fn, (long long)R);
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  SBN_TRY(check_numel(fn, "Xq (T*K)", T, K));
  SBN_TRY(check_numel(fn, "dY (T*R)", T, R));
  if (dX && dxdt != SBN_F32 && dxdt != SBN_BF16)
    return fail(SBN_ERR_DTYPE, "%s: dX dtype must be SBN_F32 or SBN_BF16", fn);
  if (flags & ~(uint32_t)SBN_GRAD_W_MASKED)
    return fail(SBN_ERR_FLAGS, "%s: flags 0x%x: only SBN_GRAD_W_MASKED is accepted", fn, (unsigned)flags);
  SBN_ALIGNED(dY);
  SBN_ALIGNED(Xq);
  SBN_ALIGNED(codes);
  if (n < m) SBN_ALIGNED(meta);
  SBN_ALIGNED(dX);
  SBN_ALIGNED(dW);
  SBN_ALIGNED(ws);
  const size_t need = bwd_ws_bytes(T, R, K, n, m);
  if (ws_bytes < need)
    return fail(SBN_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  SBN_TRY(check_finite(fn, "dY", dY, T, R, R, 2, st));
  return hip_result(launch_backward(dY, T, R, Xq, s_x, K, codes, n == m ? nullptr : meta, s_w, n,
                                    m, dX, dxdt, dW, ws, flags, st),
                    st, fn);
}

sbn_status sbn_backward(const uint16_t* dY, int64_t T, int64_t R, const int8_t* Xq,
                        const float* s_x, int64_t K, const uint8_t* codes, const uint8_t* meta,
                        const float* s_w, int n, int m, void* dX, sbn_dtype dxdt, float* dW,
                        void* ws, size_t ws_bytes, void* stream) {
  return backward_common("sbn_backward", dY, T, R, Xq, s_x, K, codes, meta, s_w, n, m, dX, dxdt, dW, 0u, ws,
                         ws_bytes, stream);
}

sbn_status sbn_decode_plane_bytes(int64_t R, int64_t K, size_t* bytes) {
  const char* fn = "sbn_decode_plane_bytes";
  SBN_NONNULL(bytes);
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  *bytes = (size_t)round_up(R * K / 4, 16);
  return ok();
}

sbn_status sbn_repack_d2(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, int n, int m,
                         uint8_t* d2, void* stream) {
  const char* fn = "sbn_repack_d2";
  SBN_NONNULL(codes);
  SBN_NONNULL(d2);
  SBN_TRY(check_nm(n, m));
  if (n < m) SBN_NONNULL(meta);
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  SBN_ALIGNED(codes);
  if (n < m) SBN_ALIGNED(meta);
  SBN_ALIGNED(d2);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_repack_d2(codes, n == m ? nullptr : meta, R, K, n, m, d2, st), st, fn);
}

sbn_status sbn_j6_bytes(int64_t R, int64_t K, size_t* nib_bytes, size_t* h_bytes) {
  const char* fn = "sbn_j6_bytes";
  SBN_NONNULL(nib_bytes);
  SBN_NONNULL(h_bytes);
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  *nib_bytes = (size_t)round_up(R * K / 8, 16);
  *h_bytes = (size_t)round_up(R * K / 16, 16);
  return ok();
}

sbn_status sbn_repack_j6(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, uint8_t* nib,
                         uint8_t* hpl, void* stream) {
  const char* fn = "sbn_repack_j6";
  SBN_NONNULL(codes);
  SBN_NONNULL(meta);
  SBN_NONNULL(nib);
  SBN_NONNULL(hpl);
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  SBN_ALIGNED(codes);
  SBN_ALIGNED(meta);
  SBN_ALIGNED(nib);
  SBN_ALIGNED(hpl);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_repack_j6(codes, meta, R, K, nib, hpl, st), st, fn);
}

static sbn_status check_d2_args(const char* fn, const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                const uint8_t* d2, const float* s_w, int64_t R, void* Y, sbn_dtype ydt,
                                int64_t ldy) {
  SBN_NONNULL(Xq);
  SBN_NONNULL(s_x);
  SBN_NONNULL(d2);
  SBN_NONNULL(s_w);
  SBN_NONNULL(Y);
  SBN_TRY(check_rows("T", T));
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  if (T > 16) return fail(SBN_ERR_SHAPE, "%s: T = %lld exceeds 16", fn, (long long)T);
  SBN_TRY(check_ld("ldy", ldy, R, T));
  if (ydt != SBN_F32 && ydt != SBN_BF16 && ydt != SBN_I32_ACC)
    return fail(SBN_ERR_DTYPE, "%s: unknown output dtype %d", fn, (int)ydt);
  SBN_ALIGNED(Xq);
  SBN_ALIGNED(d2);
  SBN_ALIGNED(Y);
  return SBN_OK;
}

sbn_status sbn_ternary_gemv_d2(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* d2,
                               const float* s_w, int64_t R, void* Y, sbn_dtype ydt, int64_t ldy, void* stream) {
  const char* fn = "sbn_ternary_gemv_d2";
  SBN_TRY(check_d2_args(fn, Xq, s_x, T, K, d2, s_w, R, Y, ydt, ldy));
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemv_d2_batched(Xq, s_x, T, K, &d2, &s_w, R, &Y, ydt, ldy, 1, st), st, fn);
}

sbn_status sbn_ternary_gemv_d2_batched(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                       const uint8_t* const* d2, const float* const* s_w, int64_t R,
                                       void* const* Y, sbn_dtype ydt, int64_t ldy, int64_t count, void* stream) {
  const char* fn = "sbn_ternary_gemv_d2_batched";
  SBN_NONNULL(d2);
  SBN_NONNULL(s_w);
  SBN_NONNULL(Y);
  if (count < 1 || count > SBN_GEMV_MAX_BATCH)
    return fail(SBN_ERR_SHAPE, "%s: count = %lld must be in [1, %d]", fn, (long long)count, SBN_GEMV_MAX_BATCH);
  for (int64_t b = 0; b < count; ++b) {
    const sbn_status st_b = check_d2_args(fn, Xq, s_x, T, K, d2[b], s_w[b], R, Y[b], ydt, ldy);
    if (st_b != SBN_OK) {
      char msg[512];
      snprintf(msg, sizeof(msg), "%s (weight %lld)", sbn_last_error(), (long long)b);
      return fail(st_b, "%s", msg);
    }
  }
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemv_d2_batched(Xq, s_x, T, K, d2, s_w, R, Y, ydt, ldy, (int)count, st), st, fn);
}

// The arguments of a table GEMV call that the host can see (the entries live
// in device memory): activations, shapes, output layout, the table pointer
// and the count.
static sbn_status check_table_call(const char* fn, const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                   const sbn_gemv_entry* table, int64_t count, int64_t R, sbn_dtype ydt,
                                   int64_t ldy) {
  SBN_NONNULL(Xq);
  SBN_NONNULL(s_x);
  SBN_NONNULL(table);
  SBN_TRY(check_rows("T", T));
  SBN_TRY(check_rows("R", R));
  SBN_TRY(check_k(K));
  SBN_TRY(check_numel(fn, "W (R*K)", R, K));
  if (T > 16) return fail(SBN_ERR_SHAPE, "%s: T = %lld exceeds 16; use the GEMM", fn, (long long)T);
  SBN_TRY(check_ld("ldy", ldy, R, T));
  if (ydt != SBN_F32 && ydt != SBN_BF16 && ydt != SBN_I32_ACC)
    return fail(SBN_ERR_DTYPE, "%s: unknown output dtype %d", fn, (int)ydt);
  if (count < 1) return fail(SBN_ERR_SHAPE, "%s: count = %lld must be at least 1", fn, (long long)count);
  if (!prod_below(count, (R + 15) / 16, (int64_t)1 << 40))
    return fail(SBN_ERR_SHAPE, "%s: count * ceil(R / 16) reaches 2^40", fn);
  SBN_ALIGNED(Xq);
  SBN_ALIGNED(table);
  return SBN_OK;
}

sbn_status sbn_sparse_ternary_gemv_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                         const sbn_gemv_entry* table, int64_t count, int64_t R, int n, int m,
                                         sbn_dtype ydt, int64_t ldy, void* stream) {
  const char* fn = "sbn_sparse_ternary_gemv_table";
  SBN_TRY(check_nm(n, m));
  SBN_TRY(check_table_call(fn, Xq, s_x, T, K, table, count, R, ydt, ldy));
  if (!((n == 2 && m == 4) || (n == 6 && m == 8)))
    return fail(SBN_ERR_UNSUPPORTED_NM, "%s: %d:%d has no table GEMV (2:4 and 6:8 only); use the batched call", fn,
                n, m);
  if (!gemv_table_shape_ok(K, n, m))
    return fail(SBN_ERR_SHAPE, "%s: K = %lld must be a multiple of 1024 up to 4096; use the batched call", fn,
                (long long)K);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemv_table(Xq, s_x, T, K, table, count, R, n, m, ydt, ldy, st), st, fn);
}

sbn_status sbn_ternary_gemv_d2_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                     const sbn_gemv_entry* table, int64_t count, int64_t R, sbn_dtype ydt,
                                     int64_t ldy, void* stream) {
  const char* fn = "sbn_ternary_gemv_d2_table";
  SBN_TRY(check_table_call(fn, Xq, s_x, T, K, table, count, R, ydt, ldy));
  if (!gemv_d2_table_shape_ok(K))
    return fail(SBN_ERR_SHAPE, "%s: K = %lld must be a multiple of 1024 up to 4096; use the batched call", fn,
                (long long)K);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemv_d2_table(Xq, s_x, T, K, table, count, R, ydt, ldy, st), st, fn);
}

sbn_status sbn_ternary_gemv_j6(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* nib,
                               const uint8_t* hpl, const float* s_w, int64_t R, void* Y, sbn_dtype ydt, int64_t ldy,
                               void* stream) {
  const char* fn = "sbn_ternary_gemv_j6";
  SBN_TRY(check_d2_args(fn, Xq, s_x, T, K, nib, s_w, R, Y, ydt, ldy));
  SBN_NONNULL(hpl);
  SBN_ALIGNED(hpl);
  if (!gemv_d2_table_shape_ok(K))
    return fail(SBN_ERR_SHAPE, "%s: K = %lld must be a multiple of 1024 up to 4096", fn, (long long)K);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemv_j6(Xq, s_x, T, K, nib, hpl, s_w, R, Y, ydt, ldy, st), st, fn);
}

sbn_status sbn_ternary_gemv_j6_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                     const sbn_gemv_entry* table, int64_t count, int64_t R, sbn_dtype ydt,
                                     int64_t ldy, void* stream) {
  const char* fn = "sbn_ternary_gemv_j6_table";
  SBN_TRY(check_table_call(fn, Xq, s_x, T, K, table, count, R, ydt, ldy));
  if (!gemv_d2_table_shape_ok(K))
    return fail(SBN_ERR_SHAPE, "%s: K = %lld must be a multiple of 1024 up to 4096", fn, (long long)K);
  hipStream_t st = (hipStream_t)stream;
  return hip_result(launch_gemv_j6_table(Xq, s_x, T, K, table, count, R, ydt, ldy, st), st, fn);
}

sbn_status sbn_gemv_table_check(const sbn_gemv_entry* table, int64_t count, int64_t T, int64_t K, int64_t R,
                                int n, int m, int form, sbn_dtype ydt, int64_t ldy) {
  const char* fn = "sbn_gemv_table_check";
  SBN_NONNULL(table);
  if (count < 1) return fail(SBN_ERR_SHAPE, "%s: count = %lld must be at least 1", fn, (long long)count);
  if (form != SBN_FORM_PACKED && form != SBN_FORM_D2 && form != SBN_FORM_J6)
    return fail(SBN_ERR_VALUE, "%s: unknown form %d", fn, form);
  // the activations are not part of the table: stand-ins that pass their checks
  alignas(16) static const int8_t xq_ok[16] = {};
  static const float sx_ok = 1.0f;
  for (int64_t b = 0; b < count; ++b) {
    const sbn_gemv_entry& e = table[b];
    sbn_status st_b =
        form != SBN_FORM_PACKED
            ? check_d2_args(fn, xq_ok, &sx_ok, T, K, e.codes, e.s_w, R, e.Y, ydt, ldy)
            : check_matmul_args(fn, xq_ok, &sx_ok, T, K, e.codes, n < m ? e.meta : nullptr, e.s_w, R, n, m, e.Y, ydt,
                                ldy);
    if (st_b == SBN_OK && form == SBN_FORM_J6) {       // the h plane travels in meta
      if (!e.meta) st_b = fail(SBN_ERR_NULL, "%s: argument 'meta' (the h plane) is NULL", fn);
      else if (!aligned16(e.meta)) st_b = fail(SBN_ERR_ALIGN, "%s: 'meta' (the h plane) is not 16-byte aligned", fn);
    }
    if (st_b != SBN_OK) {
      char msg[512];
      snprintf(msg, sizeof(msg), "%s (entry %lld)", sbn_last_error(), (long long)b);
      return fail(st_b, "%s", msg);
    }
  }
  if (T > 16) return fail(SBN_ERR_SHAPE, "%s: T = %lld exceeds 16", fn, (long long)T);
  return SBN_OK;
}

sbn_status sbn_backward_ex(const uint16_t* dY, int64_t T, int64_t R, const int8_t* Xq,
                           const float* s_x, int64_t K, const uint8_t* codes, const uint8_t* meta,
                           const float* s_w, int n, int m, void* dX, sbn_dtype dxdt, float* dW,
                           uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  return backward_common("sbn_backward_ex", dY, T, R, Xq, s_x, K, codes, meta, s_w, n, m, dX, dxdt, dW, flags, ws,
                         ws_bytes, stream);
}

}  // extern "C"
