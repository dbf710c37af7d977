// C ABI of libtpshard: host-side validation and dispatch.  Every check runs
// before the first HIP call, so each error path can be exercised on a
// machine without a GPU.  No exception crosses the ABI.
#include "../../include/tp_shard.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "launch.hpp"
#include "profile.hpp"

namespace {

thread_local std::string g_detail;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return code;
}

int ok() {
  g_detail.clear();
  return TP_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TP_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = int64_t(1) << 30;
// The kernels address an operand tile with 32-bit buffer offsets from the
// tile's first row: 256 rows of a leading dimension up to 2 * 2^21 elements
// (the SwiGLU [dG | dU] buffer) stay below 2 GiB.  The attention core keeps
// a head's keys/values (s x 128 bf16) under the same bound.
constexpr int64_t kMaxLd = int64_t(1) << 21;
constexpr int64_t kMaxSeq = int64_t(1) << 22;

int check_ld(std::initializer_list<std::pair<const char*, int64_t>> dims) {
  for (const auto& d : dims)
    if (d.second > kMaxLd)
      return fail(TP_E_DIM, "%s = %lld exceeds 2^21 (row pitch limit)", d.first, (long long)d.second);
  return TP_OK;
}

size_t esize(int dt) { return dt == TP_DT_BF16 ? 2 : 4; }

bool dtype_ok(int dt) { return dt == TP_DT_F32 || dt == TP_DT_BF16; }

struct Span {
  const char* name;
  const void* p;
  size_t bytes;
  size_t align = 16;   // required alignment in bytes
};

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Pointer presence, alignment, and output/input overlap.
int check_buffers(const std::vector<Span>& ins, const std::vector<Span>& outs,
                  const std::vector<const char*>& required) {
  auto find = [&](const char* n) -> const Span* {
    for (const auto& s : ins)
      if (std::string(s.name) == n) return &s;
    for (const auto& s : outs)
      if (std::string(s.name) == n) return &s;
    return nullptr;
  };
  for (const char* n : required) {
    const Span* s = find(n);
    if (!s || !s->p) return fail(TP_E_NULL, "%s is NULL", n);
  }
  for (const auto* v : {&ins, &outs})
    for (const auto& s : *v)
      if (s.p && (reinterpret_cast<uintptr_t>(s.p) & (s.align - 1)))
        return fail(TP_E_ALIGN, "%s (%p) is not %zu-byte aligned", s.name, s.p, s.align);
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const auto& in : ins)
      if (overlap(outs[i], in)) return fail(TP_E_ALIAS, "output %s overlaps input %s", outs[i].name, in.name);
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(TP_E_ALIAS, "output %s overlaps output %s", outs[i].name, outs[j].name);
  }
  return TP_OK;
}

int check_dims(std::initializer_list<std::pair<const char*, int64_t>> dims) {
  for (const auto& d : dims) {
    if (d.second <= 0) return fail(TP_E_DIM, "%s = %lld must be positive", d.first, (long long)d.second);
    if (d.second > kMaxDim) return fail(TP_E_DIM, "%s = %lld exceeds 2^30", d.first, (long long)d.second);
  }
  return TP_OK;
}

int check_mult8(std::initializer_list<std::pair<const char*, int64_t>> dims) {
  for (const auto& d : dims)
    if (d.second % 8) return fail(TP_E_DIVIS, "%s = %lld must be a multiple of 8", d.first, (long long)d.second);
  return TP_OK;
}

#define TP_CHECK(expr)         \
  do {                         \
    int rc_ = (expr);          \
    if (rc_ != TP_OK) return rc_; \
  } while (0)

int mlp_common(tp_dtype_t dt, int64_t M, int64_t d, int64_t f) {
  if (!dtype_ok(dt)) return fail(TP_E_DTYPE, "dtype %d is not TP_DT_F32 or TP_DT_BF16", (int)dt);
  TP_CHECK(check_dims({{"M", M}, {"d", d}, {"f", f}}));
  TP_CHECK(check_mult8({{"d", d}, {"f", f}}));
  TP_CHECK(check_ld({{"d", d}, {"f", f}}));
  if ((double)M * (double)std::max(d, f) * 2 > 9.0e15) return fail(TP_E_DIM, "operand too large");
  return TP_OK;
}

int vocab_common(tp_dtype_t dt, int64_t n_tokens, int64_t d, int64_t vocab_local, int64_t vocab_start) {
  if (!dtype_ok(dt)) return fail(TP_E_DTYPE, "dtype %d is not TP_DT_F32 or TP_DT_BF16", (int)dt);
  TP_CHECK(check_dims({{"n_tokens", n_tokens}, {"d", d}, {"vocab_local", vocab_local}}));
  TP_CHECK(check_mult8({{"d", d}, {"vocab_local", vocab_local}}));
  TP_CHECK(check_ld({{"d", d}, {"vocab_local", vocab_local}}));
  if (n_tokens > (int64_t(1) << 24)) return fail(TP_E_DIM, "n_tokens = %lld exceeds 2^24", (long long)n_tokens);
  if (vocab_start < 0 || vocab_start > (int64_t(1) << 40))
    return fail(TP_E_DIM, "vocab_start = %lld outside [0, 2^40]", (long long)vocab_start);
  if ((double)n_tokens * (double)std::max(d, vocab_local) * 2 > 9.0e15) return fail(TP_E_DIM, "operand too large");
  return TP_OK;
}

}  // namespace

namespace tpk {
ProfileState& profile_state() {
  static thread_local ProfileState ps;
  return ps;
}
}  // namespace tpk

extern "C" {

int tp_abi_version(void) { return TP_ABI_VERSION; }

int tp_profile_begin(void* const* start_events, void* const* stop_events, int capacity) {
  if (!start_events || !stop_events) return fail(TP_E_NULL, "event arrays are NULL");
  if (capacity <= 0) return fail(TP_E_DIM, "capacity must be positive");
  tpk::ProfileState& ps = tpk::profile_state();
  ps.start = reinterpret_cast<hipEvent_t const*>(start_events);
  ps.stop = reinterpret_cast<hipEvent_t const*>(stop_events);
  ps.labels.assign((size_t)capacity, nullptr);
  ps.capacity = capacity;
  ps.count = 0;
  return ok();
}

int tp_profile_only(const char* label) {
  tpk::ProfileState& ps = tpk::profile_state();
  ps.only = label ? label : "";
  return ok();
}

int tp_profile_end(void) {
  tpk::ProfileState& ps = tpk::profile_state();
  ps.only.clear();
  const int n = ps.count < ps.capacity ? ps.count : ps.capacity;
  ps.start = ps.stop = nullptr;
  ps.capacity = 0;
  return n;
}

const char* tp_profile_label(int i) {
  const tpk::ProfileState& ps = tpk::profile_state();
  if (i < 0 || i >= ps.count || i >= (int)ps.labels.size() || !ps.labels[i]) return "";
  return ps.labels[i];
}

const char* tp_last_error_detail(void) { return g_detail.c_str(); }

const char* tp_strerror(int status) {
  switch (status) {
    case TP_OK: return "ok";
    case TP_E_NULL: return "required pointer is NULL";
    case TP_E_DIM: return "size is non-positive, too large or unsupported";
    case TP_E_DIVIS: return "size is not a multiple of what it must be";
    case TP_E_DTYPE: return "unsupported dtype";
    case TP_E_ALIGN: return "pointer is not aligned as required";
    case TP_E_ALIAS: return "output overlaps an input or another output";
    case TP_E_WORKSPACE: return "workspace missing or too small";
    case TP_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int tp_shard_range(int64_t total, int64_t n_shards, int64_t index, int64_t* start, int64_t* len) {
  if (!start || !len) return fail(TP_E_NULL, "start/len output pointer is NULL");
  if (total <= 0 || n_shards <= 0) return fail(TP_E_DIM, "total and n_shards must be positive");
  if (index < 0 || index >= n_shards)
    return fail(TP_E_DIM, "index %lld outside [0, %lld)", (long long)index, (long long)n_shards);
  if (total % n_shards)
    return fail(TP_E_DIVIS, "%lld is not divisible by %lld shards", (long long)total, (long long)n_shards);
  const int64_t k = total / n_shards;
  *start = index * k;
  *len = k;
  return ok();
}

int tp_mlp_fwd(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
               const void* X, const void* W1, const void* W2, void* A, void* H, void* Z) {
  TP_CHECK(mlp_common(dt, M, d, f));
  const size_t e = esize(dt);
  TP_CHECK(check_buffers({{"X", X, M * d * e}, {"W1", W1, d * f * e}, {"W2", W2, f * d * e}},
                         {{"A", A, M * f * e}, {"H", H, M * f * e}, {"Z", Z, M * d * e}},
                         {"X", "W1", "W2", "H", "Z"}));
  return hip_status(tpk::launch_mlp_fwd(static_cast<hipStream_t>(stream), dt, M, d, f, X, W1, W2, A, H, Z),
                    "tp_mlp_fwd");
}

size_t tp_mlp_bwd_workspace_bytes(tp_dtype_t dt, int64_t M, int64_t d, int64_t f) {
  if (mlp_common(dt, M, d, f) != TP_OK) return 0;
  return tpk::mlp_bwd_ws_bytes(dt, M, d, f);
}

int tp_mlp_bwd(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
               const void* X, const void* W1, const void* W2, const void* A, const void* H,
               const void* dY, void* dX, float* dW1, float* dW2, void* ws, size_t ws_bytes) {
  TP_CHECK(mlp_common(dt, M, d, f));
  const size_t e = esize(dt);
  const size_t need = tpk::mlp_bwd_ws_bytes(dt, M, d, f);
  TP_CHECK(check_buffers(
      {{"X", X, M * d * e}, {"W1", W1, d * f * e}, {"W2", W2, f * d * e}, {"A", A, M * f * e},
       {"H", H, M * f * e}, {"dY", dY, M * d * e}},
      {{"dX", dX, M * d * e}, {"dW1", dW1, d * f * (size_t)4}, {"dW2", dW2, f * d * (size_t)4}, {"ws", ws, need}},
      {"X", "W1", "W2", "A", "H", "dY", "dX", "dW1", "dW2"}));
  if (!ws || ws_bytes < need)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes given, %zu required", ws ? ws_bytes : (size_t)0, need);
  return hip_status(tpk::launch_mlp_bwd(static_cast<hipStream_t>(stream), dt, M, d, f, X, W1, W2, A, H, dY,
                                        dX, dW1, dW2, ws),
                    "tp_mlp_bwd");
}

namespace {
int mlp_shards_common(tp_dtype_t dt, int64_t n, int64_t M, int64_t d, int64_t f) {
  TP_CHECK(mlp_common(dt, M, d, f));
  if (n < 1 || n > 64) return fail(TP_E_DIM, "n_shards = %lld is outside [1, 64]", (long long)n);
  if ((double)n * (double)M * (double)std::max(d, f) * 2 > 9.0e15) return fail(TP_E_DIM, "operands too large");
  return TP_OK;
}
}  // namespace

int tp_mlp_fwd_shards(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t M, int64_t d, int64_t f,
                      const void* X, const void* W1s, const void* W2s, void* A, void* H, void* Z) {
  TP_CHECK(mlp_shards_common(dt, n_shards, M, d, f));
  const size_t e = esize(dt), n = (size_t)n_shards;
  TP_CHECK(check_buffers({{"X", X, M * d * e}, {"W1s", W1s, n * d * f * e}, {"W2s", W2s, n * f * d * e}},
                         {{"A", A, n * M * f * e}, {"H", H, n * M * f * e}, {"Z", Z, n * M * d * e}},
                         {"X", "W1s", "W2s", "H", "Z"}));
  return hip_status(tpk::launch_mlp_fwd_shards(static_cast<hipStream_t>(stream), dt, n_shards, M, d, f, X, W1s,
                                               W2s, A, H, Z),
                    "tp_mlp_fwd_shards");
}

size_t tp_mlp_bwd_shards_workspace_bytes(tp_dtype_t dt, int64_t n_shards, int64_t M, int64_t d, int64_t f) {
  if (mlp_shards_common(dt, n_shards, M, d, f) != TP_OK) return 0;
  return tpk::mlp_shards_bwd_ws_bytes(dt, n_shards, M, d, f);
}

int tp_mlp_bwd_shards(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t M, int64_t d, int64_t f,
                      const void* X, const void* W1s, const void* W2s, const void* A, const void* H,
                      const void* dY, void* dX, float* dW1s, float* dW2s, void* ws, size_t ws_bytes) {
  TP_CHECK(mlp_shards_common(dt, n_shards, M, d, f));
  const size_t e = esize(dt), n = (size_t)n_shards;
  const size_t need = tpk::mlp_shards_bwd_ws_bytes(dt, n_shards, M, d, f);
  TP_CHECK(check_buffers(
      {{"X", X, M * d * e}, {"W1s", W1s, n * d * f * e}, {"W2s", W2s, n * f * d * e}, {"A", A, n * M * f * e},
       {"H", H, n * M * f * e}, {"dY", dY, M * d * e}},
      {{"dX", dX, n * M * d * e}, {"dW1s", dW1s, n * d * f * (size_t)4}, {"dW2s", dW2s, n * f * d * (size_t)4},
       {"ws", ws, need}},
      {"X", "W1s", "W2s", "A", "H", "dY", "dX", "dW1s", "dW2s"}));
  if (!ws || ws_bytes < need)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes given, %zu required", ws ? ws_bytes : (size_t)0, need);
  return hip_status(tpk::launch_mlp_bwd_shards(static_cast<hipStream_t>(stream), dt, n_shards, M, d, f, X, W1s, W2s,
                                               A, H, dY, dX, dW1s, dW2s, ws),
                    "tp_mlp_bwd_shards");
}

int tp_mlp_bwd_noalloc(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
                       const void* X, const void* W1, const void* W2, const void* A, const void* H,
                       const void* dY, void* dX, float* dW1, float* dW2) {
  TP_CHECK(mlp_common(dt, M, d, f));
  const size_t need = tpk::mlp_bwd_ws_bytes(dt, M, d, f);
  if (need > TP_MLP_BWD_NOALLOC_MAX_WORKSPACE)
    return fail(TP_E_WORKSPACE, "M=%lld d=%lld f=%lld needs %zu bytes of workspace; the allocation-free entry "
                "point holds %zu (use tp_mlp_bwd with a caller workspace)", (long long)M, (long long)d,
                (long long)f, need, (size_t)TP_MLP_BWD_NOALLOC_MAX_WORKSPACE);
  const size_t e = esize(dt);
  TP_CHECK(check_buffers(
      {{"X", X, M * d * e}, {"W1", W1, d * f * e}, {"W2", W2, f * d * e}, {"A", A, M * f * e},
       {"H", H, M * f * e}, {"dY", dY, M * d * e}},
      {{"dX", dX, M * d * e}, {"dW1", dW1, d * f * (size_t)4}, {"dW2", dW2, f * d * (size_t)4}},
      {"X", "W1", "W2", "A", "H", "dY", "dX", "dW1", "dW2"}));
  void* ws = nullptr;
  const hipError_t e0 = tpk::mlp_bwd_scratch(&ws);
  if (e0 != hipSuccess) return hip_status(e0, "tp_mlp_bwd_noalloc: scratch lookup");
  return hip_status(tpk::launch_mlp_bwd(static_cast<hipStream_t>(stream), dt, M, d, f, X, W1, W2, A, H, dY,
                                        dX, dW1, dW2, ws),
                    "tp_mlp_bwd_noalloc");
}

int tp_swiglu_fwd(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
                  const void* X, const void* W1, const void* W3, const void* W2,
                  void* G, void* U, void* H, void* Z) {
  TP_CHECK(mlp_common(dt, M, d, f));
  if ((G == nullptr) != (U == nullptr)) return fail(TP_E_NULL, "G and U must both be given or both be NULL");
  const size_t e = esize(dt);
  TP_CHECK(check_buffers({{"X", X, M * d * e}, {"W1", W1, d * f * e}, {"W3", W3, d * f * e},
                          {"W2", W2, f * d * e}},
                         {{"G", G, M * f * e}, {"U", U, M * f * e}, {"H", H, M * f * e}, {"Z", Z, M * d * e}},
                         {"X", "W1", "W3", "W2", "H", "Z"}));
  return hip_status(tpk::launch_swiglu_fwd(static_cast<hipStream_t>(stream), dt, M, d, f, X, W1, W3, W2,
                                           G, U, H, Z),
                    "tp_swiglu_fwd");
}

size_t tp_swiglu_bwd_workspace_bytes(tp_dtype_t dt, int64_t M, int64_t d, int64_t f) {
  if (mlp_common(dt, M, d, f) != TP_OK) return 0;
  return tpk::swiglu_bwd_ws_bytes(dt, M, d, f);
}

int tp_swiglu_bwd(void* stream, tp_dtype_t dt, int64_t M, int64_t d, int64_t f,
                  const void* X, const void* W1, const void* W3, const void* W2,
                  const void* G, const void* U, const void* H, const void* dY,
                  void* dX, float* dW1, float* dW3, float* dW2, void* ws, size_t ws_bytes) {
  TP_CHECK(mlp_common(dt, M, d, f));
  const size_t e = esize(dt);
  const size_t need = tpk::swiglu_bwd_ws_bytes(dt, M, d, f);
  TP_CHECK(check_buffers(
      {{"X", X, M * d * e}, {"W1", W1, d * f * e}, {"W3", W3, d * f * e}, {"W2", W2, f * d * e},
       {"G", G, M * f * e}, {"U", U, M * f * e}, {"H", H, M * f * e}, {"dY", dY, M * d * e}},
      {{"dX", dX, M * d * e}, {"dW1", dW1, d * f * (size_t)4}, {"dW3", dW3, d * f * (size_t)4}, {"dW2", dW2, f * d * (size_t)4},
       {"ws", ws, need}},
      {"X", "W1", "W3", "W2", "G", "U", "H", "dY", "dX", "dW1", "dW3", "dW2"}));
  if (!ws || ws_bytes < need)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes given, %zu required", ws ? ws_bytes : (size_t)0, need);
  return hip_status(tpk::launch_swiglu_bwd(static_cast<hipStream_t>(stream), dt, M, d, f, X, W1, W3, W2,
                                           G, U, H, dY, dX, dW1, dW3, dW2, ws),
                    "tp_swiglu_bwd");
}

static int attn_common(tp_dtype_t dt, int64_t b, int64_t s, int64_t d, int64_t h_local, int64_t d_head, int causal,
                float scale) {
  if (dt != TP_DT_BF16) return fail(TP_E_DTYPE, "attention supports TP_DT_BF16 only");
  TP_CHECK(check_dims({{"b", b}, {"s", s}, {"d", d}, {"h_local", h_local}, {"d_head", d_head}}));
  if (d_head != 64 && d_head != 128) return fail(TP_E_DIM, "d_head = %lld; 64 and 128 are supported", (long long)d_head);
  if (causal != 0 && causal != 1) return fail(TP_E_DIM, "causal must be 0 or 1");
  if (!std::isfinite(scale)) return fail(TP_E_DIM, "scale is not finite");
  TP_CHECK(check_mult8({{"d", d}}));
  const int64_t M = b * s, N = h_local * d_head;
  TP_CHECK(check_dims({{"b*s", M}, {"h_local*d_head", N}}));
  TP_CHECK(check_ld({{"d", d}, {"h_local*d_head", N}}));
  if (s > kMaxSeq) return fail(TP_E_DIM, "s = %lld exceeds 2^22", (long long)s);
  return TP_OK;
}

static int attn_kv_heads(int64_t h_local, int64_t h_kv) {
  if (h_kv <= 0 || h_kv > h_local || h_local % h_kv)
    return fail(TP_E_DIVIS, "h_kv_local = %lld must divide h_local = %lld", (long long)h_kv, (long long)h_local);
  return TP_OK;
}

static int attn_fwd_impl(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d, int64_t h_local,
                         int64_t h_kv, int64_t d_head, int causal, float scale, const void* X, const void* Wq,
                         const void* Wk, const void* Wv, const void* Wo, void* Q, void* K, void* V, void* O,
                         void* Z, float* L, const char* what) {
  TP_CHECK(attn_common(dt, b, s, d, h_local, d_head, causal, scale));
  TP_CHECK(attn_kv_heads(h_local, h_kv));
  const int64_t M = b * s, N = h_local * d_head, Nkv = h_kv * d_head;
  const size_t e = 2;
  TP_CHECK(check_buffers({{"X", X, M * d * e}, {"Wq", Wq, d * N * e}, {"Wk", Wk, d * Nkv * e},
                          {"Wv", Wv, d * Nkv * e}, {"Wo", Wo, N * d * e}},
                         {{"Q", Q, M * N * e}, {"K", K, M * Nkv * e}, {"V", V, M * Nkv * e},
                          {"O", O, M * N * e}, {"Z", Z, M * d * e}, {"L", L, (size_t)(b * h_local * s) * 4}},
                         {"X", "Wq", "Wk", "Wv", "Wo", "Q", "K", "V", "O", "Z"}));
  return hip_status(tpk::launch_attn_fwd(static_cast<hipStream_t>(stream), b, s, d, h_local, h_kv, d_head, causal,
                                         scale, X, Wq, Wk, Wv, Wo, Q, K, V, O, Z, L),
                    what);
}

int tp_attn_shard_fwd(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                      int64_t h_local, int64_t d_head, int causal, float scale,
                      const void* X, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                      void* Q, void* K, void* V, void* O, void* Z, float* L) {
  return attn_fwd_impl(stream, dt, b, s, d, h_local, h_local, d_head, causal, scale, X, Wq, Wk, Wv, Wo, Q, K, V,
                       O, Z, L, "tp_attn_shard_fwd");
}

int tp_attn_gqa_shard_fwd(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                          int64_t h_local, int64_t h_kv_local, int64_t d_head, int causal, float scale,
                          const void* X, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                          void* Q, void* K, void* V, void* O, void* Z, float* L) {
  return attn_fwd_impl(stream, dt, b, s, d, h_local, h_kv_local, d_head, causal, scale, X, Wq, Wk, Wv, Wo, Q, K,
                       V, O, Z, L, "tp_attn_gqa_shard_fwd");
}

static int attn_bwd_impl(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d, int64_t h_local,
                         int64_t h_kv, int64_t d_head, int causal, float scale, const void* X, const void* Wq,
                         const void* Wk, const void* Wv, const void* Wo, const void* Q, const void* K,
                         const void* V, const void* O, const float* L, const void* dY, void* dX, float* dWq,
                         float* dWk, float* dWv, float* dWo, void* ws, size_t ws_bytes, const char* what) {
  TP_CHECK(attn_common(dt, b, s, d, h_local, d_head, causal, scale));
  TP_CHECK(attn_kv_heads(h_local, h_kv));
  if (d_head != 128) return fail(TP_E_DIM, "the attention backward supports d_head = 128");
  const int64_t M = b * s, N = h_local * d_head, Nkv = h_kv * d_head;
  TP_CHECK(check_ld({{"(h_local + 2 h_kv_local)*d_head", N + 2 * Nkv}}));
  const size_t e = 2, need = tpk::attn_bwd_ws_bytes(b, s, d, h_local, h_kv, d_head);
  TP_CHECK(check_buffers(
      {{"X", X, M * d * e}, {"Wq", Wq, d * N * e}, {"Wk", Wk, d * Nkv * e}, {"Wv", Wv, d * Nkv * e},
       {"Wo", Wo, N * d * e}, {"Q", Q, M * N * e}, {"K", K, M * Nkv * e}, {"V", V, M * Nkv * e},
       {"O", O, M * N * e}, {"L", L, (size_t)(b * h_local * s) * 4}, {"dY", dY, M * d * e}},
      {{"dX", dX, M * d * e}, {"dWq", dWq, d * N * (size_t)4}, {"dWk", dWk, d * Nkv * (size_t)4},
       {"dWv", dWv, d * Nkv * (size_t)4}, {"dWo", dWo, N * d * (size_t)4}, {"ws", ws, need}},
      {"X", "Wq", "Wk", "Wv", "Wo", "Q", "K", "V", "O", "L", "dY", "dX", "dWq", "dWk", "dWv", "dWo"}));
  if (!ws || ws_bytes < need)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes given, %zu required", ws ? ws_bytes : (size_t)0, need);
  return hip_status(tpk::launch_attn_bwd(static_cast<hipStream_t>(stream), b, s, d, h_local, h_kv, d_head, causal,
                                         scale, X, Wq, Wk, Wv, Wo, Q, K, V, O, L, dY, dX, dWq, dWk, dWv, dWo,
                                         ws),
                    what);
}

size_t tp_attn_shard_bwd_workspace_bytes(tp_dtype_t dt, int64_t b, int64_t s, int64_t d, int64_t h_local,
                                         int64_t d_head) {
  if (attn_common(dt, b, s, d, h_local, d_head, 0, 1.f) != TP_OK) return 0;
  return tpk::attn_bwd_ws_bytes(b, s, d, h_local, h_local, d_head);
}

int tp_attn_shard_bwd(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                      int64_t h_local, int64_t d_head, int causal, float scale,
                      const void* X, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                      const void* Q, const void* K, const void* V, const void* O, const float* L,
                      const void* dY, void* dX, float* dWq, float* dWk, float* dWv, float* dWo,
                      void* ws, size_t ws_bytes) {
  return attn_bwd_impl(stream, dt, b, s, d, h_local, h_local, d_head, causal, scale, X, Wq, Wk, Wv, Wo, Q, K, V, O,
                       L, dY, dX, dWq, dWk, dWv, dWo, ws, ws_bytes, "tp_attn_shard_bwd");
}

size_t tp_attn_gqa_shard_bwd_workspace_bytes(tp_dtype_t dt, int64_t b, int64_t s, int64_t d, int64_t h_local,
                                             int64_t h_kv_local, int64_t d_head) {
  if (attn_common(dt, b, s, d, h_local, d_head, 0, 1.f) != TP_OK) return 0;
  if (attn_kv_heads(h_local, h_kv_local) != TP_OK) return 0;
  return tpk::attn_bwd_ws_bytes(b, s, d, h_local, h_kv_local, d_head);
}

int tp_attn_gqa_shard_bwd(void* stream, tp_dtype_t dt, int64_t b, int64_t s, int64_t d,
                          int64_t h_local, int64_t h_kv_local, int64_t d_head, int causal, float scale,
                          const void* X, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                          const void* Q, const void* K, const void* V, const void* O, const float* L,
                          const void* dY, void* dX, float* dWq, float* dWk, float* dWv, float* dWo,
                          void* ws, size_t ws_bytes) {
  return attn_bwd_impl(stream, dt, b, s, d, h_local, h_kv_local, d_head, causal, scale, X, Wq, Wk, Wv, Wo, Q, K, V,
                       O, L, dY, dX, dWq, dWk, dWv, dWo, ws, ws_bytes, "tp_attn_gqa_shard_bwd");
}

int tp_shard_reduce(void* stream, tp_dtype_t dt_in, tp_dtype_t dt_out, int64_t n_shards, int64_t numel,
                    const void* partials, int64_t shard_stride, const void* bias, int64_t bias_len,
                    void* out) {
  if (!dtype_ok(dt_in) || !dtype_ok(dt_out)) return fail(TP_E_DTYPE, "dtype is not TP_DT_F32 or TP_DT_BF16");
  if (n_shards <= 0 || n_shards > 4096) return fail(TP_E_DIM, "n_shards = %lld outside [1, 4096]", (long long)n_shards);
  if (numel <= 0) return fail(TP_E_DIM, "numel must be positive");
  if (shard_stride < numel) return fail(TP_E_DIM, "shard_stride %lld < numel %lld", (long long)shard_stride, (long long)numel);
  if (bias && bias_len <= 0) return fail(TP_E_DIM, "bias_len must be positive when bias is given");
  const size_t ei = esize(dt_in), eo = esize(dt_out);
  const size_t in_bytes = ((size_t)(n_shards - 1) * shard_stride + numel) * ei;
  const bool in_place = out == partials && dt_in == dt_out;
  const Span sp{"partials", partials, in_place ? 0 : in_bytes};
  TP_CHECK(check_buffers({sp, {"bias", bias, bias ? bias_len * ei : 0}},
                         {{"out", out, numel * eo}}, {"partials", "out"}));
  if (in_place) {  // out is block 0 itself: it must not reach into block 1 or the bias
    const Span rest{"partials[1:]", static_cast<const char*>(partials) + shard_stride * ei,
                    n_shards > 1 ? in_bytes - shard_stride * ei : 0};
    if (overlap({"out", out, numel * eo}, rest)) return fail(TP_E_ALIAS, "output out overlaps input partials");
  } else if (out == partials) {
    return fail(TP_E_ALIAS, "in-place shard-reduce needs dt_in == dt_out");
  }
  return hip_status(tpk::launch_shard_reduce(static_cast<hipStream_t>(stream), dt_in, dt_out, (int)n_shards,
                                             numel, partials, shard_stride, bias, bias ? bias_len : 0, out),
                    "tp_shard_reduce");
}

int tp_sp_reduce_scatter_ln(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t rows, int64_t cols,
                            int64_t index, const void* partials, int64_t shard_stride, const void* bias,
                            const void* residual, const uint8_t* keep, float p_drop, const void* gamma,
                            const void* beta, float eps, void* h_out, void* x_out) {
  if (!dtype_ok(dt)) return fail(TP_E_DTYPE, "dtype %d is not TP_DT_F32 or TP_DT_BF16", (int)dt);
  if (n_shards <= 0 || n_shards > 4096) return fail(TP_E_DIM, "n_shards = %lld outside [1, 4096]", (long long)n_shards);
  TP_CHECK(check_dims({{"rows", rows}, {"cols", cols}}));
  if (index < 0 || index >= n_shards)
    return fail(TP_E_DIM, "index = %lld outside [0, %lld)", (long long)index, (long long)n_shards);
  if (rows % n_shards)
    return fail(TP_E_DIVIS, "rows = %lld is not divisible by n_shards = %lld", (long long)rows, (long long)n_shards);
  TP_CHECK(check_mult8({{"cols", cols}}));
  const int64_t k = rows / n_shards;
  if (k > (int64_t(1) << 24)) return fail(TP_E_DIM, "stripe of %lld rows exceeds 2^24", (long long)k);
  const int64_t numel = rows * cols;
  if (shard_stride < numel)
    return fail(TP_E_DIM, "shard_stride %lld < rows*cols %lld", (long long)shard_stride, (long long)numel);
  if (shard_stride % 8) return fail(TP_E_DIVIS, "shard_stride = %lld must be a multiple of 8", (long long)shard_stride);
  if (keep && !(p_drop >= 0.0f && p_drop < 1.0f))
    return fail(TP_E_DIM, "p_drop = %g outside [0, 1)", (double)p_drop);
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(TP_E_DIM, "eps = %g must be positive and finite", (double)eps);
  const size_t e = esize(dt);
  const size_t stripe = (size_t)(k * cols);
  TP_CHECK(check_buffers({{"partials", partials, ((size_t)(n_shards - 1) * shard_stride + numel) * e},
                          {"bias", bias, bias ? cols * e : 0},
                          {"residual", residual, stripe * e},
                          {"keep", keep, keep ? stripe : 0},
                          {"gamma", gamma, cols * e},
                          {"beta", beta, cols * e}},
                         {{"h_out", h_out, stripe * e}, {"x_out", x_out, stripe * e}},
                         {"partials", "residual", "gamma", "beta", "h_out", "x_out"}));
  return hip_status(tpk::launch_sp_reduce_scatter_ln(static_cast<hipStream_t>(stream), dt, (int)n_shards, rows, cols,
                                                     index, partials, shard_stride, bias, residual, keep, p_drop,
                                                     gamma, beta, eps, h_out, x_out),
                    "tp_sp_reduce_scatter_ln");
}

static int sp_bwd_common(tp_dtype_t dt, int64_t n_shards, int64_t rows, int64_t cols) {
  if (!dtype_ok(dt)) return fail(TP_E_DTYPE, "dtype %d is not TP_DT_F32 or TP_DT_BF16", (int)dt);
  if (n_shards <= 0 || n_shards > 4096) return fail(TP_E_DIM, "n_shards = %lld outside [1, 4096]", (long long)n_shards);
  TP_CHECK(check_dims({{"rows", rows}, {"cols", cols}}));
  if (rows % n_shards)
    return fail(TP_E_DIVIS, "rows = %lld is not divisible by n_shards = %lld", (long long)rows, (long long)n_shards);
  TP_CHECK(check_mult8({{"cols", cols}}));
  if (cols > 16384) return fail(TP_E_DIM, "cols = %lld exceeds 16384 (the backward keeps a row in registers)",
                                (long long)cols);
  if (rows / n_shards > (int64_t(1) << 24))
    return fail(TP_E_DIM, "stripe of %lld rows exceeds 2^24", (long long)(rows / n_shards));
  return TP_OK;
}

size_t tp_sp_ln_bwd_workspace_bytes(tp_dtype_t dt, int64_t n_shards, int64_t rows, int64_t cols) {
  if (sp_bwd_common(dt, n_shards, rows, cols) != TP_OK) return 0;
  return tpk::sp_ln_bwd_ws_bytes(rows, cols, (int)n_shards);
}

int tp_sp_ln_bwd_reduce_scatter(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t rows, int64_t cols,
                                int64_t index, const void* dx_partials, int64_t shard_stride, const void* h,
                                const void* gamma, float eps, const uint8_t* keep, float p_drop,
                                const void* dres, void* dh_out, void* dy_out, float* dgamma, float* dbeta,
                                float* dbias, void* ws, size_t ws_bytes) {
  TP_CHECK(sp_bwd_common(dt, n_shards, rows, cols));
  if (index < 0 || index >= n_shards)
    return fail(TP_E_DIM, "index = %lld outside [0, %lld)", (long long)index, (long long)n_shards);
  const int64_t numel = rows * cols;
  if (shard_stride < numel)
    return fail(TP_E_DIM, "shard_stride %lld < rows*cols %lld", (long long)shard_stride, (long long)numel);
  if (shard_stride % 8) return fail(TP_E_DIVIS, "shard_stride = %lld must be a multiple of 8", (long long)shard_stride);
  if (keep && !(p_drop >= 0.0f && p_drop < 1.0f))
    return fail(TP_E_DIM, "p_drop = %g outside [0, 1)", (double)p_drop);
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(TP_E_DIM, "eps = %g must be positive and finite", (double)eps);
  const size_t e = esize(dt);
  const size_t stripe = (size_t)(rows / n_shards * cols);
  const size_t need = tpk::sp_ln_bwd_ws_bytes(rows, cols, (int)n_shards);
  TP_CHECK(check_buffers({{"dx_partials", dx_partials, ((size_t)(n_shards - 1) * shard_stride + numel) * e},
                          {"h", h, stripe * e},
                          {"gamma", gamma, cols * e},
                          {"keep", keep, keep ? stripe : 0},
                          {"dres", dres, dres ? stripe * e : 0}},
                         {{"dh_out", dh_out, stripe * e}, {"dy_out", dy_out, stripe * e},
                          {"dgamma", dgamma, (size_t)cols * 4, 4}, {"dbeta", dbeta, (size_t)cols * 4, 4},
                          {"dbias", dbias, dbias ? (size_t)cols * 4 : 0, 4}, {"ws", ws, need}},
                         {"dx_partials", "h", "gamma", "dh_out", "dy_out", "dgamma", "dbeta"}));
  if (!ws || ws_bytes < need)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes given, %zu required", ws ? ws_bytes : (size_t)0, need);
  return hip_status(tpk::launch_sp_ln_bwd(static_cast<hipStream_t>(stream), dt, (int)n_shards, rows, cols, index,
                                          dx_partials, shard_stride, h, gamma, eps, keep, p_drop, dres, dh_out,
                                          dy_out, dgamma, dbeta, dbias, ws),
                    "tp_sp_ln_bwd_reduce_scatter");
}

int tp_sp_all_gather(void* stream, tp_dtype_t dt, int64_t n_shards, int64_t stripe_rows, int64_t cols,
                     const void* const* stripes, void* full) {
  if (!dtype_ok(dt)) return fail(TP_E_DTYPE, "dtype %d is not TP_DT_F32 or TP_DT_BF16", (int)dt);
  if (n_shards <= 0 || n_shards > tpk::kSpMaxShards)
    return fail(TP_E_DIM, "n_shards = %lld outside [1, %d]", (long long)n_shards, tpk::kSpMaxShards);
  TP_CHECK(check_dims({{"stripe_rows", stripe_rows}, {"cols", cols}}));
  TP_CHECK(check_mult8({{"cols", cols}}));
  if (!stripes) return fail(TP_E_NULL, "stripes is NULL");
  const size_t bytes = (size_t)(stripe_rows * cols) * esize(dt);
  const Span out{"full", full, bytes * n_shards};
  TP_CHECK(check_buffers({}, {out}, {"full"}));
  const void* src[tpk::kSpMaxShards];
  for (int64_t j = 0; j < n_shards; ++j) {
    char name[32];
    std::snprintf(name, sizeof name, "stripes[%lld]", (long long)j);
    const void* p = stripes[j];
    if (!p) return fail(TP_E_NULL, "%s is NULL", name);
    if (reinterpret_cast<uintptr_t>(p) & 15u) return fail(TP_E_ALIGN, "%s (%p) is not 16-byte aligned", name, p);
    const void* home = static_cast<const char*>(full) + bytes * j;
    if (p == home) {          // already in place: nothing to copy
      src[j] = nullptr;
      continue;
    }
    if (overlap(out, {name, p, bytes})) return fail(TP_E_ALIAS, "output full overlaps input %s", name);
    src[j] = p;
  }
  return hip_status(tpk::launch_sp_all_gather(static_cast<hipStream_t>(stream), dt, (int)n_shards, stripe_rows, cols,
                                              src, full),
                    "tp_sp_all_gather");
}

int tp_vocab_embed_fwd(void* stream, tp_dtype_t dt, int64_t n_tokens, int64_t d, int64_t vocab_local,
                       int64_t vocab_start, const int64_t* ids, const void* E_local, void* Y) {
  TP_CHECK(vocab_common(dt, n_tokens, d, vocab_local, vocab_start));
  const size_t e = esize(dt);
  TP_CHECK(check_buffers({{"ids", ids, (size_t)n_tokens * 8, 8}, {"E_local", E_local, (size_t)(vocab_local * d) * e}},
                         {{"Y", Y, (size_t)(n_tokens * d) * e}}, {"ids", "E_local", "Y"}));
  return hip_status(tpk::launch_vocab_embed_fwd(static_cast<hipStream_t>(stream), dt, n_tokens, d, vocab_local,
                                                vocab_start, ids, E_local, Y),
                    "tp_vocab_embed_fwd");
}

int tp_vocab_embed_bwd(void* stream, tp_dtype_t dt, int64_t n_tokens, int64_t d, int64_t vocab_local,
                       int64_t vocab_start, const int64_t* ids, const void* dY, float* dE_local) {
  TP_CHECK(vocab_common(dt, n_tokens, d, vocab_local, vocab_start));
  const size_t e = esize(dt);
  TP_CHECK(check_buffers({{"ids", ids, (size_t)n_tokens * 8, 8}, {"dY", dY, (size_t)(n_tokens * d) * e}},
                         {{"dE_local", dE_local, (size_t)(vocab_local * d) * 4}}, {"ids", "dY", "dE_local"}));
  return hip_status(tpk::launch_vocab_embed_bwd(static_cast<hipStream_t>(stream), dt, n_tokens, d, vocab_local,
                                                vocab_start, ids, dY, dE_local),
                    "tp_vocab_embed_bwd");
}

size_t tp_vocab_ce_fwd_workspace_bytes(tp_dtype_t dt, int64_t n_tokens, int64_t d, int64_t vocab_local) {
  if (vocab_common(dt, n_tokens, d, vocab_local, 0) != TP_OK) return 0;
  return tpk::vocab_ce_fwd_ws_bytes(dt, n_tokens, vocab_local);
}

int tp_vocab_ce_fwd(void* stream, tp_dtype_t dt, int64_t n_tokens, int64_t d, int64_t vocab_local,
                    int64_t vocab_start, const void* X, const void* E_local, const int64_t* targets,
                    void* logits, float* stats, void* ws, size_t ws_bytes) {
  TP_CHECK(vocab_common(dt, n_tokens, d, vocab_local, vocab_start));
  const size_t e = esize(dt);
  const size_t need = tpk::vocab_ce_fwd_ws_bytes(dt, n_tokens, vocab_local);
  TP_CHECK(check_buffers({{"X", X, (size_t)(n_tokens * d) * e},
                          {"E_local", E_local, (size_t)(vocab_local * d) * e},
                          {"targets", targets, (size_t)n_tokens * 8, 8}},
                         {{"logits", logits, (size_t)(n_tokens * vocab_local) * e},
                          {"stats", stats, (size_t)n_tokens * 12, 4}, {"ws", ws, need}},
                         {"X", "E_local", "targets", "logits", "stats"}));
  if (need && (!ws || ws_bytes < need))
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes given, %zu required", ws ? ws_bytes : (size_t)0, need);
  return hip_status(tpk::launch_vocab_ce_fwd(static_cast<hipStream_t>(stream), dt, n_tokens, d, vocab_local,
                                             vocab_start, X, E_local, targets, logits, stats, ws),
                    "tp_vocab_ce_fwd");
}

int tp_vocab_ce_combine(void* stream, int64_t n_shards, int64_t n_tokens, const float* stats,
                        int64_t shard_stride, float* loss, float* lse) {
  if (n_shards <= 0 || n_shards > 4096) return fail(TP_E_DIM, "n_shards = %lld outside [1, 4096]", (long long)n_shards);
  TP_CHECK(check_dims({{"n_tokens", n_tokens}}));
  if (shard_stride < 3 * n_tokens)
    return fail(TP_E_DIM, "shard_stride %lld < 3 * n_tokens %lld", (long long)shard_stride, (long long)(3 * n_tokens));
  TP_CHECK(check_buffers({{"stats", stats, ((size_t)(n_shards - 1) * shard_stride + 3 * n_tokens) * 4, 4}},
                         {{"loss", loss, (size_t)n_tokens * 4, 4}, {"lse", lse, (size_t)n_tokens * 4, 4}},
                         {"stats", "loss", "lse"}));
  return hip_status(tpk::launch_vocab_ce_combine(static_cast<hipStream_t>(stream), (int)n_shards, n_tokens, stats,
                                                 shard_stride, loss, lse),
                    "tp_vocab_ce_combine");
}

size_t tp_vocab_ce_bwd_workspace_bytes(tp_dtype_t dt, int64_t n_tokens, int64_t d, int64_t vocab_local) {
  if (vocab_common(dt, n_tokens, d, vocab_local, 0) != TP_OK) return 0;
  return tpk::vocab_ce_bwd_ws_bytes(dt, n_tokens, d, vocab_local);
}

int tp_vocab_ce_bwd(void* stream, tp_dtype_t dt, int64_t n_tokens, int64_t d, int64_t vocab_local,
                    int64_t vocab_start, const void* X, const void* E_local, const int64_t* targets,
                    const void* logits, const float* lse, const float* dloss, void* dX, float* dE,
                    void* ws, size_t ws_bytes) {
  TP_CHECK(vocab_common(dt, n_tokens, d, vocab_local, vocab_start));
  const size_t e = esize(dt);
  const size_t need = tpk::vocab_ce_bwd_ws_bytes(dt, n_tokens, d, vocab_local);
  TP_CHECK(check_buffers({{"X", X, (size_t)(n_tokens * d) * e},
                          {"E_local", E_local, (size_t)(vocab_local * d) * e},
                          {"targets", targets, (size_t)n_tokens * 8, 8},
                          {"logits", logits, (size_t)(n_tokens * vocab_local) * e},
                          {"lse", lse, (size_t)n_tokens * 4, 4},
                          {"dloss", dloss, (size_t)n_tokens * 4, 4}},
                         {{"dX", dX, (size_t)(n_tokens * d) * e},
                          {"dE", dE, (size_t)(vocab_local * d) * 4},
                          {"ws", ws, need}},
                         {"X", "E_local", "targets", "logits", "lse", "dloss", "dX", "dE"}));
  if (!ws || ws_bytes < need)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes, %zu needed", ws ? ws_bytes : (size_t)0, need);
  return hip_status(tpk::launch_vocab_ce_bwd(static_cast<hipStream_t>(stream), dt, n_tokens, d, vocab_local,
                                             vocab_start, X, E_local, targets, logits, lse, dloss, dX, dE, ws),
                    "tp_vocab_ce_bwd");
}

}  // extern "C"
