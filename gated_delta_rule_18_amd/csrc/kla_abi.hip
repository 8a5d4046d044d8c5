// C ABI of the KLA library: argument checks, then stream-ordered launches.
// Declarations and the contract of every entry point: include/kla.h.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kla.h"
#include "kla_launch.h"

// Workspace of kla_chunk_fwd_noalloc, for callers that cannot allocate: one copy per device, held
// from the library's first use of that device until the process ends. In host code `scratch` only
// names the symbol; its device address on each device comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[KLA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

kla_status_t fail(kla_status_t st, const char* fmt, const char* what) {
  std::snprintf(g_last_error, sizeof(g_last_error), fmt, what);
  return st;
}

kla_status_t fail(kla_status_t st, const char* fmt, const char* what, const char* detail) {
  std::snprintf(g_last_error, sizeof(g_last_error), fmt, what, detail);
  return st;
}

kla_status_t launched(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_last_error[0] = '\0';
    return KLA_OK;
  }
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
  return KLA_ERR_LAUNCH;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool supported_head(int64_t d) { return d == 64 || d == 128; }

// Products of non-negative sizes, refusing anything past 2^62 elements.
bool mul_ok(int64_t& acc, int64_t x) {
  if (x < 0) return false;
  if (x != 0 && acc > (int64_t(1) << 62) / x) return false;
  acc *= x;
  return true;
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device: looked up on the first call on each device,
// with that device current, and kept per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* kla_status_string(kla_status_t status) {
  switch (status) {
    case KLA_OK: return "KLA_OK";
    case KLA_ERR_INVALID_VALUE: return "KLA_ERR_INVALID_VALUE: bad argument";
    case KLA_ERR_NOT_SUPPORTED: return "KLA_ERR_NOT_SUPPORTED: head size or chunk length not provided";
    case KLA_ERR_LAUNCH: return "KLA_ERR_LAUNCH: HIP launch failed";
  }
  return "unknown kla_status_t";
}

const char* kla_last_error(void) { return g_last_error; }

kla_status_t kla_prepare_beta(const void* k, const float* eta, const float* log_alpha, float* beta_out,
                              float* gcum_out, int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t chunk,
                              float eps, kla_dtype_t dt, void* stream) {
  if (dt != KLA_F32 && dt != KLA_BF16) return fail(KLA_ERR_INVALID_VALUE, "%s: unknown dtype", "kla_prepare_beta");
  if (B < 0 || T < 0 || H < 0) return fail(KLA_ERR_INVALID_VALUE, "%s: negative size", "kla_prepare_beta");
  if (!supported_head(d_k)) return fail(KLA_ERR_NOT_SUPPORTED, "%s: d_k must be 64 or 128", "kla_prepare_beta");
  if (chunk != kla::kChunk) return fail(KLA_ERR_NOT_SUPPORTED, "%s: chunk must be 64", "kla_prepare_beta");
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(KLA_ERR_INVALID_VALUE, "%s: eps must be finite and >= 0", "kla_prepare_beta");
  int64_t n = 1;
  if (!mul_ok(n, B) || !mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, d_k))
    return fail(KLA_ERR_INVALID_VALUE, "%s: size overflow", "kla_prepare_beta");
  if (B == 0 || T == 0 || H == 0) {
    g_last_error[0] = '\0';
    return KLA_OK;
  }
  if (B * H * ((T + kla::kChunk - 1) / kla::kChunk) > 0x7fffffffLL)
    return fail(KLA_ERR_INVALID_VALUE, "%s: grid too large", "kla_prepare_beta");
  if (!k || !eta || !log_alpha || !beta_out)
    return fail(KLA_ERR_INVALID_VALUE, "%s: null pointer", "kla_prepare_beta");
  if (!aligned(k, 16) || !aligned(eta, 4) || !aligned(log_alpha, 4) || !aligned(beta_out, 4) ||
      !aligned(gcum_out, 4))
    return fail(KLA_ERR_INVALID_VALUE, "%s: misaligned pointer", "kla_prepare_beta");
  const int64_t tok = B * T * H;
  const Range outs[2] = {range("beta_out", beta_out, tok * 4), range("gcum_out", gcum_out, tok * 4)};
  const Range ins[3] = {range("k", k, tok * d_k * (dt == KLA_BF16 ? 2 : 4)), range("eta", eta, tok * 4),
                        range("log_alpha", log_alpha, tok * 4)};
  if (overlap(outs[0], outs[1])) return fail(KLA_ERR_INVALID_VALUE, "%s: outputs overlap", "kla_prepare_beta");
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(KLA_ERR_INVALID_VALUE, "kla_prepare_beta: %s overlaps an input", o.name);
  kla::PrepareArgs a{k, eta, log_alpha, beta_out, gcum_out, B, T, H, d_k, eps, dt == KLA_BF16};
  return launched(kla::launch_prepare_beta(a, static_cast<hipStream_t>(stream)), "kla_prepare_beta");
}

size_t kla_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                    kla_dtype_t dt) {
  if (B <= 0 || T <= 0 || H <= 0 || !supported_head(d_k) || !supported_head(d_v) || chunk != kla::kChunk)
    return 0;
  return kla::chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16);
}

size_t kla_chunk_fwd_seg_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                        int64_t segments, kla_dtype_t dt) {
  if (B <= 0 || T <= 0 || H <= 0 || !supported_head(d_k) || !supported_head(d_v) || chunk != kla::kChunk ||
      segments < 0)
    return 0;
  return kla::chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16, segments);
}

size_t kla_kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                        kla_dtype_t dt) {
  if (B <= 0 || T <= 0 || H <= 0 || !supported_head(d_k) || !supported_head(d_v) || chunk != kla::kChunk)
    return 0;
  return kla::chunk_kda_fwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16);
}

size_t kla_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                    kla_dtype_t dt) {
  if (B <= 0 || T <= 0 || H <= 0 || !supported_head(d_k) || !supported_head(d_v) || chunk != kla::kChunk)
    return 0;
  return kla::chunk_bwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16);
}

size_t kla_kda_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                        kla_dtype_t dt) {
  if (B <= 0 || T <= 0 || H <= 0 || !supported_head(d_k) || !supported_head(d_v) || chunk != kla::kChunk)
    return 0;
  return kla::chunk_kda_bwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16);
}

}  // extern "C"

namespace {

// kla_chunk_fwd, kla_gdn_chunk_fwd and kla_kda_chunk_fwd: eta is eta (Kaczmarz step) or beta itself
// (beta_given, where a scalar log_alpha may be null for alpha = 1); with kda, log_alpha is the
// per-channel log a [B, T, H, d_k] and required.
// segments: the scan's sequence segments (0: the library's plan). use_scratch: the workspace is the
// library's static `scratch` (workspace and workspace_bytes are ignored).
kla_status_t chunk_fwd_impl(const char* fn, bool beta_given, bool kda, const void* q, const void* k, const void* v,
                            const float* eta, const float* log_alpha, const float* state_in, float* state_out,
                            void* o, int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                            float eps, kla_dtype_t dt, void* workspace, size_t workspace_bytes, void* stream,
                            int64_t segments = 0, bool use_scratch = false, bool train = false) {
  if (dt != KLA_F32 && dt != KLA_BF16) return fail(KLA_ERR_INVALID_VALUE, "%s: unknown dtype", fn);
  if (B < 0 || T < 0 || H < 0) return fail(KLA_ERR_INVALID_VALUE, "%s: negative size", fn);
  if (segments < 0) return fail(KLA_ERR_INVALID_VALUE, "%s: negative segment count", fn);
  if (!supported_head(d_k) || !supported_head(d_v))
    return fail(KLA_ERR_NOT_SUPPORTED, "%s: d_k and d_v must be 64 or 128", fn);
  if (chunk != kla::kChunk) return fail(KLA_ERR_NOT_SUPPORTED, "%s: chunk must be 64", fn);
  if (!std::isfinite(eps) || eps < 0.f) return fail(KLA_ERR_INVALID_VALUE, "%s: eps must be finite and >= 0", fn);
  int64_t n = 1;
  if (!mul_ok(n, B) || !mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, d_k > d_v ? d_k : d_v))
    return fail(KLA_ERR_INVALID_VALUE, "%s: size overflow", fn);
  if (B == 0 || H == 0) {
    g_last_error[0] = '\0';
    return KLA_OK;
  }
  if (B * H * 8 > 0x7fffffffLL || B * H * ((T + kla::kChunk - 1) / kla::kChunk) > 0x7fffffffLL)
    return fail(KLA_ERR_INVALID_VALUE, "%s: grid too large", fn);
  // The kernels address one batch's rows of q/k/v/o (and, with kda, of the fp32 log a), and one
  // head's workspace, with 32-bit byte offsets (up to one chunk past T).
  const int64_t row_bytes = std::max((d_k > d_v ? d_k : d_v) * (dt == KLA_BF16 ? 2 : 4), kda ? d_k * 4 : int64_t(0));
  if ((T + kla::kChunk) * H * row_bytes >= (int64_t(1) << 31))
    return fail(KLA_ERR_NOT_SUPPORTED, "%s: T * H * d of one batch entry must stay below 2 GiB", fn);
  if (T > 0 && (!q || !k || !v || !eta || (!log_alpha && (!beta_given || kda)) || !o))
    return fail(KLA_ERR_INVALID_VALUE, "%s: null pointer", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(state_in, 16) ||
      !aligned(state_out, 16) || !aligned(eta, 4) || !aligned(log_alpha, kda ? 16 : 4))
    return fail(KLA_ERR_INVALID_VALUE, "%s: misaligned pointer", fn);
  // (the training forward fills the backward's workspace)
  if (train && kda && !kla::chunk_grad_kda_supported(d_k, d_v, dt == KLA_BF16))
    return fail(KLA_ERR_NOT_SUPPORTED, "%s: fp32 gradients need d_k = d_v = 64", fn);
  const size_t need = train ? (kda ? kla::chunk_kda_bwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16)
                                   : kla::chunk_bwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16))
                      : kda ? kla::chunk_kda_fwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16)
                            : kla::chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16, segments);
  if (use_scratch) {
    workspace = nullptr;
    workspace_bytes = 0;
    if (T > 0 && need > KLA_NOALLOC_SCRATCH_BYTES) {
      char msg[160];
      std::snprintf(msg, sizeof(msg), "these sizes need %zu bytes of workspace, more than the %zu of the static scratch",
                    need, (size_t)KLA_NOALLOC_SCRATCH_BYTES);
      return fail(KLA_ERR_NOT_SUPPORTED, "%s: %s", fn, msg);
    }
    if (T > 0 && need > 0) {
      const hipError_t e = scratch_address(&workspace);
      if (e != hipSuccess) return launched(e, fn);
      workspace_bytes = KLA_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (T > 0 && need > 0 && (!workspace || workspace_bytes < need))
    return fail(KLA_ERR_INVALID_VALUE, "%s: workspace missing or too small", fn);
  const int64_t es = dt == KLA_BF16 ? 2 : 4;
  const int64_t tok = B * T * H;
  const int64_t sbytes = B * H * d_k * d_v * 4;
  const Range rq = range("q", q, tok * d_k * es), rk = range("k", k, tok * d_k * es),
              rv = range("v", v, tok * d_v * es), re = range("eta", eta, tok * 4),
              rl = range("log_alpha", log_alpha, tok * 4 * (kda ? d_k : 1)), rsi = range("state_in", state_in, sbytes),
              rso = range("state_out", state_out, sbytes), ro = range("o", o, tok * d_v * es),
              rw = range("workspace", workspace, (int64_t)(need > 0 ? workspace_bytes : 0));
  const Range* ins[6] = {&rq, &rk, &rv, &re, &rl, &rsi};
  for (const Range* i : ins) {
    if (overlap(ro, *i)) return fail(KLA_ERR_INVALID_VALUE, "%s: o overlaps %s", fn, i->name);
    if (i != &rsi && overlap(rso, *i)) return fail(KLA_ERR_INVALID_VALUE, "%s: state_out overlaps %s", fn, i->name);
    if (overlap(rw, *i)) return fail(KLA_ERR_INVALID_VALUE, "%s: workspace overlaps %s", fn, i->name);
  }
  if (overlap(ro, rso) || overlap(rw, ro) || overlap(rw, rso))
    return fail(KLA_ERR_INVALID_VALUE, "%s: outputs overlap", fn);
  if (state_in && state_out && state_in != state_out && overlap(rsi, rso))
    return fail(KLA_ERR_INVALID_VALUE, "%s: state_in and state_out overlap without being equal", fn);
  if (T == 0 && !state_out) {
    g_last_error[0] = '\0';
    return KLA_OK;
  }
  kla::ChunkArgs a{q, k, v, eta, log_alpha, state_in, state_out, o, B, T, H, d_k, d_v, eps, dt == KLA_BF16,
                   workspace, workspace_bytes, beta_given, segments};
  return launched(train ? (kda ? kla::launch_chunk_kda_fwd_train(a, static_cast<hipStream_t>(stream))
                               : kla::launch_chunk_fwd_train(a, static_cast<hipStream_t>(stream)))
                  : kda ? kla::launch_chunk_kda_fwd(a, static_cast<hipStream_t>(stream))
                        : kla::launch_chunk_fwd(a, static_cast<hipStream_t>(stream)),
                  fn);
}

// kla_chunk_bwd, kla_gdn_chunk_bwd and kla_kda_chunk_bwd (as chunk_fwd_impl; deta receives dL/dbeta
// when beta_given; with kda, log_alpha / dlog_alpha are log a / dlog a [B, T, H, d_k] and required);
// saved: the workspace holds what the training forward left (kla_chunk_bwd_saved and its gdn form).
kla_status_t chunk_bwd_impl(const char* fn, bool beta_given, bool kda, const void* q, const void* k, const void* v,
                            const float* eta, const float* log_alpha, const float* state_in, const void* dout,
                            const float* dstate_out, void* dq, void* dk, void* dv, float* deta, float* dlog_alpha,
                            float* dstate_in, int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                            int64_t chunk, float eps, kla_dtype_t dt, void* workspace, size_t workspace_bytes,
                            void* stream, bool saved = false) {
  if (dt != KLA_F32 && dt != KLA_BF16) return fail(KLA_ERR_INVALID_VALUE, "%s: unknown dtype", fn);
  if (B < 0 || T < 0 || H < 0) return fail(KLA_ERR_INVALID_VALUE, "%s: negative size", fn);
  if (!supported_head(d_k) || !supported_head(d_v))
    return fail(KLA_ERR_NOT_SUPPORTED, "%s: d_k and d_v must be 64 or 128", fn);
  if (!(kda ? kla::chunk_grad_kda_supported(d_k, d_v, dt == KLA_BF16) : kla::chunk_grad_supported(d_k, d_v, dt == KLA_BF16)))
    return fail(KLA_ERR_NOT_SUPPORTED, "%s: fp32 gradients need d_k = d_v = 64", fn);
  if (chunk != kla::kChunk) return fail(KLA_ERR_NOT_SUPPORTED, "%s: chunk must be 64", fn);
  if (!std::isfinite(eps) || eps < 0.f) return fail(KLA_ERR_INVALID_VALUE, "%s: eps must be finite and >= 0", fn);
  int64_t n = 1;
  if (!mul_ok(n, B) || !mul_ok(n, T) || !mul_ok(n, H) || !mul_ok(n, d_k > d_v ? d_k : d_v))
    return fail(KLA_ERR_INVALID_VALUE, "%s: size overflow", fn);
  if (B == 0 || H == 0) {
    g_last_error[0] = '\0';
    return KLA_OK;
  }
  const int64_t es = dt == KLA_BF16 ? 2 : 4;
  const int64_t nchunks = (T + kla::kChunk - 1) / kla::kChunk;
  if (B * H * 8 > 0x7fffffffLL || B * H * nchunks > 0x7fffffffLL)
    return fail(KLA_ERR_INVALID_VALUE, "%s: grid too large", fn);
  // 32-bit byte offsets within one batch entry's rows and within one head's workspace blocks.
  if ((T + kla::kChunk) * H * (d_k > d_v ? d_k : d_v) * es >= (int64_t(1) << 31) ||
      (kda && (T + kla::kChunk) * H * d_k * 4 >= (int64_t(1) << 31)) ||
      (nchunks + 1) * d_k * d_v * es >= (int64_t(1) << 31) ||
      (kda && (nchunks + 1) * kla::kChunk * d_k * es >= (int64_t(1) << 31)))
    return fail(KLA_ERR_NOT_SUPPORTED, "%s: T * H * d of one batch entry must stay below 2 GiB", fn);
  if (T > 0 && (!q || !k || !v || !eta || (!log_alpha && (!beta_given || kda)) || !dout || !dq || !dk || !dv ||
                !deta || (log_alpha && !dlog_alpha)))
    return fail(KLA_ERR_INVALID_VALUE, "%s: null pointer", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
      !aligned(dk, 16) || !aligned(dv, 16) || !aligned(state_in, 16) || !aligned(dstate_out, 16) ||
      !aligned(dstate_in, 16) || !aligned(eta, 4) || !aligned(log_alpha, kda ? 16 : 4) || !aligned(deta, 4) ||
      !aligned(dlog_alpha, 4) || !aligned(workspace, 16))
    return fail(KLA_ERR_INVALID_VALUE, "%s: misaligned pointer", fn);
  const size_t need = kda ? kla::chunk_kda_bwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16)
                          : kla::chunk_bwd_workspace_bytes(B, T, H, d_k, d_v, dt == KLA_BF16);
  if (T > 0 && (!workspace || workspace_bytes < need))
    return fail(KLA_ERR_INVALID_VALUE, "%s: workspace missing or too small", fn);
  const int64_t tok = B * T * H;
  const int64_t sbytes = B * H * d_k * d_v * 4;
  const Range ins[8] = {range("q", q, tok * d_k * es),          range("k", k, tok * d_k * es),
                        range("v", v, tok * d_v * es),          range("eta", eta, tok * 4),
                        range("log_alpha", log_alpha, tok * 4 * (kda ? d_k : 1)), range("state_in", state_in, sbytes),
                        range("do", dout, tok * d_v * es),      range("dstate_out", dstate_out, sbytes)};
  const Range outs[7] = {range("dq", dq, T > 0 ? tok * d_k * es : 0),
                         range("dk", dk, T > 0 ? tok * d_k * es : 0),
                         range("dv", dv, T > 0 ? tok * d_v * es : 0),
                         range("deta", deta, T > 0 ? tok * 4 : 0),
                         range("dlog_alpha", dlog_alpha, T > 0 ? tok * 4 * (kda ? d_k : 1) : 0),
                         range("dstate_in", dstate_in, sbytes),
                         range("workspace", workspace, T > 0 ? (int64_t)workspace_bytes : 0)};
  for (int i = 0; i < 7; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(KLA_ERR_INVALID_VALUE, "%s: %s overlaps an input", fn, outs[i].name);
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return fail(KLA_ERR_INVALID_VALUE, "%s: %s overlaps another output", fn,
                                                 outs[i].name);
  }
  if (T == 0 && !dstate_in) {
    g_last_error[0] = '\0';
    return KLA_OK;
  }
  kla::ChunkBwdArgs a{q,  k,  v,    eta,        log_alpha, state_in, dout, dstate_out, dq,  dk,
                      dv, deta, dlog_alpha, dstate_in, B,  T,        H,    d_k,        d_v, eps,
                      dt == KLA_BF16, workspace, workspace_bytes, beta_given, kda, saved};
  return launched(kla::launch_chunk_bwd(a, static_cast<hipStream_t>(stream)), fn);
}

// kla_decode_step, kla_gdn_decode_step and kla_kda_decode_step (as chunk_fwd_impl).
kla_status_t decode_impl(const char* fn, bool beta_given, bool kda, const void* q, const void* k, const void* v,
                         const float* eta, const float* log_alpha, float* state, void* o, int64_t B, int64_t H,
                         int64_t d_k, int64_t d_v, float eps, kla_dtype_t dt, void* stream) {
  if (dt != KLA_F32 && dt != KLA_BF16) return fail(KLA_ERR_INVALID_VALUE, "%s: unknown dtype", fn);
  if (B < 0 || H < 0) return fail(KLA_ERR_INVALID_VALUE, "%s: negative size", fn);
  if (!supported_head(d_k) || !supported_head(d_v))
    return fail(KLA_ERR_NOT_SUPPORTED, "%s: d_k and d_v must be 64 or 128", fn);
  if (!std::isfinite(eps) || eps < 0.f) return fail(KLA_ERR_INVALID_VALUE, "%s: eps must be finite and >= 0", fn);
  int64_t n = 1;
  if (!mul_ok(n, B) || !mul_ok(n, H) || !mul_ok(n, d_k) || !mul_ok(n, d_v))
    return fail(KLA_ERR_INVALID_VALUE, "%s: size overflow", fn);
  if (B == 0 || H == 0) {
    g_last_error[0] = '\0';
    return KLA_OK;
  }
  if ((B * H + 8) * 8 > 0x7fffffffLL) return fail(KLA_ERR_INVALID_VALUE, "%s: grid too large", fn);
  if (!q || !k || !v || !eta || (!log_alpha && (!beta_given || kda)) || !state || !o)
    return fail(KLA_ERR_INVALID_VALUE, "%s: null pointer", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(state, 16) ||
      !aligned(eta, 4) || !aligned(log_alpha, 4))
    return fail(KLA_ERR_INVALID_VALUE, "%s: misaligned pointer", fn);
  const int64_t es = dt == KLA_BF16 ? 2 : 4;
  const Range rs = range("state", state, B * H * d_k * d_v * 4), ro = range("o", o, B * H * d_v * es);
  const Range ins[5] = {range("q", q, B * H * d_k * es), range("k", k, B * H * d_k * es),
                        range("v", v, B * H * d_v * es), range("eta", eta, B * H * 4),
                        range("log_alpha", log_alpha, B * H * 4 * (kda ? d_k : 1))};
  if (overlap(ro, rs)) return fail(KLA_ERR_INVALID_VALUE, "%s: o overlaps state", fn);
  for (const Range& i : ins) {
    if (overlap(ro, i)) return fail(KLA_ERR_INVALID_VALUE, "%s: o overlaps %s", fn, i.name);
    if (overlap(rs, i)) return fail(KLA_ERR_INVALID_VALUE, "%s: state overlaps %s", fn, i.name);
  }
  kla::DecodeArgs a{q, k, v, eta, log_alpha, state, o, B, H, d_k, d_v, eps, dt == KLA_BF16, beta_given, kda};
  return launched(kla::launch_decode_step(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

kla_status_t kla_chunk_fwd(const void* q, const void* k, const void* v, const float* eta, const float* log_alpha,
                           const float* state_in, float* state_out, void* o, int64_t B, int64_t T, int64_t H,
                           int64_t d_k, int64_t d_v, int64_t chunk, float eps, kla_dtype_t dt, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl("kla_chunk_fwd", false, false, q, k, v, eta, log_alpha, state_in, state_out, o, B, T, H, d_k, d_v,
                        chunk, eps, dt, workspace, workspace_bytes, stream);
}

kla_status_t kla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* eta,
                                   const float* log_alpha, const float* state_in, float* state_out, void* o, int64_t B,
                                   int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk, float eps,
                                   kla_dtype_t dt, void* stream) {
  return chunk_fwd_impl("kla_chunk_fwd_noalloc", false, false, q, k, v, eta, log_alpha, state_in, state_out, o, B, T,
                        H, d_k, d_v, chunk, eps, dt, nullptr, 0, stream, 0, true);
}

kla_status_t kla_chunk_fwd_seg(const void* q, const void* k, const void* v, const float* eta, const float* log_alpha,
                               const float* state_in, float* state_out, void* o, int64_t B, int64_t T, int64_t H,
                               int64_t d_k, int64_t d_v, int64_t chunk, int64_t segments, float eps, kla_dtype_t dt,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl("kla_chunk_fwd_seg", false, false, q, k, v, eta, log_alpha, state_in, state_out, o, B, T, H,
                        d_k, d_v, chunk, eps, dt, workspace, workspace_bytes, stream, segments);
}

kla_status_t kla_gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* beta,
                               const float* log_alpha, const float* state_in, float* state_out, void* o, int64_t B,
                               int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk, kla_dtype_t dt,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl("kla_gdn_chunk_fwd", true, false, q, k, v, beta, log_alpha, state_in, state_out, o, B, T, H, d_k,
                        d_v, chunk, 0.f, dt, workspace, workspace_bytes, stream);
}

kla_status_t kla_decode_step(const void* q, const void* k, const void* v, const float* eta, const float* log_alpha,
                             float* state, void* o, int64_t B, int64_t H, int64_t d_k, int64_t d_v, float eps,
                             kla_dtype_t dt, void* stream) {
  return decode_impl("kla_decode_step", false, false, q, k, v, eta, log_alpha, state, o, B, H, d_k, d_v, eps, dt, stream);
}

kla_status_t kla_gdn_decode_step(const void* q, const void* k, const void* v, const float* beta,
                                 const float* log_alpha, float* state, void* o, int64_t B, int64_t H, int64_t d_k,
                                 int64_t d_v, kla_dtype_t dt, void* stream) {
  return decode_impl("kla_gdn_decode_step", true, false, q, k, v, beta, log_alpha, state, o, B, H, d_k, d_v, 0.f, dt,
                     stream);
}

kla_status_t kla_chunk_bwd(const void* q, const void* k, const void* v, const float* eta, const float* log_alpha,
                           const float* state_in, const void* dout, const float* dstate_out, void* dq, void* dk,
                           void* dv, float* deta, float* dlog_alpha, float* dstate_in, int64_t B, int64_t T,
                           int64_t H, int64_t d_k, int64_t d_v, int64_t chunk, float eps, kla_dtype_t dt,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl("kla_chunk_bwd", false, false, q, k, v, eta, log_alpha, state_in, dout, dstate_out, dq, dk, dv,
                        deta, dlog_alpha, dstate_in, B, T, H, d_k, d_v, chunk, eps, dt, workspace, workspace_bytes,
                        stream);
}

kla_status_t kla_gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* beta,
                               const float* log_alpha, const float* state_in, const void* dout,
                               const float* dstate_out, void* dq, void* dk, void* dv, float* dbeta,
                               float* dlog_alpha, float* dstate_in, int64_t B, int64_t T, int64_t H, int64_t d_k,
                               int64_t d_v, int64_t chunk, kla_dtype_t dt, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return chunk_bwd_impl("kla_gdn_chunk_bwd", true, false, q, k, v, beta, log_alpha, state_in, dout, dstate_out, dq, dk, dv,
                        dbeta, dlog_alpha, dstate_in, B, T, H, d_k, d_v, chunk, 0.f, dt, workspace, workspace_bytes,
                        stream);
}

kla_status_t kla_chunk_fwd_train(const void* q, const void* k, const void* v, const float* eta,
                                 const float* log_alpha, const float* state_in, float* state_out, void* o, int64_t B,
                                 int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk, float eps,
                                 kla_dtype_t dt, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl("kla_chunk_fwd_train", false, false, q, k, v, eta, log_alpha, state_in, state_out, o, B, T, H,
                        d_k, d_v, chunk, eps, dt, workspace, workspace_bytes, stream, 0, false, true);
}

kla_status_t kla_gdn_chunk_fwd_train(const void* q, const void* k, const void* v, const float* beta,
                                     const float* log_alpha, const float* state_in, float* state_out, void* o,
                                     int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                     kla_dtype_t dt, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl("kla_gdn_chunk_fwd_train", true, false, q, k, v, beta, log_alpha, state_in, state_out, o, B,
                        T, H, d_k, d_v, chunk, 0.f, dt, workspace, workspace_bytes, stream, 0, false, true);
}

kla_status_t kla_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* eta, const float* log_alpha,
                                 const float* state_in, const void* dout, const float* dstate_out, void* dq, void* dk,
                                 void* dv, float* deta, float* dlog_alpha, float* dstate_in, int64_t B, int64_t T,
                                 int64_t H, int64_t d_k, int64_t d_v, int64_t chunk, float eps, kla_dtype_t dt,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl("kla_chunk_bwd_saved", false, false, q, k, v, eta, log_alpha, state_in, dout, dstate_out, dq,
                        dk, dv, deta, dlog_alpha, dstate_in, B, T, H, d_k, d_v, chunk, eps, dt, workspace,
                        workspace_bytes, stream, true);
}

kla_status_t kla_gdn_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* beta,
                                     const float* log_alpha, const float* state_in, const void* dout,
                                     const float* dstate_out, void* dq, void* dk, void* dv, float* dbeta,
                                     float* dlog_alpha, float* dstate_in, int64_t B, int64_t T, int64_t H, int64_t d_k,
                                     int64_t d_v, int64_t chunk, kla_dtype_t dt, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl("kla_gdn_chunk_bwd_saved", true, false, q, k, v, beta, log_alpha, state_in, dout, dstate_out,
                        dq, dk, dv, dbeta, dlog_alpha, dstate_in, B, T, H, d_k, d_v, chunk, 0.f, dt, workspace,
                        workspace_bytes, stream, true);
}

kla_status_t kla_kda_chunk_fwd(const void* q, const void* k, const void* v, const float* eta, const float* log_a,
                               const float* state_in, float* state_out, void* o, int64_t B, int64_t T, int64_t H,
                               int64_t d_k, int64_t d_v, int64_t chunk, float eps, int beta_given, kla_dtype_t dt,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl("kla_kda_chunk_fwd", beta_given != 0, true, q, k, v, eta, log_a, state_in, state_out, o, B,
                        T, H, d_k, d_v, chunk, beta_given ? 0.f : eps, dt, workspace, workspace_bytes, stream);
}

kla_status_t kla_kda_chunk_bwd(const void* q, const void* k, const void* v, const float* eta, const float* log_a,
                               const float* state_in, const void* dout, const float* dstate_out, void* dq, void* dk,
                               void* dv, float* deta, float* dlog_a, float* dstate_in, int64_t B, int64_t T, int64_t H,
                               int64_t d_k, int64_t d_v, int64_t chunk, float eps, int beta_given, kla_dtype_t dt,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl("kla_kda_chunk_bwd", beta_given != 0, true, q, k, v, eta, log_a, state_in, dout, dstate_out,
                        dq, dk, dv, deta, dlog_a, dstate_in, B, T, H, d_k, d_v, chunk, beta_given ? 0.f : eps, dt,
                        workspace, workspace_bytes, stream);
}

kla_status_t kla_kda_chunk_fwd_train(const void* q, const void* k, const void* v, const float* eta,
                                     const float* log_a, const float* state_in, float* state_out, void* o, int64_t B,
                                     int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk, float eps,
                                     int beta_given, kla_dtype_t dt, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return chunk_fwd_impl("kla_kda_chunk_fwd_train", beta_given != 0, true, q, k, v, eta, log_a, state_in, state_out, o,
                        B, T, H, d_k, d_v, chunk, beta_given ? 0.f : eps, dt, workspace, workspace_bytes, stream, 0,
                        false, true);
}

kla_status_t kla_kda_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* eta,
                                     const float* log_a, const float* state_in, const void* dout,
                                     const float* dstate_out, void* dq, void* dk, void* dv, float* deta, float* dlog_a,
                                     float* dstate_in, int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                     int64_t chunk, float eps, int beta_given, kla_dtype_t dt, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl("kla_kda_chunk_bwd_saved", beta_given != 0, true, q, k, v, eta, log_a, state_in, dout,
                        dstate_out, dq, dk, dv, deta, dlog_a, dstate_in, B, T, H, d_k, d_v, chunk,
                        beta_given ? 0.f : eps, dt, workspace, workspace_bytes, stream, true);
}

kla_status_t kla_kda_decode_step(const void* q, const void* k, const void* v, const float* eta, const float* log_a,
                                 float* state, void* o, int64_t B, int64_t H, int64_t d_k, int64_t d_v, float eps,
                                 int beta_given, kla_dtype_t dt, void* stream) {
  return decode_impl("kla_kda_decode_step", beta_given != 0, true, q, k, v, eta, log_a, state, o, B, H, d_k, d_v,
                     beta_given ? 0.f : eps, dt, stream);
}

}  // extern "C"
