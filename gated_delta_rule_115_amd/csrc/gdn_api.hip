// C ABI of the GDN library: host-side argument validation, then launch on the
// caller's stream.  Nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

gdn_status ok() {
  g_last_error.clear();
  return GDN_OK;
}

gdn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_head_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// dtype of the token inputs and of the output: (bf16, bf16), (bf16, f32) or
// (f32, f32).
gdn_status check_dtypes(int dtype, int out_dtype) {
  if (dtype != GDN_BF16 && dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_ARG, "dtype %d is neither GDN_BF16 nor GDN_F32", dtype);
  if (out_dtype != GDN_BF16 && out_dtype != GDN_F32)
    return fail(GDN_ERR_INVALID_ARG, "out_dtype %d is neither GDN_BF16 nor GDN_F32",
                out_dtype);
  if (dtype == GDN_F32 && out_dtype == GDN_BF16)
    return fail(GDN_ERR_UNSUPPORTED, "f32 inputs with a bf16 output are not supported");
  return GDN_OK;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t esize(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define REQUIRE_DTYPES(dt, odt)                 \
  do {                                          \
    const gdn_status st_ = check_dtypes((dt), (odt));  \
    if (st_ != GDN_OK) return st_;              \
  } while (0)

#define REQUIRE_PTR(p)                                                        \
  do {                                                                        \
    if ((p) == nullptr) return fail(GDN_ERR_INVALID_ARG, "%s is NULL", #p);   \
    if (!aligned16(p))                                                        \
      return fail(GDN_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p);      \
  } while (0)

#define REQUIRE_ALIGNED_OR_NULL(p)                                            \
  do {                                                                        \
    if ((p) != nullptr && !aligned16(p))                                      \
      return fail(GDN_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p);      \
  } while (0)

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_last_error(void) { return g_last_error.c_str(); }

size_t gdn_prefill_workspace_bytes(int B, int T, int H, int Dk, int Dv,
                                   int chunk, int dtype) {
  if (B < 0 || T < 0 || H < 1 || !is_head_dim(Dk) || !is_head_dim(Dv)) return 0;
  if (chunk != 16 && chunk != 32 && chunk != 64) return 0;
  if (dtype != GDN_BF16 && dtype != GDN_F32) return 0;
  return gdn::prefill_workspace_bytes(B, T, H, Dk, Dv, chunk, dtype == GDN_BF16);
}

}  // extern "C"

namespace {

// Host-side checks of a gdn_prefill_chunked call, common to the entry point
// with a caller workspace and the one with the static scratch.  On success
// returns GDN_OK, fills p (without workspace and stream) and sets *need to
// the scratch bytes the launch uses.
gdn_status check_prefill(const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const float* state_in, float* state_out, void* out,
                         int B, int T, int H, int Dk, int Dv, int chunk, int dtype, int out_dtype,
                         float scale, gdn::PrefillArgs* p, size_t* need) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && T >= 0 && H >= 1, GDN_ERR_INVALID_ARG,
          "bad sizes B=%d T=%d H=%d", B, T, H);
  REQUIRE(is_head_dim(Dk) && is_head_dim(Dv), GDN_ERR_UNSUPPORTED,
          "head dims Dk=%d Dv=%d not in {16,32,64,128}", Dk, Dv);
  REQUIRE(chunk == 16 || chunk == 32 || chunk == 64, GDN_ERR_UNSUPPORTED,
          "chunk %d not in {16,32,64}", chunk);
  const long long nc = ((long long)T + chunk - 1) / chunk;
  REQUIRE((long long)B * H * nc < (1LL << 31) && (long long)B * H * 8 < (1LL << 31),
          GDN_ERR_UNSUPPORTED, "grid too large");
  *need = 0;
  if ((long long)B * H > 0) {
    REQUIRE_ALIGNED_OR_NULL(state_in);
    REQUIRE_ALIGNED_OR_NULL(state_out);
    if (T > 0) {
      REQUIRE_PTR(q);
      REQUIRE_PTR(k);
      REQUIRE_PTR(v);
      REQUIRE_PTR(out);
      REQUIRE(alpha != nullptr && beta != nullptr, GDN_ERR_INVALID_ARG,
              "alpha/beta is NULL");
      *need = gdn::prefill_workspace_bytes(B, T, H, Dk, Dv, chunk, dtype == GDN_BF16);
    }
  }
  p->q = q; p->k = k; p->v = v; p->alpha = alpha; p->beta = beta;
  p->state_in = state_in; p->state_out = state_out; p->out = out;
  p->B = B; p->T = T; p->H = H; p->Dk = Dk; p->Dv = Dv; p->chunk = chunk;
  p->bf16 = dtype == GDN_BF16; p->out_bf16 = out_dtype == GDN_BF16;
  p->scale = scale; p->workspace = nullptr; p->stream = nullptr;
  return GDN_OK;
}

// Scratch of gdn_prefill_chunked_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in); it uses the device
// address hipGetSymbolAddress returns, looked up once per device with that
// device current and kept in scratch_addr.
constexpr size_t kNoAllocScratchBytes = (size_t)GDN_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr and an error
// message on failure).
void* scratch_on_current_device(gdn_status* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = hip_status(e, "gdn_prefill_chunked_noalloc: hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(GDN_ERR_UNSUPPORTED, "gdn_prefill_chunked_noalloc: device %d out of range", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *status = hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                           "gdn_prefill_chunked_noalloc: hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    scratch_addr[dev] = ptr;
  }
  *status = GDN_OK;
  return scratch_addr[dev];
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_chunked(const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta,
                               const float* state_in, float* state_out, void* out,
                               int B, int T, int H, int Dk, int Dv, int chunk,
                               int dtype, int out_dtype, float scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
  gdn::PrefillArgs p;
  size_t need = 0;
  const gdn_status st = check_prefill(q, k, v, alpha, beta, state_in, state_out, out, B, T, H, Dk,
                               Dv, chunk, dtype, out_dtype, scale, &p, &need);
  if (st != GDN_OK) return st;
  if ((long long)B * H == 0) return ok();
  if (need > 0) {
    REQUIRE(workspace != nullptr, GDN_ERR_INVALID_ARG, "workspace is NULL");
    REQUIRE(((uintptr_t)workspace & 255u) == 0, GDN_ERR_INVALID_ARG,
            "workspace is not 256-byte aligned");
    REQUIRE(workspace_bytes >= need, GDN_ERR_INVALID_ARG,
            "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  }
  p.workspace = workspace; p.stream = stream;
  return hip_status(gdn::launch_prefill(p), "gdn_prefill_chunked launch");
}

gdn_status gdn_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const float* state_in, float* state_out, void* out,
                                       int B, int T, int H, int Dk, int Dv, int chunk,
                                       int dtype, int out_dtype, float scale, void* stream) {
  gdn::PrefillArgs p;
  size_t need = 0;
  gdn_status st = check_prefill(q, k, v, alpha, beta, state_in, state_out, out, B, T, H, Dk, Dv,
                         chunk, dtype, out_dtype, scale, &p, &need);
  if (st != GDN_OK) return st;
  if ((long long)B * H == 0) return ok();
  REQUIRE(need <= kNoAllocScratchBytes, GDN_ERR_UNSUPPORTED,
          "gdn_prefill_chunked_noalloc: these sizes need %zu bytes of scratch, more than "
          "the %zu-byte static scratch; call gdn_prefill_chunked with a workspace",
          need, kNoAllocScratchBytes);
  void* ws = scratch_on_current_device(&st);
  if (st != GDN_OK) return st;
  p.workspace = need > 0 ? ws : nullptr; p.stream = stream;
  return hip_status(gdn::launch_prefill(p), "gdn_prefill_chunked_noalloc launch");
}

gdn_status gdn_prefill_chunked_conv(const void* xq, const void* xk, const void* xv,
                                    const float* taps_q, const float* taps_k, const float* taps_v,
                                    int conv_kernel, float conv_eps, const float* alpha,
                                    const float* beta, const float* state_in, float* state_out,
                                    void* out, int B, int T, int H, int Dk, int Dv, int chunk,
                                    int dtype, int out_dtype, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  gdn::PrefillArgs p;
  size_t need = 0;
  const gdn_status st = check_prefill(xq, xk, xv, alpha, beta, state_in, state_out, out, B, T, H, Dk,
                               Dv, chunk, dtype, out_dtype, scale, &p, &need);
  if (st != GDN_OK) return st;
  REQUIRE(conv_kernel == 4, GDN_ERR_UNSUPPORTED,
          "gdn_prefill_chunked_conv: conv_kernel %d (the fused convolution has 4 taps)",
          conv_kernel);
  REQUIRE(dtype == GDN_BF16 && Dk == 128 && Dv == 128 && chunk == 64, GDN_ERR_UNSUPPORTED,
          "gdn_prefill_chunked_conv: needs bf16 inputs, Dk = Dv = 128, chunk 64");
  REQUIRE(conv_eps >= 0.f && conv_eps <= 1e30f, GDN_ERR_INVALID_ARG,
          "gdn_prefill_chunked_conv: conv_eps %g not in [0, 1e30]", (double)conv_eps);
  if ((long long)B * H == 0) return ok();
  if (T > 0)
    REQUIRE(taps_q != nullptr && taps_k != nullptr && taps_v != nullptr, GDN_ERR_INVALID_ARG,
            "gdn_prefill_chunked_conv: taps_q/taps_k/taps_v is NULL");
  if (need > 0) {
    REQUIRE(workspace != nullptr, GDN_ERR_INVALID_ARG, "workspace is NULL");
    REQUIRE(((uintptr_t)workspace & 255u) == 0, GDN_ERR_INVALID_ARG,
            "workspace is not 256-byte aligned");
    REQUIRE(workspace_bytes >= need, GDN_ERR_INVALID_ARG,
            "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  }
  p.taps_q = taps_q; p.taps_k = taps_k; p.taps_v = taps_v; p.conv_eps = conv_eps;
  p.workspace = workspace; p.stream = stream;
  return hip_status(gdn::launch_prefill(p), "gdn_prefill_chunked_conv launch");
}

gdn_status gdn_decode_step(const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta,
                           const float* state_in, float* state_out, void* out, int B,
                           int H, int Dk, int Dv, int dtype, int out_dtype,
                           float scale, void* stream) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && H >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d H=%d", B, H);
  REQUIRE(is_head_dim(Dk) && is_head_dim(Dv), GDN_ERR_UNSUPPORTED,
          "head dims Dk=%d Dv=%d not in {16,32,64,128}", Dk, Dv);
  REQUIRE((long long)B * H < (1LL << 31), GDN_ERR_UNSUPPORTED, "grid too large");
  if (B == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  REQUIRE_PTR(state_in);
  REQUIRE_PTR(state_out);
  REQUIRE(alpha != nullptr && beta != nullptr, GDN_ERR_INVALID_ARG,
          "alpha/beta is NULL");
  gdn::DecodeArgs p;
  p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state_in = state_in; p.state_out = state_out; p.out = out;
  p.B = B; p.H = H; p.Dk = Dk; p.Dv = Dv;
  p.bf16 = dtype == GDN_BF16; p.out_bf16 = out_dtype == GDN_BF16;
  p.scale = scale; p.stream = stream;
  return hip_status(gdn::launch_decode(p), "gdn_decode_step launch");
}

gdn_status gdn_short_conv_silu(const void* x, const float* taps, void* y, int B,
                               int T, int Ch, int K, int l2norm_group, float eps,
                               int dtype, int out_dtype, void* stream) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && T >= 0 && Ch >= 1, GDN_ERR_INVALID_ARG,
          "bad sizes B=%d T=%d Ch=%d", B, T, Ch);
  REQUIRE(K >= 1 && K <= 8, GDN_ERR_UNSUPPORTED, "kernel size %d not in 1..8", K);
  REQUIRE(Ch % 8 == 0, GDN_ERR_UNSUPPORTED, "Ch=%d is not a multiple of 8", Ch);
  const int g = l2norm_group;
  REQUIRE(g == 0 || (g >= 8 && g <= 512 && (g & (g - 1)) == 0 && Ch % g == 0),
          GDN_ERR_UNSUPPORTED,
          "l2norm_group %d must be 0 or a power of two in 8..512 dividing Ch", g);
  REQUIRE(B <= 65535 && ((long long)T + 63) / 64 <= 65535, GDN_ERR_UNSUPPORTED,
          "grid too large (B <= 65535, T <= 4194240)");
  if ((long long)B * T == 0) return ok();
  REQUIRE_PTR(x);
  REQUIRE_PTR(y);
  REQUIRE(taps != nullptr, GDN_ERR_INVALID_ARG, "taps is NULL");
  const size_t xbytes = (size_t)B * T * Ch * esize(dtype);
  const size_t ybytes = (size_t)B * T * Ch * esize(out_dtype);
  const char* xa = (const char*)x;
  const char* ya = (const char*)y;
  REQUIRE(ya + ybytes <= xa || xa + xbytes <= ya, GDN_ERR_INVALID_ARG,
          "y overlaps x");
  gdn::ConvArgs p;
  p.x = x; p.taps = taps; p.y = y;
  p.B = B; p.T = T; p.Ch = Ch; p.K = K; p.group = g; p.eps = eps;
  p.bf16 = dtype == GDN_BF16; p.out_bf16 = out_dtype == GDN_BF16; p.stream = stream;
  return hip_status(gdn::launch_conv(p), "gdn_short_conv_silu launch");
}

gdn_status gdn_short_conv_step(const void* x, const float* taps, void* conv_state, void* y,
                               int B, int Ch, int K, int l2norm_group, float eps, int dtype,
                               int out_dtype, void* stream) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && Ch >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d Ch=%d", B, Ch);
  REQUIRE(K >= 1 && K <= 8, GDN_ERR_UNSUPPORTED, "kernel size %d not in 1..8", K);
  REQUIRE(Ch % 8 == 0, GDN_ERR_UNSUPPORTED, "Ch=%d is not a multiple of 8", Ch);
  const int g = l2norm_group;
  REQUIRE(g == 0 || (g >= 8 && g <= 512 && (g & (g - 1)) == 0 && Ch % g == 0),
          GDN_ERR_UNSUPPORTED,
          "l2norm_group %d must be 0 or a power of two in 8..512 dividing Ch", g);
  REQUIRE((long long)B * (Ch / 8) <= (long long)INT32_MAX, GDN_ERR_UNSUPPORTED, "grid too large");
  if (B == 0) return ok();
  REQUIRE_PTR(x);
  REQUIRE_PTR(y);
  REQUIRE(taps != nullptr, GDN_ERR_INVALID_ARG, "taps is NULL");
  if (K > 1) REQUIRE_PTR(conv_state);
  const size_t xbytes = (size_t)B * Ch * esize(dtype);
  const size_t ybytes = (size_t)B * Ch * esize(out_dtype);
  const size_t sbytes = (size_t)B * (K - 1) * Ch * esize(dtype);
  const char* xa = (const char*)x;
  const char* ya = (const char*)y;
  const char* sa = (const char*)conv_state;
  REQUIRE(ya + ybytes <= xa || xa + xbytes <= ya, GDN_ERR_INVALID_ARG, "y overlaps x");
  REQUIRE(K == 1 || ya + ybytes <= sa || sa + sbytes <= ya, GDN_ERR_INVALID_ARG,
          "y overlaps conv_state");
  REQUIRE(K == 1 || xa + xbytes <= sa || sa + sbytes <= xa, GDN_ERR_INVALID_ARG,
          "x overlaps conv_state");
  gdn::ConvArgs p;
  p.x = x; p.taps = taps; p.y = y;
  p.B = B; p.T = 1; p.Ch = Ch; p.K = K; p.group = g; p.eps = eps;
  p.bf16 = dtype == GDN_BF16; p.out_bf16 = out_dtype == GDN_BF16; p.stream = stream;
  return hip_status(gdn::launch_conv_step(p, conv_state), "gdn_short_conv_step launch");
}

gdn_status gdn_swa_sink_decode(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, const int* n_tokens,
                               int B, int H, int D, int n_sink, int window,
                               float softmax_scale, int accumulate, void* out,
                               int dtype, int out_dtype, void* stream) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && H >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d H=%d", B, H);
  REQUIRE(D == 64 || D == 128, GDN_ERR_UNSUPPORTED, "head dim %d not in {64,128}", D);
  REQUIRE(n_sink >= 0 && window >= 1, GDN_ERR_INVALID_ARG,
          "bad cache shape n_sink=%d window=%d", n_sink, window);
  REQUIRE((long long)n_sink + window < (1LL << 24), GDN_ERR_UNSUPPORTED,
          "cache too long");
  REQUIRE(accumulate == 0 || accumulate == 1, GDN_ERR_INVALID_ARG,
          "accumulate must be 0 or 1");
  REQUIRE((k_new == nullptr) == (v_new == nullptr), GDN_ERR_INVALID_ARG,
          "k_new and v_new must both be given or both be NULL");
  REQUIRE((long long)B * H < (1LL << 31), GDN_ERR_UNSUPPORTED, "grid too large");
  if (B == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(out);
  REQUIRE_ALIGNED_OR_NULL(k_new);
  REQUIRE_ALIGNED_OR_NULL(v_new);
  REQUIRE(n_tokens != nullptr, GDN_ERR_INVALID_ARG, "n_tokens is NULL");
  gdn::SwaArgs p;
  p.q = q; p.k_new = k_new; p.v_new = v_new; p.k_cache = k_cache; p.v_cache = v_cache;
  p.n_tokens = n_tokens; p.B = B; p.H = H; p.D = D; p.n_sink = n_sink;
  p.window = window; p.softmax_scale = softmax_scale; p.accumulate = accumulate;
  p.out = out; p.bf16 = dtype == GDN_BF16; p.out_bf16 = out_dtype == GDN_BF16;
  p.stream = stream;
  return hip_status(gdn::launch_swa(p), "gdn_swa_sink_decode launch");
}

gdn_status gdn_swa_sink_prefill(const void* q, const void* k, const void* v, void* out, int B,
                                int T, int H, int D, int n_sink, int window, float softmax_scale,
                                int accumulate_from, int dtype, int out_dtype, void* stream) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && T >= 0 && H >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d T=%d H=%d", B, T,
          H);
  REQUIRE(n_sink >= 0 && window >= 1, GDN_ERR_INVALID_ARG, "bad n_sink=%d window=%d", n_sink,
          window);
  REQUIRE(dtype == GDN_BF16 && D == 128, GDN_ERR_UNSUPPORTED,
          "the sequence softmax path takes bf16 inputs with D = 128 (got dtype %d, D %d)",
          dtype, D);
  REQUIRE(softmax_scale > 0.f && softmax_scale < INFINITY, GDN_ERR_INVALID_ARG,
          "softmax_scale must be positive and finite");
  REQUIRE((long long)B * H * ((T + 127) / 128) < (1LL << 31) && (long long)T * H * D < (1LL << 31),
          GDN_ERR_UNSUPPORTED, "grid too large");
  if ((long long)B * T == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  gdn::SwaPrefillArgs p;
  p.q = q; p.k = k; p.v = v; p.out = out;
  p.B = B; p.T = T; p.H = H; p.n_sink = n_sink; p.window = window;
  p.acc_from = accumulate_from; p.softmax_scale = softmax_scale;
  p.out_bf16 = out_dtype == GDN_BF16; p.stream = stream;
  return hip_status(gdn::launch_swa_prefill(p), "gdn_swa_sink_prefill launch");
}

gdn_status gdn_swa_cache_fill(const void* k, const void* v, void* k_cache, void* v_cache, int B,
                              int T, int H, int D, int n_sink, int window, int dtype, void* stream) {
  REQUIRE(dtype == GDN_BF16 || dtype == GDN_F32, GDN_ERR_INVALID_ARG, "bad dtype %d", dtype);
  REQUIRE(B >= 0 && T >= 0 && H >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d T=%d H=%d", B, T,
          H);
  REQUIRE(D == 64 || D == 128, GDN_ERR_UNSUPPORTED, "head dim %d not in {64,128}", D);
  REQUIRE(n_sink >= 0 && window >= 1, GDN_ERR_INVALID_ARG, "bad n_sink=%d window=%d", n_sink,
          window);
  REQUIRE((long long)B * H < (1LL << 31), GDN_ERR_UNSUPPORTED, "grid too large");
  if ((long long)B * T == 0) return ok();
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  gdn::SwaCacheFillArgs p;
  p.k = k; p.v = v; p.k_cache = k_cache; p.v_cache = v_cache;
  p.B = B; p.T = T; p.H = H; p.D = D; p.n_sink = n_sink; p.window = window;
  p.bf16 = dtype == GDN_BF16; p.stream = stream;
  return hip_status(gdn::launch_swa_cache_fill(p), "gdn_swa_cache_fill launch");
}

size_t gdn_hybrid_prefill_workspace_bytes(int B, int T, int H, int D, int n_sink, int window) {
  if (B < 0 || T < 0 || H < 1 || D != 128 || n_sink < 0 || window < 1) return 0;
  const long long t_lin = (long long)T - window - n_sink;
  if (t_lin <= 0) return 0;
  return gdn::prefill_workspace_bytes(B, (int)t_lin, H, D, D, 64, true);
}

gdn_status gdn_hybrid_prefill(const void* q_lin, const void* k_lin, const void* v_lin,
                              const float* alpha, const float* beta, const void* q_swa,
                              const void* k_swa, const void* v_swa, float* state_out, void* out,
                              void* k_cache, void* v_cache, int B, int T, int H, int D, int n_sink,
                              int window, float lin_scale, float softmax_scale, int dtype,
                              int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && T >= 0 && H >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d T=%d H=%d", B, T,
          H);
  REQUIRE(n_sink >= 0 && window >= 1, GDN_ERR_INVALID_ARG, "bad n_sink=%d window=%d", n_sink,
          window);
  REQUIRE(dtype == GDN_BF16 && D == 128, GDN_ERR_UNSUPPORTED,
          "the hybrid prefill takes bf16 inputs with D = 128 (got dtype %d, D %d)", dtype, D);
  REQUIRE(softmax_scale > 0.f && softmax_scale < INFINITY, GDN_ERR_INVALID_ARG,
          "softmax_scale must be positive and finite");
  REQUIRE((long long)B * H * ((T + 127) / 128) < (1LL << 31) && (long long)T * H * D < (1LL << 31),
          GDN_ERR_UNSUPPORTED, "grid too large");
  REQUIRE((k_cache == nullptr) == (v_cache == nullptr), GDN_ERR_INVALID_ARG,
          "k_cache and v_cache must both be given or both be NULL");
  REQUIRE_ALIGNED_OR_NULL(state_out);
  REQUIRE_ALIGNED_OR_NULL(k_cache);
  REQUIRE_ALIGNED_OR_NULL(v_cache);
  if (B == 0) return ok();
  const long long t_lin = (long long)T - window - n_sink;
  if (T > 0) {
    REQUIRE_PTR(q_swa);
    REQUIRE_PTR(k_swa);
    REQUIRE_PTR(v_swa);
    REQUIRE_PTR(out);
  }
  if (t_lin > 0) {
    REQUIRE_PTR(q_lin);
    REQUIRE_PTR(k_lin);
    REQUIRE_PTR(v_lin);
    REQUIRE(alpha != nullptr && beta != nullptr, GDN_ERR_INVALID_ARG, "alpha/beta is NULL");
    const size_t need = gdn::prefill_workspace_bytes(B, (int)t_lin, H, D, D, 64, true);
    if (need > 0) {
      REQUIRE(workspace != nullptr, GDN_ERR_INVALID_ARG, "workspace is NULL");
      REQUIRE(((uintptr_t)workspace & 255u) == 0, GDN_ERR_INVALID_ARG,
              "workspace is not 256-byte aligned");
      REQUIRE(workspace_bytes >= need, GDN_ERR_INVALID_ARG,
              "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    }
  }
  // Linear path: the state at position t holds tokens n_sink .. t - window,
  // so with q shifted by `window` it is the chunked prefill over those
  // tokens, whose output row j is the layer's row j + window.  One launch
  // over all sequences: their rows are views with a stride of T tokens.
  const size_t row = (size_t)H * D;
  const size_t os = esize(out_dtype);
  const long long n = t_lin > 0 ? t_lin : 0;
  if (n > 0 || state_out != nullptr) {
    gdn::PrefillArgs p;
    p.q = n ? (const char*)q_lin + (size_t)(n_sink + window) * row * 2 : nullptr;
    p.k = n ? (const char*)k_lin + (size_t)n_sink * row * 2 : nullptr;
    p.v = n ? (const char*)v_lin + (size_t)n_sink * row * 2 : nullptr;
    p.alpha = n ? alpha + (size_t)n_sink * H : nullptr;
    p.beta = n ? beta + (size_t)n_sink * H : nullptr;
    p.state_in = nullptr;
    p.state_out = state_out;
    p.out = n ? (char*)out + (size_t)(n_sink + window) * row * os : nullptr;
    p.B = B; p.T = (int)n; p.H = H; p.Dk = D; p.Dv = D; p.chunk = 64;
    p.bf16 = true; p.out_bf16 = out_dtype == GDN_BF16; p.scale = lin_scale;
    p.workspace = workspace; p.stream = stream; p.seq_stride = T;
    const gdn_status st = hip_status(gdn::launch_prefill(p), "gdn_hybrid_prefill linear path");
    if (st != GDN_OK) return st;
  }
  if (T > 0) {
    gdn::SwaPrefillArgs p;
    p.q = q_swa; p.k = k_swa; p.v = v_swa; p.out = out;
    p.B = B; p.T = T; p.H = H; p.n_sink = n_sink; p.window = window;
    p.acc_from = t_lin > 0 ? n_sink + window : T;
    p.softmax_scale = softmax_scale; p.out_bf16 = out_dtype == GDN_BF16; p.stream = stream;
    const gdn_status st = hip_status(gdn::launch_swa_prefill(p), "gdn_hybrid_prefill softmax path");
    if (st != GDN_OK) return st;
  }
  if (k_cache != nullptr && T > 0) {
    gdn::SwaCacheFillArgs p;
    p.k = k_swa; p.v = v_swa; p.k_cache = k_cache; p.v_cache = v_cache;
    p.B = B; p.T = T; p.H = H; p.D = D; p.n_sink = n_sink; p.window = window;
    p.bf16 = true; p.stream = stream;
    return hip_status(gdn::launch_swa_cache_fill(p), "gdn_hybrid_prefill cache fill");
  }
  return ok();
}

size_t gdn_prefill_chgate_workspace_bytes(int B, int T, int H) {
  if (B < 0 || T < 0 || H < 1) return 0;
  return gdn::prefill_chgate_workspace_bytes(B, T, H);
}

}  // extern "C"

namespace {

// The channel-gate prefill and decode step, and kGLA on the same kernels.
gdn_status prefill_chgate_call(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, const float* state_in, float* state_out, void* out,
                               int B, int T, int H, int Dk, int Dv, int dtype, int out_dtype,
                               float scale, void* workspace, size_t workspace_bytes, void* stream,
                               bool kgla, const char* name) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && T >= 0 && H >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d T=%d H=%d", B, T,
          H);
  REQUIRE((Dk == 32 || Dk == 64 || Dk == 128) && (Dv == 32 || Dv == 64 || Dv == 128),
          GDN_ERR_UNSUPPORTED, "%s: head dims Dk=%d Dv=%d not in {32,64,128}", name, Dk, Dv);
  REQUIRE((long long)B * H * ((T + 31) / 32) < (1LL << 31), GDN_ERR_UNSUPPORTED,
          "grid too large");
  if ((long long)B * H == 0) return ok();
  REQUIRE_ALIGNED_OR_NULL(state_in);
  REQUIRE_ALIGNED_OR_NULL(state_out);
  if (T > 0) {
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    REQUIRE(alpha != nullptr && beta != nullptr, GDN_ERR_INVALID_ARG, "alpha/beta is NULL");
    REQUIRE_PTR(alpha);  // read in 16-byte pieces
    const size_t need = gdn::prefill_chgate_workspace_bytes(B, T, H);
    REQUIRE(workspace != nullptr, GDN_ERR_INVALID_ARG, "workspace is NULL");
    REQUIRE(((uintptr_t)workspace & 255u) == 0, GDN_ERR_INVALID_ARG,
            "workspace is not 256-byte aligned");
    REQUIRE(workspace_bytes >= need, GDN_ERR_INVALID_ARG,
            "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  }
  gdn::PrefillArgs p;
  p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state_in = state_in; p.state_out = state_out; p.out = out;
  p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.chunk = 32;
  p.bf16 = dtype == GDN_BF16; p.out_bf16 = out_dtype == GDN_BF16;
  p.scale = scale; p.workspace = workspace; p.stream = stream; p.kgla = kgla;
  return hip_status(gdn::launch_prefill_chgate(p), name);
}

gdn_status decode_chgate_call(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const float* state_in, float* state_out, void* out,
                              int B, int H, int Dk, int Dv, int dtype, int out_dtype, float scale,
                              void* stream, bool kgla, const char* name) {
  REQUIRE_DTYPES(dtype, out_dtype);
  REQUIRE(B >= 0 && H >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d H=%d", B, H);
  REQUIRE(is_head_dim(Dk) && is_head_dim(Dv), GDN_ERR_UNSUPPORTED,
          "head dims Dk=%d Dv=%d not in {16,32,64,128}", Dk, Dv);
  REQUIRE((long long)B * H < (1LL << 31), GDN_ERR_UNSUPPORTED, "grid too large");
  if (B == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  REQUIRE_PTR(state_in);
  REQUIRE_PTR(state_out);
  REQUIRE(alpha != nullptr && beta != nullptr, GDN_ERR_INVALID_ARG, "alpha/beta is NULL");
  gdn::DecodeArgs p;
  p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
  p.state_in = state_in; p.state_out = state_out; p.out = out;
  p.B = B; p.H = H; p.Dk = Dk; p.Dv = Dv;
  p.bf16 = dtype == GDN_BF16; p.out_bf16 = out_dtype == GDN_BF16;
  p.scale = scale; p.stream = stream; p.chgate = true; p.kgla = kgla;
  return hip_status(gdn::launch_decode(p), name);
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_chunked_chgate(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta, const float* state_in,
                                      float* state_out, void* out, int B, int T, int H, int Dk, int Dv,
                                      int dtype, int out_dtype, float scale, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return prefill_chgate_call(q, k, v, alpha, beta, state_in, state_out, out, B, T, H, Dk, Dv,
                             dtype, out_dtype, scale, workspace, workspace_bytes, stream, false,
                             "gdn_prefill_chunked_chgate launch");
}

gdn_status gdn_decode_step_chgate(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* state_in, float* state_out,
                                  void* out, int B, int H, int Dk, int Dv, int dtype, int out_dtype,
                                  float scale, void* stream) {
  return decode_chgate_call(q, k, v, alpha, beta, state_in, state_out, out, B, H, Dk, Dv, dtype,
                            out_dtype, scale, stream, false, "gdn_decode_step_chgate launch");
}

gdn_status gdn_prefill_chunked_kgla(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta, const float* state_in,
                                    float* state_out, void* out, int B, int T, int H, int Dk, int Dv,
                                    int dtype, int out_dtype, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return prefill_chgate_call(q, k, v, alpha, beta, state_in, state_out, out, B, T, H, Dk, Dv,
                             dtype, out_dtype, scale, workspace, workspace_bytes, stream, true,
                             "gdn_prefill_chunked_kgla launch");
}

gdn_status gdn_decode_step_kgla(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* state_in, float* state_out, void* out,
                                int B, int H, int Dk, int Dv, int dtype, int out_dtype, float scale,
                                void* stream) {
  return decode_chgate_call(q, k, v, alpha, beta, state_in, state_out, out, B, H, Dk, Dv, dtype,
                            out_dtype, scale, stream, true, "gdn_decode_step_kgla launch");
}

size_t gdn_prefill_backward_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
  if (B < 0 || T < 0 || H < 1 || !is_head_dim(Dk) || !is_head_dim(Dv)) return 0;
  return gdn::backward_workspace_bytes(B, T, H, Dk, Dv);
}

gdn_status gdn_prefill_backward(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* state_in, const float* dout,
                                const float* dstate_out, float* dq, float* dk, float* dv,
                                float* dalpha, float* dbeta, float* dstate_in, int B, int T, int H,
                                int Dk, int Dv, int dtype, float scale, void* workspace,
                                size_t workspace_bytes, void* stream) {
  REQUIRE(dtype == GDN_BF16 || dtype == GDN_F32, GDN_ERR_INVALID_ARG, "bad dtype %d", dtype);
  REQUIRE(B >= 0 && T >= 0 && H >= 1, GDN_ERR_INVALID_ARG, "bad sizes B=%d T=%d H=%d", B, T,
          H);
  REQUIRE(is_head_dim(Dk) && is_head_dim(Dv), GDN_ERR_UNSUPPORTED,
          "head dims Dk=%d Dv=%d not in {16,32,64,128}", Dk, Dv);
  REQUIRE((long long)B * H < (1LL << 31), GDN_ERR_UNSUPPORTED, "grid too large");
  if ((long long)B * H == 0) return ok();
  REQUIRE_ALIGNED_OR_NULL(state_in);
  REQUIRE_ALIGNED_OR_NULL(dstate_out);
  REQUIRE(dstate_in != nullptr, GDN_ERR_INVALID_ARG, "dstate_in is NULL");
  if (T > 0) {
    REQUIRE(q && k && v && alpha && beta && dout, GDN_ERR_INVALID_ARG,
            "q, k, v, alpha, beta and dout are required");
    REQUIRE(dq && dk && dv && dalpha && dbeta, GDN_ERR_INVALID_ARG,
            "dq, dk, dv, dalpha and dbeta are required");
  }
  const size_t need = gdn::backward_workspace_bytes(B, T, H, Dk, Dv);
  REQUIRE(workspace != nullptr, GDN_ERR_INVALID_ARG, "workspace is NULL");
  REQUIRE(((uintptr_t)workspace & 255u) == 0, GDN_ERR_INVALID_ARG,
          "workspace is not 256-byte aligned");
  REQUIRE(workspace_bytes >= need, GDN_ERR_INVALID_ARG, "workspace too small: %zu < %zu bytes",
          workspace_bytes, need);
  gdn::BwdArgs p;
  p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta; p.state_in = state_in;
  p.dout = dout; p.dstate_out = dstate_out; p.dq = dq; p.dk = dk; p.dv = dv;
  p.dalpha = dalpha; p.dbeta = dbeta; p.dstate_in = dstate_in;
  p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.bf16 = dtype == GDN_BF16;
  p.scale = scale; p.workspace = workspace; p.stream = stream;
  return hip_status(gdn::launch_backward(p), "gdn_prefill_backward launch");
}

}  // extern "C"
