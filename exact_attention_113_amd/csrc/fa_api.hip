// C ABI of libfa.so: argument validation, status reporting and dispatch to
// the kernel launchers. Validation runs before any HIP call, so a rejected
// call touches no device and writes nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "fa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

__attribute__((format(printf, 2, 3))) fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) != 0; }

int64_t dtype_size(int dtype) {
  switch (dtype) {
    case FA_FP32: return 4;
    case FA_FP16: return 2;
    case FA_BF16: return 2;
    default: return 0;
  }
}

// Shape checks common to forward and backward. Returns FA_OK or the status
// to report (with the error text set).
fa_status check_shape(int64_t B, int64_t H, int64_t N, int64_t D, float scale, int dtype) {
  if (B < 1) return fail(FA_ERR_INVALID_ARGUMENT, "B must be >= 1 (got %lld)", (long long)B);
  if (H < 1) return fail(FA_ERR_INVALID_ARGUMENT, "H must be >= 1 (got %lld)", (long long)H);
  if (N < 1) return fail(FA_ERR_INVALID_ARGUMENT, "N must be >= 1 (got %lld)", (long long)N);
  if (D < 1) return fail(FA_ERR_INVALID_ARGUMENT, "D must be >= 1 (got %lld)", (long long)D);
  if (dtype_size(dtype) == 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "unknown dtype code %d", dtype);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite");
  int64_t elems = 0, bytes = 0, rows = 0;
  if (__builtin_mul_overflow(B, H, &rows) || __builtin_mul_overflow(rows, N, &rows) ||
      __builtin_mul_overflow(rows, D, &elems) ||
      __builtin_mul_overflow(elems, (int64_t)4, &bytes))
    return fail(FA_ERR_INVALID_ARGUMENT, "B*H*N*D overflows 64-bit byte offsets");
  if (D != 64 && D != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)D);
  // Kernels index positions with 32-bit integers and launch one workgroup
  // per 128 query rows of each (batch, head).
  if (N > (int64_t)1 << 30)
    return fail(FA_ERR_UNSUPPORTED, "sequence length %lld above 2^30", (long long)N);
  const int64_t wgs = ((N + 127) / 128) * B * H;
  if (wgs > (int64_t)0x7fffffff)
    return fail(FA_ERR_UNSUPPORTED, "%lld workgroups exceed one grid", (long long)wgs);
  return FA_OK;
}

fa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FA_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: HIP error %d (%s)", what, (int)e,
           hipGetErrorString(e));
  return FA_ERR_HIP;
}

}  // namespace

namespace fa {

bool backward_workspace_layout(int64_t B, int64_t H, int64_t N, int64_t D, BwdWorkspace* ws) {
  if (B < 1 || H < 1 || N < 1 || D < 1) return false;
  int64_t rows = 0, dl = 0;
  if (__builtin_mul_overflow(B, H, &rows) || __builtin_mul_overflow(rows, N, &rows) ||
      __builtin_mul_overflow(rows, (int64_t)4, &dl))
    return false;
  const int64_t round = 255;
  if (dl > (INT64_MAX - 2 * round) / 2) return false;
  const int64_t padded = (dl + round) & ~round;
  ws->delta_off = 0;
  ws->delta_bytes = (size_t)dl;
  ws->lse2_off = (size_t)padded;
  ws->lse2_bytes = (size_t)dl;
  ws->total = (size_t)(2 * padded);
  return true;
}

}  // namespace fa

namespace {

// H_kv K/V heads shared by groups of H / H_kv query heads.
fa_status check_group(int64_t H, int64_t H_kv, const char* who) {
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: H_kv (%lld) must divide H (%lld)", who,
                (long long)H_kv, (long long)H);
  return FA_OK;
}

fa_status forward_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D, float scale,
                       int causal, int dtype, void* stream, const fa::DropParams& drop,
                       const char* who) {
  if (!q || !k || !v || !o || !lse)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: q, k, v, o and lse must be non-NULL", who);
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: q, k, v, o must be 16-byte aligned", who);
  if (misaligned(lse, 4)) return fail(FA_ERR_INVALID_ARGUMENT, "%s: lse must be 4-byte aligned", who);
  fa_status s = check_shape(B, H, N, D, scale, dtype);
  if (s != FA_OK) return s;
  s = check_group(H, H_kv, who);
  if (s != FA_OK) return s;
  fa::FwdArgs a{q,     k,      v,     o,     lse, B, H, N, D, scale, causal, dtype, (hipStream_t)stream,
                H_kv,  nullptr, 0,    drop};
  return hip_status(fa::launch_forward(a), who);
}

// Checks of a dense backward call except its workspace; on success ws holds
// the workspace layout the call needs.
fa_status check_backward(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D, float scale,
                         int dtype, const char* who, fa::BwdWorkspace* ws) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "%s: q, k, v, o, dout, lse, dq, dk, dv must be non-NULL", who);
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
      misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: tensors must be 16-byte aligned", who);
  if (misaligned(lse, 4)) return fail(FA_ERR_INVALID_ARGUMENT, "%s: lse must be 4-byte aligned", who);
  fa_status s = check_shape(B, H, N, D, scale, dtype);
  if (s != FA_OK) return s;
  s = check_group(H, H_kv, who);
  if (s != FA_OK) return s;
  if (dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "%s: fp32 backward is not supported", who);
  if (!fa::backward_workspace_layout(B, H, N, D, ws))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: workspace size overflows", who);
  return FA_OK;
}

fa_status backward_impl(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                        int64_t H_kv, int64_t N, int64_t D, float scale, int causal, int dtype,
                        void* stream, const fa::DropParams& drop, const char* who) {
  fa::BwdWorkspace ws;
  fa_status s = check_backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, D, scale, dtype,
                               who, &ws);
  if (s != FA_OK) return s;
  if (!workspace)
    return fail(FA_ERR_WORKSPACE, "%s: workspace is NULL (needs %lld bytes)", who,
                (long long)ws.total);
  if (workspace_bytes < ws.total)
    return fail(FA_ERR_WORKSPACE, "%s: workspace too small (needs %lld bytes)", who,
                (long long)ws.total);
  if (misaligned(workspace, 256))
    return fail(FA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, D, scale, causal, dtype,
                (hipStream_t)stream, drop, H_kv};
  return hip_status(fa::launch_backward(a, ws), who);
}

// Dropout constants from the caller's probability, seed and offset: the
// byte threshold floor(256 p + 0.5) (so p is rounded to a multiple of 1/256)
// and the scale of the kept probabilities 1 / (1 - thr / 256).
fa_status drop_params(float p, uint64_t seed, uint64_t offset, int dtype, const char* who,
                      fa::DropParams* out) {
  if (!(p >= 0.f && p < 1.f))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: dropout_p must be in [0, 1)", who);
  const uint32_t thr = (uint32_t)floor((double)p * 256.0 + 0.5);
  if (thr > 255)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: dropout_p rounds to 1 (must be below 255.5/256)",
                who);
  if (offset > 0xffffffffull)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: offset must be below 2^32", who);
  if (dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "%s: fp32 is not supported", who);
  out->thr = thr;
  out->k0 = (uint32_t)(seed & 0xffffffffu);
  out->k1 = (uint32_t)(seed >> 32);
  out->offset = (uint32_t)offset;
  out->inv_keep = (float)(1.0 / (1.0 - thr / 256.0));
  out->thr4 = thr * 0x01010101u;
  out->bias4 = 0x80808080u - (out->thr4 & 0x7f7f7f7fu);
  return FA_OK;
}

// Checks common to the packed variable-length entry points.
fa_status check_varlen(int64_t batch, int64_t max_seqlen, int64_t total, int64_t H, int64_t H_kv,
                       int64_t D, float scale, int dtype, const char* who) {
  if (batch < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: batch must be >= 1 (got %lld)", who,
                (long long)batch);
  if (H_kv < 1 || H < 1 || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: H (%lld) must be a positive multiple of H_kv (%lld)",
                who, (long long)H, (long long)H_kv);
  if (total < 1 || max_seqlen < 1 || max_seqlen > total)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: need 1 <= max_seqlen (%lld) <= total (%lld)", who,
                (long long)max_seqlen, (long long)total);
  fa_status s = check_shape(1, H, total, D, scale, dtype);
  if (s != FA_OK) return s;
  if (dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "%s: fp32 is not supported", who);
  // Query tiles of 128 (forward) or key tiles of 128 (backward) per
  // (sequence, head).
  const int64_t wgs = ((max_seqlen + 127) / 128) * batch * H;
  if (batch > (int64_t)1 << 30 || wgs > (int64_t)0x7fffffff)
    return fail(FA_ERR_UNSUPPORTED, "%s: %lld workgroups exceed one grid", who, (long long)wgs);
  return FA_OK;
}

// ---- scratch of the allocation-free backward ----------------------------
// The backward's two fp32 row statistics (delta and LSE * log2 e), laid out
// as in a caller's workspace, for calls whose workspace would exceed no more
// than kScratchBytes (B * H * N up to 2^21 rows). Each GPU the library runs
// on holds its own copy until the process ends. In host code `scratch` only
// names the symbol: its device address, different on every GPU, comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` runs on (which must be
// the current device).
fa_status scratch_address(void* stream, void** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, who);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return hip_status(e, who);
    if ((int)sdev != dev)
      return fail(FA_ERR_INVALID_ARGUMENT, "%s: the stream runs on device %d, device %d is current",
                  who, (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_ERR_UNSUPPORTED, "%s: device index %d above %d", who, dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, who);
    if (!p || misaligned(p, 256))
      return fail(FA_ERR_HIP, "%s: scratch address %p unusable", who, p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

// The packed-batch forward and backward (with dropout when drop.thr != 0).
fa_status forward_varlen_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int32_t* cu_seqlens, int64_t batch, int64_t max_seqlen,
                              int64_t total, int64_t H, int64_t H_kv, int64_t D, float scale,
                              int causal, int dtype, void* stream, const fa::DropParams& drop,
                              const char* who) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: q, k, v, o, lse and cu_seqlens must be non-NULL",
                who);
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: q, k, v, o must be 16-byte aligned", who);
  if (misaligned(lse, 4) || misaligned(cu_seqlens, 4))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: lse and cu_seqlens must be 4-byte aligned", who);
  fa_status s = check_varlen(batch, max_seqlen, total, H, H_kv, D, scale, dtype, who);
  if (s != FA_OK) return s;
  fa::FwdArgs a{q,     k,      v,     o,      lse,        batch, H,     max_seqlen, D,
                scale, causal, dtype, (hipStream_t)stream, H_kv, cu_seqlens, total, drop};
  return hip_status(fa::launch_forward(a), who);
}

fa_status backward_varlen_impl(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               const int32_t* cu_seqlens, void* workspace,
                               size_t workspace_bytes, int64_t batch, int64_t max_seqlen,
                               int64_t total, int64_t H, int64_t H_kv, int64_t D, float scale,
                               int causal, int dtype, void* stream, const fa::DropParams& drop,
                               const char* who) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "%s: q, k, v, o, dout, lse, dq, dk, dv and cu_seqlens must be non-NULL", who);
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
      misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: tensors must be 16-byte aligned", who);
  if (misaligned(lse, 4) || misaligned(cu_seqlens, 4))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: lse and cu_seqlens must be 4-byte aligned", who);
  fa_status s = check_varlen(batch, max_seqlen, total, H, H_kv, D, scale, dtype, who);
  if (s != FA_OK) return s;
  if (total > (int64_t)0x7fffffff)
    return fail(FA_ERR_UNSUPPORTED, "%s: total (%lld) above 2^31 - 1", who, (long long)total);
  fa::BwdWorkspace ws;
  if (!fa::backward_workspace_layout(1, H, total, D, &ws))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: workspace size overflows", who);
  if (!workspace)
    return fail(FA_ERR_WORKSPACE, "%s: workspace is NULL (needs %lld bytes)", who,
                (long long)ws.total);
  if (workspace_bytes < ws.total)
    return fail(FA_ERR_WORKSPACE, "%s: workspace too small (needs %lld bytes)", who,
                (long long)ws.total);
  if (misaligned(workspace, 256))
    return fail(FA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
  fa::BwdArgs a{q,     k,      v,     o,      dout,  lse,       dq,        dk,
                dv,    workspace, batch, H,     max_seqlen, D,  scale,     causal,
                dtype, (hipStream_t)stream, drop, H_kv, cu_seqlens, total};
  return hip_status(fa::launch_backward(a, ws), who);
}

extern "C" {


fa_status fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t H, int64_t N, int64_t D, float scale, int causal, int dtype,
                     void* stream) {
  g_last_error[0] = '\0';
  return forward_impl(q, k, v, o, lse, B, H, H, N, D, scale, causal, dtype, stream,
                      fa::DropParams{}, "fa_forward");
}

fa_status fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                             int dtype, float dropout_p, uint64_t seed, uint64_t offset,
                             void* stream) {
  g_last_error[0] = '\0';
  fa::DropParams dp;
  fa_status s = drop_params(dropout_p, seed, offset, dtype, "fa_forward_dropout", &dp);
  if (s != FA_OK) return s;
  return forward_impl(q, k, v, o, lse, B, H, H, N, D, scale, causal, dtype, stream, dp,
                      "fa_forward_dropout");
}

fa_status fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D, float scale,
                         int causal, int dtype, float dropout_p, uint64_t seed, uint64_t offset,
                         void* stream) {
  g_last_error[0] = '\0';
  const char* who = "fa_forward_gqa";
  fa::DropParams dp{};
  if (dropout_p != 0.f) {
    fa_status s = drop_params(dropout_p, seed, offset, dtype, who, &dp);
    if (s != FA_OK) return s;
  }
  return forward_impl(q, k, v, o, lse, B, H, H_kv, N, D, scale, causal, dtype, stream, dp, who);
}

fa_status fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens, int64_t batch, int64_t max_seqlen,
                            int64_t total, int64_t H, int64_t H_kv, int64_t D, float scale,
                            int causal, int dtype, void* stream) {
  g_last_error[0] = '\0';
  return forward_varlen_impl(q, k, v, o, lse, cu_seqlens, batch, max_seqlen, total, H, H_kv, D,
                             scale, causal, dtype, stream, fa::DropParams{}, "fa_forward_varlen");
}

fa_status fa_forward_varlen_dropout(const void* q, const void* k, const void* v, void* o,
                                    float* lse, const int32_t* cu_seqlens, int64_t batch,
                                    int64_t max_seqlen, int64_t total, int64_t H, int64_t H_kv,
                                    int64_t D, float scale, int causal, int dtype,
                                    float dropout_p, uint64_t seed, uint64_t offset,
                                    void* stream) {
  g_last_error[0] = '\0';
  const char* who = "fa_forward_varlen_dropout";
  fa::DropParams dp;
  fa_status s = drop_params(dropout_p, seed, offset, dtype, who, &dp);
  if (s != FA_OK) return s;
  return forward_varlen_impl(q, k, v, o, lse, cu_seqlens, batch, max_seqlen, total, H, H_kv, D,
                             scale, causal, dtype, stream, dp, who);
}

size_t fa_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D) {
  fa::BwdWorkspace ws;
  if (!fa::backward_workspace_layout(B, H, N, D, &ws)) return 0;
  return ws.total;
}

fa_status fa_backward(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                      int64_t D, float scale, int causal, int dtype, void* stream) {
  g_last_error[0] = '\0';
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N,
                       D, scale, causal, dtype, stream, fa::DropParams{}, "fa_backward");
}

fa_status fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                              int64_t N, int64_t D, float scale, int causal, int dtype,
                              float dropout_p, uint64_t seed, uint64_t offset, void* stream) {
  g_last_error[0] = '\0';
  fa::DropParams dp;
  fa_status s = drop_params(dropout_p, seed, offset, dtype, "fa_backward_dropout", &dp);
  if (s != FA_OK) return s;
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N,
                       D, scale, causal, dtype, stream, dp, "fa_backward_dropout");
}

fa_status fa_backward_gqa(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                          int64_t H_kv, int64_t N, int64_t D, float scale, int causal, int dtype,
                          float dropout_p, uint64_t seed, uint64_t offset, void* stream) {
  g_last_error[0] = '\0';
  const char* who = "fa_backward_gqa";
  fa::DropParams dp{};
  if (dropout_p != 0.f) {
    fa_status s = drop_params(dropout_p, seed, offset, dtype, who, &dp);
    if (s != FA_OK) return s;
  }
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H_kv,
                       N, D, scale, causal, dtype, stream, dp, who);
}

fa_status fa_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes,
                             int64_t batch, int64_t max_seqlen, int64_t total, int64_t H,
                             int64_t H_kv, int64_t D, float scale, int causal, int dtype,
                             void* stream) {
  g_last_error[0] = '\0';
  return backward_varlen_impl(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, workspace,
                              workspace_bytes, batch, max_seqlen, total, H, H_kv, D, scale,
                              causal, dtype, stream, fa::DropParams{}, "fa_backward_varlen");
}

fa_status fa_backward_varlen_dropout(const void* q, const void* k, const void* v, const void* o,
                                     const void* dout, const float* lse, void* dq, void* dk,
                                     void* dv, const int32_t* cu_seqlens, void* workspace,
                                     size_t workspace_bytes, int64_t batch, int64_t max_seqlen,
                                     int64_t total, int64_t H, int64_t H_kv, int64_t D,
                                     float scale, int causal, int dtype, float dropout_p,
                                     uint64_t seed, uint64_t offset, void* stream) {
  g_last_error[0] = '\0';
  const char* who = "fa_backward_varlen_dropout";
  fa::DropParams dp;
  fa_status s = drop_params(dropout_p, seed, offset, dtype, who, &dp);
  if (s != FA_OK) return s;
  return backward_varlen_impl(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, workspace,
                              workspace_bytes, batch, max_seqlen, total, H, H_kv, D, scale,
                              causal, dtype, stream, dp, who);
}

fa_status fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                              int dtype, void* stream) {
  g_last_error[0] = '\0';
  const char* who = "fa_backward_noalloc";
  fa::BwdWorkspace ws;
  fa_status s = check_backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, D, scale, dtype, who,
                               &ws);
  if (s != FA_OK) return s;
  if (ws.total > kScratchBytes)
    return fail(FA_ERR_UNSUPPORTED,
                "%s: B*H*N = %lld rows need %lld bytes of scratch, above the %lld this entry "
                "point holds (use fa_backward with a workspace)",
                who, (long long)(B * H * N), (long long)ws.total, (long long)kScratchBytes);
  void* ptr = nullptr;
  s = scratch_address(stream, &ptr, who);
  if (s != FA_OK) return s;
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, ptr, B, H, N, D, scale, causal, dtype,
                (hipStream_t)stream, fa::DropParams{}, H};
  return hip_status(fa::launch_backward(a, ws), who);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_UNKNOWN_STATUS";
  }
}

const char* fa_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

// Checks shared by the decode size query and the decode call.
fa_status check_decode(int64_t B, int64_t s_q, int64_t cap, int64_t max_seqlen_k, int64_t H,
                       int64_t H_kv, int64_t D, float scale, int dtype, const char* who) {
  if (B < 1 || s_q < 1 || cap < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: need batch, s_q, cache_capacity >= 1", who);
  if (max_seqlen_k < 0 || max_seqlen_k > cap)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: need 0 <= max_seqlen_k (%lld) <= capacity (%lld)",
                who, (long long)max_seqlen_k, (long long)cap);
  if (H_kv < 1 || H < 1 || H % H_kv != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: H (%lld) must be a positive multiple of H_kv (%lld)",
                who, (long long)H, (long long)H_kv);
  fa_status s = check_shape(B, H, cap, D, scale, dtype);
  if (s != FA_OK) return s;
  int64_t qelems = 0;
  if (__builtin_mul_overflow(B * H, s_q, &qelems) || __builtin_mul_overflow(qelems, D * 4, &qelems))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: B*s_q*H*D overflows", who);
  if (dtype == FA_FP32) return fail(FA_ERR_UNSUPPORTED, "%s: fp32 is not supported", who);
  if ((H / H_kv) * s_q > 32)
    return fail(FA_ERR_UNSUPPORTED,
                "%s: (H / H_kv) * s_q = %lld rows per K/V head; at most 32 are supported", who,
                (long long)((H / H_kv) * s_q));
  if (cap > (int64_t)1 << 30 || B * H_kv * fa::kMaxSplits > (int64_t)0x7fffffff)
    return fail(FA_ERR_UNSUPPORTED, "%s: sizes exceed one grid", who);
  return FA_OK;
}

}  // namespace

size_t fa_decode_workspace_bytes(int64_t batch, int64_t s_q, int64_t H, int64_t H_kv,
                                 int64_t max_seqlen_k, int64_t D) {
  fa::DecodePlan plan;
  if (!fa::decode_plan(batch, s_q, H, H_kv, max_seqlen_k, D, &plan)) return 0;
  return plan.total;
}

fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* cache_seqlens, void* o, float* lse, void* workspace,
                    size_t workspace_bytes, int64_t batch, int64_t s_q, int64_t cache_capacity,
                    int64_t max_seqlen_k, int64_t H, int64_t H_kv, int64_t D, float scale,
                    int dtype, void* stream) {
  g_last_error[0] = '\0';
  if (!q || !k_cache || !v_cache || !cache_seqlens || !o || !lse)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "fa_decode: q, k_cache, v_cache, cache_seqlens, o and lse must be non-NULL");
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(o, 16))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode: q, caches and o must be 16-byte aligned");
  if (misaligned(lse, 4) || misaligned(cache_seqlens, 4))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode: lse and cache_seqlens must be 4-byte aligned");
  fa_status s = check_decode(batch, s_q, cache_capacity, max_seqlen_k, H, H_kv, D, scale, dtype,
                             "fa_decode");
  if (s != FA_OK) return s;
  fa::DecodePlan plan;
  if (!fa::decode_plan(batch, s_q, H, H_kv, max_seqlen_k, D, &plan))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode: no plan for these sizes");
  if (plan.total > 0) {
    if (!workspace)
      return fail(FA_ERR_WORKSPACE, "fa_decode: workspace is NULL (needs %lld bytes)",
                  (long long)plan.total);
    if (workspace_bytes < plan.total)
      return fail(FA_ERR_WORKSPACE, "fa_decode: workspace too small (needs %lld bytes)",
                  (long long)plan.total);
    if (misaligned(workspace, 256))
      return fail(FA_ERR_WORKSPACE, "fa_decode: workspace must be 256-byte aligned");
  }
  fa::DecodeArgs a{q,     k_cache,        v_cache, cache_seqlens, o, lse, workspace,
                   batch, s_q,            cache_capacity, max_seqlen_k, H, H_kv, D,
                   scale, dtype, (hipStream_t)stream};
  return hip_status(fa::launch_decode(a, plan), "fa_decode");
}

fa_status fa_clock_probe(uint64_t* out, int iters, void* stream) {
  g_last_error[0] = '\0';
  if (!out) return fail(FA_ERR_INVALID_ARGUMENT, "fa_clock_probe: out must be non-NULL");
  if (misaligned(out, 8)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_clock_probe: out must be 8-byte aligned");
  if (iters < 1) return fail(FA_ERR_INVALID_ARGUMENT, "fa_clock_probe: iters must be >= 1 (got %d)", iters);
  return hip_status(fa::launch_clock_probe(out, iters, (hipStream_t)stream), "fa_clock_probe");
}
