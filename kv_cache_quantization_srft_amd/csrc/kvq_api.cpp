// C ABI of libkvq (declared in include/kvq.h): host-side validation, error reporting and
// dispatch to the gfx950 kernels.  Validation runs before any HIP call, so a rejected call
// launches nothing and touches no output.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(kvq_status_string(st)) + ": " + buf;
  return st;
}

kvq_status ok() {
  g_last_error.clear();
  return KVQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by every entry point that takes a layout.
kvq_status check_layout(const kvq_layout* L, const char* fn) {
  if (!L) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: layout is NULL", fn);
  if (L->batch < 1 || L->kv_heads < 1 || L->capacity < 1)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: batch (%d), kv_heads (%d) and capacity (%d) must be >= 1", fn,
                L->batch, L->kv_heads, L->capacity);
  if (L->head_dim != 128 && L->head_dim != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 128, 256)", fn, L->head_dim);
  if (L->group_size != 16 && L->group_size != L->head_dim)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: group_size %d (supported: 16, or head_dim for one scale per vector)", fn,
                L->group_size);
  if (L->transform != KVQ_TRANSFORM_SRFT && L->transform != KVQ_TRANSFORM_SRHT)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: transform %d (supported: 0 = SRFT, 1 = SRHT)", fn, L->transform);
  const long long rows = (long long)L->batch * L->kv_heads;
  if (rows * (long long)L->capacity > (1LL << 40))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: batch*kv_heads*capacity too large", fn);
  return KVQ_OK;
}

kvq_status check_bits(int bits, const char* fn, const char* what) {
  if (bits != 4 && bits != 8) return fail(KVQ_ERR_UNSUPPORTED, "%s: %s %d (supported: 4, 8)", fn, what, bits);
  return KVQ_OK;
}

kvq_status check_ptr(const void* p, size_t align, const char* fn, const char* name) {
  if (!p) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, name);
  if (!aligned(p, align)) return fail(KVQ_ERR_MISALIGNED, "%s: %s is not %zu-byte aligned", fn, name, align);
  return KVQ_OK;
}

kvq_status check_opt_ptr(const void* p, size_t align, const char* fn, const char* name) {
  if (p && !aligned(p, align)) return fail(KVQ_ERR_MISALIGNED, "%s: %s is not %zu-byte aligned", fn, name, align);
  return KVQ_OK;
}

kvq_status check_range(const kvq_layout* L, int32_t pos, int32_t n_tok, const char* fn) {
  if (pos < 0 || n_tok < 1 || (long long)pos + n_tok > L->capacity)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: token range [pos=%d, pos+n_tok=%lld) must lie in [0, capacity=%d)", fn,
                pos, (long long)pos + n_tok, L->capacity);
  if ((long long)L->batch * L->kv_heads * n_tok > 0x7fffffffLL)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: batch x kv_heads x n_tok exceeds 2^31 - 1 vectors", fn);
  return KVQ_OK;
}

kvq_status check_strides(int64_t sign_bs, int64_t lambda_bs, const char* fn) {
  if (sign_bs < 0 || lambda_bs < 0) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: batch strides must be >= 0", fn);
  return KVQ_OK;
}

kvq_status hip_status(hipError_t e, const char* fn) {
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

#define KVQ_TRY(expr)               \
  do {                              \
    kvq_status _s = (expr);         \
    if (_s != KVQ_OK) return _s;    \
  } while (0)

// The quantized decode reads group-of-16 scale planes only.
kvq_status check_decode_group(const kvq_layout* L, const char* fn) {
  if (L->group_size != 16)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: group_size %d (decode supports 16; one scale per vector is a write-path mode)",
                fn, L->group_size);
  return KVQ_OK;
}

// workspace == nullptr with workspace_bytes == 0 and noalloc: the built-in scratch of the
// allocation-free call, checked against its size instead
kvq_status check_decode_common(const kvq_layout* L, const void* q, int32_t seq_len, const int32_t* seq_lens,
                               float sm_scale, void* workspace, size_t workspace_bytes, float* out,
                               const char* fn, bool append = false, bool noalloc = false) {
  if (L->q_heads < 1 || L->q_heads % L->kv_heads != 0)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: q_heads (%d) must be a positive multiple of kv_heads (%d)", fn,
                L->q_heads, L->kv_heads);
  if (L->q_heads / L->kv_heads > 64)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: GQA ratio %d (supported: <= 64)", fn, L->q_heads / L->kv_heads);
  if (seq_len < 1 || seq_len > L->capacity)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: seq_len %d must lie in [1, capacity=%d]", fn, seq_len, L->capacity);
  if (!std::isfinite(sm_scale)) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: sm_scale is not finite", fn);
  KVQ_TRY(check_ptr(q, 16, fn, "q"));
  KVQ_TRY(check_ptr(out, 16, fn, "out"));
  KVQ_TRY(check_opt_ptr(seq_lens, 4, fn, "seq_lens"));
  {
    const kvq_impl::DecodePlan pl =
        kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len, seq_len, false, append);
    const long units = long(L->batch) * L->kv_heads * pl.head_tiles;
    if (units > kvq_impl::kMaxDecodeUnits)
      return fail(KVQ_ERR_UNSUPPORTED, "%s: batch x kv_heads x head tiles = %ld exceeds %d", fn, units,
                  kvq_impl::kMaxDecodeUnits);
  }
  const size_t need = kvq_impl::decode_workspace_bytes(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len);
  if (noalloc) {
    if (need > kvq_impl::kNoAllocScratchBytes)
      return fail(KVQ_ERR_WORKSPACE_TOO_SMALL,
                  "%s: the call needs %zu bytes of scratch, the built-in scratch holds %zu (use kvq_decode_attn "
                  "with a caller workspace)",
                  fn, need, kvq_impl::kNoAllocScratchBytes);
    return KVQ_OK;
  }
  KVQ_TRY(check_ptr(workspace, 256, fn, "workspace"));
  if (workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
  return KVQ_OK;
}

}  // namespace

extern "C" {

int32_t kvq_version(void) { return 100; }

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK:
      return "KVQ_OK";
    case KVQ_ERR_INVALID_ARGUMENT:
      return "KVQ_ERR_INVALID_ARGUMENT";
    case KVQ_ERR_UNSUPPORTED:
      return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_MISALIGNED:
      return "KVQ_ERR_MISALIGNED";
    case KVQ_ERR_WORKSPACE_TOO_SMALL:
      return "KVQ_ERR_WORKSPACE_TOO_SMALL";
    case KVQ_ERR_HIP:
      return "KVQ_ERR_HIP";
  }
  return "KVQ_UNKNOWN_STATUS";
}

const char* kvq_last_error_message(void) { return g_last_error.c_str(); }

size_t kvq_codes_bytes(const kvq_layout* L, int32_t bits) {
  if (check_layout(L, "kvq_codes_bytes") != KVQ_OK || (bits != 4 && bits != 8)) return 0;
  return size_t(L->batch) * L->kv_heads * L->capacity * size_t(L->head_dim) * bits / 8;
}

size_t kvq_scales_bytes(const kvq_layout* L) {
  if (check_layout(L, "kvq_scales_bytes") != KVQ_OK) return 0;
  return size_t(L->batch) * L->kv_heads * L->capacity * size_t(L->head_dim / L->group_size) * 2;
}

kvq_status kvq_quantize(const kvq_layout* L, int32_t bits, const void* x_f16, int32_t pos, int32_t n_tok,
                        const float* sign, int64_t sign_batch_stride, const float* lambda,
                        int64_t lambda_batch_stride, void* codes, void* scales, void* stream) {
  const char* fn = "kvq_quantize";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_bits(bits, fn, "bits"));
  KVQ_TRY(check_range(L, pos, n_tok, fn));
  KVQ_TRY(check_ptr(x_f16, 16, fn, "x"));
  KVQ_TRY(check_ptr(sign, 4, fn, "sign"));
  KVQ_TRY(check_opt_ptr(lambda, 4, fn, "lambda"));
  KVQ_TRY(check_ptr(codes, 16, fn, "codes"));
  KVQ_TRY(check_ptr(scales, 16, fn, "scales"));
  KVQ_TRY(check_strides(sign_batch_stride, lambda_batch_stride, fn));
  kvq_impl::QuantArgs a{L->batch, L->kv_heads, L->head_dim, bits, L->capacity, pos, n_tok, x_f16, sign,
                        sign_batch_stride, lambda, lambda_batch_stride, codes, scales};
  a.transform = L->transform;
  a.group = L->group_size;
  return hip_status(kvq_impl::launch_quantize(a, static_cast<hipStream_t>(stream)), fn);
}

kvq_status kvq_quantize_fft(const kvq_layout* L, int32_t bits, const void* x_f16, int32_t pos, int32_t n_tok,
                            const float* sign, int64_t sign_batch_stride, const float* lambda,
                            int64_t lambda_batch_stride, void* codes, void* scales, void* stream) {
  const char* fn = "kvq_quantize_fft";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_bits(bits, fn, "bits"));
  KVQ_TRY(check_range(L, pos, n_tok, fn));
  KVQ_TRY(check_ptr(x_f16, 16, fn, "x"));
  KVQ_TRY(check_ptr(sign, 4, fn, "sign"));
  KVQ_TRY(check_opt_ptr(lambda, 4, fn, "lambda"));
  KVQ_TRY(check_ptr(codes, 16, fn, "codes"));
  KVQ_TRY(check_ptr(scales, 16, fn, "scales"));
  KVQ_TRY(check_strides(sign_batch_stride, lambda_batch_stride, fn));
  kvq_impl::QuantArgs a{L->batch, L->kv_heads, L->head_dim, bits, L->capacity, pos, n_tok, x_f16, sign,
                        sign_batch_stride, lambda, lambda_batch_stride, codes, scales};
  a.transform = L->transform;
  a.group = L->group_size;
  return hip_status(kvq_impl::launch_quantize_fft(a, static_cast<hipStream_t>(stream)), fn);
}

kvq_status kvq_dequantize(const kvq_layout* L, int32_t bits, const void* codes, const void* scales, int32_t pos,
                          int32_t n_tok, const float* sign, int64_t sign_batch_stride, const float* lambda,
                          int64_t lambda_batch_stride, float* out, void* stream) {
  const char* fn = "kvq_dequantize";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_bits(bits, fn, "bits"));
  KVQ_TRY(check_range(L, pos, n_tok, fn));
  KVQ_TRY(check_ptr(codes, 16, fn, "codes"));
  KVQ_TRY(check_ptr(scales, 16, fn, "scales"));
  KVQ_TRY(check_ptr(sign, 4, fn, "sign"));
  KVQ_TRY(check_opt_ptr(lambda, 4, fn, "lambda"));
  KVQ_TRY(check_ptr(out, 16, fn, "out"));
  KVQ_TRY(check_strides(sign_batch_stride, lambda_batch_stride, fn));
  kvq_impl::DequantArgs a{L->batch, L->kv_heads, L->head_dim, bits, L->capacity, pos, n_tok, codes, scales, sign,
                          sign_batch_stride, lambda, lambda_batch_stride, out};
  a.transform = L->transform;
  a.group = L->group_size;
  return hip_status(kvq_impl::launch_dequantize(a, static_cast<hipStream_t>(stream)), fn);
}

kvq_status kvq_calibrate_lambda(const kvq_layout* L, const void* x_f16, int32_t n_tok, int32_t n_cal,
                                const float* sign, int64_t sign_batch_stride, float* lambda, void* stream) {
  const char* fn = "kvq_calibrate_lambda";
  KVQ_TRY(check_layout(L, fn));
  if (n_tok < 1 || n_cal < 1 || n_cal > n_tok)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: need 1 <= n_cal (%d) <= n_tok (%d)", fn, n_cal, n_tok);
  KVQ_TRY(check_ptr(x_f16, 16, fn, "x"));
  KVQ_TRY(check_ptr(sign, 4, fn, "sign"));
  KVQ_TRY(check_ptr(lambda, 4, fn, "lambda"));
  KVQ_TRY(check_strides(sign_batch_stride, 0, fn));
  kvq_impl::CalibArgs a{L->batch, L->kv_heads, L->head_dim, n_tok, n_cal, x_f16, sign, sign_batch_stride, lambda};
  a.transform = L->transform;
  return hip_status(kvq_impl::launch_calibrate(a, static_cast<hipStream_t>(stream)), fn);
}

size_t kvq_decode_attn_workspace_bytes(const kvq_layout* L, int32_t max_seq_len) {
  if (check_layout(L, "kvq_decode_attn_workspace_bytes") != KVQ_OK) return 0;
  if (L->q_heads < 1 || L->q_heads % L->kv_heads != 0 || max_seq_len < 1) return 0;
  return kvq_impl::decode_workspace_bytes(L->batch, L->kv_heads, L->q_heads, L->head_dim, max_seq_len);
}

kvq_status kvq_decode_attn(const kvq_layout* L, const void* q_f16, const void* k_codes, const void* k_scales,
                           const void* v_codes, const void* v_scales, int32_t seq_len, const int32_t* seq_lens,
                           const float* sign_k, const float* sign_v, int64_t sign_batch_stride,
                           const float* lambda_k, const float* lambda_v, int64_t lambda_batch_stride,
                           float sm_scale, void* workspace, size_t workspace_bytes, float* out, void* stream) {
  const char* fn = "kvq_decode_attn";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_bits(L->k_bits, fn, "k_bits"));
  KVQ_TRY(check_bits(L->v_bits, fn, "v_bits"));
  KVQ_TRY(check_decode_group(L, fn));
  KVQ_TRY(check_decode_common(L, q_f16, seq_len, seq_lens, sm_scale, workspace, workspace_bytes, out, fn));
  KVQ_TRY(check_ptr(k_codes, 16, fn, "k_codes"));
  KVQ_TRY(check_ptr(k_scales, 16, fn, "k_scales"));
  KVQ_TRY(check_ptr(v_codes, 16, fn, "v_codes"));
  KVQ_TRY(check_ptr(v_scales, 16, fn, "v_scales"));
  KVQ_TRY(check_ptr(sign_k, 4, fn, "sign_k"));
  KVQ_TRY(check_ptr(sign_v, 4, fn, "sign_v"));
  KVQ_TRY(check_opt_ptr(lambda_k, 4, fn, "lambda_k"));
  KVQ_TRY(check_opt_ptr(lambda_v, 4, fn, "lambda_v"));
  KVQ_TRY(check_strides(sign_batch_stride, lambda_batch_stride, fn));
  const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(float(L->head_dim));
  const kvq_impl::DecodePlan p =
      kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len, seq_len, false);
  kvq_impl::DecodeArgs a{L->batch,   L->kv_heads, L->q_heads, L->head_dim, L->k_bits,   L->v_bits,
                         L->capacity, seq_len,    seq_lens,   q_f16,       k_codes,     k_scales,
                         v_codes,    v_scales,    sign_k,     sign_v,      sign_batch_stride, lambda_k,
                         lambda_v,   lambda_batch_stride,     scale,       workspace,   out};
  a.transform = L->transform;
  return hip_status(kvq_impl::launch_decode(a, p, static_cast<hipStream_t>(stream)), fn);
}

kvq_status kvq_decode_attn_noalloc(const kvq_layout* L, const void* q_f16, const void* k_codes,
                                   const void* k_scales, const void* v_codes, const void* v_scales, int32_t seq_len,
                                   const int32_t* seq_lens, const float* sign_k, const float* sign_v,
                                   int64_t sign_batch_stride, const float* lambda_k, const float* lambda_v,
                                   int64_t lambda_batch_stride, float sm_scale, float* out, void* stream) {
  const char* fn = "kvq_decode_attn_noalloc";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_bits(L->k_bits, fn, "k_bits"));
  KVQ_TRY(check_bits(L->v_bits, fn, "v_bits"));
  KVQ_TRY(check_decode_group(L, fn));
  KVQ_TRY(check_decode_common(L, q_f16, seq_len, seq_lens, sm_scale, nullptr, 0, out, fn, false, true));
  KVQ_TRY(check_ptr(k_codes, 16, fn, "k_codes"));
  KVQ_TRY(check_ptr(k_scales, 16, fn, "k_scales"));
  KVQ_TRY(check_ptr(v_codes, 16, fn, "v_codes"));
  KVQ_TRY(check_ptr(v_scales, 16, fn, "v_scales"));
  KVQ_TRY(check_ptr(sign_k, 4, fn, "sign_k"));
  KVQ_TRY(check_ptr(sign_v, 4, fn, "sign_v"));
  KVQ_TRY(check_opt_ptr(lambda_k, 4, fn, "lambda_k"));
  KVQ_TRY(check_opt_ptr(lambda_v, 4, fn, "lambda_v"));
  KVQ_TRY(check_strides(sign_batch_stride, lambda_batch_stride, fn));
  void* ws = nullptr;
  const hipError_t e = kvq_impl::noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: scratch set-up: %s", fn, hipGetErrorString(e));
  const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(float(L->head_dim));
  const kvq_impl::DecodePlan p =
      kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len, seq_len, false);
  kvq_impl::DecodeArgs a{L->batch,   L->kv_heads, L->q_heads, L->head_dim, L->k_bits,   L->v_bits,
                         L->capacity, seq_len,    seq_lens,   q_f16,       k_codes,     k_scales,
                         v_codes,    v_scales,    sign_k,     sign_v,      sign_batch_stride, lambda_k,
                         lambda_v,   lambda_batch_stride,     scale,       ws,          out};
  a.transform = L->transform;
  return hip_status(kvq_impl::launch_decode(a, p, static_cast<hipStream_t>(stream)), fn);
}

kvq_status kvq_decode_attn_append(const kvq_layout* L, const void* q_f16, const void* k_new_f16,
                                  const void* v_new_f16, void* k_codes, void* k_scales, void* v_codes,
                                  void* v_scales, int32_t seq_len, const int32_t* seq_lens, const float* sign_k,
                                  const float* sign_v, int64_t sign_batch_stride, const float* lambda_k,
                                  const float* lambda_v, int64_t lambda_batch_stride, float sm_scale,
                                  void* workspace, size_t workspace_bytes, float* out, void* stream) {
  const char* fn = "kvq_decode_attn_append";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_bits(L->k_bits, fn, "k_bits"));
  KVQ_TRY(check_bits(L->v_bits, fn, "v_bits"));
  KVQ_TRY(check_decode_group(L, fn));
  KVQ_TRY(check_decode_common(L, q_f16, seq_len, seq_lens, sm_scale, workspace, workspace_bytes, out, fn, true));
  KVQ_TRY(check_ptr(k_new_f16, 16, fn, "k_new"));
  KVQ_TRY(check_ptr(v_new_f16, 16, fn, "v_new"));
  KVQ_TRY(check_ptr(k_codes, 16, fn, "k_codes"));
  KVQ_TRY(check_ptr(k_scales, 16, fn, "k_scales"));
  KVQ_TRY(check_ptr(v_codes, 16, fn, "v_codes"));
  KVQ_TRY(check_ptr(v_scales, 16, fn, "v_scales"));
  KVQ_TRY(check_ptr(sign_k, 4, fn, "sign_k"));
  KVQ_TRY(check_ptr(sign_v, 4, fn, "sign_v"));
  KVQ_TRY(check_opt_ptr(lambda_k, 4, fn, "lambda_k"));
  KVQ_TRY(check_opt_ptr(lambda_v, 4, fn, "lambda_v"));
  KVQ_TRY(check_strides(sign_batch_stride, lambda_batch_stride, fn));
  const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(float(L->head_dim));
  const kvq_impl::DecodePlan p =
      kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len, seq_len, false, true);
  kvq_impl::DecodeArgs a{L->batch,   L->kv_heads, L->q_heads, L->head_dim, L->k_bits,   L->v_bits,
                         L->capacity, seq_len,    seq_lens,   q_f16,       k_codes,     k_scales,
                         v_codes,    v_scales,    sign_k,     sign_v,      sign_batch_stride, lambda_k,
                         lambda_v,   lambda_batch_stride,     scale,       workspace,   out};
  a.transform = L->transform;
  a.k_new = k_new_f16;
  a.v_new = v_new_f16;
  return hip_status(kvq_impl::launch_decode(a, p, static_cast<hipStream_t>(stream)), fn);
}

kvq_status kvq_decode_attn_paged(const kvq_layout* L, const void* q_f16, const void* k_new_f16,
                                 const void* v_new_f16, void* k_codes, void* k_scales, void* v_codes, void* v_scales,
                                 const int32_t* page_table, int32_t pages_per_seq, int32_t page_size,
                                 int32_t num_pages, int32_t seq_len, const int32_t* seq_lens, const float* sign_k,
                                 const float* sign_v, int64_t sign_batch_stride, const float* lambda_k,
                                 const float* lambda_v, int64_t lambda_batch_stride, float sm_scale, void* workspace,
                                 size_t workspace_bytes, float* out, void* stream) {
  const char* fn = "kvq_decode_attn_paged";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_bits(L->k_bits, fn, "k_bits"));
  KVQ_TRY(check_bits(L->v_bits, fn, "v_bits"));
  KVQ_TRY(check_decode_group(L, fn));
  if (page_size < 64 || page_size % 64 != 0)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: page_size %d (supported: a positive multiple of 64)", fn, page_size);
  if (pages_per_seq < 1 || num_pages < 1)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: pages_per_seq (%d) and num_pages (%d) must be >= 1", fn,
                pages_per_seq, num_pages);
  if ((long long)pages_per_seq * page_size != L->capacity)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: capacity (%d) must equal pages_per_seq x page_size (%lld)", fn,
                L->capacity, (long long)pages_per_seq * page_size);
  if ((long long)num_pages * L->kv_heads * page_size > (1LL << 40))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: num_pages*kv_heads*page_size too large", fn);
  const bool append = k_new_f16 != nullptr || v_new_f16 != nullptr;
  KVQ_TRY(check_decode_common(L, q_f16, seq_len, seq_lens, sm_scale, workspace, workspace_bytes, out, fn, append));
  if (append) {
    KVQ_TRY(check_ptr(k_new_f16, 16, fn, "k_new"));
    KVQ_TRY(check_ptr(v_new_f16, 16, fn, "v_new"));
  }
  KVQ_TRY(check_ptr(page_table, 4, fn, "page_table"));
  KVQ_TRY(check_ptr(k_codes, 16, fn, "k_codes"));
  KVQ_TRY(check_ptr(k_scales, 16, fn, "k_scales"));
  KVQ_TRY(check_ptr(v_codes, 16, fn, "v_codes"));
  KVQ_TRY(check_ptr(v_scales, 16, fn, "v_scales"));
  KVQ_TRY(check_ptr(sign_k, 4, fn, "sign_k"));
  KVQ_TRY(check_ptr(sign_v, 4, fn, "sign_v"));
  KVQ_TRY(check_opt_ptr(lambda_k, 4, fn, "lambda_k"));
  KVQ_TRY(check_opt_ptr(lambda_v, 4, fn, "lambda_v"));
  KVQ_TRY(check_strides(sign_batch_stride, lambda_batch_stride, fn));
  const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(float(L->head_dim));
  const kvq_impl::DecodePlan p =
      kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len, seq_len, false, append, true);
  kvq_impl::DecodeArgs a{L->batch,   L->kv_heads, L->q_heads, L->head_dim, L->k_bits,   L->v_bits,
                         L->capacity, seq_len,    seq_lens,   q_f16,       k_codes,     k_scales,
                         v_codes,    v_scales,    sign_k,     sign_v,      sign_batch_stride, lambda_k,
                         lambda_v,   lambda_batch_stride,     scale,       workspace,   out};
  a.transform = L->transform;
  a.k_new = k_new_f16;
  a.v_new = v_new_f16;
  a.page_table = page_table;
  a.page_size = page_size;
  a.pages_per_seq = pages_per_seq;
  a.num_pages = num_pages;
  return hip_status(kvq_impl::launch_decode(a, p, static_cast<hipStream_t>(stream)), fn);
}

kvq_status kvq_decode_attn_fp16(const kvq_layout* L, const void* q_f16, const void* k_f16, const void* v_f16,
                                int32_t seq_len, const int32_t* seq_lens, float sm_scale, void* workspace,
                                size_t workspace_bytes, float* out, void* stream) {
  const char* fn = "kvq_decode_attn_fp16";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_decode_common(L, q_f16, seq_len, seq_lens, sm_scale, workspace, workspace_bytes, out, fn));
  KVQ_TRY(check_ptr(k_f16, 16, fn, "k"));
  KVQ_TRY(check_ptr(v_f16, 16, fn, "v"));
  const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(float(L->head_dim));
  const kvq_impl::DecodePlan p =
      kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len, seq_len, true);
  kvq_impl::DecodeF16Args a{L->batch, L->kv_heads, L->q_heads, L->head_dim, L->capacity, seq_len, seq_lens,
                            q_f16,    k_f16,       v_f16,      scale,       workspace,   out};
  return hip_status(kvq_impl::launch_decode_f16(a, p, static_cast<hipStream_t>(stream)), fn);
}

kvq_status kvq_launch_plan(const kvq_layout* L, kvq_call call, int32_t n, kvq_plan* out) {
  const char* fn = "kvq_launch_plan";
  KVQ_TRY(check_layout(L, fn));
  if (!out) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: out is NULL", fn);
  kvq_plan r{};
  if (call == KVQ_CALL_QUANTIZE) {
    KVQ_TRY(check_range(L, 0, n, fn));
    const kvq_impl::QuantPlan q = kvq_impl::plan_quantize(L->head_dim, int64_t(L->batch) * L->kv_heads * n);
    r.work_groups = q.grid;
    r.blocks = q.blocks;
    r.blocks_per_work_group = (q.blocks + q.grid - 1) / q.grid;
    *out = r;
    return ok();
  }
  if (call < KVQ_CALL_DECODE || call > KVQ_CALL_DECODE_FP16)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: unknown call %d", fn, int(call));
  if (L->q_heads < 1 || L->q_heads % L->kv_heads != 0)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: q_heads (%d) must be a positive multiple of kv_heads (%d)", fn,
                L->q_heads, L->kv_heads);
  if (L->q_heads / L->kv_heads > 64)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: GQA ratio %d (supported: <= 64)", fn, L->q_heads / L->kv_heads);
  if (n < 1 || n > L->capacity)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: seq_len %d must lie in [1, capacity=%d]", fn, n, L->capacity);
  const bool f16 = call == KVQ_CALL_DECODE_FP16;
  const bool append = call == KVQ_CALL_DECODE_APPEND || call == KVQ_CALL_DECODE_PAGED_APPEND;
  const bool paged = call == KVQ_CALL_DECODE_PAGED || call == KVQ_CALL_DECODE_PAGED_APPEND;
  const kvq_impl::DecodePlan p =
      kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, n, n, f16, append, paged);
  const int64_t units = int64_t(L->batch) * L->kv_heads * p.head_tiles;
  r.work_groups = units * p.n_chunks;
  r.head_tile = p.head_tile;
  r.head_tiles = p.head_tiles;
  r.chunk = p.chunk;
  r.n_chunks = p.n_chunks;
  r.wave_tokens = f16 ? 32 : 64;
  r.superblocks_per_wave = (p.chunk + 4 * r.wave_tokens - 1) / (4 * r.wave_tokens);
  r.query_tile = r.query_tiles = 1;
  *out = r;
  return ok();
}

// Shared checks of the multi-token / windowed attention (kvq_attn and its sizing calls).
static kvq_status check_attn_opts(const kvq_layout* L, const kvq_attn_opts* o, int32_t seq_len, const char* fn) {
  if (!o) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: opts is NULL", fn);
  if (o->n_query < 1 || o->window < 0 || (o->ring != 0 && o->ring != 1))
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: need n_query >= 1 (%d), window >= 0 (%d), ring 0 or 1 (%d)", fn,
                o->n_query, o->window, o->ring);
  if (L->q_heads < 1 || L->q_heads % L->kv_heads != 0)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: q_heads (%d) must be a positive multiple of kv_heads (%d)", fn,
                L->q_heads, L->kv_heads);
  if (L->q_heads / L->kv_heads > 64)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: GQA ratio %d (supported: <= 64)", fn, L->q_heads / L->kv_heads);
  if (seq_len < 1) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: seq_len %d must be >= 1", fn, seq_len);
  if (o->ring) {
    if (L->capacity % 64 != 0)
      return fail(KVQ_ERR_UNSUPPORTED, "%s: a ring buffer needs capacity (%d) a multiple of 64", fn, L->capacity);
    if (o->window < 1 || (long long)o->window + o->n_query - 1 > L->capacity)
      return fail(KVQ_ERR_INVALID_ARGUMENT,
                  "%s: a ring buffer needs 1 <= window and window + n_query - 1 <= capacity (window %d, n_query %d, "
                  "capacity %d)",
                  fn, o->window, o->n_query, L->capacity);
  } else if (seq_len > L->capacity) {
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: seq_len %d must lie in [1, capacity=%d] without a ring buffer", fn,
                seq_len, L->capacity);
  }
  return KVQ_OK;
}

size_t kvq_attn_workspace_bytes(const kvq_layout* L, const kvq_attn_opts* o, int32_t max_seq_len) {
  if (check_layout(L, "kvq_attn_workspace_bytes") != KVQ_OK) return 0;
  if (check_attn_opts(L, o, max_seq_len, "kvq_attn_workspace_bytes") != KVQ_OK) return 0;
  return kvq_impl::attn_workspace_bytes(L->batch, L->kv_heads, L->q_heads, L->head_dim, max_seq_len, o->n_query,
                                        o->window);
}

kvq_status kvq_attn_launch_plan(const kvq_layout* L, const kvq_attn_opts* o, int32_t seq_len, int32_t paged,
                                kvq_plan* out) {
  const char* fn = "kvq_attn_launch_plan";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_attn_opts(L, o, seq_len, fn));
  if (!out) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: out is NULL", fn);
  const kvq_impl::DecodePlan p = kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len,
                                                       seq_len, false, false, paged != 0, o->n_query, o->window);
  kvq_plan r{};
  r.work_groups = int64_t(L->batch) * L->kv_heads * p.head_tiles * p.tok_tiles * p.n_chunks;
  r.head_tile = p.head_tile;
  r.head_tiles = p.head_tiles;
  r.chunk = p.chunk;
  r.n_chunks = p.n_chunks;
  r.wave_tokens = 64;
  r.superblocks_per_wave = (p.chunk + 255) / 256;
  r.query_tile = p.tok_tile;
  r.query_tiles = p.tok_tiles;
  *out = r;
  return ok();
}

kvq_status kvq_attn(const kvq_layout* L, const kvq_attn_opts* o, const void* q_f16, const void* k_codes,
                    const void* k_scales, const void* v_codes, const void* v_scales, const int32_t* page_table,
                    int32_t pages_per_seq, int32_t page_size, int32_t num_pages, int32_t seq_len,
                    const int32_t* seq_lens, const float* sign_k, const float* sign_v, int64_t sign_batch_stride,
                    const float* lambda_k, const float* lambda_v, int64_t lambda_batch_stride, float sm_scale,
                    void* workspace, size_t workspace_bytes, float* out, void* stream) {
  const char* fn = "kvq_attn";
  KVQ_TRY(check_layout(L, fn));
  KVQ_TRY(check_bits(L->k_bits, fn, "k_bits"));
  KVQ_TRY(check_bits(L->v_bits, fn, "v_bits"));
  KVQ_TRY(check_decode_group(L, fn));
  KVQ_TRY(check_attn_opts(L, o, seq_len, fn));
  if (!std::isfinite(sm_scale)) return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: sm_scale is not finite", fn);
  const bool paged = page_table != nullptr;
  if (paged) {
    if (page_size < 64 || page_size % 64 != 0)
      return fail(KVQ_ERR_UNSUPPORTED, "%s: page_size %d (supported: a positive multiple of 64)", fn, page_size);
    if (pages_per_seq < 1 || num_pages < 1)
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: pages_per_seq (%d) and num_pages (%d) must be >= 1", fn,
                  pages_per_seq, num_pages);
    if ((long long)pages_per_seq * page_size != L->capacity)
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: capacity (%d) must equal pages_per_seq x page_size (%lld)", fn,
                  L->capacity, (long long)pages_per_seq * page_size);
    if ((long long)num_pages * L->kv_heads * page_size > (1LL << 40))
      return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: num_pages*kv_heads*page_size too large", fn);
    KVQ_TRY(check_ptr(page_table, 4, fn, "page_table"));
  }
  KVQ_TRY(check_ptr(q_f16, 16, fn, "q"));
  KVQ_TRY(check_ptr(out, 16, fn, "out"));
  KVQ_TRY(check_opt_ptr(seq_lens, 4, fn, "seq_lens"));
  KVQ_TRY(check_ptr(k_codes, 16, fn, "k_codes"));
  KVQ_TRY(check_ptr(k_scales, 16, fn, "k_scales"));
  KVQ_TRY(check_ptr(v_codes, 16, fn, "v_codes"));
  KVQ_TRY(check_ptr(v_scales, 16, fn, "v_scales"));
  KVQ_TRY(check_ptr(sign_k, 4, fn, "sign_k"));
  KVQ_TRY(check_ptr(sign_v, 4, fn, "sign_v"));
  KVQ_TRY(check_opt_ptr(lambda_k, 4, fn, "lambda_k"));
  KVQ_TRY(check_opt_ptr(lambda_v, 4, fn, "lambda_v"));
  KVQ_TRY(check_strides(sign_batch_stride, lambda_batch_stride, fn));
  const kvq_impl::DecodePlan p = kvq_impl::plan_decode(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len,
                                                       seq_len, false, false, paged, o->n_query, o->window);
  const long long units = (long long)L->batch * L->kv_heads * p.head_tiles * p.tok_tiles;
  if (units > kvq_impl::kMaxDecodeUnits)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: batch x kv_heads x head tiles x query tiles = %lld exceeds %d", fn, units,
                kvq_impl::kMaxDecodeUnits);
  if ((long long)L->batch * o->n_query * L->q_heads > 0x7fffffffLL)
    return fail(KVQ_ERR_INVALID_ARGUMENT, "%s: batch x n_query x q_heads exceeds 2^31 - 1 rows", fn);
  KVQ_TRY(check_ptr(workspace, 256, fn, "workspace"));
  const size_t need = kvq_impl::attn_workspace_bytes(L->batch, L->kv_heads, L->q_heads, L->head_dim, seq_len,
                                                     o->n_query, o->window);
  if (workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
  const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(float(L->head_dim));
  kvq_impl::DecodeArgs a{L->batch,   L->kv_heads, L->q_heads, L->head_dim, L->k_bits,   L->v_bits,
                         L->capacity, seq_len,    seq_lens,   q_f16,       k_codes,     k_scales,
                         v_codes,    v_scales,    sign_k,     sign_v,      sign_batch_stride, lambda_k,
                         lambda_v,   lambda_batch_stride,     scale,       workspace,   out};
  a.transform = L->transform;
  a.page_table = page_table;
  a.page_size = page_size;
  a.pages_per_seq = pages_per_seq;
  a.num_pages = num_pages;
  a.n_query = o->n_query;
  a.window = o->window;
  a.ring = o->ring;
  return hip_status(kvq_impl::launch_decode(a, p, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
