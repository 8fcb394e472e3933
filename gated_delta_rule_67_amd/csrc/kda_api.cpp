// kda_api.cpp -- the C ABI of libkda: argument validation and kernel dispatch.
//
// Every host-visible argument is checked before anything is enqueued and
// before any HIP runtime call, so a rejected call touches neither the device
// nor the outputs.  Errors are returned as kda_status with a thread-local
// detail string; nothing throws across the ABI.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <vector>

#include "kda_launch.h"
#include "kda_validate.h"

namespace {

thread_local char g_last_error[512] = "";

kda_status fail(kda_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

// Prefill path.  bf16 q/k/v with d = 128 run chunked on MFMA in two passes
// (parallel per-chunk preparation, then the serial state scan); everything
// else runs the token-recurrent kernel.  KDA_PREFILL_PATH=recurrent forces the
// token-recurrent kernel for any problem (a test and diagnosis switch).
enum class Path { Recurrent, TwoPass };

Path prefill_path(const kda::ChunkLaunch& a) {
  const char* e = std::getenv("KDA_PREFILL_PATH");
  if (e && std::strcmp(e, "recurrent") == 0) return Path::Recurrent;
  if (kda::twopass_supported(a)) return Path::TwoPass;
  return Path::Recurrent;
}

size_t workspace_need(Path path, const kda::ChunkLaunch& a) {
  const bool packed = a.cu_seqlens != nullptr;
  return path == Path::TwoPass ? kda::twopass_workspace_bytes(a.num_seqs, a.seq_len, a.num_heads, packed) : 0;
}

// The launch record of a descriptor (pointers left empty; cu_seqlens only
// marks a packed problem).
kda::ChunkLaunch launch_of(const kda_desc* d, bool packed) {
  kda::ChunkLaunch a{};
  a.cu_seqlens = packed ? reinterpret_cast<const int32_t*>(uintptr_t(16)) : nullptr;
  a.num_seqs = d->num_seqs;
  a.seq_len = d->seq_len;
  a.num_heads = d->num_heads;
  a.d = d->dk;
  a.bf16 = d->qkv_dtype == KDA_BF16;
  a.out_bf16 = d->out_dtype == KDA_BF16;
  a.l2 = (d->flags & KDA_FLAG_QK_L2NORM) != 0;
  return a;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Checks shared by both entry points: descriptor fields.
kda_status check_desc(const kda_desc* d, const char* fn) {
  if (!d) return fail(KDA_ERR_NULL, "%s: desc is NULL", fn);
  if (d->num_seqs < 0 || d->num_heads <= 0 || d->dk <= 0 || d->dv <= 0)
    return fail(KDA_ERR_SHAPE, "%s: need num_seqs >= 0, num_heads > 0, dk > 0, dv > 0 (got %d, %d, %d, %d)",
                fn, d->num_seqs, d->num_heads, d->dk, d->dv);
  if (d->qkv_dtype != KDA_F32 && d->qkv_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, d->qkv_dtype);
  if (d->out_dtype != KDA_F32 && d->out_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "%s: unknown out_dtype %d", fn, d->out_dtype);
  if (!std::isfinite(d->scale))
    return fail(KDA_ERR_SHAPE, "%s: scale must be finite", fn);
  if (d->dk != d->dv)
    return fail(KDA_ERR_UNSUPPORTED, "%s: dk != dv (%d vs %d) is not supported", fn, d->dk, d->dv);
  if (d->dk != 16 && d->dk != 32 && d->dk != 64 && d->dk != 128)
    return fail(KDA_ERR_UNSUPPORTED, "%s: head dim %d not in {16, 32, 64, 128}", fn, d->dk);
  if ((d->flags & ~KDA_FLAG_QK_L2NORM) != 0 || d->reserved != 0)
    return fail(KDA_ERR_UNSUPPORTED, "%s: unknown flags 0x%x (reserved %u)", fn, d->flags, d->reserved);
  if (static_cast<int64_t>(d->num_seqs) * d->num_heads > (1 << 26))
    return fail(KDA_ERR_SHAPE, "%s: num_seqs * num_heads too large", fn);
  return KDA_OK;
}

float resolve_scale(const kda_desc* d) {
  return d->scale != 0.0f ? d->scale : 1.0f / std::sqrt(static_cast<float>(d->dk));
}

bool validate_mode() {
  const char* e = std::getenv("KDA_VALIDATE");
  return e && std::strcmp(e, "1") == 0;
}

// KDA_VALIDATE=1, before a launch: cu_seqlens and log_g copied to the host
// and checked (the preconditions that live in device memory).
kda_status validate_inputs(const int32_t* cu_seqlens, int num_docs, int64_t tokens, const float* log_g,
                           size_t n_log_g, hipStream_t s, const char* fn) {
  int64_t where = 0;
  if (cu_seqlens) {
    std::vector<int32_t> cu(static_cast<size_t>(num_docs) + 1);
    if (hipMemcpyAsync(cu.data(), cu_seqlens, cu.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): copying cu_seqlens failed", fn);
    if (const char* m = kda::validate::cu_seqlens(cu.data(), num_docs, tokens, &where))
      return fail(KDA_ERR_SHAPE, "%s (KDA_VALIDATE): %s (entry %lld)", fn, m, (long long)where);
  }
  if (n_log_g > 0) {
    std::vector<float> g(n_log_g);
    if (hipMemcpyAsync(g.data(), log_g, n_log_g * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): copying log_g failed", fn);
    if (const char* m = kda::validate::log_gates(g.data(), n_log_g, &where))
      return fail(KDA_ERR_SHAPE, "%s (KDA_VALIDATE): %s (element %lld)", fn, m, (long long)where);
  }
  return KDA_OK;
}

// KDA_VALIDATE=1, after a launch: every element of an output finite (the
// outputs were filled with NaN before the launch, so an unwritten element
// shows up too).
kda_status validate_output(const void* p, size_t count, bool bf16, const char* name, hipStream_t s,
                           const char* fn) {
  if (!p || count == 0) return KDA_OK;
  int64_t where = 0;
  const char* m = nullptr;
  if (bf16) {
    std::vector<uint16_t> h(count);
    if (hipMemcpyAsync(h.data(), p, count * 2, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): copying %s failed", fn, name);
    m = kda::validate::finite_bf16(h.data(), count, &where);
  } else {
    std::vector<float> h(count);
    if (hipMemcpyAsync(h.data(), p, count * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): copying %s failed", fn, name);
    m = kda::validate::finite_f32(h.data(), count, &where);
  }
  if (m) return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): element %lld of %s %s", fn, (long long)where, name, m);
  return KDA_OK;
}

kda_status check_ptr(const void* p, const char* name, const char* fn, bool required) {
  if (!p) return required ? fail(KDA_ERR_NULL, "%s: %s is NULL", fn, name) : KDA_OK;
  if (misaligned(p)) return fail(KDA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, name);
  return KDA_OK;
}

// The decode / verify checks shared by kda_step and kda_step_rows.
kda_status check_rows(const kda_desc* d, const void* q, const void* k, const void* v, const float* log_g,
                      const float* beta, const float* state, const char* state_name, int32_t n_tok,
                      const void* out, const char* fn) {
  kda_status st = check_desc(d, fn);
  if (st != KDA_OK) return st;
  if (n_tok < 1) return fail(KDA_ERR_SHAPE, "%s: n_tok must be >= 1 (got %d)", fn, n_tok);
  if (static_cast<int64_t>(d->num_seqs) * n_tok > INT32_MAX / 2)
    return fail(KDA_ERR_SHAPE, "%s: num_seqs * n_tok too large", fn);
  const bool any = d->num_seqs > 0;
  if ((st = check_ptr(q, "q", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(k, "k", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(v, "v", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(log_g, "log_g", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(beta, "beta", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(state, state_name, fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(out, "out", fn, any)) != KDA_OK) return st;
  if (out && (out == q || out == k || out == v || out == log_g || out == beta || out == state))
    return fail(KDA_ERR_SHAPE, "%s: out aliases an input", fn);
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "required pointer is NULL";
    case KDA_ERR_SHAPE: return "invalid shape or argument";
    case KDA_ERR_DTYPE: return "unknown dtype";
    case KDA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kda_last_error(void) { return g_last_error; }

size_t kda_chunk_workspace_bytes(const kda_desc* d, int packed) {
  if (!d || d->num_seqs < 0 || d->seq_len < 0 || d->num_heads <= 0) return 0;
  if (d->dk != d->dv) return 0;
  const kda::ChunkLaunch a = launch_of(d, packed != 0);
  return workspace_need(prefill_path(a), a);
}

kda_status kda_chunk_fwd(const kda_desc* d, const void* q, const void* k, const void* v,
                         const float* log_g, const float* beta, const float* init_state,
                         const int32_t* cu_seqlens, void* out, float* final_state, void* stream) {
  return kda::chunk_fwd_checked(d, q, k, v, log_g, beta, init_state, cu_seqlens, out, final_state, stream,
                                d ? d->workspace : nullptr, d ? d->workspace_bytes : 0, false, "kda_chunk_fwd");
}

kda_status kda_chunk_fwd_gated_norm(const kda_desc* d, const void* q, const void* k, const void* v,
                                    const float* log_g, const float* beta, const float* init_state,
                                    const int32_t* cu_seqlens, const void* gate, const float* norm_weight, float eps,
                                    void* out, float* final_state, void* stream) {
  const kda::OutNorm norm{gate, norm_weight, eps};
  return kda::chunk_fwd_checked(d, q, k, v, log_g, beta, init_state, cu_seqlens, out, final_state, stream,
                                d ? d->workspace : nullptr, d ? d->workspace_bytes : 0, false,
                                "kda_chunk_fwd_gated_norm", &norm);
}

kda_status kda_step_rows(const kda_desc* d, const void* q, const void* k, const void* v,
                         const float* log_g, const float* beta, const float* state, int32_t n_tok,
                         void* out, float* deltas, void* stream) {
  static const char* fn = "kda_step_rows";
  kda_status st = check_rows(d, q, k, v, log_g, beta, state, "state", n_tok, out, fn);
  if (st != KDA_OK) return st;
  const bool any = d->num_seqs > 0;
  if ((st = check_ptr(deltas, "deltas", fn, any)) != KDA_OK) return st;
  if (deltas && (deltas == out || deltas == q || deltas == k || deltas == v || deltas == log_g ||
                 deltas == beta || deltas == state))
    return fail(KDA_ERR_SHAPE, "%s: deltas aliases another argument", fn);
  if (!any) return KDA_OK;

  kda::StepLaunch a{};
  a.q = q; a.k = k; a.v = v; a.log_g = log_g; a.beta = beta;
  a.state = const_cast<float*>(state);  // read only: keep_state
  a.keep_state = true;
  a.out = out; a.deltas = deltas;
  a.num_seqs = d->num_seqs; a.n_tok = n_tok; a.num_heads = d->num_heads;
  a.d = d->dk; a.bf16 = d->qkv_dtype == KDA_BF16; a.scale = resolve_scale(d);
  a.out_bf16 = d->out_dtype == KDA_BF16; a.l2 = (d->flags & KDA_FLAG_QK_L2NORM) != 0;
  const hipError_t e = kda::launch_step(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_step_commit(const kda_desc* d, const void* k, const float* log_g, const float* deltas,
                           const int32_t* accept, float* state_inout, int32_t n_tok, void* stream) {
  static const char* fn = "kda_step_commit";
  kda_status st = check_desc(d, fn);
  if (st != KDA_OK) return st;
  if (n_tok < 1) return fail(KDA_ERR_SHAPE, "%s: n_tok must be >= 1 (got %d)", fn, n_tok);
  if (static_cast<int64_t>(d->num_seqs) * n_tok > INT32_MAX / 2)
    return fail(KDA_ERR_SHAPE, "%s: num_seqs * n_tok too large", fn);
  const bool any = d->num_seqs > 0;
  if ((st = check_ptr(k, "k", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(log_g, "log_g", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(deltas, "deltas", fn, any)) != KDA_OK) return st;
  if (any && !accept) return fail(KDA_ERR_NULL, "%s: accept is NULL", fn);
  if ((st = check_ptr(state_inout, "state_inout", fn, any)) != KDA_OK) return st;
  if (state_inout && (static_cast<const void*>(state_inout) == k || state_inout == log_g || state_inout == deltas))
    return fail(KDA_ERR_SHAPE, "%s: state_inout aliases an input", fn);
  if (!any) return KDA_OK;

  kda::CommitLaunch a{};
  a.k = k; a.log_g = log_g; a.deltas = deltas; a.accept = accept; a.state = state_inout;
  a.num_seqs = d->num_seqs; a.n_tok = n_tok; a.num_heads = d->num_heads;
  a.d = d->dk; a.bf16 = d->qkv_dtype == KDA_BF16; a.l2 = (d->flags & KDA_FLAG_QK_L2NORM) != 0;
  const hipError_t e = kda::launch_commit(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_step(const kda_desc* d, const void* q, const void* k, const void* v,
                    const float* log_g, const float* beta, float* state_inout, int32_t n_tok,
                    void* out, void* stream) {
  static const char* fn = "kda_step";
  const kda_status st = check_rows(d, q, k, v, log_g, beta, state_inout, "state_inout", n_tok, out, fn);
  if (st != KDA_OK) return st;
  if (d->num_seqs == 0) return KDA_OK;

  kda::StepLaunch a{};
  a.q = q; a.k = k; a.v = v; a.log_g = log_g; a.beta = beta;
  a.state = state_inout; a.out = out;
  a.num_seqs = d->num_seqs; a.n_tok = n_tok; a.num_heads = d->num_heads;
  a.d = d->dk; a.bf16 = d->qkv_dtype == KDA_BF16; a.scale = resolve_scale(d);
  a.out_bf16 = d->out_dtype == KDA_BF16; a.l2 = (d->flags & KDA_FLAG_QK_L2NORM) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n_out = static_cast<size_t>(d->num_seqs) * n_tok * d->num_heads * d->dv;
  const bool check = validate_mode();
  if (check) {
    const kda_status vs = validate_inputs(nullptr, 0, 0, log_g, n_out / d->dv * d->dk, s, fn);
    if (vs != KDA_OK) return vs;
    if (hipMemsetAsync(out, 0xff, n_out * (a.out_bf16 ? 2 : 4), s) != hipSuccess)
      return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): NaN fill failed", fn);
  }
  const hipError_t e = kda::launch_step(a, s);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  if (check) {
    if (hipStreamSynchronize(s) != hipSuccess) return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): kernel failed", fn);
    kda_status vs = validate_output(out, n_out, a.out_bf16, "out", s, fn);
    if (vs != KDA_OK) return vs;
    vs = validate_output(state_inout, static_cast<size_t>(d->num_seqs) * d->num_heads * d->dk * d->dv, false,
                         "state_inout", s, fn);
    if (vs != KDA_OK) return vs;
  }
  return KDA_OK;
}

size_t kda_chunk_bwd_workspace_bytes(const kda_desc* d, int packed) {
  if (!d || d->num_seqs < 0 || d->seq_len < 0 || d->num_heads <= 0) return 0;
  if (d->dk != d->dv || (d->dk != 16 && d->dk != 32 && d->dk != 64 && d->dk != 128)) return 0;
  return kda::bwd_workspace_bytes(d->num_seqs, d->seq_len, d->num_heads, d->dk, packed != 0);
}

kda_status kda_chunk_bwd(const kda_desc* d, const void* q, const void* k, const void* v,
                         const float* log_g, const float* beta, const float* init_state,
                         const int32_t* cu_seqlens, const float* d_out, const float* d_final_state,
                         float* dq, float* dk, float* dv, float* dlog_g, float* dbeta,
                         float* d_init_state, void* stream) {
  static const char* fn = "kda_chunk_bwd";
  kda_status st = check_desc(d, fn);
  if (st != KDA_OK) return st;
  if (d->flags != 0)
    return fail(KDA_ERR_UNSUPPORTED, "%s: flags 0x%x are not supported by the backward", fn, d->flags);
  if (d->seq_len < 0) return fail(KDA_ERR_SHAPE, "%s: seq_len < 0", fn);
  const bool packed = cu_seqlens != nullptr;
  const int64_t tokens = packed ? d->seq_len : static_cast<int64_t>(d->num_seqs) * d->seq_len;
  if (tokens > INT32_MAX / 2) return fail(KDA_ERR_SHAPE, "%s: too many tokens (%lld)", fn, (long long)tokens);
  if (packed && d->num_seqs == 0 && d->seq_len != 0)
    return fail(KDA_ERR_SHAPE, "%s: packed problem with tokens but no documents", fn);
  const bool has_tok = tokens > 0;
  const char* in_names[] = {"q", "k", "v", "log_g", "beta", "d_out"};
  const void* ins[] = {q, k, v, log_g, beta, d_out};
  for (int i = 0; i < 6; ++i)
    if ((st = check_ptr(ins[i], in_names[i], fn, has_tok)) != KDA_OK) return st;
  const char* out_names[] = {"dq", "dk", "dv", "dlog_g", "dbeta"};
  float* outs[] = {dq, dk, dv, dlog_g, dbeta};
  for (int i = 0; i < 5; ++i)
    if ((st = check_ptr(outs[i], out_names[i], fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(init_state, "init_state", fn, false)) != KDA_OK) return st;
  if ((st = check_ptr(d_final_state, "d_final_state", fn, false)) != KDA_OK) return st;
  if ((st = check_ptr(d_init_state, "d_init_state", fn, false)) != KDA_OK) return st;
  if ((st = check_ptr(cu_seqlens, "cu_seqlens", fn, false)) != KDA_OK) return st;
  // outputs alias neither an input nor each other
  const void* all_in[] = {q, k, v, log_g, beta, init_state, cu_seqlens, d_out, d_final_state};
  float* all_out[] = {dq, dk, dv, dlog_g, dbeta, d_init_state};
  for (int i = 0; i < 6; ++i) {
    if (!all_out[i]) continue;
    for (const void* p : all_in)
      if (p && p == all_out[i]) return fail(KDA_ERR_SHAPE, "%s: a gradient output aliases an input", fn);
    for (int j = 0; j < i; ++j)
      if (all_out[j] == all_out[i]) return fail(KDA_ERR_SHAPE, "%s: two gradient outputs alias", fn);
  }
  kda::BwdLaunch a{};
  a.num_seqs = d->num_seqs;
  a.seq_len = d->seq_len;
  a.num_heads = d->num_heads;
  a.d = d->dk;
  a.bf16 = d->qkv_dtype == KDA_BF16;
  a.cu_seqlens = cu_seqlens;
  if (!kda::bwd_supported(a)) return fail(KDA_ERR_SHAPE, "%s: problem too large", fn);
  const size_t ws_need = kda::bwd_workspace_bytes(d->num_seqs, d->seq_len, d->num_heads, d->dk, packed);
  const bool use_ws = has_tok || (packed && d->num_seqs > 0);  // packed: the chunk map lives there
  if (use_ws) {
    if (!d->workspace || d->workspace_bytes < ws_need)
      return fail(KDA_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", fn, ws_need,
                  d->workspace ? d->workspace_bytes : size_t(0));
    if (misaligned(d->workspace)) return fail(KDA_ERR_ALIGN, "%s: workspace is not 16-byte aligned", fn);
  }
  if (d->num_seqs == 0 || (!has_tok && !d_init_state)) return KDA_OK;
  a.q = q; a.k = k; a.v = v; a.log_g = log_g; a.beta = beta; a.init_state = init_state;
  a.d_out = d_out; a.d_final = d_final_state;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_g = dlog_g; a.dbeta = dbeta; a.d_init = d_init_state;
  a.workspace = use_ws ? d->workspace : nullptr;
  a.scale = resolve_scale(d);
  const hipError_t e = kda::launch_chunk_bwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_short_conv(const kda_desc* d, int32_t channels, int32_t kernel_size, int32_t activation,
                          const void* x, const float* weight, const int32_t* cu_seqlens, const float* init_cache,
                          void* out, float* final_cache, void* stream) {
  static const char* fn = "kda_short_conv";
  if (!d) return fail(KDA_ERR_NULL, "%s: desc is NULL", fn);
  if (d->num_seqs < 0 || d->seq_len < 0)
    return fail(KDA_ERR_SHAPE, "%s: need num_seqs >= 0 and seq_len >= 0 (got %d, %d)", fn, d->num_seqs, d->seq_len);
  if (d->qkv_dtype != KDA_F32 && d->qkv_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, d->qkv_dtype);
  if (channels <= 0 || channels % 8 != 0)
    return fail(KDA_ERR_SHAPE, "%s: channels must be a positive multiple of 8 (got %d)", fn, channels);
  if (kernel_size < 1 || kernel_size > 8)
    return fail(KDA_ERR_UNSUPPORTED, "%s: kernel_size %d not in [1, 8]", fn, kernel_size);
  if (activation != 0 && activation != 1)
    return fail(KDA_ERR_SHAPE, "%s: activation must be 0 (identity) or 1 (SiLU), got %d", fn, activation);
  const bool packed = cu_seqlens != nullptr;
  const int64_t tokens = packed ? d->seq_len : static_cast<int64_t>(d->num_seqs) * d->seq_len;
  if (tokens * channels > (int64_t(1) << 40)) return fail(KDA_ERR_SHAPE, "%s: problem too large", fn);
  if (tokens / 32 >= (int64_t(1) << 31)) return fail(KDA_ERR_SHAPE, "%s: too many tokens", fn);
  if (packed && d->num_seqs == 0 && d->seq_len != 0)
    return fail(KDA_ERR_SHAPE, "%s: packed problem with tokens but no documents", fn);
  const bool has_tok = tokens > 0;
  kda_status st;
  if ((st = check_ptr(x, "x", fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(out, "out", fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(weight, "weight", fn, has_tok || (final_cache && d->num_seqs > 0))) != KDA_OK) return st;
  if ((st = check_ptr(cu_seqlens, "cu_seqlens", fn, false)) != KDA_OK) return st;
  if ((st = check_ptr(init_cache, "init_cache", fn, false)) != KDA_OK) return st;
  if ((st = check_ptr(final_cache, "final_cache", fn, false)) != KDA_OK) return st;
  if (out && (out == x || out == static_cast<const void*>(weight) || out == init_cache || out == final_cache))
    return fail(KDA_ERR_SHAPE, "%s: out aliases another argument", fn);
  // In place (final_cache == init_cache) only where every document is read and
  // written by one thread: dense sequences whose length divides the kernel's
  // 32-token run, so that no sequence straddles two runs.
  if (init_cache && final_cache == init_cache && (packed || d->seq_len == 0 || 32 % d->seq_len != 0))
    return fail(KDA_ERR_SHAPE, "%s: final_cache may alias init_cache only for dense sequences of 1, 2, 4, 8, 16 "
                "or 32 tokens", fn);
  if (d->num_seqs == 0 || (!has_tok && !final_cache)) return KDA_OK;
  kda::ConvLaunch a{};
  a.x = x; a.weight = weight; a.cu_seqlens = cu_seqlens; a.init_cache = init_cache; a.final_cache = final_cache;
  a.out = out; a.num_seqs = d->num_seqs; a.seq_len = d->seq_len; a.channels = channels;
  a.kernel_size = kernel_size; a.activation = activation; a.bf16 = d->qkv_dtype == KDA_BF16;
  const hipError_t e = kda::launch_short_conv(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_gated_rmsnorm(const kda_desc* d, const float* o, const void* gate, const float* weight, float eps,
                             void* out, void* stream) {
  static const char* fn = "kda_gated_rmsnorm";
  if (!d) return fail(KDA_ERR_NULL, "%s: desc is NULL", fn);
  if (d->num_seqs < 0 || d->seq_len < 0 || d->num_heads <= 0)
    return fail(KDA_ERR_SHAPE, "%s: need num_seqs >= 0, seq_len >= 0, num_heads > 0", fn);
  if (d->qkv_dtype != KDA_F32 && d->qkv_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "%s: unknown qkv_dtype %d", fn, d->qkv_dtype);
  if (d->out_dtype != KDA_F32 && d->out_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "%s: unknown out_dtype %d", fn, d->out_dtype);
  if (d->dv != 16 && d->dv != 32 && d->dv != 64 && d->dv != 128)
    return fail(KDA_ERR_UNSUPPORTED, "%s: head dim %d not in {16, 32, 64, 128}", fn, d->dv);
  if (!std::isfinite(eps) || eps < 0.f) return fail(KDA_ERR_SHAPE, "%s: eps must be finite and >= 0", fn);
  const int64_t rows = static_cast<int64_t>(d->num_seqs) * d->seq_len * d->num_heads;
  if (rows > (int64_t(1) << 34)) return fail(KDA_ERR_SHAPE, "%s: too many rows", fn);
  const bool any = rows > 0;
  kda_status st;
  if ((st = check_ptr(o, "o", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(gate, "gate", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(weight, "weight", fn, any)) != KDA_OK) return st;
  if ((st = check_ptr(out, "out", fn, any)) != KDA_OK) return st;
  // in place over o is fine with fp32 out (each lane reads its channels before writing them)
  if (out && (out == gate || out == static_cast<const void*>(weight) ||
              (out == static_cast<const void*>(o) && d->out_dtype != KDA_F32)))
    return fail(KDA_ERR_SHAPE, "%s: out aliases gate or weight, or o with a bf16 out", fn);
  if (!any) return KDA_OK;
  kda::NormLaunch a{o, gate, weight, out, rows, d->dv, eps, d->qkv_dtype == KDA_BF16, d->out_dtype == KDA_BF16};
  const hipError_t e = kda::launch_gated_rmsnorm(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return KDA_OK;
}

}  // extern "C"

namespace kda {

kda_status fail_hip(const char* fn, const char* what, hipError_t e) {
  return fail(KDA_ERR_HIP, "%s: %s: %s", fn, what, hipGetErrorString(e));
}

kda_status chunk_fwd_checked(const kda_desc* d, const void* q, const void* k, const void* v, const float* log_g,
                             const float* beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                             float* final_state, void* stream, void* ws, size_t ws_bytes, bool fixed_ws,
                             const char* fn, const OutNorm* norm) {
  kda_status st = check_desc(d, fn);
  if (st != KDA_OK) return st;
  if (d->seq_len < 0) return fail(KDA_ERR_SHAPE, "%s: seq_len < 0", fn);
  const bool packed = cu_seqlens != nullptr;
  const int64_t tokens = packed ? d->seq_len : static_cast<int64_t>(d->num_seqs) * d->seq_len;
  if (tokens > INT32_MAX / 2) return fail(KDA_ERR_SHAPE, "%s: too many tokens (%lld)", fn, (long long)tokens);
  if (packed && d->num_seqs == 0 && d->seq_len != 0)
    return fail(KDA_ERR_SHAPE, "%s: packed problem with tokens but no documents", fn);
  const bool has_tok = tokens > 0;
  const bool has_units = d->num_seqs > 0;
  if ((st = check_ptr(q, "q", fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(k, "k", fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(v, "v", fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(log_g, "log_g", fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(beta, "beta", fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(out, "out", fn, has_tok)) != KDA_OK) return st;
  if ((st = check_ptr(init_state, "init_state", fn, false)) != KDA_OK) return st;
  if ((st = check_ptr(final_state, "final_state", fn, false)) != KDA_OK) return st;
  if ((st = check_ptr(cu_seqlens, "cu_seqlens", fn, false)) != KDA_OK) return st;
  if (out && (out == q || out == k || out == v || out == log_g || out == beta || out == init_state))
    return fail(KDA_ERR_SHAPE, "%s: out aliases an input", fn);
  kda::ChunkLaunch a = launch_of(d, packed);
  const Path path = prefill_path(a);
  if (norm) {
    if ((st = check_ptr(norm->gate, "gate", fn, has_tok)) != KDA_OK) return st;
    if ((st = check_ptr(norm->weight, "norm_weight", fn, has_tok)) != KDA_OK) return st;
    if (!std::isfinite(norm->eps) || norm->eps < 0.f) return fail(KDA_ERR_SHAPE, "%s: eps must be finite and >= 0", fn);
    if (out && (out == norm->gate || out == static_cast<const void*>(norm->weight)))
      return fail(KDA_ERR_SHAPE, "%s: out aliases gate or norm_weight", fn);
  }
  const size_t ws_need = workspace_need(path, a);
  if (ws_need > 0) {
    if (fixed_ws && ws_bytes < ws_need)
      return fail(KDA_ERR_WORKSPACE, "%s: the problem needs %zu bytes of scratch; the fixed scratch holds %zu", fn,
                  ws_need, ws_bytes);
    if (!ws || ws_bytes < ws_need)
      return fail(KDA_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", fn, ws_need, ws ? ws_bytes : size_t(0));
    if (misaligned(ws)) return fail(KDA_ERR_ALIGN, "%s: workspace is not 16-byte aligned", fn);
  }
  if (!has_units || (!has_tok && !final_state)) return KDA_OK;

  a.q = q; a.k = k; a.v = v; a.log_g = log_g; a.beta = beta;
  a.init_state = init_state; a.cu_seqlens = cu_seqlens;
  a.out = out; a.final_state = final_state;
  a.workspace = ws_need > 0 ? ws : nullptr;
  a.scale = resolve_scale(d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n_out = static_cast<size_t>(tokens) * d->num_heads * d->dv;
  const size_t n_fin = static_cast<size_t>(d->num_seqs) * d->num_heads * d->dk * d->dv;
  const bool check = validate_mode();
  if (check) {
    st = validate_inputs(cu_seqlens, d->num_seqs, d->seq_len, log_g, static_cast<size_t>(tokens) * d->num_heads * d->dk,
                         s, fn);
    if (st != KDA_OK) return st;
    // NaN fill (all-ones bits are a NaN in fp32 and in bf16): unwritten elements stay NaN
    if (hipMemsetAsync(out, 0xff, n_out * (a.out_bf16 ? 2 : 4), s) != hipSuccess ||
        (final_state && final_state != init_state && hipMemsetAsync(final_state, 0xff, n_fin * 4, s) != hipSuccess))
      return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): NaN fill failed", fn);
  }
  hipError_t e = path == Path::TwoPass ? kda::launch_chunk_twopass(a, s) : kda::launch_chunk_recurrent(a, s);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  if (norm && has_tok) {
    // the output, as just stored in its own dtype, normalised in place
    kda::NormLaunch nl{};
    nl.o = out;
    nl.gate = norm->gate;
    nl.weight = norm->weight;
    nl.out = out;
    nl.rows = tokens * d->num_heads;
    nl.d = d->dv;
    nl.eps = norm->eps;
    nl.gate_bf16 = d->qkv_dtype == KDA_BF16;
    nl.out_bf16 = a.out_bf16;
    nl.o_bf16 = a.out_bf16;
    e = kda::launch_gated_rmsnorm(nl, s);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  }
  if (check) {
    if (hipStreamSynchronize(s) != hipSuccess) return fail(KDA_ERR_HIP, "%s (KDA_VALIDATE): kernel failed", fn);
    if ((st = validate_output(out, n_out, a.out_bf16, "out", s, fn)) != KDA_OK) return st;
    if ((st = validate_output(final_state, n_fin, false, "final_state", s, fn)) != KDA_OK) return st;
  }
  return KDA_OK;
}

}  // namespace kda
