// C ABI of libswasink: argument validation, kernel selection, error reporting.
// The operator and the conventions are documented in include/swasink.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <initializer_list>

#include "../../include/swasink.h"
#include "kernels.h"

// Scratch array of swa_sink_prefill_backward_noalloc, owned by the library: the
// backward's per-row delta and sink terms (2 x total_tokens x num_q_heads fp32) for
// callers that cannot allocate.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` only names a host-side stand-in; its device
// address is looked up once per device (hipGetSymbolAddress with that device current)
// and only that address is passed to kernels.  Nothing in it must start at zero: every
// element a call reads was written earlier in the same call.
constexpr int64_t kNoAllocScratchBytes = 16ll << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace swa {

hipError_t device_cu_count(int* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) { *out = v; return hipSuccess; }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) n = 1;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

}  // namespace swa

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return SWA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SWA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_dtype(int dtype) {
  if (dtype != SWA_DTYPE_F32 && dtype != SWA_DTYPE_BF16)
    return fail(SWA_ERR_DTYPE, "unknown dtype %d (0 = f32, 1 = bf16)", dtype);
  return SWA_OK;
}

int check_heads(int32_t hq, int32_t hkv, int32_t d) {
  if (hq < 1 || hkv < 1) return fail(SWA_ERR_SHAPE, "head counts must be >= 1 (got %d, %d)", hq, hkv);
  if (hq % hkv != 0)
    return fail(SWA_ERR_SHAPE, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", hq, hkv);
  if (d != 64 && d != 128) return fail(SWA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d);
  return SWA_OK;
}

// The kernels read and write the tensors with 16-byte vector accesses.
int check_aligned(const char* name, const char* what, std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 15u)
      return fail(SWA_ERR_UNSUPPORTED, "%s: %s must be 16-byte aligned", name, what);
  return SWA_OK;
}

float resolve_scale(float scale, int32_t d) {
  return (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf((float)d);
}

int prefill_common(const void* q, const void* k, const void* v, const float* sinks,
                   bool need_sinks, const int32_t* cu_seqlens, int32_t num_seqs,
                   int32_t total_tokens, int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t d,
                   int32_t window, float scale, int dtype, void* out, float* lse, void* stream,
                   const char* name, bool fp8 = false, float k_scale = 1.f, float v_scale = 1.f) {
  int rc = check_dtype(dtype);
  if (rc) return rc;
  if (fp8 && !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
    return fail(SWA_ERR_SHAPE, "%s: k_scale and v_scale must be finite and > 0", name);
  if (total_tokens < 0) return fail(SWA_ERR_SHAPE, "%s: total_tokens must be >= 0", name);
  if (num_seqs < 1) return fail(SWA_ERR_SHAPE, "%s: num_seqs must be >= 1", name);
  if (total_tokens > 0 && (max_seqlen < 1 || max_seqlen > total_tokens))
    return fail(SWA_ERR_SHAPE, "%s: max_seqlen must be in [1, total_tokens]", name);
  if ((rc = check_heads(hq, hkv, d))) return rc;
  if (window < 1) return fail(SWA_ERR_SHAPE, "%s: window must be >= 1 (got %d)", name, window);
  if ((long long)total_tokens * hq * d > (1LL << 40))
    return fail(SWA_ERR_UNSUPPORTED, "%s: problem too large", name);
  if (total_tokens == 0) return ok();  // nothing is read or written: pointers may be NULL
  if (!q || !k || !v || !cu_seqlens || !out || (need_sinks && !sinks))
    return fail(SWA_ERR_NULL, "%s: q, k, v, %scu_seqlens and out must be non-NULL", name,
                need_sinks ? "sinks, " : "");
  if ((rc = check_aligned(name, "q, k, v and out", {q, k, v, out}))) return rc;

  swa::PrefillArgs a;
  a.q = q; a.k = k; a.v = v;
  a.sinks = sinks;
  a.cu_seqlens = cu_seqlens;
  a.out = out; a.lse = lse;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.num_q_heads = hq; a.num_kv_heads = hkv; a.head_dim = d;
  a.window = window;
  a.scale = resolve_scale(scale, d);
  a.kv_fp8 = fp8;
  a.k_scale = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  const bool bf = dtype == SWA_DTYPE_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (swa::swa_window_mfma_supported(a, bf)) e = swa::launch_swa_window_mfma(a, s);
  else if (swa::online_mfma_supported(a, bf)) e = swa::launch_online_mfma(a, s);
  else e = swa::launch_generic_prefill(a, bf, s);
  return hip_status(e, name);
}

int check_rope_base(float base, const char* name) {
  if (!(isfinite(base) && base >= 0.f))
    return fail(SWA_ERR_SHAPE, "%s: rope_base must be finite and >= 0 (got %g)", name, (double)base);
  return 0;
}

// The previous MTP step's tokens that a decode commits to the ring before it verifies.
struct CommitIn {
  const void* prev_k;
  const void* prev_v;
  const int32_t* prev_accept;
  const int32_t* prev_pos;
  int32_t prev_t;
  int32_t* ring_head_out;
};

int ring_append_common(const void* k_new, const void* v_new, const int32_t* n_accept,
                       const int32_t* positions, void* k_cache, void* v_cache, int32_t* ring_head,
                       int32_t batch, int32_t T, int32_t num_kv_heads, int32_t head_dim,
                       int32_t window, float rope_base, swa_dtype dtype, void* stream, const char* name,
                       bool fp8 = false, float k_scale = 1.f, float v_scale = 1.f);

int decode_common(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                  const void* v_cache, bool fp8, float k_scale, float v_scale,
                  const int32_t* ring_head, const float* sinks, int32_t batch, int32_t T,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t window,
                  float scale, int dtype, void* out, float* lse, void* stream, const char* name,
                  const int32_t* rope_pos = nullptr, float rope_base = 0.f,
                  const CommitIn* commit = nullptr) {
  int rc = check_dtype(dtype);
  if (rc) return rc;
  if ((rc = check_rope_base(rope_base, name))) return rc;
  if (batch < 0) return fail(SWA_ERR_SHAPE, "%s: batch must be >= 0", name);
  if ((rc = check_heads(num_q_heads, num_kv_heads, head_dim))) return rc;
  if (window < 2) return fail(SWA_ERR_SHAPE, "%s: window must be >= 2 (got %d)", name, window);
  if (T < 1 || T >= window)
    return fail(SWA_ERR_SHAPE, "%s: T must satisfy 1 <= T < window (got T=%d, window=%d)", name, T,
                window);
  if (fp8 && !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
    return fail(SWA_ERR_SHAPE, "%s: k_scale and v_scale must be finite and > 0", name);
  if ((long long)batch * num_kv_heads * window * head_dim > (1LL << 40))
    return fail(SWA_ERR_UNSUPPORTED, "%s: problem too large", name);
  if (commit && (commit->prev_t < 1 || commit->prev_t >= window))
    return fail(SWA_ERR_SHAPE, "%s: prev_T must satisfy 1 <= prev_T < window (got prev_T=%d, window=%d)",
                name, commit->prev_t, window);
  if (batch == 0) return ok();  // nothing is read or written: pointers may be NULL
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !ring_head || !sinks || !out)
    return fail(SWA_ERR_NULL,
                "%s: q, k_new, v_new, k_cache, v_cache, ring_head, sinks and out must be non-NULL",
                name);
  if (rope_base > 0.f && !rope_pos) return fail(SWA_ERR_NULL, "%s: positions must be non-NULL", name);
  if (commit) {
    if (!commit->prev_k || !commit->prev_v || !commit->prev_accept || !commit->ring_head_out)
      return fail(SWA_ERR_NULL, "%s: prev_k, prev_v, prev_accept and ring_head_out must be non-NULL", name);
    if (rope_base > 0.f && !commit->prev_pos)
      return fail(SWA_ERR_NULL, "%s: prev_positions must be non-NULL", name);
    if (commit->ring_head_out == ring_head)
      return fail(SWA_ERR_SHAPE, "%s: ring_head_out must not be ring_head", name);
    if ((rc = check_aligned(name, "prev_k and prev_v", {commit->prev_k, commit->prev_v}))) return rc;
  }
  if ((rc = check_aligned(name, "q, k_new, v_new, k_cache, v_cache and out", {q, k_new, v_new, k_cache, v_cache, out})))
    return rc;

  swa::DecodeArgs a;
  a.q = q; a.k_new = k_new; a.v_new = v_new;
  a.k_cache = k_cache; a.v_cache = v_cache;
  a.ring_head = ring_head; a.sinks = sinks;
  a.out = out; a.lse = lse;
  a.batch = batch; a.t_new = T;
  a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.head_dim = head_dim;
  a.window = window;
  a.scale = resolve_scale(scale, head_dim);
  a.cache_fp8 = fp8;
  a.k_scale = fp8 ? k_scale : 1.f;
  a.v_scale = fp8 ? v_scale : 1.f;
  if (rope_base > 0.f) {
    a.rope_pos = rope_pos;
    a.rope_log2_base = log2((double)rope_base);
  }
  const bool bf = dtype == SWA_DTYPE_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (commit) {
    a.prev_k = commit->prev_k; a.prev_v = commit->prev_v;
    a.prev_accept = commit->prev_accept; a.prev_pos = commit->prev_pos;
    a.prev_t = commit->prev_t; a.ring_head_out = commit->ring_head_out;
    if (swa::decode_mfma_supported(a, bf)) return hip_status(swa::launch_decode_mfma(a, s), name);
    // any other shape: the same step in three launches -- the head copied to ring_head_out,
    // the append advancing that copy, the decode against the updated ring
    a.prev_k = a.prev_v = nullptr;
    a.prev_accept = a.prev_pos = nullptr;
    a.prev_t = 0; a.ring_head_out = nullptr;
    hipError_t e = hipMemcpyAsync(commit->ring_head_out, ring_head, (size_t)batch * sizeof(int32_t),
                                  hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e, name);
    int rc2 = ring_append_common(commit->prev_k, commit->prev_v, commit->prev_accept, commit->prev_pos,
                                 const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                                 commit->ring_head_out, batch, commit->prev_t, num_kv_heads, head_dim,
                                 window, rope_base, (swa_dtype)dtype, stream, name, fp8, k_scale, v_scale);
    if (rc2) return rc2;
    a.ring_head = commit->ring_head_out;
  }
  hipError_t e = swa::decode_mfma_supported(a, bf) ? swa::launch_decode_mfma(a, s)
                                                   : swa::launch_generic_decode(a, bf, s);
  return hip_status(e, name);
}

int64_t backward_workspace_bytes(int32_t total_tokens, int32_t num_q_heads) {
  if (total_tokens < 0 || num_q_heads < 1) return -1;
  const int64_t rows = (int64_t)total_tokens * num_q_heads;
  return ((2 * rows * (int64_t)sizeof(float)) + 255) / 256 * 256;  // delta and sink terms
}

int ring_append_common(const void* k_new, const void* v_new, const int32_t* n_accept,
                       const int32_t* positions, void* k_cache, void* v_cache, int32_t* ring_head,
                       int32_t batch, int32_t T, int32_t num_kv_heads, int32_t head_dim,
                       int32_t window, float rope_base, swa_dtype dtype, void* stream, const char* name,
                       bool fp8, float k_scale, float v_scale) {
  int rc = check_dtype((int)dtype);
  if (rc) return rc;
  if ((rc = check_rope_base(rope_base, name))) return rc;
  if (fp8 && !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
    return fail(SWA_ERR_SHAPE, "%s: k_scale and v_scale must be finite and > 0", name);
  if (batch < 0) return fail(SWA_ERR_SHAPE, "%s: batch must be >= 0", name);
  if (num_kv_heads < 1) return fail(SWA_ERR_SHAPE, "%s: num_kv_heads must be >= 1", name);
  if (head_dim != 64 && head_dim != 128)
    return fail(SWA_ERR_SHAPE, "%s: head_dim must be 64 or 128 (got %d)", name, head_dim);
  if (window < 2) return fail(SWA_ERR_SHAPE, "%s: window must be >= 2 (got %d)", name, window);
  if (T < 1 || T >= window)
    return fail(SWA_ERR_SHAPE, "%s: T must satisfy 1 <= T < window (got T=%d, window=%d)", name, T, window);
  if ((long long)batch * num_kv_heads * window * head_dim > (1LL << 40))
    return fail(SWA_ERR_UNSUPPORTED, "%s: problem too large", name);
  if (batch == 0) return ok();
  if (!k_new || !v_new || !n_accept || !k_cache || !v_cache || !ring_head)
    return fail(SWA_ERR_NULL, "%s: k_new, v_new, n_accept, k_cache, v_cache and ring_head must be non-NULL",
                name);
  if (rope_base > 0.f && !positions) return fail(SWA_ERR_NULL, "%s: positions must be non-NULL", name);
  if ((rc = check_aligned(name, "k_new, v_new, k_cache and v_cache", {k_new, v_new, k_cache, v_cache}))) return rc;
  swa::AppendArgs a;
  a.k_new = k_new; a.v_new = v_new; a.n_accept = n_accept;
  a.rope_pos = rope_base > 0.f ? positions : nullptr;
  a.k_cache = k_cache; a.v_cache = v_cache; a.ring_head = ring_head;
  a.batch = batch; a.t_new = T; a.num_kv_heads = num_kv_heads; a.head_dim = head_dim; a.window = window;
  a.log2_base = rope_base > 0.f ? log2((double)rope_base) : 0.0;
  a.kv_fp8 = fp8; a.k_scale = k_scale; a.v_scale = v_scale;
  return hip_status(swa::launch_ring_append(a, dtype == SWA_DTYPE_BF16, static_cast<hipStream_t>(stream)),
                    name);
}

// Device address of this device's copy of `scratch` (see the top of this file).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (resolved on the first call per device).
int scratch_address(void** out, const char* name) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, name);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SWA_ERR_UNSUPPORTED, "%s: device ordinal %d beyond the %d this library tracks", name, dev,
                kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, name);
    if (p == nullptr) return fail(SWA_ERR_HIP, "%s: no device address for the scratch array", name);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SWA_OK;
}

int backward_common(const void* q, const void* k, const void* v, const float* sinks,
                    const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t window, float scale,
                    swa_dtype dtype, const void* out, const float* lse, const void* dout, void* dq, void* dk,
                    void* dv, float* dsinks, void* workspace, int64_t workspace_bytes, bool library_scratch,
                    void* stream, const char* name) {
  int rc = check_dtype((int)dtype);
  if (rc) return rc;
  if (total_tokens < 0) return fail(SWA_ERR_SHAPE, "%s: total_tokens must be >= 0", name);
  if (num_seqs < 1) return fail(SWA_ERR_SHAPE, "%s: num_seqs must be >= 1", name);
  if (total_tokens > 0 && (max_seqlen < 1 || max_seqlen > total_tokens))
    return fail(SWA_ERR_SHAPE, "%s: max_seqlen must be in [1, total_tokens]", name);
  if ((rc = check_heads(num_q_heads, num_kv_heads, head_dim))) return rc;
  if (window < 1) return fail(SWA_ERR_SHAPE, "%s: window must be >= 1 (got %d)", name, window);
  if ((long long)total_tokens * num_q_heads * head_dim > (1LL << 40))
    return fail(SWA_ERR_UNSUPPORTED, "%s: problem too large", name);
  if ((sinks == nullptr) != (dsinks == nullptr))
    return fail(SWA_ERR_NULL, "%s: sinks and dsinks must both be given or both be NULL", name);
  if (total_tokens == 0 && dsinks == nullptr) return ok();  // nothing to read or write
  if (total_tokens > 0 && (!q || !k || !v || !cu_seqlens || !out || !lse || !dout || !dq || !dk || !dv))
    return fail(SWA_ERR_NULL, "%s: q, k, v, cu_seqlens, out, lse, dout, dq, dk and dv must be non-NULL",
                name);
  if ((rc = check_aligned(name, "q, k, v, out, dout, dq, dk, dv and workspace",
                          {q, k, v, out, dout, dq, dk, dv, library_scratch ? nullptr : workspace})))
    return rc;
  const int64_t need = backward_workspace_bytes(total_tokens, num_q_heads);
  if (library_scratch) {
    if (need > kNoAllocScratchBytes)
      return fail(SWA_ERR_UNSUPPORTED,
                  "%s: needs %lld bytes of scratch, the library's array holds %lld "
                  "(total_tokens * num_q_heads <= %lld)",
                  name, (long long)need, (long long)kNoAllocScratchBytes,
                  (long long)(kNoAllocScratchBytes / (2 * (int64_t)sizeof(float))));
    if ((rc = scratch_address(&workspace, name))) return rc;
  } else if (total_tokens > 0 && (workspace == nullptr || workspace_bytes < need)) {
    return fail(SWA_ERR_SHAPE, "%s: workspace of %lld bytes needed (got %lld)", name, (long long)need,
                (long long)workspace_bytes);
  }
  swa::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.sinks = sinks; a.cu_seqlens = cu_seqlens;
  a.out = out; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dsinks = dsinks;
  a.delta = static_cast<float*>(workspace);
  a.sink_term = a.delta + (size_t)total_tokens * num_q_heads;
  a.num_seqs = num_seqs; a.total_tokens = total_tokens;
  a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.head_dim = head_dim;
  a.window = window;
  a.scale = resolve_scale(scale, head_dim);
  const hipError_t e = swa::launch_backward(a, dtype == SWA_DTYPE_BF16, static_cast<hipStream_t>(stream));
  return hip_status(e, name);
}

}  // namespace

extern "C" {

int swa_sink_prefill(const void* q, const void* k, const void* v, const float* sinks,
                     const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                     int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t window, float scale, swa_dtype dtype, void* out,
                     float* lse, void* stream) {
  return prefill_common(q, k, v, sinks, true, cu_seqlens, num_seqs, total_tokens, max_seqlen,
                        num_q_heads, num_kv_heads, head_dim, window, scale, (int)dtype, out, lse,
                        stream, "swa_sink_prefill");
}

int ga_causal_prefill(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                      int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
                      swa_dtype dtype, void* out, float* lse, void* stream) {
  return prefill_common(q, k, v, nullptr, false, cu_seqlens, num_seqs, total_tokens, max_seqlen,
                        num_q_heads, num_kv_heads, head_dim, 0x7fffffff, scale, (int)dtype, out,
                        lse, stream, "ga_causal_prefill");
}

int swa_sink_prefill_fp8kv(const void* q, const uint8_t* k, const uint8_t* v, float k_scale,
                           float v_scale, const float* sinks, const int32_t* cu_seqlens,
                           int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t window, float scale, swa_dtype dtype, void* out, float* lse,
                           void* stream) {
  return prefill_common(q, k, v, sinks, false, cu_seqlens, num_seqs, total_tokens, max_seqlen,
                        num_q_heads, num_kv_heads, head_dim, window, scale, (int)dtype, out, lse,
                        stream, "swa_sink_prefill_fp8kv", true, k_scale, v_scale);
}

int swa_sink_decode(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                    const void* v_cache, const int32_t* ring_head, const float* sinks,
                    int32_t batch, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t window, float scale, swa_dtype dtype, void* out,
                    float* lse, void* stream) {
  return decode_common(q, k_new, v_new, k_cache, v_cache, false, 1.f, 1.f, ring_head, sinks, batch,
                       T, num_q_heads, num_kv_heads, head_dim, window, scale, (int)dtype, out, lse,
                       stream, "swa_sink_decode");
}

int swa_sink_decode_fp8kv(const void* q, const void* k_new, const void* v_new,
                          const uint8_t* k_cache, const uint8_t* v_cache, float k_scale,
                          float v_scale, const int32_t* ring_head, const float* sinks,
                          int32_t batch, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t window, float scale, swa_dtype dtype,
                          void* out, float* lse, void* stream) {
  return decode_common(q, k_new, v_new, k_cache, v_cache, true, k_scale, v_scale, ring_head, sinks,
                       batch, T, num_q_heads, num_kv_heads, head_dim, window, scale, (int)dtype,
                       out, lse, stream, "swa_sink_decode_fp8kv");
}

int swa_sink_decode_rope(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                         const void* v_cache, const int32_t* ring_head, const int32_t* positions,
                         const float* sinks, int32_t batch, int32_t T, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t window, float scale,
                         float rope_base, swa_dtype dtype, void* out, float* lse, void* stream) {
  return decode_common(q, k_new, v_new, k_cache, v_cache, false, 1.f, 1.f, ring_head, sinks, batch,
                       T, num_q_heads, num_kv_heads, head_dim, window, scale, (int)dtype, out, lse,
                       stream, "swa_sink_decode_rope", positions, rope_base);
}

int swa_sink_decode_rope_commit(const void* q, const void* k_new, const void* v_new,
                                const int32_t* positions, const void* prev_k, const void* prev_v,
                                const int32_t* prev_accept, const int32_t* prev_positions,
                                int32_t prev_T, void* k_cache, void* v_cache,
                                const int32_t* ring_head, int32_t* ring_head_out, const float* sinks,
                                int32_t batch, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t window, float scale, float rope_base,
                                swa_dtype dtype, void* out, float* lse, void* stream) {
  const CommitIn c{prev_k, prev_v, prev_accept, prev_positions, prev_T, ring_head_out};
  return decode_common(q, k_new, v_new, k_cache, v_cache, false, 1.f, 1.f, ring_head, sinks, batch,
                       T, num_q_heads, num_kv_heads, head_dim, window, scale, (int)dtype, out, lse,
                       stream, "swa_sink_decode_rope_commit", positions, rope_base, &c);
}

int swa_sink_decode_rope_commit_fp8kv(const void* q, const void* k_new, const void* v_new,
                                      const int32_t* positions, const void* prev_k, const void* prev_v,
                                      const int32_t* prev_accept, const int32_t* prev_positions,
                                      int32_t prev_T, uint8_t* k_cache, uint8_t* v_cache, float k_scale,
                                      float v_scale, const int32_t* ring_head, int32_t* ring_head_out,
                                      const float* sinks, int32_t batch, int32_t T, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t window, float scale,
                                      float rope_base, swa_dtype dtype, void* out, float* lse,
                                      void* stream) {
  const CommitIn c{prev_k, prev_v, prev_accept, prev_positions, prev_T, ring_head_out};
  return decode_common(q, k_new, v_new, k_cache, v_cache, true, k_scale, v_scale, ring_head, sinks, batch,
                       T, num_q_heads, num_kv_heads, head_dim, window, scale, (int)dtype, out, lse,
                       stream, "swa_sink_decode_rope_commit_fp8kv", positions, rope_base, &c);
}

int swa_sink_decode_rope_fp8kv(const void* q, const void* k_new, const void* v_new,
                               const uint8_t* k_cache, const uint8_t* v_cache, float k_scale,
                               float v_scale, const int32_t* ring_head, const int32_t* positions,
                               const float* sinks, int32_t batch, int32_t T, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t window, float scale,
                               float rope_base, swa_dtype dtype, void* out, float* lse, void* stream) {
  return decode_common(q, k_new, v_new, k_cache, v_cache, true, k_scale, v_scale, ring_head, sinks,
                       batch, T, num_q_heads, num_kv_heads, head_dim, window, scale, (int)dtype,
                       out, lse, stream, "swa_sink_decode_rope_fp8kv", positions, rope_base);
}

int swa_rope(void* x, const int32_t* positions, int32_t rows, int32_t heads, int32_t head_dim,
             float rope_base, swa_dtype dtype, void* stream) {
  const char* name = "swa_rope";
  int rc = check_dtype((int)dtype);
  if (rc) return rc;
  if ((rc = check_rope_base(rope_base, name))) return rc;
  if (rows < 0 || heads < 1) return fail(SWA_ERR_SHAPE, "%s: rows must be >= 0 and heads >= 1", name);
  if (head_dim != 64 && head_dim != 128)
    return fail(SWA_ERR_SHAPE, "%s: head_dim must be 64 or 128 (got %d)", name, head_dim);
  if ((long long)rows * heads * head_dim > (1LL << 40)) return fail(SWA_ERR_UNSUPPORTED, "%s: problem too large", name);
  if (rows == 0 || rope_base == 0.f) return ok();
  if (!x || !positions) return fail(SWA_ERR_NULL, "%s: x and positions must be non-NULL", name);
  if ((rc = check_aligned(name, "x", {x}))) return rc;
  swa::RopeArgs a;
  a.x = x; a.pos = positions; a.rows = rows; a.heads = heads; a.head_dim = head_dim;
  a.log2_base = log2((double)rope_base);
  return hip_status(swa::launch_rope(a, dtype == SWA_DTYPE_BF16, static_cast<hipStream_t>(stream)), name);
}

int swa_ring_append_rope(const void* k_new, const void* v_new, const int32_t* n_accept,
                         const int32_t* positions, void* k_cache, void* v_cache, int32_t* ring_head,
                         int32_t batch, int32_t T, int32_t num_kv_heads, int32_t head_dim,
                         int32_t window, float rope_base, swa_dtype dtype, void* stream) {
  return ring_append_common(k_new, v_new, n_accept, positions, k_cache, v_cache, ring_head, batch, T,
                            num_kv_heads, head_dim, window, rope_base, dtype, stream,
                            "swa_ring_append_rope");
}

int swa_ring_append_fp8kv(const void* k_new, const void* v_new, const int32_t* n_accept,
                          const int32_t* positions, uint8_t* k_cache, uint8_t* v_cache, float k_scale,
                          float v_scale, int32_t* ring_head, int32_t batch, int32_t T,
                          int32_t num_kv_heads, int32_t head_dim, int32_t window, float rope_base,
                          swa_dtype dtype, void* stream) {
  return ring_append_common(k_new, v_new, n_accept, positions, k_cache, v_cache, ring_head, batch, T,
                            num_kv_heads, head_dim, window, rope_base, dtype, stream,
                            "swa_ring_append_fp8kv", true, k_scale, v_scale);
}

int swa_topk_select(const float* scores, const int32_t* lengths, int32_t batch, int32_t num_kv_heads,
                    int32_t max_len, int32_t k, int32_t recent, int32_t* indices, int32_t* counts,
                    void* stream) {
  const char* name = "swa_topk_select";
  if (batch < 0 || num_kv_heads < 1 || max_len < 1)
    return fail(SWA_ERR_SHAPE, "%s: batch >= 0, num_kv_heads >= 1 and max_len >= 1 are required", name);
  if (k < 0 || recent < 1) return fail(SWA_ERR_SHAPE, "%s: k must be >= 0 and recent >= 1", name);
  if ((long long)batch * num_kv_heads * max_len > (1LL << 40))
    return fail(SWA_ERR_UNSUPPORTED, "%s: problem too large", name);
  if (batch == 0) return ok();
  if (!scores || !lengths || !counts || (k > 0 && !indices))
    return fail(SWA_ERR_NULL, "%s: scores, lengths, indices and counts must be non-NULL", name);
  swa::TopkArgs a;
  a.scores = scores; a.lengths = lengths; a.indices = indices; a.counts = counts;
  a.batch = batch; a.num_kv_heads = num_kv_heads; a.max_len = max_len; a.k = k; a.recent = recent;
  return hip_status(swa::launch_topk_select(a, static_cast<hipStream_t>(stream)), name);
}

// (internal: the single-token and the MTP entry points below)
static int sparse_common(const void* q, const void* k_cache, const void* v_cache, const int32_t* lengths,
                  const int32_t* indices, const int32_t* counts, const float* sinks, int32_t batch, int32_t T,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_len, int32_t k,
                  int32_t recent, float scale, swa_dtype dtype, void* out, float* lse, void* stream,
                  const char* name, bool fp8 = false, float k_scale = 1.f, float v_scale = 1.f) {
  int rc = check_dtype((int)dtype);
  if (rc) return rc;
  if ((rc = check_heads(num_q_heads, num_kv_heads, head_dim))) return rc;
  if (fp8 && !(isfinite(k_scale) && k_scale > 0.f && isfinite(v_scale) && v_scale > 0.f))
    return fail(SWA_ERR_SHAPE, "%s: k_scale and v_scale must be finite and > 0", name);
  if (batch < 0 || max_len < 1) return fail(SWA_ERR_SHAPE, "%s: batch >= 0 and max_len >= 1 are required", name);
  if (T < 1 || T > max_len)
    return fail(SWA_ERR_SHAPE, "%s: T must satisfy 1 <= T <= max_len (got T=%d, max_len=%d)", name, T, max_len);
  if (k < 0 || recent < 1 || (long long)k + recent + T - 1 > 8192)
    return fail(SWA_ERR_SHAPE, "%s: k >= 0, recent >= 1 and k + recent + T - 1 <= 8192 are required", name);
  if ((long long)batch * num_kv_heads * max_len * head_dim > (1LL << 40))
    return fail(SWA_ERR_UNSUPPORTED, "%s: problem too large", name);
  if (batch == 0) return ok();
  if (!q || !k_cache || !v_cache || !lengths || !counts || !out || (k > 0 && !indices))
    return fail(SWA_ERR_NULL, "%s: q, k_cache, v_cache, lengths, indices, counts and out must be non-NULL", name);
  if ((rc = check_aligned(name, "q, k_cache, v_cache and out", {q, k_cache, v_cache, out}))) return rc;
  swa::SparseArgs a;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.lengths = lengths; a.indices = indices;
  a.counts = counts; a.sinks = sinks; a.out = out; a.lse = lse;
  a.batch = batch; a.t_new = T; a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim; a.max_len = max_len; a.k = k; a.recent = recent; a.scale = resolve_scale(scale, head_dim);
  a.kv_fp8 = fp8; a.k_scale = fp8 ? k_scale : 1.f; a.v_scale = fp8 ? v_scale : 1.f;
  return hip_status(swa::launch_sparse_decode(a, dtype == SWA_DTYPE_BF16, static_cast<hipStream_t>(stream)), name);
}

int swa_sparse_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* lengths,
                      const int32_t* indices, const int32_t* counts, const float* sinks, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_len,
                      int32_t k, int32_t recent, float scale, swa_dtype dtype, void* out, float* lse,
                      void* stream) {
  return sparse_common(q, k_cache, v_cache, lengths, indices, counts, sinks, batch, 1, num_q_heads, num_kv_heads,
                       head_dim, max_len, k, recent, scale, dtype, out, lse, stream, "swa_sparse_decode");
}

int swa_sparse_decode_fp8kv(const void* q, const uint8_t* k_cache, const uint8_t* v_cache, float k_scale,
                            float v_scale, const int32_t* lengths, const int32_t* indices, const int32_t* counts,
                            const float* sinks, int32_t batch, int32_t T, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t max_len, int32_t k, int32_t recent,
                            float scale, swa_dtype dtype, void* out, float* lse, void* stream) {
  return sparse_common(q, k_cache, v_cache, lengths, indices, counts, sinks, batch, T, num_q_heads, num_kv_heads,
                       head_dim, max_len, k, recent, scale, dtype, out, lse, stream, "swa_sparse_decode_fp8kv", true,
                       k_scale, v_scale);
}

int swa_sparse_decode_mtp(const void* q, const void* k_cache, const void* v_cache, const int32_t* lengths,
                          const int32_t* indices, const int32_t* counts, const float* sinks, int32_t batch,
                          int32_t T, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_len,
                          int32_t k, int32_t recent, float scale, swa_dtype dtype, void* out, float* lse,
                          void* stream) {
  return sparse_common(q, k_cache, v_cache, lengths, indices, counts, sinks, batch, T, num_q_heads, num_kv_heads,
                       head_dim, max_len, k, recent, scale, dtype, out, lse, stream, "swa_sparse_decode_mtp");
}

int64_t swa_sink_prefill_backward_workspace(int32_t total_tokens, int32_t num_q_heads) {
  return backward_workspace_bytes(total_tokens, num_q_heads);
}

int swa_sink_prefill_backward(const void* q, const void* k, const void* v, const float* sinks,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                              int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t window, float scale, swa_dtype dtype,
                              const void* out, const float* lse, const void* dout, void* dq,
                              void* dk, void* dv, float* dsinks, void* workspace,
                              int64_t workspace_bytes, void* stream) {
  return backward_common(q, k, v, sinks, cu_seqlens, num_seqs, total_tokens, max_seqlen, num_q_heads,
                         num_kv_heads, head_dim, window, scale, dtype, out, lse, dout, dq, dk, dv, dsinks,
                         workspace, workspace_bytes, false, stream, "swa_sink_prefill_backward");
}

int swa_sink_prefill_backward_noalloc(const void* q, const void* k, const void* v, const float* sinks,
                                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                      int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t window, float scale, swa_dtype dtype,
                                      const void* out, const float* lse, const void* dout, void* dq,
                                      void* dk, void* dv, float* dsinks, void* stream) {
  return backward_common(q, k, v, sinks, cu_seqlens, num_seqs, total_tokens, max_seqlen, num_q_heads,
                         num_kv_heads, head_dim, window, scale, dtype, out, lse, dout, dq, dk, dv, dsinks,
                         nullptr, 0, true, stream, "swa_sink_prefill_backward_noalloc");
}

const char* swa_last_error(void) { return g_last_error; }

int32_t swa_abi_version(void) { return SWASINK_ABI_VERSION; }

}  // extern "C"
