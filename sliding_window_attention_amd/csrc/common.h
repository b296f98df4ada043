// Device-side vocabulary shared by the libswasink kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Read-only kernel inputs (sequence offsets, sinks) read through the constant
// address space: wave-uniform reads then become scalar loads, which complete on
// their own counter instead of waiting behind outstanding vector stores.
template <typename T>
using const_ptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ const_ptr<T> as_const(const T* p) {
  return (const_ptr<T>)p;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// Parameters of one prefill call (packed variable-length sequences).
struct PrefillArgs {
  const void* q;            // [N, Hq, D]
  const void* k;            // [N, Hkv, D]
  const void* v;            // [N, Hkv, D]
  const float* sinks;       // [Hq] or nullptr (no sink)
  const int32_t* cu_seqlens;  // [S+1]
  void* out;                // [N, Hq, D]
  float* lse;               // [N, Hq] or nullptr
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t window;           // keys i-window+1 .. i; INT32_MAX for unbounded
  float scale;              // logit scale (already resolved, > 0)
  bool kv_fp8 = false;      // k / v hold one-byte E4M3 codes
  float k_scale = 1.f;      // with kv_fp8: element value = code value * scale
  float v_scale = 1.f;
};

// Parameters of one decode / MTP-verify call against a ring buffer.
struct DecodeArgs {
  const void* q;            // [B, T, Hq, D]
  const void* k_new;        // [B, T, Hkv, D]
  const void* v_new;        // [B, T, Hkv, D]
  const void* k_cache;      // [B, Hkv, W, D]
  const void* v_cache;      // [B, Hkv, W, D]
  const int32_t* ring_head;  // [B]
  const float* sinks;       // [Hq]
  void* out;                // [B, T, Hq, D]
  float* lse;               // [B, T, Hq] or nullptr
  int32_t batch;
  int32_t t_new;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t window;
  float scale;
  bool cache_fp8 = false;  // k_cache / v_cache hold one-byte E4M3 codes
  float k_scale = 1.f;     // with cache_fp8: element value = code value * scale
  float v_scale = 1.f;
  const int32_t* rope_pos = nullptr;  // [B] position of new token 0: rotate q and k_new
  double rope_log2_base = 0.0;        // log2 of the rotary base (with rope_pos)
  // one-launch MTP step (with rope_pos): the previous step's accepted tokens, committed to
  // the ring before the verify; the ring is then written and ring_head is only read
  const void* prev_k = nullptr;         // [B, prev_t, Hkv, D], keys unrotated
  const void* prev_v = nullptr;         // [B, prev_t, Hkv, D]
  const int32_t* prev_accept = nullptr;  // [B] tokens of the previous step to commit
  const int32_t* prev_pos = nullptr;     // [B] position of the previous step's token 0
  int32_t prev_t = 0;
  int32_t* ring_head_out = nullptr;     // [B] head after the commit
};

// Rotary embedding of x [rows, heads, D] in place, row r at position pos[r].
struct RopeArgs {
  void* x;
  const int32_t* pos;
  int32_t rows;
  int32_t heads;
  int32_t head_dim;
  double log2_base;
};

// Commit accepted new tokens to a ring (keys rotated on the way in when rope is set).
struct AppendArgs {
  const void* k_new;        // [B, T, Hkv, D]
  const void* v_new;        // [B, T, Hkv, D]
  const int32_t* n_accept;  // [B], clamped to [0, T]
  const int32_t* rope_pos;  // [B] position of new token 0, or nullptr (no rotation)
  void* k_cache;            // [B, Hkv, W, D]
  void* v_cache;            // [B, Hkv, W, D]
  int32_t* ring_head;       // [B], advanced by the accepted count
  int32_t batch;
  int32_t t_new;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t window;
  double log2_base;
  bool kv_fp8 = false;      // caches hold E4M3 codes of value / scale
  float k_scale = 1.f, v_scale = 1.f;
};

// Token selection for the sparse layers: per (sequence, KV head) row of scores, the top
// k positions older than the recent window.
struct TopkArgs {
  const float* scores;    // [B, Hkv, Lmax]
  const int32_t* lengths;  // [B]
  int32_t* indices;       // [B, Hkv, k] increasing, padded with -1
  int32_t* counts;        // [B, Hkv]
  int32_t batch;
  int32_t num_kv_heads;
  int32_t max_len;
  int32_t k;
  int32_t recent;
};

// One query token per sequence over selected + recent keys of a [B, Hkv, Lmax, D] cache.
struct SparseArgs {
  const void* q;             // [B, T, Hq, D] (T = t_new)
  const void* k_cache;       // [B, Hkv, Lmax, D]
  const void* v_cache;
  const int32_t* lengths;    // [B]
  const int32_t* indices;    // [B, Hkv, k]
  const int32_t* counts;     // [B, Hkv]
  const float* sinks;        // [Hq] or nullptr
  void* out;                 // [B, T, Hq, D]
  float* lse;                // [B, T, Hq] or nullptr
  int32_t batch;
  int32_t t_new = 1;         // queries per sequence: its newest T tokens (MTP verify)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_len;
  int32_t k;
  int32_t recent;
  float scale;
  bool kv_fp8 = false;       // caches hold E4M3 codes; values = code value x k_scale / v_scale
  float k_scale = 1.f, v_scale = 1.f;
};

// Arguments of the backward (gradients of O).  Pointers are device pointers.
struct BackwardArgs {
  const void* q;             // [N, Hq, D]
  const void* k;             // [N, Hkv, D]
  const void* v;             // [N, Hkv, D]
  const float* sinks;        // [Hq] or nullptr (no sink)
  const int32_t* cu_seqlens;  // [S + 1]
  const void* out;           // [N, Hq, D] forward output
  const float* lse;          // [N, Hq] forward log-sum-exp (natural log, sink included)
  const void* dout;          // [N, Hq, D]
  void* dq;                  // [N, Hq, D]
  void* dk;                  // [N, Hkv, D]
  void* dv;                  // [N, Hkv, D]
  float* dsinks;             // [Hq] or nullptr (no sink)
  float* delta;              // workspace [N, Hq]: dO . O
  float* sink_term;          // workspace [N, Hq]: exp(sink - lse) * delta
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t window;
  float scale;
};

// First token of the sequence that holds packed token `t`: the largest s with
// cu[s] <= t (binary search; cu has num_seqs + 1 entries).  Clamped so that a
// malformed cu_seqlens cannot produce an index outside [0, t].
__device__ __forceinline__ int seq_start_of(const int32_t* __restrict__ cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs;  // invariant: answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  int s = cu[lo];
  s = s < 0 ? 0 : s;
  return s > t ? t : s;
}

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }

// E4M3 (OCP 8-bit float: bias 7, subnormals, no infinities) to wider types with the
// gfx950 conversion instructions.  Every E4M3 value is exactly a bf16 and an fp32
// value, so these conversions are exact.
// Eight codes (bytes 0..7 of w, element k = byte k) as bf16x8.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(u32x2 w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, true);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// One code as fp32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// E4M3 code (sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0, subnormals
// m/8 * 2^-6, S.1111.111 = NaN, largest finite 448) of y / scale: the quotient rounded
// once to the nearest E4M3 value, ties to the even mantissa; finite magnitudes past 448
// saturate to 448, and a y that is not finite gives the NaN code with y's sign.  The
// quotient is formed in fp64: y and scale carry at most 24 significant bits, so a
// quotient that is not itself halfway between two E4M3 values stays about 2^-30
// (relative) away from such a point and its fp64 rounding cannot land on one.  Every
// case is computed and the code selected, with no branches.
template <typename T>
__device__ __forceinline__ uint32_t e4m3_encode(T y, double scale) {
  uint32_t sign, nonfinite;
  if constexpr (sizeof(T) == 2) {
    const uint16_t b = __builtin_bit_cast(uint16_t, y);
    sign = (b >> 8) & 0x80u;
    nonfinite = (b & 0x7F80u) == 0x7F80u;
  } else {
    const uint32_t b = __builtin_bit_cast(uint32_t, y);
    sign = (b >> 24) & 0x80u;
    nonfinite = (b & 0x7F800000u) == 0x7F800000u;
  }
  const double q = __builtin_fabs((double)(float)y / scale);
  const uint64_t a = __builtin_bit_cast(uint64_t, q);
  const int e = (int)(a >> 52) - 1023;
  const uint64_t mant = a & ((1ull << 52) - 1);
  // mantissa rounded to 3 bits (0..8); 8 carries into the exponent field
  const int r = (int)((mant + ((1ull << 48) - 1) + ((mant >> 49) & 1)) >> 49);
  const uint32_t normal = (uint32_t)(((e + 7) << 3) + r);
  const uint32_t sub = (uint32_t)__builtin_rint(q * 512.0);  // k * 2^-9, k = 0..8
  uint32_t code = e < -6 ? sub : normal;
  code = q >= 448.0 ? 0x7Eu : code;
  code = nonfinite ? 0x7Fu : code;
  return sign | code;
}

// cos and sin of the rotary angle of pair i (of head_dim D) at an integer position:
// angle = pos * base^(-2i/D), formed and reduced to [-pi, pi] in fp64 (positions go to
// 2^31, where an angle formed in fp32 is off by whole radians), then evaluated in fp32.
__device__ __forceinline__ void rope_cos_sin(int pos, int i, int D, double log2_base, float* c, float* s) {
  const double f = exp2(-2.0 * (double)i / (double)D * log2_base);
  const double ang = (double)pos * f;
  const double r = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
  sincosf((float)r, s, c);
}

// One rotary pair (x, y) = (element i, element i + D/2) in fp32: (x cos - y sin,
// y cos + x sin), each product rounded before the sum, with no fused multiply-add
// whatever the call site, so every kernel that rotates a value produces the same bits.
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float& lo, float& hi) {
#pragma clang fp contract(off)
  lo = x * c - y * s;
  hi = y * c + x * s;
}

// Global-to-LDS loads: lane L's 16 (or 4) bytes from src land at lds + 16 L (4 L), the
// LDS base being uniform across the wavefront.  Completion is counted by vmcnt; a wait
// for vmcnt(0) and a barrier publish the block to the workgroup.
__device__ __forceinline__ void load_lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// The element of a rotary pair that a lane holds, from its own value x and its partner's p:
// x c - p s if it holds the pair's first element, else x c + p s -- rope_pair's roundings
// (each product rounded, then the sum), selected without a branch.
__device__ __forceinline__ float rope_own(float x, float p, float c, float s, bool first) {
#pragma clang fp contract(off)
  const float a = x * c, b = p * s;
  return a + (first ? -b : b);
}

// s_waitcnt immediate for vmcnt(0) with the other counters left alone (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kVmcnt0 = 0x0F70;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// The value of lane l and of lane l ^ kStride (kStride 16 or 32), in an order that
// depends on the lane.  v_permlane16_swap / v_permlane32_swap exchange 16-lane rows
// (32-lane halves) between their two register operands in one VALU instruction;
// with x in both operands the two results are x[l] and x[l ^ kStride].  Every lane
// of the wavefront must be active.
template <int kStride>
__device__ __forceinline__ f32x2 with_partner(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  if constexpr (kStride == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return (f32x2){__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return (f32x2){__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
  }
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (the lanes that hold the
// same column of a 16x16 MFMA result).  Both operations are commutative, so all
// four lanes end with bitwise the same value.  Every lane must be active.
__device__ __forceinline__ float quad_max(float x) {
  f32x2 p = with_partner<16>(x);
  p = with_partner<32>(fmaxf(p[0], p[1]));
  return fmaxf(p[0], p[1]);
}
__device__ __forceinline__ float quad_sum(float x) {
  f32x2 p = with_partner<16>(x);
  p = with_partner<32>(p[0] + p[1]);
  return p[0] + p[1];
}

}  // namespace swa
