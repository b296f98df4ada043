// Shape-general attention kernels on the vector ALUs (fp32 arithmetic).
//
// One wavefront per output row (query token, query head).  Lanes own keys while
// scoring (64 keys per step) and own head-dim elements while accumulating the
// weighted values; the softmax runs online over 64-key steps, starting from the
// sink (m = sink, running sum = 1) so that exp(sink - m) sits in the denominator
// and contributes no value (MiMo-V2-Flash Technical Report digest, section 2.2.2).
// These kernels serve every shape the matrix-core kernels do not: fp32 inputs,
// head_dim 64, group sizes that are not a multiple of 8, and ring windows other
// than 128.  They trade speed for generality.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace swa {
namespace {

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ static void load16(const float* p, float* dst) {
    f32x4 x = *reinterpret_cast<const f32x4*>(p);
    dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
  }
  __device__ static float load1(const float* p) { return *p; }
  __device__ static float store_cast(float x) { return x; }
};
template <> struct Elem<bf16> {
  static constexpr int kVec = 8;
  __device__ static void load16(const bf16* p, float* dst) {
    bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = (float)x[e];
  }
  __device__ static float load1(const bf16* p) { return (float)*p; }
  __device__ static bf16 store_cast(float x) { return (bf16)x; }
};

// Key sources hand attend_row fp32 values: load_key(j, d, dst) fills dst with
// Elem<T>::kVec head-dim elements d.. of key j, load_val(j, e) is element e of value j.

// Keys of one prefill row: positions jlo..jhi of the packed stream, KV head kvh.  FP8:
// K and V hold E4M3 codes whose values are scaled by k_scale / v_scale.
template <typename T, int D, bool FP8>
struct PrefillKeys {
  using C = typename std::conditional<FP8, uint8_t, T>::type;
  const C* k;
  const C* v;
  int row_stride;  // Hkv * D
  int kvh;
  float k_scale, v_scale;
  __device__ void load_key(int j, int d, float* dst) const {
    const C* row = k + (size_t)j * row_stride + kvh * D + d;
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < Elem<T>::kVec; ++e) dst[e] = e4m3_to_f32(row[e]) * k_scale;
    } else {
      Elem<T>::load16(row, dst);
    }
  }
  __device__ float load_val(int j, int e) const {
    const C* p = v + (size_t)j * row_stride + kvh * D + e;
    if constexpr (FP8) return e4m3_to_f32(*p) * v_scale;
    else return Elem<T>::load1(p);
  }
};

// Keys of one decode row: virtual positions 0..W-1 are ring logical slots (physical
// (head + l) mod W), W..W+T-1 are the new tokens.  FP8: the ring holds E4M3 codes
// whose values are scaled by k_scale / v_scale.
template <typename T, int D, bool FP8>
struct DecodeKeys {
  using C = typename std::conditional<FP8, uint8_t, T>::type;
  const C* kc;  // this (sequence, kv head)'s ring: [W, D]
  const C* vc;
  const T* kn;  // this sequence's new tokens: [T, Hkv, D], offset to kv head
  const T* vn;
  int W;
  int head;
  int new_stride;  // Hkv * D
  float k_scale, v_scale;
  bool rope = false;  // rotate the new keys: token t at position rope_pos0 + t
  int rope_pos0 = 0;
  double rope_l2b = 0.0;
  __device__ int phys(int j) const { int p = head + j; return p - ((p >= W) ? W : 0); }
  __device__ void load_key(int j, int d, float* dst) const {
    if (j >= W) {
      const T* row = kn + (size_t)(j - W) * new_stride;
      Elem<T>::load16(row + d, dst);
      if (rope) {  // pair element i with i + D/2; rounded to the I/O type like a stored rotation
        constexpr int H = D / 2;
        const int dp = d < H ? d + H : d - H;
        float part[Elem<T>::kVec];
        Elem<T>::load16(row + dp, part);
#pragma unroll
        for (int e = 0; e < Elem<T>::kVec; ++e) {
          float c, s;
          rope_cos_sin(rope_pos0 + (j - W), (d % H) + e, D, rope_l2b, &c, &s);
          dst[e] = (float)Elem<T>::store_cast(rope_own(dst[e], part[e], c, s, d < H));
        }
      }
      return;
    }
    const C* row = kc + (size_t)phys(j) * D + d;
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < Elem<T>::kVec; ++e) dst[e] = e4m3_to_f32(row[e]) * k_scale;
    } else {
      Elem<T>::load16(row, dst);
    }
  }
  __device__ float load_val(int j, int e) const {
    if (j >= W) return Elem<T>::load1(vn + (size_t)(j - W) * new_stride + e);
    const C* p = vc + (size_t)phys(j) * D + e;
    if constexpr (FP8) return e4m3_to_f32(*p) * v_scale;
    else return Elem<T>::load1(p);
  }
};

// Keys of one sparse-decode row: list entry m < cnt is the selected position sel[m]
// (clamped into the sequence), then the row's recent window end - nrec .. end - 1.
template <typename T, int D, bool FP8>
struct SparseKeys {
  using C = typename std::conditional<FP8, uint8_t, T>::type;  // FP8: E4M3 codes
  const C* kc;  // this (sequence, kv head)'s cache rows: [Lmax, D]
  const C* vc;
  float k_scale, v_scale;
  const int32_t* sel;
  int cnt;   // selected positions seen by the row
  int L;     // the sequence's length (selected positions are clamped into it)
  int end;   // the row's position + 1: its window is end - nrec .. end - 1
  int nrec;
  __device__ int pos(int m) const {
    if (m < cnt) {
      const int j = sel[m];
      return j < 0 ? 0 : (j >= L ? L - 1 : j);
    }
    return end - nrec + (m - cnt);
  }
  __device__ void load_key(int m, int d, float* dst) const {
    const C* row = kc + (size_t)pos(m) * D + d;
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < Elem<T>::kVec; ++e) dst[e] = e4m3_to_f32(row[e]) * k_scale;
    } else {
      Elem<T>::load16(row, dst);
    }
  }
  __device__ float load_val(int m, int e) const {
    const C* p = vc + (size_t)pos(m) * D + e;
    if constexpr (FP8) return e4m3_to_f32(*p) * v_scale;
    else return Elem<T>::load1(p);
  }
};

// One wavefront computes one row against keys jlo..jhi (inclusive, jlo <= jhi).
template <typename T, int D, class Keys>
__device__ void attend_row(const T* __restrict__ qrow, const Keys& keys, int jlo, int jhi,
                           float sink2, float c, T* __restrict__ orow, float* lse_out,
                           bool rope = false, int qpos = 0, double rope_l2b = 0.0) {
  using E = Elem<T>;
  constexpr int kPer = D / kWave;  // output elements per lane
  const int lane = threadIdx.x & (kWave - 1);
  float q[D];
#pragma unroll
  for (int d = 0; d < D; d += E::kVec) E::load16(qrow + d, q + d);
  if (rope) {  // rotary embedding of the query, rounded to the I/O type like a stored rotation
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      float cs, sn;
      rope_cos_sin(qpos, i, D, rope_l2b, &cs, &sn);
      const float u = q[i], v = q[i + D / 2];
      q[i] = (float)E::store_cast(u * cs - v * sn);
      q[i + D / 2] = (float)E::store_cast(v * cs + u * sn);
    }
  }
  float o[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) o[e] = 0.f;
  float m = sink2;                        // running max (log2 units)
  float l = (sink2 == -INFINITY) ? 0.f : 1.f;  // running sum, sink term included
  for (int jb = jlo; jb <= jhi; jb += kWave) {
    const int j = jb + lane;
    const bool valid = j <= jhi;
    float s = -INFINITY;
    if (valid) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += E::kVec) {
        float kk[E::kVec];
        keys.load_key(j, d, kk);
#pragma unroll
        for (int e = 0; e < E::kVec; ++e) acc = fmaf(q[d + e], kk[e], acc);
      }
      s = acc * c;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
    const float p = valid ? fast_exp2(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int e = 0; e < kPer; ++e) o[e] *= alpha;
    const int nk = min(kWave, jhi - jb + 1);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = __shfl(p, jj);
#pragma unroll
      for (int e = 0; e < kPer; ++e) o[e] = fmaf(pj, keys.load_val(jb + jj, lane + e * kWave), o[e]);
    }
    m = m_new;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < kPer; ++e) orow[lane + e * kWave] = E::store_cast(o[e] * inv);
  if (lse_out != nullptr && lane == 0) *lse_out = (m + fast_log2(l)) * kLn2;
}

constexpr int kRowsPerBlock = 4;

template <typename T, int D, bool FP8>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void generic_prefill_kernel(PrefillArgs a) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int hq = a.num_q_heads;
  if (row >= a.total_tokens * hq) return;
  const int n = row / hq;
  const int h = row - n * hq;
  const int kvh = h / (hq / a.num_kv_heads);
  const int start = seq_start_of(a.cu_seqlens, a.num_seqs, n);
  const int lo = (a.window >= n - start + 1) ? start : n - a.window + 1;
  using C = typename PrefillKeys<T, D, FP8>::C;
  PrefillKeys<T, D, FP8> keys{static_cast<const C*>(a.k), static_cast<const C*>(a.v),
                              a.num_kv_heads * D, kvh, a.k_scale, a.v_scale};
  const float sink2 = a.sinks ? a.sinks[h] * kLog2e : -INFINITY;
  const T* qrow = static_cast<const T*>(a.q) + (size_t)row * D;
  T* orow = static_cast<T*>(a.out) + (size_t)row * D;
  attend_row<T, D>(qrow, keys, lo, n, sink2, a.scale * kLog2e, orow,
                   a.lse ? a.lse + row : nullptr);
}

template <typename T, int D, bool FP8>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void generic_decode_kernel(DecodeArgs a) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int hq = a.num_q_heads;
  const int T_ = a.t_new;
  if (row >= a.batch * T_ * hq) return;
  const int h = row % hq;
  const int bt = row / hq;
  const int t = bt % T_;
  const int b = bt / T_;
  const int hkv = a.num_kv_heads;
  const int kvh = h / (hq / hkv);
  const int W = a.window;
  int head = a.ring_head[b] % W;
  head += (head < 0) ? W : 0;
  using Keys = DecodeKeys<T, D, FP8>;
  Keys keys;
  keys.kc = static_cast<const typename Keys::C*>(a.k_cache) + ((size_t)b * hkv + kvh) * W * D;
  keys.vc = static_cast<const typename Keys::C*>(a.v_cache) + ((size_t)b * hkv + kvh) * W * D;
  keys.k_scale = a.k_scale;
  keys.v_scale = a.v_scale;
  keys.kn = static_cast<const T*>(a.k_new) + ((size_t)b * T_ * hkv + kvh) * D;
  keys.vn = static_cast<const T*>(a.v_new) + ((size_t)b * T_ * hkv + kvh) * D;
  keys.W = W;
  keys.head = head;
  keys.new_stride = hkv * D;
  const bool rope = a.rope_pos != nullptr;
  const int pos0 = rope ? a.rope_pos[b] : 0;
  keys.rope = rope;
  keys.rope_pos0 = pos0;
  keys.rope_l2b = a.rope_log2_base;
  const T* qrow = static_cast<const T*>(a.q) + (size_t)row * D;
  T* orow = static_cast<T*>(a.out) + (size_t)row * D;
  // query t sits at virtual position W + t and sees W keys: t+1 .. W+t
  attend_row<T, D>(qrow, keys, t + 1, W + t, a.sinks[h] * kLog2e, a.scale * kLog2e, orow,
                   a.lse ? a.lse + row : nullptr, rope, pos0 + t, a.rope_log2_base);
}

template <typename T, int D, bool FP8>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void generic_sparse_kernel(SparseArgs a) {
  // row = (sequence b, query token t, head h); token t sits at position L - T + t and sees
  // the selected positions below its own window and the window itself
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int hq = a.num_q_heads, Tn = a.t_new;
  if (row >= a.batch * Tn * hq) return;
  const int h = row % hq;
  const int bt = row / hq;
  const int t = bt % Tn, b = bt / Tn;
  const int hkv = a.num_kv_heads;
  const int kvh = h / (hq / hkv);
  int L = a.lengths[b];
  L = L < Tn ? Tn : (L > a.max_len ? a.max_len : L);
  int cnt = a.counts[b * hkv + kvh];
  cnt = cnt < 0 ? 0 : (cnt > a.k ? a.k : cnt);
  using Keys = SparseKeys<T, D, FP8>;
  Keys keys;
  keys.kc = static_cast<const typename Keys::C*>(a.k_cache) + ((size_t)b * hkv + kvh) * a.max_len * D;
  keys.vc = static_cast<const typename Keys::C*>(a.v_cache) + ((size_t)b * hkv + kvh) * a.max_len * D;
  keys.k_scale = a.k_scale;
  keys.v_scale = a.v_scale;
  keys.sel = a.indices + ((size_t)b * hkv + kvh) * a.k;
  keys.L = L;
  const int p = L - Tn + t;
  keys.end = p + 1;
  keys.nrec = a.recent < p + 1 ? a.recent : p + 1;
  // the selection is increasing: only its last Tn - 1 - t entries can reach into the window
  keys.cnt = cnt;
  for (int z = 0; z < Tn - 1 - t && keys.cnt > 0 && keys.pos(keys.cnt - 1) >= p + 1 - keys.nrec; ++z) --keys.cnt;
  const int M = keys.cnt + keys.nrec;
  const float sink2 = a.sinks ? a.sinks[h] * kLog2e : -INFINITY;
  attend_row<T, D>(static_cast<const T*>(a.q) + (size_t)row * D, keys, 0, M - 1, sink2, a.scale * kLog2e,
                   static_cast<T*>(a.out) + (size_t)row * D, a.lse ? a.lse + row : nullptr);
}

template <typename T, int D>
hipError_t launch_sparse_t(const SparseArgs& a, hipStream_t s) {
  const long rows = (long)a.batch * a.t_new * a.num_q_heads;
  const long blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (a.kv_fp8)
    hipLaunchKernelGGL((generic_sparse_kernel<T, D, true>), dim3((unsigned)blocks), dim3(kRowsPerBlock * kWave), 0, s, a);
  else
    hipLaunchKernelGGL((generic_sparse_kernel<T, D, false>), dim3((unsigned)blocks), dim3(kRowsPerBlock * kWave), 0,
                       s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  const long rows = (long)a.total_tokens * a.num_q_heads;
  const long blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (a.kv_fp8)
    hipLaunchKernelGGL((generic_prefill_kernel<T, D, true>), dim3((unsigned)blocks),
                       dim3(kRowsPerBlock * kWave), 0, s, a);
  else
    hipLaunchKernelGGL((generic_prefill_kernel<T, D, false>), dim3((unsigned)blocks),
                       dim3(kRowsPerBlock * kWave), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const long rows = (long)a.batch * a.t_new * a.num_q_heads;
  const long blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (a.cache_fp8)
    hipLaunchKernelGGL((generic_decode_kernel<T, D, true>), dim3((unsigned)blocks),
                       dim3(kRowsPerBlock * kWave), 0, s, a);
  else
    hipLaunchKernelGGL((generic_decode_kernel<T, D, false>), dim3((unsigned)blocks),
                       dim3(kRowsPerBlock * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_generic_prefill(const PrefillArgs& a, bool bf16_io, hipStream_t s) {
  if (bf16_io) return a.head_dim == 64 ? launch_prefill_t<bf16, 64>(a, s) : launch_prefill_t<bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_prefill_t<float, 64>(a, s) : launch_prefill_t<float, 128>(a, s);
}

hipError_t launch_generic_sparse(const SparseArgs& a, bool bf16_io, hipStream_t s) {
  if (bf16_io) return a.head_dim == 64 ? launch_sparse_t<bf16, 64>(a, s) : launch_sparse_t<bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_sparse_t<float, 64>(a, s) : launch_sparse_t<float, 128>(a, s);
}

hipError_t launch_generic_decode(const DecodeArgs& a, bool bf16_io, hipStream_t s) {
  if (bf16_io) return a.head_dim == 64 ? launch_decode_t<bf16, 64>(a, s) : launch_decode_t<bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_decode_t<float, 64>(a, s) : launch_decode_t<float, 128>(a, s);
}

}  // namespace swa
