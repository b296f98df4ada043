// Rotary position embedding around decode: an in-place rotation of [rows, heads, D]
// tensors (queries and keys of a prefill), and the commit of accepted new tokens to a
// ring with their keys rotated on the way in; the ring holds the I/O type or, for the
// FP8 (E4M3) KV cache, one-byte codes with a per-tensor scale.
//
// Bases: 10,000 in SWA layers and 640,000 (5,000,000 after the 256K extension) in GA
// layers (MiMo-V2-Flash Technical Report digest, section 3.1); positions keep
// increasing while the window slides (ICML 2026 keynote write-up, section 06), so a
// cached key keeps the rotation of its own position.  Pairing is rotate-half: element
// i pairs with i + D/2 at angle pos * base^(-2i/D):
//   y[i] = x[i] cos - x[i + D/2] sin,   y[i + D/2] = x[i + D/2] cos + x[i] sin,
// computed in fp32 and rounded to the I/O type.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kPairs = 8;      // pairs per work item of the in-place rotation
constexpr int kHeadBatch = 8;  // heads whose loads are in flight together

template <typename T> __device__ __forceinline__ float ldf(const T* p) { return (float)*p; }
template <typename T> __device__ __forceinline__ T cvt(float x) { return (T)x; }

// Work item (row, group of kPairs pairs): the angles are shared by the row's heads.
// The heads are taken kHeadBatch at a time, all loads of a batch issued before its
// first store, so each thread keeps 2 x kHeadBatch 16-byte loads in flight instead of
// one round trip per head.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void rope_kernel(RopeArgs a) {
  constexpr int kGroups = D / 2 / kPairs;
  const long item = (long)blockIdx.x * kThreads + threadIdx.x;
  if (item >= (long)a.rows * kGroups) return;
  const long row = item / kGroups;
  const int i0 = (int)(item - row * kGroups) * kPairs;
  const int pos = a.pos[row];
  float c[kPairs], s[kPairs];
#pragma unroll
  for (int e = 0; e < kPairs; ++e) rope_cos_sin(pos, i0 + e, D, a.log2_base, &c[e], &s[e]);
  T* base = static_cast<T*>(a.x) + (size_t)row * a.heads * D + i0;
  using Vec = typename std::conditional<sizeof(T) == 2, u32x4, f32x4>::type;  // kPairs * 2 bytes for bf16
  constexpr int kVecs = kPairs * (int)sizeof(T) / 16;                         // 16-byte pieces per half
  auto rotate = [&](const Vec (&xv)[kVecs], const Vec (&yv)[kVecs], Vec (&xo)[kVecs], Vec (&yo)[kVecs]) {
    T u[kPairs], v[kPairs], uo[kPairs], vo[kPairs];
    __builtin_memcpy(u, xv, sizeof(u));
    __builtin_memcpy(v, yv, sizeof(v));
#pragma unroll
    for (int e = 0; e < kPairs; ++e) {
      float lo, hi;
      rope_pair((float)u[e], (float)v[e], c[e], s[e], lo, hi);
      uo[e] = cvt<T>(lo);
      vo[e] = cvt<T>(hi);
    }
    __builtin_memcpy(xo, uo, sizeof(uo));
    __builtin_memcpy(yo, vo, sizeof(vo));
  };
  int h = 0;
  for (; h + kHeadBatch <= a.heads; h += kHeadBatch) {
    Vec xv[kHeadBatch][kVecs], yv[kHeadBatch][kVecs];
#pragma unroll
    for (int j = 0; j < kHeadBatch; ++j) {
      const T* x1 = base + (size_t)(h + j) * D;
#pragma unroll
      for (int q = 0; q < kVecs; ++q) {
        xv[j][q] = *reinterpret_cast<const Vec*>(x1 + q * (16 / sizeof(T)));
        yv[j][q] = *reinterpret_cast<const Vec*>(x1 + D / 2 + q * (16 / sizeof(T)));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the batch's loads stay ahead of its stores
#pragma unroll
    for (int j = 0; j < kHeadBatch; ++j) {
      Vec xo[kVecs], yo[kVecs];
      rotate(xv[j], yv[j], xo, yo);
      T* x1 = base + (size_t)(h + j) * D;
#pragma unroll
      for (int q = 0; q < kVecs; ++q) {
        *reinterpret_cast<Vec*>(x1 + q * (16 / sizeof(T))) = xo[q];
        *reinterpret_cast<Vec*>(x1 + D / 2 + q * (16 / sizeof(T))) = yo[q];
      }
    }
  }
  for (; h < a.heads; ++h) {  // the heads past the last whole batch
    T* x1 = base + (size_t)h * D;
    Vec xv[kVecs], yv[kVecs], xo[kVecs], yo[kVecs];
#pragma unroll
    for (int q = 0; q < kVecs; ++q) {
      xv[q] = *reinterpret_cast<const Vec*>(x1 + q * (16 / sizeof(T)));
      yv[q] = *reinterpret_cast<const Vec*>(x1 + D / 2 + q * (16 / sizeof(T)));
    }
    rotate(xv, yv, xo, yo);
#pragma unroll
    for (int q = 0; q < kVecs; ++q) {
      *reinterpret_cast<Vec*>(x1 + q * (16 / sizeof(T))) = xo[q];
      *reinterpret_cast<Vec*>(x1 + D / 2 + q * (16 / sizeof(T))) = yo[q];
    }
  }
}

// N values of the I/O type from 8, 16 or 32 aligned bytes.
template <typename T, int N>
__device__ __forceinline__ void load_n(const T* p, T (&y)[N]) {
  constexpr int kBytes = N * (int)sizeof(T);
  static_assert(kBytes == 8 || kBytes == 16 || kBytes == 32, "8, 16 or 32 bytes");
  if constexpr (kBytes == 8) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    __builtin_memcpy(y, &w, 8);
  } else {
    u32x4 w[kBytes / 16];
#pragma unroll
    for (int k = 0; k < kBytes / 16; ++k) w[k] = reinterpret_cast<const u32x4*>(p)[k];
    __builtin_memcpy(y, w, kBytes);
  }
}

// N E4M3 codes of y / scale stored at dst (4 or 8 aligned bytes).
template <typename T, int N>
__device__ __forceinline__ void store_codes(uint8_t* dst, const T (&y)[N], double scale) {
  static_assert(N == 4 || N == 8, "4 or 8 codes");
  uint64_t w = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) w |= (uint64_t)e4m3_encode(y[e], scale) << (8 * e);
  if constexpr (N == 8) *reinterpret_cast<uint64_t*>(dst) = w;
  else *reinterpret_cast<uint32_t*>(dst) = (uint32_t)w;
}

// The accepted count and the ring head of sequence b, and the rotary cos/sin table of
// its (token, pair)s in LDS when the tokens fit it (every thread reads the head before
// the barrier that ends this).
constexpr int kMaxT = 8;  // tokens per step with a shared angle table; larger T recomputes
template <int D>
__device__ __forceinline__ void append_setup(const AppendArgs& a, int b, float (*cs)[2], int& n, int& head) {
  const int Tn = a.t_new, W = a.window;
  n = a.n_accept[b];
  n = n < 0 ? 0 : (n > Tn ? Tn : n);
  head = a.ring_head[b] % W;
  head += head < 0 ? W : 0;
  if (a.rope_pos != nullptr && n <= kMaxT) {
    const int pos0 = a.rope_pos[b];
    for (int x = threadIdx.x; x < n * (D / 2); x += blockDim.x)
      rope_cos_sin(pos0 + x / (D / 2), x % (D / 2), D, a.log2_base, &cs[x][0], &cs[x][1]);
  }
  __syncthreads();
}

// Rotate N pairs (u[e], v[e]) = (x[i], x[i + D/2]), i = i0 + e, of new token t in place,
// rounding to the I/O type.
template <typename T, int D, int N>
__device__ __forceinline__ void rotate_pairs(const AppendArgs& a, int b, int n, int t, int i0,
                                             const float (*cs)[2], T (&u)[N], T (&v)[N]) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const int i = i0 + e;
    float c, s;
    if (n <= kMaxT) {
      c = cs[t * (D / 2) + i][0];
      s = cs[t * (D / 2) + i][1];
    } else {
      rope_cos_sin(a.rope_pos[b] + t, i, D, a.log2_base, &c, &s);
    }
    float lo, hi;
    rope_pair(ldf(&u[e]), ldf(&v[e]), c, s, lo, hi);
    u[e] = cvt<T>(lo);
    v[e] = cvt<T>(hi);
  }
}

// One workgroup per sequence: write the first n accepted tokens to physical slots
// (head + t) mod W (the n oldest), then advance the head.  The rotary cos/sin of each
// (token, pair) is formed once in LDS and shared by the KV heads; keys and values move
// in 16-byte pieces.  One thread writes the new head after the last barrier.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void ring_append_kernel(AppendArgs a) {
  __shared__ float cs[kMaxT * (D / 2)][2];
  constexpr int kVec = 16 / (int)sizeof(T);  // elements per 16-byte piece
  const int b = blockIdx.x;
  int n, head;
  append_setup<D>(a, b, cs, n, head);
  const int Tn = a.t_new, hkv = a.num_kv_heads, W = a.window;
  const bool rope = a.rope_pos != nullptr;
  const T* kn = static_cast<const T*>(a.k_new) + (size_t)b * Tn * hkv * D;
  const T* vn = static_cast<const T*>(a.v_new) + (size_t)b * Tn * hkv * D;
  T* kc = static_cast<T*>(a.k_cache) + (size_t)b * hkv * W * D;
  T* vc = static_cast<T*>(a.v_cache) + (size_t)b * hkv * W * D;
  // keys: one item per (token, kv head, group of kVec pairs); values: per 16-byte piece
  constexpr int kKGroups = D / 2 / kVec, kVPieces = D / kVec;
  const int nk = n * hkv * kKGroups;
  for (int x = threadIdx.x; x < nk + n * hkv * kVPieces; x += kThreads) {
    if (x < nk) {
      const int gi = x % kKGroups, r = x / kKGroups;  // r = token * hkv + kv head
      const int t = r / hkv, g = r - t * hkv;
      const T* src = kn + ((size_t)t * hkv + g) * D + gi * kVec;
      T* dst = kc + ((size_t)g * W + (head + t) % W) * D + gi * kVec;
      T u[kVec], v[kVec];
      load_n(src, u);
      load_n(src + D / 2, v);
      if (rope) rotate_pairs<T, D>(a, b, n, t, gi * kVec, cs, u, v);
      u32x4 o1, o2;
      __builtin_memcpy(&o1, u, 16);
      __builtin_memcpy(&o2, v, 16);
      *reinterpret_cast<u32x4*>(dst) = o1;
      *reinterpret_cast<u32x4*>(dst + D / 2) = o2;
    } else {
      const int y = x - nk;
      const int pc = y % kVPieces, r = y / kVPieces;
      const int t = r / hkv, g = r - t * hkv;
      *reinterpret_cast<u32x4*>(vc + ((size_t)g * W + (head + t) % W) * D + pc * kVec) =
          *reinterpret_cast<const u32x4*>(vn + ((size_t)t * hkv + g) * D + pc * kVec);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.ring_head[b] = (head + n) % W;
}

// The same commit into an FP8 ring: every element is encoded (e4m3_encode), so the work
// is arithmetic rather than data movement and is spread thinner -- 512 threads per
// sequence, each item 8 codes: 4 pairs of a key (two 4-byte stores) or 8 elements of a
// value (one 8-byte store).
constexpr int kThreadsFp8 = 512;
template <typename T, int D>
__global__ __launch_bounds__(kThreadsFp8) void ring_append_fp8_kernel(AppendArgs a) {
  __shared__ float cs[kMaxT * (D / 2)][2];
  const int b = blockIdx.x;
  int n, head;
  append_setup<D>(a, b, cs, n, head);
  const int Tn = a.t_new, hkv = a.num_kv_heads, W = a.window;
  const bool rope = a.rope_pos != nullptr;
  const double ks = a.k_scale, vs = a.v_scale;
  const T* kn = static_cast<const T*>(a.k_new) + (size_t)b * Tn * hkv * D;
  const T* vn = static_cast<const T*>(a.v_new) + (size_t)b * Tn * hkv * D;
  uint8_t* kc = static_cast<uint8_t*>(a.k_cache) + (size_t)b * hkv * W * D;
  uint8_t* vc = static_cast<uint8_t*>(a.v_cache) + (size_t)b * hkv * W * D;
  constexpr int kKUnits = D / 2 / 4, kVUnits = D / 8;
  const int nk = n * hkv * kKUnits;
  for (int x = threadIdx.x; x < nk + n * hkv * kVUnits; x += kThreadsFp8) {
    if (x < nk) {
      const int gi = x % kKUnits, r = x / kKUnits;  // r = token * hkv + kv head
      const int t = r / hkv, g = r - t * hkv;
      const T* src = kn + ((size_t)t * hkv + g) * D + gi * 4;
      uint8_t* dst = kc + ((size_t)g * W + (head + t) % W) * D + gi * 4;
      T u[4], v[4];
      load_n(src, u);
      load_n(src + D / 2, v);
      if (rope) rotate_pairs<T, D>(a, b, n, t, gi * 4, cs, u, v);
      store_codes(dst, u, ks);
      store_codes(dst + D / 2, v, ks);
    } else {
      const int y = x - nk;
      const int pc = y % kVUnits, r = y / kVUnits;
      const int t = r / hkv, g = r - t * hkv;
      T v[8];
      load_n(vn + ((size_t)t * hkv + g) * D + pc * 8, v);
      store_codes(vc + ((size_t)g * W + (head + t) % W) * D + pc * 8, v, vs);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.ring_head[b] = (head + n) % W;
}

template <typename T, int D>
hipError_t rope_t(const RopeArgs& a, hipStream_t s) {
  const long items = (long)a.rows * (D / 2 / kPairs);
  const long blocks = (items + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((rope_kernel<T, D>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t append_t(const AppendArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (a.kv_fp8)
    hipLaunchKernelGGL((ring_append_fp8_kernel<T, D>), dim3((unsigned)a.batch), dim3(kThreadsFp8), 0, s, a);
  else
    hipLaunchKernelGGL((ring_append_kernel<T, D>), dim3((unsigned)a.batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, bool bf16_io, hipStream_t s) {
  if (bf16_io) return a.head_dim == 64 ? rope_t<bf16, 64>(a, s) : rope_t<bf16, 128>(a, s);
  return a.head_dim == 64 ? rope_t<float, 64>(a, s) : rope_t<float, 128>(a, s);
}

hipError_t launch_ring_append(const AppendArgs& a, bool bf16_io, hipStream_t s) {
  if (bf16_io) return a.head_dim == 64 ? append_t<bf16, 64>(a, s) : append_t<bf16, 128>(a, s);
  return a.head_dim == 64 ? append_t<float, 64>(a, s) : append_t<float, 128>(a, s);
}

}  // namespace swa
