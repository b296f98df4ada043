// Rotary position embedding around decode: an in-place rotation of [rows, heads, D]
// tensors (queries and keys of a prefill), and the commit of accepted new tokens to a
// ring with their keys rotated on the way in.
//
// Bases: 10,000 in SWA layers and 640,000 (5,000,000 after the 256K extension) in GA
// layers (MiMo-V2-Flash Technical Report digest, section 3.1); positions keep
// increasing while the window slides (ICML 2026 keynote write-up, section 06), so a
// cached key keeps the rotation of its own position.  Pairing is rotate-half: element
// i pairs with i + D/2 at angle pos * base^(-2i/D):
//   y[i] = x[i] cos - x[i + D/2] sin,   y[i + D/2] = x[i + D/2] cos + x[i] sin,
// computed in fp32 and rounded to the I/O type.
#include "common.h"
#include "kernels.h"

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kPairs = 8;  // pairs per work item of the in-place rotation

template <typename T> __device__ __forceinline__ float ldf(const T* p) { return (float)*p; }
template <typename T> __device__ __forceinline__ T cvt(float x) { return (T)x; }

// Work item (row, group of kPairs pairs): the angles are shared by the row's heads.
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
  for (int h = 0; h < a.heads; ++h) {
    T* x1 = base + (size_t)h * D;
    T* x2 = x1 + D / 2;
    float u[kPairs], v[kPairs];
#pragma unroll
    for (int e = 0; e < kPairs; ++e) {
      u[e] = ldf(x1 + e);
      v[e] = ldf(x2 + e);
    }
#pragma unroll
    for (int e = 0; e < kPairs; ++e) {
      x1[e] = cvt<T>(u[e] * c[e] - v[e] * s[e]);
      x2[e] = cvt<T>(v[e] * c[e] + u[e] * s[e]);
    }
  }
}

// One workgroup per sequence: write the first n accepted tokens to physical slots
// (head + t) mod W (the n oldest), then advance the head.  The rotary cos/sin of each
// (token, pair) is formed once in LDS and shared by the KV heads; keys and values move
// in 16-byte pieces.  Every thread reads the head before the barriers; one thread
// writes the new head after the last one.
constexpr int kMaxT = 8;  // tokens per step with a shared angle table; larger T recomputes
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void ring_append_kernel(AppendArgs a) {
  __shared__ float cs[kMaxT * (D / 2)][2];
  constexpr int kVec = 16 / (int)sizeof(T);  // elements per 16-byte piece
  const int b = blockIdx.x;
  const int Tn = a.t_new, hkv = a.num_kv_heads, W = a.window;
  int n = a.n_accept[b];
  n = n < 0 ? 0 : (n > Tn ? Tn : n);
  int head = a.ring_head[b] % W;
  head += head < 0 ? W : 0;
  const bool rope = a.rope_pos != nullptr;
  const int pos0 = rope ? a.rope_pos[b] : 0;
  const bool table = n <= kMaxT;
  if (rope && table)
    for (int x = threadIdx.x; x < n * (D / 2); x += kThreads)
      rope_cos_sin(pos0 + x / (D / 2), x % (D / 2), D, a.log2_base, &cs[x][0], &cs[x][1]);
  __syncthreads();
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
      const u32x4 u4 = *reinterpret_cast<const u32x4*>(src);
      const u32x4 v4 = *reinterpret_cast<const u32x4*>(src + D / 2);
      if (!rope) {
        *reinterpret_cast<u32x4*>(dst) = u4;
        *reinterpret_cast<u32x4*>(dst + D / 2) = v4;
        continue;
      }
      T u[kVec], v[kVec], yu[kVec], yv[kVec];
      __builtin_memcpy(u, &u4, 16);
      __builtin_memcpy(v, &v4, 16);
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const int i = gi * kVec + e;
        float c, s;
        if (table) {
          c = cs[t * (D / 2) + i][0];
          s = cs[t * (D / 2) + i][1];
        } else {
          rope_cos_sin(pos0 + t, i, D, a.log2_base, &c, &s);
        }
        const float fu = ldf(&u[e]), fv = ldf(&v[e]);
        yu[e] = cvt<T>(fu * c - fv * s);
        yv[e] = cvt<T>(fv * c + fu * s);
      }
      u32x4 o1, o2;
      __builtin_memcpy(&o1, yu, 16);
      __builtin_memcpy(&o2, yv, 16);
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
