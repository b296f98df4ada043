// Matrix-core prefill kernels: sliding-window attention with a per-head sink and
// global causal attention (MiMo-V2-Flash Technical Report digest, sections 2.2.1
// and 2.2.2; global layers are the same operator with no window and no sink).
//
// Work decomposition (both kernels): one workgroup of 4 wavefronts owns 16
// consecutive query tokens of the packed stream and the 8 query heads that share
// one KV head (GQA), so every K/V byte staged in LDS serves 8 heads.  Wavefront w
// owns heads 2w and 2w+1 (two 16-query MFMA tiles).  Tiles may straddle sequence
// boundaries: every query row masks keys before its own sequence start, so the
// grid depends only on the total token count and needs no host-side tile map.
//
// swa_window_kernel (window <= 128): the union of the 16 rows' windows is at most
// 143 keys, so the whole band (9 blocks of 16 keys) is staged once and scored in
// registers; the softmax is exact in one pass (no online rescaling), the sink
// entering as the initial maximum candidate and as exp(sink - m) in the
// denominator.
//
// online_kernel (any window, or none): the band is streamed in 64-key chunks
// with the next chunk prefetched into registers during the current one's
// matrix work, and the classic running max / running sum update.
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace swa {
namespace {

using namespace tile;

constexpr int kQT = 16;        // query tokens per workgroup
constexpr int kHG = 8;         // query heads per workgroup
constexpr int kThreads = 256;  // 4 wavefronts x 2 heads
constexpr int kBand = 144;     // keys staged by the window kernel (9 blocks of 16)
constexpr int kChunk = 64;     // keys per step of the online kernel

// Map a flat workgroup id to (head octet, query tile).  Workgroups are dispatched
// round-robin over the 8 XCDs (id mod 8); give each XCD a contiguous range of
// work items so that neighbouring tiles -- which share 128 of their 144 K/V
// rows -- run on the same XCD and hit in its L2.
__device__ __forceinline__ int xcd_item(int n, int total) {
  const int xcd = n & 7;
  const int j = n >> 3;
  const int per = total >> 3;
  const int rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + j;
}

// Stage `kRows` key rows starting at packed position kbase (K and V of KV head
// kvh) into LDS, zero-filling rows outside [0, N).  Loads are issued first, then
// written, so each thread has all its requests in flight together.
template <int kRows>
__device__ __forceinline__ void stage_kv(char* ks, char* vs, const bf16* __restrict__ k,
                                         const bf16* __restrict__ v, int kbase, int N, int hkv,
                                         int kvh) {
  constexpr int kUnits = kRows * kUnitsPerRow;
  constexpr int kIters = (kUnits + kThreads - 1) / kThreads;
  const int t = threadIdx.x;
  u32x4 kr[kIters], vr[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int x = it * kThreads + t;
    const int r = x >> 4, u = x & 15;
    const int key = kbase + r;
    kr[it] = (u32x4){0, 0, 0, 0};
    vr[it] = (u32x4){0, 0, 0, 0};
    if (x < kUnits && key >= 0 && key < N) {
      const size_t off = ((size_t)key * hkv + kvh) * D + u * 8;
      kr[it] = *reinterpret_cast<const u32x4*>(k + off);
      vr[it] = *reinterpret_cast<const u32x4*>(v + off);
    }
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int x = it * kThreads + t;
    if (x < kUnits) {
      const int r = x >> 4, u = x & 15;
      *reinterpret_cast<u32x4*>(ks + lds_off(r, u)) = kr[it];
      *reinterpret_cast<u32x4*>(vs + lds_off(r, u)) = vr[it];
    }
  }
}

struct RowInfo {
  int qi;      // packed query position of this lane's column
  int lo;      // first visible key (window and sequence start)
  int h0, h1;  // the wavefront's two heads
};

__device__ __forceinline__ RowInfo row_info(const PrefillArgs& a, int q0, int h_base, int w, int i) {
  RowInfo ri;
  ri.qi = q0 + i;
  const int qc = ri.qi < a.total_tokens ? ri.qi : a.total_tokens - 1;
  const int start = seq_start_of(a.cu_seqlens, a.num_seqs, qc);
  const long lw = (long)ri.qi - a.window + 1;
  ri.lo = lw > start ? (int)lw : start;
  ri.h0 = h_base + 2 * w;
  ri.h1 = ri.h0 + 1;
  return ri;
}

__device__ __forceinline__ void load_q(const PrefillArgs& a, const RowInfo& ri, int g,
                                       bf16x8 (&q0)[4], bf16x8 (&q1)[4]) {
  const bf16* q = static_cast<const bf16*>(a.q);
  const bool ok = ri.qi < a.total_tokens;
  const size_t r0 = ((size_t)ri.qi * a.num_q_heads + ri.h0) * D + 8 * g;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    q0[c] = ok ? *reinterpret_cast<const bf16x8*>(q + r0 + 32 * c) : zero8();
    q1[c] = ok ? *reinterpret_cast<const bf16x8*>(q + r0 + D + 32 * c) : zero8();
  }
}

__device__ __forceinline__ void write_out(const PrefillArgs& a, const RowInfo& ri, int g,
                                          const f32x4 (&o0)[8], const f32x4 (&o1)[8], float z0,
                                          float z1, float m0, float m1) {
  if (ri.qi >= a.total_tokens) return;
  bf16* out = static_cast<bf16*>(a.out);
  const size_t r0 = ((size_t)ri.qi * a.num_q_heads + ri.h0) * D + 32 * g;
  store_row32(out + r0, o0, 1.f / z0);
  store_row32(out + r0 + D, o1, 1.f / z1);
  if (a.lse != nullptr && g == 0) {
    float* l = a.lse + (size_t)ri.qi * a.num_q_heads + ri.h0;
    l[0] = (m0 + fast_log2(z0)) * kLn2;
    l[1] = (m1 + fast_log2(z1)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Window <= 128: whole band in registers, exact one-pass softmax.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 2) void swa_window_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kBand * kRowBytes];
  char* ks = smem;
  char* vs = smem + kBand * kRowBytes;

  const int ntiles = (a.total_tokens + kQT - 1) / kQT;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int oct = item / ntiles;
  const int q0 = (item - oct * ntiles) * kQT;
  const int h_base = oct * kHG;
  const int kvh = h_base / (a.num_q_heads / a.num_kv_heads);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int kbase = q0 - 128;  // LDS row r holds key kbase + r

  const RowInfo ri = row_info(a, q0, h_base, w, i);
  bf16x8 qa[4], qb[4];
  load_q(a, ri, g, qa, qb);
  stage_kv<kBand>(ks, vs, static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v), kbase,
                  a.total_tokens, a.num_kv_heads, kvh);

  // Row bounds relative to kbase; the lane's column is query qi.
  const int rel_lo = ri.lo - kbase;  // >= 1 because window <= 128
  const int rel_hi = ri.qi - kbase;  // = 128 + i
  const int lo_min = __shfl(rel_lo, 0);   // rows are ordered, so lane 0 / 15 bound the tile
  const int lo_max = __shfl(rel_lo, 15);
  const float c = a.scale * kLog2e;
  const float sink0 = a.sinks ? a.sinks[ri.h0] * kLog2e : -INFINITY;
  const float sink1 = a.sinks ? a.sinks[ri.h1] * kLog2e : -INFINITY;
  __syncthreads();

  // ---- S^T = K Q^T over 9 blocks of 16 keys ----
  f32x4 s0[9], s1[9];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int bl = 0; bl < 9; ++bl) {
    s0[bl] = zero4;
    s1[bl] = zero4;
    const int kr_max = bl < 8 ? 32 * (bl >> 1) + 4 * (bl & 1) + 27 : 143;
    if (kr_max < lo_min) continue;  // whole block before every row's window
    const int row = bl < 8 ? 32 * (bl >> 1) + pair_row(i, bl & 1) : 128 + i;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const bf16x8 kf = lds_read8(ks, row, 4 * cc + g);
      s0[bl] = mfma32(kf, qa[cc], s0[bl]);
      s1[bl] = mfma32(kf, qb[cc], s1[bl]);
    }
  }

  // ---- mask, row max ----
  float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
  for (int bl = 0; bl < 9; ++bl) {
    const int kr_min = bl < 8 ? 32 * (bl >> 1) + 4 * (bl & 1) : 128;
    const int kr_max = bl < 8 ? kr_min + 27 : 143;
    const bool full = kr_min >= lo_max && kr_max <= 128;  // valid for all 16 rows
    if (!full) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = bl < 8 ? 32 * (bl >> 1) + 8 * g + 4 * (bl & 1) + r : 128 + 4 * g + r;
        const bool ok = kr >= rel_lo && kr <= rel_hi;
        s0[bl][r] = ok ? s0[bl][r] : -INFINITY;
        s1[bl][r] = ok ? s1[bl][r] : -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mx0 = fmaxf(mx0, s0[bl][r]);
      mx1 = fmaxf(mx1, s1[bl][r]);
    }
  }
  const float m0 = fmaxf(quad_max(mx0) * c, sink0);
  const float m1 = fmaxf(quad_max(mx1) * c, sink1);

  // ---- exponentiate, sum ----
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int bl = 0; bl < 9; ++bl) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s0[bl][r] = fast_exp2(fmaf(s0[bl][r], c, -m0));
      s1[bl][r] = fast_exp2(fmaf(s1[bl][r], c, -m1));
      l0 += s0[bl][r];
      l1 += s1[bl][r];
    }
  }
  const float z0 = quad_sum(l0) + fast_exp2(sink0 - m0);
  const float z1 = quad_sum(l1) + fast_exp2(sink1 - m1);

  // ---- O^T = V^T P^T ----
  f32x4 o0[8], o1[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) { o0[b] = zero4; o1[b] = zero4; }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (32 * p + 31 < lo_min) continue;  // pair entirely before every window
    pv_pair(vs, 32 * p, i, g, pack_pair(s0[2 * p], s0[2 * p + 1]), pack_pair(s1[2 * p], s1[2 * p + 1]),
            o0, o1);
  }
  pv_single(vs, 128, i, g, pack_quad(s0[8]), pack_quad(s1[8]), o0, o1);

  write_out(a, ri, g, o0, o1, z0, z1, m0, m1);
}

// ---------------------------------------------------------------------------
// Any window: online softmax over 64-key chunks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 1) void online_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kChunk * kRowBytes];
  char* ks = smem;
  char* vs = smem + kChunk * kRowBytes;

  const int ntiles = (a.total_tokens + kQT - 1) / kQT;
  // Heaviest tiles (latest queries) first; consecutive ids spread over the XCDs.
  const int item = gridDim.x - 1 - blockIdx.x;
  const int oct = item / ntiles;
  const int q0 = (item - oct * ntiles) * kQT;
  const int h_base = oct * kHG;
  const int kvh = h_base / (a.num_q_heads / a.num_kv_heads);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int t = threadIdx.x;
  const int N = a.total_tokens, hkv = a.num_kv_heads;
  const bf16* kp = static_cast<const bf16*>(a.k);
  const bf16* vp = static_cast<const bf16*>(a.v);

  const RowInfo ri = row_info(a, q0, h_base, w, i);
  bf16x8 qa[4], qb[4];
  load_q(a, ri, g, qa, qb);
  const int lo_min = __shfl(ri.lo, 0);
  const int lo_max = __shfl(ri.lo, 15);
  const int kend = q0 + kQT;                       // one past the last key of the tile
  const int nchunks = (kend - lo_min + kChunk - 1) / kChunk;
  const float c = a.scale * kLog2e;
  const float sink0 = a.sinks ? a.sinks[ri.h0] * kLog2e : -INFINITY;
  const float sink1 = a.sinks ? a.sinks[ri.h1] * kLog2e : -INFINITY;

  float m0 = sink0, m1 = sink1;
  float l0 = (sink0 == -INFINITY) ? 0.f : 1.f;
  float l1 = (sink1 == -INFINITY) ? 0.f : 1.f;
  f32x4 o0[8], o1[8];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 8; ++b) { o0[b] = zero4; o1[b] = zero4; }

  constexpr int kIters = kChunk * kUnitsPerRow / kThreads;  // 4
  u32x4 pk[kIters], pv[kIters];
  auto prefetch = [&](int kb) {
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int x = it * kThreads + t;
      const int key = kb + (x >> 4);
      pk[it] = (u32x4){0, 0, 0, 0};
      pv[it] = (u32x4){0, 0, 0, 0};
      if (key >= 0 && key < N) {
        const size_t off = ((size_t)key * hkv + kvh) * D + (x & 15) * 8;
        pk[it] = *reinterpret_cast<const u32x4*>(kp + off);
        pv[it] = *reinterpret_cast<const u32x4*>(vp + off);
      }
    }
  };
  prefetch(kend - nchunks * kChunk);

  for (int ch = 0; ch < nchunks; ++ch) {
    const int kb = kend - (nchunks - ch) * kChunk;  // first key of this chunk
    __syncthreads();  // previous chunk fully consumed
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int x = it * kThreads + t;
      *reinterpret_cast<u32x4*>(ks + lds_off(x >> 4, x & 15)) = pk[it];
      *reinterpret_cast<u32x4*>(vs + lds_off(x >> 4, x & 15)) = pv[it];
    }
    __syncthreads();
    if (ch + 1 < nchunks) prefetch(kb + kChunk);

    f32x4 s0[4], s1[4];
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
      s0[bl] = zero4;
      s1[bl] = zero4;
      const int row = 32 * (bl >> 1) + pair_row(i, bl & 1);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8 kf = lds_read8(ks, row, 4 * cc + g);
        s0[bl] = mfma32(kf, qa[cc], s0[bl]);
        s1[bl] = mfma32(kf, qb[cc], s1[bl]);
      }
    }
    // mask: needed unless every key of the chunk is visible to every row
    const bool full = kb >= lo_max && kb + kChunk - 1 <= q0;
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!full) {
          const int key = kb + 32 * (bl >> 1) + 8 * g + 4 * (bl & 1) + r;
          const bool ok = key >= ri.lo && key <= ri.qi;
          s0[bl][r] = ok ? s0[bl][r] : -INFINITY;
          s1[bl][r] = ok ? s1[bl][r] : -INFINITY;
        }
        mx0 = fmaxf(mx0, s0[bl][r]);
        mx1 = fmaxf(mx1, s1[bl][r]);
      }
    }
    const float n0 = fmaxf(m0, quad_max(mx0) * c);
    const float n1 = fmaxf(m1, quad_max(mx1) * c);
    const float e0 = (n0 == -INFINITY) ? 0.f : n0;  // all-masked rows so far
    const float e1 = (n1 == -INFINITY) ? 0.f : n1;
    const float al0 = (m0 == -INFINITY) ? 0.f : fast_exp2(m0 - n0);
    const float al1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - n1);
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int bl = 0; bl < 4; ++bl) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[bl][r] = fast_exp2(fmaf(s0[bl][r], c, -e0));
        s1[bl][r] = fast_exp2(fmaf(s1[bl][r], c, -e1));
        ps0 += s0[bl][r];
        ps1 += s1[bl][r];
      }
    }
    l0 = l0 * al0 + quad_sum(ps0);
    l1 = l1 * al1 + quad_sum(ps1);
    m0 = n0;
    m1 = n1;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      o0[b] *= al0;
      o1[b] *= al1;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
      pv_pair(vs, 32 * p, i, g, pack_pair(s0[2 * p], s0[2 * p + 1]),
              pack_pair(s1[2 * p], s1[2 * p + 1]), o0, o1);
  }
  write_out(a, ri, g, o0, o1, l0, l1, m0, m1);
}

}  // namespace

bool swa_window_mfma_supported(const PrefillArgs& a, bool bf16_io) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return bf16_io && a.head_dim == 128 && G % kHG == 0 && a.window >= 1 && a.window <= 128;
}

bool online_mfma_supported(const PrefillArgs& a, bool bf16_io) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return bf16_io && a.head_dim == 128 && G % kHG == 0 && a.window >= 1;
}

hipError_t launch_swa_window_mfma(const PrefillArgs& a, hipStream_t s) {
  const long ntiles = (a.total_tokens + kQT - 1) / kQT;
  const long total = ntiles * (a.num_q_heads / kHG);
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(swa_window_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_online_mfma(const PrefillArgs& a, hipStream_t s) {
  const long ntiles = (a.total_tokens + kQT - 1) / kQT;
  const long total = ntiles * (a.num_q_heads / kHG);
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(online_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace swa
