// Gradients of the SWA-with-sink forward with respect to Q, K, V and the sinks, on
// the vector ALUs (fp32 arithmetic; any head_dim of 64 / 128, any group size and
// window, fp32 or bf16 I/O).
//
// With p_ij = exp(a_ij - lse_i) the weight of key j in row i (a_ij the scaled logit,
// lse_i the forward's log-normaliser, sink included) and p_s(i) = exp(sink - lse_i)
// the sink's weight, O_i = sum_j p_ij v_j and the sink carries no value
// (MiMo-V2-Flash Technical Report digest, section 2.2.2), so
//   delta_i = dO_i . O_i,   da_ij = p_ij (dO_i . v_j - delta_i),
//   dq_i = scale sum_j da_ij k_j,   dk_j = scale sum_i da_ij q_i,   dv_j = sum_i p_ij dO_i,
//   dsink_h = -sum_i p_s(i) delta_i,
// where dk and dv also sum over the query heads that share a KV head.  Kernels:
// (1) delta and the sink terms, a few lanes per row; (2) dq per query row and (3) dk
// and dv per key row, one wavefront per row; (4) dsink per head by a two-pass
// fixed-order reduction (deterministic: no atomics anywhere).  For bf16, head_dim
// 128, windows up to 128 and groups of 8k heads, the matrix-core kernels replace
// (1), (2) and (3): their dq kernel forms delta and the sink terms of the rows it owns.
#include "common.h"
#include "kernels.h"

namespace swa {
namespace {

constexpr int kRows = 4;  // wavefronts (rows) per workgroup

template <typename T> __device__ __forceinline__ float ld(const T* p) { return (float)*p; }
template <typename T> __device__ __forceinline__ T st(float x) { return (T)x; }

// Window of query token n: the first visible key.
__device__ __forceinline__ int first_key(const BackwardArgs& a, int n) {
  const int start = seq_start_of(a.cu_seqlens, a.num_seqs, n);
  const long lw = (long)n - a.window + 1;
  return lw > start ? (int)lw : start;
}

// (1) delta = dO . O and the sink term exp(sink - lse) * delta of each (token, head)
// row: 16-byte loads, kLpr lanes per row, kPasses rows per lane in flight.
constexpr int kPrepThreads = 256;
constexpr int kPasses = 4;
template <typename T, int D>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(BackwardArgs a) {
  constexpr int kVec = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int kLpr = D / kVec;        // lanes per row (8 .. 32, a power of two)
  constexpr int kRowsPerPass = kPrepThreads / kLpr;
  const long nrows = (long)a.total_tokens * a.num_q_heads;
  const int sub = threadIdx.x % kLpr;
  const long row0 = (long)blockIdx.x * kRowsPerPass * kPasses + threadIdx.x / kLpr;
  u32x4 ov[kPasses], dv[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const long row = row0 + p * kRowsPerPass;
    const long rr = row < nrows ? row : nrows - 1;  // every lane stays active for the shuffles
    ov[p] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.out) + rr * D + sub * kVec);
    dv[p] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dout) + rr * D + sub * kVec);
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    float acc = 0.f;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 o = __builtin_bit_cast(bf16x8, ov[p]), d = __builtin_bit_cast(bf16x8, dv[p]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)d[e], acc);
    } else {
      const f32x4 o = __builtin_bit_cast(f32x4, ov[p]), d = __builtin_bit_cast(f32x4, dv[p]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(o[e], d[e], acc);
    }
#pragma unroll
    for (int o = kLpr / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    const long row = row0 + p * kRowsPerPass;
    if (sub == 0 && row < nrows) {
      a.delta[row] = acc;
      if (a.sinks) {
        const int h = (int)(row % a.num_q_heads);
        a.sink_term[row] = expf(a.sinks[h] - a.lse[row]) * acc;
      }
    }
  }
}

// (2) dq of one (token, head) row.  Lanes own keys for the logits and dO . v; lanes
// own head-dim elements for the accumulation.
template <typename T, int D>
__global__ __launch_bounds__(kRows * kWave) void bwd_dq_kernel(BackwardArgs a) {
  __shared__ float rows[kRows][2][D];  // this row's q and dO in fp32
  const int wv = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * kRows + wv;
  if (row >= (long)a.total_tokens * a.num_q_heads) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int n = (int)(row / hq), h = (int)(row % hq);
  const int kvh = h / (hq / hkv);
  const T* qr = static_cast<const T*>(a.q) + row * D;
  const T* dor = static_cast<const T*>(a.dout) + row * D;
  for (int d = lane; d < D; d += kWave) {
    rows[wv][0][d] = ld(qr + d);
    rows[wv][1][d] = ld(dor + d);
  }
  __builtin_amdgcn_wave_barrier();
  const T* kp = static_cast<const T*>(a.k);
  const T* vp = static_cast<const T*>(a.v);
  const float c = a.scale * kLog2e, lse2 = a.lse[row] * kLog2e, delta = a.delta[row];
  float dq[D / kWave];
#pragma unroll
  for (int e = 0; e < D / kWave; ++e) dq[e] = 0.f;
  const int jlo = first_key(a, n);
  for (int jb = jlo; jb <= n; jb += kWave) {
    const int j = jb + lane;
    float ds = 0.f;
    if (j <= n) {
      const T* kr = kp + ((size_t)j * hkv + kvh) * D;
      const T* vr = vp + ((size_t)j * hkv + kvh) * D;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s = fmaf(rows[wv][0][d], ld(kr + d), s);
        dp = fmaf(rows[wv][1][d], ld(vr + d), dp);
      }
      const float p = fast_exp2(s * c - lse2);
      ds = p * (dp - delta);
    }
    const int nk = min(kWave, n - jb + 1);
    for (int jj = 0; jj < nk; ++jj) {
      const float dsj = __shfl(ds, jj);
      const T* kr = kp + ((size_t)(jb + jj) * hkv + kvh) * D;
#pragma unroll
      for (int e = 0; e < D / kWave; ++e) dq[e] = fmaf(dsj, ld(kr + lane + e * kWave), dq[e]);
    }
  }
  T* out = static_cast<T*>(a.dq) + row * D;
#pragma unroll
  for (int e = 0; e < D / kWave; ++e) out[lane + e * kWave] = st<T>(dq[e] * a.scale);
}

// (3) dk and dv of one (key token, KV head) row: every (query, head) pair that sees
// the key -- queries j .. j + window - 1 of the same sequence, the group's heads.
template <typename T, int D>
__global__ __launch_bounds__(kRows * kWave) void bwd_dkdv_kernel(BackwardArgs a) {
  __shared__ float kv[kRows][2][D];  // this key's k and v in fp32
  const int wv = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * kRows + wv;
  if (row >= (long)a.total_tokens * a.num_kv_heads) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int hq = a.num_q_heads, hkv = a.num_kv_heads, G = hq / hkv;
  const int j = (int)(row / hkv), kvh = (int)(row % hkv);
  const T* kr = static_cast<const T*>(a.k) + row * D;
  const T* vr = static_cast<const T*>(a.v) + row * D;
  for (int d = lane; d < D; d += kWave) {
    kv[wv][0][d] = ld(kr + d);
    kv[wv][1][d] = ld(vr + d);
  }
  __builtin_amdgcn_wave_barrier();
  // last query that sees key j: within the window and the key's own sequence, the
  // largest s with cu[s] <= j (so cu[s + 1] > j even past zero-length sequences)
  int seq = 0;
  {
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens[mid] <= j) lo = mid; else hi = mid;
    }
    seq = lo;
  }
  const long seq_end = a.cu_seqlens[seq + 1];  // one past the sequence's last token
  const long last = min((long)j + a.window - 1, seq_end - 1);
  const int npairs = (int)((last - j + 1) * G);
  const T* qp = static_cast<const T*>(a.q);
  const T* dop = static_cast<const T*>(a.dout);
  const float c = a.scale * kLog2e;
  float dk[D / kWave], dv[D / kWave];
#pragma unroll
  for (int e = 0; e < D / kWave; ++e) { dk[e] = 0.f; dv[e] = 0.f; }
  for (int pb = 0; pb < npairs; pb += kWave) {
    const int idx = pb + lane;
    float p = 0.f, ds = 0.f;
    if (idx < npairs) {
      const int i = j + idx / G, h = kvh * G + idx % G;
      const size_t r = (size_t)i * hq + h;
      const T* qi = qp + r * D;
      const T* doi = dop + r * D;
      float sc = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        sc = fmaf(ld(qi + d), kv[wv][0][d], sc);
        dp = fmaf(ld(doi + d), kv[wv][1][d], dp);
      }
      p = fast_exp2(sc * c - a.lse[r] * kLog2e);
      ds = p * (dp - a.delta[r]);
    }
    const int nk = min(kWave, npairs - pb);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = __shfl(p, jj), dsj = __shfl(ds, jj);
      const int id2 = pb + jj;
      const size_t r = (size_t)(j + id2 / G) * hq + kvh * G + id2 % G;
      const T* qi = qp + r * D;
      const T* doi = dop + r * D;
#pragma unroll
      for (int e = 0; e < D / kWave; ++e) {
        dv[e] = fmaf(pj, ld(doi + lane + e * kWave), dv[e]);
        dk[e] = fmaf(dsj, ld(qi + lane + e * kWave), dk[e]);
      }
    }
  }
  T* dko = static_cast<T*>(a.dk) + row * D;
  T* dvo = static_cast<T*>(a.dv) + row * D;
#pragma unroll
  for (int e = 0; e < D / kWave; ++e) {
    dko[lane + e * kWave] = st<T>(dk[e] * a.scale);
    dvo[lane + e * kWave] = st<T>(dv[e]);
  }
}

// (4) dsink_h = -sum_n sink_term[n, h] in a fixed order, in two passes: chunks of
// kSinkChunk tokens summed per head (the sum replaces the chunk's first row, which
// only the summing thread reads), then the chunk sums of each head by a tree.
constexpr int kSinkChunk = 32;
constexpr int kSinkThreads = 256;
__global__ __launch_bounds__(kSinkThreads) void bwd_sink_chunk_kernel(BackwardArgs a) {
  const int h = blockIdx.y * kSinkThreads + threadIdx.x;
  if (h >= a.num_q_heads) return;
  const long n0 = (long)blockIdx.x * kSinkChunk;
  const long n1 = min(n0 + kSinkChunk, (long)a.total_tokens);
  // every load issued before the first add (rows past the stream read its last row and
  // count as 0), then the sum in row order
  float v[kSinkChunk];
#pragma unroll
  for (int k = 0; k < kSinkChunk; ++k) {
    const long n = n0 + k < n1 ? n0 + k : n1 - 1;
    v[k] = a.sink_term[n * a.num_q_heads + h];
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kSinkChunk; ++k) acc += n0 + k < n1 ? v[k] : 0.f;
  a.sink_term[n0 * a.num_q_heads + h] = acc;
}
__global__ __launch_bounds__(kSinkThreads) void bwd_dsink_kernel(BackwardArgs a) {
  __shared__ float part[kSinkThreads];
  const int h = blockIdx.x;
  const long nchunks = ((long)a.total_tokens + kSinkChunk - 1) / kSinkChunk;
  float acc = 0.f;
#pragma unroll 8
  for (long c = threadIdx.x; c < nchunks; c += kSinkThreads)
    acc += a.sink_term[c * kSinkChunk * a.num_q_heads + h];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kSinkThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dsinks[h] = 0.f - part[0];  // +0 for an empty stream
}

template <typename T, int D>
hipError_t launch_t(const BackwardArgs& a, bool kMfma, hipStream_t s) {
  const long qrows = (long)a.total_tokens * a.num_q_heads;
  const long krows = (long)a.total_tokens * a.num_kv_heads;
  const long qblocks = (qrows + kRows - 1) / kRows, kblocks = (krows + kRows - 1) / kRows;
  const long prows = kPrepThreads / (D / (16 / (int)sizeof(T))) * kPasses;
  const long pblocks = (qrows + prows - 1) / prows;
  const long nchunks = ((long)a.total_tokens + kSinkChunk - 1) / kSinkChunk;
  const long hgroups = (a.num_q_heads + kSinkThreads - 1) / kSinkThreads;
  if (qblocks > 0x7fffffffL || kblocks > 0x7fffffffL || nchunks > 0x7fffffffL || hgroups > 0xffff)
    return hipErrorInvalidConfiguration;
  if (qrows > 0) {  // an empty stream only writes zero sink gradients
    if (kMfma) {
      // the matrix-core dq kernel forms delta and the sink terms itself (it reads dO
      // and, for this, O), before the dk/dv kernel reads them
      const hipError_t m = launch_backward_mfma(a, s);
      if (m != hipSuccess) return m;
      if (a.dsinks != nullptr)
        hipLaunchKernelGGL(bwd_sink_chunk_kernel, dim3((unsigned)nchunks, (unsigned)hgroups),
                           dim3(kSinkThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)pblocks), dim3(kPrepThreads), 0, s, a);
      if (a.dsinks != nullptr)
        hipLaunchKernelGGL(bwd_sink_chunk_kernel, dim3((unsigned)nchunks, (unsigned)hgroups),
                           dim3(kSinkThreads), 0, s, a);
      hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3((unsigned)qblocks), dim3(kRows * kWave), 0, s, a);
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D>), dim3((unsigned)kblocks), dim3(kRows * kWave), 0, s, a);
    }
  }
  if (a.dsinks != nullptr)
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3((unsigned)a.num_q_heads), dim3(kSinkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, bool bf16_io, hipStream_t s) {
  // bf16, head_dim 128, windows up to 128, groups of 8k heads: dq and dk/dv on the
  // matrix cores (backward_mfma.hip); delta and dsink stay here
  const bool mfma = backward_mfma_supported(a, bf16_io);
  if (bf16_io) return a.head_dim == 64 ? launch_t<bf16, 64>(a, false, s) : launch_t<bf16, 128>(a, mfma, s);
  return a.head_dim == 64 ? launch_t<float, 64>(a, false, s) : launch_t<float, 128>(a, false, s);
}

}  // namespace swa
