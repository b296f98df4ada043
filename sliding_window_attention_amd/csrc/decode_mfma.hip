// Matrix-core decode / MTP-verify kernel against a 128-slot ring buffer.
//
// T query tokens per sequence (the current token plus T-1 drafts verified in one
// pass: MiMo-V2-Flash Technical Report digest, section 2.3) attend the ring's
// logical slots t+1 .. 127 plus new tokens 0 .. t, with the per-head sink in the
// softmax denominator (digest, section 2.2.2).  The 8 query heads sharing a KV
// head and the T tokens form the query columns (T*8 columns, 16 per MFMA tile),
// so each ring byte is read once for all of them.
//
// One workgroup per (sequence, head octet); wavefront w scores logical slots
// 32w .. 32w+31, wavefront 0 also the new tokens.  The four partial results are
// merged exactly: the wavefronts first agree on each column's maximum (through
// LDS), exponentiate against that common maximum, and their partial sums and
// partial outputs then simply add.  Everything is read straight from HBM into
// MFMA operand registers; V rows are loaded 16 lanes per 256-byte row (fully
// coalesced) and transposed in registers.
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace swa {
namespace {

using namespace tile;

constexpr int kW = 128;         // ring slots
constexpr int kHG = 8;          // query heads per KV-head group handled together
constexpr int kThreads = 256;
constexpr int kColBytes = 528;  // fp32 partial row (512 B) padded against bank conflicts

template <int NT>
struct DecodeSmem {
  float m[4][NT * 16];
  float l[4][NT * 16];
  char o[4][NT * 16][kColBytes];
};

template <int NT>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) DecodeSmem<NT> sm;
  const int noct = a.num_q_heads / kHG;
  const int b = blockIdx.x / noct;
  const int oct = blockIdx.x - b * noct;
  const int h_base = oct * kHG;
  const int hkv = a.num_kv_heads;
  const int kvh = h_base / (a.num_q_heads / hkv);
  const int T = a.t_new;
  const int Hq = a.num_q_heads;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  int head = a.ring_head[b] % kW;
  head += head < 0 ? kW : 0;

  const bf16* qp = static_cast<const bf16*>(a.q);
  const bf16* kc = static_cast<const bf16*>(a.k_cache) + ((size_t)b * hkv + kvh) * kW * D;
  const bf16* vc = static_cast<const bf16*>(a.v_cache) + ((size_t)b * hkv + kvh) * kW * D;
  const bf16* kn = static_cast<const bf16*>(a.k_new) + ((size_t)b * T * hkv + kvh) * D;
  const bf16* vn = static_cast<const bf16*>(a.v_new) + ((size_t)b * T * hkv + kvh) * D;

  // ---- loads: ring K (A operand), ring V rows, Q (B operand) ----
  bf16x8 kf[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int kr = 32 * w + pair_row(i, s);
    const int phys = (head + kr) & (kW - 1);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      kf[s][cc] = kr != 0 ? *reinterpret_cast<const bf16x8*>(kc + (size_t)phys * D + 32 * cc + 8 * g)
                          : zero8();
  }
  bf16x8 vr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int kr = 32 * w + 8 * g + e;
    const int phys = (head + kr) & (kW - 1);
    vr[e] = kr != 0 ? *reinterpret_cast<const bf16x8*>(vc + (size_t)phys * D + 8 * i) : zero8();
  }
  bf16x8 qf[NT][4];
  int tcol[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    tcol[tt] = 2 * tt + (i >> 3);
    const int h = h_base + (i & 7);
    const bool ok = tcol[tt] < T;
    const size_t off = (((size_t)b * T + tcol[tt]) * Hq + h) * D + 8 * g;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      qf[tt][cc] = ok ? *reinterpret_cast<const bf16x8*>(qp + off + 32 * cc) : zero8();
  }
  // new tokens (wavefront 0): K rows = token i, V rows = tokens 4g .. 4g+3
  bf16x8 kfn[4], vrn[4];
  if (w == 0) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      kfn[cc] = i < T ? *reinterpret_cast<const bf16x8*>(kn + (size_t)i * hkv * D + 32 * cc + 8 * g)
                      : zero8();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int u = 4 * g + e;
      vrn[e] = u < T ? *reinterpret_cast<const bf16x8*>(vn + (size_t)u * hkv * D + 8 * i) : zero8();
    }
  }

  const float c = a.scale * kLog2e;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---- scores ----
  f32x4 s[NT][2], sn[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      s[tt][ss] = zero4;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) s[tt][ss] = mfma32(kf[ss][cc], qf[tt][cc], s[tt][ss]);
    }
    sn[tt] = zero4;
    if (w == 0) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) sn[tt] = mfma32(kfn[cc], qf[tt][cc], sn[tt]);
    }
  }

  // ---- mask (ring slot kr visible to token t iff kr >= t+1; new token u iff u <= t) ----
  float mx[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    mx[tt] = -INFINITY;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (w == 0) {
          const int kr = 8 * g + 4 * ss + r;
          s[tt][ss][r] = kr >= tcol[tt] + 1 ? s[tt][ss][r] : -INFINITY;
        }
        mx[tt] = fmaxf(mx[tt], s[tt][ss][r]);
      }
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = 4 * g + r;
        sn[tt][r] = (u <= tcol[tt] && u < T) ? sn[tt][r] : -INFINITY;
        mx[tt] = fmaxf(mx[tt], sn[tt][r]);
      }
    }
    mx[tt] = quad_max(mx[tt]);
    if (g == 0) sm.m[w][tt * 16 + i] = mx[tt] * c;
  }
  __syncthreads();

  // ---- common maximum (sink included), exponentiate, partial sums ----
  float mcol[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int col = tt * 16 + i;
    const float sink2 = a.sinks[h_base + (i & 7)] * kLog2e;
    mcol[tt] = fmaxf(fmaxf(fmaxf(sm.m[0][col], sm.m[1][col]), fmaxf(sm.m[2][col], sm.m[3][col])), sink2);
    float ps = 0.f;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[tt][ss][r] = fast_exp2(fmaf(s[tt][ss][r], c, -mcol[tt]));
        ps += s[tt][ss][r];
      }
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sn[tt][r] = fast_exp2(fmaf(sn[tt][r], c, -mcol[tt]));
        ps += sn[tt][r];
      }
    }
    ps = quad_sum(ps);
    if (g == 0) sm.l[w][col] = ps;
  }

  // ---- partial O^T = V^T P^T ----
  f32x4 o[NT][8];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) o[tt][bb] = zero4;
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    const bf16x8 av = column8(vr, bb);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) o[tt][bb] = mfma32(av, pack_pair(s[tt][0], s[tt][1]), o[tt][bb]);
  }
  if (w == 0) {
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const bf16x4 av = column4(vrn, bb);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) o[tt][bb] = mfma16(av, pack_quad(sn[tt]), o[tt][bb]);
    }
  }
  // lane (i, g) holds head-dim 32g + 8r + bb of column tt*16 + i
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    char* row = sm.o[w][tt * 16 + i];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 lo = {o[tt][0][r], o[tt][1][r], o[tt][2][r], o[tt][3][r]};
      f32x4 hi = {o[tt][4][r], o[tt][5][r], o[tt][6][r], o[tt][7][r]};
      *reinterpret_cast<f32x4*>(row + (32 * g + 8 * r) * 4) = lo;
      *reinterpret_cast<f32x4*>(row + (32 * g + 8 * r + 4) * 4) = hi;
    }
  }
  __syncthreads();

  // ---- merge the four partials; 16 threads per column, 8 head-dim elements each ----
  bf16* out = static_cast<bf16*>(a.out);
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const int item = it * kThreads + threadIdx.x;
    const int col = item >> 4, dc = item & 15;
    const int t = 2 * (col >> 4) + ((col & 15) >> 3);
    const int h = h_base + (col & 7);
    if (t >= T) continue;
    const float sink2 = a.sinks[h] * kLog2e;
    const float m = fmaxf(fmaxf(fmaxf(sm.m[0][col], sm.m[1][col]), fmaxf(sm.m[2][col], sm.m[3][col])), sink2);
    const float z = sm.l[0][col] + sm.l[1][col] + sm.l[2][col] + sm.l[3][col] + fast_exp2(sink2 - m);
    const float inv = 1.f / z;
    f32x4 acc0 = zero4, acc1 = zero4;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const char* row = sm.o[ww][col];
      acc0 += *reinterpret_cast<const f32x4*>(row + dc * 32);
      acc1 += *reinterpret_cast<const f32x4*>(row + dc * 32 + 16);
    }
    bf16x8 v8;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      bf16x2 x = __builtin_convertvector((f32x2){acc0[e] * inv, acc0[e + 1] * inv}, bf16x2);
      bf16x2 y = __builtin_convertvector((f32x2){acc1[e] * inv, acc1[e + 1] * inv}, bf16x2);
      v8[e] = x[0]; v8[e + 1] = x[1];
      v8[4 + e] = y[0]; v8[4 + e + 1] = y[1];
    }
    const size_t row_idx = ((size_t)b * T + t) * Hq + h;
    *reinterpret_cast<bf16x8*>(out + row_idx * D + 8 * dc) = v8;
    if (a.lse != nullptr && dc == 0) a.lse[row_idx] = (m + fast_log2(z)) * kLn2;
  }
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a, bool bf16_io) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return bf16_io && a.head_dim == 128 && G % kHG == 0 && a.window == kW && a.t_new >= 1 &&
         a.t_new <= 4;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  const long blocks = (long)a.batch * (a.num_q_heads / kHG);
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (a.t_new <= 2)
    hipLaunchKernelGGL(decode_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace swa
