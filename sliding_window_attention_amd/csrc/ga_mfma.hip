// Matrix-core prefill with an online softmax: global causal attention (the GA
// layers of the hybrid block: MiMo-V2-Flash Technical Report digest, section 2.2,
// the same operator with no window and no sink) and sliding windows longer than
// 128 keys (with the per-head sink of section 2.2.2).
//
// A workgroup of 8 wavefronts owns 32 consecutive query tokens and the 8 query
// heads of one KV head; wavefront w takes query sub-tile w >> 2 and heads
// 2(w & 3), 2(w & 3) + 1, i.e. two 16-query MFMA tiles sharing every K read.  Keys
// are staged 128 at a time through two LDS buffers: the next stage is loaded into
// registers while the current one is multiplied (as two 64-key steps), written to
// the other buffer, and one barrier per stage hands it over (one per 64 keys cost
// 3% more).  The running maximum is raised
// lazily: O and the running sum are rescaled only when some row's maximum grows
// by more than kSlack (log2 units); otherwise the exponent keeps the older, smaller
// reference and the weights may exceed 1 by at most 2^kSlack, which fp32 sums and
// bf16 weights hold without loss of relative precision.  Once every row has a
// finite reference, a chunk is exponentiated against it without forming maxima:
// the weights are non-negative, so a lane's partial sum of at most 2^kSlack bounds
// each of its weights by the same; a larger sum (rare once the maxima settle) sends
// the chunk through the full path with its scores formed again.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace swa {
namespace {

using namespace tile;

constexpr int kQT = 32;                  // query tokens per workgroup
constexpr int kHG = 8;                   // query heads per workgroup
constexpr int kThreads = 512;            // 8 wavefronts
constexpr int kChunk = 64;               // keys per compute step
constexpr int kStage = 128;              // keys staged in LDS per barrier (two steps)
constexpr int kKPlane = kStage * 64;     // bytes of one 32-element chunk plane of K
constexpr int kKBuf = 4 * kKPlane;       // 32768
constexpr int kVBuf = kStage * kVPitch;  // 33792
constexpr int kBuf = kKBuf + kVBuf;
constexpr float kSlack = 8.f;
constexpr float kSlackPow = 256.f;  // 2^kSlack

// Staged K/V as loaded: 16 bytes of bf16, or (FP8) 8 bytes of E4M3 codes widened to
// bf16 (exactly) only when committed to LDS, so that no conversion waits on a load.
template <bool FP8>
using GaRaw = typename std::conditional<FP8, u32x2, u32x4>::type;

// FP8: K and V arrive as E4M3 codes; the K scale joins the logit multiplier and the V
// scale the output's 1/l.
template <bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void ga_chunk_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kBuf];
  const int N = a.total_tokens, Hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int ntiles = (N + kQT - 1) / kQT;
  // latest (heaviest) tiles first; consecutive workgroups spread over the XCDs
  const int item = __builtin_amdgcn_readfirstlane(gridDim.x - 1 - blockIdx.x);
  const int oct = item / ntiles;
  const int q0 = (item - oct * ntiles) * kQT;
  const int kvh = (oct * kHG) / (Hq / hkv);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int t = threadIdx.x;
  const int h0 = oct * kHG + 2 * (w & 3);
  const int qw = q0 + 16 * (w >> 2);  // first query of this wavefront's tiles
  const int qi = qw + i;
  using KvT = typename std::conditional<FP8, uint8_t, bf16>::type;
  const KvT* kp = static_cast<const KvT*>(a.k);
  const KvT* vp = static_cast<const KvT*>(a.v);
  const bf16* qp = static_cast<const bf16*>(a.q);
  const float c = a.scale * kLog2e * (FP8 ? a.k_scale : 1.f);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---- first visible key of each row, of this wavefront and of the workgroup ----
  const int start = seq_start_of(a.cu_seqlens, a.num_seqs, qi < N ? qi : N - 1);
  const long lw = (long)qi - a.window + 1;
  const int lo = lw > start ? (int)lw : start;
  const int lo_w_min = __builtin_amdgcn_readfirstlane(lo);  // rows are ordered
  const int lo_w_max = __builtin_amdgcn_readlane(lo, 15);
  const int s0q = seq_start_of(a.cu_seqlens, a.num_seqs, q0);
  const long lw0 = (long)q0 - a.window + 1;
  const int lo_wg = __builtin_amdgcn_readfirstlane(lw0 > s0q ? (int)lw0 : s0q);
  const int kend = q0 + kQT;
  const int nstages = (kend - lo_wg + kStage - 1) / kStage;

  // ---- Q of the two tiles: lane (i, g) holds head-dim 32cc + 8g .. +8 of query qi ----
  bf16x8 qa[4], qb[4];
  {
    const bool ok = qi < N;
    const size_t r0 = ((size_t)qi * Hq + h0) * D + 8 * g;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      qa[cc] = ok ? *reinterpret_cast<const bf16x8*>(qp + r0 + 32 * cc) : zero8();
      qb[cc] = ok ? *reinterpret_cast<const bf16x8*>(qp + r0 + D + 32 * cc) : zero8();
    }
  }

  // ---- stage staging.  K: wavefront w moves plane w & 3 of the stage rows
  // r = 64 (w >> 2) + 16 j + lane / 4 (j < 4), lane L taking the unit that belongs at slot
  // L & 3 of its row (unit 4 (w & 3) + ((L & 3) ^ kswz(r))), so that each store covers 1 KB
  // of one plane and every 16 lanes write 256 contiguous bytes (rows of one unit index
  // across the four planes would share their banks: plane bases are 8 KB apart).  V:
  // thread t moves the unit su = t & 15 of rows srow + 32 j, srow = t >> 4. ----
  const int srow = t >> 4, su = t & 15;
  const size_t key_stride = (size_t)hkv * D;  // elements from one key's row to the next
  const int kcc = w & 3;
  auto krow = [&](int j) { return 64 * (w >> 2) + 16 * j + (lane >> 2); };
  auto kunit = [&](int j) { return 4 * kcc + ((lane & 3) ^ kswz(krow(j))); };
  uint32_t koff[4];  // byte offsets of the thread's K units from the stage's first key row
#pragma unroll
  for (int j = 0; j < 4; ++j)
    koff[j] = (uint32_t)((((size_t)krow(j) * hkv + kvh) * D + kunit(j) * 8) * sizeof(KvT));
  const uint32_t voff0 = (uint32_t)((((size_t)srow * hkv + kvh) * D + su * 8) * sizeof(KvT));
  const size_t gstep = 32 * key_stride;  // elements from row r to row r + 32
  GaRaw<FP8> pf[8];
  bool edge = false;  // (uniform) the staged keys reach outside [0, N)
  bool okk[4] = {true, true, true, true};  // K row krow(j) of the stage exists
  bool okv[4] = {true, true, true, true};  // V row srow + 32 j of the stage exists
  auto prefetch = [&](int kb) {
    edge = !(kb >= 0 && kb + kStage <= N);
    if (!edge) {
      // whole stage inside the token stream: a uniform base and lane-constant offsets
      const char* kbase = reinterpret_cast<const char*>(kp + (size_t)kb * key_stride);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const char* vbase = reinterpret_cast<const char*>(vp + (size_t)kb * key_stride + j * gstep);
        pf[j] = *reinterpret_cast<const GaRaw<FP8>*>(kbase + koff[j]);
        pf[4 + j] = *reinterpret_cast<const GaRaw<FP8>*>(vbase + voff0);
      }
    } else {
      // rows outside the stream load a clamped row (no masked loads, which would
      // force early waits) and are zeroed when committed
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rk = kb + krow(j), rv = kb + srow + 32 * j;
        okk[j] = rk >= 0 && rk < N;
        okv[j] = rv >= 0 && rv < N;
        pf[j] = *reinterpret_cast<const GaRaw<FP8>*>(kp + ((size_t)min(max(rk, 0), N - 1) * hkv + kvh) * D +
                                                     kunit(j) * 8);
        pf[4 + j] = *reinterpret_cast<const GaRaw<FP8>*>(vp + ((size_t)min(max(rv, 0), N - 1) * hkv + kvh) * D +
                                                         su * 8);
      }
    }
  };
  // LDS byte offsets of the thread's units (put_k / put_v layouts).  Stage bases are
  // multiples of 32, so a key's swizzle equals that of its row in the stage.
  const int ks_off = kcc * kKPlane + 64 * 64 * (w >> 2) + 16 * lane;  // + 1024 j
  const int vs_off = kKBuf + srow * kVPitch + 16 * su;
  auto commit = [&](char* buf) {
    if (edge) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!okk[j]) pf[j] = GaRaw<FP8>{};
        if (!okv[j]) pf[4 + j] = GaRaw<FP8>{};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 kx, vx;
      if constexpr (FP8) {
        kx = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(pf[j]));
        vx = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(pf[4 + j]));
      } else {
        kx = pf[j];
        vx = pf[4 + j];
      }
      *reinterpret_cast<u32x4*>(buf + ks_off + 1024 * j) = kx;
      char* v = buf + vs_off + 32 * kVPitch * j;
      *reinterpret_cast<u32x2*>(v) = (u32x2){vx[0], vx[1]};
      *reinterpret_cast<u32x2*>(v + 8) = (u32x2){vx[2], vx[3]};
    }
  };

  // Lane-constant LDS offsets.  Chunk bases are multiples of 32, so a key's low
  // five bits equal its row's and the K swizzle depends on the row alone.
  const int pr0 = pair_row(i, 0), pr1 = pair_row(i, 1);
  const int ko0 = pr0 * 64 + 16 * (g ^ kswz(pr0));
  const int ko1 = pr1 * 64 + 16 * (g ^ kswz(pr1));
  const int vrow = 16 * (g >> 1) + 8 * (g & 1) + (i >> 2);  // V row of pair 0, first half
  const int vo = kKBuf + vrow * kVPitch + vquad_bytes(i);

  const float sink0 = a.sinks ? a.sinks[h0] * kLog2e : -INFINITY;
  const float sink1 = a.sinks ? a.sinks[h0 + 1] * kLog2e : -INFINITY;
  float m0 = sink0, m1 = sink1;  // reference maxima (log2 units), equal on a row's 4 lanes
  // this lane's share of the running sums (the 4 lanes of a row are added at the end)
  float l0 = (a.sinks && g == 0) ? 1.f : 0.f, l1 = l0;
  f32x4 o0[8], o1[8];
  bool ready = false;  // (uniform) every row of the wavefront has a finite reference maximum
#pragma unroll
  for (int b = 0; b < 8; ++b) { o0[b] = zero4; o1[b] = zero4; }

  prefetch(kend - nstages * kStage);
  commit(smem);
  __syncthreads();

  for (int st = 0; st < nstages; ++st) {
    const int kst = kend - (nstages - st) * kStage;  // first key of this stage
    const char* sbuf = smem + (st & 1) * kBuf;
    if (st + 1 < nstages) prefetch(kst + kStage);
#pragma unroll
  for (int sub = 0; sub < kStage / kChunk; ++sub) {
    const int kb = kst + sub * kChunk;  // first key of this step
    // the step's K rows start 64 bytes x kChunk x sub into each plane, its V rows
    // kChunk x sub rows in
    const char* buf = sbuf + sub * kChunk * 64;
    const char* vbuf = sbuf + sub * kChunk * kVPitch;

    // chunk entirely outside this wavefront's rows (before every window / after
    // every query): nothing to do
    const bool skip = kb + kChunk - 1 < lo_w_min || kb > qw + 15;
    if (!skip) {
      // ---- S^T = K Q^T over 4 blocks of 16 keys (2 pairs), masked where a row's
      // window or the causal edge cuts the chunk ----
      f32x4 s0[4], s1[4];
      const bool full = kb >= lo_w_max && kb + kChunk - 1 <= qw;  // (uniform) no row is cut
      auto products = [&]() {
        // Raised issue priority over the MFMA runs: the two waves sharing a SIMD then
        // tend to alternate matrix work with the other's softmax instead of colliding.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
          const int off = 32 * 64 * (bl >> 1) + ((bl & 1) ? ko1 : ko0);
          bf16x8 kf = *reinterpret_cast<const bf16x8*>(buf + off);
          s0[bl] = mfma32(kf, qa[0], zero4);
          s1[bl] = mfma32(kf, qb[0], zero4);
#pragma unroll
          for (int cc = 1; cc < 4; ++cc) {
            kf = *reinterpret_cast<const bf16x8*>(buf + cc * kKPlane + off);
            s0[bl] = mfma32(kf, qa[cc], s0[bl]);
            s1[bl] = mfma32(kf, qb[cc], s1[bl]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      };
      auto mask = [&]() {
        const unsigned span = (unsigned)(qi - lo);
#pragma unroll
        for (int bl = 0; bl < 4; ++bl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kb + 32 * (bl >> 1) + 8 * g + 4 * (bl & 1) + r;
            const bool ok = (unsigned)(key - lo) <= span;
            s0[bl][r] = ok ? s0[bl][r] : -INFINITY;
            s1[bl][r] = ok ? s1[bl][r] : -INFINITY;
          }
      };
      auto scores = [&]() {
        products();
        if (!full) mask();
      };
      // ---- exponentiate against the reference maxima and sum.  Once every row of the
      // wavefront has a finite reference, the chunk is exponentiated directly: if no
      // lane's partial sum of a head exceeds 2^kSlack, no weight does, which is exactly
      // the bound the lazy rescale keeps, and the weights equal those of the full path
      // below.  A weight that overflows is +inf (the arguments are finite or -inf, the
      // weights non-negative, so no NaN arises) and its sum fails the same test.
      // Otherwise the raw scores are formed again and the full path runs: per-lane
      // maxima, the rescale where a row's maximum outgrew its reference, the
      // exponentials.  The common case (references ready, no row cut by the chunk) is
      // tested before the products, so that no mask branch splits them from the
      // exponentials. ----
      float ps0 = 0.f, ps1 = 0.f;
      auto fast = [&]() {
#pragma unroll
        for (int bl = 0; bl < 4; ++bl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s0[bl][r] = fast_exp2(fmaf(s0[bl][r], c, -m0));
            s1[bl][r] = fast_exp2(fmaf(s1[bl][r], c, -m1));
            ps0 += s0[bl][r];
            ps1 += s1[bl][r];
          }
      };
      bool need_max = !ready;
      if (ready && full) {
        products();
        fast();
        need_max = __builtin_amdgcn_ballot_w64(fmaxf(ps0, ps1) > kSlackPow) != 0;
        if (need_max) products();
      } else {
        scores();
        if (!need_max) {
          fast();
          need_max = __builtin_amdgcn_ballot_w64(fmaxf(ps0, ps1) > kSlackPow) != 0;
          if (need_max) scores();
        }
      }
      if (need_max) {
        float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
          mx0 = fmaxf(mx0, fmaxf(fmaxf(s0[bl][0], s0[bl][1]), fmaxf(s0[bl][2], s0[bl][3])));
          mx1 = fmaxf(mx1, fmaxf(fmaxf(s1[bl][0], s1[bl][1]), fmaxf(s1[bl][2], s1[bl][3])));
        }
        mx0 *= c;  // this lane's maxima: a row's maximum exceeds a bound iff one of
        mx1 *= c;  // its 4 lanes does, so the row maximum is needed only to rescale
        if (__builtin_amdgcn_ballot_w64(mx0 > m0 + kSlack) != 0) {
          const float mn = fmaxf(m0, quad_max(mx0));
          const float al = (m0 == -INFINITY) ? 0.f : fast_exp2(m0 - mn);
          l0 *= al;
#pragma unroll
          for (int b = 0; b < 8; ++b) o0[b] *= al;
          m0 = mn;
        }
        if (__builtin_amdgcn_ballot_w64(mx1 > m1 + kSlack) != 0) {
          const float mn = fmaxf(m1, quad_max(mx1));
          const float al = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - mn);
          l1 *= al;
#pragma unroll
          for (int b = 0; b < 8; ++b) o1[b] *= al;
          m1 = mn;
        }
        // rows that have seen no visible key yet keep reference -inf: exponentiate
        // against 0 so masked scores give exactly 0
        const float e0 = (m0 == -INFINITY) ? 0.f : m0;
        const float e1 = (m1 == -INFINITY) ? 0.f : m1;
        ps0 = 0.f;
        ps1 = 0.f;
#pragma unroll
        for (int bl = 0; bl < 4; ++bl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s0[bl][r] = fast_exp2(fmaf(s0[bl][r], c, -e0));
            s1[bl][r] = fast_exp2(fmaf(s1[bl][r], c, -e1));
            ps0 += s0[bl][r];
            ps1 += s1[bl][r];
          }
        ready = __builtin_amdgcn_ballot_w64(m0 == -INFINITY || m1 == -INFINITY) == 0;
      }
      bf16x8 pa[2], pb[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        pa[p] = pack_pair(s0[2 * p], s0[2 * p + 1]);
        pb[p] = pack_pair(s1[2 * p], s1[2 * p + 1]);
      }
      l0 += ps0;
      l1 += ps1;
      // ---- O^T += V^T P^T ----
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int off = vo + 32 * kVPitch * p + vblock_bytes(b);
          const bf16x4 lo4 = tr_read(vbuf, off);
          const bf16x4 hi4 = tr_read(vbuf, off + 4 * kVPitch);
          const bf16x8 av = (bf16x8){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          o0[b] = mfma32(av, pa[p], o0[b]);
          o1[b] = mfma32(av, pb[p], o1[b]);
        }
      }
    }

    __builtin_amdgcn_s_setprio(0);
  }
    if (st + 1 < nstages) commit(smem + ((st + 1) & 1) * kBuf);
    __syncthreads();  // the next buffer is written; this one is no longer read
  }

  // ---- epilogue ----
  l0 = quad_sum(l0);
  l1 = quad_sum(l1);
  if (qi < N) {
    bf16* out = static_cast<bf16*>(a.out) + ((size_t)qi * Hq + h0) * D;
    const float vmul = FP8 ? a.v_scale : 1.f;
    store_row_tr(out, g, o0, __builtin_amdgcn_rcpf(l0) * vmul);
    store_row_tr(out + D, g, o1, __builtin_amdgcn_rcpf(l1) * vmul);
    if (a.lse != nullptr && g == 0) {
      float* l = a.lse + (size_t)qi * Hq + h0;
      l[0] = (m0 + fast_log2(l0)) * kLn2;
      l[1] = (m1 + fast_log2(l1)) * kLn2;
    }
  }
}

}  // namespace

bool online_mfma_supported(const PrefillArgs& a, bool bf16_io) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return bf16_io && a.head_dim == 128 && G % kHG == 0 && a.window >= 1;
}

hipError_t launch_online_mfma(const PrefillArgs& a, hipStream_t s) {
  const long ntiles = (a.total_tokens + kQT - 1) / kQT;
  const long total = ntiles * (a.num_q_heads / kHG);
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (a.kv_fp8)
    hipLaunchKernelGGL(ga_chunk_kernel<true>, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(ga_chunk_kernel<false>, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace swa
