// Matrix-core prefill for sliding windows of at most 128 keys with a per-head
// sink (MiMo-V2-Flash Technical Report digest, sections 2.2.1 and 2.2.2).
//
// Work decomposition: a workgroup of 4 wavefronts owns 16 consecutive query
// tokens of the packed stream and the 8 query heads that share one KV head (GQA),
// so every K/V byte staged in LDS serves 8 heads; wavefront w owns heads 2w and
// 2w+1 (two 16-query MFMA tiles sharing every K read).  Tiles may straddle
// sequence boundaries: each query row masks keys before its own sequence start,
// so the grid depends only on the total token count and needs no host tile map.
//
// The union of the 16 rows' windows is at most 143 keys, so the whole band (9
// blocks of 16 keys) is scored in registers and the softmax is exact in one pass
// (no online rescaling), the sink entering as the initial maximum candidate and
// as exp(sink - m) in the denominator.  Workgroups are persistent and keep the
// band in an LDS ring across consecutive tiles, walking their run of tiles upwards
// or (odd runs) downwards, so that neighbouring runs read the rows they share at the
// same time on the same XCD.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace swa {
namespace {

using namespace tile;

constexpr int kQT = 16;        // query tokens per workgroup
constexpr int kHG = 8;         // query heads per workgroup
constexpr int kThreads = 256;  // 4 wavefronts x 2 heads

namespace ring {

constexpr int kSlots = 9;                    // ring slots of 16 keys
constexpr int kRows = 16 * kSlots;           // 144 keys
constexpr int kKPlane = kRows * 64;          // bytes of one 32-element chunk plane
constexpr int kKBytes = 4 * kKPlane;         // 36864
constexpr int kVBytes = kRows * kVPitch;     // 38016

__device__ __forceinline__ int mod9(int x) { x %= kSlots; return x < 0 ? x + kSlots : x; }

// Eight K/V elements starting at element `elem`, as loaded: bf16 in 16 bytes, or (FP8)
// eight E4M3 codes in 8 bytes, widened to bf16 only when written to the ring (widen),
// so that no conversion waits on a load where it is issued.
template <bool FP8>
using KvRaw = typename std::conditional<FP8, u32x2, u32x4>::type;
template <bool FP8>
__device__ __forceinline__ KvRaw<FP8> load_kv(const void* base, size_t elem) {
  if constexpr (FP8) return *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(base) + elem);
  else return *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(base) + elem);
}
template <bool FP8>
__device__ __forceinline__ u32x4 widen(KvRaw<FP8> x) {
  if constexpr (FP8) return __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(x));  // exact
  else return x;
}

// Load all 144 rows of a tile whose first key is kbase into the ring.
template <bool FP8>
__device__ __attribute__((noinline)) void fill(char* ks, char* vs, const void* __restrict__ k,
                                     const void* __restrict__ v, int kbase, int N, int hkv, int kvh) {
  const int t = threadIdx.x;
  const int r = t >> 4, u = t & 15;
  const int kblock0 = mod9(kbase >> 4);
  KvRaw<FP8> kr[kSlots], vr[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int key = kbase + 16 * j + r;
    kr[j] = KvRaw<FP8>{};
    vr[j] = KvRaw<FP8>{};
    if (key >= 0 && key < N) {
      const size_t off = ((size_t)key * hkv + kvh) * D + u * 8;
      kr[j] = load_kv<FP8>(k, off);
      vr[j] = load_kv<FP8>(v, off);
    }
  }
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int phys = 16 * mod9(kblock0 + j) + r;
    put_k(ks, kKPlane, phys, kbase + 16 * j + r, u, widen<FP8>(kr[j]));
    put_v(vs, phys, u, widen<FP8>(vr[j]));
  }
}

}  // namespace ring

// Index of the sequence holding packed token q: the largest s < num_seqs with
// cu[s] <= q (wave-uniform binary search on scalar loads).
__device__ __forceinline__ int find_seq(const_ptr<int32_t> cu, int num_seqs, int q) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= q) lo = mid; else hi = mid;
  }
  return lo;
}

// FP8: K and V arrive as E4M3 codes and are widened to bf16 (exactly) on their way into
// the ring; the K scale joins the logit multiplier and the V scale the output's 1/Z.
template <bool FP8>
__global__ __launch_bounds__(kThreads, 2) void swa_ring_kernel(PrefillArgs a, int items_per_wg) {
  using namespace ring;
  __shared__ __attribute__((aligned(16))) char smem[kKBytes + kVBytes];
  char* ks = smem;
  char* vs = smem + kKBytes;

  const int N = a.total_tokens, Hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int ntiles = (N + kQT - 1) / kQT;
  const int total = ntiles * (Hq / kHG);
  // Runs of neighbouring workgroups share the K/V rows of the window that straddles
  // their boundary.  Workgroups are dealt to the 8 XCDs round-robin; the logical run
  // index gives each XCD a contiguous range of runs, and odd runs walk their tiles
  // downwards, so that the two runs of every boundary read its shared rows at the same
  // time (both at their start, or both at their end) through one L2.
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, perx = nwg >> 3, remx = nwg & 7;
  const int run = xcd * perx + min(xcd, remx) + (bid >> 3);
  const bool down = run & 1;
  const int item_lo = run * items_per_wg;
  const int item_hi = min(item_lo + items_per_wg, total);
  if (item_lo >= item_hi) return;
  int item = down ? item_hi - 1 : item_lo;  // next unprocessed item
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int t = threadIdx.x;
  const int G = Hq / hkv;
  const int S = a.num_seqs;
  const const_ptr<int32_t> cu = as_const(a.cu_seqlens);
  const const_ptr<float> sinks = as_const(a.sinks);
  const void* kp = a.k;
  const void* vp = a.v;
  const bf16* qp = static_cast<const bf16*>(a.q);
  const float c = a.scale * kLog2e * (FP8 ? a.k_scale : 1.f);
  const float vmul = FP8 ? a.v_scale : 1.f;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // Lane-constant parts of the LDS addresses.
  const int pr0 = pair_row(i, 0), pr1 = pair_row(i, 1), p8 = pi8(i);
  const int vrow = 8 * (g & 1) + (i >> 2);                  // row within a 16-key block, pairs
  const int vrow8 = 8 * (g & 1) + 4 * (g >> 1) + (i >> 2);  // the single diagonal block
  const int vquad = 2 * (64 * ((i & 3) >> 1) + 16 * (i & 1));  // bytes of qoff(i & 3, 0)

  // Q of one tile: lane (i, g) holds head-dim 32cc + 8g .. +8 of query q0 + i.
  bf16x8 qa[4], qb[4];
  auto load_q_tile = [&](int q0n, int octn) {
    const int qi = q0n + i;
    const bool ok = qi < N;
    const size_t r0 = ((size_t)qi * Hq + octn * kHG + 2 * w) * D + 8 * g;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      qa[cc] = ok ? *reinterpret_cast<const bf16x8*>(qp + r0 + 32 * cc) : zero8();
      qb[cc] = ok ? *reinterpret_cast<const bf16x8*>(qp + r0 + D + 32 * cc) : zero8();
    }
  };

  // Outer loop: runs of consecutive tiles of one head octet (the ring is filled
  // once per run).  Inner loop: one tile per iteration, the ring advancing by
  // one 16-key block.
  while (down ? item >= item_lo : item < item_hi) {
    item = __builtin_amdgcn_readfirstlane(item);
    const int oct = item / ntiles;
    const int tile0 = item - oct * ntiles;  // first tile of this run
    const int run_len = __builtin_amdgcn_readfirstlane(
        down ? item - max(item_lo, oct * ntiles) + 1 : min(item_hi, (oct + 1) * ntiles) - item);
    const int dir = down ? -1 : 1;
    int seq = find_seq(cu, S, tile0 * kQT);  // sequence of the tile's first query
    const int kvh = (oct * kHG) / G;
    __syncthreads();  // the previous run is done with the ring
    fill<FP8>(ks, vs, kp, vp, tile0 * kQT - 128, N, hkv, kvh);
    load_q_tile(tile0 * kQT, oct);
    // Drain the run prologue's loads so that, at the loop head, no vector load
    // is outstanding on any path: each iteration waits for its prefetches
    // before it issues its stores.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ring slot of the tile's oldest block: (kbase / 16) mod 9 with kbase = 16 tile
    // - 128, i.e. (tile + 1) mod 9; it moves by one slot per tile, with the walk
    int kblock0 = __builtin_amdgcn_readfirstlane((tile0 + 1) % kSlots);
    for (int k = 0; k < run_len; ++k) {
      const int tile = tile0 + dir * k;
      const int q0 = tile * kQT;
      const int kbase = q0 - 128;  // ring block j holds keys kbase + 16j ..
      const int par = tile & 1;    // (kbase / 16) & 1
      // slot of ring block j, and its byte offsets in a K plane and in V
      auto slot = [&](int j) { return kblock0 + j - (kblock0 + j >= kSlots ? kSlots : 0); };
      int sk[kSlots];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) sk[j] = 16 * 64 * slot(j);
      const int h0 = oct * kHG + 2 * w;

      // ---- first visible key of each row: window and own-sequence start ----
      if (down) {
        while (seq > 0 && cu[seq] > q0) --seq;
      } else {
        while (seq + 1 < S && cu[seq + 1] <= q0) ++seq;
      }
      const int qi = q0 + i;
      int start = cu[seq];
      for (int s2 = seq + 1; s2 < S && cu[s2] < q0 + kQT; ++s2)  // boundaries inside the tile
        start = qi >= cu[s2] ? cu[s2] : start;
      const long lw = (long)qi - a.window + 1;
      const int lo = lw > start ? (int)lw : start;
      const int rel_lo = lo - kbase;
      const int rel_hi = qi - kbase;
      // rows are ordered, so lane 15 bounds the tile's window starts (wave-uniform);
      // blocks and pairs before every row's window are not skipped: the mask gives
      // their keys weight 0, and skipping would put a branch between the blocks'
      // operand reads
      const int lo_max = __builtin_amdgcn_readlane(rel_lo, 15);
      const unsigned span = (unsigned)(rel_hi - rel_lo);  // key kr is visible iff kr - rel_lo <= span
      const float sink0 = a.sinks ? sinks[h0] * kLog2e : -INFINITY;
      const float sink1 = a.sinks ? sinks[h0 + 1] * kLog2e : -INFINITY;

      // ---- S^T = K Q^T over 9 blocks of 16 keys ----
      f32x4 s0[9], s1[9];
      {
        const int ko0 = pr0 * 64 + 16 * (g ^ kswz(16 * par + pr0)) - (i >= 8 ? 16 * 64 : 0);
        const int ko1 = pr1 * 64 + 16 * (g ^ kswz(16 * par + pr1)) - (i >= 8 ? 16 * 64 : 0);
        const int ko8 = p8 * 64 + 16 * (g ^ kswz(16 * par + p8));
#pragma unroll
        for (int bl = 0; bl < 9; ++bl) {
          int off;
          if (bl < 8) {
            const int p = bl >> 1;
            off = (i >= 8 ? sk[2 * p + 1] : sk[2 * p]) + ((bl & 1) ? ko1 : ko0);
          } else {
            off = sk[8] + ko8;
          }
          bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + off);
          s0[bl] = mfma32(kf, qa[0], zero4);
          s1[bl] = mfma32(kf, qb[0], zero4);
#pragma unroll
          for (int cc = 1; cc < 4; ++cc) {
            kf = *reinterpret_cast<const bf16x8*>(ks + cc * kKPlane + off);
            s0[bl] = mfma32(kf, qa[cc], s0[bl]);
            s1[bl] = mfma32(kf, qb[cc], s1[bl]);
          }
        }
      }

      // ---- prefetch for the next tile: the 16 K/V rows it adds to the ring (its newest
      // block walking up, its oldest walking down) and its Q ----
      const bool has_next = k + 1 < run_len;
      KvRaw<FP8> pk{}, pv{};
      const int nkey = (down ? q0 - 144 : q0 + 16) + (t >> 4);
      if (has_next && nkey >= 0 && nkey < N) {
        const size_t off = ((size_t)nkey * hkv + kvh) * D + (t & 15) * 8;
        pk = load_kv<FP8>(kp, off);
        pv = load_kv<FP8>(vp, off);
      }
      if (has_next) load_q_tile(q0 + dir * kQT, oct);

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
            const int kr = bl < 8 ? 32 * (bl >> 1) + 8 * g + 4 * (bl & 1) + r
                                  : 128 + 8 * (g & 1) + 4 * (g >> 1) + r;
            const bool ok = (unsigned)(kr - rel_lo) <= span;
            s0[bl][r] = ok ? s0[bl][r] : -INFINITY;
            s1[bl][r] = ok ? s1[bl][r] : -INFINITY;
          }
        }
        mx0 = fmaxf(mx0, fmaxf(fmaxf(s0[bl][0], s0[bl][1]), fmaxf(s0[bl][2], s0[bl][3])));
        mx1 = fmaxf(mx1, fmaxf(fmaxf(s1[bl][0], s1[bl][1]), fmaxf(s1[bl][2], s1[bl][3])));
      }
      const float m0 = fmaxf(quad_max(mx0) * c, sink0);
      const float m1 = fmaxf(quad_max(mx1) * c, sink1);

      // ---- exponentiate, sum, pack P to bf16 (pairs of blocks feed one k=32 product) ----
      float l0 = 0.f, l1 = 0.f;
      bf16x8 pa[4], pb[4];
#pragma unroll
      for (int bl = 0; bl < 9; ++bl) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s0[bl][r] = fast_exp2(fmaf(s0[bl][r], c, -m0));
          s1[bl][r] = fast_exp2(fmaf(s1[bl][r], c, -m1));
          l0 += s0[bl][r];
          l1 += s1[bl][r];
        }
        if (bl & 1) {
          pa[bl >> 1] = pack_pair(s0[bl - 1], s0[bl]);
          pb[bl >> 1] = pack_pair(s1[bl - 1], s1[bl]);
        }
      }
      const bf16x4 pa8 = pack_quad(s0[8]), pb8 = pack_quad(s1[8]);
      const float z0 = quad_sum(l0) + fast_exp2(sink0 - m0);
      const float z1 = quad_sum(l1) + fast_exp2(sink1 - m1);

      // ---- O^T = V^T P^T: the single diagonal block first (initialises O), then pairs ----
      f32x4 o0[8], o1[8];
      {
        const int vb8 = 16 * slot(8) * kVPitch + vrow8 * kVPitch + vquad;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const bf16x4 av = tr_read(vs, vb8 + 2 * (32 * (b >> 2) + 4 * (b & 3)));
          o0[b] = mfma32_k16(av, pa8, zero4);
          o1[b] = mfma32_k16(av, pb8, zero4);
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // lane groups 0-1 read the pair's first 16-key block, groups 2-3 its second
        const int slot_a = 16 * slot(2 * p) * kVPitch;
        const int slot_b = 16 * slot(2 * p + 1) * kVPitch;
        const int vb = (g >= 2 ? slot_b : slot_a) + vrow * kVPitch + vquad;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int bo = 2 * (32 * (b >> 2) + 4 * (b & 3));
          const bf16x4 lo4 = tr_read(vs, vb + bo);
          const bf16x4 hi4 = tr_read(vs, vb + 4 * kVPitch + bo);
          const bf16x8 av = (bf16x8){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          o0[b] = mfma32(av, pa[p], o0[b]);
          o1[b] = mfma32(av, pb[p], o1[b]);
        }
      }

      // ---- ring update for the next tile.  Every load of this iteration is waited
      // for here, before this tile's stores are issued: loads and stores share one
      // completion counter, so a store issued ahead of a load's wait would make
      // that wait cover the store too. ----
      if (has_next) {
        __syncthreads();  // every wavefront is done with the block being replaced
        const int phys = 16 * slot(down ? 8 : 0) + (t >> 4);  // the block the next tile replaces
        put_k(ks, kKPlane, phys, nkey, t & 15, widen<FP8>(pk));
        put_v(vs, phys, t & 15, widen<FP8>(pv));
        __syncthreads();
      }
      kblock0 = down ? (kblock0 == 0 ? kSlots - 1 : kblock0 - 1) : (kblock0 == kSlots - 1 ? 0 : kblock0 + 1);

      // ---- epilogue: O and LSE of this tile ----
      // vmcnt(0) on every path (on the common one the ring update has already
      // waited): it tells the compiler that no prefetch load is outstanding past
      // this point, so the next tile need not wait at its head, where the wait
      // would also cover this tile's stores.
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      if (qi < N) {
        bf16* out = static_cast<bf16*>(a.out) + ((size_t)qi * Hq + h0) * D;
        store_row_tr(out, g, o0, __builtin_amdgcn_rcpf(z0) * vmul);
        store_row_tr(out + D, g, o1, __builtin_amdgcn_rcpf(z1) * vmul);
        if (a.lse != nullptr && g == 0) {
          float* l = a.lse + (size_t)qi * Hq + h0;
          l[0] = (m0 + fast_log2(z0)) * kLn2;
          l[1] = (m1 + fast_log2(z1)) * kLn2;
        }
      }
    }
    item += dir * run_len;  // next run
  }
}


}  // namespace

bool swa_window_mfma_supported(const PrefillArgs& a, bool bf16_io) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return bf16_io && a.head_dim == 128 && G % kHG == 0 && a.window >= 1 && a.window <= 128;
}

hipError_t launch_swa_window_mfma(const PrefillArgs& a, hipStream_t s) {
  const long ntiles = (a.total_tokens + kQT - 1) / kQT;
  const long total = ntiles * (a.num_q_heads / kHG);
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  // two resident workgroups per compute unit (LDS-bound), each walking a
  // contiguous run of tiles
  int cus = 0;
  hipError_t e = device_cu_count(&cus);
  if (e != hipSuccess) return e;
  const long slots = 2L * cus;
  const long per = (total + slots - 1) / slots;
  const long grid = (total + per - 1) / per;
  if (a.kv_fp8)
    hipLaunchKernelGGL(swa_ring_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, (int)per);
  else
    hipLaunchKernelGGL(swa_ring_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, (int)per);
  return hipGetLastError();
}


}  // namespace swa
