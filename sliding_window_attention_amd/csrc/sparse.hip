// Token-level sparse attention with a forced recent window (the HySparse2 selection of
// the MiMo-V3 / HySparse2 report: the full-attention layer's scores pick the top k
// tokens -- 1024 there -- and the most recent 128 tokens are always kept; the sparse
// layers attend to that set over the shared KV cache).
//
//  * topk_select_kernel: one workgroup per (sequence, KV head) row of scores.  The
//    candidates are the positions older than the recent window.  A radix select over
//    an order-preserving 32-bit key finds the k-th largest score (histogram passes over
//    digits of 12, 10 and 10 bits -- the first digit takes mantissa bits too, so scores
//    of one binade do not pile onto a few bins; the first pass reads the row with
//    16-byte loads and keeps the keys in LDS for the others when the row has at most
//    32768 candidates); one ordered pass then
//    writes the chosen positions in increasing order:
//    every score above the threshold, and the lowest positions among those equal to
//    it, so the result is exact and deterministic (no floating point decides a rank).
//  * sparse_decode_kernel: one workgroup per (sequence, head octet); the key list
//    (selected positions, then the recent window) is staged in LDS, and the wavefronts
//    (4, or 8 for an FP8 cache on a grid of at most one workgroup per CU) take 32-key
//    chunks in turn: K rows gathered straight into MFMA A
//    operands, S^T = K Q^T for the octet's 8 heads, an online softmax per head, V rows
//    transposed in registers for O^T += V^T P^T.  The wavefronts' partial results are
//    merged exactly through LDS, with the sink in the denominator.  MTP verify (T = 2):
//    the second token's heads take the query columns the single token leaves empty, and
//    each column masks the keys its token does not see.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace swa {
namespace {

using namespace tile;

// ---------------------------------------------------------------------------
// top-k selection
// ---------------------------------------------------------------------------

constexpr int kSelThreads = 1024;  // 16 wavefronts

// Larger float -> larger key; equal floats -> equal keys (-0 takes the key of +0, so
// the two zeros tie and the lower position wins between them); NaN below every number.
// The scores are read as their 32-bit patterns: the device code is built without NaN
// semantics, under which a test on a float value (even through its bits) may be folded
// away.
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0u;
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the workgroup (one value per thread); `tmp` holds one slot
// per wavefront.  Returns the inclusive sum; *total receives the workgroup's total.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t x, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int v = 0; v < kSelThreads / 64; ++v) {
    const uint32_t t = tmp[v];
    before += v < w ? t : 0u;
    all += t;
  }
  __syncthreads();  // tmp may be reused by the caller's next scan
  *total = all;
  return x + before;
}

constexpr int kKeyCache = 32768;  // candidates whose keys are kept in LDS (128 KB)
constexpr int kBins0 = 4096;       // first digit: bits 31..20 (sign, exponent, 3 mantissa bits)
constexpr int kBins = 1024;        // next digits: bits 19..10 and 9..0
constexpr int kList = kBins0 - kBins;  // keys of the threshold's first-digit bin kept after pass 0
constexpr int kPerWave = kList / (kSelThreads / 64);  // the part of the list each wavefront fills

// The digit holding the rem-th largest of the keys counted in hist[0, nb): thread t owns
// the nb / 1024 bins just below the top t * per (descending), and an inclusive scan over
// threads counts the keys at or above each thread's lowest bin; exactly one thread holds
// the rem-th.  After the closing barrier pick[0] is the digit and pick[1] how many keys
// with that digit are still to be taken.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, int nb, int rem, uint32_t* tmp,
                                           uint32_t* pick) {
  const int per = nb / kSelThreads;  // 4 or 1
  const int top = nb - 1 - (int)threadIdx.x * per;
  uint32_t mine = 0;
  for (int e = 0; e < per; ++e) mine += hist[top - e];
  uint32_t tot;
  const uint32_t incl = block_inclusive_scan(mine, tmp, &tot);
  uint32_t acc = incl - mine;  // keys in bins above this thread's
  if (acc < (uint32_t)rem && (uint32_t)rem <= incl) {
    int d = top;
    for (int e = 0; e < per; ++e, --d) {
      const uint32_t hv = hist[d];
      if (acc + hv >= (uint32_t)rem) break;
      acc += hv;
    }
    pick[0] = (uint32_t)d;
    pick[1] = (uint32_t)rem - acc;
  }
  __syncthreads();
}

// The ordered pass: candidate j is chosen when its key is above the threshold T, or equal
// to it and among the first `rem` such positions; its output slot is (# above T before j)
// + min(# equal to T before j, rem).  Each thread takes P consecutive candidates per chunk
// of 1024 * P (keys past ncand are read but never counted).
template <int P, typename KeysAt>
__device__ __forceinline__ void write_ordered(KeysAt keys_at, int ncand, uint32_t T, uint32_t rem, int32_t* out,
                                              uint32_t* tmp) {
  uint32_t gt_run = 0, eq_run = 0;
  for (int c0 = 0; c0 < ncand; c0 += kSelThreads * P) {
    const int j0 = c0 + (int)threadIdx.x * P;
    uint32_t key[P];
    keys_at(j0, key);
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const bool ok = j0 + e < ncand;
      ngt += (ok && key[e] > T) ? 1u : 0u;
      neq += (ok && key[e] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t incl = block_inclusive_scan((ngt << 16) | neq, tmp, &tot);
    if (ngt + neq != 0) {
      uint32_t gt_b = gt_run + ((incl >> 16) - ngt), eq_b = eq_run + ((incl & 0xffffu) - neq);
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const int j = j0 + e;
        if (j < ncand && key[e] >= T) {
          if (key[e] > T) {
            out[gt_b + min(eq_b, rem)] = j;
            ++gt_b;
          } else {
            if (eq_b < rem) out[gt_b + eq_b] = j;
            ++eq_b;
          }
        }
      }
    }
    gt_run += tot >> 16;
    eq_run += tot & 0xffffu;
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t cache[kKeyCache];  // the row's keys when it fits
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins0];  // histograms; then also the key list
  __shared__ uint32_t tmp[kSelThreads / 64];
  __shared__ uint32_t pick[2];
  __shared__ uint32_t wcount[kSelThreads / 64];  // keys of the threshold's bin found per wavefront
  const int row = blockIdx.x;  // sequence * Hkv + KV head
  const int b = row / a.num_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  int L = a.lengths[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int ncand = L - a.recent > 0 ? L - a.recent : 0;
  const int K = a.k;
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(a.scores) + (size_t)row * a.max_len;
  int32_t* out = a.indices + (size_t)row * K;
  if (ncand <= K || K == 0) {  // every candidate is chosen, or none is asked for
    for (int x = tid; x < K; x += kSelThreads) out[x] = x < ncand ? x : -1;
    if (tid == 0) a.counts[row] = ncand < K ? ncand : K;
    return;
  }

  if (ncand > kKeyCache) {
    // ---- long rows: three histogram passes straight from memory, then the ordered pass ----
    uint32_t prefix = 0, mask = 0;
    int rem = K;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
      const int nb = pass == 0 ? kBins0 : kBins;
      const uint32_t dmask = (uint32_t)nb - 1u;
      for (int x = tid; x < nb; x += kSelThreads) hist[x] = 0;
      __syncthreads();
      for (int j0 = 0; j0 < ncand; j0 += 4 * kSelThreads) {
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + e * kSelThreads + tid;
          u[e] = j < ncand ? order_key(sc[j]) : 0u;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + e * kSelThreads + tid;
          if (j < ncand && (u[e] & mask) == prefix) atomicAdd(&hist[(u[e] >> shift) & dmask], 1u);
        }
      }
      __syncthreads();
      pick_digit(hist, nb, rem, tmp, pick);
      prefix |= pick[0] << shift;
      mask |= dmask << shift;
      rem = (int)pick[1];
      __syncthreads();  // pick and hist are rewritten by the next pass
    }
    write_ordered<8>([&](int j0, uint32_t (&k)[8]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) k[e] = j0 + e < ncand ? order_key(sc[j0 + e]) : 0u;
    }, ncand, prefix, (uint32_t)rem, out, tmp);
    if (tid == 0) a.counts[row] = K;
    return;
  }

  // ---- pass 0: read the row once (16-byte loads, four in flight per thread), keep its
  // keys in LDS and histogram their first digit ----
  for (int x = tid; x < kBins0; x += kSelThreads) hist[x] = 0;
  __syncthreads();
  {
    const int head = (int)((4 - (((uintptr_t)sc >> 2) & 3)) & 3);  // scalar head where the row is unaligned
    const int h = head < ncand ? head : ncand;
    for (int j = tid; j < h; j += kSelThreads) {
      const uint32_t u = order_key(sc[j]);
      cache[j] = u;
      atomicAdd(&hist[u >> 20], 1u);
    }
    const int nvec = (ncand - h) >> 2;
    const u32x4* v4 = reinterpret_cast<const u32x4*>(sc + h);
    for (int x0 = 0; x0 < nvec; x0 += 4 * kSelThreads) {
      u32x4 ld[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = x0 + e * kSelThreads + tid;
        ld[e] = v4[x < nvec ? x : 0];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = x0 + e * kSelThreads + tid;
        if (x < nvec) {
          u32x4 k4;
#pragma unroll
          for (int c = 0; c < 4; ++c) k4[c] = order_key(ld[e][c]);
          if (h == 0) {
            reinterpret_cast<u32x4*>(cache)[x] = k4;
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) cache[h + 4 * x + c] = k4[c];
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) atomicAdd(&hist[k4[c] >> 20], 1u);
        }
      }
    }
    for (int j = h + 4 * nvec + tid; j < ncand; j += kSelThreads) {
      const uint32_t u = order_key(sc[j]);
      cache[j] = u;
      atomicAdd(&hist[u >> 20], 1u);
    }
    // keys past the row up to a multiple of 32 read as 0 (the NaN key) in the later scans
    for (int j = ncand + tid; j < ((ncand + 31) & ~31); j += kSelThreads) cache[j] = 0u;
  }
  __syncthreads();
  pick_digit(hist, kBins0, K, tmp, pick);
  const uint32_t d0 = pick[0];
  int rem = (int)pick[1];
  uint32_t T = d0 << 20;
  const int nv = (ncand + 3) >> 2;
  const u32x4* cache4 = reinterpret_cast<const u32x4*>(cache);
  uint32_t* list = hist + kBins;
  if (d0 != 0) {  // (first digit 0 holds only the NaN key 0: then T = 0 exactly)
    __syncthreads();  // pick and hist are rewritten below
    // ---- pass 1: histogram the second digit of the keys in bin d0 and collect those
    // keys, each wavefront into its own part of the list (no shared counter) ----
    for (int x = tid; x < kBins; x += kSelThreads) hist[x] = 0;
    __syncthreads();
    const int wv = tid >> 6;
    uint32_t wn = 0;  // keys this wavefront has found (uniform over the wavefront)
    for (int x0 = 0; x0 < nv; x0 += kSelThreads) {
      const int x = x0 + tid;
      const u32x4 k4 = cache4[x < nv ? x : 0];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool m = x < nv && (k4[c] >> 20) == d0;
        const uint64_t bal = __ballot(m);
        if (m) {
          atomicAdd(&hist[(k4[c] >> 10) & (kBins - 1)], 1u);
          const uint32_t slot = wn + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          if (slot < (uint32_t)kPerWave) list[wv * kPerWave + slot] = k4[c];
        }
        wn += (uint32_t)__popcll(bal);
      }
    }
    if (lane == 0) wcount[wv] = wn;
    __syncthreads();
    pick_digit(hist, kBins, rem, tmp, pick);
    const uint32_t d1 = pick[0];
    rem = (int)pick[1];
    bool fits = true;
#pragma unroll
    for (int v = 0; v < kSelThreads / 64; ++v) fits = fits && wcount[v] <= (uint32_t)kPerWave;
    __syncthreads();
    // ---- pass 2: the third digit, over the collected keys (or the whole row when a
    // wavefront found more than its part of the list holds) ----
    for (int x = tid; x < kBins; x += kSelThreads) hist[x] = 0;
    __syncthreads();
    if (fits) {
      for (int e = tid; e < kList; e += kSelThreads) {
        const int v = e / kPerWave, idx = e - v * kPerWave;
        if ((uint32_t)idx < wcount[v]) {
          const uint32_t u = list[e];
          if (((u >> 10) & (kBins - 1)) == d1) atomicAdd(&hist[u & (kBins - 1)], 1u);
        }
      }
    } else {
      const uint32_t want = (d0 << 10) | d1;
      for (int x = tid; x < nv; x += kSelThreads) {
        const u32x4 k4 = cache4[x];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if ((k4[c] >> 10) == want) atomicAdd(&hist[k4[c] & (kBins - 1)], 1u);
      }
    }
    __syncthreads();
    pick_digit(hist, kBins, rem, tmp, pick);
    T = (d0 << 20) | (d1 << 10) | pick[0];
    rem = (int)pick[1];
  }

  // ---- ordered pass over the cached keys: 32 consecutive candidates per thread, one
  // chunk.  A mask marks the keys at or above T (the padding past ncand is masked off);
  // the chosen ones, a few per thread, are then visited in increasing position ----
  {
    const int j0 = tid * 32;
    uint32_t gem = 0, ngt = 0;
    if (j0 < ncand) {
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const u32x4 k4 = cache4[(j0 >> 2) + v];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          gem |= (k4[c] >= T ? 1u : 0u) << (4 * v + c);
          ngt += k4[c] > T ? 1u : 0u;  // the zero padding is never above T
        }
      }
      if (ncand - j0 < 32) gem &= (1u << (ncand - j0)) - 1u;
    }
    const uint32_t neq = (uint32_t)__builtin_popcount(gem) - ngt;
    uint32_t tot;
    const uint32_t incl = block_inclusive_scan((ngt << 16) | neq, tmp, &tot);
    uint32_t gt_b = (incl >> 16) - ngt, eq_b = (incl & 0xffffu) - neq;
    while (gem != 0) {
      const int e = __builtin_ctz(gem);
      gem &= gem - 1u;
      const int j = j0 + e;
      if (cache[j] > T) {
        out[gt_b + min(eq_b, (uint32_t)rem)] = j;
        ++gt_b;
      } else {
        if (eq_b < (uint32_t)rem) out[gt_b + eq_b] = j;
        ++eq_b;
      }
    }
  }
  if (tid == 0) a.counts[row] = K;
}

// ---------------------------------------------------------------------------
// sparse decode (bf16, head_dim 128, heads per KV head a multiple of 8)
// ---------------------------------------------------------------------------

constexpr int kHG = 8;                 // query heads per workgroup
constexpr int kMaxList = 8192;         // selected + recent keys staged in LDS
constexpr int kQPitch = 272;           // staged bf16 query row, padded
constexpr int kOPitch = D + 4;         // fp32 partial row, padded

template <int NW>
struct SparseSmem {
  int32_t keys[kMaxList];
  char q[16][kQPitch];                 // 8 query heads; columns 8..15 zero
  float m[NW][16], l[NW][16];
  float o[NW - 1][16][kOPitch];        // partial O of wavefronts 1 .. NW-1
};

// T queries per sequence (1, or 2 for an MTP verify): the 16 query columns are token
// c >> 3, head c & 7 (T = 1: columns 8..15 zero).  Query t (position p_t = L - T + t) sees
// the selected positions below its own recent window and the window
// max(0, p_t - recent + 1) .. p_t; the staged list holds the selection and the union of
// the T windows, and each column masks the rest.
// FP8: the caches hold E4M3 codes, gathered 8 bytes per operand and kept as codes until
// they are used (so the next chunk's loads are never waited for early); the K scale joins
// the logit multiplier and the V scale the output's 1 / z.
// NW wavefronts take the chunks in turn, each with one chunk in use and the next in
// flight.  With one workgroup per CU, the FP8 gather (one 128-byte row per key and
// operand) runs 8 wavefronts to keep twice the rows in flight; bf16 rows move twice the
// bytes per load and measured no faster with 8.
template <int T, bool FP8, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void sparse_decode_kernel(SparseArgs a) {
  __shared__ __attribute__((aligned(16))) SparseSmem<NW> sm;
  const int noct = a.num_q_heads / kHG;
  const int b = blockIdx.x / noct;
  const int oct = blockIdx.x - b * noct;
  const int h_base = oct * kHG;
  const int hkv = a.num_kv_heads;
  const int kvh = h_base / (a.num_q_heads / hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;

  int L = as_const(a.lengths)[b];
  L = L < T ? T : (L > a.max_len ? a.max_len : L);  // the T queries are the newest tokens
  int cnt = as_const(a.counts)[b * hkv + kvh];
  cnt = cnt < 0 ? 0 : (cnt > a.k ? a.k : cnt);
  const int rs = max(0, L - a.recent - (T - 1));  // first position of the windows' union
  const int nrec = L - rs;
  const int M = cnt + nrec;  // keys of the list (<= kMaxList: checked on the host)

  // ---- stage the key list and the 8 query rows ----
  const int32_t* sel = a.indices + ((size_t)b * hkv + kvh) * a.k;
  for (int m = tid; m < M; m += NW * 64) {
    int j;
    if (m < cnt) {
      j = sel[m];
      j = j < 0 ? 0 : (j >= L ? L - 1 : j);  // keeps every access in bounds
    } else {
      j = L - nrec + (m - cnt);
    }
    sm.keys[m] = j;
  }
  if (tid < 256) {
    const int r = tid >> 4, u = tid & 15;  // 16 rows x 16 units: token r >> 3, head r & 7
    u32x4 x = {0, 0, 0, 0};
    if ((r >> 3) < T)
      x = *reinterpret_cast<const u32x4*>(
          static_cast<const bf16*>(a.q) + (((size_t)b * T + (r >> 3)) * a.num_q_heads + h_base + (r & 7)) * D + 8 * u);
    *reinterpret_cast<u32x4*>(&sm.q[r][16 * u]) = x;
  }
  __syncthreads();
  // this lane's column i: token tq, its window's first position wlo, and cut, the
  // selected keys below that window (the selection is increasing, and only its last
  // T - 1 - tq entries can reach into the window)
  const int tq = i >> 3;
  const int pq = L - T + tq;
  const int wlo = pq - a.recent + 1;
  int cut = cnt;
  if constexpr (T > 1) {
    for (int z = 0; z < T - 1 - tq && cut > 0 && sm.keys[cut - 1] >= wlo; ++z) --cut;
  }
  // key m of the list is seen by this lane's column
  auto visible = [&](int m) {
    if (m < cnt) return m < cut;
    const int pos = rs + (m - cnt);
    return pos >= wlo && pos <= pq;
  };

  using CacheT = typename std::conditional<FP8, uint8_t, bf16>::type;
  using Raw = typename std::conditional<FP8, u32x2, bf16x8>::type;  // one operand as gathered
  const CacheT* kc = static_cast<const CacheT*>(a.k_cache) + ((size_t)b * hkv + kvh) * a.max_len * D;
  const CacheT* vc = static_cast<const CacheT*>(a.v_cache) + ((size_t)b * hkv + kvh) * a.max_len * D;
  auto op = [](Raw r) -> bf16x8 {
    if constexpr (FP8) return e4m3x8_to_bf16x8(r);
    else return r;
  };
  auto gather = [](const CacheT* p) -> Raw {
    // each selected row is gathered once per step and not again until the layer's next
    // step: non-temporal loads, as for the dense decode's ring (measured faster for bf16)
    if constexpr (FP8) return *reinterpret_cast<const u32x2*>(p);
    else return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  };
  const float c = a.scale * kLog2e * (FP8 ? a.k_scale : 1.f);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // K operand of chunk cc: the 8 head-dim elements of unit kunit(cc) (8 elements per
  // unit): unit 4 cc + g, the chunk's 32 dims in order; for FP8 codes unit
  // 2 g + 8 (cc >> 1) + (cc & 1), so that chunks 2h and 2h + 1 of a lane are adjacent
  // codes and one 16-byte load brings both, the four lanes of a row covering 64
  // contiguous bytes.  The query operands take the same units; the contraction runs over
  // all 128 dims either way.
  auto kunit = [&](int cc) { return FP8 ? 2 * g + 8 * (cc >> 1) + (cc & 1) : 4 * cc + g; };
  bf16x8 qop[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) qop[cc] = *reinterpret_cast<const bf16x8*>(&sm.q[i][16 * kunit(cc)]);

  // operands of one 32-key chunk: K rows pair_row(i, s) (A operand, head-dim unit kunit(cc)),
  // V rows 8g + e (head-dim 8i .. 8i+7); keys past the list read the last key (their
  // weight is zero)
  const int nchunks = (M + 31) >> 5;
  auto load_chunk = [&](int ch, Raw (&kf)[2][4], Raw (&vr)[8]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int m = 32 * ch + pair_row(i, s);
      const int j = sm.keys[m < M ? m : M - 1];
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 c16 = *reinterpret_cast<const u32x4*>(kc + (size_t)j * D + 64 * h + 16 * g);
          kf[s][2 * h] = (u32x2){c16[0], c16[1]};
          kf[s][2 * h + 1] = (u32x2){c16[2], c16[3]};
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) kf[s][cc] = gather(kc + (size_t)j * D + 32 * cc + 8 * g);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = 32 * ch + 8 * g + e;
      const int j = sm.keys[m < M ? m : M - 1];
      vr[e] = gather(vc + (size_t)j * D + 8 * i);
    }
  };

  float mcol = -INFINITY, lcol = 0.f;  // running max (log2 units) and sum of column i
  f32x4 o[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) o[bb] = zero4;
  Raw kf[2][4], vr[8], nkf[2][4], nvr[8];
  if (w < nchunks) load_chunk(w, kf, vr);
  for (int ch = w; ch < nchunks; ch += NW) {
    const bool more = ch + NW < nchunks;
    if (more) load_chunk(ch + NW, nkf, nvr);
    f32x4 s2[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      s2[s] = zero4;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) s2[s] = mfma32(op(kf[s][cc]), qop[cc], s2[s]);
    }
    // lane (i, g) holds keys 8g + 4s + r of the chunk for column i
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 32 * ch + 8 * g + 4 * s + r;
        bool ok = m < M;
        if constexpr (T > 1) ok = ok && visible(m);
        s2[s][r] = ok ? s2[s][r] * c : -INFINITY;
        mx = fmaxf(mx, s2[s][r]);
      }
    // T = 1: finite, the chunk's first key is valid; T > 1: a column may have seen no key
    // yet (its reference is then 0 and every weight 0)
    const float mnew = fmaxf(mcol, quad_max(mx));
    const float mref = (T > 1 && mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2(mcol - mref);
    float ps = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s2[s][r] = fast_exp2(s2[s][r] - mref);
        ps += s2[s][r];
      }
    lcol = lcol * alpha + quad_sum(ps);
    mcol = mnew;
    const bf16x8 pp = pack_pair(s2[0], s2[1]);
    bf16x8 vb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vb[e] = op(vr[e]);
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      o[bb] *= alpha;
      o[bb] = mfma32(column8(vb, bb), pp, o[bb]);
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) kf[s][cc] = nkf[s][cc];
#pragma unroll
      for (int e = 0; e < 8; ++e) vr[e] = nvr[e];
    }
  }

  // ---- exact merge of the wavefronts' partials (lane (i, g): column i,
  // head-dim 32g + 8r + bb in register r of block bb) ----
  if (g == 0) {
    sm.m[w][i] = mcol;
    sm.l[w][i] = lcol;
  }
  if (w > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* row = &sm.o[w - 1][i][32 * g + 8 * r];
      *reinterpret_cast<f32x4*>(row) = (f32x4){o[0][r], o[1][r], o[2][r], o[3][r]};
      *reinterpret_cast<f32x4*>(row + 4) = (f32x4){o[4][r], o[5][r], o[6][r], o[7][r]};
    }
  }
  __syncthreads();
  if (w != 0 || i >= kHG * T) return;
  const int h = h_base + (i & 7);
  const size_t orow = ((size_t)b * T + tq) * a.num_q_heads + h;
  const float sink2 = a.sinks ? as_const(a.sinks)[h] * kLog2e : -INFINITY;
  float mt = sink2;
#pragma unroll
  for (int v = 0; v < NW; ++v) mt = fmaxf(mt, sm.m[v][i]);
  float z = a.sinks ? fast_exp2(sink2 - mt) : 0.f;
  float sc[NW];
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    sc[v] = fast_exp2(sm.m[v][i] - mt);  // 0 for a wavefront that had no chunk
    z += sm.l[v][i] * sc[v];
  }
  const float inv = (FP8 ? a.v_scale : 1.f) / z;
  bf16* out = static_cast<bf16*>(a.out) + orow * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float acc[8];
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) acc[bb] = o[bb][r] * sc[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) {
      const float* row = &sm.o[v - 1][i][32 * g + 8 * r];
      const f32x4 lo = *reinterpret_cast<const f32x4*>(row);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(row + 4);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        acc[bb] = fmaf(lo[bb], sc[v], acc[bb]);
        acc[bb + 4] = fmaf(hi[bb], sc[v], acc[bb + 4]);
      }
    }
    bf16x8 v8;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) v8[bb] = (bf16)(acc[bb] * inv);
    *reinterpret_cast<bf16x8*>(out + 32 * g + 8 * r) = v8;
  }
  if (a.lse != nullptr && g == 0) a.lse[orow] = (mt + fast_log2(z)) * kLn2;
}

}  // namespace

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
  const long rows = (long)a.batch * a.num_kv_heads;
  if (rows == 0) return hipSuccess;
  if (rows > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

bool sparse_mfma_supported(const SparseArgs& a, bool bf16_io) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return bf16_io && a.head_dim == 128 && G % kHG == 0 && a.t_new >= 1 && a.t_new <= 2 &&
         (long)a.k + a.recent + a.t_new - 1 <= kMaxList;
}

constexpr long kSparseWideGrid = 256;  // workgroups up to which each has a CU of its own

template <bool FP8, int NW>
hipError_t launch_sparse_nw(const SparseArgs& a, unsigned blocks, hipStream_t s) {
  const dim3 grid(blocks), block(NW * 64);
  if (a.t_new == 2) hipLaunchKernelGGL((sparse_decode_kernel<2, FP8, NW>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((sparse_decode_kernel<1, FP8, NW>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_decode(const SparseArgs& a, bool bf16_io, hipStream_t s) {
  if (!sparse_mfma_supported(a, bf16_io)) return launch_generic_sparse(a, bf16_io, s);
  const long blocks = (long)a.batch * (a.num_q_heads / kHG);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (!a.kv_fp8) return launch_sparse_nw<false, 4>(a, (unsigned)blocks, s);
  // FP8 with up to one workgroup per CU: 8 wavefronts each; beyond that 4, two
  // workgroups sharing a CU
  if (blocks <= kSparseWideGrid) return launch_sparse_nw<true, 8>(a, (unsigned)blocks, s);
  return launch_sparse_nw<true, 4>(a, (unsigned)blocks, s);
}

}  // namespace swa
