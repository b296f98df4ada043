// Matrix-core backward of the SWA-with-sink forward for windows of at most 128
// keys (bf16 I/O, head_dim 128, query heads per KV head a multiple of 8).
//
// Gradients (p_ij = exp(a_ij - lse_i) with a_ij the scaled logit and lse_i the
// forward's log-normaliser, sink included; the sink carries no value, MiMo-V2-Flash
// Technical Report digest, section 2.2.2):
//   dS_ij = p_ij (dO_i . v_j - delta_i),  delta_i = dO_i . O_i,
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i p_ij dO_i.
// Since lse is known, every score block is normalised on its own: no running max,
// no rescaling.  P and dS are rounded to bf16 as MFMA operands (fp32 accumulation).
//
// Two kernels, both deterministic (no atomics):
//  * bwd_dq_ring_kernel: the forward's decomposition -- a workgroup owns 16 query
//    tokens x 8 heads sharing one KV head (one head per wavefront), the 144-key band
//    sits in an LDS ring that advances by 16 keys per tile.  S^T = K Q^T and dP^T = V dO^T come out with
//    queries in columns, so dS^T feeds dQ^T = K^T dS^T straight from registers.  It
//    also forms delta of its rows as sum_j p_ij dP_ij over the row's keys, which is
//    dO . O for the exact O (O = sum_j p_ij v_j: the sink carries no value), so O is
//    not read; delta is written, with the sink's term, for the dk/dv kernel and the
//    sink gradient.
//  * bwd_dkdv_kernel: the transpose -- a workgroup owns 64 keys of one KV head (16
//    per wavefront) and walks the (head quad, query block) steps that see them, one
//    LDS-staged block of 16 tokens x 4 heads per step shared by the four wavefronts.
//    S = Q K^T and dP = dO V^T come out with queries in rows, so P and dS feed
//    dV^T = dO^T P and dK^T = Q^T dS from registers; each wavefront sums over all
//    heads of the group itself.
//
// Both kernels keep their streamed operands in the chunk-plane layout of the
// forward's K tiles and read it two ways: 16-byte row reads for the A operand of
// the score products and ds_read_b64_tr_b16 for the transposed A operand of the
// gradient products.  For the transposed reads the four head-dim quads addressed
// by a 16-lane group are {0, 4, 16, 20} (+ 8 for odd output blocks, + 32 per
// plane): with the plane swizzle, the 32 lanes of one half-wave then touch 64
// distinct banks for the row sets these kernels read (rows r..r+3 with r+8..r+11).
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace swa {
namespace {

using namespace tile;

constexpr int kQT = 16;        // query tokens per dq tile
constexpr int kHG = 8;         // query heads per dq workgroup
constexpr int kThreads = 256;  // 4 wavefronts (dk/dv)
constexpr int kDqPerCu = 1;    // resident dq workgroups per compute unit

// Byte offset (within a 64-byte-row plane buffer) of the 8 bytes lane (i, g) hands to
// ds_read_b64_tr_b16 for row `row` holding token/key `key`, output block 0: quad
// m = i & 3 is head-dim 16 (m >> 1) + 4 (m & 1), i.e. unit 2 (m >> 1), half m & 1.
// Output block b adds (b >> 1) planes and flips unit bit 0 when b is odd (tr_at).
__device__ __forceinline__ int tr_base(int row, int key, int i) {
  return row * 64 + 16 * ((2 * ((i >> 1) & 1)) ^ kswz(key)) + 8 * (i & 1);
}
__device__ __forceinline__ int tr_at(int base, int b, int plane_bytes) {
  return (b >> 1) * plane_bytes + (base ^ (16 * (b & 1)));
}

// Store a gradient row held in the transposed-read output layout: lane group g holds,
// in block b, head-dim 32 (b >> 1) + 8 (b & 1) + 16 (g >> 1) + 4 (g & 1) + r.
// v_permlane16_swap hands, per block pair, the even block to the even group and the
// odd block to the odd group, so that every lane stores 8 consecutive elements.
// All lanes must be active; the stores themselves are guarded by ok.
__device__ __forceinline__ void store_grad_row(bf16* row, int g, const f32x4 (&o)[8], float mul, bool ok) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f32x4 e = o[2 * p], od = o[2 * p + 1];
    const bf16x2 e0 = __builtin_convertvector((f32x2){e[0] * mul, e[1] * mul}, bf16x2);
    const bf16x2 e1 = __builtin_convertvector((f32x2){e[2] * mul, e[3] * mul}, bf16x2);
    const bf16x2 o0 = __builtin_convertvector((f32x2){od[0] * mul, od[1] * mul}, bf16x2);
    const bf16x2 o1 = __builtin_convertvector((f32x2){od[2] * mul, od[3] * mul}, bf16x2);
    const auto r0 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, e0),
                                                     __builtin_bit_cast(unsigned, o0), false, false);
    const auto r1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, e1),
                                                     __builtin_bit_cast(unsigned, o1), false, false);
    const u32x4 v = {(unsigned)r0[0], (unsigned)r1[0], (unsigned)r0[1], (unsigned)r1[1]};
    if (ok) *reinterpret_cast<u32x4*>(row + 32 * p + 16 * (g >> 1) + 8 * (g & 1)) = v;
  }
}

// ---------------------------------------------------------------------------
// dq: ring of 144 keys, K and V both in the chunk-plane layout; 8 wavefronts,
// one query head each
// ---------------------------------------------------------------------------
namespace dqring {

constexpr int kThreads = 512;
constexpr int kSlots = 9;
constexpr int kRows = 16 * kSlots;
constexpr int kPlane = kRows * 64;
constexpr int kBytes = 4 * kPlane;  // 36864 per operand

__device__ __forceinline__ int mod9(int x) { x %= kSlots; return x < 0 ? x + kSlots : x; }

// Load the 144 keys of a tile whose first key is kbase into both rings (32 rows per
// pass of the 512 threads).
__device__ __attribute__((noinline)) void fill(char* ks, char* vs, const bf16* __restrict__ k,
                                               const bf16* __restrict__ v, int kbase, int N, int hkv,
                                               int kvh) {
  const int t = threadIdx.x;
  const int r = t >> 4, u = t & 15;
  const int kblock0 = mod9(kbase >> 4);
  constexpr int kPasses = (kRows + 31) / 32;
  u32x4 kr[kPasses], vr[kPasses];
#pragma unroll
  for (int j = 0; j < kPasses; ++j) {
    const int row = 32 * j + r;
    const int key = kbase + row;
    kr[j] = (u32x4){0, 0, 0, 0};
    vr[j] = (u32x4){0, 0, 0, 0};
    if (row < kRows && key >= 0 && key < N) {
      const size_t off = ((size_t)key * hkv + kvh) * D + u * 8;
      kr[j] = *reinterpret_cast<const u32x4*>(k + off);
      vr[j] = *reinterpret_cast<const u32x4*>(v + off);
    }
  }
#pragma unroll
  for (int j = 0; j < kPasses; ++j) {
    const int row = 32 * j + r;
    if (row < kRows) {
      const int phys = 16 * mod9(kblock0 + (row >> 4)) + (row & 15);
      put_k(ks, kPlane, phys, kbase + row, u, kr[j]);
      put_k(vs, kPlane, phys, kbase + row, u, vr[j]);
    }
  }
}

}  // namespace dqring

__device__ __forceinline__ int find_seq_c(const_ptr<int32_t> cu, int num_seqs, int q) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= q) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(dqring::kThreads, 2) void bwd_dq_ring_kernel(BackwardArgs a, int items_per_wg) {
  using namespace dqring;
  __shared__ __attribute__((aligned(16))) char smem[2 * kBytes];
  char* ks = smem;
  char* vs = smem + kBytes;

  const int N = a.total_tokens, Hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int ntiles = (N + kQT - 1) / kQT;
  const int total = ntiles * (Hq / kHG);
  // Runs as in the forward ring kernel: each XCD takes a contiguous range of runs and
  // odd runs walk their tiles downwards, so that neighbouring runs read the K/V rows
  // they share at the same time through one L2.
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, perx = nwg >> 3, remx = nwg & 7;
  const int run = xcd * perx + min(xcd, remx) + (bid >> 3);
  const bool down = run & 1;
  const int item_lo = run * items_per_wg;
  const int item_hi = min(item_lo + items_per_wg, total);
  if (item_lo >= item_hi) return;
  int item = down ? item_hi - 1 : item_lo;  // next unprocessed item
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // head w of the octet
  const int i = lane & 15, g = lane >> 4;
  const int t = threadIdx.x;
  const int G = Hq / hkv;
  const int S = a.num_seqs;
  const const_ptr<int32_t> cu = as_const(a.cu_seqlens);
  const bf16* kp = static_cast<const bf16*>(a.k);
  const bf16* vp = static_cast<const bf16*>(a.v);
  const bf16* qp = static_cast<const bf16*>(a.q);
  const bf16* dop = static_cast<const bf16*>(a.dout);
  const float c = a.scale * kLog2e;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  const int pr0 = pair_row(i, 0), pr1 = pair_row(i, 1), p8 = pi8(i);
  const int vrow = 8 * (g & 1) + (i >> 2);                  // key row of the transposed reads, pairs
  const int vrow8 = 8 * (g & 1) + 4 * (g >> 1) + (i >> 2);  // the single diagonal block

  // Q and dO of one tile (lane (i, g): head-dim 32cc + 8g .. +8 of query q0 + i,
  // head w of the octet) with the row's lse.  Rows past the stream are loaded from the
  // last token (their results are never stored), so the loads are unconditional and
  // nothing waits for them before their first use.
  bf16x8 qa[4], da[4];
  float lr;
  auto load_rows = [&](int q0n, int octn) {
    const int qi = min(q0n + i, N - 1);
    const size_t hr = (size_t)qi * Hq + octn * kHG + w;
    const size_t r0 = hr * D + 8 * g;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      qa[cc] = *reinterpret_cast<const bf16x8*>(qp + r0 + 32 * cc);
      da[cc] = *reinterpret_cast<const bf16x8*>(dop + r0 + 32 * cc);
    }
    lr = a.lse[hr];
  };

  while (down ? item >= item_lo : item < item_hi) {
    item = __builtin_amdgcn_readfirstlane(item);
    const int oct = item / ntiles;
    const int tile0 = item - oct * ntiles;  // first tile of this run
    const int run_len = __builtin_amdgcn_readfirstlane(
        down ? item - max(item_lo, oct * ntiles) + 1 : min(item_hi, (oct + 1) * ntiles) - item);
    const int dir = down ? -1 : 1;
    int seq = find_seq_c(cu, S, tile0 * kQT);
    const int kvh = (oct * kHG) / G;
    __syncthreads();  // the previous run is done with the ring
    fill(ks, vs, kp, vp, tile0 * kQT - 128, N, hkv, kvh);
    load_rows(tile0 * kQT, oct);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ring slot of the tile's oldest block, (tile + 1) mod 9, moving with the walk
    int kblock0 = __builtin_amdgcn_readfirstlane((tile0 + 1) % kSlots);
    for (int k = 0; k < run_len; ++k) {
      const int tile = tile0 + dir * k;
      const int q0 = tile * kQT;
      const int kbase = q0 - 128;
      const int par = tile & 1;
      auto slot = [&](int j) { return kblock0 + j - (kblock0 + j >= kSlots ? kSlots : 0); };
      int sk[kSlots];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) sk[j] = 16 * 64 * slot(j);
      const int h0 = oct * kHG + w;

      // ---- visible keys of each row: window and own-sequence start ----
      if (down) {
        while (seq > 0 && cu[seq] > q0) --seq;
      } else {
        while (seq + 1 < S && cu[seq + 1] <= q0) ++seq;
      }
      const int qi = q0 + i;
      int start = cu[seq];
      for (int s2 = seq + 1; s2 < S && cu[s2] < q0 + kQT; ++s2)
        start = qi >= cu[s2] ? cu[s2] : start;
      const long lw = (long)qi - a.window + 1;
      const int lo = lw > start ? (int)lw : start;
      const int rel_lo = lo - kbase;
      const unsigned span = (unsigned)(qi - kbase - rel_lo);
      const float l2 = lr * kLog2e;
      const int ko0 = pr0 * 64 + 16 * (g ^ kswz(16 * par + pr0)) - (i >= 8 ? 16 * 64 : 0);
      const int ko1 = pr1 * 64 + 16 * (g ^ kswz(16 * par + pr1)) - (i >= 8 ? 16 * 64 : 0);
      const int ko8 = p8 * 64 + 16 * (g ^ kswz(16 * par + p8));
      auto block_off = [&](int bl) {
        if (bl < 8) {
          const int p = bl >> 1;
          return (i >= 8 ? sk[2 * p + 1] : sk[2 * p]) + ((bl & 1) ? ko1 : ko0);
        }
        return sk[8] + ko8;
      };
      // S^T = K Q^T and dP^T = V dO^T of block bl, the weights p formed in place of S
      auto products = [&](int bl, f32x4& s0, f32x4& t0) {
        const int off = block_off(bl);
        s0 = zero4;
        t0 = zero4;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + cc * kPlane + off);
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs + cc * kPlane + off);
          s0 = mfma32(kf, qa[cc], s0);
          t0 = mfma32(vf, da[cc], t0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kr = bl < 8 ? 32 * (bl >> 1) + 8 * g + 4 * (bl & 1) + r
                                : 128 + 8 * (g & 1) + 4 * (g >> 1) + r;
          const bool ok = (unsigned)(kr - rel_lo) <= span;
          const float e = fast_exp2(fmaf(s0[r], c, -l2));
          s0[r] = ok ? e : 0.f;
        }
      };
      // ---- p and dP of every block, delta = sum_j p_j dP_j over the row's keys (equal
      // to dO . O: the sink carries no value), then dS^T = p (dP - delta) in bf16 ----
      f32x4 ps[9], ts[9];
#pragma unroll
      for (int bl = 0; bl < 9; ++bl) products(bl, ps[bl], ts[bl]);
      float dl = 0.f;
#pragma unroll
      for (int bl = 0; bl < 9; ++bl)
#pragma unroll
        for (int r = 0; r < 4; ++r) dl = fmaf(ps[bl][r], ts[bl][r], dl);
      dl += __shfl_xor(dl, 16);
      dl += __shfl_xor(dl, 32);
      if (g == 0 && qi < N) {
        const size_t hr = (size_t)qi * Hq + h0;
        a.delta[hr] = dl;
        if (a.sinks) a.sink_term[hr] = expf(a.sinks[h0] - lr) * dl;
      }
      bf16x8 sa[4];
      bf16x4 sa8;
      {
        f32x4 x_prev;
#pragma unroll
        for (int bl = 0; bl < 9; ++bl) {
          f32x4 x;
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = ps[bl][r] * (ts[bl][r] - dl);
          if (bl == 8) {
            sa8 = pack_quad(x);
          } else if (bl & 1) {
            sa[bl >> 1] = pack_pair(x_prev, x);
          } else {
            x_prev = x;
          }
        }
      }

      // ---- prefetch for the next tile: the 16 K/V rows it adds to the ring (waves 0-3;
      // its newest block walking up, its oldest walking down), its Q, dO and lse ----
      const bool has_next = k + 1 < run_len;
      u32x4 pk = {0, 0, 0, 0}, pv = {0, 0, 0, 0};
      const int nkey = (down ? q0 - 144 : q0 + 16) + (t >> 4);
      if (has_next && t < 256 && nkey >= 0 && nkey < N) {
        const size_t off = ((size_t)nkey * hkv + kvh) * D + (t & 15) * 8;
        pk = *reinterpret_cast<const u32x4*>(kp + off);
        pv = *reinterpret_cast<const u32x4*>(vp + off);
      }
      if (has_next) load_rows(q0 + dir * kQT, oct);

      // ---- dQ^T = K^T dS^T: the diagonal block first (k = 16), then the four pairs ----
      f32x4 o0[8];
      {
        const int b8 = sk[8] + tr_base(vrow8, 16 * par + vrow8, i);
#pragma unroll
        for (int b = 0; b < 8; ++b) o0[b] = mfma32_k16(tr_read(ks, tr_at(b8, b, kPlane)), sa8, zero4);
      }
      {
        // groups 0-1 read the pair's first block, 2-3 its second; key parity of each
        const int kpar = g >= 2 ? 1 - par : par;
        const int blo = tr_base(vrow, 16 * kpar + vrow, i);
        const int bhi = tr_base(vrow + 4, 16 * kpar + vrow + 4, i);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int sbase = g >= 2 ? sk[2 * p + 1] : sk[2 * p];
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const bf16x4 lo4 = tr_read(ks, sbase + tr_at(blo, b, kPlane));
            const bf16x4 hi4 = tr_read(ks, sbase + tr_at(bhi, b, kPlane));
            const bf16x8 av = (bf16x8){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            o0[b] = mfma32(av, sa[p], o0[b]);
          }
        }
      }

      // ---- ring update for the next tile (every load of this iteration waited for
      // before the stores below are issued) ----
      if (has_next) {
        __syncthreads();
        if (t < 256) {
          const int phys = 16 * slot(down ? 8 : 0) + (t >> 4);  // the block the next tile replaces
          put_k(ks, kPlane, phys, nkey, t & 15, pk);
          put_k(vs, kPlane, phys, nkey, t & 15, pv);
        }
        __syncthreads();
      }
      kblock0 = down ? (kblock0 == 0 ? kSlots - 1 : kblock0 - 1) : (kblock0 == kSlots - 1 ? 0 : kblock0 + 1);

      // ---- epilogue: the dq row of this tile ----
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      {
        const bool ok = qi < N;
        store_grad_row(static_cast<bf16*>(a.dq) + ((size_t)(ok ? qi : 0) * Hq + h0) * D, g, o0, a.scale, ok);
      }
    }
    item += dir * run_len;  // next run
  }
}

// ---------------------------------------------------------------------------
// dk, dv: 64 keys per workgroup (16 per wavefront), one shared query block of
// 16 tokens x 4 heads per step
// ---------------------------------------------------------------------------
namespace kvtile {

constexpr int kHeads = 4;             // query heads per step
constexpr int kRows = 16 * kHeads;    // 16 tokens x 4 heads; row P = 16 * head_sel + token
constexpr int kPlane = kRows * 64;    // 4096
constexpr int kOpBytes = 4 * kPlane;  // 16384 per operand
constexpr int kStage = 2 * kOpBytes + 2 * kRows * 4;  // Q, dO, lse, delta: 33280
constexpr int kTiles = 4;             // 16-key tiles per workgroup, one per wavefront

}  // namespace kvtile

__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(BackwardArgs a, int ngrp) {
  using namespace kvtile;
  // double-buffered step, as two arrays so that the compiler can tell the buffer being
  // read from the one the next step's loads are filling
  __shared__ __attribute__((aligned(16))) char smem0[kStage];
  __shared__ __attribute__((aligned(16))) char smem1[kStage];

  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous range
  // of key tiles so that the query blocks shared by neighbouring tiles are read
  // through one L2.
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, per = nwg >> 3, rem = nwg & 7;
  const int L = xcd * per + min(xcd, rem) + (bid >> 3);
  const int kvh = L / ngrp, grp = L - kvh * ngrp;

  const int N = a.total_tokens, Hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int G = Hq / hkv;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int i = lane & 15, g = lane >> 4;
  const bf16* qp = static_cast<const bf16*>(a.q);
  const bf16* dop = static_cast<const bf16*>(a.dout);
  const float c = a.scale * kLog2e;
  const const_ptr<int32_t> cu = as_const(a.cu_seqlens);

  // Last query that sees key jj: within the window and the key's own sequence (the
  // largest s with cu[s] <= jj, so zero-length sequences are stepped over).
  auto last_query = [&](int jj) {
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= jj) lo = mid; else hi = mid;
    }
    const long lw = (long)jj + a.window - 1;
    const long end = cu[lo + 1];
    return (int)(lw < end - 1 ? lw : end - 1);
  };

  // This wavefront's keys, K and V as B operands: lane (i, g) holds key k0 + i,
  // head-dim 32cc + 8g ..
  const int kt0 = kTiles * grp;
  const int k0 = 16 * (kt0 + w);
  const int j = k0 + i;
  const bool kvalid = j < N;
  bf16x8 kb[4], vb[4];
  {
    const size_t r0 = ((size_t)(kvalid ? j : 0) * hkv + kvh) * D + 8 * g;
    const bf16* kp = static_cast<const bf16*>(a.k);
    const bf16* vp = static_cast<const bf16*>(a.v);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      kb[cc] = kvalid ? *reinterpret_cast<const bf16x8*>(kp + r0 + 32 * cc) : zero8();
      vb[cc] = kvalid ? *reinterpret_cast<const bf16x8*>(vp + r0 + 32 * cc) : zero8();
    }
  }
  const int last = kvalid ? last_query(j) : -1;
  // query q sees key j iff (unsigned)(q - jm) <= span; invalid keys see nothing
  const int jm = kvalid ? j : 0x3fffffff;
  const unsigned span = kvalid ? (unsigned)(last - j) : 0u;
  // query blocks this wavefront works on (none if it has no valid key), and the
  // workgroup's: last_query is nondecreasing in the key, so the workgroup's last
  // valid key bounds them all
  const int wlast = k0 < N ? last_query(min(k0 + 15, N - 1)) : -1;
  const int tbw_lo = k0 >> 4, tbw_hi = wlast >> 4;
  const int tb_lo = kt0;
  const int tb_hi = last_query(min(16 * (kt0 + kTiles) - 1, N - 1)) >> 4;
  const int nsteps = tb_hi - tb_lo + 1;
  const int total = (G / kHeads) * nsteps;  // (head quad, query block) steps
  // Query block of a step: within each head quad's sweep, step m takes the block tb with
  // tb = m (mod nsteps).  Neighbouring workgroups share most of their blocks and start
  // together on one XCD; with this order they read each shared block at the same step.
  auto step_block = [&](int m) {
    int r = (m - tb_lo) % nsteps;
    r += r < 0 ? nsteps : 0;
    return tb_lo + r;
  };
  // the block of local step 0; later steps advance it by one, wrapping within
  // [tb_lo, tb_lo + nsteps) (no division per step)
  const int tb_first = __builtin_amdgcn_readfirstlane(step_block(0));
  const int tb_wrap = tb_lo + nsteps;

  // Lane-constant LDS offsets: row reads (pair order) and transposed reads.
  const int pr0 = pair_row(i, 0), pr1 = pair_row(i, 1);
  const int ro0 = pr0 * 64 + 16 * (g ^ kswz(pr0));
  const int ro1 = pr1 * 64 + 16 * (g ^ kswz(pr1));
  const int tlo = tr_base(8 * g + (i >> 2), 8 * g + (i >> 2), i);
  const int thi = tr_base(8 * g + 4 + (i >> 2), 8 * g + 4 + (i >> 2), i);

  // Staging: the step's Q and dO rows go from global memory straight into LDS (16 bytes
  // per lane, 1 KB per instruction), each lane reading the unit that belongs at its slot of
  // the swizzled chunk-plane layout: wavefront w fills plane w of both operands, row groups
  // rg = 0..3 (head rg, tokens 0..15): lane L holds row P = 16 rg + L / 4, slot L & 3, i.e.
  // unit 4w + ((L & 3) ^ kswz(P)).  Wavefronts 0 and 1 bring the rows' lse and delta (4 bytes
  // per lane).  No registers hold the block; each wavefront waits for its own loads before
  // the barrier that ends the step.
  int hp_n = 0, tb_n = tb_first, m_n = 0;  // position of the step being loaded
  auto advance = [&](int& hp, int& tb, int& m) {
    ++m;
    ++tb;
    if (tb == tb_wrap) tb = tb_lo;
    if (m == nsteps) { m = 0; ++hp; tb = tb_first; }
  };
  const int srow = lane >> 2, sslot = lane & 3;
  auto issue = [&](char* buf) {
    const int hbase = kvh * G + kHeads * hp_n;
    const int q = min(16 * tb_n + srow, N - 1);
#pragma unroll
    for (int rg = 0; rg < kHeads; ++rg) {
      const int u = 4 * w + (sslot ^ kswz(16 * rg + srow));
      const size_t off = ((size_t)q * Hq + hbase + rg) * D + 8 * u;
      const int dst = w * kPlane + rg * 1024;
      load_lds16(qp + off, buf + dst);
      load_lds16(dop + off, buf + kOpBytes + dst);
    }
    if (w < 2) {  // lse (wavefront 0) or delta (1) of row P = lane: token P & 15, head P >> 4
      const size_t r = (size_t)min(16 * tb_n + (lane & 15), N - 1) * Hq + hbase + (lane >> 4);
      const float* src = w == 0 ? a.lse : a.delta;
      load_lds4(src + r, buf + 2 * kOpBytes + w * kRows * 4);
    }
  };
  f32x4 dk[8], dv[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    dk[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    dv[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // One step: its block is already in LDS buffer cur; the next step's loads into the
  // other buffer are issued first and waited for at the end.
  int hp_c = 0, tb_c = tb_first, m_c = 0;  // position of the current step
  auto do_step = [&](int step, const char* cur, char* nxt) {
    if (step + 1 < total) {
      advance(hp_n, tb_n, m_n);
      issue(nxt);
    }
    const int tb = tb_c;
    if (tb >= tbw_lo && tb <= tbw_hi) {
      const char* qs = cur;
      const char* ds = qs + kOpBytes;
      const float* ls = reinterpret_cast<const float*>(ds + kOpBytes);
      // ---- S = Q K^T and dP = dO V^T for two pairs of 16-row blocks (rows 32 pi ..) ----
      f32x4 s[2][2], tt[2][2];
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int pi = 0; pi < 2; ++pi)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          s[pi][h] = (f32x4){0.f, 0.f, 0.f, 0.f};
          tt[pi][h] = (f32x4){0.f, 0.f, 0.f, 0.f};
          const int ro = (h ? ro1 : ro0) + 32 * 64 * pi;
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qs + cc * kPlane + ro);
            const bf16x8 df = *reinterpret_cast<const bf16x8*>(ds + cc * kPlane + ro);
            s[pi][h] = mfma32(qf, kb[cc], s[pi][h]);
            tt[pi][h] = mfma32(df, vb[cc], tt[pi][h]);
          }
        }
      __builtin_amdgcn_s_setprio(0);
      // lane (i, g) holds rows P = 32 pi + 8g + 4h + r: token 8 (g & 1) + 4h + r
      bf16x8 pp[2], xp[2];
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(ls + 32 * pi + 8 * g) * kLog2e;
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(ls + 32 * pi + 8 * g + 4) * kLog2e;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(ls + kRows + 32 * pi + 8 * g);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(ls + kRows + 32 * pi + 8 * g + 4);
        f32x4 p[2], x[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = 16 * tb + 8 * (g & 1) + 4 * h + r;
            const bool ok = (unsigned)(q - jm) <= span;
            const float e = fast_exp2(fmaf(s[pi][h][r], c, -(h ? l1[r] : l0[r])));
            p[h][r] = ok ? e : 0.f;
            x[h][r] = p[h][r] * (tt[pi][h][r] - (h ? d1[r] : d0[r]));
          }
        }
        pp[pi] = pack_pair(p[0], p[1]);
        xp[pi] = pack_pair(x[0], x[1]);
      }

      // ---- dV^T += dO^T P and dK^T += Q^T dS over the step's 64 rows ----
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int lo = tr_at(tlo, b, kPlane) + 32 * 64 * pi;
          const int hi = tr_at(thi, b, kPlane) + 32 * 64 * pi;
          const bf16x4 dlo = tr_read(ds, lo);
          const bf16x4 dhi = tr_read(ds, hi);
          const bf16x4 qlo = tr_read(qs, lo);
          const bf16x4 qhi = tr_read(qs, hi);
          dv[b] = mfma32((bf16x8){dlo[0], dlo[1], dlo[2], dlo[3], dhi[0], dhi[1], dhi[2], dhi[3]}, pp[pi], dv[b]);
          dk[b] = mfma32((bf16x8){qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]}, xp[pi], dk[b]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // the buffer being filled was last read in the previous step, which every wavefront
    // had finished at the barrier that ended it; this one publishes the new block
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    advance(hp_c, tb_c, m_c);
  };

  issue(smem0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  for (int step = 0; step < total; step += 2) {
    do_step(step, smem0, smem1);
    if (step + 1 < total) do_step(step + 1, smem1, smem0);
  }

  const size_t krow = ((size_t)(kvalid ? j : 0) * hkv + kvh) * D;
  store_grad_row(static_cast<bf16*>(a.dk) + krow, g, dk, a.scale, kvalid);
  store_grad_row(static_cast<bf16*>(a.dv) + krow, g, dv, 1.f, kvalid);
}

}  // namespace

bool backward_mfma_supported(const BackwardArgs& a, bool bf16_io) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return bf16_io && a.head_dim == 128 && G % kHG == 0 && a.window >= 1 && a.window <= 128;
}

hipError_t launch_backward_mfma(const BackwardArgs& a, hipStream_t s) {
  const long ntiles = (a.total_tokens + kQT - 1) / kQT;
  const long total = ntiles * (a.num_q_heads / kHG);
  const long kvtiles = ntiles * a.num_kv_heads;
  if (total > 0x7fffffffL || kvtiles > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (total == 0) return hipSuccess;
  int cus = 0;
  hipError_t e = device_cu_count(&cus);
  if (e != hipSuccess) return e;
  // one resident 8-wavefront workgroup per compute unit (register-bound), each
  // walking a contiguous run of tiles
  const long slots = kDqPerCu * cus;
  const long per = (total + slots - 1) / slots;
  const long grid = (total + per - 1) / per;
  hipLaunchKernelGGL(bwd_dq_ring_kernel, dim3((unsigned)grid), dim3(dqring::kThreads), 0, s, a, (int)per);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long ngrp = (ntiles + kvtile::kTiles - 1) / kvtile::kTiles;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)(ngrp * a.num_kv_heads)), dim3(kThreads), 0, s, a,
                     (int)ngrp);
  return hipGetLastError();
}

}  // namespace swa
