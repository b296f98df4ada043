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
//    tokens x 8 heads sharing one KV head, the 144-key band sits in an LDS ring that
//    advances by 16 keys per tile.  S^T = K Q^T and dP^T = V dO^T come out with
//    queries in columns, so dS^T feeds dQ^T = K^T dS^T straight from registers.
//  * bwd_dkdv_kernel: the transpose -- a workgroup owns 16 keys of one KV head and
//    walks the query blocks that see them (16 tokens x 2 heads per step and
//    wavefront).  S = Q K^T and dP = dO V^T come out with queries in rows, so P and
//    dS feed dV^T = dO^T P and dK^T = Q^T dS from registers; the four wavefronts'
//    head partial sums are added in a fixed order through LDS.
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
constexpr int kThreads = 256;  // 4 wavefronts

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

// Store block pair (2p, 2p+1) of a gradient row held in the transposed-read output
// layout: lane group g holds, in block b, head-dim 32 (b >> 1) + 8 (b & 1) +
// 16 (g >> 1) + 4 (g & 1) + r.  v_permlane16_swap hands the even block to the even
// group and the odd block to the odd group, so that every lane stores 8
// consecutive elements.  All lanes must be active; the store itself is guarded.
__device__ __forceinline__ void store_pair_tr(bf16* row, int g, int p, f32x4 e, f32x4 o, float mul,
                                              bool ok) {
  const bf16x2 e0 = __builtin_convertvector((f32x2){e[0] * mul, e[1] * mul}, bf16x2);
  const bf16x2 e1 = __builtin_convertvector((f32x2){e[2] * mul, e[3] * mul}, bf16x2);
  const bf16x2 o0 = __builtin_convertvector((f32x2){o[0] * mul, o[1] * mul}, bf16x2);
  const bf16x2 o1 = __builtin_convertvector((f32x2){o[2] * mul, o[3] * mul}, bf16x2);
  const auto r0 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, e0),
                                                   __builtin_bit_cast(unsigned, o0), false, false);
  const auto r1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, e1),
                                                   __builtin_bit_cast(unsigned, o1), false, false);
  const u32x4 v = {(unsigned)r0[0], (unsigned)r1[0], (unsigned)r0[1], (unsigned)r1[1]};
  if (ok) *reinterpret_cast<u32x4*>(row + 32 * p + 16 * (g >> 1) + 8 * (g & 1)) = v;
}

// ---------------------------------------------------------------------------
// dq: ring of 144 keys, K and V both in the chunk-plane layout
// ---------------------------------------------------------------------------
namespace dqring {

constexpr int kSlots = 9;
constexpr int kRows = 16 * kSlots;
constexpr int kPlane = kRows * 64;
constexpr int kBytes = 4 * kPlane;  // 36864 per operand

__device__ __forceinline__ int mod9(int x) { x %= kSlots; return x < 0 ? x + kSlots : x; }

// Load the 144 keys of a tile whose first key is kbase into both rings.
__device__ __attribute__((noinline)) void fill(char* ks, char* vs, const bf16* __restrict__ k,
                                               const bf16* __restrict__ v, int kbase, int N, int hkv,
                                               int kvh) {
  const int t = threadIdx.x;
  const int r = t >> 4, u = t & 15;
  const int kblock0 = mod9(kbase >> 4);
  u32x4 kr[kSlots], vr[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int key = kbase + 16 * j + r;
    kr[j] = (u32x4){0, 0, 0, 0};
    vr[j] = (u32x4){0, 0, 0, 0};
    if (key >= 0 && key < N) {
      const size_t off = ((size_t)key * hkv + kvh) * D + u * 8;
      kr[j] = *reinterpret_cast<const u32x4*>(k + off);
      vr[j] = *reinterpret_cast<const u32x4*>(v + off);
    }
  }
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int phys = 16 * mod9(kblock0 + j) + r;
    put_k(ks, kPlane, phys, kbase + 16 * j + r, u, kr[j]);
    put_k(vs, kPlane, phys, kbase + 16 * j + r, u, vr[j]);
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

__global__ __launch_bounds__(kThreads, 2) void bwd_dq_ring_kernel(BackwardArgs a, int items_per_wg) {
  using namespace dqring;
  __shared__ __attribute__((aligned(16))) char smem[2 * kBytes];
  char* ks = smem;
  char* vs = smem + kBytes;

  const int N = a.total_tokens, Hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int ntiles = (N + kQT - 1) / kQT;
  const int total = ntiles * (Hq / kHG);
  int item = blockIdx.x * items_per_wg;
  const int item_end = min(item + items_per_wg, total);
  if (item >= item_end) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  // Q and dO of one tile (lane (i, g): head-dim 32cc + 8g .. +8 of query q0 + i, heads
  // 2w and 2w + 1 of the octet), with the rows' lse (log2 units) and delta.
  bf16x8 qa[4], qb[4], da[4], db[4];
  float la, lb, dla, dlb;
  auto load_rows = [&](int q0n, int octn) {
    const int qi = q0n + i;
    const bool ok = qi < N;
    const size_t hr = (size_t)qi * Hq + octn * kHG + 2 * w;
    const size_t r0 = hr * D + 8 * g;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      qa[cc] = ok ? *reinterpret_cast<const bf16x8*>(qp + r0 + 32 * cc) : zero8();
      qb[cc] = ok ? *reinterpret_cast<const bf16x8*>(qp + r0 + D + 32 * cc) : zero8();
      da[cc] = ok ? *reinterpret_cast<const bf16x8*>(dop + r0 + 32 * cc) : zero8();
      db[cc] = ok ? *reinterpret_cast<const bf16x8*>(dop + r0 + D + 32 * cc) : zero8();
    }
    la = ok ? a.lse[hr] * kLog2e : 0.f;
    lb = ok ? a.lse[hr + 1] * kLog2e : 0.f;
    dla = ok ? a.delta[hr] : 0.f;
    dlb = ok ? a.delta[hr + 1] : 0.f;
  };

  while (item < item_end) {
    item = __builtin_amdgcn_readfirstlane(item);
    const int oct = item / ntiles;
    int tile = item - oct * ntiles;
    const int run_end = min(item_end, (oct + 1) * ntiles);
    int seq = find_seq_c(cu, S, tile * kQT);
    const int kvh = (oct * kHG) / G;
    __syncthreads();  // the previous run is done with the ring
    fill(ks, vs, kp, vp, tile * kQT - 128, N, hkv, kvh);
    load_rows(tile * kQT, oct);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int run_len = __builtin_amdgcn_readfirstlane(run_end - item);
    const int tile0 = tile;
    int kblock0 = __builtin_amdgcn_readfirstlane((tile0 + 1) % kSlots);
    for (int k = 0; k < run_len; ++k) {
      tile = tile0 + k;
      const int q0 = tile * kQT;
      const int kbase = q0 - 128;
      const int par = tile & 1;
      auto slot = [&](int j) { return kblock0 + j - (kblock0 + j >= kSlots ? kSlots : 0); };
      int sk[kSlots];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) sk[j] = 16 * 64 * slot(j);
      const int h0 = oct * kHG + 2 * w;

      // ---- visible keys of each row: window and own-sequence start ----
      while (seq + 1 < S && cu[seq + 1] <= q0) ++seq;
      const int qi = q0 + i;
      int start = cu[seq];
      for (int s2 = seq + 1; s2 < S && cu[s2] < q0 + kQT; ++s2)
        start = qi >= cu[s2] ? cu[s2] : start;
      const long lw = (long)qi - a.window + 1;
      const int lo = lw > start ? (int)lw : start;
      const int rel_lo = lo - kbase;
      const unsigned span = (unsigned)(qi - kbase - rel_lo);

      // ---- per 16-key block: S^T = K Q^T, dP^T = V dO^T, then dS^T in bf16 ----
      bf16x8 sa[4], sb[4];
      bf16x4 sa8, sb8;
      {
        const int ko0 = pr0 * 64 + 16 * (g ^ kswz(16 * par + pr0)) - (i >= 8 ? 16 * 64 : 0);
        const int ko1 = pr1 * 64 + 16 * (g ^ kswz(16 * par + pr1)) - (i >= 8 ? 16 * 64 : 0);
        const int ko8 = p8 * 64 + 16 * (g ^ kswz(16 * par + p8));
        f32x4 xa_prev, xb_prev;
#pragma unroll
        for (int bl = 0; bl < 9; ++bl) {
          int off;
          if (bl < 8) {
            const int p = bl >> 1;
            off = (i >= 8 ? sk[2 * p + 1] : sk[2 * p]) + ((bl & 1) ? ko1 : ko0);
          } else {
            off = sk[8] + ko8;
          }
          f32x4 s0 = zero4, s1 = zero4, t0 = zero4, t1 = zero4;
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + cc * kPlane + off);
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs + cc * kPlane + off);
            s0 = mfma32(kf, qa[cc], s0);
            s1 = mfma32(kf, qb[cc], s1);
            t0 = mfma32(vf, da[cc], t0);
            t1 = mfma32(vf, db[cc], t1);
          }
          f32x4 xa, xb;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kr = bl < 8 ? 32 * (bl >> 1) + 8 * g + 4 * (bl & 1) + r
                                  : 128 + 8 * (g & 1) + 4 * (g >> 1) + r;
            const bool ok = (unsigned)(kr - rel_lo) <= span;
            const float ea = fast_exp2(fmaf(s0[r], c, -la));
            const float eb = fast_exp2(fmaf(s1[r], c, -lb));
            xa[r] = (ok ? ea : 0.f) * (t0[r] - dla);
            xb[r] = (ok ? eb : 0.f) * (t1[r] - dlb);
          }
          if (bl == 8) {
            sa8 = pack_quad(xa);
            sb8 = pack_quad(xb);
          } else if (bl & 1) {
            sa[bl >> 1] = pack_pair(xa_prev, xa);
            sb[bl >> 1] = pack_pair(xb_prev, xb);
          } else {
            xa_prev = xa;
            xb_prev = xb;
          }
        }
      }

      // ---- prefetch for the next tile: its 16 newest K/V rows, its Q, dO, lse, delta ----
      const bool has_next = k + 1 < run_len;
      u32x4 pk = {0, 0, 0, 0}, pv = {0, 0, 0, 0};
      const int nkey = q0 + 16 + (t >> 4);
      if (has_next && nkey < N) {
        const size_t off = ((size_t)nkey * hkv + kvh) * D + (t & 15) * 8;
        pk = *reinterpret_cast<const u32x4*>(kp + off);
        pv = *reinterpret_cast<const u32x4*>(vp + off);
      }
      if (has_next) load_rows(q0 + kQT, oct);

      // ---- dQ^T = K^T dS^T: the diagonal block first (k = 16), then the four pairs ----
      f32x4 o0[8], o1[8];
      {
        const int b8 = sk[8] + tr_base(vrow8, 16 * par + vrow8, i);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const bf16x4 av = tr_read(ks, tr_at(b8, b, kPlane));
          o0[b] = mfma16(av, sa8, zero4);
          o1[b] = mfma16(av, sb8, zero4);
        }
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
            o1[b] = mfma32(av, sb[p], o1[b]);
          }
        }
      }

      // ---- ring update for the next tile (every load of this iteration waited for
      // before the stores below are issued) ----
      if (has_next) {
        __syncthreads();
        const int phys = 16 * kblock0 + (t >> 4);
        put_k(ks, kPlane, phys, nkey, t & 15, pk);
        put_k(vs, kPlane, phys, nkey, t & 15, pv);
        __syncthreads();
      }
      kblock0 = kblock0 == kSlots - 1 ? 0 : kblock0 + 1;

      // ---- epilogue: dq rows of this tile ----
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      {
        const bool ok = qi < N;
        bf16* out = static_cast<bf16*>(a.dq) + ((size_t)(ok ? qi : 0) * Hq + h0) * D;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          store_pair_tr(out, g, p, o0[2 * p], o0[2 * p + 1], a.scale, ok);
          store_pair_tr(out + D, g, p, o1[2 * p], o1[2 * p + 1], a.scale, ok);
        }
      }
    }
    item = run_end;
  }
}

// ---------------------------------------------------------------------------
// dk, dv: 16 keys per workgroup, query blocks of 16 tokens x 2 heads per step
// ---------------------------------------------------------------------------
namespace kvtile {

constexpr int kRows = 32;             // 16 tokens x 2 heads; row P = 16 * head_sel + token
constexpr int kPlane = kRows * 64;    // 2048
constexpr int kOpBytes = 4 * kPlane;  // 8192 per operand
constexpr int kWaveBytes = 2 * kOpBytes + 2 * kRows * 4;  // Q, dO, lse, delta: 16640

}  // namespace kvtile

__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(BackwardArgs a, int nkt) {
  using namespace kvtile;
  __shared__ __attribute__((aligned(16))) char smem[4 * kWaveBytes];

  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous range
  // of key tiles so that the query blocks shared by neighbouring tiles are read
  // through one L2.
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, per = nwg >> 3, rem = nwg & 7;
  const int L = xcd * per + min(xcd, rem) + (bid >> 3);
  const int kvh = L / nkt, kt = L - kvh * nkt;

  const int N = a.total_tokens, Hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int G = Hq / hkv;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  char* qs = smem + w * kWaveBytes;
  char* ds = qs + kOpBytes;
  float* ls = reinterpret_cast<float*>(ds + kOpBytes);
  float* dls = ls + kRows;
  const bf16* qp = static_cast<const bf16*>(a.q);
  const bf16* dop = static_cast<const bf16*>(a.dout);
  const float c = a.scale * kLog2e;

  // K and V of the tile as B operands: lane (i, g) holds key k0 + i, head-dim 32cc + 8g ..
  const int k0 = kt * 16;
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
  // Last query that sees key j: within the window and the key's own sequence (the
  // largest s with cu[s] <= j, so zero-length sequences are stepped over).
  int last = -1;
  if (kvalid) {
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens[mid] <= j) lo = mid; else hi = mid;
    }
    const int end = a.cu_seqlens[lo + 1];
    const long lw = (long)j + a.window - 1;
    last = (int)(lw < end - 1 ? lw : end - 1);
  }
  // query q sees key j iff (unsigned)(q - jm) <= span; invalid keys see nothing
  const int jm = kvalid ? j : 0x3fffffff;
  const unsigned span = kvalid ? (unsigned)(last - j) : 0u;
  int qmax = last;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) qmax = max(qmax, __shfl_xor(qmax, o));
  const int tb_lo = kt, tb_hi = __builtin_amdgcn_readfirstlane(qmax) >> 4;

  // Lane-constant LDS offsets: row reads (pair order) and transposed reads.
  const int pr0 = pair_row(i, 0), pr1 = pair_row(i, 1);
  const int ro0 = pr0 * 64 + 16 * (g ^ kswz(pr0));
  const int ro1 = pr1 * 64 + 16 * (g ^ kswz(pr1));
  const int tlo = tr_base(8 * g + (i >> 2), 8 * g + (i >> 2), i);
  const int thi = tr_base(8 * g + 4 + (i >> 2), 8 * g + 4 + (i >> 2), i);
  // staging map: piece it (0..7) of lane l is row P = 16 (it >> 2) + 4 (it & 3) + (l >> 4), unit l & 15
  const int su = lane & 15;

  f32x4 dk[8], dv[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    dk[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    dv[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  const int npairs = G / 2;
  for (int hp = w; hp < npairs; hp += 4) {
    const int hbase = kvh * G + 2 * hp;
    u32x4 pq[8], pd[8];
    float pl = 0.f, pdl = 0.f;
    auto prefetch = [&](int tb) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int tok = 4 * (it & 3) + (lane >> 4);
        const int q = min(16 * tb + tok, N - 1);
        const size_t off = ((size_t)q * Hq + hbase + (it >> 2)) * D + 8 * su;
        pq[it] = *reinterpret_cast<const u32x4*>(qp + off);
        pd[it] = *reinterpret_cast<const u32x4*>(dop + off);
      }
      if (lane < kRows) {
        const int q = min(16 * tb + (lane & 15), N - 1);
        const size_t r = (size_t)q * Hq + hbase + (lane >> 4);
        pl = a.lse[r] * kLog2e;
        pdl = a.delta[r];
      }
    };
    prefetch(tb_lo);
    for (int tb = tb_lo; tb <= tb_hi; ++tb) {
      // ---- commit the staged block (the previous step's reads are complete: their
      // values were consumed by the matrix products) ----
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int P = 16 * (it >> 2) + 4 * (it & 3) + (lane >> 4);
        put_k(qs, kPlane, P, P, su, pq[it]);
        put_k(ds, kPlane, P, P, su, pd[it]);
      }
      if (lane < kRows) {
        ls[lane] = pl;
        dls[lane] = pdl;
      }
      __builtin_amdgcn_wave_barrier();
      if (tb < tb_hi) prefetch(tb + 1);

      // ---- S = Q K^T and dP = dO V^T for the two 16-row blocks of the pair ----
      f32x4 s[2], t[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[h] = (f32x4){0.f, 0.f, 0.f, 0.f};
        t[h] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const int ro = h ? ro1 : ro0;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qs + cc * kPlane + ro);
          const bf16x8 df = *reinterpret_cast<const bf16x8*>(ds + cc * kPlane + ro);
          s[h] = mfma32(qf, kb[cc], s[h]);
          t[h] = mfma32(df, vb[cc], t[h]);
        }
      }
      // lane (i, g) holds rows P = 8g + 4h + r: token 8 (g & 1) + 4h + r of head g >> 1
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(ls + 8 * g);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(ls + 8 * g + 4);
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(dls + 8 * g);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(dls + 8 * g + 4);
      f32x4 p[2], x[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = 16 * tb + 8 * (g & 1) + 4 * h + r;
          const bool ok = (unsigned)(q - jm) <= span;
          const float e = fast_exp2(fmaf(s[h][r], c, -(h ? l1[r] : l0[r])));
          p[h][r] = ok ? e : 0.f;
          x[h][r] = p[h][r] * (t[h][r] - (h ? d1[r] : d0[r]));
        }
      }
      const bf16x8 pp = pack_pair(p[0], p[1]);
      const bf16x8 xp = pack_pair(x[0], x[1]);

      // ---- dV^T += dO^T P and dK^T += Q^T dS over the pair's 32 rows ----
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bf16x4 dlo = tr_read(ds, tr_at(tlo, b, kPlane));
        const bf16x4 dhi = tr_read(ds, tr_at(thi, b, kPlane));
        const bf16x4 qlo = tr_read(qs, tr_at(tlo, b, kPlane));
        const bf16x4 qhi = tr_read(qs, tr_at(thi, b, kPlane));
        dv[b] = mfma32((bf16x8){dlo[0], dlo[1], dlo[2], dlo[3], dhi[0], dhi[1], dhi[2], dhi[3]}, pp, dv[b]);
        dk[b] = mfma32((bf16x8){qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]}, xp, dk[b]);
      }
    }
  }

  // ---- sum the four wavefronts' partial sums in a fixed order and store ----
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem + w * kWaveBytes);  // 64 registers x 64 lanes
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      red[(4 * b + r) * 64 + lane] = dk[b][r];
      red[(32 + 4 * b + r) * 64 + lane] = dv[b][r];
    }
  __syncthreads();
  // wavefront w adds registers 16w .. 16w + 15: dk blocks 0-3 / 4-7, dv blocks 0-3 / 4-7
  f32x4 sum[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int reg = 16 * w + 4 * kk + r;
      float acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
        acc += reinterpret_cast<const float*>(smem + ww * kWaveBytes)[reg * 64 + lane];
      sum[kk][r] = acc;
    }
  bf16* dst = static_cast<bf16*>(w < 2 ? a.dk : a.dv) + ((size_t)(kvalid ? j : 0) * hkv + kvh) * D;
  const float mul = w < 2 ? a.scale : 1.f;
  const int p0 = 2 * (w & 1);
  store_pair_tr(dst, g, p0, sum[0], sum[1], mul, kvalid);
  store_pair_tr(dst, g, p0 + 1, sum[2], sum[3], mul, kvalid);
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
  const long slots = 2L * cus;
  const long per = (total + slots - 1) / slots;
  const long grid = (total + per - 1) / per;
  hipLaunchKernelGGL(bwd_dq_ring_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a, (int)per);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)kvtiles), dim3(kThreads), 0, s, a, (int)ntiles);
  return hipGetLastError();
}

}  // namespace swa
