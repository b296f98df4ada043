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
// partial outputs then simply add.  The ring is read straight from HBM into MFMA
// operand registers (V rows 16 lanes per 256-byte row, fully coalesced, and
// transposed in registers); the query columns and the new tokens' K/V, shared by
// the four wavefronts, are staged once in LDS.  Template switches: an FP8 (E4M3) ring,
// the rotary embedding applied in the kernel, and the one-launch MTP step that first
// commits the previous step's accepted tokens to the ring (see decode_kernel).
#include <type_traits>

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

constexpr int kRowPitch = 272;  // staged bf16 row (256 B) padded: 16 rows hit 16 bank quads

// Partial-output slots of the merge: one per wavefront for a single query tile (one
// barrier), two for two tiles (a pairwise step first), which keeps the workgroup
// within a quarter of the LDS either way.
template <int NT>
constexpr int kMergeSlots = NT == 1 ? 4 : 2;

template <int NT>
struct DecodeSmem {
  float m[4][NT * 16];
  float l[4][NT * 16];
  float mc[NT * 16];  // column maximum (sink included), log2 units
  float zs[NT * 16];  // the sink's term of the column's denominator
  union {
    char o[kMergeSlots<NT>][NT * 16][kColBytes];  // partial outputs, fp32
    struct {
      char q[NT * 16][kRowPitch];  // query columns (dead once the scores are formed)
      char kn[16][kRowPitch];      // new-token K rows (rows past T repeat row T-1; in the one-launch
                                   // MTP step rows 4 .. 7 hold the committed tokens)
      float cs[8 * 64][2];         // rotary cos / sin per (token, pair), when rotating
    } in;
  } u;
  char vn[16][kRowPitch];  // new-token V rows (as kn)
};

// Partial O^T of lane (i, g), column tt*16 + i, head-dim 32g + 8r + b, to/from LDS.
template <int NT>
__device__ __forceinline__ void put_partial(char (*slot)[kColBytes], int i, int g,
                                            const f32x4 (&o)[NT][8]) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    char* row = slot[tt * 16 + i];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<f32x4*>(row + (32 * g + 8 * r) * 4) =
          (f32x4){o[tt][0][r], o[tt][1][r], o[tt][2][r], o[tt][3][r]};
      *reinterpret_cast<f32x4*>(row + (32 * g + 8 * r + 4) * 4) =
          (f32x4){o[tt][4][r], o[tt][5][r], o[tt][6][r], o[tt][7][r]};
    }
  }
}
template <int NT>
__device__ __forceinline__ void add_partial(const char (*slot)[kColBytes], int i, int g,
                                            f32x4 (&o)[NT][8]) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const char* row = slot[tt * 16 + i];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(row + (32 * g + 8 * r) * 4);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(row + (32 * g + 8 * r + 4) * 4);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        o[tt][bb][r] += lo[bb];
        o[tt][bb + 4][r] += hi[bb];
      }
    }
  }
}

// FP8: the ring holds E4M3 codes (8-byte operand loads, converted to bf16 in
// registers, exactly); the K scale joins the ring logits' multiplier and the V scale
// multiplies the ring weights as they are packed for P*V (the running sums stay
// unscaled), so no cache element is ever rescaled.
// ROPE: q and the new keys arrive unrotated and are rotated in registers as they are staged.
// COMMIT (with ROPE): one launch per MTP step -- the previous step's first
// prev_accept[b] tokens are committed to the ring (keys rotated at their positions, as the
// ring append does) and the drafts are verified against the ring after that commit.  The
// committed tokens are staged with the new ones (rows 4 .. 7 of the staging, free since
// T <= 4) and rotated there; the first octet of each KV head stores them to the ring from
// the staging registers, and the verify takes their rows from the staging, never from the
// ring slots being rewritten.  ring_head is read and the new head written to
// ring_head_out, so that every workgroup of a sequence sees the head before the commit.
template <int NT, bool FP8, bool ROPE, bool COMMIT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void decode_kernel(DecodeArgs a) {
  static_assert(!COMMIT || ROPE, "the one-launch step rotates the committed keys");
  __shared__ __attribute__((aligned(16))) DecodeSmem<NT> sm;
  const int noct = a.num_q_heads / kHG;
  const int b = blockIdx.x / noct;
  const int oct = blockIdx.x - b * noct;
  const int h_base = oct * kHG;
  const int hkv = a.num_kv_heads;
  const int kvh = h_base / (a.num_q_heads / hkv);
  const int T = a.t_new;
  const int Hq = a.num_q_heads;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  int head = as_const(a.ring_head)[b] % kW;  // scalar load: addresses wait on nothing else
  head += head < 0 ? kW : 0;
  // COMMIT: the verify sees the ring after the commit, whose newest ncommit logical slots
  // hold the previous step's first ncommit tokens
  int ncommit = 0;
  if constexpr (COMMIT) {
    ncommit = as_const(a.prev_accept)[b];
    ncommit = ncommit < 0 ? 0 : (ncommit > a.prev_t ? a.prev_t : ncommit);
    head = (head + ncommit) & (kW - 1);
    if (h_base == 0 && threadIdx.x == 0) a.ring_head_out[b] = head;
  }

  const bf16* qp = static_cast<const bf16*>(a.q);
  using CacheT = typename std::conditional<FP8, uint8_t, bf16>::type;
  const CacheT* kc = static_cast<const CacheT*>(a.k_cache) + ((size_t)b * hkv + kvh) * kW * D;
  const CacheT* vc = static_cast<const CacheT*>(a.v_cache) + ((size_t)b * hkv + kvh) * kW * D;
  // ring operand of 8 elements starting at element e0 of row `phys`.  A decode step reads each ring row once; the
  // layer's next step comes only after every other layer's cache has streamed through, so the bf16 loads carry the
  // non-temporal hint and leave the caches to the rows that are re-read within the step (measured faster at every
  // decode shape; the fp8 loads are 8-byte and were not).
  auto ring8 = [&](const CacheT* row, int e0) -> bf16x8 {
    if constexpr (FP8) return e4m3x8_to_bf16x8(*reinterpret_cast<const u32x2*>(row + e0));
    else return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + e0)));
  };
  // the ring row of logical slot kr (the oldest, which no query sees, replaced by slot 1)
  auto slot_row = [&](const CacheT* ring, int kr) -> const CacheT* {
    const int k2 = kr != 0 ? kr : 1;
    return ring + (size_t)((head + k2) & (kW - 1)) * D;
  };
  const bf16* kn = static_cast<const bf16*>(a.k_new) + ((size_t)b * T * hkv + kvh) * D;
  const bf16* vn = static_cast<const bf16*>(a.v_new) + ((size_t)b * T * hkv + kvh) * D;

  // ---- loads, issued in the order their data is needed: the query columns and the
  // new tokens' K/V (staged once in LDS for the four wavefronts), then ring K (A
  // operands), then ring V rows, which arrive while the scores are formed.  Every load
  // is unconditional and reads a valid row, so no wait is tied to a lane condition:
  // query columns past the T tokens repeat token T-1 (their results are never stored),
  // new-token rows past T repeat row T-1 (weight 0), and the oldest ring slot, which no
  // query sees, is replaced by logical slot 1 (weight 0 as well) and is never read. ----
  const int tid = threadIdx.x;
  // sink of this lane's head (query column i: head i & 7), loaded ahead of the bulk
  const float sink2 = a.sinks[h_base + (i & 7)] * kLog2e;
  const int nrow = min(tid >> 4, T - 1), nuu = tid & 15;  // new token of this thread
  // COMMIT: staging rows 4 .. 4 + ncommit - 1 (past the T <= 4 new tokens, whose logits
  // and weights they do not touch) carry the committed tokens, read from the previous
  // step's K / V; ctok is this thread's committed token, or -1
  const bf16* ksrc = kn + (size_t)nrow * hkv * D;
  const bf16* vsrc = vn + (size_t)nrow * hkv * D;
  int ctok = -1;
  if constexpr (COMMIT) {
    if ((tid >> 4) >= 4 && (tid >> 4) < 4 + ncommit) {
      ctok = (tid >> 4) - 4;
      const size_t off = (((size_t)b * a.prev_t + ctok) * hkv + kvh) * D;
      ksrc = static_cast<const bf16*>(a.prev_k) + off;
      vsrc = static_cast<const bf16*>(a.prev_v) + off;
    }
  }
  u32x4 st[NT + 2];
#pragma unroll
  for (int k = 0; k < NT; ++k) {  // Q column col = x >> 4: token col >> 3, head col & 7
    const int x = k * kThreads + tid;
    const int col = x >> 4, uu = x & 15, t = min(col >> 3, T - 1);
    st[k] = *reinterpret_cast<const u32x4*>(qp + (((size_t)b * T + t) * Hq + h_base + (col & 7)) * D + 8 * uu);
  }
  st[NT] = *reinterpret_cast<const u32x4*>(ksrc + 8 * nuu);
  st[NT + 1] = *reinterpret_cast<const u32x4*>(vsrc + 8 * nuu);
  // K operand of chunk cc: 8 head-dim elements of unit kunit(cc) (8 elements per unit).
  // Unit 4 cc + g, the chunk's 32 dims in order; for an FP8 ring without rotation, unit
  // 2 g + 8 (cc >> 1) + (cc & 1), so that chunks 2h and 2h + 1 of a lane are adjacent codes
  // and one 16-byte load brings both (measured 2% faster there, 5% slower with the rotation
  // in the kernel); the query operands and the new keys take the same units, and the
  // contraction runs over all 128 dims either way.
  constexpr bool kWideK = FP8 && !ROPE;
  auto kunit = [&](int cc) { return kWideK ? 2 * g + 8 * (cc >> 1) + (cc & 1) : 4 * cc + g; };
  bf16x8 kf[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const CacheT* row = slot_row(kc, 32 * w + pair_row(i, s));
    if constexpr (kWideK) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 c16 = *reinterpret_cast<const u32x4*>(row + 64 * h + 16 * g);
        kf[s][2 * h] = e4m3x8_to_bf16x8((u32x2){c16[0], c16[1]});
        kf[s][2 * h + 1] = e4m3x8_to_bf16x8((u32x2){c16[2], c16[3]});
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) kf[s][cc] = ring8(row, 32 * cc + 8 * g);
    }
  }
  bf16x8 vr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) vr[e] = ring8(slot_row(vc, 32 * w + 8 * g + e), 8 * i);
  {
    if constexpr (ROPE) {
      // the rotary cos/sin table (token, pair) is formed while the loads are in
      // flight (it depends on the position only); then each staged 8-element piece of
      // a query column or new-key row is rotated in registers before it is written:
      // element i pairs with i + 64, i.e. piece uu with piece uu ^ 8 of the same row,
      // which sits in the lane 8 away within the 16-lane row (a DPP row rotation by 8)
      // (COMMIT: rows T .. T + ncommit - 1 of the table belong to the committed tokens)
      const int pos0 = as_const(a.rope_pos)[b];
      const int ppos0 = COMMIT ? as_const(a.prev_pos)[b] : 0;
      for (int x = tid; x < (T + ncommit) * 64; x += kThreads) {
        const int tok = x >> 6;
        rope_cos_sin(tok < T ? pos0 + tok : ppos0 + (tok - T), x & 63, D, a.rope_log2_base, &sm.u.in.cs[x][0],
                     &sm.u.in.cs[x][1]);
      }
      __syncthreads();  // the table is complete
      const bool first = (tid & 8) == 0;  // this lane holds x[i], the partner x[i + 64]
      auto rotate = [&](u32x4 v4, int t) -> u32x4 {
        u32x4 p4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          p4[j] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v4[j], 0x128, 0xf, 0xf, false);  // row_ror:8
        const bf16x8 me = __builtin_bit_cast(bf16x8, v4), pa = __builtin_bit_cast(bf16x8, p4);
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = sm.u.in.cs[t * 64 + 8 * (tid & 7) + e][0];
          const float sn = sm.u.in.cs[t * 64 + 8 * (tid & 7) + e][1];
          // this lane holds x[i] (first) or x[i + 64] of pair i: the pair's lo or hi.  The
          // one-launch step keeps the branch per lane, which holds its registers under the
          // budget (the select form spills there); both round the same products.
          if constexpr (COMMIT) {
            float lo, hi;
            if (first) rope_pair((float)me[e], (float)pa[e], c, sn, lo, hi);
            else rope_pair((float)pa[e], (float)me[e], c, sn, lo, hi);
            y[e] = (bf16)(first ? lo : hi);
          } else {
            y[e] = (bf16)rope_own((float)me[e], (float)pa[e], c, sn, first);
          }
        }
        return __builtin_bit_cast(u32x4, y);
      };
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        const int col = (k * kThreads + tid) >> 4;
        st[k] = rotate(st[k], min(col >> 3, T - 1));
      }
      st[NT] = rotate(st[NT], ctok >= 0 ? T + ctok : nrow);
      if constexpr (COMMIT) {
        // the first octet of the KV head commits the staged tokens: token ctok to logical
        // slot kW - ncommit + ctok of the ring after the commit, the key as just rotated.
        // FP8: the ring takes the E4M3 codes of key / k_scale and value / v_scale (as the
        // FP8 ring append encodes them), and the staged rows become the codes' values,
        // which is what the verify reads for every other ring slot.
        const bool writer = ctok >= 0 && h_base == kvh * (Hq / hkv);
        const size_t dst = (size_t)((head + kW - ncommit + ctok) & (kW - 1)) * D + 8 * nuu;
        if constexpr (FP8) {
          if (ctok >= 0) {
            const bf16x8 kx = __builtin_bit_cast(bf16x8, st[NT]), vx = __builtin_bit_cast(bf16x8, st[NT + 1]);
            const double ks = a.k_scale, vs = a.v_scale;
            uint64_t kw = 0, vw = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              kw |= (uint64_t)e4m3_encode(kx[e], ks) << (8 * e);
              vw |= (uint64_t)e4m3_encode(vx[e], vs) << (8 * e);
            }
            if (writer) {
              *reinterpret_cast<uint64_t*>(const_cast<CacheT*>(kc) + dst) = kw;
              *reinterpret_cast<uint64_t*>(const_cast<CacheT*>(vc) + dst) = vw;
            }
            st[NT] = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(__builtin_bit_cast(u32x2, kw)));
            st[NT + 1] = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(__builtin_bit_cast(u32x2, vw)));
          }
        } else if (writer) {
          *reinterpret_cast<u32x4*>(const_cast<CacheT*>(kc) + dst) = st[NT];
          *reinterpret_cast<u32x4*>(const_cast<CacheT*>(vc) + dst) = st[NT + 1];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const int x = k * kThreads + tid;
      *reinterpret_cast<u32x4*>(&sm.u.in.q[x >> 4][16 * (x & 15)]) = st[k];
    }
    *reinterpret_cast<u32x4*>(&sm.u.in.kn[tid >> 4][16 * nuu]) = st[NT];
    *reinterpret_cast<u32x4*>(&sm.vn[tid >> 4][16 * nuu]) = st[NT + 1];
  }
  int tcol[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) tcol[tt] = 2 * tt + (i >> 3);
  __syncthreads();
  // B operand (Q^T) of tile tt, head-dim chunk cc: column tt*16 + i, unit kunit(cc)
  auto qop = [&](int tt, int cc) {
    return *reinterpret_cast<const bf16x8*>(&sm.u.in.q[tt * 16 + i][16 * kunit(cc)]);
  };

  const float c = a.scale * kLog2e;       // new tokens' logits to log2 units
  const float cr = FP8 ? c * a.k_scale : c;  // the ring's
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  if constexpr (COMMIT) {
    // wavefront 3's slots kW - ncommit .. kW - 1 are the committed tokens: their keys (as
    // rotated in staging) replace the ring rows loaded for them, which the commit rewrites
    if (w == 3 && ncommit > 0) {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const int tc = 96 + pair_row(i, ss) - (kW - ncommit);
        if (tc >= 0) {
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
            kf[ss][cc] = *reinterpret_cast<const bf16x8*>(&sm.u.in.kn[4 + tc][16 * kunit(cc)]);
        }
      }
    }
  }

  // ---- scores ----
  f32x4 s[NT][2], sn[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      s[tt][ss] = zero4;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) s[tt][ss] = mfma32(kf[ss][cc], qop(tt, cc), s[tt][ss]);
    }
    sn[tt] = zero4;
    if (w == 0) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        sn[tt] = mfma32(*reinterpret_cast<const bf16x8*>(&sm.u.in.kn[i][16 * kunit(cc)]), qop(tt, cc), sn[tt]);
    }
  }

  // ---- mask (ring slot kr visible to token t iff kr >= t+1; new token u iff u <= t) ----
  float mx[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    float mr = -INFINITY, mn = -INFINITY;  // raw maxima of the ring and new-token logits
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (w == 0) {
          const int kr = 8 * g + 4 * ss + r;
          s[tt][ss][r] = kr >= tcol[tt] + 1 ? s[tt][ss][r] : -INFINITY;
        }
        mr = fmaxf(mr, s[tt][ss][r]);
      }
    if (w == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = 4 * g + r;
        sn[tt][r] = (u <= tcol[tt] && u < T) ? sn[tt][r] : -INFINITY;
        mn = fmaxf(mn, sn[tt][r]);
      }
    }
    mx[tt] = quad_max(fmaxf(mr * cr, mn * c));  // both multipliers are > 0
    if (g == 0) sm.m[w][tt * 16 + i] = mx[tt];
  }
  __syncthreads();

  // ---- common maximum (sink included), exponentiate, partial sums ----
  float mcol[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int col = tt * 16 + i;
    mcol[tt] = fmaxf(fmaxf(fmaxf(sm.m[0][col], sm.m[1][col]), fmaxf(sm.m[2][col], sm.m[3][col])), sink2);
    float ps = 0.f;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[tt][ss][r] = fast_exp2(fmaf(s[tt][ss][r], cr, -mcol[tt]));
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
    if (w == 0 && g == 0) {
      sm.mc[col] = mcol[tt];
      sm.zs[col] = fast_exp2(sink2 - mcol[tt]);
    }
  }

  if constexpr (COMMIT) {  // likewise the committed values, from their staging rows
    if (w == 3 && ncommit > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tc = 96 + 8 * g + e - (kW - ncommit);
        if (tc >= 0) vr[e] = *reinterpret_cast<const bf16x8*>(&sm.vn[4 + tc][16 * i]);
      }
    }
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
    for (int tt = 0; tt < NT; ++tt) {
      if constexpr (FP8)
        o[tt][bb] = mfma32(av, pack_pair(s[tt][0] * a.v_scale, s[tt][1] * a.v_scale), o[tt][bb]);
      else
        o[tt][bb] = mfma32(av, pack_pair(s[tt][0], s[tt][1]), o[tt][bb]);
    }
  }
  if (w == 0) {
    bf16x8 vrn[4];  // V rows of new tokens 4g .. 4g+3, head-dim 8i .. 8i+7
#pragma unroll
    for (int e = 0; e < 4; ++e) vrn[e] = *reinterpret_cast<const bf16x8*>(&sm.vn[4 * g + e][16 * i]);
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const bf16x4 av = column4(vrn, bb);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) o[tt][bb] = mfma32_k16(av, pack_quad(sn[tt]), o[tt][bb]);
    }
  }
  // ---- merge the four partials (they share the column maxima, so they add) ----
  if constexpr (kMergeSlots<NT> == 4) {
    put_partial<NT>(sm.u.o[w], i, g, o);
  } else {  // wavefronts 2, 3 hand theirs to 0, 1, which write back the pair sums
    if (w >= 2) put_partial<NT>(sm.u.o[w - 2], i, g, o);
    __syncthreads();
    if (w < 2) {
      add_partial<NT>(sm.u.o[w], i, g, o);
      put_partial<NT>(sm.u.o[w], i, g, o);
    }
  }
  __syncthreads();

  // ---- normalise and store, all threads: thread tid owns kPer head-dim elements of one
  // query column (qc = token * 8 + head) as kPer / 8 runs of 8, run q8 starting at
  // d0 + 8 * kCol * q8, so that each store instruction's kCol threads of a column write
  // one contiguous stretch of the output row (whole 128-byte lines per instruction) ----
  constexpr int kPer = NT * 16 * D / kThreads;  // 8 or 16
  constexpr int kCol = D / kPer;                 // threads per output row
  const int qc = tid / kCol;
  const int d0 = (tid % kCol) * 8;
  const int t = qc >> 3;
  if (t >= T) return;
  float acc[kPer];
#pragma unroll
  for (int q4 = 0; q4 < kPer / 4; ++q4) {
    const int e0 = d0 + (q4 >> 1) * 8 * kCol + 4 * (q4 & 1);
    f32x4 v = *reinterpret_cast<const f32x4*>(&sm.u.o[0][qc][4 * e0]);
#pragma unroll
    for (int sl = 1; sl < kMergeSlots<NT>; ++sl) v += *reinterpret_cast<const f32x4*>(&sm.u.o[sl][qc][4 * e0]);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[4 * q4 + e] = v[e];
  }
  const float z = sm.l[0][qc] + sm.l[1][qc] + sm.l[2][qc] + sm.l[3][qc] + sm.zs[qc];
  const float inv = __builtin_amdgcn_rcpf(z);
  const size_t row_idx = ((size_t)b * T + t) * Hq + h_base + (qc & 7);
  bf16* out = static_cast<bf16*>(a.out) + row_idx * D + d0;
#pragma unroll
  for (int q8 = 0; q8 < kPer / 8; ++q8) {
    bf16x8 v8;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 x = __builtin_convertvector((f32x2){acc[8 * q8 + e] * inv, acc[8 * q8 + e + 1] * inv}, bf16x2);
      v8[e] = x[0];
      v8[e + 1] = x[1];
    }
    // written once and read by the next kernel long after: streamed past the caches.  With these stores a
    // line that one instruction covers only in part reaches HBM as separate partial writes (half lines
    // per instruction measured 1.6x the output's bytes), hence the run layout above.
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v8), reinterpret_cast<u32x4*>(out + 8 * kCol * q8));
  }
  if (a.lse != nullptr && d0 == 0) a.lse[row_idx] = (sm.mc[qc] + fast_log2(z)) * kLn2;
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a, bool bf16_io) {
  // (an FP8 ring takes the same path: only the cache element type differs)
  const int G = a.num_q_heads / a.num_kv_heads;
  // the one-launch MTP step: rotation and at most 4 committed tokens (wavefront 3's newest
  // slots)
  if (a.prev_accept != nullptr && (a.rope_pos == nullptr || a.prev_t < 1 || a.prev_t > 4)) return false;
  return bf16_io && a.head_dim == 128 && G % kHG == 0 && a.window == kW && a.t_new >= 1 &&
         a.t_new <= 4;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  const long blocks = (long)a.batch * (a.num_q_heads / kHG);
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const bool two = a.t_new > 2;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (a.prev_accept != nullptr) {  // one-launch MTP step (rotation)
    if (a.cache_fp8) {
      if (two) hipLaunchKernelGGL((decode_kernel<2, true, true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_kernel<1, true, true, true>), grid, block, 0, s, a);
    } else {
      if (two) hipLaunchKernelGGL((decode_kernel<2, false, true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_kernel<1, false, true, true>), grid, block, 0, s, a);
    }
  } else if (a.rope_pos != nullptr) {  // rotation in the kernel
    if (a.cache_fp8) {
      if (two) hipLaunchKernelGGL((decode_kernel<2, true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_kernel<1, true, true>), grid, block, 0, s, a);
    } else {
      if (two) hipLaunchKernelGGL((decode_kernel<2, false, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((decode_kernel<1, false, true>), grid, block, 0, s, a);
    }
  } else if (a.cache_fp8) {
    if (two) hipLaunchKernelGGL((decode_kernel<2, true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<1, true, false>), grid, block, 0, s, a);
  } else {
    if (two) hipLaunchKernelGGL((decode_kernel<2, false, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<1, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace swa
