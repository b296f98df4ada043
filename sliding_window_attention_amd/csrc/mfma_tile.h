// Building blocks of the matrix-core attention kernels (bf16, head_dim 128).
//
// Layout conventions (one wavefront, lane l, i = l & 15, g = l >> 4):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16:
//    A = 16 key rows x 32 head-dim, B = 32 head-dim x 16 queries.  The result
//    holds, in lane (i, g), query i against key rows 4g .. 4g+3 of the block, so a
//    query's softmax statistics need only a reduction over the four lanes
//    i, i+16, i+32, i+48.
//  * Keys come in pairs of 16-key blocks covering 32 keys.  Block s (0/1) of a
//    pair puts key 8*(row/4) + 4*s + row%4 of the pair on MFMA row `row`, so that
//    lane (i, g) ends up with keys 8g .. 8g+7 of the pair: exactly the k-slice the
//    B operand of the P*V product needs.  P therefore feeds the second product
//    straight from the score registers.
//  * O^T = V^T P^T is accumulated per 16-row block b of head-dim with row r of
//    block b standing for head-dim element 8r + b.  Lane (i, g) then holds
//    head-dim 32g .. 32g+31 of query i (element 32g + 8r + b in register r of
//    block b), which is 64 contiguous output bytes.
//  * K and V tiles live in LDS as 256-byte rows (128 bf16) whose 16-byte units are
//    XOR-swizzled per row (unit u of row r at u ^ swz(r)); every access pattern
//    below touches 16 distinct units per 16 lanes, i.e. no bank conflicts.
#pragma once

#include "common.h"

namespace swa {
namespace tile {

constexpr int D = 128;
constexpr int kRowBytes = D * 2;
constexpr int kUnitsPerRow = kRowBytes / 16;

__device__ __forceinline__ int swz(int r) {
  return (r & 3) | ((((r >> 3) ^ (r >> 2)) & 3) << 2);
}
__device__ __forceinline__ int lds_off(int r, int u) { return r * kRowBytes + ((u ^ swz(r)) << 4); }

__device__ __forceinline__ bf16x8 lds_read8(const char* base, int r, int u) {
  return *reinterpret_cast<const bf16x8*>(base + lds_off(r, u));
}

// Row (relative to the pair's first key) that MFMA row `row` of block s reads.
__device__ __forceinline__ int pair_row(int row, int s) { return 8 * (row >> 2) + 4 * s + (row & 3); }

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
  return z;
}

// Pack the two score blocks of a pair (already exponentiated) into the P^T operand.
__device__ __forceinline__ bf16x8 pack_pair(f32x4 lo, f32x4 hi) {
  bf16x2 a = __builtin_convertvector((f32x2){lo[0], lo[1]}, bf16x2);
  bf16x2 b = __builtin_convertvector((f32x2){lo[2], lo[3]}, bf16x2);
  bf16x2 c = __builtin_convertvector((f32x2){hi[0], hi[1]}, bf16x2);
  bf16x2 d = __builtin_convertvector((f32x2){hi[2], hi[3]}, bf16x2);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ bf16x4 pack_quad(f32x4 x) {
  bf16x2 a = __builtin_convertvector((f32x2){x[0], x[1]}, bf16x2);
  bf16x2 b = __builtin_convertvector((f32x2){x[2], x[3]}, bf16x2);
  return (bf16x4){a[0], a[1], b[0], b[1]};
}

// Column e of an 8x8 bf16 block held as 8 row vectors: {rows[0][e], ..., rows[7][e]}.
__device__ __forceinline__ bf16x8 column8(const bf16x8* rows, int e) {
  return (bf16x8){rows[0][e], rows[1][e], rows[2][e], rows[3][e],
                  rows[4][e], rows[5][e], rows[6][e], rows[7][e]};
}
__device__ __forceinline__ bf16x4 column4(const bf16x8* rows, int e) {
  return (bf16x4){rows[0][e], rows[1][e], rows[2][e], rows[3][e]};
}

// O^T += V^T P^T over one 32-key pair for two query tiles.  `vs` is the LDS V
// tile, `r0` the first row of the pair.  Lane (i, g) reads V rows r0 + 8g + e
// (e = 0..7) at 16-byte unit i: head-dim 8i .. 8i+7 of its 8 keys; the 8x8
// transpose turns them into the A operands of the 8 head-dim blocks.
__device__ __forceinline__ void pv_pair(const char* vs, int r0, int i, int g, bf16x8 p0, bf16x8 p1,
                                        f32x4 (&o0)[8], f32x4 (&o1)[8]) {
  bf16x8 vr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) vr[e] = lds_read8(vs, r0 + 8 * g + e, i);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bf16x8 a = column8(vr, b);
    o0[b] = mfma32(a, p0, o0[b]);
    o1[b] = mfma32(a, p1, o1[b]);
  }
}

// Same for a single 16-key block (k = 16 product); lane (i, g) holds keys 4g..4g+3.
__device__ __forceinline__ void pv_single(const char* vs, int r0, int i, int g, bf16x4 p0, bf16x4 p1,
                                          f32x4 (&o0)[8], f32x4 (&o1)[8]) {
  bf16x8 vr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) vr[e] = lds_read8(vs, r0 + 4 * g + e, i);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bf16x4 a = (bf16x4){vr[0][b], vr[1][b], vr[2][b], vr[3][b]};
    o0[b] = mfma16(a, p0, o0[b]);
    o1[b] = mfma16(a, p1, o1[b]);
  }
}

// Store 32 head-dim values (32g .. 32g+31) of one query row, scaled by inv, as bf16.
__device__ __forceinline__ void store_row32(bf16* dst, const f32x4 (&o)[8], float inv) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    bf16x8 v;
#pragma unroll
    for (int b = 0; b < 8; b += 2) {
      bf16x2 t = __builtin_convertvector((f32x2){o[b][r] * inv, o[b + 1][r] * inv}, bf16x2);
      v[b] = t[0];
      v[b + 1] = t[1];
    }
    *reinterpret_cast<bf16x8*>(dst + 8 * r) = v;
  }
}

}  // namespace tile
}  // namespace swa
