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
//  * V operands of P*V are read from LDS with ds_read_b64_tr_b16 (see tr_read).
#pragma once

#include "common.h"

namespace swa {
namespace tile {

constexpr int D = 128;
constexpr int kRowBytes = D * 2;
constexpr int kUnitsPerRow = kRowBytes / 16;

// Row (relative to the pair's first key) that MFMA row `row` of block s reads.
__device__ __forceinline__ int pair_row(int row, int s) { return 8 * (row >> 2) + 4 * s + (row & 3); }

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// A k=16 product (four k-slots per lane group) issued as the k=32 instruction with
// the other four k-slots zero in both operands.  Every accumulation chain then uses
// a single MFMA shape: a 16x16x16 result taken as the accumulator of a 16x16x32
// one wait state later has produced stale rows 2-3 on gfx950, and the compiler
// does not pad that dependency.
__device__ __forceinline__ f32x4 mfma32_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  const bf16 z = (bf16)0.f;
  return mfma32((bf16x8){a[0], a[1], a[2], a[3], z, z, z, z}, (bf16x8){b[0], b[1], b[2], b[3], z, z, z, z}, c);
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

// K tiles in LDS: four planes (one per 32-element head-dim chunk) of 64-byte rows;
// the 16-byte unit of lane group g sits at g ^ kswz(key), so the 16 rows an MFMA
// operand read touches fall on 16 distinct bank quads (for any 16-aligned run of
// keys, in the pair order of pair_row and in the order of pi8).
__device__ __forceinline__ int kswz(int key) { return ((key >> 3) ^ (key >> 2)) & 3; }
__device__ __forceinline__ void put_k(char* ks, int plane_bytes, int row, int key, int u, u32x4 x) {
  *reinterpret_cast<u32x4*>(ks + (u >> 2) * plane_bytes + row * 64 + 16 * ((u & 3) ^ kswz(key))) = x;
}

// V tiles in LDS: rows of 264 bytes (256 + 8, so consecutive rows shift banks by
// 8 bytes), read with ds_read_b64_tr_b16.  Within each 16-lane group, lane 4e+m
// addresses 4 consecutive head-dim elements of key row e and lane 4m'+c receives
// element c of rows e = 0..3 addressed by group member m' -- a 4x4 transpose that
// yields the k-contiguous V^T operand.  Head-dim quad m of output block b starts
// at qoff(m, b); the O^T result then holds head-dim 64(g>>1) + 16(g&1) + {0..15}
// and the same + 32 in lane group g.
constexpr int kVPitch = 264;
__device__ __forceinline__ void put_v(char* vs, int row, int u, u32x4 x) {
  char* p = vs + row * kVPitch + 16 * u;
  *reinterpret_cast<u32x2*>(p) = (u32x2){x[0], x[1]};
  *reinterpret_cast<u32x2*>(p + 8) = (u32x2){x[2], x[3]};
}
// Byte offset of quad (i & 3) of block 0 within a V row: lane-constant part.
__device__ __forceinline__ int vquad_bytes(int i) { return 2 * (64 * ((i & 3) >> 1) + 16 * (i & 1)); }
// Byte offset added for output block b (compile-time after unrolling).
__device__ __forceinline__ int vblock_bytes(int b) { return 2 * (32 * (b >> 2) + 4 * (b & 3)); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 tr_read(const char* vs, int off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + off));
  return __builtin_bit_cast(bf16x4, r);
}

// MFMA row -> key order of a single (unpaired) 16-key block: lane groups 0/1 get
// keys 0-3 / 8-11 so that their transposed V reads fall on different banks.
__device__ __forceinline__ int pi8(int i) { return 8 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// Store the 32 head-dim values of one query row held by lane group g (O^T layout
// of the transposed V reads), scaled by inv and rounded to bf16.
__device__ __forceinline__ void store_row_tr(bf16* row, int g, const f32x4 (&o)[8], float inv) {
  const int d0 = 64 * (g >> 1) + 16 * (g & 1);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      bf16x8 v;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int b = 4 * half + 2 * q + bb;
        bf16x2 lo = __builtin_convertvector((f32x2){o[b][0] * inv, o[b][1] * inv}, bf16x2);
        bf16x2 hi = __builtin_convertvector((f32x2){o[b][2] * inv, o[b][3] * inv}, bf16x2);
        v[4 * bb + 0] = lo[0]; v[4 * bb + 1] = lo[1];
        v[4 * bb + 2] = hi[0]; v[4 * bb + 3] = hi[1];
      }
      *reinterpret_cast<bf16x8*>(row + d0 + 32 * half + 8 * q) = v;
    }
  }
}

}  // namespace tile
}  // namespace swa
