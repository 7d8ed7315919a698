// Device-side building blocks shared by the SageSLA kernels (gfx950).
//
// MFMA conventions used throughout (CDNA3/CDNA4 16x16 matrix instructions):
//  * v_mfma_i32_16x16x64_i8 : A, B are 16 bytes per lane; lane l carries row
//    (A) / column (B) l%16 and the k-slice of lane group g = l/16.
//  * v_mfma_f32_16x16x32_bf16 : A, B are 8 bf16 per lane, same lane roles.
//  * 16x16 accumulators: lane l holds column l%16 and rows 4*(l/16) + r,
//    r = 0..3.
// The kernels only rely on A and B pairing lane group g / element e with the
// same k, so every layout below is chosen freely to make loads contiguous.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

constexpr int BLK = 64;  // query and key block size

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  v2f v = {a, b};
  v2bf r = __builtin_convertvector(v, v2bf);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16(v4u a, v4u b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// 32x32x16 bf16: lane l holds A[l%32][8(l/32) .. +7] and B[8(l/32) .. +7][l%32];
// accumulator register r of lane l is D[8(r/4) + 4(l/32) + r%4][l%32].
__device__ __forceinline__ v16f mfma32_bf16(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Layouts (byte / element offsets inside one 64-row block)
// ---------------------------------------------------------------------------

// INT8 block [64 rows][D], fragment order for v_mfma_i32_16x16x64_i8:
// fragment (row tile rt = r/16, chunk kc = c/64) is 1 KiB; lane (r%16) +
// 16*((c%64)/16) holds 16 consecutive channels.
__host__ __device__ __forceinline__ int i8_off(int r, int c, int KC) {
  return ((((r >> 4) * KC + (c >> 6)) * 64 + (r & 15) + 16 * ((c & 63) >> 4)) << 4) + (c & 15);
}

// bf16 block [64 rows][D] as the A operand of v_mfma_f32_16x16x32_bf16 with k =
// channel: fragment (row tile rt = r/16, chunk kc = c/32) is 1 KiB; lane
// (r%16) + 16*((c%32)/8) holds the 8 consecutive channels.  Element offset:
__host__ __device__ __forceinline__ int bfk_off(int r, int c, int KC32) {
  return ((((r >> 4) * KC32 + (c >> 5)) * 64 + (r & 15) + 16 * ((c & 31) >> 3)) << 3) + (c & 7);
}

// bf16 operand whose k index runs over 64 block rows (keys), fragment order for
// v_mfma_f32_16x16x32_bf16 with the 16 "rows" being channels: fragment
// (kc2 = s/32, cg = c/16) is 1 KiB; lane (c%16) + 16*g holds the 8 keys
// 32*kc2 + 16*(e/4) + 4*g + e%4, e = 0..7.  This k order is the one in which
// a 16x16 accumulator tile pair (rows 4g + r of tiles 2*kc2 and 2*kc2+1)
// already sits in a lane, so softmax probabilities feed the next product
// straight from registers.  Element offset of (key s, channel c):
__host__ __device__ __forceinline__ int kmaj_off(int s, int c, int CG) {
  int kc2 = s >> 5, sl = s & 31;
  int e = ((sl >> 4) << 2) | (sl & 3);
  int g = (sl >> 2) & 3;
  return ((kc2 * CG + (c >> 4)) * 64 + (c & 15) + 16 * g) * 8 + e;
}

// d x d matrix M[row][k] as A operand of v_mfma_f32_16x16x32_bf16 with the k
// order of kmaj_off: fragment (x = row/16, kc = k/32); element offset:
__host__ __device__ __forceinline__ int wfrag_off(int row, int k, int KC32) {
  int kc = k >> 5, kl = k & 31;
  int e = ((kl >> 4) << 2) | (kl & 3);
  int g = (kl >> 2) & 3;
  return (((row >> 4) * KC32 + kc) * 64 + (row & 15) + 16 * g) * 8 + e;
}

// Per-query-block linear state H (phi-channel c, value channel c2) as A operand
// of v_mfma_f32_16x16x32_bf16 computing O_l^T = H^T phi(Q)^T: fragment
// (x = c2/16, kc = c/32); lane (c2%16) + 16*((c%32)/8) holds the 8 consecutive
// phi channels (c%32)/8*8 .. +7.  z follows at element D*D + c.
__host__ __device__ __forceinline__ int hstate_off(int c, int c2, int KC32) {
  return (((c2 >> 4) * KC32 + (c >> 5)) * 64 + (c2 & 15) + 16 * ((c & 31) >> 3)) * 8 + (c & 7);
}

// ---------------------------------------------------------------------------
// LDS operand reads (row-major bf16 tiles)
// ---------------------------------------------------------------------------

typedef short v4s16 __attribute__((ext_vector_type(4)));

// Four consecutive rows k0 .. k0+3 of column n0 + l%16 of a row-major bf16
// LDS tile (pitch in elements), by the transposing LDS read: lane j of each
// 16-lane group supplies row k0 + j/4, columns n0 + 4(j%4) .. +3.
__device__ __forceinline__ uint2 lds_col4(const uint16_t *tile, int pitch, int k0, int n0,
                                          int lane) {
  const int j = lane & 15;
  const uint16_t *a = tile + (k0 + (j >> 2)) * pitch + n0 + 4 * (j & 3);
  const v4s16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s16 *)a);
  return __builtin_bit_cast(uint2, r);
}

// MFMA operand (16x16x32 bf16, k order of kmaj_off) of the 16 columns n0 ..
// n0+15 and the 32 keys 32 kc2 .. of a row-major [key][column] LDS tile: lane
// (column n0 + l%16, group g = l/16) holds keys 32 kc2 + 4g + 0..3 and
// 32 kc2 + 16 + 4g + 0..3.
__device__ __forceinline__ v4u lds_frag(const uint16_t *tile, int pitch, int kc2, int n0, int lane) {
  const int g = lane >> 4;
  const uint2 lo = lds_col4(tile, pitch, 32 * kc2 + 4 * g, n0, lane);
  const uint2 hi = lds_col4(tile, pitch, 32 * kc2 + 16 + 4 * g, n0, lane);
  return v4u{lo.x, lo.y, hi.x, hi.y};
}

// MFMA operand (16x16x32 bf16) of the 16 rows r0 .. r0+15 of a row-major
// [row][k] LDS tile, in the same k order as lds_frag: lane (row r0 + l%16,
// group g) holds k = 32 kc + 4g + 0..3 and 32 kc + 16 + 4g + 0..3.
__device__ __forceinline__ v4u lds_rows(const uint16_t *tile, int pitch, int r0, int kc, int lane) {
  const uint16_t *a = tile + (r0 + (lane & 15)) * pitch + 32 * kc + 4 * (lane >> 4);
  const uint2 lo = *(const uint2 *)a;
  const uint2 hi = *(const uint2 *)(a + 16);
  return v4u{lo.x, lo.y, hi.x, hi.y};
}

// Workgroup id -> logical id so that consecutive logical ids share an XCD
// (workgroups are dispatched round robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  int q = nblocks >> 3, r = nblocks & 7;
  int x = bid & 7, local = bid >> 3;
  return x * q + (x < r ? x : r) + local;
}

}  // namespace sla
