// Pieces of the MFMA attention tiles of the chunked prefill: stored-row
// chunks widened to bf16 (K) or fp16 (V), the 16x16x32 bf16 and fp16 MFMAs,
// lane reductions over the four 16-lane groups, and the padded V tile in LDS
// read back transposed.
#pragma once

#include "hws_device.h"

namespace hws {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr int V_STRIDE = 144;     // padded row of a V tile in LDS (288 B: 4 rows hit 4 bank groups)

// 8 elements of a row as stored: 16 bytes of bf16 or 8 bytes of e4m3 codes
template <bool FP8> struct KvChunk { typedef u32x4 T; };
template <> struct KvChunk<true> { typedef u32x2 T; };

__device__ __forceinline__ u32x4 chunk_bf16(u32x4 w) { return w; }

// 8 e4m3 codes -> 8 bf16 (exact; the conversion's scale operand is 1)
__device__ __forceinline__ u32x4 chunk_bf16(u32x2 w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  auto cvt = [](unsigned x, bool hi) {
    return hi ? __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true))
              : __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
  };
  return u32x4{cvt(w[0], false), cvt(w[0], true), cvt(w[1], false), cvt(w[1], true)};
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 fp32 values -> 8 fp16 bit patterns (round to nearest even), as a 16-byte chunk
__device__ __forceinline__ u32x4 chunk_f16(const float (&x)[8]) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x[2 * k], x[2 * k + 1]}, f16x2));
  return r;
}

// A stored V chunk (8 bf16 values, or 8 e4m3 codes times the page's V scale)
// as fp16: exact for bf16 values of magnitude 2^-14 .. 65504
__device__ __forceinline__ u32x4 chunk_v_f16(u32x4 w, float) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
  return chunk_f16(x);
}
__device__ __forceinline__ u32x4 chunk_v_f16(u32x2 w, float vs) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    f32x2 t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
    x[4 * k] = t.x * vs; x[4 * k + 1] = t.y * vs;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
    x[4 * k + 2] = t.x * vs; x[4 * k + 3] = t.y * vs;
  }
  return chunk_f16(x);
}

__device__ __forceinline__ bf16x8 zero8() { return (bf16x8)(__bf16)0.f; }

// Reductions over lanes i, i^16, i^32 with the gfx950 lane swaps (each call
// returns the value pair {v[i], v[i^16]} or {v[i], v[i^32]} in some order).
__device__ __forceinline__ float max_x16_x32(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_x16_x32(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A operand V^T (16 dims x 32 keys, fp16) for O^T += V^T P^T from a V tile
// stored [key][dim] with rows of V_STRIDE: dims 16 db.., keys 32 ks.. of the tile.
// The transposing reads (ds_read_b64_tr_b16): within each 16-lane group, lane
// i gets element i % 4 of the 8-byte chunks addressed by lanes 4j + i / 4
// (j = 0..3); lane k addresses dims 16db + 4 (k % 4) .. + 3 of key k / 4 of
// the quad's 4 keys, so lane i (= col) receives dim 16db + i of those 4 keys:
// keys 32ks + 4 quad + 0..3, then + 16.  This is the key order in which a
// lane of the S^T accumulator holds its P values (see pack_p).
__device__ __forceinline__ f16x8 vt_frag(const uint16_t* vtile, int ks, int db, int col, int quad) {
  const uint16_t* base = vtile + (32 * ks + 4 * quad + (col >> 2)) * V_STRIDE + 16 * db + 4 * (col & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)base);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(base + 16 * V_STRIDE));
  return __builtin_bit_cast(f16x8, (v8i16){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

}  // namespace hws
