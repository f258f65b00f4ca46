// Device helpers for the gfx950 kernels (wave64).
#pragma once

#include "hws_internal.h"

namespace hws {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// K pages are stored blocked by 32 dims: element (row r, dim d) of a page
// (16 rows x 128 dims) sits at ((d / 32) * 16 + r) * 32 + d % 32.  One
// 32-dim block of all 16 rows is then one contiguous 1 KiB (bf16) run, which
// is exactly one MFMA B-operand load of a wave, and a single row is still
// four whole 64-byte pieces.  V pages stay row-major.
__device__ __forceinline__ int kpage_off(int r, int d) { return (((d >> 5) << 4) + r) * 32 + (d & 31); }

// 16-byte load that does not allocate in the caches (data streamed once).
__device__ __forceinline__ u32x4 load_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 8 e4m3 codes -> 8 bf16, element e from byte e (exact: every e4m3 value is a
// bf16 value, and the conversion's scale operand is 1).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Full-dim scores over a K page (16 rows, blocked by 32 dims) with four
// 16x16x32 MFMA steps: lane (row, quad) supplies 8 dims of row `row` to each
// step t, and the query operand must enumerate the same dims.  bf16 pages:
// step t takes dims 32t .. 32t + 31, 8 per quad (one 16-byte load per step).
// e4m3 pages: a lane reads 16 codes at once, dims 32s + 16 (quad & 1) .. + 15
// of 32-dim block s = quad >> 1 (load 0) and s = 2 + (quad >> 1) (load 1);
// step t takes the low (t even) or high 8 codes of load t >> 1.
template <bool FP8>
__device__ __forceinline__ int mfma_dim0(int t, int quad) {
  if constexpr (FP8) return 32 * (2 * (t >> 1) + (quad >> 1)) + 16 * (quad & 1) + 8 * (t & 1);
  else return 32 * t + 8 * quad;
}

// Byte offset of this lane's first 16 codes in an e4m3 K page; the second
// load is 1024 bytes further.
__device__ __forceinline__ int fp8_page_lane_off(int row, int quad) {
  return (quad >> 1) * 512 + row * 32 + (quad & 1) * 16;
}

// The B operand of step t from the lane's two 16-byte loads of an e4m3 page.
__device__ __forceinline__ bf16x8 fp8_step(const u32x4& w, int t) {
  return (t & 1) ? fp8x8_to_bf16x8((u32x2){w[2], w[3]}) : fp8x8_to_bf16x8((u32x2){w[0], w[1]});
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 bits with a single rounding (nearest even) from the double.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  // bf16 keeps 7 explicit mantissa bits; a double has 52 -> drop 45 bits.
  u += ((1ull << 44) - 1ull) + ((u >> 45) & 1ull);
  u &= ~((1ull << 45) - 1ull);
  float f = (float)__longlong_as_double((long long)u);   // exact: value is bf16-representable
  return (uint16_t)(__float_as_uint(f) >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over the 16 lanes of a row (lanes 16r..16r+15), in every lane of the
// row: two quad swaps, then rotations of the row by 4 and by 8 (DPP moves, no
// LDS).  Quads 0/2 and 1/3 associate the four quad sums differently, so the
// lanes may differ in the last bit.
__device__ __forceinline__ float row16_sum(float a) {
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x124, 0xF, 0xF, false));  // row_ror 4
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x128, 0xF, 0xF, false));  // row_ror 8
  return a;
}

// The values of lanes i and i^16 (X16) or i and i^32 (X32), in a lane-dependent
// but register-independent order: a and b come from the same two lanes for
// every call, so symmetric combines of several registers stay consistent.
template <int X>
__device__ __forceinline__ void lane_pair(float v, float& a, float& b) {
  static_assert(X == 16 || X == 32, "lane swaps exist for 16 and 32");
  const unsigned int u = __float_as_uint(v);
  if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

// OCP e4m3fn encode of an fp32 value: saturate to +-448, round to nearest
// even, sign copied from the input.
__device__ __forceinline__ uint8_t e4m3_encode(float y) {
  uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  float a = fminf(fabsf(y), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8 (8 = smallest normal)
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);        // round mantissa to 3 bits
    uint32_t e = (u >> 23) - 127u + 7u;
    uint32_t m = (u >> 20) & 7u;
    code = (e << 3) | m;
  }
  return (uint8_t)(sign | code);
}

// Combine two (max, sum) pairs of a log2-sum-exp2.
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == NEG_INF) { m = mn; s = 0.f; return; }
  s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
  m = mn;
}

__device__ __forceinline__ unsigned long long load_u64_coherent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned int load_u32_coherent(const unsigned int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_f32_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_f32_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cross-workgroup hand-off without a device-wide fence.  A device-scope
// fence on this chip writes back and invalidates the whole L2 of the XCD,
// serialised across workgroups, so the hand-offs here use only data that is
// coherent at device scope by construction (device-scope atomics and
// agent-scope atomic stores/loads, which bypass the non-coherent cache
// levels).  The writer waits for its outstanding memory operations to be
// acknowledged before it bumps the arrival counter; the reader reads the
// data with agent-scope atomic loads after it has seen the counter.
__device__ __forceinline__ void wait_memory_ops() { __builtin_amdgcn_s_waitcnt(0); }

// Add the fixed-point mass round(a * 2^40) of this thread's kept tokens
// (bit u of `keep` marks av[u]) to *acc: a sum over the wave, then one
// device-scope atomic per wave.  Integer sums do not depend on the order in
// which the waves add them.
template <int N>
__device__ __forceinline__ void add_kept_mass(unsigned long long* acc, const float (&av)[N], unsigned int keep) {
  unsigned long long m = 0ull;
#pragma unroll
  for (int u = 0; u < N; ++u)
    if ((keep >> u) & 1u) m += __float2ull_rn(av[u] * MASS_SCALE);
  for (int off = 1; off < 64; off <<= 1) m += __shfl_xor(m, off);
  if ((threadIdx.x & 63) == 0 && m != 0ull) atomicAdd(acc, m);
}

// Fixed-point mass back to a fraction (NaN marks a head without a set).
__device__ __forceinline__ float mass_value(unsigned long long m) {
  return (float)((double)m * (1.0 / 1099511627776.0));
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Phase timestamp of this workgroup (profiling aid; p.phase_t is null unless
// the caller asked for it): the constant 100 MHz device clock.
__device__ __forceinline__ void stamp_phase(const DecodeParams& p, int k) {
  if (p.phase_t != nullptr && threadIdx.x == 0 && (int)blockIdx.x < p.phase_wgs)
    p.phase_t[(size_t)blockIdx.x * PHASES + k] = __builtin_amdgcn_s_memrealtime();
}

// Load 8 consecutive elements of a V row as fp32 (bf16 or e4m3 codes).
template <bool FP8>
__device__ __forceinline__ void load_row8(const void* pool, size_t row_off, int sub, float* x) {
  if (!FP8) {
    const uint4 w = *reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(pool) + row_off * D + 8 * sub);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(
        reinterpret_cast<const uint8_t*>(pool) + row_off * D + 8 * sub);
    f32x2 t;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false); x[0] = t.x; x[1] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);  x[2] = t.x; x[3] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false); x[4] = t.x; x[5] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);  x[6] = t.x; x[7] = t.y;
  }
}

// 8 consecutive dims 8*sub..8*sub+7 of row r of a K page (blocked layout).
template <bool FP8>
__device__ __forceinline__ void load_krow8(const void* pool, size_t page, int r, int sub, float* x) {
  const size_t off = page * (BS * D) + (size_t)(((sub >> 2) << 4) + r) * 32 + 8 * (sub & 3);
  if (!FP8) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(pool) + off);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(pool) + off);
    f32x2 t;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false); x[0] = t.x; x[1] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);  x[2] = t.x; x[3] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false); x[4] = t.x; x[5] = t.y;
    t = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);  x[6] = t.x; x[7] = t.y;
  }
}

}  // namespace hws
