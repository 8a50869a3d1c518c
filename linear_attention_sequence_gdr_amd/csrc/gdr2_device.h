// gdr2_device.h -- device-side helpers shared by the libgdr2 kernels (gfx950).
//
// Storage conversions for bf16, the CDNA4 MFMA wrappers and their lane layouts.
// MFMA 16x16 tiles (one 64-lane wavefront): lane l = 16*g + m (m = l & 15,
// g = l >> 4).  The A operand lane holds row m of A and a group of K elements
// picked by g; the B operand lane holds column m of B and the same K group.
// The accumulator lane holds C[4*g + q][m] for q = 0..3 ("C layout").  Both
// operands are always fetched with the same K grouping, so the contraction
// covers every K index exactly once whatever order the hardware uses inside a
// group.  A C-layout tile converted to 16-bit is therefore directly the B
// operand of a K = 16 product that contracts over the tile's rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr2 {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---- bf16 storage <-> fp32 ----------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t idx, float out[8]) {
  if constexpr (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    const float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void load4(const void* base, size_t idx, float out[4]) {
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    out[0] = __uint_as_float(u.x << 16);
    out[1] = __uint_as_float(u.x & 0xffff0000u);
    out[2] = __uint_as_float(u.y << 16);
    out[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  else return static_cast<const float*>(base)[idx];
}

// Store 4 consecutive fp32 values in the storage type (8- or 16-byte aligned).
template <bool BF16>
__device__ __forceinline__ void store4(void* base, size_t idx, const float v[4]) {
  if constexpr (BF16) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = u;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// ---- MFMA wrappers ---------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma32(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(const f16x8& a, const f16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const f16x4& a, const f16x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// fp32: a K = 16 block as four K = 4 instructions; lane group g supplies K
// index 4*g + q to instruction q, for A and B alike.
__device__ __forceinline__ f32x4 mma16(const float4& a, const float4& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
  return c;
}

template <typename E> struct Vec;
template <> struct Vec<__bf16> { typedef bf16x8 v8; };
template <> struct Vec<_Float16> { typedef f16x8 v8; typedef f16x4 v4; };
template <> struct Vec<float> { typedef float4 v4; };

// Accumulator chains never mix MFMA shapes: a 16x16x16 step whose C input is
// the result of a 16x16x32 step has returned wrong values in the first two
// accumulator registers, timing-dependently, so the K = 32 helper below and
// the K = 16 helper that follows are only ever chained with themselves (or
// started from a VALU-written accumulator).
//
// acc += A[16 x K] * B[K x 16], both operands K-contiguous in LDS: A row m at
// A + m*lda, B column n at Bt + n*ldb (i.e. B stored transposed).
template <typename E, int K>
__device__ __forceinline__ f32x4 mma_lds(f32x4 acc, const E* A, int lda, const E* Bt, int ldb) {
  const int m = lane_id() & 15, g = lane_id() >> 4;
  const E* a = A + m * lda;
  const E* b = Bt + m * ldb;
  if constexpr (sizeof(E) == 2) {
    static_assert(K % 32 == 0, "16-bit operands: K must be a multiple of 32");
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32)
      acc = mma32(*reinterpret_cast<const typename Vec<E>::v8*>(a + k0 + 8 * g),
                  *reinterpret_cast<const typename Vec<E>::v8*>(b + k0 + 8 * g), acc);
  } else {
    static_assert(K % 16 == 0, "K must be a multiple of 16");
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16)
      acc = mma16(*reinterpret_cast<const float4*>(a + k0 + 4 * g),
                  *reinterpret_cast<const float4*>(b + k0 + 4 * g), acc);
  }
  return acc;
}

// Same, with a K extent known only at run time (a multiple of 16, at most KMAX).
template <typename E, int KMAX>
__device__ __forceinline__ f32x4 mma_lds_k16(f32x4 acc, const E* A, int lda, const E* Bt, int ldb,
                                             int K) {
  const int m = lane_id() & 15, g = lane_id() >> 4;
  const E* a = A + m * lda;
  const E* b = Bt + m * ldb;
  typedef typename Vec<E>::v4 V4;
#pragma unroll
  for (int k0 = 0; k0 < KMAX; k0 += 16)
    if (k0 < K)
      acc = mma16(*reinterpret_cast<const V4*>(a + k0 + 4 * g),
                  *reinterpret_cast<const V4*>(b + k0 + 4 * g), acc);
  return acc;
}

// acc += A[16 x K] * B[K x 16] in fp32 from LDS, each operand either
// K-contiguous as in mma_lds (A row m at A + m*lda, B column n at B + n*ldb)
// or K-major (TA: A element (m, k) at A + k*lda + m; TB: B element (k, n) at
// B + k*ldb + n).  A K-major operand takes four 4-byte reads per K = 16
// block; within a 16-lane group they hit consecutive words.  kn (a multiple
// of 16, at most K, the same across the wavefront) cuts K short.
template <int K, bool TA, bool TB>
__device__ __forceinline__ f32x4 mma_lds_f32(f32x4 acc, const float* A, int lda, const float* B, int ldb,
                                             int kn = K) {
  static_assert(K % 16 == 0, "K must be a multiple of 16");
  const int m = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    if (k0 >= kn) break;
    float av[4], bv[4];
    if constexpr (TA) {
      const float* a = A + (k0 + 4 * g) * lda + m;
      av[0] = a[0]; av[1] = a[lda]; av[2] = a[2 * lda]; av[3] = a[3 * lda];
    } else {
      const float4 x = *reinterpret_cast<const float4*>(A + m * lda + k0 + 4 * g);
      av[0] = x.x; av[1] = x.y; av[2] = x.z; av[3] = x.w;
    }
    if constexpr (TB) {
      const float* b = B + (k0 + 4 * g) * ldb + m;
      bv[0] = b[0]; bv[1] = b[ldb]; bv[2] = b[2 * ldb]; bv[3] = b[3 * ldb];
    } else {
      const float4 x = *reinterpret_cast<const float4*>(B + m * ldb + k0 + 4 * g);
      bv[0] = x.x; bv[1] = x.y; bv[2] = x.z; bv[3] = x.w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv[q], acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- fp32 products as three bf16 products ---------------------------------------------
// x = hi + lo + e with hi = bf16(x), lo = bf16(x - hi) (both rounded to
// nearest), so |e| <= 2^-18 |x|.  A product a b then runs as hi_a hi_b +
// hi_a lo_b + lo_a hi_b on bf16 MFMA with fp32 accumulation; the dropped
// lo_a lo_b and the split residuals leave at most about 3 * 2^-18 |a b| per
// term, against 2^-24 for an fp32 product.  One 16x16x32 step of three
// instructions replaces eight 16x16x4 fp32 steps at a sixteenth of the issue
// cost each.
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

__device__ __forceinline__ void split_bf16(const f32x4& x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hi[q] = (__bf16)x[q];
    lo[q] = (__bf16)(x[q] - (float)hi[q]);
  }
}

// acc += A B over one K = 32 block, from the hi/lo halves of both operands
// (smallest terms first).
__device__ __forceinline__ f32x4 mma3x(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                       const bf16x8& bl, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}

// Transposing LDS read of 16-bit data (gfx950 ds_read_b64_tr_b16): within
// each 16-lane group, lane t receives elements t, t + 16, t + 32 and t + 48
// of the 64 elements that the group's lanes address (4 consecutive elements
// per lane, in lane order).  With lane s of the group pointing at elements
// 4 (s % 4) .. 4 (s % 4) + 3 of row s / 4 of a row-major block, lane t gets
// column t of those 4 rows: a K-major operand fragment from a row-major block.
__device__ __forceinline__ bf16x4 lds_tr16_bf16(const __bf16* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(__attribute__((address_space(3))) void*)p);
  return __builtin_bit_cast(bf16x4, v);
}

// The 16x16x32 operand fragment of lane (m, g) for a factor whose K index
// runs down the rows of a row-major bf16 block X (leading dimension ld):
// elements X[k0 + 8g + e][c0 + m], e < 8, as two transposing reads.
__device__ __forceinline__ bf16x8 frag_kmajor(const __bf16* X, int ld, int k0, int c0) {
  const int m = lane_id() & 15, g = lane_id() >> 4;
  const __bf16* p = X + (k0 + 8 * g + (m >> 2)) * ld + c0 + 4 * (m & 3);
  const bf16x4 x0 = lds_tr16_bf16(p);
  const bf16x4 x1 = lds_tr16_bf16(p + 4 * ld);
  return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// The fragment of lane (m, g) for a factor whose K index runs along the rows
// of X: elements X[c0 + m][k0 + 8g + e], e < 8, one 16-byte read.
__device__ __forceinline__ bf16x8 frag_krow(const __bf16* X, int ld, int k0, int c0) {
  const int m = lane_id() & 15, g = lane_id() >> 4;
  return *reinterpret_cast<const bf16x8*>(X + (c0 + m) * ld + k0 + 8 * g);
}

}  // namespace gdr2
