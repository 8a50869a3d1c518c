// gdr2_chunk_common.h -- device helpers shared by the chunkwise kernels (gfx950):
// storage conversions, DPP lane exchanges and scans, buffer-resource loads and
// the blocked WY inverse step.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdr2_device.h"

namespace gdr2 {

constexpr int CH = 64;   // chunk length (tokens)
constexpr float LOG2E = 1.4426950408889634f;

template <typename T> __device__ __forceinline__ T cvt(float x) { return (T)x; }

template <typename V4> __device__ __forceinline__ V4 cvt4(f32x4 a);
template <> __device__ __forceinline__ f16x4 cvt4<f16x4>(f32x4 a) {
  return f16x4{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3]};
}
template <> __device__ __forceinline__ float4 cvt4<float4>(f32x4 a) {
  return make_float4(a[0], a[1], a[2], a[3]);
}
// 2^x on the hardware exponential unit (about 1 ulp).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// x * 2^e with the integer part of e applied as an exact exponent shift, so
// that 2^e itself never underflows or overflows: only a result that is out of
// range is.  (x large and 2^e below the fp32 range still give their product.)
__device__ __forceinline__ float mul_exp2(float x, float e) {
  const float n = floorf(e);
  return __builtin_amdgcn_ldexpf(x * exp2_fast(e - n), (int)n);
}

template <typename V4> __device__ __forceinline__ V4 neg_cvt4(f32x4 a) {
  return cvt4<V4>(f32x4{-a[0], -a[1], -a[2], -a[3]});
}

// Four consecutive ST values from LDS, or gathered from a C-layout column.
template <typename ST, typename SV4>
__device__ __forceinline__ SV4 gather4(const ST* p, int stride) {
  SV4 r;
  if constexpr (std::is_same<ST, float>::value) {
    r = make_float4(p[0], p[stride], p[2 * stride], p[3 * stride]);
  } else {
    r = f16x4{p[0], p[stride], p[2 * stride], p[3 * stride]};
  }
  return r;
}

// Write 8 consecutive fp32 values as E (16 B for 16-bit types, 32 B for fp32).
template <typename E>
__device__ __forceinline__ void st8(E* dst, const float v[8]) {
  if constexpr (std::is_same<E, float>::value) {
    reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    typedef __attribute__((ext_vector_type(8))) E V8;
    V8 x;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (E)v[i];
    *reinterpret_cast<V8*>(dst) = x;
  }
}

// Write N (1, 2 or 4) consecutive values as E.
template <typename E, int N>
__device__ __forceinline__ void stn(E* dst, const float* v) {
  if constexpr (N == 4) {
    if constexpr (std::is_same<E, float>::value) *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    else *reinterpret_cast<f16x4*>(dst) = f16x4{(E)v[0], (E)v[1], (E)v[2], (E)v[3]};
  } else if constexpr (N == 2) {
    if constexpr (std::is_same<E, float>::value) *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
    else *reinterpret_cast<f16x2*>(dst) = f16x2{(E)v[0], (E)v[1]};
  } else {
    dst[0] = (E)v[0];
  }
}

__device__ __forceinline__ float dpp_shr(float v, int n) {
  int r;
  switch (n) {
    case 1: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, true); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, true); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, true); break;
    default: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, true); break;
  }
  return __builtin_bit_cast(float, r);
}

// Broadcast lane k of each group of four lanes (DPP quad_perm).
__device__ __forceinline__ float quad_bcast(float v, int k) {
  int r;
  switch (k) {
    case 0: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x00, 0xf, 0xf, false); break;
    case 1: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x55, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xaa, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xff, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, r);
}

// Inclusive prefix sum over groups of RG consecutive lanes (RG = 16, 32, 64):
// a DPP scan inside each 16-lane row (row_shr 1, 2, 4, 8), then row carries.
template <int RG>
__device__ __forceinline__ float seg_scan(float x) {
  x += dpp_shr(x, 1);
  x += dpp_shr(x, 2);
  x += dpp_shr(x, 4);
  x += dpp_shr(x, 8);
  if constexpr (RG >= 32) {
    const float c = __shfl(x, (lane_id() & ~31) + 15);
    if (lane_id() & 16) x += c;
  }
  if constexpr (RG == 64) {
    const float c = __shfl(x, 31);
    if (lane_id() & 32) x += c;
  }
  return x;
}

// The (a, b) block coordinates (b <= a) of the 10 lower-triangular 16x16
// tiles of a 64x64 chunk matrix.
__device__ __forceinline__ void tri_tile(int t, int& a, int& b) {
  a = (t >= 1) + (t >= 3) + (t >= 6);
  b = t - (a * (a + 1)) / 2;
}

template <int N>
__device__ __forceinline__ void ldw(uint32_t (&dst)[N], const void* p) {
  if constexpr (N == 8) {
    const uint4* s = static_cast<const uint4*>(p);
    const uint4 a = s[0], c = s[1];
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    dst[4] = c.x; dst[5] = c.y; dst[6] = c.z; dst[7] = c.w;
  } else if constexpr (N == 4) {
    const uint4 a = *static_cast<const uint4*>(p);
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
  } else if constexpr (N == 2) {
    const uint2 a = *static_cast<const uint2*>(p);
    dst[0] = a.x; dst[1] = a.y;
  } else {
    dst[0] = *static_cast<const uint32_t*>(p);
  }
}

// 8 stored key elements (bf16 pairs or fp32) to fp32.
template <bool F32, int KW>
__device__ __forceinline__ void unpack8(const uint32_t (&w)[KW], float out[8]) {
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// Round to the nearest bf16 value, returned as fp32 (hardware conversion).
__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }

// Write 4 consecutive fp32 values as E (8 B for 16-bit types, 16 B for fp32).
template <typename E>
__device__ __forceinline__ void st4(E* dst, const float v[4]) {
  if constexpr (std::is_same<E, float>::value) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    typedef __attribute__((ext_vector_type(4))) E V4;
    *reinterpret_cast<V4*>(dst) = V4{(E)v[0], (E)v[1], (E)v[2], (E)v[3]};
  }
}

// 4 stored key elements (bf16 pairs in 2 words, or 4 fp32 words) to fp32.
template <bool F32, int NWD>
__device__ __forceinline__ void unpack4(const uint32_t (&w)[NWD], float out[4]) {
  if constexpr (F32) {
    static_assert(NWD == 4, "fp32: 4 words");
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
  } else {
    static_assert(NWD == 2, "bf16: 2 words");
    out[0] = __uint_as_float(w[0] << 16);
    out[1] = __uint_as_float(w[0] & 0xffff0000u);
    out[2] = __uint_as_float(w[1] << 16);
    out[3] = __uint_as_float(w[1] & 0xffff0000u);
  }
}

// A raw buffer resource over [base, base + bytes): loads outside read as 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// N consecutive words through a buffer resource.
template <int N>
__device__ __forceinline__ void bld(uint32_t (&dst)[N], __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef __attribute__((ext_vector_type(2))) unsigned int u2;
  typedef __attribute__((ext_vector_type(4))) unsigned int u4;
  if constexpr (N == 4) {
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  } else if constexpr (N == 2) {
    const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    dst[0] = v.x; dst[1] = v.y;
  } else {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
  }
}

// Off-diagonal blocks of column block B of A = (I + T)^-1 by the block
// recurrence A_aB = A_aa (-sum_{B<=c<a} T_ac A_cB); Tn holds -T and the
// diagonal blocks of A are already in Am.
template <int B, typename ST, typename SV4, int LDC>
__device__ __forceinline__ void wy_column(const ST* Tn, ST* Am) {
  const int m = lane_id() & 15, g4 = lane_id() >> 4;
  SV4 xb[4];
  xb[B] = gather4<ST, SV4>(Am + (16 * B + 4 * g4) * LDC + 16 * B + m, LDC);
#pragma unroll
  for (int a = B + 1; a < 4; ++a) {
    f32x4 acc = zero4();
#pragma unroll
    for (int c = B; c < a; ++c)
      acc = mma16(*reinterpret_cast<const SV4*>(Tn + (16 * a + m) * LDC + 16 * c + 4 * g4), xb[c], acc);
    const SV4 wvec = cvt4<SV4>(acc);
    const f32x4 xa =
        mma16(*reinterpret_cast<const SV4*>(Am + (16 * a + m) * LDC + 16 * a + 4 * g4), wvec, zero4());
    xb[a] = cvt4<SV4>(xa);
#pragma unroll
    for (int q = 0; q < 4; ++q) Am[(16 * a + 4 * g4 + q) * LDC + 16 * B + m] = cvt<ST>(xa[q]);
  }
}

}  // namespace gdr2
