// gdr2_ceiling.hip -- measured ceilings of the chip for the benchmark's
// roofline figures (libgdr2_ceiling.so, loaded by the benchmark only; the
// operator library does not contain these kernels).
//
//   gdr2_ceiling_copy   dst = src over n 16-byte vectors: an HBM read stream and
//                       an HBM write stream of the same size at once.
//   gdr2_ceiling_read   reads n 16-byte vectors and writes one word per
//                       workgroup: a read-only HBM stream.
//   gdr2_ceiling_mfma   back-to-back 16x16x32 bf16 (or f16) MFMAs from
//                       registers, eight independent accumulator chains per
//                       wavefront: the dense matrix-core rate the operator's
//                       products run on.
// Every entry point enqueues one kernel on `stream` and returns the HIP status.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, unsigned* __restrict__ out,
                                                   long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  unsigned acc = 0;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup keeps the loads live
  __shared__ unsigned red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

template <bool F16>
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if constexpr (F16) {
    f16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = (_Float16)(seed * (lane + j));
      b[j] = (_Float16)(seed * (lane - j));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = (__bf16)(seed * (lane + j));
      b[j] = (__bf16)(seed * (lane - j));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

extern "C" {

// dst, src: device buffers of n16 16-byte vectors each (16-byte aligned).
int gdr2_ceiling_copy(const void* src, void* dst, long long n16, int blocks, void* stream) {
  if (!src || !dst || n16 <= 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return (int)hipGetLastError();
}

// src: n16 16-byte vectors; out: `blocks` words.
int gdr2_ceiling_read(const void* src, unsigned* out, long long n16, int blocks, void* stream) {
  if (!src || !out || n16 <= 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), out, n16);
  return (int)hipGetLastError();
}

// out: blocks * 256 floats.  Issues blocks * 4 wavefronts * iters * 8 MFMAs of
// 16 * 16 * 32 * 2 flops each.
int gdr2_ceiling_mfma(float* out, int blocks, int iters, int f16, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  if (f16)
    hipLaunchKernelGGL(mfma_kernel<true>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                       iters, 1e-3f);
  else
    hipLaunchKernelGGL(mfma_kernel<false>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                       iters, 1e-3f);
  return (int)hipGetLastError();
}

}  // extern "C"
