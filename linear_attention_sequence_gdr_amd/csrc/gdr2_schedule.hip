// gdr2_schedule.hip -- longest-first order of packed sequences.
//
// The chunked forward walks each (sequence, head) sequentially, so with
// packed sequences of very different lengths the last long sequence to start
// sets the finishing time.  One workgroup sorts (length, index) keys in LDS
// with a bitonic network and writes the sequence indices longest first; the
// forward kernel hands them out in that order.  Lengths come from cu_seqlens
// clamped to [0, T], exactly as the forward kernel reads them.
#include <hip/hip_runtime.h>

#include "gdr2_internal.h"

namespace gdr2 {

__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* cu, int N, int T,
                                                       int32_t* order) {
  __shared__ unsigned long long key[SCHED_MAX];
  int P = 1;
  while (P < N) P <<= 1;
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    if (i < N) {
      int s = cu[i], e = cu[i + 1];
      s = s < 0 ? 0 : (s > T ? T : s);
      e = e < s ? s : (e > T ? T : e);
      // ascending keys = descending length, then ascending index
      key[i] = ((unsigned long long)(0x7fffffffu - (unsigned)(e - s)) << 32) | (unsigned)i;
    } else {
      key[i] = ~0ull;
    }
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long a = key[i], b = key[l];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            key[i] = b;
            key[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < N; i += blockDim.x) order[i] = (int32_t)(key[i] & 0xffffffffu);
}

// Chunk table of packed sequences for the two-pass forward: cbase[n] is the
// index of sequence n's first 64-token chunk (an exclusive prefix sum of the
// chunk counts, one block of 1024 sequences at a time with a running carry),
// cbase[N] the number of chunks, clamped to the capacity `cap` of the table
// and of the record buffer; tab[2c], tab[2c+1] are chunk c's first token row
// and length.  Entries at or past `cap` are never written (only inputs that
// break the cu_seqlens contract can reach them).
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* cu, int N, int T, int cap,
                                                          int32_t* cbase, int32_t* tab) {
  __shared__ int part[1024];
  __shared__ int carry_s;
  const int t = threadIdx.x;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int n = base + t;
    int s = 0, len = 0;
    if (n < N) {
      s = cu[n];
      int e = cu[n + 1];
      s = s < 0 ? 0 : (s > T ? T : s);
      e = e < s ? s : (e > T ? T : e);
      len = e - s;
    }
    const int nc = (len + 63) / 64;
    part[t] = nc;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int v = t >= d ? part[t - d] : 0;
      __syncthreads();
      part[t] += v;
      __syncthreads();
    }
    const long long carry = carry_s;
    const long long first = carry + part[t] - nc;
    if (n < N) {
      cbase[n] = (int32_t)(first < cap ? first : cap);
      for (int c = 0; c < nc && first + c < cap; ++c) {
        tab[2 * (first + c)] = s + 64 * c;
        tab[2 * (first + c) + 1] = min(64, len - 64 * c);
      }
    }
    __syncthreads();
    if (t == 1023) carry_s = (int)min(carry + part[1023], (long long)cap);
    __syncthreads();
  }
  if (t == 0) cbase[N] = carry_s;
}

hipError_t launch_chunk_table(const int32_t* cu, int N, int T, int cap, int32_t* cbase, int32_t* tab,
                              hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, stream, cu, N, T, cap, cbase, tab);
  return hipGetLastError();
}

size_t schedule_bytes(int N) { return N <= 1 || N > SCHED_MAX ? 0 : (size_t)N * sizeof(int32_t); }

hipError_t launch_schedule(const int32_t* cu, int N, int T, int32_t* order, hipStream_t stream) {
  if (N <= 1 || N > SCHED_MAX) return hipSuccess;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, stream, cu, N, T, order);
  return hipGetLastError();
}

}  // namespace gdr2
