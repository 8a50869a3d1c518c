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

constexpr int SCHED_MAX = 4096;  // sequences sorted in one workgroup

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

size_t schedule_bytes(int N) { return N <= 1 || N > SCHED_MAX ? 0 : (size_t)N * sizeof(int32_t); }

hipError_t launch_schedule(const int32_t* cu, int N, int T, int32_t* order, hipStream_t stream) {
  if (N <= 1 || N > SCHED_MAX) return hipSuccess;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, stream, cu, N, T, order);
  return hipGetLastError();
}

}  // namespace gdr2
