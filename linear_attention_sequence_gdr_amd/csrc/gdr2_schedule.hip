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
// and length.  The chunks of a block of sequences are written by all threads
// at once (thread t takes chunks t, t + 1024, ... and finds its sequence by a
// binary search over the block's prefix sums), so one long sequence does not
// serialise the table.  Entries at or past `cap` are never written (only
// inputs that break the cu_seqlens contract can reach them).
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* cu, int N, int T, int cap,
                                                          int32_t* cbase, int32_t* tab) {
  __shared__ int part[1024];
  __shared__ int st[1024], ln[1024];
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
    st[t] = s;
    ln[t] = len;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int v = t >= d ? part[t - d] : 0;
      __syncthreads();
      part[t] += v;
      __syncthreads();
    }
    const long long carry = carry_s;
    const long long first = carry + part[t] - nc;
    if (n < N) cbase[n] = (int32_t)(first < cap ? first : cap);
    // chunk j of this block (j < part[1023]) belongs to the sequence i with
    // part[i - 1] <= j < part[i]
    const int nb = part[1023];
    for (int j = t; j < nb && carry + j < cap; j += 1024) {
      int lo = 0, hi = 1023;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (part[mid] > j) hi = mid;
        else lo = mid + 1;
      }
      const int c = j - (part[lo] - (ln[lo] + 63) / 64);  // chunk within sequence lo
      const long long x = carry + j;
      tab[2 * x] = st[lo] + 64 * c;
      tab[2 * x + 1] = min(64, ln[lo] - 64 * c);
    }
    __syncthreads();
    if (t == 1023) carry_s = (int)min(carry + part[1023], (long long)cap);
    __syncthreads();
  }
  if (t == 0) cbase[N] = carry_s;
}

// Segment plan of packed sequences for the split state pass (one workgroup).
// Each sequence's chain of nc_n chunks is cut into P_n = ceil(nc_n / L)
// segments of ceil(nc_n / P_n) chunks (the last shorter), where L balances
// the longest segment against the work per CU (total chunks x heads over the
// CUs), is at least PSEG_MIN chunks, and at least sqrt(2 x the longest chain)
// so that the scan over one sequence's segments stays short next to them.
// Segment ids follow the schedule order, so a sequence's segments are
// consecutive and the longest sequences' segments come first.  Ids at or past
// nsmax (only reachable by inputs that break the cu_seqlens contract) are not
// written; *nseg is the number of segments, at most nsmax.
__global__ __launch_bounds__(1024) void segment_plan_kernel(const int32_t* cu, int N, int T, const int32_t* order,
                                                           const int32_t* cbase, int H, int slots, int nsmax,
                                                           int32_t* seg, int32_t* sq, int32_t* nseg) {
  __shared__ int part[1024];
  __shared__ int carry_s, maxc_s, L_s;
  const int t = threadIdx.x;
  auto chunks_of = [&](int n) {
    int s = cu[n], e = cu[n + 1];
    s = s < 0 ? 0 : (s > T ? T : s);
    e = e < s ? s : (e > T ? T : e);
    return (e - s + 63) / 64;
  };
  if (t == 0) {
    carry_s = 0;
    maxc_s = 0;
  }
  __syncthreads();
  int mx = 0;
  for (int n = t; n < N; n += 1024) mx = max(mx, chunks_of(n));
  atomicMax(&maxc_s, mx);
  __syncthreads();
  if (t == 0) {
    const long long work = ((long long)cbase[N] * H + slots - 1) / slots;
    long long L = work > PSEG_MIN ? work : PSEG_MIN;
    const long long r = (long long)ceilf(sqrtf(2.f * (float)maxc_s));
    L = L > r ? L : r;
    L_s = (int)(L < 0x7fffffffLL ? L : 0x7fffffffLL);
  }
  __syncthreads();
  const int L = L_s;
  for (int base = 0; base < N; base += 1024) {
    const int i = base + t;
    int n = 0, nc = 0, P = 0;
    if (i < N) {
      n = order ? order[i] : i;
      nc = chunks_of(n);
      P = nc > L ? (nc + L - 1) / L : 1;
    }
    part[t] = P;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int v = t >= d ? part[t - d] : 0;
      __syncthreads();
      part[t] += v;
      __syncthreads();
    }
    const long long first = (long long)carry_s + part[t] - P;
    if (i < N) {
      const int f = (int)(first < nsmax ? first : nsmax);
      sq[2 * n] = f;
      sq[2 * n + 1] = first + P <= nsmax ? P : nsmax - f;
      const int sc = (nc + P - 1) / P;  // chunks per segment; every segment gets at least one when P > 1
      for (int j = 0; j < P && first + j < nsmax; ++j) {
        const int g = (int)first + j;
        seg[4 * g] = n;
        seg[4 * g + 1] = j * sc;
        seg[4 * g + 2] = min(sc, nc - j * sc);
        seg[4 * g + 3] = f;
      }
    }
    __syncthreads();
    if (t == 1023) carry_s = (int)min((long long)carry_s + part[1023], (long long)nsmax);
    __syncthreads();
  }
  if (t == 0) *nseg = carry_s;
}

hipError_t launch_segment_plan(const int32_t* cu, int N, int T, const int32_t* order, const int32_t* cbase,
                               int H, int slots, int nsmax, int32_t* seg, int32_t* sq, int32_t* nseg,
                               hipStream_t stream) {
  if (N <= 0 || nsmax <= 0 || H <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(segment_plan_kernel, dim3(1), dim3(1024), 0, stream, cu, N, T, order, cbase, H,
                     slots > 0 ? slots : 1, nsmax, seg, sq, nseg);
  return hipGetLastError();
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
