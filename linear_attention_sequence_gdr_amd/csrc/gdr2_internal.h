// gdr2_internal.h -- host-side launch interface between the C ABI (gdr2_api.cpp)
// and the kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr2 {

struct DecodeArgs {
  const void *q, *k, *v, *la, *b, *w;
  float* S;
  void* o;
  int N, H;
  int la_bf16;
};

struct ChunkArgs {
  const void *q, *k, *v, *la, *b, *w;
  const float* S0;
  void* o;
  float* ST;
  const int32_t* cu;      // device [N+1] or nullptr
  const int32_t* order;   // device [N] schedule (longest first) or nullptr
  int N, T, H, DV;
  int la_bf16;
};

hipError_t launch_decode(const DecodeArgs& a, int dk, int dv, bool bf16, hipStream_t stream);

// Returns hipErrorInvalidValue when no kernel variant exists for the sizes.
hipError_t launch_chunk(const ChunkArgs& a, int dk, int dv, bool bf16, hipStream_t stream);
bool chunk_supported(int dk, int dv, bool bf16);

// Schedule: a permutation of the N packed sequences, longest first, written
// into `order` (device int32 [N]) from cu_seqlens.  `scratch` holds N int32.
hipError_t launch_schedule(const int32_t* cu, int N, int T, int32_t* order, hipStream_t stream);
size_t schedule_bytes(int N);

}  // namespace gdr2
