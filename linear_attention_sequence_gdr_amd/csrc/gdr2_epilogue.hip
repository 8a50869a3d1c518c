// gdr2_epilogue.hip -- output epilogue of the Gated DeltaNet-2 block (pages,
// "Big-Picture Architecture" item 6 and "Gated DeltaNet-2 token mixer block"
// item 5: the recurrent output is RMS-normalised, then multiplied channel by
// channel by a SiLU-activated output gate):
//
//     y = o / sqrt(mean(o^2) + eps) * weight * silu(z),   silu(z) = z * sigmoid(z),
//
// with the mean taken over each group of `group` consecutive channels.
//
// HBM-bound streaming: every element of o and z is read once and every element
// of y written once (6 bytes per element in bf16, 12 in fp32) against about a
// dozen flops.  A group is spread over G lanes (a power of two, at most 64);
// each lane keeps NC chunks of 8 consecutive channels of o in registers, so o
// is read once.  Lane l of a group takes chunks l, l + G, ... so that the G
// lanes of one step read G adjacent 16-byte pieces.  The sum of squares is
// reduced over the G lanes with xor shuffles, which never leave an aligned
// group of G lanes.
#include <hip/hip_runtime.h>

#include "gdr2_device.h"
#include "gdr2_internal.h"

namespace gdr2 {

template <bool BF16>
__device__ __forceinline__ void store8(void* base, size_t idx, const float v[8]) {
  if constexpr (BF16) {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    u.z = (uint32_t)f32_to_bf16_bits(v[4]) | ((uint32_t)f32_to_bf16_bits(v[5]) << 16);
    u.w = (uint32_t)f32_to_bf16_bits(v[6]) | ((uint32_t)f32_to_bf16_bits(v[7]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) = u;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <int NC, bool BF16>
__global__ __launch_bounds__(256) void norm_gate_kernel(NormGateArgs a) {
  const int G = a.lanes;
  const int tid = threadIdx.x, gl = tid & (G - 1);
  const long long gi = (long long)blockIdx.x * (256 / G) + tid / G;  // group index
  const bool live = gi < a.groups;
  const int nch = a.group >> 3;                                      // 8-channel chunks
  const size_t base = live ? (size_t)gi * (size_t)a.group : 0;

  float x[NC][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = gl + i * G;
    if (live && c < nch) {
      load8<BF16>(a.o, base + 8 * c, x[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[i][e], x[i][e], ss);
  }
  for (int off = G >> 1; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float rn = rsqrtf(fmaf(ss, a.inv_group, a.eps));
  const int wofs = (a.period > 1 && live) ? (int)(gi % a.period) * a.group : 0;

#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = gl + i * G;
    if (!(live && c < nch)) continue;
    float zz[8], y[8];
    load8<BF16>(a.z, base + 8 * c, zz);
    float wt[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    if (a.weight) load8<false>(a.weight, (size_t)wofs + 8 * c, wt);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-zz[e]));
      y[e] = x[i][e] * rn * wt[e] * (zz[e] * sig);
    }
    store8<BF16>(a.y, base + 8 * c, y);
  }
}

int norm_gate_lanes(int group) {
  const int chunks = group / 8;
  int g = 1;
  while (g < chunks && g < 64) g <<= 1;
  return g;
}

long long norm_gate_blocks(long long groups, int group) {
  const int per_block = 256 / norm_gate_lanes(group);
  return (groups + per_block - 1) / per_block;
}

template <bool BF16>
static hipError_t launch_norm_gate_t(const NormGateArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)norm_gate_blocks(a.groups, a.group)), block(256);
  const int nc = (a.group / 8 + a.lanes - 1) / a.lanes;
  if (nc <= 1) hipLaunchKernelGGL((norm_gate_kernel<1, BF16>), grid, block, 0, stream, a);
  else if (nc <= 2) hipLaunchKernelGGL((norm_gate_kernel<2, BF16>), grid, block, 0, stream, a);
  else if (nc <= 4) hipLaunchKernelGGL((norm_gate_kernel<4, BF16>), grid, block, 0, stream, a);
  else if (nc <= 8) hipLaunchKernelGGL((norm_gate_kernel<8, BF16>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((norm_gate_kernel<16, BF16>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_norm_gate(NormGateArgs a, bool bf16, hipStream_t stream) {
  if (a.groups == 0) return hipSuccess;
  a.lanes = norm_gate_lanes(a.group);
  a.inv_group = 1.f / (float)a.group;
  return bf16 ? launch_norm_gate_t<true>(a, stream) : launch_norm_gate_t<false>(a, stream);
}

}  // namespace gdr2
