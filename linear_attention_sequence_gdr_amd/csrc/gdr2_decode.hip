// gdr2_decode.hip -- fused single-token decode step of the Gated Delta Rule-2
// operator (Gated DeltaNet-2 pages, Appendix C.5: a forward-only recurrent
// kernel that keeps the state in fp32, decays it by exp(g_t), reads it along
// b_t * k_t, writes w_t * v_t along k_t and returns S_t^T q_t).
//
// One workgroup of 256 threads owns one (sequence, head) state of dk x dv fp32.
// The state is read once and written once: with S_bar = Diag(alpha) S,
//     r = S^T (alpha * b * k),   p = S^T (alpha * q),   delta = w * v - r,
//     o = S_t^T q = p + (k . q) delta,   S_t = Diag(alpha) S + k delta^T,
// which is Steps 1-5 of the pages' state update folded so that both column
// reductions come from the same pass over S (Step 5 reads S_t = S_bar + k
// delta^T, so S_t^T q = S_bar^T q + (k^T q) delta).
//
// With the output epilogue on, the stored row is RMSNorm(o) * weight * silu(z)
// instead of o (the block's output normalisation and gate), at the cost of one
// extra read of z.
//
// Each lane owns 4 adjacent columns (one 16-byte load per row) of P rows, the
// rows of a wave are interleaved so that one wave-wide load covers whole
// contiguous state rows.  HBM-bound: 2 * dk * dv * 4 bytes of state traffic per
// (sequence, head) against 7 * dk * dv flops.
#include <hip/hip_runtime.h>

#include "gdr2_device.h"
#include "gdr2_internal.h"

namespace gdr2 {

template <int DK, int DV, bool BF16, bool GATED>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
  constexpr int NT = 256, NW = 4;
  constexpr int LPR = DV / 4;            // lanes per state row
  constexpr int RPI = 64 / LPR;          // rows per wave-wide instruction
  constexpr int RPW = DK / NW;           // rows per wave
  constexpr int P = RPW / RPI;           // rows per lane
  static_assert(P >= 1 && RPW % RPI == 0, "bad decode tiling");

  __shared__ float s_alpha[DK], s_k[DK], s_aq[DK], s_abk[DK], s_z[DV];
  __shared__ float s_red[2][NW * RPI][DV];
  __shared__ float s_qk;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t nh = blockIdx.x;
  const int cq = lane % LPR, rp = lane / LPR;
  const int col = 4 * cq;

  float* S = a.S + nh * (size_t)(DK * DV);
  // issue the state loads first: they dominate the traffic
  float4 st[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int row = wv * RPW + p * RPI + rp;
    st[p] = *reinterpret_cast<const float4*>(S + (size_t)row * DV + col);
  }

  const size_t xk = nh * DK, xv = nh * DV;
  // the output gate's pre-activation and the norm weight, needed only by the
  // lanes that store
  float zz[4] = {0.f, 0.f, 0.f, 0.f}, wt[4] = {1.f, 1.f, 1.f, 1.f};
  if (GATED && wv == 0 && rp == 0) {
    load4<BF16>(a.z, xv + col, zz);
    if (a.nw) load4<false>(a.nw, col, wt);
  }
  for (int i = tid; i < DK; i += NT) {
    const float g = a.la_bf16 ? load1<true>(a.la, xk + i) : load1<false>(a.la, xk + i);
    const float al = __expf(g);
    const float kk = load1<BF16>(a.k, xk + i);
    s_alpha[i] = al;
    s_k[i] = kk;
    s_aq[i] = al * load1<BF16>(a.q, xk + i);
    s_abk[i] = al * load1<BF16>(a.b, xk + i) * kk;
  }
  for (int j = tid; j < DV; j += NT) s_z[j] = load1<BF16>(a.w, xv + j) * load1<BF16>(a.v, xv + j);
  if (wv == 0) {
    float qk = 0.f;
    for (int i = lane; i < DK; i += 64) qk += load1<BF16>(a.q, xk + i) * load1<BF16>(a.k, xk + i);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qk += __shfl_xor(qk, off);
    if (lane == 0) s_qk = qk;
  }
  __syncthreads();

  // partial column reductions over this lane's rows
  float r[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int row = wv * RPW + p * RPI + rp;
    const float e = s_abk[row], q = s_aq[row];
    const float sv[4] = {st[p].x, st[p].y, st[p].z, st[p].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] = fmaf(sv[c], e, r[c]);
      pq[c] = fmaf(sv[c], q, pq[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    s_red[0][wv * RPI + rp][col + c] = r[c];
    s_red[1][wv * RPI + rp][col + c] = pq[c];
  }
  __syncthreads();
  float delta[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float rr = 0.f, pp = 0.f;
#pragma unroll
    for (int s = 0; s < NW * RPI; ++s) {
      rr += s_red[0][s][col + c];
      pp += s_red[1][s][col + c];
    }
    delta[c] = s_z[col + c] - rr;
    pq[c] = pp + s_qk * delta[c];
  }
  if constexpr (!GATED) {
    if (wv == 0 && rp == 0) store4<BF16>(a.o, xv + col, pq);
  }

#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int row = wv * RPW + p * RPI + rp;
    const float al = s_alpha[row], kk = s_k[row];
    float4 nv;
    nv.x = fmaf(al, st[p].x, kk * delta[0]);
    nv.y = fmaf(al, st[p].y, kk * delta[1]);
    nv.z = fmaf(al, st[p].z, kk * delta[2]);
    nv.w = fmaf(al, st[p].w, kk * delta[3]);
    *reinterpret_cast<float4*>(S + (size_t)row * DV + col) = nv;
  }

  if constexpr (GATED) {
    // Output epilogue (Gated DeltaNet-2 pages, "Big-Picture Architecture" item
    // 6), after the state stores so that it overlaps their drain.  Every
    // aligned run of LPR lanes holds the whole output row, 4 columns per lane,
    // so the sum of squares is an xor reduction inside that run; wave 0 alone
    // needs it.
    if (wv == 0) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) ss = fmaf(pq[c], pq[c], ss);
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
      const float rn = rsqrtf(fmaf(ss, 1.f / DV, a.eps));
      if (rp == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-zz[c]));
          pq[c] = pq[c] * rn * wt[c] * (zz[c] * sig);
        }
        store4<BF16>(a.o, xv + col, pq);
      }
    }
  }
}

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  decode_body<DK, DV, BF16, false>(a);
}

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(256) void decode_norm_gate_kernel(DecodeArgs a) {
  decode_body<DK, DV, BF16, true>(a);
}

template <int DK, int DV>
static hipError_t launch_decode_dv(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.N * a.H)), block(256);
  if (a.gated) {
    if (bf16) hipLaunchKernelGGL((decode_norm_gate_kernel<DK, DV, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_norm_gate_kernel<DK, DV, false>), grid, block, 0, stream, a);
  } else {
    if (bf16) hipLaunchKernelGGL((decode_kernel<DK, DV, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<DK, DV, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

template <int DK>
static hipError_t launch_decode_dk(const DecodeArgs& a, int dv, bool bf16, hipStream_t stream) {
  switch (dv) {
    case 32: return launch_decode_dv<DK, 32>(a, bf16, stream);
    case 64: return launch_decode_dv<DK, 64>(a, bf16, stream);
    default: return launch_decode_dv<DK, 128>(a, bf16, stream);
  }
}

hipError_t launch_decode(const DecodeArgs& a, int dk, int dv, bool bf16, hipStream_t stream) {
  if ((size_t)a.N * a.H == 0) return hipSuccess;
  switch (dk) {
    case 32: return launch_decode_dk<32>(a, dv, bf16, stream);
    case 64: return launch_decode_dk<64>(a, dv, bf16, stream);
    default: return launch_decode_dk<128>(a, dv, bf16, stream);
  }
}

}  // namespace gdr2
