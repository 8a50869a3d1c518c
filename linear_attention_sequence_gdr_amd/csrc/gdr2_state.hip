// gdr2_state.hip -- sequential state pass of the two-pass chunkwise forward
// (Gated DeltaNet-2 pages, "Chunkwise Parallel Training via WY
// Representation", Step 3: state and output equations, Eqs. 23-24; packed
// sequences per Appendix C.6).
//
// A workgroup owns one (sequence, head, block of 16*NWV value channels) and
// walks the sequence's chunks in order; wavefront w owns 16 value channels.
// Column j of the state, of U, R and O depends only on column j of S0 and Z,
// so every wavefront runs the whole recurrence for its channels alone, out of
// registers: per chunk, with the record of the intra-chunk pass in LDS,
//   R   = U + (-Y) S                     (residual of the chunk's writes)
//   O^T = S^T Q_g^T + R^T A_qk^T         (Eq. 24, transposed so that each lane
//                                         holds 4 adjacent output channels)
//   S  <- Diag(gamma_C) S + K_tail^T R   (Eq. 23)
// The state is an fp32 MFMA accumulator for the whole sequence.  Its 16-bit
// copy is the B operand of the products directly: an accumulator-layout tile
// holds, per lane, 4 consecutive rows of one column, and two such tiles make
// the 8 K elements of a 16x16x32 operand lane.  The record stores the other
// operands in that same K order.  All products are 16x16x32 f16 MFMAs, fed by
// fp32 accumulators or VALU-written initial values only.
//
// The workgroup copies the next chunk's record into the other half of a
// double-buffered LDS stage (direct global-to-LDS loads) while the current
// chunk is computed.
#include <hip/hip_runtime.h>

#include "gdr2_chunk_common.h"
#include "gdr2_internal.h"

namespace gdr2 {

namespace {

template <int DK, int DV, int NWV, int NP>
struct StateCfg {
  typedef Rec<DK, DV> R;
  static constexpr int NTH = 64 * (NWV + NP);
  static constexpr int DVB = 16 * NWV;                       // value channels per workgroup
  static constexpr size_t O_GC = R::GC;                      // shared part: record [0, R::U)
  static constexpr size_t O_U = R::U;                        // then this block's U tiles
  static constexpr size_t STAGE = O_U + (size_t)NWV * 4 * R::TILE;
  static constexpr int NCP = (int)(STAGE / 16);              // 16-byte pieces per stage
  static constexpr size_t BYTES = 2 * STAGE;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
};

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

// 16 bytes from global memory to LDS without a register round trip: lane l
// of the wavefront writes lds_run + 16*l (lds_run is uniform).
__device__ __forceinline__ void lds_dma16(const void* src, unsigned char* lds_run) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_run, 16, 0, 0);
}

__device__ __forceinline__ f16x8 join8(const f32x4& a, const f32x4& b) {
  return f16x8{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
               (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
}

}  // namespace

// NWV compute wavefronts and NP producer wavefronts; one workgroup per CU
// (LDS-bound), so each wavefront may use a whole SIMD's registers.
template <int DK, int DV, int NWV, int NP>
__global__ __launch_bounds__(64 * (NWV + NP), 1) void state_kernel(StateArgs p) {
  typedef StateCfg<DK, DV, NWV, NP> Cfg;
  typedef Rec<DK, DV> R;
  constexpr int NKB = R::NKB, NIB = R::NIB, NCP = Cfg::NCP;

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 15, g4 = lane >> 4;

  // ---- which (sequence, head, value block) this workgroup owns -------------------
  // the blocks of one (sequence, head) share an XCD, so their record reads hit
  // that XCD's L2
  constexpr int NB = DV / Cfg::DVB;
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const int pair = (slot / NB) * 8 + xcd;
  const int jb = slot % NB;
  if (pair >= p.N * p.H) return;
  const int H = p.H;
  const int h = pair % H;
  const int n = p.order ? p.order[pair / H] : pair / H;
  long long tok0;
  int len, cb;
  if (p.cu) {
    int s = p.cu[n], e = p.cu[n + 1];
    s = s < 0 ? 0 : (s > p.T ? p.T : s);
    e = e < s ? s : (e > p.T ? p.T : e);
    tok0 = s;
    len = e - s;
    cb = p.cbase[n];
  } else {
    tok0 = (long long)n * p.T;
    len = p.T;
    cb = n * ((p.T + CH - 1) / CH);
  }
  int nch = (len + CH - 1) / CH;
  if (cb + nch > p.cap) nch = max(0, p.cap - cb);  // only inputs that break the cu_seqlens contract
  const size_t nh = (size_t)n * H + h;
  const bool producer = wv >= NWV;
  const int col0 = Cfg::DVB * jb + 16 * (producer ? 0 : wv);  // this wavefront's first value channel
  const size_t olane = ((size_t)m * H + h) * DV + col0 + 4 * g4;  // output element of row m of a chunk

  // ---- state: fp32 accumulators, tile ib holds S[16ib + 4*g4 + q][col0 + m] -------
  f32x4 S[NIB];
#pragma unroll
  for (int ib = 0; ib < NIB; ++ib) {
    S[ib] = zero4();
    if (p.S0 && !producer) {
#pragma unroll
      for (int q = 0; q < 4; ++q) S[ib][q] = p.S0[(nh * DK + 16 * ib + 4 * g4 + q) * DV + col0 + m];
    }
  }

  // ---- record staging ------------------------------------------------------------
  // The stage is the record's shared part [0, R::U) followed by this block's
  // NWV column tiles of U (contiguous in the record).  Pieces of 16 B go
  // straight from global memory to LDS, one 1 KiB run of 64 pieces per
  // wavefront instruction, so no registers hold them in flight.
  constexpr int RUNS = (NCP + 63) / 64;
  constexpr int NSH = (int)(R::U / 16);  // shared pieces
  const size_t uoff = (size_t)jb * NWV * 4 * R::TILE;  // this block's U tiles inside the record's U
  // The producer wavefronts copy chunk c's record into stage buffer `buf`; a
  // wavefront issues its memory instructions in order, so keeping the copies
  // off the compute wavefronts lets both proceed at once.
  constexpr int KPW = (RUNS + NP - 1) / NP;  // runs per producer wavefront
  auto stage_async = [&](int c, int buf) {
    const char* rec = p.rec + ((size_t)(cb + c) * H + h) * R::BYTES;
    unsigned char* dst = smem + (size_t)buf * Cfg::STAGE;
#pragma unroll
    for (int k = 0; k < KPW; ++k) {
      const int run = k * NP + (wv - NWV);  // uniform across the wavefront
      const int xp = run * 64 + lane;
      const char* src = rec + (size_t)xp * 16 + (xp < NSH ? 0 : uoff);
      if (run < RUNS - 1 || (run == RUNS - 1 && (NCP % 64 == 0 || xp < NCP)))
        lds_dma16(src, dst + (size_t)run * 1024);
    }
  };

  if (producer && nch > 0) {
    stage_async(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's pieces have landed
  }
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    if (producer) {
      // the other buffer was last read in chunk c - 1, which every wavefront has left
      if (c + 1 < nch) stage_async(c + 1, (c + 1) & 1);
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next chunk's pieces have landed
      __syncthreads();
      continue;
    }
    const unsigned char* L = smem + (size_t)(c & 1) * Cfg::STAGE;
    const int clen = min(CH, len - c * CH);

    // 16-bit state operand: fragment kb = tiles 2kb, 2kb+1 (dk rows 32kb + ...)
    f16x8 sf[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sf[kb] = join8(S[2 * kb], S[2 * kb + 1]);

    // ---- R = U + (-Y) S and the state part of O^T, S^T Q_g^T (independent
    // of R), as eight interleaved accumulator chains.  Rt[a] holds
    // R[16a + 4*g4 + q][col0 + m]; O[a] holds O[16a + m][col0 + 4*g4 + q]. ----
    f32x4 Rt[4], O[4];
    {
      f16x8 yf[4][NKB], qf[4][NKB];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          yf[a][kb] = *reinterpret_cast<const f16x8*>(L + R::YN + ((size_t)(a * NKB + kb) * 64 + lane) * 16);
          qf[a][kb] = *reinterpret_cast<const f16x8*>(L + R::QG + ((size_t)(a * NKB + kb) * 64 + lane) * 16);
        }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f16x4 u = *reinterpret_cast<const f16x4*>(L + Cfg::O_U + ((size_t)(wv * 4 + a) * 64 + lane) * 8);
        Rt[a] = f32x4{(float)u[0], (float)u[1], (float)u[2], (float)u[3]};
        O[a] = zero4();
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          Rt[a] = mma32(yf[a][kb], sf[kb], Rt[a]);
          O[a] = mma32(sf[kb], qf[a][kb], O[a]);
        }
    }
    const f16x8 rf[2] = {join8(Rt[0], Rt[1]), join8(Rt[2], Rt[3])};

    // ---- O^T += R^T A_qk^T, then the output tile in bf16 ----
    {
      f16x8 af[6];
#pragma unroll
      for (int f = 0; f < 6; ++f)
        af[f] = *reinterpret_cast<const f16x8*>(L + R::AQK + ((size_t)f * 64 + lane) * 16);
      // A_qk tile (a, p) exists for p <= a / 2; index a for a < 2, 2a - 2 + p above
      O[0] = mma32(rf[0], af[0], O[0]);
      O[1] = mma32(rf[0], af[1], O[1]);
      O[2] = mma32(rf[0], af[2], O[2]);
      O[3] = mma32(rf[0], af[4], O[3]);
      O[2] = mma32(rf[1], af[3], O[2]);
      O[3] = mma32(rf[1], af[5], O[3]);
      __bf16* orow = static_cast<__bf16*>(p.o) + ((size_t)(tok0 + (long long)c * CH) * H) * DV + olane;
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (16 * a + m < clen)
          *reinterpret_cast<bf16x4*>(orow + (size_t)16 * a * H * DV) =
              bf16x4{(__bf16)O[a][0], (__bf16)O[a][1], (__bf16)O[a][2], (__bf16)O[a][3]};
    }

    // ---- S <- Diag(gamma_C) S + K_tail^T R ----
    {
      f16x8 kf[NIB][2];
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
          kf[ib][pp] = *reinterpret_cast<const f16x8*>(L + R::KT + ((size_t)(ib * 2 + pp) * 64 + lane) * 16);
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) {
        const float4 gc = *reinterpret_cast<const float4*>(L + Cfg::O_GC + (size_t)(16 * ib + 4 * g4) * 4);
        S[ib][0] *= gc.x;
        S[ib][1] *= gc.y;
        S[ib][2] *= gc.z;
        S[ib][3] *= gc.w;
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) S[ib] = mma32(kf[ib][pp], rf[pp], S[ib]);
    }

    __syncthreads();
  }

  if (p.ST && !producer) {
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
      for (int q = 0; q < 4; ++q) p.ST[(nh * DK + 16 * ib + 4 * g4 + q) * DV + col0 + m] = S[ib][q];
  }
}

hipError_t launch_intra(const IntraArgs& a, int dk, int dv, hipStream_t stream);

template <int DK, int DV, int NWV, int NP>
static hipError_t launch_state1(const StateArgs& a, hipStream_t stream) {
  typedef StateCfg<DK, DV, NWV, NP> Cfg;
  constexpr int NB = DV / Cfg::DVB;
  const long long pairs = (long long)a.N * a.H;
  const long long grid = (pairs + 7) / 8 * 8 * NB;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !attr_set[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&state_kernel<DK, DV, NWV, NP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::BYTES);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev] = true;
  }
  hipLaunchKernelGGL((state_kernel<DK, DV, NWV, NP>), dim3((unsigned)grid), dim3(Cfg::NTH), Cfg::BYTES,
                     stream, a);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_state_dv(const StateArgs& a, hipStream_t stream) {
  // Two compute wavefronts (32 value channels) and four producers per
  // workgroup; with too few (sequence, head) chains to cover the CUs that
  // way, blocks of 16 channels double the number of workgroups.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if ((long long)a.N * a.H * (DV / 32) < cus) return launch_state1<DK, DV, 1, 4>(a, stream);
  return launch_state1<DK, DV, 2, 4>(a, stream);
}

hipError_t launch_two_pass(const IntraArgs& ia, const StateArgs& sa, int dk, int dv, hipStream_t stream) {
  hipError_t e = launch_intra(ia, dk, dv, stream);
  if (e != hipSuccess) return e;
#define GDR2_STATE(DK, DV) \
  if (dk == DK && dv == DV) return launch_state_dv<DK, DV>(sa, stream);
  GDR2_STATE(32, 32) GDR2_STATE(32, 64) GDR2_STATE(32, 128)
  GDR2_STATE(64, 32) GDR2_STATE(64, 64) GDR2_STATE(64, 128)
  GDR2_STATE(128, 32) GDR2_STATE(128, 64) GDR2_STATE(128, 128)
#undef GDR2_STATE
  return hipErrorInvalidValue;
}

}  // namespace gdr2
