// gdr2_state.hip -- sequential state pass of the two-pass chunkwise forward
// (Gated DeltaNet-2 pages, "Chunkwise Parallel Training via WY
// Representation", Step 3: state and output equations, Eqs. 23-24; packed
// sequences per Appendix C.6).
//
// A workgroup owns one (sequence, head, block of 16*CT*NWV value channels) and
// walks the sequence's chunks in order; wavefront w owns CT tiles of 16 value
// channels and uses every operand fragment it reads for all of them.
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
// Producer wavefronts copy the records of the next chunks into LDS stage
// buffers (direct global-to-LDS loads) while the current chunk is computed.
// With one column tile per wavefront, the compute wavefronts take Q_g's
// fragments straight into registers, one chunk ahead, and the stage, compacted
// over that gap, is triple-buffered (two chunks ahead); otherwise the whole
// record is double-buffered.
//
// Split chains.  Eq. 23 makes each chunk an affine map of the state,
// S -> M S + K_tail^T U with M = Diag(gamma_C) - K_tail^T Y, so a run of chunks
// is the affine map S -> Phi S + E with Phi the product of their M.  With few
// long chains the pass is cut into segments that run at once:
//   1. the transfer pass (XF) runs the recurrence of each segment on the
//      columns of the identity with U = 0, which gives Phi, and on a zero
//      state, which gives E (segment 0 starts from S0 and gives its true end
//      state directly); it needs neither Q_g nor an output;
//   2. scan_kernel chains the segments in fp32: X_s = Phi_s X_{s-1} + E_s;
//   3. the state pass runs every segment from its true entry state X_{s-1}.
// Each chain is then about 2/P as long, at the price of the transfer pass's
// extra dk columns per segment.
#include <hip/hip_runtime.h>

#include "gdr2_chunk_common.h"
#include "gdr2_internal.h"

namespace gdr2 {

namespace {

template <int DK, int DV, int NWV, int NP, int CT, bool XF>
struct StateCfg {
  typedef Rec<DK, DV> R;
  static constexpr int NTH = 64 * (NWV + NP);
  // columns per workgroup: value channels, or for the transfer pass the dk
  // identity columns followed by the dv value channels
  static constexpr int DVB = 16 * CT * NWV;
  static_assert(!XF || DVB == DK + DV, "a transfer workgroup covers every column");
  static constexpr int UT = XF ? DV / 16 : CT * NWV;         // U column tiles staged
  static constexpr size_t O_GC = R::GC;                      // shared part: record [0, R::U)
  static constexpr size_t O_U = R::U;                        // then this block's U tiles
  static constexpr size_t STAGE = O_U + (size_t)UT * 4 * R::TILE;
  static constexpr int NCP = (int)(STAGE / 16);              // 16-byte pieces per stage
  // The state pass with one column tile per wavefront (QREG) keeps Q_g out of
  // the stage: the compute wavefronts load its fragments into registers one
  // chunk ahead, and the stage, compacted over the gap, is triple-buffered.
  static constexpr bool QREG = !XF && CT == 1;
  static constexpr size_t QGS = R::KT - R::QG;               // bytes of Q_g
  static constexpr size_t SSTR = QREG ? STAGE - QGS : STAGE; // stage stride in LDS
  static constexpr int NBUF = QREG ? 3 : 2;
  static constexpr size_t BYTES = NBUF * SSTR;
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
// XF = false: the state pass (whole chains, packed sequences, or every segment
// of split chains); XF = true: the transfer pass of split chains.
// vmcnt(n) with lgkmcnt and expcnt left open (gfx9 encoding: vmcnt bits
// [3:0] and [15:14])
constexpr unsigned vmcnt_enc(int n) { return 0x0f70u | (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14); }

template <int DK, int DV, int NWV, int NP, bool XF, int CT>
__global__ __launch_bounds__(64 * (NWV + NP), 1) void state_kernel(StateArgs p) {
  typedef StateCfg<DK, DV, NWV, NP, CT, XF> Cfg;
  typedef Rec<DK, DV> R;
  constexpr int NKB = R::NKB, NIB = R::NIB, NCP = Cfg::NCP;

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 15, g4 = lane >> 4;

  // ---- which (chain, column block) this workgroup owns ------------------------------
  // A chain is a (sequence, head), or a (sequence, segment, head) of a split
  // chain.  The blocks of one chain share an XCD, so their record reads hit
  // that XCD's L2.  A transfer workgroup covers all columns of its segment:
  // the wavefronts below DK / (16 CT) run identity columns, the rest value
  // columns.
  constexpr int NB = XF ? 1 : DV / Cfg::DVB;
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const int pair = (slot / NB) * 8 + xcd;
  const int jb = slot % NB;
  const int H = p.H;
  const int h = pair % H;
  // this chain's sequence n, its segment seg of nseg, and the slot sh of
  // (sequence, segment, head) in phi and ex
  int n, seg, nseg;
  size_t sh;
  long long tok0;
  int len, cb;
  if (p.seg) {
    // split packed sequences: chain = (segment id, head), every segment id of
    // the plan in both passes; the transfer pass skips each sequence's last
    const int g = pair / H;
    if (pair >= p.nsmax * H || g >= *p.nseg) return;
    n = p.seg[4 * g];
    seg = g - p.seg[4 * g + 3];
    nseg = p.sq[2 * n + 1];
    if (XF && seg == nseg - 1) return;
    sh = (size_t)g * H + h;
    int s = p.cu[n], e = p.cu[n + 1];
    s = s < 0 ? 0 : (s > p.T ? p.T : s);
    e = e < s ? s : (e > p.T ? p.T : e);
    const int c0 = p.seg[4 * g + 1];
    tok0 = (long long)s + (long long)c0 * CH;
    len = max(0, min(e - s - c0 * CH, p.seg[4 * g + 2] * CH));
    cb = p.cbase[n] + c0;
  } else {
    const int SP = XF ? p.P - 1 : p.P;  // segments per sequence in this pass
    if (pair >= p.N * SP * H) return;
    seg = (pair / H) % SP;
    n = p.order ? p.order[pair / H] : pair / (H * SP);
    nseg = p.P;
    sh = ((size_t)n * p.P + seg) * H + h;
    if (p.cu) {
      int s = p.cu[n], e = p.cu[n + 1];
      s = s < 0 ? 0 : (s > p.T ? p.T : s);
      e = e < s ? s : (e > p.T ? p.T : e);
      tok0 = s;
      len = e - s;
      cb = p.cbase[n];
    } else {
      // segc is the whole sequence's chunk count when chains are not split
      const int c0 = seg * p.segc;
      tok0 = (long long)n * p.T + (long long)c0 * CH;
      len = max(0, min(p.T - c0 * CH, p.segc * CH));
      cb = n * ((p.T + CH - 1) / CH) + c0;
    }
  }
  // transfer pass: this wavefront runs columns of the identity (segment 0
  // forms a transfer matrix too, unused: it starts from S0)
  const bool ident = XF && 16 * CT * wv < DK;
  int nch = (len + CH - 1) / CH;
  if (cb + nch > p.cap) nch = max(0, p.cap - cb);  // only inputs that break the cu_seqlens contract
  const size_t nh = (size_t)n * H + h;
  const bool producer = wv >= NWV;
  // this wavefront's first column (of the identity, or a value channel); its
  // tile ct covers columns col0 + 16*ct + [0, 16)
  const int col0 = producer ? 0 : XF ? (ident ? 16 * CT * wv : 16 * CT * wv - DK) : Cfg::DVB * jb + 16 * CT * wv;
  const size_t olane = ((size_t)m * H + h) * DV + col0 + 4 * g4;  // output element of row m of a chunk

  // ---- state: fp32 accumulators, tile ib holds S[16ib + 4*g4 + q][col0 + m] -------
  // S_T may alias S0, and with split chains the last segment writes S_T while
  // segment 0 of the same launch starts: the transfer pass keeps a copy of S0
  // in the spare slot ex[P - 1] for the state pass to start segment 0 from.
  float* s0copy = nseg > 1 ? p.ex + (sh + (size_t)(nseg - 1 - seg) * H) * (size_t)(DK * DV) : nullptr;
  const float* sin = nullptr;  // entry state, [DK][DV] row-major
  if (XF) {
    if (!ident && seg == 0 && p.S0) sin = p.S0 + nh * (size_t)(DK * DV);
  } else if (seg == 0) {
    if (p.S0) sin = nseg > 1 ? s0copy : p.S0 + nh * (size_t)(DK * DV);
  } else {
    sin = p.ex + (sh - H) * (size_t)(DK * DV);  // the end state of segment seg - 1
  }
  f32x4 S[CT][NIB];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      S[ct][ib] = zero4();
      if (!producer) {
        const int col = col0 + 16 * ct + m;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 16 * ib + 4 * g4 + q;
          if (XF && ident) {
            S[ct][ib][q] = row == col ? 1.f : 0.f;
          } else if (sin) {
            S[ct][ib][q] = sin[(size_t)row * DV + col];
            if (XF) s0copy[(size_t)row * DV + col] = S[ct][ib][q];
          }
        }
      }
    }

  // ---- record staging ------------------------------------------------------------
  // The stage is the record's shared part [0, R::U) followed by this block's
  // CT*NWV column tiles of U (contiguous in the record).  Pieces of 16 B go
  // straight from global memory to LDS, one 1 KiB run of 64 pieces per
  // wavefront instruction, so no registers hold them in flight.  The transfer
  // pass skips the runs of Q_g and A_qk (it forms no output) and keeps the
  // record's offsets in LDS; the QREG state pass skips Q_g and compacts.
  constexpr int RUNS = (NCP + 63) / 64;
  constexpr int NSH = (int)(R::U / 16);  // shared pieces
  static_assert(R::QG % 1024 == 0 && R::KT % 1024 == 0 && R::AQK % 1024 == 0 && R::GC % 1024 == 0,
                "Q_g and A_qk must occupy whole runs");
  constexpr bool QREG = Cfg::QREG;
  constexpr int QR0 = (XF || QREG) ? (int)(R::QG / 1024) : 0, QRN = (XF || QREG) ? (int)((R::KT - R::QG) / 1024) : 0;
  constexpr int AR0 = XF ? (int)(R::AQK / 1024) : 0, ARN = XF ? (int)((R::GC - R::AQK) / 1024) : 0;
  constexpr int npiece = NCP;
  constexpr int nrun = (npiece + 63) / 64 - QRN - ARN;
  const size_t uoff = (size_t)jb * Cfg::UT * 4 * R::TILE;  // this block's U tiles
  // The producer wavefronts copy chunk c's record into stage buffer `buf`; a
  // wavefront issues its memory instructions in order, so keeping the copies
  // off the compute wavefronts lets both proceed at once.
  constexpr int KPW = (RUNS - QRN - ARN + NP - 1) / NP;  // runs per producer wavefront
  auto stage_async = [&](int c, int buf) {
    const char* rec = p.rec + ((size_t)(cb + c) * H + h) * R::BYTES;
    unsigned char* dst = smem + (size_t)buf * Cfg::SSTR;
#pragma unroll
    for (int k = 0; k < KPW; ++k) {
      int r = k * NP + (wv - NWV);  // uniform across the wavefront
      if constexpr (QREG) {
        // every producer issues KPW loads (the last run repeated, same bytes),
        // so "this chunk has landed" is a fixed vmcnt
        r = min(r, nrun - 1);
      } else {
        if (r >= nrun) break;
      }
      int run = r < QR0 ? r : r + QRN;  // index among the record's runs
      if (XF && run >= AR0) run += ARN;
      const int xp = run * 64 + lane;
      const char* src = rec + (size_t)xp * 16 + (xp < NSH ? 0 : uoff);
      if (xp < npiece) lds_dma16(src, dst + (size_t)(QREG ? r : run) * 1024);
    }
  };

  // Producers and compute wavefronts run separate loops with one barrier per
  // chunk each, so the producers' address arithmetic is not live in the
  // compute loop.
  if (QREG && producer) {
    // chunk c goes to buffer c % 3, two chunks ahead: during chunk c the
    // producers fill the buffer chunk c - 1 used, then wait until chunk c + 1
    // has landed (chunk c + 2's loads may stay in flight)
    static_assert(KPW < 64, "vmcnt range");
    const int pre = min(2, nch);
    for (int c = 0; c < pre; ++c) stage_async(c, c);
    if (pre == 2) __builtin_amdgcn_s_waitcnt(vmcnt_enc(KPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      if (c + 2 < nch) {
        stage_async(c + 2, (c + 2) % 3);
        __builtin_amdgcn_s_waitcnt(vmcnt_enc(KPW));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
      }
      __syncthreads();
    }
    return;
  }
  if (producer) {
    if (nch > 0) {
      stage_async(0, 0);
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's pieces have landed
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      // the other buffer was last read in chunk c - 1, which every wavefront has left
      if (c + 1 < nch) stage_async(c + 1, (c + 1) & 1);
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next chunk's pieces have landed
      __syncthreads();
    }
    return;
  }
  __syncthreads();

  // operand offsets in the stage (the QREG stage lacks Q_g's bytes)
  constexpr size_t SHIFT = QREG ? Cfg::QGS : 0;
  constexpr size_t OK = R::KT - SHIFT, OA = R::AQK - SHIFT, OG = Cfg::O_GC - SHIFT, OU = Cfg::O_U - SHIFT;
  // QREG: Q_g fragments of the current chunk, loaded during the previous one
  f16x8 qreg[QREG ? 4 : 1][QREG ? NKB : 1];
  auto load_qg = [&](int c) {
    if constexpr (QREG) {
      const char* rq = p.rec + ((size_t)(cb + c) * H + h) * R::BYTES + R::QG;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          qreg[a][kb] = *reinterpret_cast<const f16x8*>(rq + ((size_t)(a * NKB + kb) * 64 + lane) * 16);
    }
  };
  if (nch > 0) load_qg(0);
  for (int c = 0; c < nch; ++c) {
    const unsigned char* L = smem + (size_t)(c % Cfg::NBUF) * Cfg::SSTR;
    const int clen = min(CH, len - c * CH);

    // 16-bit state operand: fragment kb = tiles 2kb, 2kb+1 (dk rows 32kb + ...)
    f16x8 sf[CT][NKB];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sf[ct][kb] = join8(S[ct][2 * kb], S[ct][2 * kb + 1]);

    // ---- R = U + (-Y) S and the state part of O^T, S^T Q_g^T (independent
    // of R), as interleaved accumulator chains.  Rt[ct][a] holds
    // R[16a + 4*g4 + q][col0 + 16ct + m]; O[ct][a] holds
    // O[16a + m][col0 + 16ct + 4*g4 + q]. ----
    f32x4 Rt[CT][4], O[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (XF && ident) {
          Rt[ct][a] = zero4();
        } else {
          // this tile's U columns, relative to the block's first
          const int jt = (col0 - Cfg::DVB * jb) / 16 + ct;
          const f16x4 u = *reinterpret_cast<const f16x4*>(L + OU + ((size_t)(jt * 4 + a) * 64 + lane) * 8);
          Rt[ct][a] = f32x4{(float)u[0], (float)u[1], (float)u[2], (float)u[3]};
        }
        O[ct][a] = zero4();
      }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f16x8 yf = *reinterpret_cast<const f16x8*>(L + R::YN + ((size_t)(a * NKB + kb) * 64 + lane) * 16);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Rt[ct][a] = mma32(yf, sf[ct][kb], Rt[ct][a]);
        if constexpr (!XF) {
          f16x8 qf;
          if constexpr (QREG) qf = qreg[QREG ? a : 0][QREG ? kb : 0];
          else qf = *reinterpret_cast<const f16x8*>(L + R::QG + ((size_t)(a * NKB + kb) * 64 + lane) * 16);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) O[ct][a] = mma32(sf[ct][kb], qf, O[ct][a]);
        }
      }
    // the next chunk's Q_g fragments, in flight over the rest of this chunk
    if (QREG && c + 1 < nch) load_qg(c + 1);
    f16x8 rf[CT][2];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      rf[ct][0] = join8(Rt[ct][0], Rt[ct][1]);
      rf[ct][1] = join8(Rt[ct][2], Rt[ct][3]);
    }

    // ---- O^T += R^T A_qk^T, then the output tile in bf16 ----
    if constexpr (!XF) {
      f16x8 af[6];
#pragma unroll
      for (int f = 0; f < 6; ++f)
        af[f] = *reinterpret_cast<const f16x8*>(L + OA + ((size_t)f * 64 + lane) * 16);
      const size_t obase = ((size_t)(tok0 + (long long)c * CH) * H) * DV + olane;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        // A_qk tile (a, p) exists for p <= a / 2; index a for a < 2, 2a - 2 + p above
        O[ct][0] = mma32(rf[ct][0], af[0], O[ct][0]);
        O[ct][1] = mma32(rf[ct][0], af[1], O[ct][1]);
        O[ct][2] = mma32(rf[ct][0], af[2], O[ct][2]);
        O[ct][3] = mma32(rf[ct][0], af[4], O[ct][3]);
        O[ct][2] = mma32(rf[ct][1], af[3], O[ct][2]);
        O[ct][3] = mma32(rf[ct][1], af[5], O[ct][3]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
          if (16 * a + m < clen) {
            const size_t oi = obase + (size_t)16 * a * H * DV + 16 * ct;
            if (p.o_f32)  // uniform: fp32 output rows
              *reinterpret_cast<float4*>(static_cast<float*>(p.o) + oi) =
                  make_float4(O[ct][a][0], O[ct][a][1], O[ct][a][2], O[ct][a][3]);
            else
              *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.o) + oi) =
                  bf16x4{(__bf16)O[ct][a][0], (__bf16)O[ct][a][1], (__bf16)O[ct][a][2], (__bf16)O[ct][a][3]};
          }
      }
    }

    // ---- S <- Diag(gamma_C) S + K_tail^T R ----
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      const float4 gc = *reinterpret_cast<const float4*>(L + OG + (size_t)(16 * ib + 4 * g4) * 4);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        S[ct][ib][0] *= gc.x;
        S[ct][ib][1] *= gc.y;
        S[ct][ib][2] *= gc.z;
        S[ct][ib][3] *= gc.w;
      }
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) {
        const f16x8 kf = *reinterpret_cast<const f16x8*>(L + OK + ((size_t)(ib * 2 + pp) * 64 + lane) * 16);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) S[ct][ib] = mma32(kf, rf[ct][pp], S[ct][ib]);
      }

    __syncthreads();
  }

  float* sout = nullptr;  // end state, row stride ld
  int ld = DV;
  if (XF) {
    sout = ident ? p.phi + sh * (size_t)(DK * DK) : p.ex + sh * (size_t)(DK * DV);
    ld = ident ? DK : DV;
  } else if (p.ST && seg == nseg - 1) {
    sout = p.ST + nh * (size_t)(DK * DV);
  }
  if (sout) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sout[(size_t)(16 * ib + 4 * g4 + q) * ld + col0 + 16 * ct + m] = S[ct][ib][q];
  }
}

// Chains the segments of split chains: for each (sequence, head) and block of
// 16 value columns, X_0 = ex[0] and X_s = Phi_s X_{s-1} + E_s for s = 1 .. P - 2,
// each written over ex[s].  fp32 throughout: wavefront w forms rows
// 16w .. 16w + 15 of X_s with 16x16x4 fp32 MFMAs, and X_{s-1} sits in LDS,
// transposed so that a lane's four K values are one 16-byte read; four
// accumulators split each product's K range.  Each step is short next to a
// memory latency, so the rows of Phi and the tile of E are loaded DEPTH
// steps ahead into a ring of register slots.
template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void scan_kernel(StateArgs p) {
  constexpr int NJ = DV / 16, NK = DK / 16, DEPTH = 4;
  __shared__ __align__(16) float XT[16][DK + 4];  // X_{s-1} transposed: XT[column][row]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  // the NJ column blocks of one (sequence, head) share an XCD and so read
  // each Phi_s through one L2
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const int nh = (slot / NJ) * 8 + xcd, j0 = 16 * (slot % NJ);
  const int n = nh / p.H, h = nh % p.H;
  if (n >= p.N) return;
  // (n, segment 0, h) and the segment count: fixed per sequence, or from the
  // plan of split packed sequences
  const int P = p.seg ? p.sq[2 * n + 1] : p.P;
  const size_t base = p.seg ? (size_t)p.sq[2 * n] * p.H + h : (size_t)n * p.P * p.H + h;
  const int last = P - 2;  // steps s = 1 .. last
  if (last < 1) return;
  const float* x0 = p.ex + base * (size_t)(DK * DV);
  for (int i = tid; i < DK * 16; i += 64 * NK) XT[i & 15][i >> 4] = x0[(size_t)(i >> 4) * DV + j0 + (i & 15)];

  float4 fa[DEPTH][NK];
  f32x4 ea[DEPTH];
  auto ex_of = [&](int s) { return p.ex + (base + (size_t)s * p.H) * (size_t)(DK * DV); };
  auto fetch = [&](int s, float4 (&f)[NK], f32x4& e) {
    const float* E = ex_of(s);
    const float* F = p.phi + (base + (size_t)s * p.H) * (size_t)(DK * DK);
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
      f[kb] = *reinterpret_cast<const float4*>(F + (size_t)(16 * wv + m) * DK + 16 * kb + 4 * g);
#pragma unroll
    for (int q = 0; q < 4; ++q) e[q] = E[(size_t)(16 * wv + 4 * g + q) * DV + j0 + m];
  };
  // Every step issues the same loads (step indices past the last are clamped
  // to it and their values unused), so the count of loads in flight is the
  // same on every path and each step waits only for its own slot.
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(min(1 + d, last), fa[d], ea[d]);
  __syncthreads();
  for (int s0 = 1; s0 <= last; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int s = s0 + d;
      if (s <= last) {
        float4 xb[NK];
#pragma unroll
        for (int kb = 0; kb < NK; ++kb) xb[kb] = *reinterpret_cast<const float4*>(&XT[m][16 * kb + 4 * g]);
        f32x4 part[4] = {ea[d], zero4(), zero4(), zero4()};
#pragma unroll
        for (int kb = 0; kb < NK; ++kb) part[kb & 3] = mma16(fa[d][kb], xb[kb], part[kb & 3]);
        const f32x4 acc = (part[0] + part[1]) + (part[2] + part[3]);
        __syncthreads();  // every wavefront has read X_{s-1}
        float* E = ex_of(s);
        *reinterpret_cast<float4*>(&XT[m][16 * wv + 4 * g]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
        for (int q = 0; q < 4; ++q) E[(size_t)(16 * wv + 4 * g + q) * DV + j0 + m] = acc[q];
        __syncthreads();
      }
      fetch(min(s + DEPTH, last), fa[d], ea[d]);  // refill the slot just used
    }
  }
}

hipError_t launch_intra(const IntraArgs& a, int dk, int dv, hipStream_t stream);

template <int DK, int DV, int NWV, int NP, bool XF, int CT = 1>
static hipError_t launch_state1(const StateArgs& a, hipStream_t stream) {
  typedef StateCfg<DK, DV, NWV, NP, CT, XF> Cfg;
  constexpr int NB = XF ? 1 : DV / Cfg::DVB;
  const long long pairs = a.seg ? (long long)a.nsmax * a.H : (long long)a.N * (XF ? a.P - 1 : a.P) * a.H;
  const long long grid = (pairs + 7) / 8 * 8 * NB;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  static std::atomic<bool> lds_set[64];
  const hipError_t e =
      lds_opt_in(reinterpret_cast<const void*>(&state_kernel<DK, DV, NWV, NP, XF, CT>), Cfg::BYTES, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((state_kernel<DK, DV, NWV, NP, XF, CT>), dim3((unsigned)grid), dim3(Cfg::NTH), Cfg::BYTES,
                     stream, a);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_state_dv(const StateArgs& a, hipStream_t stream) {
  if (a.P > 1 || a.seg) {
    // split chains: one workgroup per segment covers every column, so the
    // shared part of each record is staged once per segment; two column tiles
    // per wavefront halve the LDS reads of the shared operands
    if constexpr (DK == DV) {
      constexpr int NW = DV / 32;
      hipError_t e = launch_state1<DK, DV, 2 * NW, 4, true, 2>(a, stream);
      if (e != hipSuccess) return e;
      // split packed sequences: the plan on the device decides which
      // sequences have segments to chain, so the scan always runs
      if (a.P > 2 || a.seg) {
        const long long grid = ((long long)a.N * a.H + 7) / 8 * 8 * (DV / 16);
        if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL((scan_kernel<DK, DV>), dim3((unsigned)grid), dim3(64 * (DK / 16)), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      return launch_state1<DK, DV, NW, 4, false, 2>(a, stream);
    } else {
      return hipErrorInvalidValue;
    }
  }
  // With at least one (sequence, head) chain per CU the pass is bound by the
  // total record staging, so one workgroup per chain covers every value
  // channel (two column tiles per wavefront) and stages each record once.
  // With fewer chains the chain length binds: two compute wavefronts (32
  // value channels) and four producers per workgroup, or blocks of 16
  // channels when even that leaves CUs idle.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const long long chains = (long long)a.N * a.H;
  if (chains >= cus) return launch_state1<DK, DV, DV / 32, 4, false, 2>(a, stream);
  if (chains * (DV / 32) < cus) return launch_state1<DK, DV, 1, 4, false>(a, stream);
  return launch_state1<DK, DV, 2, 4, false>(a, stream);
}

int segments_for(long long chains, long long nc, int dk, int dv) {
  // Enough chains fill the CUs by themselves; otherwise split each chain into
  // a power of two of segments, at most 16, so that the state pass has up to
  // 256 segment chains (one workgroup each), each of at least 16 chunks.
  if (dk != dv || chains <= 0 || chains >= 64) return 1;
  long long P = 1;
  while (P < 16 && chains * P * 2 <= 256 && nc / (P * 2) >= 16) P *= 2;
  return (int)P;
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
