// gdr2_chunk.hip -- chunkwise forward of the Gated Delta Rule-2 operator on
// gfx950 (Gated DeltaNet-2 pages, "Chunkwise Parallel Training via WY
// Representation", Steps 1-3, Eqs. 20-24; packed sequences per Appendix C.6).
//
// One workgroup (512 threads, 8 wavefronts) owns one (sequence, head, block
// of DVB value channels) and walks the sequence's 64-token chunks in order.
// The value channels of the state are independent of each other (every
// key-side quantity is shared, and column j of S, U, R, O depends only on
// column j of S0 and Z), so splitting dv across workgroups needs no exchange.
// Each workgroup recomputes the key-side chunk quantities; the workgroups of
// one (sequence, head) are placed on the same XCD so their repeated key-side
// reads hit that XCD's L2.  Nothing is written to HBM but o and S_T.
//
// Per chunk, with G the fp32 cumulative log-decay from the chunk start (kept
// in log2 units) and c(r) = 16*(r/16) + 7 the centre row of row r's 16-row
// block:
//   L   the raw q, k, g, b, v, w of the chunk come from registers filled
//       during the previous chunk, and the next chunk's loads are issued.
//       G by a DPP scan; centred decay factors e1 = 2^(G_r - G_c(r)) and
//       e2 = 2^(G_c(r) - G_r), so no factor exceeds the decay over 8 tokens;
//       E' = e1*b*k, K' = e2*k, Q' = e1*q, and the un-centred E = gamma*b*k,
//       Q_g = gamma*q, K_tail = (gamma_C/gamma)*k, Z = w*v (Step 1, Eq. 20).
//       Each thread owns consecutive rows, so the transposed copies E^T,
//       K_tail^T and Z^T are written as vectors.
//   P   T^T = K' E'^T and A_qk^T = K' Q'^T on MFMA (Step 2 and the A_qk of
//       Eq. 24).  Inside a diagonal 16x16 tile the centring cancels; an
//       off-diagonal tile (a, b) scales K' by 2^(G_c(a) - G_c(b)) <= 1 per
//       channel first, which restores the decay between the two centres.
//       Computing the transposes lets each lane store 4 adjacent entries of
//       a row.
//   S   A = (I + T)^-1: the four 16x16 diagonal blocks by fp32 forward
//       substitution, then the off-diagonal blocks by the block recurrence
//       A_ab = A_aa (-sum_{b<=c<a} T_ac A_cb).
//   Y   Y^T = E^T A^T and U = A Z as plain MFMA products (U stays in the
//       registers of the wavefront that turns it into R).
//   R   R = U - Y S                       (chunk-local residual)
//   O   O = Q_g S + A_qk R                (Eq. 24)
//       S <- Diag(gamma_C) S + K_tail^T R (Eq. 23)
// The state stays in fp32 MFMA accumulators for the whole sequence.
//
// Operand precision: with fp32 inputs every product is fp32 MFMA.  With bf16
// inputs T uses bf16 operands, A_qk a bf16 hi/lo split (three products), and
// every state-pass operand (A, Y, Z, R, Q_g, K_tail, A_qk, S) is fp16: these
// are bounded by |q|, |k|, |b k| and the state, and fp16 keeps 3 more mantissa
// bits than bf16, which the output needs because Q_g S and A_qk Y S nearly
// cancel.  Accumulation is always fp32.  Every MFMA accumulator chain uses a
// single instruction shape (see gdr2_device.h).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdr2_chunk_common.h"
#include "gdr2_internal.h"

namespace gdr2 {

constexpr int NT = 512;  // threads per workgroup
constexpr int NW = 8;    // wavefronts per workgroup (two per SIMD)

template <int DK, int DVB, bool F32>
struct ChunkCfg {
  typedef typename std::conditional<F32, float, __bf16>::type KT;    // T / A_qk operands
  typedef typename std::conditional<F32, float, _Float16>::type ST;  // state-pass operands
  typedef typename std::conditional<F32, float4, f16x4>::type SV4;
  static constexpr int PAD = F32 ? 4 : 8;  // row padding (elements) against bank conflicts
  static constexpr int LDK = DK + PAD;     // rows of [64][DK] and [DVB][DK]
  static constexpr int LDC = CH + PAD;     // rows of [*][64]
  static constexpr size_t SK = sizeof(KT), SS = sizeof(ST);
  // region X, phase P set: E', K'hi, (K'lo), Q'hi, (Q'lo)  [64][LDK] KT
  static constexpr int NKT = F32 ? 3 : 5;
  static constexpr size_t SZK = (size_t)CH * LDK * SK;
  static constexpr size_t XP = NKT * SZK;
  // region X after phase P: E^T, K_tail^T [DK][LDC]; Q_g, -Y [64][LDK]  (ST)
  static constexpr size_t O_EHT = 0;
  static constexpr size_t O_KTT = O_EHT + (size_t)DK * LDC * SS;
  static constexpr size_t O_QG = O_KTT + (size_t)DK * LDC * SS;
  static constexpr size_t O_YN = O_QG + (size_t)CH * LDK * SS;
  static constexpr size_t XR = O_YN + (size_t)CH * LDK * SS;
  static constexpr size_t X = ((XP > XR ? XP : XR) + 15) / 16 * 16;
  static constexpr size_t O_TD = X;                                 // fp32 [4][16][16] diag T^T
  static constexpr size_t O_TN = O_TD + 4 * 16 * 16 * 4;            // ST [64][LDC]  -T
  static constexpr size_t O_A = O_TN + (size_t)CH * LDC * SS;       // ST [64][LDC]  A
  static constexpr size_t O_AQK = O_A + (size_t)CH * LDC * SS;      // ST [64][LDC]  A_qk
  static constexpr size_t O_ZT = O_AQK + (size_t)CH * LDC * SS;     // ST [DVB][LDC] Z^T
  static constexpr size_t O_RT = O_ZT + (size_t)DVB * LDC * SS;     // ST [DVB][LDC] R^T
  static constexpr size_t O_S = O_RT + (size_t)DVB * LDC * SS;      // ST [2][DVB][LDK] S^T
  static constexpr size_t O_GC = O_S + (size_t)2 * DVB * LDK * SS;  // fp32 [DK] gamma_C
  static constexpr size_t O_GCEN = O_GC + (size_t)DK * 4;           // fp32 [4][DK] block centres
  static constexpr size_t BYTES = O_GCEN + (size_t)4 * DK * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  // phase-L mapping: thread = (column group cg of EPC key channels, row group
  // rg of RPT consecutive rows); the RG row groups of a column group are
  // consecutive lanes of one wavefront.
  static constexpr int EPC = 4, CG = DK / EPC, RG = NT / CG, RPT = CH / RG;
  static_assert(RG >= 16 && RG <= 64 && CH % RG == 0, "bad phase-L mapping");
  // v/w mapping: thread = (value channel vc, row group vq of VR consecutive rows)
  static constexpr int VR = CH * DVB / NT;
  static_assert(VR == 2 || VR == 4, "DVB must be 16 or 32");
  static constexpr int NSTILE = (DK / 16) * (DVB / 16);  // 16x16 state tiles
  static constexpr int NSU = (NSTILE + NW - 1) / NW;     // state tiles per wavefront
  static constexpr int NJT = DVB / 16;                   // value column tiles
  static constexpr int ESZ = F32 ? 4 : 2;                // bytes per stored input element
  static constexpr int KW = F32 ? 4 : 2;                 // dwords per EPC key elements
};

template <int DK, int DVB, bool F32, bool LA16>
__global__ __launch_bounds__(NT) void chunk_fwd_kernel(ChunkArgs p) {
  typedef ChunkCfg<DK, DVB, F32> Cfg;
  typedef typename Cfg::KT KT;
  typedef typename Cfg::ST ST;
  typedef typename Cfg::SV4 SV4;
  constexpr bool BF16 = !F32;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, EPC = Cfg::EPC;
  constexpr int RPT = Cfg::RPT, RG = Cfg::RG, VR = Cfg::VR, NJT = Cfg::NJT;
  constexpr int ESZ = Cfg::ESZ, KW = Cfg::KW, LW = LA16 ? 2 : 4;

  extern __shared__ __align__(16) unsigned char smem[];
  KT* Ep = reinterpret_cast<KT*>(smem);
  KT* Kh = reinterpret_cast<KT*>(smem + Cfg::SZK);
  KT* Kl = reinterpret_cast<KT*>(smem + 2 * Cfg::SZK);  // bf16 path only
  KT* Qh = reinterpret_cast<KT*>(smem + (F32 ? 2 : 3) * Cfg::SZK);
  KT* Ql = reinterpret_cast<KT*>(smem + 4 * Cfg::SZK);  // bf16 path only
  ST* EhT = reinterpret_cast<ST*>(smem + Cfg::O_EHT);
  ST* KtT = reinterpret_cast<ST*>(smem + Cfg::O_KTT);
  ST* Qg = reinterpret_cast<ST*>(smem + Cfg::O_QG);
  ST* Yn = reinterpret_cast<ST*>(smem + Cfg::O_YN);
  float* Tdt = reinterpret_cast<float*>(smem + Cfg::O_TD);
  ST* Tn = reinterpret_cast<ST*>(smem + Cfg::O_TN);
  ST* Am = reinterpret_cast<ST*>(smem + Cfg::O_A);
  ST* Aqk = reinterpret_cast<ST*>(smem + Cfg::O_AQK);
  ST* ZT = reinterpret_cast<ST*>(smem + Cfg::O_ZT);
  ST* RT = reinterpret_cast<ST*>(smem + Cfg::O_RT);
  ST* Sbuf = reinterpret_cast<ST*>(smem + Cfg::O_S);
  float* gC = reinterpret_cast<float*>(smem + Cfg::O_GC);
  float* gcen = reinterpret_cast<float*>(smem + Cfg::O_GCEN);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 15, g4 = lane >> 4;

  // ---- which (sequence, head, value block) this workgroup owns -------------------
  const int NB = p.DV / DVB;
  const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const int pair = (slot / NB) * 8 + xcd;
  const int jb = slot % NB;
  if (pair >= p.N * p.H) return;
  const int h = pair % p.H;
  const int n = p.order ? p.order[pair / p.H] : pair / p.H;
  long long tok0;
  int len;
  if (p.cu) {
    int s = p.cu[n], e = p.cu[n + 1];
    s = s < 0 ? 0 : (s > p.T ? p.T : s);
    e = e < s ? s : (e > p.T ? p.T : e);
    tok0 = s;
    len = e - s;
  } else {
    tok0 = (long long)n * p.T;
    len = p.T;
  }
  const int H = p.H, DV = p.DV;
  const size_t nh = (size_t)n * H + h;
  const int jbase = jb * DVB;

  // the strictly upper blocks of A and A_qk stay zero for the whole sequence;
  // the products below run over them instead of switching instruction shape
  for (int e = tid; e < CH * LDC; e += NT) {
    Am[e] = cvt<ST>(0.f);
    Aqk[e] = cvt<ST>(0.f);
  }

  // ---- state: fp32 accumulators in C layout -------------------------------------------
  f32x4 Sacc[Cfg::NSU];
#pragma unroll
  for (int u = 0; u < Cfg::NSU; ++u) {
    const int t = wv + NW * u;
    Sacc[u] = zero4();
    if (t < Cfg::NSTILE && p.S0) {
      const int ib = t % (DK / 16), jt = t / (DK / 16);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        Sacc[u][q] = p.S0[(nh * DK + 16 * ib + 4 * g4 + q) * DV + jbase + 16 * jt + m];
    }
  }
  ST* Scur = Sbuf;
  ST* Snext = Sbuf + DVB * LDK;
#pragma unroll
  for (int u = 0; u < Cfg::NSU; ++u) {
    const int t = wv + NW * u;
    if (t < Cfg::NSTILE) {
      const int ib = t % (DK / 16), jt = t / (DK / 16);
      *reinterpret_cast<SV4*>(Scur + (16 * jt + m) * LDK + 16 * ib + 4 * g4) = cvt4<SV4>(Sacc[u]);
    }
  }

  // phase-L coordinates: rows r0 .. r0+RPT-1, key channels EPC*cg ..
  const int cg = tid / RG, rg = tid % RG, r0 = rg * RPT;
  // v/w coordinates: value channel vc, rows VR*vq .. VR*vq+VR-1
  const int vc = tid % DVB, vq = tid / DVB;
  // byte offsets of this thread's elements inside a chunk (a chunk spans 64
  // token rows, so 32 bits suffice); the chunk base itself is uniform
  const size_t krow = (size_t)H * DK, vrow = (size_t)H * DV;
  uint32_t koff[RPT], goff[RPT], voff[VR];
#pragma unroll
  for (int pr = 0; pr < RPT; ++pr) {
    koff[pr] = (uint32_t)(((r0 + pr) * krow + EPC * cg) * ESZ);
    goff[pr] = (uint32_t)(((r0 + pr) * krow + EPC * cg) * (LA16 ? 2 : 4));
  }
#pragma unroll
  for (int pr = 0; pr < VR; ++pr) voff[pr] = (uint32_t)(((VR * vq + pr) * vrow + vc) * ESZ);

  // raw inputs of the chunk in flight (registers)
  uint32_t rq[RPT][KW], rk[RPT][KW], rb[RPT][KW], rgd[RPT][LW];
  uint32_t rv[VR], rw[VR];
  // Buffer loads against a per-chunk resource whose range ends at the last
  // valid token row: rows past a ragged end read as zero without branches
  // and nothing outside the caller's tensors is touched.
  auto fetch = [&](int c) {
    const int clen = min(CH, len - c * CH);
    const size_t crow = (size_t)tok0 + (size_t)c * CH;
    const size_t kel = crow * krow + (size_t)h * DK, vel = crow * vrow + (size_t)h * DV + jbase;
    const int kbytes = (int)(clen * krow * ESZ), gbytes = (int)(clen * krow * (LA16 ? 2 : 4));
    const int vbytes = (int)(clen * vrow * ESZ);
    const auto rsq = make_rsrc(static_cast<const char*>(p.q) + kel * ESZ, kbytes);
    const auto rsk = make_rsrc(static_cast<const char*>(p.k) + kel * ESZ, kbytes);
    const auto rsb = make_rsrc(static_cast<const char*>(p.b) + kel * ESZ, kbytes);
    const auto rsg = make_rsrc(static_cast<const char*>(p.la) + kel * (LA16 ? 2 : 4), gbytes);
    const auto rsv = make_rsrc(static_cast<const char*>(p.v) + vel * ESZ, vbytes);
    const auto rsw = make_rsrc(static_cast<const char*>(p.w) + vel * ESZ, vbytes);
#pragma unroll
    for (int pr = 0; pr < RPT; ++pr) {
      bld(rq[pr], rsq, koff[pr]);
      bld(rk[pr], rsk, koff[pr]);
      bld(rb[pr], rsb, koff[pr]);
      // raw words only: expanding bf16 here would wait for the load
      bld(rgd[pr], rsg, goff[pr]);
    }
#pragma unroll
    for (int pr = 0; pr < VR; ++pr) {
      if constexpr (F32) {
        rv[pr] = __builtin_amdgcn_raw_buffer_load_b32(rsv, voff[pr], 0, 0);
        rw[pr] = __builtin_amdgcn_raw_buffer_load_b32(rsw, voff[pr], 0, 0);
      } else {
        rv[pr] = __builtin_amdgcn_raw_buffer_load_b16(rsv, voff[pr], 0, 0);
        rw[pr] = __builtin_amdgcn_raw_buffer_load_b16(rsw, voff[pr], 0, 0);
      }
    }
  };

  // the output tile of a chunk is stored during the next chunk, after its
  // prefetch is issued, so that waiting for one never waits for the other
  bool o_pending = false;
  size_t o_idx = 0;
  float o_val[4] = {0.f, 0.f, 0.f, 0.f};

  const int nchunks = (len + CH - 1) / CH;
  if (nchunks > 0) fetch(0);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const long long ctok = tok0 + (long long)c * CH;
    const int clen = min(CH, len - c * CH);

    // ================= phase L: decay scan and operand tiles ====================
    // E, Q_g, K_tail rows kept packed (16-bit on the bf16 path) until phase S
    SV4 eh[RPT], qg[RPT], kt[RPT];
    {
      float G[RPT][EPC], kv[RPT][EPC], qv[RPT][EPC], bv[RPT][EPC];
      float z[VR];
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) {
        unpack4<F32>(rq[pr], qv[pr]);
        unpack4<F32>(rk[pr], kv[pr]);
        unpack4<F32>(rb[pr], bv[pr]);
        unpack4<!LA16>(rgd[pr], G[pr]);
#pragma unroll
        for (int i = 0; i < EPC; ++i) G[pr][i] *= LOG2E;
      }
#pragma unroll
      for (int pr = 0; pr < VR; ++pr) {
        if constexpr (F32) z[pr] = __uint_as_float(rv[pr]) * __uint_as_float(rw[pr]);
        else z[pr] = __uint_as_float(rv[pr] << 16) * __uint_as_float(rw[pr] << 16);
      }
      // The raw registers are free: start the next chunk's loads now.  This
      // chunk's loads (issued a chunk ago) are waited for explicitly first;
      // otherwise the in-order memory counter makes the first use of their
      // registers wait for the new loads as well.
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      if (c + 1 < nchunks) fetch(c + 1);
      if (o_pending) store4<BF16>(p.o, o_idx, o_val);
      o_pending = false;

      // fp32 cumulative log2-decay over the chunk: serial inside the thread,
      // then a scan of thread totals across the RG row groups
#pragma unroll
      for (int pr = 1; pr < RPT; ++pr)
#pragma unroll
        for (int i = 0; i < EPC; ++i) G[pr][i] += G[pr - 1][i];
      // Each 16-row block a is centred on its row c_a = 16a + 7, so that a
      // centred factor spans at most 8 tokens of decay; the thread's rows all
      // lie in block ab.  gcen[a][channel] = G at c_a lets phase P restore the
      // decay between two block centres in the off-diagonal tiles.
      const int ab = r0 / 16;
      float egm[EPC], egcm[EPC];
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        const float tot = G[RPT - 1][i];
        const float excl = seg_scan<RG>(tot) - tot;
#pragma unroll
        for (int pr = 0; pr < RPT; ++pr) G[pr][i] += excl;
        float gca[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) gca[a] = __shfl(G[7 % RPT][i], (16 * a + 7) / RPT, RG);
        const float gm = ab == 0 ? gca[0] : ab == 1 ? gca[1] : ab == 2 ? gca[2] : gca[3];
        const float gc = __shfl(G[RPT - 1][i], RG - 1, RG);
        egm[i] = exp2_fast(gm);
        egcm[i] = exp2_fast(gc - gm);
        if (rg == 0) {
          gC[EPC * cg + i] = exp2_fast(gc);
#pragma unroll
          for (int a = 0; a < 4; ++a) gcen[a * DK + EPC * cg + i] = gca[a];
        }
#pragma unroll
        for (int pr = 0; pr < RPT; ++pr) G[pr][i] -= gm;  // centred: G - G_(c_ab)
      }
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) {
        const int r = r0 + pr;
        float ep[EPC], kh[EPC], kl[EPC], qh[EPC], ql[EPC];
#pragma unroll
        for (int i = 0; i < EPC; ++i) {
          const float e1 = exp2_fast(G[pr][i]);
          const float e2 = exp2_fast(-G[pr][i]);
          const float bk = bv[pr][i] * kv[pr][i];
          ep[i] = e1 * bk;
          const float kbv = e2 * kv[pr][i];
          const float qp = e1 * qv[pr][i];
          if constexpr (F32) {
            kh[i] = kbv;
            qh[i] = qp;
          } else {
            kh[i] = bf16_round(kbv);
            kl[i] = kbv - kh[i];
            qh[i] = bf16_round(qp);
            ql[i] = qp - qh[i];
          }
          eh[pr][i] = cvt<ST>(ep[i] * egm[i]);
          qg[pr][i] = cvt<ST>(qp * egm[i]);
          kt[pr][i] = cvt<ST>(kbv * egcm[i]);
        }
        st4<KT>(Ep + r * LDK + EPC * cg, ep);
        st4<KT>(Kh + r * LDK + EPC * cg, kh);
        st4<KT>(Qh + r * LDK + EPC * cg, qh);
        if constexpr (BF16) {
          st4<KT>(Kl + r * LDK + EPC * cg, kl);
          st4<KT>(Ql + r * LDK + EPC * cg, ql);
        }
      }
      // Z^T: VR consecutive rows of the owned value channel
      stn<ST, VR>(ZT + vc * LDC + VR * vq, z);
    }
    __syncthreads();

    // ================= phase P: T^T and A_qk^T on MFMA ==========================
    // tile t goes to wave t (and tiles 8, 9 to waves 0, 2); one wave forms
    // both T and A_qk of its tile so the K' operand is read once per K step
    {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ti = k == 0 ? wv : (wv == 0 ? 8 : wv == 2 ? 9 : -1);
        if (ti < 0) break;
        int a, b;
        tri_tile(ti, a, b);
        f32x4 acc, acct;
        if (a == b) {
          acc = mma_lds<KT, DK>(zero4(), Kh + 16 * b * LDK, LDK, Qh + 16 * a * LDK, LDK);
          if constexpr (BF16) {
            acc = mma_lds<KT, DK>(acc, Kh + 16 * b * LDK, LDK, Ql + 16 * a * LDK, LDK);
            acc = mma_lds<KT, DK>(acc, Kl + 16 * b * LDK, LDK, Qh + 16 * a * LDK, LDK);
          }
          acct = mma_lds<KT, DK>(zero4(), Kh + 16 * b * LDK, LDK, Ep + 16 * a * LDK, LDK);
        } else {
          // K' of block b is centred on c_b and E', Q' of block a on c_a: scale
          // K' by 2^(G(c_a) - G(c_b)) <= 1 per channel before the products, as
          // an exponent shift (the scale alone may be below the fp32 range)
          acc = zero4();
          acct = zero4();
          const int ob = (16 * b + m) * LDK, oa = (16 * a + m) * LDK;
          const float* ga = gcen + a * DK;
          const float* gb = gcen + b * DK;
          if constexpr (F32) {
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 16) {
              const int c0 = k0 + 4 * g4;
              float4 kk = *reinterpret_cast<const float4*>(Kh + ob + c0);
              kk.x = mul_exp2(kk.x, ga[c0] - gb[c0]);
              kk.y = mul_exp2(kk.y, ga[c0 + 1] - gb[c0 + 1]);
              kk.z = mul_exp2(kk.z, ga[c0 + 2] - gb[c0 + 2]);
              kk.w = mul_exp2(kk.w, ga[c0 + 3] - gb[c0 + 3]);
              acc = mma16(kk, *reinterpret_cast<const float4*>(Qh + oa + c0), acc);
              acct = mma16(kk, *reinterpret_cast<const float4*>(Ep + oa + c0), acct);
            }
          } else {
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) {
              const int c0 = k0 + 8 * g4;
              bf16x8 kh = *reinterpret_cast<const bf16x8*>(Kh + ob + c0);
              bf16x8 kl = *reinterpret_cast<const bf16x8*>(Kl + ob + c0);
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float x = mul_exp2((float)kh[j] + (float)kl[j], ga[c0 + j] - gb[c0 + j]);
                const float hi = bf16_round(x);
                kh[j] = (__bf16)hi;
                kl[j] = (__bf16)(x - hi);
              }
              acc = mma32(kh, *reinterpret_cast<const bf16x8*>(Qh + oa + c0), acc);
              acc = mma32(kh, *reinterpret_cast<const bf16x8*>(Ql + oa + c0), acc);
              acc = mma32(kl, *reinterpret_cast<const bf16x8*>(Qh + oa + c0), acc);
              acct = mma32(kh, *reinterpret_cast<const bf16x8*>(Ep + oa + c0), acct);
            }
          }
        }
        // lanes hold A_qk[16a + m][16b + 4*g4 + q] and T[16a + m][16b + 4*g4 + q]
        if (a == b) {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = (4 * g4 + q <= m) ? acc[q] : 0.f;
          // diagonal blocks of T transposed, fp32: Tdt[a][s][r] = T[r][s], s < r
#pragma unroll
          for (int q = 0; q < 4; ++q) Tdt[(a * 16 + 4 * g4 + q) * 16 + m] = (4 * g4 + q < m) ? acct[q] : 0.f;
        } else {
          *reinterpret_cast<SV4*>(Tn + (16 * a + m) * LDC + 16 * b + 4 * g4) = neg_cvt4<SV4>(acct);
        }
        *reinterpret_cast<SV4*>(Aqk + (16 * a + m) * LDC + 16 * b + 4 * g4) = cvt4<SV4>(acc);
      }
    }
    __syncthreads();

    // ==== phase S(i): diagonal inverses; state-pass tiles into region X ===========
    {
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        float col[RPT], col2[RPT];
#pragma unroll
        for (int pr = 0; pr < RPT; ++pr) {
          col[pr] = (float)eh[pr][i];
          col2[pr] = (float)kt[pr][i];
        }
        stn<ST, RPT>(EhT + (EPC * cg + i) * LDC + r0, col);
        stn<ST, RPT>(KtT + (EPC * cg + i) * LDC + r0, col2);
      }
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) *reinterpret_cast<SV4*>(Qg + (r0 + pr) * LDK + EPC * cg) = qg[pr];
      if (wv < 4) {
        // wave a inverts I + T_aa: lane 4*cc + part holds rows 4*part .. 4*part+3
        // of column cc and runs a right-looking fp32 forward substitution over
        // the columns s of T_aa; row s of column cc is broadcast in its quad
        const int a = wv, cc = lane >> 2, part = lane & 3;
        const float4* Tc = reinterpret_cast<const float4*>(Tdt + a * 256);
        float xs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xs[j] = (4 * part + j == cc) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < 15; ++s) {
          const float4 col = Tc[s * 4 + part];
          const float xv = quad_bcast(xs[s & 3], s >> 2);
          // T[r][s] is zero for r <= s, so finished rows are left unchanged
          xs[0] = fmaf(-col.x, xv, xs[0]);
          xs[1] = fmaf(-col.y, xv, xs[1]);
          xs[2] = fmaf(-col.z, xv, xs[2]);
          xs[3] = fmaf(-col.w, xv, xs[3]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) Am[(16 * a + 4 * part + j) * LDC + 16 * a + cc] = cvt<ST>(xs[j]);
      }
    }
    __syncthreads();

    // ==== phase S(ii): off-diagonal blocks of A ===================================
    if (wv == 3) wy_column<0, ST, SV4, LDC>(Tn, Am);
    else if (wv == 2) wy_column<1, ST, SV4, LDC>(Tn, Am);
    else if (wv == 1) wy_column<2, ST, SV4, LDC>(Tn, Am);
    __syncthreads();

    // ==== phase Y: Y^T = E^T A^T (stored as -Y), U = A Z (kept) ===================
    const int ua = wv & 3, ujt = wv >> 2;  // this wave's (row block, value tile)
    f32x4 Ureg = zero4();
    {
      if (wv < DK / 16) {
        const int ib = wv;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          f32x4 acc;
          if (a < 2) acc = mma_lds<ST, 32>(zero4(), EhT + 16 * ib * LDC, LDC, Am + 16 * a * LDC, LDC);
          else acc = mma_lds<ST, 64>(zero4(), EhT + 16 * ib * LDC, LDC, Am + 16 * a * LDC, LDC);
          // lane holds Y[16a + m][16ib + 4*g4 + q]
          *reinterpret_cast<SV4*>(Yn + (16 * a + m) * LDK + 16 * ib + 4 * g4) = neg_cvt4<SV4>(acc);
        }
      }
      if (ujt < NJT) Ureg = mma_lds<ST, CH>(zero4(), Am + 16 * ua * LDC, LDC, ZT + 16 * ujt * LDC, LDC);
    }
    __syncthreads();

    // ================= phase R: R = U - Y S =======================================
    if (ujt < NJT) {
      const f32x4 acc = mma_lds<ST, DK>(Ureg, Yn + 16 * ua * LDK, LDK, Scur + 16 * ujt * LDK, LDK);
      // lane holds R[16ua + 4*g4 + q][16ujt + m]
      *reinterpret_cast<SV4*>(RT + (16 * ujt + m) * LDC + 16 * ua + 4 * g4) = cvt4<SV4>(acc);
    }
    __syncthreads();

    // ======= phase O: O^T = S^T Q_g^T + R^T A_qk^T ;  state update ==================
    if (ujt < NJT) {
      f32x4 acc = mma_lds<ST, DK>(zero4(), Scur + 16 * ujt * LDK, LDK, Qg + 16 * ua * LDK, LDK);
      acc = mma_lds<ST, CH>(acc, RT + 16 * ujt * LDC, LDC, Aqk + 16 * ua * LDC, LDC);
      // lane holds O[16ua + m][16ujt + 4*g4 + q]
      const int r = 16 * ua + m;
      if (r < clen) {
#pragma unroll
        for (int q = 0; q < 4; ++q) o_val[q] = acc[q];
        o_idx = ((size_t)(ctok + r) * H + h) * DV + jbase + 16 * ujt + 4 * g4;
        o_pending = true;
      }
    }
#pragma unroll
    for (int u = 0; u < Cfg::NSU; ++u) {
      const int t = wv + NW * u;
      if (t < Cfg::NSTILE) {
        const int ib = t % (DK / 16), jt = t / (DK / 16);
        f32x4 acc = Sacc[u];
        const float4 gc4 = *reinterpret_cast<const float4*>(gC + 16 * ib + 4 * g4);
        acc[0] *= gc4.x;
        acc[1] *= gc4.y;
        acc[2] *= gc4.z;
        acc[3] *= gc4.w;
        acc = mma_lds<ST, CH>(acc, KtT + 16 * ib * LDC, LDC, RT + 16 * jt * LDC, LDC);
        Sacc[u] = acc;
        *reinterpret_cast<SV4*>(Snext + (16 * jt + m) * LDK + 16 * ib + 4 * g4) = cvt4<SV4>(acc);
      }
    }
    __syncthreads();
    ST* tmp = Scur;
    Scur = Snext;
    Snext = tmp;
  }

  if (o_pending) store4<BF16>(p.o, o_idx, o_val);
  if (p.ST) {
#pragma unroll
    for (int u = 0; u < Cfg::NSU; ++u) {
      const int t = wv + NW * u;
      if (t < Cfg::NSTILE) {
        const int ib = t % (DK / 16), jt = t / (DK / 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          p.ST[(nh * DK + 16 * ib + 4 * g4 + q) * DV + jbase + 16 * jt + m] = Sacc[u][q];
      }
    }
  }
}

// ---- host-side dispatch -------------------------------------------------------------

template <int DK, int DVB, bool F32, bool LA16>
static hipError_t launch_variant1(const ChunkArgs& a, hipStream_t stream) {
  typedef ChunkCfg<DK, DVB, F32> Cfg;
  const int NB = a.DV / DVB;
  const long long pairs = (long long)a.N * a.H;
  const long long grid = (pairs + 7) / 8 * 8 * NB;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // The LDS opt-in is per device; setting it again is idempotent, so racing
  // first calls from several threads are harmless.
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !attr_set[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_fwd_kernel<DK, DVB, F32, LA16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::BYTES);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev] = true;
  }
  hipLaunchKernelGGL((chunk_fwd_kernel<DK, DVB, F32, LA16>), dim3((unsigned)grid), dim3(NT), Cfg::BYTES,
                     stream, a);
  return hipGetLastError();
}

template <int DK, int DVB, bool F32>
static hipError_t launch_variant(const ChunkArgs& a, hipStream_t stream) {
  return a.la_bf16 ? launch_variant1<DK, DVB, F32, true>(a, stream)
                   : launch_variant1<DK, DVB, F32, false>(a, stream);
}

bool chunk_supported(int dk, int dv, bool bf16) {
  if (dv != 32 && dv != 64 && dv != 128) return false;
  if (bf16) return dk == 32 || dk == 64 || dk == 128;
  return dk == 32 || dk == 64;
}

hipError_t launch_chunk(const ChunkArgs& a, int dk, int dv, bool bf16, hipStream_t stream) {
  // 16-bit inputs take the two-pass forward (gdr2_intra.hip, gdr2_state.hip)
  if (!chunk_supported(dk, dv, bf16) || bf16) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return launch_variant<32, 16, true>(a, stream);
    default: return launch_variant<64, 16, true>(a, stream);
  }
}

}  // namespace gdr2
