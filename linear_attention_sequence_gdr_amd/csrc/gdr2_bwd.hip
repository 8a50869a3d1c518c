// gdr2_bwd.hip -- backward pass of the chunkwise Gated Delta Rule-2 operator
// (Gated DeltaNet-2 pages, "Gate-Aware Backward Pass", Appendix B, with the
// forward of "Chunkwise Parallel Training via WY Representation", Steps 1-3).
//
// Per 64-token chunk and head (an item), with S the state entering the chunk
// and dS' = dL/d(state leaving it):
//   forward recompute  G (fp32 cumulative log-decay), gamma = exp(G),
//                      Q_g = gamma q, K_tail = (gamma_C / gamma) k,
//                      E = gamma b k, Z = w v, T = tril(E K_bar^T, -1),
//                      A = (I + T)^-1, A_qk = tril(Q_g K_bar^T), Y = A E, U = A Z
//   state paths        R = U - Y S, dR = A_qk^T dO + K_tail dS',
//                      dS = Q_g^T dO + Diag(gamma_C) dS' - Y^T dR (chunks in reverse)
//   output paths       dQ_g = dO S^T, dY = -dR S^T, dK_tail = R dS'^T,
//                      dA_qk = tril(dO R^T)
//   gate-aware WY      dA = dR Z^T + dY E^T (Eqs. 64-65), dZ = A^T dR,
//                      dE = A^T dY + dT K_bar, dT = -tril(A^T dA A^T, -1),
//                      dK_bar = dT^T E + dA_qk^T Q_g, dQ_g += dA_qk K_bar
//   gates and decay    dq, dk, db = dE gamma k, dv = dZ w, dw = dZ v, and
//                      dg = reverse cumulative sum of dG over the chunk.
// Products whose factors carry gamma_r / gamma_s use factors centred on the
// chunk's row 31 (e1 = exp(G - G_31), e2 = exp(G_31 - G)) with the scale put
// back per row afterwards, so no 1/gamma is formed.
//
// Layout: what one kernel hands to the next is an fp32 row-major block per
// item inside the workspace (BwdLayout: G, Q_g, K_tail, Y, U, R, dR, A, A_qk,
// the entering state S, dS' and gamma_C).  Four kernels run:
//   bwd_front_kernel      per item: G, the scaled rows, T and A_qk, A, Y, U;
//   bwd_state_fwd3_kernel per chain, chunks in order: S entering each chunk
//                         and R = U - Y S;
//   bwd_state_bwd3_kernel per chain, chunks in reverse: dS' and dR, and dS0;
//   bwd_out_kernel        per item: every output-path and WY-gradient product
//                         and the gradients themselves (E, E', K', Q' are
//                         formed again from G, q, k, b rather than stored).
// The products run from LDS-staged operands with fp32 accumulation.  In the
// main launches of the backward they run as three bf16 MFMAs over hi/lo
// operand halves (mma3x, about 2^-16 of each term), except the front pass's
// WY inverse, which stays on fp32 (forward substitution and fp32 MFMA).  The
// launches that form strongly decaying chunks, and the fp32 forward (the
// front pass, then fwd32_state_kernel), keep fp32 products throughout.
#include <hip/hip_runtime.h>

#include "gdr2_device.h"
#include "gdr2_internal.h"

namespace gdr2 {

namespace {

constexpr int BC = 64;    // chunk
constexpr int DVB = 32;   // value channels per workgroup of the sequential passes
constexpr int SNT = 512;  // threads per workgroup of the sequential passes

template <int DK, int DV>
struct BwdLayout {
  static constexpr size_t CK = (size_t)BC * DK, CV = (size_t)BC * DV, CC = (size_t)BC * BC,
                          KV = (size_t)DK * DV;
  // offsets in floats inside one item's block
  static constexpr size_t G = 0, QG = G + CK, KT = QG + CK, Y_ = KT + CK;
  static constexpr size_t U = Y_ + CK, R = U + CV, DR = R + CV;
  static constexpr size_t A = DR + CV, AQK = A + CC;
  static constexpr size_t S = AQK + CC, DSP = S + KV;
  static constexpr size_t GC = DSP + KV;
  static constexpr size_t FLOATS = (GC + DK + 63) / 64 * 64;
};

// item -> first token row and valid rows; false for an item past the packed
// chunks
__device__ __forceinline__ bool bwd_locate(const BwdArgs& a, int ci, long long& row0, int& clen) {
  if (a.tab) {
    if (ci >= *a.total) return false;
    row0 = a.tab[2 * ci];
    clen = a.tab[2 * ci + 1];
  } else {
    const int n = ci / a.nc, c = ci - n * a.nc;
    row0 = (long long)n * a.T + (long long)c * BC;
    clen = min(BC, a.T - c * BC);
  }
  return true;
}

// Two independent fp32 MFMA accumulator chains advanced by one K = 4 step
// each, in one place so that their issue interleaves.
__device__ __forceinline__ void mfma2(f32x4& c0, float a0, float b0, f32x4& c1, float a1, float b1) {
  c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, c0, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, c1, 0, 0, 0);
}

// Factors centred on one row stay inside [e^-SLIM, e^SLIM] (nats); a chunk
// that needs more takes the exact path.
constexpr float BWD_SLIM = 80.f;

// e^x for the decay factors, as 2^(x log2 e) on the hardware exp2.  The
// product x log2 e is carried as its rounded value h plus a residual l: one
// FMA gives the rounding error of x * L2E exactly, a second adds x times the
// part of log2 e below fp32 (L2E_LO).  Then 2^(h + l) = 2^h (1 + l ln 2) up to
// terms in l^2, with |l| <= 2^-24 |h|.  The result is within about two ulp
// of e^x for |x| < 88 (six instructions against fourteen for expf); results
// below 2^-126 may flush to zero, and an overflowing 2^h stays +inf.
__device__ __forceinline__ float exp_dec(float x) {
  constexpr float L2E = 1.44269502162933349609375f;  // log2(e) rounded to fp32
  constexpr float L2E_LO = 1.925963033500011e-08f;    // log2(e) - L2E
  constexpr float LN2 = 0.693147180559945309f;
  const float h = x * L2E;
  const float l = fmaf(x, L2E_LO, fmaf(x, L2E, -h));
  return __builtin_amdgcn_exp2f(h) * fmaf(l, LN2, 1.f);
}

// Exact decay-weighted chunk products for one 16x16 tile in C layout: lane
// (m, g) gets, for q < 4, the sum over channels i of
//     X[r + q][i] * K[c][i] * exp(G[r + q][i] - G[c][i])
// with r = r0 (= 16 tm + 4 g), c = c0 (= 16 tn + m), from row-major [64][LD]
// LDS blocks.  Entries with c > r + q are formed too (and masked by the
// caller), so the exponent is not clamped.
template <int DK, int LD>
__device__ __forceinline__ f32x4 decay_product(const float* X, const float* K, const float* G, int r0,
                                               int c0) {
  f32x4 acc = zero4();
  const float* gc = G + c0 * LD;
  const float* kc = K + c0 * LD;
#pragma unroll 2
  for (int i = 0; i < DK; i += 4) {
    const float4 g4 = *reinterpret_cast<const float4*>(gc + i);
    const float4 k4 = *reinterpret_cast<const float4*>(kc + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 gr = *reinterpret_cast<const float4*>(G + (r0 + q) * LD + i);
      const float4 xr = *reinterpret_cast<const float4*>(X + (r0 + q) * LD + i);
      acc[q] = fmaf(xr.x * k4.x, exp_dec(gr.x - g4.x), acc[q]);
      acc[q] = fmaf(xr.y * k4.y, exp_dec(gr.y - g4.y), acc[q]);
      acc[q] = fmaf(xr.z * k4.z, exp_dec(gr.z - g4.z), acc[q]);
      acc[q] = fmaf(xr.w * k4.w, exp_dec(gr.w - g4.w), acc[q]);
    }
  }
  return acc;
}

// Exact decay-weighted products of the backward's strong chunks, for one
// 16x16 tile in C layout: lane (m, g) gets, for q < 4 and x = x0 + q
// (x0 = 16 tm + 4 g) and channel c,
//   ROW:  sum over t <= x of M[x][t] * X[t][c] * exp(G[x][c] - G[t][c])
//   !ROW: sum over t >= x of M[x][t] * X[t][c] * exp(G[t][c] - G[x][c])
// over t in [t0, t1), M row-major with stride LDM, X and G row-major with
// stride LDX.  Terms outside the triangle are discarded by a select, so an
// overflowing exponent there never reaches the sum.
template <int LDM, int LDX, bool ROW>
__device__ __forceinline__ f32x4 decay_tri(const float* M, const float* X, const float* G, int x0, int c,
                                           int t0, int t1) {
  f32x4 acc = zero4();
  float gx[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) gx[q] = G[(x0 + q) * LDX + c];
  for (int t = t0; t < t1; ++t) {
    const float xt = X[t * LDX + c], gt = G[t * LDX + c];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float term = M[(x0 + q) * LDM + t] * xt * exp_dec(ROW ? gx[q] - gt : gt - gx[q]);
      const bool in = ROW ? t <= x0 + q : t >= x0 + q;
      acc[q] = in ? acc[q] + term : acc[q];
    }
  }
  return acc;
}

// ---- front: decay, the scaled rows, T, A_qk, A = (I + T)^-1, Y and U per item ----------
// One workgroup per item:
//   phase 1  log-decay rows into LDS, q, k, b into registers; G by a column
//            scan (row blocks scanned in parallel, then offset by the totals
//            of the blocks above);
//   phase 2  Q_g and K_tail to the workspace, E', K', Q' to LDS (E and the
//            centred rows are not stored: the output pass forms them again);
//   phase 3  T = tril(E' K'^T, -1) and A_qk = tril(Q' K'^T) on MFMA (inside
//            a product the centred factors cancel);
//   phase 4  A = (I + T)^-1: forward substitution on the four diagonal 16x16
//            blocks, then the off-diagonal blocks one block row at a time,
//            A_ij = -A_ii sum_{k=j}^{i-1} T_ik A_kj;
//   phase 5  Y = A E and U = A Z (Z = w * v) on MFMA, A to the workspace.
// Rows past the end of a sequence read a clamped (valid) row and are zeroed.
// X = A B over the 64 rows of a chunk: A lower triangular [64][64] and B
// [64][16 TN], both row-major in LDS (strides LA, LB), B read K-major.  The
// NU tiles of one wavefront (t = wv + 8u: row tile t / TN, column tile
// t % TN, the same for every u since TN divides 8) run together: at each K
// step one B fragment serves every tile whose range still runs (row tile tm
// needs K < 16 (tm + 1)), and each tile accumulates in ascending K.  X goes
// to global memory with row stride ldx.
template <int NU, int TN, int LA, int LB>
__device__ __forceinline__ void tri_rows(const float* sA, const float* sB, int wv, int m, int g, float* X,
                                         int ldx) {
  static_assert(8 % TN == 0, "the column tile is the same for every u");
  const int tn = wv % TN;
  f32x4 acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = zero4();
#pragma unroll
  for (int k0 = 0; k0 < BC; k0 += 16) {
    const float* bp = sB + (k0 + 4 * g) * LB + 16 * tn + m;  // B read K-major
    const float b0 = bp[0], b1 = bp[LB], b2 = bp[2 * LB], b3 = bp[3 * LB];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int tm = (wv + 8 * u) / TN;
      if (k0 < 16 * (tm + 1)) {  // uniform
        const float4 x = *reinterpret_cast<const float4*>(sA + (16 * tm + m) * LA + k0 + 4 * g);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, b0, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, b1, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, b2, acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, b3, acc[u], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int tm = (wv + 8 * u) / TN;
#pragma unroll
    for (int q = 0; q < 4; ++q) X[(size_t)(16 * tm + 4 * g + q) * ldx + 16 * tn + m] = acc[u][q];
  }
}

// tri_rows from bf16 hi/lo halves (mma3x): A with a row's 64 hi then 64 lo
// halves (pitch LHA), B with a row's NB hi then NB lo halves (pitch LHB),
// read down its columns; K = 32 blocks past A's triangle are skipped.
template <int NU, int TN, int LHA, int LHB, int NB>
__device__ __forceinline__ void tri_rows3(const __bf16* bA, const __bf16* bB, int wv, float* X, int ldx) {
  static_assert(8 % TN == 0, "the column tile is the same for every u");
  const int tn = wv % TN, m = lane_id() & 15, g = lane_id() >> 4;
  f32x4 acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = zero4();
#pragma unroll
  for (int k0 = 0; k0 < BC; k0 += 32) {
    const bf16x8 bh = frag_kmajor(bB, LHB, k0, 16 * tn), bl = frag_kmajor(bB, LHB, k0, NB + 16 * tn);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int tm = (wv + 8 * u) / TN;
      if (k0 < 16 * (tm + 1))  // uniform
        acc[u] = mma3x(frag_krow(bA, LHA, k0, 16 * tm), frag_krow(bA, LHA, BC + k0, 16 * tm), bh, bl, acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int tm = (wv + 8 * u) / TN;
#pragma unroll
    for (int q = 0; q < 4; ++q) X[(size_t)(16 * tm + 4 * g + q) * ldx + 16 * tn + m] = acc[u][q];
  }
}

template <int DK, int DV>
struct FrontCfg {
  static constexpr int NT = 512, LA = BC + 4, LKP = DK + 4, LM = 20;
  // phases 1-2: G, E', K', Q' [64][DK]
  static constexpr int O_G = 0, O_EP = O_G + BC * LKP, O_KP = O_EP + BC * LKP,
                       O_QP = O_KP + BC * LKP, E1 = O_QP + BC * LKP;
  // phases 3-5: T, A, A^T [64][64], M^T [16][LM] for three wavefronts
  static constexpr int O_T = 0, O_A = O_T + BC * LA, O_AT = O_A + BC * LA, O_M = O_AT + BC * LA,
                       E2 = O_M + 3 * 16 * LM;
  // phase 5: E [64][DK], Z [64][DV] (row-major, read K-major)
  static constexpr int LZ = DV + 4;
  static constexpr int O_EB = E2, O_Z = O_EB + BC * LKP, O_AS = O_Z + BC * LZ;
  // the backward's main launch: A as bf16 hi/lo halves, 64 hi then 64 lo per row
  static constexpr int E3 = O_AS + BC * LA;
  static constexpr int O_PS = E1 > E3 ? E1 : E3, FLOATS = O_PS + NT;
  static constexpr size_t BYTES = (size_t)FLOATS * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(DK % 32 == 0 && DV % 32 == 0 && NT % DK == 0, "front pass tiling");
};

// One item of the front pass.  FWD: the front pass of the fp32 forward, which
// needs neither G nor A later.  SM = 0: the main launch, whose code has no
// exact-decay path: a strong chunk (see BWD_SLIM) is only flagged in
// a.sflag and left for SM = 1, the launch that forms the flagged chunks with
// the exact decay.  Keeping the exact path out of the main launch keeps its
// registers out of the common case.
template <int DK, int DV, bool BF16, bool LA16, bool FWD, int SM>
__device__ __forceinline__ void front_item(const BwdArgs& a, const int item) {
  typedef BwdLayout<DK, DV> L;
  typedef FrontCfg<DK, DV> C;
  constexpr int NT = C::NT, NWV = 8, LA = C::LA, LKP = C::LKP, LM = C::LM;
  constexpr int NEK = BC * DK / 4 / NT;  // float4 of a [64][DK] block per thread
  constexpr int NEV = BC * DV / 4 / NT;  // float4 of a [64][DV] block per thread
  constexpr int NAA = BC * BC / 4 / NT;  // float4 of a [64][64] block per thread
  constexpr int TNK = DK / 16, NKT = DK / 32, TNV = DV / 16, NVT = DV / 32;
  constexpr int NRB = NT / DK, RPB = BC / NRB;
  const int ci = item / a.H, h = item - ci * a.H;
  long long row0;
  int clen;
  if (!bwd_locate(a, ci, row0, clen) || clen <= 0) return;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* sm = reinterpret_cast<float*>(smem_raw);
  float* W = a.ws + (size_t)item * L::FLOATS;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  const size_t kr = (size_t)a.H * DK, vr = (size_t)a.H * DV;

  // ---- phase 1 ----
  float* sG = sm + C::O_G;
  f32x4 pq[NEK], pk[NEK], pb[NEK];
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, r = e / (DK / 4), i4 = e - r * (DK / 4);
    const int rr = r < clen ? r : clen - 1;
    const size_t x = (size_t)(row0 + rr) * kr + (size_t)h * DK + 4 * i4;
    const float z = r < clen ? 1.f : 0.f;
    float t[4];
    load4<LA16>(a.la, x, t);
    *reinterpret_cast<f32x4*>(sG + r * LKP + 4 * i4) = f32x4{t[0], t[1], t[2], t[3]} * z;
    load4<BF16>(a.q, x, t);
    pq[u] = f32x4{t[0], t[1], t[2], t[3]} * z;
    load4<BF16>(a.k, x, t);
    pk[u] = f32x4{t[0], t[1], t[2], t[3]} * z;
    load4<BF16>(a.b, x, t);
    pb[u] = f32x4{t[0], t[1], t[2], t[3]} * z;
  }
  __syncthreads();
  // cumulative log-decay from the chunk start, fp32 (rows past the end add 0)
  const int si = tid % DK, rb = tid / DK;
  float* sPS = sm + C::O_PS;
  float run[RPB];
  {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < RPB; ++k) {
      acc += sG[(rb * RPB + k) * LKP + si];
      run[k] = acc;
    }
    sPS[rb * DK + si] = acc;
  }
  __syncthreads();
  {
    float off = 0.f;
#pragma unroll
    for (int b = 0; b < NRB - 1; ++b)
      if (b < rb) off += sPS[b * DK + si];
#pragma unroll
    for (int k = 0; k < RPB; ++k) {
      const int r = rb * RPB + k;
      const float G = off + run[k];
      sG[r * LKP + si] = G;
      if constexpr (!FWD) W[L::G + r * DK + si] = G;
      if (r == BC - 1) W[L::GC + si] = exp_dec(G);
    }
  }
  __syncthreads();

  // ---- phase 2 ----
  // A chunk whose decay moves some channel more than SLIM nats away from row
  // 31 would take centred factors outside the fp32 range: it is "strong", and
  // its T and A_qk are formed entry by entry with the exact decay instead
  // (phase 3), from the raw rows b k, k and q.
  bool strong_t = false;
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, r = e / (DK / 4), i4 = e - r * (DK / 4);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      strong_t = strong_t || fabsf(sG[r * LKP + 4 * i4 + c] - sG[31 * LKP + 4 * i4 + c]) > BWD_SLIM;
  }
  const bool flagged = __syncthreads_or(strong_t) != 0;
  if constexpr (SM == 0) {
    if (tid == 0) a.sflag[item] = flagged ? 1 : 0;  // every item of the main launch writes its flag
    if (flagged) return;                            // uniform: the strong launch forms this chunk
  }
  constexpr bool strong = SM == 1;
  float *sEP = sm + C::O_EP, *sKP = sm + C::O_KP, *sQP = sm + C::O_QP;
  // The backward's main launch multiplies E', K' and Q' (phase 3 only) as
  // bf16 hi/lo halves (mma3x); the fp32 forward and the strong launch keep
  // fp32 operands.
  constexpr bool SPLIT = !FWD && SM == 0;
  __bf16 *bEP = reinterpret_cast<__bf16*>(sEP), *bKP = reinterpret_cast<__bf16*>(sKP),
         *bQP = reinterpret_cast<__bf16*>(sQP);
  f32x4 pg[NEK];  // G of this thread's units, for E in phase 5
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, r = e / (DK / 4), i4 = e - r * (DK / 4), o = r * LKP + 4 * i4;
    f32x4 QG, KT, EP, KP, QP;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = 4 * i4 + c;
      const float G = sG[o + c], G31 = sG[31 * LKP + i], GCl = sG[(BC - 1) * LKP + i];
      const float gam = exp_dec(G);
      const float e1 = strong ? 1.f : exp_dec(G - G31), e2 = strong ? 1.f : exp_dec(G31 - G);
      const float qv = pq[u][c], kv = pk[u][c], bv = pb[u][c];
      pg[u][c] = G;
      QG[c] = gam * qv;
      KT[c] = exp_dec(GCl - G) * kv;
      EP[c] = e1 * bv * kv;
      KP[c] = e2 * kv;
      QP[c] = e1 * qv;
    }
    const int wo = r * DK + 4 * i4;
    *reinterpret_cast<f32x4*>(W + L::QG + wo) = QG;
    *reinterpret_cast<f32x4*>(W + L::KT + wo) = KT;
    if constexpr (SPLIT) {
      // hi halves of row r at [0, DK), lo halves at [DK, 2 DK): the bytes of the fp32 row
      const int ob = r * (2 * LKP) + 4 * i4;
      bf16x4 hi, lo;
      split_bf16(EP, hi, lo);
      *reinterpret_cast<bf16x4*>(bEP + ob) = hi;
      *reinterpret_cast<bf16x4*>(bEP + ob + DK) = lo;
      split_bf16(KP, hi, lo);
      *reinterpret_cast<bf16x4*>(bKP + ob) = hi;
      *reinterpret_cast<bf16x4*>(bKP + ob + DK) = lo;
      split_bf16(QP, hi, lo);
      *reinterpret_cast<bf16x4*>(bQP + ob) = hi;
      *reinterpret_cast<bf16x4*>(bQP + ob + DK) = lo;
    } else {
      *reinterpret_cast<f32x4*>(sEP + o) = EP;
      *reinterpret_cast<f32x4*>(sKP + o) = KP;
      *reinterpret_cast<f32x4*>(sQP + o) = QP;
    }
  }
  // v and w for Z, loaded while the products run
  f32x4 pv[NEV], pw[NEV];
#pragma unroll
  for (int u = 0; u < NEV; ++u) {
    const int e = tid + NT * u, s = e / (DV / 4), j4 = e - s * (DV / 4);
    const int rr = s < clen ? s : clen - 1;
    const size_t x = (size_t)(row0 + rr) * vr + (size_t)h * DV + 4 * j4;
    const float z = s < clen ? 1.f : 0.f;
    float t[4];
    load4<BF16>(a.v, x, t);
    pv[u] = f32x4{t[0], t[1], t[2], t[3]} * z;
    load4<BF16>(a.w, x, t);
    pw[u] = f32x4{t[0], t[1], t[2], t[3]} * z;
  }
  __syncthreads();

  // ---- phase 3 ----
  // T and A_qk are lower triangular: only the ten 16x16 tiles on and below
  // the diagonal are formed.  Tile p (row-wise, p < 10) goes to wavefront
  // p % 8, so that the two wavefronts of each SIMD (w and w + 4) share at
  // most three of them; the six tiles above the diagonal are zero.
  const auto low_tile = [](int p, int& tm, int& tn) {
    tm = (p >= 1) + (p >= 3) + (p >= 6);
    tn = p - tm * (tm + 1) / 2;
  };
  f32x4 aT[2], aQ[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = wv + NWV * u;
    aT[u] = aQ[u] = zero4();
    if (p < 10) {  // uniform
      int tm, tn;
      low_tile(p, tm, tn);
      if constexpr (SPLIT) {
        // the two products share K''s fragments: two chains, interleaved
        constexpr int LH = 2 * LKP;
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
          const bf16x8 kh = frag_krow(bKP, LH, k0, 16 * tn), kl = frag_krow(bKP, LH, DK + k0, 16 * tn);
          const bf16x8 eh = frag_krow(bEP, LH, k0, 16 * tm), el = frag_krow(bEP, LH, DK + k0, 16 * tm);
          const bf16x8 qh = frag_krow(bQP, LH, k0, 16 * tm), ql = frag_krow(bQP, LH, DK + k0, 16 * tm);
          aT[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(el, kh, aT[u], 0, 0, 0);
          aQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, kh, aQ[u], 0, 0, 0);
          aT[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(eh, kl, aT[u], 0, 0, 0);
          aQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kl, aQ[u], 0, 0, 0);
          aT[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(eh, kh, aT[u], 0, 0, 0);
          aQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kh, aQ[u], 0, 0, 0);
        }
      } else if (strong) {
        aT[u] = decay_product<DK, LKP>(sEP, sKP, sG, 16 * tm + 4 * g, 16 * tn + m);
        aQ[u] = decay_product<DK, LKP>(sQP, sKP, sG, 16 * tm + 4 * g, 16 * tn + m);
      } else {
        // the two products share K''s fragments: two chains, interleaved
        const float* e = sEP + (16 * tm + m) * LKP + 4 * g;
        const float* qp = sQP + (16 * tm + m) * LKP + 4 * g;
        const float* kp = sKP + (16 * tn + m) * LKP + 4 * g;
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 16) {
          const float4 x = *reinterpret_cast<const float4*>(e + k0);
          const float4 y = *reinterpret_cast<const float4*>(qp + k0);
          const float4 z = *reinterpret_cast<const float4*>(kp + k0);
          mfma2(aT[u], x.x, z.x, aQ[u], y.x, z.x);
          mfma2(aT[u], x.y, z.y, aQ[u], y.y, z.y);
          mfma2(aT[u], x.z, z.z, aQ[u], y.z, z.z);
          mfma2(aT[u], x.w, z.w, aQ[u], y.w, z.w);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, c = 16 * tn + m;
        W[L::AQK + r * BC + c] = c <= r ? aQ[u][q] : 0.f;
      }
    }
  }
  const auto up_tile = [](int p, int& tm, int& tn) {  // p < 6, row-wise above the diagonal
    tm = (p >= 3) + (p >= 5);
    tn = p - (tm == 0 ? 0 : (tm == 1 ? 3 : 5)) + tm + 1;
  };
  if (wv >= 2) {  // the upper tiles of A_qk, one per wavefront 2-7
    int tm, tn;
    up_tile(wv - 2, tm, tn);
#pragma unroll
    for (int q = 0; q < 4; ++q) W[L::AQK + (16 * tm + 4 * g + q) * BC + 16 * tn + m] = 0.f;
  }
  __syncthreads();
  float *sT = sm + C::O_T, *sA = sm + C::O_A, *sAT = sm + C::O_AT;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = wv + NWV * u;
    if (p < 10) {
      int tm, tn;
      low_tile(p, tm, tn);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, c = 16 * tn + m;
        sT[r * LA + c] = c < r ? aT[u][q] : 0.f;
      }
    }
  }
  if (wv >= 2) {
    int tm, tn;
    up_tile(wv - 2, tm, tn);
#pragma unroll
    for (int q = 0; q < 4; ++q) sT[(16 * tm + 4 * g + q) * LA + 16 * tn + m] = 0.f;
  }
  // A is lower triangular: zero its six blocks above the diagonal (and those of A^T)
  for (int e = tid; e < 6 * 256; e += NT) {
    const int blk = e >> 8, w = e & 255, rr = w >> 4, cc = w & 15;
    const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
    const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
    sA[(16 * bi + rr) * LA + 16 * bj + cc] = 0.f;
    sAT[(16 * bj + cc) * LA + 16 * bi + rr] = 0.f;
  }
  __syncthreads();

  // ---- phase 4 ----
  if (wv == 0) {  // lane = (diagonal block b, column j)
    const int b = lane >> 4, j = lane & 15;
    const float* Tb = sT + 16 * b * LA + 16 * b;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == j ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) acc = fmaf(-Tb[r * LA + s], x[s], acc);
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sA[(16 * b + r) * LA + 16 * b + j] = x[r];
      sAT[(16 * b + j) * LA + 16 * b + r] = x[r];
    }
  }
  __syncthreads();
  float* sM = sm + C::O_M;
  for (int i = 1; i < 4; ++i) {
    if (wv < i) {  // wavefront j = wv: M = sum_{k=j}^{i-1} T_ik A_kj, kept as M^T
      f32x4 mm = zero4();
      for (int k = wv; k < i; ++k)
        mm = mma_lds<float, 16>(mm, sT + 16 * i * LA + 16 * k, LA, sAT + 16 * wv * LA + 16 * k, LA);
#pragma unroll
      for (int q = 0; q < 4; ++q) sM[wv * 16 * LM + m * LM + 4 * g + q] = mm[q];
    }
    __syncthreads();
    if (wv < i) {  // A_ij = -A_ii M
      const f32x4 x = mma_lds<float, 16>(zero4(), sA + 16 * i * LA + 16 * i, LA, sM + wv * 16 * LM, LM);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * g + q;
        sA[(16 * i + r) * LA + 16 * wv + m] = -x[q];
        sAT[(16 * wv + m) * LA + 16 * i + r] = -x[q];
      }
    }
    __syncthreads();
  }

  // ---- phase 5 ----
  float *sEB = sm + C::O_EB, *sZ = sm + C::O_Z;
  // The backward's main launch runs Y and U on hi/lo halves too: A's into a
  // region of their own (A itself stays fp32 for the workspace), E's and Z's
  // in the bytes of their fp32 rows (hi halves first, pitch twice the fp32
  // one).
  __bf16 *bAS = reinterpret_cast<__bf16*>(sm + C::O_AS), *bEB = reinterpret_cast<__bf16*>(sEB),
         *bZ = reinterpret_cast<__bf16*>(sZ);
#pragma unroll
  for (int u = 0; u < NAA; ++u) {
    const int e = tid + NT * u, s = e / (BC / 4), c4 = e - s * (BC / 4);
    const f32x4 x = *reinterpret_cast<const f32x4*>(sA + s * LA + 4 * c4);
    if constexpr (!FWD) *reinterpret_cast<f32x4*>(W + L::A + s * BC + 4 * c4) = x;
    if constexpr (SPLIT) {
      bf16x4 hi, lo;
      split_bf16(x, hi, lo);
      *reinterpret_cast<bf16x4*>(bAS + s * (2 * LA) + 4 * c4) = hi;
      *reinterpret_cast<bf16x4*>(bAS + s * (2 * LA) + BC + 4 * c4) = lo;
    }
  }
  // E = gamma * b * k from the registers of phase 1-2, and Z = w * v
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e / (DK / 4), i4 = e - s * (DK / 4);
    f32x4 eb;
#pragma unroll
    for (int c = 0; c < 4; ++c) eb[c] = exp_dec(pg[u][c]) * pb[u][c] * pk[u][c];
    if constexpr (SPLIT) {
      bf16x4 hi, lo;
      split_bf16(eb, hi, lo);
      *reinterpret_cast<bf16x4*>(bEB + s * (2 * LKP) + 4 * i4) = hi;
      *reinterpret_cast<bf16x4*>(bEB + s * (2 * LKP) + DK + 4 * i4) = lo;
    } else {
      *reinterpret_cast<f32x4*>(sEB + s * LKP + 4 * i4) = eb;
    }
  }
#pragma unroll
  for (int u = 0; u < NEV; ++u) {
    const int e = tid + NT * u, s = e / (DV / 4), j4 = e - s * (DV / 4);
    if constexpr (SPLIT) {
      bf16x4 hi, lo;
      split_bf16(pw[u] * pv[u], hi, lo);
      *reinterpret_cast<bf16x4*>(bZ + s * (2 * C::LZ) + 4 * j4) = hi;
      *reinterpret_cast<bf16x4*>(bZ + s * (2 * C::LZ) + DV + 4 * j4) = lo;
    } else {
      *reinterpret_cast<f32x4*>(sZ + s * C::LZ + 4 * j4) = pw[u] * pv[u];
    }
  }
  __syncthreads();
  // A is lower triangular: row block tm needs the first 16 (tm + 1) columns only
  // Y = A E and U = A Z: a wavefront's tiles (t = wv + 8u) share the column
  // block of E (of Z), so at each K step one fragment of it serves every
  // tile whose range (A is lower triangular: K < 16 (tm + 1)) still runs;
  // each tile accumulates in ascending K
  if constexpr (SPLIT) {
    tri_rows3<NKT, TNK, 2 * LA, 2 * LKP, DK>(bAS, bEB, wv, W + L::Y_, DK);
    tri_rows3<NVT, TNV, 2 * LA, 2 * C::LZ, DV>(bAS, bZ, wv, W + L::U, DV);
  } else {
    tri_rows<NKT, TNK, LA, LKP>(sA, sEB, wv, m, g, W + L::Y_, DK);
    tri_rows<NVT, TNV, LA, C::LZ>(sA, sZ, wv, m, g, W + L::U, DV);
  }
}

// The front pass: one workgroup per item; strong chunks are flagged only.
template <int DK, int DV, bool BF16, bool LA16, bool FWD>
__global__ __launch_bounds__(512) void bwd_front_kernel(BwdArgs a) {
  front_item<DK, DV, BF16, LA16, FWD, 0>(a, blockIdx.x);
}

// The strong chunks the main launch flagged, with the exact decay: one
// workgroup per item, which leaves at once unless its item is flagged.  The
// main launch sets the flag of every item inside the sequences; a stale flag
// of an item outside them (a packed call's spare chunks) sends its workgroup
// into front_item, which leaves at once too.  (A grid-stride loop here would
// keep values live across items and spill.)
template <int DK, int DV, bool BF16, bool LA16, bool FWD>
__global__ __launch_bounds__(512) void bwd_front_strong_kernel(BwdArgs a) {
  if (a.sflag[blockIdx.x] == 0) return;  // uniform
  front_item<DK, DV, BF16, LA16, FWD, 1>(a, blockIdx.x);
}

// Register prefetch of one chunk's operands for the sequential passes
// (16-byte loads in address order, into row-major LDS blocks).
// With FWD (the fp32 forward) Q_g and A_qk come too, for the output.
template <int DK, int DV, int NK4, int NV4, int NC4, bool FWD>
__device__ __forceinline__ void sf_load(const BwdArgs& a, int ci, int h, int jb, int tid,
                                        f32x4 (&ry)[NK4], f32x4 (&rk)[NK4], f32x4 (&ru)[NV4],
                                        f32x4& rg, f32x4 (&rq)[NK4], f32x4 (&ra)[NC4]) {
  typedef BwdLayout<DK, DV> L;
  const float* Wn = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
#pragma unroll
  for (int u = 0; u < NK4; ++u) {
    const int e4 = tid + SNT * u;
    ry[u] = reinterpret_cast<const f32x4*>(Wn + L::Y_)[e4];
    rk[u] = reinterpret_cast<const f32x4*>(Wn + L::KT)[e4];
    if constexpr (FWD) rq[u] = reinterpret_cast<const f32x4*>(Wn + L::QG)[e4];
  }
  if constexpr (FWD) {
#pragma unroll
    for (int u = 0; u < NC4; ++u) ra[u] = reinterpret_cast<const f32x4*>(Wn + L::AQK)[tid + SNT * u];
  }
#pragma unroll
  for (int u = 0; u < NV4; ++u) {
    const int e4 = tid + SNT * u, r = e4 / (DVB / 4), c4 = e4 - r * (DVB / 4);
    ru[u] = *reinterpret_cast<const f32x4*>(Wn + L::U + (size_t)r * DV + jb * DVB + 4 * c4);
  }
  if (tid < DK / 4) rg = reinterpret_cast<const f32x4*>(Wn + L::GC)[tid];
}

template <int DK, int DV, int NK4, int NV4, int NC4, bool BF16>
__device__ __forceinline__ void sb_load(const BwdArgs& a, int ci, int h, int jb, int tid,
                                        f32x4 (&rq)[NK4], f32x4 (&rk)[NK4], f32x4 (&ry)[NK4],
                                        f32x4 (&ra)[NC4], f32x4 (&ro)[NV4], f32x4& rg) {
  typedef BwdLayout<DK, DV> L;
  const float* Wn = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
  // row-major blocks, 16-byte loads in address order
#pragma unroll
  for (int u = 0; u < NK4; ++u) {
    const int e4 = tid + SNT * u;
    rq[u] = reinterpret_cast<const f32x4*>(Wn + L::QG)[e4];
    rk[u] = reinterpret_cast<const f32x4*>(Wn + L::KT)[e4];
    ry[u] = reinterpret_cast<const f32x4*>(Wn + L::Y_)[e4];
  }
#pragma unroll
  for (int u = 0; u < NC4; ++u) ra[u] = reinterpret_cast<const f32x4*>(Wn + L::AQK)[tid + SNT * u];
  // dO straight from the input (rows past the end: a clamped row, zeroed)
  long long row0 = 0;
  int clen = 0;
  bwd_locate(a, ci, row0, clen);
#pragma unroll
  for (int u = 0; u < NV4; ++u) {
    const int e4 = tid + SNT * u, t = e4 / (DVB / 4), j = 4 * (e4 - t * (DVB / 4));
    const int tt = t < clen ? t : clen - 1;
    float x[4];
    load4<BF16>(a.dO, (size_t)(row0 + tt) * a.H * DV + (size_t)h * DV + jb * DVB + j, x);
    ro[u] = f32x4{x[0], x[1], x[2], x[3]} * (t < clen ? 1.f : 0.f);
  }
  if (tid < DK / 4) rg = reinterpret_cast<const f32x4*>(Wn + L::GC)[tid];
}

// ---- sequential state pass of the fp32 forward (Eqs. 23-24) ------------------------
// One workgroup of SNT threads per (sequence, head, 32 value channels); the
// state block is kept transposed in LDS (S^T, the B operand of Y S).  The
// next two chunks' operands are loaded into registers (16-byte loads in
// address order) while the current chunk computes.  Per chunk: R = U - Y S,
// o = Q_g S + A_qk R, S <- Diag(gamma_C) S + K_tail^T R, all on fp32 MFMA;
// the final state after the last chunk.
template <int DK, int DV>
__global__ __launch_bounds__(SNT, 1) void fwd32_state_kernel(BwdArgs a) {
  constexpr bool FWD = true;
  constexpr int NB = DV / DVB, LK = DK + 4, LC = BC + 4, LV = DVB + 4;
  constexpr int NK4 = BC * DK / 4 / SNT;   // float4 per thread of a [BC][DK] block
  constexpr int NV4 = BC * DVB / 4 / SNT;  // float4 per thread of a [BC][DVB] block
  constexpr int NC4 = BC * BC / 4 / SNT;   // float4 per thread of A_qk
  static_assert(NK4 >= 1 && NV4 >= 1, "state pass tiling");
  static_assert((BC / 16) * (DVB / 16) == SNT / 64, "one output tile per wavefront");
  extern __shared__ __align__(16) unsigned char smem[];
  float* sST = reinterpret_cast<float*>(smem);  // [DVB][LK]
  float* sY = sST + DVB * LK;                   // [BC][LK]
  float* sKt = sY + BC * LK;                    // [BC][LK]
  float* sRT = sKt + BC * LK;                   // [DVB][LC]
  float* sU = sRT + DVB * LC;                   // [BC][LV]
  float* sGC = sU + BC * LV;                    // [DK]
  float* sQg = sGC + DK;                        // [BC][LK]
  float* sAq = sQg + BC * LK;                   // [BC][LC]
  // the NB value blocks of one (sequence, head) share an XCD (workgroups go
  // round the eight XCDs in order), so their reads of the chunk blocks they
  // all need hit that XCD's L2
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nh = (slot / NB) * 8 + xcd, jb = slot % NB;
  if (nh >= a.N * a.H) return;
  const int n = nh / a.H, h = nh - n * a.H;
  const int c0 = a.tab ? a.cbase[n] : n * a.nc, c1 = a.tab ? a.cbase[n + 1] : (n + 1) * a.nc;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  for (int e = tid; e < DK * DVB; e += SNT) {
    const int i = e / DVB, j = e - i * DVB;
    sST[j * LK + i] = a.S0 ? a.S0[(size_t)nh * DK * DV + (size_t)i * DV + jb * DVB + j] : 0.f;
  }
  // two register sets in turn: chunks ci + 1 and ci + 2 are in flight while chunk ci computes
  f32x4 ry0[NK4], rk0[NK4], ru0[NV4], rg0 = zero4(), rq0[NK4], ra0[NC4];
  f32x4 ry1[NK4], rk1[NK4], ru1[NV4], rg1 = zero4(), rq1[NK4], ra1[NC4];
  if (c0 < c1) sf_load<DK, DV, NK4, NV4, NC4, FWD>(a, c0, h, jb, tid, ry0, rk0, ru0, rg0, rq0, ra0);
  if (c0 + 1 < c1) sf_load<DK, DV, NK4, NV4, NC4, FWD>(a, c0 + 1, h, jb, tid, ry1, rk1, ru1, rg1, rq1, ra1);
  auto step = [&](const int ci, f32x4 (&ry)[NK4], f32x4 (&rk)[NK4], f32x4 (&ru)[NV4], f32x4& rg,
                  f32x4 (&rq)[NK4], f32x4 (&ra)[NC4]) {
#pragma unroll
    for (int u = 0; u < NK4; ++u) {
      const int e4 = tid + SNT * u, r = e4 / (DK / 4), i = 4 * (e4 - r * (DK / 4));
      *reinterpret_cast<f32x4*>(sY + r * LK + i) = ry[u];
      *reinterpret_cast<f32x4*>(sKt + r * LK + i) = rk[u];
      *reinterpret_cast<f32x4*>(sQg + r * LK + i) = rq[u];
    }
#pragma unroll
    for (int u = 0; u < NC4; ++u) {
      const int e4 = tid + SNT * u, r = e4 / (BC / 4), c4 = e4 - r * (BC / 4);
      *reinterpret_cast<f32x4*>(sAq + r * LC + 4 * c4) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
      const int e4 = tid + SNT * u, r = e4 / (DVB / 4), c4 = e4 - r * (DVB / 4);
      *reinterpret_cast<f32x4*>(sU + r * LV + 4 * c4) = ru[u];
    }
    if (tid < DK / 4) *reinterpret_cast<f32x4*>(sGC + 4 * tid) = rg;
    __syncthreads();
    // R = U - Y S  [BC][DVB] and Q_g S (same tile, from the state entering the chunk)
    f32x4 ao = zero4();
    for (int t = wv; t < (BC / 16) * (DVB / 16); t += SNT / 64) {
      const int tm = t / (DVB / 16), tn = t - tm * (DVB / 16);
      const f32x4 acc = mma_lds<float, DK>(zero4(), sY + 16 * tm * LK, LK, sST + 16 * tn * LK, LK);
      ao = mma_lds<float, DK>(zero4(), sQg + 16 * tm * LK, LK, sST + 16 * tn * LK, LK);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, j = 16 * tn + m;
        const float rv = sU[r * LV + j] - acc[q];
        sRT[j * LC + r] = rv;
      }
    }
    __syncthreads();
    {
      // o = Q_g S + A_qk R (Eq. 24); A_qk is lower triangular, so row tile
      // tm needs the first 16 (tm + 1) tokens of R only
      const int tm = wv / (DVB / 16), tn = wv - tm * (DVB / 16);
      ao = mma_lds_f32<BC, false, false>(ao, sAq + 16 * tm * LC, LC, sRT + 16 * tn * LC, LC, 16 * (tm + 1));
      long long row0 = 0;
      int clen = 0;
      bwd_locate(a, ci, row0, clen);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q;
        if (r < clen) a.o[(size_t)(row0 + r) * a.H * DV + (size_t)h * DV + jb * DVB + 16 * tn + m] = ao[q];
      }
    }
    // the chunk after next into the registers stored above (near the end the
    // current chunk is reloaded instead: no branch); issued here, after R,
    // so that R's products start at once
    sf_load<DK, DV, NK4, NV4, NC4, FWD>(a, ci + 2 < c1 ? ci + 2 : ci, h, jb, tid, ry, rk, ru, rg, rq, ra);
    // S <- Diag(gamma_C) S + K_tail^T R  [DK][DVB]; each lane owns its entries
    constexpr int NSU = (DK / 16) * (DVB / 16);
    {
      for (int t = wv; t < NSU; t += SNT / 64) {
        const int tm = t / (DVB / 16), tn = t - tm * (DVB / 16);
        // K_tail^T as the left factor: K_tail read K-major from its row-major block
        const f32x4 acc = mma_lds_f32<BC, true, false>(zero4(), sKt + 16 * tm, LK, sRT + 16 * tn * LC, LC);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 16 * tm + 4 * g + q, j = 16 * tn + m;
          sST[j * LK + i] = sGC[i] * sST[j * LK + i] + acc[q];
        }
      }
    }
    __syncthreads();
  };
  int ci = c0;
  for (; ci + 1 < c1; ci += 2) {
    step(ci, ry0, rk0, ru0, rg0, rq0, ra0);
    step(ci + 1, ry1, rk1, ru1, rg1, rq1, ra1);
  }
  if (ci < c1) step(ci, ry0, rk0, ru0, rg0, rq0, ra0);
  // the state after the sequence's last token (S0 itself for an empty one)
  if (a.ST)
    for (int e = tid; e < DK * DVB; e += SNT) {
      const int i = e / DVB, j = e - i * DVB;
      a.ST[(size_t)nh * DK * DV + (size_t)i * DV + jb * DVB + j] = sST[j * LK + i];
    }
}

// LDS plan of bwd_state_fwd3_kernel (byte offsets).  The fp32 state S^T is
// the master copy; its bf16 hi/lo halves, those of Y, K_tail and R^T feed the
// products.  Row pitches keep the 16-lane groups' reads on distinct banks:
// DK + 8 and BC + 8 halves for rows read along K, DK + 16 for K_tail, which
// is read down its columns by the transposing read.
template <int DK>
struct StateF3Cfg {
  static constexpr int LK = DK + 4, LV = DVB + 4;  // fp32 S^T, U
  static constexpr int LSB = DK + 8, LTB = DK + 16, LRB = BC + 8;
  static constexpr size_t O_ST = 0;
  static constexpr size_t O_SH = O_ST + (size_t)DVB * LK * 4, O_SL = O_SH + (size_t)DVB * LSB * 2;
  static constexpr size_t O_YH = O_SL + (size_t)DVB * LSB * 2, O_YL = O_YH + (size_t)BC * LSB * 2;
  static constexpr size_t O_KH = O_YL + (size_t)BC * LSB * 2, O_KL = O_KH + (size_t)BC * LTB * 2;
  static constexpr size_t O_RH = O_KL + (size_t)BC * LTB * 2, O_RL = O_RH + (size_t)DVB * LRB * 2;
  static constexpr size_t O_U = O_RL + (size_t)DVB * LRB * 2;
  static constexpr size_t O_GC = O_U + (size_t)BC * LV * 4;
  static constexpr size_t BYTES = O_GC + (size_t)DK * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(O_SH % 16 == 0 && O_YH % 16 == 0 && O_KH % 16 == 0 && O_RH % 16 == 0 &&
                    O_U % 16 == 0 && O_GC % 16 == 0,
                "16-byte aligned regions");
};

// ---- sequential state pass of the backward, products as three bf16 products ----------
// The state entering every chunk and R = U - Y S, saved for the output
// paths, with R = U - Y S and
// S <- Diag(gamma_C) S + K_tail^T R on 16x16x32 bf16 MFMA over hi/lo halves
// (mma3x): the chunk step's dependent chain is twelve instructions per tile
// instead of 32 fp32 ones.  Y and K_tail are split as they are staged, R where
// it is formed and S where the update writes it; the fp32 S stays the master
// copy that the update scales and the workspace receives.
template <int DK, int DV>
__global__ __launch_bounds__(SNT, 1) void bwd_state_fwd3_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  typedef StateF3Cfg<DK> C;
  constexpr int NB = DV / DVB, LK = C::LK, LV = C::LV, LSB = C::LSB, LTB = C::LTB, LRB = C::LRB;
  constexpr int NK4 = BC * DK / 4 / SNT;   // float4 per thread of a [BC][DK] block
  constexpr int NV4 = BC * DVB / 4 / SNT;  // float4 per thread of a [BC][DVB] block
  constexpr int NKB = DK / 32;             // K = 32 blocks of Y S
  static_assert(NK4 >= 1 && NV4 >= 1, "state pass tiling");
  static_assert((BC / 16) * (DVB / 16) == SNT / 64, "one R tile per wavefront");
  extern __shared__ __align__(16) unsigned char smem[];
  float* sST = reinterpret_cast<float*>(smem + C::O_ST);  // [DVB][LK] fp32 S^T
  __bf16* sSh = reinterpret_cast<__bf16*>(smem + C::O_SH);  // [DVB][LSB] S^T halves
  __bf16* sSl = reinterpret_cast<__bf16*>(smem + C::O_SL);
  __bf16* sYh = reinterpret_cast<__bf16*>(smem + C::O_YH);  // [BC][LSB] Y halves
  __bf16* sYl = reinterpret_cast<__bf16*>(smem + C::O_YL);
  __bf16* sKh = reinterpret_cast<__bf16*>(smem + C::O_KH);  // [BC][LTB] K_tail halves
  __bf16* sKl = reinterpret_cast<__bf16*>(smem + C::O_KL);
  __bf16* sRh = reinterpret_cast<__bf16*>(smem + C::O_RH);  // [DVB][LRB] R^T halves
  __bf16* sRl = reinterpret_cast<__bf16*>(smem + C::O_RL);
  float* sU = reinterpret_cast<float*>(smem + C::O_U);     // [BC][LV]
  float* sGC = reinterpret_cast<float*>(smem + C::O_GC);   // [DK]
  // the NB value blocks of one (sequence, head) share an XCD (workgroups go
  // round the eight XCDs in order), so their reads of the chunk blocks they
  // all need hit that XCD's L2
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nh = (slot / NB) * 8 + xcd, jb = slot % NB;
  if (nh >= a.N * a.H) return;
  const int n = nh / a.H, h = nh - n * a.H;
  const int c0 = a.tab ? a.cbase[n] : n * a.nc, c1 = a.tab ? a.cbase[n + 1] : (n + 1) * a.nc;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  // S0 block: thread e4 takes 4 consecutive key channels i of value column j
  for (int e4 = tid; e4 < DK * DVB / 4; e4 += SNT) {
    const int j = e4 / (DK / 4), i = 4 * (e4 - j * (DK / 4));
    f32x4 s = zero4();
    if (a.S0) {
      const float* src = a.S0 + (size_t)nh * DK * DV + (size_t)i * DV + jb * DVB + j;
      s = f32x4{src[0], src[DV], src[2 * DV], src[3 * DV]};
    }
    *reinterpret_cast<f32x4*>(sST + j * LK + i) = s;
    bf16x4 hi, lo;
    split_bf16(s, hi, lo);
    *reinterpret_cast<bf16x4*>(sSh + j * LSB + i) = hi;
    *reinterpret_cast<bf16x4*>(sSl + j * LSB + i) = lo;
  }
  __syncthreads();  // the first chunk step saves S0 in another thread mapping
  // two register sets in turn: chunks ci + 1 and ci + 2 are in flight while chunk ci computes
  f32x4 ry0[NK4], rk0[NK4], ru0[NV4], rg0 = zero4(), rq0[NK4], ra0[1];
  f32x4 ry1[NK4], rk1[NK4], ru1[NV4], rg1 = zero4(), rq1[NK4], ra1[1];
  if (c0 < c1) sf_load<DK, DV, NK4, NV4, 1, false>(a, c0, h, jb, tid, ry0, rk0, ru0, rg0, rq0, ra0);
  if (c0 + 1 < c1) sf_load<DK, DV, NK4, NV4, 1, false>(a, c0 + 1, h, jb, tid, ry1, rk1, ru1, rg1, rq1, ra1);
  auto step = [&](const int ci, f32x4 (&ry)[NK4], f32x4 (&rk)[NK4], f32x4 (&ru)[NV4], f32x4& rg,
                  f32x4 (&rq)[NK4], f32x4 (&ra)[1]) {
    float* W = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
#pragma unroll
    for (int u = 0; u < NK4; ++u) {
      const int e4 = tid + SNT * u, r = e4 / (DK / 4), i = 4 * (e4 - r * (DK / 4));
      bf16x4 hi, lo;
      split_bf16(ry[u], hi, lo);
      *reinterpret_cast<bf16x4*>(sYh + r * LSB + i) = hi;
      *reinterpret_cast<bf16x4*>(sYl + r * LSB + i) = lo;
      split_bf16(rk[u], hi, lo);
      *reinterpret_cast<bf16x4*>(sKh + r * LTB + i) = hi;
      *reinterpret_cast<bf16x4*>(sKl + r * LTB + i) = lo;
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
      const int e4 = tid + SNT * u, r = e4 / (DVB / 4), c4 = e4 - r * (DVB / 4);
      *reinterpret_cast<f32x4*>(sU + r * LV + 4 * c4) = ru[u];
    }
    if (tid < DK / 4) *reinterpret_cast<f32x4*>(sGC + 4 * tid) = rg;
    for (int e = tid; e < DK * DVB; e += SNT) {  // the state entering chunk ci
      const int i = e / DVB, j = e - i * DVB;
      W[L::S + (size_t)i * DV + jb * DVB + j] = sST[j * LK + i];
    }
    __syncthreads();
    {
      // R = U - Y S, one [16][16] tile per wavefront: Y rows and S^T rows
      // both run along K; alternate K blocks go to two chains
      const int tm = wv / (DVB / 16), tn = wv - tm * (DVB / 16);
      f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int k0 = 32 * kb;
        const bf16x8 ah = frag_krow(sYh, LSB, k0, 16 * tm), al = frag_krow(sYl, LSB, k0, 16 * tm);
        const bf16x8 bh = frag_krow(sSh, LSB, k0, 16 * tn), bl = frag_krow(sSl, LSB, k0, 16 * tn);
        if (kb & 1) acc1 = mma3x(ah, al, bh, bl, acc1);
        else acc0 = mma3x(ah, al, bh, bl, acc0);
      }
      const f32x4 acc = acc0 + acc1;
      f32x4 rv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, j = 16 * tn + m;
        rv[q] = sU[r * LV + j] - acc[q];
        W[L::R + (size_t)r * DV + jb * DVB + j] = rv[q];
      }
      bf16x4 hi, lo;
      split_bf16(rv, hi, lo);
      *reinterpret_cast<bf16x4*>(sRh + (16 * tn + m) * LRB + 16 * tm + 4 * g) = hi;
      *reinterpret_cast<bf16x4*>(sRl + (16 * tn + m) * LRB + 16 * tm + 4 * g) = lo;
    }
    __syncthreads();
    // the chunk after next into the registers stored above (near the end the
    // current chunk is reloaded instead: no branch); issued here, after R,
    // so that R's products start at once
    sf_load<DK, DV, NK4, NV4, 1, false>(a, ci + 2 < c1 ? ci + 2 : ci, h, jb, tid, ry, rk, ru, rg, rq, ra);
    // S <- Diag(gamma_C) S + K_tail^T R  [DK][DVB]; each lane owns its entries.
    // K_tail^T comes down the columns of the row-major K_tail (transposing
    // reads), R^T rows run along K.
    // The tiles t = wv + 8u of a wavefront share the column block tn, so one
    // pair of R^T fragments per K block serves every chain, interleaved.
    constexpr int NSU = (DK / 16) * (DVB / 16), NPW = (NSU + SNT / 64 - 1) / (SNT / 64);
    const int tn = wv % (DVB / 16), j = 16 * tn + m;
    f32x4 acc[NPW];
#pragma unroll
    for (int u = 0; u < NPW; ++u) acc[u] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < BC; k0 += 32) {
      const bf16x8 bh = frag_krow(sRh, LRB, k0, 16 * tn), bl = frag_krow(sRl, LRB, k0, 16 * tn);
#pragma unroll
      for (int u = 0; u < NPW; ++u) {
        const int tm = (wv + (SNT / 64) * u) / (DVB / 16);
        if (tm < DK / 16) {  // uniform per wavefront
          const bf16x8 ah = frag_kmajor(sKh, LTB, k0, 16 * tm), al = frag_kmajor(sKl, LTB, k0, 16 * tm);
          acc[u] = mma3x(ah, al, bh, bl, acc[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
      const int tm = (wv + (SNT / 64) * u) / (DVB / 16), i = 16 * tm + 4 * g;
      if (tm < DK / 16) {
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(sST + j * LK + i);
        const f32x4 gc = *reinterpret_cast<const f32x4*>(sGC + i);
        const f32x4 s = gc * s0 + acc[u];
        *reinterpret_cast<f32x4*>(sST + j * LK + i) = s;
        bf16x4 hi, lo;
        split_bf16(s, hi, lo);
        *reinterpret_cast<bf16x4*>(sSh + j * LSB + i) = hi;
        *reinterpret_cast<bf16x4*>(sSl + j * LSB + i) = lo;
      }
    }
    __syncthreads();
  };
  int ci = c0;
  for (; ci + 1 < c1; ci += 2) {
    step(ci, ry0, rk0, ru0, rg0, rq0, ra0);
    step(ci + 1, ry1, rk1, ru1, rg1, rq1, ra1);
  }
  if (ci < c1) step(ci, ry0, rk0, ru0, rg0, rq0, ra0);
}

// LDS plan of bwd_state_bwd3_kernel (byte offsets): the fp32 dS'^T master,
// and bf16 hi/lo halves of dS'^T, A_qk, dO, Q_g, -dR^T and one region X that
// holds K_tail for dR and then Y for the state gradient.  Blocks read down
// their columns (transposing reads: A_qk, dO, Q_g, Y) have pitches whose four
// rows per 16-lane group land on distinct banks; blocks read along rows
// (K_tail, dS'^T, -dR^T) pitches of 4 words mod 64.
template <int DK>
struct StateB3Cfg {
  static constexpr int LK = DK + 4;  // fp32 dS'^T
  static constexpr int LSB = DK + 8, LAB = BC + 16, LOB = DVB + 16, LTB = DK + 16, LRB = BC + 8;
  static constexpr size_t O_DST = 0;
  static constexpr size_t O_DSH = O_DST + (size_t)DVB * LK * 4, O_DSL = O_DSH + (size_t)DVB * LSB * 2;
  static constexpr size_t O_AH = O_DSL + (size_t)DVB * LSB * 2, O_AL = O_AH + (size_t)BC * LAB * 2;
  static constexpr size_t O_OH = O_AL + (size_t)BC * LAB * 2, O_OL = O_OH + (size_t)BC * LOB * 2;
  static constexpr size_t O_QH = O_OL + (size_t)BC * LOB * 2, O_QL = O_QH + (size_t)BC * LTB * 2;
  static constexpr size_t O_XH = O_QL + (size_t)BC * LTB * 2, O_XL = O_XH + (size_t)BC * LSB * 2;
  static constexpr size_t O_RH = O_XL + (size_t)BC * LSB * 2, O_RL = O_RH + (size_t)DVB * LRB * 2;
  static constexpr size_t O_GC = O_RL + (size_t)DVB * LRB * 2;
  static constexpr size_t BYTES = O_GC + (size_t)DK * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(O_DSH % 16 == 0 && O_AH % 16 == 0 && O_OH % 16 == 0 && O_QH % 16 == 0 &&
                    O_XH % 16 == 0 && O_RH % 16 == 0 && O_GC % 16 == 0,
                "16-byte aligned regions");
};

// ---- sequential reverse pass, products as three bf16 products ----------------------
// dS' and dR of every chunk, and dS0, with every product on 16x16x32 bf16 MFMA over hi/lo halves (mma3x).  A
// chunk step, chunks in reverse:
//   stage Q_g, A_qk, dO, K_tail (split as they are stored), save dS';
//   dR = A_qk^T dO + K_tail dS' (one tile per wavefront), and Q_g^T dO into
//   the state-gradient accumulators (two tiles per wavefront, same dO
//   fragments); -dR^T split into LDS;
//   stage Y over K_tail, then issue the previous chunk's loads;
//   dS <- (Q_g^T dO - Y^T dR) + Diag(gamma_C) dS', the fp32 master and its
//   halves written by the lanes that own the entries.
template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(SNT, 1) void bwd_state_bwd3_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  typedef StateB3Cfg<DK> C;
  constexpr int NB = DV / DVB, LK = C::LK, LSB = C::LSB, LAB = C::LAB, LOB = C::LOB, LTB = C::LTB,
                LRB = C::LRB;
  constexpr int NK4 = BC * DK / 4 / SNT, NV4 = BC * DVB / 4 / SNT, NC4 = BC * BC / 4 / SNT;
  constexpr int NKB = DK / 32;  // K = 32 blocks of K_tail dS'
  constexpr int NSU = (DK / 16) * (DVB / 16), NPW = (NSU + SNT / 64 - 1) / (SNT / 64);
  static_assert(NK4 >= 1 && NV4 >= 1 && NC4 >= 1, "state pass tiling");
  static_assert((BC / 16) * (DVB / 16) == SNT / 64, "one dR tile per wavefront");
  extern __shared__ __align__(16) unsigned char smem[];
  float* sdST = reinterpret_cast<float*>(smem + C::O_DST);  // [DVB][LK] fp32 dS'^T
  __bf16* sDh = reinterpret_cast<__bf16*>(smem + C::O_DSH);  // [DVB][LSB] dS'^T halves
  __bf16* sDl = reinterpret_cast<__bf16*>(smem + C::O_DSL);
  __bf16* sAh = reinterpret_cast<__bf16*>(smem + C::O_AH);   // [BC][LAB] A_qk halves
  __bf16* sAl = reinterpret_cast<__bf16*>(smem + C::O_AL);
  __bf16* sOh = reinterpret_cast<__bf16*>(smem + C::O_OH);   // [BC][LOB] dO halves
  __bf16* sOl = reinterpret_cast<__bf16*>(smem + C::O_OL);
  __bf16* sQh = reinterpret_cast<__bf16*>(smem + C::O_QH);   // [BC][LTB] Q_g halves
  __bf16* sQl = reinterpret_cast<__bf16*>(smem + C::O_QL);
  __bf16* sXh = reinterpret_cast<__bf16*>(smem + C::O_XH);   // [BC][LSB] K_tail, then Y
  __bf16* sXl = reinterpret_cast<__bf16*>(smem + C::O_XL);
  __bf16* sRh = reinterpret_cast<__bf16*>(smem + C::O_RH);   // [DVB][LRB] -dR^T halves
  __bf16* sRl = reinterpret_cast<__bf16*>(smem + C::O_RL);
  float* sGC = reinterpret_cast<float*>(smem + C::O_GC);     // [DK]
  // the NB value blocks of one (sequence, head) share an XCD (workgroups go
  // round the eight XCDs in order), so their reads of the chunk blocks they
  // all need hit that XCD's L2
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nh = (slot / NB) * 8 + xcd, jb = slot % NB;
  if (nh >= a.N * a.H) return;
  const int n = nh / a.H, h = nh - n * a.H;
  const int c0 = a.tab ? a.cbase[n] : n * a.nc, c1 = a.tab ? a.cbase[n + 1] : (n + 1) * a.nc;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  // dS_T block: thread e4 takes 4 consecutive key channels i of value column j
  for (int e4 = tid; e4 < DK * DVB / 4; e4 += SNT) {
    const int j = e4 / (DK / 4), i = 4 * (e4 - j * (DK / 4));
    f32x4 s = zero4();
    if (a.dST) {
      const float* src = a.dST + (size_t)nh * DK * DV + (size_t)i * DV + jb * DVB + j;
      s = f32x4{src[0], src[DV], src[2 * DV], src[3 * DV]};
    }
    *reinterpret_cast<f32x4*>(sdST + j * LK + i) = s;
    bf16x4 hi, lo;
    split_bf16(s, hi, lo);
    *reinterpret_cast<bf16x4*>(sDh + j * LSB + i) = hi;
    *reinterpret_cast<bf16x4*>(sDl + j * LSB + i) = lo;
  }
  __syncthreads();  // the first chunk step saves dS' in another thread mapping
  auto st_split = [](__bf16* hb, __bf16* lb, int off, const f32x4& x) {
    bf16x4 hi, lo;
    split_bf16(x, hi, lo);
    *reinterpret_cast<bf16x4*>(hb + off) = hi;
    *reinterpret_cast<bf16x4*>(lb + off) = lo;
  };
  const int tn = wv % (DVB / 16);  // column block of every tile of this wavefront
  f32x4 rq[NK4], rk[NK4], ry[NK4], ra[NC4], ro[NV4], rg = zero4();
  if (c0 < c1) sb_load<DK, DV, NK4, NV4, NC4, BF16>(a, c1 - 1, h, jb, tid, rq, rk, ry, ra, ro, rg);
  for (int ci = c1 - 1; ci >= c0; --ci) {
    float* W = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
#pragma unroll
    for (int u = 0; u < NK4; ++u) {
      const int e4 = tid + SNT * u, t = e4 / (DK / 4), i = 4 * (e4 - t * (DK / 4));
      st_split(sXh, sXl, t * LSB + i, rk[u]);
      st_split(sQh, sQl, t * LTB + i, rq[u]);
    }
#pragma unroll
    for (int u = 0; u < NC4; ++u) {
      const int e4 = tid + SNT * u, t = e4 / (BC / 4), r = 4 * (e4 - t * (BC / 4));
      st_split(sAh, sAl, t * LAB + r, ra[u]);
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
      const int e4 = tid + SNT * u, t = e4 / (DVB / 4), j = 4 * (e4 - t * (DVB / 4));
      st_split(sOh, sOl, t * LOB + j, ro[u]);
    }
    if (tid < DK / 4) *reinterpret_cast<f32x4*>(sGC + 4 * tid) = rg;
    for (int e = tid; e < DK * DVB; e += SNT) {  // dL/d(state leaving chunk ci)
      const int i = e / DVB, j = e - i * DVB;
      W[L::DSP + (size_t)i * DV + jb * DVB + j] = sdST[j * LK + i];
    }
    __syncthreads();
    // dO fragments (K = the chunk's tokens) shared by every product below
    bf16x8 oh[2], ol[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      oh[kb] = frag_kmajor(sOh, LOB, 32 * kb, 16 * tn);
      ol[kb] = frag_kmajor(sOl, LOB, 32 * kb, 16 * tn);
    }
    // Q_g^T dO, the first part of the state gradient (tiles t = wv + 8u)
    f32x4 ds[NPW];
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
      ds[u] = zero4();
      const int tm = (wv + (SNT / 64) * u) / (DVB / 16);
      if (tm < DK / 16) {  // uniform per wavefront
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 qh = frag_kmajor(sQh, LTB, 32 * kb, 16 * tm), ql = frag_kmajor(sQl, LTB, 32 * kb, 16 * tm);
          ds[u] = mma3x(qh, ql, oh[kb], ol[kb], ds[u]);
        }
      }
    }
    {
      // dR = A_qk^T dO + K_tail dS', one tile per wavefront, as two chains.
      // A_qk is lower triangular: A_qk^T rows 16 tm.. need tokens from 16 tm
      // on, so the first K block is zero for tm >= 2.
      const int tm = wv / (DVB / 16);
      f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 0 && tm >= 2) continue;  // uniform per wavefront
        const bf16x8 ah = frag_kmajor(sAh, LAB, 32 * kb, 16 * tm), al = frag_kmajor(sAl, LAB, 32 * kb, 16 * tm);
        acc0 = mma3x(ah, al, oh[kb], ol[kb], acc0);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 kh = frag_krow(sXh, LSB, 32 * kb, 16 * tm), kl = frag_krow(sXl, LSB, 32 * kb, 16 * tm);
        const bf16x8 dh = frag_krow(sDh, LSB, 32 * kb, 16 * tn), dl = frag_krow(sDl, LSB, 32 * kb, 16 * tn);
        acc1 = mma3x(kh, kl, dh, dl, acc1);
      }
      const f32x4 acc = acc0 + acc1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, j = 16 * tn + m;
        W[L::DR + (size_t)r * DV + jb * DVB + j] = acc[q];
      }
      st_split(sRh, sRl, (16 * tn + m) * LRB + 16 * tm + 4 * g, -acc);
    }
    __syncthreads();
    // Y over K_tail (every read of K_tail is done), then the previous chunk
    // into the registers just stored (the last iteration reloads the current
    // one: no branch)
#pragma unroll
    for (int u = 0; u < NK4; ++u) {
      const int e4 = tid + SNT * u, t = e4 / (DK / 4), i = 4 * (e4 - t * (DK / 4));
      st_split(sXh, sXl, t * LSB + i, ry[u]);
    }
    sb_load<DK, DV, NK4, NV4, NC4, BF16>(a, ci - 1 >= c0 ? ci - 1 : ci, h, jb, tid, rq, rk, ry, ra, ro, rg);
    __syncthreads();
    // dS <- Q_g^T dO - Y^T dR + Diag(gamma_C) dS'; each lane owns its entries
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 rh = frag_krow(sRh, LRB, 32 * kb, 16 * tn), rl = frag_krow(sRl, LRB, 32 * kb, 16 * tn);
#pragma unroll
      for (int u = 0; u < NPW; ++u) {
        const int tm = (wv + (SNT / 64) * u) / (DVB / 16);
        if (tm < DK / 16) {
          const bf16x8 yh = frag_kmajor(sXh, LSB, 32 * kb, 16 * tm), yl = frag_kmajor(sXl, LSB, 32 * kb, 16 * tm);
          ds[u] = mma3x(yh, yl, rh, rl, ds[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
      const int tm = (wv + (SNT / 64) * u) / (DVB / 16), i = 16 * tm + 4 * g, j = 16 * tn + m;
      if (tm < DK / 16) {
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(sdST + j * LK + i);
        const f32x4 gc = *reinterpret_cast<const f32x4*>(sGC + i);
        const f32x4 d = ds[u] + gc * d0;
        *reinterpret_cast<f32x4*>(sdST + j * LK + i) = d;
        st_split(sDh, sDl, j * LSB + i, d);
      }
    }
    __syncthreads();
  }
  if (a.dS0)
    for (int e = tid; e < DK * DVB; e += SNT) {
      const int i = e / DVB, j = e - i * DVB;
      a.dS0[(size_t)nh * DK * DV + (size_t)i * DV + jb * DVB + j] = sdST[j * LK + i];
    }
}

// ---- output and WY-gradient paths, fused per item ------------------------------------
// One workgroup per item forms, from the item's fp32 blocks (R, dR, A, the
// decay G), the inputs (dO, v, w, q, k, b) and the states S and dS' on either
// side of the chunk, every remaining product and the gradients themselves.
// E, E' (phase 2a) and Q', K' (phase 2b) are formed again from G, q, k, b:
//   phase 1  dQ_g = dO S^T, dY = -dR S^T, dK_tail = R dS'^T,
//            dA_qk = tril(dO R^T), dA = dR Z^T, dZ = A^T dR (-> dv, dw), and
//            the row sums of dS' * S; the value channels stream through LDS
//            in slices of 32, the results stay in the accumulators;
//   phase 2  dA += dY E^T, X = A^T dY, then dA_qk^T Q' and dA_qk K';
//   phase 3  dT = -tril(A^T dA A^T, -1);
//   phase 4  dT K' and dT^T E';
//   final    dq, dk, db from the accumulators (the centred factors put back
//            per element), and dg as the reverse cumulative sum over the
//            chunk's rows (row blocks summed in parallel, then scanned).
// Operands are staged in LDS from 16-byte loads in address order, rows padded
// by 4 floats, and read either K-contiguous (16-byte reads) or K-major (four
// 4-byte reads per K = 16 block); a 16-lane group's reads hit distinct banks
// either way.  The fp32 products run on 16x16x4 MFMA.  Tiles of a [64][N]
// result go round the eight wavefronts (tile t = wave + 8u, row tile
// t / (N/16), column tile t % (N/16)).  Each
// phase's global loads are issued into registers one phase (or one slice)
// ahead, so they overlap the products of the phase before.  Rows past the
// end of a sequence read a clamped (valid) row and are zeroed in registers.
// One [16][16] tile of M X for a triangular M over the chunk's 64 tokens,
// from bf16 hi/lo halves: M row-major with its 64 hi then 64 lo halves per row
// (pitch LHA), X a [64][DK] block whose rows are tokens, read down its columns
// (pitch LH, hi halves at column c, lo at DK + c).  Rows 16 tm.. of M are zero
// before token 16 tm when UPPER (M strictly upper triangular), or from token
// 16 (tm + 1) on otherwise, so only the K = 32 blocks that can be nonzero run.
template <int LHA, int LH, bool UPPER>
__device__ __forceinline__ f32x4 tri3x(const float* M, const float* X, int tm, int tn) {
  constexpr int DK = (LH - 8) / 2;
  const __bf16 *bm = reinterpret_cast<const __bf16*>(M), *bx = reinterpret_cast<const __bf16*>(X);
  f32x4 acc = zero4();
#pragma unroll
  for (int k0 = 0; k0 < BC; k0 += 32) {
    if (UPPER ? k0 + 32 <= 16 * tm : k0 >= 16 * (tm + 1)) continue;  // uniform
    acc = mma3x(frag_krow(bm, LHA, k0, 16 * tm), frag_krow(bm, LHA, BC + k0, 16 * tm),
                frag_kmajor(bx, LH, k0, 16 * tn), frag_kmajor(bx, LH, k0, DK + 16 * tn), acc);
  }
  return acc;
}

// One [16][16] tile of A^T X over the chunk's 64 tokens, from bf16 hi/lo
// halves (pitch LHA: a row's 64 hi then 64 lo halves): A row-major and lower
// triangular (its transpose read down the columns), X given transposed (row
// n of XT holds X[.][n] along the tokens).  Rows 16 tm.. of A^T are zero
// before token 16 tm, so a K = 32 block wholly before it is skipped.
template <int LHA>
__device__ __forceinline__ f32x4 at3x(const float* A, const float* XT, int tm, int tn) {
  const __bf16 *ba = reinterpret_cast<const __bf16*>(A), *bx = reinterpret_cast<const __bf16*>(XT);
  f32x4 acc = zero4();
#pragma unroll
  for (int k0 = 0; k0 < BC; k0 += 32) {
    if (k0 + 32 <= 16 * tm) continue;  // uniform
    acc = mma3x(frag_kmajor(ba, LHA, k0, 16 * tm), frag_kmajor(ba, LHA, k0, BC + 16 * tm),
                frag_krow(bx, LHA, k0, 16 * tn), frag_krow(bx, LHA, BC + k0, 16 * tn), acc);
  }
  return acc;
}

template <int DK, int DV>
struct OutCfg {
  static constexpr int NT = 512, NWV = 8, KC = 32, LS = KC + 4, LA = BC + 4, LKP = DK + 4;
  static constexpr int NKT = DK / 32;  // [64][DK] tiles per wavefront
  static constexpr int NCT = 2;        // [64][64] tiles per wavefront
  // LDS offsets in floats.  A (row-major) lives through phase 3; region R1
  // is reused.
  static constexpr int O_A = 0, O_R1 = O_A + BC * LA;
  // phase 1: slices of dO, dR, R, Z, w, v [64][KC], of S, dS' [DK][KC], dR^T [KC][64]
  static constexpr int O_O = O_R1, O_DR = O_O + BC * LS, O_R = O_DR + BC * LS,
                       O_Z = O_R + BC * LS, O_S = O_Z + BC * LS, O_DS = O_S + DK * LS,
                       O_DRT = O_DS + DK * LS, O_W = O_DRT + KC * LA, O_V = O_W + BC * LS,
                       E1 = O_V + BC * LS;
  // phase 2a: dY [64][DK], E [64][DK], dY^T [DK][64]
  static constexpr int O_DY = O_R1, O_EB = O_DY + BC * LKP, O_DYT = O_EB + BC * LKP,
                       E2 = O_DYT + DK * LA;
  // phases 2b-4: K' [64][DK] stays; the rest rotates behind it
  static constexpr int O_KP = O_R1, O_X = O_KP + BC * LKP;
  static constexpr int O_QP = O_X, O_AQ = O_QP + BC * LKP, O_AQT = O_AQ + BC * LA,
                       E3 = O_AQT + BC * LA;                                  // 2b
  static constexpr int O_DAT = O_X, O_WM = O_DAT + BC * LA, E4 = O_WM + BC * LA;  // 3
  static constexpr int O_DT = O_X, O_DTT = O_DT + BC * LA, E5 = O_DTT + BC * LA;  // 4
  // final: the per-element dg terms [64][DK] twice
  static constexpr int O_U = O_R1, O_V2 = O_U + BC * LKP, E6 = O_V2 + BC * LKP;
  static constexpr int mx(int x, int y) { return x > y ? x : y; }
  // E' [64][DK] from phase 2a to phase 4; per-channel values: G at row 31
  // and 63, gamma_C, the dS' * S row sums; the dg scan's row-block partial sums
  static constexpr int O_EP = mx(mx(mx(E1, E2), mx(E3, E4)), mx(E5, E6));
  // strong chunks (see BWD_SLIM): G [64][DK] takes E''s place from phase 2a to
  // phase 4, and b k [64][DK] sits behind phase 4's dT and dT^T
  static constexpr int O_BK = E5;
  static_assert(O_BK + BC * LKP <= O_EP, "b k block overlaps E'");
  static constexpr int O_G31 = O_EP + BC * LKP;
  static constexpr int O_GCL = O_G31 + DK, O_GCX = O_GCL + DK, O_RS = O_GCX + DK,
                       O_PU = O_RS + DK, O_PV = O_PU + NT, O_DQK = O_PV + NT, FLOATS = O_DQK + BC;
  static constexpr size_t BYTES = (size_t)FLOATS * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(DV % KC == 0 && DK % 32 == 0 && NT % DK == 0, "output pass tiling");
};

// One item of the output pass.  SM = 0: the main launch, without the exact
// decay path; it leaves the chunks the front pass flagged strong.  SM = 1:
// a flagged chunk, with the exact decay.
template <int DK, int DV, bool BF16, int SM>
__device__ __forceinline__ void out_item(const BwdArgs& a, const int item) {
  typedef BwdLayout<DK, DV> L;
  typedef OutCfg<DK, DV> C;
  constexpr int NT = C::NT, NWV = C::NWV, KC = C::KC, LS = C::LS, LA = C::LA, LKP = C::LKP;
  constexpr int NKT = C::NKT, NCT = C::NCT, TNK = DK / 16;
  constexpr int NS = DV / KC;                         // value slices
  constexpr int NSK = (DK * KC / 4 + NT - 1) / NT;    // float4 of an S slice per thread
  constexpr int NEK = BC * DK / 4 / NT;               // float4 of a [64][DK] block per thread
  constexpr int NAA = BC * BC / 4 / NT;               // float4 of a [64][64] block per thread
  const int ci = item / a.H, h = item - ci * a.H;
  long long row0;
  int clen;
  if (!bwd_locate(a, ci, row0, clen) || clen <= 0) return;
  // the front pass flagged this item's chunk strong (the same test on the
  // same G): it is the strong launch's
  if constexpr (SM == 0)
    if (a.sflag[item] != 0) return;  // uniform
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* sm = reinterpret_cast<float*>(smem_raw);
  const float* W = a.ws + (size_t)item * L::FLOATS;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  const size_t kr = (size_t)a.H * DK, vr = (size_t)a.H * DV;
  float* sA = sm + C::O_A;
  // The main launch multiplies every block but the value slices' fp32 copies
  // (sW, sV) as bf16 hi/lo halves (mma3x): a [64][DK] block keeps a row's DK
  // hi halves, then its DK lo halves (pitch LHK), a [.][64] block its 64 hi
  // then 64 lo halves (pitch LHA), in the bytes of the fp32 rows.  The strong
  // launch keeps fp32 blocks and products.
  constexpr bool SPLIT = SM == 0;
  constexpr int LHK = 2 * LKP, LHA = 2 * LA;
  auto st_h = [](float* base, int ld, int off, int row, int col, float x) {
    __bf16* b = reinterpret_cast<__bf16*>(base) + row * ld + col;
    const __bf16 hi = (__bf16)x;
    b[0] = hi;
    b[off] = (__bf16)(x - (float)hi);
  };
  auto st_h4 = [](float* base, int ld, int off, int row, int col, const f32x4& x) {
    __bf16* b = reinterpret_cast<__bf16*>(base) + row * ld + col;
    bf16x4 hi, lo;
    split_bf16(x, hi, lo);
    *reinterpret_cast<bf16x4*>(b) = hi;
    *reinterpret_cast<bf16x4*>(b + off) = lo;
  };
  // Products with a triangular left factor over the chunk's 64 rows run over
  // its nonzero K range only, for row tile tm: a lower-triangular factor has
  // no columns past 16 (tm + 1), an upper-triangular one none before 16 tm
  // (A, dA_qk, dT and their transposes).  A^T and the right factors Q', K',
  // E' are read K-major from row-major blocks.
  float *sO = sm + C::O_O, *sDR = sm + C::O_DR, *sR = sm + C::O_R, *sZ = sm + C::O_Z;
  float *sS = sm + C::O_S, *sDS = sm + C::O_DS, *sDRT = sm + C::O_DRT;
  float *sW = sm + C::O_W, *sV = sm + C::O_V;

  // value slice j0 of dO, w, v (inputs), R, dR (workspace) and S, dS' into
  // registers: row s = tid / 8, 4 channels at 4 * (tid % 8)
  const int ss = tid / (KC / 4), sc4 = tid - ss * (KC / 4);
  const int ssr = ss < clen ? ss : clen - 1;
  f32x4 pO, pR, pDR, pW, pV, pS[NSK], pDS[NSK];
  auto slice_load = [&](int j0) {
    const size_t xi = (size_t)(row0 + ssr) * vr + (size_t)h * DV + j0 + 4 * sc4;
    const size_t xw = (size_t)ss * DV + j0 + 4 * sc4;
    float t0[4], t1[4], t2[4];
    load4<BF16>(a.dO, xi, t0);
    load4<BF16>(a.w, xi, t1);
    load4<BF16>(a.v, xi, t2);
    const float z = ss < clen ? 1.f : 0.f;
    pO = f32x4{t0[0], t0[1], t0[2], t0[3]} * z;
    pW = f32x4{t1[0], t1[1], t1[2], t1[3]} * z;
    pV = f32x4{t2[0], t2[1], t2[2], t2[3]} * z;
    pR = *reinterpret_cast<const f32x4*>(W + L::R + xw);
    pDR = *reinterpret_cast<const f32x4*>(W + L::DR + xw);
#pragma unroll
    for (int u = 0; u < NSK; ++u) {
      const int e = tid + NT * u;
      if (e < DK * KC / 4) {
        const int i = e / (KC / 4), c4 = e - i * (KC / 4);
        pS[u] = *reinterpret_cast<const f32x4*>(W + L::S + (size_t)i * DV + j0 + 4 * c4);
        pDS[u] = *reinterpret_cast<const f32x4*>(W + L::DSP + (size_t)i * DV + j0 + 4 * c4);
      }
    }
  };
  slice_load(0);
#pragma unroll
  for (int u = 0; u < NAA; ++u) {
    const int e = tid + NT * u, s = e / (BC / 4), c4 = e - s * (BC / 4);
    const f32x4 x = *reinterpret_cast<const f32x4*>(W + L::A + s * BC + 4 * c4);
    if constexpr (SPLIT) st_h4(sA, LHA, BC, s, 4 * c4, x);
    else *reinterpret_cast<f32x4*>(sA + s * LA + 4 * c4) = x;
  }
  if (tid < DK) {
    sm[C::O_G31 + tid] = W[L::G + 31 * DK + tid];
    sm[C::O_GCL + tid] = W[L::G + (BC - 1) * DK + tid];
    sm[C::O_GCX + tid] = W[L::GC + tid];
  }

  // ---- phase 1 ----
  f32x4 aQ[NKT], aY[NKT], aK[NKT], aAQ[NCT], aA[NCT];
  f32x4 pG[NEK], pK[NEK], pB[NEK];  // G, k, b of row-major units: E, E', K', Q' are formed again
#pragma unroll
  for (int u = 0; u < NKT; ++u) aQ[u] = aY[u] = aK[u] = zero4();
#pragma unroll
  for (int u = 0; u < NCT; ++u) aAQ[u] = aA[u] = zero4();
  // Row sums over the value channels of dS' * S: each thread sums the entries
  // it stages (row (tid + NT u) / 8, 4 channels per slice); the 8 threads of a
  // row, consecutive lanes, are combined after the last slice.
  float rsp[NSK];
#pragma unroll
  for (int u = 0; u < NSK; ++u) rsp[u] = 0.f;
  // The products of this phase take their operands as bf16 hi/lo halves
  // (mma3x), split once as they are staged: a row of a [.][KC] slice holds
  // its KC hi halves, then its KC lo halves (pitch LH halves, the bytes of
  // the fp32 row it replaces).
  constexpr int LH = 2 * LS;
  static_assert(KC == 32 && LH % 8 == 0, "one K = 32 block per slice, 16-byte aligned rows");
  __bf16 *bO = reinterpret_cast<__bf16*>(sO), *bDR = reinterpret_cast<__bf16*>(sDR);
  __bf16 *bR = reinterpret_cast<__bf16*>(sR), *bZ = reinterpret_cast<__bf16*>(sZ);
  __bf16 *bS = reinterpret_cast<__bf16*>(sS), *bDS = reinterpret_cast<__bf16*>(sDS);
  auto st_split = [&](__bf16* base, int row, int c, const f32x4& x) {
    bf16x4 hi, lo;
    split_bf16(x, hi, lo);
    *reinterpret_cast<bf16x4*>(base + row * LH + c) = hi;
    *reinterpret_cast<bf16x4*>(base + row * LH + KC + c) = lo;
  };
  for (int sl = 0; sl < NS; ++sl) {
    const int j0 = sl * KC;
    {
      const int o = ss * LS + 4 * sc4;
      st_split(bO, ss, 4 * sc4, pO);
      st_split(bR, ss, 4 * sc4, pR);
      st_split(bDR, ss, 4 * sc4, pDR);
      st_split(bZ, ss, 4 * sc4, pW * pV);
      *reinterpret_cast<f32x4*>(sW + o) = pW;
      *reinterpret_cast<f32x4*>(sV + o) = pV;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (SPLIT) st_h(sDRT, LHA, BC, 4 * sc4 + q, ss, pDR[q]);
        else sDRT[(4 * sc4 + q) * LA + ss] = pDR[q];
      }
#pragma unroll
      for (int u = 0; u < NSK; ++u) {
        const int e = tid + NT * u;
        if (e < DK * KC / 4) {
          const int i = e / (KC / 4), c4 = e - i * (KC / 4);
          st_split(bS, i, 4 * c4, pS[u]);
          st_split(bDS, i, 4 * c4, pDS[u]);
#pragma unroll
          for (int q = 0; q < 4; ++q) rsp[u] = fmaf(pDS[u][q], pS[u][q], rsp[u]);
        }
      }
    }
    __syncthreads();
    {
      // aQ += dO S^T, aY += dR S^T, aK += R dS'^T over this slice (one K = 32
      // block): the wavefront's column block tn is the same for every u, so
      // its S and dS' fragments are read once; the three products run as
      // independent accumulator chains, interleaved
      const int tn = wv % TNK;
      const bf16x8 sh = frag_krow(bS, LH, 0, 16 * tn), sl2 = frag_krow(bS, LH, KC, 16 * tn);
      const bf16x8 dh = frag_krow(bDS, LH, 0, 16 * tn), dl = frag_krow(bDS, LH, KC, 16 * tn);
#pragma unroll
      for (int u = 0; u < NKT; ++u) {
        const int r0 = 16 * ((wv + NWV * u) / TNK);
        const bf16x8 oh = frag_krow(bO, LH, 0, r0), ol = frag_krow(bO, LH, KC, r0);
        const bf16x8 yh = frag_krow(bDR, LH, 0, r0), yl = frag_krow(bDR, LH, KC, r0);
        const bf16x8 rh = frag_krow(bR, LH, 0, r0), rl = frag_krow(bR, LH, KC, r0);
        aQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ol, sh, aQ[u], 0, 0, 0);
        aY[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yl, sh, aY[u], 0, 0, 0);
        aK[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rl, dh, aK[u], 0, 0, 0);
        aQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oh, sl2, aQ[u], 0, 0, 0);
        aY[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yh, sl2, aY[u], 0, 0, 0);
        aK[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh, dl, aK[u], 0, 0, 0);
        aQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oh, sh, aQ[u], 0, 0, 0);
        aY[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yh, sh, aY[u], 0, 0, 0);
        aK[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh, dh, aK[u], 0, 0, 0);
      }
    }
    // the next slice into the registers stored above, issued after the first
    // products so that they start at once
    if (sl + 1 < NS) slice_load(j0 + KC);
#pragma unroll
    for (int u = 0; u < NCT; ++u) {
      // aAQ += dO R^T (lower tiles) and aA += dR Z^T, interleaved likewise
      const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
      const bf16x8 yh = frag_krow(bDR, LH, 0, 16 * tm), yl = frag_krow(bDR, LH, KC, 16 * tm);
      const bf16x8 zh = frag_krow(bZ, LH, 0, 16 * tn), zl = frag_krow(bZ, LH, KC, 16 * tn);
      if (tn <= tm) {
        const bf16x8 oh = frag_krow(bO, LH, 0, 16 * tm), ol = frag_krow(bO, LH, KC, 16 * tm);
        const bf16x8 rh = frag_krow(bR, LH, 0, 16 * tn), rl = frag_krow(bR, LH, KC, 16 * tn);
        aAQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ol, rh, aAQ[u], 0, 0, 0);
        aA[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yl, zh, aA[u], 0, 0, 0);
        aAQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oh, rl, aAQ[u], 0, 0, 0);
        aA[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yh, zl, aA[u], 0, 0, 0);
        aAQ[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oh, rh, aAQ[u], 0, 0, 0);
        aA[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yh, zh, aA[u], 0, 0, 0);
      } else {
        aA[u] = mma3x(yh, yl, zh, zl, aA[u]);
      }
    }
    {  // dZ = A^T dR over this slice's 32 value channels: one [16][16] tile per wavefront
      const int tm = wv >> 1, tn = wv & 1;
      f32x4 z;
      if constexpr (SPLIT) z = at3x<LHA>(sA, sDRT, tm, tn);
      else z = mma_lds_f32<BC, true, false>(zero4(), sA + 16 * tm * LA + 16 * tm, LA,
                                            sDRT + 16 * tn * LA + 16 * tm, LA, BC - 16 * tm);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, c = 16 * tn + m;
        if (r < clen) {
          const size_t x = (size_t)(row0 + r) * vr + (size_t)h * DV + j0 + c;
          a.dv[x] = z[q] * sW[r * LS + c];
          a.dw[x] = z[q] * sV[r * LS + c];
        }
      }
    }
    __syncthreads();
  }

  // row sums of dS' * S: combine the 8 lanes of each row (sRS is read in the
  // final phase, after several barriers)
#pragma unroll
  for (int u = 0; u < NSK; ++u) {
    float x = rsp[u];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    const int e = tid + NT * u;
    if (e < DK * KC / 4 && (e & (KC / 4 - 1)) == 0) sm[C::O_RS + e / (KC / 4)] = x;
  }

  // ---- phase 2a: dA += dY E^T, X = A^T dY ----
  // G, k and b for E and E' (issued before dY goes to LDS)
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e / (DK / 4), i4 = e - s * (DK / 4);
    const int sr = s < clen ? s : clen - 1;
    const size_t x = (size_t)(row0 + sr) * kr + (size_t)h * DK + 4 * i4;
    const float z = s < clen ? 1.f : 0.f;
    float t[4];
    pG[u] = reinterpret_cast<const f32x4*>(W + L::G)[e];
    load4<BF16>(a.k, x, t);
    pK[u] = f32x4{t[0], t[1], t[2], t[3]} * z;
    load4<BF16>(a.b, x, t);
    pB[u] = f32x4{t[0], t[1], t[2], t[3]} * z;
  }
  float *sDY = sm + C::O_DY, *sEB = sm + C::O_EB, *sDYT = sm + C::O_DYT;
  // a strong chunk (flagged by the front pass) forms its decay-weighted
  // products exactly, with G in E''s place
  constexpr bool strong = SM == 1;
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q, i = 16 * tn + m;
      const float y = -aY[u][q];
      if constexpr (SPLIT) st_h(sDY, LHK, DK, r, i, y);
      else sDY[r * LKP + i] = y;
      if constexpr (SPLIT) st_h(sDYT, LHA, BC, i, r, y);
      else sDYT[i * LA + r] = y;
    }
  }
  // E = gamma b k and E' = e1 b k (the forms of the front pass, same order
  // of operations), e1 = exp(G - G_31)
  float* sEP = sm + C::O_EP;
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e / (DK / 4), i4 = e - s * (DK / 4), o = s * LKP + 4 * i4;
    f32x4 eb, ep;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float G = pG[u][c], gam = exp_dec(G), e1 = exp_dec(G - sm[C::O_G31 + 4 * i4 + c]);
      eb[c] = gam * pB[u][c] * pK[u][c];
      ep[c] = strong ? G : e1 * pB[u][c] * pK[u][c];
    }
    if constexpr (SPLIT) {
      st_h4(sEB, LHK, DK, s, 4 * i4, eb);
      st_h4(sEP, LHK, DK, s, 4 * i4, ep);
    } else {
      *reinterpret_cast<f32x4*>(sEB + o) = eb;
      *reinterpret_cast<f32x4*>(sEP + o) = ep;
    }
  }
  __syncthreads();
  f32x4 pQ[NEK];
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e / (DK / 4), i4 = e - s * (DK / 4);
    const int sr = s < clen ? s : clen - 1;
    float t[4];
    load4<BF16>(a.q, (size_t)(row0 + sr) * kr + (size_t)h * DK + 4 * i4, t);
    pQ[u] = f32x4{t[0], t[1], t[2], t[3]} * (s < clen ? 1.f : 0.f);
  }
  f32x4 aX[NKT];
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
    if constexpr (SPLIT) {
      const __bf16 *bY = reinterpret_cast<const __bf16*>(sDY), *bE = reinterpret_cast<const __bf16*>(sEB);
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += 32)
        aA[u] = mma3x(frag_krow(bY, LHK, k0, 16 * tm), frag_krow(bY, LHK, DK + k0, 16 * tm),
                      frag_krow(bE, LHK, k0, 16 * tn), frag_krow(bE, LHK, DK + k0, 16 * tn), aA[u]);
    } else {
      // a chain of its own, added to the bf16 chain of phase 1 (one MFMA shape per chain)
      aA[u] += mma_lds<float, DK>(zero4(), sDY + 16 * tm * LKP, LKP, sEB + 16 * tn * LKP, LKP);
    }
  }
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
    if constexpr (SPLIT) aX[u] = at3x<LHA>(sA, sDYT, tm, tn);
    else aX[u] = mma_lds_f32<BC, true, false>(zero4(), sA + 16 * tm * LA + 16 * tm, LA,
                                              sDYT + 16 * tn * LA + 16 * tm, LA, BC - 16 * tm);
  }
  __syncthreads();

  // ---- phase 2b: dA_qk^T Q' and dA_qk K' ----
  float *sKP = sm + C::O_KP, *sQP = sm + C::O_QP, *sAQ = sm + C::O_AQ, *sAQT = sm + C::O_AQT;
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q, c = 16 * tn + m;
      // strictly lower: the diagonal of dA_qk is kept apart (sDQK), so that
      // its two equal and opposite terms in dg never meet in a sum
      const float v = (tn <= tm && c < r) ? aAQ[u][q] : 0.f;
      if constexpr (SPLIT) {
        st_h(sAQ, LHA, BC, r, c, v);
        st_h(sAQT, LHA, BC, c, r, v);
      } else {
        sAQ[r * LA + c] = v;
        sAQT[c * LA + r] = v;
      }
      if (c == r) sm[C::O_DQK + r] = aAQ[u][q];
    }
  }
  // Q' = e1 q and K' = e2 k, e2 = exp(G_31 - G)
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e / (DK / 4), i4 = e - s * (DK / 4);
    f32x4 qp, kp;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float G = pG[u][c], G31 = sm[C::O_G31 + 4 * i4 + c];
      qp[c] = strong ? pQ[u][c] : exp_dec(G - G31) * pQ[u][c];
      kp[c] = strong ? pK[u][c] : exp_dec(G31 - G) * pK[u][c];
    }
    if constexpr (SPLIT) {
      st_h4(sQP, LHK, DK, s, 4 * i4, qp);
      st_h4(sKP, LHK, DK, s, 4 * i4, kp);
    } else {
      *reinterpret_cast<f32x4*>(sQP + s * LKP + 4 * i4) = qp;
      *reinterpret_cast<f32x4*>(sKP + s * LKP + 4 * i4) = kp;
    }
  }
  __syncthreads();
  f32x4 aP3[NKT], aP4[NKT];
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
    if constexpr (SPLIT) {
      aP3[u] = tri3x<LHA, LHK, true>(sAQT, sQP, tm, tn);
      aP4[u] = tri3x<LHA, LHK, false>(sAQ, sKP, tm, tn);
    } else {  // the strong launch: sEP holds G
      aP3[u] = decay_tri<LA, LKP, false>(sAQT, sQP, sEP, 16 * tm + 4 * g, 16 * tn + m, 16 * tm, BC);
      aP4[u] = decay_tri<LA, LKP, true>(sAQ, sKP, sEP, 16 * tm + 4 * g, 16 * tn + m, 0, 16 * (tm + 1));
    }
  }
  __syncthreads();

  // ---- phase 3: dT = -tril(A^T dA A^T, -1) ----
  float *sDAT = sm + C::O_DAT, *sWM = sm + C::O_WM;
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (SPLIT) st_h(sDAT, LHA, BC, 16 * tn + m, 16 * tm + 4 * g + q, aA[u][q]);
      else sDAT[(16 * tn + m) * LA + 16 * tm + 4 * g + q] = aA[u][q];
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
    f32x4 w4;
    if constexpr (SPLIT) w4 = at3x<LHA>(sA, sDAT, tm, tn);
    else w4 = mma_lds_f32<BC, true, false>(zero4(), sA + 16 * tm * LA + 16 * tm, LA,
                                           sDAT + 16 * tn * LA + 16 * tm, LA, BC - 16 * tm);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (SPLIT) st_h(sWM, LHA, BC, 16 * tm + 4 * g + q, 16 * tn + m, w4[q]);
      else sWM[(16 * tm + 4 * g + q) * LA + 16 * tn + m] = w4[q];
    }
  }
  __syncthreads();
  f32x4 aT[NCT];
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
    // A is unit lower triangular: column block tn of A^T has no rows past
    // 16 (tn + 1); tiles above the diagonal are masked out below
    if constexpr (SPLIT) {
      aT[u] = zero4();
      if (tn <= tm) {  // uniform
        const __bf16 *bw = reinterpret_cast<const __bf16*>(sWM), *ba = reinterpret_cast<const __bf16*>(sA);
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 32)
          if (k0 < 16 * (tn + 1))
            aT[u] = mma3x(frag_krow(bw, LHA, k0, 16 * tm), frag_krow(bw, LHA, BC + k0, 16 * tm),
                          frag_krow(ba, LHA, k0, 16 * tn), frag_krow(ba, LHA, BC + k0, 16 * tn), aT[u]);
      }
    } else {
      aT[u] = tn <= tm ? mma_lds_f32<BC, false, false>(zero4(), sWM + 16 * tm * LA, LA, sA + 16 * tn * LA, LA,
                                                     16 * (tn + 1))
                     : zero4();
    }
  }
  __syncthreads();

  // ---- phase 4: dT K' and dT^T E' ----
  float *sDT = sm + C::O_DT, *sDTT = sm + C::O_DTT;
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q, c = 16 * tn + m;
      const float v = c < r ? -aT[u][q] : 0.f;
      if constexpr (SPLIT) {
        st_h(sDT, LHA, BC, r, c, v);
        st_h(sDTT, LHA, BC, c, r, v);
      } else {
        sDT[r * LA + c] = v;
        sDTT[c * LA + r] = v;
      }
    }
  }
  __syncthreads();
  // the final's per-element inputs, loaded while phase 4 computes
  float fG[NKT][4], fq[NKT][4], fk[NKT][4], fb[NKT][4];
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK, i = 16 * tn + m;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q, rr = r < clen ? r : clen - 1;
      const size_t x = (size_t)(row0 + rr) * kr + (size_t)h * DK + i;
      fG[u][q] = W[L::G + r * DK + i];
      fq[u][q] = load1<BF16>(a.q, x);
      fk[u][q] = load1<BF16>(a.k, x);
      fb[u][q] = load1<BF16>(a.b, x);
    }
  }
  f32x4 aP1[NKT], aP2[NKT];
  if (strong) {
    // b k of the tile's own elements into its block behind dT and dT^T
    float* sBK = sm + C::O_BK;
#pragma unroll
    for (int u = 0; u < NKT; ++u) {
      const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK, i = 16 * tn + m;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q;
        sBK[r * LKP + i] = r < clen ? fb[u][q] * fk[u][q] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NKT; ++u) {
      const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
      aP1[u] = decay_tri<LA, LKP, true>(sDT, sKP, sEP, 16 * tm + 4 * g, 16 * tn + m, 0, 16 * (tm + 1));
      aP2[u] = decay_tri<LA, LKP, false>(sDTT, sBK, sEP, 16 * tm + 4 * g, 16 * tn + m, 16 * tm, BC);
    }
  } else {
#pragma unroll
    for (int u = 0; u < NKT; ++u) {
      const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
      aP1[u] = tri3x<LHA, LHK, false>(sDT, sKP, tm, tn);
      aP2[u] = tri3x<LHA, LHK, true>(sDTT, sEP, tm, tn);
    }
  }
  __syncthreads();

  // ---- final: dq, dk, db per element; dg by the reverse cumulative sum ----
  float *sU = sm + C::O_U, *sV2 = sm + C::O_V2, *sRS = sm + C::O_RS;
  float *sPU = sm + C::O_PU, *sPV = sm + C::O_PV;
  const float *sG31 = sm + C::O_G31, *sGCL = sm + C::O_GCL, *sGCX = sm + C::O_GCX;
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK, i = 16 * tn + m;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q;
      const bool in = r < clen;
      const float qv = in ? fq[u][q] : 0.f, kv = in ? fk[u][q] : 0.f, bv = in ? fb[u][q] : 0.f;
      const float G = fG[u][q], gam = exp_dec(G);
      // a strong chunk's products carry the whole decay already
      const float e1 = strong ? 1.f : exp_dec(G - sG31[i]), e2 = strong ? 1.f : exp_dec(sG31[i] - G);
      const float ktail = exp_dec(sGCL[i] - G);
      // off the diagonal of dA_qk, then its diagonal entry (decay 1)
      const float dqo = aQ[u][q] * gam + aP4[u][q] * e1;
      const float dkbo = (aP2[u][q] + aP3[u][q]) * e2;    // dK_bar / gamma
      const float dd = sm[C::O_DQK + r];
      const float deg = aX[u][q] * gam + aP1[u][q] * e1;  // dE * gamma
      const float dkt = aK[u][q];
      const float db = deg * kv;
      // the decay gradient of row r's own factors (the diagonal of A_qk has none)
      sU[r * LKP + i] = dqo * qv - dkbo * kv + db * bv;
      sV2[r * LKP + i] = dkt * (ktail * kv);  // dK_tail * K_tail
      if (in) {
        const size_t x = (size_t)(row0 + r) * kr + (size_t)h * DK + i;
        a.dq[x] = dqo + dd * kv;
        a.dk[x] = dkbo + dd * qv + deg * bv + dkt * ktail;
        a.db[x] = db;
      }
    }
  }
  __syncthreads();
  // The decay of row r enters the cumulative sums of rows r' >= r, gamma_C
  // (the last one) among them, and K_tail of row r' is gamma_C / gamma_r':
  //   dg_r = gamma_C * rowsum(dS' * S) + sum over r' < r of dK_tail * K_tail
  //          + sum over r' >= r of the rest.
  // Each sum runs over its own rows only, so no term is added and then taken
  // away again (under strong decay those terms dwarf dg itself).
  // Thread (row block rb, channel i): sums of its rows first, then its scans.
  constexpr int NRB = NT / DK, RPB = BC / NRB;
  const int i = tid % DK, rb = tid / DK;
  {
    float su = 0.f, sv = 0.f;
#pragma unroll
    for (int k = 0; k < RPB; ++k) {
      su += sU[(rb * RPB + k) * LKP + i];
      sv += sV2[(rb * RPB + k) * LKP + i];
    }
    sPU[rb * DK + i] = su;
    sPV[rb * DK + i] = sv;
  }
  __syncthreads();
  float base = sRS[i] * sGCX[i];
#pragma unroll
  for (int b = 0; b < NRB; ++b) {
    if (b < rb) base += sPV[b * DK + i];
    if (b > rb) base += sPU[b * DK + i];
  }
  {  // the K_tail prefix of each row, in place
    float pv = 0.f;
#pragma unroll
    for (int k = 0; k < RPB; ++k) {
      const int r = rb * RPB + k;
      const float x = sV2[r * LKP + i];
      sV2[r * LKP + i] = pv;
      pv += x;
    }
  }
  float su = 0.f;
#pragma unroll
  for (int k = RPB - 1; k >= 0; --k) {
    const int r = rb * RPB + k;
    su += sU[r * LKP + i];
    if (r < clen) a.dg[(size_t)(row0 + r) * kr + (size_t)h * DK + i] = base + sV2[r * LKP + i] + su;
  }
}

// The output pass: one workgroup per item, the flagged chunks left out.
template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(512) void bwd_out_kernel(BwdArgs a) {
  out_item<DK, DV, BF16, 0>(a, blockIdx.x);
}

// The flagged chunks of the output pass, one workgroup per item as in
// bwd_front_strong_kernel.
template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(512) void bwd_out_strong_kernel(BwdArgs a) {
  if (a.sflag[blockIdx.x] == 0) return;  // uniform
  out_item<DK, DV, BF16, 1>(a, blockIdx.x);
}

#define GDR2_CK(x)                       \
  do {                                   \
    const hipError_t e_ = (x);           \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

// Raises the dynamic LDS limit of a kernel once per device (race-free flags).
#define GDR2_LDS(kernel, bytes)                                                    \
  do {                                                                             \
    static std::atomic<bool> done_[64];                                            \
    GDR2_CK(lds_opt_in(reinterpret_cast<const void*>(&kernel), (bytes), done_));   \
  } while (0)

template <int DK, int DV, bool BF16, bool LA16, bool FWD>
hipError_t launch_front_t(const BwdArgs& a, dim3 gi, hipStream_t st) {
  typedef FrontCfg<DK, DV> FC;
  GDR2_LDS((bwd_front_kernel<DK, DV, BF16, LA16, FWD>), FC::BYTES);
  hipLaunchKernelGGL((bwd_front_kernel<DK, DV, BF16, LA16, FWD>), gi, dim3(FC::NT), FC::BYTES, st, a);
  GDR2_CK(hipGetLastError());
  GDR2_LDS((bwd_front_strong_kernel<DK, DV, BF16, LA16, FWD>), FC::BYTES);
  hipLaunchKernelGGL((bwd_front_strong_kernel<DK, DV, BF16, LA16, FWD>), gi, dim3(FC::NT), FC::BYTES, st, a);
  return hipGetLastError();
}

// The front pass, then its strong chunks.
template <int DK, int DV, bool FWD>
hipError_t launch_front(const BwdArgs& a, dim3 gi, hipStream_t st) {
  if (a.in_bf16)
    return a.la_bf16 ? launch_front_t<DK, DV, true, true, FWD>(a, gi, st)
                     : launch_front_t<DK, DV, true, false, FWD>(a, gi, st);
  return a.la_bf16 ? launch_front_t<DK, DV, false, true, FWD>(a, gi, st)
                   : launch_front_t<DK, DV, false, false, FWD>(a, gi, st);
}

// LDS of the sequential forward pass (FWD adds Q_g and A_qk)
template <int DK, bool FWD>
constexpr size_t state_fwd_lds() {
  constexpr int LK = DK + 4, LC = BC + 4, LV = DVB + 4;
  return (size_t)(DVB * LK + 2 * BC * LK + DVB * LC + BC * LV + DK + (FWD ? BC * LK + BC * LC : 0)) * 4;
}

template <int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  const int items = a.chunks * a.H;
  const dim3 gi(items > 0 ? items : 1);
  if (items > 0) GDR2_CK((launch_front<DK, DV, false>(a, gi, st)));  // decay, T, A_qk, A, Y and U
  // sequential passes (with no chunks they only pass dS_T through to dS0)
  {
    constexpr size_t lf = StateF3Cfg<DK>::BYTES;
    constexpr size_t lb = StateB3Cfg<DK>::BYTES;
    GDR2_LDS((bwd_state_fwd3_kernel<DK, DV>), lf);
    const dim3 gs((unsigned)(((size_t)a.N * a.H + 7) / 8 * 8 * (DV / DVB)));
    hipLaunchKernelGGL((bwd_state_fwd3_kernel<DK, DV>), gs, dim3(SNT), lf, st, a);
    GDR2_CK(hipGetLastError());
    if (a.in_bf16) {
      GDR2_LDS((bwd_state_bwd3_kernel<DK, DV, true>), lb);
      hipLaunchKernelGGL((bwd_state_bwd3_kernel<DK, DV, true>), gs, dim3(SNT), lb, st, a);
    } else {
      GDR2_LDS((bwd_state_bwd3_kernel<DK, DV, false>), lb);
      hipLaunchKernelGGL((bwd_state_bwd3_kernel<DK, DV, false>), gs, dim3(SNT), lb, st, a);
    }
    GDR2_CK(hipGetLastError());
  }
  if (items <= 0) return hipSuccess;
  // output paths, WY gradients and the gradients themselves, one workgroup per
  // item, then the strong chunks
  {
    typedef OutCfg<DK, DV> OC;
    if (a.in_bf16) {
      GDR2_LDS((bwd_out_kernel<DK, DV, true>), OC::BYTES);
      hipLaunchKernelGGL((bwd_out_kernel<DK, DV, true>), gi, dim3(OC::NT), OC::BYTES, st, a);
      GDR2_CK(hipGetLastError());
      GDR2_LDS((bwd_out_strong_kernel<DK, DV, true>), OC::BYTES);
      hipLaunchKernelGGL((bwd_out_strong_kernel<DK, DV, true>), gi, dim3(OC::NT), OC::BYTES, st,
                         a);
    } else {
      GDR2_LDS((bwd_out_kernel<DK, DV, false>), OC::BYTES);
      hipLaunchKernelGGL((bwd_out_kernel<DK, DV, false>), gi, dim3(OC::NT), OC::BYTES, st, a);
      GDR2_CK(hipGetLastError());
      GDR2_LDS((bwd_out_strong_kernel<DK, DV, false>), OC::BYTES);
      hipLaunchKernelGGL((bwd_out_strong_kernel<DK, DV, false>), gi, dim3(OC::NT), OC::BYTES, st,
                         a);
    }
  }
  return hipGetLastError();
}

// The fp32 forward: the front pass (decay, T, A_qk, A, Y, U per item) and the
// sequential pass that forms o and the final state.
template <int DK, int DV>
hipError_t launch_fwd32_t(const BwdArgs& a, hipStream_t st) {
  const int items = a.chunks * a.H;
  if (items > 0) GDR2_CK((launch_front<DK, DV, true>(a, dim3(items), st)));
  constexpr size_t lf = state_fwd_lds<DK, true>();
  static_assert(lf <= 160 * 1024, "LDS budget exceeded");
  GDR2_LDS((fwd32_state_kernel<DK, DV>), lf);
  const dim3 gs((unsigned)(((size_t)a.N * a.H + 7) / 8 * 8 * (DV / DVB)));
  hipLaunchKernelGGL((fwd32_state_kernel<DK, DV>), gs, dim3(SNT), lf, st, a);
  return hipGetLastError();
}

}  // namespace

size_t bwd_item_bytes(int dk, int dv) {
#define GDR2_BI(DK, DV) \
  if (dk == DK && dv == DV) return BwdLayout<DK, DV>::FLOATS * sizeof(float);
  GDR2_BI(32, 32) GDR2_BI(32, 64) GDR2_BI(32, 128)
  GDR2_BI(64, 32) GDR2_BI(64, 64) GDR2_BI(64, 128)
  GDR2_BI(128, 32) GDR2_BI(128, 64) GDR2_BI(128, 128)
#undef GDR2_BI
  return 0;
}

hipError_t launch_fwd32(const BwdArgs& a, int dk, int dv, hipStream_t st) {
#define GDR2_FW(DK, DV) \
  if (dk == DK && dv == DV) return launch_fwd32_t<DK, DV>(a, st);
  GDR2_FW(32, 32) GDR2_FW(32, 64) GDR2_FW(32, 128)
  GDR2_FW(64, 32) GDR2_FW(64, 64) GDR2_FW(64, 128)
  GDR2_FW(128, 32) GDR2_FW(128, 64) GDR2_FW(128, 128)
#undef GDR2_FW
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a, int dk, int dv, hipStream_t st) {
#define GDR2_BW(DK, DV) \
  if (dk == DK && dv == DV) return launch_bwd_t<DK, DV>(a, st);
  GDR2_BW(32, 32) GDR2_BW(32, 64) GDR2_BW(32, 128)
  GDR2_BW(64, 32) GDR2_BW(64, 64) GDR2_BW(64, 128)
  GDR2_BW(128, 32) GDR2_BW(128, 64) GDR2_BW(128, 128)
#undef GDR2_BW
  return hipErrorInvalidValue;
}

}  // namespace gdr2
