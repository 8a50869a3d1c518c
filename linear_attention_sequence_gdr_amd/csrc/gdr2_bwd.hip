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
//   bwd_state_fwd_kernel  per chain, chunks in order: S entering each chunk
//                         and R = U - Y S;
//   bwd_state_bwd_kernel  per chain, chunks in reverse: dS' and dR, and dS0;
//   bwd_out_kernel        per item: every output-path and WY-gradient product
//                         and the gradients themselves (E, E', K', Q' are
//                         formed again from G, q, k, b rather than stored).
// Every product runs on fp32 MFMA (16x16x4) from LDS-staged operands.
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
  static constexpr int O_EB = E2, O_Z = O_EB + BC * LKP, E3 = O_Z + BC * LZ;
  static constexpr int O_PS = E1 > E3 ? E1 : E3, FLOATS = O_PS + NT;
  static constexpr size_t BYTES = (size_t)FLOATS * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(DK % 32 == 0 && DV % 32 == 0 && NT % DK == 0, "front pass tiling");
};

template <int DK, int DV, bool BF16, bool LA16>
__global__ __launch_bounds__(512) void bwd_front_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  typedef FrontCfg<DK, DV> C;
  constexpr int NT = C::NT, NWV = 8, LA = C::LA, LKP = C::LKP, LM = C::LM;
  constexpr int NEK = BC * DK / 4 / NT;  // float4 of a [64][DK] block per thread
  constexpr int NEV = BC * DV / 4 / NT;  // float4 of a [64][DV] block per thread
  constexpr int NAA = BC * BC / 4 / NT;  // float4 of a [64][64] block per thread
  constexpr int TNK = DK / 16, NKT = DK / 32, TNV = DV / 16, NVT = DV / 32;
  constexpr int NRB = NT / DK, RPB = BC / NRB;
  const int item = blockIdx.x, ci = item / a.H, h = item - ci * a.H;
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
      W[L::G + r * DK + si] = G;
      if (r == BC - 1) W[L::GC + si] = expf(G);
    }
  }
  __syncthreads();

  // ---- phase 2 ----
  float *sEP = sm + C::O_EP, *sKP = sm + C::O_KP, *sQP = sm + C::O_QP;
  f32x4 pg[NEK];  // G of this thread's units, for E in phase 5
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, r = e / (DK / 4), i4 = e - r * (DK / 4), o = r * LKP + 4 * i4;
    f32x4 QG, KT, EP, KP, QP;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = 4 * i4 + c;
      const float G = sG[o + c], G31 = sG[31 * LKP + i], GCl = sG[(BC - 1) * LKP + i];
      const float gam = expf(G), e1 = expf(G - G31), e2 = expf(G31 - G);
      const float qv = pq[u][c], kv = pk[u][c], bv = pb[u][c];
      pg[u][c] = G;
      QG[c] = gam * qv;
      KT[c] = expf(GCl - G) * kv;
      EP[c] = e1 * bv * kv;
      KP[c] = e2 * kv;
      QP[c] = e1 * qv;
    }
    const int wo = r * DK + 4 * i4;
    *reinterpret_cast<f32x4*>(W + L::QG + wo) = QG;
    *reinterpret_cast<f32x4*>(W + L::KT + wo) = KT;
    *reinterpret_cast<f32x4*>(sEP + o) = EP;
    *reinterpret_cast<f32x4*>(sKP + o) = KP;
    *reinterpret_cast<f32x4*>(sQP + o) = QP;
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
  f32x4 aT[2], aQ[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
    if (tn <= tm) {
      aT[u] = mma_lds<float, DK>(zero4(), sEP + 16 * tm * LKP, LKP, sKP + 16 * tn * LKP, LKP);
      aQ[u] = mma_lds<float, DK>(zero4(), sQP + 16 * tm * LKP, LKP, sKP + 16 * tn * LKP, LKP);
    } else {
      aT[u] = aQ[u] = zero4();
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q, c = 16 * tn + m;
      W[L::AQK + r * BC + c] = c <= r ? aQ[u][q] : 0.f;
    }
  }
  __syncthreads();
  float *sT = sm + C::O_T, *sA = sm + C::O_A, *sAT = sm + C::O_AT;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q, c = 16 * tn + m;
      sT[r * LA + c] = c < r ? aT[u][q] : 0.f;
    }
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
#pragma unroll
  for (int u = 0; u < NAA; ++u) {
    const int e = tid + NT * u, s = e / (BC / 4), c4 = e - s * (BC / 4);
    *reinterpret_cast<f32x4*>(W + L::A + s * BC + 4 * c4) = *reinterpret_cast<const f32x4*>(sA + s * LA + 4 * c4);
  }
  // E = gamma * b * k from the registers of phase 1-2, and Z = w * v
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e / (DK / 4), i4 = e - s * (DK / 4);
    f32x4 eb;
#pragma unroll
    for (int c = 0; c < 4; ++c) eb[c] = expf(pg[u][c]) * pb[u][c] * pk[u][c];
    *reinterpret_cast<f32x4*>(sEB + s * LKP + 4 * i4) = eb;
  }
#pragma unroll
  for (int u = 0; u < NEV; ++u) {
    const int e = tid + NT * u, s = e / (DV / 4), j4 = e - s * (DV / 4);
    *reinterpret_cast<f32x4*>(sZ + s * C::LZ + 4 * j4) = pw[u] * pv[u];
  }
  __syncthreads();
  // A is lower triangular: row block tm needs the first 16 (tm + 1) columns only
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
    const f32x4 y = mma_lds_f32<BC, false, true>(zero4(), sA + 16 * tm * LA, LA, sEB + 16 * tn, LKP, 16 * (tm + 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) W[L::Y_ + (16 * tm + 4 * g + q) * DK + 16 * tn + m] = y[q];
  }
#pragma unroll
  for (int u = 0; u < NVT; ++u) {
    const int t = wv + NWV * u, tm = t / TNV, tn = t - tm * TNV;
    const f32x4 y = mma_lds_f32<BC, false, true>(zero4(), sA + 16 * tm * LA, LA, sZ + 16 * tn, C::LZ, 16 * (tm + 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) W[L::U + (16 * tm + 4 * g + q) * DV + 16 * tn + m] = y[q];
  }
}

// Register prefetch of one chunk's operands for the sequential passes
// (16-byte loads in address order, into row-major LDS blocks).
template <int DK, int DV, int NK4, int NV4>
__device__ __forceinline__ void sf_load(const BwdArgs& a, int ci, int h, int jb, int tid,
                                        f32x4 (&ry)[NK4], f32x4 (&rk)[NK4], f32x4 (&ru)[NV4],
                                        f32x4& rg) {
  typedef BwdLayout<DK, DV> L;
  const float* Wn = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
#pragma unroll
  for (int u = 0; u < NK4; ++u) {
    const int e4 = tid + SNT * u;
    ry[u] = reinterpret_cast<const f32x4*>(Wn + L::Y_)[e4];
    rk[u] = reinterpret_cast<const f32x4*>(Wn + L::KT)[e4];
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

// ---- sequential state pass: the state entering every chunk --------------------------
// One workgroup of SNT threads per (sequence, head, 32 value channels); the
// state block is kept transposed in LDS (S^T, the B operand of Y S).  The
// next two chunks' operands are loaded into registers (16-byte loads in
// address order) while the current chunk computes.
template <int DK, int DV>
__global__ __launch_bounds__(SNT, 1) void bwd_state_fwd_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  constexpr int NB = DV / DVB, LK = DK + 4, LC = BC + 4, LV = DVB + 4;
  constexpr int NK4 = BC * DK / 4 / SNT;   // float4 per thread of a [BC][DK] block
  constexpr int NV4 = BC * DVB / 4 / SNT;  // float4 per thread of a [BC][DVB] block
  static_assert(NK4 >= 1 && NV4 >= 1, "state pass tiling");
  extern __shared__ __align__(16) unsigned char smem[];
  float* sST = reinterpret_cast<float*>(smem);  // [DVB][LK]
  float* sY = sST + DVB * LK;                   // [BC][LK]
  float* sKt = sY + BC * LK;                    // [BC][LK]
  float* sRT = sKt + BC * LK;                   // [DVB][LC]
  float* sU = sRT + DVB * LC;                   // [BC][LV]
  float* sGC = sU + BC * LV;                    // [DK]
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
  f32x4 ry0[NK4], rk0[NK4], ru0[NV4], rg0 = zero4();
  f32x4 ry1[NK4], rk1[NK4], ru1[NV4], rg1 = zero4();
  if (c0 < c1) sf_load<DK, DV, NK4, NV4>(a, c0, h, jb, tid, ry0, rk0, ru0, rg0);
  if (c0 + 1 < c1) sf_load<DK, DV, NK4, NV4>(a, c0 + 1, h, jb, tid, ry1, rk1, ru1, rg1);
  auto step = [&](const int ci, f32x4 (&ry)[NK4], f32x4 (&rk)[NK4], f32x4 (&ru)[NV4], f32x4& rg) {
    float* W = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
#pragma unroll
    for (int u = 0; u < NK4; ++u) {
      const int e4 = tid + SNT * u, r = e4 / (DK / 4), i = 4 * (e4 - r * (DK / 4));
      *reinterpret_cast<f32x4*>(sY + r * LK + i) = ry[u];
      *reinterpret_cast<f32x4*>(sKt + r * LK + i) = rk[u];
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
    // the chunk after next into the registers just stored (near the end the
    // current chunk is reloaded instead: no branch)
    sf_load<DK, DV, NK4, NV4>(a, ci + 2 < c1 ? ci + 2 : ci, h, jb, tid, ry, rk, ru, rg);
    // R = U - Y S  [BC][DVB], kept for the output paths as well
    for (int t = wv; t < (BC / 16) * (DVB / 16); t += SNT / 64) {
      const int tm = t / (DVB / 16), tn = t - tm * (DVB / 16);
      const f32x4 acc = mma_lds<float, DK>(zero4(), sY + 16 * tm * LK, LK, sST + 16 * tn * LK, LK);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, j = 16 * tn + m;
        const float rv = sU[r * LV + j] - acc[q];
        sRT[j * LC + r] = rv;
        W[L::R + (size_t)r * DV + jb * DVB + j] = rv;
      }
    }
    __syncthreads();
    // S <- Diag(gamma_C) S + K_tail^T R  [DK][DVB]; each lane owns its entries
    for (int t = wv; t < (DK / 16) * (DVB / 16); t += SNT / 64) {
      const int tm = t / (DVB / 16), tn = t - tm * (DVB / 16);
      // K_tail^T as the left factor: K_tail read K-major from its row-major block
      const f32x4 acc = mma_lds_f32<BC, true, false>(zero4(), sKt + 16 * tm, LK, sRT + 16 * tn * LC, LC);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * tm + 4 * g + q, j = 16 * tn + m;
        sST[j * LK + i] = sGC[i] * sST[j * LK + i] + acc[q];
      }
    }
    __syncthreads();
  };
  int ci = c0;
  for (; ci + 1 < c1; ci += 2) {
    step(ci, ry0, rk0, ru0, rg0);
    step(ci + 1, ry1, rk1, ru1, rg1);
  }
  if (ci < c1) step(ci, ry0, rk0, ru0, rg0);
}

// ---- sequential reverse pass: dS' of every chunk, dR, and dS0 ------------------------
template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(SNT, 1) void bwd_state_bwd_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  constexpr int NB = DV / DVB, LK = DK + 4, LC = BC + 4;
  constexpr int NK4 = BC * DK / 4 / SNT, NV4 = BC * DVB / 4 / SNT, NC4 = BC * BC / 4 / SNT;
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int LV = DVB + 4;
  float* sdST = reinterpret_cast<float*>(smem);  // [DVB][LK]  dS^T
  float* sAqk = sdST + DVB * LK;                 // [BC][LC]   A_qk
  float* sdO = sAqk + BC * LC;                   // [BC][LV]   dO
  float* sKt = sdO + BC * LV;                    // [BC][LK]   K_tail
  float* sQg = sKt + BC * LK;                    // [BC][LK]   Q_g
  float* sY = sQg + BC * LK;                     // [BC][LK]   Y
  float* sdRT = sY + BC * LK;                    // [DVB][LC]  dR^T
  float* sGC = sdRT + DVB * LC;                  // [DK]
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
    sdST[j * LK + i] = a.dST ? a.dST[(size_t)nh * DK * DV + (size_t)i * DV + jb * DVB + j] : 0.f;
  }
  f32x4 rq[NK4], rk[NK4], ry[NK4], ra[NC4], ro[NV4], rg = zero4();
  if (c0 < c1) sb_load<DK, DV, NK4, NV4, NC4, BF16>(a, c1 - 1, h, jb, tid, rq, rk, ry, ra, ro, rg);
  for (int ci = c1 - 1; ci >= c0; --ci) {
    float* W = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
#pragma unroll
    for (int u = 0; u < NK4; ++u) {
      const int e4 = tid + SNT * u, t = e4 / (DK / 4), i = 4 * (e4 - t * (DK / 4));
      *reinterpret_cast<f32x4*>(sKt + t * LK + i) = rk[u];
      *reinterpret_cast<f32x4*>(sQg + t * LK + i) = rq[u];
      *reinterpret_cast<f32x4*>(sY + t * LK + i) = ry[u];
    }
#pragma unroll
    for (int u = 0; u < NC4; ++u) {
      const int e4 = tid + SNT * u, t = e4 / (BC / 4), r = 4 * (e4 - t * (BC / 4));
      *reinterpret_cast<f32x4*>(sAqk + t * LC + r) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
      const int e4 = tid + SNT * u, t = e4 / (DVB / 4), j = 4 * (e4 - t * (DVB / 4));
      *reinterpret_cast<f32x4*>(sdO + t * LV + j) = ro[u];
    }
    if (tid < DK / 4) *reinterpret_cast<f32x4*>(sGC + 4 * tid) = rg;
    for (int e = tid; e < DK * DVB; e += SNT) {  // dL/d(state leaving chunk ci)
      const int i = e / DVB, j = e - i * DVB;
      W[L::DSP + (size_t)i * DV + jb * DVB + j] = sdST[j * LK + i];
    }
    __syncthreads();
    // the previous chunk (the last iteration reloads the current one: no branch)
    sb_load<DK, DV, NK4, NV4, NC4, BF16>(a, ci - 1 >= c0 ? ci - 1 : ci, h, jb, tid, rq, rk, ry, ra, ro, rg);
    // dR = A_qk^T dO + K_tail dS'  [BC][DVB]
    for (int t = wv; t < (BC / 16) * (DVB / 16); t += SNT / 64) {
      const int tm = t / (DVB / 16), tn = t - tm * (DVB / 16);
      // A_qk^T and dO both read K-major from their row-major blocks
      f32x4 acc = mma_lds_f32<BC, true, true>(zero4(), sAqk + 16 * tm, LC, sdO + 16 * tn, LV);
      acc = mma_lds<float, DK>(acc, sKt + 16 * tm * LK, LK, sdST + 16 * tn * LK, LK);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, j = 16 * tn + m;
        W[L::DR + (size_t)r * DV + jb * DVB + j] = acc[q];
        sdRT[j * LC + r] = acc[q];
      }
    }
    __syncthreads();
    // dS <- Q_g^T dO + Diag(gamma_C) dS' - Y^T dR  [DK][DVB]; each lane owns its entries
    for (int t = wv; t < (DK / 16) * (DVB / 16); t += SNT / 64) {
      const int tm = t / (DVB / 16), tn = t - tm * (DVB / 16);
      const f32x4 acc = mma_lds_f32<BC, true, true>(zero4(), sQg + 16 * tm, LK, sdO + 16 * tn, LV);
      const f32x4 acy = mma_lds_f32<BC, true, false>(zero4(), sY + 16 * tm, LK, sdRT + 16 * tn * LC, LC);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * tm + 4 * g + q, j = 16 * tn + m;
        sdST[j * LK + i] = acc[q] + sGC[i] * sdST[j * LK + i] - acy[q];
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
  static constexpr int O_G31 = O_EP + BC * LKP;
  static constexpr int O_GCL = O_G31 + DK, O_GCX = O_GCL + DK, O_RS = O_GCX + DK,
                       O_PU = O_RS + DK, O_PV = O_PU + NT, FLOATS = O_PV + NT;
  static constexpr size_t BYTES = (size_t)FLOATS * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(DV % KC == 0 && DK % 32 == 0 && NT % DK == 0, "output pass tiling");
};

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(512) void bwd_out_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  typedef OutCfg<DK, DV> C;
  constexpr int NT = C::NT, NWV = C::NWV, KC = C::KC, LS = C::LS, LA = C::LA, LKP = C::LKP;
  constexpr int NKT = C::NKT, NCT = C::NCT, TNK = DK / 16;
  constexpr int NS = DV / KC;                         // value slices
  constexpr int NSK = (DK * KC / 4 + NT - 1) / NT;    // float4 of an S slice per thread
  constexpr int NEK = BC * DK / 4 / NT;               // float4 of a [64][DK] block per thread
  constexpr int NAA = BC * BC / 4 / NT;               // float4 of a [64][64] block per thread
  const int item = blockIdx.x, ci = item / a.H, h = item - ci * a.H;
  long long row0;
  int clen;
  if (!bwd_locate(a, ci, row0, clen) || clen <= 0) return;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* sm = reinterpret_cast<float*>(smem_raw);
  const float* W = a.ws + (size_t)item * L::FLOATS;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  const size_t kr = (size_t)a.H * DK, vr = (size_t)a.H * DV;
  float* sA = sm + C::O_A;
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
    *reinterpret_cast<f32x4*>(sA + s * LA + 4 * c4) = *reinterpret_cast<const f32x4*>(W + L::A + s * BC + 4 * c4);
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
  float rs = 0.f;  // sum over the value channels of dS' * S, row tid
  for (int sl = 0; sl < NS; ++sl) {
    const int j0 = sl * KC;
    {
      const int o = ss * LS + 4 * sc4;
      *reinterpret_cast<f32x4*>(sO + o) = pO;
      *reinterpret_cast<f32x4*>(sR + o) = pR;
      *reinterpret_cast<f32x4*>(sDR + o) = pDR;
      *reinterpret_cast<f32x4*>(sW + o) = pW;
      *reinterpret_cast<f32x4*>(sV + o) = pV;
      *reinterpret_cast<f32x4*>(sZ + o) = pW * pV;
#pragma unroll
      for (int q = 0; q < 4; ++q) sDRT[(4 * sc4 + q) * LA + ss] = pDR[q];
#pragma unroll
      for (int u = 0; u < NSK; ++u) {
        const int e = tid + NT * u;
        if (e < DK * KC / 4) {
          const int i = e / (KC / 4), c4 = e - i * (KC / 4);
          *reinterpret_cast<f32x4*>(sS + i * LS + 4 * c4) = pS[u];
          *reinterpret_cast<f32x4*>(sDS + i * LS + 4 * c4) = pDS[u];
        }
      }
    }
    __syncthreads();
    if (sl + 1 < NS) slice_load(j0 + KC);
    if (tid < DK)
#pragma unroll 8
      for (int c = 0; c < KC; ++c) rs = fmaf(sDS[tid * LS + c], sS[tid * LS + c], rs);
#pragma unroll
    for (int u = 0; u < NKT; ++u) {
      const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
      aQ[u] = mma_lds<float, KC>(aQ[u], sO + 16 * tm * LS, LS, sS + 16 * tn * LS, LS);
      aY[u] = mma_lds<float, KC>(aY[u], sDR + 16 * tm * LS, LS, sS + 16 * tn * LS, LS);
      aK[u] = mma_lds<float, KC>(aK[u], sR + 16 * tm * LS, LS, sDS + 16 * tn * LS, LS);
    }
#pragma unroll
    for (int u = 0; u < NCT; ++u) {
      const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
      if (tn <= tm) aAQ[u] = mma_lds<float, KC>(aAQ[u], sO + 16 * tm * LS, LS, sR + 16 * tn * LS, LS);
      aA[u] = mma_lds<float, KC>(aA[u], sDR + 16 * tm * LS, LS, sZ + 16 * tn * LS, LS);
    }
    {  // dZ = A^T dR over this slice's 32 value channels: one [16][16] tile per wavefront
      const int tm = wv >> 1, tn = wv & 1;
      const f32x4 z = mma_lds_f32<BC, true, false>(zero4(), sA + 16 * tm * LA + 16 * tm, LA,
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
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q, i = 16 * tn + m;
      const float y = -aY[u][q];
      sDY[r * LKP + i] = y;
      sDYT[i * LA + r] = y;
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
      const float G = pG[u][c], gam = expf(G), e1 = expf(G - sm[C::O_G31 + 4 * i4 + c]);
      eb[c] = gam * pB[u][c] * pK[u][c];
      ep[c] = e1 * pB[u][c] * pK[u][c];
    }
    *reinterpret_cast<f32x4*>(sEB + o) = eb;
    *reinterpret_cast<f32x4*>(sEP + o) = ep;
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
    aA[u] = mma_lds<float, DK>(aA[u], sDY + 16 * tm * LKP, LKP, sEB + 16 * tn * LKP, LKP);
  }
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
    aX[u] = mma_lds_f32<BC, true, false>(zero4(), sA + 16 * tm * LA + 16 * tm, LA,
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
      const float v = (tn <= tm && c <= r) ? aAQ[u][q] : 0.f;
      sAQ[r * LA + c] = v;
      sAQT[c * LA + r] = v;
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
      qp[c] = expf(G - G31) * pQ[u][c];
      kp[c] = expf(G31 - G) * pK[u][c];
    }
    *reinterpret_cast<f32x4*>(sQP + s * LKP + 4 * i4) = qp;
    *reinterpret_cast<f32x4*>(sKP + s * LKP + 4 * i4) = kp;
  }
  __syncthreads();
  f32x4 aP3[NKT], aP4[NKT];
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
    aP3[u] = mma_lds_f32<BC, false, true>(zero4(), sAQT + 16 * tm * LA + 16 * tm, LA,
                                          sQP + 16 * tm * LKP + 16 * tn, LKP, BC - 16 * tm);
    aP4[u] = mma_lds_f32<BC, false, true>(zero4(), sAQ + 16 * tm * LA, LA, sKP + 16 * tn, LKP, 16 * (tm + 1));
  }
  __syncthreads();

  // ---- phase 3: dT = -tril(A^T dA A^T, -1) ----
  float *sDAT = sm + C::O_DAT, *sWM = sm + C::O_WM;
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) sDAT[(16 * tn + m) * LA + 16 * tm + 4 * g + q] = aA[u][q];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
    const f32x4 w4 = mma_lds_f32<BC, true, false>(zero4(), sA + 16 * tm * LA + 16 * tm, LA,
                                                  sDAT + 16 * tn * LA + 16 * tm, LA, BC - 16 * tm);
#pragma unroll
    for (int q = 0; q < 4; ++q) sWM[(16 * tm + 4 * g + q) * LA + 16 * tn + m] = w4[q];
  }
  __syncthreads();
  f32x4 aT[NCT];
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
    // A is unit lower triangular: column block tn of A^T has no rows past
    // 16 (tn + 1); tiles above the diagonal are masked out below
    aT[u] = tn <= tm ? mma_lds_f32<BC, false, false>(zero4(), sWM + 16 * tm * LA, LA, sA + 16 * tn * LA, LA,
                                                     16 * (tn + 1))
                     : zero4();
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
      sDT[r * LA + c] = v;
      sDTT[c * LA + r] = v;
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
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
    aP1[u] = mma_lds_f32<BC, false, true>(zero4(), sDT + 16 * tm * LA, LA, sKP + 16 * tn, LKP, 16 * (tm + 1));
    aP2[u] = mma_lds_f32<BC, false, true>(zero4(), sDTT + 16 * tm * LA + 16 * tm, LA,
                                          sEP + 16 * tm * LKP + 16 * tn, LKP, BC - 16 * tm);
  }
  __syncthreads();

  // ---- final: dq, dk, db per element; dg by the reverse cumulative sum ----
  float *sU = sm + C::O_U, *sV2 = sm + C::O_V2, *sRS = sm + C::O_RS;
  float *sPU = sm + C::O_PU, *sPV = sm + C::O_PV;
  const float *sG31 = sm + C::O_G31, *sGCL = sm + C::O_GCL, *sGCX = sm + C::O_GCX;
  if (tid < DK) sRS[tid] = rs;
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK, i = 16 * tn + m;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * tm + 4 * g + q;
      const bool in = r < clen;
      const float qv = in ? fq[u][q] : 0.f, kv = in ? fk[u][q] : 0.f, bv = in ? fb[u][q] : 0.f;
      const float G = fG[u][q], gam = expf(G);
      const float e1 = expf(G - sG31[i]), e2 = expf(sG31[i] - G), ktail = expf(sGCL[i] - G);
      const float dq = aQ[u][q] * gam + aP4[u][q] * e1;
      const float dkbar = (aP2[u][q] + aP3[u][q]) * e2;   // dK_bar / gamma
      const float deg = aX[u][q] * gam + aP1[u][q] * e1;  // dE * gamma
      const float dkt = aK[u][q];
      const float db = deg * kv;
      sU[r * LKP + i] = dq * qv - dkbar * kv + db * bv - dkt * (ktail * kv);
      sV2[r * LKP + i] = dkt * (ktail * kv);  // dK_tail * K_tail
      if (in) {
        const size_t x = (size_t)(row0 + r) * kr + (size_t)h * DK + i;
        a.dq[x] = dq;
        a.dk[x] = dkbar + deg * bv + dkt * ktail;
        a.db[x] = db;
      }
    }
  }
  __syncthreads();
  // dg_r = gamma_C * rowsum(dS' * S) + sum over all rows of dK_tail * K_tail
  //        + sum over rows r' >= r of the rest (the decay of row r enters every
  //        later cumulative sum of the chunk, and gamma_C is the last one).
  // Thread (row block rb, channel i): sums of its rows first, then its scan.
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
  float acc = sRS[i] * sGCX[i];
#pragma unroll
  for (int b = 0; b < NRB; ++b) acc += sPV[b * DK + i];
#pragma unroll
  for (int b = NRB - 1; b > 0; --b)
    if (b > rb) acc += sPU[b * DK + i];
#pragma unroll
  for (int k = RPB - 1; k >= 0; --k) {
    const int r = rb * RPB + k;
    acc += sU[r * LKP + i];
    if (r < clen) a.dg[(size_t)(row0 + r) * kr + (size_t)h * DK + i] = acc;
  }
}

template <typename Kern>
hipError_t set_lds(Kern k, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

#define GDR2_CK(x)                       \
  do {                                   \
    const hipError_t e_ = (x);           \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

template <int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  const int items = a.chunks * a.H;
  const dim3 gi(items > 0 ? items : 1);
  if (items > 0) {  // decay, scaled rows, T, A_qk, A, Y and U
    typedef FrontCfg<DK, DV> FC;
    static bool attr[64] = {};
    int dev = 0;
    GDR2_CK(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64 || !attr[dev]) {
      GDR2_CK(set_lds(&bwd_front_kernel<DK, DV, true, true>, FC::BYTES));
      GDR2_CK(set_lds(&bwd_front_kernel<DK, DV, true, false>, FC::BYTES));
      GDR2_CK(set_lds(&bwd_front_kernel<DK, DV, false, true>, FC::BYTES));
      GDR2_CK(set_lds(&bwd_front_kernel<DK, DV, false, false>, FC::BYTES));
      if (dev >= 0 && dev < 64) attr[dev] = true;
    }
    if (a.in_bf16) {
      if (a.la_bf16) hipLaunchKernelGGL((bwd_front_kernel<DK, DV, true, true>), gi, dim3(FC::NT), FC::BYTES, st, a);
      else hipLaunchKernelGGL((bwd_front_kernel<DK, DV, true, false>), gi, dim3(FC::NT), FC::BYTES, st, a);
    } else {
      if (a.la_bf16) hipLaunchKernelGGL((bwd_front_kernel<DK, DV, false, true>), gi, dim3(FC::NT), FC::BYTES, st, a);
      else hipLaunchKernelGGL((bwd_front_kernel<DK, DV, false, false>), gi, dim3(FC::NT), FC::BYTES, st, a);
    }
    GDR2_CK(hipGetLastError());
  }
  // sequential passes (with no chunks they only pass dS_T through to dS0)
  {
    constexpr int LK = DK + 4, LC = BC + 4;
    constexpr int LV = DVB + 4;
    const size_t lf = (size_t)(DVB * LK + 2 * BC * LK + DVB * LC + BC * LV + DK) * 4;
    const size_t lb = (size_t)(DVB * LK + BC * LC + BC * (DVB + 4) + 3 * BC * LK + DVB * LC + DK) * 4;
    static bool attr[64] = {};
    int dev = 0;
    GDR2_CK(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64 || !attr[dev]) {
      GDR2_CK(set_lds(&bwd_state_fwd_kernel<DK, DV>, lf));
      GDR2_CK(set_lds(&bwd_state_bwd_kernel<DK, DV, true>, lb));
      GDR2_CK(set_lds(&bwd_state_bwd_kernel<DK, DV, false>, lb));
      if (dev >= 0 && dev < 64) attr[dev] = true;
    }
    const dim3 gs((unsigned)(((size_t)a.N * a.H + 7) / 8 * 8 * (DV / DVB)));
    hipLaunchKernelGGL((bwd_state_fwd_kernel<DK, DV>), gs, dim3(SNT), lf, st, a);
    GDR2_CK(hipGetLastError());
    if (a.in_bf16) hipLaunchKernelGGL((bwd_state_bwd_kernel<DK, DV, true>), gs, dim3(SNT), lb, st, a);
    else hipLaunchKernelGGL((bwd_state_bwd_kernel<DK, DV, false>), gs, dim3(SNT), lb, st, a);
    GDR2_CK(hipGetLastError());
  }
  if (items <= 0) return hipSuccess;
  // output paths, WY gradients and the gradients themselves, one workgroup per item
  {
    typedef OutCfg<DK, DV> OC;
    static bool attr[64] = {};
    int dev = 0;
    GDR2_CK(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64 || !attr[dev]) {
      GDR2_CK(set_lds(&bwd_out_kernel<DK, DV, true>, OC::BYTES));
      GDR2_CK(set_lds(&bwd_out_kernel<DK, DV, false>, OC::BYTES));
      if (dev >= 0 && dev < 64) attr[dev] = true;
    }
    if (a.in_bf16) hipLaunchKernelGGL((bwd_out_kernel<DK, DV, true>), gi, dim3(OC::NT), OC::BYTES, st, a);
    else hipLaunchKernelGGL((bwd_out_kernel<DK, DV, false>), gi, dim3(OC::NT), OC::BYTES, st, a);
  }
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
