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
// Layout: every intermediate of an item is an fp32 row-major block inside the
// workspace (BwdLayout).  The work is a chain of kernels:
//   prep (elementwise) -> batched products T, A_qk -> forward substitution A
//   -> Y, U -> sequential state pass (saves the entry state of every chunk)
//   -> sequential reverse state-gradient pass (saves dS' and dR per chunk)
//   (the state pass also saves R = U - Y S, which it forms anyway)
//   -> one fused kernel per item for the output and WY paths and the
//   gradients themselves (bwd_out_kernel).
// Every product runs on fp32 MFMA (16x16x4) from LDS-staged operands.
#include <hip/hip_runtime.h>

#include <initializer_list>

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
  static constexpr size_t G = 0, QG = G + CK, KT = QG + CK, EB = KT + CK, EP = EB + CK,
                          KP = EP + CK, QP = KP + CK, Y_ = QP + CK;
  static constexpr size_t Z = Y_ + CK, U = Z + CV, DO = U + CV, DR = DO + CV, R = DR + CV;
  static constexpr size_t T = R + CV, A = T + CC, AQK = A + CC, DAQK = AQK + CC, DA = DAQK + CC,
                          WM = DA + CC, DT = WM + CC;
  static constexpr size_t S = DT + CC, DSP = S + KV;
  static constexpr size_t DQG = DSP + KV, DY = DQG + CK, DKT = DY + CK, X1 = DKT + CK,
                          P1 = X1 + CK, P2 = P1 + CK, P3 = P2 + CK, P4 = P3 + CK;
  static constexpr size_t DZ = P4 + CK, GC = DZ + CV;
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

// ---- prep: decay, the scaled key-side rows, Z and dO ---------------------------------
template <int DK, int DV, bool BF16, bool LA16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  const int item = blockIdx.x, ci = item / a.H, h = item - ci * a.H;
  long long row0;
  int clen;
  if (!bwd_locate(a, ci, row0, clen)) return;
  float* W = a.ws + (size_t)item * L::FLOATS;
  __shared__ float sG[BC][DK];
  __shared__ float sGm[DK], sGC[DK];
  const int tid = threadIdx.x;
  const size_t kr = (size_t)a.H * DK, vr = (size_t)a.H * DV;
  if (tid < DK) {
    // cumulative log-decay from the chunk start, fp32; rows past the end add 0
    float acc = 0.f;
    for (int r = 0; r < BC; ++r) {
      if (r < clen) acc += load1<LA16>(a.la, (size_t)(row0 + r) * kr + (size_t)h * DK + tid);
      sG[r][tid] = acc;
    }
    sGm[tid] = sG[31][tid];
    sGC[tid] = acc;
    W[L::GC + tid] = expf(acc);
  }
  __syncthreads();
  for (int e = tid; e < BC * DK; e += 256) {
    const int r = e / DK, i = e - r * DK;
    float qv = 0.f, kv = 0.f, bv = 0.f;
    if (r < clen) {
      const size_t x = (size_t)(row0 + r) * kr + (size_t)h * DK + i;
      qv = load1<BF16>(a.q, x);
      kv = load1<BF16>(a.k, x);
      bv = load1<BF16>(a.b, x);
    }
    const float G = sG[r][i], gam = expf(G), e1 = expf(G - sGm[i]), e2 = expf(sGm[i] - G);
    W[L::G + e] = G;
    W[L::QG + e] = gam * qv;
    W[L::KT + e] = expf(sGC[i] - G) * kv;
    W[L::EB + e] = gam * bv * kv;
    W[L::EP + e] = e1 * bv * kv;
    W[L::KP + e] = e2 * kv;
    W[L::QP + e] = e1 * qv;
  }
  for (int e = tid; e < BC * DV; e += 256) {
    const int r = e / DV, j = e - r * DV;
    float vv = 0.f, wv = 0.f, dov = 0.f;
    if (r < clen) {
      const size_t x = (size_t)(row0 + r) * vr + (size_t)h * DV + j;
      vv = load1<BF16>(a.v, x);
      wv = load1<BF16>(a.w, x);
      dov = load1<BF16>(a.dO, x);
    }
    W[L::Z + e] = wv * vv;
    W[L::DO + e] = dov;
  }
}

// ---- batched fp32 products over items -----------------------------------------------
// C[m][n] = alpha * sum_k opA(m, k) opB(k, n) (+ D[m][n]), entries with
// n > m + diag zeroed when `mask`.  opA(m, k) = A[k][m] when transposed, else
// A[m][k] (rows of lda floats); opB(k, n) = B[n][k] when transposed, else
// B[k][n].  Both operands are staged into LDS K-contiguous ([M][K] and [N][K]),
// K in slices of 32 with 16-byte loads (the item blocks, their offsets and the
// row strides are multiples of 4 floats), so several workgroups share a CU.
// Several independent products over the items in one launch (blockIdx.y
// selects the product; none reads another's output).  M is the chunk (64);
// N and K (multiples of 32) and the transposes come from the job table.
struct BmmJob {
  size_t oa, ob, oc;  // operand offsets inside an item's block (floats)
  long long od;       // addend offset, or -1
  int lda, ldb, ldc, N, K, ta, tb, mask, diag;
  float alpha;
};
constexpr int MAXJOBS = 6;
struct BmmJobs {
  BmmJob j[MAXJOBS];
  float* ws;
  size_t stride;
  int H;
  const int32_t* total;
};

__global__ __launch_bounds__(512) void bmm_multi_kernel(BmmJobs P) {
  constexpr int M = BC, KC = 32, LD = KC + 4, TM = M / 16, NMAX = 128, TPW = TM * (NMAX / 16) / 8;
  __shared__ __align__(16) float As[M * LD];
  __shared__ __align__(16) float Bs[NMAX * LD];
  const int item = blockIdx.x;
  if (P.total && item / P.H >= *P.total) return;
  const BmmJob& J = P.j[blockIdx.y];
  const int N = J.N, K = J.K, TN = N / 16;
  const size_t base = (size_t)item * P.stride;
  const float* A = P.ws + base + J.oa;
  const float* B = P.ws + base + J.ob;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  f32x4 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = zero4();
  for (int kc = 0; kc < K; kc += KC) {
    for (int e = tid; e < M * KC / 4; e += 512) {
      if (J.ta) {
        const int k = e / (M / 4), m4 = e - k * (M / 4);
        const f32x4 x = *reinterpret_cast<const f32x4*>(A + (size_t)(kc + k) * J.lda + 4 * m4);
        As[(4 * m4 + 0) * LD + k] = x[0];
        As[(4 * m4 + 1) * LD + k] = x[1];
        As[(4 * m4 + 2) * LD + k] = x[2];
        As[(4 * m4 + 3) * LD + k] = x[3];
      } else {
        const int mm = e / (KC / 4), k4 = e - mm * (KC / 4);
        *reinterpret_cast<f32x4*>(As + mm * LD + 4 * k4) =
            *reinterpret_cast<const f32x4*>(A + (size_t)mm * J.lda + kc + 4 * k4);
      }
    }
    for (int e = tid; e < N * KC / 4; e += 512) {
      if (J.tb) {
        const int n = e / (KC / 4), k4 = e - n * (KC / 4);
        *reinterpret_cast<f32x4*>(Bs + n * LD + 4 * k4) =
            *reinterpret_cast<const f32x4*>(B + (size_t)n * J.ldb + kc + 4 * k4);
      } else {
        const int k = e / (N / 4), n4 = e - k * (N / 4);
        const f32x4 x = *reinterpret_cast<const f32x4*>(B + (size_t)(kc + k) * J.ldb + 4 * n4);
        Bs[(4 * n4 + 0) * LD + k] = x[0];
        Bs[(4 * n4 + 1) * LD + k] = x[1];
        Bs[(4 * n4 + 2) * LD + k] = x[2];
        Bs[(4 * n4 + 3) * LD + k] = x[3];
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wv + 8 * u;
      if (t < TM * TN) {
        const int tm = t / TN, tn = t - tm * TN;
        acc[u] = mma_lds<float, KC>(acc[u], As + 16 * tm * LD, LD, Bs + 16 * tn * LD, LD);
      }
    }
    __syncthreads();
  }
  float* C = P.ws + base + J.oc;
  const float* D = J.od >= 0 ? P.ws + base + J.od : nullptr;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wv + 8 * u;
    if (t >= TM * TN) continue;
    const int tm = t / TN, tn = t - tm * TN;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * tm + 4 * g + q, col = 16 * tn + m;
      float v = J.alpha * acc[u][q];
      if (D) v += D[(size_t)row * J.ldc + col];
      if (J.mask && col > row + J.diag) v = 0.f;
      C[(size_t)row * J.ldc + col] = v;
    }
  }
}

// ---- A = (I + T)^-1 by forward substitution, fp32 --------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(64) void bwd_inverse_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  const int item = blockIdx.x;
  if (a.tab && item / a.H >= *a.total) return;
  float* W = a.ws + (size_t)item * L::FLOATS;
  __shared__ float sT[BC][BC + 1], sX[BC][BC + 1];
  const int j = threadIdx.x;  // column of A
  for (int r = 0; r < BC; ++r) sT[r][j] = W[L::T + r * BC + j];
  __syncthreads();
  for (int r = 0; r < BC; ++r) {
    float x = 0.f;
    if (r == j) {
      x = 1.f;
    } else if (r > j) {
      // four independent partial sums shorten the dependent FMA chain
      float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
      int s = j;
      for (; s + 3 < r; s += 4) {
        x0 = fmaf(-sT[r][s], sX[s][j], x0);
        x1 = fmaf(-sT[r][s + 1], sX[s + 1][j], x1);
        x2 = fmaf(-sT[r][s + 2], sX[s + 2][j], x2);
        x3 = fmaf(-sT[r][s + 3], sX[s + 3][j], x3);
      }
      for (; s < r; ++s) x0 = fmaf(-sT[r][s], sX[s][j], x0);
      x = (x0 + x1) + (x2 + x3);
    }
    sX[r][j] = x;
  }
  for (int r = 0; r < BC; ++r) W[L::A + r * BC + j] = sX[r][j];
}

// Register prefetch of one chunk's operands for the sequential passes.
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
    // K_tail is stored transposed: lane = token row, so that the transposing
    // LDS stores of a wavefront hit 64 consecutive words
    const int t = e4 % BC, i = 4 * (e4 / BC);
    rk[u] = *reinterpret_cast<const f32x4*>(Wn + L::KT + (size_t)t * DK + i);
  }
#pragma unroll
  for (int u = 0; u < NV4; ++u) {
    const int e4 = tid + SNT * u, r = e4 / (DVB / 4), c4 = e4 - r * (DVB / 4);
    ru[u] = *reinterpret_cast<const f32x4*>(Wn + L::U + (size_t)r * DV + jb * DVB + 4 * c4);
  }
  if (tid < DK / 4) rg = reinterpret_cast<const f32x4*>(Wn + L::GC)[tid];
}

template <int DK, int DV, int NK4, int NV4, int NC4>
__device__ __forceinline__ void sb_load(const BwdArgs& a, int ci, int h, int jb, int tid,
                                        f32x4 (&rq)[NK4], f32x4 (&rk)[NK4], f32x4 (&ry)[NK4],
                                        f32x4 (&ra)[NC4], f32x4 (&ro)[NV4], f32x4& rg) {
  typedef BwdLayout<DK, DV> L;
  const float* Wn = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
  // Q_g, Y, A_qk and dO are stored transposed: lane = token row, so that the
  // transposing LDS stores of a wavefront hit 64 consecutive words
#pragma unroll
  for (int u = 0; u < NK4; ++u) {
    const int e4 = tid + SNT * u, t = e4 % BC, i = 4 * (e4 / BC);
    rq[u] = *reinterpret_cast<const f32x4*>(Wn + L::QG + (size_t)t * DK + i);
    rk[u] = reinterpret_cast<const f32x4*>(Wn + L::KT)[e4];
    ry[u] = *reinterpret_cast<const f32x4*>(Wn + L::Y_ + (size_t)t * DK + i);
  }
#pragma unroll
  for (int u = 0; u < NC4; ++u) {
    const int e4 = tid + SNT * u, t = e4 % BC, r = 4 * (e4 / BC);
    ra[u] = *reinterpret_cast<const f32x4*>(Wn + L::AQK + (size_t)t * BC + r);
  }
#pragma unroll
  for (int u = 0; u < NV4; ++u) {
    const int e4 = tid + SNT * u, t = e4 % BC, j = 4 * (e4 / BC);
    ro[u] = *reinterpret_cast<const f32x4*>(Wn + L::DO + (size_t)t * DV + jb * DVB + j);
  }
  if (tid < DK / 4) rg = reinterpret_cast<const f32x4*>(Wn + L::GC)[tid];
}

// ---- sequential state pass: the state entering every chunk --------------------------
// One workgroup of SNT threads per (sequence, head, 32 value channels); the
// state block is
// kept transposed in LDS (S^T, the B operand of Y S).  The next chunk's
// operands are loaded into registers (16-byte loads) while the current chunk
// computes.
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
  float* sKtT = sY + BC * LK;                   // [DK][LC]
  float* sRT = sKtT + DK * LC;                  // [DVB][LC]
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
  f32x4 ry[NK4], rk[NK4], ru[NV4], rg = zero4();
  if (c0 < c1) sf_load<DK, DV, NK4, NV4>(a, c0, h, jb, tid, ry, rk, ru, rg);
  for (int ci = c0; ci < c1; ++ci) {
    float* W = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
#pragma unroll
    for (int u = 0; u < NK4; ++u) {
      const int e4 = tid + SNT * u, r = e4 / (DK / 4), i = 4 * (e4 - r * (DK / 4));
      *reinterpret_cast<f32x4*>(sY + r * LK + i) = ry[u];
      const int t = e4 % BC, it = 4 * (e4 / BC);  // K_tail: lane = token row (sf_load)
      sKtT[(it + 0) * LC + t] = rk[u][0];
      sKtT[(it + 1) * LC + t] = rk[u][1];
      sKtT[(it + 2) * LC + t] = rk[u][2];
      sKtT[(it + 3) * LC + t] = rk[u][3];
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
    // the next chunk (the last iteration reloads the current one: no branch)
    sf_load<DK, DV, NK4, NV4>(a, ci + 1 < c1 ? ci + 1 : ci, h, jb, tid, ry, rk, ru, rg);
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
      const f32x4 acc = mma_lds<float, BC>(zero4(), sKtT + 16 * tm * LC, LC, sRT + 16 * tn * LC, LC);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * tm + 4 * g + q, j = 16 * tn + m;
        sST[j * LK + i] = sGC[i] * sST[j * LK + i] + acc[q];
      }
    }
    __syncthreads();
  }
}

// ---- sequential reverse pass: dS' of every chunk, dR, and dS0 ------------------------
template <int DK, int DV>
__global__ __launch_bounds__(SNT, 1) void bwd_state_bwd_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  constexpr int NB = DV / DVB, LK = DK + 4, LC = BC + 4;
  constexpr int NK4 = BC * DK / 4 / SNT, NV4 = BC * DVB / 4 / SNT, NC4 = BC * BC / 4 / SNT;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sdST = reinterpret_cast<float*>(smem);  // [DVB][LK]  dS^T
  float* sAqkT = sdST + DVB * LK;                // [BC][LC]   A_qk^T
  float* sdOT = sAqkT + BC * LC;                 // [DVB][LC]  dO^T
  float* sKt = sdOT + DVB * LC;                  // [BC][LK]   K_tail
  float* sQgT = sKt + BC * LK;                   // [DK][LC]   Q_g^T
  float* sYT = sQgT + DK * LC;                   // [DK][LC]   Y^T
  float* sdRT = sYT + DK * LC;                   // [DVB][LC]  dR^T
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
  if (c0 < c1) sb_load<DK, DV, NK4, NV4, NC4>(a, c1 - 1, h, jb, tid, rq, rk, ry, ra, ro, rg);
  for (int ci = c1 - 1; ci >= c0; --ci) {
    float* W = a.ws + ((size_t)ci * a.H + h) * L::FLOATS;
#pragma unroll
    for (int u = 0; u < NK4; ++u) {
      const int e4 = tid + SNT * u;
      {
        const int t = e4 / (DK / 4), i = 4 * (e4 - t * (DK / 4));
        *reinterpret_cast<f32x4*>(sKt + t * LK + i) = rk[u];
      }
      const int t = e4 % BC, i = 4 * (e4 / BC);  // lane = token row (sb_load)
      sQgT[(i + 0) * LC + t] = rq[u][0];
      sQgT[(i + 1) * LC + t] = rq[u][1];
      sQgT[(i + 2) * LC + t] = rq[u][2];
      sQgT[(i + 3) * LC + t] = rq[u][3];
      sYT[(i + 0) * LC + t] = ry[u][0];
      sYT[(i + 1) * LC + t] = ry[u][1];
      sYT[(i + 2) * LC + t] = ry[u][2];
      sYT[(i + 3) * LC + t] = ry[u][3];
    }
#pragma unroll
    for (int u = 0; u < NC4; ++u) {  // A_qk[t][r..r+3] -> A_qk^T
      const int e4 = tid + SNT * u, t = e4 % BC, r = 4 * (e4 / BC);
      sAqkT[(r + 0) * LC + t] = ra[u][0];
      sAqkT[(r + 1) * LC + t] = ra[u][1];
      sAqkT[(r + 2) * LC + t] = ra[u][2];
      sAqkT[(r + 3) * LC + t] = ra[u][3];
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {  // dO[t][j..j+3] -> dO^T
      const int e4 = tid + SNT * u, t = e4 % BC, j = 4 * (e4 / BC);
      sdOT[(j + 0) * LC + t] = ro[u][0];
      sdOT[(j + 1) * LC + t] = ro[u][1];
      sdOT[(j + 2) * LC + t] = ro[u][2];
      sdOT[(j + 3) * LC + t] = ro[u][3];
    }
    if (tid < DK / 4) *reinterpret_cast<f32x4*>(sGC + 4 * tid) = rg;
    for (int e = tid; e < DK * DVB; e += SNT) {  // dL/d(state leaving chunk ci)
      const int i = e / DVB, j = e - i * DVB;
      W[L::DSP + (size_t)i * DV + jb * DVB + j] = sdST[j * LK + i];
    }
    __syncthreads();
    // the previous chunk (the last iteration reloads the current one: no branch)
    sb_load<DK, DV, NK4, NV4, NC4>(a, ci - 1 >= c0 ? ci - 1 : ci, h, jb, tid, rq, rk, ry, ra, ro, rg);
    // dR = A_qk^T dO + K_tail dS'  [BC][DVB]
    for (int t = wv; t < (BC / 16) * (DVB / 16); t += SNT / 64) {
      const int tm = t / (DVB / 16), tn = t - tm * (DVB / 16);
      f32x4 acc = mma_lds<float, BC>(zero4(), sAqkT + 16 * tm * LC, LC, sdOT + 16 * tn * LC, LC);
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
      const f32x4 acc = mma_lds<float, BC>(zero4(), sQgT + 16 * tm * LC, LC, sdOT + 16 * tn * LC, LC);
      const f32x4 acy = mma_lds<float, BC>(zero4(), sYT + 16 * tm * LC, LC, sdRT + 16 * tn * LC, LC);
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
// One workgroup per item forms, from the item's fp32 blocks (R, dR, A, E, Q',
// K', E', the decay G), the inputs (dO, v, w, q, k, b) and the states S and
// dS' on either side of the chunk, every remaining product and the gradients
// themselves:
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
// Every operand is staged K-contiguous in LDS (rows padded by 4 floats, so a
// 16-lane group's 16-byte reads hit distinct banks); the fp32 products run on
// 16x16x4 MFMA.  Tiles of a [64][N] result go round the eight wavefronts
// (tile t = wave + 8u, row tile t / (N/16), column tile t % (N/16)).  Each
// phase's global loads are issued into registers one phase (or one slice)
// ahead, so they overlap the products of the phase before.  Rows past the
// end of a sequence read a clamped (valid) row and are zeroed in registers.
template <int DK, int DV>
struct OutCfg {
  static constexpr int NT = 512, NWV = 8, KC = 32, LS = KC + 4, LA = BC + 4, LKP = DK + 4;
  static constexpr int NKT = DK / 32;  // [64][DK] tiles per wavefront
  static constexpr int NCT = 2;        // [64][64] tiles per wavefront
  // LDS offsets in floats.  A^T lives through phase 3; region R1 is reused.
  static constexpr int O_AT = 0, O_R1 = O_AT + BC * LA;
  // phase 1: slices of dO, dR, R, Z, w, v [64][KC], of S, dS' [DK][KC], dR^T [KC][64]
  static constexpr int O_O = O_R1, O_DR = O_O + BC * LS, O_R = O_DR + BC * LS,
                       O_Z = O_R + BC * LS, O_S = O_Z + BC * LS, O_DS = O_S + DK * LS,
                       O_DRT = O_DS + DK * LS, O_W = O_DRT + KC * LA, O_V = O_W + BC * LS,
                       E1 = O_V + BC * LS;
  // phase 2a: dY [64][DK], E [64][DK], dY^T [DK][64]
  static constexpr int O_DY = O_R1, O_EB = O_DY + BC * LKP, O_DYT = O_EB + BC * LKP,
                       E2 = O_DYT + DK * LA;
  // phases 2b-4: K'^T [DK][64] stays; the rest rotates behind it
  static constexpr int O_KPT = O_R1, O_X = O_KPT + DK * LA;
  static constexpr int O_QPT = O_X, O_AQ = O_QPT + DK * LA, O_AQT = O_AQ + BC * LA,
                       E3 = O_AQT + BC * LA;                                  // 2b
  static constexpr int O_DAT = O_X, O_WM = O_DAT + BC * LA, O_A = O_WM + BC * LA,
                       E4 = O_A + BC * LA;                                    // 3
  static constexpr int O_EPT = O_X, O_DT = O_EPT + DK * LA, O_DTT = O_DT + BC * LA,
                       E5 = O_DTT + BC * LA;                                  // 4
  // final: the per-element dg terms [64][DK] twice
  static constexpr int O_U = O_R1, O_V2 = O_U + BC * LKP, E6 = O_V2 + BC * LKP;
  static constexpr int mx(int x, int y) { return x > y ? x : y; }
  // per-channel values: G at row 31 and 63, gamma_C, the dS' * S row sums;
  // the dg scan's row-block partial sums
  static constexpr int O_G31 = mx(mx(mx(E1, E2), mx(E3, E4)), mx(E5, E6));
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
  float* sAT = sm + C::O_AT;
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
  // A^T (lane = row of A: consecutive lanes write consecutive words)
#pragma unroll
  for (int u = 0; u < NAA; ++u) {
    const int e = tid + NT * u, k = e % BC, c4 = e / BC;
    const f32x4 x = *reinterpret_cast<const f32x4*>(W + L::A + k * BC + 4 * c4);
#pragma unroll
    for (int q = 0; q < 4; ++q) sAT[(4 * c4 + q) * LA + k] = x[q];
  }
  if (tid < DK) {
    sm[C::O_G31 + tid] = W[L::G + 31 * DK + tid];
    sm[C::O_GCL + tid] = W[L::G + (BC - 1) * DK + tid];
    sm[C::O_GCX + tid] = W[L::GC + tid];
  }

  // ---- phase 1 ----
  f32x4 aQ[NKT], aY[NKT], aK[NKT], aAQ[NCT], aA[NCT], pEB[NEK];
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
    if (sl + 1 < NS) {
      slice_load(j0 + KC);
    } else {
#pragma unroll
      for (int u = 0; u < NEK; ++u) {
        const int e = tid + NT * u, s = e / (DK / 4), i4 = e - s * (DK / 4);
        pEB[u] = *reinterpret_cast<const f32x4*>(W + L::EB + s * DK + 4 * i4);
      }
    }
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
      const f32x4 z = mma_lds<float, BC>(zero4(), sAT + 16 * tm * LA, LA, sDRT + 16 * tn * LA, LA);
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
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e / (DK / 4), i4 = e - s * (DK / 4);
    *reinterpret_cast<f32x4*>(sEB + s * LKP + 4 * i4) = pEB[u];
  }
  __syncthreads();
  f32x4 pQP[NEK], pKP[NEK];  // lane = token row
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e % BC, i4 = e / BC;
    pQP[u] = *reinterpret_cast<const f32x4*>(W + L::QP + s * DK + 4 * i4);
    pKP[u] = *reinterpret_cast<const f32x4*>(W + L::KP + s * DK + 4 * i4);
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
    aX[u] = mma_lds<float, BC>(zero4(), sAT + 16 * tm * LA, LA, sDYT + 16 * tn * LA, LA);
  }
  __syncthreads();

  // ---- phase 2b: dA_qk^T Q' and dA_qk K' ----
  float *sKPT = sm + C::O_KPT, *sQPT = sm + C::O_QPT, *sAQ = sm + C::O_AQ, *sAQT = sm + C::O_AQT;
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
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e % BC, i4 = e / BC;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sQPT[(4 * i4 + q) * LA + s] = pQP[u][q];
      sKPT[(4 * i4 + q) * LA + s] = pKP[u][q];
    }
  }
  __syncthreads();
  f32x4 pA[NAA], pEP[NEK];
#pragma unroll
  for (int u = 0; u < NAA; ++u) {
    const int e = tid + NT * u, s = e / (BC / 4), c4 = e - s * (BC / 4);
    pA[u] = *reinterpret_cast<const f32x4*>(W + L::A + s * BC + 4 * c4);
  }
#pragma unroll
  for (int u = 0; u < NEK; ++u) {  // lane = token row
    const int e = tid + NT * u, s = e % BC, i4 = e / BC;
    pEP[u] = *reinterpret_cast<const f32x4*>(W + L::EP + s * DK + 4 * i4);
  }
  f32x4 aP3[NKT], aP4[NKT];
#pragma unroll
  for (int u = 0; u < NKT; ++u) {
    const int t = wv + NWV * u, tm = t / TNK, tn = t - tm * TNK;
    aP3[u] = mma_lds<float, BC>(zero4(), sAQT + 16 * tm * LA, LA, sQPT + 16 * tn * LA, LA);
    aP4[u] = mma_lds<float, BC>(zero4(), sAQ + 16 * tm * LA, LA, sKPT + 16 * tn * LA, LA);
  }
  __syncthreads();

  // ---- phase 3: dT = -tril(A^T dA A^T, -1) ----
  float *sDAT = sm + C::O_DAT, *sWM = sm + C::O_WM, *sA = sm + C::O_A;
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) sDAT[(16 * tn + m) * LA + 16 * tm + 4 * g + q] = aA[u][q];
  }
#pragma unroll
  for (int u = 0; u < NAA; ++u) {
    const int e = tid + NT * u, s = e / (BC / 4), c4 = e - s * (BC / 4);
    *reinterpret_cast<f32x4*>(sA + s * LA + 4 * c4) = pA[u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int t = wv + NWV * u, tm = t >> 2, tn = t & 3;
    const f32x4 w4 = mma_lds<float, BC>(zero4(), sAT + 16 * tm * LA, LA, sDAT + 16 * tn * LA, LA);
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
    aT[u] = tn <= tm ? mma_lds_k16<float, BC>(zero4(), sWM + 16 * tm * LA, LA, sA + 16 * tn * LA, LA,
                                              16 * (tn + 1))
                     : zero4();
  }
  __syncthreads();

  // ---- phase 4: dT K' and dT^T E' ----
  float *sEPT = sm + C::O_EPT, *sDT = sm + C::O_DT, *sDTT = sm + C::O_DTT;
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
#pragma unroll
  for (int u = 0; u < NEK; ++u) {
    const int e = tid + NT * u, s = e % BC, i4 = e / BC;
#pragma unroll
    for (int q = 0; q < 4; ++q) sEPT[(4 * i4 + q) * LA + s] = pEP[u][q];
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
    aP1[u] = mma_lds<float, BC>(zero4(), sDT + 16 * tm * LA, LA, sKPT + 16 * tn * LA, LA);
    aP2[u] = mma_lds<float, BC>(zero4(), sDTT + 16 * tm * LA, LA, sEPT + 16 * tn * LA, LA);
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

BmmJob job(size_t oa, int lda, bool ta, size_t ob, int ldb, bool tb, size_t oc, int ldc, int N, int K,
           float alpha = 1.f, long long od = -1, int mask = 0, int diag = 0) {
  BmmJob j;
  j.oa = oa; j.ob = ob; j.oc = oc; j.od = od;
  j.lda = lda; j.ldb = ldb; j.ldc = ldc; j.N = N; j.K = K;
  j.ta = ta; j.tb = tb; j.mask = mask; j.diag = diag;
  j.alpha = alpha;
  return j;
}

hipError_t bmm_group(const BwdArgs& a, size_t stride, int items, std::initializer_list<BmmJob> jobs,
                     hipStream_t st) {
  BmmJobs P{};
  int n = 0;
  for (const BmmJob& j : jobs) {
    if (n >= MAXJOBS || j.N % 32 || j.K % 32 || j.N > 128) return hipErrorInvalidValue;
    P.j[n++] = j;
  }
  P.ws = a.ws;
  P.stride = stride;
  P.H = a.H;
  P.total = a.tab ? a.total : nullptr;
  hipLaunchKernelGGL(bmm_multi_kernel, dim3(items, n), dim3(512), 0, st, P);
  return hipGetLastError();
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
  typedef BwdLayout<DK, DV> L;
  const int items = a.chunks * a.H;
  const size_t F = L::FLOATS;
  const dim3 gi(items > 0 ? items : 1);
  if (items > 0) {
  if (a.in_bf16) {
    if (a.la_bf16) hipLaunchKernelGGL((bwd_prep_kernel<DK, DV, true, true>), gi, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_prep_kernel<DK, DV, true, false>), gi, dim3(256), 0, st, a);
  } else {
    if (a.la_bf16) hipLaunchKernelGGL((bwd_prep_kernel<DK, DV, false, true>), gi, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_prep_kernel<DK, DV, false, false>), gi, dim3(256), 0, st, a);
  }
  GDR2_CK(hipGetLastError());
  // T = tril(E' K'^T, -1), A_qk = tril(Q' K'^T, 0)  (centred factors cancel)
  GDR2_CK(bmm_group(a, F, items, {job(L::EP, DK, 0, L::KP, DK, 1, L::T, BC, BC, DK, 1.f, -1, 1, -1),
                                  job(L::QP, DK, 0, L::KP, DK, 1, L::AQK, BC, BC, DK, 1.f, -1, 1, 0)}, st));
  hipLaunchKernelGGL((bwd_inverse_kernel<DK, DV>), gi, dim3(64), 0, st, a);
  GDR2_CK(hipGetLastError());
  // Y = A E, U = A Z
  GDR2_CK(bmm_group(a, F, items, {job(L::A, BC, 0, L::EB, DK, 0, L::Y_, DK, DK, BC),
                                  job(L::A, BC, 0, L::Z, DV, 0, L::U, DV, DV, BC)}, st));
  }
  // sequential passes (with no chunks they only pass dS_T through to dS0)
  {
    constexpr int LK = DK + 4, LC = BC + 4;
    constexpr int LV = DVB + 4;
    const size_t lf = (size_t)(DVB * LK + BC * LK + DK * LC + DVB * LC + BC * LV + DK) * 4;
    const size_t lb = (size_t)(DVB * LK + BC * LC + DVB * LC + BC * LK + 2 * DK * LC + DVB * LC + DK) * 4;
    static bool attr[64] = {};
    int dev = 0;
    GDR2_CK(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64 || !attr[dev]) {
      GDR2_CK(set_lds(&bwd_state_fwd_kernel<DK, DV>, lf));
      GDR2_CK(set_lds(&bwd_state_bwd_kernel<DK, DV>, lb));
      if (dev >= 0 && dev < 64) attr[dev] = true;
    }
    const dim3 gs((unsigned)(((size_t)a.N * a.H + 7) / 8 * 8 * (DV / DVB)));
    hipLaunchKernelGGL((bwd_state_fwd_kernel<DK, DV>), gs, dim3(SNT), lf, st, a);
    GDR2_CK(hipGetLastError());
    hipLaunchKernelGGL((bwd_state_bwd_kernel<DK, DV>), gs, dim3(SNT), lb, st, a);
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
