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
// workspace (BwdLayout).  The work is a chain of simple kernels:
//   prep (elementwise) -> batched products T, A_qk -> forward substitution A
//   -> Y, U -> sequential state pass (saves the entry state of every chunk)
//   -> sequential reverse state-gradient pass (saves dS' and dR per chunk)
//   -> batched products of the output and WY paths -> final elementwise pass.
// The batched products run on fp32 MFMA (16x16x4) from LDS-staged operands.
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
// n > m + diag zeroed when `mask`.  opA(m, k) = TA ? A[k][m] : A[m][k] (rows of
// lda floats); opB(k, n) = TB ? B[n][k] : B[k][n] (rows of ldb floats).  Both
// operands are staged into LDS K-contiguous ([M][K] and [N][K]).
struct BmmArgs {
  const float* A;
  const float* B;
  float* C;
  const float* D;
  size_t stride;  // floats between consecutive items (all operands)
  int lda, ldb, ldc;
  float alpha;
  int mask, diag;
  int H;
  const int32_t* total;  // packed sequences: valid chunks; else nullptr
};

template <int M, int N, int K, bool TA, bool TB>
__global__ __launch_bounds__(512) void bmm_kernel(BmmArgs p) {
  // K is staged in slices of KC so that several workgroups fit on a CU; every
  // global access is a 16-byte load (the item blocks, their offsets and the
  // row strides are multiples of 4 floats)
  constexpr int KC = 32, LD = KC + 4;
  constexpr int TM = M / 16, TN = N / 16, TPW = (TM * TN + 7) / 8;
  __shared__ __align__(16) float As[M * LD];
  __shared__ __align__(16) float Bs[N * LD];
  const int item = blockIdx.x;
  if (p.total && item / p.H >= *p.total) return;
  const size_t base = (size_t)item * p.stride;
  const float* A = p.A + base;
  const float* B = p.B + base;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
  f32x4 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = zero4();
  for (int kc = 0; kc < K; kc += KC) {
    for (int e = tid; e < M * KC / 4; e += 512) {
      if constexpr (TA) {  // As[m][k] = A[k][m]: 4 consecutive m per load
        const int k = e / (M / 4), m4 = e - k * (M / 4);
        const float4 x = *reinterpret_cast<const float4*>(A + (size_t)(kc + k) * p.lda + 4 * m4);
        As[(4 * m4 + 0) * LD + k] = x.x;
        As[(4 * m4 + 1) * LD + k] = x.y;
        As[(4 * m4 + 2) * LD + k] = x.z;
        As[(4 * m4 + 3) * LD + k] = x.w;
      } else {
        const int mm = e / (KC / 4), k4 = e - mm * (KC / 4);
        *reinterpret_cast<float4*>(As + mm * LD + 4 * k4) =
            *reinterpret_cast<const float4*>(A + (size_t)mm * p.lda + kc + 4 * k4);
      }
    }
    for (int e = tid; e < N * KC / 4; e += 512) {
      if constexpr (TB) {
        const int n = e / (KC / 4), k4 = e - n * (KC / 4);
        *reinterpret_cast<float4*>(Bs + n * LD + 4 * k4) =
            *reinterpret_cast<const float4*>(B + (size_t)n * p.ldb + kc + 4 * k4);
      } else {  // Bs[n][k] = B[k][n]: 4 consecutive n per load
        const int k = e / (N / 4), n4 = e - k * (N / 4);
        const float4 x = *reinterpret_cast<const float4*>(B + (size_t)(kc + k) * p.ldb + 4 * n4);
        Bs[(4 * n4 + 0) * LD + k] = x.x;
        Bs[(4 * n4 + 1) * LD + k] = x.y;
        Bs[(4 * n4 + 2) * LD + k] = x.z;
        Bs[(4 * n4 + 3) * LD + k] = x.w;
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
  float* C = p.C + base;
  const float* D = p.D ? p.D + base : nullptr;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wv + 8 * u;
    if (t >= TM * TN) continue;
    const int tm = t / TN, tn = t - tm * TN;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * tm + 4 * g + q, col = 16 * tn + m;
      float v = p.alpha * acc[u][q];
      if (D) v += D[(size_t)row * p.ldc + col];
      if (p.mask && col > row + p.diag) v = 0.f;
      C[(size_t)row * p.ldc + col] = v;
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
      for (int s = j; s < r; ++s) x = fmaf(-sT[r][s], sX[s][j], x);
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
    rk[u] = reinterpret_cast<const f32x4*>(Wn + L::KT)[e4];
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
#pragma unroll
  for (int u = 0; u < NK4; ++u) {
    const int e4 = tid + SNT * u;
    rq[u] = reinterpret_cast<const f32x4*>(Wn + L::QG)[e4];
    rk[u] = reinterpret_cast<const f32x4*>(Wn + L::KT)[e4];
    ry[u] = reinterpret_cast<const f32x4*>(Wn + L::Y_)[e4];
  }
#pragma unroll
  for (int u = 0; u < NC4; ++u) ra[u] = reinterpret_cast<const f32x4*>(Wn + L::AQK)[tid + SNT * u];
#pragma unroll
  for (int u = 0; u < NV4; ++u) {
    const int e4 = tid + SNT * u, t = e4 / (DVB / 4), c4 = e4 - t * (DVB / 4);
    ro[u] = *reinterpret_cast<const f32x4*>(Wn + L::DO + (size_t)t * DV + jb * DVB + 4 * c4);
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
  const int jb = blockIdx.x % NB, nh = blockIdx.x / NB, n = nh / a.H, h = nh - n * a.H;
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
      sKtT[(i + 0) * LC + r] = rk[u][0];
      sKtT[(i + 1) * LC + r] = rk[u][1];
      sKtT[(i + 2) * LC + r] = rk[u][2];
      sKtT[(i + 3) * LC + r] = rk[u][3];
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
    // R = U - Y S  [BC][DVB]
    for (int t = wv; t < (BC / 16) * (DVB / 16); t += SNT / 64) {
      const int tm = t / (DVB / 16), tn = t - tm * (DVB / 16);
      const f32x4 acc = mma_lds<float, DK>(zero4(), sY + 16 * tm * LK, LK, sST + 16 * tn * LK, LK);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tm + 4 * g + q, j = 16 * tn + m;
        sRT[j * LC + r] = sU[r * LV + j] - acc[q];
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
  const int jb = blockIdx.x % NB, nh = blockIdx.x / NB, n = nh / a.H, h = nh - n * a.H;
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
      const int e4 = tid + SNT * u, t = e4 / (DK / 4), i = 4 * (e4 - t * (DK / 4));
      *reinterpret_cast<f32x4*>(sKt + t * LK + i) = rk[u];
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
      const int e4 = tid + SNT * u, t = e4 / (BC / 4), r = 4 * (e4 - t * (BC / 4));
      sAqkT[(r + 0) * LC + t] = ra[u][0];
      sAqkT[(r + 1) * LC + t] = ra[u][1];
      sAqkT[(r + 2) * LC + t] = ra[u][2];
      sAqkT[(r + 3) * LC + t] = ra[u][3];
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {  // dO[t][j..j+3] -> dO^T
      const int e4 = tid + SNT * u, t = e4 / (DVB / 4), j = 4 * (e4 - t * (DVB / 4));
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

// ---- final elementwise pass: dq, dk, db, dv, dw and the reverse cumsum for dg -------
template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(256) void bwd_final_kernel(BwdArgs a) {
  typedef BwdLayout<DK, DV> L;
  const int item = blockIdx.x, ci = item / a.H, h = item - ci * a.H;
  long long row0;
  int clen;
  if (!bwd_locate(a, ci, row0, clen)) return;
  const float* W = a.ws + (size_t)item * L::FLOATS;
  __shared__ float sdG[BC][DK];
  __shared__ float sGm[DK], sGC[DK];
  const int tid = threadIdx.x;
  const size_t kr = (size_t)a.H * DK, vr = (size_t)a.H * DV;
  if (tid < DK) {
    sGm[tid] = W[L::G + 31 * DK + tid];
    sGC[tid] = W[L::G + 63 * DK + tid];
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
    const float G = W[L::G + e], gam = expf(G);
    const float e1 = expf(G - sGm[i]), e2 = expf(sGm[i] - G), ktail = expf(sGC[i] - G);
    const float dq = W[L::DQG + e] * gam + W[L::P4 + e] * e1;
    const float dkbar = (W[L::P2 + e] + W[L::P3 + e]) * e2;   // dK_bar / gamma
    const float deg = W[L::X1 + e] * gam + W[L::P1 + e] * e1;  // dE * gamma
    const float dkt = W[L::DKT + e];
    const float dk = dkbar + deg * bv + dkt * ktail;
    const float db = deg * kv;
    sdG[r][i] = dq * qv - dkbar * kv + db * bv - dkt * (ktail * kv);
    if (r < clen) {
      const size_t x = (size_t)(row0 + r) * kr + (size_t)h * DK + i;
      a.dq[x] = dq;
      a.dk[x] = dk;
      a.db[x] = db;
    }
  }
  for (int e = tid; e < BC * DV; e += 256) {
    const int r = e / DV, j = e - r * DV;
    if (r < clen) {
      const size_t x = (size_t)(row0 + r) * vr + (size_t)h * DV + j;
      const float dz = W[L::DZ + e];
      a.dv[x] = dz * load1<BF16>(a.w, x);
      a.dw[x] = dz * load1<BF16>(a.v, x);
    }
  }
  __syncthreads();
  if (tid < DK) {
    // gamma_C enters the state update (Diag(gamma_C) S) and every K_tail row
    float acc = 0.f;
    for (int j = 0; j < DV; ++j) acc = fmaf(W[L::DSP + (size_t)tid * DV + j], W[L::S + (size_t)tid * DV + j], acc);
    acc *= W[L::GC + tid];
    for (int r = 0; r < BC; ++r) acc = fmaf(W[L::DKT + r * DK + tid], W[L::KT + r * DK + tid], acc);
    // dg_r = sum over rows r' >= r of dG (the decay of row r enters every
    // later cumulative sum of the chunk, and gamma_C is the last one)
    for (int r = BC - 1; r >= 0; --r) {
      acc += sdG[r][tid];
      if (r < clen) a.dg[(size_t)(row0 + r) * kr + (size_t)h * DK + tid] = acc;
    }
  }
}

template <int M, int N, int K, bool TA, bool TB>
hipError_t bmm(const BwdArgs& a, size_t stride, size_t oa, int lda, size_t ob, int ldb, size_t oc,
               int ldc, float alpha, long long od, int mask, int diag, int items, hipStream_t st) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 32 == 0, "bmm tile shapes");
  BmmArgs p;
  p.A = a.ws + oa;
  p.B = a.ws + ob;
  p.C = a.ws + oc;
  p.D = od >= 0 ? a.ws + od : nullptr;
  p.stride = stride;
  p.lda = lda; p.ldb = ldb; p.ldc = ldc;
  p.alpha = alpha;
  p.mask = mask; p.diag = diag;
  p.H = a.H;
  p.total = a.tab ? a.total : nullptr;
  hipLaunchKernelGGL((bmm_kernel<M, N, K, TA, TB>), dim3(items), dim3(512), 0, st, p);
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
  GDR2_CK((bmm<BC, BC, DK, false, true>(a, F, L::EP, DK, L::KP, DK, L::T, BC, 1.f, -1, 1, -1, items, st)));
  GDR2_CK((bmm<BC, BC, DK, false, true>(a, F, L::QP, DK, L::KP, DK, L::AQK, BC, 1.f, -1, 1, 0, items, st)));
  hipLaunchKernelGGL((bwd_inverse_kernel<DK, DV>), gi, dim3(64), 0, st, a);
  GDR2_CK(hipGetLastError());
  // Y = A E, U = A Z
  GDR2_CK((bmm<BC, DK, BC, false, false>(a, F, L::A, BC, L::EB, DK, L::Y_, DK, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DV, BC, false, false>(a, F, L::A, BC, L::Z, DV, L::U, DV, 1.f, -1, 0, 0, items, st)));
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
    const dim3 gs((unsigned)((size_t)a.N * a.H * (DV / DVB)));
    hipLaunchKernelGGL((bwd_state_fwd_kernel<DK, DV>), gs, dim3(SNT), lf, st, a);
    GDR2_CK(hipGetLastError());
    hipLaunchKernelGGL((bwd_state_bwd_kernel<DK, DV>), gs, dim3(SNT), lb, st, a);
    GDR2_CK(hipGetLastError());
  }
  if (items <= 0) return hipSuccess;
  // output paths
  GDR2_CK((bmm<BC, DV, DK, false, false>(a, F, L::Y_, DK, L::S, DV, L::R, DV, -1.f, (long long)L::U, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DK, DV, false, true>(a, F, L::DO, DV, L::S, DV, L::DQG, DK, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DK, DV, false, true>(a, F, L::DR, DV, L::S, DV, L::DY, DK, -1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DK, DV, false, true>(a, F, L::R, DV, L::DSP, DV, L::DKT, DK, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, BC, DV, false, true>(a, F, L::DO, DV, L::R, DV, L::DAQK, BC, 1.f, -1, 1, 0, items, st)));
  // gate-aware WY inverse path (Eqs. 64-65)
  GDR2_CK((bmm<BC, BC, DV, false, true>(a, F, L::DR, DV, L::Z, DV, L::DA, BC, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, BC, DK, false, true>(a, F, L::DY, DK, L::EB, DK, L::DA, BC, 1.f, (long long)L::DA, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DV, BC, true, false>(a, F, L::A, BC, L::DR, DV, L::DZ, DV, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DK, BC, true, false>(a, F, L::A, BC, L::DY, DK, L::X1, DK, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, BC, BC, true, false>(a, F, L::A, BC, L::DA, BC, L::WM, BC, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, BC, BC, false, true>(a, F, L::WM, BC, L::A, BC, L::DT, BC, -1.f, -1, 1, -1, items, st)));
  // decay-weighted products through the centred factors
  GDR2_CK((bmm<BC, DK, BC, false, false>(a, F, L::DT, BC, L::KP, DK, L::P1, DK, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DK, BC, true, false>(a, F, L::DT, BC, L::EP, DK, L::P2, DK, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DK, BC, true, false>(a, F, L::DAQK, BC, L::QP, DK, L::P3, DK, 1.f, -1, 0, 0, items, st)));
  GDR2_CK((bmm<BC, DK, BC, false, false>(a, F, L::DAQK, BC, L::KP, DK, L::P4, DK, 1.f, -1, 0, 0, items, st)));
  if (a.in_bf16) hipLaunchKernelGGL((bwd_final_kernel<DK, DV, true>), gi, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((bwd_final_kernel<DK, DV, false>), gi, dim3(256), 0, st, a);
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
