// gdr2_intra.hip -- intra-chunk pass of the two-pass chunkwise forward of the
// Gated Delta Rule-2 operator, 16-bit inputs (Gated DeltaNet-2 pages,
// "Chunkwise Parallel Training via WY Representation", Step 1 decay
// normalisation and Step 2 WY representation, Eqs. 20-22).
//
// Everything in a chunk that does not depend on the incoming state is
// computed here, for all chunks of all sequences and heads at once: one
// (chunk, head) item per workgroup iteration, in a persistent grid that
// prefetches the next item's raw inputs into registers while it works on the
// current one.  Per item, with G the fp32 cumulative log-decay from the chunk
// start (log2 units) and c(r) = 16*(r/16) + 7 the centre row of row r's
// 16-row block:
//   L  G by a DPP scan; centred factors e1 = 2^(G_r - G_c(r)), e2 = 2^(G_c(r)
//      - G_r) so that no factor exceeds the decay over 8 tokens; E' = e1*b*k,
//      K' = e2*k, Q' = e1*q (bf16, hi/lo for K' and Q'), the un-centred
//      E = gamma*b*k, Q_g = gamma*q, K_tail = (gamma_C/gamma)*k and Z = w*v.
//   P  T^T = K' E'^T and A_qk^T = K' Q'^T on MFMA.  Inside a diagonal 16x16
//      tile the centring cancels; an off-diagonal tile (a, b) first scales K'
//      by 2^(G_c(a) - G_c(b)) <= 1 per channel (and splits it into hi/lo
//      again), which restores the decay between the two centres.
//   S  A = (I + T)^-1: fp32 forward substitution on the four 16x16 diagonal
//      blocks, then the block recurrence for the off-diagonal blocks.
//   Y  Y = A E and U = A Z on MFMA.
// The record (layout in gdr2_internal.h) gets gamma_C in phase L, A_qk in
// phase P straight from the accumulators, Q_g and K_tail through LDS in phase
// S, and -Y and U from the accumulators in phase Y.
// The state pass (gdr2_state.hip) then needs only three small products per
// chunk and value tile.
#include <hip/hip_runtime.h>

#include "gdr2_chunk_common.h"
#include "gdr2_internal.h"

namespace gdr2 {

namespace {

constexpr int NT = 512;  // threads per workgroup
constexpr int NW = 8;    // wavefronts per workgroup (the prologue's row sums read NW = 8 partials)

template <int DK, int DV>
struct IntraCfg {
  typedef __bf16 KT;    // T / A_qk operands
  typedef _Float16 ST;  // record and state-pass operands
  static constexpr int PAD = 8;
  static constexpr int LDK = DK + PAD;  // rows of [64][DK]
  static constexpr int LDC = CH + PAD;  // rows of [*][64]
  // region X, phase P set: E', K'hi, K'lo, Q'hi, Q'lo  [64][LDK] bf16
  static constexpr size_t SZK = (size_t)CH * LDK * 2;
  static constexpr size_t XP = 5 * SZK;
  // region X after phase P: E^T, K_tail^T [DK][LDC]; Q_g [64][LDK]  (fp16)
  static constexpr size_t O_EHT = 0;
  static constexpr size_t O_KTT = O_EHT + (size_t)DK * LDC * 2;
  static constexpr size_t O_QG = O_KTT + (size_t)DK * LDC * 2;
  static constexpr size_t XR = O_QG + (size_t)CH * LDK * 2;
  static constexpr size_t X = ((XP > XR ? XP : XR) + 15) / 16 * 16;
  static constexpr size_t O_TD = X;                                // fp32 [4][16][16] diag T^T
  static constexpr size_t O_TN = O_TD + 4 * 16 * 16 * 4;           // [64][LDC] -T
  static constexpr size_t O_A = O_TN + (size_t)CH * LDC * 2;       // [64][LDC] A
  static constexpr int LDZ = DV + PAD;                             // rows of Z
  static constexpr size_t O_Z = O_A + (size_t)CH * LDC * 2;        // [64][LDZ] Z (row major)
  // per (block pair a > b, channel): 2^(G(c_a) - G(c_b)) as fp32 factor and
  // integer exponent, float2 [6][DK]
  static constexpr size_t O_DSC = O_Z + (size_t)CH * LDZ * 2;
  static constexpr size_t O_NRM = O_DSC + (size_t)6 * DK * 8;      // fp32 [64][2] q, k row sums
  static constexpr size_t O_SCL = O_NRM + (size_t)CH * 2 * 4;      // fp32 [64][2] q, k row scales
  static constexpr size_t O_FLAG = O_SCL + (size_t)CH * 2 * 4;     // ints: block centres, strong item
  static constexpr size_t BYTES = O_FLAG + 16;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  // region X of a strong item in phase P: the uncentred G (fp32 [64][LDG]) and
  // the raw k, q (bf16) and activated b (fp16) rows, [64][LDK] each
  static constexpr int LDG = DK + 4;
  static constexpr size_t O_SG = 0;
  static constexpr size_t O_SK = O_SG + (size_t)CH * LDG * 4;
  static constexpr size_t O_SQ = O_SK + SZK;
  static constexpr size_t O_SB = O_SQ + SZK;
  static_assert(O_SB + SZK <= X, "strong-item rows exceed region X");
  // key-side mapping: thread = (column group cg of EPC channels, row group rg
  // of RPT consecutive rows); the RG row groups of a column group are
  // consecutive lanes of one wavefront
  static constexpr int EPC = 4, CG = DK / EPC, RG = NT / CG, RPT = CH / RG;
  static_assert(RG >= 16 && RG <= 64 && CH % RG == 0, "bad key-side mapping");
  // value-side mapping: units of VE consecutive channels of one row
  static constexpr int VPT = CH * DV / NT;          // elements per thread
  static constexpr int VE = VPT < 8 ? VPT : 8;      // elements per unit (one load)
  static constexpr int NVU = VPT / VE;              // units per thread
  static constexpr int UPR = DV / VE;               // units per row
  static_assert(VE == 4 || VE == 8, "bad value-side mapping");
};

// Transposing LDS read of 16-bit data: within each 16-lane group, lane t
// receives element t, t + 16, t + 32 and t + 48 of the 64 elements that the
// group's lanes address (4 consecutive elements per lane, in lane order).
__device__ __forceinline__ f16x4 lds_tr16(const _Float16* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(__attribute__((address_space(3))) void*)p);
  return __builtin_bit_cast(f16x4, v);
}

// Exact chunk-matrix tile of a strong item (decay that centred factors cannot
// carry): lane (m, g4) gets, for q < 4, row r = r0 + m and column s = s0 + q
// (s0 = 16 b + 4 g4), in the layout of the MFMA path,
//   aq[q] = nq_r nk_s sum_c q[r][c] k[s][c] 2^(G[r][c] - G[s][c])        (A_qk)
//   at[q] = nk_r nk_s sum_c b[r][c] k[r][c] k[s][c] 2^(G[r][c] - G[s][c]) (T)
// from the rows staged in region X (G in log2 units) and the per-row L2
// scales (nq, nk) in scl.  Entries above the diagonal are formed too and
// masked by the caller.
template <int DK, int LDG, int LDK>
__device__ __forceinline__ void strong_tile(const float* SG, const __bf16* SK, const __bf16* SQ,
                                            const _Float16* SB, const float* scl, int r, int s0,
                                            f32x4& aq, f32x4& at) {
  typedef __attribute__((ext_vector_type(4))) __bf16 b4;
  typedef __attribute__((ext_vector_type(4))) _Float16 h4;
  aq = zero4();
  at = zero4();
#pragma unroll 1
  for (int c = 0; c < DK; c += 4) {
    const float4 gr = *reinterpret_cast<const float4*>(SG + r * LDG + c);
    const b4 kr = *reinterpret_cast<const b4*>(SK + r * LDK + c);
    const b4 qr = *reinterpret_cast<const b4*>(SQ + r * LDK + c);
    const h4 br = *reinterpret_cast<const h4*>(SB + r * LDK + c);
    const float bk[4] = {(float)br[0] * (float)kr[0], (float)br[1] * (float)kr[1],
                         (float)br[2] * (float)kr[2], (float)br[3] * (float)kr[3]};
    const float qq[4] = {(float)qr[0], (float)qr[1], (float)qr[2], (float)qr[3]};
    const float g[4] = {gr.x, gr.y, gr.z, gr.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 gs = *reinterpret_cast<const float4*>(SG + (s0 + q) * LDG + c);
      const b4 ks = *reinterpret_cast<const b4*>(SK + (s0 + q) * LDK + c);
      const float gsv[4] = {gs.x, gs.y, gs.z, gs.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = (float)ks[j] * exp2_fast(g[j] - gsv[j]);
        aq[q] = fmaf(qq[j], x, aq[q]);
        at[q] = fmaf(bk[j], x, at[q]);
      }
    }
  }
  const float2 sr = *reinterpret_cast<const float2*>(scl + 2 * r);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float nks = scl[2 * (s0 + q) + 1];
    aq[q] *= sr.x * nks;
    at[q] *= sr.y * nks;
  }
}

}  // namespace

// fp32 activations of the gate prologue.  softplus(x) = max(x, 0) +
// log1p(e^-|x|), with log1p(u) = u - u^2/2 (its Taylor series) below 1e-3
// where 1 + u would round away u.
__device__ __forceinline__ float softplus_f(float x) {
  const float u = __expf(-fabsf(x));
  const float l = u < 1e-3f ? u * (1.f - 0.5f * u) : __logf(1.f + u);
  return fmaxf(x, 0.f) + l;
}
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// Gate-prologue steps of an instantiation: PRO = 0 runs none, PRO_ALL all
// three with the choice fixed at compile time, PRO_ANY the steps the call's
// flags select, read at run time.  The all-steps case is the usual one, and
// fixing it at compile time keeps the registers of the branches it never
// skips from weighing on the rest of the item (its main loop spills 8 bytes
// per lane instead of 56).
constexpr int PRO_ALL = PRO_QK_L2NORM | PRO_DECAY | PRO_GATES;
constexpr int PRO_ANY = 8;
template <int PRO>
__device__ __forceinline__ bool pro_step(const IntraArgs& p, int step) {
  if constexpr (PRO == PRO_ANY) return (p.pro & step) != 0;
  else return (PRO & step) != 0;
}

// Stages a strong item's rows in region X for the exact products of phase P
// (strong_tile): the uncentred cumulative log2-decay G (fp32), the raw k and
// q rows (bf16) and the erase gate b (fp16, activated under the prologue),
// read again from the inputs of token rows [row0, row0 + clen) of value head
// h's key head; rows past the end get zero q, k and log-decay.  Thread tid
// owns channel tid % DK and a group of consecutive rows; the group totals of
// the decay scan meet in the diagonal-T buffer, free until the tiles.
template <int DK, int DV, bool LA16, int PRO>
__device__ __forceinline__ void strong_stage(const IntraArgs& p, long long row0, int clen, int h) {
  typedef IntraCfg<DK, DV> Cfg;
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NGR = NT / DK, RPG = CH / NGR, LDK = Cfg::LDK, LDG = Cfg::LDG;
  float* SG = reinterpret_cast<float*>(smem + Cfg::O_SG);
  __bf16* SK = reinterpret_cast<__bf16*>(smem + Cfg::O_SK);
  __bf16* SQ = reinterpret_cast<__bf16*>(smem + Cfg::O_SQ);
  _Float16* SB = reinterpret_cast<_Float16*>(smem + Cfg::O_SB);
  float* part = reinterpret_cast<float*>(smem + Cfg::O_TD);
  const int tid = threadIdx.x, c = tid % DK, gr = tid / DK;
  const int hk = h / p.grp;  // key head of value head h (grp = 1 without grouping)
  const size_t krow = (size_t)p.Hk * DK;
  float ea = 0.f, dl = 0.f;
  if constexpr (PRO != 0) {
    if (pro_step<PRO>(p, PRO_DECAY)) {
      ea = __expf(p.da[(size_t)hk * DK + c]);
      dl = p.db[(size_t)hk * DK + c];
    }
  }
  float acc = 0.f;
#pragma unroll 2
  for (int j = 0; j < RPG; ++j) {
    const int r = gr * RPG + j;
    float gv = 0.f, kv = 0.f, qv = 0.f, bv = 0.f;
    if (r < clen) {
      const size_t x = (size_t)(row0 + r) * krow + (size_t)hk * DK + c;
      gv = load1<LA16>(p.la, x);
      kv = load1<true>(p.k, x);
      qv = load1<true>(p.q, x);
      bv = load1<true>(p.b, x);
      if constexpr (PRO != 0) {
        if (pro_step<PRO>(p, PRO_DECAY)) gv = -ea * softplus_f(gv + dl);
        if (pro_step<PRO>(p, PRO_GATES)) bv = p.b_scale * sigmoid_f(bv);
      }
    }
    acc += gv * LOG2E;
    SG[r * LDG + c] = acc;  // the group's own partial sum; offset below
    SK[r * LDK + c] = (__bf16)kv;
    SQ[r * LDK + c] = (__bf16)qv;
    SB[r * LDK + c] = (_Float16)bv;
  }
  part[gr * DK + c] = acc;
  // Z = w * v rows (the write gate activated under the prologue)
  _Float16* Zr = reinterpret_cast<_Float16*>(smem + Cfg::O_Z);
  const size_t vrow = (size_t)p.H * DV;
  for (int e = tid; e < CH * DV; e += NT) {
    const int r = e / DV, j = e - r * DV;
    float z = 0.f;
    if (r < clen) {
      const size_t x = (size_t)(row0 + r) * vrow + (size_t)h * DV + j;
      float wv = load1<true>(p.w, x);
      if constexpr (PRO != 0) {
        if (pro_step<PRO>(p, PRO_GATES)) wv = sigmoid_f(wv);
      }
      z = load1<true>(p.v, x) * wv;
    }
    Zr[r * Cfg::LDZ + j] = (_Float16)z;
  }
  __syncthreads();
  float off = 0.f;
#pragma unroll
  for (int q = 0; q < NGR - 1; ++q)
    if (q < gr) off += part[q * DK + c];
#pragma unroll 4
  for (int j = 0; j < RPG; ++j) SG[(gr * RPG + j) * LDG + c] += off;
  // per-row scales of the q, k L2 norm (1 without it; 0 past the end)
  float* scl = reinterpret_cast<float*>(smem + Cfg::O_SCL);
  if (tid < 2 * CH) {
    const int r = tid >> 1, which = tid & 1;
    float sc = 1.f;
    if constexpr (PRO != 0) {
      if (pro_step<PRO>(p, PRO_QK_L2NORM)) {
        const __bf16* row = (which ? SK : SQ) + r * LDK;
        float ss = 0.f;
        for (int cc = 0; cc < DK; ++cc) ss = fmaf((float)row[cc], (float)row[cc], ss);
        sc = r < clen ? rsqrtf(ss + p.qk_eps) : 0.f;
      }
    }
    scl[2 * r + which] = sc;
  }
}

// Stores one lower tile (a, b) of phase P, lane layout of the MFMA products
// (acc: A_qk[16a + m][16b + 4 g4 + q], acct: T likewise): the diagonal blocks
// of T transposed in fp32 (Tdt), -T of the off-diagonal blocks in fp16 (Tn),
// and A_qk as record fragments.
template <int DK, int DV>
__device__ __forceinline__ void tile_store(int a, int b, f32x4 acc, f32x4 acct, char* rec) {
  typedef IntraCfg<DK, DV> Cfg;
  typedef Rec<DK, DV> R;
  typedef _Float16 ST;
  typedef f16x4 SV4;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Tdt = reinterpret_cast<float*>(smem + Cfg::O_TD);
  ST* Tn = reinterpret_cast<ST*>(smem + Cfg::O_TN);
  const int lane = lane_id(), m = lane & 15, g4 = lane >> 4;
  if (a == b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = (4 * g4 + q <= m) ? acc[q] : 0.f;
    // diagonal blocks of T transposed, fp32: Tdt[a][s][r] = T[r][s], s < r
#pragma unroll
    for (int q = 0; q < 4; ++q) Tdt[(a * 16 + 4 * g4 + q) * 16 + m] = (4 * g4 + q < m) ? acct[q] : 0.f;
  } else {
    *reinterpret_cast<SV4*>(Tn + (16 * a + m) * Cfg::LDC + 16 * b + 4 * g4) = neg_cvt4<SV4>(acct);
  }
  // A_qk fragment (a, p = b/2) half b&1, lane (m, g4); the upper halves of
  // fragments (0, 0) and (2, 1) are zero
  const int f = a < 2 ? a : 2 * a - 2 + (b >> 1);
  char* dst = rec + R::AQK + ((size_t)f * 64 + lane) * 16;
  *reinterpret_cast<SV4*>(dst + 8 * (b & 1)) = cvt4<SV4>(acc);
  if (a == b && (a & 1) == 0) *reinterpret_cast<SV4*>(dst + 8) = SV4{(ST)0.f, (ST)0.f, (ST)0.f, (ST)0.f};
}

// MODE 0: every item, then again the strong ones this workgroup met; MODE 1:
// every item, strong ones only flagged; MODE 2: the flagged items only (the
// second launch after MODE 1).  Variants whose main loop is near the register
// limit take MODE 1 and 2, so that the exact path's registers never weigh on
// their main loop.
template <int DK, int DV, bool LA16, int PRO, int MODE>
__global__ __launch_bounds__(NT) void intra_kernel(IntraArgs p) {
  typedef IntraCfg<DK, DV> Cfg;
  typedef Rec<DK, DV> R;
  typedef __bf16 KT;
  typedef _Float16 ST;
  typedef f16x4 SV4;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, EPC = Cfg::EPC;
  constexpr int RPT = Cfg::RPT, RG = Cfg::RG, LW = LA16 ? 2 : 4;
  constexpr int VE = Cfg::VE, NVU = Cfg::NVU, UPR = Cfg::UPR;

  extern __shared__ __align__(16) unsigned char smem[];
  KT* Ep = reinterpret_cast<KT*>(smem);
  KT* Kh = reinterpret_cast<KT*>(smem + Cfg::SZK);
  KT* Kl = reinterpret_cast<KT*>(smem + 2 * Cfg::SZK);
  KT* Qh = reinterpret_cast<KT*>(smem + 3 * Cfg::SZK);
  KT* Ql = reinterpret_cast<KT*>(smem + 4 * Cfg::SZK);
  ST* EhT = reinterpret_cast<ST*>(smem + Cfg::O_EHT);
  ST* KtT = reinterpret_cast<ST*>(smem + Cfg::O_KTT);
  ST* Qg = reinterpret_cast<ST*>(smem + Cfg::O_QG);
  float* Tdt = reinterpret_cast<float*>(smem + Cfg::O_TD);
  ST* Tn = reinterpret_cast<ST*>(smem + Cfg::O_TN);
  ST* Am = reinterpret_cast<ST*>(smem + Cfg::O_A);
  ST* Zr = reinterpret_cast<ST*>(smem + Cfg::O_Z);
  float2* dsc = reinterpret_cast<float2*>(smem + Cfg::O_DSC);
  float* nrm = reinterpret_cast<float*>(smem + Cfg::O_NRM);
  int* blocked = reinterpret_cast<int*>(smem + Cfg::O_FLAG);
  int* strongf = blocked + 1;
  float* scl = reinterpret_cast<float*>(smem + Cfg::O_SCL);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = lane & 15, g4 = lane >> 4;
  const int H = p.H;
  const int items = (p.total ? *p.total : p.chunks) * H;
  if ((int)blockIdx.x >= items) return;

  // the strictly upper blocks of A stay zero; the products run over them
  for (int e = tid; e < CH * LDC; e += NT) Am[e] = (ST)0.f;
  if (tid == 0) *blocked = *strongf = 0;
  for (int e = tid; e < 6 * DK; e += NT) dsc[e] = make_float2(1.f, __int_as_float(0));

  // item -> first token row, valid rows, head.  The values are uniform across
  // the workgroup; reading them through readfirstlane keeps them in scalar
  // registers, so the buffer descriptors built from them need no per-lane loop.
  auto locate = [&](int it, long long& row0, int& clen, int& h) {
    const int ci = it / H;
    h = it - ci * H;
    int r, l;
    if (p.tab) {
      r = p.tab[2 * ci];
      l = p.tab[2 * ci + 1];
      row0 = __builtin_amdgcn_readfirstlane(r);
      clen = __builtin_amdgcn_readfirstlane(l);
    } else {
      const int n = ci / p.nc, c = ci - n * p.nc;
      row0 = (long long)n * p.T + (long long)c * CH;
      clen = min(CH, p.T - c * CH);
    }
  };

  // processing order -> record index.  With equal-length sequences the items
  // go last chunk first, so the records the state pass reads first are the
  // most recently written ones (still in the last-level cache when the state
  // pass starts); packed sequences keep the record order.
  auto order = [&](int it) -> int {
    if (p.tab) return it;
    const int pairs = p.chunks / p.nc * H, step = it / pairs, rem = it - step * pairs;
    const int n = rem / H, hh = rem - n * H;
    return ((n * p.nc) + (p.nc - 1 - step)) * H + hh;
  };

  const int cg = tid / RG, rg = tid % RG, r0 = rg * RPT;
  // key-side rows hold Hk heads (grouped value heads), value-side rows H
  const size_t krow = (size_t)p.Hk * DK, vrow = (size_t)H * DV;
  uint32_t koff[RPT], goff[RPT], voff[NVU];
  int vr[NVU], vc0[NVU];
#pragma unroll
  for (int pr = 0; pr < RPT; ++pr) {
    koff[pr] = (uint32_t)(((r0 + pr) * krow + EPC * cg) * 2);
    goff[pr] = (uint32_t)(((r0 + pr) * krow + EPC * cg) * (LA16 ? 2 : 4));
  }
#pragma unroll
  for (int i = 0; i < NVU; ++i) {
    const int u = tid + NT * i;
    vr[i] = u / UPR;
    vc0[i] = VE * (u % UPR);
    voff[i] = (uint32_t)((vr[i] * vrow + vc0[i]) * 2);
  }

  uint32_t rq[RPT][2], rk[RPT][2], rb[RPT][2], rgd[RPT][LW];
  uint32_t rv[NVU][VE / 2], rw[NVU][VE / 2];
  // prologue: a and delta of this thread's 4 key channels for the next item,
  // loaded at the end of the previous one so that they are live only across
  // the item boundary
  float4 rda = make_float4(0.f, 0.f, 0.f, 0.f), rdb = rda;
  auto fetch_decay = [&](int h) {
    if constexpr (PRO != 0) {
      if (pro_step<PRO>(p, PRO_DECAY)) {
        const size_t o = (size_t)(h / p.grp) * DK + EPC * cg;
        rda = *reinterpret_cast<const float4*>(p.da + o);
        rdb = *reinterpret_cast<const float4*>(p.db + o);
      }
    }
  };
  // Range-limited buffer loads: rows past the chunk's last valid token read
  // as zero and nothing outside the caller's tensors is touched.
  // One input tensor per batch (q, k, b, log_alpha, v, w).  A CU keeps only
  // a limited amount of memory traffic in flight, and issuing a whole item at
  // once stalls the issuing wavefronts until it drains, so the batches go out
  // at six points of the current item (two in phase L, then one at the start
  // of each later phase).
  auto fetch = [&](long long row0, int clen, int h, int batch) {
    const int hk = h / p.grp;  // key head of value head h (grp = 1 without grouping)
    const size_t kel = (size_t)row0 * krow + (size_t)hk * DK, vel = (size_t)row0 * vrow + (size_t)h * DV;
    const int kbytes = (int)(clen * krow * 2), gbytes = (int)(clen * krow * (LA16 ? 2 : 4));
    const int vbytes = (int)(clen * vrow * 2);
    if (batch <= 2) {
      const void* src = batch == 0 ? p.q : batch == 1 ? p.k : p.b;
      const auto rs = make_rsrc(static_cast<const char*>(src) + kel * 2, kbytes);
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) bld(batch == 0 ? rq[pr] : batch == 1 ? rk[pr] : rb[pr], rs, koff[pr]);
    } else if (batch == 3) {
      const auto rsg = make_rsrc(static_cast<const char*>(p.la) + kel * (LA16 ? 2 : 4), gbytes);
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) bld(rgd[pr], rsg, goff[pr]);  // raw words: expanding bf16 here would wait
    } else {
      const auto rs = make_rsrc(static_cast<const char*>(batch == 4 ? p.v : p.w) + vel * 2, vbytes);
#pragma unroll
      for (int i = 0; i < NVU; ++i) bld(batch == 4 ? rv[i] : rw[i], rs, voff[i]);
    }
  };

  // ---- phases S and Y, shared by the main loop and the strong items' loop -----
  // S(i): wave a < 4 inverts I + T_aa (diagonal blocks of A)
  auto inv_diag = [&]() __attribute__((always_inline)) {
      if (wv < 4) {
      // wave a inverts I + T_aa: lane 4*cc + part holds rows 4*part .. 4*part+3
      // of column cc and runs a right-looking fp32 forward substitution over
      // the columns s of T_aa; row s of column cc is broadcast in its quad
      const int a = wv, cc = lane >> 2, part = lane & 3;
      const float4* Tc = reinterpret_cast<const float4*>(Tdt + a * 256);
      // all 15 column pieces first, so the substitution chain waits on no LDS read
      float4 tcol[15];
#pragma unroll
      for (int s = 0; s < 15; ++s) tcol[s] = Tc[s * 4 + part];
      float xs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xs[j] = (4 * part + j == cc) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < 15; ++s) {
        const float4 col = tcol[s];
        const float xv = quad_bcast(xs[s & 3], s >> 2);
        // T[r][s] is zero for r <= s, so finished rows are left unchanged
        xs[0] = fmaf(-col.x, xv, xs[0]);
        xs[1] = fmaf(-col.y, xv, xs[1]);
        xs[2] = fmaf(-col.z, xv, xs[2]);
        xs[3] = fmaf(-col.w, xv, xs[3]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) Am[(16 * a + 4 * part + j) * LDC + 16 * a + cc] = (ST)xs[j];
    }
  };
  // S(ii): the off-diagonal blocks of A; the Q_g and K_tail fragments into the record
  auto phase_s2 = [&](char* rec, bool copy_fragments) __attribute__((always_inline)) {
    if (wv == 3) wy_column<0, ST, SV4, LDC>(Tn, Am);
    else if (wv == 2) wy_column<1, ST, SV4, LDC>(Tn, Am);
    else if (wv == 1) wy_column<2, ST, SV4, LDC>(Tn, Am);
    else if (copy_fragments) {
      // waves 0, 4..7 copy the Q_g and K_tail fragments, complete since phase
      // S(i), while the others solve (16-byte pieces, 1 KiB per instruction)
      constexpr int NQG = 4 * R::NKB, NF = NQG + 2 * R::NIB;
      const int w5 = wv == 0 ? 0 : wv - 3;  // 0..4
      for (int f = w5; f < NF; f += 5) {
        const ST* src;
        char* dst;
        if (f < NQG) {
          const int a = f / R::NKB, kb = f % R::NKB;
          src = Qg + (16 * a + m) * LDK + 32 * kb + 4 * g4;
          dst = rec + R::QG + (size_t)f * R::FRAG;
        } else {
          const int ff = f - NQG, ib = ff >> 1, pp = ff & 1;
          src = KtT + (16 * ib + m) * LDC + 32 * pp + 4 * g4;
          dst = rec + R::KT + (size_t)ff * R::FRAG;
        }
        const SV4 lo = *reinterpret_cast<const SV4*>(src);
        const SV4 hi = *reinterpret_cast<const SV4*>(src + 16);
        *reinterpret_cast<f16x8*>(dst + lane * 16) =
            f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
  };
  // Y: -Y and U into the record
  auto phase_y = [&](char* rec) __attribute__((always_inline)) {
    {
      // -Y fragments (a, kb): wave -> kb = wv / 2 and row blocks {wv & 1, 3 - (wv & 1)}
      const int kb = wv >> 1;
      if (kb < R::NKB) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int a = s == 0 ? (wv & 1) : 3 - (wv & 1);
          f32x4 y0, y1;
          if (a < 2) {
            y0 = mma_lds<ST, 32>(zero4(), EhT + 32 * kb * LDC, LDC, Am + 16 * a * LDC, LDC);
            y1 = mma_lds<ST, 32>(zero4(), EhT + (32 * kb + 16) * LDC, LDC, Am + 16 * a * LDC, LDC);
          } else {
            y0 = mma_lds<ST, 64>(zero4(), EhT + 32 * kb * LDC, LDC, Am + 16 * a * LDC, LDC);
            y1 = mma_lds<ST, 64>(zero4(), EhT + (32 * kb + 16) * LDC, LDC, Am + 16 * a * LDC, LDC);
          }
          // lane holds Y[16a + m][32kb + 4*g4 + q] (y0) and Y[16a + m][32kb + 16 + 4*g4 + q] (y1)
          *reinterpret_cast<f16x8*>(rec + R::YN + ((size_t)(a * R::NKB + kb) * 64 + lane) * 16) =
              f16x8{(ST)-y0[0], (ST)-y0[1], (ST)-y0[2], (ST)-y0[3],
                    (ST)-y1[0], (ST)-y1[1], (ST)-y1[2], (ST)-y1[3]};
        }
      }
      // U tiles (jt, a): U = A Z over tokens.  K position 8*g4 + j of a 32-token
      // step p is token 32p + 4*g4 + j (j < 4) or 32p + 16 + 4*g4 + j - 4; the
      // A operand reads those columns of row 16a + m of A, and the Z operand
      // comes from row-major Z through the LDS transpose read (lane s of a
      // 16-lane group points at 4 channels of one token row; lane m then holds
      // channel m of 4 consecutive token rows)
      for (int t = wv; t < 4 * R::NJT; t += NW) {
        const int a = t / R::NJT, jt = t % R::NJT;
        f32x4 u = zero4();
        const int s = m;  // source lane inside the 16-lane group
        for (int pp = 0; pp <= (a >> 1); ++pp) {
          const ST* arow = Am + (16 * a + m) * LDC + 32 * pp + 4 * g4;
          const f16x4 a0 = *reinterpret_cast<const f16x4*>(arow);
          const f16x4 a1 = *reinterpret_cast<const f16x4*>(arow + 16);
          const ST* z0 = Zr + (32 * pp + 4 * g4 + (s >> 2)) * Cfg::LDZ + 16 * jt + 4 * (s & 3);
          const f16x4 b0 = lds_tr16(z0);
          const f16x4 b1 = lds_tr16(z0 + 16 * Cfg::LDZ);
          u = mma32(f16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]},
                    f16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]}, u);
        }
        // lane holds U[16a + 4*g4 + q][16jt + m]
        *reinterpret_cast<SV4*>(rec + R::U + ((size_t)(jt * 4 + a) * 64 + lane) * 8) = cvt4<SV4>(u);
      }
    }
  };

  int nstrong = 0;  // strong items this workgroup met (the same in every thread)
  if constexpr (MODE != 2) {
  long long row0;
  int clen, h;
  locate(order(blockIdx.x), row0, clen, h);
  for (int b = 0; b < 6; ++b) fetch(row0, clen, h, b);
  fetch_decay(h);
  __syncthreads();

  // the thread's indices under other names, for the loop's per-item copies
  const int tid_o = tid, lane_o = lane, wv_o = wv, m_o = m, g4_o = g4, cg_o = cg, rg_o = rg, r0_o = r0;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    // With the prologue's steps read at run time, the compiler hoists every
    // index computed from the thread index out of this loop and holds them
    // across the item, and the variant spilled (56 bytes per lane at the
    // 256-register limit); an empty asm makes the index opaque per item, so
    // they are recomputed inside (230 registers, no spill: B4 T4096 H16 Hv16
    // flags 3, 0.393 -> 0.359 ms).  The other variants keep the hoisting
    // (the copies below are then the outer values themselves), which
    // measured slightly faster for them.
    int tid_i = tid_o;
    if constexpr (PRO == PRO_ANY) asm volatile("" : "+v"(tid_i));
    const int tid = PRO == PRO_ANY ? tid_i : tid_o;
    const int lane = PRO == PRO_ANY ? (tid & 63) : lane_o, wv = PRO == PRO_ANY ? (tid >> 6) : wv_o;
    const int m = PRO == PRO_ANY ? (lane & 15) : m_o, g4 = PRO == PRO_ANY ? (lane >> 4) : g4_o;
    const int cg = PRO == PRO_ANY ? (tid / RG) : cg_o, rg = PRO == PRO_ANY ? (tid % RG) : rg_o;
    const int r0 = PRO == PRO_ANY ? (rg * RPT) : r0_o;
    (void)m; (void)g4; (void)cg; (void)rg; (void)r0; (void)wv;
    const int itn = it + gridDim.x;
    long long nrow0 = 0;
    int nclen = 0, nh = 0;
    if (itn < items) locate(order(itn), nrow0, nclen, nh);
    const int ri = order(it);  // record index
    char* rec = p.rec + (size_t)ri * R::BYTES;

    // ================= phase L: decay scan and operand tiles ====================
    SV4 eh[RPT], qg[RPT], kt[RPT];
    {
      float G[RPT][EPC], kv[RPT][EPC], qv[RPT][EPC], bv[RPT][EPC];
      float z[NVU][VE];
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) {
        unpack4<false>(rq[pr], qv[pr]);
        unpack4<false>(rk[pr], kv[pr]);
      }
      // q, k L2 norm of the gate prologue: per-row scales, applied where the
      // operand tiles are formed so that q and k can stay packed until then
      float nq[RPT], nk[RPT];
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) nq[pr] = nk[pr] = 1.f;
      if constexpr (PRO != 0) {
        if (pro_step<PRO>(p, PRO_QK_L2NORM)) {
          // A token row's DK channels sit in all CG column groups: 64/RG of
          // them per wavefront (lanes RG apart) and NW wavefronts.  Reduce
          // inside the wavefront by xor shuffles, then across wavefronts in
          // a fixed order through the diagonal-T buffer, which is idle during
          // this phase: red[row][q or k][wavefront] -> nrm[row][q or k].
          float sq[RPT], sk[RPT];
#pragma unroll
          for (int pr = 0; pr < RPT; ++pr) {
            sq[pr] = 0.f;
            sk[pr] = 0.f;
#pragma unroll
            for (int i = 0; i < EPC; ++i) {
              sq[pr] = fmaf(qv[pr][i], qv[pr][i], sq[pr]);
              sk[pr] = fmaf(kv[pr][i], kv[pr][i], sk[pr]);
            }
#pragma unroll
            for (int off = RG; off < 64; off <<= 1) {
              sq[pr] += __shfl_xor(sq[pr], off);
              sk[pr] += __shfl_xor(sk[pr], off);
            }
          }
          float* red = Tdt;
          static_assert(CH * 2 * NW * 4 <= 4 * 16 * 16 * 4, "row sums exceed the diagonal-T buffer");
          if (lane < RG) {
#pragma unroll
            for (int pr = 0; pr < RPT; ++pr) {
              red[((r0 + pr) * 2 + 0) * NW + wv] = sq[pr];
              red[((r0 + pr) * 2 + 1) * NW + wv] = sk[pr];
            }
          }
          __syncthreads();
          if (tid < CH * 2) {
            const float4* r4 = reinterpret_cast<const float4*>(red + tid * NW);
            const float4 x0 = r4[0], x1 = r4[1];
            nrm[tid] = ((x0.x + x0.y) + (x0.z + x0.w)) + ((x1.x + x1.y) + (x1.z + x1.w));
          }
          __syncthreads();
#pragma unroll
          for (int pr = 0; pr < RPT; ++pr) {
            const float2 t = *reinterpret_cast<const float2*>(nrm + (r0 + pr) * 2);
            const float tq = t.x, tk = t.y;
            // rows past the chunk's end stay zero (also with qk_eps = 0)
            const bool live = r0 + pr < clen;
            nq[pr] = live ? rsqrtf(tq + p.qk_eps) : 0.f;
            nk[pr] = live ? rsqrtf(tk + p.qk_eps) : 0.f;
          }
        }
      }
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) {
        unpack4<false>(rb[pr], bv[pr]);
        unpack4<!LA16>(rgd[pr], G[pr]);
        if constexpr (PRO == 0) {
#pragma unroll
          for (int i = 0; i < EPC; ++i) G[pr][i] *= LOG2E;
        }
      }
#pragma unroll
      for (int i = 0; i < NVU; ++i)
#pragma unroll
        for (int j = 0; j < VE / 2; ++j) {
          float w0 = __uint_as_float(rw[i][j] << 16), w1 = __uint_as_float(rw[i][j] & 0xffff0000u);
          if constexpr (PRO != 0) {
            if (pro_step<PRO>(p, PRO_GATES)) {  // write gate w = sigmoid(W_w x)  (Eq. 11)
              w0 = sigmoid_f(w0);
              w1 = sigmoid_f(w1);
            }
          }
          z[i][2 * j] = __uint_as_float(rv[i][j] << 16) * w0;
          z[i][2 * j + 1] = __uint_as_float(rv[i][j] & 0xffff0000u) * w1;
        }
      // The raw registers are free: the next item's loads go out in six
      // batches from here on.  The loads of this item are waited for
      // explicitly first, so that the first use of their registers does not
      // also wait for the new ones.
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      if (itn < items) fetch(nrow0, nclen, nh, 0);

      if constexpr (PRO != 0) {
        // Gate prologue (Gated DeltaNet-2 pages, "Gate Parameterization":
        // Eq. 12 log-decay g = -exp(a) * softplus(f + delta) and Eq. 11 erase
        // gate b = b_scale * sigmoid(W_b x); q and k L2-normalised per head),
        // in fp32 on the loaded values.
        if (pro_step<PRO>(p, PRO_DECAY)) {
          const float ea[4] = {__expf(rda.x), __expf(rda.y), __expf(rda.z), __expf(rda.w)};
          const float dl[4] = {rdb.x, rdb.y, rdb.z, rdb.w};
#pragma unroll
          for (int pr = 0; pr < RPT; ++pr)
#pragma unroll
            for (int i = 0; i < EPC; ++i)  // rows past the chunk's end keep g = 0
              G[pr][i] = r0 + pr < clen ? -ea[i] * softplus_f(G[pr][i] + dl[i]) : 0.f;
        }
        if (pro_step<PRO>(p, PRO_GATES)) {
#pragma unroll
          for (int pr = 0; pr < RPT; ++pr)
#pragma unroll
            for (int i = 0; i < EPC; ++i) bv[pr][i] = p.b_scale * sigmoid_f(bv[pr][i]);
        }
#pragma unroll
        for (int pr = 0; pr < RPT; ++pr)
#pragma unroll
          for (int i = 0; i < EPC; ++i) G[pr][i] *= LOG2E;
      }

      // fp32 cumulative log2-decay: serial inside the thread, then a scan of
      // the thread totals across the RG row groups of the column group
#pragma unroll
      for (int pr = 1; pr < RPT; ++pr)
#pragma unroll
        for (int i = 0; i < EPC; ++i) G[pr][i] += G[pr - 1][i];
      // Centring.  A channel whose decay on each side of row 31 stays below
      // 2^CLIM is centred on row 31 for the whole chunk, as one centre keeps
      // every factor of that channel in range.  A channel with stronger decay
      // centres each 16-row block a on its row c_a = 16a + 7 instead, so that
      // a factor spans at most 8 tokens of decay.  The thread's rows all lie
      // in block ab.  dsc[pair (a, b)][channel] = 2^(G(c_a) - G(c_b)) (1 for a
      // row-31 channel, the value the table holds between items) as (factor in
      // [1, 2), integer exponent) lets phase P
      // restore the decay between two block centres in the off-diagonal
      // tiles; it spans 16 tokens of decay and may lie below the fp32 range
      // while the scaled K' (at most ~23 tokens from c_a) does not, so it is
      // kept as an exponent shift.  The workgroup flag `blocked` tells phase
      // P whether any channel of the item needs the scaling.
      constexpr float CLIM = 100.f;
      const int ab = r0 / 16;
      float egm[EPC], egcm[EPC];
      bool blocked_t = false;
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        const float tot = G[RPT - 1][i];
        const float excl = seg_scan<RG>(tot) - tot;
#pragma unroll
        for (int pr = 0; pr < RPT; ++pr) G[pr][i] += excl;
        const float g31 = __shfl(G[(CH / 2 - 1) % RPT][i], (CH / 2 - 1) / RPT, RG);
        const float gc = __shfl(G[RPT - 1][i], RG - 1, RG);
        // G is 0 before row 0; with either sign of decay the factors of a
        // row-31 centre stay within 2^max(|G_31|, |G_31 - G_63|)
        const bool mild = fabsf(g31) < CLIM && fabsf(g31 - gc) < CLIM;
        float gca[4] = {g31, g31, g31, g31};
        if (__any(!mild)) {  // wave-uniform: the shuffles need every lane
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float v = __shfl(G[7 % RPT][i], (16 * a + 7) / RPT, RG);
            if (!mild) gca[a] = v;
          }
        }
        const float gm = ab == 0 ? gca[0] : ab == 1 ? gca[1] : ab == 2 ? gca[2] : gca[3];
        egm[i] = exp2_fast(gm);
        egcm[i] = exp2_fast(gc - gm);
        if (rg == 0) reinterpret_cast<float*>(rec + R::GC)[EPC * cg + i] = exp2_fast(gc);
        if (rg == 0 && !mild) {  // dsc holds 1 (factor 1, exponent 0) for every other channel
#pragma unroll
          for (int a = 1; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < a; ++b) {
              const float dg = gca[a] - gca[b], n = floorf(dg);
              dsc[(a * (a - 1) / 2 + b) * DK + EPC * cg + i] =
                  make_float2(exp2_fast(dg - n), __int_as_float((int)n));
            }
        }
        blocked_t = blocked_t || !mild;
#pragma unroll
        for (int pr = 0; pr < RPT; ++pr) G[pr][i] -= gm;  // centred
      }
      if (blocked_t) *blocked = 1;  // every writer stores the same value
      // A strong item has some centred factor beyond 2^SLIM: decay that even
      // the per-block centres cannot carry in 16-bit operands.  This pass
      // still runs it (with out-of-range factors and a record that means
      // nothing); the item is flagged, and the workgroup forms its record
      // again after its last item, from the inputs, with the exact decay.
      constexpr float SLIM = 112.f;
      bool strong_t = false;
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr)
#pragma unroll
        for (int i = 0; i < EPC; ++i) strong_t = strong_t || fabsf(G[pr][i]) > SLIM;
      if (strong_t) *strongf = 1;  // every writer stores the same value
      {
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) {
        const int r = r0 + pr;
        float ep[EPC], kh[EPC], kl[EPC], qh[EPC], ql[EPC];
#pragma unroll
        for (int i = 0; i < EPC; ++i) {
          const float e1 = exp2_fast(G[pr][i]);
          const float e2 = exp2_fast(-G[pr][i]);
          const float kk = kv[pr][i] * nk[pr], qq = qv[pr][i] * nq[pr];  // L2 norm (prologue)
          ep[i] = e1 * (bv[pr][i] * kk);
          const float kbv = e2 * kk;
          const float qp = e1 * qq;
          kh[i] = bf16_round(kbv);
          kl[i] = kbv - kh[i];
          qh[i] = bf16_round(qp);
          ql[i] = qp - qh[i];
          eh[pr][i] = (ST)(ep[i] * egm[i]);
          qg[pr][i] = (ST)(qp * egm[i]);
          kt[pr][i] = (ST)(kbv * egcm[i]);
        }
        st4<KT>(Ep + r * LDK + EPC * cg, ep);
        st4<KT>(Kh + r * LDK + EPC * cg, kh);
        st4<KT>(Kl + r * LDK + EPC * cg, kl);
        st4<KT>(Qh + r * LDK + EPC * cg, qh);
        st4<KT>(Ql + r * LDK + EPC * cg, ql);
      }
      }
      if (itn < items) fetch(nrow0, nclen, nh, 1);
      // Z row major: each unit is VE consecutive channels of one row
#pragma unroll
      for (int i = 0; i < NVU; ++i) {
        if constexpr (VE == 8) st8<ST>(Zr + vr[i] * Cfg::LDZ + vc0[i], z[i]);
        else st4<ST>(Zr + vr[i] * Cfg::LDZ + vc0[i], z[i]);
      }
    }
    __syncthreads();

    // ================= phase P: T^T and A_qk^T on MFMA ==========================
    // tile t goes to wave t (tiles 8, 9 to waves 0, 2); one wave forms both T
    // and A_qk of its tile so the K' operand is read once per K step
    if (itn < items) fetch(nrow0, nclen, nh, 2);
    {
      const bool blk = *blocked != 0;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ti = k == 0 ? wv : (wv == 0 ? 8 : wv == 2 ? 9 : -1);
        if (ti < 0) break;
        int a, b;
        tri_tile(ti, a, b);
        // each operand fragment is read from LDS once per K step and feeds the
        // three hi/lo products of A_qk and the product of T
        f32x4 acc = zero4(), acct = zero4();
        {
          const int ob = (16 * b + m) * LDK + 8 * g4, oa = (16 * a + m) * LDK + 8 * g4;
#pragma unroll
          for (int k0 = 0; k0 < DK; k0 += 32) {
            bf16x8 kh = *reinterpret_cast<const bf16x8*>(Kh + ob + k0);
            bf16x8 kl = *reinterpret_cast<const bf16x8*>(Kl + ob + k0);
            if (a != b && blk) {
              // K' of block b is centred on c_b and E', Q' of block a on c_a:
              // scale K' by 2^(G(c_a) - G(c_b)) <= 1 per channel (factor, then
              // exponent shift) and split it into hi/lo again
              const float4* pd = reinterpret_cast<const float4*>(dsc + (a * (a - 1) / 2 + b) * DK + k0 + 8 * g4);
#pragma unroll
              for (int hf = 0; hf < 2; ++hf) {  // two halves of 4 channels: fewer live registers
                const float4 d0 = pd[2 * hf], d1 = pd[2 * hf + 1];
                const float df[4] = {d0.x, d0.z, d1.x, d1.z};
                const int dn[4] = {__float_as_int(d0.y), __float_as_int(d0.w), __float_as_int(d1.y),
                                   __float_as_int(d1.w)};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const int jj = 4 * hf + j;
                  const float x = __builtin_amdgcn_ldexpf(((float)kh[jj] + (float)kl[jj]) * df[j], dn[j]);
                  const float hi = bf16_round(x);
                  kh[jj] = (__bf16)hi;
                  kl[jj] = (__bf16)(x - hi);
                }
              }
            }
            const bf16x8 qh = *reinterpret_cast<const bf16x8*>(Qh + oa + k0);
            const bf16x8 ql = *reinterpret_cast<const bf16x8*>(Ql + oa + k0);
            const bf16x8 ep = *reinterpret_cast<const bf16x8*>(Ep + oa + k0);
            acc = mma32(kh, qh, acc);
            acct = mma32(kh, ep, acct);
            acc = mma32(kh, ql, acc);
            acc = mma32(kl, qh, acc);
          }
        }
        tile_store<DK, DV>(a, b, acc, acct, rec);
      }
    }
    __syncthreads();

    // ==== phase S(i): diagonal inverses; E^T, K_tail^T, Q_g into region X ==========
    if (itn < items) fetch(nrow0, nclen, nh, 3);
    const bool strong = *strongf != 0;  // uniform
    if (tid == 0) p.sflag[ri] = strong ? 1 : 0;
    nstrong += strong ? 1 : 0;
    if (*blocked || strong) {  // uniform; phase P has read the flags and the table
      __syncthreads();  // every thread has read the flags before they are cleared
      for (int e = tid; e < 6 * DK; e += NT) dsc[e] = make_float2(1.f, __int_as_float(0));
      if (tid == 0) *blocked = *strongf = 0;
    }
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
      inv_diag();
    }
    __syncthreads();

    // ==== phase S(ii): off-diagonal blocks of A ===================================
    if (itn < items) fetch(nrow0, nclen, nh, 4);
    phase_s2(rec, true);
    __syncthreads();

    // ==== phase Y: -Y and U into the record ======================================
    if (itn < items) fetch(nrow0, nclen, nh, 5);
    phase_y(rec);
    if (itn < items) fetch_decay(nh);
    clen = nclen;  // valid rows of the next item (the prologue masks the rest)
    __syncthreads();
  }
  }  // MODE != 2

  // ==== strong items, again: exact decay from the inputs ===========================
  // Every item of this workgroup that the main loop flagged (its flag was
  // written by this workgroup, before a barrier) is staged again from the
  // inputs; T and A_qk are formed entry by entry with the exact decay, E,
  // K_tail and Q_g from the uncentred G, and phases S and Y run as above.
  auto strong_item = [&](int ri) __attribute__((always_inline)) {
    long long frow0;
    int fclen, fh;
    locate(ri, frow0, fclen, fh);
    char* rec = p.rec + (size_t)ri * R::BYTES;
    strong_stage<DK, DV, LA16, PRO>(p, frow0, fclen, fh);
    __syncthreads();
    {
      const float* SG = reinterpret_cast<const float*>(smem + Cfg::O_SG);
      const KT* SK = reinterpret_cast<const KT*>(smem + Cfg::O_SK);
      const KT* SQ = reinterpret_cast<const KT*>(smem + Cfg::O_SQ);
      const ST* SB = reinterpret_cast<const ST*>(smem + Cfg::O_SB);
      for (int k = 0; k < 2; ++k) {
        const int ti = k == 0 ? wv : (wv == 0 ? 8 : wv == 2 ? 9 : -1);
        if (ti < 0) break;
        int a, b;
        tri_tile(ti, a, b);
        f32x4 acc, acct;
        strong_tile<DK, Cfg::LDG, LDK>(SG, SK, SQ, SB, scl, 16 * a + m, 16 * b + 4 * g4, acc, acct);
        tile_store<DK, DV>(a, b, acc, acct, rec);
      }
      // this thread's rows and channels (the phase-L layout) of Q_g = gamma q
      // and K_tail = (gamma_C / gamma) k go straight into their record
      // fragments; E = gamma b k waits in registers for region X
      float fe[RPT][EPC], kcol[EPC][RPT];
#pragma unroll
      for (int pr = 0; pr < RPT; ++pr) {
        const int r = r0 + pr;
        const float2 sc = *reinterpret_cast<const float2*>(scl + 2 * r);
        float qrow[EPC];
#pragma unroll
        for (int i = 0; i < EPC; ++i) {
          const int c = EPC * cg + i;
          const float gr = SG[r * Cfg::LDG + c], gam = exp2_fast(gr);
          const float kk = (float)SK[r * LDK + c] * sc.y;
          fe[pr][i] = gam * ((float)SB[r * LDK + c] * kk);
          qrow[i] = gam * ((float)SQ[r * LDK + c] * sc.x);
          kcol[i][pr] = exp2_fast(SG[(CH - 1) * Cfg::LDG + c] - gr) * kk;
        }
        // Q_g fragment (a, kb), lane (m, g4): channels 32 kb + 4 g4 + [0, 4)
        // (first half) or 32 kb + 16 + 4 g4 + [0, 4) (second half) of row 16 a + m
        const int c0 = EPC * cg, kb = c0 / 32, w = c0 % 32, half = w / 16, g4q = (w % 16) / 4;
        char* dq = rec + R::QG + ((size_t)((r / 16) * R::NKB + kb) * 64 + 16 * g4q + (r % 16)) * 16 + 8 * half;
        *reinterpret_cast<SV4*>(dq) = SV4{(ST)qrow[0], (ST)qrow[1], (ST)qrow[2], (ST)qrow[3]};
      }
      // K_tail fragment (ib, p), lane (m, g4): tokens 32 p + 4 g4 + [0, 4) (first
      // half) or 32 p + 16 + 4 g4 + [0, 4) (second half) of channel 16 ib + m;
      // this thread's RPT rows (RPT <= 4, aligned) are RPT of those 4 tokens
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        const int c = EPC * cg + i, pp = r0 / 32, w = r0 % 32, half = w / 16, g4k = (w % 16) / 4;
        ST* dk = reinterpret_cast<ST*>(rec + R::KT + ((size_t)((c / 16) * 2 + pp) * 64 + 16 * g4k + (c % 16)) * 16 +
                                       8 * half);
        stn<ST, RPT>(dk + r0 % 4, kcol[i]);
      }
      __syncthreads();  // the staged rows are read; region X takes E^T
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        float col[RPT];
#pragma unroll
        for (int pr = 0; pr < RPT; ++pr) col[pr] = fe[pr][i];
        stn<ST, RPT>(EhT + (EPC * cg + i) * LDC + r0, col);
      }
      inv_diag();
    }
    __syncthreads();
    phase_s2(rec, false);
    __syncthreads();
    phase_y(rec);
    __syncthreads();
  };
  if constexpr (MODE == 0) {
    for (int it = blockIdx.x; nstrong > 0 && it < items; it += gridDim.x) {
      const int ri = order(it);
      if (p.sflag[ri] == 0) continue;  // uniform
      --nstrong;
      strong_item(ri);
    }
  }
  if constexpr (MODE == 2) {
    // the flags of NT of this workgroup's items at a time, one per thread
    for (int base = blockIdx.x; base < items; base += gridDim.x * NT) {
      const int mine = base + tid * gridDim.x;
      if (__syncthreads_or(mine < items && p.sflag[order(mine)] != 0) == 0) continue;
      for (int j = 0; j < NT; ++j) {
        const int it = base + j * gridDim.x;
        if (it >= items) break;
        const int ri = order(it);
        if (p.sflag[ri] != 0) strong_item(ri);  // uniform
      }
    }
  }
}

size_t record_bytes(int dk, int dv) {
#define GDR2_REC(DK, DV) \
  if (dk == DK && dv == DV) return Rec<DK, DV>::BYTES;
  GDR2_REC(32, 32) GDR2_REC(32, 64) GDR2_REC(32, 128)
  GDR2_REC(64, 32) GDR2_REC(64, 64) GDR2_REC(64, 128)
  GDR2_REC(128, 32) GDR2_REC(128, 64) GDR2_REC(128, 128)
#undef GDR2_REC
  return 0;
}

template <int DK, int DV, bool LA16, int PRO, int MODE>
static hipError_t launch_intra_mode(const IntraArgs& a, long long grid, hipStream_t stream) {
  typedef IntraCfg<DK, DV> Cfg;
  static std::atomic<bool> lds_set[64];
  const hipError_t e =
      lds_opt_in(reinterpret_cast<const void*>(&intra_kernel<DK, DV, LA16, PRO, MODE>), Cfg::BYTES, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((intra_kernel<DK, DV, LA16, PRO, MODE>), dim3((unsigned)grid), dim3(NT), Cfg::BYTES, stream,
                     a);
  return hipGetLastError();
}

template <int DK, int DV, bool LA16, int PRO>
static hipError_t launch_intra1(const IntraArgs& a, hipStream_t stream) {
  const long long items = (long long)a.chunks * a.H;
  if (items <= 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const long long grid = items < cus ? items : cus;  // persistent: one workgroup per CU
  // the variants whose main loop is lightest keep the exact path in the same
  // launch; the others run it as a second launch
  if constexpr (LA16 && PRO == 0) {
    return launch_intra_mode<DK, DV, LA16, PRO, 0>(a, grid, stream);
  } else {
    e = launch_intra_mode<DK, DV, LA16, PRO, 1>(a, grid, stream);
    if (e != hipSuccess) return e;
    // the second launch reads the flags at run time: one instantiation serves
    // every prologue choice
    return launch_intra_mode<DK, DV, LA16, PRO == 0 ? 0 : PRO_ANY, 2>(a, grid, stream);
  }
}

hipError_t launch_intra(const IntraArgs& a, int dk, int dv, hipStream_t stream) {
  // the prologue variants: all three steps fixed at compile time, or any
  // other choice read at run time; grouped value heads need no variant of
  // their own (every variant reads key head h / grp)
  const bool pro = a.pro != 0;
#define GDR2_INTRA(DK, DV)                                                                  \
  if (dk == DK && dv == DV) {                                                               \
    if (pro && a.pro == PRO_ALL)                                                            \
      return a.la_bf16 ? launch_intra1<DK, DV, true, PRO_ALL>(a, stream)                    \
                       : launch_intra1<DK, DV, false, PRO_ALL>(a, stream);                  \
    if (pro)                                                                                \
      return a.la_bf16 ? launch_intra1<DK, DV, true, PRO_ANY>(a, stream)                    \
                       : launch_intra1<DK, DV, false, PRO_ANY>(a, stream);                  \
    return a.la_bf16 ? launch_intra1<DK, DV, true, 0>(a, stream)                            \
                     : launch_intra1<DK, DV, false, 0>(a, stream);                          \
  }
  GDR2_INTRA(32, 32) GDR2_INTRA(32, 64) GDR2_INTRA(32, 128)
  GDR2_INTRA(64, 32) GDR2_INTRA(64, 64) GDR2_INTRA(64, 128)
  GDR2_INTRA(128, 32) GDR2_INTRA(128, 64) GDR2_INTRA(128, 128)
#undef GDR2_INTRA
  return hipErrorInvalidValue;
}

}  // namespace gdr2
