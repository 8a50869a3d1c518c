// gdr2_internal.h -- host-side launch interface between the C ABI (gdr2_api.cpp)
// and the kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace gdr2 {

// Raises `kernel`'s dynamic LDS limit to `bytes` on the current device the
// first time it is launched there.  `done` is that kernel's own per-device
// flag array (64 devices; others set the attribute on every call).  The flags
// are atomic: first calls from several threads may each set the attribute,
// which is idempotent, but never race on a flag.
inline hipError_t lds_opt_in(const void* kernel, size_t bytes, std::atomic<bool>* done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool slot = dev >= 0 && dev < 64;
  if (slot && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && slot) done[dev].store(true, std::memory_order_release);
  return e;
}

struct DecodeArgs {
  const void *q, *k, *v, *la, *b, *w;
  float* S;
  void* o;
  int N, H;
  int la_bf16;
  // Output epilogue applied before o is stored (gated != 0): o becomes
  // RMSNorm(o) over dv, times nw (fp32 [dv], or NULL for ones), times silu(z).
  const void* z;
  const float* nw;
  float eps;
  int gated;
};

// Output epilogue over `groups` groups of `group` channels (a multiple of 8).
// `period` = channels per row / group: the weight (fp32, one entry per channel
// of a row, or NULL) is indexed by (group index % period) * group + channel.
struct NormGateArgs {
  const void *o, *z;
  const float* weight;
  void* y;
  long long groups;
  int group, period;
  float eps;
  float inv_group;  // set by launch_norm_gate
  int lanes;        // set by launch_norm_gate
};

// ---- two-pass chunkwise forward (16-bit inputs) ------------------------------------
//
// The intra-chunk pass writes one record per (chunk, head); the state pass
// reads them in chunk order.  Record r = chunk_index * H + head.  Every matrix
// in a record is fp16 and stored as MFMA operand fragments: 64 lanes x 16 B
// (8 halves) for the A/B operands of a 16x16x32 product, 64 lanes x 8 B (4
// halves) for an accumulator-layout tile.  Lane l = 16*g + m.
//   YN [a][kb]  (a < 4, kb < DK/32)  lane: -Y[16a+m][32kb+4g+j], -Y[16a+m][32kb+16+4g+j]  (j < 4)
//   QG [a][kb]                       lane:  Qg[16a+m][...same columns...]
//   KT [ib][p]  (ib < DK/16, p < 2)  lane:  Kt[32p+4g+j][16ib+m], Kt[32p+16+4g+j][16ib+m]
//   AQK (a, p), p <= a/2 (6 tiles)   lane:  Aqk[16a+m][32p+4g+j], Aqk[16a+m][32p+16+4g+j]
//   GC          fp32 [DK]                   gamma_C per key channel
//   U  [jt][a]  (jt < DV/16)         lane:  U[16a+4g+q][16jt+m]  (q < 4, accumulator layout)
// Everything before U is shared by all value channels; U is last so that a
// block of value channels reads one contiguous range of it.
template <int DK, int DV>
struct Rec {
  static constexpr int NKB = DK / 32, NIB = DK / 16, NJT = DV / 16;
  static constexpr size_t FRAG = 1024, TILE = 512;
  static constexpr size_t YN = 0;
  static constexpr size_t QG = YN + 4 * NKB * FRAG;
  static constexpr size_t KT = QG + 4 * NKB * FRAG;
  static constexpr size_t AQK = KT + NIB * 2 * FRAG;
  static constexpr size_t GC = AQK + 6 * FRAG;
  static constexpr size_t U = GC + DK * 4;
  static constexpr size_t BYTES = U + NJT * 4 * TILE;
};
size_t record_bytes(int dk, int dv);

// Packed-sequence tables for the two-pass forward: cbase[n] = index of the
// first chunk of sequence n (cbase[N] = total chunks), tab[2c], tab[2c+1] =
// first token row and length of chunk c.
// Gate prologue flags (the values of the public GDR2_PRO_* flags).
enum { PRO_QK_L2NORM = 1, PRO_DECAY = 2, PRO_GATES = 4 };

struct IntraArgs {
  const void *q, *k, *v, *la, *b, *w;
  char* rec;
  int* sflag;             // per record: 1 when its chunk's decay needs the exact path
  const int32_t* tab;     // packed sequences: per chunk (row, length); else nullptr
  const int32_t* total;   // packed sequences: device total chunk count; else nullptr
  int nc;                 // chunks per sequence (equal-length sequences)
  int chunks;             // total chunks (equal-length) or an upper bound (packed)
  int T, H;               // H: value heads (one record per chunk and value head)
  int la_bf16;
  // Grouped value heads: q, k, la, b have Hk heads and value head h reads key
  // head h / grp (H = Hk * grp).  The plain forward has Hk = H, grp = 1.
  int Hk, grp;
  // Gate prologue, applied to the loaded inputs (pro = 0: none).
  int pro;                // PRO_* flags
  const float* da;        // PRO_DECAY: a, fp32 [Hk][DK]
  const float* db;        // PRO_DECAY: delta, fp32 [Hk][DK]
  float b_scale;          // PRO_GATES: b = b_scale * sigmoid(b)
  float qk_eps;           // PRO_QK_L2NORM: x / sqrt(sum(x^2) + qk_eps)
};
struct StateArgs {
  const char* rec;
  const float* S0;
  void* o;                // bf16, or fp32 when o_f32
  int o_f32;
  float* ST;
  const int32_t* cu;      // device [N+1] or nullptr
  const int32_t* order;   // longest-first schedule or nullptr
  const int32_t* cbase;   // packed sequences: first chunk per sequence; else nullptr
  int cap;                // records available (chunks); chunks past it are skipped
  int N, T, H, DV;
  // Split chains (equal-length sequences, dk == dv, P > 1): the chunks of
  // each sequence form P segments of segc chunks (the last may be shorter).
  // A transfer pass gives every segment but the last its transfer matrix
  // (phi, fp32 [N][P][H][dk][dk]) and its end state from a zero start (ex,
  // fp32 [N][P][H][dk][dv]; segment 0 starts from S0 instead).  A scan turns
  // ex[s] into the true end state of segment s, and the state pass then runs
  // every segment at once, segment s > 0 starting from ex[s - 1].
  int P, segc;
  float* phi;
  float* ex;
  // Split packed sequences (cu set, seg set): sequence n's chunks form sq[2n+1]
  // segments with global ids sq[2n] + [0, sq[2n+1]), numbered in schedule
  // order; segment g (g < *nseg <= nsmax) is seg[4g..4g+3] = (sequence, first
  // chunk within the sequence, chunks, the sequence's first segment id).  phi
  // and ex are then [nsmax][H][..], indexed by (segment id, head).
  const int32_t* seg;
  const int32_t* sq;
  const int32_t* nseg;
  int nsmax;
};
hipError_t launch_two_pass(const IntraArgs& ia, const StateArgs& sa, int dk, int dv, hipStream_t stream);
// Segments per sequence for the state pass of `chains` equal-length
// (sequence, value head) chains of nc chunks each (1 = no split).  It depends
// on the shape only, so the workspace size can be computed without a device.
int segments_for(long long chains, long long nc, int dk, int dv);

// ---- backward ------------------------------------------------------------------------
// One fp32 workspace block of bwd_item_bytes() per (chunk, head) item, item =
// chunk_index * H + head; chunk indices as in the two-pass forward.
struct BwdArgs {
  const void *q, *k, *v, *la, *b, *w, *dO;
  const float *S0, *dST;
  float *dq, *dk, *dv, *dg, *db, *dw, *dS0;
  float *o, *ST;          // the fp32 forward's outputs (launch_fwd32); unused by the backward
  float* ws;
  int* sflag;             // per item: its chunk took the exact-decay path (written by the front pass)
  const int32_t* tab;     // packed sequences: per chunk (row, length); else nullptr
  const int32_t* cbase;   // packed sequences: first chunk per sequence, [N+1]
  const int32_t* total;   // packed sequences: cbase + N
  int nc, chunks, N, T, H;
  int in_bf16, la_bf16;
};
size_t bwd_item_bytes(int dk, int dv);
hipError_t launch_bwd(const BwdArgs& a, int dk, int dv, hipStream_t stream);
// The forward for fp32 inputs, on the backward's fp32 front pass and the
// forward variant of its sequential state pass: q..w, S0, o (fp32), ST, the
// packed-sequence tables and the workspace as for the backward.
hipError_t launch_fwd32(const BwdArgs& a, int dk, int dv, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, int dk, int dv, bool bf16, hipStream_t stream);

hipError_t launch_norm_gate(NormGateArgs a, bool bf16, hipStream_t stream);
// Lanes per group and 256-thread blocks of the epilogue launch (host-side
// bounds checks use them).
int norm_gate_lanes(int group);
long long norm_gate_blocks(long long groups, int group);


// Schedule: a permutation of the N packed sequences, longest first, written
// into `order` (device int32 [N]) from cu_seqlens.  `scratch` holds N int32.
hipError_t launch_schedule(const int32_t* cu, int N, int T, int32_t* order, hipStream_t stream);
size_t schedule_bytes(int N);
// cbase (int32 [N+1]) and tab (int32 [2 * chunks]) of packed sequences.
hipError_t launch_chunk_table(const int32_t* cu, int N, int T, int cap, int32_t* cbase, int32_t* tab,
                              hipStream_t stream);
constexpr int SCHED_MAX = 4096;  // sequences the longest-first sort handles
// Segment plan of packed sequences for the split state pass (StateArgs::seg):
// sequence n of nc_n chunks gets P_n = ceil(nc_n / L) segments of balanced
// length, L = max(PSEG_MIN, ceil(total chunks * H / slots), ceil(sqrt(2 * the
// longest nc_n))); reads cbase[N] (the chunk total) from the chunk table and
// `order` (or the identity when NULL).  At most N + cap / PSEG_MIN segments.
constexpr int PSEG_MIN = 32;
hipError_t launch_segment_plan(const int32_t* cu, int N, int T, const int32_t* order, const int32_t* cbase,
                               int H, int slots, int nsmax, int32_t* seg, int32_t* sq, int32_t* nseg,
                               hipStream_t stream);

}  // namespace gdr2
