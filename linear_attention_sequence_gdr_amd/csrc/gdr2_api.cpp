// gdr2_api.cpp -- the C ABI of libgdr2 (declared in include/gdr2.h).
//
// Every argument is validated on the host before any HIP call, so a rejected
// call touches no device memory and needs no GPU.  Valid calls enqueue their
// kernels on the caller's stream and return without synchronising.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "gdr2.h"
#include "gdr2_internal.h"

// Workspace of gdr2_chunk_fwd_noalloc: one static array per device that the
// library runs on, held until the process ends.  Host code never uses this
// name as an address (on the host it only stands for the symbol): the device
// address comes from hipGetSymbolAddress, once per device (scratch_address).
static __device__ __align__(256) unsigned char scratch[GDR2_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

gdr2_status fail(gdr2_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool dtype_ok(int t) { return t == GDR2_F32 || t == GDR2_BF16; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the two-pass forward (16-bit inputs): for packed sequences the
// longest-first order, the chunk base per sequence and the chunk table, then
// one record per (chunk, head).  Packed sequences add at most one partial
// chunk each, so ceil(T/64) + N chunks bound the record count.  Equal-length
// sequences with few (sequence, head) chains split each chain into P segments
// of segc chunks; they add the segments' transfer matrices and end states.
// Packed sequences with dk == dv and more than PSEG_MIN chunks in all may be
// split too, as the segment plan built on the device decides: they add the
// plan (per segment 4 ints, per sequence 2, and the count) and transfer
// matrices and end states for its largest possible number of segments,
// nsmax = N + cap / PSEG_MIN.
struct Layout {
  size_t order, cbase, tab, seg, sq, nseg, rec, phi, ex, sflag, total;
  long long cap;  // chunks with a record
  int P, segc;
  int nsmax;      // split packed sequences: segment capacity (0: never split)
};
Layout two_pass_layout(int B, int T, int H, int dk, int dv, int num_seqs) {
  Layout l{};
  const long long nc = ((long long)T + 63) / 64;
  size_t off = 0;
  l.P = 1;
  l.segc = (int)nc;
  if (num_seqs > 0) {
    l.cap = nc + num_seqs;
    l.order = off;
    off += align256(gdr2::schedule_bytes(num_seqs));
    l.cbase = off;
    off += align256(sizeof(int32_t) * ((size_t)num_seqs + 1));
    l.tab = off;
    off += align256(2 * sizeof(int32_t) * (size_t)l.cap);
    if (dk == dv && nc > gdr2::PSEG_MIN) {
      l.nsmax = (int)(num_seqs + l.cap / gdr2::PSEG_MIN);
      l.seg = off;
      off += align256(4 * sizeof(int32_t) * (size_t)l.nsmax);
      l.sq = off;
      off += align256(2 * sizeof(int32_t) * (size_t)num_seqs);
      l.nseg = off;
      off += 256;
    }
  } else {
    l.cap = (long long)B * nc;
    const int P = gdr2::segments_for((long long)B * H, nc, dk, dv);
    if (P > 1) {
      l.segc = (int)((nc + P - 1) / P);
      l.P = (int)((nc + l.segc - 1) / l.segc);
    }
  }
  l.rec = off;
  off += (size_t)l.cap * (size_t)H * gdr2::record_bytes(dk, dv);
  if (l.P > 1 || l.nsmax > 0) {
    const size_t chains = l.nsmax > 0 ? (size_t)l.nsmax * H : (size_t)B * l.P * H;
    l.phi = align256(off);
    l.ex = l.phi + chains * dk * dk * sizeof(float);
    off = l.ex + chains * dk * dv * sizeof(float);
  }
  // one int per record: its chunk needed the exact-decay path
  l.sflag = align256(off);
  off = l.sflag + (size_t)l.cap * (size_t)H * sizeof(int32_t);
  l.total = off;
  return l;
}

// Workspace of the backward: packed-sequence tables, then one fp32 block per
// (chunk, head) item, then from the next 256-byte boundary one int per item
// (its chunk took the exact-decay path).
struct BwdLayoutHost {
  size_t cbase, tab, items, sflag, total;
  long long cap;
};
BwdLayoutHost bwd_layout(int B, int T, int H, int dk, int dv, int num_seqs) {
  BwdLayoutHost l{};
  const long long nc = ((long long)T + 63) / 64;
  size_t off = 0;
  if (num_seqs > 0) {
    l.cap = nc + num_seqs;
    l.cbase = off;
    off += align256(sizeof(int32_t) * ((size_t)num_seqs + 1));
    l.tab = off;
    off += align256(2 * sizeof(int32_t) * (size_t)l.cap);
  } else {
    l.cap = (long long)B * nc;
  }
  l.items = off;
  off += (size_t)l.cap * (size_t)H * gdr2::bwd_item_bytes(dk, dv);
  l.sflag = align256(off);
  l.total = l.sflag + (size_t)l.cap * (size_t)H * sizeof(int32_t);
  return l;
}

// The two-pass forward (16-bit inputs), arguments already validated: Hv value
// heads (records, o, S0, S_T), Hk key heads (q, k, log_alpha, b).
gdr2_status two_pass(const char* fn, const void* q, const void* k, const void* v,
                     const void* log_alpha, const void* b, const void* w, const float* S0, void* o,
                     float* S_T, const int32_t* cu_seqlens, int N, int B, int T, int Hk, int Hv,
                     int dk, int dv, bool la_bf16, int pro, const float* da, const float* db,
                     float b_scale, float qk_eps, bool o_f32, char* ws, hipStream_t st) {
  // intra-chunk pass over all (chunk, value head) items, then the state pass
  const int ns = cu_seqlens ? N : 0;
  const Layout l = two_pass_layout(B, T, Hv, dk, dv, ns);
  int32_t* order = nullptr;
  int32_t* cbase = nullptr;
  int32_t* tab = nullptr;
  if (cu_seqlens) {
    cbase = reinterpret_cast<int32_t*>(ws + l.cbase);
    tab = reinterpret_cast<int32_t*>(ws + l.tab);
    if (gdr2::schedule_bytes(N)) {
      order = reinterpret_cast<int32_t*>(ws + l.order);
      const hipError_t e = gdr2::launch_schedule(cu_seqlens, N, T, order, st);
      if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: schedule launch: %s", fn, hipGetErrorString(e));
    }
    const hipError_t e = gdr2::launch_chunk_table(cu_seqlens, N, T, (int)l.cap, cbase, tab, st);
    if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: chunk table launch: %s", fn, hipGetErrorString(e));
    if (l.nsmax > 0) {
      // the segment plan balances the longest segment against the work per CU
      int dev = 0, cus = 256;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
      const hipError_t ep = gdr2::launch_segment_plan(
          cu_seqlens, N, T, order, cbase, Hv, cus, l.nsmax, reinterpret_cast<int32_t*>(ws + l.seg),
          reinterpret_cast<int32_t*>(ws + l.sq), reinterpret_cast<int32_t*>(ws + l.nseg), st);
      if (ep != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: segment plan launch: %s", fn, hipGetErrorString(ep));
    }
  }
  gdr2::IntraArgs ia;
  ia.q = q; ia.k = k; ia.v = v; ia.la = log_alpha; ia.b = b; ia.w = w;
  ia.rec = ws + l.rec;
  ia.sflag = reinterpret_cast<int*>(ws + l.sflag);
  ia.tab = tab;
  ia.total = cu_seqlens ? cbase + N : nullptr;
  ia.nc = (T + 63) / 64;
  ia.chunks = (int)l.cap;
  ia.T = T; ia.H = Hv;
  ia.la_bf16 = la_bf16;
  ia.Hk = Hk; ia.grp = Hv / Hk;
  ia.pro = pro; ia.da = da; ia.db = db; ia.b_scale = b_scale; ia.qk_eps = qk_eps;
  gdr2::StateArgs sa;
  sa.rec = ws + l.rec;
  sa.S0 = S0; sa.o = o; sa.o_f32 = o_f32 ? 1 : 0; sa.ST = S_T; sa.cu = cu_seqlens; sa.order = order; sa.cbase = cbase;
  sa.cap = (int)l.cap;
  sa.N = N; sa.T = T; sa.H = Hv; sa.DV = dv;
  sa.P = l.P; sa.segc = l.segc;
  const bool split = l.P > 1 || l.nsmax > 0;
  sa.phi = split ? reinterpret_cast<float*>(ws + l.phi) : nullptr;
  sa.ex = split ? reinterpret_cast<float*>(ws + l.ex) : nullptr;
  sa.seg = l.nsmax > 0 ? reinterpret_cast<const int32_t*>(ws + l.seg) : nullptr;
  sa.sq = l.nsmax > 0 ? reinterpret_cast<const int32_t*>(ws + l.sq) : nullptr;
  sa.nseg = l.nsmax > 0 ? reinterpret_cast<const int32_t*>(ws + l.nseg) : nullptr;
  sa.nsmax = l.nsmax;
  const hipError_t e = gdr2::launch_two_pass(ia, sa, dk, dv, st);
  if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: launch: %s", fn, hipGetErrorString(e));
  return GDR2_OK;
}

}  // namespace

extern "C" {

const char* gdr2_status_string(gdr2_status s) {
  switch (s) {
    case GDR2_OK: return "ok";
    case GDR2_E_NULL: return "a required pointer is NULL";
    case GDR2_E_SHAPE: return "invalid or inconsistent sizes";
    case GDR2_E_DTYPE: return "unknown dtype code";
    case GDR2_E_ALIGN: return "a base pointer is not 16-byte aligned";
    case GDR2_E_UNSUPPORTED: return "unsupported head dimension";
    case GDR2_E_WORKSPACE: return "workspace missing or too small";
    case GDR2_E_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* gdr2_last_error(void) { return g_err; }

int gdr2_version(void) { return 300; }

size_t gdr2_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs,
                                      gdr2_dtype in_dtype) {
  if (B <= 0 || T < 0 || H <= 0 || !dim_ok(dk) || !dim_ok(dv) || num_seqs < 0 ||
      !dtype_ok(in_dtype))
    return 0;
  if (in_dtype == GDR2_F32) return bwd_layout(B, T, H, dk, dv, num_seqs).total;
  const Layout l = two_pass_layout(B, T, H, dk, dv, num_seqs);
  return l.total;
}

}  // extern "C"

namespace {

// gdr2_chunk_fwd and gdr2_chunk_fwd_f32_out: o in in_dtype, or fp32 (o_f32).
// dry_run: validate every argument but the workspace, and return.
gdr2_status chunk_fwd_common(const char* fn, const void* q, const void* k, const void* v,
                             const void* log_alpha, const void* b, const void* w, const float* S0,
                             void* o, float* S_T, const int32_t* cu_seqlens, int num_seqs, int B,
                             int T, int H, int dk, int dv, gdr2_dtype in_dtype,
                             gdr2_dtype log_alpha_dtype, bool o_f32, void* workspace,
                             size_t workspace_bytes, void* stream, bool dry_run = false) {
  if (!q || !k || !v || !log_alpha || !b || !w || !o)
    return fail(GDR2_E_NULL, "%s: q, k, v, log_alpha, b, w and o must be non-NULL", fn);
  if (!dtype_ok(in_dtype) || !dtype_ok(log_alpha_dtype))
    return fail(GDR2_E_DTYPE, "%s: dtype codes %d/%d are not GDR2_F32 or GDR2_BF16", fn,
                (int)in_dtype, (int)log_alpha_dtype);
  if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
    return fail(GDR2_E_SHAPE, "%s: need B >= 1, T >= 0, H >= 1, dk, dv >= 1 (got B=%d T=%d H=%d dk=%d dv=%d)",
                fn, B, T, H, dk, dv);
  if (!dim_ok(dk) || !dim_ok(dv))
    return fail(GDR2_E_UNSUPPORTED, "%s: dk=%d dv=%d; each must be 32, 64 or 128", fn, dk, dv);
  const bool bf16 = in_dtype == GDR2_BF16;
  int N = B;
  if (cu_seqlens) {
    if (B != 1)
      return fail(GDR2_E_SHAPE, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
    if (num_seqs < 1)
      return fail(GDR2_E_SHAPE, "%s: num_seqs must be >= 1 with cu_seqlens, got %d", fn, num_seqs);
    N = num_seqs;
  }
  if ((long long)N * H > (1LL << 26))
    return fail(GDR2_E_SHAPE, "%s: N*H = %lld (sequence, head) pairs is too many", fn, (long long)N * H);
  const void* ptrs[] = {q, k, v, log_alpha, b, w, o, S0, S_T, cu_seqlens, workspace};
  const char* names[] = {"q", "k", "v", "log_alpha", "b", "w", "o", "S0", "S_T", "cu_seqlens", "workspace"};
  for (int i = 0; i < 11; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GDR2_E_ALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
  const int ns = cu_seqlens ? N : 0;
  const long long items =
      bf16 ? two_pass_layout(B, T, H, dk, dv, ns).cap * H : bwd_layout(B, T, H, dk, dv, ns).cap * H;
  if (items > 0x7fffffffLL)
    return fail(GDR2_E_SHAPE, "%s: %lld (chunk, head) items exceed 2^31 - 1", fn, items);
  if (dry_run) return GDR2_OK;
  const size_t need = gdr2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, ns, in_dtype);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GDR2_E_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu%s", fn, need,
                workspace_bytes, workspace ? "" : " (NULL)");

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (!bf16) {
    // fp32 inputs: the fp32 front pass per (chunk, head), then the sequential
    // pass per (sequence, head, 32 value channels) that forms o and S_T
    const BwdLayoutHost l = bwd_layout(B, T, H, dk, dv, ns);
    gdr2::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.b = b; a.w = w;
    a.S0 = S0; a.o = static_cast<float*>(o); a.ST = S_T;
    a.ws = reinterpret_cast<float*>(ws + l.items);
    a.sflag = reinterpret_cast<int*>(ws + l.sflag);
    if (cu_seqlens) {
      int32_t* cbase = reinterpret_cast<int32_t*>(ws + l.cbase);
      int32_t* tab = reinterpret_cast<int32_t*>(ws + l.tab);
      const hipError_t e = gdr2::launch_chunk_table(cu_seqlens, N, T, (int)l.cap, cbase, tab, st);
      if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: chunk table launch: %s", fn, hipGetErrorString(e));
      a.tab = tab; a.cbase = cbase; a.total = cbase + N;
    }
    a.nc = (T + 63) / 64;
    a.chunks = (int)l.cap;
    a.N = N; a.T = T; a.H = H;
    a.in_bf16 = 0;
    a.la_bf16 = log_alpha_dtype == GDR2_BF16;
    const hipError_t e = gdr2::launch_fwd32(a, dk, dv, st);
    if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: launch: %s", fn, hipGetErrorString(e));
    return GDR2_OK;
  }

  return two_pass(fn, q, k, v, log_alpha, b, w, S0, o, S_T, cu_seqlens, N, B, T, H, H, dk, dv,
                  log_alpha_dtype == GDR2_BF16, 0, nullptr, nullptr, 1.f, 0.f, o_f32, ws, st);
}

// The device address of this device's static scratch, looked up once per
// device with that device current (each device holds its own copy).
constexpr int SCRATCH_DEVICES = 64;
std::once_flag g_scratch_once[SCRATCH_DEVICES];
void* g_scratch_addr[SCRATCH_DEVICES];
hipError_t g_scratch_err[SCRATCH_DEVICES];

hipError_t scratch_address(void** addr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_addr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

gdr2_status gdr2_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const void* log_alpha, const void* b, const void* w,
                                   const float* S0, void* o, float* S_T,
                                   const int32_t* cu_seqlens, int num_seqs, int B, int T, int H,
                                   int dk, int dv, gdr2_dtype in_dtype,
                                   gdr2_dtype log_alpha_dtype, void* stream) {
  const char* fn = "gdr2_chunk_fwd_noalloc";
  gdr2_status st = chunk_fwd_common(fn, q, k, v, log_alpha, b, w, S0, o, S_T, cu_seqlens, num_seqs,
                                    B, T, H, dk, dv, in_dtype, log_alpha_dtype, in_dtype == GDR2_F32,
                                    nullptr, 0, stream, true);
  if (st != GDR2_OK) return st;
  const size_t need = gdr2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, cu_seqlens ? num_seqs : 0, in_dtype);
  if (need > (size_t)GDR2_NOALLOC_SCRATCH_BYTES)
    return fail(GDR2_E_WORKSPACE,
                "%s: these sizes need %zu bytes of workspace, more than the %zu bytes of static "
                "scratch (use gdr2_chunk_fwd with a workspace)",
                fn, need, (size_t)GDR2_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess)
    return fail(GDR2_E_LAUNCH, "%s: address of the static scratch: %s", fn, hipGetErrorString(e));
  return chunk_fwd_common(fn, q, k, v, log_alpha, b, w, S0, o, S_T, cu_seqlens, num_seqs, B, T, H, dk,
                          dv, in_dtype, log_alpha_dtype, in_dtype == GDR2_F32, ws,
                          (size_t)GDR2_NOALLOC_SCRATCH_BYTES, stream);
}

gdr2_status gdr2_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* b, const void* w, const float* S0, void* o, float* S_T,
                           const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int dk,
                           int dv, gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_common("gdr2_chunk_fwd", q, k, v, log_alpha, b, w, S0, o, S_T, cu_seqlens,
                          num_seqs, B, T, H, dk, dv, in_dtype, log_alpha_dtype,
                          in_dtype == GDR2_F32, workspace, workspace_bytes, stream);
}

gdr2_status gdr2_chunk_fwd_f32_out(const void* q, const void* k, const void* v,
                                   const void* log_alpha, const void* b, const void* w,
                                   const float* S0, float* o, float* S_T,
                                   const int32_t* cu_seqlens, int num_seqs, int B, int T, int H,
                                   int dk, int dv, gdr2_dtype in_dtype,
                                   gdr2_dtype log_alpha_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return chunk_fwd_common("gdr2_chunk_fwd_f32_out", q, k, v, log_alpha, b, w, S0, o, S_T,
                          cu_seqlens, num_seqs, B, T, H, dk, dv, in_dtype, log_alpha_dtype, true,
                          workspace, workspace_bytes, stream);
}

gdr2_status gdr2_chunk_fwd_block(const void* q, const void* k, const void* v, const void* f,
                                 const void* b, const void* w, const float* decay_a,
                                 const float* decay_bias, unsigned flags, float b_scale,
                                 float qk_eps, const float* S0, void* o, float* S_T,
                                 const int32_t* cu_seqlens, int num_seqs, int B, int T, int H,
                                 int Hv, int dk, int dv, gdr2_dtype f_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const char* fn = "gdr2_chunk_fwd_block";
  if (!q || !k || !v || !f || !b || !w || !o)
    return fail(GDR2_E_NULL, "%s: q, k, v, f, b, w and o must be non-NULL", fn);
  if ((flags & GDR2_PRO_DECAY) && (!decay_a || !decay_bias))
    return fail(GDR2_E_NULL, "%s: GDR2_PRO_DECAY needs decay_a and decay_bias", fn);
  if (!dtype_ok(f_dtype))
    return fail(GDR2_E_DTYPE, "%s: f dtype code %d is not GDR2_F32 or GDR2_BF16", fn, (int)f_dtype);
  if (flags & ~(unsigned)(GDR2_PRO_QK_L2NORM | GDR2_PRO_DECAY | GDR2_PRO_GATES))
    return fail(GDR2_E_UNSUPPORTED, "%s: unknown flag bits 0x%x", fn, flags);
  if (B <= 0 || T < 0 || H <= 0 || Hv <= 0 || dk <= 0 || dv <= 0)
    return fail(GDR2_E_SHAPE, "%s: need B >= 1, T >= 0, H, Hv, dk, dv >= 1 (got B=%d T=%d H=%d Hv=%d dk=%d dv=%d)",
                fn, B, T, H, Hv, dk, dv);
  if (Hv % H != 0)
    return fail(GDR2_E_SHAPE, "%s: Hv=%d must be a multiple of H=%d", fn, Hv, H);
  if (!dim_ok(dk) || !dim_ok(dv))
    return fail(GDR2_E_UNSUPPORTED, "%s: dk=%d dv=%d; each must be 32, 64 or 128", fn, dk, dv);
  if ((flags & GDR2_PRO_GATES) && !isfinite(b_scale))
    return fail(GDR2_E_SHAPE, "%s: b_scale must be finite (got %g)", fn, (double)b_scale);
  if ((flags & GDR2_PRO_QK_L2NORM) && !(qk_eps >= 0.f && isfinite(qk_eps)))
    return fail(GDR2_E_SHAPE, "%s: qk_eps must be finite and >= 0 (got %g)", fn, (double)qk_eps);
  int N = B;
  if (cu_seqlens) {
    if (B != 1) return fail(GDR2_E_SHAPE, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
    if (num_seqs < 1) return fail(GDR2_E_SHAPE, "%s: num_seqs must be >= 1 with cu_seqlens, got %d", fn, num_seqs);
    N = num_seqs;
  }
  if ((long long)N * Hv > (1LL << 26))
    return fail(GDR2_E_SHAPE, "%s: N*Hv = %lld (sequence, head) pairs is too many", fn, (long long)N * Hv);
  const void* ptrs[] = {q, k, v, f, b, w, o, S0, S_T, cu_seqlens, workspace, decay_a, decay_bias};
  const char* names[] = {"q", "k", "v", "f", "b", "w", "o", "S0", "S_T", "cu_seqlens", "workspace",
                         "decay_a", "decay_bias"};
  for (int i = 0; i < 13; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GDR2_E_ALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
  const int ns = cu_seqlens ? N : 0;
  const Layout l = two_pass_layout(B, T, Hv, dk, dv, ns);
  if (l.cap * Hv > 0x7fffffffLL)
    return fail(GDR2_E_SHAPE, "%s: %lld (chunk, head) items exceed 2^31 - 1", fn, l.cap * Hv);
  const size_t need = gdr2_chunk_fwd_workspace_bytes(B, T, Hv, dk, dv, ns, GDR2_BF16);
  if (need && (!workspace || workspace_bytes < need))
    return fail(GDR2_E_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu%s", fn, need,
                workspace_bytes, workspace ? "" : " (NULL)");
  return two_pass(fn, q, k, v, f, b, w, S0, o, S_T, cu_seqlens, N, B, T, H, Hv, dk, dv,
                  f_dtype == GDR2_BF16, (int)flags, decay_a, decay_bias, b_scale, qk_eps, false,
                  static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}


size_t gdr2_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs) {
  if (B <= 0 || T < 0 || H <= 0 || !dim_ok(dk) || !dim_ok(dv) || num_seqs < 0) return 0;
  return bwd_layout(B, T, H, dk, dv, num_seqs).total;
}

gdr2_status gdr2_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* b, const void* w, const float* S0, const void* dO,
                           const float* dS_T, float* dq, float* dk, float* dv, float* dlog_alpha,
                           float* db, float* dw, float* dS0, const int32_t* cu_seqlens,
                           int num_seqs, int B, int T, int H, int dk_, int dv_, gdr2_dtype in_dtype,
                           gdr2_dtype log_alpha_dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const char* fn = "gdr2_chunk_bwd";
  if (T != 0 &&
      (!q || !k || !v || !log_alpha || !b || !w || !dO || !dq || !dk || !dv || !dlog_alpha || !db || !dw))
    return fail(GDR2_E_NULL, "%s: inputs, dO and every input gradient must be non-NULL", fn);
  if (!dtype_ok(in_dtype) || !dtype_ok(log_alpha_dtype))
    return fail(GDR2_E_DTYPE, "%s: dtype codes %d/%d are not GDR2_F32 or GDR2_BF16", fn, (int)in_dtype,
                (int)log_alpha_dtype);
  if (B <= 0 || T < 0 || H <= 0 || dk_ <= 0 || dv_ <= 0)
    return fail(GDR2_E_SHAPE, "%s: need B >= 1, T >= 0, H >= 1, dk, dv >= 1 (got B=%d T=%d H=%d dk=%d dv=%d)",
                fn, B, T, H, dk_, dv_);
  if (!dim_ok(dk_) || !dim_ok(dv_))
    return fail(GDR2_E_UNSUPPORTED, "%s: dk=%d dv=%d; each must be 32, 64 or 128", fn, dk_, dv_);
  int N = B;
  if (cu_seqlens) {
    if (B != 1) return fail(GDR2_E_SHAPE, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
    if (num_seqs < 1) return fail(GDR2_E_SHAPE, "%s: num_seqs must be >= 1 with cu_seqlens, got %d", fn, num_seqs);
    N = num_seqs;
  }
  if ((long long)N * H > (1LL << 26))
    return fail(GDR2_E_SHAPE, "%s: N*H = %lld (sequence, head) pairs is too many", fn, (long long)N * H);
  const void* ptrs[] = {q, k, v, log_alpha, b, w, S0, dO, dS_T, dq, dk, dv, dlog_alpha, db, dw, dS0,
                        cu_seqlens, workspace};
  const char* names[] = {"q", "k", "v", "log_alpha", "b", "w", "S0", "dO", "dS_T", "dq", "dk", "dv",
                         "dlog_alpha", "db", "dw", "dS0", "cu_seqlens", "workspace"};
  for (int i = 0; i < 18; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GDR2_E_ALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
  const int ns = cu_seqlens ? N : 0;
  const BwdLayoutHost l = bwd_layout(B, T, H, dk_, dv_, ns);
  if (l.cap * H > 0x7fffffffLL)
    return fail(GDR2_E_SHAPE, "%s: %lld (chunk, head) items exceed 2^31 - 1", fn, l.cap * H);
  if (!workspace || workspace_bytes < l.total)
    return fail(GDR2_E_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu%s", fn, l.total,
                workspace_bytes, workspace ? "" : " (NULL)");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  gdr2::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.b = b; a.w = w; a.dO = dO;
  a.S0 = S0; a.dST = dS_T;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dlog_alpha; a.db = db; a.dw = dw; a.dS0 = dS0;
  a.ws = reinterpret_cast<float*>(ws + l.items);
  a.sflag = reinterpret_cast<int*>(ws + l.sflag);
  if (cu_seqlens) {
    int32_t* cbase = reinterpret_cast<int32_t*>(ws + l.cbase);
    int32_t* tab = reinterpret_cast<int32_t*>(ws + l.tab);
    const hipError_t e = gdr2::launch_chunk_table(cu_seqlens, N, T, (int)l.cap, cbase, tab, st);
    if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: chunk table launch: %s", fn, hipGetErrorString(e));
    a.tab = tab; a.cbase = cbase; a.total = cbase + N;
  }
  a.nc = (T + 63) / 64;
  a.chunks = (int)l.cap;
  a.N = N; a.T = T; a.H = H;
  a.in_bf16 = in_dtype == GDR2_BF16;
  a.la_bf16 = log_alpha_dtype == GDR2_BF16;
  const hipError_t e = gdr2::launch_bwd(a, dk_, dv_, st);
  if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: launch: %s", fn, hipGetErrorString(e));
  return GDR2_OK;
}

namespace {

gdr2_status decode_common(const char* fn, const void* q, const void* k, const void* v,
                          const void* log_alpha, const void* b, const void* w, float* S, void* o,
                          const void* z, const float* nw, float eps, bool gated, int N, int H,
                          int dk, int dv, gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype,
                          void* stream) {
  const char* out = gated ? "y" : "o";
  if (!q || !k || !v || !log_alpha || !b || !w || !S || !o || (gated && !z))
    return fail(GDR2_E_NULL, "%s: q, k, v, log_alpha, b, w, S%s and %s must be non-NULL", fn,
                gated ? ", z" : "", out);
  if (!dtype_ok(in_dtype) || !dtype_ok(log_alpha_dtype))
    return fail(GDR2_E_DTYPE, "%s: dtype codes %d/%d are not GDR2_F32 or GDR2_BF16", fn,
                (int)in_dtype, (int)log_alpha_dtype);
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0)
    return fail(GDR2_E_SHAPE, "%s: need N >= 0, H >= 1, dk, dv >= 1 (got N=%d H=%d dk=%d dv=%d)",
                fn, N, H, dk, dv);
  if (!dim_ok(dk) || !dim_ok(dv))
    return fail(GDR2_E_UNSUPPORTED, "%s: dk=%d dv=%d; each must be 32, 64 or 128", fn, dk, dv);
  if ((long long)N * H > 0x7fffffffLL)
    return fail(GDR2_E_SHAPE, "%s: N*H = %lld is too many", fn, (long long)N * H);
  if (gated && !(eps >= 0.f && isfinite(eps)))
    return fail(GDR2_E_SHAPE, "%s: eps must be finite and >= 0 (got %g)", fn, (double)eps);
  const void* ptrs[] = {q, k, v, log_alpha, b, w, S, o, z, nw};
  const char* names[] = {"q", "k", "v", "log_alpha", "b", "w", "S", out, "z", "norm_weight"};
  for (int i = 0; i < 10; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GDR2_E_ALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
  gdr2::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.b = b; a.w = w;
  a.S = S; a.o = o; a.N = N; a.H = H;
  a.la_bf16 = log_alpha_dtype == GDR2_BF16;
  a.z = gated ? z : nullptr;
  a.nw = gated ? nw : nullptr;
  a.eps = gated ? eps : 0.f;
  a.gated = gated ? 1 : 0;
  const hipError_t e = gdr2::launch_decode(a, dk, dv, in_dtype == GDR2_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: launch: %s", fn, hipGetErrorString(e));
  return GDR2_OK;
}

}  // namespace

gdr2_status gdr2_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                             const void* b, const void* w, float* S, void* o, int N, int H, int dk,
                             int dv, gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype, void* stream) {
  return decode_common("gdr2_decode_step", q, k, v, log_alpha, b, w, S, o, nullptr, nullptr, 0.f,
                       false, N, H, dk, dv, in_dtype, log_alpha_dtype, stream);
}

gdr2_status gdr2_decode_step_norm_gate(const void* q, const void* k, const void* v,
                                       const void* log_alpha, const void* b, const void* w,
                                       float* S, const void* z, const float* norm_weight, float eps,
                                       void* y, int N, int H, int dk, int dv, gdr2_dtype in_dtype,
                                       gdr2_dtype log_alpha_dtype, void* stream) {
  return decode_common("gdr2_decode_step_norm_gate", q, k, v, log_alpha, b, w, S, y, z, norm_weight,
                       eps, true, N, H, dk, dv, in_dtype, log_alpha_dtype, stream);
}

gdr2_status gdr2_norm_gate(const void* o, const void* z, const float* weight, void* y,
                           long long rows, int d, int group, float eps, gdr2_dtype dtype,
                           void* stream) {
  const char* fn = "gdr2_norm_gate";
  if (rows > 0 && (!o || !z || !y)) return fail(GDR2_E_NULL, "%s: o, z and y must be non-NULL", fn);
  if (!dtype_ok(dtype)) return fail(GDR2_E_DTYPE, "%s: dtype code %d is not GDR2_F32 or GDR2_BF16", fn, (int)dtype);
  if (rows < 0 || d <= 0 || group <= 0)
    return fail(GDR2_E_SHAPE, "%s: need rows >= 0, d >= 1, group >= 1 (got rows=%lld d=%d group=%d)", fn,
                rows, d, group);
  if (group % 8 != 0 || group > GDR2_NORM_GATE_MAX_GROUP || d % group != 0)
    return fail(GDR2_E_SHAPE, "%s: group=%d must be a multiple of 8, at most %d, and divide d=%d", fn,
                group, GDR2_NORM_GATE_MAX_GROUP, d);
  if (!(eps >= 0.f && isfinite(eps)))
    return fail(GDR2_E_SHAPE, "%s: eps must be finite and >= 0 (got %g)", fn, (double)eps);
  const long long period = d / group;
  if (rows > (1LL << 62) / d || gdr2::norm_gate_blocks(rows * period, group) > 0x7fffffffLL)
    return fail(GDR2_E_SHAPE, "%s: rows=%lld x d=%d is too large for one launch", fn, rows, d);
  const void* ptrs[] = {o, z, y, weight};
  const char* names[] = {"o", "z", "y", "weight"};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(GDR2_E_ALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
  gdr2::NormGateArgs a{};
  a.o = o; a.z = z; a.weight = weight; a.y = y;
  a.groups = rows * period;
  a.group = group;
  a.period = (int)period;
  a.eps = eps;
  const hipError_t e = gdr2::launch_norm_gate(a, dtype == GDR2_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDR2_E_LAUNCH, "%s: launch: %s", fn, hipGetErrorString(e));
  return GDR2_OK;
}

}  // extern "C"
