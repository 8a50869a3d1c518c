// Host-side driver of libgdr2's C ABI for the AddressSanitizer /
// UndefinedBehaviorSanitizer build of gdr2_api.cpp (tests/test_api_sanitizers.py).
// It makes only calls that the library must reject on the host, plus the
// size queries and the string functions, so no device is touched: device
// pointers are fake addresses that are never dereferenced.  Each call's
// status must be the one include/gdr2.h documents, and the thread-local
// detail must name the entry point.  Prints "ok" when every check passed.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdr2.h"

static int failures = 0;

static void expect(int got, int want, const char* fn, const char* what) {
  const char* err = gdr2_last_error();
  if (got != want) {
    printf("FAIL %s (%s): status %d, expected %d (%s)\n", fn, what, got, want, err ? err : "");
    ++failures;
  } else if (want != GDR2_OK && (!err || strncmp(err, fn, strlen(fn)) != 0)) {
    printf("FAIL %s (%s): detail \"%s\" does not name the entry point\n", fn, what, err ? err : "");
    ++failures;
  }
}

static void* const A = (void*)0x10000;    // 16-byte aligned fake device address
static void* const MIS = (void*)0x10008;  // misaligned

struct Fwd {
  const void *q = A, *k = A, *v = A, *la = A, *b = A, *w = A;
  const float* S0 = nullptr;
  void* o = A;
  float* ST = nullptr;
  const int32_t* cu = nullptr;
  int ns = 0, B = 2, T = 100, H = 4, dk = 128, dv = 128;
  gdr2_dtype dt = GDR2_BF16, ldt = GDR2_BF16;
  void* ws = nullptr;
  size_t wsb = 0;
  int run() const {
    return gdr2_chunk_fwd(q, k, v, la, b, w, S0, o, ST, cu, ns, B, T, H, dk, dv, dt, ldt, ws, wsb, nullptr);
  }
  int run_f32() const {
    return gdr2_chunk_fwd_f32_out(q, k, v, la, b, w, S0, (float*)o, ST, cu, ns, B, T, H, dk, dv, dt, ldt, ws,
                                  wsb, nullptr);
  }
  int run_noalloc() const {
    return gdr2_chunk_fwd_noalloc(q, k, v, la, b, w, S0, o, ST, cu, ns, B, T, H, dk, dv, dt, ldt, nullptr);
  }
};

static void chunk_fwd_cases() {
  struct Case { const char* what; Fwd f; int want; };
  Case cases[32];
  int n = 0;
  auto add = [&](const char* what, Fwd f, int want) { cases[n++] = Case{what, f, want}; };
  Fwd f;
  { Fwd x = f; x.q = nullptr; add("q NULL", x, GDR2_E_NULL); }
  { Fwd x = f; x.o = nullptr; add("o NULL", x, GDR2_E_NULL); }
  { Fwd x = f; x.la = nullptr; add("log_alpha NULL", x, GDR2_E_NULL); }
  { Fwd x = f; x.dt = (gdr2_dtype)7; add("dtype 7", x, GDR2_E_DTYPE); }
  { Fwd x = f; x.ldt = (gdr2_dtype)-1; add("log_alpha dtype -1", x, GDR2_E_DTYPE); }
  { Fwd x = f; x.B = 0; add("B 0", x, GDR2_E_SHAPE); }
  { Fwd x = f; x.T = -1; add("T -1", x, GDR2_E_SHAPE); }
  { Fwd x = f; x.H = 0; add("H 0", x, GDR2_E_SHAPE); }
  { Fwd x = f; x.dk = 0; add("dk 0", x, GDR2_E_SHAPE); }
  { Fwd x = f; x.dk = 48; add("dk 48", x, GDR2_E_UNSUPPORTED); }
  { Fwd x = f; x.dv = 256; add("dv 256", x, GDR2_E_UNSUPPORTED); }
  { Fwd x = f; x.dt = GDR2_F32; add("fp32 without workspace", x, GDR2_E_WORKSPACE); }
  { Fwd x = f; x.cu = (const int32_t*)A; x.ns = 3; add("cu_seqlens with B 2", x, GDR2_E_SHAPE); }
  { Fwd x = f; x.cu = (const int32_t*)A; x.B = 1; x.ns = 0; add("cu_seqlens with 0 sequences", x, GDR2_E_SHAPE); }
  { Fwd x = f; x.q = MIS; add("q misaligned", x, GDR2_E_ALIGN); }
  { Fwd x = f; x.S0 = (const float*)MIS; add("S0 misaligned", x, GDR2_E_ALIGN); }
  { Fwd x = f; x.cu = (const int32_t*)MIS; x.B = 1; x.ns = 3; add("cu_seqlens misaligned", x, GDR2_E_ALIGN); }
  { Fwd x = f; x.cu = (const int32_t*)A; x.B = 1; x.ns = 3; add("packed without workspace", x, GDR2_E_WORKSPACE); }
  { Fwd x = f; x.cu = (const int32_t*)A; x.B = 1; x.ns = 3; x.ws = A; x.wsb = 8; add("workspace of 8 B", x, GDR2_E_WORKSPACE); }
  { Fwd x = f; x.B = 1; x.T = INT_MAX / 2; add("T near INT_MAX / 2", x, GDR2_E_WORKSPACE); }
  { Fwd x = f; x.B = 1; x.T = INT_MAX; x.cu = (const int32_t*)A; x.ns = INT_MAX / 4; add("huge packed: too many (sequence, head) pairs", x, GDR2_E_SHAPE); }
  for (int i = 0; i < n; ++i) {
    expect(cases[i].f.run(), cases[i].want, "gdr2_chunk_fwd", cases[i].what);
    expect(cases[i].f.run_f32(), cases[i].want, "gdr2_chunk_fwd_f32_out", cases[i].what);
  }
  { Fwd x = f; x.q = nullptr; expect(x.run_noalloc(), GDR2_E_NULL, "gdr2_chunk_fwd_noalloc", "q NULL"); }
  { Fwd x = f; x.dk = 48; expect(x.run_noalloc(), GDR2_E_UNSUPPORTED, "gdr2_chunk_fwd_noalloc", "dk 48"); }
  { Fwd x = f; x.B = 4; x.T = 4096; x.H = 16; expect(x.run_noalloc(), GDR2_E_WORKSPACE, "gdr2_chunk_fwd_noalloc", "beyond the scratch"); }
  { Fwd x = f; x.B = 1; x.T = INT_MAX; x.H = INT_MAX; expect(x.run_noalloc(), GDR2_E_SHAPE, "gdr2_chunk_fwd_noalloc", "T and H at INT_MAX: too many pairs"); }
}

static void decode_cases() {
  const char* fn = "gdr2_decode_step";
  auto dec = [](const void* q, float* S, void* o, int N, int dk, gdr2_dtype dt) {
    return gdr2_decode_step(q, A, A, A, A, A, S, o, N, 4, dk, 128, dt, GDR2_F32, nullptr);
  };
  expect(dec(A, nullptr, A, 8, 128, GDR2_F32), GDR2_E_NULL, fn, "S NULL");
  expect(dec(nullptr, (float*)A, A, 8, 128, GDR2_F32), GDR2_E_NULL, fn, "q NULL");
  expect(dec(A, (float*)A, A, 8, 128, (gdr2_dtype)5), GDR2_E_DTYPE, fn, "dtype 5");
  expect(dec(A, (float*)A, A, -1, 128, GDR2_F32), GDR2_E_SHAPE, fn, "N -1");
  expect(dec(A, (float*)A, A, 8, 16, GDR2_F32), GDR2_E_UNSUPPORTED, fn, "dk 16");
  expect(dec(A, (float*)A, MIS, 8, 128, GDR2_F32), GDR2_E_ALIGN, fn, "o misaligned");
  expect(dec(A, (float*)MIS, A, 8, 128, GDR2_F32), GDR2_E_ALIGN, fn, "S misaligned");
  const char* fg = "gdr2_decode_step_norm_gate";
  auto decg = [](const void* z, const float* nw, float eps, void* y, int dv, gdr2_dtype dt) {
    return gdr2_decode_step_norm_gate(A, A, A, A, A, A, (float*)A, z, nw, eps, y, 8, 4, 128, dv, dt, GDR2_F32,
                                      nullptr);
  };
  expect(decg(nullptr, nullptr, 1e-6f, A, 128, GDR2_BF16), GDR2_E_NULL, fg, "z NULL");
  expect(decg(A, nullptr, 1e-6f, nullptr, 128, GDR2_BF16), GDR2_E_NULL, fg, "y NULL");
  expect(decg(A, nullptr, 1e-6f, A, 128, (gdr2_dtype)3), GDR2_E_DTYPE, fg, "dtype 3");
  expect(decg(A, nullptr, -0.5f, A, 128, GDR2_BF16), GDR2_E_SHAPE, fg, "eps -0.5");
  expect(decg(A, nullptr, NAN, A, 128, GDR2_BF16), GDR2_E_SHAPE, fg, "eps NaN");
  expect(decg(A, nullptr, 1e-6f, A, 96, GDR2_BF16), GDR2_E_UNSUPPORTED, fg, "dv 96");
  expect(decg(MIS, nullptr, 1e-6f, A, 128, GDR2_BF16), GDR2_E_ALIGN, fg, "z misaligned");
  expect(decg(A, (const float*)MIS, 1e-6f, A, 128, GDR2_BF16), GDR2_E_ALIGN, fg, "weight misaligned");
}

static void backward_cases() {
  const char* fn = "gdr2_chunk_bwd";
  struct Bw {
    const void* dO = A;
    float* dg = (float*)A;
    float* dS0 = nullptr;
    const float* dST = nullptr;
    const int32_t* cu = nullptr;
    int ns = 0, B = 2, T = 100, dk = 128, dv = 128;
    gdr2_dtype dt = GDR2_BF16;
    void* ws = nullptr;
    size_t wsb = 0;
    int run() const {
      return gdr2_chunk_bwd(A, A, A, A, A, A, nullptr, dO, dST, (float*)A, (float*)A, (float*)A, dg, (float*)A,
                            (float*)A, dS0, cu, ns, B, T, 4, dk, dv, dt, GDR2_F32, ws, wsb, nullptr);
    }
  };
  Bw w;
  { Bw x = w; x.dO = nullptr; expect(x.run(), GDR2_E_NULL, fn, "dO NULL"); }
  { Bw x = w; x.dg = nullptr; expect(x.run(), GDR2_E_NULL, fn, "dlog_alpha NULL"); }
  { Bw x = w; x.dt = (gdr2_dtype)2; expect(x.run(), GDR2_E_DTYPE, fn, "dtype 2"); }
  { Bw x = w; x.B = 0; expect(x.run(), GDR2_E_SHAPE, fn, "B 0"); }
  { Bw x = w; x.T = -1; expect(x.run(), GDR2_E_SHAPE, fn, "T -1"); }
  { Bw x = w; x.dk = 48; expect(x.run(), GDR2_E_UNSUPPORTED, fn, "dk 48"); }
  { Bw x = w; x.cu = (const int32_t*)A; x.ns = 3; expect(x.run(), GDR2_E_SHAPE, fn, "cu_seqlens with B 2"); }
  { Bw x = w; x.dO = MIS; expect(x.run(), GDR2_E_ALIGN, fn, "dO misaligned"); }
  { Bw x = w; x.dS0 = (float*)MIS; expect(x.run(), GDR2_E_ALIGN, fn, "dS0 misaligned"); }
  { Bw x = w; x.dST = (const float*)MIS; expect(x.run(), GDR2_E_ALIGN, fn, "dS_T misaligned"); }
  { Bw x = w; expect(x.run(), GDR2_E_WORKSPACE, fn, "no workspace"); }
  { Bw x = w; x.ws = A; x.wsb = 64; expect(x.run(), GDR2_E_WORKSPACE, fn, "workspace of 64 B"); }
  { Bw x = w; x.B = 1; x.T = INT_MAX; expect(x.run(), GDR2_E_WORKSPACE, fn, "T at INT_MAX"); }
}

static void block_cases() {
  const char* fn = "gdr2_chunk_fwd_block";
  struct Bl {
    const void* q = A;
    const void* f = A;
    const float *da = (const float*)A, *db = (const float*)A;
    unsigned flags = 7;
    float bs = 1.f, eps = 1e-6f;
    void* o = A;
    const int32_t* cu = nullptr;
    int ns = 0, B = 2, T = 100, H = 4, Hv = 8, dk = 128, dv = 128;
    gdr2_dtype fdt = GDR2_F32;
    void* ws = nullptr;
    size_t wsb = 0;
    int run() const {
      return gdr2_chunk_fwd_block(q, A, A, f, A, A, da, db, flags, bs, eps, nullptr, o, nullptr, cu, ns, B, T,
                                  H, Hv, dk, dv, fdt, ws, wsb, nullptr);
    }
  };
  Bl b;
  { Bl x = b; x.q = nullptr; expect(x.run(), GDR2_E_NULL, fn, "q NULL"); }
  { Bl x = b; x.f = nullptr; expect(x.run(), GDR2_E_NULL, fn, "f NULL"); }
  { Bl x = b; x.da = nullptr; expect(x.run(), GDR2_E_NULL, fn, "decay_a NULL"); }
  { Bl x = b; x.fdt = (gdr2_dtype)9; expect(x.run(), GDR2_E_DTYPE, fn, "f dtype 9"); }
  { Bl x = b; x.flags = 8; expect(x.run(), GDR2_E_UNSUPPORTED, fn, "flags 8"); }
  { Bl x = b; x.Hv = 6; expect(x.run(), GDR2_E_SHAPE, fn, "Hv 6 with H 4"); }
  { Bl x = b; x.dk = 96; expect(x.run(), GDR2_E_UNSUPPORTED, fn, "dk 96"); }
  { Bl x = b; x.bs = INFINITY; expect(x.run(), GDR2_E_SHAPE, fn, "b_scale inf"); }
  { Bl x = b; x.eps = NAN; expect(x.run(), GDR2_E_SHAPE, fn, "qk_eps NaN"); }
  { Bl x = b; x.cu = (const int32_t*)A; x.ns = 2; expect(x.run(), GDR2_E_SHAPE, fn, "cu_seqlens with B 2"); }
  { Bl x = b; x.q = MIS; expect(x.run(), GDR2_E_ALIGN, fn, "q misaligned"); }
  { Bl x = b; x.o = MIS; expect(x.run(), GDR2_E_ALIGN, fn, "o misaligned"); }
  { Bl x = b; expect(x.run(), GDR2_E_WORKSPACE, fn, "no workspace"); }
  { Bl x = b; x.da = nullptr; x.db = nullptr; x.flags = 5; expect(x.run(), GDR2_E_WORKSPACE, fn, "no decay step"); }
}

static void norm_gate_cases() {
  const char* fn = "gdr2_norm_gate";
  auto ng = [](const void* o, const float* wt, void* y, long long rows, int d, int group, float eps,
               gdr2_dtype dt) { return gdr2_norm_gate(o, A, wt, y, rows, d, group, eps, dt, nullptr); };
  expect(ng(nullptr, nullptr, A, 64, 128, 128, 1e-6f, GDR2_BF16), GDR2_E_NULL, fn, "o NULL");
  expect(ng(A, nullptr, A, 64, 128, 128, 1e-6f, (gdr2_dtype)4), GDR2_E_DTYPE, fn, "dtype 4");
  expect(ng(A, nullptr, A, -1, 128, 128, 1e-6f, GDR2_BF16), GDR2_E_SHAPE, fn, "rows -1");
  expect(ng(A, nullptr, A, 64, 24, 12, 1e-6f, GDR2_BF16), GDR2_E_SHAPE, fn, "group 12");
  expect(ng(A, nullptr, A, 64, 96, 64, 1e-6f, GDR2_BF16), GDR2_E_SHAPE, fn, "group does not divide d");
  expect(ng(A, nullptr, A, 64, 128, 128, NAN, GDR2_BF16), GDR2_E_SHAPE, fn, "eps NaN");
  expect(ng(A, nullptr, A, 1LL << 60, 128, 128, 1e-6f, GDR2_BF16), GDR2_E_SHAPE, fn, "rows 2^60");
  expect(ng(A, nullptr, A, LLONG_MAX, INT_MAX, 8, 1e-6f, GDR2_BF16), GDR2_E_SHAPE, fn, "rows and d at their maxima");
  expect(ng(MIS, nullptr, A, 64, 128, 128, 1e-6f, GDR2_BF16), GDR2_E_ALIGN, fn, "o misaligned");
  expect(ng(A, (const float*)MIS, A, 64, 128, 128, 1e-6f, GDR2_BF16), GDR2_E_ALIGN, fn, "weight misaligned");
  expect(ng(A, nullptr, A, 0, 128, 128, 1e-6f, GDR2_BF16), GDR2_OK, fn, "no rows");
}

static void query_cases() {
  // size queries over valid and invalid sizes: every invalid one is 0, and a
  // valid one is monotone in T
  const int dims[] = {0, 16, 32, 48, 64, 128, 256};
  for (int dk : dims)
    for (int dv : dims)
      for (int dt = -1; dt <= 2; ++dt) {
        const bool ok = (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128) &&
                        (dt == 0 || dt == 1);
        size_t prev = 0;
        for (int T : {0, 1, 63, 64, 65, 4096, 32768, 1 << 24}) {
          const size_t a = gdr2_chunk_fwd_workspace_bytes(2, T, 3, dk, dv, 0, (gdr2_dtype)dt);
          const size_t p = gdr2_chunk_fwd_workspace_bytes(1, T, 3, dk, dv, 5, (gdr2_dtype)dt);
          if (!ok && (a != 0 || p != 0)) {
            printf("FAIL workspace query of invalid sizes dk %d dv %d dtype %d: %zu %zu\n", dk, dv, dt, a, p);
            ++failures;
          }
          if (ok && a < prev) {
            printf("FAIL workspace query not monotone in T at %d\n", T);
            ++failures;
          }
          prev = a;
        }
        (void)gdr2_chunk_bwd_workspace_bytes(2, 100, 3, dk, dv, 0);
      }
  if (gdr2_chunk_fwd_workspace_bytes(-1, 100, 4, 128, 128, 0, GDR2_BF16) != 0 ||
      gdr2_chunk_fwd_workspace_bytes(1, 100, 4, 128, 128, -3, GDR2_BF16) != 0 ||
      gdr2_chunk_bwd_workspace_bytes(1, -5, 4, 128, 128, 0) != 0) {
    printf("FAIL workspace query of negative sizes\n");
    ++failures;
  }
  (void)gdr2_chunk_fwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 128, 128, 0, GDR2_BF16);
  (void)gdr2_chunk_fwd_workspace_bytes(1, INT_MAX, INT_MAX, 128, 128, INT_MAX, GDR2_BF16);
  (void)gdr2_chunk_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 128, 128, 0);
  for (int s = -1; s <= 8; ++s) {
    const char* t = gdr2_status_string((gdr2_status)s);
    if (!t || !*t) {
      printf("FAIL status string %d\n", s);
      ++failures;
    }
  }
  if (gdr2_version() < 100) {
    printf("FAIL version\n");
    ++failures;
  }
}

int main() {
  chunk_fwd_cases();
  decode_cases();
  backward_cases();
  block_cases();
  norm_gate_cases();
  query_cases();
  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
