/* Host-side driver of the C ABI (include/vdm.h), built with AddressSanitizer and
 * UndefinedBehaviorSanitizer together with a host-only build of the library
 * (tests/test_abi_sanitized.py). It needs no GPU: every call below either
 * returns before any device work (argument, dimension and workspace checks,
 * zero-sized calls) or is a size query or the timing API. The sanitizers watch
 * the library's host code on these paths: validation, workspace carving and
 * size arithmetic, error-message formatting.
 *
 * Exit status 0 when every check holds; each failed check prints its line. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "vdm.h"

static int failures = 0;
#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      printf("FAILED line %d: %s (last error: %s)\n", __LINE__, #cond,      \
             vdm_last_error());                                             \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

/* fake device addresses: never dereferenced, every call using them fails
 * validation first */
#define FAKE ((void*)(uintptr_t)0x100000)
#define AT(off) ((void*)(uintptr_t)(0x100000 + (off)))

static vdm_decoder decoder(int D, int F, int dtype) {
  vdm_decoder d;
  memset(&d, 0, sizeof d);
  d.D = D;
  d.H = D / 64;
  d.F = F;
  d.n_freq = 8;
  d.dtype = dtype;
  d.net_scale = 0.05f;
  d.Wq = d.Wk = d.Wv = d.Wo = d.W1 = d.W2 = FAKE;
  d.w_head = (const float*)FAKE;
  d.n_prims = 1;
  d.prims[0].kind = VDM_PRIM_SPHERE;
  d.prims[0].size[0] = 0.5f;
  return d;
}

static vdm_hier_params hier(int R0, int levels) {
  vdm_hier_params p;
  memset(&p, 0, sizeof p);
  p.R0 = R0;
  p.levels = levels;
  p.dilation = 1;
  p.tau = 4.f / (R0 << (levels - 1));
  p.block = 8;
  p.k = 64;
  p.cap = 512;
  return p;
}

static void decoders_and_zero_sizes(void) {
  vdm_decoder d = decoder(256, 1024, VDM_BF16);
  CHECK(vdm_version() == VDM_VERSION);
  CHECK(vdm_embed_queries(NULL, NULL, 5, NULL, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(strstr(vdm_last_error(), "NULL") != NULL);
  vdm_decoder bad = decoder(128, 1024, VDM_BF16);
  CHECK(vdm_embed_queries(&bad, NULL, 5, NULL, NULL) == VDM_ERR_UNSUPPORTED);
  bad = decoder(256, 1000, VDM_BF16);
  CHECK(vdm_embed_queries(&bad, NULL, 5, NULL, NULL) == VDM_ERR_UNSUPPORTED);
  bad = decoder(256, 1024, 7);
  CHECK(vdm_embed_queries(&bad, NULL, 5, NULL, NULL) == VDM_ERR_INVALID_ARG);
  bad = d;
  bad.n_prims = 0;
  CHECK(vdm_embed_queries(&bad, NULL, 5, NULL, NULL) == VDM_ERR_INVALID_ARG);
  bad.n_prims = VDM_MAX_PRIMS + 1;
  CHECK(vdm_embed_queries(&bad, NULL, 5, NULL, NULL) == VDM_ERR_INVALID_ARG);
  bad = d;
  bad.n_freq = 6;
  CHECK(vdm_embed_queries(&bad, NULL, 5, NULL, NULL) == VDM_ERR_UNSUPPORTED);
  bad = d;
  bad.Wk = AT(2);
  CHECK(vdm_project_kv(&bad, AT(0x1000), 4, AT(0x2000), AT(0x3000), NULL) == VDM_ERR_INVALID_ARG);
  /* zero-sized calls do nothing and succeed */
  CHECK(vdm_embed_queries(&d, NULL, 0, NULL, NULL) == VDM_OK);
  CHECK(vdm_project_kv(&d, NULL, 0, NULL, NULL, NULL) == VDM_OK);
  vdm_queries q0 = {VDM_Q_POINTS, 0, 0, NULL, NULL};
  CHECK(vdm_decode_dense(&d, &q0, NULL, NULL, 1, NULL, NULL, NULL, 0, NULL) == VDM_OK);
  CHECK(vdm_decode_dense_noalloc(&d, &q0, NULL, NULL, 1, NULL, NULL) == VDM_OK);
}

static void dense(void) {
  vdm_decoder d = decoder(256, 1024, VDM_BF16);
  vdm_queries q = {VDM_Q_GRID, 16, 17 * 17 * 17 - 1, NULL, NULL};
  CHECK(vdm_decode_dense(&d, &q, FAKE, FAKE, 10, NULL, (float*)FAKE, FAKE, (size_t)1 << 30, NULL) ==
        VDM_ERR_INVALID_ARG);
  q.N = 17 * 17 * 17;
  CHECK(vdm_decode_dense(&d, &q, FAKE, FAKE, 0, NULL, (float*)FAKE, FAKE, (size_t)1 << 30, NULL) ==
        VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_dense(&d, &q, FAKE, FAKE, 10, NULL, (float*)FAKE, FAKE, 16, NULL) == VDM_ERR_WORKSPACE);
  vdm_kvsel sel = {8, 64, (const int32_t*)FAKE, (const int32_t*)FAKE, NULL, 0};
  CHECK(vdm_decode_dense(&d, &q, FAKE, FAKE, 10, &sel, (float*)FAKE, FAKE, (size_t)1 << 30, NULL) ==
        VDM_ERR_INVALID_ARG);
  vdm_queries qr = {VDM_Q_GRID, 5000, 1, NULL, NULL};
  CHECK(vdm_decode_dense(&d, &qr, FAKE, FAKE, 10, NULL, (float*)FAKE, FAKE, (size_t)1 << 30, NULL) ==
        VDM_ERR_INVALID_ARG);
  vdm_queries qm = {9, 16, 10, NULL, NULL};
  CHECK(vdm_decode_dense(&d, &qm, FAKE, FAKE, 10, NULL, (float*)FAKE, FAKE, (size_t)1 << 30, NULL) ==
        VDM_ERR_INVALID_ARG);
  /* no-allocation decode: a token count whose scratch exceeds the fixed array */
  CHECK(vdm_decode_dense_noalloc(&d, &q, FAKE, FAKE, 60000, (float*)FAKE, NULL) == VDM_ERR_WORKSPACE);
  CHECK(strstr(vdm_last_error(), "scratch") != NULL);
  CHECK(vdm_decode_dense_noalloc(&d, &q, NULL, FAKE, 10, (float*)FAKE, NULL) == VDM_ERR_INVALID_ARG);
  /* batch */
  size_t need = vdm_dense_batch_workspace_size(&d, 4, 3072);
  CHECK(vdm_dense_batch_workspace_size(&d, 0, 3072) == 0);
  CHECK(need > 0);
  CHECK(vdm_decode_dense_batch(&d, &q, 0, FAKE, FAKE, 3072, (float*)FAKE, FAKE, need, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_dense_batch(&d, &q, 4, FAKE, FAKE, 3072, (float*)FAKE, FAKE, need - 1, NULL) ==
        VDM_ERR_WORKSPACE);
}

static void select_and_hier(void) {
  vdm_decoder d = decoder(256, 1024, VDM_BF16);
  int32_t* I = (int32_t*)FAKE;
  CHECK(vdm_select_kv(&d, 75, 8, 65, 512, 0, 0, FAKE, 64, NULL, 1000, I, I, NULL, 0, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_select_kv(&d, 75, 8, 64, 32, 0, 0, FAKE, 3072, NULL, 1000, I, I, NULL, 0, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_select_kv(&d, 75, 8, 64, 512, 0, 0, FAKE, 65537, NULL, 1000, I, I, NULL, 0, NULL) ==
        VDM_ERR_UNSUPPORTED);
  CHECK(vdm_select_kv(&d, 75, 8, 103, 1024, 0, 0, FAKE, 40960, NULL, 1000, I, I, NULL, 0, NULL) ==
        VDM_ERR_UNSUPPORTED);
  CHECK(vdm_select_kv(&d, 75, 8, 64, 512, 0, 0, FAKE, 40960, NULL, 1000, I, I, NULL, 0, NULL) ==
        VDM_ERR_WORKSPACE);
  CHECK(vdm_select_kv_heads(&d, 75, 8, 64, 512, 0, 0, FAKE, 16385, NULL, 1000, I, I, NULL, 0, NULL) ==
        VDM_ERR_UNSUPPORTED);
  CHECK(vdm_select_kv(&d, 75, 8, 64, 512, 2, 0, FAKE, 3072, NULL, 1000, I, I, NULL, 0, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_select_kv(&d, 75, 8, 64, 512, 0, 0, FAKE, 3072, NULL, 999, I, I, NULL, 0, NULL) == VDM_ERR_INVALID_ARG);
  const size_t sneed = vdm_select_workspace_size(&d, 3072);
  CHECK(sneed >= (size_t)32 * 3072 * 4);
  CHECK(vdm_select_kv(&d, 75, 8, 64, 512, 0, 0, FAKE, 3072, NULL, 1000, I, I, FAKE, sneed - 1, NULL) ==
        VDM_ERR_WORKSPACE);
  CHECK(vdm_select_heads_workspace_size(&d, 3072) >= sneed);
  CHECK(vdm_select_kv_heads(&d, 75, 8, 64, 512, 0, 0, FAKE, 3072, NULL, 1000, I, I, FAKE, sneed - 1, NULL) ==
        VDM_ERR_WORKSPACE);

  vdm_hier_params p = hier(75, 3);
  CHECK(vdm_hier_workspace_size(&d, &p, 3072) > (size_t)27000000 * 4);
  vdm_hier_params bad = hier(75, 3);
  bad.levels = VDM_MAX_LEVELS + 1;
  CHECK(vdm_hier_workspace_size(&d, &bad, 3072) == 0);
  bad = hier(75, 3);
  bad.use_kvsel = 1;
  bad.probes = 3;
  CHECK(vdm_hier_workspace_size(&d, &bad, 3072) == 0);
  CHECK(strstr(vdm_last_error(), "probes") != NULL);
  bad = hier(75, 3);
  bad.tau = NAN;
  CHECK(vdm_decode_hier(&d, &bad, FAKE, FAKE, 3072, (float*)FAKE, 301 * 301 * 301, NULL, NULL, FAKE,
                        (size_t)1 << 40, NULL) == VDM_ERR_INVALID_ARG);
  bad = hier(600, 2); /* finest grid 1200: allowed; 1201 points per axis */
  CHECK(vdm_hier_workspace_size(&d, &bad, 3072) > 0);
  bad = hier(601, 2); /* finest grid 1202: refused */
  CHECK(vdm_hier_workspace_size(&d, &bad, 3072) == 0);
  CHECK(vdm_decode_hier(&d, &p, FAKE, FAKE, 3072, (float*)FAKE, 300 * 300 * 300, NULL, NULL, FAKE,
                        (size_t)1 << 40, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_hier(&d, &p, FAKE, FAKE, 3072, (float*)FAKE, 301 * 301 * 301, NULL, NULL, FAKE, 1024, NULL) ==
        VDM_ERR_WORKSPACE);
  /* batch */
  const size_t one = vdm_hier_workspace_size(&d, &p, 3072), four = vdm_hier_batch_workspace_size(&d, &p, 4, 3072);
  CHECK(vdm_hier_batch_workspace_size(&d, &p, 0, 3072) == 0);
  CHECK(four % 4 == 0 && four / 4 >= one && four / 4 - one < 256);
  const int64_t P3 = 301 * 301 * 301;
  CHECK(vdm_decode_hier_batch(&d, &p, 0, FAKE, FAKE, 3072, (float*)FAKE, 4 * P3, NULL, FAKE, four, NULL) ==
        VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_hier_batch(&d, &p, 4097, FAKE, FAKE, 3072, (float*)FAKE, 4 * P3, NULL, FAKE, four, NULL) ==
        VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_hier_batch(&d, &p, 4, AT(8), FAKE, 3072, (float*)FAKE, 4 * P3, NULL, FAKE, four, NULL) ==
        VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_hier_batch(&d, &p, 4, FAKE, FAKE, 3072, (float*)FAKE, 4 * P3 - 1, NULL, FAKE, four, NULL) ==
        VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_hier_batch(&d, &p, 4, FAKE, FAKE, 3072, (float*)FAKE, 4 * P3, NULL, FAKE, four - 1, NULL) ==
        VDM_ERR_WORKSPACE);
}

static void surface_and_local(void) {
  CHECK(vdm_surface_workspace_size(0) == 0);
  CHECK(strstr(vdm_last_error(), "R=0") != NULL);
  const size_t n300 = vdm_surface_workspace_size(300);
  CHECK(n300 > 0);
  float* F = (float*)FAKE;
  int32_t* T = (int32_t*)FAKE;
  int64_t* C = (int64_t*)FAKE;
  CHECK(vdm_extract_surface(NULL, 300, NULL, F, 10, T, 10, NULL, C, FAKE, n300, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_extract_surface(F, 0, NULL, F, 10, T, 10, NULL, C, FAKE, n300, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_extract_surface((float*)AT(2), 300, NULL, F, 10, T, 10, NULL, C, FAKE, n300, NULL) ==
        VDM_ERR_INVALID_ARG);
  CHECK(strstr(vdm_last_error(), "misaligned") != NULL);
  CHECK(vdm_extract_surface(F, 300, NULL, F, 10, T, 10, NULL, C, FAKE, n300 - 1, NULL) == VDM_ERR_WORKSPACE);

  vdm_local_decoder l;
  memset(&l, 0, sizeof l);
  l.C = 256;
  l.F = 1024;
  l.K = 16;
  l.hidden = 32;
  l.net_scale = 0.05f;
  l.A = l.a = l.w_head = (const float*)FAKE;
  l.B = l.W1 = l.W2 = FAKE;
  l.n_prims = 1;
  CHECK(vdm_decode_local(NULL, F, FAKE, 100, F, 50, F, NULL, FAKE, (size_t)1 << 30, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_local(&l, F, FAKE, 100, F, 0, NULL, NULL, NULL, 0, NULL) == VDM_OK);
  l.K = 8;
  CHECK(vdm_decode_local(&l, F, FAKE, 100, F, 50, F, NULL, FAKE, (size_t)1 << 30, NULL) == VDM_ERR_UNSUPPORTED);
  l.K = 16;
  CHECK(vdm_decode_local(&l, F, FAKE, 15, F, 50, F, NULL, FAKE, (size_t)1 << 30, NULL) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_decode_local(&l, F, FAKE, 100, F, 50, F, NULL, FAKE, 64, NULL) == VDM_ERR_WORKSPACE);
  CHECK(vdm_local_workspace_size(&l, 40960, 200000) >= (size_t)200000 * 256 * 2);
}

/* Size queries over wide ranges, including sizes far beyond any GPU: each call
 * returns a size or 0 (refused); UBSan reports any signed overflow on the way. */
static void size_sweeps(void) {
  vdm_decoder d = decoder(256, 1024, VDM_BF16), d1 = decoder(64, 128, VDM_F32);
  const int64_t Ms[] = {1, 33, 3072, 40960, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX / 4};
  const int64_t Ns[] = {0, 1, 4097, 2146689, (int64_t)1 << 33, INT64_MAX / 8};
  for (unsigned i = 0; i < sizeof Ms / sizeof *Ms; ++i) {
    for (unsigned j = 0; j < sizeof Ns / sizeof *Ns; ++j)
      for (int s = 0; s < 2; ++s) {
        (void)vdm_dense_workspace_size(&d, Ms[i], Ns[j], s);
        (void)vdm_dense_workspace_size(&d1, Ms[i], Ns[j], s);
      }
    (void)vdm_select_workspace_size(&d, Ms[i]);
    (void)vdm_select_heads_workspace_size(&d, Ms[i]);
    for (int B = 1; B <= 4096; B *= 16) {
      (void)vdm_dense_batch_workspace_size(&d, B, Ms[i]);
      vdm_hier_params p = hier(75, 3);
      (void)vdm_hier_batch_workspace_size(&d, &p, B, Ms[i]);
    }
    for (int R0 = 1; R0 <= 1200; R0 = R0 * 3 + 1)
      for (int L = 1; L <= VDM_MAX_LEVELS; ++L) {
        vdm_hier_params p = hier(R0, L);
        (void)vdm_hier_workspace_size(&d, &p, Ms[i]);
        p.use_kvsel = 1;
        (void)vdm_hier_workspace_size(&d, &p, Ms[i]);
      }
  }
  for (int R = -1; R <= 5000; R += 37) (void)vdm_surface_workspace_size(R);
  vdm_local_decoder l;
  memset(&l, 0, sizeof l);
  l.C = 256;
  l.F = 1024;
  l.K = 16;
  l.hidden = 32;
  for (unsigned i = 0; i < sizeof Ms / sizeof *Ms; ++i)
    for (unsigned j = 0; j < sizeof Ns / sizeof *Ns; ++j) (void)vdm_local_workspace_size(&l, Ms[i], Ns[j]);
  CHECK(vdm_dense_workspace_size(&d, 3072, 1000, 0) >= (size_t)2 * 3072 * 256 * 2);
}

static void timing(void) {
  CHECK(vdm_timing(2) == VDM_OK);
  CHECK(vdm_timing(1) == VDM_OK);
  int64_t n = -1;
  double ms = -1.0;
  CHECK(vdm_timing_read(VDM_TIME_DECODE, &n, &ms) == VDM_OK);
  CHECK(n == 0 && ms == 0.0);
  CHECK(vdm_timing(0) == VDM_OK);
  CHECK(vdm_timing(3) == VDM_ERR_INVALID_ARG);
  CHECK(strstr(vdm_last_error(), "timing mode") != NULL);
  CHECK(vdm_timing_read(VDM_TIME_KINDS, &n, &ms) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_timing_read(-1, &n, &ms) == VDM_ERR_INVALID_ARG);
  CHECK(vdm_timing_read(0, NULL, &ms) == VDM_ERR_INVALID_ARG);
}

int main(void) {
  decoders_and_zero_sizes();
  dense();
  select_and_hier();
  surface_and_local();
  size_sweeps();
  timing();
  printf("%s: %d failed checks\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
