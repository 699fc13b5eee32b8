/*
 * Host-side check of the C ABI (test infrastructure): linked against the library's host code
 * built under AddressSanitizer and UndefinedBehaviorSanitizer, it drives every entry point
 * through argument validation and every workspace-size query, including sizes near the int64
 * range, so signed overflow, an out-of-bounds host access or an unexpected status aborts or
 * fails the program.  No call here passes validation with device pointers: the fake addresses
 * below are never dereferenced, and nothing is launched.  Exit status 0 means every case
 * returned the expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mamba_scan.h"

#define FAKE ((void*)0x10000)
#define ODD ((void*)0x10001)
#define BIG INT64_MAX

static int failures = 0;

/* Extreme values for a size field.  Each one is invalid wherever it is used below (a product
 * past 2^40 elements, a value at or past 2^31 where that is the bound, or <= 0), so no call in
 * the sweeps can pass validation and launch. */
static const int64_t extremes[] = {BIG, BIG - 15, (int64_t)1 << 62, (int64_t)1 << 40, INT64_MIN,
                                   -1, 0};
#define NEX ((int)(sizeof extremes / sizeof extremes[0]))

static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

static mamba_dims dims(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io,
                       int chunk) {
  mamba_dims d;
  memset(&d, 0, sizeof d);
  d.batch = batch; d.dim = dim; d.dstate = dstate; d.seqlen = seqlen;
  d.io_dtype = io; d.chunk_len = chunk;
  return d;
}

static int scan(const mamba_dims* d, void* u, void* ws, size_t wsb) {
  return mamba_scan_fwd(u, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL, 1, FAKE, NULL, d, ws, wsb,
                        NULL);
}

static int conv(const mamba_dims* d, int width, void* u_out) {
  return mamba_scan_fwd_conv(FAKE, FAKE, NULL, width, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL, 1,
                             FAKE, NULL, u_out, d, NULL, 0, NULL);
}

static int step(const mamba_dims* d, float* state) {
  return mamba_state_update(state, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL, 1, FAKE, d,
                            NULL);
}

static int bwd(const mamba_dims* d, void* ws, size_t wsb) {
  return mamba_scan_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL, 1, FAKE, NULL, FAKE, FAKE,
                        FAKE, FAKE, FAKE, NULL, NULL, NULL, d, ws, wsb, NULL);
}

static mamba_block_dims bdims(int64_t batch, int64_t L, int64_t dm, int64_t E, int64_t R,
                              int width) {
  mamba_block_dims d;
  memset(&d, 0, sizeof d);
  d.batch = batch; d.seqlen = L; d.d_model = dm; d.d_inner = E; d.dstate = 16; d.dt_rank = R;
  d.conv_width = width;
  return d;
}

static int block(const mamba_block_dims* d, void* ws, size_t wsb) {
  return mamba_block_fwd(FAKE, FAKE, FAKE, NULL, FAKE, FAKE, NULL, FAKE, NULL, FAKE, FAKE, d, ws,
                         wsb, NULL);
}

static int gemm(int64_t M, int64_t N, int64_t K, int64_t batch, int64_t lda, int64_t ldb,
                int64_t bs, int64_t ldc, int64_t cs, int kc, int tr, void* A) {
  return mamba_gemm_bf16(A, FAKE, FAKE, M, N, K, batch, lda, ldb, bs, ldc, cs, kc, tr, NULL);
}

int main(void) {
  EXPECT(mamba_abi_version(), MAMBA_SCAN_ABI_VERSION);
  for (int s = -100; s <= 100; ++s)
    if (!mamba_status_string(s)) { fprintf(stderr, "NULL status string %d\n", s); ++failures; }

  /* scan: the validation order of the header (pointers, shape, dtype, alignment, workspace) */
  mamba_dims d = dims(2, 64, 16, 128, MAMBA_F32, 0);
  EXPECT(scan(NULL, FAKE, NULL, 0), MAMBA_ERR_NULL);
  EXPECT(scan(&d, NULL, NULL, 0), MAMBA_ERR_NULL);
  EXPECT(scan(&d, ODD, NULL, 0), MAMBA_ERR_ALIGN);
  d = dims(2, 64, 8, 128, 0, 0);
  EXPECT(scan(&d, FAKE, NULL, 0), MAMBA_ERR_UNSUPPORTED);
  d = dims(2, 64, 16, 128, 7, 0);
  EXPECT(scan(&d, FAKE, NULL, 0), MAMBA_ERR_DTYPE);
  d = dims(2, 64, 16, 128, 0, 24);
  EXPECT(scan(&d, FAKE, NULL, 0), MAMBA_ERR_SHAPE);
  d = dims(1, 1, 16, (int64_t)1 << 25, MAMBA_F32, 0);
  EXPECT(scan(&d, FAKE, NULL, 0), MAMBA_ERR_SHAPE);
  d = dims(2, 64, 16, 4096, MAMBA_F32, 256);
  const size_t need = mamba_scan_workspace_bytes(&d);
  if (need == 0) { fprintf(stderr, "chunked plan without workspace\n"); ++failures; }
  EXPECT(scan(&d, FAKE, NULL, 0), MAMBA_ERR_WORKSPACE);
  EXPECT(scan(&d, FAKE, FAKE, need - 1), MAMBA_ERR_WORKSPACE);
  /* every field at the extremes: a shape error and a zero workspace, never an overflow */
  for (int f = 0; f < 4; ++f)
    for (int i = 0; i < NEX; ++i) {
      int64_t v[4] = {2, 64, 16, 128};
      v[f] = extremes[i];
      for (int io = 0; io < 2; ++io) {
        d = dims(v[0], v[1], v[2], v[3], io, 0);
        const int want = (f == 2 && extremes[i] > 0) ? MAMBA_ERR_UNSUPPORTED : MAMBA_ERR_SHAPE;
        EXPECT(scan(&d, FAKE, NULL, 0), want);
        EXPECT(conv(&d, 4, NULL), want);
        EXPECT(bwd(&d, FAKE, 1 << 20), want);
        EXPECT(mamba_scan_workspace_bytes(&d) != 0, 0);
        EXPECT(mamba_scan_bwd_workspace_bytes(&d) != 0, 0);
        d.seqlen = f == 3 ? d.seqlen : 1;
        if (f != 3) EXPECT(step(&d, FAKE), want);
      }
    }
  d = dims(2, 64, 16, 128, 0, -16);
  EXPECT(scan(&d, FAKE, NULL, 0), MAMBA_ERR_SHAPE);

  /* the allocation-free forward: the same validation, and its scratch bound before any HIP call */
  EXPECT(mamba_scan_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL, 1, FAKE, NULL, NULL,
                                NULL), MAMBA_ERR_NULL);
  d = dims(2, 64, 16, 128, 7, 0);
  EXPECT(mamba_scan_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL, 1, FAKE, NULL, &d,
                                NULL), MAMBA_ERR_DTYPE);
  d = dims(1, 64, 16, (int64_t)1 << 16, MAMBA_F32, 16);
  EXPECT(mamba_scan_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL, 1, FAKE, NULL, &d,
                                NULL), MAMBA_ERR_SCRATCH);

  /* workspace queries over a sweep of valid shapes and chunk lengths */
  for (int64_t b = 1; b <= 3; ++b)
    for (int64_t dim = 1; dim <= 130; dim += 43)
      for (int64_t L = 1; L <= ((int64_t)1 << 24); L = L * 5 + 3)
        for (int chunk = 0; chunk <= 4096; chunk = chunk ? chunk * 4 : 16) {
          d = dims(b, dim, 16, L, (int)(L & 1), chunk);
          const size_t f = mamba_scan_workspace_bytes(&d);
          const size_t g = mamba_scan_bwd_workspace_bytes(&d);
          if (f > ((size_t)1 << 40) || g > ((size_t)1 << 44)) {
            fprintf(stderr, "implausible workspace %zu / %zu\n", f, g);
            ++failures;
          }
        }

  /* conv and step specifics */
  d = dims(1, 64, 16, 128, 0, 0);
  EXPECT(conv(&d, 0, NULL), MAMBA_ERR_UNSUPPORTED);
  EXPECT(conv(&d, 5, NULL), MAMBA_ERR_UNSUPPORTED);
  EXPECT(conv(&d, 4, ODD), MAMBA_ERR_ALIGN);
  d = dims(1, 64, 16, 2, 0, 0);
  EXPECT(step(&d, FAKE), MAMBA_ERR_SHAPE);
  d = dims(1, 64, 16, 1, 0, 0);
  EXPECT(step(&d, (float*)0x10004), MAMBA_ERR_ALIGN);
  d = dims(70000, 64, 16, 1, 0, 0);
  EXPECT(step(&d, FAKE), MAMBA_ERR_SHAPE);

  /* backward: workspace presence, size and alignment */
  d = dims(2, 64, 16, 128, 0, 0);
  const size_t bneed = mamba_scan_bwd_workspace_bytes(&d);
  EXPECT(bwd(&d, NULL, bneed), MAMBA_ERR_WORKSPACE);
  EXPECT(bwd(&d, FAKE, bneed - 1), MAMBA_ERR_WORKSPACE);
  EXPECT(bwd(&d, (void*)0x10008, bneed), MAMBA_ERR_ALIGN);

  /* GEMM: every size, leading dimension and stride at the extremes is rejected */
  EXPECT(gemm(256, 128, 64, 1, 64, 64, 0, 128, 0, 1, 0, NULL), MAMBA_ERR_NULL);
  EXPECT(gemm(256, 128, 64, 1, 64, 64, 0, 128, 0, 1, 0, ODD), MAMBA_ERR_ALIGN);
  EXPECT(gemm(250, 128, 64, 1, 64, 64, 0, 128, 0, 1, 0, FAKE), MAMBA_ERR_SHAPE);
  EXPECT(gemm(256, 128, 64, 0, 64, 64, 0, 128, 0, 1, 0, FAKE), MAMBA_ERR_SHAPE);
  EXPECT(gemm(256, 128, 64, 65536, 64, 64, 0, 128, 0, 1, 0, FAKE), MAMBA_ERR_SHAPE);
  EXPECT(gemm(256, 128, 64, 1, 64, 32, 0, 128, 0, 1, 0, FAKE), MAMBA_ERR_SHAPE);
  EXPECT(gemm(256, 128, 64, 1, 64, 64, 0, 100, 0, 1, 0, FAKE), MAMBA_ERR_SHAPE);
  for (int f = 0; f < 8; ++f)
    for (int i = 0; i < NEX; ++i) {
      int64_t v[8] = {256, 128, 64, 1, 64, 64, 0, 128};
      v[f] = extremes[i] - (f < 3 && extremes[i] > 0 ? extremes[i] % 16 : 0);
      if (f == 6 && extremes[i] == 0) continue;                    /* a zero stride is valid */
      EXPECT(gemm(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], 0, 1, 0, FAKE),
             MAMBA_ERR_SHAPE);
    }
  /* output batch stride, transposed and row-major */
  for (int i = 0; i < NEX; ++i) {
    if (extremes[i] == 0) continue;
    EXPECT(gemm(256, 128, 64, 1, 64, 64, 0, 256, extremes[i], 1, 1, FAKE), MAMBA_ERR_SHAPE);
    EXPECT(gemm(256, 128, 64, 1, 64, 64, 0, 128, extremes[i], 1, 0, FAKE), MAMBA_ERR_SHAPE);
  }

  /* block: shape rules, extremes in every field, the scan's token bound before any launch */
  mamba_block_dims bd = bdims(1, 128, 64, 128, 16, 4);
  const size_t bw = mamba_block_workspace_bytes(&bd);
  if (bw == 0) { fprintf(stderr, "block workspace 0 for a valid shape\n"); ++failures; }
  EXPECT(block(NULL, FAKE, bw), MAMBA_ERR_NULL);
  EXPECT(block(&bd, NULL, bw), MAMBA_ERR_WORKSPACE);
  EXPECT(block(&bd, FAKE, bw - 1), MAMBA_ERR_WORKSPACE);
  EXPECT(block(&bd, (void*)0x10010, bw), MAMBA_ERR_ALIGN);
  bd.reserved = 0; bd.dstate = 8;
  EXPECT(block(&bd, FAKE, bw), MAMBA_ERR_UNSUPPORTED);
  bd = bdims(1, 128, 64, 128, 16, 5);
  EXPECT(block(&bd, FAKE, bw), MAMBA_ERR_UNSUPPORTED);
  bd = bdims(1, 124, 64, 128, 16, 4);
  EXPECT(block(&bd, FAKE, bw), MAMBA_ERR_SHAPE);
  bd = bdims(1, (int64_t)1 << 26, 16, 16, 16, 4);        /* 2^26 bf16 tokens: past the scan's bound */
  EXPECT(block(&bd, FAKE, (size_t)1 << 40), MAMBA_ERR_SHAPE);
  EXPECT(mamba_block_workspace_bytes(&bd) != 0, 0);
  for (int f = 0; f < 5; ++f)
    for (int i = 0; i < NEX; ++i) {
      int64_t v[5] = {1, 128, 64, 128, 16};
      v[f] = extremes[i] - (extremes[i] > 0 ? extremes[i] % 16 : 0);
      bd = bdims(v[0], v[1], v[2], v[3], v[4], 4);
      EXPECT(block(&bd, FAKE, (size_t)-1), MAMBA_ERR_SHAPE);
      EXPECT(mamba_block_workspace_bytes(&bd) != 0, 0);
    }

  if (failures)
    printf("C ABI sanitizer checks: %d FAILED\n", failures);
  else
    printf("C ABI sanitizer checks: clean\n");
  return failures ? 1 : 0;
}
