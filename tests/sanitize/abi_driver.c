/*
 * Drives the host-side argument validation of the C ABI (include/kda.h):
 * every rejection path returns before any GPU work, so this runs on a CPU.
 * Built against a build of the library whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py);
 * an out-of-bounds access,
 * a signed overflow or a misaligned access in validation or workspace sizing
 * aborts the run.  Prints "ok" on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int fails = 0;
static void expect(kda_status_t got, kda_status_t want, const char *what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, kda_last_error());
    ++fails;
  }
}

static kda_fwd_desc_t desc(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V) {
  kda_fwd_desc_t d;
  memset(&d, 0, sizeof d);
  d.B = B; d.T = T; d.H = H; d.K = K; d.V = V;
  d.dtype = KDA_BF16;
  d.o_dtype = KDA_F32;
  d.scale = NAN;
  d.chunk_size = 64;
  d.lower_bound = -5.f;
  return d;
}

int main(void) {
  size_t n = 0;
  void *fake = (void *)(uintptr_t)0x100000;      /* never dereferenced: validation fails first */
  void *odd = (void *)(uintptr_t)0x100008;       /* not 16-byte aligned */
  kda_fwd_desc_t d = desc(1, 128, 2, 128, 128);

  expect(kda_chunk_fwd_workspace_size(NULL, 0, &n), KDA_ERR_INVALID_ARGUMENT, "NULL desc");
  expect(kda_chunk_fwd_workspace_size(&d, 0, NULL), KDA_ERR_INVALID_ARGUMENT, "NULL bytes");
  expect(kda_chunk_fwd_workspace_size(&d, 0, &n), KDA_OK, "fixed size");
  const size_t fixed = n;
  d.max_segments = 4;
  expect(kda_chunk_fwd_workspace_size(&d, 1, &n), KDA_OK, "packed size");
  if (!(n > fixed)) { fprintf(stderr, "packed workspace %zu not above fixed %zu\n", n, fixed); ++fails; }
  d.max_segments = 0;
  expect(kda_chunk_fwd_workspace_size(&d, 1, &n), KDA_ERR_INVALID_ARGUMENT, "packed without max_segments");

  kda_fwd_desc_t b = d;
  b.K = 96;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_NOT_IMPLEMENTED, "K = 96");
  b = d; b.V = 256;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_NOT_IMPLEMENTED, "V = 256");
  b = d; b.chunk_size = 32;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_NOT_IMPLEMENTED, "chunk 32");
  b = d; b.safe_gate = 1; b.lower_bound = 0.f;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_INVALID_ARGUMENT, "safe gate bound 0");
  b = d; b.safe_gate = 1; b.lower_bound = -6.f;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_INVALID_ARGUMENT, "safe gate bound -6");
  b = d; b.scale = INFINITY;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_INVALID_ARGUMENT, "infinite scale");
  b = d; b.B = -1;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_INVALID_ARGUMENT, "negative B");
  b = d; b.T = (int64_t)1 << 40;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_NOT_IMPLEMENTED, "huge T");
  b = d; b.B = (int64_t)1 << 20; b.T = (int64_t)1 << 20;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_NOT_IMPLEMENTED, "huge B*T");
  b = d; b.dtype = (kda_dtype_t)7;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_INVALID_ARGUMENT, "bad dtype");
  b = d; b.o_dtype = (kda_dtype_t)-3;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_INVALID_ARGUMENT, "bad o_dtype");
  b = d; b.H = (int64_t)1 << 40;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_NOT_IMPLEMENTED, "huge H");
  b = d; b.B = (int64_t)1 << 40; b.T = 0;
  expect(kda_chunk_fwd_workspace_size(&b, 1, &n), KDA_ERR_INVALID_ARGUMENT, "huge B, no max_segments");
  b = d; b.B = (int64_t)1 << 30; b.T = 1; b.max_segments = 1 << 30;
  expect(kda_chunk_fwd_workspace_size(&b, 1, &n), KDA_ERR_NOT_IMPLEMENTED, "huge B * max_segments");
  b = d; b.B = (int64_t)1 << 62; b.T = 4;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_NOT_IMPLEMENTED, "B * T overflows");
  b = d; b.use_qk_l2norm = 2;
  expect(kda_chunk_fwd_workspace_size(&b, 0, &n), KDA_ERR_INVALID_ARGUMENT, "bad l2norm flag");

  /* forward: pointer checks and workspace size, all before any launch */
  expect(kda_chunk_fwd(&d, NULL, fake, fake, fake, fake, NULL, NULL, fake, NULL, fake, fixed, NULL),
         KDA_ERR_INVALID_ARGUMENT, "NULL q");
  expect(kda_chunk_fwd(&d, fake, fake, fake, fake, fake, NULL, NULL, NULL, NULL, fake, fixed, NULL),
         KDA_ERR_INVALID_ARGUMENT, "NULL o");
  expect(kda_chunk_fwd(&d, odd, fake, fake, fake, fake, NULL, NULL, fake, NULL, fake, fixed, NULL),
         KDA_ERR_INVALID_ARGUMENT, "misaligned q");
  expect(kda_chunk_fwd(&d, fake, fake, fake, fake, fake, NULL, NULL, fake, NULL, fake, fixed - 1, NULL),
         KDA_ERR_WORKSPACE_TOO_SMALL, "workspace short by one byte");
  expect(kda_chunk_fwd(&d, fake, fake, fake, fake, fake, NULL, NULL, fake, NULL, NULL, fixed, NULL),
         KDA_ERR_WORKSPACE_TOO_SMALL, "NULL workspace");
  b = d; b.B = 0;
  expect(kda_chunk_fwd(&b, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, fake, fixed, NULL), KDA_OK,
         "B = 0 is a no-op");
  expect(kda_chunk_fwd_gated(&d, fake, fake, fake, fake, fake, (const float *)(uintptr_t)0x100002, NULL, NULL, NULL,
                             fake, NULL, fake, fixed, NULL),
         KDA_ERR_INVALID_ARGUMENT, "misaligned A_log");
  expect(kda_chunk_fwd_transition(&d, fake, fake, fake, fake, fake, NULL, NULL, fake, NULL, NULL, fake, fixed, NULL),
         KDA_ERR_INVALID_ARGUMENT, "NULL transition");

  /* backward */
  expect(kda_chunk_bwd_workspace_size(NULL, 0, &n), KDA_ERR_INVALID_ARGUMENT, "bwd NULL desc");
  expect(kda_chunk_bwd_workspace_size(&d, 0, &n), KDA_OK, "bwd size");
  expect(kda_chunk_bwd(&d, fake, fake, fake, fake, fake, NULL, NULL, fake, NULL, (float *)fake, (float *)fake,
                       (float *)fake, (float *)fake, (float *)fake, NULL, fake, 1, NULL),
         KDA_ERR_WORKSPACE_TOO_SMALL, "bwd workspace too small");

  /* context-parallel glue */
  kda_cp_desc_t c = {1, 128, 2, 128, 128, 2, 1};
  expect(kda_cp_plan(NULL, NULL, fake, NULL), KDA_ERR_INVALID_ARGUMENT, "cp NULL desc");
  c.P = 0;
  expect(kda_cp_plan(&c, NULL, fake, NULL), KDA_ERR_INVALID_ARGUMENT, "cp P = 0");
  c.P = 3;
  expect(kda_cp_plan(&c, NULL, fake, NULL), KDA_ERR_INVALID_ARGUMENT, "cp T not a multiple of P");
  c.P = 2; c.K = 32;
  expect(kda_cp_chain(&c, fake, fake, fake, fake, NULL), KDA_ERR_NOT_IMPLEMENTED, "cp K = 32");

  /* layer steps */
  expect(kda_short_conv_fwd(1, 16, 64, 0, KDA_BF16, fake, fake, NULL, fake, NULL), KDA_ERR_INVALID_ARGUMENT,
         "conv W = 0");
  expect(kda_short_conv_fwd(1, 16, 64, 9, KDA_BF16, fake, fake, NULL, fake, NULL), KDA_ERR_NOT_IMPLEMENTED,
         "conv W = 9");
  expect(kda_short_conv_fwd(1, 16, 60, 4, KDA_BF16, fake, fake, NULL, fake, NULL), KDA_ERR_NOT_IMPLEMENTED,
         "conv D = 60");
  expect(kda_short_conv_fwd(1, 16, 64, 4, (kda_dtype_t)9, fake, fake, NULL, fake, NULL), KDA_ERR_INVALID_ARGUMENT,
         "conv bad dtype");
  expect(kda_gated_rmsnorm_fwd(4, 128, KDA_F32, (kda_dtype_t)5, KDA_BF16, fake, fake, fake, 1e-6f, fake, NULL),
         KDA_ERR_INVALID_ARGUMENT, "rmsnorm bad gate dtype");
  c.K = 128; c.B = (int64_t)1 << 40; c.n_states = 1 << 30;
  expect(kda_cp_plan(&c, NULL, fake, NULL), KDA_ERR_NOT_IMPLEMENTED, "cp sizes overflow");
  expect(kda_gated_rmsnorm_fwd(4, 96, KDA_F32, KDA_BF16, KDA_BF16, fake, fake, fake, 1e-6f, fake, NULL),
         KDA_ERR_NOT_IMPLEMENTED, "rmsnorm V = 96");
  expect(kda_gated_rmsnorm_fwd(4, 128, KDA_F32, KDA_BF16, KDA_BF16, fake, fake, fake, -1.f, fake, NULL),
         KDA_ERR_INVALID_ARGUMENT, "rmsnorm eps < 0");
  expect(kda_chunk_fwd_flags(NULL, 0, NULL, NULL), KDA_ERR_INVALID_ARGUMENT, "flags NULL");

  if (kda_version() == NULL || strncmp(kda_version(), "kda-mi355x", 10) != 0) {
    fprintf(stderr, "version string\n");
    ++fails;
  }
  if (fails) return 1;
  printf("ok\n");
  return 0;
}
