/* Host-side driver for the sanitizer build of libmpq: exercises argument
 * validation, workspace sizing, codebook recognition and table building
 * (which run on the host before any device work) with no GPU present.
 * argv[1]: a raw float32 file holding an E8-prefix codebook (K x 8),
 * argv[2]: its K.  Prints one line per check and "ok" at the end; exits
 * non-zero on the first unexpected status. */
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>
#include "mpq.h"

static int fails = 0;
#define EXPECT(cond, what)                          \
  do {                                              \
    if (!(cond)) {                                  \
      fprintf(stderr, "FAILED: %s\n", what);        \
      ++fails;                                      \
    }                                               \
  } while (0)

int main(int argc, char** argv) {
  if (argc < 3) return 2;
  const int64_t K = atoll(argv[2]);
  float* E = (float*)malloc((size_t)K * 8 * sizeof(float));
  FILE* f = fopen(argv[1], "rb");
  if (!f || fread(E, sizeof(float), (size_t)K * 8, f) != (size_t)K * 8) return 3;
  fclose(f);
  void* fake = (void*)(uintptr_t)(1 << 20);   /* never dereferenced: validation fails first */

  /* sizes */
  EXPECT(mpq_workspace_bytes(64, 256, 256, 8, 1) > 0, "workspace bytes scalar");
  EXPECT(mpq_workspace_bytes(4096, 14336, 14336, 65536, 8) > 0, "workspace bytes lattice");
  EXPECT(mpq_workspace_bytes(4, 10, 11, 8, 1) == 0, "workspace r > n");
  EXPECT(mpq_workspace_bytes(4, 16, 16, 8, 3) == 0, "workspace d");
  EXPECT(mpq_codebook_bytes(K, 8) > 0 && mpq_codebook_bytes(70000, 8) == 0, "codebook bytes");
  EXPECT(mpq_greedy_workspace_bytes(64, 256, 256, 8, 1) > mpq_workspace_bytes(64, 256, 256, 8, 1), "greedy bytes");

  /* codebook recognition and the automaton (host tables) */
  EXPECT(mpq_codebook_kind(E, K, 8) == MPQ_CB_E8_PREFIX, "E8 prefix recognised");
  EXPECT(mpq_e8dp_transitions(E, K) > 0, "E8 transitions");
  float* Es = (float*)malloc((size_t)K * 8 * sizeof(float));
  memcpy(Es, E, (size_t)K * 8 * sizeof(float));
  float tmp[8];
  memcpy(tmp, Es, sizeof(tmp));
  memcpy(Es, Es + 8 * (K - 1), sizeof(tmp));
  memcpy(Es + 8 * (K - 1), tmp, sizeof(tmp));
  EXPECT(mpq_codebook_kind(Es, K, 8) == MPQ_CB_GENERIC, "shuffled codebook is generic");
  EXPECT(mpq_e8dp_transitions(Es, K) == 0, "no transitions for a generic codebook");

  /* codebook preparation: validation, then the host tables (the copy to the
     fake device address fails without a GPU, after the tables are built) */
  mpq_codebook cb;
  memset(&cb, 0, sizeof(cb));
  EXPECT(mpq_codebook_prepare(NULL, K, 8, fake, 1u << 30, NULL, &cb) == MPQ_ENULL, "prepare null");
  EXPECT(mpq_codebook_prepare(E, K, 8, fake, 1024, NULL, &cb) == MPQ_EWORKSPACE, "prepare small");
  EXPECT(mpq_codebook_prepare(E, K, 3, fake, 1u << 30, NULL, &cb) == MPQ_EUNSUPPORTED, "prepare d");
  {
    int rc = mpq_codebook_prepare(E, K, 8, fake, 1u << 30, NULL, &cb);
    EXPECT(rc == MPQ_EHIP || rc == MPQ_OK, "prepare builds its tables");
    rc = mpq_codebook_prepare(Es, K, 8, fake, 1u << 30, NULL, &cb);
    EXPECT(rc == MPQ_EHIP || rc == MPQ_OK, "prepare builds generic tables");
  }
  float lv[8] = {0, 1, 2, 3, 4, 5, 6, 7};
  {
    int rc = mpq_codebook_prepare(lv, 8, 1, fake, 1u << 30, NULL, &cb);
    EXPECT(rc == MPQ_EHIP || rc == MPQ_OK, "prepare scalar");
  }

  /* solve validation with a hand-filled prepared codebook */
  mpq_codebook fcb;
  memset(&fcb, 0, sizeof(fcb));
  fcb.K = 8;
  fcb.d = 1;
  fcb.tables = fake;
  fcb.magic = 0x4d50514342763200ull;
  int32_t* codes = (int32_t*)fake;
  EXPECT(mpq_quantize_layer(fake, 4, 16, fake, fake, 16, &fcb, fake, fake, -1, 1, 0.5f, NULL, codes, NULL, NULL,
                            NULL, NULL, fake, 1u << 30, NULL) == MPQ_EPARAM, "T_vamp < 0");
  EXPECT(mpq_quantize_layer(fake, 4, 16, fake, fake, 17, &fcb, fake, fake, 2, 1, 0.5f, NULL, codes, NULL, NULL,
                            NULL, NULL, fake, 1u << 30, NULL) == MPQ_ESHAPE, "r > n");
  EXPECT(mpq_quantize_layer(fake, 4, 16, fake, fake, 16, &fcb, fake, fake, 2, 1, 0.5f, NULL, codes, NULL, NULL,
                            NULL, NULL, fake, 1024, NULL) == MPQ_EWORKSPACE, "small workspace");
  mpq_options opt;
  memset(&opt, 0, sizeof(opt));
  opt.safeguard_eps = -1.f;
  EXPECT(mpq_quantize_layer(fake, 4, 16, fake, fake, 16, &fcb, fake, fake, 2, 1, 0.5f, &opt, codes, NULL, NULL,
                            NULL, NULL, fake, 1u << 30, NULL) == MPQ_EPARAM, "safeguard_eps < 0");
  memset(&opt, 0, sizeof(opt));
  opt.group = 4;
  opt.anchor_tau = 0.2f;
  EXPECT(mpq_quantize_layer(fake, 4, 16, fake, fake, 16, &fcb, fake, fake, 2, 1, 0.5f, &opt, codes, NULL, NULL,
                            NULL, NULL, fake, 1u << 30, NULL) == MPQ_EUNSUPPORTED, "groups with the anchor");
  fcb.magic = 0;
  EXPECT(mpq_quantize_layer(fake, 4, 16, fake, fake, 16, &fcb, fake, fake, 2, 1, 0.5f, NULL, codes, NULL, NULL,
                            NULL, NULL, fake, 1u << 30, NULL) == MPQ_EPARAM, "unprepared codebook");
  EXPECT(mpq_linear_step(fake, fake, fake, fake, 4, 16, fake, fake, 17, 0.5f, NULL, fake, fake, fake, 1u << 30,
                         NULL) == MPQ_ESHAPE, "linear step r > n");
  EXPECT(mpq_rht(fake, 4, 12, fake, NULL) == MPQ_EUNSUPPORTED, "rht n");
  EXPECT(mpq_gram(fake, 10, 0, fake, fake, 1u << 30, NULL) == MPQ_ESHAPE, "gram n");
  for (int s = 0; s >= -9; --s) EXPECT(strlen(mpq_strerror(s)) > 0, "strerror");
  EXPECT(strlen(mpq_hip_error_name()) > 0, "hip error name");

  /* profiler: created and destroyed (event creation fails without a GPU) */
  mpq_profiler* p = NULL;
  EXPECT(mpq_profiler_create(0, &p) == MPQ_EPARAM, "profiler capacity");
  {
    int rc = mpq_profiler_create(4, &p);
    EXPECT(rc == MPQ_OK || rc == MPQ_EHIP, "profiler create");
    mpq_profiler_destroy(p);
  }
  free(E);
  free(Es);
  if (fails) return 1;
  printf("ok\n");
  return 0;
}
