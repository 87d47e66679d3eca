/* Runs every oracle entry point on small inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer (the oracle is plain C; this driver only
 * checks that it reads and writes inside its buffers and stays defined). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/mole_oracle.c"  /* the oracle itself, compiled into this driver */

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); return 1; } } while (0)

static float frand(unsigned* s) { *s = *s * 1664525u + 1013904223u; return ((*s >> 8) / 16777216.0f - 0.5f) * 0.1f; }

int main(void) {
  const int64_t V = 40, D = 128, F = 96, N = 3, T = 33;
  unsigned s = 7;
  float* emb = malloc(sizeof(float) * V * D);
  float* wu = malloc(sizeof(float) * N * F * D);
  float* wd = malloc(sizeof(float) * N * D * F);
  float* wr = malloc(sizeof(float) * N * D);
  float* h = malloc(sizeof(float) * T * D);
  float* lutf = malloc(sizeof(float) * V * N * D);
  double* lut = malloc(sizeof(double) * V * N * D);
  double* y = malloc(sizeof(double) * T * D);
  double* g = malloc(sizeof(double) * T * N);
  int64_t* ids = malloc(sizeof(int64_t) * T);
  for (int64_t i = 0; i < V * D; ++i) emb[i] = frand(&s);
  for (int64_t i = 0; i < N * F * D; ++i) { wu[i] = frand(&s); wd[i] = frand(&s); }
  for (int64_t i = 0; i < N * D; ++i) wr[i] = frand(&s) * 10.f;
  for (int64_t i = 0; i < T * D; ++i) h[i] = frand(&s) * 10.f;
  for (int64_t t = 0; t < T; ++t) ids[t] = (t * 7) % V;
  int64_t* rows = malloc(sizeof(int64_t) * V);
  for (int64_t v = 0; v < V; ++v) rows[v] = v;
  CHECK(oracle_build_lut_rows(emb, wu, wd, 0, V, D, F, N, rows, V, lut, 2) == 0);
  for (int64_t i = 0; i < V * N * D; ++i) lutf[i] = (float)lut[i];
  CHECK(oracle_router_gates(h, wr, 0, T, D, N, g, 2) == 0);
  CHECK(oracle_lookup_combine(ids, h, wr, 0, lutf, 0, T, V, D, N, y, 2) == 0);
  uint8_t* c3 = malloc(V * N * 3 * D / 8);
  uint16_t* s3 = malloc(sizeof(uint16_t) * V * N * (D / 64));
  uint8_t* u3 = malloc(V * N * D);
  double* dq = malloc(sizeof(double) * V * N * D);
  int64_t nsat = 0;
  CHECK(oracle_pack_nf3(lutf, 0, V * N, D, c3, s3, &nsat, 2) == 0);
  CHECK(oracle_unpack_nf3(c3, V * N, D, u3) == 0);
  CHECK(oracle_dequant_nf3(c3, s3, V * N, D, dq) == 0);
  CHECK(oracle_lookup_combine_nf3(ids, h, wr, 0, c3, s3, T, V, D, N, y, 2) == 0);
  uint8_t* c4 = malloc(V * N * D / 2);
  CHECK(oracle_pack_nf4(lutf, 0, V * N, D, c4, s3, &nsat, 2) == 0);
  int8_t* c8 = malloc(V * N * D);
  float* s8 = malloc(sizeof(float) * V * N);
  CHECK(oracle_pack_int8(lutf, 0, V * N, D, c8, s8, 2) == 0);
  ids[3] = V;  /* out of range: rejected */
  CHECK(oracle_lookup_combine(ids, h, wr, 0, lutf, 0, T, V, D, N, y, 2) != 0);
  free(emb); free(wu); free(wd); free(wr); free(h); free(lutf); free(lut); free(y); free(g); free(ids);
  free(rows); free(c3); free(s3); free(u3); free(dq); free(c4); free(c8); free(s8);
  printf("oracle driver: ok\n");
  return 0;
}
