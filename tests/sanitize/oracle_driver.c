/* Drives every entry point of the CPU oracle on small random problems, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers_cpu.py).
 * Includes the oracle's source so that its static helpers are built with the same
 * flags; prints "ok" and returns 0 when every call returns the expected status. */
#include "../../oracle/paged_attention_ref.c"

#include <stdio.h>

static uint32_t rng = 12345u;
static uint32_t next_u32(void) {
  rng = rng * 1664525u + 1013904223u;
  return rng;
}
static uint16_t rand_bf16(void) { /* values in about [-2, 2]: sign, exponent 120..127, mantissa */
  return (uint16_t)(((next_u32() & 1u) << 15) | ((120u + next_u32() % 8u) << 7) | (next_u32() & 0x7Fu));
}
static uint8_t rand_fp8(void) { uint8_t c = (uint8_t)(next_u32() & 0xFF); return (c & 0x7F) == 0x7F ? 0 : c; }

#define CHECK(x, want)                                                   \
  do {                                                                   \
    int st_ = (x);                                                       \
    if (st_ != (want)) {                                                 \
      printf("line %d: status %d, expected %d\n", __LINE__, st_, want); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main(void) {
  enum { B = 3, HQ = 8, HKV = 2, D = 32, PS = 5, MP = 8, NP = 24, QL = 3 };
  const int lens[B] = {0, 17, 40};
  int32_t bt[B * MP];
  int32_t sl[B];
  for (int b = 0; b < B; ++b) {
    sl[b] = lens[b];
    for (int i = 0; i < MP; ++i) bt[b * MP + i] = i < (lens[b] + PS - 1) / PS ? (b * MP + i) % NP : -1;
  }
  static uint16_t q[B * QL * HQ * D], kc[NP * PS * HKV * D], vc[NP * PS * HKV * D];
  static uint8_t k8[NP * PS * HKV * D], v8[NP * PS * HKV * D];
  for (size_t i = 0; i < sizeof(q) / 2; ++i) q[i] = rand_bf16();
  for (size_t i = 0; i < sizeof(kc) / 2; ++i) { kc[i] = rand_bf16(); vc[i] = rand_bf16(); k8[i] = rand_fp8(); v8[i] = rand_fp8(); }
  const float ks[HKV] = {0.5f, 0.25f}, vs[HKV] = {0.75f, 1.5f}, sinks[HQ] = {0, 1, -1, 2, -INFINITY, 0.5f, 3, -2};
  static double out[B * QL * HQ * D], lse[B * QL * HQ];
  for (int fp8 = 0; fp8 < 2; ++fp8) {
    const void* K = fp8 ? (const void*)k8 : (const void*)kc;
    const void* V = fp8 ? (const void*)v8 : (const void*)vc;
    const float* sk = fp8 ? ks : NULL;
    const float* sv = fp8 ? vs : NULL;
    for (int threads = 1; threads <= 3; threads += 2) {
      CHECK(pkd_oracle_paged_decode(B, HQ, HKV, D, PS, NP, MP, fp8, q, K, V, bt, sl, sk, sv, 0.17, out, lse, threads), 0);
      for (int S = 1; S <= 9; S += 4)
        CHECK(pkd_oracle_paged_decode_split(B, HQ, HKV, D, PS, NP, MP, fp8, q, K, V, bt, sl, sk, sv, 0.17, S, out, lse,
                                            threads), 0);
      for (int causal = 0; causal < 2; ++causal)
        CHECK(pkd_oracle_paged_decode_multi(B, HQ, HKV, D, PS, NP, MP, fp8, QL, causal, q, K, V, bt, sl, sk, sv, 0.17,
                                            out, lse, threads), 0);
      for (int window = 0; window <= 7; window += 7)
        CHECK(pkd_oracle_paged_decode_ext(B, HQ, HKV, D, PS, NP, MP, fp8, QL, 1, window, sinks, q, K, V, bt, sl, sk, sv,
                                          0.17, out, lse, threads), 0);
    }
    const int64_t rows[4] = {0, 5, 23, 23};
    CHECK(pkd_oracle_paged_decode_rows(B, HQ, HKV, D, PS, NP, MP, fp8, q, K, V, bt, sl, sk, sv, 0.17, 4, rows, out, lse), 0);
    CHECK(pkd_oracle_paged_decode_ext_rows(B, HQ, HKV, D, PS, NP, MP, fp8, QL, 1, 9, sinks, q, K, V, bt, sl, sk, sv,
                                           0.17, 4, rows, out, lse), 0);
    /* strided contiguous form: [B][L][Hkv][D] with L = MP * PS */
    const int64_t qs[3] = {QL * HQ * D, HQ * D, D}, kvs[3] = {(int64_t)MP * PS * HKV * D, HKV * D, D};
    static uint16_t ckc[B * MP * PS * HKV * D], cvc[B * MP * PS * HKV * D];
    for (size_t i = 0; i < sizeof(ckc) / 2; ++i) { ckc[i] = rand_bf16(); cvc[i] = rand_bf16(); }
    CHECK(pkd_oracle_contiguous_decode(B, HQ, HKV, D, MP * PS, 0, QL, 1, 6, sinks, q, qs, ckc, cvc, kvs, sl, NULL, NULL,
                                       0.17, out, lse, 2), 0);
  }
  /* contract violations are reported, not read */
  int32_t bad_bt[B * MP];
  memcpy(bad_bt, bt, sizeof(bt));
  bad_bt[2 * MP + 1] = NP;
  CHECK(pkd_oracle_paged_decode(B, HQ, HKV, D, PS, NP, MP, 0, q, kc, vc, bad_bt, sl, NULL, NULL, 0.1, out, lse, 1),
        PKD_ORACLE_BAD_PAGE);
  int32_t bad_sl[B] = {0, 17, MP * PS + 1};
  CHECK(pkd_oracle_paged_decode(B, HQ, HKV, D, PS, NP, MP, 0, q, kc, vc, bt, bad_sl, NULL, NULL, 0.1, out, lse, 1),
        PKD_ORACLE_BAD_LEN);
  /* merge */
  static double op[6 * 4 * D], lp[6 * 4], mo[6 * D], ml[6];
  for (int i = 0; i < 6 * 4 * D; ++i) op[i] = (double)(int)(next_u32() % 100) / 50.0 - 1.0;
  for (int i = 0; i < 24; ++i) lp[i] = i % 5 == 0 ? -INFINITY : (double)(next_u32() % 7);
  pkd_oracle_lse_merge(6, 4, D, op, lp, mo, ml);
  /* append, bf16 and FP8, with RoPE and padding */
  enum { N = 9, MAXPOS = 6 };
  static uint16_t kn[N * HKV * D], vn[N * HKV * D];
  for (int i = 0; i < N * HKV * D; ++i) { kn[i] = rand_bf16(); vn[i] = rand_bf16(); }
  int64_t slots[N], pos[N];
  for (int i = 0; i < N; ++i) { slots[i] = (i * 13) % (NP * PS); pos[i] = i % (MAXPOS + 2) - 1; }
  slots[3] = -1;
  slots[4] = NP * PS + 2;
  static float cs[MAXPOS * D];
  for (int i = 0; i < MAXPOS * D; ++i) cs[i] = (float)((int)(next_u32() % 200) - 100) / 100.0f;
  CHECK(pkd_oracle_kv_append(HKV, D, PS, NP, 0, N, kn, vn, slots, pos, cs, MAXPOS, kc, vc, NULL, NULL), 0);
  CHECK(pkd_oracle_kv_append(HKV, D, PS, NP, 1, N, kn, vn, slots, NULL, NULL, 0, k8, v8, ks, vs), 0);
  /* metadata with invalid entries */
  enum { MB = 4, RR = 5, RS = 30 };
  static int32_t r2t[RR * RS];
  for (int i = 0; i < RR * RS; ++i) r2t[i] = (int32_t)(next_u32() % (NP * PS));
  const int64_t rpi[MB] = {0, 4, 7, 2}, msl[MB] = {3, 29, 5, -2};
  int32_t cache_sl[MB], cu[MB + 1], pt[MB * MP], swa_sl[MB], swa_pt[MB * MP];
  CHECK(pkd_oracle_decode_metadata(MB, RR, RS, PS, MP, 2, 11, 1, r2t, rpi, msl, cache_sl, cu, pt, swa_sl, swa_pt), 2);
  /* scalar helpers on every code */
  double acc = 0;
  for (int c = 0; c < 65536; ++c) acc += isnan(pkd_oracle_bf16_value((uint16_t)c)) ? 0 : 1;
  for (int c = 0; c < 256; ++c) acc += isnan(pkd_oracle_fp8e4m3_value((uint8_t)c)) ? 0 : 1;
  for (int i = -460; i <= 460; ++i) acc += pkd_oracle_fp8e4m3_encode((float)i * 0.97f) + pkd_oracle_bf16_round((float)i / 7.0f);
  printf("ok %g\n", acc);
  return 0;
}
