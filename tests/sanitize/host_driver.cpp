// Drives the library's host-side code (argument checks, the split heuristic, the
// workspace and launch planning of every entry point) with valid, invalid and
// extreme arguments, for a build of the host code with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers_cpu.py).  Pointer arguments
// are fake non-NULL addresses that the library must never dereference on these
// paths: without a device every call ends before a launch.  Prints "ok" and
// returns 0 when every status is the expected one.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/paged_kv_decode.h"
#include "../../include/pkd_stream.h"
#include "../../include/pkd_lds.h"
#include "../../include/pkd_valu.h"

namespace {

void* const F = reinterpret_cast<void*>(0x1000);
const int32_t* const FI = reinterpret_cast<const int32_t*>(0x1000);
float* const FF = reinterpret_cast<float*>(0x1000);
int failures = 0;

void expect(int got, int want, int line) {
  if (got != want) {
    std::printf("line %d: status %d, expected %d\n", line, got, want);
    ++failures;
  }
}
#define EXPECT(x, want) expect((x), (want), __LINE__)

pkd_dims dims(int b, int hq, int hkv, int d, int ps, int np, int mp, int dt) {
  pkd_dims x;
  x.batch = b;
  x.num_q_heads = hq;
  x.num_kv_heads = hkv;
  x.head_dim = d;
  x.page_size = ps;
  x.num_pages = np;
  x.max_pages_per_seq = mp;
  x.kv_dtype = dt;
  return x;
}

}  // namespace

int main() {
  const int S_MODES[] = {PKD_SPLITS_AUTO, 1, 2, 7, PKD_MAX_SPLITS, PKD_MAX_SPLITS + 1, -1, -77, PKD_SPLITS_BALANCED,
                         INT32_MIN, INT32_MAX};
  const int EXT_Q[] = {1, 2, 5, PKD_MAX_Q_LEN};
  const int BATCHES[] = {0, 1, 31, 32, 33, 128, 1024, 1025, 65535, INT32_MAX};
  const int HEADS[][2] = {{32, 8}, {16, 2}, {4, 4}, {64, 1}, {6, 4}, {INT32_MAX, 1}};
  const int DIMS[] = {32, 64, 128, 256, 96, 0};
  const int PAGES[][2] = {{16, 64}, {64, 2048}, {24, 171}, {1, 1}, {4096, 1 << 20}, {INT32_MAX, 2}};
  long calls = 0;
  for (int b : BATCHES)
    for (auto& h : HEADS)
      for (int d : DIMS)
        for (auto& pg : PAGES)
          for (int dt = 0; dt < 3; ++dt) {
            const pkd_dims x = dims(b, h[0], h[1], d, pg[0], 1 << 20, pg[1], dt);
            const float* sc = dt == PKD_DTYPE_FP8_E4M3 ? FF : nullptr;
            for (int S : S_MODES) {
              for (int ql : EXT_Q)
                for (int causal = 0; causal < 2; ++causal)
                  for (int win : {0, 1, 1000, INT32_MAX}) {
                    pkd_ext e{ql, causal, win, 0};
                    const size_t ws = paged_decode_workspace_bytes_ext(&x, &e, S);
                    const int ns = paged_decode_num_splits_ext(&x, &e, 4096);
                    const int nl = paged_decode_launches(&x, &e, S);
                    const int np = paged_decode_path(&x, &e, S);
                    (void)ns;
                    (void)nl;
                    (void)np;
                    const int st = paged_decode_ext(&x, &e, F, F, F, FI, FI, sc, sc, FF, 0.125f, F, FF, S, F,
                                                    ws ? ws : 256, nullptr);
                    // without a device: an argument error, or the missing device
                    if (st >= 0) EXPECT(st == 0 && b == 0 ? 0 : st, 0);
                    paged_decode_partition(&x, &e, F, F, F, FI, FI, sc, sc, 0.125f, S, F, ws, nullptr);
                    paged_decode_finish(&x, &e, S, F, ws, FF, F, FF, nullptr);
                    paged_decode_partials(&x, &e, F, F, F, FI, FI, sc, sc, 0.125f, S, FF, FF, nullptr);
                    paged_decode_ext_noalloc(&x, &e, F, F, F, FI, FI, sc, sc, FF, 0.125f, F, FF, S, nullptr);
                    calls += 6;
                  }
              const size_t ws = paged_decode_workspace_bytes(&x, S);
              paged_decode(&x, F, F, F, FI, FI, sc, sc, 0.125f, F, FF, S, F, ws ? ws : 256, nullptr);
              paged_decode_num_splits(&x, S);
              paged_kv_append(&x, S, F, F, reinterpret_cast<const int64_t*>(F), nullptr, nullptr, 0, F, F, sc, sc,
                              nullptr);
              pkd_decode_valu(&x, F, F, F, FI, FI, 0.125f, F, FF, nullptr);
              pkd_decode_lds(&x, F, F, F, FI, FI, 0.125f, F, FF, nullptr);
              pkd_decode_registers(&x, F, F, F, FI, FI, 0.125f, F, FF, nullptr);
              paged_decode_check_tables(&x, FI, FI, reinterpret_cast<int32_t*>(F), nullptr);
              calls += 5;
            }
          }
  // the merge, metadata, contiguous and stream entries
  for (int64_t rows : {(int64_t)0, (int64_t)1, (int64_t)1 << 40, (int64_t)-1})
    for (int S : {0, 1, 512, 513})
      for (int d : {32, 256, 100}) paged_decode_merge(rows, S, d, FF, FF, F, FF, nullptr);
  for (int b : {0, 1, 65535, 65536})
    for (int w : {0, 5, INT32_MAX}) {
      pkd_meta_dims md{b, 4, 100, 16, 7, 1, w, 1};
      paged_decode_metadata(&md, FI, reinterpret_cast<const int64_t*>(F), reinterpret_cast<const int64_t*>(F),
                            reinterpret_cast<int32_t*>(F), reinterpret_cast<int32_t*>(F), reinterpret_cast<int32_t*>(F),
                            reinterpret_cast<int32_t*>(F), reinterpret_cast<int32_t*>(F),
                            reinterpret_cast<int32_t*>(F), nullptr);
    }
  for (int b : {0, 3, INT32_MAX})
    for (int L : {1, 4096, INT32_MAX}) {
      pkd_contig_dims cd;
      std::memset(&cd, 0, sizeof cd);
      cd.batch = b;
      cd.num_q_heads = 8;
      cd.num_kv_heads = 2;
      cd.head_dim = 128;
      cd.max_seq_len = L;
      cd.q_len = 1;
      for (int i = 0; i < 3; ++i) {
        cd.q_strides[i] = cd.out_strides[i] = (int64_t)8 << (4 * i);
        cd.kv_strides[i] = (int64_t)128 << (5 * i);
      }
      for (int S : {0, 1, 5, PKD_SPLITS_BALANCED}) {
        const size_t ws = contiguous_decode_workspace_bytes(&cd, S);
        contiguous_decode(&cd, F, F, F, FI, nullptr, nullptr, nullptr, 0.1f, F, FF, S, F, ws, nullptr);
      }
    }
  for (int64_t bytes : {(int64_t)1 << 20, (int64_t)1 << 40, (int64_t)3})
    for (int wgs : {1, 256, 1 << 20, (1 << 20) + 1})
      for (int pattern : {0, 1, 2, 3})
        for (int waves : {4, 8})
          for (int kb : {4, 16, 32})
            pkd_stream_read(F, bytes, 2048, 256, pattern, wgs, waves, kb, 1, reinterpret_cast<uint32_t*>(F), nullptr);
  size_t text = 0;
  for (int st = -20; st <= 1; ++st) text += std::strlen(paged_decode_status_string(st));
  if (text == 0) ++failures;
  // a valid plain call without a device reports the missing device (or runs, on a GPU machine)
  const pkd_dims ok = dims(32, 32, 8, 128, 64, 2048, 64, PKD_DTYPE_BF16);
  const int st = paged_decode(&ok, F, F, F, FI, FI, nullptr, nullptr, 0.125f, F, nullptr, 1, nullptr, 0, nullptr);
  EXPECT(st == PKD_ERR_DEVICE || st == PKD_OK ? 0 : st, 0);
  std::printf("ok %ld calls, %d failures\n", calls, failures);
  return failures ? 1 : 0;
}
