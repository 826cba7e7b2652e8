// Host-only checks of the arithmetic the decode kernels share with the host
// (pkd_internal.hpp): the in-place merge's counter words, the balanced
// partition's pieces per segment, and the paired deal of whole items.
// Prints "ok" and returns 0 when every check holds; otherwise prints the first
// failure and returns 1.  Seeded, deterministic.
#include "pkd_internal.hpp"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

namespace {

int fail(const char* what, long long a, long long b) {
  std::printf("FAIL %s: %lld %lld\n", what, a, b);
  return 1;
}

// Every piece of a segment counts itself in, in a random order, starting from
// `start` (a stale word): exactly the last one sees the count complete, and it
// leaves the reset word behind.
int check_counter(std::mt19937_64& rng, uint64_t start, uint64_t tag, int npieces, uint64_t* left) {
  uint64_t w = start;
  int completed = 0, completed_at = -1;
  for (int i = 0; i < npieces; ++i) {
    w = pkd::count_word_add(w, tag);
    if (pkd::count_word_pieces(w) == npieces) {
      ++completed;
      completed_at = i;
      w = pkd::count_word_reset(tag);
    }
  }
  (void)rng;
  if (completed != 1) return fail("pieces completing the count", completed, npieces);
  if (completed_at != npieces - 1) return fail("completing piece", completed_at, npieces - 1);
  *left = w;
  return 0;
}

int counters() {
  std::mt19937_64 rng(1);
  const uint64_t mask40 = (1ull << 40) - 1;
  for (int trial = 0; trial < 20000; ++trial) {
    const uint64_t tag = pkd::call_tag(rng());
    if (tag == 0 || tag > mask40) return fail("tag range", (long long)tag, 0);
    const int npieces = 1 + (int)(rng() % 300);
    // Stale words: garbage, a word of another tag part-way through a count, a
    // completed call's reset word (another tag, or this one).
    uint64_t other = pkd::call_tag(tag + 1 + rng() % 1000);
    const uint64_t starts[4] = {rng(), (other << 24) | (rng() % 300), pkd::count_word_reset(other),
                                pkd::count_word_reset(tag)};
    for (uint64_t s : starts) {
      if ((s >> 24) == tag && s != pkd::count_word_reset(tag)) continue;  // a live count of this very call
      uint64_t left;
      if (check_counter(rng, s, tag, npieces, &left)) return 1;
      if (left != pkd::count_word_reset(tag)) return fail("word left behind", (long long)left, 0);
      // The next call counts from what this one left.
      const uint64_t next = pkd::call_tag(tag + 1);
      if (check_counter(rng, left, next, npieces, &left)) return 1;
    }
  }
  // Tags wrap at 2^40 and are never 0.
  if (pkd::call_tag(0) != 1 || pkd::call_tag(1ull << 40) != 1 || pkd::call_tag((1ull << 40) + 5) != 5 ||
      pkd::call_tag(mask40) != mask40)
    return fail("call_tag wrap", (long long)pkd::call_tag(1ull << 40), 1);
  // The largest tag still leaves the count's 24 bits intact.
  uint64_t w = pkd::count_word_reset(mask40);
  for (int i = 0; i < 5; ++i) w = pkd::count_word_add(w, mask40);
  if (pkd::count_word_pieces(w) != 5 || (w >> 24) != mask40) return fail("largest tag", (long long)w, 5);
  return 0;
}

// The balanced partition, walked workgroup by workgroup as the kernel does,
// against segment_pieces' closed form; slots w + s are distinct and below
// nwe + segments.
int partition() {
  std::mt19937_64 rng(2);
  for (int trial = 0; trial < 3000; ++trial) {
    const int B = 1 + (int)(rng() % 64);
    const int spb = 1 + (int)(rng() % 9);
    std::vector<int64_t> nb(B);
    std::vector<int64_t> pre(B + 1, 0);
    for (int b = 0; b < B; ++b) {
      const int r = (int)(rng() % 10);
      nb[b] = r == 0 ? 0 : r == 1 ? 1 : (int64_t)(rng() % 400);
      pre[b + 1] = pre[b] + nb[b] * spb;
    }
    const int64_t T = pre[B];
    if (T == 0) continue;
    const int64_t W = 1 + (int64_t)(rng() % 300);
    const int64_t nwe = std::min(W, T);
    const int64_t segs = (int64_t)B * spb;
    std::vector<int> pieces(segs, 0);
    std::vector<int64_t> first(segs, -1);
    std::vector<char> slot_used(nwe + segs, 0);
    for (int64_t w = 0; w < nwe; ++w) {
      const int64_t lo = w * T / nwe, hi = (w + 1) * T / nwe;
      if (hi <= lo) return fail("empty range", w, T);
      for (int64_t pos = lo; pos < hi;) {
        int b = (int)(std::upper_bound(pre.begin(), pre.end(), pos) - pre.begin()) - 1;
        const int seg = (int)((pos - pre[b]) / nb[b]);
        const int64_t s = (int64_t)b * spb + seg;
        const int64_t seg_end = pre[b] + (int64_t)(seg + 1) * nb[b];
        if (first[s] < 0) first[s] = w;
        ++pieces[s];
        if (slot_used[w + s]) return fail("slot reused", w, s);
        slot_used[w + s] = 1;
        pos = std::min(hi, seg_end);
      }
    }
    for (int b = 0; b < B; ++b)
      for (int seg = 0; seg < spb; ++seg) {
        const int64_t s = (int64_t)b * spb + seg;
        if (nb[b] == 0) {
          if (pieces[s] != 0) return fail("piece of an empty segment", s, pieces[s]);
          continue;
        }
        int64_t wf;
        int np;
        pkd::segment_pieces(pre[b] + (int64_t)seg * nb[b], nb[b], nwe, T, &wf, &np);
        if (wf != first[s] || np != pieces[s]) return fail("segment pieces", np, pieces[s]);
      }
  }
  return 0;
}

// The paired deal: every item to exactly one workgroup, at most two each, the
// longest 2W - N alone, and each pair's ranks adding up to 2E - 1.
int pairs() {
  for (int W = 1; W <= 300; W += (W < 20 ? 1 : 7)) {
    for (int N = 0; N <= 2 * W; ++N) {
      std::vector<int> owner(N, -1);
      for (int g = 0; g < W; ++g) {
        int a, b;
        pkd::paired_items(g, N, W, &a, &b);
        for (int it : {a, b}) {
          if (it < -1 || it >= N) return fail("item range", it, N);
          if (it < 0) continue;
          if (owner[it] >= 0) return fail("item dealt twice", it, g);
          owner[it] = g;
        }
        const int E = N - W;
        if (b >= 0 && (E <= 0 || a + b != 2 * E - 1 || a < b)) return fail("pair ranks", a, b);
        if (b < 0 && a >= 0 && E > 0 && a < 2 * E) return fail("a short item alone", a, E);
      }
      for (int it = 0; it < N; ++it)
        if (owner[it] < 0) return fail("item not dealt", it, N);
    }
  }
  return 0;
}

}  // namespace

int main() {
  if (counters() || partition() || pairs()) return 1;
  std::printf("ok\n");
  return 0;
}
