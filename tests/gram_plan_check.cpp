// Host check of the Gram's work plan (csrc/gram.hip): for each (K, Mp) given on
// the command line as K:Mp, every tile on or above the diagonal is covered
// exactly once over all calibration stages (whole, or as pieces that partition
// the stages on flush-chunk boundaries), no tile below it is touched, every
// partial-buffer slot is written by exactly one piece and lies inside
// gram_partial_bytes, and the fix-up pass visits each split tile once.
// Prints one line per case and exits non-zero on the first inconsistency.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "gram.hip"

using namespace awq;

static int check(int K, long Mp) {
  const GramPlan p = gram_plan(K, Mp);
  const int nb = K / kGT, stages = (int)(Mp / 64);
  std::vector<int> covered((size_t)nb * nb, 0), whole((size_t)nb * nb, 0), slot_use(p.piece_slots, 0);
  for (int x = 0; x < 8; ++x)
    for (int q = 0; q < p.blocks_per_xcd; ++q) {
      const GramWork w = gram_work(p, x, q, Mp);
      if (w.tq < 0) continue;
      int I, J;
      if (!gram_tile(x, w.tq, nb, I, J)) {
        if (w.slot >= 0) return printf("K=%d Mp=%ld: piece of a tile past XCD %d's list\n", K, Mp, x), 1;
        continue;
      }
      if (w.t0 >= w.t1 || w.t1 > stages || w.t0 % kGFlush != 0)
        return printf("K=%d Mp=%ld: stages [%d, %d) of %d\n", K, Mp, w.t0, w.t1, stages), 1;
      covered[(size_t)I * nb + J] += w.t1 - w.t0;
      if (w.slot < 0) {
        whole[(size_t)I * nb + J] += 1;
      } else {
        if (w.slot >= p.piece_slots) return printf("K=%d Mp=%ld: slot %d of %d\n", K, Mp, w.slot, p.piece_slots), 1;
        slot_use[w.slot] += 1;
      }
    }
  for (int I = 0; I < nb; ++I)
    for (int J = 0; J < nb; ++J) {
      const int c = covered[(size_t)I * nb + J], want = J >= I ? stages : 0;
      if (c != want) return printf("K=%d Mp=%ld: tile (%d, %d) covers %d stages, not %d\n", K, Mp, I, J, c, want), 1;
    }
  for (int s = 0; s < p.piece_slots; ++s)
    if (slot_use[s] != 1) return printf("K=%d Mp=%ld: slot %d written %d times\n", K, Mp, s, slot_use[s]), 1;
  if ((size_t)p.piece_slots * kGT * kGT * sizeof(double) != gram_partial_bytes(K, Mp))
    return printf("K=%d Mp=%ld: partial bytes disagree\n", K, Mp), 1;
  int fixed = 0;
  for (int x = 0; x < 8; ++x)
    for (int l = 0; l < p.fixup_per_xcd; ++l) {
      if (l >= p.left[x]) continue;
      int I, J;
      if (!gram_tile(x, p.full[x] + l, nb, I, J) || whole[(size_t)I * nb + J] != 0)
        return printf("K=%d Mp=%ld: fix-up block (%d, %d) has no split tile\n", K, Mp, x, l), 1;
      ++fixed;
    }
  int split = 0;
  for (int x = 0; x < 8; ++x) split += p.left[x];
  if (fixed != split) return printf("K=%d Mp=%ld: %d split tiles, %d fixed up\n", K, Mp, split, fixed), 1;
  printf("K=%d Mp=%ld blocks=%d split=%d slots=%d\n", K, Mp, 8 * p.blocks_per_xcd, split, p.piece_slots);
  return 0;
}

int main(int argc, char** argv) {
  for (int i = 1; i < argc; ++i) {
    int K = 0;
    long Mp = 0;
    if (sscanf(argv[i], "%d:%ld", &K, &Mp) != 2 || K % kGT != 0 || Mp % 64 != 0 || K <= 0 || Mp <= 0)
      return printf("bad case %s\n", argv[i]), 2;
    if (check(K, Mp)) return 1;
  }
  return 0;
}
