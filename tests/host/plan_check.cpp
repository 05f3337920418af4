// Host-side driver of the kernels' mask geometry (attn_common.h), compiled
// with hipcc for the CPU only.  Reads cases "Sq Sk causal window input_pos
// k_len tile_m tile_n prefix" from stdin; for each prints the tile plan (one line of
// digits per query tile) and then the per-row [lo, hi) key intervals.
#include <cstdio>

#include "attn_common.h"

int main() {
  int Sq, Sk, causal, window, ip, kl, tm, tn, prefix;
  while (std::scanf("%d %d %d %d %d %d %d %d %d", &Sq, &Sk, &causal, &window,
                    &ip, &kl, &tm, &tn, &prefix) == 9) {
    const int nqt = (Sq + tm - 1) / tm, nkt = (Sk + tn - 1) / tn;
    const int k = kl < 0 ? 0 : (kl > Sk ? Sk : kl);
    std::printf("plan %d %d\n", nqt, nkt);
    for (int qt = 0; qt < nqt; ++qt) {
      const int i0 = qt * tm, i1 = (i0 + tm < Sq) ? i0 + tm : Sq;
      const attn::KvGeometry g = attn::kv_geometry(i0, i1, k, causal, window, ip, prefix);
      for (int kt = 0; kt < nkt; ++kt)
        std::printf("%d", attn::tile_class(g, kt * tn, tn));
      std::printf("\n");
    }
    std::printf("rows %d\n", Sq);
    for (int i = 0; i < Sq; ++i) {
      const attn::RowRange r = attn::row_range(i, k, causal, window, ip, prefix);
      std::printf("%d %d\n", r.lo, r.hi);
    }
  }
  return 0;
}
