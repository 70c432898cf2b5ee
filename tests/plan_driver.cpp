// Reads single-launch planning inputs, one case per line:
//   n_chunks kmax share share_max cand_max num_pages page_limit resident pairs xcds max_rounds
// and prints, per case: single n_val bg_round n_xcd
#include <cstdio>

#include "plan.hpp"

int main() {
  ckv::plan::Inputs in;
  while (std::scanf("%d %d %d %d %d %d %d %d %d %d %d", &in.n_chunks, &in.kmax, &in.share, &in.share_max,
                    &in.cand_max, &in.num_pages, &in.page_limit, &in.resident, &in.pairs, &in.xcds,
                    &in.max_rounds) == 11) {
    const ckv::plan::Layout L = ckv::plan::single_launch(in);
    std::printf("%d %d %d %d\n", L.single ? 1 : 0, L.n_val, L.bg_round, L.n_xcd);
  }
  return 0;
}
