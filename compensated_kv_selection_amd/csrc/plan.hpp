// Layout of the single-launch decode step on a device: which (sequence, KV
// head) pairs run at once, how many value workgroups each pair gets, and
// whether each pair keeps to one XCD.  Plain host C++ (no HIP), so that the
// rules can be checked on a machine without a GPU.
#pragma once

#include <algorithm>

namespace ckv {
namespace plan {

// Value workgroups per pair and pairs per round when `pairs` pairs of
// `n_chunks` control workgroups each share `cap` resident workgroups: the
// fewest rounds, then the most value workgroups (one per chunk, down to one
// per four chunks).  rounds == 0: not even one pair fits.
struct Fit {
  int n_val = 0, per_round = 0, rounds = 0;
};
inline Fit fit_pairs(int n_chunks, int cap, int pairs) {
  Fit best;
  for (int nv = n_chunks; nv >= (n_chunks + 3) / 4; --nv) {
    const int per = std::min(pairs, cap / (n_chunks + nv));
    if (per < 1) continue;
    const int rounds = (pairs + per - 1) / per;
    if (best.rounds == 0 || rounds < best.rounds) best = Fit{nv, per, rounds};
  }
  return best;
}

struct Inputs {
  int n_chunks;     // control workgroups per pair
  int kmax;         // selected-block capacity per pair
  int share;        // selected blocks one control workgroup may attend to
  int share_max;    // ... that its shared memory holds
  int cand_max;     // candidates of all chunks its shared memory holds
  int num_pages;    // pages of the cache
  int page_limit;   // pages the selection keys can name
  int resident;     // workgroups of the kernel resident on the device at once
  int pairs;        // (sequence, KV head) pairs of the call
  int xcds;         // > 0: the device sends workgroup i to XCD i % xcds; 0: unknown / not so
  int max_rounds;   // rounds of pairs beyond which the three launches are faster
};

struct Layout {
  bool single = false;  // false: the three-launch path
  int n_val = 0;        // value workgroups per pair
  int bg_round = 0;     // pairs per round of the persistent grid
  int n_xcd = 0;        // > 0: every pair on one XCD (workgroup i on XCD i % n_xcd)
};

// One launch when its whole grid - at least the control workgroups of every
// chunk of one pair and a value workgroup per four chunks - can be resident
// at once, the pairs take at most max_rounds rounds of it, the pair's
// candidates fit in shared memory and page ids fit in its selection keys.
// (Every round is a full chain of dependent hand-offs; the three launches
// stream all pairs at once instead.)  Keeping every pair on one XCD is
// preferred when it takes no more rounds than spreading them.
inline Layout single_launch(const Inputs& in) {
  Layout out;
  if (in.share > in.share_max || in.n_chunks * in.kmax > in.cand_max) return out;
  if (in.num_pages >= in.page_limit) return out;
  const Fit spread = fit_pairs(in.n_chunks, in.resident, in.pairs);
  if (spread.rounds == 0 || spread.rounds > in.max_rounds) return out;
  out.single = true;
  out.n_val = spread.n_val;
  out.bg_round = spread.per_round;
  if (in.xcds > 0) {
    const Fit local = fit_pairs(in.n_chunks, in.resident / in.xcds, (in.pairs + in.xcds - 1) / in.xcds);
    if (local.rounds > 0 && local.rounds <= spread.rounds) {
      out.n_xcd = in.xcds;
      out.n_val = local.n_val;
      out.bg_round = std::min(in.pairs, in.xcds * local.per_round);
    }
  }
  return out;
}

}  // namespace plan
}  // namespace ckv
