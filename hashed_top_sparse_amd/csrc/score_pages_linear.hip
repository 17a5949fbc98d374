// score_pages_linear.hip -- the streaming filter for page candidates, linear radius weight.
#include "score_filter.h"

namespace dkv {

DKV_FILTER_DECL(launch_filter_pages_linear) {
  return launch_filter_impl<true, true>(d, codes, radii, block_table, tasks, qop,
                                       qneg, lthr, cand, tcount, scores_out, stream);
}

} // namespace dkv
