// score_keys_linear.hip -- the streaming filter for key candidates, linear radius weight.
#include "score_filter.h"

namespace dkv {

DKV_FILTER_DECL(launch_filter_keys_linear) {
  return launch_filter_impl<true, false>(d, codes, radii, block_table, tasks, qop,
                                       qneg, lthr, cand, tcount, scores_out, stream);
}

} // namespace dkv
