// score_pages_log.hip -- the streaming filter for page candidates, log radius weight.
#include "score_filter.h"

namespace dkv {

DKV_FILTER_DECL(launch_filter_pages_log) {
  return launch_filter_impl<false, true>(d, codes, radii, block_table, tasks, qop,
                                       qneg, lthr, cand, tcount, scores_out, stream);
}

} // namespace dkv
