// score.hip -- picks the streaming filter (score_filter.h) for the call's
// selection granularity and radius weight.
#include "internal.h"

namespace dkv {

hipError_t launch_score(const DecodeDims &d, const uint32_t *codes,
                        const uint8_t *radii, const int32_t *block_table,
                        const uint32_t *tasks, const uint32_t *qop,
                        const float *qneg, const uint32_t *lthr, uint2 *cand,
                        uint32_t *tcount, int32_t *scores_out,
                        hipStream_t stream) {
  auto *f = d.pages ? (d.lin ? launch_filter_pages_linear : launch_filter_pages_log)
                    : (d.lin ? launch_filter_keys_linear : launch_filter_keys_log);
  return f(d, codes, radii, block_table, tasks, qop, qneg, lthr, cand, tcount,
           scores_out, stream);
}

} // namespace dkv
