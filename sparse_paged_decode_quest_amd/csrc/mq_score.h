// Launcher of the several-query-token page scorer (mq_score.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/spd.h"
#include "spd_launch.h"

namespace spd {

constexpr int kMqScoreMaxTokens = SPD_MQ_MAX_TOKENS;  // query groups a scorer lane holds

// Scores of the num_tokens token rows of every request: `a` describes the requests (seq_lens: the
// last token's length L), a.q is [B, T, Hq, d] and a.scores [B * T, Hkv, max_pages].  Returns
// SPD_ERR_UNSUPPORTED for a (head_dim, kv_dtype) without a compiled kernel.
int launch_mq_page_score(const ScoreArgs& a, int num_tokens, int head_dim, int kv_dtype, hipStream_t stream);

}  // namespace spd
