// plan.hpp -- host-only argument validation and launch planning.
// Compiled without any HIP header so it can be unit-tested on a CPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "diffattn.h"

namespace da {

// Split-KV decode plan: the pages of each sequence are cut into splits of
// split_pages pages; every (sequence, KV head, split) is one work item whose
// partial softmax state (max, sum, unnormalised output per query row) goes to
// the workspace, and a second pass merges the splits.
struct DecodePlan {
    int split_pages = 0;  // pages per split
    int num_splits = 0;   // splits per sequence (for the longest possible sequence)
    int qrows = 0;        // query rows per KV head = 2 * (H / H_kv)
    size_t ws_bytes = 0;  // workspace bytes
};

// Prefill kernel selection.
enum class PrefillKind { None, F32, Bf16 };

struct PrefillPlan {
    PrefillKind kind = PrefillKind::None;
    bool shared_k = false;  // k1 and k2 are the same tensor (one key tile feeds both branches)
    bool empty = false;     // nothing to compute (B == 0 or N == 0)
};

// lambda_init(depth) = 0.8 - 0.6 exp(-0.3 (depth - 1)); NaN for depth < 1.
double lambda_init(int depth);

// Validate prefill arguments. Returns DIFFATTN_OK or a negative status with *msg set.
int check_prefill(const diffattn_prefill_args *a, PrefillPlan *plan, std::string *msg);

// Validate the sizes and flags of decode arguments (no pointer is examined)
// and build the plan.
int check_decode_sizes(const diffattn_decode_args *a, DecodePlan *plan, std::string *msg);

// Validate decode arguments (workspace excluded) and build the plan.
int check_decode(const diffattn_decode_args *a, DecodePlan *plan, std::string *msg);

// Validate diffattn_lambda arguments.
int check_lambda(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                 int d_lambda, int depth, const float *out, std::string *msg);

}  // namespace da
