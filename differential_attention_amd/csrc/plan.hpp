// plan.hpp -- host-only argument validation and launch planning.
// Compiled without any HIP header so it can be unit-tested on a CPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "diffattn.h"

namespace da {

// Split-KV decode plan. The work is the list of (sequence, KV head) units in
// order, each holding its sequence's pages; the split pass cuts this global
// page list into equal contiguous ranges, one per work-group, so every
// work-group streams the same number of pages whatever the length mix. A
// range may end inside a unit and may span several; each (work-group, unit)
// pair it touches yields one partial softmax state (max, sum, unnormalised
// output per query row) in the workspace, and a second pass merges the
// partial states of each unit.
constexpr int kDecodeMaxWgs = 2048;   // work-groups of the split pass, at most
constexpr int kDecodeMinPages = 4;    // pages per work-group, at least (library's choice)
constexpr int kDecodeMaxTarget = 1 << 24;
// Bytes of the static device scratch diffattn_decode_noalloc uses in place of
// a workspace (one array per device, for the life of the process).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;

struct DecodePlan {
    int target_pages = 0;      // pages per work-group asked for; 0 = library's choice
    int max_wgs = 0;           // work-groups the workspace is sized for
    int qrows = 0;             // query rows per KV head = 2 * (H / H_kv)
    size_t header_bytes = 0;   // int32 page prefix [B + 1], rounded up to 256 bytes
    size_t record_bytes = 0;   // one partial state: qrows * (d_v + 2) floats
    size_t ws_bytes = 0;       // workspace bytes: header + (max_wgs + B * H_kv) records
};

// Prefill kernel selection.
enum class PrefillKind { None, F32, Bf16 };

struct PrefillPlan {
    PrefillKind kind = PrefillKind::None;
    bool shared_k = false;  // k1 and k2 are the same tensor (one key tile feeds both branches)
    bool empty = false;     // nothing to compute (B == 0 or N == 0)
};

// Backward plan: the workspace holds the output gradient after the norm
// (bf16, one d_v row per query row), two per-row reductions (rowsum of the
// output gradient times each branch's normalised output) and, per block of
// kBwdPrepRows rows, the partial sums of dlambda and dgamma.
constexpr int kBwdPrepRows = 64;

struct BackwardPlan {
    bool shared_k = false;
    bool empty = false;
    int64_t rows = 0;        // B * H * N
    int64_t prep_blocks = 0; // B * H * ceil(N / kBwdPrepRows)
    size_t off_dy = 0, off_dt1 = 0, off_dt2 = 0, off_ls1 = 0, off_ls2 = 0, off_part = 0;
    size_t ws_bytes = 0;
};

// Validate backward sizes and flags (no pointer examined) and build the plan.
int check_backward_sizes(const diffattn_backward_args *a, BackwardPlan *plan, std::string *msg);

// Validate backward arguments (workspace excluded) and build the plan.
int check_backward(const diffattn_backward_args *a, BackwardPlan *plan, std::string *msg);

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

// Validate diffattn_lambda_backward arguments: sizes, null pointers, 4-byte
// alignment, and no output overlapping an input or another output.
int check_lambda_backward(const float *lq1, const float *lk1, const float *lq2, const float *lk2, int H,
                          int d_lambda, const float *dlambda, const float *dlq1, const float *dlk1,
                          const float *dlq2, const float *dlk2, std::string *msg);

}  // namespace da
