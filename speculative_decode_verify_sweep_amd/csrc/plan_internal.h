// Host-side plan object shared by the planner and the launch code.
#pragma once
#include <cstddef>
#include <cstdint>
#include <vector>

#include "smallw.h"

struct smallw_plan {
    smallw_problem prob;          // scale and num_cus resolved
    int32_t G = 0;                // query heads per KV head
    int32_t R = 0;                // rows per work unit: W * G
    int32_t U = 0;                // work units
    bool any_split = false;
    std::vector<int32_t> seq;     // host lengths the plan was built from
    std::vector<int32_t> npg;     // pages per request
    std::vector<int32_t> splits;  // S_p
    std::vector<int32_t> unit_off;// P + 1 prefix offsets of work units
    size_t part_o_off = 0, part_rec_off = 0, ws_bytes = 0;
    size_t max_unit_pages = 0;
};

namespace smallw {
// Planner core shared by small_w_attention_plan; num_cus must be resolved (> 0).
int build_plan(const smallw_problem& pr, const int32_t* seq_lens_host, smallw_plan** out);
void set_device_error(const char* what, int hip_status);
}  // namespace smallw
