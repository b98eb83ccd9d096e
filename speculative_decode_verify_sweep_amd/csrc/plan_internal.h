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
    bool any_split = false;       // some request has S_p > 1
    bool combine = false;         // partials + combine kernel: any_split or row-exact
    std::vector<int32_t> seq;     // host lengths the plan was built from
    std::vector<int32_t> npg;     // pages per request
    std::vector<int32_t> splits;  // S_p
    std::vector<int32_t> unit_off;// P + 1 prefix offsets of work units
    size_t part_o_off = 0, part_rec_off = 0, ws_bytes = 0;
    size_t max_unit_pages = 0;
};

namespace smallw {
// Page range [*pb, *pe) of split s of a request with n pages and S splits:
// balanced (split_pages == 0) or at multiples of split_pages.
inline void split_range(int64_t n, int64_t S, int64_t s, int32_t split_pages, int64_t* pb,
                        int64_t* pe) {
    if (split_pages > 0) {
        *pb = s * split_pages;
        *pe = (s + 1 == S) ? n : (s + 1) * split_pages;
    } else {
        *pb = s * n / S;
        *pe = (s + 1) * n / S;
    }
}
// Planner core shared by small_w_attention_plan; num_cus must be resolved (> 0).
int build_plan(const smallw_problem& pr, const int32_t* seq_lens_host, smallw_plan** out);
void set_device_error(const char* what, int hip_status);
}  // namespace smallw
