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
    std::vector<int32_t> nlo;     // first page streamed (sliding window), else 0
    std::vector<int32_t> splits;  // S_p
    std::vector<int32_t> unit_off;// P + 1 prefix offsets of work units
    size_t part_o_off = 0, part_rec_off = 0, ws_bytes = 0;
    size_t max_unit_pages = 0;
};

namespace smallw {
// First page any row of a request needs (0 without a sliding window): row 0
// has the lowest last key h0 = L - W (causal) or L - 1, and sees keys from
// h0 - window_left + 1 on.
inline int64_t first_page(int64_t L, int32_t W, int32_t causal, int32_t window_left) {
    if (window_left <= 0 || L <= 0) return 0;
    const int64_t lo = (causal ? L - W : L - 1) - window_left + 1;
    return lo > 0 ? lo / SMALLW_PAGE_SIZE : 0;
}

// Pages the sweep groups together for one step of its arithmetic: two-page
// chunks for bf16 pools, eight-page steps (128 tokens, one softmax each) for
// e4m3 and MXFP4 pools.  A row-exact piece must start on this grid so that
// every call groups the piece's pages the same way.
inline int32_t piece_align(int32_t kv_dtype) { return kv_dtype == SMALLW_KV_BF16 ? 2 : 8; }

// Page range [*pb, *pe) of split s of a request whose pages [n_lo, n) are
// streamed in S splits: balanced (split_pages == 0) or on the absolute grid of
// multiples of split_pages, the last piece ending at n and the first starting
// at n_lo moved down to a multiple of `align` pages from the piece's own grid
// point (so that every call groups the pages of a piece the same way).
inline void split_range(int64_t n_lo, int64_t n, int64_t S, int64_t s, int32_t split_pages,
                        int32_t align, int64_t* pb, int64_t* pe) {
    if (split_pages > 0) {
        const int64_t k = n_lo / split_pages + s;
        *pb = s == 0 ? k * split_pages + ((n_lo - k * split_pages) & ~int64_t(align - 1))
                     : k * split_pages;
        *pe = (s + 1 == S) ? n : (k + 1) * split_pages;
    } else {
        *pb = n_lo + s * (n - n_lo) / S;
        *pe = n_lo + (s + 1) * (n - n_lo) / S;
    }
}
// Planner core shared by small_w_attention_plan; num_cus must be resolved (> 0).
int build_plan(const smallw_problem& pr, const int32_t* seq_lens_host, smallw_plan** out);
void set_device_error(const char* what, int hip_status);
}  // namespace smallw
