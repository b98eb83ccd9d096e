// Planner stress for host sanitizer builds (AddressSanitizer, UBSan): random
// problems, valid and invalid, through build_plan, plan export (buffer too
// small, then exact), workspace size, largest unit and destroy.  For every
// accepted plan it also checks that the export partitions each request's
// streamed pages among its units.  Test infrastructure: host C++ only.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>
#include <vector>

#include "plan_internal.h"

namespace {

std::mt19937_64 rng(20261202);

template <typename T>
T pick(std::initializer_list<T> v) {
    return *(v.begin() + std::uniform_int_distribution<size_t>(0, v.size() - 1)(rng));
}

int fail(const char* what, int it) {
    std::fprintf(stderr, "plan_stress: %s (iteration %d)\n", what, it);
    return 1;
}

}  // namespace

int main(int argc, char** argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
    int accepted = 0, rejected = 0;
    for (int it = 0; it < iters; ++it) {
        // a valid problem, then (30% of the time) one field made invalid
        smallw_problem pr{};
        pr.num_reqs = pick<int32_t>({1, 1, 2, 3, 8, 64, 256});
        pr.num_kv_heads = pick<int32_t>({1, 2, 4, 8});
        pr.head_dim = pick<int32_t>({64, 128, 256, 256});
        pr.kv_dtype = pick<int32_t>({0, 1, 2});
        if (pr.kv_dtype == 2 && pr.head_dim == 64) pr.head_dim = 128;
        const int32_t G = pick<int32_t>({1, 2, 3, 4, 6, 8});
        pr.num_q_heads = pr.num_kv_heads * G;
        pr.window = std::uniform_int_distribution<int32_t>(1, std::min(16, 128 / G))(rng);
        pr.page_size = 16;
        pr.max_pages_per_req = pick<int32_t>({1, 2, 17, 300, 4097, 100000});
        pr.num_pages = pick<int32_t>({1, 5000, 1 << 20});
        pr.causal = pick<int32_t>({0, 1, 1});
        pr.scale = pick<float>({0.f, 0.0625f, -1.f});
        pr.num_cus = pick<int32_t>({1, 80, 256, 304, 512});
        pr.force_splits = pick<int32_t>({0, 0, 0, 1, 2, 3, 17, 200});
        pr.split_pages = pr.force_splits ? 0 : pick<int32_t>({0, 0, 0, 1, 5, 9, 65});
        pr.window_left = pick<int32_t>({0, 0, 1, 7, 4096, 1 << 30});
        pr.v_layout = pr.kv_dtype == 0 ? pick<int32_t>({0, 1}) : 0;
        const int64_t cap = int64_t(pr.max_pages_per_req) * 16;
        std::vector<int32_t> seq(SMALLW_MAX_REQS + 1);
        for (auto& L : seq) {
            const int64_t r = std::uniform_int_distribution<int64_t>(pr.window, cap)(rng);
            L = int32_t(r >= pr.window ? pick<int64_t>({0, pr.window, r, r, r, cap}) : 0);
            if (L > cap) L = int32_t(cap);
        }
        if (std::uniform_int_distribution<int>(0, 9)(rng) < 3) {
            switch (std::uniform_int_distribution<int>(0, 15)(rng)) {
                case 0: pr.num_reqs = pick<int32_t>({0, -1, 257}); break;
                case 1: pr.window = pick<int32_t>({0, 17}); break;
                case 2: pr.num_kv_heads = pick<int32_t>({0, 3}); break;
                case 3: pr.num_q_heads += 1; break;
                case 4: pr.head_dim = pick<int32_t>({0, 96}); break;
                case 5: pr.page_size = 8; break;
                case 6: pr.num_pages = 0; break;
                case 7: pr.causal = 2; break;
                case 8: pr.kv_dtype = 3; break;
                case 9: pr.scale = pick<float>({std::numeric_limits<float>::quiet_NaN(),
                                               std::numeric_limits<float>::infinity()}); break;
                case 10: pr.force_splits = -1; break;
                case 11: pr.split_pages = -2; break;
                case 12: pr.window_left = -1; break;
                case 13: seq[0] = pick<int32_t>({-1, int32_t(cap + 1)}); break;
                case 14: pr.v_layout = pick<int32_t>({-1, 2}); break;
                default: if (pr.window > 1) { pr.causal = 1; seq[0] = pr.window - 1; } break;
            }
        }
        smallw_plan* pl = nullptr;
        const int rc = smallw::build_plan(pr, seq.data(), &pl);
        if (rc != SMALLW_OK) {
            if (pl) return fail("a rejected problem returned a plan", it);
            ++rejected;
            continue;
        }
        ++accepted;
        size_t need = 0;
        if (small_w_attention_plan_export(pl, nullptr, 0, &need) != SMALLW_EINVAL || need < 4)
            return fail("export into a null buffer was not refused with the size", it);
        std::vector<int32_t> buf(need);
        size_t need2 = 0;
        if (small_w_attention_plan_export(pl, buf.data(), need, &need2) != SMALLW_OK || need2 != need)
            return fail("export into an exact buffer failed", it);
        (void)small_w_attention_workspace_bytes(pl);
        const size_t maxp = small_w_attention_plan_max_unit_pages(pl);
        // [P, Hkv, U, R], S_p x P, unit_off x (P+1), (p, kvh, s, pb, pe) x U
        const int P = buf[0], Hkv = buf[1], U = buf[2];
        if (P != pr.num_reqs || Hkv != pr.num_kv_heads || U < P * Hkv)
            return fail("export header", it);
        const int32_t* Sp = buf.data() + 4;
        const int32_t* uoff = Sp + P;
        const int32_t* units = uoff + (P + 1);
        if (size_t(4 + P + (P + 1) + 5 * int64_t(U)) != need || uoff[P] != U)
            return fail("export size", it);
        // unit u = unit_off[p] + kvh*S_p + s; a (p, kvh) group's ranges are contiguous and end at
        // the request's last page (the first starts at the sliding window's first page)
        for (int p = 0; p < P; ++p) {
            const int S = Sp[p];
            if (S < 1 || uoff[p + 1] - uoff[p] != int64_t(Hkv) * S) return fail("unit offsets", it);
            const int64_t np = (int64_t(seq[p]) + 15) / 16;
            for (int h = 0; h < Hkv; ++h) {
                int64_t prev_pe = -1;
                for (int sp = 0; sp < S; ++sp) {
                    const int32_t* e = units + 5 * (int64_t(uoff[p]) + int64_t(h) * S + sp);
                    if (e[0] != p || e[1] != h || e[2] != sp) return fail("unit order", it);
                    if (e[3] > e[4] || size_t(e[4] - e[3]) > maxp) return fail("unit range", it);
                    if (sp > 0 && e[3] != prev_pe) return fail("units not contiguous", it);
                    prev_pe = e[4];
                }
                if (np > 0 && prev_pe != np) return fail("last unit does not end at the last page", it);
            }
        }
        small_w_attention_plan_destroy(pl);
    }
    std::printf("plan_stress: %d accepted, %d rejected\n", accepted, rejected);
    return 0;
}
