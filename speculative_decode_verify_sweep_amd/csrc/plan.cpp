// Split-K planner: validates a call and decides its work decomposition.
//
// The pages name key splitting with a reduce step ("ChunkedSmallT re-streams
// full KV per query chunk", section Finding) and a capacity function that
// throws past the tile width (section Why no PR yet); they give no formula.
// A call ends with its longest work unit, so this planner hands the splits of
// one round of resident work-unit slots to the requests so that the largest
// pages-per-split is as small as it can be, with at least 8 pages per split so
// the per-split pipeline start and the partial traffic stay small against the
// KV stream:
//   n_p   = ceil(L_p / 16), n_eff = pages streamed (n_p less a window's skip)
//   slots = num_cus * (2 if bf16 pool and D < 256 else 1)   (units resident
//           per CU: a D=256 unit, and every e4m3 or MXFP4 unit, needs one CU's
//           VGPRs; bf16 units of smaller heads fit two)
//   round = max(1, floor(slots / Hkv))         (splits one round of units holds)
//   S_p   = 1 (empty request) | min(force_splits, n_eff) | apportioned:
//           every request starts at 1; while sum S < budget, the request with
//           the largest n_eff / S_p (ties: the lower index) whose next split
//           keeps 8 pages (S_p < floor(n_eff / 8)) gets one more.  budget =
//           round when P <= round (one round, no second), else P + round.
//   unit  u = unit_off[p] + kvh*S_p + s,  pages [floor(s n/S), floor((s+1) n/S))
// Giving each next split to the largest pages-per-split (the D'Hondt
// apportionment) minimises the largest n_eff / S_p for every total: a
// proportional share with floors can leave it up to twice as large.
// Row-exact mode (split_pages = B > 0): S_p = max(1, ceil(n_p / B)), split s covers [s B, min((s+1) B, n_p)),
// and every row goes through the combine, so split boundaries sit at fixed
// page indices whatever W, P or the other lengths are.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "plan_internal.h"

namespace {

constexpr int kMinPagesPerSplit = 8;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Automatic split counts (S starts at 1 for every request): one split at a time
// to the request with the most streamed pages per split, ties to the lower
// index, while the budget lasts and the split keeps kMinPagesPerSplit pages.
void apportion(const std::vector<int64_t>& ne, int64_t budget, std::vector<int64_t>& S) {
    const int P = int(ne.size());
    auto cap = [&](int p) { return std::max<int64_t>(1, ne[p] / kMinPagesPerSplit); };
    // heap order: a below b when ne[a]/S[a] < ne[b]/S[b], or equal and a > b
    auto below = [&](int a, int b) {
        const int64_t l = ne[a] * S[b], r = ne[b] * S[a];
        return l != r ? l < r : a > b;
    };
    std::vector<int> heap;
    for (int p = 0; p < P; ++p)
        if (ne[p] > 0 && S[p] < cap(p)) heap.push_back(p);
    std::make_heap(heap.begin(), heap.end(), below);
    for (int64_t used = P; used < budget && !heap.empty(); ++used) {
        std::pop_heap(heap.begin(), heap.end(), below);
        const int p = heap.back();
        heap.pop_back();
        if (++S[p] < cap(p)) {
            heap.push_back(p);
            std::push_heap(heap.begin(), heap.end(), below);
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int validate(const smallw_problem& pr, const int32_t* seq) {
    if (pr.num_reqs < 1 || pr.window < 1 || pr.num_q_heads < 1 || pr.num_kv_heads < 1 ||
        pr.head_dim < 1 || pr.page_size < 1 || pr.num_pages < 1 || pr.max_pages_per_req < 1 ||
        pr.num_cus < 0 || pr.force_splits < 0 || pr.split_pages < 0 || pr.window_left < 0)
        return SMALLW_EINVAL;
    if (pr.v_layout != SMALLW_V_DMAJOR && pr.v_layout != SMALLW_V_TOKEN_MAJOR) return SMALLW_EINVAL;
    if (pr.force_splits > 0 && pr.split_pages > 0) return SMALLW_EINVAL;
    if (pr.causal != 0 && pr.causal != 1) return SMALLW_EINVAL;
    if (pr.kv_dtype != SMALLW_KV_BF16 && pr.kv_dtype != SMALLW_KV_FP8_E4M3 &&
        pr.kv_dtype != SMALLW_KV_MXFP4)
        return SMALLW_EINVAL;
    if (std::isnan(pr.scale) || std::isinf(pr.scale)) return SMALLW_EINVAL;
    if (pr.num_q_heads % pr.num_kv_heads != 0) return SMALLW_EINVAL;
    if (pr.num_reqs > SMALLW_MAX_REQS) return SMALLW_EUNSUPPORTED;
    if (pr.window > SMALLW_MAX_WINDOW) return SMALLW_EUNSUPPORTED;
    if (pr.page_size != SMALLW_PAGE_SIZE) return SMALLW_EUNSUPPORTED;
    if (pr.head_dim != 64 && pr.head_dim != 128 && pr.head_dim != 256) return SMALLW_EUNSUPPORTED;
    if (pr.kv_dtype == SMALLW_KV_MXFP4 && pr.head_dim == 64) return SMALLW_EUNSUPPORTED;
    if (pr.v_layout == SMALLW_V_TOKEN_MAJOR && pr.kv_dtype != SMALLW_KV_BF16)
        return SMALLW_EUNSUPPORTED;
    const int64_t rows = int64_t(pr.window) * (pr.num_q_heads / pr.num_kv_heads);
    if (rows > SMALLW_MAX_ROWS) return SMALLW_EUNSUPPORTED;
    if (!seq) return SMALLW_EINVAL;
    const int64_t cap = int64_t(pr.max_pages_per_req) * SMALLW_PAGE_SIZE;
    for (int p = 0; p < pr.num_reqs; ++p) {
        if (seq[p] < 0 || seq[p] > cap) return SMALLW_EINVAL;
        if (pr.causal && seq[p] > 0 && seq[p] < pr.window) return SMALLW_EINVAL;
    }
    return SMALLW_OK;
}

}  // namespace

namespace smallw {

int build_plan(const smallw_problem& in, const int32_t* seq, smallw_plan** out) {
    int rc = validate(in, seq);
    if (rc != SMALLW_OK) return rc;
    smallw_plan* pl = new (std::nothrow) smallw_plan();
    if (!pl) return SMALLW_ENOMEM;
    try {
        pl->prob = in;
        if (!(pl->prob.scale > 0.f)) pl->prob.scale = 1.0f / std::sqrt(float(in.head_dim));
        const int P = in.num_reqs, Hkv = in.num_kv_heads, D = in.head_dim;
        pl->G = in.num_q_heads / Hkv;
        pl->R = in.window * pl->G;
        pl->seq.assign(seq, seq + P);
        pl->npg.resize(P);
        pl->nlo.resize(P);
        std::vector<int64_t> ne(P), Sv(P, 1);
        for (int p = 0; p < P; ++p) {
            pl->npg[p] = int32_t(ceil_div(seq[p], SMALLW_PAGE_SIZE));
            pl->nlo[p] = int32_t(smallw::first_page(seq[p], in.window, in.causal, in.window_left));
            const int64_t n = pl->npg[p], lo = pl->nlo[p];
            ne[p] = n - lo;
            if (n == 0) Sv[p] = 1;
            else if (in.split_pages > 0) Sv[p] = ceil_div(n, in.split_pages) - lo / in.split_pages;
            else if (in.force_splits > 0) Sv[p] = std::min<int64_t>(in.force_splits, ne[p]);
        }
        if (in.split_pages == 0 && in.force_splits == 0) {
            const int64_t slots =
                int64_t(in.num_cus) * (D < 256 && in.kv_dtype == SMALLW_KV_BF16 ? 2 : 1);
            const int64_t round = std::max<int64_t>(1, slots / Hkv);
            apportion(ne, P <= round ? round : P + round, Sv);
        }
        pl->splits.resize(P);
        pl->unit_off.assign(P + 1, 0);
        for (int p = 0; p < P; ++p) {
            const int64_t n = pl->npg[p], lo = pl->nlo[p], S = Sv[p];
            pl->splits[p] = int32_t(S);
            if (S > 1) pl->any_split = true;
            const int64_t next = int64_t(pl->unit_off[p]) + Hkv * S;
            if (next > INT32_MAX / 2) { delete pl; return SMALLW_EUNSUPPORTED; }
            pl->unit_off[p + 1] = int32_t(next);
            for (int64_t s = 0; s < S; ++s) {
                int64_t pb, pe;
                smallw::split_range(lo, n, S, s, in.split_pages, smallw::piece_align(in.kv_dtype), &pb,
                                    &pe);
                if (size_t(pe - pb) > pl->max_unit_pages) pl->max_unit_pages = size_t(pe - pb);
            }
        }
        pl->U = pl->unit_off[P];
        pl->combine = pl->any_split || in.split_pages > 0;
        if (pl->combine) {
            // fp16 partials (16-row tiles, the last one padded), then one
            // {lse, scale} float pair per (unit, row)
            const size_t po = size_t(pl->U) * ((pl->R + 15) / 16 * 16) * D * 2;
            const size_t prec = size_t(pl->U) * pl->R * 2 * sizeof(float);
            pl->part_o_off = 0;
            pl->part_rec_off = align256(po);
            pl->ws_bytes = pl->part_rec_off + align256(prec);
        }
    } catch (...) {
        delete pl;
        return SMALLW_ENOMEM;
    }
    *out = pl;
    return SMALLW_OK;
}

}  // namespace smallw

extern "C" {

size_t small_w_attention_workspace_bytes(const smallw_plan* plan) {
    return plan ? plan->ws_bytes : 0;
}

size_t small_w_attention_plan_max_unit_pages(const smallw_plan* plan) {
    return plan ? plan->max_unit_pages : 0;
}

int small_w_attention_plan_export(const smallw_plan* plan, int32_t* buf, size_t cap,
                                  size_t* needed) {
    if (!plan) return SMALLW_EINVAL;
    const int P = plan->prob.num_reqs, Hkv = plan->prob.num_kv_heads;
    const size_t n = 4 + size_t(P) + size_t(P + 1) + 5 * size_t(plan->U);
    if (needed) *needed = n;
    if (!buf || cap < n) return SMALLW_EINVAL;
    size_t k = 0;
    buf[k++] = P;
    buf[k++] = Hkv;
    buf[k++] = plan->U;
    buf[k++] = plan->R;
    for (int p = 0; p < P; ++p) buf[k++] = plan->splits[p];
    for (int p = 0; p <= P; ++p) buf[k++] = plan->unit_off[p];
    for (int p = 0; p < P; ++p) {
        const int64_t npg = plan->npg[p], lo = plan->nlo[p], S = plan->splits[p];
        for (int kvh = 0; kvh < Hkv; ++kvh)
            for (int64_t s = 0; s < S; ++s) {
                int64_t pb, pe;
                smallw::split_range(lo, npg, S, s, plan->prob.split_pages,
                                    smallw::piece_align(plan->prob.kv_dtype), &pb, &pe);
                buf[k++] = p;
                buf[k++] = kvh;
                buf[k++] = int32_t(s);
                buf[k++] = int32_t(pb);
                buf[k++] = int32_t(pe);
            }
    }
    return SMALLW_OK;
}

void small_w_attention_plan_destroy(smallw_plan* plan) { delete plan; }

}  // extern "C"
