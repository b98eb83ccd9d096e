/* A C caller of include/smallw.h, host calls only (no GPU needed): plan a
 * 64K-key verify call, read its workspace size and integer export, check the
 * documented status codes of bad problems and null arguments, and release the
 * plan.  Built as C11 with every warning an error, so the header stays usable
 * from C.  Prints "ok" and exits 0 when every check holds. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "smallw.h"

#define CHECK(cond)                                                    \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                                  \
        }                                                              \
    } while (0)

static smallw_problem verify_64k(void) {
    smallw_problem pr;
    memset(&pr, 0, sizeof pr);
    pr.num_reqs = 1;
    pr.window = 16;
    pr.num_q_heads = 24;
    pr.num_kv_heads = 4;
    pr.head_dim = 256;
    pr.page_size = SMALLW_PAGE_SIZE;
    pr.num_pages = 5000;
    pr.max_pages_per_req = 4097;
    pr.causal = 1;
    pr.kv_dtype = SMALLW_KV_BF16;
    pr.scale = 0.0f; /* 1/sqrt(D) */
    pr.num_cus = 256;
    pr.v_layout = SMALLW_V_DMAJOR;
    return pr;
}

int main(void) {
    const int32_t len = 65536 + 16;
    smallw_problem pr = verify_64k();
    smallw_plan* plan = NULL;
    CHECK(small_w_attention_plan(&pr, &len, &plan) == SMALLW_OK && plan != NULL);

    /* 256 units for 256 compute units: 64 splits of each of the 4 KV heads */
    size_t needed = 0;
    CHECK(small_w_attention_plan_export(plan, NULL, 0, &needed) == SMALLW_EINVAL);
    CHECK(needed == 4 + 1 + 2 + 5 * 256);
    int32_t* buf = (int32_t*)malloc(needed * sizeof(int32_t));
    CHECK(buf != NULL);
    CHECK(small_w_attention_plan_export(plan, buf, needed, &needed) == SMALLW_OK);
    CHECK(buf[0] == 1 && buf[1] == 4 && buf[2] == 256 && buf[3] == 16 * 6);
    CHECK(buf[4] == 64 && buf[5] == 0 && buf[6] == 256);
    /* units tile the 4097 pages of every head in order, without gaps */
    int32_t next = 0;
    for (int u = 0; u < 256; ++u) {
        const int32_t* e = buf + 7 + 5 * u;
        CHECK(e[0] == 0 && e[1] == u / 64 && e[2] == u % 64);
        if (e[2] == 0) next = 0;
        CHECK(e[3] == next && e[4] > e[3]);
        next = e[4];
        if (e[2] == 63) CHECK(e[4] == 4097);
    }
    free(buf);
    CHECK(small_w_attention_workspace_bytes(plan) > 0);
    CHECK(small_w_attention_plan_max_unit_pages(plan) == 65);

    /* status codes: unsupported shapes, malformed problems, null arguments */
    smallw_plan* none = NULL;
    smallw_problem bad = verify_64k();
    bad.window = SMALLW_MAX_WINDOW + 1;
    CHECK(small_w_attention_plan(&bad, &len, &none) == SMALLW_EUNSUPPORTED && none == NULL);
    bad = verify_64k();
    bad.head_dim = 96;
    CHECK(small_w_attention_plan(&bad, &len, &none) == SMALLW_EUNSUPPORTED && none == NULL);
    bad = verify_64k();
    bad.num_q_heads = 25;
    CHECK(small_w_attention_plan(&bad, &len, &none) == SMALLW_EINVAL && none == NULL);
    const int32_t too_long = 16 * 4097 + 1;
    CHECK(small_w_attention_plan(&pr, &too_long, &none) == SMALLW_EINVAL && none == NULL);
    CHECK(small_w_attention_plan(&pr, NULL, &none) == SMALLW_EINVAL);
    CHECK(small_w_attention_run(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                NULL, 0, NULL) == SMALLW_EINVAL);
    CHECK(small_w_attention_check_pages(plan, NULL, NULL, NULL, NULL) == SMALLW_EINVAL);
    CHECK(strcmp(small_w_attention_strerror(SMALLW_OK), "ok") == 0);
    CHECK(small_w_attention_strerror(SMALLW_EWORKSPACE)[0] != '\0');

    small_w_attention_plan_destroy(plan);
    small_w_attention_plan_destroy(NULL);
    printf("ok\n");
    return 0;
}
