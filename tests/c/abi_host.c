/* A plain C99 client of libdpstep.so: it includes both headers as C and calls
 * the entry points that need no GPU (plan creation and its checks, the chunk
 * table, flat bindings, status strings, and the checkpoint host layer).  It
 * prints "ok" and exits 0 when every check holds, else names the failing
 * check and exits 1.  argv[1] is an empty directory for the checkpoint. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dpckpt.h"
#include "dpstep.h"

static int failures = 0;

#define CHECK(cond)                                                  \
    do {                                                             \
        if (!(cond)) {                                               \
            printf("FAILED line %d: %s (last error: %s)\n", __LINE__, \
                   #cond, dp_last_error());                          \
            ++failures;                                              \
        }                                                            \
    } while (0)

int main(int argc, char** argv) {
    if (argc < 2) return 2;
    const char* dir = argv[1];

    CHECK(dp_abi_version() == DP_ABI_VERSION);
    CHECK(strcmp(dp_status_string(DP_ERR_CORRUPT), "checkpoint corrupt") == 0);

    /* a ragged layout: 1000 | 0 | 20000 | 3 elements */
    const int64_t numel[4] = {1000, 0, 20000, 3};
    dp_layout L;
    memset(&L, 0, sizeof(L));
    L.num_tensors = 4;
    L.n_replicas = 3;
    L.numel = numel;
    L.grad_dtype = DP_BF16;
    L.param_dtype = DP_F16;
    L.chunk_elems = 4096;

    dp_plan* plan = NULL;
    CHECK(dp_plan_create(&L, &plan) == DP_OK && plan != NULL);

    dp_plan_info info;
    CHECK(dp_plan_info_get(plan, &info) == DP_OK);
    CHECK(info.params == 21003 && info.num_tensors == 4 && info.n_replicas == 3 && info.chunk_elems == 4096);
    /* tensor 0: 1 chunk; tensor 2: ceil(20000 / 4096) = 5 chunks; tensor 3: 1 */
    CHECK(info.num_chunks == 7);
    CHECK(info.bytes_adam == 21003.0 * 30.0);

    /* the chunk table of a range that starts inside tensor 2 */
    dp_chunk ch[8];
    int64_t count = -1;
    CHECK(dp_plan_chunks(plan, 5000, 21003, 0, 8, ch, &count) == DP_OK);
    /* tensor 2 is cut at multiples of 4096 counted from its own start:
     * offsets [4000, 4096), [4096, 8192), ..., [16384, 20000); then tensor 3 */
    CHECK(count == 6);
    if (count == 6) {
        CHECK(ch[0].flat == 5000 && ch[0].offset == 4000 && ch[0].tensor == 2 && ch[0].len == 96);
        CHECK(ch[1].offset == 4096 && ch[1].len == 4096);
        CHECK(ch[4].flat == 1000 + 16384 && ch[4].len == 20000 - 16384);
        CHECK(ch[5].flat == 21000 && ch[5].offset == 0 && ch[5].tensor == 3 && ch[5].len == 3);
    }
    CHECK(dp_plan_chunks(plan, 0, 21004, 0, 0, NULL, &count) == DP_ERR_RANGE);

    /* binding checks are host work */
    static float fake[1];
    CHECK(dp_plan_bind_flat(plan, DP_ROLE_MASTER, 1, fake) == DP_OK);
    CHECK(dp_plan_bind_flat(plan, DP_ROLE_MASTER, 2, fake) == DP_ERR_INVALID_ARG);
    CHECK(dp_plan_bind_flat(plan, DP_ROLE_ACC, 3, fake) == DP_ERR_INVALID_ARG);
    CHECK(dp_plan_bind_flat(plan, (dp_role)7, 0, fake) == DP_ERR_INVALID_ARG);
    /* order checks fail before any GPU work */
    dp_adam_hparams hp = {1e-3, 1e-8, 0.01};
    CHECK(dp_adam_step(plan, &hp, 0, 21003, NULL) == DP_ERR_STATE);
    CHECK(dp_adam_step(plan, &hp, 0, 21004, NULL) == DP_ERR_RANGE);
    /* the bucket calls fail validation before any GPU work */
    CHECK(dp_accumulate_all_range(plan, 1, 0, 256, NULL) == DP_ERR_UNBOUND);
    CHECK(dp_accumulate_all_range(NULL, 1, 0, 256, NULL) == DP_ERR_INVALID_ARG);
    CHECK(dp_reduce_replicas_range(plan, DP_ROLE_MASTER, 0, 256, NULL) == DP_ERR_INVALID_ARG);
    CHECK(dp_reduce_replicas_range(plan, DP_ROLE_ACC, 0, 256, NULL) == DP_ERR_STATE); /* before dp_state_init */
    CHECK(dp_plan_drop_ranges(plan) == DP_OK); /* nothing cached: no GPU work */
    CHECK(dp_plan_drop_ranges(NULL) == DP_ERR_INVALID_ARG);
    CHECK(dp_plan_destroy(plan) == DP_OK);

    /* rejected layouts */
    L.n_replicas = 0;
    CHECK(dp_plan_create(&L, &plan) == DP_ERR_BAD_LAYOUT);
    L.n_replicas = 3;
    L.chunk_elems = 768;
    CHECK(dp_plan_create(&L, &plan) == DP_ERR_BAD_LAYOUT);
    L.chunk_elems = 4096;

    /* checkpoint host layer: two shards written, read back across them */
    enum { P = 21003, CUT = 7777 };
    static float w[P], m[P], v[P];
    static uint16_t p[P];
    for (int i = 0; i < P; ++i) {
        w[i] = (float)i * 0.5f;
        m[i] = -(float)i;
        v[i] = (float)i * (float)i;
        p[i] = (uint16_t)(i * 7);
    }
    CHECK(dp_ckpt_write_shard(dir, 3, &L, 0, CUT, w, m, v, p) == DP_OK);
    CHECK(dp_ckpt_write_shard(dir, 3, &L, CUT, P, w + CUT, m + CUT, v + CUT, p + CUT) == DP_OK);
    dp_step_state st;
    memset(&st, 0, sizeof(st));
    st.t = 41;
    st.iter = 42;
    st.scale = 1024.0;
    dp_state_cfg cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.beta1 = 0.9;
    cfg.beta2 = 0.999;
    CHECK(dp_ckpt_commit(dir, 3, &L, &st, &cfg) == DP_OK);

    static float rw[P], rm[P], rv[P];
    static uint16_t rp[P];
    dp_step_state rs;
    dp_state_cfg rc;
    int64_t gen = -1;
    CHECK(dp_ckpt_read(dir, &L, 100, 20000, rw, rm, rv, rp, &rs, &rc, &gen) == DP_OK);
    CHECK(gen == 3 && rs.t == 41 && rs.iter == 42 && rs.scale == 1024.0 && rc.beta2 == 0.999);
    CHECK(memcmp(rw, w + 100, (20000 - 100) * sizeof(float)) == 0);
    CHECK(memcmp(rm, m + 100, (20000 - 100) * sizeof(float)) == 0);
    CHECK(memcmp(rv, v + 100, (20000 - 100) * sizeof(float)) == 0);
    CHECK(memcmp(rp, p + 100, (20000 - 100) * sizeof(uint16_t)) == 0);

    /* another tensor list is refused */
    const int64_t other[4] = {1000, 1, 20000, 2};
    L.numel = other;
    CHECK(dp_ckpt_read(dir, &L, 0, 10, rw, NULL, NULL, NULL, NULL, NULL, NULL) == DP_ERR_BAD_LAYOUT);

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
