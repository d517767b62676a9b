/* A plain C99 program that runs whole steps of the data-parallel update on
 * the GPU through libdpstep.so alone: its own hipMalloc'd buffers, its own
 * stream, no torch.  The inputs come from files written by the test:
 *
 *   config.txt  P T n a steps grad_dtype param_dtype max_norm lr eps wd beta1
 *               beta2, then the T tensor sizes, then a shard cut c (the
 *               update runs as [0, c) and [c, P))
 *   master.bin  binary32 [P], the initial master weights
 *   grads.bin   16-bit [steps][a][n][P], the gradient of every micro-step
 *
 * and the outputs go to state.bin (binary32 master, m, v [P] each, then the
 * 16-bit params [P]) and scalars.txt (t iter growth_tracker found_inf, then
 * beta1^t, beta2^t, scale, norm, clip as C99 hex floats).  argv[1] is the directory of
 * these files.  With argv[2] = "buckets", every micro-step and the reduction
 * run in two buckets split at the last tensor start at or before the cut, the
 * later bucket first (dp_accumulate_all_range, dp_accumulate_reduce_range).
 * Exit status 0 on success; a failing call prints its status and
 * dp_last_error(). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dpstep.h"

#define CALL(x)                                                                        \
    do {                                                                               \
        dp_status s_ = (x);                                                            \
        if (s_ != DP_OK) {                                                             \
            printf("%s failed: %s: %s\n", #x, dp_status_string(s_), dp_last_error()); \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

#define HIPCALL(x)                                                          \
    do {                                                                    \
        hipError_t e_ = (x);                                                \
        if (e_ != hipSuccess) {                                             \
            printf("%s failed: %s\n", #x, hipGetErrorString(e_));           \
            return 1;                                                       \
        }                                                                   \
    } while (0)

static char path_buf[4096];

static const char* path(const char* dir, const char* name) {
    snprintf(path_buf, sizeof(path_buf), "%s/%s", dir, name);
    return path_buf;
}

static int read_file(const char* p, void* dst, size_t bytes) {
    FILE* f = fopen(p, "rb");
    if (!f) return 1;
    const size_t got = fread(dst, 1, bytes, f);
    fclose(f);
    return got == bytes ? 0 : 1;
}

int main(int argc, char** argv) {
    if (argc < 2) return 2;
    const char* dir = argv[1];
    FILE* cf = fopen(path(dir, "config.txt"), "r");
    if (!cf) return 2;
    long long P, T, n, a, steps, cut;
    int gdt, pdt;
    double max_norm, lr, eps, wd, b1, b2;
    if (fscanf(cf, "%lld %lld %lld %lld %lld %d %d %lf %lf %lf %lf %lf %lf", &P, &T, &n, &a, &steps, &gdt, &pdt,
               &max_norm, &lr, &eps, &wd, &b1, &b2) != 13 || T < 0 || T > 4096 || n < 1 || n > DP_MAX_REPLICAS ||
        a < 1 || steps < 1 || P < 0) {
        fclose(cf);
        return 2;
    }
    int64_t* numel = (int64_t*)calloc((size_t)(T > 0 ? T : 1), sizeof(int64_t));
    long long sum = 0;
    for (long long i = 0; i < T; ++i) {
        long long x;
        if (fscanf(cf, "%lld", &x) != 1 || x < 0) return 2;
        numel[i] = x;
        sum += x;
    }
    if (fscanf(cf, "%lld", &cut) != 1 || sum != P || cut < 0 || cut > P) return 2;
    fclose(cf);
    const int buckets = argc > 2 && strcmp(argv[2], "buckets") == 0;
    long long bcut = 0;  /* the last tensor start at or before the cut */
    for (long long i = 0, at = 0; i < T; at += numel[i], ++i)
        if (at <= cut) bcut = at;

    const size_t np = (size_t)P;
    float* master = (float*)malloc(np * 4 + 4);
    uint16_t* grads = (uint16_t*)malloc((size_t)(steps * a * n) * np * 2 + 2);
    if (!master || !grads) return 3;
    if (read_file(path(dir, "master.bin"), master, np * 4) ||
        read_file(path(dir, "grads.bin"), grads, (size_t)(steps * a * n) * np * 2)) {
        printf("cannot read the inputs\n");
        return 2;
    }

    dp_layout L;
    memset(&L, 0, sizeof(L));
    L.num_tensors = (int32_t)T;
    L.n_replicas = (int32_t)n;
    L.numel = numel;
    L.grad_dtype = (dp_dtype)gdt;
    L.param_dtype = (dp_dtype)pdt;
    dp_plan* plan = NULL;
    CALL(dp_plan_create(&L, &plan));

    /* device memory: state, params, accumulators (one allocation), g_bar, and
     * every micro-step's gradients (the inputs, copied up once) */
    float *w_d, *m_d, *v_d, *acc_d, *gbar_d;
    uint16_t *p_d, *g_d;
    HIPCALL(hipMalloc((void**)&w_d, np * 4 + 4));
    HIPCALL(hipMalloc((void**)&m_d, np * 4 + 4));
    HIPCALL(hipMalloc((void**)&v_d, np * 4 + 4));
    HIPCALL(hipMalloc((void**)&p_d, np * 2 + 2));
    HIPCALL(hipMalloc((void**)&acc_d, (size_t)n * np * 4 + 4));
    HIPCALL(hipMalloc((void**)&gbar_d, np * 4 + 4));
    HIPCALL(hipMalloc((void**)&g_d, (size_t)(steps * a * n) * np * 2 + 2));
    HIPCALL(hipMemcpy(w_d, master, np * 4, hipMemcpyHostToDevice));
    HIPCALL(hipMemset(m_d, 0, np * 4));
    HIPCALL(hipMemset(v_d, 0, np * 4));
    HIPCALL(hipMemset(p_d, 0, np * 2));
    HIPCALL(hipMemcpy(g_d, grads, (size_t)(steps * a * n) * np * 2, hipMemcpyHostToDevice));
    hipStream_t s;
    HIPCALL(hipStreamCreate(&s));

    CALL(dp_plan_bind_flat(plan, DP_ROLE_MASTER, 0, w_d));
    CALL(dp_plan_bind_flat(plan, DP_ROLE_EXP_AVG, 0, m_d));
    CALL(dp_plan_bind_flat(plan, DP_ROLE_EXP_AVG_SQ, 0, v_d));
    CALL(dp_plan_bind_flat(plan, DP_ROLE_PARAM, 0, p_d));
    for (long long r = 0; r < n; ++r) CALL(dp_plan_bind_flat(plan, DP_ROLE_ACC, (int32_t)r, acc_d + r * P));
    if (n > 1) CALL(dp_plan_bind_flat(plan, DP_ROLE_GBAR, 0, gbar_d));
    CALL(dp_plan_prepare_range(plan, 0, cut));
    CALL(dp_plan_prepare_range(plan, cut, P));

    dp_state_cfg cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.beta1 = b1;
    cfg.beta2 = b2;
    cfg.scaler_mode = DP_SCALER_NONE;
    CALL(dp_state_init(plan, &cfg, s));
    const dp_adam_hparams hp = {lr, eps, wd};

    for (long long st = 0; st < steps; ++st) {
        for (long long k = 0; k < a; ++k) {
            for (long long r = 0; r < n; ++r)
                CALL(dp_plan_bind_flat(plan, DP_ROLE_GRAD, (int32_t)r, g_d + ((st * a + k) * n + r) * P));
            if (buckets && k + 1 < a) {
                CALL(dp_accumulate_all_range(plan, k == 0, bcut, P, s));
                CALL(dp_accumulate_all_range(plan, k == 0, 0, bcut, s));
            } else if (buckets) {
                CALL(dp_accumulate_reduce_range(plan, bcut, P, s));
                CALL(dp_accumulate_reduce_range(plan, 0, bcut, s));
            } else if (k + 1 < a) {
                CALL(dp_accumulate_all(plan, k == 0, s));
            } else {
                CALL(dp_accumulate_reduce(plan, s));
            }
        }
        CALL(dp_grad_stats(plan, 0, max_norm, s));
        CALL(dp_adam_step(plan, &hp, cut, P, s));  /* the shards in either order */
        CALL(dp_adam_step(plan, &hp, 0, cut, s));
    }
    dp_step_state out;
    CALL(dp_read_state(plan, &out, s));

    float* back = (float*)malloc(np * 12 + 4);
    uint16_t* pb = (uint16_t*)malloc(np * 2 + 2);
    if (!back || !pb) return 3;
    HIPCALL(hipMemcpy(back, w_d, np * 4, hipMemcpyDeviceToHost));
    HIPCALL(hipMemcpy(back + np, m_d, np * 4, hipMemcpyDeviceToHost));
    HIPCALL(hipMemcpy(back + 2 * np, v_d, np * 4, hipMemcpyDeviceToHost));
    HIPCALL(hipMemcpy(pb, p_d, np * 2, hipMemcpyDeviceToHost));
    FILE* of = fopen(path(dir, "state.bin"), "wb");
    if (!of || fwrite(back, 4, np * 3, of) != np * 3 || fwrite(pb, 2, np, of) != np) return 4;
    fclose(of);
    FILE* sf = fopen(path(dir, "scalars.txt"), "w");
    if (!sf) return 4;
    fprintf(sf, "%lld %lld %lld %d %a %a %a %a %a\n", (long long)out.t, (long long)out.iter,
            (long long)out.growth_tracker, out.found_inf, out.beta1_pow, out.beta2_pow, out.scale, out.norm, out.clip);
    fclose(sf);

    CALL(dp_plan_destroy(plan));
    HIPCALL(hipStreamDestroy(s));
    hipFree(w_d);
    hipFree(m_d);
    hipFree(v_d);
    hipFree(p_d);
    hipFree(acc_d);
    hipFree(gbar_d);
    hipFree(g_d);
    free(master);
    free(grads);
    free(back);
    free(pb);
    free(numel);
    printf("ok\n");
    return 0;
}
