/* Seeded corruption of a committed checkpoint, read back through the host
 * layer of libdpstep (dpckpt.h).  A checkpoint of three shards is written and
 * committed; then, iteration by iteration, one file (the manifest or a shard)
 * is damaged (bytes flipped, a range zeroed, or the file cut short), a random
 * range is read, and the file is put back.  Every read must return a status
 * and never crash; a read that returns DP_OK must return exactly the data
 * and scalars that were written (damage it did not detect must lie where the
 * read does not look).  Built with a sanitizer, this also checks the parsers
 * for out-of-bounds accesses.
 *
 * Usage: ckpt_fuzz DIR ITERATIONS SEED.  Prints "ok <reads> <detected>" and
 * exits 0, or names the failing iteration and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dpckpt.h"

static uint64_t rng_state;

static uint64_t next_u64(void) { /* xorshift64* (Vigna) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

static uint64_t below(uint64_t n) { return n ? next_u64() % n : 0; }

static unsigned char* slurp(const char* path, size_t* size) {
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    fseek(f, 0, SEEK_END);
    const long n = ftell(f);
    fseek(f, 0, SEEK_SET);
    unsigned char* b = (unsigned char*)malloc((size_t)n + 1);
    if (b && fread(b, 1, (size_t)n, f) != (size_t)n) {
        free(b);
        b = NULL;
    }
    fclose(f);
    *size = (size_t)n;
    return b;
}

static int spill(const char* path, const unsigned char* b, size_t n) {
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    const int bad = fwrite(b, 1, n, f) != n;
    fclose(f);
    return bad;
}

enum { T = 3, P = 5000 + 3 + 70001, NFILES = 4 };

int main(int argc, char** argv) {
    if (argc < 4) return 2;
    const char* dir = argv[1];
    const long iters = atol(argv[2]);
    rng_state = (uint64_t)atoll(argv[3]) * 0x9E3779B97F4A7C15ull + 1;

    const int64_t numel[T] = {5000, 3, 70001};
    dp_layout L;
    memset(&L, 0, sizeof(L));
    L.num_tensors = T;
    L.n_replicas = 1;
    L.numel = numel;
    L.grad_dtype = DP_BF16;
    L.param_dtype = DP_F16;

    static float w[P], m[P], v[P];
    static uint16_t p[P];
    for (int i = 0; i < P; ++i) {
        w[i] = (float)(i % 977) * 0.25f - 7.0f;
        m[i] = (float)(i % 31) * 1e-3f;
        v[i] = (float)(i % 13) * 1e-6f;
        p[i] = (uint16_t)(i * 2654435761u >> 16);
    }
    const int64_t cuts[4] = {0, 4097, 40000, P};
    for (int s = 0; s < 3; ++s)
        if (dp_ckpt_write_shard(dir, 7, &L, cuts[s], cuts[s + 1], w + cuts[s], m + cuts[s], v + cuts[s],
                                p + cuts[s]) != DP_OK) {
            printf("write failed: %s\n", dp_last_error());
            return 1;
        }
    dp_step_state st;
    memset(&st, 0, sizeof(st));
    st.t = 12;
    st.iter = 13;
    st.scale = 32768.0;
    st.beta1_pow = 0.28242953648100017;
    dp_state_cfg cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.beta1 = 0.9;
    cfg.beta2 = 0.999;
    cfg.scaler_mode = 2;
    cfg.growth_interval = 2000;
    if (dp_ckpt_commit(dir, 7, &L, &st, &cfg) != DP_OK) {
        printf("commit failed: %s\n", dp_last_error());
        return 1;
    }

    char paths[NFILES][512];
    snprintf(paths[0], sizeof(paths[0]), "%s/manifest.dpck", dir);
    for (int s = 0; s < 3; ++s)
        snprintf(paths[s + 1], sizeof(paths[s + 1]), "%s/g7-%lld-%lld.dpshard", dir, (long long)cuts[s],
                 (long long)cuts[s + 1]);
    unsigned char* orig[NFILES];
    size_t size[NFILES];
    for (int f = 0; f < NFILES; ++f) {
        orig[f] = slurp(paths[f], &size[f]);
        if (!orig[f]) {
            printf("cannot read %s\n", paths[f]);
            return 1;
        }
    }

    static float rw[P], rm[P], rv[P];
    static uint16_t rp[P];
    size_t largest = 0;
    for (int f = 0; f < NFILES; ++f) largest = size[f] > largest ? size[f] : largest;
    unsigned char* work = (unsigned char*)malloc(largest + 1);
    if (!work) return 1;
    long reads = 0, detected = 0;
    for (long it = 0; it < iters; ++it) {
        const int f = (int)below(NFILES);
        size_t n = size[f];
        memcpy(work, orig[f], n);
        const int kind = (int)below(4);
        if (kind == 0) { /* flip 1..8 bytes */
            const int k = 1 + (int)below(8);
            for (int j = 0; j < k; ++j) work[below(n)] ^= (unsigned char)(1 + below(255));
        } else if (kind == 1) { /* zero a range */
            const size_t a = below(n), len = 1 + below(4096);
            memset(work + a, 0, a + len > n ? n - a : len);
        } else if (kind == 2) { /* cut short */
            n = below(n);
        } else { /* flip one bit in the first 512 bytes (headers, manifest fields) */
            work[below(n < 512 ? n : 512)] ^= (unsigned char)(1u << below(8));
        }
        if (spill(paths[f], work, n)) return 1;
        int64_t b = (int64_t)below(P + 1), e = (int64_t)below(P + 1);
        if (b > e) {
            const int64_t x = b;
            b = e;
            e = x;
        }
        dp_step_state rs;
        dp_state_cfg rc;
        int64_t gen = -1;
        const dp_status s = dp_ckpt_read(dir, &L, b, e, rw, rm, rv, rp, &rs, &rc, &gen);
        ++reads;
        if (s == DP_OK) {
            const size_t cnt = (size_t)(e - b);
            if (gen != 7 || rs.t != st.t || rs.iter != st.iter || rs.scale != st.scale ||
                rs.beta1_pow != st.beta1_pow || rc.beta2 != cfg.beta2 || rc.growth_interval != cfg.growth_interval ||
                memcmp(rw, w + b, cnt * 4) || memcmp(rm, m + b, cnt * 4) || memcmp(rv, v + b, cnt * 4) ||
                memcmp(rp, p + b, cnt * 2)) {
                printf("iteration %ld: file %d, damage %d, range [%lld, %lld): DP_OK with wrong data\n", it, f, kind,
                       (long long)b, (long long)e);
                return 1;
            }
        } else if (s == DP_ERR_CORRUPT || s == DP_ERR_STATE || s == DP_ERR_BAD_LAYOUT || s == DP_ERR_IO) {
            ++detected;
        } else {
            printf("iteration %ld: unexpected status %d: %s\n", it, (int)s, dp_last_error());
            return 1;
        }
        if (spill(paths[f], orig[f], size[f])) return 1;
    }
    /* the intact checkpoint still reads in full */
    if (dp_ckpt_read(dir, &L, 0, P, rw, rm, rv, rp, NULL, NULL, NULL) != DP_OK || memcmp(rw, w, sizeof(w))) {
        printf("the restored checkpoint does not read back\n");
        return 1;
    }
    for (int f = 0; f < NFILES; ++f) free(orig[f]);
    free(work);
    printf("ok %ld %ld\n", reads, detected);
    return 0;
}
