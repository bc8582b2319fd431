/* A plain C99 caller of the library's C ABI (host-only calls): the header
 * compiles as C, the declared functions link, and the host paths answer as
 * documented.  Built and run by tests/test_abi_c.py; prints "ok" on success. */
#include <stdio.h>
#include <string.h>

#include "ada.h"

#define CHECK(c)                                                \
    do {                                                        \
        if (!(c)) {                                             \
            fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                           \
        }                                                       \
    } while (0)

int main(void) {
    ada_config_t cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.head_dim = 128;
    cfg.page_size = 16;
    cfg.num_q_heads = 32;
    cfg.num_kv_heads = 8;
    cfg.pair_layout = ADA_PAIRS_ADJACENT;

    ada_cache_t cache;
    memset(&cache, 0, sizeof cache);
    cache.num_seqs = 8;
    cache.max_pages_per_head = 1600;
    cache.page_capacity = 100000;
    cache.arena_capacity16 = 1 << 24;

    /* sizes and strings */
    CHECK(ada_block_bytes(ADA_TIER_T8, 16) == 16 * (130 + 256));
    CHECK(ada_block_bytes(ADA_TIER_T4, 16) == 16 * (66 + 256));
    CHECK(ada_block_bytes(ADA_TIER_T2, 32) == 32 * (42 + 256));
    CHECK(ada_block_bytes(ADA_TIER_T2V8, 16) == 16 * (42 + 132));
    CHECK(ada_block_bytes(ADA_NUM_TIERS, 16) == -1);
    CHECK(ada_lut_floats(&cfg) == (size_t)64 * (256 + 16 + 4));
    CHECK(strncmp(ada_status_str(ADA_OK), "ADA_OK", 6) == 0);
    CHECK(strncmp(ada_status_str((ada_status_t)99), "ADA_UNKNOWN", 11) == 0);
    CHECK(ada_host_f64_to_f16(1.0) == 0x3C00);

    /* workspace queries: the partials of 8 sequences x 32 query heads fit */
    size_t n = 0;
    CHECK(ada_decode_workspace(&cfg, &cache, 8, &n) == ADA_OK);
    CHECK(n >= (size_t)8 * 32 * 130 * 4);
    size_t n2 = 0;
    CHECK(ada_decode_multi_workspace(&cfg, &cache, 8, 2, &n2) == ADA_OK && n2 > n);
    CHECK(ada_decode_multi_workspace(&cfg, &cache, 8, 3, &n2) == ADA_EUNSUPPORTED);
    CHECK(ada_pack_workspace(&cfg, &cache, 8, 32768, &n) == ADA_OK && n > 0);
    CHECK(ada_rdr_workspace(&cfg, 8, 32768, &n) == ADA_OK && n >= (size_t)8 * 8 * 32768);
    CHECK(ada_repack_workspace(&cfg, &cache, 8, &n) == ADA_OK && n > 0);
    CHECK(ada_dense_workspace(&cfg, 8, 2048, &n) == ADA_OK && n > 0);

    /* validation before any device work */
    cfg.head_dim = 64;
    CHECK(ada_decode_workspace(&cfg, &cache, 8, &n) == ADA_EUNSUPPORTED);
    cfg.head_dim = 128;
    CHECK(ada_decode(&cfg, &cache, NULL, 8, 1.0f, NULL, NULL, NULL, 0, NULL) == ADA_EINVAL);
    CHECK(ada_read_status(NULL, NULL) == ADA_EINVAL);
    printf("ok\n");
    return 0;
}
