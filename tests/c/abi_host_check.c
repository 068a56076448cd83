/* A plain C program against include/zero.h: the host-only entry points
 * (layout, index maps, step scalars, clip coefficient, ledger, traffic,
 * diagnostics) called without Python or torch.  Exits 0 when every check
 * holds; prints the first failure otherwise.  No GPU is touched. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero.h"

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            printf("FAIL line %d: %s\n", __LINE__, #c);                 \
            return 1;                                                   \
        }                                                               \
    } while (0)

int main(void)
{
    CHECK(zero_abi_version() == ZERO_ABI_VERSION);
    const int64_t numel[3] = {1000, 1001, 7};
    size_t need = 0;
    CHECK(zero_pack(4, 3, numel, NULL, 0, &need) == ZERO_OK);
    CHECK(need == zero_layout_bytes(3));
    zero_layout *L = (zero_layout *)malloc(need);
    CHECK(zero_pack(4, 3, numel, L, need - 1, NULL) == ZERO_ENOSPC);
    CHECK(zero_pack(4, 3, numel, L, need, NULL) == ZERO_OK);
    CHECK(L->padded == 1000 + 1004 + 8 && L->shard == 250 + 251 + 2);
    CHECK(L->unit[1].offset == 1000 && L->unit[2].local_offset == 501);
    /* every local index of every rank maps to a distinct global index whose
     * owner is that rank and local index */
    for (int r = 0; r < 4; ++r)
        for (int64_t k = 0; k < L->shard; ++k) {
            int64_t j = -1, k2 = -1;
            int32_t r2 = -1;
            CHECK(zero_global_index(L, r, k, &j) == ZERO_OK);
            CHECK(zero_owner(L, j, &r2, &k2) == ZERO_OK);
            CHECK(r2 == r && k2 == k);
        }
    zero_adamw_scalars s1, s2, s3;
    CHECK(zero_adamw_scalars_for(1, 0.01f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, &s1) == ZERO_OK);
    CHECK(zero_adamw_scalars_next(&s1, &s2) == ZERO_OK);
    CHECK(zero_adamw_scalars_for(2, 0.01f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, &s3) == ZERO_OK);
    CHECK(memcmp(&s2, &s3, sizeof s2) == 0);
    CHECK(s1.pow1 == 0.9f && s1.bc1 == 1.0f - 0.9f);
    float c = 0.0f;
    CHECK(zero_clip_coef(4.0, 1.0, &c) == ZERO_OK && fabsf(c - 0.5f) < 1e-6f);
    zero_ledger_out o;
    CHECK(zero_ledger(70e9, 64, 3, 0, &o) == ZERO_OK);
    CHECK(fabs(o.model_state_bytes / 1e9 - 17.5) < 1e-9 && o.comm_elements == 3 * 70e9);
    CHECK(zero_ledger(1000, 4, 1, 0, &o) == ZERO_OK && o.optimizer_floats_per_rank == 750.0);
    double bytes = 0;
    int64_t el = 0;
    CHECK(zero_step_traffic(L, -1, 4, ZERO_BF16, 1, &bytes, &el) == ZERO_OK);
    CHECK(el == L->padded && bytes == (2.0 * 4 + 26) * (double)el);
    CHECK(strcmp(zero_strerror(ZERO_EINVAL), "invalid argument") == 0);
    CHECK(zero_last_hip_error()[0] == '\0');
    /* invalid calls are rejected before any device work */
    CHECK(zero_step(NULL, -1, NULL, 1, ZERO_BF16, ZERO_GLOBAL, 4.0f, NULL, NULL, NULL, 0, NULL, 0,
                    &s1, NULL) == ZERO_EINVAL);
    CHECK(zero_pack(0, 3, numel, L, need, NULL) == ZERO_EINVAL);
    free(L);
    printf("ok\n");
    return 0;
}
