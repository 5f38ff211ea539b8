/* A plain C11 consumer of libzero1.so: compiled by tests/test_abi.py to show
 * that include/zero1.h is valid C and that the library links and answers its
 * host-only calls without any device work (no GPU is touched).  Prints one
 * line per check; exits non-zero on the first failure. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "zero1.h"

#define CHECK(cond, what)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            printf("FAIL %s: %s\n", what, zero1_last_error()); \
            return 1;                                       \
        }                                                   \
        printf("ok %s\n", what);                            \
    } while (0)

int main(void)
{
    CHECK(zero1_abi_version() == ZERO1_ABI_VERSION, "abi version");
    CHECK(strcmp(zero1_status_string(ZERO1_EINVAL), "ZERO1_EINVAL") == 0, "status string");

    int64_t b = -1, n = -1;
    CHECK(zero1_shard_range(10, 4, 3, &b, &n) == ZERO1_OK && b + n == 10, "shard range");
    CHECK(zero1_shard_range(10, 0, 0, &b, &n) == ZERO1_EINVAL && strlen(zero1_last_error()) > 0,
          "shard range rejects W=0");

    CHECK(zero1_workspace_bytes(1 << 20, 8, ZERO1_STORE_G) >= (size_t)(1 << 20) * 4, "workspace bytes");

    zero1_hparams hp = {1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 7, NULL};
    zero1_step_scalars s;
    CHECK(zero1_step_scalars_derive(&hp, &s) == ZERO1_OK, "step scalars");
    {
        const double want = 1e-3 * sqrt(1.0 - pow(0.95, 7.0)) / (1.0 - pow(0.9, 7.0));
        CHECK(s.step_size == (float)want && s.decay == (float)(1.0 - 1e-3 * 0.1) && s.max_norm == 1.0,
              "step scalars values");
    }
    hp.step = 0;
    CHECK(zero1_step_scalars_derive(&hp, &s) == ZERO1_EINVAL, "step scalars reject t=0");

    zero1_arena_request q;
    memset(&q, 0, sizeof q);
    q.shard_len = 15554976;
    q.W = 8;
    q.grad_elems = 124439808;
    q.grad_offset = 4 * 15554976;
    q.param_elems = 124439808;
    q.param_offset = 4 * 15554976;
    q.capacity = (size_t)200 << 30;
    zero1_arena_layout L;
    CHECK(zero1_arena_plan(&q, &L) == ZERO1_OK && L.spacing == ZERO1_ARENA_SPACING &&
              L.master == L.ws + L.spacing && L.total_bytes <= q.capacity,
          "arena plan");
    q.capacity = 1 << 20;
    CHECK(zero1_arena_plan(&q, &L) == ZERO1_EINVAL, "arena plan rejects a small capacity");

    /* an invalid call is rejected on the host before anything is launched */
    CHECK(zero1_grad_norm(NULL, 10, NULL, NULL, 0, NULL) == ZERO1_EINVAL, "grad norm rejects NULL");
    /* a timing request with no events is accepted (host only) */
    CHECK(zero1_time_next_launch(NULL, NULL) == ZERO1_OK, "timing request");
    printf("all ok\n");
    return 0;
}
