/* A plain C99 caller of the library's host-side entry points: the header
 * must compile as strict C, the library must link from C, and the calls that
 * need no GPU must behave as declared.  Prints one line per check and exits
 * non-zero on the first failure. */
#include "bf16opt.h"

#include <math.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

static void check(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok) ++failures;
}

int main(int argc, char **argv) {
    uint64_t b = 0, e = 0;
    check(shard_range(1557686400ull, 8, 1, &b, &e) == BFO_OK && b == 194710800ull && e == 389421600ull,
          "shard_range of the 1.5B buffer, rank 1 of 8");
    check(shard_range(10, 3, 0, &b, &e) == BFO_ENOTDIVISIBLE, "shard_range refuses 10 over 3");
    check(shard_range(10, 2, 2, &b, &e) == BFO_ERANGE, "shard_range refuses rank 2 of 2");
    check(shard_range(10, 0, 0, &b, &e) == BFO_EINVAL, "shard_range refuses world 0");

    bfo_tensor bad[2];
    memset(bad, 0, sizeof bad);
    bad[0].offset = 0; bad[0].numel = 4;
    bad[1].offset = 5; bad[1].numel = 4;   /* gap: not contiguous */
    bfo_table tb = NULL;
    check(bfo_table_create(bad, 2, 1, 0, &tb) == BFO_ETABLE && tb == NULL, "a table with a gap is refused");

    bfo_lr_schedule sch;
    memset(&sch, 0, sizeof sch);
    sch.kind = BFO_LR_COSINE;
    sch.warmup_steps = 10;
    sch.total_steps = 110;
    sch.lr_max = 1e-3f;
    sch.final_frac = 0.1f;
    float lr = 0.0f;
    check(bfo_lr_at(&sch, 0, &lr) == BFO_OK && fabsf(lr - 1e-4f) < 1e-10f, "cosine warm-up starts at lr/10");
    check(bfo_lr_at(&sch, 60, &lr) == BFO_OK && fabsf(lr - 5.5e-4f) < 1e-9f, "cosine midpoint is the mean of peak and floor");
    check(bfo_lr_at(&sch, 110, &lr) == BFO_OK && fabsf(lr - 1e-4f) < 1e-10f, "cosine ends at the floor");

    check(strcmp(bfo_status_string(BFO_OK), "ok") == 0, "status string of BFO_OK");

    bfo_adamw_hparams hp;
    memset(&hp, 0, sizeof hp);
    check(grad_global_norm(NULL, NULL, 1.0f, NULL, NULL, NULL) == BFO_EINVAL, "grad_global_norm refuses a null table");
    check(adamw_sr_step(NULL, NULL, NULL, NULL, NULL, NULL, &hp, NULL, NULL, 1, 0, BFO_ROUND_SR, NULL) == BFO_EINVAL,
          "adamw_sr_step refuses a null table");
    check(master_to_bf16_sr(NULL, NULL, NULL, 0, NULL) == BFO_EINVAL, "master_to_bf16_sr refuses a null table");

    if (argc > 1) {   /* an empty directory: no checkpoint yet */
        uint64_t step = 0;
        check(bfo_checkpoint_latest(argv[1], &step) == BFO_ENOTFOUND, "no DONE marker -> BFO_ENOTFOUND");
        check(bfo_checkpoint_done(argv[1], 42) == BFO_OK && bfo_checkpoint_latest(argv[1], &step) == BFO_OK &&
                  step == 42,
              "a DONE marker is found as the latest step");
    }
    return failures ? 1 : 0;
}
