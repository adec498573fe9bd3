/*
 * A plain C99 client of include/ccl.h, built with gcc by the CPU tests: the
 * header must compile as C, and the host-only parts of the library (status
 * strings, argument checks that reject a call before any HIP call, the
 * reshard planner) must work through the C ABI alone.
 *
 * The planner is checked on the weight reshard of the NCCL M2N write-up's
 * Example A (TP4 -> TP2 x DP2): [8192, 28672] bf16, source mesh [1, 4] from
 * rank 0 with (Replicate, Shard(0)), destination mesh [2, 2] from rank 4 with
 * (Replicate, Shard(0)).  Each source block of 2048 rows lands in destination
 * shard r / 2 at byte offset (r mod 2) * 2048 rows, and every destination
 * shard has two replicas.
 *
 * Prints "ok" and exits 0 on success; prints the failed check and exits 1.
 */
#include <stdio.h>
#include <string.h>

#include "ccl.h"

static int failures = 0;

#define CHECK(cond)                                                  \
    do {                                                             \
        if (!(cond)) {                                               \
            printf("FAILED line %d: %s\n", __LINE__, #cond);         \
            ++failures;                                              \
        }                                                            \
    } while (0)

static int check_example_a(void) {
    const uint64_t rows = 8192, cols = 28672, esz = 2;
    const uint64_t block = rows / 4 * cols * esz; /* 117,440,512 bytes */
    ccl_tensor_desc_t t;
    ccl_mesh_t src, dst;
    ccl_placement_t src_pl[2], dst_pl[2];
    ccl_plan_t *plan = NULL;
    uint64_t n = 0, i, bytes = 0;
    int32_t shards = 0;
    int side, k;

    memset(&t, 0, sizeof t);
    memset(&src, 0, sizeof src);
    memset(&dst, 0, sizeof dst);
    t.ndim = 2;
    t.dtype = CCL_BFLOAT16;
    t.shape[0] = (int64_t)rows;
    t.shape[1] = (int64_t)cols;
    src.ndims = 2;
    src.start_rank = 0;
    src.dims[0] = 1;
    src.dims[1] = 4;
    dst.ndims = 2;
    dst.start_rank = 4;
    dst.dims[0] = 2;
    dst.dims[1] = 2;
    src_pl[0].kind = CCL_REPLICATE;
    src_pl[0].dim = 0;
    src_pl[1].kind = CCL_SHARD;
    src_pl[1].dim = 0;
    dst_pl[0] = src_pl[0];
    dst_pl[1] = src_pl[1];

    CHECK(ccl_reshard_plan(&t, &src, src_pl, &dst, dst_pl, &plan) == CCL_OK);
    if (!plan) return 1;
    CHECK(ccl_plan_num_intervals(plan, &n) == CCL_OK);
    CHECK(n == 4);
    CHECK(ccl_plan_num_dst_shards(plan, &shards) == CCL_OK);
    CHECK(shards == 2);
    for (i = 0; i < n; ++i) {
        ccl_interval_t iv;
        int32_t reps[4], nrep = 0;
        CHECK(ccl_plan_get_interval(plan, i, &iv) == CCL_OK);
        CHECK(iv.length == block);
        CHECK(iv.src_offset == 0);
        CHECK(iv.dst_shard == iv.src_rank / 2);
        CHECK(iv.dst_offset == (uint64_t)(iv.src_rank % 2) * block);
        CHECK(iv.num_replicas == 2);
        CHECK(ccl_plan_shard_replicas(plan, iv.dst_shard, reps, 4, &nrep) == CCL_OK);
        CHECK(nrep == 2);
        /* row-major numbering: shard 0 on ranks 4 and 6, shard 1 on 5 and 7 */
        CHECK(reps[0] == 4 + iv.dst_shard && reps[1] == 6 + iv.dst_shard);
        CHECK(iv.leader == reps[0] || iv.leader == reps[1]);
    }
    for (side = 0; side < 2; ++side)
        for (k = 0; k < 4; ++k) {
            CHECK(ccl_plan_local_bytes(plan, side, k, &bytes) == CCL_OK);
            CHECK(bytes == (side == 0 ? block : 2 * block));
        }
    CHECK(ccl_plan_local_bytes(plan, 1, 4, &bytes) != CCL_OK);
    CHECK(ccl_plan_get_interval(plan, n, NULL) != CCL_OK);
    CHECK(ccl_plan_destroy(plan) == CCL_OK);

    /* two sharded mesh axes break the one-sharded-axis rule */
    src_pl[0].kind = CCL_SHARD;
    src_pl[0].dim = 1;
    plan = NULL;
    CHECK(ccl_reshard_plan(&t, &src, src_pl, &dst, dst_pl, &plan) == CCL_ERR_LAYOUT);
    CHECK(plan == NULL);
    return 0;
}

int main(void) {
    const void *send[2] = {NULL, NULL};
    void *recv[2] = {NULL, NULL};
    int s;

    CHECK(ccl_version() > 0);
    for (s = CCL_OK; s <= CCL_ERR_SCRATCH_LIMIT; ++s) CHECK(ccl_get_error_string((ccl_status_t)s) != NULL);

    /* rejected before any HIP call: null buffers, bad rank counts, bad dtype */
    CHECK(ccl_all_reduce(send, recv, 2, 16, CCL_FLOAT32, CCL_SUM, NULL, NULL) ==
          CCL_ERR_INVALID_ARG);
    CHECK(ccl_all_reduce(send, recv, 0, 16, CCL_FLOAT32, CCL_SUM, NULL, NULL) ==
          CCL_ERR_INVALID_ARG);
    CHECK(ccl_reduce_scatter(send, recv, 2, 16, 99, CCL_SUM, NULL, NULL) == CCL_ERR_INVALID_ARG);
    CHECK(ccl_all_gather(NULL, recv, 2, 16, CCL_INT32, NULL, NULL) == CCL_ERR_INVALID_ARG);
    /* zero elements is a no-op that succeeds */
    CHECK(ccl_all_reduce(send, recv, 2, 0, CCL_BFLOAT16, CCL_MAX, NULL, NULL) == CCL_OK);

    /* launch configuration: store_policy 0..2 accepted, anything else rejected */
    {
        ccl_launch_config_t cfg;
        memset(&cfg, 0, sizeof cfg);
        cfg.store_policy = 1;
        CHECK(ccl_all_reduce(send, recv, 2, 0, CCL_BFLOAT16, CCL_SUM, NULL, &cfg) == CCL_OK);
        cfg.store_policy = 2;
        CHECK(ccl_all_gather(send, recv, 2, 0, CCL_BFLOAT16, NULL, &cfg) == CCL_OK);
        cfg.store_policy = 3;
        CHECK(ccl_all_reduce(send, recv, 2, 0, CCL_BFLOAT16, CCL_SUM, NULL, &cfg) ==
              CCL_ERR_INVALID_ARG);
        cfg.store_policy = -1;
        CHECK(ccl_reduce_scatter(send, recv, 2, 0, CCL_FLOAT32, CCL_SUM, NULL, &cfg) ==
              CCL_ERR_INVALID_ARG);
    }

    check_example_a();
    if (failures) return 1;
    printf("ok\n");
    return 0;
}
