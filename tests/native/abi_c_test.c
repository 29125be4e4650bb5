/* abi_c_test.c - a C11 program that uses kvx through include/kvx.h alone,
 * as a caller without Python or C++ would. Built by tests/native/build.py
 * with the host C compiler and linked against libkvx.so and the HIP runtime
 * (for hipMalloc / hipMemcpy of the caller's own memory).
 *
 *   abi_c_test cpu   checks that need no GPU: version, registration and its
 *                    refusals (with their messages), packed sizes, the run
 *                    plan, the host tier and a ring's round trip.
 *   abi_c_test gpu   a backup of 8 pages and a publishing restore into 8
 *                    other pages of a device pool, zero-copy: every restored
 *                    piece equals its source piece, every other byte of the
 *                    allocation keeps its value, every layer publishes 8.
 * Prints one line per check and "ok" at the end; exits 1 on the first
 * failure. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include "kvx.h"

#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "check failed line %d: %s (last error: %s)\n", __LINE__, \
                    #cond, kvx_last_error());                                        \
            exit(1);                                                                 \
        }                                                                            \
    } while (0)

/* A [2 layers][K,V][64 pages][16 tokens][2 heads][64] bf16 pool. */
enum { NB = 64, NL = 2, KV = 2, T = 16, H = 2, D = 64, EB = 2, N = 8 };

static kvx_layout tiny_layout(void)
{
    kvx_layout L;
    L.outer[0] = KVX_AX_LAYER;
    L.outer[1] = KVX_AX_KV;
    L.outer[2] = KVX_AX_PAGE;
    L.inner = KVX_NHD;
    L.num_pages = NB;
    L.num_layers = NL;
    L.num_kv = KV;
    L.page_size = T;
    L.num_heads = H;
    L.head_dim = D;
    return L;
}

static void dense(const int64_t* shape, int nd, int64_t* stride)
{
    int64_t acc = 1;
    for (int k = nd - 1; k >= 0; k--) {
        stride[k] = acc;
        acc *= shape[k];
    }
}

static int cpu_checks(void)
{
    CHECK(kvx_version() == KVX_ABI_VERSION);
    kvx_layout L = tiny_layout();
    int64_t shape[6] = {NL, KV, NB, T, H, D}, stride[6];
    dense(shape, 6, stride);
    void* fake = (void*)(uintptr_t)0x7f0000000000ull;   /* never dereferenced */
    kvx_pool* pool = NULL;
    CHECK(kvx_register_pool(&L, fake, 0, EB, 6, shape, stride, 3, &pool) == KVX_OK && pool);
    kvx_pool_info info;
    CHECK(kvx_pool_get_info(pool, &info) == KVX_OK);
    CHECK(info.piece_bytes == (uint64_t)T * H * D * EB && info.page_stride == info.piece_bytes);
    uint64_t bytes = 0;
    CHECK(kvx_packed_bytes(pool, N, &bytes) == KVX_OK && bytes == (uint64_t)NL * KV * N * info.piece_bytes);
    printf("register, geometry, packed size: ok\n");

    /* refusals, before any HIP call */
    int64_t padded[6];
    memcpy(padded, stride, sizeof padded);
    padded[0] += 8;
    kvx_pool* bad = NULL;
    CHECK(kvx_register_pool(&L, fake, 0, EB, 6, shape, padded, 3, &bad) == KVX_E_NONCONTIG);
    CHECK(strstr(kvx_last_error(), "stride") != NULL);
    CHECK(kvx_register_pool(&L, fake, 8, EB, 6, shape, stride, 3, &bad) == KVX_E_ALIGN);
    int32_t ids[N] = {5, 1, 9, 63, 2, 3, 4, 40};
    int32_t dup[2] = {7, 7}, outside[1] = {NB};
    CHECK(kvx_backup(pool, outside, 1, fake, bytes, 0, NL, NULL, KVX_PATH_ZEROCOPY) == KVX_E_RANGE);
    CHECK(kvx_restore(pool, fake, bytes, dup, 2, 0, NL, NULL, 0, NULL, KVX_PATH_ZEROCOPY) == KVX_E_DUP);
    CHECK(kvx_backup(pool, ids, N, fake, bytes, 0, NL + 1, NULL, KVX_PATH_ZEROCOPY) == KVX_E_RANGE);
    CHECK(kvx_backup(pool, ids, 0, fake, bytes, 0, NL, NULL, KVX_PATH_ZEROCOPY) == KVX_OK);   /* no-op */
    printf("refusals and messages: ok\n");

    int32_t runs[3 * N], nruns = 0;
    CHECK(kvx_plan_runs(pool, ids, N, runs, N, &nruns) == KVX_OK);
    CHECK(nruns >= 1 && nruns <= N && runs[0] == 1);   /* sorted by page */
    printf("run plan: %d runs\n", nruns);

    /* host tier: two slots, a third key evicts the least recently used */
    kvx_tier* tier = NULL;
    CHECK(kvx_tier_create(2, 3, &tier) == KVX_OK);
    uint64_t keys[3] = {101, 102, 103}, evicted[1];
    int32_t slots[2], ne = 0, hits = 0;
    CHECK(kvx_tier_reserve(tier, keys, 2, slots, evicted, &ne) == KVX_OK && ne == 0);
    CHECK(kvx_tier_commit(tier, slots, 2) == KVX_OK);
    CHECK(kvx_tier_lookup(tier, keys + 1, 1, slots, &hits) == KVX_OK && hits == 1);
    CHECK(kvx_tier_release(tier, slots, 1) == KVX_OK);
    CHECK(kvx_tier_reserve(tier, keys + 2, 1, slots, evicted, &ne) == KVX_OK);
    CHECK(ne == 1 && evicted[0] == 101 && slots[0] == 0);
    CHECK(kvx_tier_destroy(tier) == KVX_OK);
    printf("host tier: ok\n");

    /* a ring, both sides in this process */
    char name[64];
    snprintf(name, sizeof name, "/kvx-c-test-%d", (int)getpid());
    kvx_ring *sched = NULL, *plane = NULL;
    CHECK(kvx_ring_create(name, 4, 3, &sched) == KVX_OK);
    CHECK(kvx_ring_open(name, &plane) == KVX_OK);
    kvx_sqe* q = (kvx_sqe*)calloc(1, sizeof *q);
    CHECK(q != NULL);
    q->op_id = 42;
    q->generation = 2;   /* not the pool's: the executor refuses it at once */
    q->op = KVX_OP_BACKUP;
    q->n = N;
    q->layer_end = NL;
    q->path = KVX_PATH_ZEROCOPY;
    q->ready_slot_base = -1;
    memcpy(q->page_ids, ids, sizeof ids);
    CHECK(kvx_ring_submit(sched, q) == KVX_OK);
    void* bufs[1] = {fake};
    uint64_t sizes[1] = {bytes};
    int32_t taken = 0, done = 0, got = 0;
    CHECK(kvx_ring_serve(plane, &pool, 1, bufs, sizes, 1, NULL, NULL, 8, &taken, &done) == KVX_OK);
    CHECK(taken == 1 && done == 1);
    kvx_cqe c;
    CHECK(kvx_ring_reap(sched, &c, 1, &got) == KVX_OK && got == 1);
    CHECK(c.op_id == 42 && c.status == KVX_E_STALE);
    free(q);
    CHECK(kvx_ring_close(plane) == KVX_OK && kvx_ring_close(sched) == KVX_OK);
    printf("ring: ok\n");

    CHECK(kvx_unregister_pool(pool) == KVX_OK);
    CHECK(kvx_unregister_pool(pool) == KVX_OK);   /* teardown never fails loudly */
    return 0;
}

static uint8_t pattern(uint64_t a)
{
    uint64_t x = (a + 1) * 0x9E3779B97F4A7C15ull;
    return (uint8_t)(x >> 56);
}

static int gpu_checks(void)
{
    kvx_layout L = tiny_layout();
    int64_t shape[6] = {NL, KV, NB, T, H, D}, stride[6];
    dense(shape, 6, stride);
    const size_t piece = (size_t)T * H * D * EB;
    const size_t pool_bytes = (size_t)NB * NL * KV * piece;
    uint8_t* img = (uint8_t*)malloc(pool_bytes);
    uint8_t* after = (uint8_t*)malloc(pool_bytes);
    CHECK(img && after);
    for (size_t a = 0; a < pool_bytes; a++) img[a] = pattern(a);
    void* dev = NULL;
    CHECK(hipMalloc(&dev, pool_bytes) == hipSuccess);
    CHECK(hipMemcpy(dev, img, pool_bytes, hipMemcpyHostToDevice) == hipSuccess);
    kvx_pool* pool = NULL;
    CHECK(kvx_register_pool(&L, dev, 0, EB, 6, shape, stride, 5, &pool) == KVX_OK);
    uint64_t bytes = 0;
    CHECK(kvx_packed_bytes(pool, N, &bytes) == KVX_OK);
    void* host = NULL;
    CHECK(kvx_host_alloc(bytes, &host) == KVX_OK);
    kvx_ready* ready = NULL;
    CHECK(kvx_ready_create(NL, 5, &ready) == KVX_OK);
    int32_t src[N] = {5, 1, 9, 63, 2, 3, 4, 40}, dst[N] = {10, 11, 20, 21, 30, 31, 50, 60};
    CHECK(kvx_backup(pool, src, N, host, bytes, 0, NL, NULL, KVX_PATH_ZEROCOPY) == KVX_OK);
    CHECK(kvx_restore(pool, host, bytes, dst, N, 0, NL, ready, 0, NULL, KVX_PATH_ZEROCOPY) == KVX_OK);
    CHECK(kvx_sync(NULL) == KVX_OK);
    int32_t prefix = -1;
    CHECK(kvx_ready_prefix(ready, &prefix) == KVX_OK && prefix == N);
    CHECK(hipMemcpy(after, dev, pool_bytes, hipMemcpyDeviceToHost) == hipSuccess);
    /* layer-major pool: piece (p, l, c) starts at ((l * KV + c) * NB + p) * piece */
    char* written = (char*)calloc(pool_bytes / piece, 1);
    CHECK(written != NULL);
    for (int i = 0; i < N; i++)
        for (int l = 0; l < NL; l++)
            for (int c = 0; c < KV; c++) {
                const size_t s = ((size_t)(l * KV + c) * NB + src[i]) * piece;
                const size_t d = ((size_t)(l * KV + c) * NB + dst[i]) * piece;
                CHECK(memcmp(after + d, img + s, piece) == 0);
                written[d / piece] = 1;
            }
    for (size_t k = 0; k < pool_bytes / piece; k++)
        if (!written[k]) CHECK(memcmp(after + k * piece, img + k * piece, piece) == 0);
    printf("round trip: %d pages x %d layers x %d, other pieces unchanged, prefix %d: ok\n", N, NL,
           KV, prefix);
    CHECK(kvx_ready_destroy(ready) == KVX_OK);
    CHECK(kvx_unregister_pool(pool) == KVX_OK);
    CHECK(kvx_host_free(host) == KVX_OK);
    CHECK(hipFree(dev) == hipSuccess);
    free(written);
    free(img);
    free(after);
    return 0;
}

int main(int argc, char** argv)
{
    if (argc != 2 || (strcmp(argv[1], "cpu") != 0 && strcmp(argv[1], "gpu") != 0)) {
        fprintf(stderr, "usage: %s cpu|gpu\n", argv[0]);
        return 2;
    }
    const int rc = strcmp(argv[1], "cpu") == 0 ? cpu_checks() : gpu_checks();
    if (rc == 0) printf("ok\n");
    return rc;
}
