// host_threads.cpp - the host tier and the rings used from several threads
// at once, built with ThreadSanitizer by tests/test_host_sanitizers.py:
//   - a ring: a producer thread submits and reaps, a consumer thread sleeps
//     in kvx_ring_wait, takes and completes, a third thread reads the
//     counts and the peer state meanwhile;
//   - a tier: four threads reserve, commit, look up, release and invalidate
//     overlapping keys; afterwards the counts must add up.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>
#include <unistd.h>

#include "ring.h"
#include "tier.h"

namespace kvx {
int fail(int code, const std::string&) { return code; }
void clear_error() {}
void log_warn(const std::string&) {}
void log_info(const std::string&) {}
}  // namespace kvx

#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            std::exit(1);                                                   \
        }                                                                   \
    } while (0)

static void ring_threads()
{
    char name[64];
    std::snprintf(name, sizeof name, "/kvx-tsan-%d", int(getpid()));
    kvx_ring *r = nullptr, *o = nullptr;
    CHECK(kvx_ring_create(name, 8, 1, &r) == KVX_OK);
    CHECK(kvx_ring_open(name, &o) == KVX_OK);
    const uint64_t total = 50000;
    std::atomic<bool> done{false};
    std::thread consumer([&] {
        kvx_sqe q;
        for (uint64_t want = 1; want <= total;) {
            int32_t ready = 0, got = 0;
            CHECK(kvx_ring_wait(o, 100000, &ready) == KVX_OK);
            if (!ready) continue;
            CHECK(kvx_ring_take(o, &q, &got) == KVX_OK);
            if (!got) continue;
            CHECK(q.op_id == want && q.page_ids[0] == int32_t(want & 1023));
            kvx_cqe c{want, 1, 0, 0};
            while (kvx_ring_complete(o, &c) != KVX_OK) {}
            want++;
        }
    });
    std::thread watcher([&] {
        while (!done.load()) {
            int32_t a = 0, b = 0, alive = 0;
            CHECK(kvx_ring_pending(r, &a, &b) == KVX_OK && a >= 0 && a <= 8 && b >= 0 && b <= 8);
            CHECK(kvx_ring_peer_alive(r, &alive) == KVX_OK && alive == 1);
        }
    });
    kvx_sqe q;
    std::memset(&q, 0, sizeof q);
    uint64_t sent = 1, reaped = 1;
    while (reaped <= total) {
        if (sent <= total) {
            q.op_id = sent;
            q.n = 1;
            q.page_ids[0] = int32_t(sent & 1023);
            if (kvx_ring_submit(r, &q) == KVX_OK) sent++;
        }
        kvx_cqe out[4];
        int32_t got = 0;
        CHECK(kvx_ring_reap(r, out, 4, &got) == KVX_OK);
        for (int32_t i = 0; i < got; i++) CHECK(out[i].op_id == reaped++);
    }
    consumer.join();
    done.store(true);
    watcher.join();
    CHECK(kvx_ring_close(o) == KVX_OK && kvx_ring_close(r) == KVX_OK);
    std::printf("ring: %llu descriptors across three threads\n", static_cast<unsigned long long>(total));
}

static void tier_threads()
{
    kvx_tier* t = nullptr;
    CHECK(kvx_tier_create(64, 1, &t) == KVX_OK);
    std::vector<std::thread> th;
    for (int k = 0; k < 4; k++)
        th.emplace_back([t, k] {
            std::mt19937_64 rng(1000 + k);
            for (int it = 0; it < 4000; it++) {
                uint64_t keys[8];
                int32_t slots[8], n = int32_t(rng() % 8) + 1, ne = 0, hits = 0, nd = 0;
                uint64_t ev[8];
                for (int i = 0; i < n; i++) keys[i] = rng() % 200;
                switch (rng() % 3) {
                case 0:
                    if (kvx_tier_reserve(t, keys, n, slots, ev, &ne) == KVX_OK) {
                        // this thread's reservations are its own to commit
                        CHECK(kvx_tier_commit(t, slots, n) == KVX_OK);
                    }
                    break;
                case 1:
                    CHECK(kvx_tier_lookup(t, keys, n, slots, &hits) == KVX_OK);
                    CHECK(kvx_tier_release(t, slots, n) == KVX_OK);
                    break;
                default:
                    CHECK(kvx_tier_invalidate(t, keys, 1, &nd) == KVX_OK);
                }
            }
        });
    for (auto& x : th) x.join();
    kvx_tier_info info;
    CHECK(kvx_tier_get_info(t, &info) == KVX_OK);
    CHECK(info.writing == 0 && info.pinned == 0 && info.doomed == 0);
    CHECK(info.free_slots + info.resident == 64);
    CHECK(kvx_tier_destroy(t) == KVX_OK);
    std::printf("tier: four threads, %d resident, %llu evictions\n", info.resident,
                static_cast<unsigned long long>(info.evictions));
}

int main()
{
    ring_threads();
    tier_threads();
    std::printf("host threads ok\n");
    return 0;
}
