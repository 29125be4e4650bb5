// host_fuzz.cpp - randomized checks of kvx's host-only logic (pool layout
// validator, page-list checks, run planning), built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py. Each
// accepted layout is compared with a brute-force row-major index; each plan
// must cover every (page, slot) pair exactly once with valid runs.
#include <algorithm>
#include <deque>
#include <thread>
#include <unistd.h>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "kvx_host.h"
#include "ring.h"
#include "tier.h"

namespace kvx {
static int g_last_code = 0;
int fail(int code, const std::string&) { g_last_code = code; return code; }
void clear_error() {}
void log_warn(const std::string&) {}
void log_info(const std::string&) {}
}  // namespace kvx

using namespace kvx;

#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            std::exit(1);                                                   \
        }                                                                   \
    } while (0)

static std::mt19937_64 rng(12345);
static int64_t rnd(int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); }

// byte offset of piece (p, l, c) by brute force: walk the row-major index
static int64_t piece_offset(const kvx_layout& L, int64_t piece_bytes, int64_t p, int64_t l, int64_t c)
{
    const int64_t size[3] = {L.num_pages, L.num_layers, L.num_kv};
    const int64_t coord[3] = {p, l, c};
    int64_t idx = 0;
    for (int k = 0; k < 3; k++) idx = idx * size[L.outer[k]] + coord[L.outer[k]];
    return idx * piece_bytes;
}

static void fuzz_geometry(int iters)
{
    int accepted = 0;
    for (int it = 0; it < iters; it++) {
        kvx_layout L;
        int perm[3] = {0, 1, 2};
        std::shuffle(perm, perm + 3, rng);
        for (int k = 0; k < 3; k++) L.outer[k] = perm[k];
        L.inner = static_cast<int32_t>(rnd(0, 1));
        L.num_pages = static_cast<int32_t>(rnd(1, 9));
        L.num_layers = static_cast<int32_t>(rnd(1, 5));
        L.num_kv = static_cast<int32_t>(rnd(1, 2));
        L.page_size = static_cast<int32_t>(rnd(1, 7));
        L.num_heads = static_cast<int32_t>(rnd(1, 5));
        L.head_dim = static_cast<int32_t>(8 * rnd(1, 4));
        const uint32_t eb = static_cast<uint32_t>(1 << rnd(0, 2));
        if (rnd(0, 20) == 0) L.num_heads = 0;                 // invalid dim
        if (rnd(0, 20) == 0) L.outer[1] = L.outer[0];          // not a permutation
        const int64_t sz[3] = {L.num_pages, L.num_layers, L.num_kv};
        std::vector<int64_t> phys = {sz[L.outer[0]], sz[L.outer[1]], sz[L.outer[2]],
                                     L.inner ? L.num_heads : L.page_size,
                                     L.inner ? L.page_size : L.num_heads, L.head_dim};
        // a view: the physical dims with random neighbours merged, sometimes broken
        std::vector<int64_t> shape;
        for (int64_t d : phys) {
            if (!shape.empty() && rnd(0, 2) == 0) shape.back() *= d;
            else shape.push_back(d);
        }
        if (rnd(0, 15) == 0 && shape.size() > 1) std::swap(shape[0], shape[1]);   // wrong split
        if (rnd(0, 15) == 0) shape.back() += 1;                                   // wrong count
        std::vector<int64_t> stride(shape.size());
        int64_t acc = 1;
        for (size_t k = shape.size(); k-- > 0;) { stride[k] = acc; acc *= shape[k]; }
        if (rnd(0, 10) == 0 && shape.size() > 1) stride[0] += 1;                  // not dense
        const uint64_t base = 0x10000ull * rnd(1, 1000) + (rnd(0, 12) == 0 ? 8 : 0);
        const uint64_t off = 16ull * rnd(0, 64);
        PoolGeom g;
        int rc = derive_geometry(&L, reinterpret_cast<void*>(base), off, eb,
                                 static_cast<int32_t>(shape.size()), shape.data(), stride.data(), &g);
        if (rc != KVX_OK) continue;
        accepted++;
        CHECK(g.row_bytes == L.head_dim * int64_t(eb));
        CHECK(g.piece_bytes == L.page_size * L.num_heads * g.row_bytes);
        CHECK(g.pool_bytes == int64_t(L.num_pages) * L.num_layers * L.num_kv * g.piece_bytes);
        CHECK((base + off) % 16 == 0 && g.row_bytes % 16 == 0);
        for (int64_t p = 0; p < L.num_pages; p++)
            for (int64_t l = 0; l < L.num_layers; l++)
                for (int64_t c = 0; c < L.num_kv; c++)
                    CHECK(p * g.page_stride + l * g.layer_stride + c * g.kv_stride ==
                          piece_offset(L, g.piece_bytes, p, l, c));
    }
    CHECK(accepted > iters / 4);
    std::printf("geometry: %d of %d accepted and verified\n", accepted, iters);
}

static void fuzz_extremes()
{
    kvx_layout L{{0, 1, 2}, 0, 2147483647, 2147483647, 2, 2147483647, 2147483647, 2147483647};
    int64_t shape[1] = {1}, stride[1] = {1};
    PoolGeom g;
    CHECK(derive_geometry(&L, reinterpret_cast<void*>(0x1000), 0, 2, 1, shape, stride, &g) == KVX_E_INVAL);
    kvx_layout M{{1, 2, 0}, 1, 4, 2, 2, 8, 4, 64};
    int64_t s9[9] = {1, 1, 1, 1, 1, 1, 1, 1, 1}, t9[9] = {1, 1, 1, 1, 1, 1, 1, 1, 1};
    CHECK(derive_geometry(&M, reinterpret_cast<void*>(0x1000), 0, 2, 9, s9, t9, &g) == KVX_E_INVAL);
    CHECK(derive_geometry(&M, reinterpret_cast<void*>(0x1000), 0, 2, 0, s9, t9, &g) == KVX_E_INVAL);
    CHECK(derive_geometry(nullptr, reinterpret_cast<void*>(0x1000), 0, 2, 1, s9, t9, &g) == KVX_E_INVAL);
    CHECK(derive_geometry(&M, nullptr, 0, 2, 1, s9, t9, &g) == KVX_E_INVAL);
    CHECK(derive_geometry(&M, reinterpret_cast<void*>(0x1000), 0, 0, 1, s9, t9, &g) == KVX_E_INVAL);
    int64_t neg[2] = {-4, 2}, st2[2] = {2, 1};
    CHECK(derive_geometry(&M, reinterpret_cast<void*>(0x1000), 0, 2, 2, neg, st2, &g) == KVX_E_INVAL);
    std::printf("extremes: ok\n");
}

static void fuzz_pages(int iters)
{
    for (int it = 0; it < iters; it++) {
        PoolGeom g;
        g.num_pages = rnd(1, 5000);
        g.piece_bytes = 4096;
        g.pages_adjacent = rnd(0, 1) != 0;
        const int32_t n = static_cast<int32_t>(rnd(0, 3000));
        std::vector<int32_t> ids(n);
        const bool contiguous = rnd(0, 3) == 0;
        int32_t start = static_cast<int32_t>(rnd(0, g.num_pages - 1));
        for (int32_t i = 0; i < n; i++)
            ids[i] = contiguous ? static_cast<int32_t>((start + i) % g.num_pages)
                                : static_cast<int32_t>(rnd(0, g.num_pages - 1));
        if (n > 0 && rnd(0, 10) == 0) ids[rnd(0, n - 1)] = static_cast<int32_t>(g.num_pages + rnd(0, 3));
        if (n > 0 && rnd(0, 10) == 0) ids[rnd(0, n - 1)] = -1 - static_cast<int32_t>(rnd(0, 3));
        bool in_range = true;
        for (int32_t v : ids) in_range = in_range && v >= 0 && v < g.num_pages;
        const int rc = check_page_ids(g, ids.data(), n, false);
        CHECK((rc == KVX_OK) == in_range);
        if (!in_range) continue;
        const bool distinct = std::set<int32_t>(ids.begin(), ids.end()).size() == ids.size();
        CHECK((check_page_ids(g, ids.data(), n, true) == KVX_OK) == distinct);
        for (bool sorted : {false, true}) {
            std::vector<PageSlot> pairs;
            order_pages(ids.data(), n, sorted, &pairs);
            CHECK(static_cast<int32_t>(pairs.size()) == n);
            for (size_t j = 0; j + 1 < pairs.size() && sorted; j++) CHECK(pairs[j].page <= pairs[j + 1].page);
            std::vector<int> seen(n, 0);
            for (const PageSlot& ps : pairs) {
                CHECK(ps.slot >= 0 && ps.slot < n && ids[ps.slot] == ps.page);
                seen[ps.slot]++;
            }
            for (int v : seen) CHECK(v == 1);
            if (!sorted) continue;
            std::vector<Run> runs;
            plan_runs(g, pairs, &runs);
            std::vector<int> covered(n, 0);
            for (const Run& r : runs) {
                CHECK(r.count >= 1 && (r.count == 1 || g.pages_adjacent));
                for (int32_t k = 0; k < r.count; k++) {
                    CHECK(r.slot + k < n && ids[r.slot + k] == r.page + k);
                    covered[r.slot + k]++;
                }
            }
            for (int v : covered) CHECK(v == 1);
        }
    }
    std::printf("pages: %d random lists checked\n", iters);
}

// Host-slot lists: check_host_slots accepts exactly the in-range lists
// (and, when asked, only distinct ones); order_pairs keeps every
// (page, slot) pair of the caller and sorts by page when asked.
static void fuzz_slots(int iters)
{
    for (int it = 0; it < iters; it++) {
        const int64_t S = rnd(0, 4000);
        const int32_t n = static_cast<int32_t>(rnd(0, 2000));
        std::vector<int32_t> slots(n), ids(n);
        for (int32_t i = 0; i < n; i++) {
            slots[i] = S ? static_cast<int32_t>(rnd(0, S - 1)) : 0;
            ids[i] = static_cast<int32_t>(rnd(0, 9999));
        }
        if (n > 0 && rnd(0, 8) == 0) slots[rnd(0, n - 1)] = static_cast<int32_t>(S + rnd(0, 3));
        if (n > 0 && rnd(0, 8) == 0) slots[rnd(0, n - 1)] = -1 - static_cast<int32_t>(rnd(0, 3));
        bool in_range = true;
        for (int32_t v : slots) in_range = in_range && v >= 0 && v < S;
        CHECK((check_host_slots(slots.data(), n, S, false) == KVX_OK) == in_range);
        if (!in_range) continue;
        const bool distinct = std::set<int32_t>(slots.begin(), slots.end()).size() == slots.size();
        CHECK((check_host_slots(slots.data(), n, S, true) == KVX_OK) == distinct);
        for (bool sorted : {false, true}) {
            std::vector<PageSlot> pairs;
            order_pairs(ids.data(), slots.data(), n, sorted, &pairs);
            CHECK(static_cast<int32_t>(pairs.size()) == n);
            std::multiset<std::pair<int32_t, int32_t>> want, got;
            for (int32_t i = 0; i < n; i++) {
                want.insert({ids[i], slots[i]});
                got.insert({pairs[i].page, pairs[i].slot});
                if (!sorted) CHECK(pairs[i].page == ids[i] && pairs[i].slot == slots[i]);
            }
            CHECK(want == got);
            for (size_t j = 0; j + 1 < pairs.size() && sorted; j++) CHECK(pairs[j].page <= pairs[j + 1].page);
        }
    }
    std::printf("slots: %d random lists checked\n", iters);
}

// Host tier: random operations through the C entry points; after each
// one the tier's index structures must agree with its entries (the free set
// holds exactly the FREE slots, the key map exactly the present entries,
// the LRU set exactly the evictable ones) and every count must add up.
static void check_tier(const kvx_tier* t)
{
    size_t nfree = 0, npresent = 0, nevict = 0;
    for (int32_t s = 0; s < int32_t(t->e.size()); s++) {
        const TierEntry& x = t->e[s];
        CHECK(x.pins >= 0);
        CHECK(x.pins == 0 || x.state == TIER_RESIDENT);
        if (x.state == TIER_FREE) {
            CHECK(t->free_slots.count(s) && x.key == 0 && !x.doomed && x.pins == 0);
            nfree++;
            continue;
        }
        CHECK(!t->free_slots.count(s));
        if (!x.doomed) {
            auto it = t->where.find(x.key);
            CHECK(it != t->where.end() && it->second == s);
            npresent++;
        }
        const bool ev = x.state == TIER_RESIDENT && x.pins == 0 && !x.doomed;
        CHECK(t->lru.count({x.last, s}) == (ev ? 1u : 0u));
        nevict += ev;
        CHECK(x.last <= t->clock);
    }
    CHECK(nfree == t->free_slots.size() && npresent == t->where.size() && nevict == t->lru.size());
}

static void fuzz_tier(int iters)
{
    int ok = 0;
    for (int it = 0; it < iters; it++) {
        const int32_t S = static_cast<int32_t>(rnd(0, 40));
        kvx_tier* t = nullptr;
        CHECK(kvx_tier_create(S, 1, &t) == KVX_OK);
        std::vector<int32_t> writing, held;
        const uint64_t nkeys = static_cast<uint64_t>(rnd(1, 3 * S + 3));
        for (int step = 0; step < 200; step++) {
            const int op = static_cast<int>(rnd(0, 6));
            const int32_t n = static_cast<int32_t>(rnd(0, S + 2));
            std::vector<uint64_t> keys(n), ev(n + 1);
            std::vector<int32_t> slots(n + 1);
            for (auto& k : keys) k = static_cast<uint64_t>(rnd(0, nkeys - 1)) * 0x9E3779B97F4A7C15ull;
            int32_t cnt = 0;
            int rc = KVX_OK;
            if (op == 0) {
                rc = kvx_tier_reserve(t, keys.data(), n, slots.data(), ev.data(), &cnt);
                if (rc == KVX_OK) {
                    CHECK(cnt >= 0 && cnt <= n);
                    for (int32_t i = 0; i < n; i++) if (slots[i] >= 0) writing.push_back(slots[i]);
                } else {
                    CHECK(rc == KVX_E_FULL);
                }
            } else if (op == 1 || op == 2) {
                std::shuffle(writing.begin(), writing.end(), rng);
                const size_t k = static_cast<size_t>(rnd(0, int64_t(writing.size())));
                std::vector<int32_t> sl(writing.begin(), writing.begin() + k);
                writing.erase(writing.begin(), writing.begin() + k);
                if (rnd(0, 9) == 0) sl.push_back(static_cast<int32_t>(rnd(-3, S + 3)));
                rc = op == 1 ? kvx_tier_commit(t, sl.data(), int32_t(sl.size()))
                             : kvx_tier_abort(t, sl.data(), int32_t(sl.size()));
            } else if (op == 3) {
                rc = kvx_tier_lookup(t, keys.data(), n, slots.data(), &cnt);
                CHECK(rc == KVX_OK);
                for (int32_t i = 0; i < n; i++) if (slots[i] >= 0) held.push_back(slots[i]);
            } else if (op == 4) {
                std::shuffle(held.begin(), held.end(), rng);
                const size_t k = static_cast<size_t>(rnd(0, int64_t(held.size())));
                std::vector<int32_t> sl(held.begin(), held.begin() + k);
                held.erase(held.begin(), held.begin() + k);
                if (rnd(0, 9) == 0) sl.push_back(static_cast<int32_t>(rnd(-3, S + 3)));
                rc = kvx_tier_release(t, sl.data(), int32_t(sl.size()));
                if (rc != KVX_OK) held.insert(held.end(), sl.begin(), sl.end() - 1);
            } else {
                rc = kvx_tier_invalidate(t, keys.data(), n, &cnt);
                CHECK(rc == KVX_OK && cnt >= 0 && cnt <= n);
            }
            ok += rc == KVX_OK;
            std::vector<int32_t> still;
            for (int32_t s : writing) if (t->e[s].state == TIER_WRITING) still.push_back(s);
            writing.swap(still);
            check_tier(t);
        }
        kvx_tier_info info;
        CHECK(kvx_tier_get_info(t, &info) == KVX_OK);
        CHECK(info.num_slots == S && info.free_slots + info.writing + info.resident == S);
        CHECK(kvx_tier_destroy(t) == KVX_OK);
        CHECK(kvx_tier_lookup(t, nullptr, 0, nullptr, &info.pinned) == KVX_E_STALE);
    }
    std::printf("tier: %d sequences, %d successful operations checked\n", iters, ok);
}

// Rings: random submit / take / complete / reap / discard on one ring from
// both ends, against two deques; then a producer and a consumer thread
// pushing 200000 descriptors through a small ring, in order.
static void fuzz_ring(int iters)
{
    char name[64];
    for (int it = 0; it < iters; it++) {
        std::snprintf(name, sizeof name, "/kvx-fuzz-%d-%d", int(getpid()), it);
        const int32_t entries = 1 << rnd(1, 6);
        kvx_ring *r = nullptr, *o = nullptr;
        CHECK(kvx_ring_create(name, entries, 3, &r) == KVX_OK);
        CHECK(kvx_ring_open(name, &o) == KVX_OK);
        std::deque<uint64_t> sq, cq;
        uint64_t next = 1;
        kvx_sqe q;
        kvx_cqe c;
        for (int step = 0; step < 400; step++) {
            const int op = static_cast<int>(rnd(0, 4));
            int32_t got = 0;
            if (op == 0) {
                std::memset(&q, 0, sizeof q);
                q.op_id = next;
                q.n = static_cast<int32_t>(rnd(0, KVX_RING_MAX_PAGES));
                for (int32_t i = 0; i < q.n; i++) q.page_ids[i] = static_cast<int32_t>(next + i);
                const int rc = kvx_ring_submit(r, &q);
                CHECK((rc == KVX_OK) == (sq.size() < size_t(entries)));
                if (rc == KVX_OK) sq.push_back(next++);
            } else if (op == 1) {
                CHECK(kvx_ring_take(o, &q, &got) == KVX_OK);
                CHECK(got == (sq.empty() ? 0 : 1));
                if (got) {
                    CHECK(q.op_id == sq.front());
                    for (int32_t i = 0; i < q.n; i++) CHECK(q.page_ids[i] == int32_t(q.op_id + i));
                    sq.pop_front();
                    c = kvx_cqe{q.op_id, 3, -static_cast<int32_t>(q.n), 0};
                    if (kvx_ring_complete(o, &c) == KVX_OK) {
                        cq.push_back(q.op_id);
                    } else {
                        CHECK(cq.size() == size_t(entries));
                    }
                }
            } else if (op == 2) {
                kvx_cqe out[8];
                const int32_t max = static_cast<int32_t>(rnd(0, 8));
                CHECK(kvx_ring_reap(r, out, max, &got) == KVX_OK);
                CHECK(got == std::min<int32_t>(max, int32_t(cq.size())));
                for (int32_t i = 0; i < got; i++) {
                    CHECK(out[i].op_id == cq.front() && out[i].generation == 3);
                    cq.pop_front();
                }
            } else if (op == 3 && rnd(0, 9) == 0) {
                CHECK(kvx_ring_discard(o, &got) == KVX_OK);
                CHECK(got == int32_t(sq.size()));
                sq.clear();
            } else {
                int32_t a = 0, b = 0;
                CHECK(kvx_ring_pending(r, &a, &b) == KVX_OK);
                CHECK(a == int32_t(sq.size()) && b == int32_t(cq.size()));
            }
        }
        int32_t alive = 0;
        CHECK(kvx_ring_peer_alive(r, &alive) == KVX_OK && alive == 1);
        CHECK(kvx_ring_close(o) == KVX_OK);
        CHECK(kvx_ring_peer_alive(r, &alive) == KVX_OK && alive == 0);
        CHECK(kvx_ring_close(r) == KVX_OK);
        CHECK(kvx_ring_open(name, &o) == KVX_E_INVAL);   // the name is gone
    }
    // two threads, one per side
    std::snprintf(name, sizeof name, "/kvx-fuzz-%d-threads", int(getpid()));
    kvx_ring *r = nullptr, *o = nullptr;
    CHECK(kvx_ring_create(name, 8, 1, &r) == KVX_OK);
    CHECK(kvx_ring_open(name, &o) == KVX_OK);
    const uint64_t total = 200000;
    std::thread consumer([&] {
        kvx_sqe q;
        uint64_t want = 1;
        while (want <= total) {
            int32_t got = 0;
            CHECK(kvx_ring_take(o, &q, &got) == KVX_OK);
            if (!got) continue;
            CHECK(q.op_id == want && q.n == 1 && q.page_ids[0] == int32_t(want % 1000));
            kvx_cqe c{want, 1, 0, 0};
            while (kvx_ring_complete(o, &c) != KVX_OK) {}
            want++;
        }
    });
    uint64_t sent = 1, reaped = 1;
    kvx_sqe q;
    std::memset(&q, 0, sizeof q);
    while (reaped <= total) {
        if (sent <= total) {
            q.op_id = sent;
            q.n = 1;
            q.page_ids[0] = int32_t(sent % 1000);
            if (kvx_ring_submit(r, &q) == KVX_OK) sent++;
        }
        kvx_cqe out[4];
        int32_t got = 0;
        CHECK(kvx_ring_reap(r, out, 4, &got) == KVX_OK);
        for (int32_t i = 0; i < got; i++) CHECK(out[i].op_id == reaped++);
    }
    consumer.join();
    CHECK(kvx_ring_close(o) == KVX_OK && kvx_ring_close(r) == KVX_OK);
    std::printf("ring: %d random sequences and %llu descriptors across two threads checked\n",
                iters, static_cast<unsigned long long>(total));
}

// The host-link grid policy against its rule, case by case: alone, beside
// calls of the same direction, both directions (shares of 6 and 18 and their
// rounding), beside staged copies, and with the duplex shares switched off.
static void check_link_policy()
{
    struct Case {
        int w, r, dw, dr, dir;
        int64_t dup_w, dup_r;
        int want;
    };
    const int W = kLinkWrites, R = kLinkReads;
    const Case cases[] = {
        {0, 0, 0, 0, W, 6, 18, 32},  {0, 0, 0, 0, R, 6, 18, 32},    // alone
        {1, 0, 0, 0, W, 6, 18, 24},  {3, 0, 0, 0, W, 6, 18, 12},    // same direction only
        {0, 2, 0, 0, R, 6, 18, 16},  {9, 0, 0, 0, W, 6, 18, 8},     // ... at least 8
        {0, 1, 0, 0, W, 6, 18, 6},   {1, 1, 0, 0, W, 6, 18, 3},     // writers beside a reader kernel
        {2, 1, 0, 0, W, 6, 18, 2},   {3, 2, 0, 0, W, 6, 18, 2},     // 6 / 3 = 2, 6 / 4 = 1.5 -> 2
        {6, 1, 0, 0, W, 6, 18, 1},                                  // at least 1
        {1, 0, 0, 0, R, 6, 18, 18},  {1, 1, 0, 0, R, 6, 18, 9},     // readers beside a writer
        {2, 2, 0, 0, R, 6, 18, 6},   {2, 3, 0, 0, R, 6, 18, 5},     // 18 / 4 = 4.5 -> 5
        {0, 0, 1, 0, R, 6, 18, 18},  {0, 1, 2, 0, R, 6, 18, 9},     // readers beside staged backups
        {0, 0, 0, 2, W, 6, 18, 32},  {1, 0, 0, 2, W, 6, 18, 32},    // writers beside staged restores only
        {0, 1, 0, 2, W, 6, 18, 6},                                  // ... and a reader kernel
        {0, 0, 2, 0, W, 6, 18, 16},  {0, 0, 0, 2, R, 6, 18, 16},    // staged calls of its own direction
        {1, 1, 0, 0, W, 0, 18, 16},  {1, 1, 0, 0, R, 6, 0, 16},     // duplex shares off: 48 / 3
        {1, 1, 1, 1, R, 0, 0, 9},    {0, 1, 0, 2, W, 0, 18, 12},
        {1, 1, 0, 0, W, 12, 18, 6},  {1, 1, 0, 0, R, 6, 30, 15},    // other totals
    };
    for (const Case& c : cases) {
        LinkLoad o;
        o.writers = c.w;
        o.readers = c.r;
        o.dma_writers = c.dw;
        o.dma_readers = c.dr;
        const int got = link_grid_for(o, c.dir, c.dup_w, c.dup_r);
        if (got != c.want) {
            std::printf("link policy: writers %d readers %d dma %d/%d dir %d shares %lld/%lld: %d, want %d\n",
                        c.w, c.r, c.dw, c.dr, c.dir, static_cast<long long>(c.dup_w),
                        static_cast<long long>(c.dup_r), got, c.want);
            std::exit(1);
        }
    }
}

int main()
{
    check_link_policy();
    fuzz_extremes();
    fuzz_geometry(20000);
    fuzz_pages(3000);
    fuzz_slots(3000);
    fuzz_tier(300);
    fuzz_ring(100);
    std::printf("host fuzz ok\n");
    return 0;
}
