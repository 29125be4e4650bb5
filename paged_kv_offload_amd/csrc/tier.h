// tier.h - the host tier's slot allocator and residency bookkeeping (host
// only, no HIP). The C entry points are declared in kvx.h; this header gives
// the runtime's own code (kvx_tier_backup / kvx_tier_restore) the lock and
// the undo log that make those two calls all-or-nothing.
#pragma once

#include <atomic>
#include <cstdint>
#include <mutex>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "kvx_host.h"

namespace kvx {

constexpr uint32_t TIER_MAGIC = 0x6b767874u;   // "kvxt"

enum TierState : int32_t { TIER_FREE = 0, TIER_WRITING = 1, TIER_RESIDENT = 2 };

struct TierEntry {
    uint64_t key = 0;
    int32_t state = TIER_FREE;
    int32_t pins = 0;
    bool doomed = false;     // invalidated; freed when the last pin or the backup ends
    uint64_t last = 0;       // clock value of the last touch
};

}  // namespace kvx

struct kvx_tier {
    uint32_t magic = kvx::TIER_MAGIC;
    std::atomic<bool> live{true};
    uint64_t generation = 0;
    std::mutex mu;

    // Each structure below is a function of the entries: `free_slots` holds
    // the FREE slots, `where` maps the key of every entry that is not FREE
    // and not doomed to its slot, `lru` holds (last, slot) of every RESIDENT
    // entry with no pin that is not doomed (the evictable ones).
    std::vector<kvx::TierEntry> e;
    std::set<int32_t> free_slots;
    std::unordered_map<uint64_t, int32_t> where;
    std::set<std::pair<uint64_t, int32_t>> lru;
    uint64_t clock = 0;
    uint64_t evictions = 0;

    // undo log of one transaction (begin .. commit_txn / rollback)
    bool logging = false;
    std::vector<std::pair<int32_t, kvx::TierEntry>> saved;
    uint64_t saved_clock = 0, saved_evictions = 0;

    explicit kvx_tier(int32_t num_slots, uint64_t gen);

    void detach(int32_t s);                          // drop slot s from the structures
    void attach(int32_t s);                          // insert slot s as its entry says
    void set(int32_t s, const kvx::TierEntry& v);    // replace an entry (logged)

    void begin();
    void end();
    void rollback();

    // The operations of kvx.h, called with `mu` held. Every check comes
    // first; an operation that fails has changed nothing.
    int reserve(const uint64_t* keys, int32_t n, int32_t* slots, uint64_t* evicted,
                int32_t* num_evicted);
    int commit(const int32_t* slots, int32_t n);
    int abort(const int32_t* slots, int32_t n);
    int lookup(const uint64_t* keys, int32_t n, int32_t* slots, int32_t* hits);
    int release(const int32_t* slots, int32_t n);
    int invalidate(const uint64_t* keys, int32_t n, int32_t* num_dropped);

private:
    int check_writing(const int32_t* slots, int32_t n, const char* op) const;
};

namespace kvx {
bool tier_known(const kvx_tier* t);
}  // namespace kvx
