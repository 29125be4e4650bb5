// tier.cpp - host-tier slot allocator and residency protocol (host only).
//
// The data plane owns the host KV physical allocation while the scheduler's
// cache index stays authoritative for cache semantics ([RFC] "Ownership",
// which leaves open how the two sides then agree on when a page's host copy
// exists). The rules here make every answer current:
//   - a backup first reserves slots (WRITING: invisible to lookups, never
//     evicted) and commits them once its bytes have landed;
//   - a restore looks keys up, which pins their slots until it releases
//     them; a pinned slot is never evicted or reused;
//   - a full tier evicts the least recently used unpinned resident entry
//     and reports its key to the caller that caused the eviction;
//   - invalidation hides a key at once and frees its slot when the last pin
//     or the backup in flight ends.
// Every operation checks all of its arguments before it changes anything.
#include <algorithm>
#include <map>
#include <string>
#include <unordered_set>

#include "tier.h"

using kvx::TierEntry;

kvx_tier::kvx_tier(int32_t num_slots, uint64_t gen) : generation(gen), e(num_slots)
{
    for (int32_t s = 0; s < num_slots; s++) free_slots.insert(free_slots.end(), s);
}

void kvx_tier::detach(int32_t s)
{
    const TierEntry& x = e[s];
    if (x.state == kvx::TIER_FREE) {
        free_slots.erase(s);
        return;
    }
    if (!x.doomed) where.erase(x.key);
    if (x.state == kvx::TIER_RESIDENT && x.pins == 0 && !x.doomed) lru.erase({x.last, s});
}

void kvx_tier::attach(int32_t s)
{
    const TierEntry& x = e[s];
    if (x.state == kvx::TIER_FREE) {
        free_slots.insert(s);
        return;
    }
    if (!x.doomed) where[x.key] = s;
    if (x.state == kvx::TIER_RESIDENT && x.pins == 0 && !x.doomed) lru.insert({x.last, s});
}

void kvx_tier::set(int32_t s, const TierEntry& v)
{
    if (logging) saved.emplace_back(s, e[s]);
    detach(s);
    e[s] = v;
    attach(s);
}

void kvx_tier::begin()
{
    logging = true;
    saved.clear();
    saved_clock = clock;
    saved_evictions = evictions;
}

void kvx_tier::end()
{
    logging = false;
    saved.clear();
}

void kvx_tier::rollback()
{
    logging = false;
    for (auto it = saved.rbegin(); it != saved.rend(); ++it) {
        detach(it->first);
        e[it->first] = it->second;
        attach(it->first);
    }
    saved.clear();
    clock = saved_clock;
    evictions = saved_evictions;
}

namespace {

int check_list(const void* p, int32_t n, const char* op, const char* what)
{
    if (n < 0) return kvx::fail(KVX_E_RANGE, std::string(op) + ": negative length");
    if (n > 0 && !p) return kvx::fail(KVX_E_INVAL, std::string(op) + ": " + what + " is NULL");
    return KVX_OK;
}

}  // namespace

int kvx_tier::reserve(const uint64_t* keys, int32_t n, int32_t* slots, uint64_t* evicted,
                      int32_t* num_evicted)
{
    int rc = check_list(keys, n, "tier_reserve", "keys");
    if (rc != KVX_OK) return rc;
    if (n > 0 && (!slots || !evicted))
        return kvx::fail(KVX_E_INVAL, "tier_reserve: slots or evicted is NULL");
    if (!num_evicted) return kvx::fail(KVX_E_INVAL, "tier_reserve: num_evicted is NULL");
    // keys present at the start are touched, never evicted by this call
    std::unordered_set<uint64_t> fresh;
    std::unordered_set<int32_t> kept;
    int64_t protected_evictable = 0;
    for (int32_t i = 0; i < n; i++) {
        auto it = where.find(keys[i]);
        if (it == where.end()) {
            fresh.insert(keys[i]);
        } else if (kept.insert(it->second).second) {
            const TierEntry& x = e[it->second];
            if (x.state == kvx::TIER_RESIDENT && x.pins == 0) protected_evictable++;
        }
    }
    const int64_t room = int64_t(free_slots.size()) + int64_t(lru.size()) - protected_evictable;
    if (int64_t(fresh.size()) > room)
        return kvx::fail(KVX_E_FULL, "tier_reserve: " + std::to_string(fresh.size()) +
                                         " new keys but only " + std::to_string(free_slots.size()) +
                                         " free and " + std::to_string(lru.size() - protected_evictable) +
                                         " evictable slots");
    *num_evicted = 0;
    for (int32_t i = 0; i < n; i++) {
        auto it = where.find(keys[i]);
        if (it != where.end()) {
            TierEntry x = e[it->second];
            x.last = ++clock;
            slots[i] = -1;
            set(it->second, x);
            continue;
        }
        int32_t s;
        if (!free_slots.empty()) {
            s = *free_slots.begin();
        } else {
            auto v = lru.begin();
            while (kept.count(v->second)) ++v;   // room was counted: a victim exists
            s = v->second;
            evicted[(*num_evicted)++] = e[s].key;
            evictions++;
        }
        TierEntry x;
        x.key = keys[i];
        x.state = kvx::TIER_WRITING;
        x.last = ++clock;
        set(s, x);
        slots[i] = s;
    }
    return KVX_OK;
}

int kvx_tier::check_writing(const int32_t* slots, int32_t n, const char* op) const
{
    int rc = check_list(slots, n, op, "slots");
    if (rc != KVX_OK) return rc;
    std::unordered_set<int32_t> seen;
    for (int32_t i = 0; i < n; i++) {
        const int32_t s = slots[i];
        if (s == -1) continue;
        if (s < 0 || s >= int32_t(e.size()))
            return kvx::fail(KVX_E_RANGE, std::string(op) + ": slots[" + std::to_string(i) + "] = " +
                                              std::to_string(s) + " is outside [0, " +
                                              std::to_string(e.size()) + ")");
        if (e[s].state != kvx::TIER_WRITING)
            return kvx::fail(KVX_E_INVAL, std::string(op) + ": slot " + std::to_string(s) +
                                              " has no backup in flight");
        if (!seen.insert(s).second)
            return kvx::fail(KVX_E_INVAL, std::string(op) + ": slot " + std::to_string(s) +
                                              " is named twice");
    }
    return KVX_OK;
}

int kvx_tier::commit(const int32_t* slots, int32_t n)
{
    int rc = check_writing(slots, n, "tier_commit");
    if (rc != KVX_OK) return rc;
    for (int32_t i = 0; i < n; i++) {
        const int32_t s = slots[i];
        if (s == -1) continue;
        TierEntry x = e[s];
        if (x.doomed) {
            x = TierEntry();
        } else {
            x.state = kvx::TIER_RESIDENT;
            x.last = ++clock;
        }
        set(s, x);
    }
    return KVX_OK;
}

int kvx_tier::abort(const int32_t* slots, int32_t n)
{
    int rc = check_writing(slots, n, "tier_abort");
    if (rc != KVX_OK) return rc;
    for (int32_t i = 0; i < n; i++)
        if (slots[i] != -1) set(slots[i], TierEntry());
    return KVX_OK;
}

int kvx_tier::lookup(const uint64_t* keys, int32_t n, int32_t* slots, int32_t* hits)
{
    int rc = check_list(keys, n, "tier_lookup", "keys");
    if (rc != KVX_OK) return rc;
    if (n > 0 && !slots) return kvx::fail(KVX_E_INVAL, "tier_lookup: slots is NULL");
    if (!hits) return kvx::fail(KVX_E_INVAL, "tier_lookup: hits is NULL");
    *hits = 0;
    for (int32_t i = 0; i < n; i++) {
        auto it = where.find(keys[i]);
        if (it == where.end() || e[it->second].state != kvx::TIER_RESIDENT) {
            slots[i] = -1;
            continue;
        }
        TierEntry x = e[it->second];
        x.pins++;
        x.last = ++clock;
        slots[i] = it->second;
        set(it->second, x);
        (*hits)++;
    }
    return KVX_OK;
}

int kvx_tier::release(const int32_t* slots, int32_t n)
{
    int rc = check_list(slots, n, "tier_release", "slots");
    if (rc != KVX_OK) return rc;
    std::map<int32_t, int32_t> times;
    for (int32_t i = 0; i < n; i++) {
        const int32_t s = slots[i];
        if (s == -1) continue;
        if (s < 0 || s >= int32_t(e.size()))
            return kvx::fail(KVX_E_RANGE, "tier_release: slots[" + std::to_string(i) + "] = " +
                                              std::to_string(s) + " is outside [0, " +
                                              std::to_string(e.size()) + ")");
        times[s]++;
    }
    for (const auto& st : times)
        if (e[st.first].state != kvx::TIER_RESIDENT || e[st.first].pins < st.second)
            return kvx::fail(KVX_E_INVAL, "tier_release: slot " + std::to_string(st.first) +
                                              " is released " + std::to_string(st.second) +
                                              " times but holds " + std::to_string(e[st.first].pins) +
                                              " pins");
    for (int32_t i = 0; i < n; i++) {
        const int32_t s = slots[i];
        if (s == -1) continue;
        TierEntry x = e[s];
        x.pins--;
        if (x.pins == 0 && x.doomed) x = TierEntry();
        set(s, x);
    }
    return KVX_OK;
}

int kvx_tier::invalidate(const uint64_t* keys, int32_t n, int32_t* num_dropped)
{
    int rc = check_list(keys, n, "tier_invalidate", "keys");
    if (rc != KVX_OK) return rc;
    if (!num_dropped) return kvx::fail(KVX_E_INVAL, "tier_invalidate: num_dropped is NULL");
    *num_dropped = 0;
    for (int32_t i = 0; i < n; i++) {
        auto it = where.find(keys[i]);
        if (it == where.end()) continue;
        const int32_t s = it->second;
        TierEntry x = e[s];
        if (x.state == kvx::TIER_RESIDENT && x.pins == 0)
            x = TierEntry();
        else
            x.doomed = true;
        set(s, x);
        (*num_dropped)++;
    }
    return KVX_OK;
}

// ---------------------------------------------------------------------------
// handles and the C entry points
// ---------------------------------------------------------------------------
namespace {

// Handles stay registered after destruction (so later calls fail as STALE);
// the registry itself is never destroyed, so a call made while the process
// exits still finds it.
std::mutex g_tier_mu;
std::set<const kvx_tier*>& tiers()
{
    static auto* s = new std::set<const kvx_tier*>();
    return *s;
}

// The tier behind a handle, or an error (unknown or destroyed handle).
int open_tier(const kvx_tier* t, const char* op)
{
    kvx::clear_error();
    if (!kvx::tier_known(t)) return kvx::fail(KVX_E_INVAL, std::string(op) + ": unknown tier handle");
    if (!t->live.load()) return kvx::fail(KVX_E_STALE, std::string(op) + ": tier was destroyed");
    return KVX_OK;
}

}  // namespace

namespace kvx {
bool tier_known(const kvx_tier* t)
{
    std::lock_guard<std::mutex> lk(g_tier_mu);
    return t && tiers().count(t) && t->magic == TIER_MAGIC;
}
}  // namespace kvx

extern "C" {

int kvx_tier_create(int32_t num_slots, uint64_t generation, kvx_tier** out)
{
    kvx::clear_error();
    if (!out) return kvx::fail(KVX_E_INVAL, "tier_create: out is NULL");
    *out = nullptr;
    if (num_slots < 0) return kvx::fail(KVX_E_RANGE, "tier_create: negative num_slots");
    kvx_tier* t = nullptr;
    try {
        t = new kvx_tier(num_slots, generation);
    } catch (...) {
        return kvx::fail(KVX_E_NOMEM, "tier_create: cannot allocate " + std::to_string(num_slots) +
                                          " slots");
    }
    std::lock_guard<std::mutex> lk(g_tier_mu);
    tiers().insert(t);
    *out = t;
    return KVX_OK;
}

int kvx_tier_destroy(kvx_tier* t)
{
    kvx::clear_error();
    if (!t) return KVX_OK;
    {
        std::lock_guard<std::mutex> lk(g_tier_mu);
        if (!tiers().count(t) || t->magic != kvx::TIER_MAGIC) {
            kvx::log_warn("tier_destroy: unknown or already destroyed tier handle");
            return KVX_OK;
        }
        // the handle stays registered (stale) so later calls fail as STALE
        if (!t->live.exchange(false)) {
            kvx::log_warn("tier_destroy: tier already destroyed");
            return KVX_OK;
        }
    }
    std::lock_guard<std::mutex> lk(t->mu);
    std::vector<kvx::TierEntry>().swap(t->e);
    std::set<int32_t>().swap(t->free_slots);
    std::unordered_map<uint64_t, int32_t>().swap(t->where);
    std::set<std::pair<uint64_t, int32_t>>().swap(t->lru);
    std::vector<std::pair<int32_t, kvx::TierEntry>>().swap(t->saved);
    return KVX_OK;
}

#define KVX_TIER_CALL(op, call)                       \
    int rc_ = open_tier(tier, op);                    \
    if (rc_ != KVX_OK) return rc_;                    \
    std::lock_guard<std::mutex> lk_(tier->mu);        \
    if (!tier->live.load()) return kvx::fail(KVX_E_STALE, std::string(op) + ": tier was destroyed"); \
    return tier->call;

int kvx_tier_reserve(kvx_tier* tier, const uint64_t* keys, int32_t n, int32_t* slots,
                     uint64_t* evicted, int32_t* num_evicted)
{
    KVX_TIER_CALL("tier_reserve", reserve(keys, n, slots, evicted, num_evicted))
}

int kvx_tier_commit(kvx_tier* tier, const int32_t* slots, int32_t n)
{
    KVX_TIER_CALL("tier_commit", commit(slots, n))
}

int kvx_tier_abort(kvx_tier* tier, const int32_t* slots, int32_t n)
{
    KVX_TIER_CALL("tier_abort", abort(slots, n))
}

int kvx_tier_lookup(kvx_tier* tier, const uint64_t* keys, int32_t n, int32_t* slots, int32_t* hits)
{
    KVX_TIER_CALL("tier_lookup", lookup(keys, n, slots, hits))
}

int kvx_tier_release(kvx_tier* tier, const int32_t* slots, int32_t n)
{
    KVX_TIER_CALL("tier_release", release(slots, n))
}

int kvx_tier_invalidate(kvx_tier* tier, const uint64_t* keys, int32_t n, int32_t* num_dropped)
{
    KVX_TIER_CALL("tier_invalidate", invalidate(keys, n, num_dropped))
}

#undef KVX_TIER_CALL

int kvx_tier_get_info(const kvx_tier* tier, kvx_tier_info* info)
{
    int rc = open_tier(tier, "tier_get_info");
    if (rc != KVX_OK) return rc;
    if (!info) return kvx::fail(KVX_E_INVAL, "tier_get_info: info is NULL");
    kvx_tier* t = const_cast<kvx_tier*>(tier);
    std::lock_guard<std::mutex> lk(t->mu);
    kvx_tier_info o{};
    o.num_slots = static_cast<int32_t>(t->e.size());
    o.free_slots = static_cast<int32_t>(t->free_slots.size());
    for (const kvx::TierEntry& x : t->e) {
        o.writing += x.state == kvx::TIER_WRITING;
        o.resident += x.state == kvx::TIER_RESIDENT;
        o.pinned += x.state == kvx::TIER_RESIDENT && x.pins > 0;
        o.doomed += x.doomed;
    }
    o.evictions = t->evictions;
    o.generation = t->generation;
    *info = o;
    return KVX_OK;
}

int kvx_tier_slot(const kvx_tier* tier, int32_t slot, uint64_t* key, int32_t* state, int32_t* pins)
{
    int rc = open_tier(tier, "tier_slot");
    if (rc != KVX_OK) return rc;
    if (!key || !state || !pins) return kvx::fail(KVX_E_INVAL, "tier_slot: NULL output");
    kvx_tier* t = const_cast<kvx_tier*>(tier);
    std::lock_guard<std::mutex> lk(t->mu);
    if (slot < 0 || slot >= int32_t(t->e.size()))
        return kvx::fail(KVX_E_RANGE, "tier_slot: slot " + std::to_string(slot) + " is outside [0, " +
                                          std::to_string(t->e.size()) + ")");
    *key = t->e[slot].key;
    *state = t->e[slot].state;
    *pins = t->e[slot].pins;
    return KVX_OK;
}

}  // extern "C"
