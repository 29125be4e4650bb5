// tier_policy.cpp - the host tier's policy calls (kvx_tier_backup,
// kvx_tier_restore, kvx_tier_exchange): the tier's bookkeeping (tier.cpp)
// and the slot transfers, under the tier's lock, all or nothing
// ([RFC] "Ownership": the data plane owns host KV physical allocation while
// backup decisions stay with the scheduler).
#include <vector>

#include "kvx_internal.h"
#include "tier.h"

using namespace kvx;
using kvx::TierEntry;

extern "C" {

// ---- host-tier policy calls --------------------------------------------------

namespace {

// Tier handle check and its generation against the pool's.
int tier_for_pool(kvx_tier* tier, const kvx_pool* pool, const char* op)
{
    if (!tier_known(tier)) return fail(KVX_E_INVAL, std::string(op) + ": unknown tier handle");
    if (!tier->live.load()) return fail(KVX_E_STALE, std::string(op) + ": tier was destroyed");
    if (!pool_known(pool)) return fail(KVX_E_INVAL, std::string(op) + ": unknown pool handle");
    if (!pool->live.load()) return fail(KVX_E_STALE, std::string(op) + ": pool handle was unregistered");
    if (tier->generation != pool->generation)
        return fail(KVX_E_STALE, std::string(op) + ": tier generation " +
                                     std::to_string(tier->generation) +
                                     " does not match pool generation " +
                                     std::to_string(pool->generation));
    return KVX_OK;
}

}  // namespace

int kvx_tier_backup(kvx_tier* tier, kvx_pool* pool, const uint64_t* keys, const int32_t* page_ids,
                    int32_t n, void* host_pool, uint64_t host_pool_bytes, void* stream,
                    int32_t path, int32_t* slots, uint64_t* evicted, int32_t* num_evicted)
{
    const TraceRange tr("kvx_tier_backup");
    clear_error();
    int rc = tier_for_pool(tier, pool, "tier_backup");
    if (rc != KVX_OK) return rc;
    rc = check_page_ids(pool->geom, page_ids, n, false);
    if (rc != KVX_OK) return rc;
    std::lock_guard<std::mutex> lk(tier->mu);
    if (!tier->live.load()) return fail(KVX_E_STALE, "tier_backup: tier was destroyed");
    tier->begin();
    rc = tier->reserve(keys, n, slots, evicted, num_evicted);
    if (rc != KVX_OK) {
        tier->rollback();
        return rc;
    }
    std::vector<int32_t> ids, sl;
    for (int32_t i = 0; i < n; i++)
        if (slots[i] >= 0) {
            ids.push_back(page_ids[i]);
            sl.push_back(slots[i]);
        }
    rc = kvx_backup_slots(pool, ids.data(), sl.data(), static_cast<int32_t>(ids.size()), host_pool,
                          host_pool_bytes, static_cast<int32_t>(tier->e.size()), 0,
                          static_cast<int32_t>(pool->geom.num_layers), stream, path);
    if (rc != KVX_OK && rc != KVX_E_HIP) {
        // refused before anything was enqueued: the tier as before the call,
        // evicted entries included
        tier->rollback();
        for (int32_t i = 0; i < n; i++) slots[i] = -1;
        *num_evicted = 0;
        return rc;
    }
    if (rc != KVX_OK) {
        // a launch failed part way: the reserved slots may hold part of a
        // backup, so they are freed and the evictions stand (still reported)
        tier->end();
        for (int32_t i = 0; i < n; i++)
            if (slots[i] >= 0) tier->set(slots[i], TierEntry());
        for (int32_t i = 0; i < n; i++) slots[i] = -1;
        return rc;
    }
    tier->end();
    return KVX_OK;
}

int kvx_tier_restore(kvx_tier* tier, kvx_pool* pool, const uint64_t* keys, const int32_t* page_ids,
                     int32_t n, const void* host_pool, uint64_t host_pool_bytes,
                     kvx_ready* ready, int32_t slot_base, void* stream, int32_t path,
                     int32_t* slots, int32_t* hits)
{
    const TraceRange tr("kvx_tier_restore");
    clear_error();
    int rc = tier_for_pool(tier, pool, "tier_restore");
    if (rc != KVX_OK) return rc;
    rc = check_page_ids(pool->geom, page_ids, n, true);
    if (rc != KVX_OK) return rc;
    std::lock_guard<std::mutex> lk(tier->mu);
    if (!tier->live.load()) return fail(KVX_E_STALE, "tier_restore: tier was destroyed");
    tier->begin();
    rc = tier->lookup(keys, n, slots, hits);
    if (rc != KVX_OK) {
        tier->rollback();
        return rc;
    }
    std::vector<int32_t> ids, sl;
    for (int32_t i = 0; i < n; i++)
        if (slots[i] >= 0) {
            ids.push_back(page_ids[i]);
            sl.push_back(slots[i]);
        }
    rc = kvx_restore_slots(pool, host_pool, host_pool_bytes, static_cast<int32_t>(tier->e.size()),
                           sl.data(), ids.data(), static_cast<int32_t>(ids.size()), 0,
                           static_cast<int32_t>(pool->geom.num_layers), ready, slot_base, stream,
                           path);
    if (rc != KVX_OK) {
        tier->rollback();   // pins and recency as before the call
        for (int32_t i = 0; i < n; i++) slots[i] = -1;
        *hits = 0;
        return rc;
    }
    tier->end();
    return KVX_OK;
}

int kvx_tier_exchange(kvx_tier* tier, kvx_pool* pool, const uint64_t* backup_keys,
                      const int32_t* backup_pages, int32_t nb, const uint64_t* restore_keys,
                      const int32_t* restore_pages, int32_t nr, void* host_pool,
                      uint64_t host_pool_bytes, kvx_ready* ready, int32_t slot_base, void* stream,
                      int32_t path, int32_t* backup_slots, uint64_t* evicted, int32_t* num_evicted,
                      int32_t* restore_slots, int32_t* hits)
{
    const TraceRange tr("kvx_tier_exchange");
    clear_error();
    int rc = tier_for_pool(tier, pool, "tier_exchange");
    if (rc != KVX_OK) return rc;
    rc = check_page_ids(pool->geom, backup_pages, nb, false);
    if (rc != KVX_OK) return rc;
    rc = check_page_ids(pool->geom, restore_pages, nr, true);
    if (rc != KVX_OK) return rc;
    std::lock_guard<std::mutex> lk(tier->mu);
    if (!tier->live.load()) return fail(KVX_E_STALE, "tier_exchange: tier was destroyed");
    tier->begin();
    // hits first: pinned, they cannot be the reservation's victims
    rc = tier->lookup(restore_keys, nr, restore_slots, hits);
    if (rc == KVX_OK) rc = tier->reserve(backup_keys, nb, backup_slots, evicted, num_evicted);
    if (rc != KVX_OK) {
        tier->rollback();
        return rc;
    }
    std::vector<int32_t> bi, bs, ri, rs;
    for (int32_t i = 0; i < nb; i++)
        if (backup_slots[i] >= 0) {
            bi.push_back(backup_pages[i]);
            bs.push_back(backup_slots[i]);
        }
    for (int32_t i = 0; i < nr; i++)
        if (restore_slots[i] >= 0) {
            ri.push_back(restore_pages[i]);
            rs.push_back(restore_slots[i]);
        }
    const int32_t S = static_cast<int32_t>(tier->e.size());
    const int32_t L = static_cast<int32_t>(pool->geom.num_layers);
    const kvx_xfer_slots xb{bi.data(), bs.data(), static_cast<int32_t>(bi.size()), S, host_pool,
                            host_pool_bytes, 0, L};
    const kvx_xfer_slots xr{ri.data(), rs.data(), static_cast<int32_t>(ri.size()), S, host_pool,
                            host_pool_bytes, 0, L};
    rc = kvx_exchange_slots(pool, &xb, &xr, ready, slot_base, stream, path);
    if (rc != KVX_OK && rc != KVX_E_HIP) {
        tier->rollback();   // refused before anything was enqueued
        for (int32_t i = 0; i < nb; i++) backup_slots[i] = -1;
        for (int32_t i = 0; i < nr; i++) restore_slots[i] = -1;
        *num_evicted = 0;
        *hits = 0;
        return rc;
    }
    if (rc != KVX_OK) {
        // a launch failed part way: free the reservations (they may hold part
        // of a backup) and drop the pins; the evictions stand
        tier->end();
        for (int32_t i = 0; i < nb; i++)
            if (backup_slots[i] >= 0) tier->set(backup_slots[i], TierEntry());
        (void)tier->release(restore_slots, nr);
        for (int32_t i = 0; i < nb; i++) backup_slots[i] = -1;
        for (int32_t i = 0; i < nr; i++) restore_slots[i] = -1;
        *hits = 0;
        return rc;
    }
    tier->end();
    return KVX_OK;
}

}  // extern "C"
