// pages.cpp - page-ID list validation and run planning (host only).
//
// Operations address the pool by page IDs that the caller allocated ([RFC]
// "Device IPC data path" and "Ownership": BACKUP names source pages the
// scheduler published as safe, RESTORE names destination pages it
// allocated). Slot i of the packed buffer holds page_ids[i], or slot
// host_slots[i] of a slot-addressed host pool ([RFC] "Ownership": the data
// plane owns host KV physical allocation); planning only changes the order
// in which pieces are visited, never where they land.
#include <algorithm>

#include "kvx_host.h"

namespace kvx {

int check_page_ids(const PoolGeom& g, const int32_t* ids, int32_t n, bool reject_dups)
{
    if (n < 0) return fail(KVX_E_RANGE, "page list length is negative");
    if (n > 0 && !ids) return fail(KVX_E_INVAL, "page_ids is NULL");
    for (int32_t i = 0; i < n; i++)
        if (ids[i] < 0 || ids[i] >= g.num_pages)
            return fail(KVX_E_RANGE, "page_ids[" + std::to_string(i) + "] = " +
                                         std::to_string(ids[i]) + " is outside [0, " +
                                         std::to_string(g.num_pages) + ")");
    if (reject_dups && n > 1) {
        std::vector<int32_t> s(ids, ids + n);
        std::sort(s.begin(), s.end());
        auto it = std::adjacent_find(s.begin(), s.end());
        if (it != s.end())
            return fail(KVX_E_DUP, "destination page " + std::to_string(*it) +
                                       " appears more than once; concurrent writes to one page "
                                       "would race");
    }
    return KVX_OK;
}

int check_host_slots(const int32_t* slots, int32_t n, int64_t num_slots, bool reject_dups)
{
    if (n > 0 && !slots) return fail(KVX_E_INVAL, "host_slots is NULL");
    for (int32_t i = 0; i < n; i++)
        if (slots[i] < 0 || slots[i] >= num_slots)
            return fail(KVX_E_RANGE, "host_slots[" + std::to_string(i) + "] = " +
                                         std::to_string(slots[i]) + " is outside [0, " +
                                         std::to_string(num_slots) + ")");
    if (reject_dups && n > 1) {
        std::vector<int32_t> s(slots, slots + n);
        std::sort(s.begin(), s.end());
        auto it = std::adjacent_find(s.begin(), s.end());
        if (it != s.end())
            return fail(KVX_E_DUP, "host slot " + std::to_string(*it) +
                                       " appears more than once; concurrent writes to one slot "
                                       "would race");
    }
    return KVX_OK;
}

void order_pages(const int32_t* ids, int32_t n, bool sorted, std::vector<PageSlot>* out)
{
    order_pairs(ids, nullptr, n, sorted, out);
}

void order_pairs(const int32_t* ids, const int32_t* slots, int32_t n, bool sorted,
                 std::vector<PageSlot>* out)
{
    out->resize(n);
    for (int32_t i = 0; i < n; i++) (*out)[i] = PageSlot{ids[i], slots ? slots[i] : i};
    if (sorted)
        std::stable_sort(out->begin(), out->end(),
                         [](const PageSlot& a, const PageSlot& b) { return a.page < b.page; });
}

void plan_runs(const PoolGeom& g, const std::vector<PageSlot>& pairs, std::vector<Run>* runs)
{
    runs->clear();
    for (const PageSlot& ps : pairs) {
        if (!runs->empty()) {
            Run& r = runs->back();
            // extend when the next pair continues both the page run in the pool
            // (pages adjacent in memory) and the slot run in the packed buffer
            if (g.pages_adjacent && ps.page == r.page + r.count && ps.slot == r.slot + r.count) {
                r.count++;
                continue;
            }
        }
        runs->push_back(Run{ps.page, ps.slot, 1});
    }
}

}  // namespace kvx
