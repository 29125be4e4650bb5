// kvx_host.h - host-only declarations of the kvx runtime: errors, the pool
// geometry and its validator, page-list checks and run planning. Includes
// no HIP header, so these parts also build with a plain host compiler (the
// sanitizer tests do that). Not part of the ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "kvx.h"

namespace kvx {

// ---------------------------------------------------------------------------
// errors and logging
// ---------------------------------------------------------------------------
int fail(int code, const std::string& msg);   // records the thread's message, returns code
void clear_error();
void log_warn(const std::string& msg);
void log_info(const std::string& msg);


// ---------------------------------------------------------------------------
// pool geometry (derived and validated at registration; host only)
// ---------------------------------------------------------------------------
struct PoolGeom {
    int64_t num_pages = 0, num_layers = 0, num_kv = 0, page_size = 0, num_heads = 0,
            head_dim = 0;
    int32_t inner = KVX_NHD;
    int32_t outer[3] = {0, 1, 2};
    int64_t dtype_bytes = 0;
    int64_t row_bytes = 0, piece_bytes = 0, pool_bytes = 0;
    int64_t page_stride = 0, layer_stride = 0, kv_stride = 0;   // bytes
    bool pages_adjacent = false;   // page_stride == piece_bytes
};

// Validates layout + tensor view; fills geom. Host only, calls no HIP API.
int derive_geometry(const kvx_layout* layout, const void* base, uint64_t byte_offset,
                    uint32_t dtype_bytes, int32_t ndim, const int64_t* shape,
                    const int64_t* stride, PoolGeom* geom);

// ---------------------------------------------------------------------------
// page lists (host only)
// ---------------------------------------------------------------------------
struct PageSlot {
    int32_t page, slot;
};
struct Run {
    int32_t page, slot, count;
};
int check_page_ids(const PoolGeom& g, const int32_t* ids, int32_t n, bool reject_dups);
// Pairs (page, slot) in visiting order: sorted by page when `sorted`, else
// caller order.
void order_pages(const int32_t* ids, int32_t n, bool sorted, std::vector<PageSlot>* out);
// As order_pages with slot slots[i] for page ids[i] (slots == NULL: slot i).
void order_pairs(const int32_t* ids, const int32_t* slots, int32_t n, bool sorted,
                 std::vector<PageSlot>* out);
// Host slots in [0, num_slots); with reject_dups, distinct (KVX_E_DUP).
int check_host_slots(const int32_t* slots, int32_t n, int64_t num_slots, bool reject_dups);
void plan_runs(const PoolGeom& g, const std::vector<PageSlot>& sorted_pairs,
               std::vector<Run>* runs);

constexpr int kVecBytes = 16;        // one dwordx4 per lane access

}  // namespace kvx
