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

// ---------------------------------------------------------------------------
// host-link grid policy (pure; api.cpp counts the calls in flight)
// ---------------------------------------------------------------------------
constexpr int kHostGridAuto = 32;    // default workgroups of a kernel streaming over the host link
constexpr int kHostLinkBudget = 48;  // workgroups that concurrent host-link kernels share
constexpr int kLinkWrites = 1;       // a call's host-link traffic: a kernel writes host memory (zero-copy BACKUP)
constexpr int kLinkReads = 2;        // a kernel reads host memory (zero-copy RESTORE)
constexpr int kLinkDmaWrites = 4;    // copies write host memory (staged BACKUP)
constexpr int kLinkDmaReads = 8;     // copies read host memory (staged RESTORE)

// Host-link calls of other streams in flight on a GPU, by direction
// (BACKUPs write host memory, RESTOREs read it) and by mover (the zero-copy
// kernel, or the staged path's copies).
struct LinkLoad {
    int writers = 0, readers = 0;           // zero-copy kernels
    int dma_writers = 0, dma_readers = 0;   // staged copies
    int all() const { return writers + readers + dma_writers + dma_readers; }
};

// Workgroups of a one-direction kernel over the host link (dir: kLinkWrites
// or kLinkReads), given the other streams' host-link calls in flight. Alone,
// kHostGridAuto (32 x 8 KiB units in flight cover the link's round trip).
// A kernel that reads host memory, beside any call that writes it, and a
// kernel that writes host memory, beside a zero-copy RESTORE kernel, take a
// share of a per-direction total (duplex_writers or duplex_readers) over
// the zero-copy kernels of their own direction, themselves included. A
// kernel that writes host memory beside staged RESTOREs only (whose copies
// read it) takes kHostGridAuto. Else a share of kHostLinkBudget over all
// the calls in flight.
//
// Measured on MI355X (zero-copy, 2 GiB requests of 128 KiB pieces):
//  - alone: backup 22.6 / 33.5 / 44.5 / 55.5 / 56.9 GB/s at 2 / 3 / 4 / 6 /
//    32 workgroups, restore 25.6 / 36.7 / 48.4 / 57.4 / 57.5 at 6 / 9 / 12 /
//    16 / 32: a workgroup writing host memory keeps about 11 GB/s going, one
//    reading it about 4;
//  - both directions at once, backups on one stream and restores on another
//    (workgroups per backup / restore kernel: GB/s both ways): 24 / 24 83.3,
//    8 / 8 52.2, 4 / 16 87.0, 6 / 16 87.3, 6 / 18 98.5-98.7, 7 / 18 99.4,
//    5 / 18 97.1, 6 / 20 91.6, 7 / 21 81.5, 6 / 24 66.5, 4 / 24 59.7: the
//    two directions share the link best when each is held just below what
//    it reaches alone (about 50 GB/s each); a direction given more than that
//    slows the other one far more than it gains;
//  - the mixed stream's 128 requests as separate calls on four streams (two
//    backups and two restores in flight): a share of 48 regardless of
//    direction (12 each) 84.6-84.9, 3 / 9 per kernel 99.1-99.9, 4 / 9 93.7,
//    3 / 8 87.4, 3 / 12 68.2, 2 / 9 82.5;
//  - the same with staged calls in one direction (their copies move that
//    direction; GB/s both ways, the duplex shares on / a share of 48):
//    zero-copy restores beside staged backups 98.6-98.8 / 69.6, zero-copy
//    backups beside staged restores 66.1 / 82.1, and at 6 / 8 / 16 / 24 /
//    32 workgroups a backup kernel 69.8 / 77.6 / 84.7 / 90.5 / 92.5: kernels
//    that read host memory need holding back beside the copies' writes too,
//    while kernels that write it beside the copies' reads do best with a
//    full grid.
// A kernel keeps the grid it was launched with: one sized beside calls that
// then finish runs on at its share (a share of 6 writers still moves 55
// GB/s alone, of 18 readers 57; half of either about 35).
inline int link_grid_for(const LinkLoad& o, int dir, int64_t duplex_writers, int64_t duplex_readers)
{
    const int same = dir == kLinkWrites ? o.writers : o.readers;
    const int opp = dir == kLinkWrites ? o.readers : o.writers + o.dma_writers;
    const int64_t total = dir == kLinkWrites ? duplex_writers : duplex_readers;
    if (dir == kLinkWrites && opp == 0 && o.dma_readers > 0 && total > 0) return kHostGridAuto;
    if (opp == 0 || total <= 0) {
        const int share = kHostLinkBudget / (o.all() + 1);
        return share < 8 ? 8 : share > kHostGridAuto ? kHostGridAuto : share;
    }
    // total / (same + 1), rounded to the nearest, at least 1
    const int64_t share = (2 * total + same + 1) / (2 * (same + 1));
    return static_cast<int>(share < 1 ? 1 : share);
}

}  // namespace kvx
