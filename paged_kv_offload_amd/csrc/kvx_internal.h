// kvx_internal.h - shared declarations of the kvx runtime (host side) and the
// kernel launchers. Not part of the ABI.
#pragma once

#include <atomic>
#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "kvx.h"

namespace kvx {

// ---------------------------------------------------------------------------
// errors and logging
// ---------------------------------------------------------------------------
int fail(int code, const std::string& msg);   // records the thread's message, returns code
void clear_error();
void log_warn(const std::string& msg);
void log_info(const std::string& msg);
int hip_fail(hipError_t e, const char* what);  // KVX_E_HIP with the runtime's message

#define KVX_HIP(call)                                   \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

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
void plan_runs(const PoolGeom& g, const std::vector<PageSlot>& sorted_pairs,
               std::vector<Run>* runs);

// ---------------------------------------------------------------------------
// handles
// ---------------------------------------------------------------------------
constexpr uint32_t POOL_MAGIC = 0x6b767870u;    // "kvxp"
constexpr uint32_t READY_MAGIC = 0x6b767872u;   // "kvxr"

}  // namespace kvx

struct kvx_pool {
    uint32_t magic = kvx::POOL_MAGIC;
    std::atomic<bool> live{true};
    kvx::PoolGeom geom;
    uint8_t* base = nullptr;
    uint64_t byte_offset = 0;
    uint8_t* start = nullptr;   // base + byte_offset (device)
    uint64_t generation = 0;
    int device = -1;            // resolved at first data call
    std::mutex mu;
    std::map<hipStream_t, hipEvent_t> last_op;   // per caller stream: end of our last op
};

struct kvx_ready {
    uint32_t magic = kvx::READY_MAGIC;
    std::atomic<bool> live{true};
    int32_t num_slots = 0;
    uint64_t generation = 0;
    uint32_t* counts = nullptr;      // host view (fine-grained pinned)
    uint32_t* counts_dev = nullptr;  // device view of the same memory
};

namespace kvx {

bool pool_known(const kvx_pool* p);
bool ready_known(const kvx_ready* r);

// ---------------------------------------------------------------------------
// tuning
// ---------------------------------------------------------------------------
struct Tuning {
    int64_t grid_max = 0;                 // 0 = auto
    int64_t stage_slot_bytes = 128ll << 20;
    int64_t stage_slots = 3;
    int64_t sort_pages = 0;
    int64_t nontemporal = -1;             // bit 0 loads, bit 1 stores; -1 = auto
    int64_t restore_chunk_layers = 0;     // 0 = auto (chunks of >= kRestoreChunkMin bytes)
    int64_t host_grid_max = 0;            // 0 = auto
    int64_t unit_order = -1;              // MoveArgs::unit_order bits, -1 = auto
    int64_t max_unroll = 16;              // largest 16-byte vectors per lane per unit
    int64_t staged_dma_on_caller = 0;     // staged DMA on the caller's stream instead of a side stream
};
Tuning tuning();

// ---------------------------------------------------------------------------
// kernel launch interface
// ---------------------------------------------------------------------------
constexpr int kThreads = 256;        // 4 wave64 per workgroup
constexpr int kVecBytes = 16;        // one dwordx4 per lane access
constexpr int kMaxPairs = 448;       // (page, slot) pairs carried in the kernel arguments
constexpr int kHostGridAuto = 32;    // default workgroups of a kernel streaming over the host link
constexpr int64_t kRestoreChunkMin = 32ll << 20;   // default minimum staged restore chunk

enum Dir : int32_t { GATHER = 0, SCATTER = 1 };

// One launch moves pieces (page, layer, kv) for layers [layer_begin,
// layer_begin + num_layers), every kv, and the `npairs` (page, slot) pairs.
struct MoveArgs {
    uint8_t* pool;           // pool start (base + byte_offset)
    uint8_t* packed;         // packed buffer holding layers >= pk_layer0, slots >= pk_slot0
    int64_t page_stride, layer_stride, kv_stride;   // pool byte strides
    int64_t pk_lc_stride;    // packed bytes per (layer, kv) = pk_slots * piece_bytes
    int32_t pk_layer0, pk_slot0;
    uint32_t piece_bytes;
    uint32_t chunk_bytes;    // bytes of one work unit (kThreads * 16 * unroll)
    uint32_t chunks_per_piece;
    int32_t layer_begin;
    uint32_t num_kv;
    uint32_t npairs;
    uint32_t total_units;    // num_layers * num_kv * npairs * chunks_per_piece
    // pool HND <-> packed NHD permutation (unused for NHD pools)
    uint32_t T, H, row_vec;              // row_vec = row_bytes / 16
    uint32_t mg_row_vec, mg_H, mg_T;     // magic multipliers (0 means divisor 1)
    // per-layer publish (RESTORE with a ready object)
    uint32_t* layer_done;    // device counters, indexed by absolute layer
    uint32_t* ready;         // device view of counts + slot_base, indexed by layer
    uint32_t layer_target;   // work units of one layer over the whole call
    uint32_t publish_value;  // n
    uint32_t unit_order;     // bit 0: XCD-contiguous unit numbering; bit 1: rotate chunks
    int32_t pairs[2 * kMaxPairs];
};

struct LaunchCfg {
    int unroll;        // 16-byte vectors per lane per unit: 1, 2, 4, 8 or 16
    bool permute;      // pool inner layout is HND
    bool publish;
    int nontemporal;   // bit 0: non-temporal loads, bit 1: non-temporal stores
    int grid;
};

uint32_t magic_u32(uint32_t d);   // multiplier for exact x / d with x * d < 2^32
int pick_unroll(int64_t piece_bytes, int max_unroll);
hipError_t launch_move(Dir dir, const LaunchCfg& cfg, const MoveArgs& a, hipStream_t s);
hipError_t launch_ready_wait(const uint32_t* slot, uint32_t min_count, uint32_t spin_limit,
                             int32_t* status, hipStream_t s);

}  // namespace kvx
