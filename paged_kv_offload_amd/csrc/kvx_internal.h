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
#include "kvx_host.h"

namespace kvx {

int hip_fail(hipError_t e, const char* what);  // KVX_E_HIP with the runtime's message

// A roctx range around a data-moving call while KVX_TRACE is set.
struct TraceRange {
    explicit TraceRange(const char* name);
    ~TraceRange();
    TraceRange(const TraceRange&) = delete;
    TraceRange& operator=(const TraceRange&) = delete;
    bool on;
};

#define KVX_HIP(call)                                   \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

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
    uint32_t* counts = nullptr;      // host view (fine-grained pinned); null for device counts
    uint32_t* counts_dev = nullptr;  // device view of the same memory, or the device counts
    int device = -1;                 // GPU holding device counts; -1 for pinned host counts
    bool owned = true;               // allocated here (freed by kvx_ready_destroy)
    hipStream_t query = nullptr;     // non-blocking stream for copies of device counts
};

namespace kvx {

bool pool_known(const kvx_pool* p);
bool ready_known(const kvx_ready* r);
void register_ready(const kvx_ready* r);   // enters a new ready handle in the registry

// ---------------------------------------------------------------------------
// tuning
// ---------------------------------------------------------------------------
struct Tuning {
    int64_t grid_max = 0;                 // 0 = auto
    int64_t stage_slot_bytes = 128ll << 20;
    int64_t stage_slots = 3;
    int64_t sort_pages = 0;
    int64_t cache_policy = -1;            // bit 0 nt loads, bit 1 nt stores, bit 2 sc1 stores; -1 = auto
    int64_t restore_chunk_layers = 0;     // 0 = auto (chunks of >= kRestoreChunkMin bytes)
    int64_t host_grid_max = 0;            // 0 = auto
    int64_t unit_order = -1;              // MoveArgs::unit_order bits, -1 = auto
    int64_t max_unroll = 32;              // largest 16-byte vectors per lane per unit
    int64_t unit_rounds = 0;              // 0 = auto; else the unit's vector rounds
    int64_t staged_dma_on_caller = -1;    // staged DMA: 1 caller's stream, 0 side stream, -1 auto
    int64_t hnd_lds = -1;                 // HND<->NHD through LDS: 1 both, 0 never, -1 scatter only
    int64_t fail_allocs = 0;              // test hook: internal device allocations left to fail
    int64_t ring_pairing = 1;             // ring executor runs BACKUP + RESTORE as one exchange
    int64_t publish_block = 0;            // units per queue draw of device-memory publishing kernels (0 = auto)
    int64_t coalesce_runs = 1;            // move runs of adjacent pages as spans when that takes fewer units
    int64_t tail_units = 1;               // the tails of pieces that 128 KiB units do not tile share units
    int64_t device_lists = 1;             // lists longer than the kernel arguments carry go to device memory
    int64_t duplex_writers = 6;           // workgroups writing host memory while host reads are in flight (0 = share of 48)
    int64_t duplex_readers = 18;          // workgroups reading host memory while host writes are in flight (0 = share of 48)
};
Tuning tuning();

// ---------------------------------------------------------------------------
// kernel launch interface
// ---------------------------------------------------------------------------
constexpr int kThreads = 256;        // 4 wave64 per workgroup
constexpr int kMaxPairs = 448;       // (page, slot) pairs carried in the kernel arguments
constexpr int kListHostSlots = 4;    // pinned host buffers a stream's long page lists rotate through
constexpr int64_t kRestoreChunkMin = 32ll << 20;   // default minimum staged restore chunk
constexpr int64_t kPublishBlockBytes = 2ll << 20;  // auto publish block: about this many bytes
// kvx_restore_noalloc: layers of a pool it serves, and the words of its device
// scratch (one counter per layer, the unit queue, padding)
constexpr int64_t kNoAllocMaxLayers = KVX_NOALLOC_MAX_LAYERS;
constexpr int64_t kNoAllocScratchWords = kNoAllocMaxLayers + 64;

enum Dir : int32_t { GATHER = 0, SCATTER = 1 };

// Pool and work-unit geometry shared by every unit of a launch.
struct UnitGeom {
    uint8_t* pool;           // pool start (base + byte_offset)
    int64_t page_stride, layer_stride, kv_stride;   // pool byte strides
    uint32_t piece_bytes;
    uint32_t chunk_bytes;    // bytes of one work unit (kThreads * 16 * unroll)
    uint32_t chunks_per_piece;
    uint32_t num_kv;
    // pool HND <-> packed NHD permutation (unused for NHD pools)
    uint32_t T, H, row_vec;              // row_vec = row_bytes / 16
    uint32_t mg_row_vec, mg_H, mg_T;     // magic multipliers (0 means divisor 1)
    uint32_t TU, seg, mg_seg;            // LDS token blocks: tokens per unit, TU * row_vec
    uint32_t unit_order;     // bit 0: XCD-contiguous unit numbering; bit 1: rotate chunks
    uint32_t runs;           // move launches: 1 = the pair list holds runs of adjacent pages
    uint32_t units_lc;       // runs: work units of one (layer, kv) in the launch
    // tails (launches over pairs, not runs; units of 32 rounds in device
    // memory or 2 over the host link): a piece is main_units whole units
    // (possibly none) and a tail of tail_bytes; the tails of
    // tails_per_wave * 4 consecutive pairs of a side share one unit, each
    // wave moving tails_per_wave of them
    uint32_t tails_per_wave; // 0: no tail units (a piece's last unit may be partial)
    uint32_t main_units;
    uint32_t tail_bytes;
};

// One direction's share of a launch: the pieces (page, layer, kv) of layers
// [layer_begin, layer_begin + num_layers), every kv, and `npairs` pages,
// against a packed buffer holding layers >= pk_layer0 and slots >= pk_slot0.
struct Side {
    uint8_t* packed;
    int64_t pk_lc_stride;    // packed bytes per (layer, kv) = pk_slots * piece_bytes
    int32_t pk_layer0, pk_slot0;
    int32_t layer_begin;
    uint32_t npairs;
    uint32_t total_units;    // num_layers * num_kv * npairs * chunks_per_piece
};

// Per-layer publish of a RESTORE with a ready object, and the unit queue.
struct PublishArgs {
    uint32_t* layer_done;    // device counters, indexed by absolute layer
    uint32_t* queue;         // queue-driven kernels: next unit number (zero between launches)
    uint32_t* ready;         // device view of counts + slot_base, indexed by layer
    uint32_t layer_target;   // work units of one layer over the whole call
    uint32_t publish_value;  // n
    uint32_t block;          // move kernels: consecutive units per queue draw (>= 1)
};

// Runs of adjacent pages per move launch: (first page, first slot, pages,
// units before the run in its (layer, kv)) in the pair array.
constexpr int kMaxRuns = kMaxPairs / 2;

// One direction: pairs[2j] is the page and pairs[2j + 1] its slot; in a
// launch over runs (g.runs), pairs[4r .. 4r + 3] describe run r.
struct MoveArgs {
    UnitGeom g;
    Side s;
    PublishArgs p;
    // the launch's (page, slot) pairs or runs: in device memory when `list`
    // is set (lists longer than the kernel arguments carry), else in `pairs`
    const int32_t* list;
    int32_t pairs[2 * kMaxPairs];
};
static_assert(sizeof(MoveArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// Both directions in one launch (kvx_exchange): a BACKUP side `b` and a
// RESTORE side `r`, each listing its pages in slot order (the slot of
// pages_x[j] is first_x + j; the sides' pk_slot0 is 0, the buffer start).
struct ExchangeArgs {
    UnitGeom g;
    Side b, r;
    PublishArgs p;
    const int32_t* list_b;   // the sides' pages in device memory (lists longer than
    const int32_t* list_r;   // the arguments carry), else pages_b / pages_r
    int32_t first_b, first_r;
    int32_t pages_b[kMaxPairs];
    int32_t pages_r[kMaxPairs];
};
static_assert(sizeof(ExchangeArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// Both directions against slot-addressed host pools (kvx_exchange_slots):
// pairs_x[2j] is a page and pairs_x[2j + 1] its host slot.
constexpr int kMaxSlotPairs = 224;
struct ExchangeSlotArgs {
    UnitGeom g;
    Side b, r;
    PublishArgs p;
    const int32_t* list_b;   // the sides' (page, slot) pairs in device memory, else
    const int32_t* list_r;   // pairs_b / pairs_r
    int32_t pairs_b[2 * kMaxSlotPairs];
    int32_t pairs_r[2 * kMaxSlotPairs];
};
static_assert(sizeof(ExchangeSlotArgs) <= 4096, "kernel arguments are limited to 4 KiB");

struct LaunchCfg {
    int unroll;        // 16-byte vectors per lane per unit: 1, 2, 4, 8 or 16
    int permute;       // 0: same inner layout; 1: HND<->NHD by rows; 2: through LDS
    bool publish;
    int cache_policy;  // bit 0: non-temporal loads, bit 1: non-temporal stores, bit 2: device-scope stores
    bool host_link;    // exchange: both packed buffers are pinned host memory
    int grid;
};

// Makes `dev` current for the guard's lifetime.
struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev)
            changed = (hipSetDevice(dev) == hipSuccess);
    }
    ~DeviceGuard()
    {
        if (changed) (void)hipSetDevice(prev);
    }
};

// True if `p` lies in a mapping imported with kvx_ipc_import; then *device is
// its GPU and *bytes_after the mapping's bytes from p to its end.
bool ipc_lookup(const void* p, int* device, uint64_t* bytes_after);

uint32_t magic_u32(uint32_t d);   // multiplier for exact x / d with x * d < 2^32
// unit rounds for a piece: `forced` (> 0) if given, else the measured choice
int pick_unroll(int64_t piece_bytes, int max_unroll, int forced);
hipError_t launch_move(Dir dir, const LaunchCfg& cfg, const MoveArgs& a, hipStream_t s);
hipError_t launch_exchange(const LaunchCfg& cfg, const ExchangeArgs& a, hipStream_t s);
hipError_t launch_exchange(const LaunchCfg& cfg, const ExchangeSlotArgs& a, hipStream_t s);
hipError_t launch_clear_u32(uint32_t* p, uint32_t count, hipStream_t s);
// Device address of this GPU's copy of the no-alloc scratch (looked up once
// per device, with the device current).
int noalloc_scratch(int device, uint32_t** out);
hipError_t launch_ready_wait(const uint32_t* slot, uint32_t min_count, uint32_t spin_limit,
                             int32_t* status, hipStream_t s);

}  // namespace kvx
