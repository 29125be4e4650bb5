// api.cpp - the C ABI of kvx: handles and their lifecycle, the order of
// validation (everything is checked before anything is enqueued), the path
// executor (staged DMA through a device ring on a side stream, zero-copy
// kernels on pinned host memory, or device-to-device), the exchange of a
// backup and a restore in one launch sequence and small utilities. Ready
// objects are in ready.cpp, the host tier's policy calls in tier_policy.cpp
// and the ring executor in ring_exec.cpp.
//
// Ownership follows the RFC's split ([RFC] "Ownership"): the caller owns the
// pool allocation, page IDs and the decision that pages are safe to read or
// write; the library owns its side streams, staging rings, events and
// completion counters. Lifecycle follows [RFC] "Failure and lifecycle
// handling" (generation-tagged handles, fail closed) and the RawCudaIPCWrapper
// article's lifecycle section (teardown logs, never raises).
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iterator>
#include <set>
#include <type_traits>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "kvx_internal.h"

namespace kvx {

// ---------------------------------------------------------------------------
// errors and logging
// ---------------------------------------------------------------------------
namespace {
thread_local std::string t_error;

int log_level()
{
    static const int lvl = [] {
        const char* e = std::getenv("KVX_LOG");
        return e ? std::atoi(e) : 1;
    }();
    return lvl;
}
}  // namespace

int fail(int code, const std::string& msg)
{
    t_error = msg;
    if (log_level() >= 2) std::fprintf(stderr, "kvx: error %d: %s\n", code, msg.c_str());
    return code;
}

void clear_error() { t_error.clear(); }

// KVX_TRACE=1: every data-moving call is a roctx range named after it, so a
// marker trace (rocprofv3 --marker-trace) shows the calls around their
// kernels and copies. Read once; off by default.
bool trace_on()
{
    static const bool on = [] {
        const char* e = std::getenv("KVX_TRACE");
        return e && std::atoi(e) > 0;
    }();
    return on;
}

TraceRange::TraceRange(const char* name) : on(trace_on())
{
    if (on) roctxRangePushA(name);
}

TraceRange::~TraceRange()
{
    if (on) roctxRangePop();
}

void log_warn(const std::string& msg)
{
    if (log_level() >= 1) std::fprintf(stderr, "kvx: warning: %s\n", msg.c_str());
}

void log_info(const std::string& msg)
{
    if (log_level() >= 2) std::fprintf(stderr, "kvx: %s\n", msg.c_str());
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(KVX_E_HIP, std::string(what) + " failed: " + hipGetErrorName(e) + " (" +
                               hipGetErrorString(e) + ")");
}

// ---------------------------------------------------------------------------
// handle registries: handles are never freed, only marked dead, so a stale
// handle is recognised instead of being undefined behaviour
// ---------------------------------------------------------------------------
namespace {
std::mutex g_reg_mu;
std::set<const kvx_pool*> g_pools;
std::set<const kvx_ready*> g_readies;

std::mutex g_tune_mu;
Tuning g_tune;
}  // namespace

bool pool_known(const kvx_pool* p)
{
    std::lock_guard<std::mutex> lk(g_reg_mu);
    return p && g_pools.count(p) && p->magic == POOL_MAGIC;
}

bool ready_known(const kvx_ready* r)
{
    std::lock_guard<std::mutex> lk(g_reg_mu);
    return r && g_readies.count(r) && r->magic == READY_MAGIC;
}

void register_ready(const kvx_ready* r)
{
    std::lock_guard<std::mutex> lk(g_reg_mu);
    g_readies.insert(r);
}

Tuning tuning()
{
    std::lock_guard<std::mutex> lk(g_tune_mu);
    return g_tune;
}

// Test hook (KVX_OPT_FAIL_ALLOCS): true if this internal allocation is to
// fail as if the device were out of memory.
bool injected_alloc_failure()
{
    std::lock_guard<std::mutex> lk(g_tune_mu);
    if (g_tune.fail_allocs <= 0) return false;
    g_tune.fail_allocs--;
    return true;
}

namespace {

// ---------------------------------------------------------------------------
// lanes: per (device, caller stream) state of the executor
// ---------------------------------------------------------------------------
struct Lane {
    int device = -1;
    hipStream_t caller = nullptr;
    hipStream_t side = nullptr;     // library-owned, default priority; created by the first
                                    // staged operation (a HIP process has few hardware queues,
                                    // and every stream takes a share of one)
    int cu_count = 0;
    uint8_t* ring = nullptr;        // device staging ring
    int64_t slot_bytes = 0;
    int nslots = 0;
    std::vector<hipEvent_t> slot_free, slot_ready;
    std::vector<bool> slot_pending;
    hipEvent_t ev_start = nullptr, ev_done = nullptr;
    uint32_t* layer_done = nullptr; // per-layer unit counters for publish, then the unit queue
    int64_t layer_cap = 0;          // counters; the queue is layer_done[layer_cap]
    bool counters_dirty = false;
    int next_slot = 0;
    // a call's pair or run list when it is longer than one launch's kernel
    // arguments carry: copied on the caller's stream into list_dev (one
    // buffer: the next call's copy is stream-ordered after this call's
    // launches) from a ring of pinned host buffers (a host buffer is refilled
    // only once its previous copy has run)
    int32_t* list_dev = nullptr;
    int64_t list_cap = 0;           // int32 words
    int32_t* list_host[kListHostSlots] = {};
    int64_t list_host_cap[kListHostSlots] = {};
    hipEvent_t list_sent[kListHostSlots] = {};
    int list_next = 0;
    // recorded after each zero-copy or staged call (under g_link_mu): other
    // streams' calls see whether this one still uses the host link
    hipEvent_t link_ev = nullptr;
    bool link_busy = false;         // link_ev recorded and not yet seen complete
    int link_dir = 0;               // kLink* traffic of the calls link_ev covers
    std::mutex mu;
};

std::mutex g_lanes_mu;
std::map<std::pair<int, hipStream_t>, Lane*> g_lanes;

// Lanes that ran host-link calls, and every lane's link_ev and link_busy.
// Taken inside a lane's mutex (or with none held), never around one.
std::mutex g_link_mu;
std::vector<Lane*> g_link_lanes;

// Zero-copy and staged BACKUP and RESTORE calls of other streams whose work
// has not finished on L's GPU (LinkLoad).
LinkLoad link_others(const Lane* L)
{
    std::lock_guard<std::mutex> lk(g_link_mu);
    LinkLoad n;
    for (Lane* o : g_link_lanes) {
        if (o == L || o->device != L->device || !o->link_busy) continue;
        if (hipEventQuery(o->link_ev) == hipErrorNotReady) {
            (void)hipGetLastError();
            if (o->link_dir & kLinkWrites) n.writers++;
            if (o->link_dir & kLinkReads) n.readers++;
            if (o->link_dir & kLinkDmaWrites) n.dma_writers++;
            if (o->link_dir & kLinkDmaReads) n.dma_readers++;
        } else {
            o->link_busy = false;   // done: not queried again until its next call
        }
    }
    return n;
}

// Records the end of L's latest host-link call (traffic dir). Calls queued
// on the stream before it that have not finished keep their directions.
int link_record(Lane* L, hipStream_t s, int dir)
{
    std::lock_guard<std::mutex> lk(g_link_mu);
    if (!L->link_ev) {
        KVX_HIP(hipEventCreateWithFlags(&L->link_ev, hipEventDisableTiming));
        g_link_lanes.push_back(L);
    }
    if (L->link_busy) {   // the previous calls' event, recorded after them
        if (hipEventQuery(L->link_ev) == hipErrorNotReady)
            (void)hipGetLastError();
        else
            L->link_busy = false;
    }
    KVX_HIP(hipEventRecord(L->link_ev, s));
    L->link_dir = L->link_busy ? (L->link_dir | dir) : dir;
    L->link_busy = true;
    return KVX_OK;
}

// Workgroups of a one-direction zero-copy kernel (dir: kLinkWrites or
// kLinkReads), given the other streams' host-link calls in flight now
// (link_grid_for states the policy and its measurements).
int link_grid(const Lane* L, int dir, const Tuning& t)
{
    return link_grid_for(link_others(L), dir, t.duplex_writers, t.duplex_readers);
}

int lane_init(Lane* L)
{
    KVX_HIP(hipDeviceGetAttribute(&L->cu_count, hipDeviceAttributeMultiprocessorCount, L->device));
    KVX_HIP(hipEventCreateWithFlags(&L->ev_start, hipEventDisableTiming));
    KVX_HIP(hipEventCreateWithFlags(&L->ev_done, hipEventDisableTiming));
    return KVX_OK;
}

// The lane of (device, caller stream), created on first use, returned with
// its mutex held by *held. The mutex is taken while the registry's is held,
// so kvx_release_stream (which takes both in the same order) never frees a
// lane that a call has found.
int get_lane(int device, hipStream_t caller, Lane** out, std::unique_lock<std::mutex>* held)
{
    std::lock_guard<std::mutex> lk(g_lanes_mu);
    auto key = std::make_pair(device, caller);
    auto it = g_lanes.find(key);
    if (it != g_lanes.end()) {
        *held = std::unique_lock<std::mutex>(it->second->mu);
        *out = it->second;
        return KVX_OK;
    }
    Lane* L = new (std::nothrow) Lane();
    if (!L) return fail(KVX_E_NOMEM, "cannot allocate an executor lane");
    L->device = device;
    L->caller = caller;
    int rc = lane_init(L);
    if (rc != KVX_OK) return rc;   // a half-built lane is leaked on purpose: never reused
    g_lanes[key] = L;
    *held = std::unique_lock<std::mutex>(L->mu);
    *out = L;
    return KVX_OK;
}

// Waits for everything a lane enqueued and frees what it holds: the staging
// ring, the per-layer counters, the side stream and the events. Failures are
// logged; the lane is not used again either way.
void lane_free(Lane* L)
{
    DeviceGuard dg(L->device);
    auto check = [](hipError_t e, const char* what) {
        if (e != hipSuccess) {
            (void)hipGetLastError();
            log_warn(std::string("release_stream: ") + what + " failed: " + hipGetErrorString(e));
        }
    };
    check(hipStreamSynchronize(L->caller), "waiting for the caller's stream");
    if (L->side) {
        check(hipStreamSynchronize(L->side), "waiting for the side stream");
        check(hipStreamDestroy(L->side), "hipStreamDestroy");
    }
    for (hipEvent_t e : L->slot_free) check(hipEventDestroy(e), "hipEventDestroy");
    for (hipEvent_t e : L->slot_ready) check(hipEventDestroy(e), "hipEventDestroy");
    if (L->ev_start) check(hipEventDestroy(L->ev_start), "hipEventDestroy");
    if (L->ev_done) check(hipEventDestroy(L->ev_done), "hipEventDestroy");
    if (L->ring) check(hipFree(L->ring), "hipFree of the staging ring");
    if (L->layer_done) check(hipFree(L->layer_done), "hipFree of the per-layer counters");
    {
        std::lock_guard<std::mutex> lk(g_link_mu);
        g_link_lanes.erase(std::remove(g_link_lanes.begin(), g_link_lanes.end(), L), g_link_lanes.end());
        if (L->link_ev) check(hipEventDestroy(L->link_ev), "hipEventDestroy");
        L->link_ev = nullptr;
    }
    if (L->list_dev) check(hipFree(L->list_dev), "hipFree of the page list");
    for (int h = 0; h < kListHostSlots; h++) {
        if (L->list_sent[h]) check(hipEventDestroy(L->list_sent[h]), "hipEventDestroy");
        if (L->list_host[h]) check(hipHostFree(L->list_host[h]), "hipHostFree of the page list");
    }
}

// waits until no earlier operation of this lane still reads or writes the
// ring: DMA on the side stream through the slots' events, and operations
// that ran on the caller's stream alone (their slots are not pending)
// through the caller's stream, which is live: this runs inside a call on it
int lane_drain_ring(Lane* L)
{
    for (int r = 0; r < L->nslots; r++)
        if (L->slot_pending[r]) KVX_HIP(hipEventSynchronize(L->slot_free[r]));
    if (L->ring) KVX_HIP(hipStreamSynchronize(L->caller));
    return KVX_OK;
}

int lane_ring(Lane* L, int64_t slot_bytes, int nslots)
{
    if (L->ring && L->slot_bytes == slot_bytes && L->nslots == nslots) return KVX_OK;
    int rc = lane_drain_ring(L);
    if (rc != KVX_OK) return rc;
    if (L->ring) {
        KVX_HIP(hipFree(L->ring));
        L->ring = nullptr;
    }
    for (hipEvent_t e : L->slot_free) (void)hipEventDestroy(e);
    for (hipEvent_t e : L->slot_ready) (void)hipEventDestroy(e);
    L->slot_free.clear();
    L->slot_ready.clear();
    L->slot_pending.assign(nslots, false);
    L->nslots = 0;
    void* p = nullptr;
    hipError_t e = injected_alloc_failure() ? hipErrorOutOfMemory
                                            : hipMalloc(&p, static_cast<size_t>(slot_bytes) * nslots);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(KVX_E_NOMEM, "cannot allocate the device staging ring (" +
                                     std::to_string(slot_bytes * nslots) + " bytes)");
    }
    L->ring = static_cast<uint8_t*>(p);
    L->slot_free.resize(nslots);
    L->slot_ready.resize(nslots);
    for (int r = 0; r < nslots; r++) {
        KVX_HIP(hipEventCreateWithFlags(&L->slot_free[r], hipEventDisableTiming));
        KVX_HIP(hipEventCreateWithFlags(&L->slot_ready[r], hipEventDisableTiming));
    }
    L->slot_bytes = slot_bytes;
    L->nslots = nslots;
    L->next_slot = 0;
    return KVX_OK;
}

// Copies `words` (a call's pair or run list) to the lane's device list on
// the caller's stream; *out is the device copy.
int lane_upload_list(Lane* L, const std::vector<int32_t>& words, const int32_t** out)
{
    const int64_t count = static_cast<int64_t>(words.size());
    if (L->list_cap < count) {
        if (L->list_dev) {
            KVX_HIP(hipStreamSynchronize(L->caller));   // earlier launches may still read it
            KVX_HIP(hipFree(L->list_dev));
            L->list_dev = nullptr;
            L->list_cap = 0;
        }
        const int64_t cap = std::max<int64_t>(count, int64_t(1) << 16);
        void* p = nullptr;
        hipError_t e = injected_alloc_failure() ? hipErrorOutOfMemory : hipMalloc(&p, cap * sizeof(int32_t));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(KVX_E_NOMEM, "cannot allocate the device page list");
        }
        L->list_dev = static_cast<int32_t*>(p);
        L->list_cap = cap;
    }
    const int h = L->list_next;
    L->list_next = (h + 1) % kListHostSlots;
    if (L->list_sent[h])
        KVX_HIP(hipEventSynchronize(L->list_sent[h]));   // the buffer's previous copy has run
    else
        KVX_HIP(hipEventCreateWithFlags(&L->list_sent[h], hipEventDisableTiming));
    if (L->list_host_cap[h] < count) {
        if (L->list_host[h]) KVX_HIP(hipHostFree(L->list_host[h]));
        L->list_host[h] = nullptr;
        L->list_host_cap[h] = 0;
        const int64_t cap = std::max<int64_t>(count, int64_t(1) << 16);
        void* p = nullptr;
        hipError_t e = hipHostMalloc(&p, cap * sizeof(int32_t), hipHostMallocDefault);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(KVX_E_NOMEM, "cannot allocate the pinned page list");
        }
        L->list_host[h] = static_cast<int32_t*>(p);
        L->list_host_cap[h] = cap;
    }
    std::memcpy(L->list_host[h], words.data(), words.size() * sizeof(int32_t));
    KVX_HIP(hipMemcpyAsync(L->list_dev, L->list_host[h], words.size() * sizeof(int32_t),
                           hipMemcpyHostToDevice, L->caller));
    KVX_HIP(hipEventRecord(L->list_sent[h], L->caller));
    *out = L->list_dev;
    return KVX_OK;
}

int lane_counters(Lane* L, int64_t num_layers)
{
    if (L->layer_done && L->layer_cap >= num_layers && !L->counters_dirty) return KVX_OK;
    if (!L->layer_done || L->layer_cap < num_layers) {
        if (L->layer_done) {
            KVX_HIP(hipStreamSynchronize(L->caller));   // earlier publishes may still count
            KVX_HIP(hipFree(L->layer_done));
            L->layer_done = nullptr;
        }
        const int64_t cap = std::max<int64_t>(num_layers, 256);
        void* p = nullptr;
        hipError_t e = injected_alloc_failure() ? hipErrorOutOfMemory
                                                : hipMalloc(&p, (cap + 1) * sizeof(uint32_t));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(KVX_E_NOMEM, "cannot allocate per-layer completion counters");
        }
        L->layer_done = static_cast<uint32_t*>(p);
        L->layer_cap = cap;
    }
    // stream-ordered clear before the first kernel that counts into them
    KVX_HIP(launch_clear_u32(L->layer_done, static_cast<uint32_t>(L->layer_cap + 1), L->caller));
    L->counters_dirty = false;
    return KVX_OK;
}

// ---------------------------------------------------------------------------
// memory classification
// ---------------------------------------------------------------------------
enum class MemKind { PinnedHost, Device, Other };

MemKind classify(const void* p, int device, uint8_t** dev_view)
{
    hipPointerAttribute_t at;
    std::memset(&at, 0, sizeof at);
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return MemKind::Other;
    }
    if (at.type == hipMemoryTypeHost) {
        void* d = nullptr;
        if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
            (void)hipGetLastError();
            return MemKind::Other;
        }
        *dev_view = static_cast<uint8_t*>(d);
        return MemKind::PinnedHost;
    }
    if (at.type == hipMemoryTypeDevice && at.device == device) {
        *dev_view = static_cast<uint8_t*>(const_cast<void*>(p));
        return MemKind::Device;
    }
    return MemKind::Other;
}

int resolve_device(kvx_pool* pool)
{
    std::lock_guard<std::mutex> lk(pool->mu);
    if (pool->device >= 0) return KVX_OK;
    hipPointerAttribute_t at;
    std::memset(&at, 0, sizeof at);
    // a mapping imported with kvx_ipc_import is known by its registry entry
    int ipc_dev = -1;
    uint64_t ipc_after = 0;
    if (ipc_lookup(pool->start, &ipc_dev, &ipc_after)) {
        if (static_cast<uint64_t>(pool->geom.pool_bytes) > ipc_after)
            return fail(KVX_E_RANGE, "pool (" + std::to_string(pool->geom.pool_bytes) +
                                         " bytes) extends past the end of its imported allocation");
        pool->device = ipc_dev;
        return KVX_OK;
    }
    hipError_t e = hipPointerGetAttributes(&at, pool->start);
    if (e != hipSuccess || at.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        return fail(KVX_E_INVAL, "pool memory is not device memory");
    }
    void* abase = nullptr;
    size_t asize = 0;
    e = hipMemGetAddressRange(reinterpret_cast<hipDeviceptr_t*>(&abase), &asize, pool->start);
    if (e == hipSuccess && abase) {
        const uint64_t end = reinterpret_cast<uintptr_t>(pool->start) + pool->geom.pool_bytes;
        if (end > reinterpret_cast<uintptr_t>(abase) + asize)
            return fail(KVX_E_RANGE, "pool (" + std::to_string(pool->geom.pool_bytes) +
                                         " bytes) extends past the end of its allocation");
    } else {
        (void)hipGetLastError();
    }
    pool->device = at.device;
    return KVX_OK;
}

// ---------------------------------------------------------------------------
// kernel launches over a layer range and a pair list
// ---------------------------------------------------------------------------
struct Target {
    uint8_t* packed;       // device view of the packed region
    int32_t pk_layer0, pk_slot0;
    int64_t pk_slots;      // slots stored per (layer, kv) in `packed`
    bool host;             // `packed` is pinned host memory read or written over the link
    int host_grid = 0;     // host: workgroups per launch (0: kHostGridAuto)
};

struct Publish {
    uint32_t* layer_done = nullptr;
    uint32_t* queue = nullptr;   // unit queue of the publishing kernels
    uint32_t* ready = nullptr;   // device view of counts + slot_base
    uint32_t layer_target = 0;   // units of one layer over the call (unless target_here)
    uint32_t value = 0;
    bool target_here = false;    // the launch sequence is the whole call: it counts the target
};

// Unit size (vector rounds of 4 KiB per workgroup) of a launch; the publish
// target of a RESTORE is counted in the same units.
int unroll_for(const PoolGeom& g, const Tuning& t, bool host)
{
    const bool permute = (g.inner == KVX_HND) && g.num_heads > 1 && g.page_size > 1;
    // the LDS form runs units of 4, 8 or 16 rounds
    int max_unroll = static_cast<int>(permute && t.hnd_lds != 0 ? std::min<int64_t>(t.max_unroll, 16)
                                                                : t.max_unroll);
    // over the host link, 8 KiB units (measured on the llama8b request: the
    // same 57 GB/s one way as 32 or 128 KiB units, the first layer of a
    // zero-copy restore ready at 1.19 ms instead of 1.22 and 1.8, and the
    // layer-pipelined exchange step at 95.4 GB/s against 88.9 with 32 KiB
    // units; 4 KiB units hold the restore to 42 GB/s)
    if (host) max_unroll = std::min(max_unroll, 2);
    return pick_unroll(g.piece_bytes, max_unroll, static_cast<int>(t.unit_rounds));
}

// Tail units of a launch over (page, slot) pairs: a piece is main_units whole
// units and a tail, and the tails of 4 * tails_per_wave pieces share one unit,
// each wave moving tails_per_wave whole tails (the kernels carry this form
// for units of 32 rounds in device memory and of 2 over the host link).
//  - Pieces that such units do not tile (the MLA pool's 144 KiB pieces: a
//    16 KiB tail after one 128 KiB unit) lose their mostly idle partial
//    unit.
//  - Pieces no longer than a wave's share of such a unit (32 KiB in device
//    memory, 2 KiB over the host link; a pool of one token per page has
//    2 KiB pieces) are all tail: 4 * tails_per_wave of them travel in one
//    unit instead of one piece in a unit of its own.
// Not for reordered rows, nor where the unit size is forced.
struct TailPlan {
    int unroll = 0;
    uint32_t tails_per_wave = 0, main_units = 0, tail_bytes = 0;
};

// Whether short pieces travel whole, several to a unit, rather than one to a
// unit of their own size. Measured on MI355X, fragmented 1 GiB requests of a
// 32-layer K+V pool (TB/s read + write, one piece a unit -> whole pieces):
//   piece   plain pack     plain unpack   publishing unpack
//   1 KiB   2.10 -> 3.42   1.99 -> 3.07   0.28 -> 1.57
//   2 KiB   3.96 -> 4.40   3.82 -> 3.98   0.72 -> 2.37
//   4 KiB   5.35 -> 4.80   4.82 -> 4.40   1.63 -> 3.23
//   8 KiB   5.45 -> 5.39   4.97 -> 4.83   2.67 -> 3.87
//  16 KiB   5.55 -> 5.84   5.08 -> 5.10   3.87 -> 3.54
//  32 KiB   5.60 -> 6.05   5.23 -> 5.53   3.75 -> 3.93
// and zero-copy restores of 1 and 2 KiB pieces at 54.5 and 55.9 GB/s
// against 17.1 and 34.2.
bool whole_pieces_pay(int64_t piece_bytes, bool host, bool publish)
{
    if (host) return true;
    if (publish) return piece_bytes <= 8192 || piece_bytes > 16384;
    return piece_bytes <= 2048 || piece_bytes >= 16384;
}

bool plan_tails(const PoolGeom& g, const Tuning& t, bool host, bool publish, TailPlan* tp)
{
    const bool permute = (g.inner == KVX_HND) && g.num_heads > 1 && g.page_size > 1;
    if (permute || t.tail_units == 0) return false;
    const int umax = host ? 2 : 32;
    const int64_t wave_round = 64 * kVecBytes;   // one round of one wave
    const int unroll = unroll_for(g, t, host);
    int64_t main = 0, tail = 0;
    if (unroll == umax) {
        main = g.piece_bytes / (4 * wave_round * umax);
        tail = g.piece_bytes - main * 4 * wave_round * umax;
    } else if (t.unit_rounds == 0 && t.max_unroll >= umax && g.piece_bytes <= umax * wave_round &&
               whole_pieces_pay(g.piece_bytes, host, publish)) {
        tail = g.piece_bytes;
    } else {
        return false;
    }
    if (tail <= 0) return false;
    for (int tpw = 8; tpw >= 1; tpw /= 2) {
        if (tpw <= umax && tail <= (umax / tpw) * wave_round) {
            tp->unroll = umax;
            tp->tails_per_wave = static_cast<uint32_t>(tpw);
            tp->main_units = static_cast<uint32_t>(main);
            tp->tail_bytes = static_cast<uint32_t>(tail);
            return true;
        }
    }
    return false;
}

// Work units of one (layer, kv) of a launch over np pairs.
int64_t pair_units(const TailPlan* tp, int64_t chunks_per_piece, int64_t np)
{
    if (tp && tp->tails_per_wave)
        return np * tp->main_units + (np + 4 * tp->tails_per_wave - 1) / (4 * tp->tails_per_wave);
    return np * chunks_per_piece;
}

// Unit geometry of launches on `pool`; sets cfg.unroll and cfg.permute.
void setup_geom(const kvx_pool* pool, bool host, const Tuning& t, UnitGeom* ug, LaunchCfg* cfg)
{
    const PoolGeom& g = pool->geom;
    std::memset(ug, 0, sizeof *ug);
    cfg->permute = ((g.inner == KVX_HND) && g.num_heads > 1 && g.page_size > 1) ? 1 : 0;
    // HND<->NHD through LDS token blocks unless switched off (measured on the
    // TRT-LLM-shaped pool with equal counter traffic: 64 KiB token blocks
    // pack at 6.30 TB/s against 5.93 row by row, and unpack at 5.96 against
    // 5.71)
    const bool lds = cfg->permute && t.hnd_lds != 0;
    cfg->unroll = unroll_for(g, t, host);
    ug->pool = pool->start;
    ug->page_stride = g.page_stride;
    ug->layer_stride = g.layer_stride;
    ug->kv_stride = g.kv_stride;
    ug->piece_bytes = static_cast<uint32_t>(g.piece_bytes);
    ug->chunk_bytes = static_cast<uint32_t>(kThreads * kVecBytes * cfg->unroll);
    ug->chunks_per_piece = static_cast<uint32_t>((g.piece_bytes + ug->chunk_bytes - 1) / ug->chunk_bytes);
    ug->num_kv = static_cast<uint32_t>(g.num_kv);
    ug->T = static_cast<uint32_t>(g.page_size);
    ug->H = static_cast<uint32_t>(g.num_heads);
    ug->row_vec = static_cast<uint32_t>(g.row_bytes / kVecBytes);
    ug->mg_row_vec = magic_u32(ug->row_vec);
    ug->mg_H = magic_u32(ug->H);
    ug->mg_T = magic_u32(ug->T);
    if (lds && (cfg->unroll == 4 || cfg->unroll == 8 || cfg->unroll == 16)) {
        // an LDS unit is a block of whole tokens over all heads
        const int64_t block = g.num_heads * g.row_bytes;
        if (ug->chunk_bytes % block == 0 && g.page_size % (ug->chunk_bytes / block) == 0) {
            cfg->permute = 2;
            ug->TU = static_cast<uint32_t>(ug->chunk_bytes / block);
            ug->seg = ug->TU * ug->row_vec;
            ug->mg_seg = magic_u32(ug->seg);
        }
    }
}

void set_publish(const Publish* pub, PublishArgs* p)
{
    std::memset(p, 0, sizeof *p);
    if (!pub) return;
    p->layer_done = pub->layer_done;
    p->queue = pub->queue;
    p->ready = pub->ready;
    p->layer_target = pub->layer_target;
    p->publish_value = pub->value;
    p->block = 1;
}

// Runs of adjacent pages for a launch sequence over `pairs` (in visiting
// order): consecutive pages that land in consecutive slots, in a pool whose
// pages are adjacent in memory (the page is the innermost outer axis). On
// both sides a run is one span of count x piece_bytes, cut into units like
// a piece. Used when rows are not reordered (a span is moved as it is) and
// the runs need fewer units than the pieces do: small pieces get fewer,
// fuller units, and pieces that a unit does not tile lose their partial
// unit.
struct RunPlan {
    std::vector<Run> runs;
    int unroll = 0;          // vector rounds of a unit
    int64_t units_lc = 0;    // units of one (layer, kv) over all runs
};

bool plan_run_units(const PoolGeom& g, const Tuning& t, bool host, bool publish,
                    const std::vector<PageSlot>& pairs, RunPlan* rp)
{
    const bool permute = (g.inner == KVX_HND) && g.num_heads > 1 && g.page_size > 1;
    if (t.coalesce_runs == 0 || permute || !g.pages_adjacent || pairs.size() < 2) return false;
    plan_runs(g, pairs, &rp->runs);
    if (rp->runs.size() == pairs.size()) return false;
    const int64_t round = int64_t(kThreads) * kVecBytes;
    const int64_t piece_chunk = round * unroll_for(g, t, host);
    // what the pairs would take (tail units where they apply)
    TailPlan tp;
    const int64_t piece_units = pair_units(plan_tails(g, t, host, publish, &tp) ? &tp : nullptr,
                                           (g.piece_bytes + piece_chunk - 1) / piece_chunk,
                                           static_cast<int64_t>(pairs.size()));
    int64_t span = 0;
    for (const Run& r : rp->runs) {
        const int64_t b = int64_t(r.count) * g.piece_bytes;
        if (b >= (int64_t(1) << 31)) return false;   // a buffer resource spans < 2 GiB
        span += b;
    }
    // the unit of a piece of the runs' average span
    int max_unroll = static_cast<int>(t.max_unroll);
    if (host) max_unroll = std::min(max_unroll, 2);
    rp->unroll = pick_unroll(span / int64_t(rp->runs.size()), max_unroll, static_cast<int>(t.unit_rounds));
    const int64_t chunk = round * rp->unroll;
    int64_t units = 0;
    for (const Run& r : rp->runs) units += (int64_t(r.count) * g.piece_bytes + chunk - 1) / chunk;
    // only for a clear gain: a few accidental runs in a fragmented list
    // would mostly add launches (fewer runs than pairs fit one)
    if (4 * units > 3 * piece_units) return false;
    rp->units_lc = units;
    return true;
}

// The device-memory form of a launch's list: (page, slot) per pair, or
// (page, slot, pages, first unit) per run with the first units of a single
// launch over all runs.
std::vector<int32_t> pair_words(const std::vector<PageSlot>& pairs)
{
    std::vector<int32_t> w(2 * pairs.size());
    for (size_t j = 0; j < pairs.size(); j++) {
        w[2 * j] = pairs[j].page;
        w[2 * j + 1] = pairs[j].slot;
    }
    return w;
}

std::vector<int32_t> run_words(const PoolGeom& g, const RunPlan& rp)
{
    const int64_t chunk = int64_t(kThreads) * kVecBytes * rp.unroll;
    std::vector<int32_t> w(4 * rp.runs.size());
    int64_t units = 0;
    for (size_t j = 0; j < rp.runs.size(); j++) {
        const Run& r = rp.runs[j];
        w[4 * j] = r.page;
        w[4 * j + 1] = r.slot;
        w[4 * j + 2] = r.count;
        w[4 * j + 3] = static_cast<int32_t>(units);
        units += (int64_t(r.count) * g.piece_bytes + chunk - 1) / chunk;
    }
    return w;
}

// pairs: (page, slot) in visiting order; NULL: ids[i] in slot i, caller order.
// rp: launch over the plan's runs instead (pairs then unused).
// dev_list: the same pairs (or runs) in device memory (pair_words /
// run_words): one launch over all of them.
int launch_range(Dir dir, const kvx_pool* pool, const Target& tg, int32_t la, int32_t lb,
                 const PageSlot* pairs, size_t npairs, const Publish* pub, const Tuning& t,
                 int cu_count, hipStream_t s, const int32_t* ids = nullptr, const RunPlan* rp = nullptr,
                 const int32_t* dev_list = nullptr)
{
    const PoolGeom& g = pool->geom;
    MoveArgs a;
    std::memset(&a, 0, sizeof a);
    LaunchCfg cfg;
    cfg.host_link = tg.host;
    setup_geom(pool, tg.host, t, &a.g, &cfg);
    if (rp) {
        // whole runs, never reordered rows (the plan requires the same inner layout)
        cfg.unroll = rp->unroll;
        cfg.permute = 0;
        a.g.chunk_bytes = static_cast<uint32_t>(kThreads * kVecBytes * rp->unroll);
        a.g.runs = 1;
    }
    cfg.publish = pub != nullptr;
    // cache policy (measured on MI355X): HBM to HBM, non-temporal loads and
    // non-temporal device-scope stores; into pinned host memory, non-temporal
    // loads and device-scope stores; out of pinned host memory, plain loads
    int cp = 7;
    if (tg.host) cp = (dir == GATHER) ? 5 : 6;
    cfg.cache_policy = t.cache_policy >= 0 ? static_cast<int>(t.cache_policy) : cp;
    a.s.packed = tg.packed;
    a.s.pk_lc_stride = tg.pk_slots * g.piece_bytes;
    a.s.pk_layer0 = tg.pk_layer0;
    a.s.pk_slot0 = tg.pk_slot0;
    set_publish(pub, &a.p);
    const int64_t limit = (int64_t(1) << 31) - 1;
    // tail units (not for a publishing call whose target is counted outside
    // this launch sequence: the staged path's chunks)
    TailPlan tp;
    const bool tails = !rp && (!pub || pub->target_here) && plan_tails(g, t, tg.host, pub != nullptr, &tp);
    if (tails) {
        cfg.unroll = tp.unroll;
        a.g.chunk_bytes = static_cast<uint32_t>(kThreads * kVecBytes * tp.unroll);
        a.g.chunks_per_piece = static_cast<uint32_t>((g.piece_bytes + a.g.chunk_bytes - 1) / a.g.chunk_bytes);
        a.g.tails_per_wave = tp.tails_per_wave;
        a.g.main_units = tp.main_units;
        a.g.tail_bytes = tp.tail_bytes;
    }
    // work units of one (layer, kv) of a launch over np pairs
    auto units_of = [&](int64_t np) -> int64_t {
        return pair_units(tails ? &tp : nullptr, a.g.chunks_per_piece, np);
    };

    // launches over layers [la, lb) of the pairs or runs now in `a`, each
    // (layer, kv) holding per_lc work units
    auto launch_layers = [&](int64_t per_lc) -> int {
        const int64_t per_layer = g.num_kv * per_lc;
        if (per_layer > limit) return fail(KVX_E_INVAL, "one layer of this call has too many work units");
        const int32_t step = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(lb - la, limit / per_layer)));
        for (int32_t l = la; l < lb; l += step) {
            const int32_t nl = std::min(step, lb - l);
            a.s.layer_begin = l;
            a.s.total_units = static_cast<uint32_t>(per_layer * nl);
            // Grid policy, all measured on MI355X:
            //  - a kernel streaming over the host link needs only a few
            //    workgroups (32 x 32 KiB in flight covers the link's round
            //    trip); more only take compute units from concurrent work;
            //  - a publishing workgroup fences once per layer it leaves, so
            //    each gets a few units of every layer;
            //  - HBM-to-HBM with units of >= 32 KiB: one workgroup per unit,
            //    numbered so each XCD takes consecutive units and chunk
            //    offsets rotate between pieces (5-8% over a persistent grid);
            //  - smaller units share persistent workgroups (32 per CU).
            int64_t gmax;
            uint32_t order = 0;
            if (t.grid_max > 0) {
                gmax = t.grid_max;
            } else if (tg.host) {
                gmax = t.host_grid_max > 0 ? t.host_grid_max : tg.host_grid > 0 ? tg.host_grid : kHostGridAuto;
            } else if (pub) {
                gmax = std::min<int64_t>(int64_t(cu_count) * 8, std::max<int64_t>(cu_count, per_layer / 4));
            } else if (a.g.chunk_bytes >= (32u << 10)) {
                gmax = a.s.total_units;
                order = a.g.runs ? 1 : 3;   // chunk rotation is per piece
            } else {
                gmax = int64_t(cu_count) * 32;
            }
            if (t.unit_order >= 0) order = static_cast<uint32_t>(t.unit_order);
            if (a.g.runs) order &= 1u;
            a.g.unit_order = order;
            int64_t grid = std::max<int64_t>(1, std::min<int64_t>(a.s.total_units, gmax));
            if ((order & 1u) && grid > 8) grid &= ~int64_t(7);   // whole rounds of 8 XCDs
            cfg.grid = static_cast<int>(grid);
            // publishing kernels draw blocks of units: one per draw over the
            // host link (a slow read holds back one unit); in device memory,
            // where each count's L2 write-back is what costs, blocks of about
            // 2 MiB that tile each layer, at least one per workgroup.
            // Measured on the device path, restore with publish: llama8b
            // 5.37 TB/s, trtllm_hnd 6.00, mla_fp8 4.94 (16, 32 and 16 units),
            // against 4.15, 3.28 and 2.11 one unit per draw; blocks that
            // straddle layers (mla_fp8, 14 or 15 units) lose about 12%.
            // Among the block sizes that tile a layer, from that size down
            // to half of it (smaller blocks mean more counts: one unit per
            // draw ran the MLA pool at 2.1 TB/s), the one whose last round of
            // draws is fullest: the fewest units a workgroup may have to move
            // (rounds x block), ties to the larger block. Measured on the MLA
            // pool's 144 KiB pieces as 9 MiB runs (72 units of 128 KiB a
            // layer): 12-unit blocks left the second round 43% full
            // (4.46 TB/s).
            if (pub && !tg.host) {
                int64_t b = t.publish_block;
                if (b <= 0) {
                    // bytes a unit moves: its capacity, or the whole short
                    // pieces it holds
                    int64_t unit_bytes = a.g.chunk_bytes;
                    if (tails && tp.main_units == 0)
                        unit_bytes = std::min<int64_t>(unit_bytes, int64_t(4) * tp.tails_per_wave * tp.tail_bytes);
                    const int64_t bmax = std::max<int64_t>(1, std::min<int64_t>(
                        kPublishBlockBytes / unit_bytes, std::max<int64_t>(1, a.s.total_units / grid)));
                    int64_t best = 1, best_cost = INT64_MAX;
                    for (int64_t c = bmax; c >= std::max<int64_t>(1, bmax / 2); c--) {
                        if (per_layer % c != 0) continue;
                        const int64_t blocks = (a.s.total_units + c - 1) / c;
                        const int64_t cost = (blocks + grid - 1) / grid * c;
                        if (cost < best_cost) {
                            best = c;
                            best_cost = cost;
                        }
                    }
                    if (best_cost == INT64_MAX) {   // no size in the range tiles a layer
                        best = bmax;
                        while (best > 1 && per_layer % best != 0) best--;
                    }
                    b = best;
                }
                a.p.block = static_cast<uint32_t>(b);
            }
            hipError_t e = launch_move(dir, cfg, a, s);
            if (e != hipSuccess) return hip_fail(e, "kernel launch");
        }
        return KVX_OK;
    };

    // a list in device memory (run_words / pair_words of the same list) is
    // read by one launch over all of it
    a.list = dev_list;
    if (rp) {
        // runs per launch: at most kMaxRuns, spread evenly over the launches
        const size_t nr = rp->runs.size();
        const size_t nl = dev_list ? 1 : (nr + kMaxRuns - 1) / kMaxRuns;
        const size_t per_launch = (nr + nl - 1) / nl;
        const int64_t chunk = a.g.chunk_bytes;
        if (pub && pub->target_here) {
            int64_t units = 0;
            for (const Run& r : rp->runs) units += (int64_t(r.count) * g.piece_bytes + chunk - 1) / chunk;
            if (g.num_kv * units >= (int64_t(1) << 32))
                return fail(KVX_E_INVAL, "too many work units for per-layer publish");
            a.p.layer_target = static_cast<uint32_t>(g.num_kv * units);
        }
        for (size_t r0 = 0; r0 < nr; r0 += per_launch) {
            const size_t k = std::min(per_launch, nr - r0);
            int64_t units = 0;
            for (size_t j = 0; j < k; j++) {
                const Run& r = rp->runs[r0 + j];
                if (!dev_list) {
                    a.pairs[4 * j] = r.page;
                    a.pairs[4 * j + 1] = r.slot;
                    a.pairs[4 * j + 2] = r.count;
                    a.pairs[4 * j + 3] = static_cast<int32_t>(units);
                }
                units += (int64_t(r.count) * g.piece_bytes + chunk - 1) / chunk;
            }
            if (units > limit) return fail(KVX_E_INVAL, "one layer of this call has too many work units");
            a.s.npairs = static_cast<uint32_t>(k);
            a.g.units_lc = static_cast<uint32_t>(units);
            const int rc = launch_layers(units);
            if (rc != KVX_OK) return rc;
        }
        return KVX_OK;
    }
    // pairs per launch: at most kMaxPairs, spread evenly over the launches
    // (512 pages as 256 + 256, not 448 + 64); all of a list in device memory
    const size_t launches = dev_list ? 1 : (npairs + kMaxPairs - 1) / kMaxPairs;
    const size_t per_launch = npairs ? (npairs + launches - 1) / launches : 1;
    if (pub && pub->target_here) {
        int64_t units = 0;
        for (size_t p0 = 0; p0 < npairs; p0 += per_launch)
            units += units_of(static_cast<int64_t>(std::min<size_t>(per_launch, npairs - p0)));
        if (g.num_kv * units >= (int64_t(1) << 32))
            return fail(KVX_E_INVAL, "too many work units for per-layer publish");
        a.p.layer_target = static_cast<uint32_t>(g.num_kv * units);
    }
    for (size_t p0 = 0; p0 < npairs; p0 += per_launch) {
        const size_t np = std::min<size_t>(per_launch, npairs - p0);
        for (size_t j = 0; j < np && !dev_list; j++) {
            a.pairs[2 * j] = pairs ? pairs[p0 + j].page : ids[p0 + j];
            a.pairs[2 * j + 1] = pairs ? pairs[p0 + j].slot : static_cast<int32_t>(p0 + j);
        }
        a.s.npairs = static_cast<uint32_t>(np);
        a.g.units_lc = static_cast<uint32_t>(units_of(static_cast<int64_t>(np)));
        const int rc = launch_layers(units_of(static_cast<int64_t>(np)));
        if (rc != KVX_OK) return rc;
    }
    return KVX_OK;
}

// ---------------------------------------------------------------------------
// the operation
// ---------------------------------------------------------------------------
// A slot-addressed host pool: page ids[i] lands in (or comes from) slot
// slots[i] of a buffer holding `num` slots per (layer, kv). NULL in the
// functions below means the packed buffer (slot i, n slots).
struct HostSlots {
    const int32_t* slots;
    int64_t num;
};

int enqueue(kvx_pool* pool, Dir dir, const int32_t* ids, int32_t n, uint8_t* host, uint8_t* view,
            int32_t l0, int32_t l1, kvx_ready* ready, int32_t slot_base, hipStream_t s,
            int32_t path, const Tuning& t, Lane* L, const HostSlots* hs);

// Checks of one BACKUP or RESTORE that need no HIP call: layer range, page
// list, ready object, packed buffer size and alignment. Leaves *active false
// when there is nothing to move (n == 0 or an empty layer range).
int validate_side(const kvx_pool* pool, Dir dir, const int32_t* ids, int32_t n, const void* buf,
                  uint64_t buf_bytes, int32_t l0, int32_t l1, const kvx_ready* ready,
                  int32_t slot_base, const std::string& op, bool* active,
                  const HostSlots* hs = nullptr)
{
    const PoolGeom& g = pool->geom;
    *active = false;
    if (l0 < 0 || l1 > g.num_layers || l0 > l1)
        return fail(KVX_E_RANGE, op + ": layer range [" + std::to_string(l0) + ", " +
                                     std::to_string(l1) + ") is outside [0, " +
                                     std::to_string(g.num_layers) + ")");
    int rc = check_page_ids(g, ids, n, dir == SCATTER);
    if (rc != KVX_OK) return rc;
    if (hs) {
        if (hs->num < 0)
            return fail(KVX_E_RANGE, op + ": num_host_slots " + std::to_string(hs->num) + " is negative");
        // a backup writes each named slot once; a restore may read one slot
        // into several pages
        rc = check_host_slots(hs->slots, n, hs->num, dir == GATHER);
        if (rc != KVX_OK) return rc;
    }
    if (ready) {
        if (!ready_known(ready)) return fail(KVX_E_INVAL, op + ": unknown ready handle");
        if (!ready->live.load()) return fail(KVX_E_STALE, op + ": ready object was destroyed");
        if (ready->generation != pool->generation)
            return fail(KVX_E_STALE, op + ": ready object generation " +
                                         std::to_string(ready->generation) +
                                         " does not match pool generation " +
                                         std::to_string(pool->generation));
        if (slot_base < 0 || int64_t(slot_base) + l1 > ready->num_slots)
            return fail(KVX_E_RANGE, op + ": slots [" + std::to_string(int64_t(slot_base) + l0) +
                                         ", " + std::to_string(int64_t(slot_base) + l1) +
                                         ") are outside the ready object's " +
                                         std::to_string(ready->num_slots) + " slots");
    }
    if (n == 0 || l0 == l1) return KVX_OK;
    if (!buf) return fail(KVX_E_INVAL, op + ": packed buffer is NULL");
    const int64_t need = g.num_layers * g.num_kv * (hs ? hs->num : int64_t(n)) * g.piece_bytes;
    if (buf_bytes < static_cast<uint64_t>(need))
        return fail(KVX_E_RANGE, op + ": packed buffer holds " + std::to_string(buf_bytes) +
                                     " bytes, needs " + std::to_string(need));
    if (reinterpret_cast<uintptr_t>(buf) % kVecBytes != 0)
        return fail(KVX_E_ALIGN, op + ": packed buffer is not 16-byte aligned");
    if (ready && int64_t(n) * g.num_kv * ((g.piece_bytes + 4095) / 4096) >= (int64_t(1) << 32))
        return fail(KVX_E_INVAL, op + ": too many pages for per-layer publish");
    *active = true;
    return KVX_OK;
}

// The memory kind `path` needs for a packed buffer (HIP call); *view is its
// device view.
int check_packed_kind(const kvx_pool* pool, void* buf, int32_t path, const std::string& op,
                      uint8_t** view)
{
    const MemKind kind = classify(buf, pool->device, view);
    if (path == KVX_PATH_DEVICE && kind != MemKind::Device)
        return fail(KVX_E_INVAL, op + ": path DEVICE needs device memory of the pool's GPU");
    if (path != KVX_PATH_DEVICE && kind != MemKind::PinnedHost)
        return fail(kind == MemKind::Device ? KVX_E_INVAL : KVX_E_NOTPINNED,
                    op + (kind == MemKind::Device
                              ? ": host path given device memory"
                              : ": packed buffer is not pinned host memory (pageable memory is "
                                "refused; use kvx_host_alloc)"));
    return KVX_OK;
}

int run_op(kvx_pool* pool, Dir dir, const int32_t* ids, int32_t n, void* buf, uint64_t buf_bytes,
         int32_t l0, int32_t l1, kvx_ready* ready, int32_t slot_base, void* stream_v, int32_t path,
         const HostSlots* hs = nullptr)
{
    clear_error();
    const char* op = hs ? (dir == GATHER ? "backup_slots" : "restore_slots")
                        : (dir == GATHER ? "backup" : "restore");
    if (!pool_known(pool)) return fail(KVX_E_INVAL, std::string(op) + ": unknown pool handle");
    if (!pool->live.load()) return fail(KVX_E_STALE, std::string(op) + ": pool handle was unregistered");
    if (path != KVX_PATH_STAGED && path != KVX_PATH_ZEROCOPY && path != KVX_PATH_DEVICE)
        return fail(KVX_E_INVAL, std::string(op) + ": unknown path " + std::to_string(path));
    if (hs && path == KVX_PATH_STAGED)
        return fail(KVX_E_INVAL, std::string(op) + ": a slot-addressed host pool is moved on the "
                                                   "zero-copy or device path");
    bool active = false;
    int rc = validate_side(pool, dir, ids, n, buf, buf_bytes, l0, l1, ready, slot_base, op, &active, hs);
    if (rc != KVX_OK || !active) return rc;

    // ---- HIP from here on; nothing has been enqueued yet ----
    rc = resolve_device(pool);
    if (rc != KVX_OK) return rc;
    if (ready && ready->device >= 0 && ready->device != pool->device)
        return fail(KVX_E_INVAL, std::string(op) + ": the ready object's counts are on GPU " +
                                     std::to_string(ready->device) + ", the pool on GPU " +
                                     std::to_string(pool->device));
    DeviceGuard dg(pool->device);
    hipStream_t s = static_cast<hipStream_t>(stream_v);
    uint8_t* view = nullptr;
    rc = check_packed_kind(pool, buf, path, op, &view);
    if (rc != KVX_OK) return rc;
    const Tuning t = tuning();
    Lane* L = nullptr;
    std::unique_lock<std::mutex> lk;
    rc = get_lane(pool->device, s, &L, &lk);
    if (rc != KVX_OK) return rc;
    rc = enqueue(pool, dir, ids, n, static_cast<uint8_t*>(buf), view, l0, l1, ready, slot_base, s,
                 path, t, L, hs);
    if (rc != KVX_OK) {
        if (ready) L->counters_dirty = true;   // a partial publish may have left counts
        return rc;
    }
    // remember the end of this operation for teardown
    std::lock_guard<std::mutex> plk(pool->mu);
    hipEvent_t& ev = pool->last_op[s];
    if (!ev) KVX_HIP(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    KVX_HIP(hipEventRecord(ev, s));
    return KVX_OK;
}

// Enqueues the whole operation on `s` (and the lane's side stream). Called
// with the lane locked, after every validation has passed.
int enqueue(kvx_pool* pool, Dir dir, const int32_t* ids, int32_t n, uint8_t* host, uint8_t* view,
            int32_t l0, int32_t l1, kvx_ready* ready, int32_t slot_base, hipStream_t s,
            int32_t path, const Tuning& t, Lane* L, const HostSlots* hs)
{
    const PoolGeom& g = pool->geom;
    int rc = KVX_OK;

    std::vector<PageSlot> pairs;
    order_pairs(ids, hs ? hs->slots : nullptr, n, t.sort_pages != 0, &pairs);

    // runs of adjacent pages (zero-copy and device paths: the staged path
    // cuts layers into slot ranges of its ring)
    RunPlan runs;
    const bool use_runs = path != KVX_PATH_STAGED &&
                          plan_run_units(g, t, path == KVX_PATH_ZEROCOPY, ready != nullptr, pairs, &runs);
    Publish pub;
    const Publish* pubp = nullptr;
    if (ready) {
        rc = lane_counters(L, g.num_layers);
        if (rc != KVX_OK) return rc;
        const int64_t chunk = int64_t(kThreads) * kVecBytes * unroll_for(g, t, path == KVX_PATH_ZEROCOPY);
        pub.layer_done = L->layer_done;
        pub.queue = L->layer_done + L->layer_cap;
        pub.ready = ready->counts_dev + slot_base;
        // the staged path's chunks each launch part of a layer: the target is
        // counted here; the other paths' single launch sequence counts it
        pub.layer_target = static_cast<uint32_t>(g.num_kv * int64_t(n) * ((g.piece_bytes + chunk - 1) / chunk));
        pub.target_here = path != KVX_PATH_STAGED;
        pub.value = static_cast<uint32_t>(n);
        pubp = &pub;
    }
    // A list longer than one launch's kernel arguments carry goes to device
    // memory once, and one launch covers every page and layer, where it was
    // launches of at most kMaxPairs pairs, each over all layers (so a
    // publishing restore finished no layer before its last launch).
    // Measured on MI355X, fragmented 1 GiB requests of a 32-layer K+V pool
    // (TB/s read + write, launches of 448 pairs -> one launch):
    //   piece              pack           unpack         publishing unpack
    //   1 KiB, 16384 pages 3.35 -> 5.01   2.91 -> 3.39   1.54 -> 3.31
    //   2 KiB,  8192 pages 4.44 -> 5.76   4.04 -> 4.76   2.44 -> 4.39
    //   4 KiB,  4096 pages 5.33 -> 4.56   4.80 -> 4.55   3.21 -> 4.65
    //  64 KiB,   512 pages 6.10 -> 6.12   6.07 -> 6.11   4.93 -> 5.03
    // and zero-copy restores 54.3 -> 55.5, 56.0 -> 56.6, 55.3 -> 56.9 GB/s.
    // Plain device-memory kernels of small units (the persistent grid of
    // 4 KiB units above) wait for each unit's page lookup, which the kernel
    // arguments serve from cache: they keep launches of kMaxPairs.
    const int32_t* dev_list = nullptr;
    auto upload_list = [&]() -> int {
        if (dev_list || t.device_lists == 0) return KVX_OK;
        if (use_runs ? runs.runs.size() <= size_t(kMaxRuns) : pairs.size() <= size_t(kMaxPairs)) return KVX_OK;
        const bool host_link = path == KVX_PATH_ZEROCOPY;
        if (!ready && !host_link) {
            TailPlan tp;
            const int unroll = use_runs ? runs.unroll
                                        : plan_tails(g, t, false, false, &tp) ? tp.unroll : unroll_for(g, t, false);
            if (int64_t(kThreads) * kVecBytes * unroll < (32 << 10)) return KVX_OK;
        }
        return lane_upload_list(L, use_runs ? run_words(g, runs) : pair_words(pairs), &dev_list);
    };
    if (path != KVX_PATH_STAGED) {
        rc = upload_list();
        if (rc != KVX_OK) return rc;
        const bool zc = path == KVX_PATH_ZEROCOPY;
        const int link_dir = dir == GATHER ? kLinkWrites : kLinkReads;
        Target tg{view, 0, 0, hs ? hs->num : int64_t(n), zc, zc ? link_grid(L, link_dir, t) : 0};
        rc = launch_range(dir, pool, tg, l0, l1, pairs.data(), pairs.size(), pubp, t, L->cu_count, s,
                          nullptr, use_runs ? &runs : nullptr, dev_list);
        if (rc == KVX_OK && zc) rc = link_record(L, s, link_dir);
    } else {
        // chunks of whole layers when one layer fits a ring slot, else slot
        // ranges of one layer
        const int64_t layer_bytes = g.num_kv * int64_t(n) * g.piece_bytes;
        int64_t slot_bytes = std::max<int64_t>(t.stage_slot_bytes, g.num_kv * g.piece_bytes);
        slot_bytes = (slot_bytes + 4095) / 4096 * 4096;
        const int nslots = static_cast<int>(std::min<int64_t>(8, std::max<int64_t>(2, t.stage_slots)));
        rc = lane_ring(L, slot_bytes, nslots);
        if (rc != KVX_OK) return rc;
        int32_t layers_per_chunk = 1, slots_per_chunk = n;
        if (layer_bytes <= slot_bytes) {
            layers_per_chunk = static_cast<int32_t>(slot_bytes / layer_bytes);
            if (dir == SCATTER) {
                // restore chunks are kept small so early layers publish early,
                // but at least kRestoreChunkMin bytes so each DMA runs at speed
                const int64_t want = t.restore_chunk_layers > 0
                                         ? t.restore_chunk_layers
                                         : (kRestoreChunkMin + layer_bytes - 1) / layer_bytes;
                layers_per_chunk = static_cast<int32_t>(
                    std::max<int64_t>(1, std::min<int64_t>(layers_per_chunk, want)));
            }
        } else {
            slots_per_chunk = static_cast<int32_t>(slot_bytes / (g.num_kv * g.piece_bytes));
        }
        // DMA on the library's side stream (overlaps the next chunk's kernel)
        // or on the caller's stream (stream order alone; no cross-stream
        // events). Auto: the side stream when there is a next chunk to
        // overlap and no other stream's host-link call is in flight, else
        // the caller's stream. Measured on MI355X: the tiny pool's 128 KiB
        // request (one chunk), call to completion: backup 62 -> 32 us,
        // restore 52 -> 24 us on the caller's stream; a 2 GiB llama8b call
        // alone: 56.3 / 55.9 GB/s (backup / restore) with the side stream,
        // 55.5 / 55.3 without; the mixed stream as separate staged calls on
        // four streams: 42.0 GB/s with side streams, 80.4 without.
        const bool one_chunk = (l1 - l0) <= layers_per_chunk && slots_per_chunk >= n;
        const bool on_caller = t.staged_dma_on_caller > 0 ||
                               (t.staged_dma_on_caller < 0 && (one_chunk || link_others(L).all() > 0));
        if (!on_caller && !L->side) KVX_HIP(hipStreamCreateWithFlags(&L->side, hipStreamNonBlocking));
        hipStream_t dma = on_caller ? s : L->side;
        const bool split = dma != s;
        if (dir == SCATTER && split) {
            KVX_HIP(hipEventRecord(L->ev_start, s));
            KVX_HIP(hipStreamWaitEvent(dma, L->ev_start, 0));
        }
        // A restore of several chunks of whole layers starts with one layer
        // and doubles each chunk up to layers_per_chunk, so that layer 0 is
        // published after one layer's copy instead of a whole chunk's
        // (measured on MI355X, the MLA pool's 576 MB restore, call to layer 0
        // published: 0.72-0.77 -> 0.66 ms at the same rate; most of what is
        // left is the host enqueueing the chunks' copies and launches).
        const bool grow = dir == SCATTER && t.restore_chunk_layers <= 0 && !one_chunk &&
                          slots_per_chunk >= n && layers_per_chunk > 1;
        int32_t step = grow ? 1 : layers_per_chunk;
        std::vector<PageSlot> sub;
        for (int32_t la = l0; la < l1 && rc == KVX_OK; la += step, step = std::min(2 * step, layers_per_chunk)) {
            const int32_t lb = std::min(l1, la + step);
            for (int32_t s0 = 0; s0 < n && rc == KVX_OK; s0 += slots_per_chunk) {
                const int32_t s1 = std::min(n, s0 + slots_per_chunk);
                const bool full = (s0 == 0 && s1 == n);
                const PageSlot* cp = pairs.data();
                size_t cn = pairs.size();
                if (!full) {
                    sub.clear();
                    for (const PageSlot& ps : pairs)
                        if (ps.slot >= s0 && ps.slot < s1) sub.push_back(ps);
                    cp = sub.data();
                    cn = sub.size();
                }
                const int r = L->next_slot;
                L->next_slot = (r + 1) % L->nslots;
                uint8_t* slot_mem = L->ring + int64_t(r) * L->slot_bytes;
                Target tg{slot_mem, la, s0, s1 - s0, false};
                const int64_t strip = int64_t(s1 - s0) * g.piece_bytes;
                // host byte offset of (layer l, kv c, slot s0) and of its ring copy
                auto host_off = [&](int32_t l, int64_t c) { return ((int64_t(l) * g.num_kv + c) * n + s0) * g.piece_bytes; };
                auto ring_off = [&](int32_t l, int64_t c) { return ((int64_t(l - la) * g.num_kv + c) * (s1 - s0)) * g.piece_bytes; };
                if (dir == GATHER) {
                    if (split && L->slot_pending[r]) KVX_HIP(hipStreamWaitEvent(s, L->slot_free[r], 0));
                    if (full) rc = upload_list();
                    if (rc != KVX_OK) break;
                    rc = launch_range(dir, pool, tg, la, lb, cp, cn, nullptr, t, L->cu_count, s, nullptr,
                                      nullptr, full ? dev_list : nullptr);
                    if (rc != KVX_OK) break;
                    if (split) {
                        KVX_HIP(hipEventRecord(L->slot_ready[r], s));
                        KVX_HIP(hipStreamWaitEvent(dma, L->slot_ready[r], 0));
                    }
                    if (full) {
                        KVX_HIP(hipMemcpyAsync(host + host_off(la, 0), slot_mem, int64_t(lb - la) * g.num_kv * strip,
                                               hipMemcpyDeviceToHost, dma));
                    } else {
                        for (int32_t l = la; l < lb; l++)
                            for (int64_t c = 0; c < g.num_kv; c++)
                                KVX_HIP(hipMemcpyAsync(host + host_off(l, c), slot_mem + ring_off(l, c), strip,
                                                       hipMemcpyDeviceToHost, dma));
                    }
                    if (split) KVX_HIP(hipEventRecord(L->slot_free[r], dma));
                } else {
                    if (split && L->slot_pending[r]) KVX_HIP(hipStreamWaitEvent(dma, L->slot_free[r], 0));
                    if (full) {
                        KVX_HIP(hipMemcpyAsync(slot_mem, host + host_off(la, 0), int64_t(lb - la) * g.num_kv * strip,
                                               hipMemcpyHostToDevice, dma));
                    } else {
                        for (int32_t l = la; l < lb; l++)
                            for (int64_t c = 0; c < g.num_kv; c++)
                                KVX_HIP(hipMemcpyAsync(slot_mem + ring_off(l, c), host + host_off(l, c), strip,
                                                       hipMemcpyHostToDevice, dma));
                    }
                    if (split) {
                        KVX_HIP(hipEventRecord(L->slot_ready[r], dma));
                        KVX_HIP(hipStreamWaitEvent(s, L->slot_ready[r], 0));
                    }
                    if (full) rc = upload_list();
                    if (rc != KVX_OK) break;
                    rc = launch_range(dir, pool, tg, la, lb, cp, cn, pubp, t, L->cu_count, s, nullptr,
                                      nullptr, full ? dev_list : nullptr);
                    if (rc != KVX_OK) break;
                    if (split) KVX_HIP(hipEventRecord(L->slot_free[r], s));
                }
                L->slot_pending[r] = split;
            }
        }
        if (rc == KVX_OK && dir == GATHER && split) {
            KVX_HIP(hipEventRecord(L->ev_done, dma));
            KVX_HIP(hipStreamWaitEvent(s, L->ev_done, 0));
        }
        // the caller's stream has passed the call once its copies are done
        if (rc == KVX_OK) rc = link_record(L, s, dir == GATHER ? kLinkDmaWrites : kLinkDmaReads);
    }
    return rc;
}

// One side of an exchange: pages in visiting order with their packed slots
// (slots == NULL: slot i), the device view of the packed buffer or host pool
// of pk_slots slots per (layer, kv), and the layer range.
struct XSide {
    const int32_t* pages;
    const int32_t* slots;
    int32_t n;
    void* packed;
    int64_t pk_slots;
    int32_t l0, l1;
    uint8_t* view = nullptr;
};

// Fills side x of launch args `a` with pairs [p0, p0 + per) of `xs`;
// returns the side's work units.
// The side's list in the kernel arguments (fill) or, with a device list,
// only its count; units_of(np) is the side's work units of one (layer, kv).
template <class F>
int64_t exchange_side(const PoolGeom& g, F units_of, const XSide& xs, Side* x, int64_t p0, int64_t per,
                      ExchangeArgs& a, bool backup, bool fill)
{
    const int64_t np = std::max<int64_t>(0, std::min<int64_t>(per, xs.n - p0));
    x->packed = xs.view;
    x->pk_lc_stride = xs.pk_slots * g.piece_bytes;
    x->pk_layer0 = 0;
    x->pk_slot0 = 0;
    x->layer_begin = xs.l0;
    x->npairs = static_cast<uint32_t>(np);
    int32_t* pages = backup ? a.pages_b : a.pages_r;
    for (int64_t j = 0; j < np && fill; j++) pages[j] = xs.pages[p0 + j];
    (backup ? a.first_b : a.first_r) = static_cast<int32_t>(p0);
    return int64_t(xs.l1 - xs.l0) * g.num_kv * units_of(np);
}

template <class F>
int64_t exchange_side(const PoolGeom& g, F units_of, const XSide& xs, Side* x, int64_t p0, int64_t per,
                      ExchangeSlotArgs& a, bool backup, bool fill)
{
    const int64_t np = std::max<int64_t>(0, std::min<int64_t>(per, xs.n - p0));
    x->packed = xs.view;
    x->pk_lc_stride = xs.pk_slots * g.piece_bytes;
    x->pk_layer0 = 0;
    x->pk_slot0 = 0;
    x->layer_begin = xs.l0;
    x->npairs = static_cast<uint32_t>(np);
    int32_t* pairs = backup ? a.pairs_b : a.pairs_r;
    for (int64_t j = 0; j < np && fill; j++) {
        pairs[2 * j] = xs.pages[p0 + j];
        pairs[2 * j + 1] = xs.slots[p0 + j];
    }
    return int64_t(xs.l1 - xs.l0) * g.num_kv * units_of(np);
}

// The device-memory form of an exchange side's list: pages in slot order
// (packed buffers) or (page, slot) pairs (host pools).
void side_words(const XSide& xs, bool slot_pairs, std::vector<int32_t>* w)
{
    for (int32_t j = 0; j < xs.n; j++) {
        w->push_back(xs.pages[j]);
        if (slot_pairs) w->push_back(xs.slots[j]);
    }
}

// The launches of one exchange: each interleaves one share of both sides'
// pages (at most max_pairs per side per launch, spread evenly).
template <class A>
int exchange_launches(kvx_pool* pool, const XSide& bk, const XSide& rs, kvx_ready* ready,
                      int32_t slot_base, hipStream_t s, bool host, const Tuning& t, Lane* L,
                      int64_t max_pairs)
{
    const PoolGeom& g = pool->geom;
    A a;
    std::memset(&a, 0, sizeof a);
    LaunchCfg cfg;
    cfg.host_link = host;
    cfg.cache_policy = 0;   // fixed per side inside the exchange kernel
    setup_geom(pool, host, t, &a.g, &cfg);
    cfg.publish = ready != nullptr;
    // tail units (tails and whole short pieces) as in one-direction launches
    TailPlan tp;
    const bool tails = plan_tails(g, t, host, ready != nullptr, &tp);
    if (tails) {
        cfg.unroll = tp.unroll;
        a.g.chunk_bytes = static_cast<uint32_t>(kThreads * kVecBytes * tp.unroll);
        a.g.chunks_per_piece = static_cast<uint32_t>((g.piece_bytes + a.g.chunk_bytes - 1) / a.g.chunk_bytes);
        a.g.tails_per_wave = tp.tails_per_wave;
        a.g.main_units = tp.main_units;
        a.g.tail_bytes = tp.tail_bytes;
    }
    const int64_t cpp = a.g.chunks_per_piece;
    auto units_of = [&](int64_t np) { return pair_units(tails ? &tp : nullptr, cpp, np); };
    // lists longer than the kernel arguments carry: both sides in device
    // memory and one launch
    const int32_t* dev = nullptr;
    if (t.device_lists != 0 && (bk.n > max_pairs || rs.n > max_pairs)) {
        constexpr bool slot_pairs = std::is_same<A, ExchangeSlotArgs>::value;
        std::vector<int32_t> words;
        words.reserve((slot_pairs ? 2 : 1) * (size_t(bk.n) + size_t(rs.n)));
        side_words(bk, slot_pairs, &words);
        const size_t len_b = words.size();
        side_words(rs, slot_pairs, &words);
        const int rc = lane_upload_list(L, words, &dev);
        if (rc != KVX_OK) return rc;
        a.list_b = dev;
        a.list_r = dev + len_b;
    }
    const int64_t launches = dev ? 1
                                 : std::max<int64_t>((bk.n + max_pairs - 1) / max_pairs,
                                                     (rs.n + max_pairs - 1) / max_pairs);
    const int64_t per_b = (bk.n + launches - 1) / launches;
    const int64_t per_r = (rs.n + launches - 1) / launches;
    Publish pub;
    pub.layer_done = L->layer_done;
    pub.queue = L->layer_done + L->layer_cap;
    if (ready) {
        // the RESTORE side's units of one layer over all launches
        int64_t units = 0;
        for (int64_t k = 0; k < launches; k++)
            units += units_of(std::max<int64_t>(0, std::min<int64_t>(per_r, rs.n - k * per_r)));
        if (g.num_kv * units >= (int64_t(1) << 32))
            return fail(KVX_E_INVAL, "exchange: too many work units for per-layer publish");
        pub.ready = ready->counts_dev + slot_base;
        pub.layer_target = static_cast<uint32_t>(g.num_kv * units);
        pub.value = static_cast<uint32_t>(rs.n);
    }
    set_publish(&pub, &a.p);
    a.g.unit_order = 0;
    for (int64_t k = 0; k < launches; k++) {
        const int64_t ub = exchange_side(g, units_of, bk, &a.b, k * per_b, per_b, a, true, !dev);
        const int64_t ur = exchange_side(g, units_of, rs, &a.r, k * per_r, per_r, a, false, !dev);
        if (ub + ur >= (int64_t(1) << 31))
            return fail(KVX_E_INVAL, "exchange: one launch would have too many work units");
        a.b.total_units = static_cast<uint32_t>(ub);
        a.r.total_units = static_cast<uint32_t>(ur);
        // grid: over the host link, the two single-direction host grids
        // together (measured: 64 workgroups sustain 90-91 GB/s for both
        // directions); in device memory, one workgroup per CU drawing blocks
        // of units (KVX_OPT_PUBLISH_BLOCK; auto: about 1 MiB of each side,
        // at least one block per workgroup), so the restore side counts once
        // per block. Measured on the device path with publish, half the
        // layers each way: llama8b 5.45 TB/s, mla_fp8 4.92, against 4.48 and
        // 2.82 with 8 workgroups per CU and one unit per draw.
        int64_t gmax;
        if (t.grid_max > 0)
            gmax = t.grid_max;
        else if (host)
            gmax = 2 * (t.host_grid_max > 0 ? t.host_grid_max : kHostGridAuto);
        else
            gmax = L->cu_count;
        cfg.grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ub + ur, gmax)));
        a.p.block = 1;
        if (!host) {
            int64_t b = t.publish_block;
            // bytes a unit moves: its capacity, or the whole short pieces it holds
            int64_t unit_bytes = a.g.chunk_bytes;
            if (tails && tp.main_units == 0)
                unit_bytes = std::min<int64_t>(unit_bytes, int64_t(4) * tp.tails_per_wave * tp.tail_bytes);
            if (b <= 0)
                b = std::min<int64_t>(std::max<int64_t>(1, kPublishBlockBytes / unit_bytes),
                                      std::max<int64_t>(1, (ub + ur) / cfg.grid));
            a.p.block = static_cast<uint32_t>(b);
        }
        const hipError_t e = launch_exchange(cfg, a, s);
        if (e != hipSuccess) return hip_fail(e, "exchange kernel launch");
    }
    return KVX_OK;
}

// BACKUP and RESTORE sides of kvx_exchange / kvx_exchange_slots, enqueued as
// launches that each interleave one share of the pages of both sides.
int run_exchange(kvx_pool* pool, XSide bk, XSide rs, kvx_ready* ready, int32_t slot_base,
                 void* stream_v, int32_t path)
{
    const PoolGeom& g = pool->geom;
    const bool host = path == KVX_PATH_ZEROCOPY;
    int rc = resolve_device(pool);
    if (rc != KVX_OK) return rc;
    if (ready && ready->device >= 0 && ready->device != pool->device)
        return fail(KVX_E_INVAL, "exchange: the ready object's counts are on GPU " +
                                     std::to_string(ready->device) + ", the pool on GPU " +
                                     std::to_string(pool->device));
    DeviceGuard dg(pool->device);
    hipStream_t s = static_cast<hipStream_t>(stream_v);
    rc = check_packed_kind(pool, bk.packed, path, "exchange backup", &bk.view);
    if (rc != KVX_OK) return rc;
    rc = check_packed_kind(pool, rs.packed, path, "exchange restore", &rs.view);
    if (rc != KVX_OK) return rc;
    const Tuning t = tuning();
    Lane* L = nullptr;
    std::unique_lock<std::mutex> lk;
    rc = get_lane(pool->device, s, &L, &lk);
    if (rc != KVX_OK) return rc;
    rc = lane_counters(L, g.num_layers);   // the unit queue, and the publish counters
    if (rc != KVX_OK) return rc;
    rc = bk.slots ? exchange_launches<ExchangeSlotArgs>(pool, bk, rs, ready, slot_base, s, host, t, L,
                                                        kMaxSlotPairs)
                  : exchange_launches<ExchangeArgs>(pool, bk, rs, ready, slot_base, s, host, t, L,
                                                    kMaxPairs);
    if (rc != KVX_OK) {
        L->counters_dirty = true;   // a partial launch may have left counts and the queue
        return rc;
    }
    std::lock_guard<std::mutex> plk(pool->mu);
    hipEvent_t& ev = pool->last_op[s];
    if (!ev) KVX_HIP(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    KVX_HIP(hipEventRecord(ev, s));
    return KVX_OK;
}

}  // namespace
}  // namespace kvx

using namespace kvx;

// ===========================================================================
// exported C ABI
// ===========================================================================
extern "C" {

int kvx_version(void) { return KVX_ABI_VERSION; }

const char* kvx_last_error(void) { return t_error.c_str(); }

int kvx_register_pool(const kvx_layout* layout, void* base, uint64_t byte_offset,
                      uint32_t dtype_bytes, int32_t ndim, const int64_t* shape,
                      const int64_t* stride, uint64_t generation, kvx_pool** out)
{
    clear_error();
    if (!out) return fail(KVX_E_INVAL, "register: out is NULL");
    *out = nullptr;
    PoolGeom g;
    int rc = derive_geometry(layout, base, byte_offset, dtype_bytes, ndim, shape, stride, &g);
    if (rc != KVX_OK) return rc;
    kvx_pool* p = new (std::nothrow) kvx_pool();
    if (!p) return fail(KVX_E_NOMEM, "register: out of host memory");
    p->geom = g;
    p->base = static_cast<uint8_t*>(base);
    p->byte_offset = byte_offset;
    p->start = p->base + byte_offset;
    p->generation = generation;
    {
        std::lock_guard<std::mutex> lk(g_reg_mu);
        g_pools.insert(p);
    }
    *out = p;
    return KVX_OK;
}

int kvx_unregister_pool(kvx_pool* pool)
{
    clear_error();
    if (!pool) return KVX_OK;
    if (!pool_known(pool)) {
        log_warn("unregister: unknown pool handle ignored");
        return fail(KVX_E_INVAL, "unregister: unknown pool handle");
    }
    if (!pool->live.exchange(false)) {
        log_warn("unregister: pool handle was already unregistered");
        return KVX_OK;
    }
    std::lock_guard<std::mutex> lk(pool->mu);
    if (pool->device >= 0) {
        DeviceGuard dg(pool->device);
        for (auto& kv : pool->last_op) {
            hipError_t e = hipEventSynchronize(kv.second);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                log_warn(std::string("unregister: waiting for in-flight work failed: ") +
                         hipGetErrorString(e));
            }
            if (hipEventDestroy(kv.second) != hipSuccess) (void)hipGetLastError();
        }
    }
    pool->last_op.clear();
    return KVX_OK;
}

int kvx_pool_get_info(const kvx_pool* pool, kvx_pool_info* info)
{
    clear_error();
    if (!pool_known(pool)) return fail(KVX_E_INVAL, "pool_get_info: unknown pool handle");
    if (!pool->live.load()) return fail(KVX_E_STALE, "pool_get_info: pool handle was unregistered");
    if (!info) return fail(KVX_E_INVAL, "pool_get_info: info is NULL");
    const PoolGeom& g = pool->geom;
    info->row_bytes = g.row_bytes;
    info->piece_bytes = g.piece_bytes;
    info->page_stride = g.page_stride;
    info->layer_stride = g.layer_stride;
    info->kv_stride = g.kv_stride;
    info->pool_bytes = g.pool_bytes;
    info->generation = pool->generation;
    return KVX_OK;
}

int kvx_packed_bytes(const kvx_pool* pool, int32_t n, uint64_t* bytes)
{
    clear_error();
    if (!pool_known(pool)) return fail(KVX_E_INVAL, "packed_bytes: unknown pool handle");
    if (!pool->live.load()) return fail(KVX_E_STALE, "packed_bytes: pool handle was unregistered");
    if (n < 0 || !bytes) return fail(KVX_E_INVAL, "packed_bytes: bad arguments");
    const PoolGeom& g = pool->geom;
    *bytes = static_cast<uint64_t>(g.num_layers * g.num_kv * int64_t(n) * g.piece_bytes);
    return KVX_OK;
}

int kvx_backup(kvx_pool* pool, const int32_t* page_ids, int32_t n, void* dst, uint64_t dst_bytes,
               int32_t layer_begin, int32_t layer_end, void* stream, int32_t path)
{
    const TraceRange tr("kvx_backup");
    return run_op(pool, GATHER, page_ids, n, dst, dst_bytes, layer_begin, layer_end, nullptr, 0,
                stream, path);
}

int kvx_restore(kvx_pool* pool, const void* src, uint64_t src_bytes, const int32_t* page_ids,
                int32_t n, int32_t layer_begin, int32_t layer_end, kvx_ready* ready,
                int32_t slot_base, void* stream, int32_t path)
{
    const TraceRange tr("kvx_restore");
    return run_op(pool, SCATTER, page_ids, n, const_cast<void*>(src), src_bytes, layer_begin,
                layer_end, ready, slot_base, stream, path);
}

int kvx_restore_noalloc(kvx_pool* pool, const void* src, uint64_t src_bytes, const int32_t* page_ids,
                        int32_t n, int32_t layer_begin, int32_t layer_end, kvx_ready* ready,
                        int32_t slot_base, void* stream, int32_t path)
{
    const TraceRange tr("kvx_restore_noalloc");
    clear_error();
    if (!pool_known(pool)) return fail(KVX_E_INVAL, "restore_noalloc: unknown pool handle");
    if (!pool->live.load()) return fail(KVX_E_STALE, "restore_noalloc: pool handle was unregistered");
    if (path != KVX_PATH_ZEROCOPY && path != KVX_PATH_DEVICE)
        return fail(KVX_E_INVAL, "restore_noalloc: runs on the zero-copy or device path (the staged "
                                 "path needs the library's staging ring)");
    if (pool->geom.num_layers > kNoAllocMaxLayers)
        return fail(KVX_E_RANGE, "restore_noalloc: the pool has " + std::to_string(pool->geom.num_layers) +
                                     " layers; its scratch serves at most " +
                                     std::to_string(kNoAllocMaxLayers));
    bool active = false;
    int rc = validate_side(pool, SCATTER, page_ids, n, src, src_bytes, layer_begin, layer_end, ready,
                           slot_base, "restore_noalloc", &active);
    if (rc != KVX_OK || !active) return rc;

    // ---- HIP from here on; nothing has been enqueued yet ----
    rc = resolve_device(pool);
    if (rc != KVX_OK) return rc;
    if (ready && ready->device >= 0 && ready->device != pool->device)
        return fail(KVX_E_INVAL, "restore_noalloc: the ready object's counts are on GPU " +
                                     std::to_string(ready->device) + ", the pool on GPU " +
                                     std::to_string(pool->device));
    DeviceGuard dg(pool->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* view = nullptr;
    rc = check_packed_kind(pool, const_cast<void*>(src), path, "restore_noalloc", &view);
    if (rc != KVX_OK) return rc;
    int cu_count = 0;
    KVX_HIP(hipDeviceGetAttribute(&cu_count, hipDeviceAttributeMultiprocessorCount, pool->device));
    const Tuning t = tuning();
    const PoolGeom& g = pool->geom;
    Publish pub;
    const Publish* pubp = nullptr;
    if (ready) {
        uint32_t* scratch = nullptr;
        rc = noalloc_scratch(pool->device, &scratch);
        if (rc != KVX_OK) return rc;
        // the counters and the queue start at zero in stream order (a kernel,
        // not a memset node, for callers that capture the stream)
        KVX_HIP(launch_clear_u32(scratch, static_cast<uint32_t>(g.num_layers), s));
        KVX_HIP(launch_clear_u32(scratch + kNoAllocMaxLayers, 1, s));
        const int64_t chunk = int64_t(kThreads) * kVecBytes * unroll_for(g, t, path == KVX_PATH_ZEROCOPY);
        pub.layer_done = scratch;
        pub.queue = scratch + kNoAllocMaxLayers;
        pub.ready = ready->counts_dev + slot_base;
        pub.layer_target = static_cast<uint32_t>(g.num_kv * int64_t(n) * ((g.piece_bytes + chunk - 1) / chunk));
        pub.target_here = true;
        pub.value = static_cast<uint32_t>(n);
        pubp = &pub;
    }
    // pages in the caller's order, page_ids[i] from packed slot i
    const Target tg{view, 0, 0, int64_t(n), path == KVX_PATH_ZEROCOPY};
    return launch_range(SCATTER, pool, tg, layer_begin, layer_end, nullptr, static_cast<size_t>(n), pubp,
                        t, cu_count, s, page_ids);
}

int kvx_backup_slots(kvx_pool* pool, const int32_t* page_ids, const int32_t* host_slots, int32_t n,
                     void* host_pool, uint64_t host_pool_bytes, int32_t num_host_slots,
                     int32_t layer_begin, int32_t layer_end, void* stream, int32_t path)
{
    const TraceRange tr("kvx_backup_slots");
    const HostSlots hs{host_slots, num_host_slots};
    return run_op(pool, GATHER, page_ids, n, host_pool, host_pool_bytes, layer_begin, layer_end,
                  nullptr, 0, stream, path, &hs);
}

int kvx_restore_slots(kvx_pool* pool, const void* host_pool, uint64_t host_pool_bytes,
                      int32_t num_host_slots, const int32_t* host_slots, const int32_t* page_ids,
                      int32_t n, int32_t layer_begin, int32_t layer_end, kvx_ready* ready,
                      int32_t slot_base, void* stream, int32_t path)
{
    const TraceRange tr("kvx_restore_slots");
    const HostSlots hs{host_slots, num_host_slots};
    return run_op(pool, SCATTER, page_ids, n, const_cast<void*>(host_pool), host_pool_bytes,
                  layer_begin, layer_end, ready, slot_base, stream, path, &hs);
}

int kvx_exchange(kvx_pool* pool, const kvx_xfer* backup, const kvx_xfer* restore, kvx_ready* ready,
                 int32_t slot_base, void* stream, int32_t path)
{
    const TraceRange tr("kvx_exchange");
    clear_error();
    if (!backup || !restore) return fail(KVX_E_INVAL, "exchange: NULL transfer description");
    if (!pool_known(pool)) return fail(KVX_E_INVAL, "exchange: unknown pool handle");
    if (!pool->live.load()) return fail(KVX_E_STALE, "exchange: pool handle was unregistered");
    if (path != KVX_PATH_ZEROCOPY && path != KVX_PATH_DEVICE)
        return fail(KVX_E_INVAL, "exchange: runs on the zero-copy or device path (use kvx_backup and "
                                 "kvx_restore for the staged path)");
    bool ab = false, ar = false;
    int rc = validate_side(pool, GATHER, backup->page_ids, backup->n, backup->packed,
                           backup->packed_bytes, backup->layer_begin, backup->layer_end, nullptr, 0,
                           "exchange backup", &ab);
    if (rc != KVX_OK) return rc;
    rc = validate_side(pool, SCATTER, restore->page_ids, restore->n, restore->packed,
                       restore->packed_bytes, restore->layer_begin, restore->layer_end, ready,
                       slot_base, "exchange restore", &ar);
    if (rc != KVX_OK) return rc;
    if (!ab && !ar) return KVX_OK;
    if (!ar) return kvx_backup(pool, backup->page_ids, backup->n, backup->packed, backup->packed_bytes,
                               backup->layer_begin, backup->layer_end, stream, path);
    if (!ab) return kvx_restore(pool, restore->packed, restore->packed_bytes, restore->page_ids,
                                restore->n, restore->layer_begin, restore->layer_end, ready, slot_base,
                                stream, path);
    // the two sides run concurrently: they must not touch the same bytes
    // (packed bytes: the layer slices each side touches; the packed layout is
    // layer-major, so one request's buffer may serve a backup of some layers
    // and a restore of others)
    const PoolGeom& g = pool->geom;
    const int64_t lay_b = g.num_kv * int64_t(backup->n) * g.piece_bytes;
    const int64_t lay_r = g.num_kv * int64_t(restore->n) * g.piece_bytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(backup->packed) + backup->layer_begin * lay_b;
    const uintptr_t b1 = reinterpret_cast<uintptr_t>(backup->packed) + backup->layer_end * lay_b;
    const uintptr_t r0 = reinterpret_cast<uintptr_t>(restore->packed) + restore->layer_begin * lay_r;
    const uintptr_t r1 = reinterpret_cast<uintptr_t>(restore->packed) + restore->layer_end * lay_r;
    if (b0 < r1 && r0 < b1)
        return fail(KVX_E_INVAL, "exchange: the packed bytes the backup writes overlap those the "
                                 "restore reads");
    if (std::max(backup->layer_begin, restore->layer_begin) <
        std::min(backup->layer_end, restore->layer_end)) {
        std::vector<int32_t> a(backup->page_ids, backup->page_ids + backup->n);
        std::vector<int32_t> b(restore->page_ids, restore->page_ids + restore->n);
        std::sort(a.begin(), a.end());
        std::sort(b.begin(), b.end());
        std::vector<int32_t> both;
        std::set_intersection(a.begin(), a.end(), b.begin(), b.end(), std::back_inserter(both));
        if (!both.empty())
            return fail(KVX_E_INVAL, "exchange: page " + std::to_string(both[0]) +
                                         " is read by the backup and written by the restore in the "
                                         "same layers; run them one after the other");
    }
    const XSide xb{backup->page_ids, nullptr, backup->n, backup->packed, backup->n,
                   backup->layer_begin, backup->layer_end};
    const XSide xr{restore->page_ids, nullptr, restore->n, restore->packed, restore->n,
                   restore->layer_begin, restore->layer_end};
    return run_exchange(pool, xb, xr, ready, slot_base, stream, path);
}

int kvx_exchange_slots(kvx_pool* pool, const kvx_xfer_slots* backup, const kvx_xfer_slots* restore,
                       kvx_ready* ready, int32_t slot_base, void* stream, int32_t path)
{
    const TraceRange tr("kvx_exchange_slots");
    clear_error();
    if (!backup || !restore) return fail(KVX_E_INVAL, "exchange_slots: NULL transfer description");
    if (!pool_known(pool)) return fail(KVX_E_INVAL, "exchange_slots: unknown pool handle");
    if (!pool->live.load()) return fail(KVX_E_STALE, "exchange_slots: pool handle was unregistered");
    if (path != KVX_PATH_ZEROCOPY && path != KVX_PATH_DEVICE)
        return fail(KVX_E_INVAL, "exchange_slots: runs on the zero-copy or device path");
    const HostSlots hb{backup->host_slots, backup->num_host_slots};
    const HostSlots hr{restore->host_slots, restore->num_host_slots};
    bool ab = false, ar = false;
    int rc = validate_side(pool, GATHER, backup->page_ids, backup->n, backup->host_pool,
                           backup->host_pool_bytes, backup->layer_begin, backup->layer_end, nullptr, 0,
                           "exchange_slots backup", &ab, &hb);
    if (rc != KVX_OK) return rc;
    rc = validate_side(pool, SCATTER, restore->page_ids, restore->n, restore->host_pool,
                       restore->host_pool_bytes, restore->layer_begin, restore->layer_end, ready,
                       slot_base, "exchange_slots restore", &ar, &hr);
    if (rc != KVX_OK) return rc;
    if (!ab && !ar) return KVX_OK;
    if (!ar)
        return kvx_backup_slots(pool, backup->page_ids, backup->host_slots, backup->n, backup->host_pool,
                                backup->host_pool_bytes, backup->num_host_slots, backup->layer_begin,
                                backup->layer_end, stream, path);
    if (!ab)
        return kvx_restore_slots(pool, restore->host_pool, restore->host_pool_bytes,
                                 restore->num_host_slots, restore->host_slots, restore->page_ids,
                                 restore->n, restore->layer_begin, restore->layer_end, ready, slot_base,
                                 stream, path);
    // the two sides run concurrently: they must not touch the same bytes
    const PoolGeom& g = pool->geom;
    const bool common_layers = std::max(backup->layer_begin, restore->layer_begin) <
                               std::min(backup->layer_end, restore->layer_end);
    auto intersect = [](const int32_t* x, int32_t nx, const int32_t* y, int32_t ny, int32_t* first) {
        std::vector<int32_t> a(x, x + nx), b(y, y + ny);
        std::sort(a.begin(), a.end());
        std::sort(b.begin(), b.end());
        std::vector<int32_t> both;
        std::set_intersection(a.begin(), a.end(), b.begin(), b.end(), std::back_inserter(both));
        if (!both.empty()) *first = both[0];
        return !both.empty();
    };
    int32_t first = 0;
    if (backup->host_pool == restore->host_pool && backup->num_host_slots == restore->num_host_slots) {
        // one host pool: a slot the backup writes and the restore reads in a
        // common layer
        if (common_layers &&
            intersect(backup->host_slots, backup->n, restore->host_slots, restore->n, &first))
            return fail(KVX_E_INVAL, "exchange_slots: host slot " + std::to_string(first) +
                                         " is written by the backup and read by the restore in the "
                                         "same layers");
    } else {
        const int64_t lay_b = g.num_kv * int64_t(backup->num_host_slots) * g.piece_bytes;
        const int64_t lay_r = g.num_kv * int64_t(restore->num_host_slots) * g.piece_bytes;
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(backup->host_pool) + backup->layer_begin * lay_b;
        const uintptr_t b1 = reinterpret_cast<uintptr_t>(backup->host_pool) + backup->layer_end * lay_b;
        const uintptr_t r0 = reinterpret_cast<uintptr_t>(restore->host_pool) + restore->layer_begin * lay_r;
        const uintptr_t r1 = reinterpret_cast<uintptr_t>(restore->host_pool) + restore->layer_end * lay_r;
        if (b0 < r1 && r0 < b1)
            return fail(KVX_E_INVAL, "exchange_slots: the host bytes the backup writes overlap those "
                                     "the restore reads");
    }
    if (common_layers && intersect(backup->page_ids, backup->n, restore->page_ids, restore->n, &first))
        return fail(KVX_E_INVAL, "exchange_slots: page " + std::to_string(first) +
                                     " is read by the backup and written by the restore in the same "
                                     "layers; run them one after the other");
    const XSide xb{backup->page_ids, backup->host_slots, backup->n, backup->host_pool,
                   backup->num_host_slots, backup->layer_begin, backup->layer_end};
    const XSide xr{restore->page_ids, restore->host_slots, restore->n, restore->host_pool,
                   restore->num_host_slots, restore->layer_begin, restore->layer_end};
    return run_exchange(pool, xb, xr, ready, slot_base, stream, path);
}

int kvx_plan_runs(const kvx_pool* pool, const int32_t* page_ids, int32_t n, int32_t* runs,
                  int32_t max_runs, int32_t* num_runs)
{
    clear_error();
    if (!pool_known(pool)) return fail(KVX_E_INVAL, "plan_runs: unknown pool handle");
    if (!pool->live.load()) return fail(KVX_E_STALE, "plan_runs: pool handle was unregistered");
    if (!num_runs || (max_runs > 0 && !runs) || max_runs < 0)
        return fail(KVX_E_INVAL, "plan_runs: bad output arguments");
    int rc = check_page_ids(pool->geom, page_ids, n, false);
    if (rc != KVX_OK) return rc;
    std::vector<PageSlot> pairs;
    order_pages(page_ids, n, true, &pairs);
    std::vector<Run> rr;
    plan_runs(pool->geom, pairs, &rr);
    *num_runs = static_cast<int32_t>(rr.size());
    for (int32_t k = 0; k < max_runs && k < *num_runs; k++) {
        runs[3 * k] = rr[k].page;
        runs[3 * k + 1] = rr[k].slot;
        runs[3 * k + 2] = rr[k].count;
    }
    return KVX_OK;
}

// ---- memory / misc -------------------------------------------------------------

int kvx_host_alloc(uint64_t bytes, void** out)
{
    clear_error();
    if (!out || bytes == 0) return fail(KVX_E_INVAL, "host_alloc: bad arguments");
    *out = nullptr;
    hipError_t e = hipHostMalloc(out, bytes,
                                 hipHostMallocMapped | hipHostMallocPortable | hipHostMallocNonCoherent);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *out = nullptr;
        return fail(e == hipErrorOutOfMemory ? KVX_E_NOMEM : KVX_E_HIP,
                    std::string("host_alloc: hipHostMalloc failed: ") + hipGetErrorString(e));
    }
    return KVX_OK;
}

int kvx_host_free(void* p)
{
    clear_error();
    if (!p) return KVX_OK;
    hipError_t e = hipHostFree(p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_fail(e, "hipHostFree");
    }
    return KVX_OK;
}

int kvx_alloc_range(const void* ptr, void** base, uint64_t* size)
{
    clear_error();
    if (!ptr || !base || !size) return fail(KVX_E_INVAL, "alloc_range: bad arguments");
    hipDeviceptr_t b = nullptr;
    size_t sz = 0;
    hipError_t e = hipMemGetAddressRange(&b, &sz, const_cast<void*>(ptr));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_fail(e, "hipMemGetAddressRange");
    }
    *base = b;
    *size = sz;
    return KVX_OK;
}

int kvx_release_stream(void* stream)
{
    const TraceRange tr("kvx_release_stream");
    clear_error();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // take the stream's lanes out of the registry, each with its mutex held
    // (a call still enqueueing on one finishes first)
    std::vector<Lane*> gone;
    {
        std::lock_guard<std::mutex> lk(g_lanes_mu);
        for (auto it = g_lanes.begin(); it != g_lanes.end();) {
            if (it->first.second == s) {
                it->second->mu.lock();
                gone.push_back(it->second);
                it = g_lanes.erase(it);
            } else {
                ++it;
            }
        }
    }
    for (Lane* L : gone) {
        lane_free(L);
        L->mu.unlock();
        delete L;
    }
    // the pools' records of their last operation on this stream
    std::vector<kvx_pool*> pools;
    {
        std::lock_guard<std::mutex> lk(g_reg_mu);
        for (const kvx_pool* p : g_pools) pools.push_back(const_cast<kvx_pool*>(p));
    }
    for (kvx_pool* p : pools) {
        std::lock_guard<std::mutex> lk(p->mu);
        auto it = p->last_op.find(s);
        if (it == p->last_op.end()) continue;
        DeviceGuard dg(p->device);
        hipError_t e = hipEventSynchronize(it->second);
        if (e == hipSuccess) e = hipEventDestroy(it->second);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            log_warn(std::string("release_stream: an end-of-operation event failed: ") +
                     hipGetErrorString(e));
        }
        p->last_op.erase(it);
    }
    return KVX_OK;
}

int kvx_sync(void* stream)
{
    clear_error();
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return KVX_OK;
}

int kvx_set_option(int32_t option, int64_t value)
{
    clear_error();
    std::lock_guard<std::mutex> lk(g_tune_mu);
    switch (option) {
    case KVX_OPT_GRID_MAX:
        if (value < 0 || value > (1 << 24)) break;
        g_tune.grid_max = value;
        return KVX_OK;
    case KVX_OPT_STAGE_SLOT_BYTES:
        if (value < (1 << 20) || value > (int64_t(1) << 34)) break;
        g_tune.stage_slot_bytes = value;
        return KVX_OK;
    case KVX_OPT_STAGE_SLOTS:
        if (value < 2 || value > 8) break;
        g_tune.stage_slots = value;
        return KVX_OK;
    case KVX_OPT_SORT_PAGES:
        if (value != 0 && value != 1) break;
        g_tune.sort_pages = value;
        return KVX_OK;
    case KVX_OPT_CACHE_POLICY:
        if (value < -1 || value > 7) break;
        g_tune.cache_policy = value;
        return KVX_OK;
    case KVX_OPT_RESTORE_CHUNK_LAYERS:
        if (value < 0 || value > 4096) break;
        g_tune.restore_chunk_layers = value;
        return KVX_OK;
    case KVX_OPT_HOST_GRID_MAX:
        if (value < 0 || value > (1 << 24)) break;
        g_tune.host_grid_max = value;
        return KVX_OK;
    case KVX_OPT_UNIT_ORDER:
        if (value < -1 || value > 3) break;
        g_tune.unit_order = value;
        return KVX_OK;
    case KVX_OPT_STAGED_DMA_ON_CALLER:
        if (value < -1 || value > 1) break;
        g_tune.staged_dma_on_caller = value;
        return KVX_OK;
    case KVX_OPT_HND_LDS:
        if (value < -1 || value > 1) break;
        g_tune.hnd_lds = value;
        return KVX_OK;
    case KVX_OPT_MAX_UNROLL:
        if (value < 1 || value > 32) break;
        g_tune.max_unroll = value;
        return KVX_OK;
    case KVX_OPT_UNIT_ROUNDS:
        if (value != 0 && value != 1 && value != 2 && value != 3 && value != 4 && value != 6 &&
            value != 8 && value != 12 && value != 16 && value != 32)
            break;
        g_tune.unit_rounds = value;
        return KVX_OK;
    case KVX_OPT_FAIL_ALLOCS:
        if (value < 0 || value > 1000) break;
        g_tune.fail_allocs = value;
        return KVX_OK;
    case KVX_OPT_RING_PAIRING:
        if (value != 0 && value != 1) break;
        g_tune.ring_pairing = value;
        return KVX_OK;
    case KVX_OPT_PUBLISH_BLOCK:
        if (value < 0 || value > 4096) break;
        g_tune.publish_block = value;
        return KVX_OK;
    case KVX_OPT_COALESCE_RUNS:
        if (value != 0 && value != 1) break;
        g_tune.coalesce_runs = value;
        return KVX_OK;
    case KVX_OPT_TAIL_UNITS:
        if (value != 0 && value != 1) break;
        g_tune.tail_units = value;
        return KVX_OK;
    case KVX_OPT_DEVICE_LISTS:
        if (value != 0 && value != 1) break;
        g_tune.device_lists = value;
        return KVX_OK;
    case KVX_OPT_DUPLEX_WRITERS:
        if (value < 0 || value > 1024) break;
        g_tune.duplex_writers = value;
        return KVX_OK;
    case KVX_OPT_DUPLEX_READERS:
        if (value < 0 || value > 1024) break;
        g_tune.duplex_readers = value;
        return KVX_OK;
    default:
        return fail(KVX_E_INVAL, "set_option: unknown option " + std::to_string(option));
    }
    return fail(KVX_E_INVAL, "set_option: value " + std::to_string(value) +
                                 " out of range for option " + std::to_string(option));
}

int kvx_get_option(int32_t option, int64_t* value)
{
    clear_error();
    if (!value) return fail(KVX_E_INVAL, "get_option: value is NULL");
    std::lock_guard<std::mutex> lk(g_tune_mu);
    switch (option) {
    case KVX_OPT_GRID_MAX: *value = g_tune.grid_max; return KVX_OK;
    case KVX_OPT_STAGE_SLOT_BYTES: *value = g_tune.stage_slot_bytes; return KVX_OK;
    case KVX_OPT_STAGE_SLOTS: *value = g_tune.stage_slots; return KVX_OK;
    case KVX_OPT_SORT_PAGES: *value = g_tune.sort_pages; return KVX_OK;
    case KVX_OPT_CACHE_POLICY: *value = g_tune.cache_policy; return KVX_OK;
    case KVX_OPT_RESTORE_CHUNK_LAYERS: *value = g_tune.restore_chunk_layers; return KVX_OK;
    case KVX_OPT_HOST_GRID_MAX: *value = g_tune.host_grid_max; return KVX_OK;
    case KVX_OPT_UNIT_ORDER: *value = g_tune.unit_order; return KVX_OK;
    case KVX_OPT_MAX_UNROLL: *value = g_tune.max_unroll; return KVX_OK;
    case KVX_OPT_UNIT_ROUNDS: *value = g_tune.unit_rounds; return KVX_OK;
    case KVX_OPT_STAGED_DMA_ON_CALLER: *value = g_tune.staged_dma_on_caller; return KVX_OK;
    case KVX_OPT_HND_LDS: *value = g_tune.hnd_lds; return KVX_OK;
    case KVX_OPT_FAIL_ALLOCS: *value = g_tune.fail_allocs; return KVX_OK;
    case KVX_OPT_RING_PAIRING: *value = g_tune.ring_pairing; return KVX_OK;
    case KVX_OPT_PUBLISH_BLOCK: *value = g_tune.publish_block; return KVX_OK;
    case KVX_OPT_COALESCE_RUNS: *value = g_tune.coalesce_runs; return KVX_OK;
    case KVX_OPT_TAIL_UNITS: *value = g_tune.tail_units; return KVX_OK;
    case KVX_OPT_DEVICE_LISTS: *value = g_tune.device_lists; return KVX_OK;
    case KVX_OPT_DUPLEX_WRITERS: *value = g_tune.duplex_writers; return KVX_OK;
    case KVX_OPT_DUPLEX_READERS: *value = g_tune.duplex_readers; return KVX_OK;
    default: return fail(KVX_E_INVAL, "get_option: unknown option " + std::to_string(option));
    }
}

}  // extern "C"
