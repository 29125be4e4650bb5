// ring.h - submission / completion rings between a scheduler process and a
// data-plane process, in POSIX shared memory (host only, no HIP). The C
// entry points are declared in kvx.h; the executor (kvx_ring_serve /
// kvx_ring_drain, which enqueue GPU work) lives in ring_exec.cpp and keeps its
// in-flight list here.
#pragma once

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

#include "kvx_host.h"

namespace kvx {

constexpr uint32_t RING_MAGIC = 0x6b767867u;        // "kvxg": the local handle
constexpr uint32_t RING_SHM_MAGIC = 0x6b767853u;    // "kvxS": the shared header
constexpr uint32_t RING_SHM_VERSION = 2;

static_assert(std::atomic<uint64_t>::is_always_lock_free, "shared atomics must be lock free");
static_assert(std::atomic<int32_t>::is_always_lock_free, "shared atomics must be lock free");

// The shared header. Each index is written by one side only: the SQ tail
// and the CQ head by the creator (scheduler), the SQ head and the CQ tail
// by the opener (data plane). A descriptor or completion is written before
// the release store of the index that publishes it and read after the
// acquire load that observes it.
struct RingShared {
    uint32_t magic;
    uint32_t version;
    uint32_t entries;
    uint32_t reserved;
    uint64_t generation;
    std::atomic<int32_t> creator_pid;
    std::atomic<int32_t> opener_pid;
    std::atomic<uint64_t> creator_start;   // start time (clock ticks since boot)
    std::atomic<uint64_t> opener_start;
    alignas(64) std::atomic<uint64_t> sq_head;
    alignas(64) std::atomic<uint64_t> sq_tail;
    alignas(64) std::atomic<uint64_t> cq_head;
    alignas(64) std::atomic<uint64_t> cq_tail;
    // wakeups: each push bumps its ring's sequence word and, if a waiter
    // has announced itself, wakes it with a futex on that word
    alignas(64) std::atomic<uint32_t> sq_seq;
    std::atomic<uint32_t> sq_waiters;
    alignas(64) std::atomic<uint32_t> cq_seq;
    std::atomic<uint32_t> cq_waiters;
};
static_assert(sizeof(std::atomic<uint32_t>) == 4, "futex words are 32 bits");

// Bytes of the shared object for `entries` descriptors per ring, and the
// offsets of the two arrays in it.
size_t ring_sq_offset();
size_t ring_cq_offset(uint32_t entries);
size_t ring_bytes(uint32_t entries);

// Start time of process `pid` from /proc (0 if it does not exist or has
// exited and awaits its parent).
uint64_t process_start(int32_t pid);

// An operation of the executor, in submission order.
struct RingFlight {
    uint64_t op_id = 0;
    uint64_t generation = 0;
    int32_t status = 0;      // the call's status (KVX_OK: wait for `event`)
    void* event = nullptr;   // hipEvent_t recorded after the operation's work
};

bool ring_known(const kvx_ring* r);

}  // namespace kvx

struct kvx_ring {
    uint32_t magic = kvx::RING_MAGIC;
    std::atomic<bool> live{true};
    bool creator = false;
    std::string name;
    void* map = nullptr;
    size_t map_bytes = 0;
    kvx::RingShared* sh = nullptr;
    kvx_sqe* sq = nullptr;
    kvx_cqe* cq = nullptr;
    uint32_t mask = 0;
    std::mutex mu;

    // executor state (data-plane side, this process only)
    std::deque<kvx::RingFlight> flights;
    std::vector<void*> spare_events;                // fired events, reused by later flights
    void (*release_flights)(kvx_ring*) = nullptr;   // frees events at close

    // SPSC steps, called with `mu` held
    bool push_sqe(const kvx_sqe& e);
    bool pop_sqe(kvx_sqe* e);
    bool push_cqe(const kvx_cqe& e);
    bool pop_cqe(kvx_cqe* e);
    uint32_t cq_room() const;
};
