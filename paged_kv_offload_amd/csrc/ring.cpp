// ring.cpp - submission / completion rings in POSIX shared memory between a
// scheduler process (creator: submits descriptors, reaps completions) and a
// data-plane process (opener: takes descriptors, posts completions). Host
// only; the executor that runs descriptors on the GPU is in ring_exec.cpp.
//
// [RFC] "Device IPC data path" gives the control path its shape (BACKUP /
// RESTORE descriptors, completions), and "Failure and lifecycle handling"
// its rules: operations carry the generation they were issued under, a
// restarted scheduler starts a new generation, and when a peer dies the
// survivor releases what it held for it. Each side therefore records its
// process ID and start time in the ring; either can tell whether the other
// still runs (a reused process ID has another start time).
#include <algorithm>
#include <cerrno>
#include <cstdio>
#include <cstring>
#include <climits>
#include <ctime>
#include <fcntl.h>
#include <linux/futex.h>
#include <new>
#include <sys/syscall.h>
#include <set>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include "ring.h"

namespace kvx {

size_t ring_sq_offset()
{
    return (sizeof(RingShared) + 4095) / 4096 * 4096;
}

size_t ring_cq_offset(uint32_t entries)
{
    return ring_sq_offset() + size_t(entries) * sizeof(kvx_sqe);
}

size_t ring_bytes(uint32_t entries)
{
    return (ring_cq_offset(entries) + size_t(entries) * sizeof(kvx_cqe) + 4095) / 4096 * 4096;
}

uint64_t process_start(int32_t pid)
{
    if (pid <= 0) return 0;
    char path[64];
    std::snprintf(path, sizeof path, "/proc/%d/stat", pid);
    FILE* f = std::fopen(path, "r");
    if (!f) return 0;
    char buf[1024];
    const size_t got = std::fread(buf, 1, sizeof buf - 1, f);
    std::fclose(f);
    buf[got] = 0;
    // fields after the command name (which may hold spaces and parentheses)
    const char* p = std::strrchr(buf, ')');
    if (!p) return 0;
    p++;
    char state = 0;
    unsigned long long start = 0;
    // state is field 3, the start time field 22
    if (std::sscanf(p, " %c %*d %*d %*d %*d %*d %*u %*u %*u %*u %*u %*u %*u %*d %*d %*d %*d %*d %*d %llu",
                    &state, &start) != 2)
        return 0;
    if (state == 'Z' || state == 'X') return 0;   // exited
    return start;
}

namespace {

std::mutex g_ring_mu;
std::set<const kvx_ring*>& rings()
{
    static auto* s = new std::set<const kvx_ring*>();
    return *s;
}

bool name_ok(const char* name)
{
    if (!name || name[0] != '/') return false;
    const size_t len = std::strlen(name);
    if (len < 2 || len >= KVX_RING_NAME_MAX) return false;
    return std::strchr(name + 1, '/') == nullptr;
}

int map_ring(kvx_ring* r, int fd, size_t bytes)
{
    void* m = mmap(nullptr, bytes, PROT_READ | PROT_WRITE, MAP_SHARED, fd, 0);
    if (m == MAP_FAILED) return fail(KVX_E_NOMEM, "ring: mmap failed: " + std::string(std::strerror(errno)));
    r->map = m;
    r->map_bytes = bytes;
    r->sh = static_cast<RingShared*>(m);
    return KVX_OK;
}

void attach_arrays(kvx_ring* r)
{
    auto* base = static_cast<uint8_t*>(r->map);
    r->sq = reinterpret_cast<kvx_sqe*>(base + ring_sq_offset());
    r->cq = reinterpret_cast<kvx_cqe*>(base + ring_cq_offset(r->sh->entries));
    r->mask = r->sh->entries - 1;
}

void add_ring(kvx_ring* r)
{
    std::lock_guard<std::mutex> lk(g_ring_mu);
    rings().insert(r);
}

int open_ring(const kvx_ring* r, const char* op, bool want_creator)
{
    clear_error();
    if (!ring_known(r)) return fail(KVX_E_INVAL, std::string(op) + ": unknown ring handle");
    if (!r->live.load()) return fail(KVX_E_STALE, std::string(op) + ": ring was closed");
    if (r->creator != want_creator)
        return fail(KVX_E_INVAL, std::string(op) + (want_creator ? ": only the ring's creator (scheduler side) may do this"
                                                                 : ": only the side that opened the ring (data plane) may do this"));
    return KVX_OK;
}

}  // namespace

bool ring_known(const kvx_ring* r)
{
    std::lock_guard<std::mutex> lk(g_ring_mu);
    return r && rings().count(r) && r->magic == RING_MAGIC;
}

}  // namespace kvx

using namespace kvx;

namespace {

// futex on a word of the shared mapping (not FUTEX_PRIVATE: the other
// process waits on the same physical word)
void futex_wake_all(std::atomic<uint32_t>* w)
{
    syscall(SYS_futex, reinterpret_cast<uint32_t*>(w), FUTEX_WAKE, INT_MAX, nullptr, nullptr, 0);
}

void futex_wait_for(std::atomic<uint32_t>* w, uint32_t expected, int64_t ns)
{
    struct timespec ts;
    ts.tv_sec = static_cast<time_t>(ns / 1000000000);
    ts.tv_nsec = static_cast<long>(ns % 1000000000);
    syscall(SYS_futex, reinterpret_cast<uint32_t*>(w), FUTEX_WAIT, expected, &ts, nullptr, 0);
}

void bump(std::atomic<uint32_t>& seq, std::atomic<uint32_t>& waiters)
{
    seq.fetch_add(1, std::memory_order_seq_cst);
    if (waiters.load(std::memory_order_seq_cst) != 0) futex_wake_all(&seq);
}

}  // namespace

bool kvx_ring::push_sqe(const kvx_sqe& e)
{
    const uint64_t tail = sh->sq_tail.load(std::memory_order_relaxed);
    if (tail - sh->sq_head.load(std::memory_order_acquire) >= sh->entries) return false;
    sq[tail & mask] = e;
    sh->sq_tail.store(tail + 1, std::memory_order_release);
    bump(sh->sq_seq, sh->sq_waiters);
    return true;
}

bool kvx_ring::pop_sqe(kvx_sqe* e)
{
    const uint64_t head = sh->sq_head.load(std::memory_order_relaxed);
    if (head == sh->sq_tail.load(std::memory_order_acquire)) return false;
    *e = sq[head & mask];
    sh->sq_head.store(head + 1, std::memory_order_release);
    return true;
}

bool kvx_ring::push_cqe(const kvx_cqe& e)
{
    const uint64_t tail = sh->cq_tail.load(std::memory_order_relaxed);
    if (tail - sh->cq_head.load(std::memory_order_acquire) >= sh->entries) return false;
    cq[tail & mask] = e;
    sh->cq_tail.store(tail + 1, std::memory_order_release);
    bump(sh->cq_seq, sh->cq_waiters);
    return true;
}

bool kvx_ring::pop_cqe(kvx_cqe* e)
{
    const uint64_t head = sh->cq_head.load(std::memory_order_relaxed);
    if (head == sh->cq_tail.load(std::memory_order_acquire)) return false;
    *e = cq[head & mask];
    sh->cq_head.store(head + 1, std::memory_order_release);
    return true;
}

uint32_t kvx_ring::cq_room() const
{
    const uint64_t used = sh->cq_tail.load(std::memory_order_relaxed) -
                          sh->cq_head.load(std::memory_order_acquire);
    return used >= sh->entries ? 0u : static_cast<uint32_t>(sh->entries - used);
}

extern "C" {

int kvx_ring_create(const char* name, int32_t entries, uint64_t generation, kvx_ring** out)
{
    clear_error();
    if (!out) return fail(KVX_E_INVAL, "ring_create: out is NULL");
    *out = nullptr;
    if (!name_ok(name))
        return fail(KVX_E_INVAL, "ring_create: the name must be '/' and 1 to " +
                                     std::to_string(KVX_RING_NAME_MAX - 2) + " characters other than '/'");
    if (entries < 2 || entries > 4096 || (entries & (entries - 1)))
        return fail(KVX_E_RANGE, "ring_create: entries " + std::to_string(entries) +
                                     " is not a power of two in [2, 4096]");
    const int fd = shm_open(name, O_CREAT | O_EXCL | O_RDWR, 0600);
    if (fd < 0)
        return fail(errno == EEXIST ? KVX_E_INVAL : KVX_E_NOMEM,
                    std::string("ring_create: shm_open(") + name + ") failed: " + std::strerror(errno));
    const size_t bytes = ring_bytes(static_cast<uint32_t>(entries));
    kvx_ring* r = new (std::nothrow) kvx_ring();
    int rc = KVX_OK;
    if (!r) rc = fail(KVX_E_NOMEM, "ring_create: out of memory");
    if (rc == KVX_OK && ftruncate(fd, static_cast<off_t>(bytes)) != 0)
        rc = fail(KVX_E_NOMEM, "ring_create: ftruncate failed: " + std::string(std::strerror(errno)));
    if (rc == KVX_OK) rc = map_ring(r, fd, bytes);
    close(fd);
    if (rc != KVX_OK) {
        shm_unlink(name);
        delete r;
        return rc;
    }
    r->creator = true;
    r->name = name;
    RingShared* sh = new (r->map) RingShared();
    sh->version = RING_SHM_VERSION;
    sh->entries = static_cast<uint32_t>(entries);
    sh->generation = generation;
    sh->creator_pid.store(static_cast<int32_t>(getpid()));
    sh->creator_start.store(process_start(getpid()));
    sh->opener_pid.store(0);
    sh->opener_start.store(0);
    sh->sq_head.store(0);
    sh->sq_tail.store(0);
    sh->cq_head.store(0);
    sh->cq_tail.store(0);
    sh->sq_seq.store(0);
    sh->sq_waiters.store(0);
    sh->cq_seq.store(0);
    sh->cq_waiters.store(0);
    std::atomic_thread_fence(std::memory_order_release);
    reinterpret_cast<std::atomic<uint32_t>*>(&sh->magic)->store(RING_SHM_MAGIC, std::memory_order_release);
    attach_arrays(r);
    add_ring(r);
    *out = r;
    return KVX_OK;
}

int kvx_ring_open(const char* name, kvx_ring** out)
{
    clear_error();
    if (!out) return fail(KVX_E_INVAL, "ring_open: out is NULL");
    *out = nullptr;
    if (!name_ok(name)) return fail(KVX_E_INVAL, "ring_open: malformed name");
    const int fd = shm_open(name, O_RDWR, 0);
    if (fd < 0)
        return fail(KVX_E_INVAL, std::string("ring_open: shm_open(") + name + ") failed: " + std::strerror(errno));
    struct stat st;
    if (fstat(fd, &st) != 0 || size_t(st.st_size) < ring_sq_offset()) {
        close(fd);
        return fail(KVX_E_INVAL, "ring_open: not a kvx ring (too small)");
    }
    kvx_ring* r = new (std::nothrow) kvx_ring();
    if (!r) {
        close(fd);
        return fail(KVX_E_NOMEM, "ring_open: out of memory");
    }
    int rc = map_ring(r, fd, size_t(st.st_size));
    close(fd);
    if (rc == KVX_OK) {
        const RingShared* sh = r->sh;
        const uint32_t magic = reinterpret_cast<const std::atomic<uint32_t>*>(&sh->magic)->load(std::memory_order_acquire);
        if (magic != RING_SHM_MAGIC || sh->version != RING_SHM_VERSION || sh->entries < 2 ||
            (sh->entries & (sh->entries - 1)) || ring_bytes(sh->entries) != size_t(st.st_size))
            rc = fail(KVX_E_INVAL, "ring_open: not a kvx ring of this version");
    }
    if (rc == KVX_OK) {
        // one data-plane side at a time; a dead one's place may be taken
        const int32_t me = static_cast<int32_t>(getpid());
        int32_t cur = r->sh->opener_pid.load();
        for (;;) {
            if (cur != 0 && process_start(cur) == r->sh->opener_start.load() && process_start(cur) != 0) {
                rc = fail(KVX_E_INVAL, "ring_open: process " + std::to_string(cur) + " has the ring open");
                break;
            }
            if (r->sh->opener_pid.compare_exchange_strong(cur, me)) {
                r->sh->opener_start.store(process_start(me));
                break;
            }
        }
    }
    if (rc != KVX_OK) {
        munmap(r->map, r->map_bytes);
        delete r;
        return rc;
    }
    r->creator = false;
    r->name = name;
    attach_arrays(r);
    add_ring(r);
    *out = r;
    return KVX_OK;
}

int kvx_ring_close(kvx_ring* r)
{
    clear_error();
    if (!r) return KVX_OK;
    {
        std::lock_guard<std::mutex> lk(g_ring_mu);
        if (!rings().count(r) || r->magic != RING_MAGIC || !r->live.exchange(false)) {
            log_warn("ring_close: unknown or already closed ring handle");
            return KVX_OK;
        }
    }
    std::lock_guard<std::mutex> lk(r->mu);
    if (r->release_flights) r->release_flights(r);
    r->flights.clear();
    if (r->creator) {
        if (shm_unlink(r->name.c_str()) != 0)
            log_warn("ring_close: shm_unlink(" + r->name + ") failed: " + std::strerror(errno));
    } else {
        int32_t me = static_cast<int32_t>(getpid());
        r->sh->opener_pid.compare_exchange_strong(me, 0);
        // a creator that died cannot remove the name any more
        const int32_t cp = r->sh->creator_pid.load();
        if (process_start(cp) != r->sh->creator_start.load() || process_start(cp) == 0)
            (void)shm_unlink(r->name.c_str());
    }
    if (munmap(r->map, r->map_bytes) != 0) log_warn("ring_close: munmap failed");
    r->map = nullptr;
    r->sh = nullptr;
    r->sq = nullptr;
    r->cq = nullptr;
    return KVX_OK;
}

int kvx_ring_submit(kvx_ring* r, const kvx_sqe* sqe)
{
    int rc = open_ring(r, "ring_submit", true);
    if (rc != KVX_OK) return rc;
    if (!sqe) return fail(KVX_E_INVAL, "ring_submit: sqe is NULL");
    if (sqe->n < 0 || sqe->n > KVX_RING_MAX_PAGES)
        return fail(KVX_E_RANGE, "ring_submit: n = " + std::to_string(sqe->n) + " is outside [0, " +
                                     std::to_string(KVX_RING_MAX_PAGES) + "]");
    std::lock_guard<std::mutex> lk(r->mu);
    if (!r->push_sqe(*sqe)) return fail(KVX_E_FULL, "ring_submit: the submission ring is full");
    return KVX_OK;
}

int kvx_ring_reap(kvx_ring* r, kvx_cqe* out, int32_t max, int32_t* got)
{
    int rc = open_ring(r, "ring_reap", true);
    if (rc != KVX_OK) return rc;
    if (!got || (max > 0 && !out)) return fail(KVX_E_INVAL, "ring_reap: NULL output");
    *got = 0;
    std::lock_guard<std::mutex> lk(r->mu);
    while (*got < max && r->pop_cqe(out + *got)) (*got)++;
    return KVX_OK;
}

int kvx_ring_take(kvx_ring* r, kvx_sqe* out, int32_t* got)
{
    int rc = open_ring(r, "ring_take", false);
    if (rc != KVX_OK) return rc;
    if (!out || !got) return fail(KVX_E_INVAL, "ring_take: NULL output");
    std::lock_guard<std::mutex> lk(r->mu);
    *got = r->pop_sqe(out) ? 1 : 0;
    return KVX_OK;
}

int kvx_ring_complete(kvx_ring* r, const kvx_cqe* cqe)
{
    int rc = open_ring(r, "ring_complete", false);
    if (rc != KVX_OK) return rc;
    if (!cqe) return fail(KVX_E_INVAL, "ring_complete: cqe is NULL");
    std::lock_guard<std::mutex> lk(r->mu);
    if (!r->push_cqe(*cqe)) return fail(KVX_E_FULL, "ring_complete: the completion ring is full");
    return KVX_OK;
}

int kvx_ring_peer_alive(const kvx_ring* r, int32_t* alive)
{
    clear_error();
    if (!ring_known(r)) return fail(KVX_E_INVAL, "ring_peer_alive: unknown ring handle");
    if (!r->live.load()) return fail(KVX_E_STALE, "ring_peer_alive: ring was closed");
    if (!alive) return fail(KVX_E_INVAL, "ring_peer_alive: alive is NULL");
    const RingShared* sh = r->sh;
    const int32_t pid = r->creator ? sh->opener_pid.load() : sh->creator_pid.load();
    const uint64_t start = r->creator ? sh->opener_start.load() : sh->creator_start.load();
    *alive = (pid != 0 && start != 0 && process_start(pid) == start) ? 1 : 0;
    return KVX_OK;
}

int kvx_ring_pending(const kvx_ring* r, int32_t* submitted, int32_t* completed)
{
    clear_error();
    if (!ring_known(r)) return fail(KVX_E_INVAL, "ring_pending: unknown ring handle");
    if (!r->live.load()) return fail(KVX_E_STALE, "ring_pending: ring was closed");
    if (!submitted || !completed) return fail(KVX_E_INVAL, "ring_pending: NULL output");
    const RingShared* sh = r->sh;
    // a snapshot while both sides run: each head is read before its tail, so
    // the difference is never negative; it is capped at the ring's size
    auto count = [&](const std::atomic<uint64_t>& head, const std::atomic<uint64_t>& tail) {
        const uint64_t h = head.load(std::memory_order_acquire);
        const uint64_t t = tail.load(std::memory_order_acquire);
        return static_cast<int32_t>(std::min<uint64_t>(t - h, sh->entries));
    };
    *submitted = count(sh->sq_head, sh->sq_tail);
    *completed = count(sh->cq_head, sh->cq_tail);
    return KVX_OK;
}

int kvx_ring_wait(kvx_ring* r, int32_t timeout_us, int32_t* ready)
{
    clear_error();
    if (!ring_known(r)) return fail(KVX_E_INVAL, "ring_wait: unknown ring handle");
    if (!r->live.load()) return fail(KVX_E_STALE, "ring_wait: ring was closed");
    if (!ready) return fail(KVX_E_INVAL, "ring_wait: ready is NULL");
    if (timeout_us < 0) return fail(KVX_E_RANGE, "ring_wait: negative timeout");
    RingShared* sh = r->sh;
    // the data plane waits for descriptors, the scheduler for completions
    std::atomic<uint64_t>& head = r->creator ? sh->cq_head : sh->sq_head;
    std::atomic<uint64_t>& tail = r->creator ? sh->cq_tail : sh->sq_tail;
    std::atomic<uint32_t>& seq = r->creator ? sh->cq_seq : sh->sq_seq;
    std::atomic<uint32_t>& waiters = r->creator ? sh->cq_waiters : sh->sq_waiters;
    struct timespec t0;
    clock_gettime(CLOCK_MONOTONIC, &t0);
    const int64_t limit = int64_t(timeout_us) * 1000;
    for (;;) {
        const uint32_t s = seq.load(std::memory_order_seq_cst);
        if (tail.load(std::memory_order_acquire) != head.load(std::memory_order_acquire)) {
            *ready = 1;
            return KVX_OK;
        }
        struct timespec t1;
        clock_gettime(CLOCK_MONOTONIC, &t1);
        const int64_t spent = (t1.tv_sec - t0.tv_sec) * 1000000000ll + (t1.tv_nsec - t0.tv_nsec);
        const int32_t peer = r->creator ? sh->opener_pid.load() : sh->creator_pid.load();
        const uint64_t peer_start = r->creator ? sh->opener_start.load() : sh->creator_start.load();
        const bool peer_alive = peer != 0 && peer_start != 0 && process_start(peer) == peer_start;
        if (spent >= limit || !peer_alive) {
            *ready = 0;
            return KVX_OK;
        }
        // sleep until the next push (the sequence word moves) or 10 ms, then
        // look again (a dead peer never pushes)
        waiters.fetch_add(1, std::memory_order_seq_cst);
        if (seq.load(std::memory_order_seq_cst) == s)
            futex_wait_for(&seq, s, std::min<int64_t>(limit - spent, 10000000));
        waiters.fetch_sub(1, std::memory_order_seq_cst);
    }
}

int kvx_ring_discard(kvx_ring* r, int32_t* dropped)
{
    int rc = open_ring(r, "ring_discard", false);
    if (rc != KVX_OK) return rc;
    if (!dropped) return fail(KVX_E_INVAL, "ring_discard: dropped is NULL");
    std::lock_guard<std::mutex> lk(r->mu);
    const uint64_t head = r->sh->sq_head.load(std::memory_order_relaxed);
    const uint64_t tail = r->sh->sq_tail.load(std::memory_order_acquire);
    r->sh->sq_head.store(tail, std::memory_order_release);
    *dropped = static_cast<int32_t>(tail - head);
    return KVX_OK;
}

}  // extern "C"
