// ring_exec.cpp - the data-plane executor of the submission / completion
// rings (ring.cpp): descriptors taken from the ring run as the calls they
// name, a BACKUP next to a RESTORE of one pool as one exchange, and
// completions are posted in submission order once an event recorded after
// each operation's work has fired ([RFC] "Device IPC data path" and
// "Ownership": the data plane runs and batches the transfers the scheduler
// submits).
#include <algorithm>
#include <string>

#include "kvx_internal.h"
#include "ring.h"

using namespace kvx;

extern "C" {

// ---- ring executor ---------------------------------------------------------

namespace {

void release_ring_flights(kvx_ring* r)
{
    for (RingFlight& f : r->flights)
        if (f.event) {
            (void)hipEventSynchronize(static_cast<hipEvent_t>(f.event));
            (void)hipEventDestroy(static_cast<hipEvent_t>(f.event));
            f.event = nullptr;
        }
    for (void* ev : r->spare_events) (void)hipEventDestroy(static_cast<hipEvent_t>(ev));
    r->spare_events.clear();
}

// Events of finished flights are reused by later flights instead of one
// create / destroy pair per operation. At most this many are kept.
constexpr size_t kSpareEvents = 256;

void recycle_event(kvx_ring* r, hipEvent_t ev)
{
    if (r->spare_events.size() < kSpareEvents)
        r->spare_events.push_back(ev);
    else
        (void)hipEventDestroy(ev);
}

// Looks a descriptor's pool and buffer up in the data plane's tables and
// checks its generation: *pool, and the buffer from its offset on.
int resolve_sqe(const kvx_sqe& q, kvx_pool* const* pools, int32_t num_pools, void* const* buffers,
                const uint64_t* buffer_bytes, int32_t num_buffers, kvx_pool** pool, uint8_t** buf,
                uint64_t* bytes)
{
    if (q.pool < 0 || q.pool >= num_pools || !pools[q.pool])
        return fail(KVX_E_RANGE, "ring op " + std::to_string(q.op_id) + ": pool " +
                                     std::to_string(q.pool) + " is not in the data plane's table");
    if (q.buffer < 0 || q.buffer >= num_buffers || !buffers[q.buffer])
        return fail(KVX_E_RANGE, "ring op " + std::to_string(q.op_id) + ": buffer " +
                                     std::to_string(q.buffer) + " is not in the data plane's table");
    if (q.buffer_offset > buffer_bytes[q.buffer])
        return fail(KVX_E_RANGE, "ring op " + std::to_string(q.op_id) + ": buffer offset " +
                                     std::to_string(q.buffer_offset) + " is past the buffer's " +
                                     std::to_string(buffer_bytes[q.buffer]) + " bytes");
    if (q.n < 0 || q.n > KVX_RING_MAX_PAGES)
        return fail(KVX_E_RANGE, "ring op " + std::to_string(q.op_id) + ": bad page count");
    *pool = pools[q.pool];
    if (!pool_known(*pool)) return fail(KVX_E_INVAL, "ring op: unknown pool handle in the table");
    if (q.generation != (*pool)->generation)
        return fail(KVX_E_STALE, "ring op " + std::to_string(q.op_id) + ": generation " +
                                     std::to_string(q.generation) + " does not match pool generation " +
                                     std::to_string((*pool)->generation));
    *buf = static_cast<uint8_t*>(buffers[q.buffer]) + q.buffer_offset;
    *bytes = buffer_bytes[q.buffer] - q.buffer_offset;
    return KVX_OK;
}

// The ready object a RESTORE descriptor publishes into (NULL: none).
int sqe_ready(const kvx_sqe& q, kvx_ready* ready, kvx_ready** out)
{
    *out = nullptr;
    if (q.ready_slot_base < 0) return KVX_OK;
    if (!ready)
        return fail(KVX_E_INVAL, "ring op " + std::to_string(q.op_id) +
                                     ": publish asked for but the data plane has no ready object");
    *out = ready;
    return KVX_OK;
}

// Runs one descriptor: the call it names, against the data plane's tables.
int run_sqe(const kvx_sqe& q, kvx_pool* const* pools, int32_t num_pools, void* const* buffers,
            const uint64_t* buffer_bytes, int32_t num_buffers, kvx_ready* ready, void* stream)
{
    kvx_pool* pool = nullptr;
    uint8_t* buf = nullptr;
    uint64_t bytes = 0;
    int rc = resolve_sqe(q, pools, num_pools, buffers, buffer_bytes, num_buffers, &pool, &buf, &bytes);
    if (rc != KVX_OK) return rc;
    kvx_ready* rd = nullptr;
    rc = sqe_ready(q, ready, &rd);
    if (rc != KVX_OK) return rc;
    const int32_t sb = q.ready_slot_base >= 0 ? q.ready_slot_base : 0;
    switch (q.op) {
    case KVX_OP_BACKUP:
        return kvx_backup(pool, q.page_ids, q.n, buf, bytes, q.layer_begin, q.layer_end, stream, q.path);
    case KVX_OP_RESTORE:
        return kvx_restore(pool, buf, bytes, q.page_ids, q.n, q.layer_begin, q.layer_end, rd, sb, stream,
                           q.path);
    case KVX_OP_BACKUP_SLOTS:
        return kvx_backup_slots(pool, q.page_ids, q.host_slots, q.n, buf, bytes, q.num_host_slots,
                                q.layer_begin, q.layer_end, stream, q.path);
    case KVX_OP_RESTORE_SLOTS:
        return kvx_restore_slots(pool, buf, bytes, q.num_host_slots, q.host_slots, q.page_ids, q.n,
                                 q.layer_begin, q.layer_end, rd, sb, stream, q.path);
    default:
        return fail(KVX_E_INVAL, "ring op " + std::to_string(q.op_id) + ": unknown operation " +
                                     std::to_string(q.op));
    }
}

// A BACKUP and a RESTORE of one pool on the zero-copy or device path, taken
// one after the other, can run as one kvx_exchange (both link directions
// busy together).
bool pairable(const kvx_sqe& a, const kvx_sqe& b)
{
    const bool ops = (a.op == KVX_OP_BACKUP && b.op == KVX_OP_RESTORE) ||
                     (a.op == KVX_OP_RESTORE && b.op == KVX_OP_BACKUP) ||
                     (a.op == KVX_OP_BACKUP_SLOTS && b.op == KVX_OP_RESTORE_SLOTS) ||
                     (a.op == KVX_OP_RESTORE_SLOTS && b.op == KVX_OP_BACKUP_SLOTS);
    return ops && a.pool == b.pool && a.path == b.path &&
           (a.path == KVX_PATH_ZEROCOPY || a.path == KVX_PATH_DEVICE);
}

// Runs a pairable BACKUP and RESTORE as one kvx_exchange. Any refusal
// (either descriptor's checks, or the two touching the same bytes) leaves
// nothing enqueued, and the caller runs them one by one instead.
int run_pair(const kvx_sqe& a, const kvx_sqe& b, kvx_pool* const* pools, int32_t num_pools,
             void* const* buffers, const uint64_t* buffer_bytes, int32_t num_buffers, kvx_ready* ready,
             void* stream)
{
    const bool a_backs_up = a.op == KVX_OP_BACKUP || a.op == KVX_OP_BACKUP_SLOTS;
    const kvx_sqe& bk = a_backs_up ? a : b;
    const kvx_sqe& rs = a_backs_up ? b : a;
    kvx_pool *pb = nullptr, *pr = nullptr;
    uint8_t *bb = nullptr, *br = nullptr;
    uint64_t nb = 0, nr = 0;
    int rc = resolve_sqe(bk, pools, num_pools, buffers, buffer_bytes, num_buffers, &pb, &bb, &nb);
    if (rc != KVX_OK) return rc;
    rc = resolve_sqe(rs, pools, num_pools, buffers, buffer_bytes, num_buffers, &pr, &br, &nr);
    if (rc != KVX_OK) return rc;
    kvx_ready* rd = nullptr;
    rc = sqe_ready(rs, ready, &rd);
    if (rc != KVX_OK) return rc;
    const int32_t sb = rs.ready_slot_base >= 0 ? rs.ready_slot_base : 0;
    if (bk.op == KVX_OP_BACKUP_SLOTS) {
        const kvx_xfer_slots xb{bk.page_ids, bk.host_slots, bk.n, bk.num_host_slots, bb, nb,
                                bk.layer_begin, bk.layer_end};
        const kvx_xfer_slots xr{rs.page_ids, rs.host_slots, rs.n, rs.num_host_slots, br, nr,
                                rs.layer_begin, rs.layer_end};
        return kvx_exchange_slots(pb, &xb, &xr, rd, sb, stream, bk.path);
    }
    const kvx_xfer xb{bk.page_ids, bk.n, bb, nb, bk.layer_begin, bk.layer_end};
    const kvx_xfer xr{rs.page_ids, rs.n, br, nr, rs.layer_begin, rs.layer_end};
    return kvx_exchange(pb, &xb, &xr, rd, sb, stream, bk.path);
}

// Queues the completion of descriptor q whose call returned `status`; a
// call that enqueued work completes when an event recorded after it fires.
void push_flight(kvx_ring* r, const kvx_sqe& q, int status, void* stream)
{
    RingFlight f;
    f.op_id = q.op_id;
    f.generation = q.generation;
    f.status = status;
    if (f.status == KVX_OK) {
        hipEvent_t ev = nullptr;
        hipError_t e = hipSuccess;
        if (!r->spare_events.empty()) {
            ev = static_cast<hipEvent_t>(r->spare_events.back());
            r->spare_events.pop_back();
        } else {
            e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        }
        if (e == hipSuccess) e = hipEventRecord(ev, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) {
            // the work is enqueued but cannot be tracked: wait for it
            if (ev) (void)hipEventDestroy(ev);
            ev = nullptr;
            f.status = hipStreamSynchronize(static_cast<hipStream_t>(stream)) == hipSuccess ? KVX_OK
                                                                                             : KVX_E_HIP;
        }
        f.event = ev;
    }
    r->flights.push_back(f);
}

// Posts the completions of finished operations at the front, in order,
// while the completion ring has room. With `wait`, waits for each.
int post_finished(kvx_ring* r, bool wait, int32_t* posted)
{
    while (!r->flights.empty() && r->cq_room() > 0) {
        RingFlight& f = r->flights.front();
        if (f.event) {
            hipEvent_t ev = static_cast<hipEvent_t>(f.event);
            hipError_t e = wait ? hipEventSynchronize(ev) : hipEventQuery(ev);
            if (e == hipErrorNotReady) break;
            if (e != hipSuccess) {
                (void)hipGetLastError();
                f.status = KVX_E_HIP;
                (void)hipEventDestroy(ev);
            } else {
                recycle_event(r, ev);
            }
            f.event = nullptr;
        }
        kvx_cqe c{};
        c.op_id = f.op_id;
        c.generation = f.generation;
        c.status = f.status;
        r->push_cqe(c);
        r->flights.pop_front();
        (*posted)++;
    }
    return KVX_OK;
}

int open_server(kvx_ring* r, const char* op)
{
    clear_error();
    if (!ring_known(r)) return fail(KVX_E_INVAL, std::string(op) + ": unknown ring handle");
    if (!r->live.load()) return fail(KVX_E_STALE, std::string(op) + ": ring was closed");
    if (r->creator) return fail(KVX_E_INVAL, std::string(op) + ": only the data-plane side serves");
    return KVX_OK;
}

}  // namespace

int kvx_ring_serve(kvx_ring* r, kvx_pool* const* pools, int32_t num_pools, void* const* buffers,
                   const uint64_t* buffer_bytes, int32_t num_buffers, kvx_ready* ready, void* stream,
                   int32_t max_ops, int32_t* taken, int32_t* completed)
{
    const TraceRange tr("kvx_ring_serve");
    int rc = open_server(r, "ring_serve");
    if (rc != KVX_OK) return rc;
    if (!taken || !completed) return fail(KVX_E_INVAL, "ring_serve: NULL output");
    if (num_pools < 0 || num_buffers < 0 || (num_pools > 0 && !pools) ||
        (num_buffers > 0 && (!buffers || !buffer_bytes)))
        return fail(KVX_E_INVAL, "ring_serve: malformed tables");
    *taken = *completed = 0;
    std::lock_guard<std::mutex> lk(r->mu);
    r->release_flights = release_ring_flights;
    post_finished(r, false, completed);
    const bool pairing = tuning().ring_pairing != 0;
    static thread_local kvx_sqe qa, qb;   // 8 KiB each: kept off the stack
    kvx_sqe* cur = &qa;
    kvx_sqe* nxt = &qb;
    bool has_nxt = false;
    while (*taken < max_ops) {
        if (has_nxt) {
            std::swap(cur, nxt);
            has_nxt = false;
        } else if (!r->pop_sqe(cur)) {
            break;
        }
        (*taken)++;
        // a BACKUP next to a RESTORE of the same pool share one launch
        // sequence ([RFC] "Ownership": the data plane batches transfers)
        if (pairing && *taken < max_ops && cur->op >= KVX_OP_BACKUP && cur->op <= KVX_OP_RESTORE_SLOTS &&
            r->pop_sqe(nxt)) {
            has_nxt = true;
            if (pairable(*cur, *nxt)) {
                const int prc = run_pair(*cur, *nxt, pools, num_pools, buffers, buffer_bytes,
                                         num_buffers, ready, stream);
                if (prc == KVX_OK || prc == KVX_E_HIP) {
                    (*taken)++;
                    has_nxt = false;
                    push_flight(r, *cur, prc, stream);
                    push_flight(r, *nxt, prc, stream);
                    continue;
                }
            }
        }
        push_flight(r, *cur, run_sqe(*cur, pools, num_pools, buffers, buffer_bytes, num_buffers, ready,
                                     stream),
                    stream);
    }
    if (has_nxt) {
        (*taken)++;
        push_flight(r, *nxt, run_sqe(*nxt, pools, num_pools, buffers, buffer_bytes, num_buffers, ready,
                                     stream),
                    stream);
    }
    post_finished(r, false, completed);
    return KVX_OK;
}

int kvx_ring_drain(kvx_ring* r, int32_t* completed)
{
    const TraceRange tr("kvx_ring_drain");
    int rc = open_server(r, "ring_drain");
    if (rc != KVX_OK) return rc;
    if (!completed) return fail(KVX_E_INVAL, "ring_drain: completed is NULL");
    *completed = 0;
    std::lock_guard<std::mutex> lk(r->mu);
    post_finished(r, true, completed);
    // completions that do not fit (nobody reaps any more) are dropped once
    // their work has finished
    for (RingFlight& f : r->flights) {
        if (f.event) {
            (void)hipEventSynchronize(static_cast<hipEvent_t>(f.event));
            (void)hipEventDestroy(static_cast<hipEvent_t>(f.event));
        }
        (*completed)++;
    }
    r->flights.clear();
    return KVX_OK;
}

}  // extern "C"
