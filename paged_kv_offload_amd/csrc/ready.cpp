// ready.cpp - ready objects: the per-layer published counts that RESTOREs
// write and consumers read ([TICKET] "PP Prefetch Ticket Path": layer-wise
// progress and the minimum over layers and sidecars as the safe prefix;
// [RFC] "Device IPC data path": completion as a capability of its own). The
// counts live in fine-grained pinned host memory, or in device memory that
// another process can share through the device-memory IPC.
#include <cstring>
#include <string>

#include "kvx_internal.h"

using namespace kvx;

extern "C" {

// ---- ready objects -----------------------------------------------------------

namespace {

constexpr size_t kDeviceCountsMin = 2u << 20;   // own allocation, never a carved-out piece

// Copies device counts [0, num) to `out` through the object's own stream.
int read_device_counts(const kvx_ready* r, uint32_t* out, int32_t num)
{
    DeviceGuard dg(r->device);
    KVX_HIP(hipMemcpyAsync(out, r->counts_dev, sizeof(uint32_t) * num, hipMemcpyDeviceToHost, r->query));
    KVX_HIP(hipStreamSynchronize(r->query));
    return KVX_OK;
}

int make_device_ready(int device, uint32_t* counts, bool owned, int32_t num_slots,
                      uint64_t generation, kvx_ready** out)
{
    DeviceGuard dg(device);
    hipStream_t q = nullptr;
    KVX_HIP(hipStreamCreateWithFlags(&q, hipStreamNonBlocking));
    kvx_ready* r = new (std::nothrow) kvx_ready();
    if (!r) {
        (void)hipStreamDestroy(q);
        return fail(KVX_E_NOMEM, "ready: out of host memory");
    }
    r->num_slots = num_slots;
    r->generation = generation;
    r->counts_dev = counts;
    r->device = device;
    r->owned = owned;
    r->query = q;
    register_ready(r);
    *out = r;
    return KVX_OK;
}

}  // namespace

int kvx_ready_create(int32_t num_slots, uint64_t generation, kvx_ready** out)
{
    clear_error();
    if (!out) return fail(KVX_E_INVAL, "ready_create: out is NULL");
    *out = nullptr;
    if (num_slots < 1 || num_slots > (1 << 24))
        return fail(KVX_E_INVAL, "ready_create: num_slots must be in [1, 2^24]");
    void* p = nullptr;
    hipError_t e = hipHostMalloc(&p, sizeof(uint32_t) * num_slots,
                                 hipHostMallocMapped | hipHostMallocPortable | hipHostMallocCoherent);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(e == hipErrorOutOfMemory ? KVX_E_NOMEM : KVX_E_HIP,
                    std::string("ready_create: hipHostMalloc failed: ") + hipGetErrorString(e));
    }
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, p, 0);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        (void)hipHostFree(p);
        return hip_fail(e, "hipHostGetDevicePointer");
    }
    kvx_ready* r = new (std::nothrow) kvx_ready();
    if (!r) {
        (void)hipHostFree(p);
        return fail(KVX_E_NOMEM, "ready_create: out of host memory");
    }
    r->num_slots = num_slots;
    r->generation = generation;
    r->counts = static_cast<uint32_t*>(p);
    r->counts_dev = static_cast<uint32_t*>(d);
    for (int32_t k = 0; k < num_slots; k++) __atomic_store_n(&r->counts[k], 0u, __ATOMIC_RELEASE);
    register_ready(r);
    *out = r;
    return KVX_OK;
}


int kvx_ready_create_device(int32_t device, int32_t num_slots, uint64_t generation, kvx_ready** out)
{
    clear_error();
    if (!out) return fail(KVX_E_INVAL, "ready_create_device: out is NULL");
    *out = nullptr;
    if (num_slots < 1 || num_slots > (1 << 24))
        return fail(KVX_E_INVAL, "ready_create_device: num_slots must be in [1, 2^24]");
    int count = 0;
    KVX_HIP(hipGetDeviceCount(&count));
    if (device < 0 || device >= count)
        return fail(KVX_E_INVAL, "ready_create_device: no GPU " + std::to_string(device));
    DeviceGuard dg(device);
    const size_t bytes = std::max(kDeviceCountsMin, sizeof(uint32_t) * num_slots);
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(KVX_E_NOMEM, std::string("ready_create_device: hipMalloc failed: ") +
                                     hipGetErrorString(e));
    }
    int rc = make_device_ready(device, static_cast<uint32_t*>(p), true, num_slots, generation, out);
    if (rc != KVX_OK) {
        (void)hipFree(p);
        return rc;
    }
    e = hipMemsetAsync(p, 0, sizeof(uint32_t) * num_slots, (*out)->query);
    if (e == hipSuccess) e = hipStreamSynchronize((*out)->query);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        kvx_ready* r = *out;
        *out = nullptr;
        (void)kvx_ready_destroy(r);   // frees the counts and the stream
        return hip_fail(e, "ready_create_device: clearing the counts");
    }
    return KVX_OK;
}

int kvx_ready_attach_device(void* counts_dev, int32_t num_slots, uint64_t generation, kvx_ready** out)
{
    clear_error();
    if (!out) return fail(KVX_E_INVAL, "ready_attach_device: out is NULL");
    *out = nullptr;
    if (num_slots < 1 || num_slots > (1 << 24))
        return fail(KVX_E_INVAL, "ready_attach_device: num_slots must be in [1, 2^24]");
    if (!counts_dev || reinterpret_cast<uintptr_t>(counts_dev) % sizeof(uint32_t))
        return fail(KVX_E_INVAL, "ready_attach_device: counts must be 4-byte aligned device memory");
    int device = -1;
    uint64_t after = 0;
    if (!ipc_lookup(counts_dev, &device, &after)) {
        hipPointerAttribute_t at;
        std::memset(&at, 0, sizeof at);
        if (hipPointerGetAttributes(&at, counts_dev) != hipSuccess || at.type != hipMemoryTypeDevice) {
            (void)hipGetLastError();
            return fail(KVX_E_INVAL, "ready_attach_device: counts are not device memory");
        }
        device = at.device;
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        DeviceGuard dg(device);
        if (hipMemGetAddressRange(&base, &size, counts_dev) == hipSuccess && base)
            after = reinterpret_cast<uintptr_t>(base) + size - reinterpret_cast<uintptr_t>(counts_dev);
        else
            (void)hipGetLastError();
    }
    if (after && after < sizeof(uint32_t) * uint64_t(num_slots))
        return fail(KVX_E_RANGE, "ready_attach_device: the allocation has no room for " +
                                     std::to_string(num_slots) + " counts");
    return make_device_ready(device, static_cast<uint32_t*>(counts_dev), false, num_slots, generation,
                             out);
}

int kvx_ready_reset(kvx_ready* r)
{
    clear_error();
    if (!ready_known(r)) return fail(KVX_E_INVAL, "ready_reset: unknown ready handle");
    if (!r->live.load()) return fail(KVX_E_STALE, "ready_reset: ready object was destroyed");
    if (r->device >= 0) {
        DeviceGuard dg(r->device);
        KVX_HIP(hipMemsetAsync(r->counts_dev, 0, sizeof(uint32_t) * r->num_slots, r->query));
        KVX_HIP(hipStreamSynchronize(r->query));
        return KVX_OK;
    }
    for (int32_t k = 0; k < r->num_slots; k++) __atomic_store_n(&r->counts[k], 0u, __ATOMIC_RELEASE);
    return KVX_OK;
}

int kvx_ready_destroy(kvx_ready* r)
{
    clear_error();
    if (!r) return KVX_OK;
    if (!ready_known(r)) {
        log_warn("ready_destroy: unknown ready handle ignored");
        return fail(KVX_E_INVAL, "ready_destroy: unknown ready handle");
    }
    if (!r->live.exchange(false)) {
        log_warn("ready_destroy: ready object was already destroyed");
        return KVX_OK;
    }
    if (r->device >= 0) {
        DeviceGuard dg(r->device);
        hipError_t e = hipStreamSynchronize(r->query);
        if (e == hipSuccess && r->owned) e = hipFree(r->counts_dev);
        if (e == hipSuccess) e = hipStreamDestroy(r->query);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            log_warn(std::string("ready_destroy: releasing device counts failed: ") + hipGetErrorString(e));
        }
    } else {
        hipError_t e = hipHostFree(r->counts);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            log_warn(std::string("ready_destroy: hipHostFree failed: ") + hipGetErrorString(e));
        }
    }
    r->counts = nullptr;
    r->counts_dev = nullptr;
    return KVX_OK;
}

int kvx_layer_ready(const kvx_ready* r, int32_t slot, int32_t* published)
{
    clear_error();
    if (!ready_known(r)) return fail(KVX_E_INVAL, "layer_ready: unknown ready handle");
    if (!r->live.load()) return fail(KVX_E_STALE, "layer_ready: ready object was destroyed");
    if (slot < 0 || slot >= r->num_slots || !published)
        return fail(KVX_E_RANGE, "layer_ready: slot out of range");
    if (r->device >= 0) {
        std::vector<uint32_t> c(slot + 1);
        int rc = read_device_counts(r, c.data(), slot + 1);
        if (rc != KVX_OK) return rc;
        *published = static_cast<int32_t>(c[slot]);
        return KVX_OK;
    }
    *published = static_cast<int32_t>(__atomic_load_n(&r->counts[slot], __ATOMIC_ACQUIRE));
    return KVX_OK;
}

int kvx_ready_prefix(const kvx_ready* r, int32_t* prefix)
{
    clear_error();
    if (!ready_known(r)) return fail(KVX_E_INVAL, "ready_prefix: unknown ready handle");
    if (!r->live.load()) return fail(KVX_E_STALE, "ready_prefix: ready object was destroyed");
    if (!prefix) return fail(KVX_E_INVAL, "ready_prefix: prefix is NULL");
    if (r->device >= 0) {
        std::vector<uint32_t> c(r->num_slots);
        int rc = read_device_counts(r, c.data(), r->num_slots);
        if (rc != KVX_OK) return rc;
        *prefix = static_cast<int32_t>(*std::min_element(c.begin(), c.end()));
        return KVX_OK;
    }
    uint32_t m = __atomic_load_n(&r->counts[0], __ATOMIC_ACQUIRE);
    for (int32_t k = 1; k < r->num_slots; k++)
        m = std::min(m, __atomic_load_n(&r->counts[k], __ATOMIC_ACQUIRE));
    *prefix = static_cast<int32_t>(m);
    return KVX_OK;
}

int kvx_ready_slot_ptr(const kvx_ready* r, int32_t slot, void** dev_ptr)
{
    clear_error();
    if (!ready_known(r)) return fail(KVX_E_INVAL, "ready_slot_ptr: unknown ready handle");
    if (!r->live.load()) return fail(KVX_E_STALE, "ready_slot_ptr: ready object was destroyed");
    if (slot < 0 || slot >= r->num_slots || !dev_ptr)
        return fail(KVX_E_RANGE, "ready_slot_ptr: slot out of range");
    *dev_ptr = r->counts_dev + slot;
    return KVX_OK;
}

int kvx_ready_wait_gpu(const kvx_ready* r, int32_t slot, int32_t min_count, void* stream,
                       uint32_t spin_limit, int32_t* status_dev)
{
    clear_error();
    if (!ready_known(r)) return fail(KVX_E_INVAL, "ready_wait_gpu: unknown ready handle");
    if (!r->live.load()) return fail(KVX_E_STALE, "ready_wait_gpu: ready object was destroyed");
    if (slot < 0 || slot >= r->num_slots) return fail(KVX_E_RANGE, "ready_wait_gpu: slot out of range");
    if (min_count < 0 || !status_dev || reinterpret_cast<uintptr_t>(status_dev) % 4)
        return fail(KVX_E_INVAL, "ready_wait_gpu: bad min_count or status pointer");
    hipPointerAttribute_t at;
    std::memset(&at, 0, sizeof at);
    if (hipPointerGetAttributes(&at, status_dev) != hipSuccess || at.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        return fail(KVX_E_INVAL, "ready_wait_gpu: status must be device memory");
    }
    DeviceGuard dg(at.device);
    hipError_t e = launch_ready_wait(r->counts_dev + slot, static_cast<uint32_t>(min_count),
                                     spin_limit, status_dev, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "ready wait launch");
    return KVX_OK;
}

}  // extern "C"
