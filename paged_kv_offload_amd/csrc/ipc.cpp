// ipc.cpp - device-memory IPC: export a pool's allocation, import it once
// per process, close the mapping.
//
// [RFC] "Device IPC data path": the data plane imports each registered KV
// allocation once, and memory sharing is a capability of its own (export,
// import, close), separate from cross-process completion. [RAWIPC] "the full
// share/rebuild chain": an IPC handle always names a whole allocation, so
// the exporter takes the handle of the allocation base and sends the byte
// offset of the pool inside it and the exporting GPU's UUID; the importer
// resolves its local device ordinal from the UUID and keeps one mapping per
// handle. [RAWIPC] "rebuild lifecycle and refcounts": a process-wide
// registry keyed by the handle bytes counts the opens of each mapping; the
// last close unmaps it, and a failure to unmap is logged, never raised,
// because closes run on teardown paths.
#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "kvx_internal.h"

namespace kvx {
namespace {

struct Mapping {
    void* base = nullptr;
    uint64_t bytes = 0;
    int device = -1;
    int64_t opens = 0;
};

std::mutex g_ipc_mu;
std::map<std::string, Mapping> g_by_handle;   // handle bytes -> mapping
std::map<uintptr_t, std::string> g_by_base;   // mapping base -> handle bytes

int device_by_uuid(const uint8_t uuid[16], int* out)
{
    int count = 0;
    KVX_HIP(hipGetDeviceCount(&count));
    for (int d = 0; d < count; d++) {
        hipDevice_t dev;
        hipUUID u;
        if (hipDeviceGet(&dev, d) != hipSuccess || hipDeviceGetUuid(&u, dev) != hipSuccess) {
            (void)hipGetLastError();
            continue;
        }
        if (std::memcmp(u.bytes, uuid, 16) == 0) {
            *out = d;
            return KVX_OK;
        }
    }
    return fail(KVX_E_INVAL, "ipc_import: no visible GPU has the exporting GPU's UUID");
}

}  // namespace

bool ipc_lookup(const void* p, int* device, uint64_t* bytes_after)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    std::lock_guard<std::mutex> lk(g_ipc_mu);
    auto it = g_by_base.upper_bound(a);
    if (it == g_by_base.begin()) return false;
    --it;
    const Mapping& m = g_by_handle.at(it->second);
    if (a >= it->first + m.bytes) return false;
    *device = m.device;
    *bytes_after = it->first + m.bytes - a;
    return true;
}

}  // namespace kvx

using namespace kvx;

extern "C" int kvx_ipc_export(const void* device_ptr, kvx_ipc_handle* out)
{
    clear_error();
    if (!device_ptr || !out) return fail(KVX_E_INVAL, "ipc_export: NULL argument");
    hipPointerAttribute_t at;
    std::memset(&at, 0, sizeof at);
    if (hipPointerGetAttributes(&at, device_ptr) != hipSuccess || at.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        return fail(KVX_E_INVAL, "ipc_export: pointer is not device memory");
    }
    DeviceGuard dg(at.device);
    hipDeviceptr_t base = nullptr;
    size_t bytes = 0;
    KVX_HIP(hipMemGetAddressRange(&base, &bytes, const_cast<void*>(device_ptr)));
    if (bytes >= KVX_IPC_MAX_BYTES)
        return fail(KVX_E_RANGE, "ipc_export: the allocation holds " + std::to_string(bytes) +
                                     " bytes; only allocations below " +
                                     std::to_string(KVX_IPC_MAX_BYTES) + " bytes are shared");
    hipIpcMemHandle_t mh;
    KVX_HIP(hipIpcGetMemHandle(&mh, base));
    hipDevice_t dev;
    hipUUID uuid;
    KVX_HIP(hipDeviceGet(&dev, at.device));
    KVX_HIP(hipDeviceGetUuid(&uuid, dev));
    kvx_ipc_handle h;
    std::memset(&h, 0, sizeof h);
    static_assert(sizeof(mh) == sizeof(h.mem_handle), "IPC handle size");
    std::memcpy(h.mem_handle, &mh, sizeof mh);
    std::memcpy(h.device_uuid, uuid.bytes, sizeof h.device_uuid);
    h.alloc_bytes = bytes;
    h.offset = reinterpret_cast<uintptr_t>(device_ptr) - reinterpret_cast<uintptr_t>(base);
    h.version = KVX_IPC_HANDLE_VERSION;
    *out = h;
    return KVX_OK;
}

extern "C" int kvx_ipc_import(const kvx_ipc_handle* handle, void** base_out, int32_t* device_out)
{
    clear_error();
    if (!handle || !base_out || !device_out) return fail(KVX_E_INVAL, "ipc_import: NULL argument");
    if (handle->version != KVX_IPC_HANDLE_VERSION || handle->reserved != 0 || handle->alloc_bytes == 0 ||
        handle->offset >= handle->alloc_bytes)
        return fail(KVX_E_INVAL, "ipc_import: malformed handle");
    if (handle->alloc_bytes >= KVX_IPC_MAX_BYTES)
        return fail(KVX_E_RANGE, "ipc_import: the allocation holds " +
                                     std::to_string(handle->alloc_bytes) + " bytes; only allocations below " +
                                     std::to_string(KVX_IPC_MAX_BYTES) + " bytes are shared");
    const std::string key(reinterpret_cast<const char*>(handle->mem_handle), sizeof handle->mem_handle);
    std::lock_guard<std::mutex> lk(g_ipc_mu);
    auto it = g_by_handle.find(key);
    if (it != g_by_handle.end()) {
        it->second.opens++;
        *base_out = it->second.base;
        *device_out = it->second.device;
        return KVX_OK;
    }
    int dev = -1;
    int rc = device_by_uuid(handle->device_uuid, &dev);
    if (rc != KVX_OK) return rc;
    DeviceGuard dg(dev);
    hipIpcMemHandle_t mh;
    std::memcpy(&mh, handle->mem_handle, sizeof mh);
    void* base = nullptr;
    KVX_HIP(hipIpcOpenMemHandle(&base, mh, hipIpcMemLazyEnablePeerAccess));
    Mapping m;
    m.base = base;
    m.bytes = handle->alloc_bytes;
    m.device = dev;
    m.opens = 1;
    g_by_handle[key] = m;
    g_by_base[reinterpret_cast<uintptr_t>(base)] = key;
    *base_out = base;
    *device_out = dev;
    return KVX_OK;
}

extern "C" int kvx_ipc_close(void* base)
{
    clear_error();
    std::lock_guard<std::mutex> lk(g_ipc_mu);
    auto bit = g_by_base.find(reinterpret_cast<uintptr_t>(base));
    if (bit == g_by_base.end())
        return fail(KVX_E_INVAL, "ipc_close: not the base of a mapping imported by kvx_ipc_import");
    Mapping& m = g_by_handle.at(bit->second);
    if (--m.opens > 0) return KVX_OK;
    {
        DeviceGuard dg(m.device);
        const hipError_t e = hipIpcCloseMemHandle(base);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            log_warn(std::string("ipc_close: hipIpcCloseMemHandle failed: ") + hipGetErrorString(e));
        }
    }
    g_by_handle.erase(bit->second);
    g_by_base.erase(bit);
    return KVX_OK;
}
