// geometry.cpp - pool layout descriptor and validator (host only, no HIP
// calls).
//
// The layout of a registered pool is described once ([RFC] "Device IPC data
// path": REGISTER_KV_POOL carries a layout). The tensor view the caller hands
// in must be dense: the LMCache RawCudaIPCWrapper article ("sender
// validation") makes non-contiguity a hard error, because the transfer
// kernels assume the logical layout is the physical one and a silent
// .contiguous() copy of gigabytes of KV would hide a caller bug.
#include <cinttypes>
#include <cstdio>
#include <sstream>

#include "kvx_host.h"

namespace kvx {

namespace {

std::string dims_str(int32_t ndim, const int64_t* v)
{
    std::ostringstream o;
    o << "[";
    for (int32_t k = 0; k < ndim; k++) o << (k ? ", " : "") << v[k];
    o << "]";
    return o.str();
}

// a * b with an overflow check against 2^62
bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > (int64_t(1) << 62) / a) return false;
    *out = a * b;
    return true;
}

}  // namespace

int derive_geometry(const kvx_layout* L, const void* base, uint64_t byte_offset,
                    uint32_t dtype_bytes, int32_t ndim, const int64_t* shape,
                    const int64_t* stride, PoolGeom* g)
{
    if (!L || !g) return fail(KVX_E_INVAL, "register: layout and output must not be NULL");
    if (!base) return fail(KVX_E_INVAL, "register: base pointer is NULL");
    if (dtype_bytes < 1 || dtype_bytes > 64)
        return fail(KVX_E_INVAL, "register: dtype_bytes must be in [1, 64]");
    if (L->inner != KVX_NHD && L->inner != KVX_HND)
        return fail(KVX_E_INVAL, "register: layout.inner must be KVX_NHD or KVX_HND");
    {
        bool seen[3] = {false, false, false};
        for (int k = 0; k < 3; k++) {
            int ax = L->outer[k];
            if (ax < 0 || ax > 2 || seen[ax])
                return fail(KVX_E_INVAL,
                            "register: layout.outer must be a permutation of {PAGE, LAYER, KV}");
            seen[ax] = true;
        }
    }
    const int32_t d6[6] = {L->num_pages, L->num_layers, L->num_kv,
                           L->page_size, L->num_heads, L->head_dim};
    for (int k = 0; k < 6; k++)
        if (d6[k] < 1) return fail(KVX_E_INVAL, "register: every layout dimension must be >= 1");

    PoolGeom G;
    G.num_pages = L->num_pages;
    G.num_layers = L->num_layers;
    G.num_kv = L->num_kv;
    G.page_size = L->page_size;
    G.num_heads = L->num_heads;
    G.head_dim = L->head_dim;
    G.inner = L->inner;
    for (int k = 0; k < 3; k++) G.outer[k] = L->outer[k];
    G.dtype_bytes = dtype_bytes;

    // physical dims, outermost first, in elements
    const int64_t axis_size[3] = {G.num_pages, G.num_layers, G.num_kv};
    int64_t phys[6] = {axis_size[G.outer[0]], axis_size[G.outer[1]], axis_size[G.outer[2]],
                       G.inner == KVX_NHD ? G.page_size : G.num_heads,
                       G.inner == KVX_NHD ? G.num_heads : G.page_size, G.head_dim};
    int64_t total = 1;
    for (int k = 0; k < 6; k++)
        if (!mul_ok(total, phys[k], &total))
            return fail(KVX_E_INVAL, "register: pool size overflows");
    int64_t pool_bytes;
    if (!mul_ok(total, dtype_bytes, &pool_bytes))
        return fail(KVX_E_INVAL, "register: pool size overflows");

    // tensor view: shape/stride in elements
    if (ndim < 1 || ndim > 8 || !shape || !stride)
        return fail(KVX_E_INVAL, "register: tensor view needs 1..8 dims with shape and stride");
    int64_t numel = 1;
    for (int32_t k = 0; k < ndim; k++) {
        if (shape[k] < 1)
            return fail(KVX_E_INVAL, "register: tensor shape " + dims_str(ndim, shape) +
                                         " has an empty dimension");
        if (!mul_ok(numel, shape[k], &numel))
            return fail(KVX_E_INVAL, "register: tensor size overflows");
    }
    if (numel != total) {
        char b[160];
        snprintf(b, sizeof b, " holds %" PRId64 " elements but the layout describes %" PRId64,
                 numel, total);
        return fail(KVX_E_INVAL, "register: tensor shape " + dims_str(ndim, shape) + b);
    }
    {
        int64_t want = 1;
        std::vector<int64_t> expect(ndim);
        bool dense = true;
        for (int32_t k = ndim - 1; k >= 0; k--) {
            expect[k] = want;
            if (shape[k] != 1 && stride[k] != want) dense = false;
            want *= shape[k];
        }
        if (!dense)
            return fail(KVX_E_NONCONTIG,
                        "register: pool tensor is not contiguous: shape " + dims_str(ndim, shape) +
                            " stride " + dims_str(ndim, stride) + " (dense would be " +
                            dims_str(ndim, expect.data()) +
                            "); kvx never copies a pool to make it contiguous");
    }
    // the view's dims must be the physical dims with neighbours merged: every
    // prefix product of the view is a prefix product of the physical dims
    {
        int64_t pp[7];
        pp[0] = 1;
        for (int k = 0; k < 6; k++) pp[k + 1] = pp[k] * phys[k];
        int64_t acc = 1;
        for (int32_t k = 0; k < ndim; k++) {
            acc *= shape[k];
            bool hit = false;
            for (int j = 0; j <= 6; j++) hit = hit || pp[j] == acc;
            if (!hit)
                return fail(KVX_E_INVAL, "register: tensor shape " + dims_str(ndim, shape) +
                                             " does not split at the layout's dimension "
                                             "boundaries " + dims_str(6, phys));
        }
    }

    G.row_bytes = G.head_dim * G.dtype_bytes;
    G.piece_bytes = G.page_size * G.num_heads * G.row_bytes;
    G.pool_bytes = pool_bytes;
    // byte strides of the outer axes: row-major over outer[] with pieces innermost
    int64_t s = G.piece_bytes;
    int64_t* axis_stride[3] = {&G.page_stride, &G.layer_stride, &G.kv_stride};
    for (int k = 2; k >= 0; k--) {
        *axis_stride[G.outer[k]] = s;
        s *= axis_size[G.outer[k]];
    }
    G.pages_adjacent = (G.page_stride == G.piece_bytes);

    const uint64_t start = reinterpret_cast<uintptr_t>(base) + byte_offset;
    if (start % kVecBytes != 0)
        return fail(KVX_E_ALIGN, "register: pool start (base + byte_offset) is not 16-byte aligned");
    if (G.row_bytes % kVecBytes != 0)
        return fail(KVX_E_ALIGN, "register: head_dim * dtype_bytes (" +
                                     std::to_string(G.row_bytes) +
                                     ") must be a multiple of 16 bytes");
    if (G.piece_bytes > (int64_t(1) << 30))
        return fail(KVX_E_INVAL, "register: one piece (page x layer x kv) exceeds 1 GiB");
    if (G.inner == KVX_HND) {
        // the permuting kernels divide by row_vec, H and T with 32-bit
        // multiply-high, exact while dividend * divisor < 2^32
        const int64_t pv = G.piece_bytes / kVecBytes, rv = G.row_bytes / kVecBytes;
        const int64_t rows = G.page_size * G.num_heads;
        const int64_t lim = int64_t(1) << 32;
        if (pv * rv >= lim || rows * G.page_size >= lim || rows * G.num_heads >= lim)
            return fail(KVX_E_INVAL, "register: head-major piece geometry too large "
                                     "(need piece_vecs * row_vecs and rows * max(T, H) < 2^32)");
    }
    *g = G;
    return KVX_OK;
}

}  // namespace kvx
