// kernels.hip - gfx950 kernels of kvx: the piece gather (BACKUP pack), the
// piece scatter (RESTORE unpack) with per-layer publish, both in one launch
// (kvx_exchange), and the bounded ready-wait used by GPU-side consumers.
//
// Work decomposition. A launch moves the pieces (page, layer, kv) of a layer
// range, every kv and a list of (page, slot) pairs (or runs of adjacent
// pages) carried in the kernel arguments, or in device memory when the list
// is longer than they hold. Each piece (T*H*D*eb bytes, contiguous in every
// supported pool layout and in the packed buffer) is cut into units of
// kThreads * 16 * U bytes, and the tails of pieces that such units do not
// tile, or short pieces whole, share units; one workgroup moves one unit at
// a time (a
// grid-stride loop, or unit numbers drawn from a queue where the order of
// completion matters), every lane issuing U independent 16-byte (dwordx4)
// loads before its U stores. Each wave owns U KiB of the unit, contiguous,
// and moves it 1 KiB per instruction (measured on MI355X: 6-8% faster than
// the workgroup sweeping the unit 4 KiB per round, for the same bytes).
// Units are numbered layer-major, so the units of layer l are all handed out
// before those of layer l+1 and layers complete roughly in order.
//
// Every access is a buffer load or store against a resource that spans one
// piece, so the hardware drops any access past the piece. The cache policy
// is a template argument: non-temporal loads and stores, and stores at
// device scope, which write through the XCD's L2 instead of leaving dirty
// lines for the end-of-kernel write-back (measured: +3-4% HBM to HBM).
//
// Head-major pools ([RAWIPC] integration: TRT-LLM's HND pool) are converted
// either row by row - a row of D elements is contiguous on both sides, so
// every 16-byte access stays within one row and each wave reads and writes
// whole 64-byte segments; the destination is walked linearly and the source
// address is the permuted row - or through LDS in token blocks, where both
// global sides are linear runs.
//
// Publish ([TICKET] "PP Prefetch Ticket Path": layer-wise H2D and a
// published safe prefix): a workgroup counts the units it finished of layer
// l into layer_done[l] when it moves on to the next layer (one release fence
// per workgroup and layer, not per unit); the add that completes the layer
// adds n to the ready slot with a system-scope release, so no reader can see
// the new count before every byte of the layer, and a count only grows: a
// consumer of the k-th restore into a slot waits for the pages of the first
// k. That add also resets the counter, leaving it zero for the next call on
// the same stream.
#include "kvx_internal.h"

namespace kvx {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fast_div(uint32_t x, uint32_t magic)
{
    return magic ? __umulhi(x, magic) : x;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw (stride 0, unswizzled) buffer resource over [base, base + bytes); the
// 32-bit data format in the last word is what untyped buffer accesses need
// on gfx9-family parts. An access at or past `bytes` reads zero and a store
// there is dropped.
constexpr int kRsrcFormat = 0x00020000;

__device__ __forceinline__ rsrc_t piece_rsrc(const uint8_t* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, static_cast<int>(bytes),
                                             kRsrcFormat);
}

// Cache-policy bits of a buffer instruction on gfx950: nt (streaming) and
// sc1 (device scope).
constexpr int kAuxNT = 2;
constexpr int kAuxSC1 = 16;

// CP bit 0: non-temporal loads; bit 1: non-temporal stores; bit 2: stores at
// device scope
template <int CP>
__device__ __forceinline__ v4u load16(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, (CP & 1) ? kAuxNT : 0);
}

template <int CP>
__device__ __forceinline__ void store16(rsrc_t r, uint32_t off, v4u v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0,
                                           ((CP & 2) ? kAuxNT : 0) | ((CP & 4) ? kAuxSC1 : 0));
}

// The same with a scalar part of the offset (soffset) next to the lane's
// vector part: per-round offsets then need no vector registers.
template <int CP>
__device__ __forceinline__ v4u load16s(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff),
                                                 (CP & 1) ? kAuxNT : 0);
}

template <int CP>
__device__ __forceinline__ void store16s(rsrc_t r, uint32_t voff, uint32_t soff, v4u v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(voff), static_cast<int>(soff),
                                           ((CP & 2) ? kAuxNT : 0) | ((CP & 4) ? kAuxSC1 : 0));
}

// Vector index of lane `tid`'s round u inside a unit of U rounds: wave w owns
// vectors [w * 64U, (w + 1) * 64U), one 64-vector (1 KiB) run per round.
template <int U>
__device__ __forceinline__ uint32_t unit_vec(uint32_t tid, int u)
{
    return (tid >> 6) * (64u * U) + static_cast<uint32_t>(u) * 64u + (tid & 63u);
}

// Byte offset, inside the source piece, of the 16 bytes that land at byte
// offset `off` of the destination piece.
template <Dir D, bool PERMUTE>
__device__ __forceinline__ uint32_t source_offset(const UnitGeom& a, uint32_t off)
{
    if constexpr (!PERMUTE) {
        return off;
    } else {
        const uint32_t vi = off >> 4;
        const uint32_t row = fast_div(vi, a.mg_row_vec);
        const uint32_t w = vi - row * a.row_vec;
        uint32_t src_row;
        if constexpr (D == GATHER) {
            // destination: packed NHD row t*H + h; source: pool HND row h*T + t
            const uint32_t t = fast_div(row, a.mg_H);
            const uint32_t h = row - t * a.H;
            src_row = h * a.T + t;
        } else {
            // destination: pool HND row h*T + t; source: packed NHD row t*H + h
            const uint32_t h = fast_div(row, a.mg_T);
            const uint32_t t = row - h * a.T;
            src_row = t * a.H + h;
        }
        return (src_row * a.row_vec + w) << 4;
    }
}

// Moves one unit: the bytes [unit_base, unit_base + U * 4 KiB) of one piece
// (or of a run of adjacent pieces, `span` bytes; for a piece span is
// piece_bytes),
// without per-access predicates, so that all U loads are in flight before
// the first store and the stores issue back to back. The destination
// resource (and the source one, when the layouts match) starts at the unit
// and ends with the piece: each access's offset is the lane's fixed part
// plus a per-round constant that the instruction's immediate offset absorbs,
// and in the last unit of a piece that the unit does not tile, the accesses
// past the piece are dropped by the hardware's range check (loads read zero,
// stores are discarded), so a partial unit runs the same code. Piece sizes
// are multiples of 16 bytes, so no access straddles the end. Reordered
// (HND<->NHD) sources span the whole piece; a dropped store may pair with
// any in-range load.
template <Dir D, int U, bool PERMUTE, int CP>
__device__ __forceinline__ void move_unit(const UnitGeom& a, const uint8_t* src_piece,
                                          uint8_t* dst_piece, uint32_t span, uint32_t unit_base,
                                          uint32_t tid)
{
    const uint32_t rest = span - unit_base;
    const rsrc_t dst = piece_rsrc(dst_piece + unit_base, rest);
    const rsrc_t src = PERMUTE ? piece_rsrc(src_piece, a.piece_bytes)
                               : piece_rsrc(src_piece + unit_base, rest);
    const uint32_t lane_off = unit_vec<U>(tid, 0) * kVecBytes;
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const uint32_t off = lane_off + u * (64u * kVecBytes);
        v[u] = load16<CP>(src, PERMUTE ? source_offset<D, true>(a, unit_base + off) : off);
    }
#pragma unroll
    for (int u = 0; u < U; u++) store16<CP>(dst, lane_off + u * (64u * kVecBytes), v[u]);
}

// s_waitcnt with vmcnt 0 and the other counters at their maximum (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8): waits until
// every vector memory access of this wave has completed.
constexpr int kWaitVmcnt0 = 0x0F70;

// Counts `units` finished units of layer l. Every wave first waits until its
// own stores have completed, the barrier gathers the workgroup, and thread 0
// releases at agent scope: one L2 write-back then covers the stores of the
// whole workgroup (a release fence in every wave, plus a release on the add,
// cost five write-backs per count; measured on the device path, publishing
// restores ran 2.3-3x slower with them). Thread 0 waits for the write-back
// and adds to the layer's counter; the add that completes the layer acquires
// the other workgroups' releases, clears the counter for the next call and
// adds the page count to the ready slot with a system-scope release.
__device__ __forceinline__ void count_units(const PublishArgs& a, int32_t l, uint32_t units,
                                            uint32_t tid)
{
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        const uint32_t done = __hip_atomic_fetch_add(&a.layer_done[l], units, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) + units;
        if (done == a.layer_target) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(&a.layer_done[l], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // this add is the call's only write of the slot, and calls that
            // publish into one slot run one after the other (stream order),
            // so a read and a store add n without an atomic read-modify-write
            // on host memory
            const uint32_t prev = __hip_atomic_load(&a.ready[l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&a.ready[l], prev + a.publish_value, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

// One unit of a head-major piece through LDS: tokens [t0, t0 + TU) of all H
// heads, the token-major (NHD) side one contiguous run and the head-major
// (HND) side H contiguous segments of TU rows. Global reads and writes are
// both linear runs; LDS does the (t, h) exchange. Used when a unit is a
// whole number of token blocks (chunk_bytes = TU * H * row_bytes).
template <Dir D, int U, int CP>
__device__ __forceinline__ void move_unit_lds(const UnitGeom& a, rsrc_t src, rsrc_t dst,
                                              uint32_t k, uint32_t tid, v4u* lds)
{
    const uint32_t t0 = k * a.TU;
    const uint32_t nhd0 = t0 * a.H * a.row_vec;   // first vector of the unit on the NHD side
    v4u v[U];
    __syncthreads();   // the previous unit's readers are done with lds
#pragma unroll
    for (int u = 0; u < U; u++) {
        const uint32_t i = unit_vec<U>(tid, u);
        if constexpr (D == GATHER) {
            // source: pool HND, read head segment by head segment
            const uint32_t h = fast_div(i, a.mg_seg);
            const uint32_t r = i - h * a.seg;
            const uint32_t tt = fast_div(r, a.mg_row_vec);
            const uint32_t w = r - tt * a.row_vec;
            v[u] = load16<CP>(src, ((h * a.T + t0 + tt) * a.row_vec + w) << 4);
        } else {
            // source: packed NHD, one contiguous run
            v[u] = load16<CP>(src, (nhd0 + i) << 4);
        }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
        const uint32_t i = unit_vec<U>(tid, u);
        if constexpr (D == GATHER) {
            const uint32_t h = fast_div(i, a.mg_seg);
            const uint32_t r = i - h * a.seg;
            const uint32_t tt = fast_div(r, a.mg_row_vec);
            const uint32_t w = r - tt * a.row_vec;
            lds[(tt * a.H + h) * a.row_vec + w] = v[u];   // into NHD order
        } else {
            lds[i] = v[u];
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; u++) {
        const uint32_t i = unit_vec<U>(tid, u);
        if constexpr (D == GATHER) {
            store16<CP>(dst, (nhd0 + i) << 4, lds[i]);
        } else {
            // destination: pool HND, written head segment by head segment
            const uint32_t h = fast_div(i, a.mg_seg);
            const uint32_t r = i - h * a.seg;
            const uint32_t tt = fast_div(r, a.mg_row_vec);
            const uint32_t w = r - tt * a.row_vec;
            store16<CP>(dst, ((h * a.T + t0 + tt) * a.row_vec + w) << 4,
                        lds[(tt * a.H + h) * a.row_vec + w]);
        }
    }
}

// Position of unit q of a side: layer, kv, pair index j and chunk k of the
// piece; all wave-uniform scalar math.
struct UnitPos {
    int32_t l;
    uint32_t c, j, k;
};

__device__ __forceinline__ UnitPos decode_unit(const UnitGeom& g, const Side& s, uint32_t q)
{
    if (g.tails_per_wave) {
        // per (layer, kv): the side's pieces' whole units, then its tail
        // units; a tail unit is marked k == main_units, j its first piece
        const uint32_t per_unit = 4u * g.tails_per_wave;   // pieces a tail unit holds
        const uint32_t main = s.npairs * g.main_units;
        const uint32_t units_lc = main + (s.npairs + per_unit - 1) / per_unit;
        const uint32_t lc = q / units_lc;
        const uint32_t rem = q - lc * units_lc;
        uint32_t j, k;
        if (rem < main) {
            j = rem / g.main_units;
            k = rem - j * g.main_units;
        } else {
            j = (rem - main) * per_unit;
            k = g.main_units;
        }
        const uint32_t lrel = lc / g.num_kv;
        return UnitPos{s.layer_begin + static_cast<int32_t>(lrel), lc - lrel * g.num_kv, j, k};
    }
    const uint32_t cpp = g.chunks_per_piece;
    const uint32_t pu = q / cpp;
    uint32_t k = q - pu * cpp;
    const uint32_t lc = pu / s.npairs;
    const uint32_t j = pu - lc * s.npairs;
    if (g.unit_order & 2u) {   // rotate the chunk order from piece to piece
        k += j % cpp;
        if (k >= cpp) k -= cpp;
    }
    const uint32_t lrel = lc / g.num_kv;
    return UnitPos{s.layer_begin + static_cast<int32_t>(lrel), lc - lrel * g.num_kv, j, k};
}

// Moves the unit at `u` of a side between pool page `page` and packed slot
// `slot`; `span` is the bytes the unit's piece or run covers from there.
// PERM: 0 = same inner layout, 1 = HND<->NHD row by row, 2 = HND<->NHD
// through LDS token blocks (`lds` holds U * kThreads vectors).
template <Dir D, int U, int PERM, int CP>
__device__ __forceinline__ void move_at(const UnitGeom& g, const Side& s, const UnitPos& u,
                                        int32_t page, int32_t slot, uint32_t span, uint32_t tid,
                                        v4u* lds)
{
    uint8_t* pool_piece = g.pool + static_cast<int64_t>(page) * g.page_stride +
                          static_cast<int64_t>(u.l) * g.layer_stride +
                          static_cast<int64_t>(u.c) * g.kv_stride;
    uint8_t* pk_piece = s.packed +
                        (static_cast<int64_t>(u.l - s.pk_layer0) * g.num_kv + u.c) * s.pk_lc_stride +
                        static_cast<int64_t>(slot - s.pk_slot0) * g.piece_bytes;
    const uint8_t* src = (D == GATHER) ? pool_piece : pk_piece;
    uint8_t* dst = (D == GATHER) ? pk_piece : pool_piece;
    if constexpr (PERM == 2)
        move_unit_lds<D, U, CP>(g, piece_rsrc(src, g.piece_bytes), piece_rsrc(dst, g.piece_bytes), u.k,
                                tid, lds);
    else
        move_unit<D, U, PERM == 1, CP>(g, src, dst, span, u.k * g.chunk_bytes, tid);
}

// Word i of a move launch's pair or run list: from device memory when the
// list is longer than the kernel arguments carry, else from the arguments.
// The device list is read through a constant-address-space pointer: it does
// not change during the launch, and the index is wave-uniform, so the reads
// are scalar loads through the scalar cache.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

__device__ __forceinline__ int32_t pair_word(const MoveArgs& a, uint32_t i)
{
    return a.list ? ((const_i32_ptr)(a.list))[i] : a.pairs[i];
}

// A tail unit: the tails of the pieces j0 .. j0 + 4 * TPW - 1 of a move
// launch (those that exist), the last tail_bytes of each after its
// main_units whole units; with main_units 0 the tail is the whole piece, so
// pieces shorter than a wave's share of a unit travel 4 * TPW to a unit
// instead of one. Wave w moves the tails of pieces j0 + w * TPW ..
// j0 + (w + 1) * TPW - 1, U / TPW rounds of 1 KiB each; a tail shorter than
// that, or a piece past the launch's last, is bounded by its buffer
// resource (a missing piece gets a resource of length zero). Wave-uniform
// throughout: the wave index is read through readfirstlane so that every
// resource stays scalar.
template <Dir D, int U, int TPW, int CP, class PS>
__device__ __forceinline__ void move_tails(const UnitGeom& g, const Side& s, const UnitPos& u, PS page_slot,
                                           uint32_t tid)
{
    constexpr int TR = U / TPW;   // rounds per tail
    const uint32_t wave = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(tid >> 6)));
    const uint32_t lane_off = (tid & 63u) * kVecBytes;
    const uint32_t tail0 = g.main_units * g.chunk_bytes;
    rsrc_t src[TPW], dst[TPW];
#pragma unroll
    for (int t = 0; t < TPW; t++) {
        const uint32_t j = u.j + wave * TPW + t;
        const bool live = j < s.npairs;
        const uint32_t jj = live ? j : u.j;
        const int32_t page = page_slot.page(jj), slot = page_slot.slot(jj);
        uint8_t* pool_piece = g.pool + static_cast<int64_t>(page) * g.page_stride +
                              static_cast<int64_t>(u.l) * g.layer_stride +
                              static_cast<int64_t>(u.c) * g.kv_stride;
        uint8_t* pk_piece = s.packed + (static_cast<int64_t>(u.l - s.pk_layer0) * g.num_kv + u.c) * s.pk_lc_stride +
                            static_cast<int64_t>(slot - s.pk_slot0) * g.piece_bytes;
        const uint32_t bytes = live ? g.tail_bytes : 0u;
        src[t] = piece_rsrc((D == GATHER ? pool_piece : pk_piece) + tail0, bytes);
        dst[t] = piece_rsrc((D == GATHER ? pk_piece : pool_piece) + tail0, bytes);
    }
    v4u v[U];
#pragma unroll
    for (int r = 0; r < U; r++) v[r] = load16s<CP>(src[r / TR], lane_off, (r % TR) * (64u * kVecBytes));
#pragma unroll
    for (int r = 0; r < U; r++) store16s<CP>(dst[r / TR], lane_off, (r % TR) * (64u * kVecBytes), v[r]);
}

// Moves unit `u` of a side: a tail unit (tail units are built for units of
// 32 rounds in device memory and 2 over the host link, without reordered
// rows) or a chunk of the piece or run at (page, slot) spanning `span`
// bytes. page_slot(j) gives pair j of the side for tail units.
template <Dir D, int U, int PERM, int CP, class PS>
__device__ __forceinline__ void move_side(const UnitGeom& g, const Side& s, const UnitPos& u, int32_t page,
                                          int32_t slot, uint32_t span, PS page_slot, uint32_t tid, v4u* lds)
{
    if constexpr ((U == 32 || U == 2) && PERM == 0) {
        if (g.tails_per_wave != 0 && u.k == g.main_units) {
            if constexpr (U == 32) {
                switch (g.tails_per_wave) {
                case 1: move_tails<D, U, 1, CP>(g, s, u, page_slot, tid); break;
                case 2: move_tails<D, U, 2, CP>(g, s, u, page_slot, tid); break;
                case 4: move_tails<D, U, 4, CP>(g, s, u, page_slot, tid); break;
                default: move_tails<D, U, 8, CP>(g, s, u, page_slot, tid); break;
                }
            } else {
                // the host link's 8 KiB units: one or two short pieces a wave
                if (g.tails_per_wave == 1)
                    move_tails<D, U, 1, CP>(g, s, u, page_slot, tid);
                else
                    move_tails<D, U, 2, CP>(g, s, u, page_slot, tid);
            }
            return;
        }
    }
    move_at<D, U, PERM, CP>(g, s, u, page, slot, span, tid, lds);
}

// Pair j of a move launch's (page, slot) list.
struct MovePairs {
    const MoveArgs& a;
    __device__ int32_t page(uint32_t j) const { return pair_word(a, 2 * j); }
    __device__ int32_t slot(uint32_t j) const { return pair_word(a, 2 * j + 1); }
};

// Position of unit q of a move launch over runs of adjacent pages: run r of
// the launch starts at pairs[4r] (page) and pairs[4r + 1] (slot), spans
// pairs[4r + 2] pieces and holds the units [pairs[4r + 3], pairs[4r + 3] +
// its units) of each (layer, kv); j is the run, k the unit inside it.
__device__ __forceinline__ UnitPos decode_run_unit(const MoveArgs& a, uint32_t q)
{
    const uint32_t per = a.g.units_lc;
    const uint32_t lc = q / per;
    const uint32_t rem = q - lc * per;
    uint32_t lo = 0, hi = a.s.npairs - 1;   // the last run whose first unit is <= rem
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (static_cast<uint32_t>(pair_word(a, 4 * mid + 3)) <= rem)
            lo = mid;
        else
            hi = mid - 1;
    }
    const uint32_t lrel = lc / a.g.num_kv;
    return UnitPos{a.s.layer_begin + static_cast<int32_t>(lrel), lc - lrel * a.g.num_kv, lo,
                   rem - static_cast<uint32_t>(pair_word(a, 4 * lo + 3))};
}

// Runs f(q) for the unit numbers [0, total) drawn from `queue` in number
// order. Lane 0 draws the next number while the workgroup moves the current
// unit; two LDS words alternate so one barrier per unit suffices. Each
// workgroup stops at its first draw past the end, so draw number
// total + gridDim.x - 1 is the launch's last: whoever makes it resets the
// queue for the next launch on the stream.
//
// Every lane reads the same LDS word after the barrier; readfirstlane tells
// the compiler so. Without it the unit number, and every buffer resource
// derived from it, counts as divergent, and each buffer access is wrapped in
// a readfirstlane loop (measured on MI355X, device-path restore publishing
// every layer: 5.36 TB/s with the loops on llama8b against 5.69 without,
// 181 VGPRs against 164).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v)
{
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

template <class F>
__device__ __forceinline__ void for_queued_units(uint32_t* queue, uint32_t total, uint32_t tid, F&& f)
{
    __shared__ uint32_t next[2];
    const uint32_t last_draw = total + gridDim.x - 1;
    if (tid == 0) {
        const uint32_t d = __hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == last_draw) __hip_atomic_store(queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        next[0] = d;
    }
    __syncthreads();
    uint32_t q = uniform_u32(next[0]);
    for (uint32_t it = 1; q < total; it++) {
        uint32_t d = 0;
        if (tid == 0) d = __hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        f(q);
        if (tid == 0) {
            if (d == last_draw) __hip_atomic_store(queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            next[it & 1u] = d;
        }
        __syncthreads();
        q = uniform_u32(next[it & 1u]);
    }
}

template <Dir D, int U, int PERM, bool PUBLISH, int CP>
__global__ __launch_bounds__(kThreads) void kvx_move_kernel(MoveArgs a)
{
    const uint32_t tid = threadIdx.x;
    int32_t pend_layer = -1;   // PUBLISH: layer of the units finished but not yet counted
    uint32_t pend = 0;
    __shared__ v4u lds[PERM == 2 ? U * kThreads : 1];
    auto do_unit = [&](uint32_t q) {
        UnitPos u;
        int32_t page, slot;
        uint32_t span;
        if (a.g.runs) {
            u = decode_run_unit(a, q);
            page = pair_word(a, 4 * u.j);
            slot = pair_word(a, 4 * u.j + 1);
            span = static_cast<uint32_t>(pair_word(a, 4 * u.j + 2)) * a.g.piece_bytes;
        } else {
            u = decode_unit(a.g, a.s, q);
            page = pair_word(a, 2 * u.j);
            slot = pair_word(a, 2 * u.j + 1);
            span = a.g.piece_bytes;
        }
        if constexpr (PUBLISH) {
            // units arrive layer by layer: count a layer once this workgroup leaves it
            if (u.l != pend_layer) {
                if (pend) count_units(a.p, pend_layer, pend, tid);
                pend_layer = u.l;
                pend = 0;
            }
        }
        move_side<D, U, PERM, CP>(a.g, a.s, u, page, slot, span, MovePairs{a}, tid, lds);
        if constexpr (PUBLISH) pend++;
    };

    if constexpr (PUBLISH) {
        // Blocks of a.p.block consecutive units come from the queue in
        // number order, so every unit of layer l is handed out before any of
        // layer l + 1 and a workgroup that runs slowly (measured: reads of
        // pinned host memory are not served evenly across workgroups) holds
        // back at most the block it is on. A workgroup counts once per layer
        // it leaves, so larger blocks mean fewer counts.
        const uint32_t B = a.p.block;
        const uint32_t total = a.s.total_units;
        for_queued_units(a.p.queue, (total + B - 1) / B, tid, [&](uint32_t b) {
            const uint32_t q1 = (b + 1) * B < total ? (b + 1) * B : total;
            for (uint32_t q = b * B; q < q1; q++) do_unit(q);
        });
        if (pend) count_units(a.p, pend_layer, pend, tid);
    } else {
        // Workgroups are dispatched round-robin over the 8 XCDs (block b runs
        // on XCD b mod 8). With XCD ordering, the workgroups of one XCD take
        // consecutive unit numbers in every round of the loop, so each XCD
        // walks whole pieces instead of one fixed chunk offset of many pieces.
        uint32_t v = blockIdx.x;
        if ((a.g.unit_order & 1u) && (gridDim.x & 7u) == 0)
            v = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
        for (uint32_t q = v; q < a.s.total_units; q += gridDim.x) do_unit(q);
    }
}

// BACKUP side b and RESTORE side r in one launch. Units are drawn from the
// queue and alternate between the sides (b, r, b, r, ... until the shorter
// side runs out), so both directions of the host link stay busy together:
// measured on MI355X, a gather to pinned host memory and a scatter from it
// sharing one launch sustain 90-91 GB/s over back-to-back launches, where
// the same work as two kernels on two streams drifts out of step and falls
// to 67-76 GB/s. Only the RESTORE side publishes.
// Page and packed slot of pair j of a side: listed in slot order from
// first_x (packed buffers), or as explicit (page, slot) pairs (host pools);
// in device memory (list_x, read through scalar loads) when the list is
// longer than the kernel arguments carry.
__device__ __forceinline__ int32_t list_word(const int32_t* list, const int32_t* args, uint32_t i)
{
    return list ? ((const_i32_ptr)(list))[i] : args[i];
}
__device__ __forceinline__ int32_t page_b(const ExchangeArgs& a, uint32_t j) { return list_word(a.list_b, a.pages_b, j); }
__device__ __forceinline__ int32_t slot_b(const ExchangeArgs& a, uint32_t j)
{
    return a.first_b + static_cast<int32_t>(j);
}
__device__ __forceinline__ int32_t page_r(const ExchangeArgs& a, uint32_t j) { return list_word(a.list_r, a.pages_r, j); }
__device__ __forceinline__ int32_t slot_r(const ExchangeArgs& a, uint32_t j)
{
    return a.first_r + static_cast<int32_t>(j);
}
__device__ __forceinline__ int32_t page_b(const ExchangeSlotArgs& a, uint32_t j)
{
    return list_word(a.list_b, a.pairs_b, 2 * j);
}
__device__ __forceinline__ int32_t slot_b(const ExchangeSlotArgs& a, uint32_t j)
{
    return list_word(a.list_b, a.pairs_b, 2 * j + 1);
}
__device__ __forceinline__ int32_t page_r(const ExchangeSlotArgs& a, uint32_t j)
{
    return list_word(a.list_r, a.pairs_r, 2 * j);
}
__device__ __forceinline__ int32_t slot_r(const ExchangeSlotArgs& a, uint32_t j)
{
    return list_word(a.list_r, a.pairs_r, 2 * j + 1);
}

// Pair j of an exchange's BACKUP (B) or RESTORE side.
template <class A, bool B>
struct SidePairs {
    const A& a;
    __device__ int32_t page(uint32_t j) const { return B ? page_b(a, j) : page_r(a, j); }
    __device__ int32_t slot(uint32_t j) const { return B ? slot_b(a, j) : slot_r(a, j); }
};

template <int U, int PERM, bool PUBLISH, bool HOST, class A>
__global__ __launch_bounds__(kThreads) void kvx_exchange_kernel(A a)
{
    // cache policy: pinned host memory is written at device scope and read
    // plainly; pool memory is read non-temporally
    constexpr int CPG = HOST ? 5 : 7;
    constexpr int CPS = HOST ? 6 : 7;
    const uint32_t tid = threadIdx.x;
    const uint32_t tb = a.b.total_units, tr = a.r.total_units;
    const uint32_t m = tb < tr ? tb : tr;
    int32_t pend_layer = -1;
    uint32_t pend = 0;
    __shared__ v4u lds[PERM == 2 ? U * kThreads : 1];
    auto do_unit = [&](uint32_t q) {
        bool gather;
        uint32_t idx;
        if (q < 2 * m) {
            gather = (q & 1u) == 0;
            idx = q >> 1;
        } else {
            gather = tb > tr;
            idx = m + (q - 2 * m);
        }
        if (gather) {
            const UnitPos u = decode_unit(a.g, a.b, idx);
            move_side<GATHER, U, PERM, CPG>(a.g, a.b, u, page_b(a, u.j), slot_b(a, u.j), a.g.piece_bytes,
                                            SidePairs<A, true>{a}, tid, lds);
        } else {
            const UnitPos u = decode_unit(a.g, a.r, idx);
            if constexpr (PUBLISH) {
                if (u.l != pend_layer) {
                    if (pend) count_units(a.p, pend_layer, pend, tid);
                    pend_layer = u.l;
                    pend = 0;
                }
            }
            move_side<SCATTER, U, PERM, CPS>(a.g, a.r, u, page_r(a, u.j), slot_r(a, u.j), a.g.piece_bytes,
                                             SidePairs<A, false>{a}, tid, lds);
            if constexpr (PUBLISH) pend++;
        }
    };
    // blocks of a.p.block consecutive unit numbers per draw (both sides
    // alternating inside a block), as in the move kernel
    const uint32_t B = a.p.block, total = tb + tr;
    for_queued_units(a.p.queue, (total + B - 1) / B, tid, [&](uint32_t blk) {
        const uint32_t q1 = (blk + 1) * B < total ? (blk + 1) * B : total;
        for (uint32_t q = blk * B; q < q1; q++) do_unit(q);
    });
    if constexpr (PUBLISH) {
        if (pend) count_units(a.p, pend_layer, pend, tid);
    }
}

// One wave polls a ready slot with bounded patience; see kvx_ready_wait_gpu.
// Zeroes count words: clears the per-layer counters and the unit queue in
// stream order. A kernel rather than a memset node, so that a caller who
// captures the stream into a graph records a node that replays correctly.
__global__ __launch_bounds__(256) void kvx_clear_kernel(uint32_t* p, uint32_t count)
{
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i < count) p[i] = 0u;
}

__global__ __launch_bounds__(64) void kvx_ready_wait_kernel(const uint32_t* slot, uint32_t min_count,
                                                            uint32_t spin_limit, int32_t* status)
{
    if (threadIdx.x != 0) return;
    int32_t reached = 0;
    for (uint32_t i = 0; i < spin_limit; i++) {
        const uint32_t v = __hip_atomic_load(slot, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM);
        if (v >= min_count) {
            reached = 1;
            break;
        }
        __builtin_amdgcn_s_sleep(64);
    }
    *status = reached;
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
uint32_t magic_u32(uint32_t d)
{
    // floor(x / d) == umulhi(x, floor(2^32 / d) + 1) whenever x * d < 2^32;
    // divisor 1 is flagged with 0 (the multiplier would not fit in 32 bits)
    if (d <= 1) return 0;
    return static_cast<uint32_t>((uint64_t(1) << 32) / d + 1);
}

int pick_unroll(int64_t piece_bytes, int max_unroll, int forced)
{
    if (forced > 0) return forced;
    // the largest power-of-two unit, up to 32 rounds of 4 KiB, that fits in
    // the piece; what is left of the piece forms one partial unit. Measured
    // on MI355X (HBM to HBM): 128 KiB pieces move fastest as one 128 KiB
    // unit (6.3 TB/s against 6.1 in 64 KiB units and 5.3-5.6 in 32 or 48
    // KiB units); 144 KiB pieces as 128 KiB plus 16 KiB (5.6 TB/s both ways)
    // rather than nine exact 16 KiB units (5.0 unpack) or three of 48 KiB
    // (5.0); 64 KiB head-major pieces as one 64 KiB unit
    const int64_t rounds = piece_bytes / (kThreads * kVecBytes);
    int u = 1;
    while (u < 32 && 2 * u <= max_unroll && 2 * u <= rounds) u *= 2;
    return u;
}

namespace {

template <Dir D, int U, int P, bool PUB, int CP>
hipError_t go(const LaunchCfg& cfg, const MoveArgs& a, hipStream_t s)
{
    void* args[] = {const_cast<MoveArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&kvx_move_kernel<D, U, P, PUB, CP>),
                           dim3(cfg.grid), dim3(kThreads), args, 0, s);
}

template <Dir D, int U, int P, bool PUB>
hipError_t go_nt(const LaunchCfg& cfg, const MoveArgs& a, hipStream_t s)
{
    switch (cfg.cache_policy & 7) {
    case 7: return go<D, U, P, PUB, 7>(cfg, a, s);
    case 6: return go<D, U, P, PUB, 6>(cfg, a, s);
    case 5: return go<D, U, P, PUB, 5>(cfg, a, s);
    case 4: return go<D, U, P, PUB, 4>(cfg, a, s);
    case 3: return go<D, U, P, PUB, 3>(cfg, a, s);
    case 2: return go<D, U, P, PUB, 2>(cfg, a, s);
    case 1: return go<D, U, P, PUB, 1>(cfg, a, s);
    default: return go<D, U, P, PUB, 0>(cfg, a, s);
    }
}

template <Dir D, int U, int P>
hipError_t go_pub(const LaunchCfg& cfg, const MoveArgs& a, hipStream_t s)
{
    if constexpr (D == SCATTER) {
        if (cfg.publish) return go_nt<D, U, P, true>(cfg, a, s);
    }
    return go_nt<D, U, P, false>(cfg, a, s);
}

template <Dir D, int U>
hipError_t go_perm(const LaunchCfg& cfg, const MoveArgs& a, hipStream_t s)
{
    if constexpr (U == 4 || U == 8 || U == 16) {
        if (cfg.permute == 2) return go_pub<D, U, 2>(cfg, a, s);
    }
    return cfg.permute ? go_pub<D, U, 1>(cfg, a, s) : go_pub<D, U, 0>(cfg, a, s);
}

template <Dir D>
hipError_t go_unroll(const LaunchCfg& cfg, const MoveArgs& a, hipStream_t s)
{
    switch (cfg.unroll) {
    case 32: return go_perm<D, 32>(cfg, a, s);
    case 16: return go_perm<D, 16>(cfg, a, s);
    case 12: return go_perm<D, 12>(cfg, a, s);
    case 8: return go_perm<D, 8>(cfg, a, s);
    case 6: return go_perm<D, 6>(cfg, a, s);
    case 4: return go_perm<D, 4>(cfg, a, s);
    case 3: return go_perm<D, 3>(cfg, a, s);
    case 2: return go_perm<D, 2>(cfg, a, s);
    case 1: return go_perm<D, 1>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_move(Dir dir, const LaunchCfg& cfg, const MoveArgs& a, hipStream_t s)
{
    if (cfg.grid < 1 || a.s.total_units == 0) return hipErrorInvalidValue;
    return dir == GATHER ? go_unroll<GATHER>(cfg, a, s) : go_unroll<SCATTER>(cfg, a, s);
}

namespace {

template <int U, int P, bool PUB, bool HOST, class A>
hipError_t xgo(const LaunchCfg& cfg, const A& a, hipStream_t s)
{
    void* args[] = {const_cast<A*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&kvx_exchange_kernel<U, P, PUB, HOST, A>),
                           dim3(cfg.grid), dim3(kThreads), args, 0, s);
}

template <int U, int P, class A>
hipError_t xgo_pub(const LaunchCfg& cfg, const A& a, hipStream_t s)
{
    if (cfg.publish)
        return cfg.host_link ? xgo<U, P, true, true>(cfg, a, s) : xgo<U, P, true, false>(cfg, a, s);
    return cfg.host_link ? xgo<U, P, false, true>(cfg, a, s) : xgo<U, P, false, false>(cfg, a, s);
}

template <int U, class A>
hipError_t xgo_perm(const LaunchCfg& cfg, const A& a, hipStream_t s)
{
    if constexpr (U == 4 || U == 8 || U == 16) {
        if (cfg.permute == 2) return xgo_pub<U, 2>(cfg, a, s);
    }
    return cfg.permute ? xgo_pub<U, 1>(cfg, a, s) : xgo_pub<U, 0>(cfg, a, s);
}

template <class A>
hipError_t xgo_unroll(const LaunchCfg& cfg, const A& a, hipStream_t s)
{
    if (cfg.grid < 1 || a.b.total_units + a.r.total_units == 0 || !a.p.queue) return hipErrorInvalidValue;
    switch (cfg.unroll) {
    case 32: return xgo_perm<32>(cfg, a, s);
    case 16: return xgo_perm<16>(cfg, a, s);
    case 12: return xgo_perm<12>(cfg, a, s);
    case 8: return xgo_perm<8>(cfg, a, s);
    case 6: return xgo_perm<6>(cfg, a, s);
    case 4: return xgo_perm<4>(cfg, a, s);
    case 3: return xgo_perm<3>(cfg, a, s);
    case 2: return xgo_perm<2>(cfg, a, s);
    case 1: return xgo_perm<1>(cfg, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_exchange(const LaunchCfg& cfg, const ExchangeArgs& a, hipStream_t s)
{
    return xgo_unroll(cfg, a, s);
}

hipError_t launch_exchange(const LaunchCfg& cfg, const ExchangeSlotArgs& a, hipStream_t s)
{
    return xgo_unroll(cfg, a, s);
}

hipError_t launch_clear_u32(uint32_t* p, uint32_t count, hipStream_t s)
{
    if (count == 0) return hipSuccess;
    const uint32_t blocks = (count + 255u) / 256u;
    void* args[] = {&p, &count};
    return hipLaunchKernel(reinterpret_cast<const void*>(&kvx_clear_kernel), dim3(blocks), dim3(256),
                           args, 0, s);
}

hipError_t launch_ready_wait(const uint32_t* slot, uint32_t min_count, uint32_t spin_limit,
                             int32_t* status, hipStream_t s)
{
    void* args[] = {&slot, &min_count, &spin_limit, &status};
    return hipLaunchKernel(reinterpret_cast<const void*>(&kvx_ready_wait_kernel), dim3(1), dim3(64),
                           args, 0, s);
}

}  // namespace kvx
