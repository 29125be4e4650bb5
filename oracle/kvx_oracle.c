/*
 * kvx_oracle.c - the CPU oracle for paged-KV backup, restore and layout
 * permutation.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The product path (the HIP library and
 * its Python binding) never calls, links or imports it, and it includes no
 * header and shares no helper with that path.
 *
 * Everything here is a plain byte loop written straight from the definitions
 * below, in int64 index arithmetic, with no blocking, fusion or reordering.
 * Each function cites the passage of the source pages it follows:
 *
 *   [RFC]     SGLang issue #37372, "[Feature] [RFC] [HiCache] Out-of-process
 *             HiCache data plane with device-memory IPC"
 *   [TICKET]  SGLang PR #36700, "[PP + HiCache] Add PP Prefetch Tickets for
 *             eager cross-stage storage prefetch"
 *   [RAWIPC]  the article analysing LMCache's RawCudaIPCWrapper
 *             ("LMCacheRawCudaIPCWrapper深度解析")
 *
 * Readings taken where the pages are silent (each one is also listed in the
 * design notes of the repository):
 *   - A pool is NB pages x NL layers x KV (1 or 2) pieces. The three outer
 *     axes {page, layer, kv} are laid out row-major in the order given by
 *     `outer`; one piece (one page of one layer of K or V) is T tokens x H
 *     heads x D elements of `dtype_bytes` bytes, stored either tokens-major
 *     (NHD: [T][H][D]) or heads-major (HND: [H][T][D]). D is innermost.
 *   - The packed host buffer is layer-major NHD over absolute layer
 *     indices: host[l][c][i][t][h][d], slot i holding page_ids[i], K before
 *     V. A call for layers [l0, l1) touches only those layers' slices.
 *   - Bytes are never interpreted: dtype_bytes only sizes a row.
 *
 * Pins (checked by the CPU tests): numpy advanced indexing of the same pool,
 * the memcpy special case, brute force over all short page-ID tuples of a
 * tiny pool, round trip and untouched-byte invariance, permutation inverses,
 * a hand-derived worked example, and the published SplitMix64 outputs for
 * the generator. No function here is left without a pin.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>

typedef struct kvxo_layout {
    int32_t outer[3];      /* physical order of the outer axes, outermost first:
                              0 = page, 1 = layer, 2 = kv                        */
    int32_t inner;         /* 0 = NHD [T][H][D], 1 = HND [H][T][D]              */
    int64_t num_pages;     /* NB */
    int64_t num_layers;    /* NL */
    int64_t num_kv;        /* KV: 2 for separate K and V, 1 for a latent pool   */
    int64_t page_size;     /* T: tokens per page                                */
    int64_t num_heads;     /* H: KV heads                                       */
    int64_t head_dim;      /* D: elements per row                               */
    int64_t dtype_bytes;   /* eb: bytes per element (sizes rows only)           */
    int64_t byte_offset;   /* pool start, in bytes from the allocation start    */
} kvxo_layout;

/* ---------------------------------------------------------------------------
 * Addressing.
 * [RFC, "Device IPC data path"]: operations carry page IDs into a pool that
 * was registered once with its layout.
 * [RAWIPC, "share/rebuild chain"]: the mapping covers the whole allocation
 * and the tensor starts at a byte offset from its base, which must be applied.
 * ------------------------------------------------------------------------- */

int64_t kvxo_row_bytes(const kvxo_layout* L) { return L->head_dim * L->dtype_bytes; }

int64_t kvxo_piece_bytes(const kvxo_layout* L)
{
    return L->page_size * L->num_heads * L->head_dim * L->dtype_bytes;
}

int64_t kvxo_pool_bytes(const kvxo_layout* L)
{
    return L->num_pages * L->num_layers * L->num_kv * kvxo_piece_bytes(L);
}

/* Row-major index of piece (page, layer, kv) over the outer axes in their
 * physical order. */
int64_t kvxo_piece_index(const kvxo_layout* L, int64_t page, int64_t layer, int64_t kv)
{
    int64_t coord[3] = { page, layer, kv };
    int64_t size[3] = { L->num_pages, L->num_layers, L->num_kv };
    int64_t idx = 0;
    for (int k = 0; k < 3; k++) {
        int ax = L->outer[k];
        idx = idx * size[ax] + coord[ax];
    }
    return idx;
}

/* Allocation-relative byte address of the first byte of piece (page, layer, kv). */
int64_t kvxo_piece_start(const kvxo_layout* L, int64_t page, int64_t layer, int64_t kv)
{
    return L->byte_offset + kvxo_piece_index(L, page, layer, kv) * kvxo_piece_bytes(L);
}

/* Row number (in rows of D elements) of token t, head h inside one piece. */
int64_t kvxo_row_in_piece(const kvxo_layout* L, int64_t t, int64_t h)
{
    if (L->inner == 0)
        return t * L->num_heads + h;       /* NHD: [T][H][D] */
    return h * L->page_size + t;           /* HND: [H][T][D] */
}

/* Row number of (layer l, kv c, slot i, token t, head h) in the packed host
 * buffer of n slots: host[l][c][i][t][h][:]. */
int64_t kvxo_host_row(const kvxo_layout* L, int64_t n, int64_t l, int64_t c, int64_t i,
                      int64_t t, int64_t h)
{
    return (((l * L->num_kv + c) * n + i) * L->page_size + t) * L->num_heads + h;
}

/* ---------------------------------------------------------------------------
 * BACKUP.
 * [RFC, "Device IPC data path"]: BACKUP names source pages; the data plane
 * copies them device-to-host. [RFC, "Ownership"]: the scheduler publishes
 * which pages are safe to read. [RAWIPC, "uint8 round trip"]: the transfer
 * moves numel*element_size bytes and never looks at the dtype.
 * [RAWIPC, "integration"]: the TRT-LLM pool is head-major (HND) and is
 * converted to the token-major host layout here.
 * ------------------------------------------------------------------------- */
void kvxo_backup(const kvxo_layout* L, const uint8_t* alloc, const int32_t* ids, int64_t n,
                 int64_t l0, int64_t l1, uint8_t* host)
{
    const int64_t rb = kvxo_row_bytes(L);
    for (int64_t l = l0; l < l1; l++)
        for (int64_t c = 0; c < L->num_kv; c++)
            for (int64_t i = 0; i < n; i++)
                for (int64_t t = 0; t < L->page_size; t++)
                    for (int64_t h = 0; h < L->num_heads; h++)
                        for (int64_t b = 0; b < rb; b++) {
                            int64_t src = kvxo_piece_start(L, ids[i], l, c)
                                        + kvxo_row_in_piece(L, t, h) * rb + b;
                            int64_t dst = kvxo_host_row(L, n, l, c, i, t, h) * rb + b;
                            host[dst] = alloc[src];
                        }
}

/* ---------------------------------------------------------------------------
 * RESTORE.
 * [RFC, "Device IPC data path"]: RESTORE scatters host KV into destination
 * pages that the scheduler allocated and passed in. [TICKET, "PP Prefetch
 * Ticket Path" diagram]: restore is layer-wise so a forward can use layer 0
 * before the last layer lands. Every byte of the allocation outside the
 * destination pieces of layers [l0, l1) is left as it was.
 * ------------------------------------------------------------------------- */
void kvxo_restore(const kvxo_layout* L, uint8_t* alloc, const uint8_t* host, const int32_t* ids,
                  int64_t n, int64_t l0, int64_t l1)
{
    const int64_t rb = kvxo_row_bytes(L);
    for (int64_t l = l0; l < l1; l++)
        for (int64_t c = 0; c < L->num_kv; c++)
            for (int64_t i = 0; i < n; i++)
                for (int64_t t = 0; t < L->page_size; t++)
                    for (int64_t h = 0; h < L->num_heads; h++)
                        for (int64_t b = 0; b < rb; b++) {
                            int64_t dst = kvxo_piece_start(L, ids[i], l, c)
                                        + kvxo_row_in_piece(L, t, h) * rb + b;
                            int64_t src = kvxo_host_row(L, n, l, c, i, t, h) * rb + b;
                            alloc[dst] = host[src];
                        }
}

/* ---------------------------------------------------------------------------
 * BACKUP and RESTORE against a slot-addressed host pool.
 * [RFC, "Ownership"]: the data plane owns the host KV physical allocation,
 * so host pages live in slots of a host pool that it hands out, and a
 * BACKUP names, next to each source page, the host slot that receives it;
 * a RESTORE names the host slot to read for each destination page. Reading
 * (the pages give no host layout): the pool is layer-major NHD like the
 * packed buffer, host[l][c][s][t][h][d] with S slots per (layer, kv), and
 * host slot slots[i] pairs with page ids[i]. With slots = 0..n-1 and S = n
 * this is the packed buffer of kvxo_backup / kvxo_restore.
 * ------------------------------------------------------------------------- */
void kvxo_backup_slots(const kvxo_layout* L, const uint8_t* alloc, const int32_t* ids,
                       const int32_t* slots, int64_t n, int64_t num_slots, int64_t l0, int64_t l1,
                       uint8_t* host)
{
    const int64_t rb = kvxo_row_bytes(L);
    for (int64_t l = l0; l < l1; l++)
        for (int64_t c = 0; c < L->num_kv; c++)
            for (int64_t i = 0; i < n; i++)
                for (int64_t t = 0; t < L->page_size; t++)
                    for (int64_t h = 0; h < L->num_heads; h++)
                        for (int64_t b = 0; b < rb; b++) {
                            int64_t src = kvxo_piece_start(L, ids[i], l, c)
                                        + kvxo_row_in_piece(L, t, h) * rb + b;
                            int64_t dst = kvxo_host_row(L, num_slots, l, c, slots[i], t, h) * rb + b;
                            host[dst] = alloc[src];
                        }
}

void kvxo_restore_slots(const kvxo_layout* L, uint8_t* alloc, const uint8_t* host,
                        const int32_t* slots, const int32_t* ids, int64_t n, int64_t num_slots,
                        int64_t l0, int64_t l1)
{
    const int64_t rb = kvxo_row_bytes(L);
    for (int64_t l = l0; l < l1; l++)
        for (int64_t c = 0; c < L->num_kv; c++)
            for (int64_t i = 0; i < n; i++)
                for (int64_t t = 0; t < L->page_size; t++)
                    for (int64_t h = 0; h < L->num_heads; h++)
                        for (int64_t b = 0; b < rb; b++) {
                            int64_t dst = kvxo_piece_start(L, ids[i], l, c)
                                        + kvxo_row_in_piece(L, t, h) * rb + b;
                            int64_t src = kvxo_host_row(L, num_slots, l, c, slots[i], t, h) * rb + b;
                            alloc[dst] = host[src];
                        }
}

/* ---------------------------------------------------------------------------
 * Layout permutation of one piece.
 * [RAWIPC, "share/rebuild chain" and "integration"]: NHD is token-major,
 * HND is head-major; a row of D elements stays contiguous in both.
 * ------------------------------------------------------------------------- */
void kvxo_nhd_to_hnd(const uint8_t* in, uint8_t* out, int64_t T, int64_t H, int64_t row_bytes)
{
    for (int64_t t = 0; t < T; t++)
        for (int64_t h = 0; h < H; h++)
            for (int64_t b = 0; b < row_bytes; b++)
                out[(h * T + t) * row_bytes + b] = in[(t * H + h) * row_bytes + b];
}

void kvxo_hnd_to_nhd(const uint8_t* in, uint8_t* out, int64_t T, int64_t H, int64_t row_bytes)
{
    for (int64_t t = 0; t < T; t++)
        for (int64_t h = 0; h < H; h++)
            for (int64_t b = 0; b < row_bytes; b++)
                out[(t * H + h) * row_bytes + b] = in[(h * T + t) * row_bytes + b];
}

/* ---------------------------------------------------------------------------
 * Ready prefix.
 * [TICKET, "PP Prefetch Ticket Path" diagram]: the globally safe prefix is
 * the minimum of the progress that every KV layer and sidecar has
 * published. Counts are in pages.
 * ------------------------------------------------------------------------- */
int64_t kvxo_ready_prefix(const uint32_t* counts, int64_t num_slots)
{
    int64_t m = 0;
    for (int64_t s = 0; s < num_slots; s++)
        if (s == 0 || (int64_t)counts[s] < m)
            m = (int64_t)counts[s];
    return m;
}

/* ---------------------------------------------------------------------------
 * Per-layer publish of one RESTORE.
 * [TICKET, "PP Prefetch Ticket Path" diagram]: KV arrives layer by layer and
 * each KV layer and sidecar publishes its own progress; the safe prefix is
 * the minimum of that progress. The page leaves open what a count holds
 * when a ready object serves one restore after another. The reading taken
 * here: a count is the number of pages published into its slot since the
 * object was created or reset, so a RESTORE of n pages over layers
 * [l0, l1) from slot_base adds n to slots [slot_base + l0, slot_base + l1)
 * once each of those layers is complete; counts only grow, and a consumer
 * of the k-th restore waits for the sum of the n of the first k. Counts are
 * 32-bit and wrap modulo 2^32.
 * ------------------------------------------------------------------------- */
void kvxo_ready_publish(uint32_t* counts, int64_t num_slots, int64_t slot_base, int64_t l0,
                        int64_t l1, uint32_t n)
{
    for (int64_t l = l0; l < l1; l++) {
        int64_t s = slot_base + l;
        if (s >= 0 && s < num_slots)
            counts[s] = counts[s] + n;
    }
}

/* ---------------------------------------------------------------------------
 * The synthetic-input generator, written here independently of the input
 * module so that the closed forms below do not depend on it.
 * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): the state advances by the golden gamma
 * 0x9e3779b97f4a7c15 and each output is the variant-13 style mix of the new
 * state with shifts 30, 27, 31.
 * Word j of stream `seed` is the (j+1)-th output of the generator started at
 * state `seed`; byte a of the stream is byte (a mod 8), little-endian, of
 * word floor(a / 8).
 * ------------------------------------------------------------------------- */
uint64_t kvxo_splitmix64_next(uint64_t* state)
{
    uint64_t z = (*state += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

uint64_t kvxo_gen_word(uint64_t seed, uint64_t j)
{
    uint64_t state = seed + j * 0x9e3779b97f4a7c15ULL;   /* j steps already taken */
    return kvxo_splitmix64_next(&state);
}

typedef struct { uint64_t seed, j, w; int valid; } gen_cache;

static uint8_t gen_byte(gen_cache* g, uint64_t seed, uint64_t a)
{
    uint64_t j = a >> 3;
    if (!g->valid || g->seed != seed || g->j != j) {
        g->seed = seed;
        g->j = j;
        g->w = kvxo_gen_word(seed, j);
        g->valid = 1;
    }
    return (uint8_t)(g->w >> (8 * (a & 7)));
}

void kvxo_gen_fill(uint64_t seed, uint64_t addr, uint64_t len, uint8_t* out)
{
    gen_cache g = { 0, 0, 0, 0 };
    for (uint64_t k = 0; k < len; k++)
        out[k] = gen_byte(&g, seed, addr + k);
}

/* ---------------------------------------------------------------------------
 * Closed forms for pools filled by the generator, used to check full-size
 * results one byte at a time without a host copy of the pool.
 * A pool allocation of `alloc_bytes` is filled with stream `pad_seed`, then
 * the pool region [byte_offset, byte_offset + pool_bytes) with stream
 * `seed`, both indexed by allocation-relative address.
 * ------------------------------------------------------------------------- */

/* Counts the bytes of host[0, len) - which hold packed host bytes
 * [host_begin, host_begin + len) of a BACKUP of `ids` over layers [l0, l1) -
 * that differ from the definition of BACKUP applied to a generator-filled
 * pool. *first_bad receives the packed offset of the first difference or -1. */
int64_t kvxo_check_backup_gen(const kvxo_layout* L, uint64_t seed, const int32_t* ids, int64_t n,
                              int64_t l0, int64_t l1, const uint8_t* host, int64_t host_begin,
                              int64_t len, int64_t* first_bad)
{
    const int64_t rb = kvxo_row_bytes(L);
    gen_cache g = { 0, 0, 0, 0 };
    int64_t bad = 0;
    *first_bad = -1;
    for (int64_t o = host_begin; o < host_begin + len;) {
        /* decode host row -> (l, c, i, t, h) */
        int64_t row = o / rb, b0 = o % rb;
        int64_t h = row % L->num_heads;
        int64_t t = (row / L->num_heads) % L->page_size;
        int64_t i = (row / (L->num_heads * L->page_size)) % n;
        int64_t lc = row / (L->num_heads * L->page_size * n);
        int64_t c = lc % L->num_kv, l = lc / L->num_kv;
        int64_t src_row = kvxo_piece_start(L, ids[i], l, c) + kvxo_row_in_piece(L, t, h) * rb;
        for (int64_t b = b0; b < rb && o < host_begin + len; b++, o++) {
            uint8_t want = (l >= l0 && l < l1) ? gen_byte(&g, seed, (uint64_t)(src_row + b)) : 0;
            uint8_t got = host[o - host_begin];
            if (l < l0 || l >= l1 || got != want) {
                if (bad == 0)
                    *first_bad = o;
                bad++;
            }
        }
    }
    return bad;
}

/* Counts the bytes of buf[0, len) - which hold allocation bytes
 * [addr_begin, addr_begin + len) after BACKUP of `src` followed by RESTORE of
 * that host buffer into `dst`, both over layers [l0, l1), starting from a
 * generator-filled allocation - that differ from the definitions. The
 * composition moves piece (src[i], l, c) onto piece (dst[i], l, c) byte for
 * byte and leaves every other byte as it was. `dst` must hold distinct
 * pages (duplicate destinations have no defined result). Returns -1 if
 * memory for the page-to-slot table cannot be had. */
int64_t kvxo_check_alloc_roundtrip(const kvxo_layout* L, uint64_t seed, uint64_t pad_seed,
                                   const int32_t* src, const int32_t* dst, int64_t n,
                                   int64_t l0, int64_t l1, const uint8_t* buf,
                                   int64_t addr_begin, int64_t len, int64_t* first_bad)
{
    const int64_t pb = kvxo_piece_bytes(L);
    const int64_t pool_end = L->byte_offset + kvxo_pool_bytes(L);
    const int64_t end = addr_begin + len;
    gen_cache g = { 0, 0, 0, 0 };
    int64_t bad = 0;
    int64_t* slot_of = (int64_t*)malloc((size_t)L->num_pages * sizeof(int64_t));
    *first_bad = -1;
    if (!slot_of)
        return -1;
    for (int64_t p = 0; p < L->num_pages; p++)
        slot_of[p] = -1;
    for (int64_t i = 0; i < n; i++)
        slot_of[dst[i]] = i;

    for (int64_t a = addr_begin; a < end;) {
        int64_t seg_end;
        uint64_t stream;
        int64_t shift;        /* expected byte at a is stream byte (a + shift) */
        if (a < L->byte_offset || a >= pool_end) {
            seg_end = a < L->byte_offset ? L->byte_offset : end;
            stream = pad_seed;
            shift = 0;
        } else {
            int64_t q = a - L->byte_offset;
            int64_t P = q / pb;
            int64_t size[3] = { L->num_pages, L->num_layers, L->num_kv };
            int64_t coord[3];
            int64_t piece_begin = L->byte_offset + P * pb;
            for (int k = 2; k >= 0; k--) {       /* undo the row-major outer index */
                int ax = L->outer[k];
                coord[ax] = P % size[ax];
                P /= size[ax];
            }
            seg_end = piece_begin + pb;
            stream = seed;
            shift = 0;
            if (coord[1] >= l0 && coord[1] < l1 && slot_of[coord[0]] >= 0) {
                int64_t i = slot_of[coord[0]];
                shift = kvxo_piece_start(L, src[i], coord[1], coord[2]) - piece_begin;
            }
        }
        if (seg_end > end)
            seg_end = end;
        for (; a < seg_end; a++) {
            uint8_t want = gen_byte(&g, stream, (uint64_t)(a + shift));
            if (buf[a - addr_begin] != want) {
                if (bad == 0)
                    *first_bad = a;
                bad++;
            }
        }
    }
    free(slot_of);
    return bad;
}
