// wq_abi.cpp -- the C ABI: host-side validation, dispatch by M, planning of the
// grouped decode and prefill launches and the 64-byte-aligned tensor table.
//
// Every check runs on the host before anything is launched; a failing check
// returns a status and touches no HIP state. Launches go to the caller's
// stream; nothing is synchronized here. The only allocation is the prefill
// workspace of wq_gemm (a per-(device, stream) buffer from a stream-ordered
// memory pool, reused across calls).
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "wq_internal.h"

namespace {

// ---------------------------------------------------------------- workspace
// One stream-ordered memory pool per device, created on first use and kept
// until the process ends (its release threshold is the maximum, so freed
// blocks stay in the pool). On top of it, each (device, stream handle) keeps
// the workspace of its last prefill call and reuses it while it is large
// enough. Each buffer carries an event recorded after its last use; a call
// makes its stream wait for that event before using the buffer, so two uses
// never overlap even when a stream handle is reused after a stream was
// destroyed with work still pending. A larger need replaces the buffer (the
// old one is freed on the stream of its last use, after that work); with more
// streams than cache entries the least recently used entry is released the
// same way. Calls made while the stream is being captured into a graph take a
// fresh pool allocation, freed inside the capture.
constexpr int kMaxDevices = 64;
constexpr int kWsEntries = 16;
std::mutex g_ws_mu;
hipMemPool_t g_pools[kMaxDevices] = {};

struct WsEntry {
    int dev;
    hipStream_t stream;      // stream of the last use
    void *ptr;
    size_t bytes;
    hipEvent_t done;         // recorded on `stream` after the last use
    uint64_t last;
};
WsEntry g_ws[kWsEntries] = {};
uint64_t g_ws_clock = 0;

// The device's pool (g_ws_mu held).
hipError_t device_pool(int dev, hipMemPool_t *out)
{
    if (!g_pools[dev]) {
        hipMemPoolProps props;
        memset(&props, 0, sizeof props);
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t created = nullptr;
        hipError_t e = hipMemPoolCreate(&created, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(created, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(created);
            return e;
        }
        g_pools[dev] = created;
    }
    *out = g_pools[dev];
    return hipSuccess;
}

// A workspace of at least `bytes` for work on `stream`. *entry is set for a
// cached buffer (the caller records its event after the launches) and null for
// a fresh allocation the caller frees on the stream (capture). The caller
// holds g_ws_mu until its launches and that record or free are enqueued, so
// no other call can release the buffer in between.
hipError_t workspace(size_t bytes, hipStream_t stream, void **p, WsEntry **entry)
{
    *entry = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    hipMemPool_t pool;
    e = device_pool(dev, &pool);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return hipMallocFromPoolAsync(p, bytes, pool, stream);
    WsEntry *hit = nullptr, *lru = &g_ws[0];
    for (WsEntry &w : g_ws) {
        if (w.ptr && w.dev == dev && w.stream == stream) hit = &w;
        if (!w.ptr) lru = &w;
        else if (lru->ptr && w.last < lru->last) lru = &w;
    }
    WsEntry *slot = hit ? hit : lru;
    if (!hit || slot->bytes < bytes) {
        if (slot->ptr) {
            e = hipFreeAsync(slot->ptr, slot->stream);   // after the work of its last use
            slot->ptr = nullptr;
            if (e != hipSuccess) return e;
        }
        if (!slot->done) {
            e = hipEventCreateWithFlags(&slot->done, hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        const size_t want = hit && bytes < 2 * hit->bytes ? 2 * hit->bytes : bytes;   // grow geometrically
        void *np = nullptr;
        e = hipMallocFromPoolAsync(&np, want, pool, stream);
        if (e != hipSuccess) return e;
        slot->dev = dev;
        slot->stream = stream;
        slot->ptr = np;
        slot->bytes = want;
    } else {
        e = hipStreamWaitEvent(stream, slot->done, 0);   // after the buffer's last use
        if (e != hipSuccess) return e;
    }
    slot->last = ++g_ws_clock;
    *p = slot->ptr;
    *entry = slot;
    return hipSuccess;
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;     // bound on M, N, K (index arithmetic)
constexpr int64_t kMaxK = (int64_t)1 << 24;

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int check_bits(int bits) { return (bits == 4 || bits == 5 || bits == 8) ? WQ_OK : WQ_ERR_BITS; }

// int5 rows are 5K/8 bytes; K % 128 == 0 keeps every row 16-byte aligned.
inline int check_row(int64_t K, int bits) { return (bits == 5 && K % 128 != 0) ? WQ_ERR_SHAPE : WQ_OK; }

inline int check_shape(int64_t M, int64_t K, int64_t N)
{
    if (K <= 0 || K % WQ_BLOCK != 0 || K > kMaxK) return WQ_ERR_SHAPE;
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return WQ_ERR_SHAPE;
    return WQ_OK;
}

// Common checks of the matmul entry points. Returns WQ_OK with *empty set when
// there is nothing to compute.
int check_matmul(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                 const uint16_t *scales, const float *y, bool *empty)
{
    *empty = false;
    int st = check_bits(bits);
    if (st) return st;
    st = check_shape(M, K, N);
    if (st) return st;
    st = check_row(K, bits);
    if (st) return st;
    if (M == 0 || N == 0) { *empty = true; return WQ_OK; }
    if (!x || !q || !scales || !y) return WQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 16) || !aligned(y, 16)) return WQ_ERR_ALIGN;
    return WQ_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_ERR_HIP; }

inline uint64_t align64(uint64_t v) { return (v + (WQ_TABLE_ALIGN - 1)) & ~(uint64_t)(WQ_TABLE_ALIGN - 1); }

// The decode kernels address a tensor's codes and scales with 32-bit offsets.
inline int gemv_offsets_ok(int64_t K, int64_t N, int bits)
{
    const uint64_t lim = (uint64_t)1 << 32;
    if ((uint64_t)N * (uint64_t)K * (uint64_t)bits / 8 >= lim) return WQ_ERR_SHAPE;
    if ((uint64_t)N * (uint64_t)(K / WQ_BLOCK) * 2 >= lim) return WQ_ERR_SHAPE;
    return WQ_OK;
}

int gemm_grid_ok(int64_t M, int64_t N)
{
    // the prefill tile is 64 x 128; the grid is rounded up to a multiple of 8
    const int64_t tiles = ((M + 63) / 64) * ((N + 127) / 128);
    return tiles <= (int64_t)0x7FFFFFF0 ? WQ_OK : WQ_ERR_SHAPE;
}

// Limits of the prefill kernels: 32-bit byte offsets into the prepared x
// (binary16, M x K), the codes and the scales.
int gemm_sizes_ok(int64_t M, int64_t K, int64_t N, int bits)
{
    const uint64_t lim = (uint64_t)1 << 32;
    if ((uint64_t)M * (uint64_t)K * 2 >= lim) return WQ_ERR_SHAPE;
    if (N >= ((int64_t)1 << 22)) return WQ_ERR_SHAPE;      // y offsets within a 128-row tile stay below 2^32
    if ((uint64_t)N * (uint64_t)K * (uint64_t)bits / 8 >= lim) return WQ_ERR_SHAPE;
    if ((uint64_t)N * (uint64_t)(K / WQ_BLOCK) * 2 >= lim) return WQ_ERR_SHAPE;
    return gemm_grid_ok(M, N);
}

// Checks of one tensor-table entry of a grouped call with M rows.
int check_entry(const wq_desc &d, int64_t M)
{
    int st = check_bits(d.bits);
    if (st) return st;
    st = check_shape(M, d.K, d.N);
    if (st) return st;
    st = check_row(d.K, d.bits);
    if (st) return st;
    st = gemv_offsets_ok(d.K, d.N, d.bits);
    if (st) return st;
    if ((d.q_off % WQ_TABLE_ALIGN) || (d.s_off % WQ_TABLE_ALIGN)) return WQ_ERR_ALIGN;
    if (d.s_off < d.q_off + (uint64_t)d.N * (uint64_t)d.K * (uint64_t)d.bits / 8 &&
        d.q_off < d.s_off + (uint64_t)d.N * (uint64_t)(d.K / WQ_BLOCK) * 2 && d.N > 0)
        return WQ_ERR_TABLE;                    // codes and scales overlap
    if (d.N > 0) {
        if (!d.x || !d.y) return WQ_ERR_NULL;
        if (!aligned(d.x, 16) || !aligned(d.y, 16)) return WQ_ERR_ALIGN;
    }
    return WQ_OK;
}

}  // namespace

extern "C" {

size_t wq_q_bytes(int64_t N, int64_t K, int bits)
{
    if (check_bits(bits) || check_shape(0, K, N) || check_row(K, bits)) return 0;
    return (size_t)N * (size_t)K * (size_t)bits / 8;
}

size_t wq_s_bytes(int64_t N, int64_t K)
{
    if (check_shape(0, K, N)) return 0;
    return (size_t)N * (size_t)(K / WQ_BLOCK) * 2;
}

int wq_pack(const float *w, int64_t N, int64_t K, int bits, void *q, uint16_t *scales,
            hipStream_t stream)
{
    int st = check_bits(bits);
    if (st) return st;
    st = check_shape(0, K, N);
    if (st) return st;
    st = check_row(K, bits);
    if (st) return st;
    if (N == 0) return WQ_OK;
    if (!w || !q || !scales) return WQ_ERR_NULL;
    if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scales, 16)) return WQ_ERR_ALIGN;
    return hip_status(wq::launch_pack(w, N, K, bits, q, scales, stream));
}

int wq_unpack(const void *q, int64_t N, int64_t K, int bits, int8_t *codes, hipStream_t stream)
{
    int st = check_bits(bits);
    if (st) return st;
    st = check_shape(0, K, N);
    if (st) return st;
    st = check_row(K, bits);
    if (st) return st;
    if (N == 0) return WQ_OK;
    if (!q || !codes) return WQ_ERR_NULL;
    if (!aligned(q, 16) || !aligned(codes, 16)) return WQ_ERR_ALIGN;
    return hip_status(wq::launch_unpack(q, N, K, bits, codes, stream));
}

int wq_gemv(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
            const uint16_t *scales, float *y, hipStream_t stream)
{
    bool empty;
    int st = check_matmul(x, M, K, N, bits, q, scales, y, &empty);
    if (st) return st;
    if (M > WQ_GEMV_MAX_M) return WQ_ERR_M_RANGE;
    if (empty) return WQ_OK;
    st = gemv_offsets_ok(K, N, bits);
    if (st) return st;
    if (M >= wq::kMgemvMinM) return hip_status(wq::launch_mgemv(x, M, K, N, bits, q, scales, y, stream));
    return hip_status(wq::launch_gemv(x, M, K, N, bits, q, scales, y, stream));
}

int wq_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
            const uint16_t *scales, float *y, hipStream_t stream)
{
    bool empty;
    int st = check_matmul(x, M, K, N, bits, q, scales, y, &empty);
    if (st) return st;
    if (empty) return WQ_OK;
    st = gemm_sizes_ok(M, K, N, bits);
    if (st) return st;
    if (wq::gemm_skinny(M, K, N, bits))          // prepares x itself: no workspace
        return hip_status(wq::launch_gemm(x, M, K, N, bits, q, scales, y, nullptr, stream));
    std::lock_guard<std::mutex> lk(g_ws_mu);
    void *ws = nullptr;
    WsEntry *entry = nullptr;
    if (workspace((size_t)wq::gemm_ws_bytes(M, K), stream, &ws, &entry) != hipSuccess) return WQ_ERR_HIP;
    const hipError_t e = wq::launch_gemm(x, M, K, N, bits, q, scales, y, ws, stream);
    // the buffer's last use so far (cached), or its release (capture)
    const hipError_t f = entry ? hipEventRecord(entry->done, stream) : hipFreeAsync(ws, stream);
    return (e == hipSuccess && f == hipSuccess) ? WQ_OK : WQ_ERR_HIP;
}

int wq_gemm_noalloc(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                    const uint16_t *scales, float *y, hipStream_t stream)
{
    bool empty;
    int st = check_matmul(x, M, K, N, bits, q, scales, y, &empty);
    if (st) return st;
    if (empty) return WQ_OK;
    st = gemm_sizes_ok(M, K, N, bits);
    if (st) return st;
    if (wq::gemm_ws_bytes(M, K) > wq::kGemmNoAllocScratch) return WQ_ERR_SCRATCH;
    void *ws = nullptr;
    if (wq::gemm_noalloc_scratch(&ws) != hipSuccess) return WQ_ERR_HIP;
    return hip_status(wq::launch_gemm(x, M, K, N, bits, q, scales, y, ws, stream));
}

int wq_embed(const int32_t *ids, int64_t n_ids, int64_t K, int64_t N, int bits, const void *q,
             const uint16_t *scales, float *out, hipStream_t stream)
{
    int st = check_bits(bits);
    if (st) return st;
    st = check_shape(n_ids, K, N);
    if (st) return st;
    st = check_row(K, bits);
    if (st) return st;
    if (n_ids == 0) return WQ_OK;
    if (!ids || !out) return WQ_ERR_NULL;
    if (N > 0 && (!q || !scales)) return WQ_ERR_NULL;
    if (!aligned(ids, 4) || !aligned(out, 16)) return WQ_ERR_ALIGN;
    if (N > 0 && (!aligned(q, 16) || !aligned(scales, 16))) return WQ_ERR_ALIGN;
    // one thread per 8 outputs; the grid must fit in 32 bits
    if ((uint64_t)n_ids * (uint64_t)(K / 8) > (uint64_t)0x7FFFFFFF * 256) return WQ_ERR_SHAPE;
    return hip_status(wq::launch_embed(ids, n_ids, K, N, bits, q, scales, out, stream));
}

int wq_linear(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
              const uint16_t *scales, float *y, hipStream_t stream)
{
    if (M >= 0 && M <= WQ_GEMV_MAX_M)
        return wq_gemv(x, M, K, N, bits, q, scales, y, stream);
    return wq_gemm(x, M, K, N, bits, q, scales, y, stream);
}

int wq_table_layout(wq_desc *table, int count, uint64_t *package_bytes)
{
    if (count < 0) return WQ_ERR_SHAPE;
    if (!package_bytes || (count > 0 && !table)) return WQ_ERR_NULL;
    uint64_t cur = 0;
    for (int i = 0; i < count; ++i) {
        wq_desc &d = table[i];
        int st = check_bits(d.bits);
        if (st) return st;
        st = check_shape(0, d.K, d.N);
        if (st) return st;
        st = check_row(d.K, d.bits);
        if (st) return st;
        d.q_off = align64(cur);
        cur = d.q_off + (uint64_t)d.N * (uint64_t)d.K * (uint64_t)d.bits / 8;
        d.s_off = align64(cur);
        cur = d.s_off + (uint64_t)d.N * (uint64_t)(d.K / WQ_BLOCK) * 2;
    }
    *package_bytes = align64(cur);
    return WQ_OK;
}

int wq_table_plan(wq_desc *table, int count, int64_t M, int64_t *total_tiles)
{
    if (count < 0) return WQ_ERR_SHAPE;
    if (!total_tiles || (count > 0 && !table)) return WQ_ERR_NULL;
    if (M < 1 || M > WQ_GEMV_MAX_M) return WQ_ERR_M_RANGE;
    int64_t cur = 0;
    for (int i = 0; i < count; ++i) {
        wq_desc &d = table[i];
        const int st = check_entry(d, M);
        if (st) return st;
        d.tile_begin = cur;
        d.ws_slot = 0;
        const int64_t rows = wq::decode_item_rows(d.K, d.bits, d.N, true, M);
        cur += (d.N + rows - 1) / rows;
        if (cur > (int64_t)0x7FFFFFFF) return WQ_ERR_SHAPE;
    }
    *total_tiles = cur;
    return WQ_OK;
}

int wq_gemv_grouped(const void *base, const wq_desc *table_dev, int count, int64_t total_tiles,
                    int64_t M, hipStream_t stream)
{
    if (M < 1 || M > WQ_GEMV_MAX_M) return WQ_ERR_M_RANGE;
    if (count < 0 || total_tiles < 0 || total_tiles > (int64_t)0x7FFFFFFF) return WQ_ERR_SHAPE;
    if (count == 0 || total_tiles == 0) return WQ_OK;
    if (!base || !table_dev) return WQ_ERR_NULL;
    if (!aligned(base, WQ_TABLE_ALIGN) || !aligned(table_dev, WQ_TABLE_ALIGN)) return WQ_ERR_ALIGN;
    if (M >= wq::kMgemvMinM) return hip_status(wq::launch_mgemv_grouped(base, table_dev, count, total_tiles, M, stream));
    return hip_status(wq::launch_gemv_grouped(base, table_dev, count, total_tiles, M, stream));
}

int wq_table_plan_gemm(wq_desc *table, int count, int64_t M, int64_t *total_tiles, uint64_t *workspace_bytes)
{
    if (count < 0) return WQ_ERR_SHAPE;
    if (!total_tiles || !workspace_bytes || (count > 0 && !table)) return WQ_ERR_NULL;
    if (M < 1 || M > kMaxDim) return WQ_ERR_M_RANGE;
    for (int i = 0; i < count; ++i) {
        const int st = check_entry(table[i], M);
        if (st) return st;
        const int sz = gemm_sizes_ok(M, table[i].K, table[i].N, table[i].bits);
        if (sz) return sz;
    }
    // workspace slots: one per distinct (x, K, code order) of the non-empty
    // entries, in table order
    uint64_t ws = 0;
    for (int i = 0; i < count; ++i) {
        wq_desc &d = table[i];
        d.ws_slot = 0;
        if (d.N == 0) continue;
        const bool ord8 = d.bits == 8;
        int owner = -1;
        for (int j = 0; j < i && owner < 0; ++j)
            if (table[j].N > 0 && table[j].x == d.x && table[j].K == d.K && (table[j].bits == 8) == ord8) owner = j;
        if (owner >= 0) {
            d.ws_slot = table[owner].ws_slot;
            continue;
        }
        if (ws / wq::kGemmWsUnit > (uint64_t)INT32_MAX) return WQ_ERR_SHAPE;
        d.ws_slot = (int32_t)(ws / wq::kGemmWsUnit);
        ws += wq::gemm_ws_bytes(M, d.K);
    }
    // dispatch order: longest K first (the longest K loops start first), ties in
    // table order; each entry starts at a multiple of 8 work items
    int64_t cur = 0, prev = INT64_MAX;
    for (;;) {
        int64_t k = -1;                         // the longest K below prev
        for (int i = 0; i < count; ++i)
            if (table[i].K < prev && table[i].K > k) k = table[i].K;
        if (k < 0) break;
        for (int i = 0; i < count; ++i) {
            wq_desc &d = table[i];
            if (d.K != k) continue;
            cur = (cur + wq::kGemmGroupAlign - 1) / wq::kGemmGroupAlign * wq::kGemmGroupAlign;
            d.tile_begin = cur;
            cur += wq::gemm_grouped_items(M, d.N, d.K);
            if (cur > (int64_t)0x7FFFFFFF) return WQ_ERR_SHAPE;
        }
        prev = k;
    }
    // the split-K header (flags and partial tiles) comes first; the slots follow.
    // An entry that shares an earlier entry's slot gets the slot's complement.
    const uint64_t head = wq::gemm_grouped_header_bytes(M, cur);
    for (int i = 0; i < count; ++i) {
        if (table[i].N == 0) continue;
        const uint64_t slot = (uint64_t)table[i].ws_slot + head / wq::kGemmWsUnit;
        if (slot > (uint64_t)INT32_MAX) return WQ_ERR_SHAPE;
        table[i].ws_slot = (int32_t)slot;
    }
    for (int i = count - 1; i >= 0; --i) {
        if (table[i].N == 0) continue;
        for (int j = 0; j < i; ++j)
            if (table[j].N > 0 && table[j].ws_slot == table[i].ws_slot) {
                table[i].ws_slot = ~table[i].ws_slot;
                break;
            }
    }
    *total_tiles = cur;
    *workspace_bytes = ws + head;
    return WQ_OK;
}

int wq_gemm_grouped(const void *base, const wq_desc *table_dev, int count, int64_t total_tiles, int64_t M,
                    void *workspace, uint64_t workspace_bytes, hipStream_t stream)
{
    if (M < 1 || M > kMaxDim) return WQ_ERR_M_RANGE;
    if (count < 0 || total_tiles < 0 || total_tiles > (int64_t)0x7FFFFFFF) return WQ_ERR_SHAPE;
    if (count > 65535) return WQ_ERR_SHAPE;                 // one preparation grid row per entry
    if (count == 0 || total_tiles == 0) return WQ_OK;
    if (!base || !table_dev) return WQ_ERR_NULL;
    if (workspace_bytes > 0 && !workspace) return WQ_ERR_NULL;
    if (!aligned(base, WQ_TABLE_ALIGN) || !aligned(table_dev, WQ_TABLE_ALIGN) ||
        !aligned(workspace, (uintptr_t)wq::kGemmWsUnit))
        return WQ_ERR_ALIGN;
    if (workspace_bytes < wq::gemm_grouped_header_bytes(M, total_tiles)) return WQ_ERR_SHAPE;
    return hip_status(wq::launch_gemm_grouped(base, table_dev, count, total_tiles, M, workspace, stream));
}

const char *wq_strerror(int status)
{
    switch (status) {
    case WQ_OK: return "ok";
    case WQ_ERR_NULL: return "null pointer argument";
    case WQ_ERR_SHAPE: return "invalid shape (K must be a positive multiple of 32; M, N >= 0; sizes in range)";
    case WQ_ERR_BITS: return "bits must be 4, 5 or 8";
    case WQ_ERR_ALIGN: return "misaligned pointer or table offset";
    case WQ_ERR_M_RANGE: return "M outside the range of this entry point";
    case WQ_ERR_HIP: return "HIP runtime error at launch";
    case WQ_ERR_TABLE: return "inconsistent tensor-table entry";
    case WQ_ERR_SCRATCH: return "workspace larger than the scratch of wq_gemm_noalloc";
    default: return "unknown status";
    }
}

int wq_abi_version(void) { return 7; }

}  // extern "C"
