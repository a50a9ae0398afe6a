// The host-side C ABI layer (wq_abi.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_sanitize_host.py with g++
// -fsanitize=address,undefined and no recovery; any report ends the run with
// a non-zero status).
//
// The kernel launchers are replaced by stubs that count calls and launch
// nothing, and only paths that end before any HIP runtime call are taken:
// argument validation of every entry point, the empty calls, the size
// queries, the package layout and both planners (over random tables of up to
// 300 entries, with empty entries, shared activations and every code width),
// wq_gemm_noalloc's scratch limit and wq_strerror. Results are checked as
// well, so the run also fails on a wrong status or plan.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "wq.h"
#include "../../weight_only_bit_block_amd/csrc/wq_internal.h"

static int launches = 0;

namespace wq {
hipError_t launch_pack(const float *, int64_t, int64_t, int, void *, uint16_t *, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_unpack(const void *, int64_t, int64_t, int, int8_t *, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_gemv(const float *, int64_t, int64_t, int64_t, int, const void *, const uint16_t *, float *,
                       hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_gemv_grouped(const void *, const wq_desc *, int, int64_t, int64_t, hipStream_t) { ++launches; return hipSuccess; }
bool gemm_skinny(int64_t, int64_t, int64_t, int) { return false; }
hipError_t launch_gemm(const float *, int64_t, int64_t, int64_t, int, const void *, const uint16_t *, float *, void *,
                       hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_gemm_grouped(const void *, const wq_desc *, int, int64_t, int64_t, void *, hipStream_t) { ++launches; return hipSuccess; }
hipError_t gemm_noalloc_scratch(void **) { ++launches; return hipErrorInvalidValue; }
hipError_t launch_mgemv(const float *, int64_t, int64_t, int64_t, int, const void *, const uint16_t *, float *,
                        hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_mgemv_grouped(const void *, const wq_desc *, int, int64_t, int64_t, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_embed(const int32_t *, int64_t, int64_t, int64_t, int, const void *, const uint16_t *, float *,
                        hipStream_t) { ++launches; return hipSuccess; }
}  // namespace wq

static int failures = 0;
#define EXPECT(c)                                                        \
    do {                                                                 \
        if (!(c)) {                                                      \
            std::fprintf(stderr, "line %d: %s\n", __LINE__, #c);        \
            failures++;                                                  \
        }                                                                \
    } while (0)

static uint64_t rng_state = 12345;
static uint64_t rnd()
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main()
{
    float *const FAKE = reinterpret_cast<float *>(0x10000);   // aligned, never dereferenced
    float *const MIS = reinterpret_cast<float *>(0x10004);
    const void *FQ = FAKE;
    const uint16_t *FS = reinterpret_cast<const uint16_t *>(FAKE);

    // sizes
    EXPECT(wq_q_bytes(2048, 1024, 4) == 2048u * 512);
    EXPECT(wq_q_bytes(10, 128, 5) == 800 && wq_q_bytes(10, 96, 5) == 0 && wq_q_bytes(10, 32, 6) == 0);
    EXPECT(wq_s_bytes(2048, 1024) == 2048u * 64 && wq_s_bytes(-1, 32) == 0);

    // validation of the matmul entry points: every failure is reported before a launch
    typedef int (*mm_t)(const float *, int64_t, int64_t, int64_t, int, const void *, const uint16_t *, float *,
                        hipStream_t);
    const mm_t fns[4] = {wq_gemv, wq_gemm, wq_linear, wq_gemm_noalloc};
    for (mm_t f : fns) {
        EXPECT(f(FAKE, 1, 32, 8, 6, FQ, FS, FAKE, nullptr) == WQ_ERR_BITS);
        EXPECT(f(FAKE, 1, 33, 8, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_SHAPE);
        EXPECT(f(FAKE, 1, 96, 8, 5, FQ, FS, FAKE, nullptr) == WQ_ERR_SHAPE);
        EXPECT(f(FAKE, -1, 32, 8, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_SHAPE);
        EXPECT(f(FAKE, 1, 32, -8, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_SHAPE);
        EXPECT(f(nullptr, 0, 32, 8, 4, nullptr, nullptr, nullptr, nullptr) == WQ_OK);
        EXPECT(f(nullptr, 3, 32, 0, 8, nullptr, nullptr, nullptr, nullptr) == WQ_OK);
        EXPECT(f(nullptr, 1, 32, 8, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_NULL);
        EXPECT(f(FAKE, 1, 32, 8, 4, nullptr, FS, FAKE, nullptr) == WQ_ERR_NULL);
        EXPECT(f(MIS, 1, 32, 8, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_ALIGN);
        EXPECT(f(FAKE, 1, 32, 8, 4, FQ, FS, MIS, nullptr) == WQ_ERR_ALIGN);
    }
    EXPECT(wq_gemv(FAKE, 17, 32, 8, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_M_RANGE);
    EXPECT(wq_gemm(FAKE, (int64_t)1 << 21, 1024, 8, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_SHAPE);   // 2 M K >= 2^32
    EXPECT(wq_gemm(FAKE, 4, 1024, (int64_t)1 << 22, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_SHAPE);
    EXPECT(wq_gemm_noalloc(FAKE, 4097, 4096, 64, 4, FQ, FS, FAKE, nullptr) == WQ_ERR_SCRATCH);
    EXPECT(wq_pack(FAKE, 4, 32, 3, FAKE, nullptr, nullptr) == WQ_ERR_BITS);
    EXPECT(wq_pack(FAKE, 4, 48, 4, FAKE, reinterpret_cast<uint16_t *>(FAKE), nullptr) == WQ_ERR_SHAPE);
    EXPECT(wq_unpack(FQ, 4, 32, 4, nullptr, nullptr) == WQ_ERR_NULL);
    EXPECT(wq_embed(reinterpret_cast<const int32_t *>(FAKE), 3, 33, 8, 8, FQ, FS, FAKE, nullptr) == WQ_ERR_SHAPE);
    EXPECT(wq_embed(nullptr, 0, 32, 8, 8, nullptr, nullptr, nullptr, nullptr) == WQ_OK);
    for (int st = 0; st <= 9; ++st) EXPECT(wq_strerror(st) != nullptr && std::strlen(wq_strerror(st)) > 0);
    EXPECT(wq_abi_version() == 7);

    // layout and planners over random tables
    for (int trial = 0; trial < 200; ++trial) {
        const int count = 1 + (int)(rnd() % 300);
        std::vector<wq_desc> t(count);
        std::memset(t.data(), 0, sizeof(wq_desc) * count);
        const int bits_of[3] = {4, 5, 8};
        for (int i = 0; i < count; ++i) {
            t[i].bits = bits_of[rnd() % 3];
            t[i].K = 128 * (int64_t)(1 + rnd() % 24);
            t[i].N = (rnd() % 10 == 0) ? 0 : (int64_t)(1 + rnd() % 5000);
        }
        uint64_t bytes = 0;
        EXPECT(wq_table_layout(t.data(), count, &bytes) == WQ_OK);
        uint64_t end = 0;
        for (int i = 0; i < count; ++i) {
            EXPECT(t[i].q_off % 64 == 0 && t[i].s_off % 64 == 0 && t[i].q_off >= end);
            end = t[i].s_off + wq_s_bytes(t[i].N, t[i].K);
            EXPECT(t[i].s_off >= t[i].q_off + wq_q_bytes(t[i].N, t[i].K, t[i].bits));
        }
        EXPECT(bytes >= end);
        // activations: a few shared ones (same x and K), 256-byte aligned fake addresses
        for (int i = 0; i < count; ++i) {
            const int share = (int)(rnd() % 4);
            t[i].x = reinterpret_cast<const float *>((uintptr_t)0x1000000 + (uintptr_t)(share * 0x100000 + (i % 7) * 0x40000));
            t[i].y = reinterpret_cast<float *>((uintptr_t)0x80000000u + (uintptr_t)i * 0x10000);
        }
        const int64_t M = 1 + (int64_t)(rnd() % 700);
        int64_t tiles = -1;
        if (M <= 16) {
            EXPECT(wq_table_plan(t.data(), count, M, &tiles) == WQ_OK);
            EXPECT(tiles >= 0);
        }
        uint64_t ws = 0;
        int64_t gt = -1;
        const int st = wq_table_plan_gemm(t.data(), count, M, &gt, &ws);
        EXPECT(st == WQ_OK);
        if (st == WQ_OK) {
            // entries with the same (x, K, int8 order) share a workspace slot; others get
            // distinct ones; the first entry of a slot prepares it (ws_slot >= 0), later
            // sharers hold the slot's complement
            auto slot_of = [](int32_t s) { return s >= 0 ? s : ~s; };
            for (int i = 0; i < count; ++i) {
                if (t[i].N == 0) continue;
                bool earlier = false;
                for (int j = 0; j < i; ++j) {
                    if (t[j].N == 0) continue;
                    const bool same = t[i].x == t[j].x && t[i].K == t[j].K && (t[i].bits == 8) == (t[j].bits == 8);
                    EXPECT(same == (slot_of(t[i].ws_slot) == slot_of(t[j].ws_slot)));
                    earlier = earlier || same;
                }
                EXPECT(earlier == (t[i].ws_slot < 0));
            }
            // work items of non-empty entries are disjoint and inside the launch
            std::vector<uint8_t> used((size_t)gt, 0);
            for (int i = 0; i < count; ++i) {
                if (t[i].N == 0) continue;
                const int64_t n = wq::gemm_grouped_items(M, t[i].N, t[i].K);
                EXPECT(t[i].tile_begin % 8 == 0 && t[i].tile_begin + n <= gt);
                for (int64_t k = 0; k < n && t[i].tile_begin + k < gt; ++k) {
                    EXPECT(!used[(size_t)(t[i].tile_begin + k)]);
                    used[(size_t)(t[i].tile_begin + k)] = 1;
                }
            }
            EXPECT(ws % 256 == 0);
            // the prepared-x slots lie after the split-K header and inside the workspace
            const uint64_t head = wq::gemm_grouped_header_bytes(M, gt);
            for (int i = 0; i < count; ++i)
                if (t[i].N > 0) {
                    const uint64_t off = (uint64_t)slot_of(t[i].ws_slot) * 256;
                    EXPECT(off >= head && off + wq::gemm_ws_bytes(M, t[i].K) <= ws);
                }
        }
        // an inconsistent entry is refused
        if (count > 1) {
            t[count / 2].q_off += 1;
            EXPECT(wq_table_plan_gemm(t.data(), count, M, &gt, &ws) != WQ_OK);
        }
    }
    EXPECT(launches == 0);
    if (failures) {
        std::fprintf(stderr, "%d expectations failed\n", failures);
        return 1;
    }
    std::printf("abi sanitize run: all checks passed\n");
    return 0;
}
