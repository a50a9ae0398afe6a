/*
 * wq.h -- weight-only block-32 int4/int5/int8 matmul for AMD MI355X (gfx950).
 *
 * The operation (TinyMOSS-Diarize devpost page, "How we built it": strictly
 * weight-only kernels, FP32 activations, dequantization fused into the matmul,
 * no dequantized weight tensor ever materialized; moss-transcribe-diarize-litert
 * card, "v2 decoder": int4 block-32; soniqo MOSS guide RU, implementation notes:
 * symmetric linear INT8 block-32):
 *
 *     y[m,n] = sum_b s[n,b] * sum_{k in block b} q[n,k] * x[m,k]
 *
 * Layouts (one canonical layout, all row-major and contiguous):
 *   x       fp32  [M][K]
 *   y       fp32  [M][N]            (overwritten; no bias, no accumulate)
 *   q int4  uint8 [N][K/2]          two codes per byte, low nibble = even k,
 *                                   two's complement, codes in [-8, 7]
 *   q int5  uint8 [N][5K/8]         per row: K/2 bytes of the low 4 bits of every
 *                                   code as for int4, then K/8 bytes of bit 4 of
 *                                   every code (code k in bit k%8 of byte k/8);
 *                                   5-bit two's complement, codes in [-16, 15].
 *                                   (INT5 is the MLX default of the soniqo MOSS
 *                                   guide, "INT5 vs INT8"; the pages give no
 *                                   layout or scale rule, this is the library's.)
 *   q int8  int8  [N][K]            two's complement, codes in [-128, 127]
 *   scales  binary16 bits [N][K/32] one scale per 32 consecutive k
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers on the current HIP device, owned by the
 *     caller. The only state the library keeps is the workspace of wq_gemm
 *     (and wq_linear for M > 16): one stream-ordered device memory pool per
 *     device (created on first use, kept until the process ends) and, per
 *     (device, stream), the workspace of the last call on that stream, reused
 *     while large enough (calls on one stream run in order; streams are told
 *     apart by their process-unique id), and the fixed device scratch of
 *     wq_gemm_noalloc. No other entry point allocates.
 *   - Arguments are validated on the host before any launch; a non-zero
 *     wq_status is returned and nothing is launched. Requirements: bits in
 *     {4, 5, 8}; K > 0 and K % 32 == 0 (K % 128 == 0 for int5, so rows stay
 *     16-byte aligned); N >= 0; M >= 0; non-null pointers for
 *     non-empty calls; x, y, q, scales 16-byte aligned. y must not alias an
 *     input.
 *   - Empty calls (M == 0 or N == 0) return WQ_OK without launching.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); a
 *     launch error is reported as WQ_ERR_HIP. There is no implicit sync.
 *   - Results are deterministic: no read-modify-write atomics, a fixed
 *     reduction order (split K loops of the grouped prefill hand partial sums
 *     over through flag stores and loads and add them in piece order).
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum wq_status {
    WQ_OK = 0,
    WQ_ERR_NULL = 1,      /* a required pointer is null */
    WQ_ERR_SHAPE = 2,     /* K <= 0, K % 32 != 0 (int5: K % 128 != 0), negative M or N, or too large */
    WQ_ERR_BITS = 3,      /* bits not 4, 5 or 8 */
    WQ_ERR_ALIGN = 4,     /* a pointer or table offset is misaligned */
    WQ_ERR_M_RANGE = 5,   /* M outside the entry point's range (wq_gemv: 1..16) */
    WQ_ERR_HIP = 6,       /* the HIP runtime reported an error at launch */
    WQ_ERR_TABLE = 7,     /* a tensor-table entry is inconsistent */
    WQ_ERR_SCRATCH = 8    /* wq_gemm_noalloc: the workspace exceeds WQ_NOALLOC_SCRATCH_BYTES */
};

#define WQ_BLOCK 32           /* values per quantization block along K */
#define WQ_GEMV_MAX_M 16      /* largest M accepted by wq_gemv */
#define WQ_TABLE_ALIGN 64     /* alignment of tensors in a package and of table entries */
#define WQ_NOALLOC_SCRATCH_BYTES (32u << 20)   /* per-device scratch of wq_gemm_noalloc */

/* Bytes of packed codes for an [N][K] tensor: N*K*bits/8. 0 on bad arguments. */
size_t wq_q_bytes(int64_t N, int64_t K, int bits);
/* Bytes of binary16 scales for an [N][K] tensor: N*(K/32)*2. 0 on bad arguments. */
size_t wq_s_bytes(int64_t N, int64_t K);

/*
 * wq_pack -- quantize and pack fp32 weights w [N][K] into q and scales.
 * Per row n and block b of 32 consecutive k (the block-32 symmetric scheme of
 * the pages above; the scale rule and rounding are this library's reading):
 *   amax = max |w|;  s = binary16_rne(amax / Q) with fp32 division,
 *   Q = 7 (int4), 15 (int5) or 127 (int8);  if s == 0 every code is 0;
 *   else q = clamp(round_half_even(w / s), -Q-1, Q) with fp32 division by the
 *   stored binary16 scale.
 * Inputs must be finite with amax / Q <= 65504 (not checked here).
 * Output is bit-exact: one correct result exists for every input.
 */
int wq_pack(const float *w, int64_t N, int64_t K, int bits,
            void *q, uint16_t *scales, hipStream_t stream);

/*
 * wq_unpack -- decode packed codes q into one int8 per code, codes [N][K].
 * Inverse of the packing layout above (test and inspection aid).
 */
int wq_unpack(const void *q, int64_t N, int64_t K, int bits,
              int8_t *codes, hipStream_t stream);

/*
 * wq_gemv -- decode path (the devpost page's separate GEMV path for decode),
 * 1 <= M <= 16. M <= 2: codes are unpacked in registers and multiplied in fp32
 * with fused multiply-adds against the fp32 activations; each block's partial
 * is scaled by its fp32-converted scale; lanes along K are reduced within a
 * wavefront. 3 <= M <= 16: x is split exactly into three binary16 parts per
 * (row, block) after a power-of-two normalisation, and the block partials come
 * from fp16 matrix-core instructions with exact products and fp32 sums, then
 * are scaled per block in fp32 as above.
 * Error: |y - y_exact| <= 1e-5 * sum_k |x[m,k]| |w^[n,k]| for M <= 2. For
 * 3 <= M <= 16 the three binary16 parts hold every value within 2^16 of its
 * (row, block)'s largest magnitude exactly and smaller values with an absolute
 * error of at most 2^-39 of that largest (2^-151 where it is below 2^-112), so
 * the bound gains sum_b (2^-39 max_{k in b} |x[m,k]| + 2^-151) sum_{k in b}
 * |w^[n,k]| over the blocks b of the row; for blocks spread over no more than
 * 2^16 it is the plain bound.
 */
int wq_gemv(const float *x, int64_t M, int64_t K, int64_t N, int bits,
            const void *q, const uint16_t *scales, float *y, hipStream_t stream);

/*
 * wq_gemm -- prefill path (the devpost page's blocked prefill GEMM that unpacks
 * each weight group once and reuses it across all activation rows), any M >= 1,
 * tuned for M >= 128. Two kernels on `stream`:
 *   1. x is rounded to binary16 once per call into a workspace: each row m is
 *      scaled by a power of two 2^e_m so that its largest magnitude lies in
 *      [2^14, 2^15), then rounded to nearest even (for rows inside binary16's
 *      normal range this is exactly the binary16 rounding of x, times 2^e_m);
 *   2. packed weight tiles are staged in LDS and every code is unpacked exactly
 *      once per output tile into binary16 (the integer codes are exact there);
 *      each 32-wide K step is one quantization block, computed by fp16
 *      matrix-core instructions into an fp32 partial that is scaled by that
 *      block's scale and accumulated in fp32; y = acc * 2^-e_m.
 * The workspace (about 2*M*K bytes) is the calling stream's buffer from the
 * library's pool on the current device (grown when too small; a fresh pool
 * allocation, freed inside the capture, while the stream is being captured).
 * Few rows and many columns (M <= 64, K = 512 or 1024, or 2048 with M <= 32,
 * and at least 128 columns per compute unit: the M = 64 lm_head) run as one
 * kernel instead, which keeps the prepared x (same rounding) in LDS and needs
 * no workspace.
 * Error: ||Y - Y_exact||_F <= 2e-3 * ||Y_exact||_F per call for finite x whose
 * rows' largest magnitudes are at least 2^-112. Elementwise, for any finite x:
 * |y - y_exact| <= (2^-11 + 1e-5) sum_k |x[m,k]| |w^[n,k]| + 2^-25 2^-e_m
 * sum_k |w^[n,k]|, where 2^-e_m is row m's scaling (its largest magnitude
 * times 2^e_m lies in [2^14, 2^15), e_m <= 126): values whose scaled magnitude
 * is at least 2^-14 keep 11 significant bits, smaller ones an absolute error
 * of at most 2^-25 scaled. A row holding inf or NaN gives non-finite outputs
 * in every column of that row and changes no other row.
 * Sizes: M * K * 2, N * K * bits / 8 and N * K / 16 must each be below 2^32,
 * and N below 2^22 (32-bit offsets in the kernels), else WQ_ERR_SHAPE. A pool
 * allocation failure is reported as WQ_ERR_HIP.
 */
int wq_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits,
            const void *q, const uint16_t *scales, float *y, hipStream_t stream);

/*
 * wq_gemm_noalloc -- wq_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc). Same arguments, kernels, results (bitwise) and error bound as
 * wq_gemm, but the workspace is a fixed per-device scratch array that lives as
 * long as the library is loaded: ceil256(2*M*K) + ceil256(4*M) bytes must not
 * exceed WQ_NOALLOC_SCRATCH_BYTES (32 MiB, e.g. M = 4096 at K = 4096), else
 * WQ_ERR_SCRATCH and nothing is launched. No allocation is made; the first
 * call on a device looks up the scratch's address. Every call on a device
 * shares that device's scratch (nothing in it needs to start at zero), so
 * calls that overlap on one device, e.g. on two streams, race; calls on one
 * stream are ordered and safe.
 */
int wq_gemm_noalloc(const float *x, int64_t M, int64_t K, int64_t N, int bits,
                    const void *q, const uint16_t *scales, float *y, hipStream_t stream);

/* wq_linear -- dispatch by M: M <= 16 -> wq_gemv, M > 16 -> wq_gemm. */
int wq_linear(const float *x, int64_t M, int64_t K, int64_t N, int bits,
              const void *q, const uint16_t *scales, float *y, hipStream_t stream);

/*
 * wq_embed -- tied token embedding (the MOSS-Transcribe-Diarize LiteRT card,
 * "Files": the embedder file holds one tied table for the token embedding and
 * the lm_head, with `embed_1` / `embed_128` lookups beside `logits`). The table
 * is a packed [N][K] tensor in the layout above (normally the int8 lm_head):
 *   out[i][k] = s[ids[i], k/32] * q[ids[i], k]   for 0 <= i < n_ids,
 * in fp32, which is exact. ids: int32 [n_ids], 4-byte aligned; out: fp32
 * [n_ids][K], 16-byte aligned, must not alias the table. A row whose id lies
 * outside [0, N) is filled with quiet NaN and the table is not read for it
 * (ids live on the device, so they are not checked on the host). n_ids == 0
 * returns WQ_OK without launching; with N == 0, q and scales may be null.
 */
int wq_embed(const int32_t *ids, int64_t n_ids, int64_t K, int64_t N, int bits,
             const void *q, const uint16_t *scales, float *out, hipStream_t stream);

/*
 * Packed package and tensor table (the devpost page, "How we built it": the
 * packed tensors live in one container with a 64-byte-aligned tensor table).
 * A package is one device allocation; each tensor's codes and scales start at
 * a multiple of 64 bytes from its base. The table is an array of 64-byte
 * descriptors; a device copy of it drives wq_gemv_grouped.
 */
typedef struct wq_desc {
    int32_t bits;          /* 4, 5 or 8 */
    int32_t ws_slot;       /* prefill plans (set by wq_table_plan_gemm): the offset
                              of this entry's prepared x in the grouped workspace,
                              in 256-byte units, when this entry prepares it, or
                              its bitwise complement (a negative value) when an
                              earlier entry reading the same x prepares it;
                              decode plans set it to 0 */
    int64_t N;             /* output features (rows of q) */
    int64_t K;             /* input features, multiple of 32 */
    uint64_t q_off;        /* byte offset of q from the package base, multiple of 64 */
    uint64_t s_off;        /* byte offset of scales from the package base, multiple of 64 */
    const float *x;        /* device pointer to this call's x [M][K], 16-byte aligned */
    float *y;              /* device pointer to this call's y [M][N], 16-byte aligned */
    int64_t tile_begin;    /* first work item (workgroup) of this tensor; set by wq_table_plan */
} wq_desc;

/*
 * wq_table_layout -- host only. Given bits, N, K in each of `count` entries,
 * assign q_off / s_off in table order (each at the next multiple of 64) and
 * return the package size in *package_bytes. Other fields are left alone.
 */
int wq_table_layout(wq_desc *table, int count, uint64_t *package_bytes);

/*
 * wq_table_plan -- host only. For a grouped call with M rows, set tile_begin of
 * every entry and return the total number of work items (the launch size) in
 * *total_tiles. Validates every entry (bits, shape, 64-byte offsets, 16-byte
 * x / y, non-overlapping codes and scales). Work items are dispatched in table
 * order.
 */
int wq_table_plan(wq_desc *table, int count, int64_t M, int64_t *total_tiles);

/*
 * wq_gemv_grouped -- one launch that runs the decode GEMV of every tensor in a
 * planned table (the per-token decode step over all projections), 1 <= M <= 16.
 * `table_dev` is a device copy of a table planned with the same M; `base` is the
 * package base. Every call's result is bitwise equal to wq_gemv on that tensor.
 * The calls must be independent (no call reads another call's y).
 */
int wq_gemv_grouped(const void *base, const wq_desc *table_dev, int count,
                    int64_t total_tiles, int64_t M, hipStream_t stream);

/*
 * wq_table_plan_gemm -- host only. For a grouped prefill call (wq_gemm_grouped)
 * with M >= 1 rows, set tile_begin and ws_slot of every entry, return the
 * launch size in *total_tiles and the workspace size in *workspace_bytes.
 * Validates every entry as wq_table_plan does, and wq_gemm's size limits for each.
 * Work items are dispatched longest K first (ties in table order), and each
 * entry's items start at a multiple of 8. Entries that read the same x (same
 * pointer and K) with the same code order (int8, or int4/int5) share one
 * workspace slot, prepared by the first of them. For M <= 128 each tile of an
 * entry with K >= 2048 is min(K / 1024, 8) work items (pieces of its K loop),
 * and the workspace starts with a header of one 32-bit flag per work item
 * (rounded up to 256 bytes) and one 64 x 128 fp32 partial tile per work item.
 * The tile shape and split depend on M and K only, so a plan is valid for
 * exactly the M it was made with.
 */
int wq_table_plan_gemm(wq_desc *table, int count, int64_t M, int64_t *total_tiles,
                       uint64_t *workspace_bytes);

/*
 * wq_gemm_grouped -- one launch of x preparation and one of the prefill GEMM
 * over every tensor in a planned table (the devpost page's blocked prefill
 * GEMM, "How we built it", over all projections of a layer at once, so that
 * short prefills fill the chip). `table_dev` is a device copy of a table
 * planned by wq_table_plan_gemm with the same M; `base` is the package base
 * (64-byte aligned); `workspace` is caller-owned device memory of at least the
 * planned workspace_bytes, 256-byte aligned (it may be null when that is 0).
 * Each call's y [M][N] is computed as wq_gemm computes it (same preparation of
 * x, unpack and per-block fp32 scaling), with one tile shape for the whole
 * launch: 64-row tiles with each tile's K loop split two ways within the
 * workgroup for M <= 128, 128-row tiles above. For M <= 128 the K loops of
 * 2048 and more are also split across workgroups (see wq_table_plan_gemm): the
 * leading pieces leave their fp32 partials in the workspace and then set a
 * flag, both with device-scope coherent stores; the last piece of the tile, a
 * workgroup of higher index, waits for those flags (a bounded wait: if a flag never
 * comes, that tile's outputs are NaN), adds the partials in piece order to its
 * own and stores y. Nothing is accumulated with atomic read-modify-write
 * operations. The result is deterministic and meets wq_gemm's error bound; it
 * equals wq_gemm bitwise when both use the same tile shape and no split. The
 * calls must be independent (no call reads another call's y, the y of
 * different entries do not overlap, and no y overlaps the workspace); the
 * workspace must be at least the split-K header of total_tiles work items
 * (else WQ_ERR_SHAPE).
 */
int wq_gemm_grouped(const void *base, const wq_desc *table_dev, int count,
                    int64_t total_tiles, int64_t M, void *workspace,
                    uint64_t workspace_bytes, hipStream_t stream);

/* Human-readable text for a wq_status value (static storage). */
const char *wq_strerror(int status);

/* Library ABI version (increments on any signature or layout change). */
int wq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
