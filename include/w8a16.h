/*
 * w8a16.h -- C ABI of the block-scaled FP8 W8A16 small-M GEMM for MI355X
 * (gfx950).
 *
 * The operation (page "w8a16_gemm_pipelined_m32.rs", doc comment of
 * `w8a16_gemm_pipelined_m32_strided`; one FP8 scale block per 128-wide K
 * step, doc comment of `W8A16_M32_K_BLOCK`):
 *
 *   C[i][j] = bf16( sum_{b < K/128} S[j/128][b] * sum_{t < 128} A[i][128b+t] * W[j][128b+t] )
 *
 *   A  BF16 (bits, 2 bytes)   [m, a_row_stride]   first k elements of each row are read
 *   W  FP8 E4M3 (OCP E4M3FN)  [n, k]              row-major, contiguous, 1 byte per weight
 *   S  FP32                   [ceil(n/128), k/128] row-major: scale of W block (j/128, k/128)
 *   C  BF16                   [m, c_row_stride]   first n elements of each row are written
 *
 * Strides are in elements.  Products are taken in BF16 x BF16 with FP32
 * accumulation; each 128-wide K step's partial sum is multiplied by its
 * block scale once and added in FP32; the result is rounded to BF16 with
 * round-to-nearest-even.  The association of the K reduction inside a step,
 * across the waves of a workgroup and across K splits is fixed by the plan,
 * so a given plan gives the same bits on every run.
 *
 * Ownership: every pointer passed to w8a16_gemm* is a DEVICE pointer owned
 * by the caller, who keeps the buffers alive until the stream has passed
 * the call.  The library keeps no pointer to them.  It owns one split-K
 * workspace and counter array per (device, stream), allocated with
 * hipMalloc on first use and grown when a larger plan needs it.  Growing
 * allocates new buffers and keeps the old ones until the process ends, so
 * calls in flight and HIP graphs captured earlier on that stream stay
 * valid; it needs no synchronisation.  Growth cannot happen while the
 * stream is being captured: such a call returns W8A16_ERR_WORKSPACE and
 * enqueues nothing, so make one call with the largest plan on a stream
 * before capturing it.  A graph keeps using the workspace of the stream it
 * was captured on: two replays of graphs captured on one stream must not
 * overlap in time.
 *
 * Alignment and aliasing: A, W, S and C must be 16-byte aligned (torch
 * allocations are).  C must not overlap A, W or S.  c_row_stride may be any
 * value >= n.
 *
 * Errors: every entry point returns a w8a16_status.  Argument errors are
 * detected before anything is enqueued, in the order of the enum below
 * (codes 1..4 in the order the page checks them; 5..7 and 9 are checks the
 * page does not make; 10, a bad diagnostic setting, is checked first).
 * w8a16_last_error() then holds a message for the calling thread.  Launches are asynchronous: the call returns once the kernel is
 * enqueued on `stream`; a failed enqueue returns W8A16_ERR_HIP.
 */
#ifndef W8A16_H
#define W8A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w8a16_status {
    W8A16_OK = 0,
    W8A16_ERR_M_ZERO = 1,            /* m == 0: no rows to compute */
    W8A16_ERR_K_NOT_MULT_128 = 2,    /* k == 0 or k % 128 != 0 */
    W8A16_ERR_PITCH_TOO_SHORT = 3,   /* a_row_stride < k or c_row_stride < n */
    W8A16_ERR_A_STRIDE_ALIGN = 4,    /* a_row_stride % 8 != 0 (16-byte rows) */
    W8A16_ERR_N_ZERO = 5,            /* n == 0: empty launch */
    W8A16_ERR_NULL_PTR = 6,          /* a, w_fp8, block_scale or c is null */
    W8A16_ERR_BAD_PLAN = 7,          /* a plan that does not fit the problem */
    W8A16_ERR_HIP = 8,               /* allocation or launch failed in HIP */
    W8A16_ERR_WORKSPACE = 9,         /* the plan's split-K workspace cannot be provided:
                                        it would have to grow during stream capture,
                                        or it exceeds w8a16_gemm_noalloc's scratch */
    W8A16_ERR_ENV = 10               /* a diagnostic environment variable holds a value
                                        other than 0 or 1 (see Diagnostics below) */
} w8a16_status;

/* Diagnostics.  Two environment variables, read once per process at the
 * first call of an entry point that enqueues work (w8a16_gemm,
 * _gemm_planned, _gemm_noalloc, _gemm_batched, _act_quant_fp8,
 * _gemm_w8a8[_planned], _gemm_w4a4[_planned]); unset, empty or "0" is off,
 * "1" is on, and any other value makes each of those calls return
 * W8A16_ERR_ENV, before any other check, with the variable named in
 * w8a16_last_error().  The pure planning calls ignore them.
 *   W8A16_LOG=1: each distinct launch (entry point, m, n, k and plan) is
 *     printed once to stderr: kernel, tile, K splits, waves, grid, LDS,
 *     workspace, and for a default plan the planner rule that chose it.
 *   W8A16_DEBUG_SYNC=1: after enqueuing, the call waits for the stream and
 *     returns W8A16_ERR_HIP if the kernel failed.  On a stream being
 *     captured into a graph it does not wait (nothing runs until replay).
 *     It serialises the caller with the GPU: for debugging only. */

/* Kernel families a plan can name. */
typedef enum w8a16_kernel {
    /* Weight-streaming kernel: a workgroup owns n_blocks 16-column blocks
     * of C and m_blocks 16-row blocks, its waves take interleaved 128-wide
     * K steps, and K may be split across workgroups with a fixed-order
     * FP32 fix-up. */
    W8A16_KERNEL_STREAM = 1,
    /* Tiled kernel for m above 32: a workgroup owns a 16*m_blocks-row
     * (64 or 128) x 16*n_blocks-column (64 or 128) tile of C, stages A and
     * the FP8 weight of each K step in LDS rings (a_depth and depth
     * buffers), and its waves split the tile (8 waves: also each K step). */
    W8A16_KERNEL_TILE = 2,
    /* Ring kernel for small m: a workgroup owns n_blocks 16-column blocks
     * and m_blocks 16-row blocks of C over all of K, streams K in stages of
     * stage_steps steps with a ring of `depth` stages in flight (1 KiB
     * row-contiguous LDS-DMA loads), and its waves, grouped per column
     * block, take the stages' steps round-robin.  No K split. */
    W8A16_KERNEL_RING = 3,
    /* W8A8 kernel (w8a16_gemm_w8a8 only): A given as FP8 codes with one
     * scale per (row, K step); the stream kernel's organisation with A
     * staged like the weight and one FP8 MFMA per K step.  No K split. */
    W8A16_KERNEL_W8A8 = 4,
    /* W4A4 MX kernel (w8a16_gemm_w4a4 only): a workgroup owns n_blocks
     * 16-column blocks and m_blocks 16-row blocks of C over all of K, its
     * waves take interleaved groups of four 128-wide K steps with one scaled
     * FP4 MFMA per block and step, each activation fragment feeding the
     * n_blocks weight blocks.  No K split. */
    W8A16_KERNEL_W4A4 = 5,
    /* Persistent W4A4 MX kernel: one workgroup per CU owns an equal
     * contiguous range of 16-row weight tiles and stages all of A in LDS;
     * its waves split the range's (tile, 4-step K group) items evenly and
     * add the partials of tiles split between them in wave order. */
    W8A16_KERNEL_W4A4_PS = 6
} w8a16_kernel;

/* Launch plan.  w8a16_plan() fills every field; callers may change
 * kernel, m_blocks, n_blocks, splits, depth, flags, waves, stage_steps and
 * a_depth and pass the result to
 * w8a16_gemm_planned(), which recomputes the derived fields and rejects a
 * plan the kernels do not support (W8A16_ERR_BAD_PLAN). */
typedef struct w8a16_plan {
    uint32_t kernel;          /* w8a16_kernel */
    uint32_t m_blocks;        /* 16-row blocks of C per workgroup tile */
    uint32_t n_blocks;        /* 16-column blocks of C per workgroup tile */
    uint32_t splits;          /* K splits across workgroups (>= 1) */
    uint32_t steps_per_split; /* 128-wide K steps per split (derived) */
    uint32_t m_tiles;         /* ceil(m / (16 * m_blocks)) (derived) */
    uint32_t n_tiles;         /* ceil(n / (16 * n_blocks)) (derived) */
    uint32_t grid;            /* workgroups launched (derived) */
    uint32_t block;           /* threads per workgroup (derived) */
    uint32_t lds_bytes;       /* LDS per workgroup (derived) */
    uint64_t workspace_bytes; /* split-K FP32 partials (derived; 0 if splits == 1) */
    uint32_t counter_count;   /* 32-bit words of split-K arrival counters, one counter
                                 per tile every 64 words (derived) */
    uint32_t cu_count;        /* compute units the plan was sized for */
    uint32_t depth;           /* stream: K steps each wave keeps in flight (1, 2, 4);
                                 tile: weight ring buffers; ring: stages in flight (2..4) */
    uint32_t flags;           /* W8A16_FLAG_* bits */
    uint32_t waves;           /* waves per workgroup (stream 4/8/16, ring 8/16,
                                 tile 4/6/8/10) */
    uint32_t stage_steps;     /* ring: K steps per stage (4 or 8); 0 for the others */
    uint32_t a_depth;         /* tile: A ring buffers (2..6; 0 means 2); 0 for the others */
} w8a16_plan_t;

/* Plan flags. */
enum {
    /* Stream kernel: load A fragments straight into the MFMA register
     * layout instead of staging coalesced loads through LDS (the weight is
     * always staged). */
    W8A16_FLAG_DIRECT = 1u,
    /* Ring kernel, m <= 8 with m_blocks == 1: stage 8 A rows instead of 16
     * (derived by w8a16_plan_finalize from m; callers need not set it). */
    W8A16_FLAG_A8 = 2u,
    /* Stream kernel with splits > 1: the K splits of every tile run on one
     * XCD (consecutive logical workgroups inside one XCD's contiguous range
     * of the grid), so the partials they exchange stay in that XCD's L2.
     * w8a16_plan() sets it on every plan that splits K.
     * w8a16_plan_finalize() rejects it (W8A16_ERR_BAD_PLAN) unless
     * splits >= 2, the grid is a multiple of 8 and each eighth of the grid
     * holds whole tiles.  The publication itself is the same with or
     * without the flag: each split stores its partial with agent-scope
     * (write-through) stores, waits for them, then counts its arrival; the
     * last one acquires at agent scope and reads the partials with
     * agent-scope loads.  It is correct on whichever XCDs the splits run. */
    W8A16_FLAG_XCD_LOCAL = 4u
};

/* Validate the scalar arguments alone, in the documented order.  Pure: no
 * GPU call.  Returns W8A16_OK or the first failing check's code. */
int w8a16_check_args(uint32_t m, uint32_t n, uint32_t k,
                     uint32_t a_row_stride, uint32_t c_row_stride);

/* Default plan for (m, n, k) on a device with `cu_count` compute units
 * (0 means 256, MI355X).  Pure: no GPU call.  Checks m, n and k as
 * w8a16_check_args does (pitches are not part of a plan). */
int w8a16_plan(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count,
               w8a16_plan_t *out);

/* Recompute the derived fields of a caller-edited plan and check it.
 * Pure: no GPU call. */
int w8a16_plan_finalize(uint32_t m, uint32_t n, uint32_t k, w8a16_plan_t *plan);

/* The GEMM.  a: BF16 [m, a_row_stride]; w_fp8: E4M3 [n, k]; block_scale:
 * FP32 [ceil(n/128), k/128]; c: BF16 [m, c_row_stride].  All device
 * pointers.  stream: a hipStream_t (NULL for the null stream).  Picks the
 * plan with w8a16_plan() for the current device's CU count. */
int w8a16_gemm(const void *a, uint32_t a_row_stride,
               const void *w_fp8, const float *block_scale,
               void *c, uint32_t c_row_stride,
               uint32_t m, uint32_t n, uint32_t k, void *stream);

/* The GEMM with an explicit plan (kernel, m_blocks, n_blocks, splits taken
 * from *plan; derived fields recomputed).  For tests and tuning: every
 * valid plan computes the same operation; plans differ only in the order of
 * the FP32 additions. */
int w8a16_gemm_planned(const void *a, uint32_t a_row_stride,
                       const void *w_fp8, const float *block_scale,
                       void *c, uint32_t c_row_stride,
                       uint32_t m, uint32_t n, uint32_t k,
                       const w8a16_plan_t *plan, void *stream);

/* ---- No-allocation entry point --------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * w8a16_gemm_noalloc() computes exactly what w8a16_gemm() computes, with
 * the same default plan, arguments, checks (codes 1..6) and asynchronous
 * launch, but the split-K partials and arrival counters of a plan that
 * splits K come from a static device array the library holds on each GPU
 * it runs on until the process ends (W8A16_NOALLOC_WORKSPACE_BYTES of
 * partials plus W8A16_NOALLOC_COUNTERS 32-bit counter words, 17 MiB).  It
 * calls no hipMalloc, hipFree or other allocating routine.  A plan needing
 * more than that returns W8A16_ERR_WORKSPACE and enqueues nothing.  The
 * first call on a device looks the array up and clears its counters with a
 * small kernel on `stream`; every later call leaves them at zero.
 *
 * All calls on one GPU share its array: calls that overlap in time on that
 * GPU (other streams, concurrent graph replays) race and give wrong
 * results.  Order them (one stream, or events). */
#define W8A16_NOALLOC_WORKSPACE_BYTES (16u << 20)
#define W8A16_NOALLOC_COUNTERS (1u << 18)

int w8a16_gemm_noalloc(const void *a, uint32_t a_row_stride,
                       const void *w_fp8, const float *block_scale,
                       void *c, uint32_t c_row_stride,
                       uint32_t m, uint32_t n, uint32_t k, void *stream);

/* ---- Batched tier ------------------------------------------------------
 * The pages' strided launch exists so that a multi-sequence Q/K/V tier can
 * hold it as one arm among several with their own pitches (page
 * "w8a16_gemm_pipelined_m32.rs", module doc and the doc comment of
 * `w8a16_gemm_pipelined_m32_strided`).  Here the arms run in one launch. */

/* Most GEMMs one batched call takes. */
#define W8A16_MAX_BATCH 8

/* One GEMM of a batch: the arguments of w8a16_gemm(), same meaning, layout
 * and ownership (device pointers owned by the caller). */
typedef struct w8a16_gemm_desc {
    const void *a;            /* BF16 [m, a_row_stride] */
    const void *w_fp8;        /* E4M3 [n, k] */
    const float *block_scale; /* FP32 [ceil(n/128), k/128] */
    void *c;                  /* BF16 [m, c_row_stride] */
    uint32_t a_row_stride;
    uint32_t c_row_stride;
    uint32_t m, n, k;
} w8a16_gemm_desc_t;

/* Plan of a batched call from the descriptors' m, n and k (pointers and
 * pitches are not read).  Pure: no GPU call.  One stream-kernel variant
 * serves every problem, without K splits; grid is the total workgroup
 * count, m_tiles the largest per problem and n_tiles the sum.  Errors:
 * W8A16_ERR_NULL_PTR (descs or out null), W8A16_ERR_BAD_PLAN (count not in
 * 1..W8A16_MAX_BATCH, or some m above 64), or the first failing problem's
 * w8a16_check_args() code, with its index in w8a16_last_error(). */
int w8a16_plan_batched(const w8a16_gemm_desc_t *descs, uint32_t count, uint32_t cu_count,
                       w8a16_plan_t *out);

/* `count` independent GEMMs (descs is a host array) in one launch of the
 * stream kernel on `stream`; problem i computes exactly what w8a16_gemm()
 * would with descs[i].  Each descriptor is checked as w8a16_gemm() checks
 * its arguments, in order; on the first failure nothing is launched and
 * that code is returned (index in w8a16_last_error()).  Asynchronous.  The
 * problems' outputs must not overlap each other or any input. */
int w8a16_gemm_batched(const w8a16_gemm_desc_t *descs, uint32_t count, void *stream);

/* ---- FP8 activations and the W8A8 GEMM ----------------------------------
 * The per-token FP8 activation quantizer of page "fp8_act_quant.rs" (one
 * group = 128 consecutive K elements of one token; tokens on grid X, groups
 * on grid Y) and the block-scaled GEMM that consumes its output.  The page
 * gives the grouping, not the arithmetic; the reading used: per (token,
 * group) s = amax / 448 and code = E4M3 round-to-nearest-even of x / s, both
 * divisions in binary32, saturated to +-448; an all-zero group gets s = 0
 * and zero codes. */

/* Quantize a: BF16 [m, a_row_stride] (first k of each row) into q: E4M3
 * [m, q_row_stride] (first k of each row written) and scales: FP32
 * [m, k/128] row-major.  Device pointers owned by the caller.  Errors, in
 * order: m == 0; k not a positive multiple of 128; a_row_stride or
 * q_row_stride below k (W8A16_ERR_PITCH_TOO_SHORT); a_row_stride not a
 * multiple of 8 or q_row_stride not a multiple of 16 (16-byte rows,
 * W8A16_ERR_A_STRIDE_ALIGN); a null pointer.  Nothing is launched on an
 * error.  Asynchronous on `stream`. */
int w8a16_act_quant_fp8(const void *a, uint32_t a_row_stride, void *q, uint32_t q_row_stride,
                        float *scales, uint32_t m, uint32_t k, void *stream);

/* Default plan of the W8A8 GEMM (kernel W8A16_KERNEL_W8A8).  Pure. */
int w8a16_plan_w8a8(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count,
                    w8a16_plan_t *out);

/*   C[i, j] = bf16( sum_b a_scales[i, b] * block_scale[j/128, b] *
 *                   sum_t qa[i, 128b + t] * w_fp8[j, 128b + t] )
 * qa: E4M3 [m, qa_row_stride]; a_scales: FP32 [m, k/128]; w_fp8 and
 * block_scale as for w8a16_gemm; c: BF16 [m, c_row_stride].  The two scales
 * are multiplied in FP32 and folded once per K step.  Checks as w8a16_gemm
 * with qa_row_stride in place of a_row_stride, which must be a multiple of
 * 16 (16-byte rows).  Asynchronous. */
int w8a16_gemm_w8a8(const void *qa, uint32_t qa_row_stride, const float *a_scales,
                    const void *w_fp8, const float *block_scale, void *c,
                    uint32_t c_row_stride, uint32_t m, uint32_t n, uint32_t k, void *stream);

/* w8a16_gemm_w8a8 with an explicit plan (kernel must be W8A16_KERNEL_W8A8;
 * m_blocks, n_blocks and waves taken from it).  For tests and tuning. */
int w8a16_gemm_w8a8_planned(const void *qa, uint32_t qa_row_stride, const float *a_scales,
                            const void *w_fp8, const float *block_scale, void *c,
                            uint32_t c_row_stride, uint32_t m, uint32_t n, uint32_t k,
                            const w8a16_plan_t *plan, void *stream);

/* ---- W4A4 MX projection GEMV ---------------------------------------------
 * The m-row W4A4 projection of page "w4a4_proj/mx_plan.rs" (up to 64 rows;
 * weight rows in 16-row tiles; tiers by m; activation reuse across weight
 * tiles; a persistent entry for wide weights).  The page states no number
 * format; the reading is OCP MXFP4 for both operands: FP4 E2M1 elements
 * (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives), two per byte with the
 * even element in the low nibble, and one E8M0 scale byte (2^(e - 127)) per
 * 32 consecutive K elements of a row:
 *
 *   C[i][j] = bf16( sum_b 2^(ea[i][b]-127) * 2^(ew[j][b]-127) * sum_{t<32} a[i][32b+t] * w[j][32b+t] )
 *
 *   a        FP4   [m, a_row_stride]  elements; a row is a_row_stride / 2 bytes
 *   a_scale  E8M0  [m, k/32]          row-major, contiguous
 *   w_fp4    FP4   [n, k]             row-major, contiguous (k/2 bytes per row)
 *   w_scale  E8M0  [n, k/32]          row-major, contiguous
 *   c        BF16  [m, c_row_stride]  first n elements of each row written
 *
 * Products are exact, sums FP32 (the matrix cores apply the two block scales
 * to each 32-element partial), one round-to-nearest-even to BF16.  Device
 * pointers owned by the caller, 16-byte aligned.  Errors, in order: m == 0;
 * k not a positive multiple of 128; a_row_stride < k or c_row_stride < n;
 * a_row_stride not a multiple of 32 (16-byte rows); n == 0; k or
 * a_row_stride above 2^24 elements (W8A16_ERR_BAD_PLAN: the kernels address
 * a tile's rows through 32-bit buffer ranges); a null pointer; m above 64
 * (W8A16_ERR_BAD_PLAN).  No workspace.  Asynchronous. */
int w8a16_gemm_w4a4(const void *a, uint32_t a_row_stride, const uint8_t *a_scale,
                    const void *w_fp4, const uint8_t *w_scale, void *c, uint32_t c_row_stride,
                    uint32_t m, uint32_t n, uint32_t k, void *stream);

/* Default plan of the W4A4 GEMV (kernel W8A16_KERNEL_W4A4 or _W4A4_PS).
 * Pure: no GPU call. */
int w8a16_plan_w4a4(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count,
                    w8a16_plan_t *out);

/* w8a16_gemm_w4a4 with an explicit plan (kernel W8A16_KERNEL_W4A4:
 * m_blocks 1, 2 or 4 and n_blocks 1, 2 or 4, not both 4, with 4 waves, 8
 * waves up to m_blocks + n_blocks = 4, 16 waves for 1 x 1; kernel
 * W8A16_KERNEL_W4A4_PS: m_blocks 1, 2 or 4 covering m, 4, 8 or 16 waves,
 * and the staged activations plus two partial tiles per wave within the
 * LDS, else W8A16_ERR_BAD_PLAN).  For tests and tuning. */
int w8a16_gemm_w4a4_planned(const void *a, uint32_t a_row_stride, const uint8_t *a_scale,
                            const void *w_fp4, const uint8_t *w_scale, void *c,
                            uint32_t c_row_stride, uint32_t m, uint32_t n, uint32_t k,
                            const w8a16_plan_t *plan, void *stream);

/* Static text for a status code (never null). */
const char *w8a16_status_string(int status);

/* Message of the calling thread's last failing call ("" if none). */
const char *w8a16_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A16_H */
