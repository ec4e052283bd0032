/*
 * psi.h -- C ABI of the MI355X paged BF16 block operator.
 *
 * Precision-Preserving Subtensor Inference (cited as [PSI]: "Precision-
 * Preserving Subtensor Inference for a 22B Joint Audio-Video Generator under
 * a Fixed GPU Working Set", arXiv 2611.08023) computes linear projections,
 * the FFN and attention from weight sub-block PAGES that are copied from
 * pinned host memory into a fixed, reusable device ARENA.  The managed
 * device footprint is bounded by the pages, the declared live state and a
 * bounded workspace ([PSI] sec. II-A, eq. (1)):
 *
 *     M_managed <= S_live + W + n_pages * P + eps
 *
 * Conventions for every entry point:
 *   - Return value: PSI_OK (0) or a negative PSI_E_* code.  On error nothing
 *     has been enqueued and the arena/journal state is unchanged; a message
 *     is available from psi_last_error() (thread-local).
 *   - BF16 values are passed as uint16_t bit patterns (bfloat16).
 *   - Pointers named *_dev are device pointers owned by the caller (the
 *     declared live state).  Pointers named *_host point to pinned host
 *     memory (hipHostMalloc / torch pin_memory), owned by the caller, which
 *     must stay valid and unmodified until the compute stream has passed
 *     the operation (psi_arena_sync).
 *   - Streams are hipStream_t passed as void*; NULL means the null stream.
 *   - All operators are asynchronous on the arena's compute stream: a call
 *     returns after enqueueing.  Page copies run on a library-owned copy
 *     stream and are ordered with cross-stream events ([PSI] sec. II-D).
 *   - Matrices are row-major; weights use the Linear layout W[out, in], so
 *     a projection computes y = x W^T + b.
 *   - One arena per host thread; an arena is not thread-safe.
 */
#ifndef PSI_H
#define PSI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int psi_status;

/* ---------------------------------------------------------------- status */
#define PSI_OK 0
#define PSI_E_INVALID (-1)           /* bad shape, pointer or flag; masked/causal attention unsupported */
#define PSI_E_ARENA_TOO_SMALL (-2)   /* n_pages * P + 2 bias slots + W exceeds the arena */
#define PSI_E_SCRATCH_EXHAUSTED (-3) /* an operator's tiles do not fit the arena scratch ([PSI] Table V) */
#define PSI_E_PAGE_TOO_SMALL (-4)    /* a weight tile does not fit one page ([PSI] Table V) */
#define PSI_E_PAGE_BUSY (-5)         /* second unreleased request for a page ([PSI] sec. II-A, rule 2) */
#define PSI_E_NOT_PINNED (-6)        /* host pointer is not pinned (page-locked) memory */
#define PSI_E_ALIGN (-7)             /* pointer or leading dimension not 16-byte aligned */
#define PSI_E_JOURNAL_KEY (-8)       /* journal key missing, duplicated, or size mismatch */
#define PSI_E_HIP (-9)               /* HIP runtime error */
#define PSI_E_STATE (-10)            /* page released/acquired in the wrong lifecycle state */
#define PSI_E_JOURNAL_FULL (-11)     /* journal host store capacity exceeded */

/* ------------------------------------------------------------ arena flags */
#define PSI_ARENA_SYNC_COPY 0x1u /* page copies on the compute stream (transport control) */
#define PSI_ARENA_PROFILE 0x2u   /* time every kernel launch with HIP events */
#define PSI_ARENA_DRY_RUN 0x4u   /* no device memory and no HIP calls: plans, lifecycle and
                                    byte accounting only (host-side tests) */
#define PSI_ARENA_PROFILE_COPIES 0x8u /* with PSI_ARENA_PROFILE: time page copies too (two more
                                         events per copy on the copy streams); also on while a
                                         device timeline is being kept */
#define PSI_ARENA_JITTER 0x10u /* transport control ([PSI] sec. II-D): delay every page or
                                  bias copy and every kernel launch by a deterministic
                                  pseudo-random 0-63 us (a one-wave wait kernel on the copy
                                  or compute stream); results must not change */

/* --------------------------------------------------------- operator flags */
#define PSI_OP_BASELINE_BIAS 0x1u /* [PSI] sec. III-A baseline: round the product to BF16,
                                     then add the bias (default: bias added in fp32) */
#define PSI_OP_RESIDUAL 0x2u      /* y = B(f(x) + f(B(acc + b))) */
#define PSI_OP_STORE_ACC 0x4u     /* also store the final fp32 accumulator to acc_dev */
#define PSI_OP_BF16_SOFTMAX 0x8u  /* attention: BF16 softmax numerator weights (the
                                     [PSI] sec. III-A baseline); default: fp32 weights
                                     (modified PSI), fed to the BF16 matrix cores as
                                     three BF16 terms */
#define PSI_OP_ATTN_P2 0x10u      /* attention: fp32 weights carried as two BF16 terms
                                     (about 17 significant bits; one MFMA fewer per
                                     step); ignored with PSI_OP_BF16_SOFTMAX */
/* Attention kernel (bits 8-10 of the flags): 0 = the automatic choice (the
   ping-pong kernel for 512 or more keys or 256 or more workgroups of 256
   queries, else 128-query workgroups); 1 = 128-query workgroups; 2 = 256-query
   workgroups; 3 = 256-query, software-pipelined with the waves in lock step;
   4 = 256-query ping-pong (the two wave groups alternate softmax and matrix
   phases).  Every choice gives the same bits (a comparison path); other
   values are PSI_E_INVALID. */
#define PSI_OP_ATTN_CONFIG(c) (((unsigned)(c) & 7u) << 8)
#define PSI_OP_ATTN_CONFIG_MASK 0x700u
#define PSI_OP_ATTN_PIPELINED PSI_OP_ATTN_CONFIG(3) /* the lock-step kernel at every size */

/* -------------------------------------------------------- matrix layouts */
#define PSI_SPLIT_ROWS 0 /* page p = rows [p*block, (p+1)*block) of W: an output-column
                            partition of y = x W^T ([PSI] sec. IV-B projections) */
#define PSI_SPLIT_COLS 1 /* page p = columns [p*block, (p+1)*block) of W stored as a
                            contiguous [rows, block] slice: a K-split with a carried fp32
                            accumulator ([PSI] sec. II-B eq. (2), bias added once) */
#define PSI_SPLIT_TILES 2 /* 2-D page tiles: page (o, q) = rows [o*block, ...) x columns
                             [q*block_cols, ...) of W stored as a contiguous [rows, cols]
                             block; pages ordered o-major (p = o * ceil(cols/block_cols) + q).
                             An output tile of `block` rows may then span several pages
                             (the output-tile schedules of psi_ffn_tiled and psi_attn_tiled) */

#define PSI_MAX_PAGES 8

typedef struct psi_arena psi_arena;
typedef struct psi_journal psi_journal;

/* Arena description ([PSI] Fig. 1: two pages, workspace, state/scratch). */
typedef struct psi_arena_desc {
  size_t arena_bytes;     /* A: the single device allocation */
  size_t page_bytes;      /* P: capacity of one weight page */
  int n_pages;            /* reusable page slots, 1..PSI_MAX_PAGES (the paper uses 2) */
  size_t workspace_bytes; /* W: fixed library workspace (reserved, may be 0) */
  size_t bias_slot_bytes; /* each of the two bias slots (an operator's biases are staged
                             in one slot, slots alternate between operators); 0 -> 64 KiB */
  void* compute_stream;   /* hipStream_t the operators run on (caller-owned) */
  unsigned flags;         /* PSI_ARENA_* */
} psi_arena_desc;

/* Byte offsets of the carve inside the arena (256-byte aligned). */
typedef struct psi_arena_layout {
  size_t page_off[PSI_MAX_PAGES];
  size_t bias_off[2];
  size_t bias_slot_bytes;
  size_t workspace_off;
  size_t scratch_off;
  size_t scratch_bytes;
  size_t total_bytes;
} psi_arena_layout;

/* Accounting ([PSI] sec. IV-A/IV-C: arena, scratch high-water, bytes moved,
 * blocking synchronisations). */
typedef struct psi_stats {
  size_t arena_bytes;
  size_t page_bytes;
  size_t workspace_bytes;
  size_t scratch_bytes;
  size_t scratch_high_water;
  uint64_t bytes_h2d;       /* page + bias bytes copied host -> device */
  uint64_t page_copies;     /* page submissions */
  uint64_t event_waits;     /* cross-stream waits enqueued */
  uint64_t host_syncs;      /* blocking host synchronisations performed */
  uint64_t kernel_launches;
  /* PSI_ARENA_PROFILE only (0 otherwise): summed device time per kind */
  double gemm_ms;
  uint64_t gemm_launches;
  double gemm_flops;        /* algorithmic 2*M*N*K of the timed GEMM launches */
  double attn_ms;
  uint64_t attn_launches;
  double attn_flops;        /* algorithmic 4*Mq*Mk*dh per head of the timed launches */
  double copy_ms;           /* busy time of the busier of the two page-copy streams
                               (PSI_ARENA_PROFILE_COPIES or while tracing) */
  uint64_t copy_bytes_timed;
  uint64_t lent_page_copies; /* page copies into slots lent from an operator's idle scratch */
  uint64_t ahead_page_copies; /* page copies of a block's FFN started during its attention sub-block */
} psi_stats;

/* A weight matrix W[rows, cols] in pinned host memory, already packed into
 * page-contiguous slices by psi_pack_matrix or psi_pack_tiles ([PSI] Fig. 1
 * "checkpoint slices"): for ROWS / COLS page p starts at byte offset
 * p * block * (split == ROWS ? cols : rows) * 2; for TILES page (o, q) starts
 * at (o * block * cols + e_o * q * block_cols) * 2 with e_o the rows of row
 * tile o.  The last page of a row or column may be narrower (ragged). */
typedef struct psi_matrix {
  const void* pages_host;   /* pinned, packed image of W (rows*cols bf16) */
  const uint16_t* bias_host;/* pinned [rows] bf16, or NULL for no bias */
  int rows;                 /* output features */
  int cols;                 /* input features */
  int split;                /* PSI_SPLIT_ROWS, PSI_SPLIT_COLS or PSI_SPLIT_TILES */
  int block;                /* rows (ROWS, TILES) or columns (COLS) per page */
  int resident;             /* 0: streamed through the arena pages.  1: the image and
                               bias are DEVICE pointers (weights already resident in
                               HBM); pages are consumed in place, nothing is copied and
                               no page slot is used (the resident-weight comparison) */
  int block_cols;           /* TILES: columns per page (a multiple of 8); ignored (0) for
                               ROWS and COLS */
} psi_matrix;

/* ------------------------------------------------------------ host utils */

/* Pack a row-major W[rows, cols] (any host memory) into the page image
 * layout of psi_matrix; dst must hold rows*cols bf16.  Host-only. */
psi_status psi_pack_matrix(const uint16_t* W, int rows, int cols, int split, int block,
                           void* dst);

/* Pack a row-major W[rows, cols] into the PSI_SPLIT_TILES page image of
 * block_rows x block_cols pages (row tiles in order, each row tile's column
 * blocks in order, each page row-major); dst (rows*cols bf16) must not
 * overlap W.  Host-only.  Errors: PSI_E_INVALID. */
psi_status psi_pack_tiles(const uint16_t* W, int rows, int cols, int block_rows, int block_cols, void* dst);

/* Number of pages and bytes of page p of a matrix.  Host-only. */
int psi_matrix_pages(const psi_matrix* m);
size_t psi_matrix_page_bytes(const psi_matrix* m, int p);

/* Compute the arena carve without allocating.  Fails with
 * PSI_E_ARENA_TOO_SMALL when the pages, bias slots and workspace exceed
 * arena_bytes.  Host-only. */
psi_status psi_arena_plan(const psi_arena_desc* d, psi_arena_layout* out);

/* Scratch and page feasibility of each operator for a given arena, without
 * allocating or enqueueing anything (host-only).  *scratch_needed receives
 * the scratch bytes the operator would use.  Errors: PSI_E_PAGE_TOO_SMALL
 * when a page slice exceeds P, PSI_E_SCRATCH_EXHAUSTED when the scratch
 * does not fit, PSI_E_INVALID for bad shapes. */
psi_status psi_linear_plan(const psi_arena_desc* d, int M, int K, const psi_matrix* W,
                           int acc_external, size_t* scratch_needed);
psi_status psi_ffn_plan(const psi_arena_desc* d, int M, int dmodel, const psi_matrix* U,
                        const psi_matrix* V, int token_chunks, int acc_external,
                        size_t* scratch_needed);
psi_status psi_attn_plan(const psi_arena_desc* d, int M, int Mc, int heads, int head_dim,
                         const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                         const psi_matrix* Wo, int acc_external, size_t* scratch_needed);

/* Thread-local message describing the last error. */
const char* psi_last_error(void);
/* Library version string. */
const char* psi_version(void);

/* ----------------------------------------------------------------- arena */

/* [PSI] sec. II-A, Fig. 1: one device allocation of arena_bytes carved into
 * n_pages page slots, two bias slots (the bounded metadata term eps of
 * eq. (1)), the workspace and scratch.  Creates two page-copy streams and
 * the per-slot events (a bias-copy stream follows on the first bias copy).  While an operator runs, the whole pages of scratch
 * above its own allocations serve as extra page slots for its requests
 * (psi_stats.lent_page_copies; not in a PSI_ARENA_SYNC_COPY arena).
 * *out is the caller's handle until psi_arena_destroy.
 * Errors: PSI_E_INVALID, PSI_E_ARENA_TOO_SMALL, PSI_E_HIP. */
psi_status psi_arena_create(const psi_arena_desc* d, psi_arena** out);

/* Synchronises the compute and copy streams and frees the one allocation. */
psi_status psi_arena_destroy(psi_arena* a);

/* Blocks the host until every enqueued page copy and operator completed. */
psi_status psi_arena_sync(psi_arena* a);

/* Copies the accounting counters (synchronises first if PSI_ARENA_PROFILE,
 * to read the event timers). */
psi_status psi_arena_stats(psi_arena* a, psi_stats* out);

/* Zeroes the counters and the scratch high-water mark. */
psi_status psi_arena_reset_stats(psi_arena* a);

/* Per-launch timing of a profiled arena (PSI_ARENA_PROFILE) on (on != 0,
 * the initial state) or off for the launches and traced page copies
 * enqueued from now on; timings already enqueued are kept.  The two events
 * around each launch cost the compute stream a few microseconds, so a
 * caller can time a sample of its launches (e.g. one invocation of many).
 * Errors: PSI_E_INVALID for a null arena or one without PSI_ARENA_PROFILE. */
psi_status psi_arena_set_timing(psi_arena* a, int on);

/* Device timeline of a profiled arena (PSI_ARENA_PROFILE), for overlap
 * analysis of the page lifecycle of [PSI] sec. II-D: every timed GEMM and
 * attention launch and every timed half-page copy, with its start relative
 * to a base event.
 *   psi_arena_trace_start synchronises the arena's streams, records the base
 *   event on the compute stream and starts keeping up to `capacity` events
 *   (older ones are not overwritten: later events are dropped once full);
 *   page copies are timed from then on, as with PSI_ARENA_PROFILE_COPIES.
 *   psi_arena_trace_read synchronises (to read the timers), copies up to
 *   `capacity` events into `out` (caller-owned host array) and stores the
 *   number recorded in *count.
 * Errors: PSI_E_INVALID without PSI_ARENA_PROFILE or for a null arena;
 * PSI_E_HIP if an event cannot be created or read. */
typedef struct psi_trace_event {
  int32_t kind;     /* 0 GEMM, 1 attention, 2 / 3 page copy on copy stream 0 / 1,
                       4 query/key normalisation-rotary kernel */
  int32_t reserved;
  double start_ms;  /* from the base event */
  double dur_ms;
  double work;      /* algorithmic FLOPs (kernels) or bytes (copies) */
} psi_trace_event;
psi_status psi_arena_trace_start(psi_arena* a, size_t capacity);
psi_status psi_arena_trace_read(psi_arena* a, psi_trace_event* out, size_t capacity, size_t* count);

/* Device address of the arena base (for footprint checks). */
psi_status psi_arena_device_base(psi_arena* a, void** base_out, size_t* bytes_out);

/* Stage probes ([PSI] sec. III-C and sec. IV-B compare stage tensors of a
 * block on identical inputs).  With a journal attached, every following
 * operator also commits its intermediate BF16 stage tensors under
 * key (step, block, branch = head group or hidden tile, role):
 *   PSI_ROLE_ATTN_O   attention output O_g of head group g, [M, group cols]
 *                     (Wo split by columns); with Wo split into output
 *                     tiles, every group's outputs at once, [M, d], under
 *                     branch -1
 *   PSI_ROLE_FFN_H    FFN hidden tile H_J (after GELU), [M, tile]; with
 *                     token_chunks > 1, chunk c's rows under branch
 *                     J * token_chunks + c
 * and the compute stream waits for each copy before the scratch holding
 * the tensor is reused (probes cost time; they are a diagnostic).  Pass
 * NULL to detach.  Errors: PSI_E_INVALID. */
#define PSI_ROLE_ATTN_O 16
#define PSI_ROLE_FFN_H 17
#define PSI_ROLE_FFN_HSTATE 18  /* hidden tiles journaled by PSI_FFN_REUSE */
#define PSI_ROLE_ATTN_OSTATE 19 /* head-group outputs journaled by psi_attn_tiled */
psi_status psi_arena_set_probe(psi_arena* a, psi_journal* j, int32_t step, int32_t block);

/* ------------------------------------------------------------ page API */

/* Slice request ([PSI] sec. II-D): take the first free page slot from the
 * round-robin position on (the next slot after the last one taken) and
 * enqueue an H2D copy of `bytes` from pinned host memory into it (free ->
 * filling).  The copy follows the slot's previous release event: if that
 * has not completed yet, the host waits for it before enqueueing (counted
 * in host_syncs), so the host never runs more than one round of slots
 * ahead of the consumers.
 * Errors: PSI_E_PAGE_TOO_SMALL (bytes > P), PSI_E_PAGE_BUSY (every slot
 * still has an unreleased request), PSI_E_NOT_PINNED, PSI_E_ALIGN. */
psi_status psi_page_submit(psi_arena* a, const void* host_pinned, size_t bytes, int* page_out);

/* Makes the compute stream wait for the page's copy (filling -> consuming)
 * and returns its device address, so caller kernels may consume it. */
psi_status psi_page_acquire(psi_arena* a, int page, void** dev_out);

/* Ends the request: records the release event after every use enqueued so
 * far on the compute stream; the next copy into this slot waits for it
 * ([PSI] sec. II-D).  Releasing a page that was never acquired acquires it
 * implicitly.  Errors: PSI_E_STATE for a free page. */
psi_status psi_page_release(psi_arena* a, int page);

/* ------------------------------------------------------------- operators */

/* Paged projection y = B(x W^T + b) ([PSI] sec. III-A numerics, sec. IV-B
 * output-column groups).
 *   x_dev [M, K] bf16 (16-byte aligned rows: K % 8 == 0)
 *   W: PSI_SPLIT_ROWS -> each page computes y[:, page columns] directly;
 *      PSI_SPLIT_COLS -> K-split, fp32 accumulator carried in page order in
 *      acc_dev (or arena scratch when acc_dev is NULL and it fits), bias
 *      added once after the last page.
 *   acc_dev nullable [M, N] fp32; y_dev [M, N] bf16 (N = W->rows).  y must
 *   not overlap x: every page launch reads x while earlier launches have
 *   written y (PSI_E_INVALID otherwise).
 *   flags: PSI_OP_BASELINE_BIAS, PSI_OP_RESIDUAL (y = B(x + ...), needs
 *   K == N), PSI_OP_STORE_ACC. */
psi_status psi_linear_paged(psi_arena* a, const uint16_t* x_dev, int M, int K,
                            const psi_matrix* W, float* acc_dev, uint16_t* y_dev,
                            unsigned flags);

/* For callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * projection of psi_linear_paged over RESIDENT weight pages (W->resident
 * = 1: image and bias are device pointers) with no arena.  The K-split's
 * fp32 accumulator lives in a library-owned static device array of
 * PSI_NOALLOC_SCRATCH_BYTES per device (held until the process ends); the
 * call allocates nothing and enqueues only GEMM launches on `stream`
 * (hipStream_t; NULL = null stream), in the page order of
 * psi_linear_paged, so its bits equal psi_linear_paged's on the same
 * resident matrix.
 *   x_dev [M, K] bf16, y_dev [M, N] bf16 (N = W->rows), y must not overlap x;
 *   W split by ROWS (no scratch used) or COLS (M * N * 4 bytes of scratch).
 *   flags: PSI_OP_BASELINE_BIAS, PSI_OP_RESIDUAL (needs K == N).
 * Every call on a device shares that device's array and finds the last
 * call's contents in it (the first K-split page never reads them): calls
 * that overlap on one device (two streams, two threads) race and must be
 * ordered by the caller.
 * Errors (before anything is enqueued): PSI_E_INVALID (not resident,
 * shapes, flags, y overlapping x), PSI_E_SCRATCH_EXHAUSTED (M * N * 4 >
 * PSI_NOALLOC_SCRATCH_BYTES for a K-split), PSI_E_ALIGN, PSI_E_HIP. */
#define PSI_NOALLOC_SCRATCH_BYTES (16u << 20)
psi_status psi_linear_resident_noalloc(const uint16_t* x_dev, int M, int K, const psi_matrix* W,
                                       uint16_t* y_dev, unsigned flags, void* stream);

/* Paged FFN F(X) = phi(X U^T + a) V^T + b ([PSI] sec. II-B eq. (2)) with the
 * declared BF16 writes of sec. III-A: pre-GELU B(acc + a), post-GELU
 * B(phi(.)), output B(ACC + b).
 *   U: [h, d] PSI_SPLIT_ROWS with block t_h (hidden tile J); bias a [h].
 *   V: [d, h] PSI_SPLIT_COLS with the same block t_h; bias b [d].
 *   token_chunks >= 1: x is cut into contiguous chunks of ceil(M/chunks)
 *   rows.  With one chunk every page is one launch over all tokens.  With
 *   several, U_J and V_J are held together (two page slots) while every
 *   chunk runs its up-projection into H_J and its carried down-projection,
 *   so each page is streamed once and serves all chunks (page reuse across
 *   token chunks); H_J [ceil(M/chunks), t_h] BF16 lives in arena scratch,
 *   so the scratch bound does not grow with M.  Rows are independent: the
 *   result is bitwise the same for every chunk count.
 *   The fp32 accumulator [M, d] lives in acc_dev or scratch.
 *   y_dev may be x_dev itself (with PSI_OP_RESIDUAL: y = B(x + F(x))) or
 *   must not overlap it.
 * Errors: PSI_E_INVALID (shapes, token_chunks < 1, several chunks in a
 * one-slot arena with streamed weights, y partly overlapping x),
 * PSI_E_SCRATCH_EXHAUSTED (one chunk's H_J, plus the accumulator without
 * acc_dev, exceeds the scratch), PSI_E_PAGE_TOO_SMALL, PSI_E_NOT_PINNED. */
psi_status psi_ffn_paged(psi_arena* a, const uint16_t* x_dev, int M, int d,
                         const psi_matrix* U, const psi_matrix* V, int token_chunks,
                         float* acc_dev, uint16_t* y_dev, unsigned flags);

/* FFN over output tiles of the down-projection ([PSI] sec. III-B "FFN
 * reuse"): V is split by rows into output tiles V_o = V[o t_o:(o+1) t_o, :]
 * (PSI_SPLIT_ROWS, block t_o; one page holds t_o x h), U as in
 * psi_ffn_paged (PSI_SPLIT_ROWS, block t_h).  Per output tile o:
 * ACC_o = sum over J ascending of H_J V_o[:, J]^T (fp32, carried across J),
 * y[:, o] = B(ACC_o + b_o) (+ residual), with H_J = B(phi(B(x U_J^T + a_J))).
 *   PSI_FFN_REUSE      each H_J is computed once for all tokens, committed to
 *                      the journal `j` under key (step, block, J,
 *                      PSI_ROLE_FFN_HSTATE) and reloaded for every output
 *                      tile (the paper's FFN reuse)
 *   PSI_FFN_RECOMPUTE  scheduling baseline: for every output tile each U_J
 *                      page is streamed again and H_J recomputed; `j` unused
 * Per output the accumulation is the one of psi_ffn_paged (same hidden
 * tiles in the same order), so both schedules give its bits.
 *   x_dev [M, d], y_dev [M, d].  y_dev may alias x_dev with PSI_FFN_REUSE
 *   (every read of x precedes the output tiles, and tile o reads and writes
 *   only its own columns), with PSI_FFN_RECOMPUTE only when t_o == d.
 *   Scratch: H_J [M, t_h] bf16 (two such buffers with PSI_FFN_REUSE, so
 *   that journal copies of one overlap the GEMMs on the other) and ACC_o
 *   [M, t_o] fp32.  flags: PSI_OP_BASELINE_BIAS, PSI_OP_RESIDUAL.  The
 *   journal store must hold h x M x 2 bytes more than it holds
 *   (PSI_FFN_REUSE).
 * Errors: PSI_E_INVALID (shapes, unknown schedule, missing journal, y
 * aliasing x under recomputation over more than one output tile),
 * PSI_E_SCRATCH_EXHAUSTED, PSI_E_PAGE_TOO_SMALL, PSI_E_JOURNAL_KEY /
 * PSI_E_JOURNAL_FULL. */
#define PSI_FFN_REUSE 1
#define PSI_FFN_RECOMPUTE 2
psi_status psi_ffn_tiled_plan(const psi_arena_desc* d, int M, int dmodel, const psi_matrix* U,
                              const psi_matrix* Vo, int schedule, size_t* scratch_needed);
psi_status psi_ffn_tiled(psi_arena* a, const uint16_t* x_dev, int M, int d, const psi_matrix* U,
                         const psi_matrix* Vo, int schedule, psi_journal* j, int32_t step,
                         int32_t block, uint16_t* y_dev, unsigned flags);

/* Paged attention sub-block ([PSI] sec. II-B eqs. (3)-(4)): per head group
 * g (heads_per_group = Wq->block / head_dim): Q_g = x Wq_g^T + bq_g,
 * K_g/V_g from ctx (cross-attention) or x (self), fp32 online-softmax
 * attention per head (unmasked, noncausal, dropout-free), then the
 * O-projection y = B(O Wo^T + bo) (+ residual), in one of two layouts of
 * Wo with the same summation per output (same bits):
 *   - Wo PSI_SPLIT_COLS with the head-group block: K-split over the groups,
 *     ACC += O_g Wo[:, g]^T in group order with the fp32 ACC carried in
 *     acc_dev (or scratch when it fits);
 *   - Wo PSI_SPLIT_ROWS (output tiles of any block): every group's O is kept
 *     in an [M, d] BF16 buffer and each tile y[:, o] is one GEMM over the
 *     full K.  No fp32 accumulator exists: acc_dev (M x d x 4 bytes,
 *     16-byte aligned) then serves as working memory, holding that buffer
 *     and, behind it, K_g and V_g^T when they fit (else scratch); without
 *     acc_dev the buffer takes scratch.  PSI_OP_STORE_ACC is refused.
 *   Wq, Wk, Wv: [d, d] PSI_SPLIT_ROWS, block = heads_per_group*head_dim.
 *   head_dim is 128 or 64.  ctx_dev nullable [Mc, d]; y_dev may alias x_dev.
 * Errors: PSI_E_INVALID (shapes, blocks, PSI_OP_STORE_ACC without acc_dev
 * or with output tiles), PSI_E_ALIGN (acc_dev holding the outputs not
 * 16-byte aligned), PSI_E_SCRATCH_EXHAUSTED, PSI_E_PAGE_TOO_SMALL,
 * PSI_E_NOT_PINNED. */
psi_status psi_attn_paged(psi_arena* a, const uint16_t* x_dev, int M,
                          const uint16_t* ctx_dev, int Mc, int heads, int head_dim,
                          const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                          const psi_matrix* Wo, float* acc_dev, uint16_t* y_dev,
                          unsigned flags);

/* Query/key normalisation and rotary positions of the attention sub-block
 * ([PSI] sec. II-B, full-row RMS and split RoPE), each a declared BF16 write:
 *   Q = B(x Wq^T + bq); if gamma_q: Q = B(gamma_q * Q / sqrt(s/d + eps)),
 *   s = sum over column tiles J (width norm_tile, ascending) of the tile's
 *   sum of squares, ONE denominator per row for all tiles; if cos_q:
 *   per head the pair (Q_j, Q_{j+dh/2}), j < dh/2, becomes
 *   B(c Q_j - s Q_{j+dh/2}), B(s Q_j + c Q_{j+dh/2}) with c = cos[t][j],
 *   s = sin[t][j] of the row's token t.  K likewise with gamma_k and the
 *   key tables (NULL cos_k: the query tables, which needs Mk == M).
 * Fields:
 *   gamma_q, gamma_k  BF16 [d] or NULL (no normalisation of that operand);
 *                     pinned host memory staged with the biases, or device
 *                     memory when the projection matrices are resident
 *   eps               > 0 when a gamma is given (fp32)
 *   norm_tile         width of the partial sums, a multiple of 8;
 *                     0 = the head-group block (one tile per weight page)
 *   cos_q, sin_q      device fp32 [M, head_dim/2], 16-byte aligned, or NULL
 *                     (no rotary embedding)
 *   cos_k, sin_k      device fp32 [Mk, head_dim/2] or NULL */
typedef struct psi_qk_norm_rope {
  const uint16_t* gamma_q;
  const uint16_t* gamma_k;
  float eps;
  int norm_tile;
  const float* cos_q;
  const float* sin_q;
  const float* cos_k;
  const float* sin_k;
} psi_qk_norm_rope;

/* psi_attn_paged with the normalisation/rotary stage above between the
 * Q/K projections and attention.  Because the row statistic spans every
 * head group, the Q and K projections of all groups are computed first
 * (pages Wq_g, Wk_g for g ascending), then normalised/rotated in place,
 * then per group V_g and attention (pages Wv_g), with the O-projection per
 * group (Wo[:, g], column split) or over output tiles after every group
 * (row split; the tiles read the Q buffer, which the attention overwrote
 * with O).  Scratch: Q [M, d] and K [Mk, d] BF16, V_g^T, and, for the
 * column split, ACC unless acc_dev.
 * nr == NULL (or nothing enabled in it) gives psi_attn_paged's bits.
 * Errors: as psi_attn_paged, plus PSI_E_INVALID for eps <= 0 with a gamma,
 * a bad norm_tile, a missing sin table, or NULL cos_k with Mk != M;
 * PSI_E_ALIGN for misaligned tables. */
psi_status psi_attn_ext_plan(const psi_arena_desc* d, int M, int Mc, int heads, int head_dim,
                             const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                             const psi_matrix* Wo, const psi_qk_norm_rope* nr, int acc_external,
                             size_t* scratch_needed);
psi_status psi_attn_paged_ext(psi_arena* a, const uint16_t* x_dev, int M,
                              const uint16_t* ctx_dev, int Mc, int heads, int head_dim,
                              const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                              const psi_matrix* Wo, const psi_qk_norm_rope* nr, float* acc_dev,
                              uint16_t* y_dev, unsigned flags);

/* Attention sub-block with the O-projection over output tiles and the
 * head-group outputs held in the journal instead of device memory ([PSI]
 * sec. III-B: intermediate state is retained on device or stored in the
 * host journal for later use).  Per head group g (pages Wq_g, Wk_g, Wv_g):
 * Q_g, K_g, V_g^T and attention as psi_attn_paged, then O_g [M, e_g] is
 * committed under key (step, block, g, PSI_ROLE_ATTN_OSTATE).  Then per
 * output tile o (Wo split by ROWS, block t_o; one page holds t_o x d):
 * ACC_o = sum over g ascending of O_g Wo[o rows, g cols]^T (fp32, carried),
 * y[:, o] = B(ACC_o + bo_o) (+ x[:, o]), with every O_g reloaded from the
 * journal (two device buffers: the reload of the next group overlaps the
 * GEMM of the current one).  Each output element sums over the same
 * channels in the same order as psi_attn_paged, so the result is its bits.
 * The device holds no [M, d] intermediate: scratch is two [M, gw] buffers
 * plus max(K_g and V_g^T, ACC_o [M, t_o] fp32).
 *   y_dev may alias x_dev.  flags as psi_attn_paged except PSI_OP_STORE_ACC.
 *   Journal traffic: M x d x 2 bytes D2H, (d / t_o) x M x d x 2 bytes H2D.
 * Errors: as psi_attn_paged, plus PSI_E_INVALID for a missing journal and
 * PSI_E_JOURNAL_KEY / PSI_E_JOURNAL_FULL. */
psi_status psi_attn_tiled_plan(const psi_arena_desc* d, int M, int Mc, int heads, int head_dim,
                               const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                               const psi_matrix* Wo, size_t* scratch_needed);
psi_status psi_attn_tiled(psi_arena* a, const uint16_t* x_dev, int M, const uint16_t* ctx_dev,
                          int Mc, int heads, int head_dim, const psi_matrix* Wq,
                          const psi_matrix* Wk, const psi_matrix* Wv, const psi_matrix* Wo,
                          psi_journal* j, int32_t step, int32_t block, uint16_t* y_dev,
                          unsigned flags);

/* One synthetic transformer block in place: x_tmp = x + Attn(x) (self),
 * then x = x_tmp + FFN(x_tmp), both with the residual write.  x_tmp_dev
 * NULL (or x_dev) runs both sub-blocks in place on x with the same bits, so
 * x is the only [M, d] BF16 live state; otherwise x_tmp must not overlap x.
 * w->Wo may be split by columns or by rows (psi_attn_paged's two
 * O-projection layouts); acc_dev serves both sub-blocks in turn;
 * token_chunks as psi_ffn_paged.  If `fence` is non-NULL, the first launch
 * that writes x first waits for every journal copy enqueued so far (the
 * journal's reads of x are previous consumers, [PSI] sec. II-D). */
typedef struct psi_block_weights {
  psi_matrix Wq, Wk, Wv, Wo; /* attention projections */
  psi_matrix U, V;           /* FFN */
} psi_block_weights;
psi_status psi_block_paged(psi_arena* a, uint16_t* x_dev, uint16_t* x_tmp_dev, int M,
                           int heads, int head_dim, const psi_block_weights* w,
                           int token_chunks, float* acc_dev, psi_journal* fence,
                           unsigned flags);

/* One synthetic block in place with only x as device state (low-live-state
 * mode): psi_journal_reset(j), then psi_attn_tiled (x -> x, residual) and
 * psi_ffn_tiled with PSI_FFN_REUSE (x -> x, residual); the head-group
 * outputs and hidden tiles live in the journal `j` (its store needs
 * M x (d + h) x 2 bytes; it is reused by every call).  w->Wo and w->V are
 * split by ROWS (output tiles).  Same bits as psi_block_paged.
 * flags: PSI_OP_BASELINE_BIAS, PSI_OP_BF16_SOFTMAX, PSI_OP_ATTN_P2. */
psi_status psi_block_lowlive(psi_arena* a, uint16_t* x_dev, int M, int heads, int head_dim,
                             const psi_block_weights* w, psi_journal* j, unsigned flags);

/* --------------------------------------------------------------- journal */

/* Indexed host journal of BF16 state ([PSI] sec. II-D, sec. III-B):
 * key = (step, block, branch, role).  Commit copies device bytes to the
 * host store on the journal's own stream after the producer's work; reload
 * copies them back after the consumer's previous work.  Byte-preserving.
 * Store modes:
 *   default           the store is pinned host memory; commits and reloads
 *                     are single DMA copies straight to/from the entry
 *   PSI_JOURNAL_RING  the store is pageable memory; bytes are staged
 *                     through a pinned ring of ring_slots x ring_slot_bytes
 *                     and moved by a host commit after each copy (the
 *                     paper's pinned-ring transport)
 *   PSI_JOURNAL_SYNC  transport control: copies on the caller's stream and
 *                     the host blocks until each one completes */
typedef struct psi_key {
  int32_t step;
  int32_t block;
  int32_t branch;
  int32_t role;
} psi_key;

typedef struct psi_journal_desc {
  size_t ring_slot_bytes; /* staging slot size (ring mode / sync mode), e.g. 8 MiB */
  int ring_slots;         /* >= 2 in ring mode */
  size_t store_bytes;     /* host store capacity, allocated and touched up front */
  unsigned flags;         /* PSI_JOURNAL_SYNC, PSI_JOURNAL_RING */
} psi_journal_desc;
#define PSI_JOURNAL_SYNC 0x1u
#define PSI_JOURNAL_RING 0x2u

psi_status psi_journal_create(const psi_journal_desc* d, psi_journal** out);
psi_status psi_journal_destroy(psi_journal* j);

/* Drop every entry and reuse the store from its start.  GPU-ordered: all
 * journal copies enqueued before the reset precede those enqueued after
 * it, so the host need not wait.  Counters are kept. */
psi_status psi_journal_reset(psi_journal* j);

/* Enqueue a byte copy of dev[0, bytes) into the store under key k, ordered
 * after all work enqueued so far on `producer`.  Errors: PSI_E_JOURNAL_KEY
 * for a duplicate key, PSI_E_JOURNAL_FULL. */
psi_status psi_journal_commit(psi_journal* j, psi_key k, const void* dev, size_t bytes,
                              void* producer_stream);

/* Enqueue the reload of key k into dev, ordered after all work enqueued so
 * far on `consumer`; `consumer` then waits for the reload.  Errors:
 * PSI_E_JOURNAL_KEY when the key is missing or sizes differ. */
psi_status psi_journal_reload(psi_journal* j, psi_key k, void* dev, size_t bytes,
                              void* consumer_stream);

/* Make `stream` wait until every commit enqueued so far has finished
 * reading its device buffer (device-buffer overwrites follow the journal's
 * copies). */
psi_status psi_journal_fence(psi_journal* j, void* stream);

/* Block the host until every enqueued commit and reload is complete. */
psi_status psi_journal_sync(psi_journal* j);

/* Copy a committed entry to host memory (synchronises first). */
psi_status psi_journal_read(psi_journal* j, psi_key k, void* host_dst, size_t bytes);

/* Bytes moved and entries held. */
psi_status psi_journal_counters(psi_journal* j, uint64_t* bytes_d2h, uint64_t* bytes_h2d,
                                uint64_t* entries);

#ifdef __cplusplus
}
#endif

#endif /* PSI_H */
