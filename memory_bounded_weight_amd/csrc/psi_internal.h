// psi_internal.h -- shared declarations of the paged-operator runtime.
//
// [PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint
// Audio-Video Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "psi.h"

namespace psi {

// ------------------------------------------------------------- errors
psi_status fail(psi_status code, const std::string& msg);
psi_status hip_fail(hipError_t e, const char* what);
#define PSI_HIP(call)                                     \
  do {                                                    \
    hipError_t e_ = (call);                               \
    if (e_ != hipSuccess) return ::psi::hip_fail(e_, #call); \
  } while (0)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
constexpr size_t kAlign = 256;
constexpr size_t kDefaultSide = 64 * 1024;

// ------------------------------------------------------------- kernels
// Events that the next kernel launch binds to its own start and end
// (hipExtLaunchKernelGGL), set by the arena around one launch: bound to the
// kernel they time the kernel alone, and they add no packet to the stream.
// `launched` is set once a kernel has taken them; a launch function that
// launches several kernels binds `start` to the first and `stop` to the last.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool launched = false;
};
LaunchEvents& launch_events();  // this host thread's

template <typename F, typename... Args>
hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  LaunchEvents& ev = launch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    ev.launched = true;
    ev.start = nullptr;
  }
  return e;
}

enum GemmEpilogue : int {
  EPI_ACC = 0,   // store fp32 accumulator only
  EPI_BIAS = 1,  // out = B(acc + bias)  [+ residual]
  EPI_GELU = 2,  // out = B(phi(f(B(acc + bias))))
};

// C[M,N] = A[M,K] * B[N,K]^T (both operands K-contiguous bf16), fp32
// accumulation on MFMA, optional carried initial accumulator and fused
// epilogue.  All pointers are device pointers; leading dimensions are in
// elements.
struct GemmArgs {
  const uint16_t* A;
  long lda;
  const uint16_t* B;
  long ldb;
  int M, N, K;
  const float* acc_in;  // nullable [M, ld_acc]: initial accumulator
  long ld_acc_in;
  float* acc_out;       // nullable: fp32 accumulator store
  long ld_acc_out;
  const uint16_t* bias; // nullable
  int bias_on_m;        // bias indexed by row (1) or column (0)
  uint16_t* out;        // nullable bf16 output
  long ldo;
  const uint16_t* resid;// nullable residual, indexed like out (may alias out)
  long ldr;
  int epi;
  int baseline_bias;
  int config;           // tile configuration; 0 = chosen from the shape
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
int gemm_auto_config(const GemmArgs& a);

struct AttnArgs {
  uint16_t* q;         // [Mq, ldq]; head h occupies columns h*dh..(h+1)*dh-1; O overwrites it
  long ldq;
  const uint16_t* k;   // [Mk, ldk]
  long ldk;
  const uint16_t* vt;  // [heads*dh, ldvt]: V transposed (row = channel, column = key)
  long ldvt;
  int Mq, Mk, heads;
  int dh;              // head dimension: 128 or 64
  float alpha;         // 1/sqrt(dh) rounded to fp32
  int p_terms;         // BF16 terms per softmax weight in P*V: 3 = fp32 weights,
                       // 2 = hi + lo (about 17 bits), 1 = BF16 numerator weights
  int config;          // 0: chosen from the shape; 1: 128-query, 2: 256-query, 3: 256-query
                       // pipelined (waves in lock step), 4: 256-query ping-pong
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// In place on rows of x: optional full-row RMS normalisation (gamma
// non-null; sum of squares as ascending partial sums over column tiles of
// width `tile`), then optional split RoPE per head (cs/sn non-null, fp32
// tables [M, dh/2]); each a BF16 write.  x, gamma, cs, sn 16-byte aligned,
// ldx % 8 == 0, d % 16 == 0, tile % 8 == 0.
struct NormRopeArgs {
  uint16_t* x;
  long ldx;
  int M, d, dh;
  const uint16_t* gamma;  // nullable, [d]
  float eps;
  int tile;
  const float* cs;        // nullable, [M, dh/2]
  const float* sn;
};
hipError_t launch_qk_norm_rope(const NormRopeArgs& a, hipStream_t s);

// One-wave kernel that waits the given time (bounded spin on the real-time
// counter); PSI_ARENA_JITTER transport control.
hipError_t launch_delay(uint32_t microseconds, hipStream_t s);

// ------------------------------------------------------------- planning
struct MatrixInfo {
  int pages;
  size_t max_page_bytes;
};
// expect_split: PSI_SPLIT_ROWS / PSI_SPLIT_COLS, -1 for either of the two,
// or kSplitOutputTiles for the output-tile schedules (ROWS or TILES).
// TILES is refused everywhere else.
constexpr int kSplitOutputTiles = -2;
psi_status check_matrix(const psi_matrix* m, const char* name, int expect_split);
// A device pointer that must be 16-byte aligned (and non-null unless
// allow_null): PSI_E_INVALID / PSI_E_ALIGN otherwise.
psi_status check_ptr(const void* p, const char* what, bool allow_null = false);
// Output and input ranges: disjoint, or (where the operator reads each
// element of x before writing the same element of y, and every other read
// of x comes earlier on the stream) exactly the same buffer.
psi_status check_alias(const void* x, size_t xbytes, const void* y, size_t ybytes, bool allow_same,
                       const char* op);
// True when the query/key normalisation-rotary stage does any work.
inline bool qk_stage_active(const psi_qk_norm_rope* nr) {
  return nr && (nr->gamma_q || nr->gamma_k || nr->cos_q || nr->sin_q || nr->cos_k || nr->sin_k);
}
MatrixInfo matrix_info(const psi_matrix* m);
// Rows of one FFN token chunk: ceil(M / chunks) (the last chunk may be
// shorter); chunks < 1 is treated as 1.
inline size_t ffn_chunk_rows(int M, int chunks) {
  if (M <= 0) return 0;
  if (chunks < 1) chunks = 1;
  return ((size_t)M + chunks - 1) / chunks;
}
const void* matrix_page_ptr(const psi_matrix* m, int p);
int matrix_page_extent(const psi_matrix* m, int p);  // rows (ROWS, TILES) or cols (COLS) in page p
int matrix_page_cols(const psi_matrix* m, int p);    // columns held by page p
int matrix_page_col0(const psi_matrix* m, int p);    // first column of W in page p
int matrix_page_row0(const psi_matrix* m, int p);    // first row of W in page p

// One weight-page request of an operator, in consumption order.
struct PageReq {
  const void* host;  // device address when `resident`
  size_t bytes;
  bool resident;
};

}  // namespace psi

// ------------------------------------------------------------- arena
struct psi_page_slot {
  enum State { FREE = 0, FILLING = 1, CONSUMING = 2 };
  State state = FREE;
  hipEvent_t ready = nullptr;    // recorded on the copy stream after the copy
  hipEvent_t release = nullptr;  // recorded on the compute stream after the last consumer
  // The event that marks the last release: `release`, or the end event bound
  // to the consuming kernel's launch (entry `rel_ring` of the arena's ring
  // while that entry still carries launch number `rel_seq`; a profiling
  // event when `rel_ring` is -1, dropped once harvested); nullptr once known
  // to be complete.
  hipEvent_t rel_ev = nullptr;
  int rel_ring = -1;
  uint64_t rel_seq = 0;
  uint64_t acq_launch = 0;  // kernel launches before the slot's consumers were ordered after its copy
  bool released_once = false;
  void* dev = nullptr;
};

struct psi_timed {
  hipEvent_t start, stop;
  int kind;      // 0 gemm, 1 attention, 2 copy on stream 0, 3 copy on stream 1, 4 norm/rope
  double work;   // flops (kernels) or bytes (copies)
};

struct psi_arena {
  psi_arena_desc desc{};
  psi_arena_layout layout{};
  bool dry = false;
  char* base = nullptr;
  hipStream_t compute = nullptr;
  hipStream_t copy = nullptr;   // even page copies and bias copies
  hipStream_t copy1 = nullptr;  // odd page copies (a second DMA engine)
  hipStream_t copyb = nullptr;  // bias copies: small, never queued behind page copies (created on first use)
  int next_copy = 0;            // copy stream of the next page
  psi_page_slot slots[PSI_MAX_PAGES];
  int next_slot = 0;
  // The slot freed by the consumer the host enqueued last.  While that
  // consumer may still run, page fills that are not needed yet go elsewhere:
  // filling it would make the host wait for the kernel it has just
  // enqueued, and the compute stream would run dry until the next launch.
  int hold_slot = -1;
  // the running operator's page feeder, called after a launch that ends a hold
  psi_status (*refill)(void*) = nullptr;
  void* refill_ctx = nullptr;
  // Page slots lent by the running operator from the whole pages of scratch
  // above its own allocations (indices n_pages .. n_pages + n_lent - 1).
  // A lent slot is filled only when no host wait is needed: on first use
  // once `scratch_free` (the compute stream before the operator) has
  // completed, later once its own release has.
  static constexpr int kMaxLent = 4;
  psi_page_slot lent[kMaxLent];
  bool lent_fresh[kMaxLent] = {};
  int n_lent = 0;
  hipEvent_t scratch_free = nullptr;
  psi_page_slot bias_slots[2];  // same lifecycle as pages, one per operator, alternating
  int next_bias = 0;
  // scratch stack (offsets relative to layout.scratch_off)
  size_t scratch_top = 0;
  psi_stats stats{};
  // stage probes
  psi_journal* probe = nullptr;
  int32_t probe_step = 0, probe_block = 0;
  // profiling
  std::vector<psi_timed> pending;
  std::vector<hipEvent_t> event_pool;
  double copy_ms_stream[2] = {0.0, 0.0};
  // device timeline (psi_arena_trace_start / _read)
  hipEvent_t trace_base = nullptr;
  size_t trace_cap = 0;
  std::vector<psi_trace_event> trace;
  // double-buffered journal transport inside operators (commit-read and
  // reload-done events of two buffers)
  hipEvent_t pipe_ev[4] = {nullptr, nullptr, nullptr, nullptr};
  uint32_t jitter_state = 0x9E3779B9u;  // PSI_ARENA_JITTER sequence
  bool timing_off = false;               // psi_arena_set_timing(a, 0)
  int device = 0;
  // End events bound to the kernels the arena launches (launch_kernel).  A
  // release made by an operator right after its consuming kernel borrows
  // that kernel's end event instead of recording one more event on the
  // compute stream: each recorded event delays the next kernel by a few
  // microseconds (measured on MI355X), one bound to a launch does not.  An
  // entry is bound again only after its previous kernel has ended.
  static constexpr int kStopRing = 32;
  hipEvent_t stop_ring[kStopRing] = {};
  uint64_t stop_seq[kStopRing] = {};  // launch number an entry is bound to (0: never)
  int stop_next = 0;
  uint64_t launches = 0;              // kernels launched through the arena
  hipEvent_t last_stop = nullptr;     // end event of the last launch, if it has one
  int last_stop_ring = -1;            // its ring entry, or -1 for a profiling event
  // Page requests of the operator that runs next, set by a block driver for
  // the operator before it.  Once that operator's feeder has submitted all
  // of its own requests, page slots it frees (never lent ones: those are its
  // scratch) take these in order, so the copy engines keep working through
  // the end of a compute-bound operator; the next operator's feeder adopts
  // the submitted ones (`ahead_slot`, -1 for a resident page).
  std::vector<psi::PageReq> ahead;
  std::vector<int> ahead_slot;
  bool ahead_producing = false;  // the running operator's feeder still submits them
};

namespace psi {
// Scratch bump allocation inside the arena; nullptr in a dry run.
void* scratch_alloc(psi_arena* a, size_t bytes, psi_status* st);
void scratch_reset(psi_arena* a, size_t mark);

// Page request (slice copy into a lent slot that is ready, else into the
// next round-robin page slot).
int first_free_slot(const psi_arena* a, int skip = -1);  // -1 when every slot is taken
// Lends the whole pages of scratch above scratch_top as page slots to the
// running operator (none in a sync-copy arena); returns how many.  The
// operator must not allocate scratch afterwards, and returns them with
// return_lent_slots once every request is released.
int lend_scratch_slots(psi_arena* a);
psi_status return_lent_slots(psi_arena* a);
// The slot the next page_submit_ex would fill (-1: none free), and the
// device address of slot s (regular or lent).
// `regular_only`: never a lent slot.
int submit_slot(psi_arena* a, bool avoid_hold = false, bool regular_only = false);
void* slot_dev(psi_arena* a, int s);
psi_status page_submit_ex(psi_arena* a, const void* host, size_t bytes, int* page_out,
                          bool check_pinned, bool avoid_hold = false, bool regular_only = false);
psi_status page_acquire(psi_arena* a, int page);
// `borrow`: the caller releases right after launching the slot's last
// consumer (an operator's own sequence, nothing of the caller's between), so
// the release may take that kernel's end event (see psi_arena::stop_ring).
psi_status page_release(psi_arena* a, int page, bool borrow = false);

// An operator's biases: one request into the next bias slot (several
// pinned host arrays, each placed 256-byte aligned); *dev_out[i] receives
// the device address of part i.  slot_out is -1 when nothing was copied.
struct BiasPart {
  const void* host;
  size_t bytes;
};
psi_status bias_submit(psi_arena* a, const BiasPart* parts, int n, const uint16_t** dev_out,
                       int* slot_out);
psi_status bias_acquire(psi_arena* a, int slot);
psi_status bias_release(psi_arena* a, int slot, bool borrow = false);

// Kernel launch through the arena (profiling, counters).
psi_status run_gemm(psi_arena* a, const GemmArgs& g);
psi_status run_attention(psi_arena* a, const AttnArgs& g);
psi_status run_norm_rope(psi_arena* a, const NormRopeArgs& g);

psi_status check_pinned(const void* p, const char* what);

// PSI_ARENA_JITTER: enqueue a delay of 0-63 us (deterministic sequence) on s.
psi_status jitter(psi_arena* a, hipStream_t s);

// Stage probe: journal a device tensor of the current operator (no-op when
// no probe journal is attached) and make the compute stream wait for the
// copy before the buffer is reused.
psi_status probe_commit(psi_arena* a, int32_t branch, int32_t role, const void* dev, size_t bytes);

// Journal transport with caller events, so that an operator can keep two
// buffers in flight: a commit records `read_ev` once the device bytes have
// been read (the buffer may then be overwritten); a reload records `done`
// once the bytes are in place and does NOT make the consumer wait (the
// caller waits on `done` right before the reading kernel).  Null events
// give psi_journal_commit / psi_journal_reload.
psi_status journal_commit_ev(psi_journal* j, psi_key k, const void* dev, size_t bytes, hipStream_t prod,
                             hipEvent_t read_ev);
psi_status journal_reload_ev(psi_journal* j, psi_key k, void* dev, size_t bytes, hipStream_t cons,
                             hipEvent_t done);
}  // namespace psi
