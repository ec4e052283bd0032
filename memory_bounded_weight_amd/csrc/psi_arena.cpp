// psi_arena.cpp -- the fixed device arena and the weight-page lifecycle.
//
// [PSI] sec. II-A and Fig. 1 ("Precision-Preserving Subtensor Inference for
// a 22B Joint Audio-Video Generator under a Fixed GPU Working Set", arXiv
// 2611.08023): all managed device memory is ONE allocation carved into
// reusable pages, a workspace and scratch.  [PSI] sec. II-D: a page has at
// most one outstanding slice request; its lifecycle is free -> filling ->
// ready -> consuming; copy completion permits consumption and completion of
// the last consumer permits the next write.  Here the copy runs on one of
// two library streams and records `ready`; consumers on the compute stream
// wait on `ready`; release records `release` on the compute stream after
// every enqueued use, and the next copy into the slot is enqueued once the
// host has seen `release` complete (a host wait when it has not: see
// wait_release).  An operator's own release right after the consuming
// kernel takes that kernel's end event instead of recording one (see
// psi_arena::stop_ring).  Inside an operator, whole pages of idle scratch
// serve as extra (lent) slots, filled only when that needs no wait.
#include <cstring>

#include "psi_internal.h"

namespace psi {

LaunchEvents& launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}

psi_status probe_commit(psi_arena* a, int32_t branch, int32_t role, const void* dev, size_t bytes) {
  if (!a->probe || a->dry) return PSI_OK;
  psi_key k{a->probe_step, a->probe_block, branch, role};
  psi_status st = psi_journal_commit(a->probe, k, dev, bytes, a->compute);
  if (st) return st;
  return psi_journal_fence(a->probe, a->compute);
}

psi_status jitter(psi_arena* a, hipStream_t s) {
  if (a->dry || !(a->desc.flags & PSI_ARENA_JITTER)) return PSI_OK;
  uint32_t x = a->jitter_state;  // xorshift32
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  a->jitter_state = x;
  PSI_HIP(launch_delay(x % 64u, s));
  return PSI_OK;
}

psi_status check_pinned(const void* p, const char* what) {
  if (!p) return PSI_OK;
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of an unknown pointer
    return fail(PSI_E_NOT_PINNED, std::string(what) + " is not pinned host memory");
  }
  if (attr.type != hipMemoryTypeHost)
    return fail(PSI_E_NOT_PINNED, std::string(what) + " is not pinned host memory (type " +
                                      std::to_string((int)attr.type) + ")");
  return PSI_OK;
}

void* scratch_alloc(psi_arena* a, size_t bytes, psi_status* st) {
  size_t off = a->scratch_top;
  size_t end = off + align_up(bytes, kAlign);
  if (end > a->layout.scratch_bytes) {
    *st = fail(PSI_E_SCRATCH_EXHAUSTED, "scratch exhausted: need " + std::to_string(end) +
                                            " B of " + std::to_string(a->layout.scratch_bytes));
    return nullptr;
  }
  *st = PSI_OK;
  a->scratch_top = end;
  if (end > a->stats.scratch_high_water) a->stats.scratch_high_water = end;
  if (a->dry) return nullptr;
  return a->base + a->layout.scratch_off + off;
}

void scratch_reset(psi_arena* a, size_t mark) { a->scratch_top = mark; }

static hipEvent_t pool_event(psi_arena* a) {
  if (!a->event_pool.empty()) {
    hipEvent_t e = a->event_pool.back();
    a->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Before a copy into a slot, the host waits until the slot's previous
// consumers have finished (the release event).  Ordering the copy after them
// on the GPU instead (a copy-stream wait on the compute stream's event) lets
// the host run ahead, and the runtime then blocks an H2D enqueue for
// milliseconds at a time while the DMA engines idle (measured: 22 vs 43 GB/s
// for 8 MiB pages in a slot/event pipeline).  With the wait on the host the
// host stays at most one slot round ahead of the consumers, which keeps the
// compute stream fed.
static hipEvent_t release_event(const psi_arena* a, const psi_page_slot& slot) {
  // a ring entry bound again has seen its earlier kernel end
  if (slot.rel_ring >= 0 && a->stop_seq[slot.rel_ring] != slot.rel_seq) return nullptr;
  return slot.rel_ev;
}

static psi_status wait_release(psi_arena* a, psi_page_slot& slot) {
  hipEvent_t ev = release_event(a, slot);
  if (!ev) return PSI_OK;
  hipError_t q = hipEventQuery(ev);
  if (q == hipSuccess) return PSI_OK;
  if (q != hipErrorNotReady) return hip_fail(q, "hipEventQuery(release)");
  PSI_HIP(hipEventSynchronize(ev));
  a->stats.host_syncs++;
  return PSI_OK;
}

int first_free_slot(const psi_arena* a, int skip) {
  for (int i = 0; i < a->desc.n_pages; ++i) {
    const int c = (a->next_slot + i) % a->desc.n_pages;
    if (c != skip && a->slots[c].state == psi_page_slot::FREE) return c;
  }
  return -1;
}

static psi_page_slot* slot_ptr(psi_arena* a, int s) {
  if (s >= 0 && s < a->desc.n_pages) return &a->slots[s];
  if (s >= a->desc.n_pages && s < a->desc.n_pages + a->n_lent) return &a->lent[s - a->desc.n_pages];
  return nullptr;
}

static bool event_done(hipEvent_t e) {
  if (!e) return true;
  const hipError_t q = hipEventQuery(e);
  if (q == hipSuccess) return true;
  if (q != hipErrorNotReady) (void)hipGetLastError();  // not ready for this purpose; the waits report it
  return false;
}

static bool release_done(const psi_arena* a, const psi_page_slot& slot) {
  return !slot.released_once || event_done(release_event(a, slot));
}

// Marks the slot's release after every use enqueued so far: with `borrow`,
// and a kernel launched after the slot's consumers were ordered, the end
// event of the last launch (which follows them in stream order); else an
// event recorded on the compute stream now.
static psi_status mark_release(psi_arena* a, psi_page_slot& slot, bool borrow) {
  if (a->dry) return PSI_OK;
  if (borrow && a->last_stop && a->launches > slot.acq_launch) {
    slot.rel_ev = a->last_stop;
    slot.rel_ring = a->last_stop_ring;
    slot.rel_seq = a->launches;
    return PSI_OK;
  }
  PSI_HIP(hipEventRecord(slot.release, a->compute));
  slot.rel_ev = slot.release;
  slot.rel_ring = -1;
  return PSI_OK;
}

// A lent slot that can be filled without a host wait, or -1.
static int ready_lent_slot(psi_arena* a) {
  for (int i = 0; i < a->n_lent; ++i) {
    const psi_page_slot& l = a->lent[i];
    if (l.state != psi_page_slot::FREE) continue;
    if (a->dry) return a->desc.n_pages + i;
    if (a->lent_fresh[i] ? event_done(a->scratch_free) : release_done(a, l))
      return a->desc.n_pages + i;
  }
  return -1;
}

// A free lent slot whose fill needs a host wait, or -1.
static int free_lent_slot(const psi_arena* a, int skip) {
  for (int i = 0; i < a->n_lent; ++i)
    if (a->desc.n_pages + i != skip && a->lent[i].state == psi_page_slot::FREE) return a->desc.n_pages + i;
  return -1;
}

// The held slot while its consumer may still run, else -1 (dry runs keep
// the plain order).
static int pending_hold(psi_arena* a) {
  const int h = a->hold_slot;
  if (h < 0 || a->dry) return -1;
  psi_page_slot* p = slot_ptr(a, h);
  if (!p || p->state != psi_page_slot::FREE || !p->released_once) return -1;
  return release_done(a, *p) ? -1 : h;
}

int submit_slot(psi_arena* a, bool avoid_hold, bool regular_only) {
  const int skip = avoid_hold ? pending_hold(a) : -1;
  if (regular_only) return first_free_slot(a, skip);
  int s = ready_lent_slot(a);
  if (s < 0) s = first_free_slot(a, skip);
  if (s < 0) s = free_lent_slot(a, skip);
  return s;
}

void* slot_dev(psi_arena* a, int s) {
  psi_page_slot* p = slot_ptr(a, s);
  return p ? p->dev : nullptr;
}

int lend_scratch_slots(psi_arena* a) {
  if (a->desc.flags & PSI_ARENA_SYNC_COPY) return 0;
  const size_t start = align_up(a->scratch_top, kAlign);
  const size_t stride = align_up(a->desc.page_bytes, kAlign);
  if (stride == 0 || start >= a->layout.scratch_bytes) return 0;
  size_t n = (a->layout.scratch_bytes - start) / stride;
  if (n > (size_t)psi_arena::kMaxLent) n = psi_arena::kMaxLent;
  for (size_t i = 0; i < n; ++i) {
    psi_page_slot& l = a->lent[i];
    l.state = psi_page_slot::FREE;
    l.released_once = false;
    l.dev = a->dry ? nullptr : a->base + a->layout.scratch_off + start + i * stride;
    a->lent_fresh[i] = true;
  }
  if (a->hold_slot >= a->desc.n_pages) a->hold_slot = -1;
  a->n_lent = (int)n;
  if (n) {
    // the scratch's earlier users (previous operators) precede any copy into
    // it; the scratch high-water mark stays the operators' own allocations
    if (!a->dry && hipEventRecord(a->scratch_free, a->compute) != hipSuccess) {
      a->n_lent = 0;
      return 0;
    }
  }
  return (int)n;
}

psi_status return_lent_slots(psi_arena* a) {
  bool busy = false;
  for (int i = 0; i < a->n_lent; ++i) busy |= a->lent[i].state != psi_page_slot::FREE;
  if (a->hold_slot >= a->desc.n_pages) a->hold_slot = -1;
  a->n_lent = 0;
  if (busy) return fail(PSI_E_STATE, "a lent page slot is still in use at the end of the operator");
  return PSI_OK;
}

psi_status page_submit_ex(psi_arena* a, const void* host, size_t bytes, int* page_out,
                          bool pinned_check, bool avoid_hold, bool regular_only) {
  if (!host || bytes == 0) return fail(PSI_E_INVALID, "page submit: empty slice");
  if (bytes > a->desc.page_bytes)
    return fail(PSI_E_PAGE_TOO_SMALL, "weight tile exceeds page: " + std::to_string(bytes) +
                                          " B > " + std::to_string(a->desc.page_bytes) + " B");
  // a lent slot that needs no wait, else the first free slot from the
  // round-robin position on (a page held across many requests does not
  // stall the others)
  // (a lent slot that is not ready comes last and then takes a host wait)
  const int s = submit_slot(a, avoid_hold, regular_only);
  if (s < 0) return fail(PSI_E_PAGE_BUSY, "every page slot still has an unreleased request");
  const bool lent = s >= a->desc.n_pages;
  psi_page_slot& slot = *slot_ptr(a, s);
  if (!a->dry && pinned_check) {
    psi_status st = check_pinned(host, "page slice");
    if (st) return st;
  }
  if (!a->dry) {
    const bool sync = a->desc.flags & PSI_ARENA_SYNC_COPY;
    if (sync) {
      psi_status st = jitter(a, a->compute);
      if (st) return st;
      PSI_HIP(hipMemcpyAsync(slot.dev, host, bytes, hipMemcpyHostToDevice, a->compute));
      PSI_HIP(hipEventRecord(slot.ready, a->compute));
    } else {
      // Whole pages, alternating between the two copy streams (two DMA
      // engines): while one engine pays the start-up of its next copy, the
      // other one is streaming, so back-to-back 8 MiB pages keep the host
      // link near its bulk rate.
      const int ci = a->next_copy;
      hipStream_t cs = ci ? a->copy1 : a->copy;
      a->next_copy = ci ^ 1;
      if (lent) {
        const int li = s - a->desc.n_pages;
        if (a->lent_fresh[li]) {
          if (!event_done(a->scratch_free)) {
            PSI_HIP(hipEventSynchronize(a->scratch_free));
            a->stats.host_syncs++;
          }
        } else if (slot.released_once) {
          psi_status st = wait_release(a, slot);
          if (st) return st;
        }
      } else if (slot.released_once) {
        psi_status st = wait_release(a, slot);
        if (st) return st;
      }
      if (psi_status st = jitter(a, cs)) return st;
      hipEvent_t t0 = nullptr, t1 = nullptr;
      if ((a->desc.flags & PSI_ARENA_PROFILE) && !a->timing_off &&
          ((a->desc.flags & PSI_ARENA_PROFILE_COPIES) || a->trace_base)) {
        t0 = pool_event(a);
        t1 = pool_event(a);
        if (!t0 || !t1) return fail(PSI_E_HIP, "event pool");
        PSI_HIP(hipEventRecord(t0, cs));
      }
      PSI_HIP(hipMemcpyAsync(slot.dev, host, bytes, hipMemcpyHostToDevice, cs));
      if (t0) {
        PSI_HIP(hipEventRecord(t1, cs));
        a->pending.push_back({t0, t1, 2 + ci, (double)bytes});
      }
      PSI_HIP(hipEventRecord(slot.ready, cs));
    }
  }
  slot.state = psi_page_slot::FILLING;
  a->stats.bytes_h2d += bytes;
  a->stats.page_copies++;
  if (lent) {
    a->lent_fresh[s - a->desc.n_pages] = false;
    a->stats.lent_page_copies++;
  } else {
    a->next_slot = (s + 1) % a->desc.n_pages;
  }
  if (page_out) *page_out = s;
  return PSI_OK;
}

psi_status bias_submit(psi_arena* a, const BiasPart* parts, int n, const uint16_t** dev_out,
                       int* slot_out) {
  *slot_out = -1;
  size_t total = 0;
  for (int i = 0; i < n; ++i)
    if (parts[i].host && parts[i].bytes) total += align_up(parts[i].bytes, kAlign);
  for (int i = 0; i < n; ++i) dev_out[i] = nullptr;
  if (total == 0) return PSI_OK;
  if (total > a->layout.bias_slot_bytes)
    return fail(PSI_E_PAGE_TOO_SMALL, "the operator's biases exceed a bias slot");
  const int s = a->next_bias;
  psi_page_slot& slot = a->bias_slots[s];
  if (slot.state != psi_page_slot::FREE)
    return fail(PSI_E_STATE, "bias slot " + std::to_string(s) + " still in use");
  const bool sync = a->desc.flags & PSI_ARENA_SYNC_COPY;
  // Created on the first bias copy rather than with the arena: HIP assigns
  // a process's streams to its hardware queues in creation order, and a
  // stream created with the arena moved the journal's streams (created
  // after it) onto other queues, which slowed the low-live blocks by 13%
  // (measured on MI355X).
  if (!a->dry && !sync && !a->copyb) PSI_HIP(hipStreamCreateWithFlags(&a->copyb, hipStreamNonBlocking));
  hipStream_t cs = sync ? a->compute : a->copyb;
  if (!a->dry && !sync && slot.released_once) {
    psi_status st = wait_release(a, slot);
    if (st) return st;
  }
  if (psi_status st = jitter(a, cs)) return st;
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    if (!parts[i].host || !parts[i].bytes) continue;
    char* dst = a->dry ? nullptr : static_cast<char*>(slot.dev) + off;
    if (!a->dry) PSI_HIP(hipMemcpyAsync(dst, parts[i].host, parts[i].bytes, hipMemcpyHostToDevice, cs));
    dev_out[i] = reinterpret_cast<const uint16_t*>(dst);
    off += align_up(parts[i].bytes, kAlign);
    a->stats.bytes_h2d += parts[i].bytes;
  }
  if (!a->dry) PSI_HIP(hipEventRecord(slot.ready, cs));
  slot.state = psi_page_slot::FILLING;
  a->next_bias = (s + 1) % 2;
  *slot_out = s;
  return PSI_OK;
}

psi_status bias_acquire(psi_arena* a, int s) {
  if (s < 0) return PSI_OK;
  psi_page_slot& slot = a->bias_slots[s];
  if (slot.state == psi_page_slot::FILLING) {
    if (!a->dry && !(a->desc.flags & PSI_ARENA_SYNC_COPY)) {
      PSI_HIP(hipStreamWaitEvent(a->compute, slot.ready, 0));
      a->stats.event_waits++;
    }
    slot.state = psi_page_slot::CONSUMING;
    slot.acq_launch = a->launches;
  }
  return PSI_OK;
}

psi_status bias_release(psi_arena* a, int s, bool borrow) {
  if (s < 0) return PSI_OK;
  psi_page_slot& slot = a->bias_slots[s];
  if (slot.state == psi_page_slot::FREE) return PSI_OK;
  if (slot.state == psi_page_slot::FILLING) {
    psi_status st = bias_acquire(a, s);
    if (st) return st;
  }
  if (psi_status st = mark_release(a, slot, borrow)) return st;
  slot.released_once = true;
  slot.state = psi_page_slot::FREE;
  return PSI_OK;
}

psi_status page_acquire(psi_arena* a, int page) {
  psi_page_slot* sp = slot_ptr(a, page);
  if (!sp) return fail(PSI_E_INVALID, "bad page index");
  psi_page_slot& slot = *sp;
  if (slot.state == psi_page_slot::FREE)
    return fail(PSI_E_STATE, "page " + std::to_string(page) + " has no outstanding request");
  if (slot.state == psi_page_slot::CONSUMING) return PSI_OK;
  if (!a->dry && !(a->desc.flags & PSI_ARENA_SYNC_COPY)) {
    PSI_HIP(hipStreamWaitEvent(a->compute, slot.ready, 0));
    a->stats.event_waits++;
  }
  slot.state = psi_page_slot::CONSUMING;
  slot.acq_launch = a->launches;
  return PSI_OK;
}

psi_status page_release(psi_arena* a, int page, bool borrow) {
  psi_page_slot* sp = slot_ptr(a, page);
  if (!sp) return fail(PSI_E_INVALID, "bad page index");
  psi_page_slot& slot = *sp;
  if (slot.state == psi_page_slot::FREE)
    return fail(PSI_E_STATE, "page " + std::to_string(page) + " released while free");
  if (slot.state == psi_page_slot::FILLING) {
    psi_status st = page_acquire(a, page);
    if (st) return st;
  }
  if (psi_status st = mark_release(a, slot, borrow)) return st;
  slot.released_once = true;
  slot.state = psi_page_slot::FREE;
  return PSI_OK;
}

static psi_status timed_launch(psi_arena* a, int kind, double work, hipError_t (*fn)(const void*, hipStream_t),
                               const void* args) {
  a->stats.kernel_launches++;
  if (a->dry) return PSI_OK;
  if (psi_status st = jitter(a, a->compute)) return st;  // delays the consumer, not the copies
  a->last_stop = nullptr;
  LaunchEvents& ev = launch_events();
  ev = LaunchEvents{};
  hipEvent_t t0 = nullptr, t1 = nullptr;
  int ring = -1;
  if ((a->desc.flags & PSI_ARENA_PROFILE) && !a->timing_off) {
    // bound to the kernel: its own start and end, as a kernel trace has them
    t0 = pool_event(a);
    t1 = pool_event(a);
    if (!t0 || !t1) return fail(PSI_E_HIP, "event pool");
    ev.start = t0;
    ev.stop = t1;
  } else {
    const int j = a->stop_next;
    if (a->stop_seq[j] == 0 || event_done(a->stop_ring[j])) {
      ring = j;
      ev.stop = a->stop_ring[j];
    }
  }
  const hipError_t e = fn(args, a->compute);
  const bool launched = ev.launched;
  ev = LaunchEvents{};
  if (e != hipSuccess)
    return hip_fail(e, kind == 0 ? "gemm launch" : kind == 1 ? "attention launch" : "norm/rope launch");
  if (launched) {
    a->launches++;
    if (ring >= 0) {
      a->stop_seq[ring] = a->launches;
      a->stop_next = (ring + 1) % psi_arena::kStopRing;
      a->last_stop = a->stop_ring[ring];
      a->last_stop_ring = ring;
    } else if (t1) {
      a->last_stop = t1;
      a->last_stop_ring = -1;
    }
  }
  if (t0) {
    if (!launched) {  // nothing to bind (an empty launch): time the empty interval
      PSI_HIP(hipEventRecord(t0, a->compute));
      PSI_HIP(hipEventRecord(t1, a->compute));
    }
    a->pending.push_back({t0, t1, kind, work});
  }
  // A consumer enqueued after the held slot's one: fills of that slot no
  // longer leave the compute stream empty.
  if (a->hold_slot >= 0) {
    a->hold_slot = -1;
    if (a->refill) return a->refill(a->refill_ctx);
  }
  return PSI_OK;
}

static hipError_t gemm_thunk(const void* p, hipStream_t s) {
  return launch_gemm(*static_cast<const GemmArgs*>(p), s);
}
static hipError_t attn_thunk(const void* p, hipStream_t s) {
  return launch_attention(*static_cast<const AttnArgs*>(p), s);
}

psi_status run_gemm(psi_arena* a, const GemmArgs& g) {
  double flops = 2.0 * g.M * (double)g.N * g.K;
  return timed_launch(a, 0, flops, gemm_thunk, &g);
}

psi_status run_attention(psi_arena* a, const AttnArgs& g) {
  double flops = 4.0 * g.Mq * (double)g.Mk * g.dh * g.heads;
  return timed_launch(a, 1, flops, attn_thunk, &g);
}

static hipError_t norm_thunk(const void* p, hipStream_t s) {
  return launch_qk_norm_rope(*static_cast<const NormRopeArgs*>(p), s);
}

psi_status run_norm_rope(psi_arena* a, const NormRopeArgs& g) {
  if (g.M <= 0) return PSI_OK;
  double bytes = 4.0 * g.M * (double)g.d;  // one read and one write of each BF16 row
  return timed_launch(a, 4, bytes, norm_thunk, &g);
}

static psi_status harvest(psi_arena* a) {
  if (a->dry) return PSI_OK;
  PSI_HIP(hipStreamSynchronize(a->copy));
  PSI_HIP(hipStreamSynchronize(a->copy1));
  if (a->copyb) PSI_HIP(hipStreamSynchronize(a->copyb));
  PSI_HIP(hipStreamSynchronize(a->compute));
  a->stats.host_syncs += 4;
  // every release is complete now; profiling events go back to the pool
  auto drop = [](psi_page_slot& sl) {
    if (sl.rel_ring < 0 && sl.rel_ev != sl.release) sl.rel_ev = nullptr;
  };
  for (int i = 0; i < a->desc.n_pages; ++i) drop(a->slots[i]);
  for (psi_page_slot& sl : a->lent) drop(sl);
  for (psi_page_slot& sl : a->bias_slots) drop(sl);
  if (a->last_stop_ring < 0) a->last_stop = nullptr;
  for (const psi_timed& t : a->pending) {
    float ms = 0.0f;
    PSI_HIP(hipEventElapsedTime(&ms, t.start, t.stop));
    if (t.kind == 0) {
      a->stats.gemm_ms += ms;
      a->stats.gemm_launches++;
      a->stats.gemm_flops += t.work;
    } else if (t.kind == 1) {
      a->stats.attn_ms += ms;
      a->stats.attn_launches++;
      a->stats.attn_flops += t.work;
    } else if (t.kind == 4) {
      // normalisation / rotary kernels: device timeline only
    } else {
      // copy_ms = busy time of the busier copy stream
      a->copy_ms_stream[t.kind - 2] += ms;
      a->stats.copy_ms = a->copy_ms_stream[0] > a->copy_ms_stream[1] ? a->copy_ms_stream[0] : a->copy_ms_stream[1];
      a->stats.copy_bytes_timed += (uint64_t)t.work;
    }
    if (a->trace_base && a->trace.size() < a->trace_cap) {
      float off = 0.0f;
      PSI_HIP(hipEventElapsedTime(&off, a->trace_base, t.start));
      a->trace.push_back(psi_trace_event{t.kind, 0, (double)off, (double)ms, t.work});
    }
    a->event_pool.push_back(t.start);
    a->event_pool.push_back(t.stop);
  }
  a->pending.clear();
  return PSI_OK;
}

}  // namespace psi

using namespace psi;

extern "C" {

psi_status psi_arena_create(const psi_arena_desc* d, psi_arena** out) {
  if (!out) return fail(PSI_E_INVALID, "psi_arena_create: null out");
  psi_arena_layout L;
  psi_status st = psi_arena_plan(d, &L);
  if (st) return st;
  psi_arena* a = new psi_arena();
  a->desc = *d;
  a->layout = L;
  a->dry = d->flags & PSI_ARENA_DRY_RUN;
  a->compute = static_cast<hipStream_t>(d->compute_stream);
  a->stats.arena_bytes = d->arena_bytes;
  a->stats.page_bytes = d->page_bytes;
  a->stats.workspace_bytes = d->workspace_bytes;
  a->stats.scratch_bytes = L.scratch_bytes;
  if (!a->dry) {
    hipError_t e = hipGetDevice(&a->device);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&a->base), d->arena_bytes);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&a->copy, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&a->copy1, hipStreamNonBlocking);
    for (int i = 0; e == hipSuccess && i < d->n_pages; ++i) {
      e = hipEventCreateWithFlags(&a->slots[i].ready, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&a->slots[i].release, hipEventDisableTiming);
      a->slots[i].dev = a->base + L.page_off[i];
    }
    for (int i = 0; e == hipSuccess && i < 2; ++i) {
      e = hipEventCreateWithFlags(&a->bias_slots[i].ready, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&a->bias_slots[i].release, hipEventDisableTiming);
      a->bias_slots[i].dev = a->base + L.bias_off[i];
    }
    for (int i = 0; e == hipSuccess && i < 4; ++i)
      e = hipEventCreateWithFlags(&a->pipe_ev[i], hipEventDisableTiming);
    for (int i = 0; e == hipSuccess && i < psi_arena::kMaxLent; ++i) {
      e = hipEventCreateWithFlags(&a->lent[i].ready, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&a->lent[i].release, hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&a->scratch_free, hipEventDisableTiming);
    for (int i = 0; e == hipSuccess && i < psi_arena::kStopRing; ++i)
      e = hipEventCreateWithFlags(&a->stop_ring[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      psi_status r = hip_fail(e, "psi_arena_create");
      psi_arena_destroy(a);
      return r;
    }
  }
  *out = a;
  return PSI_OK;
}

psi_status psi_arena_destroy(psi_arena* a) {
  if (!a) return PSI_OK;
  psi_status st = PSI_OK;
  if (!a->dry) {
    if (a->copy) (void)hipStreamSynchronize(a->copy);
    if (a->copy1) (void)hipStreamSynchronize(a->copy1);
    if (a->copyb) (void)hipStreamSynchronize(a->copyb);
    (void)hipStreamSynchronize(a->compute);
    for (psi_timed& t : a->pending) {
      a->event_pool.push_back(t.start);
      a->event_pool.push_back(t.stop);
    }
    for (hipEvent_t e : a->event_pool) (void)hipEventDestroy(e);
    if (a->trace_base) (void)hipEventDestroy(a->trace_base);
    for (int i = 0; i < a->desc.n_pages; ++i) {
      if (a->slots[i].ready) (void)hipEventDestroy(a->slots[i].ready);
      if (a->slots[i].release) (void)hipEventDestroy(a->slots[i].release);
    }
    for (int i = 0; i < 2; ++i) {
      if (a->bias_slots[i].ready) (void)hipEventDestroy(a->bias_slots[i].ready);
      if (a->bias_slots[i].release) (void)hipEventDestroy(a->bias_slots[i].release);
    }
    for (hipEvent_t e : a->pipe_ev)
      if (e) (void)hipEventDestroy(e);
    for (psi_page_slot& l : a->lent) {
      if (l.ready) (void)hipEventDestroy(l.ready);
      if (l.release) (void)hipEventDestroy(l.release);
    }
    if (a->scratch_free) (void)hipEventDestroy(a->scratch_free);
    for (hipEvent_t e : a->stop_ring)
      if (e) (void)hipEventDestroy(e);
    if (a->copy) (void)hipStreamDestroy(a->copy);
    if (a->copy1) (void)hipStreamDestroy(a->copy1);
    if (a->copyb) (void)hipStreamDestroy(a->copyb);
    if (a->base) {
      hipError_t e = hipFree(a->base);
      if (e != hipSuccess) st = hip_fail(e, "hipFree(arena)");
    }
  }
  delete a;
  return st;
}

psi_status psi_arena_sync(psi_arena* a) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (a->dry) return PSI_OK;
  PSI_HIP(hipStreamSynchronize(a->copy));
  PSI_HIP(hipStreamSynchronize(a->copy1));
  if (a->copyb) PSI_HIP(hipStreamSynchronize(a->copyb));
  PSI_HIP(hipStreamSynchronize(a->compute));
  a->stats.host_syncs += 4;
  return PSI_OK;
}

psi_status psi_arena_stats(psi_arena* a, psi_stats* out) {
  if (!a || !out) return fail(PSI_E_INVALID, "null argument");
  if ((a->desc.flags & PSI_ARENA_PROFILE) && !a->pending.empty()) {
    psi_status st = harvest(a);
    if (st) return st;
  }
  *out = a->stats;
  return PSI_OK;
}

psi_status psi_arena_reset_stats(psi_arena* a) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (!a->pending.empty()) {
    psi_status st = harvest(a);
    if (st) return st;
  }
  psi_stats s;
  std::memset(&s, 0, sizeof s);
  s.arena_bytes = a->stats.arena_bytes;
  s.page_bytes = a->stats.page_bytes;
  s.workspace_bytes = a->stats.workspace_bytes;
  s.scratch_bytes = a->stats.scratch_bytes;
  s.scratch_high_water = a->scratch_top;
  a->stats = s;
  a->copy_ms_stream[0] = a->copy_ms_stream[1] = 0.0;
  return PSI_OK;
}

psi_status psi_arena_trace_start(psi_arena* a, size_t capacity) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (!(a->desc.flags & PSI_ARENA_PROFILE)) return fail(PSI_E_INVALID, "trace needs PSI_ARENA_PROFILE");
  if (a->dry) return PSI_OK;
  psi_status st = harvest(a);  // synchronises the three streams
  if (st) return st;
  if (!a->trace_base) PSI_HIP(hipEventCreate(&a->trace_base));
  PSI_HIP(hipEventRecord(a->trace_base, a->compute));
  a->trace.clear();
  a->trace.reserve(capacity < (1u << 20) ? capacity : (1u << 20));
  a->trace_cap = capacity;
  return PSI_OK;
}

psi_status psi_arena_trace_read(psi_arena* a, psi_trace_event* out, size_t capacity, size_t* count) {
  if (!a || (capacity && !out)) return fail(PSI_E_INVALID, "null argument");
  if (!(a->desc.flags & PSI_ARENA_PROFILE)) return fail(PSI_E_INVALID, "trace needs PSI_ARENA_PROFILE");
  if (!a->pending.empty()) {
    psi_status st = harvest(a);
    if (st) return st;
  }
  const size_t n = a->trace.size() < capacity ? a->trace.size() : capacity;
  for (size_t i = 0; i < n; ++i) out[i] = a->trace[i];
  if (count) *count = a->trace.size();
  return PSI_OK;
}

psi_status psi_arena_set_timing(psi_arena* a, int on) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (!(a->desc.flags & PSI_ARENA_PROFILE)) return fail(PSI_E_INVALID, "timing needs PSI_ARENA_PROFILE");
  a->timing_off = !on;
  return PSI_OK;
}

psi_status psi_arena_device_base(psi_arena* a, void** base_out, size_t* bytes_out) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (base_out) *base_out = a->base;
  if (bytes_out) *bytes_out = a->desc.arena_bytes;
  return PSI_OK;
}

psi_status psi_arena_set_probe(psi_arena* a, psi_journal* j, int32_t step, int32_t block) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  a->probe = j;
  a->probe_step = step;
  a->probe_block = block;
  return PSI_OK;
}

psi_status psi_page_submit(psi_arena* a, const void* host_pinned, size_t bytes, int* page_out) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  return page_submit_ex(a, host_pinned, bytes, page_out, true);
}

psi_status psi_page_acquire(psi_arena* a, int page, void** dev_out) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  psi_status st = page_acquire(a, page);
  if (st) return st;
  if (dev_out) *dev_out = a->dry ? nullptr : a->slots[page].dev;
  return PSI_OK;
}

psi_status psi_page_release(psi_arena* a, int page) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  return page_release(a, page);
}

}  // extern "C"
