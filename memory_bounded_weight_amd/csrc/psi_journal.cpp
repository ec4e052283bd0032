// psi_journal.cpp -- indexed host journal of BF16 state.
//
// [PSI] sec. II-D and sec. III-B ("Precision-Preserving Subtensor Inference
// for a 22B Joint Audio-Video Generator under a Fixed GPU Working Set",
// arXiv 2611.08023): an indexed host journal stores values by block,
// branch and tensor role.  The device-to-host copy waits for its producer,
// host commit waits for that copy before moving the staged bytes into the
// journal location, and device-buffer overwrites and later reloads keep the
// previous-consumer dependencies.  Asynchronous transport stages state
// through a pinned host ring.
//
// Default mode: the store is pinned host memory, so a commit is one DMA
// copy into the entry's location on the journal's D2H stream (the "host
// commit" is the index update) and a reload is one DMA copy back on its
// H2D stream.  Ring mode (PSI_JOURNAL_RING): the store is pageable; two
// library streams alternate over the pinned ring slots (slot s belongs to
// stream s % 2, so stream order alone makes slot reuse follow the previous
// host commit); a D2H copy into the slot is followed on the same stream by a
// host callback that moves the bytes into the store.  The store is
// allocated and touched when the journal is created.
#include <cstdlib>
#include <cstring>
#include <map>
#include <tuple>

#include "psi_internal.h"

namespace {

struct KeyLess {
  bool operator()(const psi_key& a, const psi_key& b) const {
    return std::tie(a.step, a.block, a.branch, a.role) < std::tie(b.step, b.block, b.branch, b.role);
  }
};

struct Entry {
  size_t off;
  size_t bytes;
};

struct HostCopy {
  void* dst;
  const void* src;
  size_t n;
};

void host_copy_cb(void* arg) {
  HostCopy* c = static_cast<HostCopy*>(arg);
  std::memcpy(c->dst, c->src, c->n);
  delete c;
}

}  // namespace

struct psi_journal {
  psi_journal_desc desc{};
  bool ring_mode = false;
  char* ring = nullptr;   // pinned staging (ring and sync modes)
  char* store = nullptr;  // pinned (default) or pageable, pre-touched (ring mode)
  size_t store_top = 0;
  std::map<psi_key, Entry, KeyLess> index;
  hipStream_t stream[2] = {nullptr, nullptr};
  hipEvent_t read_done[2] = {nullptr, nullptr};  // last D2H read of a device buffer per stream
  hipEvent_t write_done[2] = {nullptr, nullptr}; // last H2D reload per stream
  hipEvent_t dep = nullptr;
  hipEvent_t cross[2] = {nullptr, nullptr};     // orders the two streams before a reload
  bool used[2] = {false, false};
  int next_slot = 0;
  uint64_t bytes_d2h = 0, bytes_h2d = 0;
};

namespace psi {

// Records `ev` on journal stream 1 once the work enqueued so far on the
// streams marked in `touched` has completed.
static psi_status join_record(psi_journal* j, hipEvent_t ev, const bool touched[2]) {
  if (touched[0]) {
    PSI_HIP(hipEventRecord(j->cross[0], j->stream[0]));
    PSI_HIP(hipStreamWaitEvent(j->stream[1], j->cross[0], 0));
  }
  return hipEventRecord(ev, j->stream[1]) == hipSuccess ? PSI_OK : fail(PSI_E_HIP, "journal event");
}

psi_status journal_commit_ev(psi_journal* j, psi_key k, const void* dev, size_t bytes, hipStream_t prod,
                             hipEvent_t read_ev) {
  if (!j || !dev || bytes == 0) return fail(PSI_E_INVALID, "journal commit: bad arguments");
  if (j->index.count(k)) return fail(PSI_E_JOURNAL_KEY, "journal commit: duplicate key");
  const size_t need = align_up(bytes, 64);
  if (j->store_top + need > j->desc.store_bytes)
    return fail(PSI_E_JOURNAL_FULL, "journal store full: " + std::to_string(j->store_top + need) +
                                        " B > " + std::to_string(j->desc.store_bytes) + " B");
  const Entry ent{j->store_top, bytes};
  const size_t S = j->desc.ring_slot_bytes;
  const char* src = static_cast<const char*>(dev);
  if (j->desc.flags & PSI_JOURNAL_SYNC) {
    // transport control: copies on the producer's stream, host blocks per slot
    for (size_t off = 0; off < bytes; off += S) {
      size_t n = bytes - off < S ? bytes - off : S;
      PSI_HIP(hipMemcpyAsync(j->ring, src + off, n, hipMemcpyDeviceToHost, prod));
      PSI_HIP(hipStreamSynchronize(prod));
      std::memcpy(j->store + ent.off + off, j->ring, n);
    }
    if (read_ev) PSI_HIP(hipEventRecord(read_ev, prod));
  } else if (!j->ring_mode) {
    // one DMA copy straight into the pinned entry, after the producer's work
    PSI_HIP(hipEventRecord(j->dep, prod));
    PSI_HIP(hipStreamWaitEvent(j->stream[0], j->dep, 0));
    PSI_HIP(hipMemcpyAsync(j->store + ent.off, src, bytes, hipMemcpyDeviceToHost, j->stream[0]));
    PSI_HIP(hipEventRecord(j->read_done[0], j->stream[0]));
    if (read_ev) PSI_HIP(hipEventRecord(read_ev, j->stream[0]));
    j->used[0] = true;
  } else {
    PSI_HIP(hipEventRecord(j->dep, prod));
    for (int i = 0; i < 2; ++i) PSI_HIP(hipStreamWaitEvent(j->stream[i], j->dep, 0));
    bool touched[2] = {false, false};
    for (size_t off = 0; off < bytes; off += S) {
      size_t n = bytes - off < S ? bytes - off : S;
      const int slot = j->next_slot;
      j->next_slot = (slot + 1) % j->desc.ring_slots;
      const int si = slot % 2;
      char* stage = j->ring + (size_t)slot * S;
      PSI_HIP(hipMemcpyAsync(stage, src + off, n, hipMemcpyDeviceToHost, j->stream[si]));
      PSI_HIP(hipEventRecord(j->read_done[si], j->stream[si]));
      j->used[si] = true;
      touched[si] = true;
      HostCopy* c = new HostCopy{j->store + ent.off + off, stage, n};
      hipError_t e = hipLaunchHostFunc(j->stream[si], host_copy_cb, c);
      if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "hipLaunchHostFunc(journal commit)");
      }
    }
    if (read_ev) {
      psi_status st = join_record(j, read_ev, touched);
      if (st) return st;
    }
  }
  j->index[k] = ent;
  j->store_top += need;
  j->bytes_d2h += bytes;
  return PSI_OK;
}

psi_status journal_reload_ev(psi_journal* j, psi_key k, void* dev, size_t bytes, hipStream_t cons,
                             hipEvent_t done) {
  if (!j || !dev) return fail(PSI_E_INVALID, "journal reload: bad arguments");
  auto it = j->index.find(k);
  if (it == j->index.end()) return fail(PSI_E_JOURNAL_KEY, "journal reload: key not found");
  if (it->second.bytes != bytes) return fail(PSI_E_JOURNAL_KEY, "journal reload: size mismatch");
  const size_t S = j->desc.ring_slot_bytes;
  char* dst = static_cast<char*>(dev);
  const Entry ent = it->second;
  if (j->desc.flags & PSI_JOURNAL_SYNC) {
    PSI_HIP(hipStreamSynchronize(j->stream[0]));
    PSI_HIP(hipStreamSynchronize(j->stream[1]));
    for (size_t off = 0; off < bytes; off += S) {
      size_t n = bytes - off < S ? bytes - off : S;
      PSI_HIP(hipStreamSynchronize(cons));
      std::memcpy(j->ring, j->store + ent.off + off, n);
      PSI_HIP(hipMemcpyAsync(dst + off, j->ring, n, hipMemcpyHostToDevice, cons));
    }
    PSI_HIP(hipStreamSynchronize(cons));
    if (done) PSI_HIP(hipEventRecord(done, cons));
  } else if (!j->ring_mode) {
    // the overwrite of dev follows its previous consumers on `cons`, and the
    // entry's commit (both on the journal's streams) precedes the read
    PSI_HIP(hipEventRecord(j->dep, cons));
    PSI_HIP(hipEventRecord(j->cross[0], j->stream[0]));
    PSI_HIP(hipStreamWaitEvent(j->stream[1], j->dep, 0));
    PSI_HIP(hipStreamWaitEvent(j->stream[1], j->cross[0], 0));
    PSI_HIP(hipMemcpyAsync(dst, j->store + ent.off, bytes, hipMemcpyHostToDevice, j->stream[1]));
    if (done) {
      PSI_HIP(hipEventRecord(done, j->stream[1]));
    } else {
      PSI_HIP(hipEventRecord(j->write_done[1], j->stream[1]));
      PSI_HIP(hipStreamWaitEvent(cons, j->write_done[1], 0));
    }
  } else {
    // the overwrite of dev follows its previous consumers on `cons`, and
    // every earlier host commit (on either stream) precedes the reads of
    // the store
    PSI_HIP(hipEventRecord(j->dep, cons));
    for (int i = 0; i < 2; ++i) PSI_HIP(hipEventRecord(j->cross[i], j->stream[i]));
    for (int i = 0; i < 2; ++i) {
      PSI_HIP(hipStreamWaitEvent(j->stream[i], j->dep, 0));
      PSI_HIP(hipStreamWaitEvent(j->stream[i], j->cross[1 - i], 0));
    }
    bool touched[2] = {false, false};
    for (size_t off = 0; off < bytes; off += S) {
      size_t n = bytes - off < S ? bytes - off : S;
      const int slot = j->next_slot;
      j->next_slot = (slot + 1) % j->desc.ring_slots;
      const int si = slot % 2;
      char* stage = j->ring + (size_t)slot * S;
      HostCopy* c = new HostCopy{stage, j->store + ent.off + off, n};
      hipError_t e = hipLaunchHostFunc(j->stream[si], host_copy_cb, c);
      if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "hipLaunchHostFunc(journal reload)");
      }
      PSI_HIP(hipMemcpyAsync(dst + off, stage, n, hipMemcpyHostToDevice, j->stream[si]));
      touched[si] = true;
    }
    if (done) {
      psi_status st = join_record(j, done, touched);
      if (st) return st;
    } else {
      for (int i = 0; i < 2; ++i)
        if (touched[i]) {
          PSI_HIP(hipEventRecord(j->write_done[i], j->stream[i]));
          PSI_HIP(hipStreamWaitEvent(cons, j->write_done[i], 0));
        }
    }
  }
  j->bytes_h2d += bytes;
  return PSI_OK;
}

}  // namespace psi

using namespace psi;

extern "C" {

psi_status psi_journal_destroy(psi_journal* j);

psi_status psi_journal_create(const psi_journal_desc* d, psi_journal** out) {
  if (!d || !out) return fail(PSI_E_INVALID, "psi_journal_create: null argument");
  const bool ring_mode = d->flags & PSI_JOURNAL_RING;
  const bool sync = d->flags & PSI_JOURNAL_SYNC;
  if ((ring_mode || sync) && (d->ring_slot_bytes == 0 || d->ring_slots < 2))
    return fail(PSI_E_INVALID, "journal: ring and sync modes need ring_slots >= 2 and a non-empty slot");
  psi_journal* j = new psi_journal();
  j->desc = *d;
  j->ring_mode = ring_mode;
  hipError_t e = hipSuccess;
  if (ring_mode || sync) {
    e = hipHostMalloc(reinterpret_cast<void**>(&j->ring), d->ring_slot_bytes * d->ring_slots,
                      hipHostMallocDefault);
    if (e != hipSuccess) {
      delete j;
      return hip_fail(e, "hipHostMalloc(journal ring)");
    }
  }
  if (d->store_bytes) {
    if (ring_mode) {
      j->store = static_cast<char*>(std::malloc(d->store_bytes));
      if (!j->store) {
        psi_journal_destroy(j);
        return fail(PSI_E_INVALID, "journal: cannot allocate the host store");
      }
    } else {
      e = hipHostMalloc(reinterpret_cast<void**>(&j->store), d->store_bytes, hipHostMallocDefault);
      if (e != hipSuccess) {
        j->store = nullptr;
        psi_journal_destroy(j);
        return hip_fail(e, "hipHostMalloc(journal store)");
      }
    }
    std::memset(j->store, 0, d->store_bytes);  // touch every page now, not during commits
  }
  for (int i = 0; i < 2 && e == hipSuccess; ++i) {
    e = hipStreamCreateWithFlags(&j->stream[i], hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j->read_done[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j->write_done[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j->cross[i], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&j->dep, hipEventDisableTiming);
  if (e != hipSuccess) {
    psi_status st = hip_fail(e, "psi_journal_create");
    psi_journal_destroy(j);
    return st;
  }
  *out = j;
  return PSI_OK;
}

psi_status psi_journal_destroy(psi_journal* j) {
  if (!j) return PSI_OK;
  for (int i = 0; i < 2; ++i) {
    if (j->stream[i]) {
      (void)hipStreamSynchronize(j->stream[i]);
      (void)hipStreamDestroy(j->stream[i]);
    }
    if (j->read_done[i]) (void)hipEventDestroy(j->read_done[i]);
    if (j->write_done[i]) (void)hipEventDestroy(j->write_done[i]);
    if (j->cross[i]) (void)hipEventDestroy(j->cross[i]);
  }
  if (j->dep) (void)hipEventDestroy(j->dep);
  if (j->ring) (void)hipHostFree(j->ring);
  if (j->ring_mode)
    std::free(j->store);
  else if (j->store)
    (void)hipHostFree(j->store);
  delete j;
  return PSI_OK;
}

psi_status psi_journal_commit(psi_journal* j, psi_key k, const void* dev, size_t bytes,
                              void* producer_stream) {
  return journal_commit_ev(j, k, dev, bytes, static_cast<hipStream_t>(producer_stream), nullptr);
}

psi_status psi_journal_reload(psi_journal* j, psi_key k, void* dev, size_t bytes, void* consumer_stream) {
  return journal_reload_ev(j, k, dev, bytes, static_cast<hipStream_t>(consumer_stream), nullptr);
}

psi_status psi_journal_reset(psi_journal* j) {
  if (!j) return fail(PSI_E_INVALID, "null journal");
  // everything enqueued so far on either journal stream (reloads reading
  // the store, host commits writing it) precedes everything enqueued later
  for (int i = 0; i < 2; ++i) PSI_HIP(hipEventRecord(j->cross[i], j->stream[i]));
  for (int i = 0; i < 2; ++i) PSI_HIP(hipStreamWaitEvent(j->stream[i], j->cross[1 - i], 0));
  j->index.clear();
  j->store_top = 0;
  return PSI_OK;
}

psi_status psi_journal_fence(psi_journal* j, void* stream) {
  if (!j) return fail(PSI_E_INVALID, "null journal");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < 2; ++i)
    if (j->used[i]) PSI_HIP(hipStreamWaitEvent(s, j->read_done[i], 0));
  return PSI_OK;
}

psi_status psi_journal_sync(psi_journal* j) {
  if (!j) return fail(PSI_E_INVALID, "null journal");
  for (int i = 0; i < 2; ++i) PSI_HIP(hipStreamSynchronize(j->stream[i]));
  return PSI_OK;
}

psi_status psi_journal_read(psi_journal* j, psi_key k, void* host_dst, size_t bytes) {
  if (!j || !host_dst) return fail(PSI_E_INVALID, "journal read: bad arguments");
  auto it = j->index.find(k);
  if (it == j->index.end()) return fail(PSI_E_JOURNAL_KEY, "journal read: key not found");
  if (it->second.bytes != bytes) return fail(PSI_E_JOURNAL_KEY, "journal read: size mismatch");
  psi_status st = psi_journal_sync(j);
  if (st) return st;
  std::memcpy(host_dst, j->store + it->second.off, bytes);
  return PSI_OK;
}

psi_status psi_journal_counters(psi_journal* j, uint64_t* d2h, uint64_t* h2d, uint64_t* entries) {
  if (!j) return fail(PSI_E_INVALID, "null journal");
  if (d2h) *d2h = j->bytes_d2h;
  if (h2d) *h2d = j->bytes_h2d;
  if (entries) *entries = j->index.size();
  return PSI_OK;
}

}  // extern "C"
