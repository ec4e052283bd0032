// psi_ops.cpp -- the paged operators: projection, FFN, attention sub-block
// and the block.  Host code only enqueues: page copies on the copy stream,
// kernels on the compute stream, ordered by the page events.
//
// [PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint
// Audio-Video Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
#include <cmath>
#include <vector>

#include "psi_internal.h"

namespace psi {
namespace {

void matrix_requests(const psi_matrix* m, std::vector<PageReq>& out) {
  const int n = psi_matrix_pages(m);
  for (int p = 0; p < n; ++p)
    out.push_back(PageReq{matrix_page_ptr(m, p), psi_matrix_page_bytes(m, p), m->resident != 0});
}

// The biases of an operator's matrices, staged together in one bias slot
// (resident matrices are used in place).  A split-by-rows page uses the
// slice of its output rows; a K-split matrix adds its whole bias once,
// after the last partial sum ([PSI] sec. II-B).
class OpBiases {
 public:
  // Stages the biases of matrices ms[0..n) and then n_extra further BF16
  // parameter vectors (pinned host, or device when `extra_resident`) in
  // one bias-slot request; get(i) for i >= n returns extra vector i - n.
  psi_status stage(psi_arena* a, const psi_matrix* const* ms, int n, const BiasPart* extra = nullptr,
                   int n_extra = 0, bool extra_resident = false) {
    a_ = a;
    BiasPart parts[kMax];
    const uint16_t* dev[kMax];
    if (n + n_extra > kMax) return fail(PSI_E_INVALID, "too many bias parts");
    for (int i = 0; i < n; ++i) {
      const bool copy = ms[i]->bias_host && !ms[i]->resident;
      parts[i] = BiasPart{copy ? ms[i]->bias_host : nullptr, copy ? (size_t)ms[i]->rows * 2 : 0};
    }
    for (int i = 0; i < n_extra; ++i)
      parts[n + i] = extra_resident ? BiasPart{nullptr, 0} : extra[i];
    psi_status st = bias_submit(a, parts, n + n_extra, dev, &slot_);
    if (st) return st;
    for (int i = 0; i < n; ++i) ptr_[i] = ms[i]->resident ? ms[i]->bias_host : dev[i];
    for (int i = 0; i < n_extra; ++i)
      ptr_[n + i] = extra_resident ? static_cast<const uint16_t*>(extra[i].host) : dev[n + i];
    return PSI_OK;
  }
  // Device address of part i (nullable); the compute stream first waits
  // for the bias copy.
  psi_status get(int i, const uint16_t** out) {
    psi_status st = bias_acquire(a_, slot_);
    if (st) return st;
    *out = ptr_[i];
    return PSI_OK;
  }
  // called by the operator right after its last kernel
  psi_status release() { return bias_release(a_, slot_, true); }

 private:
  static constexpr int kMax = 6;
  psi_arena* a_ = nullptr;
  int slot_ = -1;
  const uint16_t* ptr_[kMax] = {};
};

// Streams a list of page requests through the arena's slots: requests are
// submitted as soon as a slot is free (a lent slot that needs no wait, else
// the round-robin slot), so the copy of the next pages overlaps the
// consumers of the current one; with two slots this is the paper's two
// alternating pages ([PSI] sec. III-B weight prefetch).  Refilling a slot
// waits on the host for its last consumer (see page_submit_ex), so each copy
// starts right after that consumer ends (submitting only slots whose
// consumer had already finished started copies later and cost the
// copy-bound workloads 2-6%).  The one exception is the slot freed by the
// consumer enqueued last: waiting for that kernel would leave the compute
// stream empty until the host enqueues the next one.  A page not needed yet
// goes to another slot, and that slot is refilled right after the next
// launch (the arena's hold, ended in its launch path through `refill`).
//
// Given the next operator's requests (`next`), the feeder goes on with them
// once its own are all submitted, into regular slots only, and leaves them
// in the arena, where the next operator's feeder adopts them: a
// compute-bound operator (attention) then no longer leaves the copy engines
// idle while its last kernels run.
class PageFeeder {
 public:
  PageFeeder(psi_arena* a, std::vector<PageReq> reqs, const std::vector<PageReq>* next = nullptr)
      : a_(a), reqs_(std::move(reqs)), slot_(reqs_.size(), -1) {
    if (!a_->ahead.empty() && !a_->ahead_producing) {
      // pages the previous operator submitted for this one
      const size_t n = a_->ahead_slot.size();
      for (size_t i = 0; i < n && !mismatch_; ++i) {
        const PageReq& q = a_->ahead[i];
        mismatch_ = i >= reqs_.size() || reqs_[i].host != q.host || reqs_[i].bytes != q.bytes ||
                    reqs_[i].resident != q.resident;
      }
      if (!mismatch_) {
        for (size_t i = 0; i < n; ++i) slot_[i] = a_->ahead_slot[i];
        submitted_ = n;
        a_->ahead.clear();
        a_->ahead_slot.clear();
      }
    }
    if (next && !next->empty() && !mismatch_) {
      a_->ahead = *next;
      a_->ahead_slot.clear();
      a_->ahead_producing = true;
      producer_ = true;
    }
    a_->refill = &PageFeeder::refill_cb;
    a_->refill_ctx = this;
  }
  ~PageFeeder() {
    if (a_->refill_ctx == this) {
      a_->refill = nullptr;
      a_->refill_ctx = nullptr;
    }
    if (producer_) a_->ahead_producing = false;  // from now on the next feeder adopts them
  }
  PageFeeder(const PageFeeder&) = delete;
  PageFeeder& operator=(const PageFeeder&) = delete;
  static psi_status refill_cb(void* self) { return static_cast<PageFeeder*>(self)->feed(); }

  // Submits requests in order while a slot is free.  Requests below `need`
  // are wanted now and may take any slot; later ones avoid the slot freed by
  // the last enqueued consumer while it may still run.
  psi_status feed(size_t need = 0) {
    if (mismatch_) return fail(PSI_E_STATE, "pages submitted ahead do not match the operator's requests");
    while (submitted_ < reqs_.size()) {
      const PageReq& r = reqs_[submitted_];
      if (r.resident) {  // consumed in place: no copy, no slot
        ++submitted_;
        continue;
      }
      const bool avoid = submitted_ >= need;
      if (submit_slot(a_, avoid) < 0) break;
      int s = -1;
      psi_status st = page_submit_ex(a_, r.host, r.bytes, &s, false, avoid);
      if (st) return st;
      slot_[submitted_++] = s;
    }
    if (producer_ && submitted_ == reqs_.size()) return feed_ahead();
    return PSI_OK;
  }
  // Waits (on the compute stream) for request i and returns its page.
  psi_status take(size_t i, const uint16_t** page) {
    psi_status st = feed(i + 1);
    if (st) return st;
    const PageReq& r = reqs_[i];
    if (r.resident) {
      *page = static_cast<const uint16_t*>(r.host);
      return PSI_OK;
    }
    if (i >= submitted_) return fail(PSI_E_STATE, "page request not submitted (slots exhausted)");
    st = page_acquire(a_, slot_[i]);
    if (st) return st;
    *page = static_cast<const uint16_t*>(slot_dev(a_, slot_[i]));
    return PSI_OK;
  }
  psi_status give_back(size_t i) {
    if (!reqs_[i].resident) {
      psi_status st = page_release(a_, slot_[i], true);
      if (st) return st;
      a_->hold_slot = slot_[i];
    }
    return feed();
  }

 private:
  // The next operator's requests, into free regular slots; none of them is
  // wanted yet.
  psi_status feed_ahead() {
    while (a_->ahead_slot.size() < a_->ahead.size()) {
      const PageReq& r = a_->ahead[a_->ahead_slot.size()];
      if (r.resident) {
        a_->ahead_slot.push_back(-1);
        continue;
      }
      if (submit_slot(a_, true, true) < 0) break;
      int s = -1;
      psi_status st = page_submit_ex(a_, r.host, r.bytes, &s, false, true, true);
      if (st) return st;
      a_->ahead_slot.push_back(s);
      a_->stats.ahead_page_copies++;
    }
    return PSI_OK;
  }

  psi_arena* a_;
  std::vector<PageReq> reqs_;
  std::vector<int> slot_;
  size_t submitted_ = 0;
  bool producer_ = false;
  bool mismatch_ = false;
};

// Releases the pages submitted ahead for an operator that did not adopt
// them (an error before it ran), so that their slots serve again.
psi_status drop_ahead(psi_arena* a) {
  psi_status first = PSI_OK;
  for (int s : a->ahead_slot) {
    if (s < 0) continue;
    psi_status st = page_release(a, s);
    if (st && !first) first = st;
  }
  a->ahead.clear();
  a->ahead_slot.clear();
  a->ahead_producing = false;
  return first;
}

psi_status check_matrix_pinned(psi_arena* a, const psi_matrix* m, const char* name) {
  if (a->dry) return PSI_OK;
  if (m->resident) {
    if (reinterpret_cast<uintptr_t>(m->pages_host) % 16 != 0)
      return fail(PSI_E_ALIGN, std::string(name) + ": resident image must be 16-byte aligned");
    return PSI_OK;
  }
  psi_status st = check_pinned(m->pages_host, name);
  if (st) return st;
  if (m->bias_host) st = check_pinned(m->bias_host, "bias");
  return st;
}

// Restores the scratch stack when an operator returns.
struct ScratchMark {
  psi_arena* a;
  size_t mark;
  explicit ScratchMark(psi_arena* a_) : a(a_), mark(a_->scratch_top) {}
  ~ScratchMark() { scratch_reset(a, mark); }
};

// The attention kernel choice in the flags: 0 (automatic) to 4.
psi_status check_attn_config(unsigned flags) {
  if ((flags & PSI_OP_ATTN_CONFIG_MASK) > PSI_OP_ATTN_CONFIG(4))
    return fail(PSI_E_INVALID, "attention kernel choice (PSI_OP_ATTN_CONFIG) must be 0-4");
  return PSI_OK;
}

int attn_p_terms(unsigned flags) {
  if (flags & PSI_OP_BF16_SOFTMAX) return 1;
  return (flags & PSI_OP_ATTN_P2) ? 2 : 3;
}

// Lends the operator's idle scratch (the whole pages above its own
// allocations) as page slots for its requests, and takes them back when
// the operator returns; construct it after the last scratch allocation.
// Those pages wait behind compute less often: a lent slot is filled only
// when that needs no host wait.
class LentSlots {
 public:
  explicit LentSlots(psi_arena* a, bool lend = true) : a_(a) {
    if (lend) lend_scratch_slots(a);
  }
  ~LentSlots() { (void)return_lent_slots(a_); }
  LentSlots(const LentSlots&) = delete;
  LentSlots& operator=(const LentSlots&) = delete;

 private:
  psi_arena* a_;
};

GemmArgs gemm_args() {
  GemmArgs g{};
  g.epi = EPI_BIAS;
  return g;
}

const uint16_t* offset(const uint16_t* v, size_t off) { return v ? v + off : nullptr; }

// Projection of one head group from a page of rows (Wq_g or Wk_g):
// out[Ms, ext] (row stride ldo) = B(src page^T + bias).
psi_status project(psi_arena* a, const uint16_t* src, int Ms, int dm, const uint16_t* page, int ext,
                   const uint16_t* bias, uint16_t* out, long ldo, int bbase) {
  GemmArgs G = gemm_args();
  G.A = src; G.lda = dm; G.B = page; G.ldb = dm;
  G.M = Ms; G.N = ext; G.K = dm;
  G.bias = bias; G.out = out; G.ldo = ldo; G.baseline_bias = bbase;
  return run_gemm(a, G);
}

// V_g^T [ext, Ms] (row stride ldvt) = B(page src^T + bias), the bias along
// rows: V written transposed, so that P.V reads keys contiguously.
psi_status project_vt(psi_arena* a, const uint16_t* src, int Ms, int dm, const uint16_t* page, int ext,
                      const uint16_t* bias, uint16_t* vt, long ldvt, int bbase) {
  GemmArgs G = gemm_args();
  G.A = page; G.lda = dm; G.B = src; G.ldb = dm;
  G.M = ext; G.N = Ms; G.K = dm;
  G.bias = bias; G.bias_on_m = 1; G.out = vt; G.ldo = ldvt; G.baseline_bias = bbase;
  return run_gemm(a, G);
}

// Online-softmax attention of the heads of one group; O overwrites Q.
psi_status attend(psi_arena* a, uint16_t* q, long ldq, const uint16_t* k, long ldk, const uint16_t* vt,
                  long ldvt, int Mq, int Mk, int heads, int dh, unsigned flags) {
  AttnArgs A{};
  A.q = q; A.ldq = ldq;
  A.k = k; A.ldk = ldk;
  A.vt = vt; A.ldvt = ldvt;
  A.Mq = Mq; A.Mk = Mk; A.heads = heads; A.dh = dh;
  A.alpha = (float)(1.0 / std::sqrt((double)dh));
  A.p_terms = attn_p_terms(flags);
  A.config = (int)((flags & PSI_OP_ATTN_CONFIG_MASK) >> 8);  // 0-4, checked at the operator's entry
  return run_attention(a, A);
}

// K-split O-projection step: ACC (+)= O_g Wo[:, g]^T over the group's K
// extent; after the last group y = B(ACC + bo) (+ x).
psi_status oproj_ksplit(psi_arena* a, const uint16_t* og, long ldog, int M, int dm, const uint16_t* page,
                        int ext, bool first, bool last, float* acc, const uint16_t* bo, uint16_t* y,
                        const uint16_t* x, unsigned flags, int bbase) {
  GemmArgs G = gemm_args();
  G.A = og; G.lda = ldog; G.B = page; G.ldb = ext;
  G.M = M; G.N = dm; G.K = ext;
  G.baseline_bias = bbase;
  if (!first) { G.acc_in = acc; G.ld_acc_in = dm; }
  if (last) {
    G.bias = bo; G.out = y; G.ldo = dm;
    if (flags & PSI_OP_RESIDUAL) { G.resid = x; G.ldr = dm; }
    if (flags & PSI_OP_STORE_ACC) { G.acc_out = acc; G.ld_acc_out = dm; }
  } else {
    G.epi = EPI_ACC; G.acc_out = acc; G.ld_acc_out = dm;
  }
  return run_gemm(a, G);
}

// O-projection output tile: y[:, c0 : c0+eo] = B(O Wo[c0 : c0+eo, :]^T + bo)
// (+ x) over the full K, O holding every head group's output ([M, dm]).
// Each output sums the same products in the same order as the K-split.
psi_status oproj_tile(psi_arena* a, const uint16_t* O, int M, int dm, const uint16_t* page, int eo, size_t c0,
                      const uint16_t* bo, uint16_t* y, const uint16_t* x, unsigned flags, int bbase) {
  GemmArgs G = gemm_args();
  G.A = O; G.lda = dm; G.B = page; G.ldb = dm;
  G.M = M; G.N = eo; G.K = dm;
  G.bias = offset(bo, c0); G.out = y + c0; G.ldo = dm; G.baseline_bias = bbase;
  if (flags & PSI_OP_RESIDUAL) { G.resid = x + c0; G.ldr = dm; }
  return run_gemm(a, G);
}

// Device pointers and pinned page images of an attention operator.
psi_status check_attn_args(psi_arena* a, const uint16_t* x, const uint16_t* y, const uint16_t* ctx,
                           const float* acc, const psi_matrix* Wq, const psi_matrix* Wk,
                           const psi_matrix* Wv, const psi_matrix* Wo) {
  if (a->dry) return PSI_OK;
  psi_status st;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(y, "y")) || (st = check_ptr(ctx, "ctx", true)) ||
      (st = check_ptr(acc, "acc", true)))
    return st;
  if ((st = check_matrix_pinned(a, Wq, "Wq")) || (st = check_matrix_pinned(a, Wk, "Wk")) ||
      (st = check_matrix_pinned(a, Wv, "Wv")) || (st = check_matrix_pinned(a, Wo, "Wo")))
    return st;
  return PSI_OK;
}

}  // namespace
}  // namespace psi

using namespace psi;

extern "C" {

psi_status psi_linear_paged(psi_arena* a, const uint16_t* x, int M, int K, const psi_matrix* W,
                            float* acc_dev, uint16_t* y, unsigned flags) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  size_t need = 0;
  psi_status st = psi_linear_plan(&a->desc, M, K, W, acc_dev != nullptr, &need);
  if (st) return st;
  const int N = W->rows;
  const bool resid = flags & PSI_OP_RESIDUAL;
  if (resid && K != N) return fail(PSI_E_INVALID, "linear residual needs K == N");
  if ((flags & PSI_OP_STORE_ACC) && !acc_dev) return fail(PSI_E_INVALID, "PSI_OP_STORE_ACC needs acc_dev");
  // every page reads all of x (output-column pages) or x's next columns
  // (K-split) while earlier launches have written y: no in-place form
  if ((st = check_alias(x, (size_t)M * K * 2, y, (size_t)M * N * 2, false, "linear"))) return st;
  if (!a->dry) {
    if ((st = check_ptr(x, "x")) || (st = check_ptr(y, "y")) || (st = check_ptr(acc_dev, "acc", true)))
      return st;
    if (N % 8 != 0 && W->split == PSI_SPLIT_COLS) return fail(PSI_E_ALIGN, "N must be a multiple of 8");
    if ((st = check_matrix_pinned(a, W, "W"))) return st;
  }
  if (M == 0) return PSI_OK;
  ScratchMark mark(a);
  float* acc = acc_dev;
  if (W->split == PSI_SPLIT_COLS && !acc) {
    acc = static_cast<float*>(scratch_alloc(a, (size_t)M * N * 4, &st));
    if (st) return st;
  }
  OpBiases bias;
  if ((st = bias.stage(a, &W, 1))) return st;
  std::vector<PageReq> reqs;
  matrix_requests(W, reqs);
  LentSlots lent(a);
  PageFeeder feeder(a, reqs);
  if ((st = feeder.feed())) return st;
  const uint16_t* b = nullptr;
  const int n = (int)reqs.size();
  for (int p = 0; p < n; ++p) {
    const uint16_t* page;
    if ((st = feeder.take(p, &page))) return st;
    const int ext = matrix_page_extent(W, p);
    GemmArgs g = gemm_args();
    g.M = M;
    g.baseline_bias = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
    if (W->split == PSI_SPLIT_ROWS) {
      const int c0 = p * W->block;
      if ((st = bias.get(0, &b))) return st;
      g.A = x; g.lda = K;
      g.B = page; g.ldb = K;
      g.N = ext; g.K = K;
      g.bias = b ? b + c0 : nullptr;
      g.out = y + c0; g.ldo = N;
      if (resid) { g.resid = x + c0; g.ldr = K; }
      if (flags & PSI_OP_STORE_ACC) { g.acc_out = acc_dev + c0; g.ld_acc_out = N; }
    } else {
      const int k0 = p * W->block;
      const bool last = p == n - 1;
      g.A = x + k0; g.lda = K;
      g.B = page; g.ldb = ext;
      g.N = N; g.K = ext;
      if (p > 0) { g.acc_in = acc; g.ld_acc_in = N; }
      if (last) {
        if ((st = bias.get(0, &b))) return st;
        g.bias = b;
        g.out = y; g.ldo = N;
        if (resid) { g.resid = x; g.ldr = K; }
        if (flags & PSI_OP_STORE_ACC) { g.acc_out = acc; g.ld_acc_out = N; }
      } else {
        g.epi = EPI_ACC;
        g.acc_out = acc; g.ld_acc_out = N;
      }
    }
    if ((st = run_gemm(a, g))) return st;
    if ((st = feeder.give_back(p))) return st;
  }
  return bias.release();
}

// The FFN; with out_fence, the compute stream first waits for every journal
// copy enqueued so far right before the first launch that writes y (the
// journal's reads of y's previous contents are earlier consumers).
// The FFN's page requests, U_0, V_0, U_1, V_1, ...: each hidden tile J is
// produced from U_J, then consumed by V_J ([PSI] eq. (2)).
std::vector<PageReq> ffn_requests(const psi_matrix* U, const psi_matrix* V) {
  std::vector<PageReq> ru, rv, reqs;
  matrix_requests(U, ru);
  matrix_requests(V, rv);
  for (size_t J = 0; J < ru.size(); ++J) {
    reqs.push_back(ru[J]);
    reqs.push_back(rv[J]);
  }
  return reqs;
}

static psi_status ffn_paged(psi_arena* a, const uint16_t* x, int M, int d, const psi_matrix* U,
                            const psi_matrix* V, int token_chunks, float* acc_dev, uint16_t* y,
                            unsigned flags, psi_journal* out_fence) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  size_t need = 0;
  psi_status st = psi_ffn_plan(&a->desc, M, d, U, V, token_chunks, acc_dev != nullptr, &need);
  if (st) return st;
  if ((flags & PSI_OP_STORE_ACC) && !acc_dev) return fail(PSI_E_INVALID, "PSI_OP_STORE_ACC needs acc_dev");
  if ((st = check_alias(x, (size_t)M * d * 2, y, (size_t)M * d * 2, true, "ffn"))) return st;
  if (!a->dry) {
    if ((st = check_ptr(x, "x")) || (st = check_ptr(y, "y")) || (st = check_ptr(acc_dev, "acc", true)))
      return st;
    if (d % 8 != 0) return fail(PSI_E_ALIGN, "d must be a multiple of 8");
    if ((st = check_matrix_pinned(a, U, "U")) || (st = check_matrix_pinned(a, V, "V"))) return st;
  }
  if (M == 0) return PSI_OK;
  const bool resid = flags & PSI_OP_RESIDUAL;
  const int th = U->block;
  // Token chunks: contiguous row ranges of x of `rows_per` rows.  One chunk
  // (the default) runs every page in a single launch over all tokens.  With
  // several, U_J and V_J stay acquired while every chunk runs its
  // up-projection and its carried down-projection, so each page is streamed
  // once and serves all chunks (page reuse across token chunks, [PSI]
  // sec. II-B eq. (2) with the bounded scratch of sec. II-A eq. (1)): the
  // hidden tile H_J holds one chunk's rows.  Rows are independent, so the
  // arithmetic of every output is the same whatever the chunk count.
  const int rows_per = (int)ffn_chunk_rows(M, token_chunks);
  const int nC = (M + rows_per - 1) / rows_per;
  ScratchMark mark(a);
  uint16_t* H = static_cast<uint16_t*>(scratch_alloc(a, (size_t)rows_per * th * 2, &st));
  if (st) return st;
  float* acc = acc_dev;
  if (!acc) {
    acc = static_cast<float*>(scratch_alloc(a, (size_t)M * d * 4, &st));
    if (st) return st;
  }
  const psi_matrix* ms[2] = {U, V};
  OpBiases bias;
  if ((st = bias.stage(a, ms, 2))) return st;
  const std::vector<PageReq> reqs = ffn_requests(U, V);
  const int nJ = (int)reqs.size() / 2;
  LentSlots lent(a);
  PageFeeder feeder(a, reqs);
  if ((st = feeder.feed())) return st;
  const uint16_t *ba = nullptr, *bb = nullptr;
  const unsigned baseline = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
  // H[0:mr] = B(phi(B(x[r0:r0+mr] U_J^T + a_J)))
  auto up = [&](int J, const uint16_t* page, int r0, int mr) -> psi_status {
    GemmArgs g = gemm_args();
    g.A = x + (size_t)r0 * d; g.lda = d;
    g.B = page; g.ldb = d;
    g.M = mr; g.N = matrix_page_extent(U, J); g.K = d;
    g.bias = ba ? ba + (size_t)J * th : nullptr;
    g.out = H; g.ldo = th;
    g.epi = EPI_GELU;
    g.baseline_bias = baseline;
    return run_gemm(a, g);
  };
  // ACC[r0:r0+mr] (+)= H V_J^T; after the last tile y = B(ACC + b) (+ x)
  auto down = [&](int J, const uint16_t* page, int r0, int mr) -> psi_status {
    const int ext = matrix_page_extent(U, J);
    const bool last = J == nJ - 1;
    GemmArgs g = gemm_args();
    g.A = H; g.lda = th;
    g.B = page; g.ldb = ext;
    g.M = mr; g.N = d; g.K = ext;
    float* ar = acc + (size_t)r0 * d;
    if (J > 0) { g.acc_in = ar; g.ld_acc_in = d; }
    if (last) {
      g.bias = bb;
      g.out = y + (size_t)r0 * d; g.ldo = d;
      if (resid) { g.resid = x + (size_t)r0 * d; g.ldr = d; }
      if (flags & PSI_OP_STORE_ACC) { g.acc_out = ar; g.ld_acc_out = d; }
    } else {
      g.epi = EPI_ACC;
      g.acc_out = ar; g.ld_acc_out = d;
    }
    return run_gemm(a, g);
  };
  for (int J = 0; J < nJ; ++J) {
    const int ext = matrix_page_extent(U, J);
    const bool last = J == nJ - 1;
    const uint16_t *upage, *vpage;
    if ((st = feeder.take(2 * J, &upage)) || (st = bias.get(0, &ba))) return st;
    if (nC == 1) {
      // up-projection + bias + BF16 + GELU + BF16 for all tokens; U_J goes
      // back before V_J is waited for, so the next copy overlaps the GEMMs
      if ((st = up(J, upage, 0, M)) || (st = feeder.give_back(2 * J))) return st;
      const int branch = token_chunks > 1 ? J * token_chunks : J;
      if (ext == th && (st = probe_commit(a, branch, PSI_ROLE_FFN_H, H, (size_t)M * th * 2))) return st;
      if ((st = feeder.take(2 * J + 1, &vpage))) return st;
      if (last && (st = bias.get(1, &bb))) return st;
      if (last && out_fence && !a->dry && (st = psi_journal_fence(out_fence, a->compute))) return st;
      if ((st = down(J, vpage, 0, M)) || (st = feeder.give_back(2 * J + 1))) return st;
      continue;
    }
    // several chunks: both pages of tile J held across the chunk launches
    if ((st = feeder.take(2 * J + 1, &vpage))) return st;
    if (last && (st = bias.get(1, &bb))) return st;
    if (last && out_fence && !a->dry && (st = psi_journal_fence(out_fence, a->compute))) return st;
    for (int c = 0; c < nC; ++c) {
      const int r0 = c * rows_per;
      const int mr = M - r0 < rows_per ? M - r0 : rows_per;
      if ((st = up(J, upage, r0, mr))) return st;
      // U_J's last use is the last chunk's up-projection
      if (c == nC - 1 && (st = feeder.give_back(2 * J))) return st;
      if (ext == th &&
          (st = probe_commit(a, J * token_chunks + c, PSI_ROLE_FFN_H, H, (size_t)mr * th * 2)))
        return st;
      if ((st = down(J, vpage, r0, mr))) return st;
    }
    if ((st = feeder.give_back(2 * J + 1))) return st;
  }
  return bias.release();
}

psi_status psi_ffn_paged(psi_arena* a, const uint16_t* x, int M, int d, const psi_matrix* U,
                         const psi_matrix* V, int token_chunks, float* acc_dev, uint16_t* y,
                         unsigned flags) {
  return ffn_paged(a, x, M, d, U, V, token_chunks, acc_dev, y, flags, nullptr);
}

psi_status psi_ffn_tiled(psi_arena* a, const uint16_t* x, int M, int d, const psi_matrix* U,
                         const psi_matrix* Vo, int schedule, psi_journal* j, int32_t step, int32_t block,
                         uint16_t* y, unsigned flags) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  psi_status st = psi_ffn_tiled_plan(&a->desc, M, d, U, Vo, schedule, nullptr);
  if (st) return st;
  if (schedule == PSI_FFN_REUSE && !j) return fail(PSI_E_INVALID, "ffn tiled: FFN reuse needs a journal");
  if (flags & PSI_OP_STORE_ACC) return fail(PSI_E_INVALID, "ffn tiled: no full accumulator to store");
  // output tiles: row tiles of Vo (a page each when split by rows, several
  // pages of whole hidden tiles each with 2-D page tiles)
  const int nO = (Vo->rows + Vo->block - 1) / Vo->block;
  const int nP = psi_matrix_pages(Vo);
  if ((st = check_alias(x, (size_t)M * d * 2, y, (size_t)M * d * 2, true, "ffn tiled"))) return st;
  if (x == y && nO > 1 && schedule != PSI_FFN_REUSE)
    return fail(PSI_E_INVALID, "ffn tiled: with recomputation y may alias x only with a single output tile");
  if (!a->dry) {
    if ((st = check_ptr(x, "x")) || (st = check_ptr(y, "y"))) return st;
    if (d % 8 != 0) return fail(PSI_E_ALIGN, "d must be a multiple of 8");
    if ((st = check_matrix_pinned(a, U, "U")) || (st = check_matrix_pinned(a, Vo, "V"))) return st;
  }
  if (M == 0) return PSI_OK;
  const bool resid = flags & PSI_OP_RESIDUAL;
  const int th = U->block, to = Vo->block;
  const int nJ = psi_matrix_pages(U);
  const bool reuse = schedule == PSI_FFN_REUSE;
  // hidden tiles J of page p: J * th in [col0, col0 + cols) (whole tiles,
  // checked by the plan)
  auto j_first = [&](int p) { return matrix_page_col0(Vo, p) / th; };
  auto j_end = [&](int p) { return (matrix_page_col0(Vo, p) + matrix_page_cols(Vo, p) + th - 1) / th; };
  ScratchMark mark(a);
  uint16_t* Hb[2];
  Hb[0] = static_cast<uint16_t*>(scratch_alloc(a, (size_t)M * th * 2, &st));
  if (st) return st;
  Hb[1] = Hb[0];
  if (reuse) {  // two hidden-tile buffers: journal copies overlap the GEMMs
    Hb[1] = static_cast<uint16_t*>(scratch_alloc(a, (size_t)M * th * 2, &st));
    if (st) return st;
  }
  float* acc = static_cast<float*>(scratch_alloc(a, (size_t)M * to * 4, &st));
  if (st) return st;
  const psi_matrix* ms[2] = {U, Vo};
  OpBiases bias;
  if ((st = bias.stage(a, ms, 2))) return st;
  std::vector<PageReq> ru, rv, reqs;
  matrix_requests(U, ru);
  matrix_requests(Vo, rv);
  if (schedule == PSI_FFN_REUSE) {
    reqs = ru;
    reqs.insert(reqs.end(), rv.begin(), rv.end());
  } else {
    for (int p = 0; p < nP; ++p) {
      reqs.push_back(rv[p]);
      for (int J = j_first(p); J < j_end(p); ++J) reqs.push_back(ru[J]);
    }
  }
  // not with the journal's reloads: more pages in flight delay the hidden
  // tiles the GEMMs wait for on the same host link (low-live blocks ran 7%
  // slower)
  LentSlots lent(a, !reuse);
  PageFeeder feeder(a, reqs);
  if ((st = feeder.feed())) return st;
  const uint16_t *ba = nullptr, *bb = nullptr;
  const unsigned baseline = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
  // H_J = B(phi(B(x U_J^T + a_J))) for all tokens, stored compactly
  // ([M, e_J], row stride e_J) so that a ragged last tile is also one
  // contiguous journal entry
  auto up = [&](int J, const uint16_t* page, uint16_t* H) -> psi_status {
    psi_status s2 = bias.get(0, &ba);
    if (s2) return s2;
    const int ej = matrix_page_extent(U, J);
    GemmArgs g = gemm_args();
    g.A = x; g.lda = d;
    g.B = page; g.ldb = d;
    g.M = M; g.N = ej; g.K = d;
    g.bias = ba ? ba + (size_t)J * th : nullptr;
    g.out = H; g.ldo = ej;
    g.epi = EPI_GELU;
    g.baseline_bias = baseline;
    return run_gemm(a, g);
  };
  // ACC_o (+)= H_J V[o rows, J cols]^T from page p of row tile o; the last
  // hidden tile writes y[:, o rows]
  auto down = [&](int p, int J, const uint16_t* vpage, const uint16_t* H) -> psi_status {
    const int eo = matrix_page_extent(Vo, p), ej = matrix_page_extent(U, J);
    const bool last = J == nJ - 1;
    GemmArgs g = gemm_args();
    g.A = H; g.lda = ej;
    g.B = vpage + ((size_t)J * th - matrix_page_col0(Vo, p)); g.ldb = matrix_page_cols(Vo, p);
    g.M = M; g.N = eo; g.K = ej;
    if (J > 0) { g.acc_in = acc; g.ld_acc_in = eo; }
    if (last) {
      psi_status s2 = bias.get(1, &bb);
      if (s2) return s2;
      const size_t c0 = (size_t)matrix_page_row0(Vo, p);
      g.bias = bb ? bb + c0 : nullptr;
      g.out = y + c0; g.ldo = d;
      if (resid) { g.resid = x + c0; g.ldr = d; }
      g.baseline_bias = baseline;
    } else {
      g.epi = EPI_ACC;
      g.acc_out = acc; g.ld_acc_out = eo;
    }
    return run_gemm(a, g);
  };
  const uint16_t* page;
  if (reuse) {
    // H_J in buffer J % 2: the commit of H_J records rd[b] once the journal
    // has read it, and up(J + 2) overwrites the buffer only after that
    hipEvent_t* rd = a->pipe_ev;
    hipEvent_t* ld = a->pipe_ev + 2;
    auto hkey = [&](int J) { return psi_key{step, block, J, PSI_ROLE_FFN_HSTATE}; };
    auto hbytes = [&](int J) { return (size_t)M * matrix_page_extent(U, J) * 2; };
    for (int J = 0; J < nJ; ++J) {
      const int b = J % 2;
      if (!a->dry && J >= 2) PSI_HIP(hipStreamWaitEvent(a->compute, rd[b], 0));
      if ((st = feeder.take(J, &page)) || (st = up(J, page, Hb[b])) || (st = feeder.give_back(J))) return st;
      if (!a->dry && (st = journal_commit_ev(j, hkey(J), Hb[b], hbytes(J), a->compute, rd[b]))) return st;
    }
    // down-projection steps t (over the pages in order, the hidden tiles of
    // each page in order) read buffer t % 2; the reload of step t + 1 is
    // issued before the GEMM of step t (after the GEMM of step t - 1, the
    // buffer's previous reader), so copies overlap GEMMs
    std::vector<int> step_j;
    for (int p = 0; p < nP; ++p)
      for (int J = j_first(p); J < j_end(p); ++J) step_j.push_back(J);
    const int T = (int)step_j.size();
    auto issue = [&](int t) -> psi_status {
      const int J = step_j[t];
      return journal_reload_ev(j, hkey(J), Hb[t % 2], hbytes(J), a->compute, ld[t % 2]);
    };
    if (!a->dry && (st = issue(0))) return st;
    int t = 0;
    for (int p = 0; p < nP; ++p) {
      const uint16_t* vpage;
      if ((st = feeder.take(nJ + p, &vpage))) return st;
      for (int J = j_first(p); J < j_end(p); ++J, ++t) {
        if (!a->dry) {
          if (t + 1 < T && (st = issue(t + 1))) return st;
          PSI_HIP(hipStreamWaitEvent(a->compute, ld[t % 2], 0));
        }
        if ((st = down(p, J, vpage, Hb[t % 2]))) return st;
      }
      if ((st = feeder.give_back(nJ + p))) return st;
    }
  } else {
    size_t r = 0;
    for (int p = 0; p < nP; ++p) {
      const size_t vi = r++;
      const uint16_t* vpage;
      if ((st = feeder.take(vi, &vpage))) return st;
      for (int J = j_first(p); J < j_end(p); ++J) {
        const size_t ui = r++;
        if ((st = feeder.take(ui, &page)) || (st = up(J, page, Hb[0])) || (st = feeder.give_back(ui))) return st;
        if ((st = down(p, J, vpage, Hb[0]))) return st;
      }
      if ((st = feeder.give_back(vi))) return st;
    }
  }
  return bias.release();
}

// The attention sub-block; with out_fence, the compute stream first waits
// for every journal copy enqueued so far right before the first launch that
// writes y (as in ffn_paged).
static psi_status attn_paged(psi_arena* a, const uint16_t* x, int M, const uint16_t* ctx, int Mc, int heads,
                             int head_dim, const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                             const psi_matrix* Wo, float* acc_dev, uint16_t* y, unsigned flags,
                             psi_journal* out_fence, const std::vector<PageReq>* next = nullptr) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (psi_status st = check_attn_config(flags)) return st;
  if (ctx && Mc < 1) return fail(PSI_E_INVALID, "attention: cross-attention needs Mc >= 1 keys");
  if (!ctx) Mc = 0;
  size_t need = 0;
  psi_status st = psi_attn_plan(&a->desc, M, Mc, heads, head_dim, Wq, Wk, Wv, Wo, acc_dev != nullptr, &need);
  if (st) return st;
  const bool otiles = Wo->split == PSI_SPLIT_ROWS;
  if ((flags & PSI_OP_STORE_ACC) && (!acc_dev || otiles))
    return fail(PSI_E_INVALID, "PSI_OP_STORE_ACC needs acc_dev and a column-split Wo");
  if (otiles && (reinterpret_cast<uintptr_t>(acc_dev) & 15))
    return fail(PSI_E_ALIGN, "attention: acc_dev must be 16-byte aligned when it holds the head-group outputs");
  if ((st = check_attn_args(a, x, y, ctx, acc_dev, Wq, Wk, Wv, Wo))) return st;
  const int dm = heads * head_dim;
  if ((st = check_alias(x, (size_t)M * dm * 2, y, (size_t)M * dm * 2, true, "attention"))) return st;
  if (M == 0) return PSI_OK;
  const int gw = Wq->block;
  const uint16_t* src = ctx ? ctx : x;
  const int Ms = ctx ? Mc : M;
  const long ldvt = (long)align_up((size_t)Ms, 64);
  const int bbase = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
  auto fence = [&]() -> psi_status {
    return out_fence && !a->dry ? psi_journal_fence(out_fence, a->compute) : PSI_OK;
  };
  ScratchMark mark(a);
  // Q_g, overwritten by O_g: one group's tile [M, gw] for the K-split, or
  // columns g of an [M, dm] buffer that keeps every group's O for the
  // output tiles.  With output tiles acc_dev holds no fp32 accumulator: its
  // memory takes that buffer and, where they fit behind it, K_g and V_g^T
  // (the plan's scratch figure follows the same rule).
  uint16_t* Q;
  uint16_t* Kb;
  uint16_t* Vt;
  long ldq;
  const size_t kbytes = align_up((size_t)Ms * gw * 2, kAlign);
  const size_t kvbytes = kbytes + align_up((size_t)gw * ldvt * 2, kAlign);
  const size_t obytes = align_up((size_t)M * dm * 2, kAlign);
  const bool kv_in_acc = otiles && acc_dev && obytes + kvbytes <= (size_t)M * dm * 4;
  if (otiles) {
    Q = acc_dev ? reinterpret_cast<uint16_t*>(acc_dev)
                : static_cast<uint16_t*>(scratch_alloc(a, (size_t)M * dm * 2, &st));
    ldq = dm;
  } else {
    Q = static_cast<uint16_t*>(scratch_alloc(a, (size_t)M * gw * 2, &st));
    ldq = gw;
  }
  if (st) return st;
  if (kv_in_acc) {
    char* base = reinterpret_cast<char*>(acc_dev) + obytes;
    Kb = reinterpret_cast<uint16_t*>(base);
    Vt = reinterpret_cast<uint16_t*>(base + kbytes);
  } else {
    Kb = static_cast<uint16_t*>(scratch_alloc(a, (size_t)Ms * gw * 2, &st));
    if (st) return st;
    Vt = static_cast<uint16_t*>(scratch_alloc(a, (size_t)gw * ldvt * 2, &st));
    if (st) return st;
  }
  float* acc = acc_dev;
  if (!acc && !otiles) {
    acc = static_cast<float*>(scratch_alloc(a, (size_t)M * dm * 4, &st));
    if (st) return st;
  }
  const psi_matrix* ms[4] = {Wq, Wk, Wv, Wo};
  OpBiases bias;
  if ((st = bias.stage(a, ms, 4))) return st;
  // pages: Wq_g, Wk_g, Wv_g (, Wo[:, g]) per group; output tiles Wo_o last
  std::vector<PageReq> rq, rk, rv, ro, reqs;
  matrix_requests(Wq, rq);
  matrix_requests(Wk, rk);
  matrix_requests(Wv, rv);
  matrix_requests(Wo, ro);
  const int nG = (int)rq.size();
  const int per = otiles ? 3 : 4;
  for (int g = 0; g < nG; ++g) {
    reqs.push_back(rq[g]);
    reqs.push_back(rk[g]);
    reqs.push_back(rv[g]);
    if (!otiles) reqs.push_back(ro[g]);
  }
  if (otiles) reqs.insert(reqs.end(), ro.begin(), ro.end());
  LentSlots lent(a);
  PageFeeder feeder(a, reqs, next);
  if ((st = feeder.feed())) return st;
  const uint16_t* bq[4];
  for (int g = 0; g < nG; ++g) {
    const int ext = matrix_page_extent(Wq, g);
    const size_t c0 = (size_t)g * gw;
    const size_t r0 = (size_t)per * g;
    uint16_t* Qg = otiles ? Q + c0 : Q;
    const uint16_t* page;
    if (g == 0)
      for (int i = 0; i < 4; ++i)
        if ((st = bias.get(i, &bq[i]))) return st;
    // Q_g = x Wq_g^T + bq_g, K_g = src Wk_g^T + bk_g, V_g^T = Wv_g src^T + bv_g
    if ((st = feeder.take(r0, &page)) ||
        (st = project(a, x, M, dm, page, ext, offset(bq[0], c0), Qg, ldq, bbase)) ||
        (st = feeder.give_back(r0)))
      return st;
    if ((st = feeder.take(r0 + 1, &page)) ||
        (st = project(a, src, Ms, dm, page, ext, offset(bq[1], c0), Kb, gw, bbase)) ||
        (st = feeder.give_back(r0 + 1)))
      return st;
    if ((st = feeder.take(r0 + 2, &page)) ||
        (st = project_vt(a, src, Ms, dm, page, ext, offset(bq[2], c0), Vt, ldvt, bbase)) ||
        (st = feeder.give_back(r0 + 2)))
      return st;
    // O_g over Q_g (online softmax, fp32 state)
    if ((st = attend(a, Qg, ldq, Kb, gw, Vt, ldvt, M, Ms, ext / head_dim, head_dim, flags))) return st;
    if (otiles) continue;
    if (ext == gw && (st = probe_commit(a, g, PSI_ROLE_ATTN_O, Q, (size_t)M * gw * 2))) return st;
    if ((st = feeder.take(r0 + 3, &page)) || (g == nG - 1 && (st = fence())) ||
        (st = oproj_ksplit(a, Q, gw, M, dm, page, ext, g == 0, g == nG - 1, acc, bq[3], y, x, flags, bbase)) ||
        (st = feeder.give_back(r0 + 3)))
      return st;
  }
  if (otiles) {
    if ((st = probe_commit(a, -1, PSI_ROLE_ATTN_O, Q, (size_t)M * dm * 2))) return st;
    const size_t r0 = (size_t)per * nG;
    const uint16_t* page;
    for (int o = 0; o < (int)ro.size(); ++o)
      if ((st = feeder.take(r0 + o, &page)) || (o == 0 && (st = fence())) ||
          (st = oproj_tile(a, Q, M, dm, page, matrix_page_extent(Wo, o), (size_t)o * Wo->block, bq[3], y, x,
                           flags, bbase)) ||
          (st = feeder.give_back(r0 + o)))
        return st;
  }
  return bias.release();
}

psi_status psi_attn_paged(psi_arena* a, const uint16_t* x, int M, const uint16_t* ctx, int Mc,
                          int heads, int head_dim, const psi_matrix* Wq, const psi_matrix* Wk,
                          const psi_matrix* Wv, const psi_matrix* Wo, float* acc_dev, uint16_t* y,
                          unsigned flags) {
  return attn_paged(a, x, M, ctx, Mc, heads, head_dim, Wq, Wk, Wv, Wo, acc_dev, y, flags, nullptr);
}

psi_status psi_attn_paged_ext(psi_arena* a, const uint16_t* x, int M, const uint16_t* ctx, int Mc,
                              int heads, int head_dim, const psi_matrix* Wq, const psi_matrix* Wk,
                              const psi_matrix* Wv, const psi_matrix* Wo, const psi_qk_norm_rope* nr,
                              float* acc_dev, uint16_t* y, unsigned flags) {
  if (psi_status st = check_attn_config(flags)) return st;
  if (!qk_stage_active(nr))
    return psi_attn_paged(a, x, M, ctx, Mc, heads, head_dim, Wq, Wk, Wv, Wo, acc_dev, y, flags);
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (ctx && Mc < 1) return fail(PSI_E_INVALID, "attention: cross-attention needs Mc >= 1 keys");
  if (!ctx) Mc = 0;
  psi_status st = psi_attn_ext_plan(&a->desc, M, Mc, heads, head_dim, Wq, Wk, Wv, Wo, nr,
                                    acc_dev != nullptr, nullptr);
  if (st) return st;
  const bool otiles = Wo->split == PSI_SPLIT_ROWS;
  if ((flags & PSI_OP_STORE_ACC) && (!acc_dev || otiles))
    return fail(PSI_E_INVALID, "PSI_OP_STORE_ACC needs acc_dev and a column-split Wo");
  if ((st = check_attn_args(a, x, y, ctx, acc_dev, Wq, Wk, Wv, Wo))) return st;
  if (!a->dry) {
    for (const uint16_t* g : {nr->gamma_q, nr->gamma_k}) {
      if (!g) continue;
      if ((st = Wq->resident ? check_ptr(g, "gamma") : check_pinned(g, "gamma"))) return st;
    }
  }
  const int dm = heads * head_dim;
  if ((st = check_alias(x, (size_t)M * dm * 2, y, (size_t)M * dm * 2, true, "attention"))) return st;
  if (M == 0) return PSI_OK;
  const int gw = Wq->block;
  const uint16_t* src = ctx ? ctx : x;
  const int Ms = ctx ? Mc : M;
  const long ldvt = (long)align_up((size_t)Ms, 64);
  const int bbase = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
  ScratchMark mark(a);
  uint16_t* Q = static_cast<uint16_t*>(scratch_alloc(a, (size_t)M * dm * 2, &st));
  if (st) return st;
  uint16_t* Kb = static_cast<uint16_t*>(scratch_alloc(a, (size_t)Ms * dm * 2, &st));
  if (st) return st;
  uint16_t* Vt = static_cast<uint16_t*>(scratch_alloc(a, (size_t)gw * ldvt * 2, &st));
  if (st) return st;
  float* acc = acc_dev;
  if (!acc && !otiles) {
    acc = static_cast<float*>(scratch_alloc(a, (size_t)M * dm * 4, &st));
    if (st) return st;
  }
  const psi_matrix* ms[4] = {Wq, Wk, Wv, Wo};
  const BiasPart gam[2] = {{nr->gamma_q, nr->gamma_q ? (size_t)dm * 2 : 0},
                           {nr->gamma_k, nr->gamma_k ? (size_t)dm * 2 : 0}};
  OpBiases bias;
  if ((st = bias.stage(a, ms, 4, gam, 2, Wq->resident != 0))) return st;
  // pages: Wq_g, Wk_g for every group, then Wv_g (, Wo[:, g]) for every
  // group; output tiles Wo_o last
  std::vector<PageReq> rq, rk, rv, ro, reqs;
  matrix_requests(Wq, rq);
  matrix_requests(Wk, rk);
  matrix_requests(Wv, rv);
  matrix_requests(Wo, ro);
  const int nG = (int)rq.size();
  const int per = otiles ? 1 : 2;
  for (int g = 0; g < nG; ++g) {
    reqs.push_back(rq[g]);
    reqs.push_back(rk[g]);
  }
  for (int g = 0; g < nG; ++g) {
    reqs.push_back(rv[g]);
    if (!otiles) reqs.push_back(ro[g]);
  }
  if (otiles) reqs.insert(reqs.end(), ro.begin(), ro.end());
  LentSlots lent(a);
  PageFeeder feeder(a, reqs);
  if ((st = feeder.feed())) return st;
  const uint16_t* bq[6];
  for (int i = 0; i < 6; ++i)
    if ((st = bias.get(i, &bq[i]))) return st;
  const uint16_t* page;
  // Q[:, g] = x Wq_g^T + bq_g and K[:, g] = src Wk_g^T + bk_g for all groups
  for (int g = 0; g < nG; ++g) {
    const int ext = matrix_page_extent(Wq, g);
    const size_t c0 = (size_t)g * gw;
    if ((st = feeder.take(2 * g, &page)) ||
        (st = project(a, x, M, dm, page, ext, offset(bq[0], c0), Q + c0, dm, bbase)) ||
        (st = feeder.give_back(2 * g)))
      return st;
    if ((st = feeder.take(2 * g + 1, &page)) ||
        (st = project(a, src, Ms, dm, page, ext, offset(bq[1], c0), Kb + c0, dm, bbase)) ||
        (st = feeder.give_back(2 * g + 1)))
      return st;
  }
  // full-row RMS and split RoPE, in place
  {
    NormRopeArgs N{};
    N.x = Q; N.ldx = dm; N.M = M; N.d = dm; N.dh = head_dim;
    N.gamma = bq[4]; N.eps = nr->eps; N.tile = nr->norm_tile > 0 ? nr->norm_tile : gw;
    N.cs = nr->cos_q; N.sn = nr->sin_q;
    if ((nr->gamma_q || nr->cos_q) && (st = run_norm_rope(a, N))) return st;
    N.x = Kb; N.M = Ms; N.gamma = bq[5];
    N.cs = nr->cos_k ? nr->cos_k : nr->cos_q;
    N.sn = nr->cos_k ? nr->sin_k : nr->sin_q;
    if ((nr->gamma_k || nr->cos_q) && (st = run_norm_rope(a, N))) return st;
  }
  const size_t base = 2 * (size_t)nG;
  for (int g = 0; g < nG; ++g) {
    const int ext = matrix_page_extent(Wq, g);
    const size_t c0 = (size_t)g * gw;
    const size_t r0 = base + (size_t)per * g;
    // V_g^T = Wv_g src^T + bv_g, then O_g over Q[:, g] in place
    if ((st = feeder.take(r0, &page)) ||
        (st = project_vt(a, src, Ms, dm, page, ext, offset(bq[2], c0), Vt, ldvt, bbase)) ||
        (st = feeder.give_back(r0)))
      return st;
    if ((st = attend(a, Q + c0, dm, Kb + c0, dm, Vt, ldvt, M, Ms, ext / head_dim, head_dim, flags))) return st;
    if (otiles) continue;
    if ((st = feeder.take(r0 + 1, &page)) ||
        (st = oproj_ksplit(a, Q + c0, dm, M, dm, page, ext, g == 0, g == nG - 1, acc, bq[3], y, x, flags,
                           bbase)) ||
        (st = feeder.give_back(r0 + 1)))
      return st;
  }
  if (otiles) {
    const size_t r0 = base + (size_t)per * nG;
    for (int o = 0; o < (int)ro.size(); ++o)
      if ((st = feeder.take(r0 + o, &page)) ||
          (st = oproj_tile(a, Q, M, dm, page, matrix_page_extent(Wo, o), (size_t)o * Wo->block, bq[3], y, x,
                           flags, bbase)) ||
          (st = feeder.give_back(r0 + o)))
        return st;
  }
  return bias.release();
}

psi_status psi_attn_tiled(psi_arena* a, const uint16_t* x, int M, const uint16_t* ctx, int Mc, int heads,
                          int head_dim, const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                          const psi_matrix* Wo, psi_journal* j, int32_t step, int32_t block, uint16_t* y,
                          unsigned flags) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (psi_status st = check_attn_config(flags)) return st;
  if (ctx && Mc < 1) return fail(PSI_E_INVALID, "attention: cross-attention needs Mc >= 1 keys");
  if (!ctx) Mc = 0;
  psi_status st = psi_attn_tiled_plan(&a->desc, M, Mc, heads, head_dim, Wq, Wk, Wv, Wo, nullptr);
  if (st) return st;
  if (!j) return fail(PSI_E_INVALID, "attention tiled: needs a journal for the head-group outputs");
  if (flags & PSI_OP_STORE_ACC) return fail(PSI_E_INVALID, "attention tiled: no full accumulator to store");
  if ((st = check_attn_args(a, x, y, ctx, nullptr, Wq, Wk, Wv, Wo))) return st;
  const int dm = heads * head_dim;
  if ((st = check_alias(x, (size_t)M * dm * 2, y, (size_t)M * dm * 2, true, "attention tiled"))) return st;
  if (M == 0) return PSI_OK;
  const int gw = Wq->block, to = Wo->block;
  const uint16_t* src = ctx ? ctx : x;
  const int Ms = ctx ? Mc : M;
  const long ldvt = (long)align_up((size_t)Ms, 64);
  const int bbase = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
  ScratchMark mark(a);
  uint16_t* Ob[2];  // Q_g, then O_g in place; later the reloaded O_g
  for (int i = 0; i < 2; ++i) {
    Ob[i] = static_cast<uint16_t*>(scratch_alloc(a, (size_t)M * gw * 2, &st));
    if (st) return st;
  }
  const size_t phase_mark = a->scratch_top;
  uint16_t* Kb = static_cast<uint16_t*>(scratch_alloc(a, (size_t)Ms * gw * 2, &st));
  if (st) return st;
  uint16_t* Vt = static_cast<uint16_t*>(scratch_alloc(a, (size_t)gw * ldvt * 2, &st));
  if (st) return st;
  const psi_matrix* ms[4] = {Wq, Wk, Wv, Wo};
  OpBiases bias;
  if ((st = bias.stage(a, ms, 4))) return st;
  std::vector<PageReq> rq, rk, rv, ro, reqs;
  matrix_requests(Wq, rq);
  matrix_requests(Wk, rk);
  matrix_requests(Wv, rv);
  matrix_requests(Wo, ro);
  const int nG = (int)rq.size(), nP = (int)ro.size();
  for (int g = 0; g < nG; ++g) {
    reqs.push_back(rq[g]);
    reqs.push_back(rk[g]);
    reqs.push_back(rv[g]);
  }
  reqs.insert(reqs.end(), ro.begin(), ro.end());
  PageFeeder feeder(a, reqs);
  if ((st = feeder.feed())) return st;
  const uint16_t* bq[4];
  for (int i = 0; i < 4; ++i)
    if ((st = bias.get(i, &bq[i]))) return st;
  hipEvent_t* rd = a->pipe_ev;
  hipEvent_t* ld = a->pipe_ev + 2;
  auto okey = [&](int g) { return psi_key{step, block, g, PSI_ROLE_ATTN_OSTATE}; };
  auto obytes = [&](int g) { return (size_t)M * matrix_page_extent(Wq, g) * 2; };
  const uint16_t* page;
  // per head group: Q_g, K_g, V_g^T, attention; O_g (compact [M, e_g]) to the journal
  for (int g = 0; g < nG; ++g) {
    const int ext = matrix_page_extent(Wq, g);
    const size_t c0 = (size_t)g * gw;
    uint16_t* Q = Ob[g % 2];
    if (!a->dry && g >= 2) PSI_HIP(hipStreamWaitEvent(a->compute, rd[g % 2], 0));
    if ((st = feeder.take(3 * g, &page)) ||
        (st = project(a, x, M, dm, page, ext, offset(bq[0], c0), Q, ext, bbase)) ||
        (st = feeder.give_back(3 * g)))
      return st;
    if ((st = feeder.take(3 * g + 1, &page)) ||
        (st = project(a, src, Ms, dm, page, ext, offset(bq[1], c0), Kb, ext, bbase)) ||
        (st = feeder.give_back(3 * g + 1)))
      return st;
    if ((st = feeder.take(3 * g + 2, &page)) ||
        (st = project_vt(a, src, Ms, dm, page, ext, offset(bq[2], c0), Vt, ldvt, bbase)) ||
        (st = feeder.give_back(3 * g + 2)))
      return st;
    if ((st = attend(a, Q, ext, Kb, ext, Vt, ldvt, M, Ms, ext / head_dim, head_dim, flags))) return st;
    if (ext == gw && (st = probe_commit(a, g, PSI_ROLE_ATTN_O, Q, obytes(g)))) return st;
    if (!a->dry && (st = journal_commit_ev(j, okey(g), Q, obytes(g), a->compute, rd[g % 2]))) return st;
  }
  // per output tile o (rows of Wo: one page, or several pages of whole head
  // groups with 2-D page tiles): ACC_o = sum over g ascending of
  // O_g Wo[o, g]^T, then y[:, o] = B(ACC_o + bo_o) (+ x[:, o]); O_g reloads
  // alternate buffers
  scratch_reset(a, phase_mark);
  float* acc = static_cast<float*>(scratch_alloc(a, (size_t)M * to * 4, &st));
  if (st) return st;
  auto g_first = [&](int p) { return matrix_page_col0(Wo, p) / gw; };
  auto g_end = [&](int p) { return (matrix_page_col0(Wo, p) + matrix_page_cols(Wo, p) + gw - 1) / gw; };
  std::vector<int> step_g;
  for (int p = 0; p < nP; ++p)
    for (int g = g_first(p); g < g_end(p); ++g) step_g.push_back(g);
  const int T = (int)step_g.size();
  auto issue = [&](int t) -> psi_status {
    const int g = step_g[t];
    return journal_reload_ev(j, okey(g), Ob[t % 2], obytes(g), a->compute, ld[t % 2]);
  };
  if (!a->dry && (st = issue(0))) return st;
  int t = 0;
  for (int p = 0; p < nP; ++p) {
    const int eo = matrix_page_extent(Wo, p);
    const size_t c0 = (size_t)matrix_page_row0(Wo, p);
    if ((st = feeder.take(3 * nG + p, &page))) return st;
    for (int g = g_first(p); g < g_end(p); ++g, ++t) {
      const int ext = matrix_page_extent(Wq, g);
      if (!a->dry) {
        if (t + 1 < T && (st = issue(t + 1))) return st;
        PSI_HIP(hipStreamWaitEvent(a->compute, ld[t % 2], 0));
      }
      GemmArgs G = gemm_args();
      G.A = Ob[t % 2]; G.lda = ext;
      G.B = page + ((size_t)g * gw - matrix_page_col0(Wo, p)); G.ldb = matrix_page_cols(Wo, p);
      G.M = M; G.N = eo; G.K = ext;
      G.baseline_bias = bbase;
      if (g > 0) { G.acc_in = acc; G.ld_acc_in = eo; }
      if (g == nG - 1) {
        G.bias = bq[3] ? bq[3] + c0 : nullptr; G.out = y + c0; G.ldo = dm;
        if (flags & PSI_OP_RESIDUAL) { G.resid = x + c0; G.ldr = dm; }
      } else {
        G.epi = EPI_ACC; G.acc_out = acc; G.ld_acc_out = eo;
      }
      if ((st = run_gemm(a, G))) return st;
    }
    if ((st = feeder.give_back(3 * nG + p))) return st;
  }
  return bias.release();
}

psi_status psi_block_lowlive(psi_arena* a, uint16_t* x, int M, int heads, int head_dim,
                             const psi_block_weights* w, psi_journal* j, unsigned flags) {
  if (!a || !w || !j) return fail(PSI_E_INVALID, "null argument");
  if (psi_status st = check_attn_config(flags)) return st;
  const unsigned f = (flags & (PSI_OP_BASELINE_BIAS | PSI_OP_BF16_SOFTMAX | PSI_OP_ATTN_P2 | PSI_OP_ATTN_CONFIG_MASK)) |
                     PSI_OP_RESIDUAL;
  const int dm = heads * head_dim;
  psi_status st = psi_attn_tiled_plan(&a->desc, M, 0, heads, head_dim, &w->Wq, &w->Wk, &w->Wv, &w->Wo, nullptr);
  if (st) return st;
  if ((st = psi_ffn_tiled_plan(&a->desc, M, dm, &w->U, &w->V, PSI_FFN_REUSE, nullptr))) return st;
  if (!a->dry && (st = psi_journal_reset(j))) return st;
  if ((st = psi_attn_tiled(a, x, M, nullptr, 0, heads, head_dim, &w->Wq, &w->Wk, &w->Wv, &w->Wo, j, 0, 0, x, f)))
    return st;
  return psi_ffn_tiled(a, x, M, dm, &w->U, &w->V, PSI_FFN_REUSE, j, 0, 1, x, f & ~PSI_OP_BF16_SOFTMAX);
}

psi_status psi_block_paged(psi_arena* a, uint16_t* x, uint16_t* xt, int M, int heads, int head_dim,
                           const psi_block_weights* w, int token_chunks, float* acc_dev,
                           psi_journal* fence, unsigned flags) {
  if (!a || !w) return fail(PSI_E_INVALID, "null argument");
  if (psi_status st = check_attn_config(flags)) return st;
  const unsigned f = (flags & (PSI_OP_BASELINE_BIAS | PSI_OP_BF16_SOFTMAX | PSI_OP_ATTN_P2 | PSI_OP_ATTN_CONFIG_MASK)) |
                     PSI_OP_RESIDUAL;
  // validate both halves before enqueueing anything
  const int dm = heads * head_dim;
  psi_status st = psi_attn_plan(&a->desc, M, 0, heads, head_dim, &w->Wq, &w->Wk, &w->Wv, &w->Wo,
                                acc_dev != nullptr, nullptr);
  if (st) return st;
  if ((st = psi_ffn_plan(&a->desc, M, dm, &w->U, &w->V, token_chunks, acc_dev != nullptr, nullptr)))
    return st;
  const size_t xbytes = (size_t)M * dm * 2;
  if (xt && xt != x && (st = check_alias(x, xbytes, xt, xbytes, false, "block x_tmp"))) return st;
  // The FFN's first pages are copied while the attention sub-block's last
  // kernels run (PageFeeder lookahead).
  const std::vector<PageReq> ffn_reqs = ffn_requests(&w->U, &w->V);
  const bool inplace = !xt || xt == x;
  // In place, the attention sub-block's output tiles write x after its last
  // read of x, and the FFN's last down-projection writes each row after
  // every read of that row; the journal's reads of x's previous contents
  // precede the attention's first write.
  st = attn_paged(a, x, M, nullptr, 0, heads, head_dim, &w->Wq, &w->Wk, &w->Wv, &w->Wo, acc_dev, inplace ? x : xt,
                  f, inplace ? fence : nullptr, &ffn_reqs);
  if (!st)
    st = inplace ? ffn_paged(a, x, M, dm, &w->U, &w->V, token_chunks, acc_dev, x, f, nullptr)
                 : ffn_paged(a, xt, M, dm, &w->U, &w->V, token_chunks, acc_dev, x, f, fence);
  if (st && !a->ahead.empty()) (void)drop_ahead(a);  // the error is the one to report
  return st;
}

}  // extern "C"
