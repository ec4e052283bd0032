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

// One weight-page request of an operator, in consumption order.
struct PageReq {
  const void* host;  // device address when `resident`
  size_t bytes;
  const void* side;
  size_t side_bytes;
  bool resident;
};

// Page requests of a matrix: ROWS pages carry their bias slice; a COLS
// (K-split) matrix carries its whole bias on the last page, because the
// bias is added once after the last partial sum ([PSI] sec. II-B).
void matrix_requests(const psi_matrix* m, std::vector<PageReq>& out) {
  const int n = psi_matrix_pages(m);
  for (int p = 0; p < n; ++p) {
    PageReq r{matrix_page_ptr(m, p), psi_matrix_page_bytes(m, p), nullptr, 0, m->resident != 0};
    if (m->bias_host) {
      if (m->split == PSI_SPLIT_ROWS) {
        r.side = m->bias_host + (size_t)p * m->block;
        r.side_bytes = (size_t)matrix_page_extent(m, p) * 2;
      } else if (p == n - 1) {
        r.side = m->bias_host;
        r.side_bytes = (size_t)m->rows * 2;
      }
    }
    out.push_back(r);
  }
}

// Streams a list of page requests through the arena's slots: requests are
// submitted as soon as their (round-robin) slot is free, so the copy of the
// next pages overlaps the consumers of the current one; with two slots this
// is the paper's two alternating pages ([PSI] sec. III-B weight prefetch).
class PageFeeder {
 public:
  PageFeeder(psi_arena* a, std::vector<PageReq> reqs) : a_(a), reqs_(std::move(reqs)), slot_(reqs_.size(), -1) {}

  psi_status feed() {
    while (submitted_ < reqs_.size()) {
      const PageReq& r = reqs_[submitted_];
      if (r.resident) {  // consumed in place: no copy, no slot
        ++submitted_;
        continue;
      }
      if (a_->slots[a_->next_slot].state != psi_page_slot::FREE) break;
      int s = -1;
      psi_status st = page_submit_ex(a_, r.host, r.bytes, r.side, r.side_bytes, &s, false);
      if (st) return st;
      slot_[submitted_++] = s;
    }
    return PSI_OK;
  }
  // Waits (on the compute stream) for request i and returns its page/side.
  psi_status take(size_t i, const uint16_t** page, const uint16_t** side) {
    psi_status st = feed();
    if (st) return st;
    const PageReq& r = reqs_[i];
    if (r.resident) {
      *page = static_cast<const uint16_t*>(r.host);
      *side = static_cast<const uint16_t*>(r.side);
      return PSI_OK;
    }
    if (i >= submitted_) return fail(PSI_E_STATE, "page request not submitted (slots exhausted)");
    st = page_acquire(a_, slot_[i]);
    if (st) return st;
    *page = static_cast<const uint16_t*>(a_->dry ? nullptr : a_->slots[slot_[i]].dev);
    *side = r.side ? static_cast<const uint16_t*>(a_->dry ? nullptr : a_->slots[slot_[i]].side_dev)
                   : nullptr;
    return PSI_OK;
  }
  psi_status give_back(size_t i) {
    if (!reqs_[i].resident) {
      psi_status st = page_release(a_, slot_[i]);
      if (st) return st;
    }
    return feed();
  }

 private:
  psi_arena* a_;
  std::vector<PageReq> reqs_;
  std::vector<int> slot_;
  size_t submitted_ = 0;
};

psi_status check_ptr(const void* p, const char* what, bool allow_null = false) {
  if (!p) return allow_null ? PSI_OK : fail(PSI_E_INVALID, std::string(what) + " is null");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(PSI_E_ALIGN, std::string(what) + " must be 16-byte aligned");
  return PSI_OK;
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

GemmArgs gemm_args() {
  GemmArgs g{};
  g.epi = EPI_BIAS;
  return g;
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
  std::vector<PageReq> reqs;
  matrix_requests(W, reqs);
  PageFeeder feeder(a, reqs);
  if ((st = feeder.feed())) return st;
  const int n = (int)reqs.size();
  for (int p = 0; p < n; ++p) {
    const uint16_t *page, *side;
    if ((st = feeder.take(p, &page, &side))) return st;
    const int ext = matrix_page_extent(W, p);
    GemmArgs g = gemm_args();
    g.M = M;
    g.baseline_bias = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
    if (W->split == PSI_SPLIT_ROWS) {
      const int c0 = p * W->block;
      g.A = x; g.lda = K;
      g.B = page; g.ldb = K;
      g.N = ext; g.K = K;
      g.bias = side;
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
        g.bias = side;
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
  return PSI_OK;
}

psi_status psi_ffn_paged(psi_arena* a, const uint16_t* x, int M, int d, const psi_matrix* U,
                         const psi_matrix* V, int token_chunks, float* acc_dev, uint16_t* y,
                         unsigned flags) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  size_t need = 0;
  psi_status st = psi_ffn_plan(&a->desc, M, d, U, V, token_chunks, acc_dev != nullptr, &need);
  if (st) return st;
  if ((flags & PSI_OP_STORE_ACC) && !acc_dev) return fail(PSI_E_INVALID, "PSI_OP_STORE_ACC needs acc_dev");
  if (!a->dry) {
    if ((st = check_ptr(x, "x")) || (st = check_ptr(y, "y")) || (st = check_ptr(acc_dev, "acc", true)))
      return st;
    if (d % 8 != 0) return fail(PSI_E_ALIGN, "d must be a multiple of 8");
    if ((st = check_matrix_pinned(a, U, "U")) || (st = check_matrix_pinned(a, V, "V"))) return st;
  }
  if (M == 0) return PSI_OK;
  const bool resid = flags & PSI_OP_RESIDUAL;
  const int th = U->block;
  ScratchMark mark(a);
  uint16_t* H = static_cast<uint16_t*>(scratch_alloc(a, (size_t)M * th * 2, &st));
  if (st) return st;
  float* acc = acc_dev;
  if (!acc) {
    acc = static_cast<float*>(scratch_alloc(a, (size_t)M * d * 4, &st));
    if (st) return st;
  }
  // Request order U_0, V_0, U_1, V_1, ...: each hidden tile J is produced
  // for all tokens from U_J, then consumed by V_J ([PSI] eq. (2)).
  std::vector<PageReq> ru, rv, reqs;
  matrix_requests(U, ru);
  matrix_requests(V, rv);
  const int nJ = (int)ru.size();
  for (int J = 0; J < nJ; ++J) {
    reqs.push_back(ru[J]);
    reqs.push_back(rv[J]);
  }
  const int chunks = token_chunks > M ? M : token_chunks;
  const int rows_per = (M + chunks - 1) / chunks;
  PageFeeder feeder(a, reqs);
  if ((st = feeder.feed())) return st;
  for (int J = 0; J < nJ; ++J) {
    const int ext = matrix_page_extent(U, J);
    const bool last = J == nJ - 1;
    const uint16_t *page, *side;
    // up-projection + bias + BF16 + GELU + BF16 for every token chunk
    if ((st = feeder.take(2 * J, &page, &side))) return st;
    for (int r0 = 0; r0 < M; r0 += rows_per) {
      const int mr = M - r0 < rows_per ? M - r0 : rows_per;
      GemmArgs g = gemm_args();
      g.A = x + (size_t)r0 * d; g.lda = d;
      g.B = page; g.ldb = d;
      g.M = mr; g.N = ext; g.K = d;
      g.bias = side;
      g.out = H + (size_t)r0 * th; g.ldo = th;
      g.epi = EPI_GELU;
      g.baseline_bias = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
      if ((st = run_gemm(a, g))) return st;
    }
    if ((st = feeder.give_back(2 * J))) return st;
    // down-projection: carried fp32 accumulator, bias once after the last tile
    if ((st = feeder.take(2 * J + 1, &page, &side))) return st;
    for (int r0 = 0; r0 < M; r0 += rows_per) {
      const int mr = M - r0 < rows_per ? M - r0 : rows_per;
      GemmArgs g = gemm_args();
      g.A = H + (size_t)r0 * th; g.lda = th;
      g.B = page; g.ldb = ext;
      g.M = mr; g.N = d; g.K = ext;
      if (J > 0) { g.acc_in = acc + (size_t)r0 * d; g.ld_acc_in = d; }
      if (last) {
        g.bias = side;
        g.out = y + (size_t)r0 * d; g.ldo = d;
        if (resid) { g.resid = x + (size_t)r0 * d; g.ldr = d; }
        if (flags & PSI_OP_STORE_ACC) { g.acc_out = acc + (size_t)r0 * d; g.ld_acc_out = d; }
      } else {
        g.epi = EPI_ACC;
        g.acc_out = acc + (size_t)r0 * d; g.ld_acc_out = d;
      }
      if ((st = run_gemm(a, g))) return st;
    }
    if ((st = feeder.give_back(2 * J + 1))) return st;
  }
  return PSI_OK;
}

psi_status psi_attn_paged(psi_arena* a, const uint16_t* x, int M, const uint16_t* ctx, int Mc,
                          int heads, int head_dim, const psi_matrix* Wq, const psi_matrix* Wk,
                          const psi_matrix* Wv, const psi_matrix* Wo, float* acc_dev, uint16_t* y,
                          unsigned flags) {
  if (!a) return fail(PSI_E_INVALID, "null arena");
  if (ctx && Mc < 1) return fail(PSI_E_INVALID, "attention: cross-attention needs Mc >= 1 keys");
  if (!ctx) Mc = 0;
  size_t need = 0;
  psi_status st = psi_attn_plan(&a->desc, M, Mc, heads, head_dim, Wq, Wk, Wv, Wo, acc_dev != nullptr, &need);
  if (st) return st;
  if ((flags & PSI_OP_STORE_ACC) && !acc_dev) return fail(PSI_E_INVALID, "PSI_OP_STORE_ACC needs acc_dev");
  if (!a->dry) {
    if ((st = check_ptr(x, "x")) || (st = check_ptr(y, "y")) || (st = check_ptr(ctx, "ctx", true)) ||
        (st = check_ptr(acc_dev, "acc", true)))
      return st;
    if ((st = check_matrix_pinned(a, Wq, "Wq")) || (st = check_matrix_pinned(a, Wk, "Wk")) ||
        (st = check_matrix_pinned(a, Wv, "Wv")) || (st = check_matrix_pinned(a, Wo, "Wo")))
      return st;
  }
  if (M == 0) return PSI_OK;
  const int dm = heads * head_dim;
  const int gw = Wq->block;
  const uint16_t* src = ctx ? ctx : x;
  const int Ms = ctx ? Mc : M;
  const long ldvt = (long)align_up((size_t)Ms, 64);
  const int bb = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
  ScratchMark mark(a);
  uint16_t* Q = static_cast<uint16_t*>(scratch_alloc(a, (size_t)M * gw * 2, &st));
  if (st) return st;
  uint16_t* Kb = static_cast<uint16_t*>(scratch_alloc(a, (size_t)Ms * gw * 2, &st));
  if (st) return st;
  uint16_t* Vt = static_cast<uint16_t*>(scratch_alloc(a, (size_t)gw * ldvt * 2, &st));
  if (st) return st;
  float* acc = acc_dev;
  if (!acc) {
    acc = static_cast<float*>(scratch_alloc(a, (size_t)M * dm * 4, &st));
    if (st) return st;
  }
  std::vector<PageReq> rq, rk, rv, ro, reqs;
  matrix_requests(Wq, rq);
  matrix_requests(Wk, rk);
  matrix_requests(Wv, rv);
  matrix_requests(Wo, ro);
  const int nG = (int)rq.size();
  for (int g = 0; g < nG; ++g) {
    reqs.push_back(rq[g]);
    reqs.push_back(rk[g]);
    reqs.push_back(rv[g]);
    reqs.push_back(ro[g]);
  }
  const float alpha = (float)(1.0 / std::sqrt((double)head_dim));
  PageFeeder feeder(a, reqs);
  if ((st = feeder.feed())) return st;
  for (int g = 0; g < nG; ++g) {
    const int ext = matrix_page_extent(Wq, g);
    const bool last = g == nG - 1;
    const uint16_t *page, *side;
    // Q_g = x Wq_g^T + bq_g
    if ((st = feeder.take(4 * g, &page, &side))) return st;
    {
      GemmArgs G = gemm_args();
      G.A = x; G.lda = dm; G.B = page; G.ldb = dm;
      G.M = M; G.N = ext; G.K = dm;
      G.bias = side; G.out = Q; G.ldo = gw; G.baseline_bias = bb;
      if ((st = run_gemm(a, G))) return st;
    }
    if ((st = feeder.give_back(4 * g))) return st;
    // K_g = src Wk_g^T + bk_g
    if ((st = feeder.take(4 * g + 1, &page, &side))) return st;
    {
      GemmArgs G = gemm_args();
      G.A = src; G.lda = dm; G.B = page; G.ldb = dm;
      G.M = Ms; G.N = ext; G.K = dm;
      G.bias = side; G.out = Kb; G.ldo = gw; G.baseline_bias = bb;
      if ((st = run_gemm(a, G))) return st;
    }
    if ((st = feeder.give_back(4 * g + 1))) return st;
    // V_g^T = Wv_g src^T + bv_g (bias along rows): written transposed
    if ((st = feeder.take(4 * g + 2, &page, &side))) return st;
    {
      GemmArgs G = gemm_args();
      G.A = page; G.lda = dm; G.B = src; G.ldb = dm;
      G.M = ext; G.N = Ms; G.K = dm;
      G.bias = side; G.bias_on_m = 1; G.out = Vt; G.ldo = ldvt; G.baseline_bias = bb;
      if ((st = run_gemm(a, G))) return st;
    }
    if ((st = feeder.give_back(4 * g + 2))) return st;
    // O_g over Q_g (online softmax, fp32 state)
    {
      AttnArgs A{};
      A.q = Q; A.ldq = gw;
      A.k = Kb; A.ldk = gw;
      A.vt = Vt; A.ldvt = ldvt;
      A.Mq = M; A.Mk = Ms; A.heads = ext / head_dim;
      A.alpha = alpha;
      A.bf16_p = (flags & PSI_OP_BF16_SOFTMAX) ? 1 : 0;
      if ((st = run_attention(a, A))) return st;
    }
    // ACC (+)= O_g Wo[:, g]^T; after the last group y = B(ACC + bo) (+ x)
    if ((st = feeder.take(4 * g + 3, &page, &side))) return st;
    {
      GemmArgs G = gemm_args();
      G.A = Q; G.lda = gw; G.B = page; G.ldb = ext;
      G.M = M; G.N = dm; G.K = ext;
      G.baseline_bias = bb;
      if (g > 0) { G.acc_in = acc; G.ld_acc_in = dm; }
      if (last) {
        G.bias = side; G.out = y; G.ldo = dm;
        if (flags & PSI_OP_RESIDUAL) { G.resid = x; G.ldr = dm; }
        if (flags & PSI_OP_STORE_ACC) { G.acc_out = acc; G.ld_acc_out = dm; }
      } else {
        G.epi = EPI_ACC; G.acc_out = acc; G.ld_acc_out = dm;
      }
      if ((st = run_gemm(a, G))) return st;
    }
    if ((st = feeder.give_back(4 * g + 3))) return st;
  }
  return PSI_OK;
}

psi_status psi_journal_fence(psi_journal* j, void* stream);

psi_status psi_block_paged(psi_arena* a, uint16_t* x, uint16_t* xt, int M, int heads, int head_dim,
                           const psi_block_weights* w, int token_chunks, float* acc_dev,
                           psi_journal* fence, unsigned flags) {
  if (!a || !w) return fail(PSI_E_INVALID, "null argument");
  if (x == xt && M > 0) return fail(PSI_E_INVALID, "block: x_tmp must be a separate buffer");
  const unsigned f = (flags & (PSI_OP_BASELINE_BIAS | PSI_OP_BF16_SOFTMAX)) | PSI_OP_RESIDUAL;
  // validate both halves before enqueueing anything
  const int dm = heads * head_dim;
  psi_status st = psi_attn_plan(&a->desc, M, 0, heads, head_dim, &w->Wq, &w->Wk, &w->Wv, &w->Wo,
                                acc_dev != nullptr, nullptr);
  if (st) return st;
  if ((st = psi_ffn_plan(&a->desc, M, dm, &w->U, &w->V, token_chunks, acc_dev != nullptr, nullptr)))
    return st;
  if ((st = psi_attn_paged(a, x, M, nullptr, 0, heads, head_dim, &w->Wq, &w->Wk, &w->Wv, &w->Wo,
                           acc_dev, xt, f)))
    return st;
  if (fence && !a->dry && (st = psi_journal_fence(fence, a->compute))) return st;
  return psi_ffn_paged(a, xt, M, dm, &w->U, &w->V, token_chunks, acc_dev, x, f);
}

}  // extern "C"
