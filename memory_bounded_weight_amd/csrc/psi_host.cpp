// psi_host.cpp -- host-only parts of the runtime: error reporting, page-image
// packing, arena carve and operator feasibility plans.  Nothing here touches
// the device, so all of it runs (and is tested) without a GPU.
//
// [PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint
// Audio-Video Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
#include <cstring>
#include <string>

#include "psi_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace psi {

psi_status fail(psi_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

psi_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return PSI_E_HIP;
}

psi_status check_matrix(const psi_matrix* m, const char* name, int expect_split) {
  if (!m) return fail(PSI_E_INVALID, std::string(name) + ": null matrix");
  if (m->rows <= 0 || m->cols <= 0 || m->block <= 0)
    return fail(PSI_E_INVALID, std::string(name) + ": non-positive rows/cols/block");
  if (m->split != PSI_SPLIT_ROWS && m->split != PSI_SPLIT_COLS && m->split != PSI_SPLIT_TILES)
    return fail(PSI_E_INVALID, std::string(name) + ": unknown split");
  if (expect_split == kSplitOutputTiles) {
    if (m->split == PSI_SPLIT_COLS)
      return fail(PSI_E_INVALID, std::string(name) + ": must be split into output tiles (by rows or 2-D tiles)");
  } else if (m->split == PSI_SPLIT_TILES) {
    return fail(PSI_E_INVALID, std::string(name) + ": 2-D page tiles serve only the output-tile schedules");
  } else if (expect_split >= 0 && m->split != expect_split) {
    return fail(PSI_E_INVALID, std::string(name) + (expect_split == PSI_SPLIT_ROWS
                                                         ? ": must be split by rows (output columns)"
                                                         : ": must be split by columns (K-split)"));
  }
  if (m->split == PSI_SPLIT_TILES && (m->block_cols <= 0 || m->block_cols % 8 != 0))
    return fail(PSI_E_ALIGN, std::string(name) + ": 2-D page tiles need block_cols a positive multiple of 8");
  if (m->cols % 8 != 0 || (m->split == PSI_SPLIT_COLS && m->block % 8 != 0))
    return fail(PSI_E_ALIGN, std::string(name) + ": K extents must be multiples of 8 (16-byte rows)");
  if (!m->pages_host) return fail(PSI_E_INVALID, std::string(name) + ": null page image");
  return PSI_OK;
}

// Column blocks per row tile of a TILES matrix (1 otherwise).
static int tile_cols_per_row(const psi_matrix* m) {
  return m->split == PSI_SPLIT_TILES ? (m->cols + m->block_cols - 1) / m->block_cols : 1;
}

int matrix_page_cols(const psi_matrix* m, int p) {
  if (m->split == PSI_SPLIT_ROWS) return m->cols;
  if (m->split == PSI_SPLIT_COLS) return matrix_page_extent(m, p);
  const int q = p % tile_cols_per_row(m);
  const int ext = m->cols - q * m->block_cols;
  return ext < m->block_cols ? ext : m->block_cols;
}

int matrix_page_col0(const psi_matrix* m, int p) {
  if (m->split == PSI_SPLIT_ROWS) return 0;
  if (m->split == PSI_SPLIT_COLS) return p * m->block;
  return (p % tile_cols_per_row(m)) * m->block_cols;
}

int matrix_page_row0(const psi_matrix* m, int p) {
  if (m->split == PSI_SPLIT_COLS) return 0;
  return (p / tile_cols_per_row(m)) * m->block;
}

psi_status check_ptr(const void* p, const char* what, bool allow_null) {
  if (!p) return allow_null ? PSI_OK : fail(PSI_E_INVALID, std::string(what) + " is null");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(PSI_E_ALIGN, std::string(what) + " must be 16-byte aligned");
  return PSI_OK;
}

psi_status check_alias(const void* x, size_t xbytes, const void* y, size_t ybytes, bool allow_same,
                       const char* op) {
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), y0 = reinterpret_cast<uintptr_t>(y);
  if (!x || !y || xbytes == 0 || ybytes == 0) return PSI_OK;
  if (x0 + xbytes <= y0 || y0 + ybytes <= x0) return PSI_OK;
  if (allow_same && x0 == y0 && xbytes == ybytes) return PSI_OK;
  return fail(PSI_E_INVALID, std::string(op) + (allow_same ? ": y must be x itself or not overlap it"
                                                           : ": y must not overlap x"));
}

int matrix_page_extent(const psi_matrix* m, int p) {
  if (m->split == PSI_SPLIT_TILES) p /= tile_cols_per_row(m);  // row tile of page p
  int total = m->split == PSI_SPLIT_COLS ? m->cols : m->rows;
  int start = p * m->block;
  int ext = total - start;
  return ext < m->block ? ext : m->block;
}

MatrixInfo matrix_info(const psi_matrix* m) {
  MatrixInfo mi;
  if (m->split == PSI_SPLIT_TILES) {
    const int nq = tile_cols_per_row(m);
    mi.pages = (m->rows + m->block - 1) / m->block * nq;
    mi.max_page_bytes = (size_t)(m->block < m->rows ? m->block : m->rows) *
                        (size_t)(m->block_cols < m->cols ? m->block_cols : m->cols) * 2;
    return mi;
  }
  int total = m->split == PSI_SPLIT_ROWS ? m->rows : m->cols;
  mi.pages = (total + m->block - 1) / m->block;
  size_t other = m->split == PSI_SPLIT_ROWS ? (size_t)m->cols : (size_t)m->rows;
  mi.max_page_bytes = (size_t)(m->block < total ? m->block : total) * other * 2;
  return mi;
}

const void* matrix_page_ptr(const psi_matrix* m, int p) {
  if (m->split == PSI_SPLIT_TILES) {
    const int nq = tile_cols_per_row(m), o = p / nq, q = p % nq;
    const size_t off = (size_t)o * m->block * m->cols + (size_t)matrix_page_extent(m, p) * q * m->block_cols;
    return static_cast<const char*>(m->pages_host) + off * 2;
  }
  size_t other = m->split == PSI_SPLIT_ROWS ? (size_t)m->cols : (size_t)m->rows;
  return static_cast<const char*>(m->pages_host) + (size_t)p * m->block * other * 2;
}

}  // namespace psi

using namespace psi;

extern "C" {

const char* psi_last_error(void) { return g_last_error.c_str(); }

const char* psi_version(void) { return "psi-mi355x 0.1 (gfx950)"; }

psi_status psi_pack_matrix(const uint16_t* W, int rows, int cols, int split, int block, void* dst) {
  if (!W || !dst || rows <= 0 || cols <= 0 || block <= 0)
    return fail(PSI_E_INVALID, "psi_pack_matrix: bad arguments");
  uint16_t* out = static_cast<uint16_t*>(dst);
  if (split == PSI_SPLIT_ROWS) {
    // row blocks of a row-major matrix are already contiguous
    if (out != W) std::memmove(out, W, (size_t)rows * cols * 2);
    return PSI_OK;
  }
  if (split != PSI_SPLIT_COLS) return fail(PSI_E_INVALID, "psi_pack_matrix: unknown split");
  if (out == W) return fail(PSI_E_INVALID, "psi_pack_matrix: column split cannot be packed in place");
  size_t off = 0;
  for (int c0 = 0; c0 < cols; c0 += block) {
    int w = cols - c0 < block ? cols - c0 : block;
    for (int r = 0; r < rows; ++r) {
      std::memcpy(out + off, W + (size_t)r * cols + c0, (size_t)w * 2);
      off += (size_t)w;
    }
  }
  return PSI_OK;
}

psi_status psi_pack_tiles(const uint16_t* W, int rows, int cols, int block_rows, int block_cols, void* dst) {
  if (!W || !dst || rows <= 0 || cols <= 0 || block_rows <= 0 || block_cols <= 0)
    return fail(PSI_E_INVALID, "psi_pack_tiles: bad arguments");
  uint16_t* out = static_cast<uint16_t*>(dst);
  const size_t n = (size_t)rows * cols;
  if (!(out + n <= W || W + n <= out)) return fail(PSI_E_INVALID, "psi_pack_tiles: dst overlaps W");
  size_t off = 0;
  for (int r0 = 0; r0 < rows; r0 += block_rows) {
    const int er = rows - r0 < block_rows ? rows - r0 : block_rows;
    for (int c0 = 0; c0 < cols; c0 += block_cols) {
      const int ec = cols - c0 < block_cols ? cols - c0 : block_cols;
      for (int r = 0; r < er; ++r) {
        std::memcpy(out + off, W + (size_t)(r0 + r) * cols + c0, (size_t)ec * 2);
        off += (size_t)ec;
      }
    }
  }
  return PSI_OK;
}

int psi_matrix_pages(const psi_matrix* m) {
  if (!m || m->block <= 0) return 0;
  return matrix_info(m).pages;
}

size_t psi_matrix_page_bytes(const psi_matrix* m, int p) {
  if (!m || p < 0 || p >= psi_matrix_pages(m)) return 0;
  if (m->split == PSI_SPLIT_TILES) return (size_t)matrix_page_extent(m, p) * matrix_page_cols(m, p) * 2;
  size_t other = m->split == PSI_SPLIT_ROWS ? (size_t)m->cols : (size_t)m->rows;
  return (size_t)matrix_page_extent(m, p) * other * 2;
}

psi_status psi_arena_plan(const psi_arena_desc* d, psi_arena_layout* out) {
  if (!d || !out) return fail(PSI_E_INVALID, "psi_arena_plan: null argument");
  if (d->n_pages < 1 || d->n_pages > PSI_MAX_PAGES)
    return fail(PSI_E_INVALID, "psi_arena_plan: n_pages must be 1.." + std::to_string(PSI_MAX_PAGES));
  if (d->page_bytes == 0 || d->arena_bytes == 0)
    return fail(PSI_E_INVALID, "psi_arena_plan: zero arena or page size");
  psi_arena_layout L;
  std::memset(&L, 0, sizeof L);
  L.bias_slot_bytes = align_up(d->bias_slot_bytes ? d->bias_slot_bytes : kDefaultSide, kAlign);
  size_t off = 0;
  for (int i = 0; i < d->n_pages; ++i) {
    L.page_off[i] = off;
    off += align_up(d->page_bytes, kAlign);
  }
  for (int i = 0; i < 2; ++i) {
    L.bias_off[i] = off;
    off += L.bias_slot_bytes;
  }
  L.workspace_off = off;
  off += align_up(d->workspace_bytes, kAlign);
  if (off > d->arena_bytes)
    return fail(PSI_E_ARENA_TOO_SMALL,
                "arena of " + std::to_string(d->arena_bytes) + " B cannot hold " +
                    std::to_string(d->n_pages) + " pages of " + std::to_string(d->page_bytes) +
                    " B, two bias slots and " + std::to_string(d->workspace_bytes) + " B workspace");
  L.scratch_off = off;
  L.scratch_bytes = (d->arena_bytes - off) / kAlign * kAlign;
  L.total_bytes = d->arena_bytes;
  *out = L;
  return PSI_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- plans
namespace psi {

static psi_status page_fit(const psi_arena_desc* d, const psi_matrix* m, const char* name) {
  if (m->resident) return PSI_OK;  // consumed in place, never copied into a page
  MatrixInfo mi = matrix_info(m);
  if (mi.max_page_bytes > d->page_bytes)
    return fail(PSI_E_PAGE_TOO_SMALL, std::string("weight tile exceeds page: ") + name + " needs " +
                                          std::to_string(mi.max_page_bytes) + " B per page, page is " +
                                          std::to_string(d->page_bytes) + " B");
  return PSI_OK;
}

// Bytes an operator stages in its bias slot (streamed matrices with a bias).
static psi_status bias_fit(const psi_arena_layout& L, const psi_matrix* const* ms, int n) {
  size_t need = 0;
  for (int i = 0; i < n; ++i)
    if (ms[i]->bias_host && !ms[i]->resident) need += align_up((size_t)ms[i]->rows * 2, kAlign);
  if (need > L.bias_slot_bytes)
    return fail(PSI_E_PAGE_TOO_SMALL, "the operator's biases (" + std::to_string(need) +
                                          " B) exceed a bias slot (" + std::to_string(L.bias_slot_bytes) + " B)");
  return PSI_OK;
}

static psi_status scratch_fit(const psi_arena_layout& L, size_t need, const char* what) {
  if (need > L.scratch_bytes)
    return fail(PSI_E_SCRATCH_EXHAUSTED, std::string("scratch exhausted: ") + what + " needs " +
                                             std::to_string(need) + " B, scratch is " +
                                             std::to_string(L.scratch_bytes) + " B");
  return PSI_OK;
}

}  // namespace psi

extern "C" {

psi_status psi_linear_plan(const psi_arena_desc* d, int M, int K, const psi_matrix* W,
                           int acc_external, size_t* scratch_needed) {
  psi_arena_layout L;
  psi_status st = psi_arena_plan(d, &L);
  if (st) return st;
  if ((st = check_matrix(W, "W", -1))) return st;
  if (M < 0 || K <= 0 || K != W->cols) return fail(PSI_E_INVALID, "linear: x is [M, K] with K == W.cols");
  if ((st = page_fit(d, W, "W"))) return st;
  if ((st = bias_fit(L, &W, 1))) return st;
  size_t need = 0;
  if (W->split == PSI_SPLIT_COLS && !acc_external) need += align_up((size_t)M * W->rows * 4, kAlign);
  if ((st = scratch_fit(L, need, "linear accumulator"))) return st;
  if (scratch_needed) *scratch_needed = need;
  return PSI_OK;
}

psi_status psi_ffn_plan(const psi_arena_desc* d, int M, int dmodel, const psi_matrix* U,
                        const psi_matrix* V, int token_chunks, int acc_external,
                        size_t* scratch_needed) {
  psi_arena_layout L;
  psi_status st = psi_arena_plan(d, &L);
  if (st) return st;
  if ((st = check_matrix(U, "U", PSI_SPLIT_ROWS))) return st;
  if ((st = check_matrix(V, "V", PSI_SPLIT_COLS))) return st;
  if (M < 0 || dmodel <= 0 || U->cols != dmodel || V->rows != dmodel || V->cols != U->rows)
    return fail(PSI_E_INVALID, "ffn: need U [h, d] and V [d, h]");
  if (U->block != V->block) return fail(PSI_E_INVALID, "ffn: U and V must share the hidden tile");
  if (U->block % 8 != 0) return fail(PSI_E_ALIGN, "ffn: hidden tile must be a multiple of 8");
  if (token_chunks < 1) return fail(PSI_E_INVALID, "ffn: token_chunks must be >= 1");
  if ((st = page_fit(d, U, "U")) || (st = page_fit(d, V, "V"))) return st;
  // several chunks hold U_J and V_J in two slots at once (every chunk's
  // up-projection is followed by its down-projection)
  if (token_chunks > 1 && d->n_pages < 2 && !(U->resident && V->resident))
    return fail(PSI_E_INVALID, "ffn: token chunks keep U_J and V_J acquired together: need two page slots");
  const psi_matrix* uv[2] = {U, V};
  if ((st = bias_fit(L, uv, 2))) return st;
  // hidden tile H_J for the rows of one token chunk
  const size_t rows = ffn_chunk_rows(M, token_chunks);
  size_t need = align_up(rows * U->block * 2, kAlign);
  if (!acc_external) need += align_up((size_t)M * dmodel * 4, kAlign);
  if ((st = scratch_fit(L, need, "FFN hidden tile and accumulator"))) return st;
  if (scratch_needed) *scratch_needed = need;
  return PSI_OK;
}

psi_status psi_ffn_tiled_plan(const psi_arena_desc* d, int M, int dmodel, const psi_matrix* U,
                              const psi_matrix* Vo, int schedule, size_t* scratch_needed) {
  psi_arena_layout L;
  psi_status st = psi_arena_plan(d, &L);
  if (st) return st;
  if (schedule != PSI_FFN_REUSE && schedule != PSI_FFN_RECOMPUTE)
    return fail(PSI_E_INVALID, "ffn tiled: unknown schedule");
  if ((st = check_matrix(U, "U", PSI_SPLIT_ROWS))) return st;
  if ((st = check_matrix(Vo, "V", kSplitOutputTiles))) return st;
  if (M < 0 || dmodel <= 0 || U->cols != dmodel || Vo->rows != dmodel || Vo->cols != U->rows)
    return fail(PSI_E_INVALID, "ffn tiled: need U [h, d] and V [d, h]");
  if (U->block % 8 != 0) return fail(PSI_E_ALIGN, "ffn tiled: hidden tile must be a multiple of 8");
  if (Vo->split == PSI_SPLIT_TILES && Vo->block_cols % U->block != 0)
    return fail(PSI_E_INVALID, "ffn tiled: V's page columns must hold whole hidden tiles");
  if ((st = page_fit(d, U, "U")) || (st = page_fit(d, Vo, "V"))) return st;
  if (schedule == PSI_FFN_RECOMPUTE && d->n_pages < 2 && !(U->resident && Vo->resident))
    return fail(PSI_E_INVALID, "ffn tiled: the recompute schedule holds an output tile while U streams: "
                               "needs two page slots");
  const psi_matrix* uv[2] = {U, Vo};
  if ((st = bias_fit(L, uv, 2))) return st;
  const size_t hbuf = align_up((size_t)M * U->block * 2, kAlign);
  size_t need = (schedule == PSI_FFN_REUSE ? 2 : 1) * hbuf + align_up((size_t)M * Vo->block * 4, kAlign);
  if ((st = scratch_fit(L, need, "FFN hidden tile and output-tile accumulator"))) return st;
  if (scratch_needed) *scratch_needed = need;
  return PSI_OK;
}

psi_status psi_attn_plan(const psi_arena_desc* d, int M, int Mc, int heads, int head_dim,
                         const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                         const psi_matrix* Wo, int acc_external, size_t* scratch_needed) {
  psi_arena_layout L;
  psi_status st = psi_arena_plan(d, &L);
  if (st) return st;
  if (head_dim != 128 && head_dim != 64)
    return fail(PSI_E_INVALID, "attention: head_dim must be 128 or 64");
  if (heads <= 0 || M < 0 || Mc < 0) return fail(PSI_E_INVALID, "attention: bad sizes");
  const int dm = heads * head_dim;
  if ((st = check_matrix(Wq, "Wq", PSI_SPLIT_ROWS))) return st;
  if ((st = check_matrix(Wk, "Wk", PSI_SPLIT_ROWS))) return st;
  if ((st = check_matrix(Wv, "Wv", PSI_SPLIT_ROWS))) return st;
  // Wo split by columns: K-split over the head groups with the fp32 ACC
  // carried; split by rows: output tiles over the full K from every
  // group's O (the same summation per output)
  if ((st = check_matrix(Wo, "Wo", -1))) return st;
  const bool otiles = Wo->split == PSI_SPLIT_ROWS;
  const psi_matrix* ms[4] = {Wq, Wk, Wv, Wo};
  for (const psi_matrix* m : ms)
    if (m->rows != dm || m->cols != dm)
      return fail(PSI_E_INVALID, "attention: projections must be [heads*head_dim, heads*head_dim]");
  const int gw = Wq->block;
  if (gw % head_dim != 0 || Wk->block != gw || Wv->block != gw || (!otiles && Wo->block != gw))
    return fail(PSI_E_INVALID, "attention: Wq, Wk, Wv (and a column-split Wo) need the same head-group "
                               "block (a multiple of head_dim)");
  const char* names[4] = {"Wq", "Wk", "Wv", "Wo"};
  for (int i = 0; i < 4; ++i)
    if ((st = page_fit(d, ms[i], names[i]))) return st;
  if ((st = bias_fit(L, ms, 4))) return st;
  const int Ms = Mc > 0 ? Mc : M;
  if (Ms < 1 && M > 0) return fail(PSI_E_INVALID, "attention: at least one key per row is required");
  size_t ldvt = align_up((size_t)Ms, 64);
  size_t need = align_up((size_t)Ms * gw * 2, kAlign) + align_up((size_t)gw * ldvt * 2, kAlign);
  if (otiles) {
    // every group's O [M, dm] BF16, then one group's K and V^T: in acc_dev
    // (M dm 4 bytes) when given, K and V^T only where they fit behind O
    const size_t obytes = align_up((size_t)M * dm * 2, kAlign);
    if (!acc_external) need += obytes;
    else if (obytes + need <= (size_t)M * dm * 4) need = 0;
  } else {
    need += align_up((size_t)M * gw * 2, kAlign);
    if (!acc_external) need += align_up((size_t)M * dm * 4, kAlign);
  }
  if ((st = scratch_fit(L, need, "attention Q/K/V head-group tiles"))) return st;
  if (scratch_needed) *scratch_needed = need;
  return PSI_OK;
}

psi_status psi_attn_tiled_plan(const psi_arena_desc* d, int M, int Mc, int heads, int head_dim,
                               const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                               const psi_matrix* Wo, size_t* scratch_needed) {
  psi_arena_layout L;
  psi_status st = psi_arena_plan(d, &L);
  if (st) return st;
  if (head_dim != 128 && head_dim != 64)
    return fail(PSI_E_INVALID, "attention: head_dim must be 128 or 64");
  if (heads <= 0 || M < 0 || Mc < 0) return fail(PSI_E_INVALID, "attention: bad sizes");
  const int dm = heads * head_dim;
  if ((st = check_matrix(Wq, "Wq", PSI_SPLIT_ROWS)) || (st = check_matrix(Wk, "Wk", PSI_SPLIT_ROWS)) ||
      (st = check_matrix(Wv, "Wv", PSI_SPLIT_ROWS)))
    return st;
  if ((st = check_matrix(Wo, "Wo", kSplitOutputTiles))) return st;  // output tiles of the O-projection
  const psi_matrix* ms[4] = {Wq, Wk, Wv, Wo};
  for (const psi_matrix* m : ms)
    if (m->rows != dm || m->cols != dm)
      return fail(PSI_E_INVALID, "attention: projections must be [heads*head_dim, heads*head_dim]");
  const int gw = Wq->block;
  if (gw % head_dim != 0 || Wk->block != gw || Wv->block != gw)
    return fail(PSI_E_INVALID, "attention: Wq, Wk, Wv need the same head-group block (a multiple of head_dim)");
  if (gw % 8 != 0 || Wo->block % 8 != 0)
    return fail(PSI_E_ALIGN, "attention: head-group and output tiles must be multiples of 8");
  if (Wo->split == PSI_SPLIT_TILES && Wo->block_cols % gw != 0)
    return fail(PSI_E_INVALID, "attention tiled: Wo's page columns must hold whole head groups");
  const char* names[4] = {"Wq", "Wk", "Wv", "Wo"};
  for (int i = 0; i < 4; ++i)
    if ((st = page_fit(d, ms[i], names[i]))) return st;
  if ((st = bias_fit(L, ms, 4))) return st;
  const int Ms = Mc > 0 ? Mc : M;
  if (Ms < 1 && M > 0) return fail(PSI_E_INVALID, "attention: at least one key per row is required");
  const size_t ldvt = align_up((size_t)Ms, 64);
  const size_t obuf = align_up((size_t)M * gw * 2, kAlign);
  const size_t kv = align_up((size_t)Ms * gw * 2, kAlign) + align_up((size_t)gw * ldvt * 2, kAlign);
  const size_t acc = align_up((size_t)M * Wo->block * 4, kAlign);
  const size_t need = 2 * obuf + (kv > acc ? kv : acc);
  if ((st = scratch_fit(L, need, "attention Q/O buffers, K/V^T tiles, output-tile accumulator"))) return st;
  if (scratch_needed) *scratch_needed = need;
  return PSI_OK;
}

psi_status psi_attn_ext_plan(const psi_arena_desc* d, int M, int Mc, int heads, int head_dim,
                             const psi_matrix* Wq, const psi_matrix* Wk, const psi_matrix* Wv,
                             const psi_matrix* Wo, const psi_qk_norm_rope* nr, int acc_external,
                             size_t* scratch_needed) {
  psi_status st = psi_attn_plan(d, M, Mc, heads, head_dim, Wq, Wk, Wv, Wo, acc_external, scratch_needed);
  if (st || !qk_stage_active(nr)) return st;
  psi_arena_layout L;
  if ((st = psi_arena_plan(d, &L))) return st;
  if ((nr->gamma_q || nr->gamma_k) && !(nr->eps > 0.0f))
    return fail(PSI_E_INVALID, "attention: eps must be > 0 with a normalisation gamma");
  if (nr->norm_tile < 0 || nr->norm_tile % 8 != 0)
    return fail(PSI_E_INVALID, "attention: norm_tile must be 0 or a positive multiple of 8");
  if (!nr->cos_q && (nr->sin_q || nr->cos_k || nr->sin_k))
    return fail(PSI_E_INVALID, "attention: rotary tables given without the query cosine table");
  if (nr->cos_q && !nr->sin_q) return fail(PSI_E_INVALID, "attention: sin_q is missing");
  if (nr->cos_k && !nr->sin_k) return fail(PSI_E_INVALID, "attention: sin_k is missing");
  const int Ms = Mc > 0 ? Mc : M;
  if (nr->cos_q && !nr->cos_k && Ms != M)
    return fail(PSI_E_INVALID, "attention: keys need their own rotary tables when Mk != M");
  const void* tabs[4] = {nr->cos_q, nr->sin_q, nr->cos_k, nr->sin_k};
  for (const void* t : tabs)
    if (reinterpret_cast<uintptr_t>(t) % 16 != 0)
      return fail(PSI_E_ALIGN, "attention: rotary tables must be 16-byte aligned");
  const int dm = heads * head_dim;
  const psi_matrix* ms[4] = {Wq, Wk, Wv, Wo};
  size_t bias = 0;
  for (const psi_matrix* m : ms)
    if (m->bias_host && !m->resident) bias += align_up((size_t)m->rows * 2, kAlign);
  if (!Wq->resident) {
    if (nr->gamma_q) bias += align_up((size_t)dm * 2, kAlign);
    if (nr->gamma_k) bias += align_up((size_t)dm * 2, kAlign);
  }
  if (bias > L.bias_slot_bytes)
    return fail(PSI_E_PAGE_TOO_SMALL, "the operator's biases and gammas (" + std::to_string(bias) +
                                          " B) exceed a bias slot (" + std::to_string(L.bias_slot_bytes) + " B)");
  const size_t ldvt = align_up((size_t)Ms, 64);
  size_t need = align_up((size_t)M * dm * 2, kAlign) + align_up((size_t)Ms * dm * 2, kAlign) +
                align_up((size_t)Wq->block * ldvt * 2, kAlign);
  if (!acc_external && Wo->split == PSI_SPLIT_COLS) need += align_up((size_t)M * dm * 4, kAlign);
  if ((st = scratch_fit(L, need, "attention Q/K (all head groups) and V^T tiles"))) return st;
  if (scratch_needed) *scratch_needed = need;
  return PSI_OK;
}

}  // extern "C"
