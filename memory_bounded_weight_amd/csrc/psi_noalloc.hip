// psi_noalloc.hip -- the projection over resident weight pages for callers
// that cannot allocate device memory (code under stream capture, tight
// serving loops, harnesses that forbid allocation).
//
// It is psi_linear_paged with resident pages (psi_matrix.resident = 1) and
// no arena: the K-split's carried fp32 accumulator, which psi_linear_paged
// keeps in arena scratch, lives in the file-scope array `scratch` below,
// one copy per device, held until the process ends.  The kernels are the
// same GEMM launches in the same page order, so the bits are those of
// psi_linear_paged.
#include <mutex>

#include "psi_internal.h"

namespace {

constexpr size_t kScratchBytes = PSI_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The device array.  Host code never passes its name to a kernel or a copy:
// the name is a host-side stand-in; the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
psi_status scratch_address(void** out) {
  int dev = 0;
  PSI_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return psi::fail(PSI_E_INVALID, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    PSI_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return psi::fail(PSI_E_HIP, "hipGetSymbolAddress returned a null address");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return PSI_OK;
}

}  // namespace

using namespace psi;

extern "C" {

psi_status psi_linear_resident_noalloc(const uint16_t* x, int M, int K, const psi_matrix* W, uint16_t* y,
                                       unsigned flags, void* stream) {
  psi_status st = check_matrix(W, "W", -1);
  if (st) return st;
  if (!W->resident) return fail(PSI_E_INVALID, "noalloc linear: W must be resident (device pages)");
  if (M < 0 || K <= 0 || K != W->cols) return fail(PSI_E_INVALID, "noalloc linear: x is [M, K] with K == W.cols");
  const int N = W->rows;
  const bool ksplit = W->split == PSI_SPLIT_COLS;
  const bool resid = flags & PSI_OP_RESIDUAL;
  if (flags & ~(unsigned)(PSI_OP_BASELINE_BIAS | PSI_OP_RESIDUAL))
    return fail(PSI_E_INVALID, "noalloc linear: only PSI_OP_BASELINE_BIAS and PSI_OP_RESIDUAL");
  if (resid && K != N) return fail(PSI_E_INVALID, "linear residual needs K == N");
  if (ksplit && (size_t)M * N * 4 > kScratchBytes)
    return fail(PSI_E_SCRATCH_EXHAUSTED, "noalloc linear: the fp32 accumulator (" +
                                             std::to_string((size_t)M * N * 4) + " B) exceeds the " +
                                             std::to_string(kScratchBytes) + " B static scratch");
  if ((st = check_alias(x, (size_t)M * K * 2, y, (size_t)M * N * 2, false, "noalloc linear"))) return st;
  if ((st = check_ptr(x, "x")) || (st = check_ptr(y, "y")) || (st = check_ptr(W->pages_host, "W pages")))
    return st;
  if (ksplit && N % 8 != 0) return fail(PSI_E_ALIGN, "N must be a multiple of 8");
  if (M == 0) return PSI_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* acc = nullptr;
  if (ksplit) {
    void* p = nullptr;
    if ((st = scratch_address(&p))) return st;
    acc = static_cast<float*>(p);
  }
  const uint16_t* b = W->bias_host;
  const int n = psi_matrix_pages(W);
  for (int p = 0; p < n; ++p) {
    const uint16_t* page = static_cast<const uint16_t*>(matrix_page_ptr(W, p));
    const int ext = matrix_page_extent(W, p);
    GemmArgs g{};
    g.epi = EPI_BIAS;
    g.M = M;
    g.baseline_bias = (flags & PSI_OP_BASELINE_BIAS) ? 1 : 0;
    if (!ksplit) {
      const int c0 = p * W->block;
      g.A = x; g.lda = K;
      g.B = page; g.ldb = K;
      g.N = ext; g.K = K;
      g.bias = b ? b + c0 : nullptr;
      g.out = y + c0; g.ldo = N;
      if (resid) { g.resid = x + c0; g.ldr = K; }
    } else {
      // ACC (+)= x[:, k0:k0+ext] page^T in page order (the first page starts
      // from zero and reads nothing of the previous call's contents); the
      // last page adds the bias once and writes y
      const int k0 = p * W->block;
      const bool last = p == n - 1;
      g.A = x + k0; g.lda = K;
      g.B = page; g.ldb = ext;
      g.N = N; g.K = ext;
      if (p > 0) { g.acc_in = acc; g.ld_acc_in = N; }
      if (last) {
        g.bias = b;
        g.out = y; g.ldo = N;
        if (resid) { g.resid = x; g.ldr = K; }
      } else {
        g.epi = EPI_ACC;
        g.acc_out = acc; g.ld_acc_out = N;
      }
    }
    PSI_HIP(launch_gemm(g, s));
  }
  return PSI_OK;
}

}  // extern "C"
