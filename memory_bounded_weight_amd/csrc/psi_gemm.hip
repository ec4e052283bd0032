// psi_gemm.hip -- page-sliced BF16 GEMM for gfx950 (CDNA4).
//
// Computes C[M,N] = A[M,K] * B[N,K]^T with fp32 accumulation on the matrix
// cores (v_mfma_f32_32x32x16_bf16), operands staged through LDS with a
// double buffer, and a fused epilogue:
//   * carried fp32 accumulator: the MFMA accumulators start from acc_in, so
//     a K-split over weight pages continues one accumulation chain per
//     output in page order ([PSI] sec. II-B eq. (2): disjoint
//     down-projection sum, output bias added once);
//   * bias in fp32 before the single BF16 write (modified PSI, [PSI] sec.
//     III-A) or after rounding the product (baseline PSI);
//   * tanh-GELU between the two declared BF16 writes of the up-projection
//     ([PSI] sec. III-A);
//   * residual write B(f(x) + f(y)).
// [PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint
// Audio-Video Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
//
// Determinism: one fixed instruction sequence per output element for every
// shape (no split-K inside a launch, no atomics), so the same operands give
// the same bits on every run and for every page partition of the output.
#include "psi_internal.h"

namespace psi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// Round to bfloat16, nearest with ties to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t f2bf(float v) {
  uint32_t w = __float_as_uint(v);
  if ((w & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  w += 0x7FFFu + ((w >> 16) & 1u);
  return (uint16_t)(w >> 16);
}

// tanh-GELU, phi(v) = v/2 (1 + tanh(z)), z = sqrt(2/pi) (v + 0.044715 v^3),
// through 1 + tanh(z) = 2 / (1 + e^(-2z)) = 2 e^(2z) / (1 + e^(2z)); the
// second form for z < 0 neither cancels nor overflows, so the tiny negative
// values of the left tail keep their relative precision.
__device__ __forceinline__ float gelu_tanh(float v) {
  const float c = 0.7978845608028654f;
  const float z = c * (v + 0.044715f * v * v * v);
  if (z >= 0.0f) return v / (1.0f + expf(-2.0f * z));
  const float e = expf(2.0f * z);
  return v * e / (1.0f + e);
}

constexpr int kThreads = 256;  // 4 waves of 64, arranged 2 x 2

template <int BM, int BN, int BK>
struct Tile {
  static constexpr int LDS = BK + 8;            // padded row stride (elements)
  static constexpr int A_CHUNKS = BM * BK / 8;  // 16-byte chunks per tile
  static constexpr int B_CHUNKS = BN * BK / 8;
  static constexpr int A_PER_T = A_CHUNKS / kThreads;
  static constexpr int B_PER_T = B_CHUNKS / kThreads;
  static constexpr int WM = BM / 2;  // wave tile (2 x 2 waves)
  static constexpr int WN = BN / 2;
  static constexpr int TM = WM / 32;  // 32x32 MFMA tiles per wave
  static constexpr int TN = WN / 32;
  static constexpr int STAGE = (BM + BN) * LDS;  // elements per LDS stage
  static_assert(A_CHUNKS % kThreads == 0 && B_CHUNKS % kThreads == 0, "tile/threads");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
};

// STAGES = 2: double-buffered LDS, one barrier per K tile.
// STAGES = 1: one LDS buffer (half the LDS, so two workgroups fit a CU),
// the register stage still prefetches the next K tile.
template <int BM, int BN, int BK, int STAGES>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  using T = Tile<BM, BN, BK>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * T::STAGE];

  // Workgroup ids are dealt round-robin to the 8 XCDs (each with its own
  // L2).  Remap so that every XCD owns a contiguous range of logical tiles,
  // and walk that range with N fastest: concurrently running tiles of an
  // XCD then share their A row bands (and the page's B bands) in its L2.
  const int nt = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (nt % 8 == 0) t = (t % 8) * (nt / 8) + t / 8;
  const int tm = t / tiles_n;
  const int tn = t % tiles_n;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  constexpr int CPR = BK / 8;  // 16-byte chunks per row
  uint4 ra[T::A_PER_T], rb[T::B_PER_T];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::A_PER_T; ++i) {
      int c = tid + i * kThreads;
      int r = c / CPR, kc = (c % CPR) * 8;
      int gr = m0 + r, gk = k0 + kc;
      if (gr < p.M && gk < p.K)
        ra[i] = *reinterpret_cast<const uint4*>(p.A + (long)gr * p.lda + gk);
      else
        ra[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < T::B_PER_T; ++i) {
      int c = tid + i * kThreads;
      int r = c / CPR, kc = (c % CPR) * 8;
      int gr = n0 + r, gk = k0 + kc;
      if (gr < p.N && gk < p.K)
        rb[i] = *reinterpret_cast<const uint4*>(p.B + (long)gr * p.ldb + gk);
      else
        rb[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_lds = [&](int buf) {
    uint16_t* sa = smem + buf * T::STAGE;
    uint16_t* sb = sa + BM * T::LDS;
#pragma unroll
    for (int i = 0; i < T::A_PER_T; ++i) {
      int c = tid + i * kThreads;
      int r = c / CPR, kc = (c % CPR) * 8;
      *reinterpret_cast<uint4*>(sa + r * T::LDS + kc) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < T::B_PER_T; ++i) {
      int c = tid + i * kThreads;
      int r = c / CPR, kc = (c % CPR) * 8;
      *reinterpret_cast<uint4*>(sb + r * T::LDS + kc) = rb[i];
    }
  };

  // Accumulators, C layout of the 32x32 MFMA: lane holds column l32 and
  // rows 8*(i/4) + 4*half + (i%4), i = 0..15.
  f32x16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (p.acc_in) {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const int gn = n0 + wn * T::WN + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gm = m0 + wm * T::WM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          if (gm < p.M && gn < p.N) acc[i][j][r] = p.acc_in[(long)gm * p.ld_acc_in + gn];
        }
      }
  }

  const int nk = (p.K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = STAGES == 2 ? (kt & 1) : 0;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const uint16_t* sa = smem + cur * T::STAGE + (wm * T::WM) * T::LDS;
    const uint16_t* sb = smem + cur * T::STAGE + BM * T::LDS + (wn * T::WN) * T::LDS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kofs = ks * 16 + half * 8;
      bf16x8 af[T::TM], bfr[T::TN];
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sa + (i * 32 + l32) * T::LDS + kofs);
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(sb + (j * 32 + l32) * T::LDS + kofs);
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (STAGES == 1) __syncthreads();
    if (kt + 1 < nk) store_lds(STAGES == 2 ? (cur ^ 1) : 0);
    __syncthreads();
  }

  // Epilogue.
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int gn = n0 + wn * T::WN + j * 32 + l32;
      if (gn >= p.N) continue;
      const float bn = (p.bias && !p.bias_on_m) ? bf2f(p.bias[gn]) : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm * T::WM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
        if (gm >= p.M) continue;
        const float v = acc[i][j][r];
        if (p.acc_out) p.acc_out[(long)gm * p.ld_acc_out + gn] = v;
        if (p.out) {
          float t;
          if (p.bias) {
            const float bv = p.bias_on_m ? bf2f(p.bias[gm]) : bn;
            t = p.baseline_bias ? bf2f(f2bf(v)) + bv : v + bv;
          } else {
            t = v;
          }
          uint16_t y = f2bf(t);
          if (p.epi == EPI_GELU) y = f2bf(gelu_tanh(bf2f(y)));
          if (p.resid) y = f2bf(bf2f(p.resid[(long)gm * p.ldr + gn]) + bf2f(y));
          p.out[(long)gm * p.ldo + gn] = y;
        }
      }
    }
}

// Deep-prefetch variant: K tiles are fetched two iterations ahead into two
// register stages (the loop is unrolled by two so stage indices are
// compile-time), loads are branch-free (rows past M or N are clamped to
// the last row: they only feed outputs that are never stored; the K tail
// is zeroed with a select), and LDS is double-buffered.
template <int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads) void gemm_kernel_pf(GemmArgs p, int tiles_m, int tiles_n) {
  using T = Tile<BM, BN, BK>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];

  const int nt = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (nt % 8 == 0) t = (t % 8) * (nt / 8) + t / 8;
  const int tm = t / tiles_n;
  const int tn = t % tiles_n;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  constexpr int CPR = BK / 8;
  // per-thread chunk coordinates (row within the tile, k offset)
  const uint16_t* pa[T::A_PER_T];
  const uint16_t* pb[T::B_PER_T];
  int ka[T::A_PER_T], kb[T::B_PER_T];
#pragma unroll
  for (int i = 0; i < T::A_PER_T; ++i) {
    int c = tid + i * kThreads;
    int r = m0 + c / CPR;
    r = r < p.M ? r : p.M - 1;
    ka[i] = (c % CPR) * 8;
    pa[i] = p.A + (long)r * p.lda;
  }
#pragma unroll
  for (int i = 0; i < T::B_PER_T; ++i) {
    int c = tid + i * kThreads;
    int r = n0 + c / CPR;
    r = r < p.N ? r : p.N - 1;
    kb[i] = (c % CPR) * 8;
    pb[i] = p.B + (long)r * p.ldb;
  }
  uint4 ra[2][T::A_PER_T], rb[2][T::B_PER_T];

  auto load = [&](int k0, uint4* xa, uint4* xb) {
#pragma unroll
    for (int i = 0; i < T::A_PER_T; ++i) {
      const int gk = k0 + ka[i];
      const bool ok = gk < p.K;
      uint4 v = *reinterpret_cast<const uint4*>(pa[i] + (ok ? gk : 0));
      xa[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < T::B_PER_T; ++i) {
      const int gk = k0 + kb[i];
      const bool ok = gk < p.K;
      uint4 v = *reinterpret_cast<const uint4*>(pb[i] + (ok ? gk : 0));
      xb[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf, const uint4* xa, const uint4* xb) {
    uint16_t* sa = smem + buf * T::STAGE;
    uint16_t* sb = sa + BM * T::LDS;
#pragma unroll
    for (int i = 0; i < T::A_PER_T; ++i) {
      int c = tid + i * kThreads;
      *reinterpret_cast<uint4*>(sa + (c / CPR) * T::LDS + (c % CPR) * 8) = xa[i];
    }
#pragma unroll
    for (int i = 0; i < T::B_PER_T; ++i) {
      int c = tid + i * kThreads;
      *reinterpret_cast<uint4*>(sb + (c / CPR) * T::LDS + (c % CPR) * 8) = xb[i];
    }
  };

  f32x16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (p.acc_in) {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const int gn = n0 + wn * T::WN + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gm = m0 + wm * T::WM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          if (gm < p.M && gn < p.N) acc[i][j][r] = p.acc_in[(long)gm * p.ld_acc_in + gn];
        }
      }
  }

  auto compute = [&](int buf) {
    const uint16_t* sa = smem + buf * T::STAGE + (wm * T::WM) * T::LDS;
    const uint16_t* sb = smem + buf * T::STAGE + BM * T::LDS + (wn * T::WN) * T::LDS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kofs = ks * 16 + half * 8;
      bf16x8 af[T::TM], bfr[T::TN];
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sa + (i * 32 + l32) * T::LDS + kofs);
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(sb + (j * 32 + l32) * T::LDS + kofs);
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = (p.K + BK - 1) / BK;
  // prologue: tile 0 in LDS buffer 0, tile 1 in register stage 1
  load(0, ra[0], rb[0]);
  store(0, ra[0], rb[0]);
  if (nk > 1) load(BK, ra[1], rb[1]);
  __syncthreads();

  // iteration kt: issue tile kt+2 into register stage kt&1, compute tile kt
  // from LDS buffer kt&1, then move tile kt+1 (register stage (kt+1)&1) into
  // LDS buffer (kt+1)&1.
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 2 < nk) load((kt + 2) * BK, ra[0], rb[0]);
    compute(0);
    if (kt + 1 < nk) store(1, ra[1], rb[1]);
    __syncthreads();
    if (kt + 1 >= nk) break;
    if (kt + 3 < nk) load((kt + 3) * BK, ra[1], rb[1]);
    compute(1);
    if (kt + 2 < nk) store(0, ra[0], rb[0]);
    __syncthreads();
  }

  // Epilogue.
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int gn = n0 + wn * T::WN + j * 32 + l32;
      if (gn >= p.N) continue;
      const float bn = (p.bias && !p.bias_on_m) ? bf2f(p.bias[gn]) : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm * T::WM + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
        if (gm >= p.M) continue;
        const float v = acc[i][j][r];
        if (p.acc_out) p.acc_out[(long)gm * p.ld_acc_out + gn] = v;
        if (p.out) {
          float t;
          if (p.bias) {
            const float bv = p.bias_on_m ? bf2f(p.bias[gm]) : bn;
            t = p.baseline_bias ? bf2f(f2bf(v)) + bv : v + bv;
          } else {
            t = v;
          }
          uint16_t y = f2bf(t);
          if (p.epi == EPI_GELU) y = f2bf(gelu_tanh(bf2f(y)));
          if (p.resid) y = f2bf(bf2f(p.resid[(long)gm * p.ldr + gn]) + bf2f(y));
          p.out[(long)gm * p.ldo + gn] = y;
        }
      }
    }
}

template <int BM, int BN, int BK>
hipError_t launch_pf(const GemmArgs& a, hipStream_t s) {
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel_pf<BM, BN, BK>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, s, a,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int STAGES>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, STAGES>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, s, a,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

// Tile configurations (every one gives the same bits: each output sees the
// same ascending sequence of k16 MFMA steps whatever the tile).
//   1: 256x256, 2: 256x128, 3: 128x256, 4: 128x128 (double-buffered LDS)
//   5: 256x128, 6: 128x256 with one LDS stage (two workgroups per CU)
//   7: 128x128 (BK 64), 8: 128x128 (BK 32), 9: 256x128 (BK 32), 10: 128x256
//      (BK 32): two register stages, tiles fetched two iterations ahead
// Measured on MI355X: the 128x128 tile, at two waves per SIMD (two
// workgroups per CU), is the fastest on every page shape of this path;
// the single-wave large tiles are latency-bound.
int gemm_auto_config(int M, int N) {
  (void)M;
  (void)N;
  return 4;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  int cfg = a.config > 0 ? a.config : gemm_auto_config(a.M, a.N);
  switch (cfg) {
    case 1: return launch_cfg<256, 256, 64, 2>(a, s);
    case 2: return launch_cfg<256, 128, 64, 2>(a, s);
    case 3: return launch_cfg<128, 256, 64, 2>(a, s);
    case 5: return launch_cfg<256, 128, 64, 1>(a, s);
    case 6: return launch_cfg<128, 256, 64, 1>(a, s);
    case 7: return launch_pf<128, 128, 64>(a, s);
    case 8: return launch_pf<128, 128, 32>(a, s);
    case 9: return launch_pf<256, 128, 32>(a, s);
    case 10: return launch_pf<128, 256, 32>(a, s);
    default: return launch_cfg<128, 128, 64, 2>(a, s);
  }
}

}  // namespace psi
