// psi_gemm.hip -- page-sliced BF16 GEMM for gfx950 (CDNA4).
//
// Computes C[M,N] = A[M,K] * B[N,K]^T with fp32 accumulation on the matrix
// cores (v_mfma_f32_32x32x16_bf16) and a fused epilogue:
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
// Main kernel: operand tiles move from global memory straight into LDS
// (global_load_lds_dwordx4, no register staging) through a ring of S LDS
// stages, so S-1 K tiles are in flight while the matrix cores work on the
// current one.  LDS rows are unpadded; the 16-byte chunks of a row are
// XOR-swizzled by the row index so that the MFMA fragment reads
// (ds_read_b128 down 32 rows) hit distinct banks.  Fragments of the next
// k16 step are read while the MFMAs of the current step run.
//
// Determinism: one fixed instruction sequence per output element for every
// shape (no split-K inside a launch, no atomics), so the same operands give
// the same bits on every run and for every page partition of the output;
// all tile configurations below give identical bits (each output sees the
// same ascending sequence of k16 MFMA steps with the same lane mapping).
#include <atomic>

#include "psi_internal.h"

namespace psi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// Round to bfloat16, nearest with ties to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t f2bf(float v) {
  uint32_t w = __float_as_uint(v);
  if ((w & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  w += 0x7FFFu + ((w >> 16) & 1u);
  return (uint16_t)(w >> 16);
}

// Round a pair to bfloat16 with the packed conversion instruction (a in
// the low half).  It rounds to nearest with ties to even and gives f2bf's
// bits for every input but NaN, whose sign and payload it keeps; a value
// that is stored canonicalises NaN first (nan_canon), so NaN still gives
// 0x7FC0.  An intermediate rounding needs no canonical NaN: only NaN-ness
// reaches the stored value, and both conversions keep it.
__device__ __forceinline__ uint32_t cvt_pair(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float nan_canon(float v) {
  return __uint_as_float(v != v ? 0x7FC00000u : __float_as_uint(v));
}
__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// tanh-GELU, phi(v) = v/2 (1 + tanh(z)), z = sqrt(2/pi) (v + 0.044715 v^3),
// through 1 + tanh(z) = 2 / (1 + e^(-2z)) = 2 e^(2z) / (1 + e^(2z)); with
// e = e^(-2|z|) <= 1 that is v / (1 + e) for z >= 0 and v e / (1 + e) for
// z < 0, which neither cancels nor overflows, so the tiny negative values of
// the left tail keep their relative precision.  e comes from exp2f (which
// keeps denormal results) of -2 log2(e) |z|, and 1 / (1 + e) (in [1/2, 1])
// from the reciprocal instruction: about 2^-18 relative error against the
// exact function, well inside the BF16 rounding that follows (a result moves
// by one BF16 ulp only next to a rounding boundary).
__device__ __forceinline__ float gelu_tanh(float v) {
  const float c = 0.7978845608028654f;
  const float z = c * (v + 0.044715f * v * v * v);
  const float e = exp2f(-2.8853900817779268f * fabsf(z));
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  return z >= 0.0f ? v * r : (v * e) * r;
}

// Epilogue of one wave's TM x TN block of 32x32 accumulator tiles.  C layout
// of the 32x32 MFMA: lane holds column l32 and rows
// 8*(r/4) + 4*half + (r%4), r = 0..15.
//
// The residual (and a bias along rows) of each 32-row group is loaded
// before the group's first store.  The output may alias the residual, so
// the compiler cannot move a load above an earlier store: loaded element by
// element, each of the 16 TN values of a group would wait a full memory
// round trip.  Every element is still read by the lane that writes it,
// before its write.
template <int TM, int TN>
__device__ __forceinline__ void epilogue(const GemmArgs& p, f32x16 (&acc)[TM][TN], int mb, int nb, int half,
                                         int l32) {
  const bool resid = p.out && p.resid;
  const bool row_bias = p.out && p.bias && p.bias_on_m;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float rv[TN][16];
    float bm[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gm = min(mb + i * 32 + 8 * (r / 4) + 4 * half + (r % 4), p.M - 1);
      bm[r] = row_bias ? bf2f(p.bias[gm]) : 0.0f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int gn = min(nb + j * 32 + l32, p.N - 1);
        rv[j][r] = resid ? bf2f(p.resid[(long)gm * p.ldr + gn]) : 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int gn = nb + j * 32 + l32;
      if (gn >= p.N) continue;
      const float bn = (p.bias && !p.bias_on_m) ? bf2f(p.bias[gn]) : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = mb + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
        if (gm >= p.M) continue;
        const float v = acc[i][j][r];
        if (p.acc_out) p.acc_out[(long)gm * p.ld_acc_out + gn] = v;
        if (p.out) {
          float t;
          if (p.bias) {
            const float bv = p.bias_on_m ? bm[r] : bn;
            t = p.baseline_bias ? bf2f(f2bf(v)) + bv : v + bv;
          } else {
            t = v;
          }
          uint16_t y = f2bf(t);
          if (p.epi == EPI_GELU) y = f2bf(gelu_tanh(bf2f(y)));
          if (resid) y = f2bf(rv[j][r] + bf2f(y));
          p.out[(long)gm * p.ldo + gn] = y;
        }
      }
    }
  }
}

// Wave blocks wholly inside the output, on the epilogues of the hot path.
// A row's address is the same for every lane of the wave (a scalar base)
// plus a per-lane 32-bit byte offset (rows 4*half, column l32) and the
// tile's column offset as an immediate, so an element costs no address
// arithmetic and no bounds test; rows 2k and 2k+1 of a column are rounded
// by one conversion.  The arithmetic is epilogue()'s, in the same order,
// so both give the same bits.  Row offsets in bytes must fit 32 bits:
// leading dimensions below 2^26 (checked by finish()).
__device__ __forceinline__ int block_row(int mb, int i, int r) { return mb + i * 32 + 8 * (r / 4) + (r % 4); }

// BF16 output = B(acc + bias), then optionally GELU and a residual; no
// fp32 store.  The bias runs along columns, or along rows (BIAS_M: the
// transposed V projection).
template <int TM, int TN, bool GELU, bool RESID, bool BIAS_M>
__device__ __forceinline__ void epilogue_full(const GemmArgs& p, f32x16 (&acc)[TM][TN], int mb, int nb, int half,
                                              int l32) {
  const uint32_t lane_out = (uint32_t)(4 * half * (int)p.ldo + l32) * 2u;
  const uint32_t lane_res = RESID ? (uint32_t)(4 * half * (int)p.ldr + l32) * 2u : 0u;
  float bn[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) bn[j] = BIAS_M ? 0.0f : bf2f(p.bias[nb + j * 32 + l32]);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float bm[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) bm[r] = BIAS_M ? bf2f(p.bias[block_row(mb, i, r) + 4 * half]) : 0.0f;
    // the residual of the 32-row group, read before its first store (the
    // output may alias it; each element is read by the lane that writes it)
    float rv[TN][16];
    if (RESID) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const char* rb = (const char*)(p.resid + (long)block_row(mb, i, r) * p.ldr + nb) + lane_res;
#pragma unroll
        for (int j = 0; j < TN; ++j) rv[j][r] = bf2f(*(const uint16_t*)(rb + j * 64));
      }
    }
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      char* o0 = (char*)(p.out + (long)block_row(mb, i, r) * p.ldo + nb) + lane_out;
      char* o1 = (char*)(p.out + (long)block_row(mb, i, r + 1) * p.ldo + nb) + lane_out;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const float t0 = acc[i][j][r] + (BIAS_M ? bm[r] : bn[j]);
        const float t1 = acc[i][j][r + 1] + (BIAS_M ? bm[r + 1] : bn[j]);
        uint32_t y;
        if (!GELU && !RESID) {
          y = cvt_pair(nan_canon(t0), nan_canon(t1));
        } else {
          y = cvt_pair(t0, t1);
          if (GELU) {
            const float g0 = gelu_tanh(lo_f(y)), g1 = gelu_tanh(hi_f(y));
            y = RESID ? cvt_pair(g0, g1) : cvt_pair(nan_canon(g0), nan_canon(g1));
          }
          if (RESID) y = cvt_pair(nan_canon(rv[j][r] + lo_f(y)), nan_canon(rv[j][r + 1] + hi_f(y)));
        }
        *(uint16_t*)(o0 + j * 64) = (uint16_t)y;
        *(uint16_t*)(o1 + j * 64) = (uint16_t)(y >> 16);
      }
    }
  }
}

// fp32 accumulator store only (a step of a carried K-split chain).
template <int TM, int TN>
__device__ __forceinline__ void store_acc_full(const GemmArgs& p, f32x16 (&acc)[TM][TN], int mb, int nb, int half,
                                               int l32) {
  const uint32_t lane = (uint32_t)(4 * half * (int)p.ld_acc_out + l32) * 4u;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      char* ob = (char*)(p.acc_out + (long)block_row(mb, i, r) * p.ld_acc_out + nb) + lane;
#pragma unroll
      for (int j = 0; j < TN; ++j) *(float*)(ob + j * 128) = acc[i][j][r];
    }
}

__device__ __forceinline__ bool ld_ok(long ld) { return ld >= 0 && ld < (1L << 26); }

// The epilogue of a wave block: the whole-block paths above where they
// apply, epilogue() otherwise (ragged blocks, fp32 store beside the BF16
// output, the baseline bias rounding, no bias, a bias along rows with GELU
// or a residual).
template <int TM, int TN>
__device__ __forceinline__ void finish(const GemmArgs& p, f32x16 (&acc)[TM][TN], int mb, int nb, int half,
                                       int l32) {
  mb = __builtin_amdgcn_readfirstlane(mb);
  nb = __builtin_amdgcn_readfirstlane(nb);
  const bool full = mb + TM * 32 <= p.M && nb + TN * 32 <= p.N;
  if (full && !p.out && p.acc_out && ld_ok(p.ld_acc_out)) {
    store_acc_full<TM, TN>(p, acc, mb, nb, half, l32);
    return;
  }
  if (full && p.out && !p.acc_out && p.bias && !p.baseline_bias && ld_ok(p.ldo) && (!p.resid || ld_ok(p.ldr))) {
    const bool gelu = p.epi == EPI_GELU;
    if (p.bias_on_m) {
      if (!gelu && !p.resid) {
        epilogue_full<TM, TN, false, false, true>(p, acc, mb, nb, half, l32);
        return;
      }
    } else if (p.resid) {
      if (gelu) epilogue_full<TM, TN, true, true, false>(p, acc, mb, nb, half, l32);
      else epilogue_full<TM, TN, false, true, false>(p, acc, mb, nb, half, l32);
      return;
    } else {
      if (gelu) epilogue_full<TM, TN, true, false, false>(p, acc, mb, nb, half, l32);
      else epilogue_full<TM, TN, false, false, false>(p, acc, mb, nb, half, l32);
      return;
    }
  }
  epilogue<TM, TN>(p, acc, mb, nb, half, l32);
}

// Accumulators start from acc_in (carried K-split chain) or zero.
template <int TM, int TN>
__device__ __forceinline__ void init_acc(const GemmArgs& p, f32x16 (&acc)[TM][TN], int mb, int nb, int half,
                                         int l32) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (!p.acc_in) return;
  // whole block inside the output: scalar row bases, as in epilogue_full
  mb = __builtin_amdgcn_readfirstlane(mb);
  nb = __builtin_amdgcn_readfirstlane(nb);
  if (mb + TM * 32 <= p.M && nb + TN * 32 <= p.N && p.ld_acc_in >= 0 && p.ld_acc_in < (1L << 26)) {
    const uint32_t lane = (uint32_t)(4 * half * (int)p.ld_acc_in + l32) * 4u;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const char* ib = (const char*)(p.acc_in + (long)(mb + i * 32 + 8 * (r / 4) + (r % 4)) * p.ld_acc_in + nb) + lane;
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j][r] = *(const float*)(ib + j * 128);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int gn = nb + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = mb + i * 32 + 8 * (r / 4) + 4 * half + (r % 4);
        if (gm < p.M && gn < p.N) acc[i][j][r] = p.acc_in[(long)gm * p.ld_acc_in + gn];
      }
    }
}

// Tile order.  Workgroup ids are dealt round-robin to the 8 XCDs (each
// with its own L2); remap them so that every XCD owns a contiguous range of
// logical tiles.  Within that range tiles are walked in groups of gm tile
// rows: consecutive tiles go down the gm rows of a group, then to the next
// column.  The tiles an XCD runs at the same time then cover about gm rows
// x (concurrent / gm) columns, and share both operands' K slices in its L2
// (gm = 1 walks whole rows, N fastest).
__device__ __forceinline__ void tile_coords_of(int t, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  const int nt = tiles_m * tiles_n;
  if (nt % 8 == 0) t = (t % 8) * (nt / 8) + t / 8;
  const int per_group = gm * tiles_n;
  const int first_m = (t / per_group) * gm;
  const int rows = min(tiles_m - first_m, gm);
  const int r = t % per_group;
  tm = first_m + r % rows;
  tn = r / rows;
}
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  tile_coords_of(blockIdx.x, tiles_m, tiles_n, gm, tm, tn);
}

// s_waitcnt immediate for gfx9: vmcnt = n (6 bits), expcnt and lgkmcnt not
// waited on.
#define PSI_VMCNT(n) ((((n) & 0xF)) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 0x3) << 14))
#define PSI_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// ---------------------------------------------------------------------------
// Direct-to-LDS kernel.  BM x BN workgroup tile, WGM x WGN waves (each
// (BM/WGM) x (BN/WGN)), BK = 64, S LDS stages.  Requires K % 64 == 0 and
// 16-byte aligned rows (checked by the dispatcher).
//
// Stage layout: A rows [0, BM) then B rows [BM, BM+BN), 128 bytes per row;
// chunk c (8 elements) of row r sits at chunk position c ^ ((r / 2) % 8).
// One global_load_lds_dwordx4 moves 64 chunks = 8 rows: lane l fetches the
// global chunk that belongs at LDS position l of those 8 rows.
//
// Pipeline (per K tile kt): stage kt+S-1 is issued into the buffer that
// stage kt-1 used (all waves left it at the previous barrier); before the
// last k16 step of tile kt each wave waits until its own loads of stage kt+1
// have landed (vmcnt) and the workgroup meets at a barrier, after which the
// first fragments of tile kt+1 are read while the last MFMAs of kt run.
//
// Launch bound: at least two waves per SIMD (at most 256 registers per
// lane), so that two 4-wave workgroups share a CU where LDS allows it.
template <int BM, int BN, int WGM, int WGN, int S>
__global__ __launch_bounds__(64 * WGM * WGN, 2) void gemm_kernel_dma(GemmArgs p, int tiles_m, int tiles_n, int gm) {
  constexpr int BK = 64, NW = WGM * WGN;
  constexpr int CPR = BK / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;        // rows per load instruction
  constexpr int STAGE = (BM + BN) * BK;
  constexpr int LA = BM / RPI / NW, LB = BN / RPI / NW, NL = LA + LB;  // loads per wave per stage
  static_assert(LA * RPI * NW == BM && LB * RPI * NW == BN, "tile rows must split evenly over the waves");
  constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 32, TN = WN / 32, KS = BK / 16;
  static_assert(S >= 2 && S <= 4, "stages");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[S * STAGE];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, gm, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave / WGN, wn = wave % WGN;

  // Global sources of this lane's chunks (rows past M or N clamped to the
  // last row: they feed only outputs the epilogue discards).
  const uint16_t* ga[LA];
  const uint16_t* gb[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int r = (j * NW + wave) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ ((r / 2) % CPR);
    const int gr = min(m0 + r, p.M - 1);
    ga[j] = p.A + (long)gr * p.lda + c * 8;
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int r = (j * NW + wave) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ ((r / 2) % CPR);
    const int gr = min(n0 + r, p.N - 1);
    gb[j] = p.B + (long)gr * p.ldb + c * 8;
  }
  auto issue = [&](int kt) {
    uint16_t* st = smem + (kt % S) * STAGE;
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < LA; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(ga[j] + k0), PSI_LDS(st + (j * NW + wave) * RPI * BK), 16, 0,
                                       0);
#pragma unroll
    for (int j = 0; j < LB; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(gb[j] + k0),
                                       PSI_LDS(st + BM * BK + (j * NW + wave) * RPI * BK), 16, 0, 0);
  };
  // Let n stages of this wave's loads stay in flight (loads retire in order).
  auto wait_stages = [&](int n) {
    if (S >= 4 && n >= 2) __builtin_amdgcn_s_waitcnt(PSI_VMCNT(2 * NL));
    else if (S >= 3 && n >= 1) __builtin_amdgcn_s_waitcnt(PSI_VMCNT(NL));
    else __builtin_amdgcn_s_waitcnt(PSI_VMCNT(0));
  };
  // Fragment reads: row r of the wave's block, logical chunk 2*ks + half.
  // Rows 32 apart share the swizzle, so one per-lane term serves all tiles.
  int offa[TM], offb[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) offa[i] = (wm * WM + i * 32 + l32) * BK;
#pragma unroll
  for (int j = 0; j < TN; ++j) offb[j] = BM * BK + (wn * WN + j * 32 + l32) * BK;
  const int swz = (l32 / 2) % CPR;
  auto frags = [&](const uint16_t* st, int ks, bf16x8* af, bf16x8* bf) {
    const int pc = ((ks * 2 + half) ^ swz) * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(st + offa[i] + pc);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const bf16x8*>(st + offb[j] + pc);
  };

  f32x16 acc[TM][TN];
  init_acc<TM, TN>(p, acc, m0 + wm * WM, n0 + wn * WN, half, l32);

  // k16 step of tile kt after whose MFMAs stage kt+S-1 is issued; always
  // before the wait for stage kt+1 in the last step, so the vmcnt counts
  // hold.  Measured on MI355X: one step in is 1.5% faster with 3 stages and
  // 3-7% slower with 4.
  constexpr int kIssueStep = S == 3 ? 1 : 0;
  static_assert(kIssueStep < KS - 1, "stage issue must precede the last step's wait");
  const int nk = p.K / BK;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s);
  wait_stages(min(S - 2, nk - 1));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  bf16x8 fa[2][TM], fb[2][TN];
  frags(smem, 0, fa[0], fb[0]);
  for (int kt = 0; kt < nk; ++kt) {
    const uint16_t* st = smem + (kt % S) * STAGE;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < KS) {
        frags(st, ks + 1, fa[nxt], fb[nxt]);
      } else if (kt + 1 < nk) {
        wait_stages(min(S - 2, nk - 2 - kt));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        frags(smem + ((kt + 1) % S) * STAGE, 0, fa[nxt], fb[nxt]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
      if (ks == kIssueStep && kt + S - 1 < nk) issue(kt + S - 1);
    }
  }
  __builtin_amdgcn_s_waitcnt(PSI_VMCNT(0));
  finish<TM, TN>(p, acc, m0 + wm * WM, n0 + wn * WN, half, l32);
}

// ---------------------------------------------------------------------------
// Carried-chain kernel: a middle step of a K-split chain (fp32 accumulator in
// and out, no bias, no BF16 output) over whole 256 x 128 tiles, K = 1024,
// with the waves and LDS ring of the direct-to-LDS kernel (8 waves of
// 64 x 64, three stages).  In that kernel each workgroup loads its 128 KiB
// of acc_in before its first MFMA and stores 128 KiB after its last, with
// the matrix cores idle in both.  Here each workgroup stays resident and
// walks T tiles (t = blockIdx.x + i * gridDim.x, in the same XCD-local tile
// order), and two accumulator register sets alternate: while the MFMAs of
// tile i run on one, the other first gives up tile i-1's result (stores)
// and then takes tile i+1's acc_in (loads into the same registers), four or
// five elements in each of the first fourteen K tiles.  The LDS ring runs on
// across tiles: the first two stages of tile i+1 are issued during the last
// two K tiles of tile i.  Every output still starts from its acc_in and sees
// the same ascending k16 MFMA steps with the same lane mapping, so the bits
// are those of the other kernels.  The accumulator moves with non-temporal
// loads and stores, which leaves more of each XCD's L2 to the operand tiles.
//
// Wait counts.  One counter covers loads and stores, retired in issue order.
// In K tile kt, stage kt+2 is issued after the MFMAs of the second k16 step;
// the accumulator operations follow, half after that step and half after
// the third, and the wait for stage kt+1 before the last step leaves in
// flight exactly what was issued after stage kt+1: the accumulator
// operations of K tile kt-1, stage kt+2 and the accumulator operations of
// K tile kt.  A store or load thus has about two K tiles to complete.
#define PSI_VM_CASE(n) \
  case n: __builtin_amdgcn_s_waitcnt(PSI_VMCNT(n)); break;
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {  // immediates only; folded once the K loop is unrolled
    PSI_VM_CASE(1) PSI_VM_CASE(2) PSI_VM_CASE(3) PSI_VM_CASE(4) PSI_VM_CASE(5) PSI_VM_CASE(6) PSI_VM_CASE(7)
    PSI_VM_CASE(8) PSI_VM_CASE(9) PSI_VM_CASE(10) PSI_VM_CASE(11) PSI_VM_CASE(12) PSI_VM_CASE(13)
    PSI_VM_CASE(14) PSI_VM_CASE(15) PSI_VM_CASE(16) PSI_VM_CASE(17) PSI_VM_CASE(18) PSI_VM_CASE(19)
    PSI_VM_CASE(20) PSI_VM_CASE(21) PSI_VM_CASE(22) PSI_VM_CASE(23) PSI_VM_CASE(24) PSI_VM_CASE(25)
    PSI_VM_CASE(26) PSI_VM_CASE(27) PSI_VM_CASE(28) PSI_VM_CASE(29) PSI_VM_CASE(30) PSI_VM_CASE(31)
    PSI_VM_CASE(32) PSI_VM_CASE(33) PSI_VM_CASE(34) PSI_VM_CASE(35) PSI_VM_CASE(36) PSI_VM_CASE(37)
    PSI_VM_CASE(38) PSI_VM_CASE(39) PSI_VM_CASE(40)
    default: __builtin_amdgcn_s_waitcnt(PSI_VMCNT(0)); break;  // fewer in flight is always safe
  }
}
#undef PSI_VM_CASE

constexpr int kChainNK = 16;  // K tiles of 64 per step: K = 1024
// The accumulator traffic of a tile (64 elements per lane each way) is
// spread over its first 14 K tiles: element range [chain_e0(kt),
// chain_e0(kt + 1)) in K tile kt, 4 or 5 elements.  The last two K tiles
// stay free, so the next tile's accumulator has arrived before its first
// MFMA without a wait.  (Over the first 8 K tiles the kernel measured the
// same.)
constexpr int kChainAccTiles = 14;
__host__ __device__ constexpr int chain_e0(int kt) { return kt * 64 / kChainAccTiles; }

template <int KIND>
struct ChainKind {  // 0: first tile (no previous), 1: middle, 2: last (no next)
  static constexpr bool prev = KIND != 0, next = KIND != 2;
};

__global__ __launch_bounds__(512, 2) void gemm_kernel_chain(GemmArgs p, int tiles_m, int tiles_n, int gm, int T) {
  constexpr int BM = 256, BN = 128, WGN = 2, NW = 8, S = 3, BK = 64, NK = kChainNK;
  constexpr int CPR = BK / 8, RPI = 64 / CPR, STAGE = (BM + BN) * BK;
  constexpr int LA = BM / RPI / NW, LB = BN / RPI / NW, NL = LA + LB;
  constexpr int WM = 64, WN = 64, TM = 2, TN = 2, KS = BK / 16;
  static_assert(kChainAccTiles + 2 <= NK, "accumulator traffic must end two K tiles before a tile's end");
  static_assert(chain_e0(kChainAccTiles) == TM * TN * 16, "every accumulator element is moved");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave / WGN, wn = wave % WGN;

  // Tile i of this workgroup: operand bases (scalar) and the wave block's origin.
  struct Tile {
    const uint16_t* a;
    const uint16_t* b;
    int mb, nb;
  };
  auto tile = [&](int i) {
    int tm, tn;
    tile_coords_of(blockIdx.x + i * gridDim.x, tiles_m, tiles_n, gm, tm, tn);
    Tile t;
    t.a = p.A + (long)(tm * BM) * p.lda;
    t.b = p.B + (long)(tn * BN) * p.ldb;
    t.mb = __builtin_amdgcn_readfirstlane(tm * BM + wm * WM);
    t.nb = __builtin_amdgcn_readfirstlane(tn * BN + wn * WN);
    return t;
  };
  // Per-lane element offsets of the stage loads within a tile's operand rows
  // (32-bit: the dispatcher bounds lda and ldb).
  uint32_t oa[LA], ob[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int r = (j * NW + wave) * RPI + lane / CPR;
    oa[j] = (uint32_t)r * (uint32_t)p.lda + (uint32_t)((lane % CPR) ^ ((r / 2) % CPR)) * 8u;
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int r = (j * NW + wave) * RPI + lane / CPR;
    ob[j] = (uint32_t)r * (uint32_t)p.ldb + (uint32_t)((lane % CPR) ^ ((r / 2) % CPR)) * 8u;
  }
  auto issue = [&](const Tile& t, int kk, int buf) {
    uint16_t* st = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < LA; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(t.a + oa[j] + kk * BK),
                                       PSI_LDS(st + (j * NW + wave) * RPI * BK), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < LB; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(t.b + ob[j] + kk * BK),
                                       PSI_LDS(st + BM * BK + (j * NW + wave) * RPI * BK), 16, 0, 0);
  };
  int offa[TM], offb[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) offa[i] = (wm * WM + i * 32 + l32) * BK;
#pragma unroll
  for (int j = 0; j < TN; ++j) offb[j] = BM * BK + (wn * WN + j * 32 + l32) * BK;
  const int swz = (l32 / 2) % CPR;
  auto frags = [&](const uint16_t* st, int ks, bf16x8* af, bf16x8* bf) {
    const int pc = ((ks * 2 + half) ^ swz) * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(st + offa[i] + pc);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const bf16x8*>(st + offb[j] + pc);
  };
  // Accumulator element e of a wave block: tile (e / 32, e % 2), register
  // (e % 32) / 2; row and column as in the MFMA C layout.  Addresses: the
  // wave block's origin (scalar, per tile) plus a 32-bit byte offset, the
  // row's (scalar) and the lane's (the dispatcher bounds the leading
  // dimensions so that both fit).
  const uint32_t ld_in = (uint32_t)p.ld_acc_in * 4u, ld_out = (uint32_t)p.ld_acc_out * 4u;
  const uint32_t lane_in = 4u * (uint32_t)half * ld_in + (uint32_t)l32 * 4u;
  const uint32_t lane_out = 4u * (uint32_t)half * ld_out + (uint32_t)l32 * 4u;
  auto acc_src = [&](const char* base, uint32_t ld, int i, int r, int j) {
    const char* row = base + (uint32_t)block_row(0, i, r) * ld;  // scalar
    return (const float*)(row + lane_in + j * 128);
  };
  auto acc_dst = [&](char* base, uint32_t ld, int i, int r, int j) {
    char* row = base + (uint32_t)block_row(0, i, r) * ld;  // scalar
    return (float*)(row + lane_out + j * 128);
  };
  auto src_base = [&](const Tile& t) { return (const char*)(p.acc_in + (long)t.mb * p.ld_acc_in + t.nb); };
  auto dst_base = [&](const Tile& t) { return (char*)(p.acc_out + (long)t.mb * p.ld_acc_out + t.nb); };

  bf16x8 fa[2][TM], fb[2][TN];
  f32x16 P[TM][TN], Q[TM][TN];

  // One tile: MFMAs into cur; side gives up tile i-1 and takes tile i+1's
  // acc_in; the ring index of the tile's first K tile is (i * NK) % S.
  auto body = [&](auto kind, int i, f32x16 (&cur)[TM][TN], f32x16 (&side)[TM][TN]) {
    constexpr bool has_prev = decltype(kind)::prev, has_next = decltype(kind)::next;
    constexpr int OPS = (has_prev ? 1 : 0) + (has_next ? 1 : 0);  // per element
    // accumulator operations issued in K tile x of this tile
    auto acc_ops = [&](int x) { return (x >= 0 && x < kChainAccTiles) ? OPS * (chain_e0(x + 1) - chain_e0(x)) : 0; };
    const Tile tc = tile(i);
    Tile tn = tc;
    char* dst = nullptr;
    const char* src = nullptr;
    if (has_prev) dst = dst_base(tile(i - 1));
    if (has_next) {
      tn = tile(i + 1);
      src = src_base(tn);
    }
    const int b0 = (i * NK) % S;
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      const int bc = (b0 + kt) % S, bn = (b0 + kt + 1) % S, bi = (b0 + kt + 2) % S;
      const uint16_t* st = smem + bc * STAGE;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks & 1, n = c ^ 1;
        if (ks + 1 < KS) {
          frags(st, ks + 1, fa[n], fb[n]);
        } else if (kt + 1 < NK || has_next) {
          const bool issued = kt + 2 < NK || has_next;
          wait_vmcnt(acc_ops(kt - 1) + (issued ? NL : 0) + acc_ops(kt));
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          frags(smem + bn * STAGE, 0, fa[n], fb[n]);
        }
#pragma unroll
        for (int ti = 0; ti < TM; ++ti)
#pragma unroll
          for (int tj = 0; tj < TN; ++tj)
            cur[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][ti], fb[c][tj], cur[ti][tj], 0, 0, 0);
        if (ks == 1) {
          // The wait counts above need every accumulator operation of a K
          // tile issued after that tile's stage loads: the scheduler may not
          // move instructions across this fence.
          __builtin_amdgcn_sched_barrier(0);
          if (kt + 2 < NK) issue(tc, kt + 2, bi);
          else if (has_next) issue(tn, kt + 2 - NK, bi);
          __builtin_amdgcn_sched_barrier(0);
        }
        // Accumulator operations: half after the MFMAs of the second k16
        // step, half after the third (both before the wait in the last).
        if (kt < kChainAccTiles && (ks == 1 || ks == 2)) {
          // row offsets computed here, not hoisted (they would hold 128 scalar registers)
          uint32_t li = ld_in, lo = ld_out;
          asm volatile("" : "+s"(li), "+s"(lo));
          const int e0 = chain_e0(kt), e1 = chain_e0(kt + 1), em = (e0 + e1) / 2;
#pragma unroll
          for (int e = ks == 1 ? e0 : em; e < (ks == 1 ? em : e1); ++e) {
            const int ei = e / 32, er = (e % 32) / 2, ej = e % 2;
            if (has_prev) __builtin_nontemporal_store(side[ei][ej][er], acc_dst(dst, lo, ei, er, ej));
            if (has_next) side[ei][ej][er] = __builtin_nontemporal_load(acc_src(src, li, ei, er, ej));
          }
        }
      }
    }
  };

  // Prologue: tile 0's acc_in, then its first two stages.
  {
    const Tile t0 = tile(0);
    const char* src = src_base(t0);
#pragma unroll
    for (int ti = 0; ti < TM; ++ti)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int tj = 0; tj < TN; ++tj) P[ti][tj][r] = __builtin_nontemporal_load(acc_src(src, ld_in, ti, r, tj));
    issue(t0, 0, 0);
    issue(t0, 1, 1);
    wait_vmcnt(NL);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    frags(smem, 0, fa[0], fb[0]);
  }
  body(ChainKind<0>{}, 0, P, Q);
  int i = 1;
  for (; i + 2 < T; i += 2) {  // T is even: tiles 1 .. T-2 in pairs
    body(ChainKind<1>{}, i, Q, P);
    body(ChainKind<1>{}, i + 1, P, Q);
  }
  body(ChainKind<2>{}, i, Q, P);
  char* dst = dst_base(tile(i));
#pragma unroll
  for (int ti = 0; ti < TM; ++ti)
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int tj = 0; tj < TN; ++tj) __builtin_nontemporal_store(Q[ti][tj][r], acc_dst(dst, ld_out, ti, r, tj));
}

// ---------------------------------------------------------------------------
// Register-staged kernel for any K and 8-element-aligned rows: 128 x 128 x 64
// tile, 2 x 2 waves of 64 x 64, padded LDS rows (BK + 8), the next K tile
// loaded into registers while the current one is multiplied, K tail zeroed.
constexpr int kRegThreads = 256;

__global__ __launch_bounds__(kRegThreads, 2) void gemm_kernel_reg(GemmArgs p, int tiles_m, int tiles_n, int gm) {
  constexpr int BM = 128, BN = 128, BK = 64, LDS = BK + 8, CPR = BK / 8;
  constexpr int A_PER_T = BM * BK / 8 / kRegThreads, B_PER_T = BN * BK / 8 / kRegThreads;
  constexpr int WM = 64, WN = 64, TM = 2, TN = 2, STAGE = (BM + BN) * LDS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, gm, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  uint4 ra[A_PER_T], rb[B_PER_T];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * kRegThreads;
      const int gr = m0 + c / CPR, gk = k0 + (c % CPR) * 8;
      ra[i] = (gr < p.M && gk < p.K) ? *reinterpret_cast<const uint4*>(p.A + (long)gr * p.lda + gk)
                                     : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int c = tid + i * kRegThreads;
      const int gr = n0 + c / CPR, gk = k0 + (c % CPR) * 8;
      rb[i] = (gr < p.N && gk < p.K) ? *reinterpret_cast<const uint4*>(p.B + (long)gr * p.ldb + gk)
                                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_lds = [&](int buf) {
    uint16_t* sa = smem + buf * STAGE;
    uint16_t* sb = sa + BM * LDS;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * kRegThreads;
      *reinterpret_cast<uint4*>(sa + (c / CPR) * LDS + (c % CPR) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int c = tid + i * kRegThreads;
      *reinterpret_cast<uint4*>(sb + (c / CPR) * LDS + (c % CPR) * 8) = rb[i];
    }
  };

  f32x16 acc[TM][TN];
  init_acc<TM, TN>(p, acc, m0 + wm * WM, n0 + wn * WN, half, l32);

  const int nk = (p.K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const uint16_t* sa = smem + cur * STAGE + (wm * WM) * LDS;
    const uint16_t* sb = smem + cur * STAGE + BM * LDS + (wn * WN) * LDS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kofs = ks * 16 + half * 8;
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(sa + (i * 32 + l32) * LDS + kofs);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(sb + (j * 32 + l32) * LDS + kofs);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }
  finish<TM, TN>(p, acc, m0 + wm * WM, n0 + wn * WN, half, l32);
}

// Group height of the tile order: with C tiles of one XCD in flight, a
// window of g rows x C/g columns reads about g*BM + (C/g)*BN operand rows
// per K slice, least near g = sqrt(C * BN / BM); a power of two, at most
// the number of tile rows.
int group_rows(int tiles_m, int concurrent, int bm, int bn) {
  int g = 1;
  while (g * 2 <= tiles_m && (double)(g * 2) * (g * 2) <= (double)concurrent * bn / bm) g *= 2;
  return g;
}

constexpr int kXcdCUs = 32;  // CUs per XCD on MI355X

template <int BM, int BN, int WGM, int WGN, int S>
hipError_t launch_dma(const GemmArgs& a, hipStream_t s) {
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  constexpr int per_cu = (160 * 1024) / (S * (BM + BN) * 64 * 2);  // workgroups per CU by LDS
  const int gm = group_rows(tiles_m, kXcdCUs * per_cu, BM, BN);
  return launch_kernel(gemm_kernel_dma<BM, BN, WGM, WGN, S>, dim3(tiles_m * tiles_n), dim3(64 * WGM * WGN), s, a,
                       tiles_m, tiles_n, gm);
}

hipError_t launch_reg(const GemmArgs& a, hipStream_t s) {
  const int tiles_m = (a.M + 127) / 128;
  const int tiles_n = (a.N + 127) / 128;
  const int gm = group_rows(tiles_m, kXcdCUs * 2, 128, 128);
  return launch_kernel(gemm_kernel_reg, dim3(tiles_m * tiles_n), dim3(kRegThreads), s, a, tiles_m, tiles_n, gm);
}

bool dma_ok(const GemmArgs& a) {
  const uintptr_t al = (uintptr_t)a.A | (uintptr_t)a.B;
  return a.K > 0 && a.K % 64 == 0 && (al & 15) == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0;
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups of the carried-chain kernel for this step, or 0 where it does
// not apply: a middle step of a K-split chain (fp32 accumulator in and out
// only) of K = 1024 over whole 256 x 128 tiles, one workgroup per CU, each
// with an even number of tiles; operand rows of the stage loads addressed
// with 32-bit offsets.
int chain_workgroups(const GemmArgs& a) {
  if (!a.acc_in || !a.acc_out || a.out || a.bias || a.resid || !dma_ok(a)) return 0;
  if (a.K != kChainNK * 64 || a.M % 256 != 0 || a.N % 128 != 0) return 0;
  if (a.lda >= (1L << 22) || a.ldb >= (1L << 22) || !(a.ld_acc_in >= 0 && a.ld_acc_in < (1L << 24)) ||
      !(a.ld_acc_out >= 0 && a.ld_acc_out < (1L << 24)))
    return 0;
  const int G = device_cus();
  const long nt = (long)(a.M / 256) * (a.N / 128);
  if (G <= 0 || G % 8 != 0 || nt % G != 0 || (nt / G) % 2 != 0) return 0;
  return G;
}

hipError_t launch_chain(const GemmArgs& a, int G, hipStream_t s) {
  const int tiles_m = a.M / 256, tiles_n = a.N / 128;
  const int gm = group_rows(tiles_m, kXcdCUs, 256, 128);
  const int T = (int)((long)tiles_m * tiles_n / G);
  return launch_kernel(gemm_kernel_chain, dim3(G), dim3(512), s, a, tiles_m, tiles_n, gm, T);
}

}  // namespace

// Tile configurations (all give identical bits):
//   1: direct-to-LDS 256 x 128, 8 waves of 64 x 64, 3 LDS stages (144 KiB,
//      one workgroup per CU); a middle step of a carried K-split chain
//      that fits the carried-chain kernel runs on that kernel instead
//      (same tile and waves, resident workgroups) unless configuration 1
//      is asked for explicitly;
//   2: direct-to-LDS 128 x 128, 4 waves of 64 x 64, 2 LDS stages (64 KiB,
//      two workgroups per CU);
//   3: register-staged 128 x 128 (any K, 8-element-aligned rows).
// Configurations 1 and 2 need K % 64 == 0 and 16-byte aligned rows; other
// operands take configuration 3 whatever is asked.  Measured on MI355X on the
// page shapes of this path: 1 is fastest where it still yields >= 256 tiles
// and no fp32 accumulator streams through the epilogue; 2 overlaps one
// workgroup's accumulator traffic with the other's MFMAs (K-split pages)
// and fills more CUs on small outputs.
int gemm_auto_config(const GemmArgs& a) {
  if (!dma_ok(a)) return 3;
  // Outputs of more than 256 tiles of 128 x 128 fill the chip with 256 x 128
  // workgroups; smaller ones (few tokens, or a narrow page) are bound by the
  // latency of the K loop of a few workgroups, and 64 x 64 tiles with four
  // stages in flight run 2-2.5x faster there.
  const long tiles128 = (long)((a.M + 127) / 128) * ((a.N + 127) / 128);
  return tiles128 > 256 ? 1 : 4;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  int cfg = a.config > 0 ? a.config : gemm_auto_config(a);
  if (cfg != 3 && !dma_ok(a)) cfg = 3;
  if (a.config == 0 && cfg == 1)
    if (const int G = chain_workgroups(a)) return launch_chain(a, G, s);
  switch (cfg) {
    case 1: return launch_dma<256, 128, 4, 2, 3>(a, s);
    case 2: return launch_dma<128, 128, 2, 2, 2>(a, s);
    case 4: return launch_dma<64, 64, 2, 2, 4>(a, s);
    default: return launch_reg(a, s);
  }
}

}  // namespace psi
