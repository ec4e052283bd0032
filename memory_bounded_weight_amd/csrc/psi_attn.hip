// psi_attn.hip -- row-blocked attention with fp32 online softmax, gfx950.
//
// [PSI] sec. II-B eqs. (3)-(4) ("Precision-Preserving Subtensor Inference
// for a 22B Joint Audio-Video Generator under a Fixed GPU Working Set",
// arXiv 2611.08023): for every query, keys are processed in disjoint tiles
// T while a running maximum m, normaliser l and weighted value sum z are
// kept; for each tile m' = max(m, max_T s_j), eta = e^(m - m'),
// l' = eta l + sum_T e^(s_j - m'), z' = eta z + sum_T e^(s_j - m') v_j.
// After the last tile z / l is dense softmax attention (unmasked,
// noncausal, no dropout, at least one key).
//
// Layout of the work (head_dim 128 or 64, 64 keys per tile):
//   * one workgroup = 4 or 8 waves = 128 or 256 queries of one head; each
//     wave owns 32 queries;
//   * scores are computed transposed, S^T = K Q^T, with the 32x32x16 BF16
//     MFMA: in its accumulator layout a lane holds ONE query (column) and
//     16 keys, so m, l and the rescale factor of a query live in one lane
//     (and its partner lane l^32), with no cross-lane shuffles of the
//     output accumulator;
//   * the output is also accumulated transposed, O^T = V^T P^T: V^T comes
//     from the value projection, which writes V transposed, and P^T is fed
//     straight from the score registers as the B operand;
//   * the softmax weights stay fp32 on the BF16 matrix cores by splitting
//     p = hi + lo + lo2 into three BF16 numbers (each the rounding of what
//     the previous ones leave, so the three hold p's 24-bit significand)
//     and issuing one MFMA per term: the FP32 online accumulation of
//     modified PSI (sec. III-A).  With two terms (hi + lo) the weights keep
//     about 17 significant bits; with one (hi) they are the BF16 numerator
//     weights of baseline PSI.
#include "psi_internal.h"

namespace psi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// Round to bfloat16, nearest with ties to even (output values; finite).
__device__ __forceinline__ uint16_t f2bf(float v) {
  uint32_t w = __float_as_uint(v);
  if ((w & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  w += 0x7FFFu + ((w >> 16) & 1u);
  return (uint16_t)(w >> 16);
}

constexpr int KT = 64;        // keys per tile
constexpr int VS = KT + 4;    // V^T tile row stride in LDS (elements): 136 B

// Splits fp32 weights (two at a time) into NP BF16 terms, each the
// round-to-nearest of the exact remainder left by the previous terms.
template <int NP>
__device__ __forceinline__ void split_p(f32x2 pv, bf16x2 (&t)[3]) {
  t[0] = __builtin_convertvector(pv, bf16x2);  // round to nearest even
  if (NP >= 2) {
    const f32x2 h = __builtin_convertvector(t[0], f32x2);
    const f32x2 r = {pv[0] - h[0], pv[1] - h[1]};  // exact
    t[1] = __builtin_convertvector(r, bf16x2);
    if (NP >= 3) {
      const f32x2 l = __builtin_convertvector(t[1], f32x2);
      const f32x2 r2 = {r[0] - l[0], r[1] - l[1]};  // exact
      t[2] = __builtin_convertvector(r2, bf16x2);
    }
  }
}

// One workgroup = QB/32 waves = QB queries of one head.  Two waves per SIMD
// (<= 256 registers each): while one wave runs its softmax arithmetic the
// other keeps the matrix cores busy.  NP = BF16 terms per weight (1, 2, 3).
template <int QB, int NP, int DH>
__global__ __launch_bounds__(QB * 2, 2) void attn_kernel(AttnArgs p) {
  constexpr int KS = DH + 8;     // K tile row stride in LDS (elements)
  constexpr int CPRK = DH / 8;   // 16-byte chunks per K row
  constexpr int NT = QB * 2;  // threads
  constexpr int KCH = KT * DH / 8 / NT;  // 16-byte K chunks per thread and tile
  constexpr int VCH = DH * KT / 8 / NT;  // 16-byte V^T chunks per thread and tile
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][DH * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int h = blockIdx.y;
  const int qrow = blockIdx.x * QB + wave * 32 + l32;  // this lane's query
  const bool qvalid = qrow < p.Mq;
  // scores in exp2 units: s * log2(e) = dot * (alpha * log2(e))
  const float c = p.alpha * 1.4426950408889634f;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][kk*16 + half*8 + 0..7]
  // (rows past Mq read the last row; their outputs are not stored).
  bf16x8 qf[DH / 16];
  {
    const int qr = qvalid ? qrow : p.Mq - 1;
    const uint16_t* qp = p.q + (long)qr * p.ldq + h * DH + half * 8;
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qp + kk * 16));
  }

  // Global -> register staging of one key tile: K rows (keys) and V^T rows
  // (channels of this head), 16-byte chunks.  In full tiles every load is
  // in range; the last (ragged) tile clamps K rows (their scores are masked)
  // and zeroes V^T entries past the last key (their weights are 0 and the
  // padding of V^T is not initialised).
  uint4 rk[KCH], rv[VCH];
  const uint16_t* kbase = p.k + h * DH;
  const uint16_t* vbase = p.vt + (long)h * DH * p.ldvt;
  auto load_tile = [&](int key0, bool ragged) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int c2 = tid + i * NT;
      int key = key0 + c2 / CPRK;
      if (ragged) key = key < p.Mk ? key : p.Mk - 1;
      rk[i] = *reinterpret_cast<const uint4*>(kbase + (long)key * p.ldk + (c2 % CPRK) * 8);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      int c2 = tid + i * NT;
      int vr = c2 >> 3, vkey = key0 + (c2 & 7) * 8;
      if (!ragged) {
        rv[i] = *reinterpret_cast<const uint4*>(vbase + (long)vr * p.ldvt + vkey);
      } else {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (vkey < p.Mk) {
          v = *reinterpret_cast<const uint4*>(vbase + (long)vr * p.ldvt + vkey);
          uint16_t* e = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (vkey + t >= p.Mk) e[t] = 0;
        }
        rv[i] = v;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int c2 = tid + i * NT;
      *reinterpret_cast<uint4*>(&k_lds[buf][(c2 / CPRK) * KS + (c2 % CPRK) * 8]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      int c2 = tid + i * NT;
      uint2* dst = reinterpret_cast<uint2*>(&v_lds[buf][(c2 >> 3) * VS + (c2 & 7) * 8]);  // 8-byte aligned rows
      dst[0] = make_uint2(rv[i].x, rv[i].y);
      dst[1] = make_uint2(rv[i].z, rv[i].w);
    }
  };

  // Running maximum m (in raw dot-product units), normaliser l, and the
  // output accumulator z (= O^T), all fp32.
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[DH / 32];
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;

  // one key tile: scores, online-softmax update, P.V
  auto tile = [&](int cur, int key0, bool ragged) {
    // S^T for 64 keys x this wave's 32 queries: two 32x32 accumulator tiles.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(&k_lds[cur][(kb * 32 + l32) * KS + kk * 16 + half * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
      }
    }
    if (ragged) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + kb * 32 + 8 * (r / 4) + 4 * half + (r % 4) >= p.Mk) s[kb][r] = -INFINITY;
    }
    // tile maximum of this query (max commutes with the positive scale, so
    // it is taken on the raw dot products)
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float mc = m_new * c;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
        s[kb][r] = e;
        lsum += e;
      }
    lsum += __shfl_xor(lsum, 32);
    // rescale only when some query's maximum moved (eta = 1 exactly otherwise)
    if (__any(m_new != m_run)) {
      const float eta = __builtin_amdgcn_exp2f(m_run * c - mc);
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= eta;
      l_run *= eta;
    }
    l_run += lsum;
    m_run = m_new;

    // O^T += V^T P^T over 4 groups of 16 keys.  Slot j of a lane's B operand
    // holds score register i = (g%2)*8 + j of tile g/2, i.e. key
    // 16g + 4*half + j (j < 4) or 16g + 8 + 4*half + (j-4) (j >= 4); the A
    // operand (V^T) uses the same key for the same slot.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x8 bt[NP];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        f32x2 pv = {s[g >> 1][(g & 1) * 8 + j], s[g >> 1][(g & 1) * 8 + j + 1]};
        bf16x2 t[3];
        split_p<NP>(pv, t);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
          bt[n][j] = t[n][0];
          bt[n][j + 1] = t[n][1];
        }
      }
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) {
        const uint16_t* vr = &v_lds[cur][(dt * 32 + l32) * VS + 16 * g + 4 * half];
        uint2 x0 = *reinterpret_cast<const uint2*>(vr);
        uint2 x1 = *reinterpret_cast<const uint2*>(vr + 8);
        bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
#pragma unroll
        for (int n = 0; n < NP; ++n) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bt[n], o[dt], 0, 0, 0);
      }
    }
  };

  const int nfull = p.Mk / KT;          // tiles with every key in range
  const int ntiles = (p.Mk + KT - 1) / KT;
  load_tile(0, nfull == 0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < nfull; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) load_tile((t + 1) * KT, t + 1 >= nfull);
    tile(cur, t * KT, false);
    if (t + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }
  if (nfull < ntiles) tile(nfull & 1, nfull * KT, true);

  // O = B(z / l).  O^T layout: lane holds query qrow, channels
  // dt*32 + 8*(r/4) + 4*half + (r%4): four consecutive channels per store.
  if (qvalid) {
    uint16_t* op = p.q + (long)qrow * p.ldq + h * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c0 = dt * 32 + 8 * rg + 4 * half;
        uint16_t b0 = f2bf(o[dt][rg * 4 + 0] / l_run);
        uint16_t b1 = f2bf(o[dt][rg * 4 + 1] / l_run);
        uint16_t b2 = f2bf(o[dt][rg * 4 + 2] / l_run);
        uint16_t b3 = f2bf(o[dt][rg * 4 + 3] / l_run);
        uint2 w = make_uint2((uint32_t)b0 | ((uint32_t)b1 << 16), (uint32_t)b2 | ((uint32_t)b3 << 16));
        *reinterpret_cast<uint2*>(op + c0) = w;
      }
  }
}

// Software-pipelined variant.  The scores of key tile t+1 (S^T = K Q^T,
// 16 MFMAs) are issued before the softmax of tile t (fp32 VALU and exp2),
// so every wave always has independent matrix-core and vector work in
// flight and the two waves of a SIMD no longer alternate between an
// MFMA-only and a VALU-only phase.  K and V^T tiles are triple-buffered in
// LDS: iteration t reads K of tile t+1 and V^T of tile t while tile t+2 is
// stored.  Same arithmetic, in the same order per query, as attn_kernel.
template <int QB, int NP, int DH>
__global__ __launch_bounds__(QB * 2) void attn_kernel_pipe(AttnArgs p) {
  constexpr int KS = DH + 8;
  constexpr int CPRK = DH / 8;
  constexpr int NT = QB * 2;
  constexpr int KCH = KT * DH / 8 / NT;
  constexpr int VCH = DH * KT / 8 / NT;
  constexpr int NB = 3;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NB][KT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[NB][DH * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int h = blockIdx.y;
  const int qrow = blockIdx.x * QB + wave * 32 + l32;
  const bool qvalid = qrow < p.Mq;
  const float c = p.alpha * 1.4426950408889634f;

  bf16x8 qf[DH / 16];
  {
    const int qr = qvalid ? qrow : p.Mq - 1;
    const uint16_t* qp = p.q + (long)qr * p.ldq + h * DH + half * 8;
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qp + kk * 16));
  }

  uint4 rk[KCH], rv[VCH];
  const uint16_t* kbase = p.k + h * DH;
  const uint16_t* vbase = p.vt + (long)h * DH * p.ldvt;
  // Tile loads: K rows past Mk are clamped (their scores are masked), V^T
  // entries past Mk are zeroed (their weights are 0; the padding of V^T is
  // not initialised).
  auto load_tile = [&](int key0) {
    const bool ragged = key0 + KT > p.Mk;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int c2 = tid + i * NT;
      int key = key0 + c2 / CPRK;
      if (ragged) key = key < p.Mk ? key : p.Mk - 1;
      rk[i] = *reinterpret_cast<const uint4*>(kbase + (long)key * p.ldk + (c2 % CPRK) * 8);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      int c2 = tid + i * NT;
      int vr = c2 >> 3, vkey = key0 + (c2 & 7) * 8;
      if (!ragged) {
        rv[i] = *reinterpret_cast<const uint4*>(vbase + (long)vr * p.ldvt + vkey);
      } else {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (vkey < p.Mk) {
          v = *reinterpret_cast<const uint4*>(vbase + (long)vr * p.ldvt + vkey);
          const int keep = p.Mk - vkey;  // elements of this chunk in range (>= 1)
          uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t mlo = (2 * q < keep) ? 0x0000FFFFu : 0u;
            const uint32_t mhi = (2 * q + 1 < keep) ? 0xFFFF0000u : 0u;
            w[q] &= (mlo | mhi);
          }
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
        rv[i] = v;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int c2 = tid + i * NT;
      *reinterpret_cast<uint4*>(&k_lds[buf][(c2 / CPRK) * KS + (c2 % CPRK) * 8]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      int c2 = tid + i * NT;
      uint2* dst = reinterpret_cast<uint2*>(&v_lds[buf][(c2 >> 3) * VS + (c2 & 7) * 8]);
      dst[0] = make_uint2(rv[i].x, rv[i].y);
      dst[1] = make_uint2(rv[i].z, rv[i].w);
    }
  };
  // S^T of one tile: the two 32-key accumulator chains alternate, and the
  // K fragments of step kk+1 are read while the MFMAs of step kk run.
  auto scores = [&](int buf, f32x16 (&s)[2]) {
    const uint16_t* kr0 = &k_lds[buf][l32 * KS + half * 8];
    const uint16_t* kr1 = kr0 + 32 * KS;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[0][r] = 0.0f;
      s[1][r] = 0.0f;
    }
    bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kr0);
    bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kr1);
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) {
      bf16x8 n0 = a0, n1 = a1;
      if (kk + 1 < DH / 16) {
        n0 = *reinterpret_cast<const bf16x8*>(kr0 + (kk + 1) * 16);
        n1 = *reinterpret_cast<const bf16x8*>(kr1 + (kk + 1) * 16);
      }
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], s[1], 0, 0, 0);
      a0 = n0;
      a1 = n1;
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[DH / 32];
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;

  // softmax of tile scores s (key0: first key of the tile) and O^T += V^T P^T
  auto softmax_pv = [&](f32x16 (&s)[2], int buf, int key0) {
    if (key0 + KT > p.Mk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + kb * 32 + 8 * (r / 4) + 4 * half + (r % 4) >= p.Mk) s[kb][r] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float mc = m_new * c;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
        s[kb][r] = e;
        lsum += e;
      }
    lsum += __shfl_xor(lsum, 32);
    if (__any(m_new != m_run)) {
      const float eta = __builtin_amdgcn_exp2f(m_run * c - mc);
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= eta;
      l_run *= eta;
    }
    l_run += lsum;
    m_run = m_new;
    // P^T as B operands for the 4 groups of 16 keys, NP terms each
    bf16x8 bt[NP][4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        f32x2 pv = {s[g >> 1][(g & 1) * 8 + j], s[g >> 1][(g & 1) * 8 + j + 1]};
        bf16x2 t[3];
        split_p<NP>(pv, t);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
          bt[n][g][j] = t[n][0];
          bt[n][g][j + 1] = t[n][1];
        }
      }
    }
    // O^T += V^T P^T: per group the channel tiles' MFMAs of term 0, then of
    // term 1, ... (each accumulator still sees the terms of every group in
    // order); the V^T fragments of group g+1 are read during group g.
    auto vfrag = [&](int g, int dt) {
      const uint16_t* vr = &v_lds[buf][(dt * 32 + l32) * VS + 16 * g + 4 * half];
      uint2 x0 = *reinterpret_cast<const uint2*>(vr);
      uint2 x1 = *reinterpret_cast<const uint2*>(vr + 8);
      return __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
    };
    bf16x8 va[DH / 32];
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt) va[dt] = vfrag(0, dt);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x8 vn[DH / 32];
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) vn[dt] = g + 1 < 4 ? vfrag(g + 1, dt) : va[dt];
#pragma unroll
      for (int n = 0; n < NP; ++n)
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], bt[n][g], o[dt], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) va[dt] = vn[dt];
    }
  };

  const int ntiles = (p.Mk + KT - 1) / KT;
  load_tile(0);
  store_tile(0);
  if (ntiles > 1) {
    load_tile(KT);
    store_tile(1);
  }
  __syncthreads();
  f32x16 s_cur[2], s_nxt[2];
  scores(0, s_cur);
  for (int t = 0; t < ntiles; ++t) {
    const int b = t % NB;
    if (t + 2 < ntiles) load_tile((t + 2) * KT);
    if (t + 1 < ntiles) scores((t + 1) % NB, s_nxt);
    softmax_pv(s_cur, b, t * KT);
    if (t + 2 < ntiles) store_tile((t + 2) % NB);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_nxt[kb];
  }

  if (qvalid) {
    uint16_t* op = p.q + (long)qrow * p.ldq + h * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c0 = dt * 32 + 8 * rg + 4 * half;
        uint16_t b0 = f2bf(o[dt][rg * 4 + 0] / l_run);
        uint16_t b1 = f2bf(o[dt][rg * 4 + 1] / l_run);
        uint16_t b2 = f2bf(o[dt][rg * 4 + 2] / l_run);
        uint16_t b3 = f2bf(o[dt][rg * 4 + 3] / l_run);
        uint2 w = make_uint2((uint32_t)b0 | ((uint32_t)b1 << 16), (uint32_t)b2 | ((uint32_t)b3 << 16));
        *reinterpret_cast<uint2*>(op + c0) = w;
      }
  }
}

// Ping-pong variant.  The vector work of a key tile (mask, maximum, exp2,
// normaliser, rescale, BF16 split) and its matrix work (P.V of the tile and
// the scores of the next) are separate phases, and the two waves that share
// a SIMD run opposite phases: waves 0-3 (queries 0-127 of the workgroup)
// run the vector phase of tile t while waves 4-7 (queries 128-255) run the
// matrix phase of tile t-1 and the scores of tile t, then they swap at a
// workgroup barrier.  A SIMD's matrix core then works on one wave's MFMAs
// while its vector unit works on the other wave's softmax, where in
// attn_kernel_pipe both waves of a SIMD reach the same phase together.
// Per query the arithmetic and its order are those of attn_kernel_pipe (same
// score chains, softmax updates, split and P.V sequence per accumulator), so
// the bits are the same.
//
// Half-iteration h (one barrier after each): group A (waves 0-3) runs the
// vector phase V(t) at h = 2t and the matrix phase M(t) = P.V(t) + S(t+1) at
// h = 2t+1; group B runs S(0) at h = 0, V(t) at h = 2t+1 and M(t) at
// h = 2t+2.  Tile i's K is read at h = 2i-1 and 2i (the groups' S(i)), its
// V^T at h = 2i to 2i+2 (the groups' P.V(i), whose first fragment group each
// reads during its vector phase V(i)); three LDS buffers of each hold the
// tiles.  Group A stages K: the global loads of K(i) at the start of
// its M(i-2) (h = 2i-3), the LDS stores at the end of its V(i-1)
// (h = 2i-2), after K(i-3) was last read at h = 2i-6.  Group B stages V^T
// the same way one half-iteration later: loads at the start of its M(i-2)
// (h = 2i-2), stores at the end of its V(i-1) (h = 2i-1), after V^T(i-3)
// was last read at h = 2i-4.  Each group runs its own loop (2 ntiles + 2
// barriers in both), so that the compiler allocates registers for one
// group's phases at a time.
template <int NP, int DH>
__global__ __launch_bounds__(512) void attn_kernel_pp(AttnArgs p) {
  constexpr int QB = 256;
  constexpr int KS = DH + 8;
  constexpr int CPRK = DH / 8;
  constexpr int NT = QB;                  // the 256 threads of one group stage a part
  constexpr int KCH = KT * DH / 8 / NT;   // 16-byte K chunks per thread of group A
  constexpr int VCH = DH * KT / 8 / NT;   // 16-byte V^T chunks per thread of group B
  constexpr int NB = 3;
  constexpr int KSTEPS = DH / 16;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NB][KT * KS];
  // V^T rows of 72 elements (144 B: 16-byte aligned, 16 lanes reading
  // 16 bytes each at row stride 36 banks touch all 64 banks once)
  constexpr int VP = KT + 8;
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[NB][DH * VP];

  const int tid = threadIdx.x;
  const int gtid = tid & (NT - 1);  // thread index inside its group
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool group_a = wave < 4;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int h = blockIdx.y;
  const int qrow = blockIdx.x * QB + wave * 32 + l32;
  const bool qvalid = qrow < p.Mq;
  const float c = p.alpha * 1.4426950408889634f;

  bf16x8 qf[KSTEPS];
  {
    const int qr = qvalid ? qrow : p.Mq - 1;
    const uint16_t* qp = p.q + (long)qr * p.ldq + h * DH + half * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qp + kk * 16));
  }

  // Tile staging as attn_kernel_pipe's, split by operand: K rows past Mk are
  // clamped (their scores are masked), V^T entries past Mk are zeroed.
  uint4 rs[KCH > VCH ? KCH : VCH];
  const uint16_t* kbase = p.k + h * DH;
  const uint16_t* vbase = p.vt + (long)h * DH * p.ldvt;
  // Byte offsets of this thread's chunks inside a full tile, so that a tile
  // costs one wave-uniform base address (scalar arithmetic) plus these.
  uint32_t koff[KCH > VCH ? KCH : VCH];
#pragma unroll
  for (int i = 0; i < (KCH > VCH ? KCH : VCH); ++i) {
    const int c2 = gtid + i * NT;
    koff[i] = group_a ? (uint32_t)(((long)(c2 / CPRK) * p.ldk + (c2 % CPRK) * 8) * 2)
                      : (uint32_t)(((long)(c2 >> 3) * p.ldvt + (c2 & 7) * 8) * 2);
  }
  auto load_k = [&](int key0) {
    if (key0 + KT <= p.Mk) {
      const char* base = reinterpret_cast<const char*>(kbase + (long)key0 * p.ldk);
#pragma unroll
      for (int i = 0; i < KCH; ++i) rs[i] = *reinterpret_cast<const uint4*>(base + koff[i]);
      return;
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int c2 = gtid + i * NT;
      int key = key0 + c2 / CPRK;
      key = key < p.Mk ? key : p.Mk - 1;
      rs[i] = *reinterpret_cast<const uint4*>(kbase + (long)key * p.ldk + (c2 % CPRK) * 8);
    }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int c2 = gtid + i * NT;
      *reinterpret_cast<uint4*>(&k_lds[buf][(c2 / CPRK) * KS + (c2 % CPRK) * 8]) = rs[i];
    }
  };
  auto load_v = [&](int key0) {
    if (key0 + KT <= p.Mk) {
      const char* base = reinterpret_cast<const char*>(vbase + key0);
#pragma unroll
      for (int i = 0; i < VCH; ++i) rs[i] = *reinterpret_cast<const uint4*>(base + koff[i]);
      return;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      int c2 = gtid + i * NT;
      int vr = c2 >> 3, vkey = key0 + (c2 & 7) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (vkey < p.Mk) {
        v = *reinterpret_cast<const uint4*>(vbase + (long)vr * p.ldvt + vkey);
        const int keep = p.Mk - vkey;
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t mlo = (2 * q < keep) ? 0x0000FFFFu : 0u;
          const uint32_t mhi = (2 * q + 1 < keep) ? 0xFFFF0000u : 0u;
          w[q] &= (mlo | mhi);
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
      rs[i] = v;
    }
  };
  // Within each 16-key group the V^T row holds the keys in the order of the
  // P^T operand's lanes: keys 0-3 and 8-11 (read by lanes 0-31), then 4-7
  // and 12-15 (lanes 32-63), so that one fragment is one 16-byte read.  A
  // chunk of 8 keys starting at an even multiple of 8 puts keys 0-3 at
  // positions 0-3 and 4-7 at 8-11; an odd one puts 8-11 at 4-7 and 12-15
  // at 12-15.
  auto store_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      int c2 = gtid + i * NT;
      uint16_t* row = &v_lds[buf][(c2 >> 3) * VP + ((c2 & 7) >> 1) * 16 + (c2 & 1) * 4];
      *reinterpret_cast<uint2*>(row) = make_uint2(rs[i].x, rs[i].y);
      *reinterpret_cast<uint2*>(row + 8) = make_uint2(rs[i].z, rs[i].w);
    }
  };
  auto kfrag = [&](int buf, int kb, int kk) {
    return *reinterpret_cast<const bf16x8*>(&k_lds[buf][(kb * 32 + l32) * KS + kk * 16 + half * 8]);
  };
  auto vfrag = [&](int buf, int g, int dt) {
    return *reinterpret_cast<const bf16x8*>(&v_lds[buf][(dt * 32 + l32) * VP + 16 * g + 8 * half]);
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 o[DH / 32];
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  f32x16 s[2];
  bf16x8 bt[NP][4];

  // The matrix phase runs one wave's MFMAs with no other MFMA stream on its
  // SIMD to hide LDS latency behind, so fragments are read well ahead: the
  // reads of P.V group g+1 are issued with the MFMAs of group g, the K
  // fragments of score step kk+KPF before the MFMAs of step kk (held there
  // by sched_barrier fences), and the first V^T group during the vector
  // phase.  Fencing the P.V reads as well measured slower with three terms.
  constexpr int KPF = KSTEPS < 3 ? KSTEPS : 3;  // score steps read ahead
  auto fence = []() { __builtin_amdgcn_sched_barrier(0); };

  // S^T of the tile in buffer kb: the two 32-key chains alternate (as in
  // attn_kernel_pipe); f holds the fragments of steps 0 .. KPF-1 on entry
  auto scores = [&](int kb, bf16x8 (&f)[KPF][2]) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int cur = kk % KPF;
      const bf16x8 a0 = f[cur][0], a1 = f[cur][1];
      if (kk + KPF < KSTEPS) {
        f[cur][0] = kfrag(kb, 0, kk + KPF);
        f[cur][1] = kfrag(kb, 1, kk + KPF);
      }
      fence();
      if (kk == 0) {
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], f32x16{}, 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], f32x16{}, 0, 0, 0);
      } else {
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], s[1], 0, 0, 0);
      }
      fence();
    }
  };

  // vector phase of the tile starting at key0: the online-softmax update and
  // the BF16 terms of the weights (attn_kernel_pipe's arithmetic, in order);
  // va receives group 0 of the V^T tile in buffer vb for the next matrix phase
  auto vector_phase = [&](int key0, int vb, bf16x8 (&va)[DH / 32]) {
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt) va[dt] = vfrag(vb, 0, dt);
    fence();
    if (key0 + KT > p.Mk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + kb * 32 + 8 * (r / 4) + 4 * half + (r % 4) >= p.Mk) s[kb][r] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float mc = m_new * c;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
        s[kb][r] = e;
        lsum += e;
      }
    lsum += __shfl_xor(lsum, 32);
    if (__any(m_new != m_run)) {
      const float eta = __builtin_amdgcn_exp2f(m_run * c - mc);
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= eta;
      l_run *= eta;
    }
    l_run += lsum;
    m_run = m_new;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        f32x2 pv = {s[g >> 1][(g & 1) * 8 + j], s[g >> 1][(g & 1) * 8 + j + 1]};
        bf16x2 t[3];
        split_p<NP>(pv, t);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
          bt[n][g][j] = t[n][0];
          bt[n][g][j + 1] = t[n][1];
        }
      }
    }
  };
  // matrix phase: O^T += V^T P^T of the tile in buffer vb (attn_kernel_pipe's
  // MFMA order per accumulator; va holds its group 0), then the scores of
  // the tile in buffer kb.  Without a next tile kb = vb: the scores are
  // computed from a valid buffer and never used, so that the phase has no
  // branch.
  auto matrix_phase = [&](int vb, int kb, bf16x8 (&va)[DH / 32]) {
    bf16x8 kf[KPF][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x8 vn[DH / 32];
      if (g + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt) vn[dt] = vfrag(vb, g + 1, dt);
      } else {
#pragma unroll
        for (int kk = 0; kk < KPF; ++kk) {
          kf[kk][0] = kfrag(kb, 0, kk);
          kf[kk][1] = kfrag(kb, 1, kk);
        }
      }
#pragma unroll
      for (int n = 0; n < NP; ++n)
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], bt[n][g], o[dt], 0, 0, 0);
      if (g + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < DH / 32; ++dt) va[dt] = vn[dt];
      }
    }
    scores(kb, kf);
  };
  // the stores of this half-iteration are visible after it
  auto barrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  const int ntiles = (p.Mk + KT - 1) / KT;
  // tiles 0 and 1: K by group A, V^T by group B
  if (group_a) {
    load_k(0);
    store_k(0);
    if (ntiles > 1) {
      load_k(KT);
      store_k(1);
    }
  } else {
    load_v(0);
    store_v(0);
    if (ntiles > 1) {
      load_v(KT);
      store_v(1);
    }
  }
  barrier();
  {
    bf16x8 kf[KPF][2];
#pragma unroll
    for (int kk = 0; kk < KPF; ++kk) {
      kf[kk][0] = kfrag(0, 0, kk);
      kf[kk][1] = kfrag(0, 1, kk);
    }
    bf16x8 va[DH / 32];
    if (group_a) {
      scores(0, kf);
      for (int t = 0; t < ntiles; ++t) {
        vector_phase(t * KT, t % NB, va);                     // h = 2t
        if (t >= 1 && t + 1 < ntiles) store_k((t + 1) % NB);  // loaded in M(t-1)
        barrier();
        if (t + 2 < ntiles) load_k((t + 2) * KT);             // h = 2t+1
        matrix_phase(t % NB, t + 1 < ntiles ? (t + 1) % NB : t % NB, va);
        barrier();
      }
      barrier();  // h = 2 ntiles: group B's last matrix phase
    } else {
      scores(0, kf);  // h = 0
      barrier();
      for (int t = 0; t < ntiles; ++t) {
        vector_phase(t * KT, t % NB, va);                     // h = 2t+1
        if (t >= 1 && t + 1 < ntiles) store_v((t + 1) % NB);  // loaded in M(t-1)
        barrier();
        if (t + 2 < ntiles) load_v((t + 2) * KT);             // h = 2t+2
        matrix_phase(t % NB, t + 1 < ntiles ? (t + 1) % NB : t % NB, va);
        barrier();
      }
    }
  }

  if (qvalid) {
    uint16_t* op = p.q + (long)qrow * p.ldq + h * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c0 = dt * 32 + 8 * rg + 4 * half;
        uint16_t b0 = f2bf(o[dt][rg * 4 + 0] / l_run);
        uint16_t b1 = f2bf(o[dt][rg * 4 + 1] / l_run);
        uint16_t b2 = f2bf(o[dt][rg * 4 + 2] / l_run);
        uint16_t b3 = f2bf(o[dt][rg * 4 + 3] / l_run);
        uint2 w = make_uint2((uint32_t)b0 | ((uint32_t)b1 << 16), (uint32_t)b2 | ((uint32_t)b3 << 16));
        *reinterpret_cast<uint2*>(op + c0) = w;
      }
  }
}

template <int QB, int NP, int DH>
hipError_t launch_pipe(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.Mq + QB - 1) / QB, a.heads);
  return launch_kernel(attn_kernel_pipe<QB, NP, DH>, grid, dim3(QB * 2), s, a);
}

template <int NP, int DH>
hipError_t launch_pp(const AttnArgs& a, hipStream_t s) {
  // the kernel addresses a tile's chunks by 32-bit byte offsets
  if ((long)KT * a.ldk * 2 >= (1L << 32) || (long)DH * a.ldvt * 2 >= (1L << 32))
    return launch_pipe<256, NP, DH>(a, s);
  dim3 grid((a.Mq + 255) / 256, a.heads);
  return launch_kernel(attn_kernel_pp<NP, DH>, grid, dim3(512), s, a);
}

template <int QB, int NP, int DH>
hipError_t launch_q(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.Mq + QB - 1) / QB, a.heads);
  return launch_kernel(attn_kernel<QB, NP, DH>, grid, dim3(QB * 2), s, a);
}

template <int NP, int DH>
hipError_t launch_cfg(const AttnArgs& a, int cfg, hipStream_t s) {
  switch (cfg) {
    case 2: return launch_q<256, NP, DH>(a, s);
    case 3: return launch_pipe<256, NP, DH>(a, s);
    case 4: return launch_pp<NP, DH>(a, s);
    default: return launch_q<128, NP, DH>(a, s);
  }
}

template <int DH>
hipError_t launch_dh(const AttnArgs& a, int cfg, hipStream_t s) {
  switch (a.p_terms) {
    case 1: return launch_cfg<1, DH>(a, cfg, s);
    case 2: return launch_cfg<2, DH>(a, cfg, s);
    case 3: return launch_cfg<3, DH>(a, cfg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.Mq <= 0) return hipSuccess;
  if (a.Mk <= 0) return hipErrorInvalidValue;  // softmax over no keys
  // 256-query workgroups (8 waves sharing each K/V tile, the two wave
  // groups in ping-pong) when there are at least 512 keys or the grid gives
  // every CU a workgroup, else 128-query ones (measured on MI355X: with 8 or
  // more key tiles the ping-pong kernel is faster even on grids of 64
  // workgroups; with fewer, more and smaller workgroups win unless the grid
  // is large).  Configurations: 1 = 128-query, 2 = 256-query, 3 = 256-query
  // pipelined in lock step, 4 = 256-query ping-pong; all give identical
  // bits.  Head dimension 128 or 64.
  int cfg = a.config;
  if (cfg == 0) cfg = (a.Mk >= 512 || ((a.Mq + 255) / 256) * a.heads >= 256) ? 4 : 1;
  if (a.dh == 64) return launch_dh<64>(a, cfg, s);
  if (a.dh != 128) return hipErrorInvalidValue;
  return launch_dh<128>(a, cfg, s);
}

}  // namespace psi
