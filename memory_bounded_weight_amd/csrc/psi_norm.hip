// psi_norm.hip -- full-row RMS normalisation and split rotary embedding of
// the query/key projections, in place, gfx950.
//
// [PSI] sec. II-B ("Precision-Preserving Subtensor Inference for a 22B Joint
// Audio-Video Generator under a Fixed GPU Working Set", arXiv 2611.08023):
//   * full-row RMS: y_i = gamma_i x_i / sqrt(s/d + eps), where the sum of
//     squares s is taken over the WHOLE row of width d as a sum over column
//     tiles J of the tile partial sums, and every tile uses the same single
//     positive denominator;
//   * split RoPE: inside each head of width dh the pair
//     (a, b) = (x_j, x_{j+dh/2}), j < dh/2, becomes (c a - s b, s a + c b),
//     with the cosine/sine of the pair's table index.
// Each is a declared BF16 write: the normalised row is rounded to BF16 and
// the rotation reads those rounded values (then rounds again).
//
// Memory-bound (one read and one write of the row, plus a re-read that hits
// the cache): one wave per row, 16-byte loads, the row's sum of squares in
// fp32 -- per lane, then a fixed xor-butterfly across the wave per tile,
// then the tile partials added in ascending tile order.
#include "psi_internal.h"

namespace psi {
namespace {

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to bfloat16, nearest with ties to even (finite values; NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float v) {
  uint32_t w = __float_as_uint(v);
  if ((w & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  w += 0x7FFFu + ((w >> 16) & 1u);
  return (uint16_t)(w >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void unpack8(const uint4& u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const uint16_t (&b)[8]) {
  return make_uint4((uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16),
                    (uint32_t)b[4] | ((uint32_t)b[5] << 16), (uint32_t)b[6] | ((uint32_t)b[7] << 16));
}

constexpr int kRowsPerBlock = 4;  // one wave per row

__global__ __launch_bounds__(64 * kRowsPerBlock) void qk_norm_rope_kernel(NormRopeArgs p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= p.M) return;  // whole wave; the kernel has no barriers
  uint16_t* xr = p.x + (long)row * p.ldx;

  // one denominator for the whole row
  float den = 1.0f;
  if (p.gamma) {
    float s = 0.0f;
    for (int j0 = 0; j0 < p.d; j0 += p.tile) {
      const int j1 = min(j0 + p.tile, p.d);
      float part = 0.0f;
      for (int c = j0 + lane * 8; c < j1; c += 64 * 8) {  // tile widths are multiples of 8
        float f[8];
        unpack8(*reinterpret_cast<const uint4*>(xr + c), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) part = __builtin_fmaf(f[i], f[i], part);
      }
      s += wave_sum(part);
    }
    den = __fsqrt_rn(s / (float)p.d + p.eps);
  }

  // pairs (j, j + dh/2) of each head, 8 consecutive j per lane
  const int hh = p.dh / 2;
  const int per_head = hh / 8;
  const int npairs = p.d / 16;
  const float* cs = p.cs ? p.cs + (long)row * hh : nullptr;
  const float* sn = p.sn ? p.sn + (long)row * hh : nullptr;
  for (int pc = lane; pc < npairs; pc += 64) {
    const int h = pc / per_head;
    const int j = (pc - h * per_head) * 8;
    const int ca = h * p.dh + j, cb = ca + hh;
    float a[8], b[8];
    unpack8(*reinterpret_cast<const uint4*>(xr + ca), a);
    unpack8(*reinterpret_cast<const uint4*>(xr + cb), b);
    uint16_t ua[8], ub[8];
    if (p.gamma) {
      float ga[8], gb[8];
      unpack8(*reinterpret_cast<const uint4*>(p.gamma + ca), ga);
      unpack8(*reinterpret_cast<const uint4*>(p.gamma + cb), gb);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // gamma*x is exact in fp32 (two 8-bit significands); one division
        ua[i] = f2bf(__fdiv_rn(ga[i] * a[i], den));
        ub[i] = f2bf(__fdiv_rn(gb[i] * b[i], den));
        a[i] = bf2f(ua[i]);
        b[i] = bf2f(ub[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ua[i] = f2bf(a[i]);
        ub[i] = f2bf(b[i]);
      }
    }
    if (cs) {
      const float4 c0 = *reinterpret_cast<const float4*>(cs + j);
      const float4 c1 = *reinterpret_cast<const float4*>(cs + j + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(sn + j);
      const float4 s1 = *reinterpret_cast<const float4*>(sn + j + 4);
      const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ua[i] = f2bf(__builtin_fmaf(c[i], a[i], -(sv[i] * b[i])));
        ub[i] = f2bf(__builtin_fmaf(sv[i], a[i], c[i] * b[i]));
      }
    }
    *reinterpret_cast<uint4*>(xr + ca) = pack8(ua);
    *reinterpret_cast<uint4*>(xr + cb) = pack8(ub);
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(const NormRopeArgs& a, hipStream_t s) {
  if (a.M <= 0 || (!a.gamma && !a.cs)) return hipSuccess;
  const dim3 grid((a.M + kRowsPerBlock - 1) / kRowsPerBlock);
  return launch_kernel(qk_norm_rope_kernel, grid, dim3(64 * kRowsPerBlock), s, a);
}

}  // namespace psi
