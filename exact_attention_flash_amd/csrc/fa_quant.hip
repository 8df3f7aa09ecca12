// FP8 (E4M3) quantisation of Q or K for the FP8 forward, with optional
// incoherent processing.
//
// "FlashAttention 系列技术详解" (FlashAttention-3 section) lowers the
// quantisation error by multiplying the queries and keys by a random
// orthogonal matrix, a Hadamard transform, which spreads large entries over
// all coordinates and costs O(d log d) per row.  Here that matrix is
// M = diag(signs) H_d / sqrt(d) (H_d the Sylvester Hadamard matrix, the
// signs given by the caller); Q M (K M)^T = Q K^T, so the attention is
// unchanged up to rounding, and V is quantised without it.
//
// Per tensor: y = x M (or y = x), descale = amax|y| / 448 (fp32),
// codes = E4M3(y / descale), round to nearest even (of the exact quotient,
// not of an fp32 rounding of it).  Two launches:
//   amax pass  - every workgroup strides over row blocks and writes the
//                largest |y| it saw to its own workspace slot (no atomics:
//                atomics on one address serialise, about 11 ns each);
//   codes pass - every workgroup reduces the slots, derives the descale,
//                recomputes y and writes the codes; block 0 writes the
//                descale.
//
// Layout: a wave handles 16 rows; lane l takes row l % 16 and the d / 4
// contiguous values at position l / 16 of it.  The fast Walsh-Hadamard
// transform runs all but two butterfly levels inside a lane; the other two
// pair lanes 16 and 32 apart through v_permlane16_swap / v_permlane32_swap,
// which exchange half-waves of two registers at once: after the swap every
// lane holds both halves of one butterfly (for one of the two registers)
// and all lanes run the same add and subtract.  The swap trades a lane bit
// for a register bit, so the output indices come out permuted (see
// out_index).  Memory-bound in principle (2 bytes read per element in each
// pass, 1 byte written); the VALU work, about 9 (amax) and 14 (codes)
// operations per element, sits close to what the HBM time allows.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct QuantCfg {
  static constexpr int E = D / 4;          // values per lane
  static constexpr int LOGE = D == 128 ? 5 : 4;
  static constexpr int NT = 256;           // threads per workgroup
  static constexpr int RPB = 64;           // rows per workgroup and step
  // 1 / sqrt(d), the scale of M
  static constexpr float kInvSqrtD = D == 128 ? 0.08838834764831845f : 0.125f;
};

// Sign bits of the rotation for the E / 2 packed bf16 pairs of lane
// position lp: XOR-ing them into the raw words multiplies by the signs.
template <int D, bool ROT>
__device__ __forceinline__ void load_sign_masks(const QuantArgs& a, int lp,
                                                uint32_t mask[QuantCfg<D>::E / 2]) {
  constexpr int E = QuantCfg<D>::E;
#pragma unroll
  for (int c = 0; c < E / 4; ++c) {
    if (!ROT) {
      mask[2 * c] = mask[2 * c + 1] = 0u;
      continue;
    }
    const f32x4 s = load_global<f32x4>(a.signs + E * lp + 4 * c);
    mask[2 * c] = ((__float_as_uint(s[0]) >> 16) & 0x8000u) | (__float_as_uint(s[1]) & 0x80000000u);
    mask[2 * c + 1] =
        ((__float_as_uint(s[2]) >> 16) & 0x8000u) | (__float_as_uint(s[3]) & 0x80000000u);
  }
}

template <int D>
__device__ __forceinline__ void load_row(const QuantArgs& a, int64_t row, int lp,
                                         uint32_t w[QuantCfg<D>::E / 2]) {
  constexpr int E = QuantCfg<D>::E;
#pragma unroll
  for (int c = 0; c < E / 8; ++c) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (row < a.rows) z = load_global<u32x4>(a.x + row * D + E * lp + 8 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) w[4 * c + j] = z[j];
  }
}

// v = (x M) sqrt(d) (or v = x) for the E values of the lane.  Every lane of
// the wave must call it (the swaps are wave-wide); lanes without a row pass
// zero words.  Index bits of x M held by lane l, slot e (T = log2 E - 1):
//   bits 0 .. T-2 : slot bits 0 .. T-2
//   bit T-1       : lane bit 5            bit T   : lane bit 4
//   bit T+1       : slot bit T            bit T+2 : slot bit T-1
// (without rotation, index = E * (l / 16) + e).
template <int D, bool ROT>
__device__ __forceinline__ void rotate_row(const uint32_t w[QuantCfg<D>::E / 2],
                                           const uint32_t mask[QuantCfg<D>::E / 2],
                                           float v[QuantCfg<D>::E]) {
  constexpr int E = QuantCfg<D>::E;
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    const uint32_t t = w[i] ^ mask[i];
    v[2 * i] = __uint_as_float(t << 16);
    v[2 * i + 1] = __uint_as_float(t & 0xffff0000u);
  }
  if (!ROT) return;
#pragma unroll
  for (int h = 1; h < E; h <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((e & h) == 0) {
        const float x0 = v[e], x1 = v[e + h];
        v[e] = x0 + x1;
        v[e + h] = x0 - x1;
      }
  // lane bit 4 (index bit T+1) against slot bit T: v_permlane16_swap(X, Y)
  // leaves in every lane the (lane bit 4 = 0, = 1) pair of X (even 16-lane
  // rows) or of Y (odd rows)
#pragma unroll
  for (int e = 0; e < E / 2; ++e) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[e]),
                                                    __float_as_uint(v[e + E / 2]), false, false);
    const float x0 = __uint_as_float(r[0]), x1 = __uint_as_float(r[1]);
    v[e] = x0 + x1;
    v[e + E / 2] = x0 - x1;
  }
  // lane bit 5 (index bit T+2) against slot bit T-1, the same way
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((e & (E / 4)) == 0) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[e]),
                                                      __float_as_uint(v[e + E / 4]), false, false);
      const float x0 = __uint_as_float(r[0]), x1 = __uint_as_float(r[1]);
      v[e] = x0 + x1;
      v[e + E / 4] = x0 - x1;
    }
}

// Row offset of the run of E / 4 consecutive slots starting at slot s
// (s a multiple of E / 4) of lane l: E / 4 consecutive indices.
template <int D, bool ROT>
__device__ __forceinline__ int out_index(int s, int l) {
  constexpr int E = QuantCfg<D>::E;
  if (!ROT) return E * (l >> 4) + s;
  const int b4 = (l >> 4) & 1, b5 = (l >> 5) & 1;
  const int sT = (s / (E / 2)) & 1, sT1 = (s / (E / 4)) & 1;
  return (E / 4) * b5 + (E / 2) * b4 + E * sT + 2 * E * sT1;
}

// The E4M3 rounding (nearest even) of the exact quotient y / ds, returned as
// an fp32 value whose own nearest-even E4M3 rounding is that code.
// q = y * inv (inv = 1 / ds rounded) is within two ulps of the quotient, so
// unless q lies within a few ulps of an E4M3 midpoint it is on the same side
// of every midpoint as the quotient and converts to the right code.  Near a
// midpoint the sign of y - mid * ds (exact through the FMA) tells on which
// side the quotient lies (or that it is the midpoint), and q is set one ulp
// that way from the midpoint (or to it, a true tie).  Below the normal E4M3
// range (|q| < 2^-6, midpoints at odd multiples of 2^-10) the same test runs
// on the correctly rounded division.  Used only for the rare values whose
// code the fast path cannot settle.
__device__ __forceinline__ float e4m3_ready_quotient(float y, float ds, float inv) {
  float q = y * inv;
  const uint32_t b = __float_as_uint(q);
  const uint32_t mag = b & 0x7fffffffu;
  // normal range: mantissa bits below E4M3's top three read 100..0 at a
  // midpoint
  const float mid = __uint_as_float((b & 0xfff00000u) | 0x80000u);
  const float r = fmaf(-mid, ds, y);
  const uint32_t mb = __float_as_uint(mid);
  const float qm = r == 0.f ? mid : __uint_as_float((r > 0.f) == (mid > 0.f) ? mb + 1u : mb - 1u);
  q = (mag & 0xfffffu) - 0x7fffcu <= 8u ? qm : q;
  if (mag < 0x3c800000u) {
    q = y / ds;
    const float rr = fmaf(-q, ds, y);
    const uint32_t bq = __float_as_uint(q);
    const float t = fabsf(q) * 1024.f;
    if (t == rintf(t) && (((int)t) & 1) && rr != 0.f)
      q = __uint_as_float((rr > 0.f) == (q > 0.f) ? bq + 1u : bq - 1u);
  }
  return q;
}

// Four E4M3 codes (nearest even, the first value in the low byte).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false),
                                                   true);
}

// Largest |v| of a wave, in every lane.
__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  return m;
}

// Each workgroup strides over row blocks (the stride is uniform per
// workgroup, so every wave runs the same iterations and reaches every swap)
// with the next block's words loaded before the current one is processed.
template <int D, bool ROT>
__global__ void __launch_bounds__(256) fa_quant_amax_kernel(QuantArgs a) {
  using C = QuantCfg<D>;
  __shared__ float wmax[C::NT / 64];
  const int l = threadIdx.x & 63, lp = l >> 4;
  const int64_t stride = (int64_t)gridDim.x * C::RPB;
  const int64_t row0 = (int64_t)blockIdx.x * C::RPB + (threadIdx.x >> 6) * 16 + (l & 15);
  uint32_t mask[C::E / 2], w[C::E / 2];
  load_row<D>(a, row0, lp, w);
  load_sign_masks<D, ROT>(a, lp, mask);
  float m = 0.f;
  for (int64_t r0 = (int64_t)blockIdx.x * C::RPB; r0 < a.rows; r0 += stride) {
    uint32_t wn[C::E / 2];
    load_row<D>(a, row0 + (r0 - (int64_t)blockIdx.x * C::RPB) + stride, lp, wn);
    float v[C::E];
    rotate_row<D, ROT>(w, mask, v);
#pragma unroll
    for (int e = 0; e < C::E; ++e) m = fmaxf(m, fabsf(v[e]));
#pragma unroll
    for (int i = 0; i < C::E / 2; ++i) w[i] = wn[i];
  }
  m = wave_max(m);
  if (l == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int i = 1; i < C::NT / 64; ++i) b = fmaxf(b, wmax[i]);
    a.part[blockIdx.x] = b;  // max |x M| sqrt(d), or max |x|
  }
}

template <int D, bool ROT>
__global__ void __launch_bounds__(256) fa_quant_codes_kernel(QuantArgs a) {
  using C = QuantCfg<D>;
  const int l = threadIdx.x & 63, lp = l >> 4;
  const int64_t stride = (int64_t)gridDim.x * C::RPB;
  const int64_t row0 = (int64_t)blockIdx.x * C::RPB + (threadIdx.x >> 6) * 16 + (l & 15);
  uint32_t mask[C::E / 2], w[C::E / 2];
  load_row<D>(a, row0, lp, w);
  load_sign_masks<D, ROT>(a, lp, mask);
  // every wave reduces the partial maxima itself (no barrier): lane l
  // takes slots 4 l .. 4 l + 3 and 256 + 4 l .. 256 + 4 l + 3
  float m = 0.f;
#pragma unroll
  for (int h = 0; h < kQuantParts / 256; ++h) {
    const int i = 256 * h + 4 * l;
    if (i < a.parts) {
      const f32x4 p = load_global<f32x4>(a.part + i);
#pragma unroll
      for (int k = 0; k < 4; ++k) m = i + k < a.parts ? fmaxf(m, p[k]) : m;
    }
  }
  m = wave_max(m);
  // y = v c; rounding is monotone, so max fl(|v| c) = fl(max |v| c)
  const float c = ROT ? C::kInvSqrtD : 1.f;
  const float amax = m * c;
  const float descale = amax > 0.f ? amax / 448.f : 1.f;
  const float inv = 1.f / descale;
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.descale = descale;
  const float cinv = c * inv;
  // The fast path takes q = v cinv, within 4.0001 units of 2^-24 (relative)
  // of the quotient fl(v c) / ds.  If q (1 - 2^-21) and q (1 + 2^-21) have
  // q's code they bracket the quotient inside one rounding interval, so q's
  // code is its code; otherwise (a value at or near a code boundary) the
  // exact path decides, element by element.  Such values are not rare
  // without rotation: when amax has a short mantissa, x / ds sits at or
  // next to a midpoint for a fixed subset of bf16 mantissas (0.5 - 6 % of
  // the elements).  q stays below 448 (1 + 2^-20), which rounds to 448: no
  // saturation is needed.
  constexpr float kLo = 1.f - 1.f / (1 << 21), kHi = 1.f + 1.f / (1 << 21);
  for (int64_t r0 = (int64_t)blockIdx.x * C::RPB; r0 < a.rows; r0 += stride) {
    const int64_t row = row0 + (r0 - (int64_t)blockIdx.x * C::RPB);
    uint32_t wn[C::E / 2];
    load_row<D>(a, row + stride, lp, wn);
    float v[C::E];
    rotate_row<D, ROT>(w, mask, v);
#pragma unroll
    for (int i = 0; i < C::E / 2; ++i) w[i] = wn[i];
    uint32_t out[C::E / 4], dif[C::E / 4];  // dif: non-zero bytes need the exact path
    uint32_t anyd = 0u;
#pragma unroll
    for (int j = 0; j < C::E / 4; ++j) {
      float q[4], lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // fma with +0 turns the -0 of cancelled sums into +0, as an exact
        // rotation gives; without rotation x's own -0 is kept
        q[e] = ROT ? fmaf(v[4 * j + e], cinv, 0.f) : v[4 * j + e] * cinv;
        lo[e] = q[e] * kLo;
        hi[e] = q[e] * kHi;
      }
      out[j] = e4m3x4(q[0], q[1], q[2], q[3]);
      dif[j] = (e4m3x4(lo[0], lo[1], lo[2], lo[3]) ^ out[j]) |
               (e4m3x4(hi[0], hi[1], hi[2], hi[3]) ^ out[j]);
      anyd |= dif[j];
    }
    if (__builtin_amdgcn_ballot_w64(anyd != 0u)) {
#pragma unroll
      for (int j = 0; j < C::E / 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool be = ((dif[j] >> (8 * b)) & 0xffu) != 0u;
          if (__builtin_amdgcn_ballot_w64(be) && be) {
            const float y = ROT ? fmaf(v[4 * j + b], c, 0.f) : v[4 * j + b];
            const float q = e4m3_ready_quotient(y, descale, inv);
            const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0xffu;
            out[j] = (out[j] & ~(0xffu << (8 * b))) | (code << (8 * b));
          }
        }
    }
    if (row < a.rows) {
      uint8_t* dst = a.codes + row * D;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int off = out_index<D, ROT>(s4 * (C::E / 4), l);
        if constexpr (D == 128) {
          const u32x2 o = {out[2 * s4], out[2 * s4 + 1]};
          *reinterpret_cast<u32x2*>(dst + off) = o;
        } else {
          *reinterpret_cast<uint32_t*>(dst + off) = out[s4];
        }
      }
    }
  }
}

// Workgroups of each pass: enough to fill the chip several times over; each
// strides over row blocks, so the per-workgroup set-up (rotation signs,
// partial maxima) is paid a few times per workgroup rather than per block.
constexpr int64_t kQuantCodesGrid = 1024;
static_assert(kQuantParts % 256 == 0, "the codes pass reads the partials 256 at a time");

template <int D, bool ROT>
static hipError_t launch_quant_t(const QuantArgs& a0, hipStream_t stream) {
  using C = QuantCfg<D>;
  const int64_t blocks = (a0.rows + C::RPB - 1) / C::RPB;
  QuantArgs a = a0;
  a.parts = (int)min(blocks, (int64_t)kQuantParts);
  hipLaunchKernelGGL((fa_quant_amax_kernel<D, ROT>), dim3((unsigned)a.parts), dim3(C::NT), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_quant_codes_kernel<D, ROT>), dim3((unsigned)min(blocks, kQuantCodesGrid)),
                     dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const QuantArgs& a, int d, hipStream_t stream) {
  if (a.signs)
    return d == 64 ? launch_quant_t<64, true>(a, stream) : launch_quant_t<128, true>(a, stream);
  return d == 64 ? launch_quant_t<64, false>(a, stream) : launch_quant_t<128, false>(a, stream);
}

}  // namespace fa
