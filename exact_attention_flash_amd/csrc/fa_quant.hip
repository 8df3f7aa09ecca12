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
// not of its fp32 rounding: see e4m3_ready_quotient).  Three launches: clear
// the amax word, reduce amax|y| (atomic max on the fp32 bits, which order
// like the values for y >= 0), then recompute y and write the codes; block
// 0 of the last launch writes the descale.
//
// Layout: a row of d bf16 values is handled by d / 8 consecutive lanes, 8
// values (16 bytes) each.  The fast Walsh-Hadamard transform runs its first
// three butterfly levels inside a lane and the rest across lanes with XOR
// shuffles (lane distance 1, 2, 4, 8).  Memory-bound: 2 bytes read per
// element in each of the two passes, 1 byte written.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct QuantCfg {
  static constexpr int L = D / 8;          // lanes per row
  static constexpr int NT = 256;           // threads per workgroup
  static constexpr int RPB = NT / L;       // rows per workgroup
};

// y for the 8 values of lane position lr (0 .. D/8 - 1) of a row.  Every
// lane of the wave must call it (the shuffles are wave-wide); lanes without a
// row pass zeros.
template <int D>
__device__ __forceinline__ void load_rotate(const QuantArgs& a, int64_t row, int lr, float v[8]) {
  constexpr int L = D / 8;
  if (row < a.rows) {
    const u32x4 w = load_global<u32x4>(a.x + row * D + 8 * lr);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32((uint16_t)(w[j] & 0xffffu));
      v[2 * j + 1] = bf16_to_f32((uint16_t)(w[j] >> 16));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  if (a.signs == nullptr) return;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] *= a.signs[8 * lr + e];
  // butterflies over index bits 0..2 (inside the lane)
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((e & h) == 0) {
        const float x0 = v[e], x1 = v[e + h];
        v[e] = x0 + x1;
        v[e + h] = x0 - x1;
      }
  // bits 3.. log2(D) - 1: the partner lane holds the other half of each pair;
  // the lane with the bit clear keeps the sum, the other the difference
#pragma unroll
  for (int m = 1; m < L; m <<= 1) {
    const bool upper = (lr & m) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __shfl_xor(v[e], m, 64);
      v[e] = upper ? p - v[e] : v[e] + p;
    }
  }
  constexpr float kInvSqrtD = D == 128 ? 0.08838834764831845f : 0.125f;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] *= kInvSqrtD;
}

// The E4M3 rounding (nearest even) of the exact quotient v / ds, returned as
// an fp32 value whose own nearest-even E4M3 rounding is that code.  q = v / ds
// rounded to fp32 lands on the same side of every E4M3 midpoint as the exact
// quotient, or on the midpoint itself; in that case the remainder
// v - q ds (exact through the FMA) tells on which side the quotient lies, and
// q moves one ulp that way so that the conversion does not see a tie.
__device__ __forceinline__ float e4m3_ready_quotient(float v, float ds) {
  float q = v / ds;
  const float r = fmaf(-q, ds, v);
  const uint32_t b = __float_as_uint(q);
  const uint32_t mag = b & 0x7fffffffu;
  bool mid;
  if (mag >= 0x3c800000u) {          // |q| >= 2^-6: normal E4M3 range
    mid = (mag & 0xfffffu) == 0x80000u;  // the mantissa bits below E4M3's three are 100..0
  } else {                           // subnormal range: midpoints are odd multiples of 2^-10
    const float t = fabsf(q) * 1024.f;
    mid = t == rintf(t) && (((int)t) & 1);
  }
  if (mid && r != 0.f) q = __uint_as_float((r > 0.f) == (q > 0.f) ? b + 1u : b - 1u);
  return q;
}

__global__ void fa_quant_clear_kernel(QuantArgs a) { *a.amax = 0u; }

template <int D>
__global__ void __launch_bounds__(256) fa_quant_amax_kernel(QuantArgs a) {
  using C = QuantCfg<D>;
  const int64_t row = (int64_t)blockIdx.x * C::RPB + threadIdx.x / C::L;
  const int lr = threadIdx.x % C::L;
  float v[8];
  load_rotate<D>(a, row, lr, v);
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(a.amax, __float_as_uint(m));
}

template <int D>
__global__ void __launch_bounds__(256) fa_quant_codes_kernel(QuantArgs a) {
  using C = QuantCfg<D>;
  const int64_t row = (int64_t)blockIdx.x * C::RPB + threadIdx.x / C::L;
  const int lr = threadIdx.x % C::L;
  float v[8];
  load_rotate<D>(a, row, lr, v);
  const float amax = __uint_as_float(*a.amax);
  const float descale = amax > 0.f ? amax / 448.f : 1.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.descale = descale;
  if (row >= a.rows) return;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(e4m3_ready_quotient(v[e], descale), -448.f), 448.f);
  u32x2 out;
  out.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
      y[2], y[3], __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false), true);
  out.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
      y[6], y[7], __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false), true);
  *reinterpret_cast<u32x2*>(a.codes + row * D + 8 * lr) = out;
}

template <int D>
static hipError_t launch_quant_t(const QuantArgs& a, hipStream_t stream) {
  using C = QuantCfg<D>;
  const int64_t grid = (a.rows + C::RPB - 1) / C::RPB;
  hipLaunchKernelGGL(fa_quant_clear_kernel, dim3(1), dim3(1), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_quant_amax_kernel<D>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((fa_quant_codes_kernel<D>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const QuantArgs& a, int d, hipStream_t stream) {
  return d == 64 ? launch_quant_t<64>(a, stream) : launch_quant_t<128>(a, stream);
}

}  // namespace fa
