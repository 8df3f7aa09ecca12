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
// not of an fp32 rounding of it: see e4m3_ready_quotient).  Three launches: clear
// the amax word, reduce amax|y| (atomic max on the fp32 bits, which order
// like the values for y >= 0), then recompute y and write the codes; block
// 0 of the last launch writes the descale.  The amax pass strides over the
// rows with a bounded grid and issues one atomic per workgroup.
//
// Layout: a row of d bf16 values is handled by 4 consecutive lanes, d / 4
// values each (contiguous, so a wave reads 16 whole rows).  The fast
// Walsh-Hadamard transform runs all but its two top butterfly levels inside
// a lane and those two with XOR shuffles inside a quad (lane distance 1, 2).
// Memory-bound: 2 bytes read per element in each of the two passes, 1 byte
// written.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct QuantCfg {
  static constexpr int L = 4;              // lanes per row
  static constexpr int E = D / L;          // values per lane
  static constexpr int NT = 256;           // threads per workgroup
  static constexpr int RPB = NT / L;       // rows per workgroup
};

// The value of lane (lane ^ m) for m = 1 or 2: a DPP quad permutation
// (quad_perm [1,0,3,2] or [2,3,0,1]), a plain VALU move.
__device__ __forceinline__ float quad_xor(float x, int m) {
  const int r = m == 1 ? __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)
                       : __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false);
  return __int_as_float(r);
}

// y for the E values of lane position lr (0 .. 3) of a row.  Every lane of
// the wave must call it (the shuffles are wave-wide); lanes without a row
// pass zeros.
template <int D>
__device__ __forceinline__ void load_rotate(const QuantArgs& a, int64_t row, int lr,
                                            float v[QuantCfg<D>::E]) {
  constexpr int E = QuantCfg<D>::E;
  if (row < a.rows) {
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      const u32x4 w = load_global<u32x4>(a.x + row * D + E * lr + 8 * c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * c + 2 * j] = bf16_to_f32((uint16_t)(w[j] & 0xffffu));
        v[8 * c + 2 * j + 1] = bf16_to_f32((uint16_t)(w[j] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = 0.f;
  }
  if (a.signs == nullptr) return;
#pragma unroll
  for (int c = 0; c < E / 4; ++c) {
    const f32x4 sg = load_global<f32x4>(a.signs + E * lr + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * c + e] *= sg[e];
  }
  // butterflies over the index bits inside the lane
#pragma unroll
  for (int h = 1; h < E; h <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((e & h) == 0) {
        const float x0 = v[e], x1 = v[e + h];
        v[e] = x0 + x1;
        v[e + h] = x0 - x1;
      }
  // the two top index bits are the lane position: the partner lane (xor 1,
  // then xor 2, inside a quad) holds the other half of each pair; the lane
  // with the bit clear keeps the sum, the other the difference
#pragma unroll
  for (int m = 1; m < 4; m <<= 1) {
    const bool upper = (lr & m) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float p = quad_xor(v[e], m);
      v[e] = upper ? p - v[e] : v[e] + p;
    }
  }
  constexpr float kInvSqrtD = D == 128 ? 0.08838834764831845f : 0.125f;
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] *= kInvSqrtD;
}

// The E4M3 rounding (nearest even) of the exact quotient v / ds, returned as
// an fp32 value whose own nearest-even E4M3 rounding is that code.
// q = v * inv (inv = 1 / ds rounded) is within two ulps of the quotient, so
// unless q lies within a few ulps of an E4M3 midpoint it is on the same side
// of every midpoint as the quotient and converts to the right code.  Near a
// midpoint the sign of v - mid * ds (exact through the FMA) tells on which
// side the quotient lies (or that it is the midpoint), and q is set one ulp
// that way from the midpoint (or to it, a true tie).  Below the normal E4M3
// range (|q| < 2^-6, midpoints at odd multiples of 2^-10) the same test runs
// on the correctly rounded division.
__device__ __forceinline__ float e4m3_ready_quotient(float v, float ds, float inv) {
  float q = v * inv;
  const uint32_t b = __float_as_uint(q);
  const uint32_t mag = b & 0x7fffffffu;
  // normal range, branch-free: mantissa bits below E4M3's top three read
  // 100..0 at a midpoint
  const float mid = __uint_as_float((b & 0xfff00000u) | 0x80000u);
  const float r = fmaf(-mid, ds, v);
  const uint32_t mb = __float_as_uint(mid);
  const float qm = r == 0.f ? mid : __uint_as_float((r > 0.f) == (mid > 0.f) ? mb + 1u : mb - 1u);
  q = (mag & 0xfffffu) - 0x7fffcu <= 8u ? qm : q;
  const bool sub = mag < 0x3c800000u;
  if (__builtin_amdgcn_ballot_w64(sub)) {  // wave-uniform; rare for amax-scaled data
    if (sub) {
      q = v / ds;
      const float rr = fmaf(-q, ds, v);
      const uint32_t bq = __float_as_uint(q);
      const float t = fabsf(q) * 1024.f;
      if (t == rintf(t) && (((int)t) & 1) && rr != 0.f)
        q = __uint_as_float((rr > 0.f) == (q > 0.f) ? bq + 1u : bq - 1u);
    }
  }
  return q;
}

__global__ void fa_quant_clear_kernel(QuantArgs a) { *a.amax = 0u; }

// Grid-stride over row blocks (the stride is uniform per workgroup, so every
// wave runs the same iterations and reaches every shuffle), then one atomic
// per workgroup: atomics on one address serialise in L2.
template <int D>
__global__ void __launch_bounds__(256) fa_quant_amax_kernel(QuantArgs a) {
  using C = QuantCfg<D>;
  __shared__ float wmax[C::NT / 64];
  const int lr = threadIdx.x % C::L;
  float m = 0.f;
  for (int64_t r0 = (int64_t)blockIdx.x * C::RPB; r0 < a.rows; r0 += (int64_t)gridDim.x * C::RPB) {
    float v[C::E];
    load_rotate<D>(a, r0 + threadIdx.x / C::L, lr, v);
#pragma unroll
    for (int e = 0; e < C::E; ++e) m = fmaxf(m, fabsf(v[e]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int i = 1; i < C::NT / 64; ++i) b = fmaxf(b, wmax[i]);
    atomicMax(a.amax, __float_as_uint(b));
  }
}

// Workgroups of the amax pass: enough to fill the chip several times over.
constexpr int64_t kQuantAmaxGrid = 2048;

template <int D>
__global__ void __launch_bounds__(256) fa_quant_codes_kernel(QuantArgs a) {
  using C = QuantCfg<D>;
  const int64_t row = (int64_t)blockIdx.x * C::RPB + threadIdx.x / C::L;
  const int lr = threadIdx.x % C::L;
  float v[C::E];
  load_rotate<D>(a, row, lr, v);
  const float amax = __uint_as_float(*a.amax);
  const float descale = amax > 0.f ? amax / 448.f : 1.f;
  const float inv = 1.f / descale;
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.descale = descale;
  if (row >= a.rows) return;
#pragma unroll
  for (int c = 0; c < C::E / 16; ++c) {
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = fminf(fmaxf(e4m3_ready_quotient(v[16 * c + 4 * j + e], descale, inv), -448.f),
                     448.f);
      out[j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
          y[2], y[3], __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false), true);
    }
    *reinterpret_cast<u32x4*>(a.codes + row * D + C::E * lr + 16 * c) = out;
  }
}

template <int D>
static hipError_t launch_quant_t(const QuantArgs& a, hipStream_t stream) {
  using C = QuantCfg<D>;
  const int64_t grid = (a.rows + C::RPB - 1) / C::RPB;
  hipLaunchKernelGGL(fa_quant_clear_kernel, dim3(1), dim3(1), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_quant_amax_kernel<D>), dim3((unsigned)min(grid, kQuantAmaxGrid)),
                     dim3(C::NT), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((fa_quant_codes_kernel<D>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const QuantArgs& a, int d, hipStream_t stream) {
  return d == 64 ? launch_quant_t<64>(a, stream) : launch_quant_t<128>(a, stream);
}

}  // namespace fa
