// FP8 attention forward for gfx950: Q, K, V as OCP E4M3 codes with one
// dequantisation factor per tensor; O (bf16) and LSE (fp32) as in the bf16
// forward.
//
// Method: the same FlashAttention-2 forward as the bf16 kernel (CMU notes
// "Transformer、注意力机制与优化", sections "FlashAttention-2 算法" and
// "安全 Softmax 与在线 Softmax"), with both matrix products in FP8, which
// "FlashAttention 系列技术详解" lists among the FlashAttention-3 changes
// (hardware low-precision GEMM, FP8 doubling matrix throughput).  On gfx950
// both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32
// accumulate, unit block scales), twice the bf16 MFMA rate:
//  * S^T = K Q^T: exact products of E4M3 values summed in fp32, then scaled
//    by softmax_scale * descale_q * descale_k * log2(e) inside the softmax;
//  * O^T += V^T P^T: the probabilities are rounded to E4M3 for the product.
//    They are taken as 2^4 * 2^(s - m) with a running max m that is moved
//    only when a tile's max exceeds it by more than 2^4, so every value lies
//    in (0, 2^8] (E4M3 reaches 448) and values down to 2^-14 of the max
//    keep a nonzero code.  The row sum l adds the unrounded fp32 values, so
//    LSE carries no rounding from the FP8 probabilities; O = descale_v *
//    acc / l.
//
// gfx950 mapping: the ping-pong structure of the bf16 forward (one workgroup
// = 8 waves = 256 query rows, 32 per wave; waves w and w + 4 share a SIMD
// and alternate a matrix phase with a softmax phase, half a period apart),
// with tiles of BC = 128 keys (16 KB for d = 128, 8 KB for d = 64) in three
// K and three V buffers; the larger tile than the bf16 kernel's halves the
// per-key cost of the period's fixed work (barriers, branches, copy issue),
// which matters here because the softmax phase, not the matrix phase, sets
// the period.  MFMA operands (lane l = 32 g + c):
//  * A (K rows): lane (c, g) holds 32 bytes of row c; B (Q^T): lane holds 32
//    bytes of its query's row; byte j of the A lane pairs with byte j of the
//    B lane of the same g (measured: any k order shared by both operands
//    gives the product).  So K is read with two ds_read_b128 per operand
//    from row-major tiles, Q stays in registers, and S^T lane (c, g) value i
//    of 32-key block sb is key 32 sb + 8 (i / 4) + 4 g + i % 4;
//  * P^T (B) is those values, rounded and packed in that same order: byte j
//    of 64-key slice ps is key 64 ps + 32 (j / 16) + 8 ((j % 16) / 4) + 4 g
//    + j % 4;
//  * V^T (A) must list the same keys: ds_read_b64_tr_b8 transposes an
//    8-row x 16-byte block per group of 16 lanes, each lane supplying one
//    row address, so each lane points at exactly the key rows its group
//    needs and four such reads make one 32-byte operand;
//  * the K tile swizzles its 16-byte chunks by row bits 1-3 (d = 128) or
//    2-3 (d = 64), the V tile its 32-byte segments by row bits 1 and 3
//    (d = 128) or 3 (d = 64), which keeps both kinds of operand read free of
//    bank conflicts under the LDS lane grouping measured on this chip (four
//    cycles of 16 lanes for 16-byte reads, two cycles of 32 lanes for
//    transposed reads).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E4M3 (format 0) and
// both block scales 2^0 (E8M0 exponent 127).
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join8(const i32x4& lo, const i32x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed LDS read of 8-bit elements (ds_read_b64_tr_b8): within each
// group of 16 lanes, lane 2 r + h supplies the address of 8 bytes (row r of
// an 8-row block, byte half h of 16 columns); lane i of the group receives
// byte i % 8 of the run supplied by lane 2 r + i / 8, for r = 0..7, i.e.
// column i of the block.
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// Four fp32 values rounded to E4M3 (nearest even) into the bytes of one
// word, a in byte 0 .. d in byte 3.  The first conversion keeps bytes 2-3 of
// its `old` operand, which the second one overwrites, so any register does
// (here a's own, which needs no copy).
__device__ __forceinline__ int cvt_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int D>
struct Fp8Cfg {
  static constexpr int NW = 8;                  // waves per workgroup
  static constexpr int NT = NW * 64;            // threads per workgroup
  static constexpr int QW = 32;                 // query rows per wave
  static constexpr int BR = NW * QW;            // query rows per workgroup
  static constexpr int BC = 128;                // keys per K/V tile
  static constexpr int CPR = D / 16;            // 16-byte chunks per row
  static constexpr int TILE = BC * D;           // bytes per tile
  static constexpr int COPIES = TILE / 16 / NT; // 16-byte copies per thread per tile
  static constexpr int KS = D / 64;             // 64-deep slices of S^T = K Q^T
  static constexpr int SB = BC / 32;            // 32-key blocks of S^T
  static constexpr int PS = BC / 64;            // 64-key slices of O^T += V^T P^T
  static constexpr int DB = D / 32;             // 32-column blocks of O^T
  static_assert(COPIES >= 1 && COPIES * 16 * NT == TILE, "tile copies must split evenly");
};

// Growth of the probabilities (log2 units) tolerated before the running max
// moves, and the power of two they are multiplied by before rounding:
// 2^(kP + threshold) = 256 stays inside E4M3's range.
constexpr float kFp8RescaleThreshold = 4.f;
constexpr float kFp8PExp = 4.f;

// Chunk (K) and 32-byte segment (V) swizzles of the row-major tiles.
template <int D>
__device__ __forceinline__ int fp8_k_swizzle(int r) {
  return D == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int fp8_v_swizzle(int r) {
  return D == 128 ? ((r >> 1) & 1) | (((r >> 3) & 1) << 1) : (r >> 3) & 1;
}

// Per-lane source offsets of the tile copies: lane `lane` of wave w fills
// 16-byte slot 64 w + lane of a tile (row r = slot / CPR, physical chunk
// slot % CPR) with the logical chunk that the swizzle puts there.  A tile
// that runs past the end of the sequence clamps its rows to N - 1 (finite
// data for keys that are masked anyway).
template <int D>
struct Fp8TileCopy {
  using C = Fp8Cfg<D>;
  uint32_t koff[C::COPIES], voff[C::COPIES];

  __device__ __forceinline__ static int slot_row(int t, int w, int lane) {
    return ((t * C::NW + w) * 64 + lane) / C::CPR;
  }

  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int t = 0; t < C::COPIES; ++t) {
      const int slot = (t * C::NW + w) * 64 + lane;
      const int r = slot / C::CPR, pc = slot % C::CPR;
      koff[t] = r * D + 16 * (pc ^ fp8_k_swizzle<D>(r));
      voff[t] = r * D + 16 * (pc ^ (fp8_v_swizzle<D>(r) << 1));
    }
  }

  template <bool KEYS>
  __device__ __forceinline__ void issue(const uint8_t* X, uint8_t* Ts, int k0, int N, int w,
                                        int lane) const {
    // the resource is rebuilt from the laundered head pointer at each issue,
    // so that its words do not sit in scalar registers across the loop
    const i32x4 rs = make_rsrc_words(opaque_s(X) + (int64_t)k0 * D, C::TILE);
    const int wb = opaque_s(w * 64 * 16);  // this wave's slots
    if (k0 + C::BC <= N) {
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t)
        buffer_load_lds16_unseen(rs, KEYS ? koff[t] : voff[t], Ts + t * C::NW * 64 * 16 + wb);
    } else {
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t) {
        const int r = opaque(slot_row(t, w, lane));
        const uint32_t shift = (uint32_t)((min(k0 + r, N - 1) - (k0 + r)) * D);
        buffer_load_lds16_unseen(rs, (KEYS ? koff[t] : voff[t]) + shift,
                                 Ts + t * C::NW * 64 * 16 + wb);
      }
    }
  }
};

struct Fp8Smem {
  uint8_t* k[3];
  uint8_t* v[3];
};

template <int D, bool CAUSAL>
struct Fp8Wave {
  using C = Fp8Cfg<D>;
  static constexpr int BC = C::BC;

  Fp8Smem sm;
  const uint8_t* Kh;
  const uint8_t* Vh;
  int w, grp, lane, c32, g, N, qw0, qrow;
  int t0, nt, ntw;
  float sl2;
  float m_run;   // running max of the scaled log2 scores (possibly stale)
  float l_part;  // this lane's share of the running row sum (times 2^kP)
  i32x8 qf[C::KS];      // Q^T operand: bytes 64 kc + 32 g + 0..31 of qrow
  f32x16 oacc[C::DB];   // O^T: lane holds O[qrow][32 db + 8(i/4) + 4g + i%4]
  f32x16 s[C::SB];
  i32x8 pb[C::PS];
  int kb;  // K operand read: row c32, logical chunk 2 g, swizzled (bytes)
  int vb;  // V operand read: the lane's row and 8-byte half, swizzled (bytes)
  Fp8TileCopy<D> cp;

  template <int KB>
  __device__ __forceinline__ void scores() {
    const uint8_t* Ks = sm.k[KB];
    const int b = opaque(kb);
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb) s[sb] = zero16();
#pragma unroll
    for (int kc = 0; kc < C::KS; ++kc)
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb) {
        const uint8_t* row = Ks + sb * 32 * D;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(row + (b ^ (16 * (4 * kc))));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(row + (b ^ (16 * (4 * kc + 1))));
        s[sb] = mfma_fp8(join8(lo, hi), qf[kc], s[sb]);
      }
    sched_pipeline<C::KS * C::SB, 2, 1, 2>();
  }

  template <int VB>
  __device__ __forceinline__ void pv() {
    const uint8_t* Vs = sm.v[VB];
    const int b = opaque(vb);
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        i32x2 r[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          r[t] = lds_read_tr8(Vs + (64 * ps + 32 * (t >> 1) + 16 * (t & 1)) * D + (b ^ (32 * db)));
        i32x8 a;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          a[2 * t] = r[t][0];
          a[2 * t + 1] = r[t][1];
        }
        oacc[db] = mfma_fp8(a, pb[ps], oacc[db]);
      }
    sched_pipeline<C::PS * C::DB, 4, 1, 2>();
  }

  template <int KB, int VB>
  __device__ __forceinline__ void matrix_phase(int t) {
    const bool do_s = t < ntw;
    const bool do_pv = t >= 1 && t - 1 < ntw;
    if (do_s) scores<KB>();
    if (do_pv) pv<VB>();
  }

  __device__ __forceinline__ void softmax_phase(int t) {
    if (t < 0 || t >= ntw) return;
    const int k0 = (t0 + t) * BC;
    const bool need_mask = (k0 + BC > N) || (CAUSAL && (k0 + BC - 1 > qw0));
    if (need_mask) {
      // key k0 + 32 sb + 8 (i / 4) + 4 g + i % 4 is visible iff its offset
      // from k0 + 4 g is <= lim
      // The select is bit arithmetic on a sign mask kept opaque, so that it
      // stays in vector registers instead of 64 live compare masks in scalar
      // register pairs.
      const int lim = opaque((CAUSAL ? min(N - 1, qrow) : N - 1) - k0 - 4 * g);
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t hide = (uint32_t)opaque((lim - (32 * sb + 8 * (i >> 2) + (i & 3))) >> 31);
          s[sb][i] = __uint_as_float((__float_as_uint(s[sb][i]) & ~hide) | (0xff800000u & hide));
        }
    }
    // row max in four independent chains (a single chain of dependent
    // v_max3 is latency bound)
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i) m4[i & 3] = fmaxf(m4[i & 3], s[sb][i]);
    float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    mx = max_halves(mx) * sl2;
    if (__ballot(mx > m_run + kFp8RescaleThreshold)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    const float m_use = (m_run == -INFINITY ? 0.f : m_run) - kFp8PExp;
    float rs = 0.f;
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps)
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int sb = 2 * ps + (wd >> 2), i0 = 4 * (wd & 3);
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = exp2_fast(fmaf(s[sb][i0 + e], sl2, -m_use));
          rs += p[e];
        }
        pb[ps][wd] = cvt_e4m3x4(p[0], p[1], p[2], p[3]);
      }
    l_part += rs;
  }

  // One period of the ping-pong schedule; see the bf16 forward for the
  // buffer rotation.  Unlike there, a barrier separates the two slots: the
  // softmax phase is the longer one here, and without the barrier the two
  // groups' softmax phases overlap on the SIMD's vector unit (5% slower on
  // causal B=4 H=16 N=4096 d=128).
  template <int R, int GRP>
  __device__ __forceinline__ void period(int t) {
    constexpr int KB = R, VB = (R + 2) % 3, KN = (R + 2) % 3, VN = (R + 1) % 3;
    const bool kn = t + 2 < nt, vn = t + 1 < nt;
    if (GRP == 0) {
      matrix_phase<KB, VB>(t);
    } else {
      if (kn) cp.template issue<true>(Kh, sm.k[KN], (t0 + t + 2) * BC, N, w, lane);
      if (vn) cp.template issue<false>(Vh, sm.v[VN], (t0 + t + 1) * BC, N, w, lane);
      softmax_phase(t - 1);
    }
    block_barrier();
    if (GRP == 0) {
      if (kn) cp.template issue<true>(Kh, sm.k[KN], (t0 + t + 2) * BC, N, w, lane);
      if (vn) cp.template issue<false>(Vh, sm.v[VN], (t0 + t + 1) * BC, N, w, lane);
      softmax_phase(t);
    } else {
      matrix_phase<KB, VB>(t);
    }
    if (kn) wait_vmem_except_last<2 * C::COPIES>();
    else if (vn) wait_vmem_except_last<C::COPIES>();
    else wait_vmem();
    block_barrier();
  }

  template <int GRP>
  __device__ __forceinline__ void run() {
    for (int t = 0; t <= nt; t += 3) {
      period<0, GRP>(t);
      if (t + 1 > nt) break;
      period<1, GRP>(t + 1);
      if (t + 2 > nt) break;
      period<2, GRP>(t + 2);
    }
  }
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_fp8_kernel(Fp8FwdArgs a) {
  using C = Fp8Cfg<D>;
  constexpr int TILE = C::TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t k0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t k1s[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t k2s[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v1s[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v2s[TILE];

  const int tid = threadIdx.x;
  const int N = a.N;
  const int nqb = (N + C::BR - 1) / C::BR;

  // per-lane constants, the same for every item
  Fp8Wave<D, CAUSAL> f;
  f.sm = Fp8Smem{{k0s, k1s, k2s}, {v0s, v1s, v2s}};
  f.w = __builtin_amdgcn_readfirstlane(tid >> 6);
  f.grp = f.w >> 2;
  f.lane = tid & 63;
  f.c32 = f.lane & 31;
  f.g = f.lane >> 5;
  f.N = N;
  f.t0 = 0;
  f.sl2 = a.scale_log2;
  f.kb = f.c32 * D + 16 * ((2 * f.g) ^ fp8_k_swizzle<D>(f.c32));
  {
    // lane 16 u + 2 jj + h of the transposed V reads: group u = (g, column
    // half), key row 8 (jj / 4) + 4 g + jj % 4 of the block, byte half h
    const int i16 = f.lane & 15, jj = i16 >> 1, h = i16 & 1, dh = (f.lane >> 4) & 1;
    const int r = 8 * (jj >> 2) + 4 * f.g + (jj & 3);
    f.vb = r * D + 16 * dh + 8 * h + 32 * fp8_v_swizzle<D>(r);
  }
  f.cp.init(f.w, f.lane);

  // Item (head bh, query block qb): its fields with a fresh running max and
  // sum, the copies of K tiles 0 and 1 and V tile 0, and Q into registers.
  auto begin = [&](int bh, int qb) {
    const int64_t hoff = (int64_t)bh * N * D;
    f.Kh = a.k + hoff;
    f.Vh = a.v + hoff;
    const int q0 = qb * C::BR;
    f.qw0 = q0 + (2 * (f.w & 3) + f.grp) * C::QW;
    f.qrow = f.qw0 + f.c32;
    int nt_all = (N + C::BC - 1) / C::BC;
    if (CAUSAL) nt_all = min(nt_all, (q0 + C::BR + C::BC - 1) / C::BC);
    f.nt = nt_all;
    f.ntw = CAUSAL ? min(nt_all, (f.qw0 + C::QW + C::BC - 1) / C::BC) : nt_all;
    asm volatile("" : "+s"(f.ntw));  // keep the per-tile tests: knowing ntw == nt hoists more
    f.m_run = -INFINITY;
    f.l_part = 0.f;
    f.cp.template issue<true>(f.Kh, k0s, 0, N, f.w, f.lane);
    if (f.nt > 1) f.cp.template issue<true>(f.Kh, k1s, C::BC, N, f.w, f.lane);
    f.cp.template issue<false>(f.Vh, v0s, 0, N, f.w, f.lane);
    const uint8_t* Qh = a.q + hoff;
#pragma unroll
    for (int kc = 0; kc < C::KS; ++kc) {
      if (f.qrow < N) {
        const uint8_t* src = Qh + (int64_t)f.qrow * D + 64 * kc + 32 * f.g;
        f.qf[kc] = join8(load_global<i32x4>(src), load_global<i32x4>(src + 16));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.qf[kc][e] = 0;
      }
    }
  };
  // O = descale_v * acc / l; LSE = (m - kP + log2 l) ln 2 (both acc and l
  // carry the factor 2^kP).
  auto finish = [&](int bh, int row, float l, float m) {
    if (row >= N) return;
    const float inv = a.descale_v / l;
    uint16_t* Orow = a.o + (int64_t)bh * N * D + (int64_t)row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 val;
        val.x = pack2(f.oacc[db][4 * r4 + 0] * inv, f.oacc[db][4 * r4 + 1] * inv);
        val.y = pack2(f.oacc[db][4 * r4 + 2] * inv, f.oacc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2*>(Orow + db * 32 + 8 * r4 + 4 * f.g) = val;
      }
    if (f.g == 0) a.lse[(int64_t)bh * N + row] = (m - kFp8PExp + log2_fast(l)) * kLn2;
  };

  // Persistent: the grid walks the (head, query block) items in run order
  // (heads grouped per XCD, heaviest causal query blocks first); the next
  // item's first copies and Q loads overlap the current item's epilogue.
  const ItemWalk walk{(int)blockIdx.x, (int)gridDim.x, a.BH * nqb};
  int bh, qb;
  xcd_head_block<kHeadsPerGroup>(walk.item(0), walk.total, a.BH, nqb, bh, qb);
  begin(bh, CAUSAL ? nqb - 1 - qb : qb);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) f.oacc[db] = zero16();
  wait_vmem();
  block_barrier();
  for (int r = 1;; ++r) {
    // fresh copies of the per-lane constants each item, so that nothing
    // derived from them is hoisted out of the item loop and held across it
    f.kb = opaque(f.kb);
    f.vb = opaque(f.vb);
#pragma unroll
    for (int t = 0; t < C::COPIES; ++t) {
      f.cp.koff[t] = (uint32_t)opaque((int)f.cp.koff[t]);
      f.cp.voff[t] = (uint32_t)opaque((int)f.cp.voff[t]);
    }
    if (f.grp == 0) f.template run<0>();
    else f.template run<1>();
    const float l = sum_halves(f.l_part);
    const float m = f.m_run;
    const int cur_bh = bh, cur_row = f.qrow;
    const int L = walk.item(r);
    if (L >= 0) {
      xcd_head_block<kHeadsPerGroup>(L, walk.total, a.BH, nqb, bh, qb);
      begin(bh, CAUSAL ? nqb - 1 - qb : qb);
    }
    finish(cur_bh, cur_row, l, m);
    if (L < 0) break;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) f.oacc[db] = zero16();
    // the previous item's scores and probabilities are dead: say so
#pragma unroll
    for (int sb = 0; sb < C::SB; ++sb) f.s[sb] = zero16();
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps)
#pragma unroll
      for (int e = 0; e < 8; ++e) f.pb[ps][e] = 0;
    wait_vmem();
    block_barrier();
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_fp8_t(const Fp8FwdArgs& a, hipStream_t stream) {
  using C = Fp8Cfg<D>;
  const int64_t nqb = (a.N + C::BR - 1) / C::BR;
  // persistent: one workgroup per CU (the kernel's registers allow no more)
  const int64_t grid = persistent_grid(nqb * a.BH);
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_fwd_fp8_t<64, true>(a, stream) : launch_fwd_fp8_t<64, false>(a, stream);
  return causal ? launch_fwd_fp8_t<128, true>(a, stream) : launch_fwd_fp8_t<128, false>(a, stream);
}

}  // namespace fa
