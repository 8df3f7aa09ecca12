// Fused attention backward for gfx950 (recompute from the stored LSE).
//
// Method ("FlashAttention 的基本原理", section 2.4; "FlashAttention 系列技术
// 详解", section "反向传播步骤"; CMU 15-442/642 notes, section
// "为什么前向和反向的并行化策略不同"): the scores are recomputed block by
// block, and because LSE is known the probabilities P = exp(scale*S - LSE)
// are final at once, with no running max.  Then
//   dV += P^T dO,   dP = dO V^T,   dS = P o (dP - D),   D_i = sum_c dO_ic O_ic,
//   dK += scale * dS^T Q,   dQ += scale * dS K.
// The work is split over key blocks (each workgroup owns one K/V block and
// accumulates its dK, dV in registers); every key block adds into the same
// dQ rows, so dQ is accumulated in an fp32 buffer with atomic adds and
// converted to bf16 at the end, as the CMU notes describe.
//
// Three kernels on the caller's stream:
//   fa_bwd_pre   D = rowsum(dO o O), LSE * log2(e), dQ accumulator := 0
//   fa_bwd_main  one workgroup per (batch, head, 128-key block)
//   fa_bwd_dq    dQ = bf16(scale * dQ accumulator)
//
// gfx950 mapping of fa_bwd_main (4 waves, wave w owns keys 32w .. 32w+31 of
// the block; query blocks of 64 rows are streamed through LDS):
//  * S = Q K^T and dP = dO V^T come out of v_mfma_f32_32x32x16_bf16 with a
//    lane owning one key and 16 queries; Q and dO rows sit in LDS in swap23
//    order so those 16 queries are two runs of eight consecutive rows;
//  * in that layout P and dS, rounded to bf16, are directly the B operands
//    of dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T staged transposed);
//  * dQ needs dS with keys as the contraction index, so dS goes through LDS
//    once; each wave then computes a 32-column slice of dS K against K^T
//    (kept in LDS for the workgroup's lifetime) and adds it into the fp32
//    accumulator: a lane owns one column, so each atomic instruction covers
//    whole 128-byte row segments.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// ------------------------------------------------------------------ pre pass
template <int D>
__global__ void __launch_bounds__(256) fa_bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;       // threads per row (16-byte chunks)
  constexpr int RPB = 256 / TPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int ch = tid % TPR;
  const int64_t rows = (int64_t)a.BH * a.N;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = load_global<u32x4>(a.o + row * D + ch * 8);
    const u32x4 d = load_global<u32x4>(a.dout + row * D + ch * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(bf16_to_f32((uint16_t)(o[j] & 0xffffu)), bf16_to_f32((uint16_t)(d[j] & 0xffffu)), acc);
      acc = fmaf(bf16_to_f32((uint16_t)(o[j] >> 16)), bf16_to_f32((uint16_t)(d[j] >> 16)), acc);
    }
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(a.dq_acc + row * D + ch * 8) = z;
    *reinterpret_cast<f32x4*>(a.dq_acc + row * D + ch * 8 + 4) = z;
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && ch == 0) {
    a.delta[row] = acc;
    a.lse2[row] = a.lse[row] * kLog2e;
  }
}

// ------------------------------------------------------------------ main pass
template <int D>
struct BwdCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int KW = 32;            // keys per wave
  static constexpr int BCK = NW * KW;      // keys per workgroup
  static constexpr int BRQ = 64;           // queries per iteration
  static constexpr int QP = D + 8;         // Q / dO row-major pitch
  static constexpr int TP = BRQ + 8;       // Q^T / dO^T pitch
  static constexpr int SP = BCK + 8;       // dS pitch ([query][key])
  static constexpr int KTP = BCK + 8;      // K^T pitch ([d][key])
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) fa_bwd_main_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int BRQ = C::BRQ, BCK = C::BCK, QP = C::QP, TP = C::TP, SP = C::SP, KTP = C::KTP;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BRQ * QP];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[BRQ * QP];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TP];
  __shared__ __attribute__((aligned(16))) uint16_t dOt[D * TP];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[BRQ * SP];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * KTP];
  __shared__ __attribute__((aligned(16))) float lse_s[BRQ];
  __shared__ __attribute__((aligned(16))) float del_s[BRQ];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, c32 = lane & 31, g = lane >> 5;
  const int N = a.N;
  const int nkb = (N + BCK - 1) / BCK;

  // Workgroup -> (head, key block), XCD-contiguous like the forward pass.
  // Causal key blocks near the start see the most query blocks, so the
  // natural order is already heaviest first.
  const int total = gridDim.x;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int bh = L / nkb;
  const int kb = L - bh * nkb;
  const int kb0 = kb * BCK;
  const int kw0 = kb0 + w * C::KW;
  const int key = kw0 + c32;  // the key this lane owns

  const int64_t hoff = (int64_t)bh * N * D;
  const uint16_t* Qh = a.q + hoff;
  const uint16_t* dOh = a.dout + hoff;
  const float* lse2h = a.lse2 + (int64_t)bh * N;
  const float* delh = a.delta + (int64_t)bh * N;
  float* dQh = a.dq_acc + hoff;

  // K and V of this lane's key as B operands (K[key][16 kc + 8 g + 0..7]).
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    const int64_t off = hoff + (int64_t)key * D + kc * 16 + g * 8;
    kf[kc] = key < N ? load_global<bf16x8>(a.k + off) : zero_bf16x8();
    vf[kc] = key < N ? load_global<bf16x8>(a.v + off) : zero_bf16x8();
  }
  {
    TransTile<BCK, D, C::NT> kt;
    kt.load(a.k + hoff, kb0, N, tid);
    kt.store(Kt, KTP, tid);
  }

  f32x16 dk[D / 32], dv[D / 32];  // dK^T, dV^T: lane holds [32 db + 8(i/4) + 4g + i%4][key]
#pragma unroll
  for (int db = 0; db < D / 32; ++db) { dk[db] = zero16(); dv[db] = zero16(); }

  const float sl2 = a.scale_log2;
  const int nqb = (N + BRQ - 1) / BRQ;
  const int i0 = CAUSAL ? kb0 / BRQ : 0;

  RowTile<BRQ, D, C::NT, true> qrow, dorow;
  TransTile<BRQ, D, C::NT> qtr, dotr;

  for (int i = i0; i < nqb; ++i) {
    const int q0 = i * BRQ;
    qrow.load(Qh, q0, N, tid);
    dorow.load(dOh, q0, N, tid);
    qtr.load(Qh, q0, N, tid);
    dotr.load(dOh, q0, N, tid);
    __syncthreads();  // previous iteration is done with every LDS tile
    qrow.store(Qs, QP, tid);
    dorow.store(dOs, QP, tid);
    qtr.store(Qt, TP, tid);
    dotr.store(dOt, TP, tid);
    if (tid < BRQ) {
      const int q = q0 + tid;
      lse_s[tid] = q < N ? lse2h[q] : INFINITY;  // padded rows get P = 0
      del_s[tid] = q < N ? delh[q] : 0.f;
    }
    __syncthreads();

#pragma unroll
    for (int qs = 0; qs < BRQ / 32; ++qs) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + (qs * 32 + c32) * QP + kc * 16 + g * 8);
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(dOs + (qs * 32 + c32) * QP + kc * 16 + g * 8);
        s = mfma32(qa, kf[kc], s);
        dp = mfma32(da, vf[kc], dp);
      }
      // value i <-> query q0 + 32 qs + 16 (i/8) + 8 g + i%8, key `key`
      const bool need_mask = (kb0 + BCK > N) || (CAUSAL && kw0 + C::KW - 1 > q0 + 32 * qs);
      float p[16], ds[16];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ql = 32 * qs + 16 * c + 8 * g;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse_s + ql);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse_s + ql + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(del_s + ql);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(del_s + ql + 4);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int idx = 8 * c + jj;
          const float lv = jj < 4 ? l0[jj] : l1[jj - 4];
          const float dv_ = jj < 4 ? d0[jj] : d1[jj - 4];
          float pv = exp2_fast(fmaf(s[idx], sl2, -lv));
          if (need_mask) {
            const int q = q0 + ql + jj;
            if (key >= N || (CAUSAL && key > q)) pv = 0.f;
          }
          p[idx] = pv;
          ds[idx] = pv * (dp[idx] - dv_);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over this sub-block's 32 queries.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 pb = pack8(p + 8 * c);
        const bf16x8 sb = pack8(ds + 8 * c);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 oa = *reinterpret_cast<const bf16x8*>(dOt + (db * 32 + c32) * TP + qs * 32 + 16 * c + 8 * g);
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qt + (db * 32 + c32) * TP + qs * 32 + 16 * c + 8 * g);
          dv[db] = mfma32(oa, pb, dv[db]);
          dk[db] = mfma32(qa, sb, dk[db]);
        }
      }
      // dS (bf16) into LDS as [query][key] for the dQ product.
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int ql = 32 * qs + 16 * (idx >> 3) + 8 * g + (idx & 7);
        const __bf16 h = (__bf16)ds[idx];
        dSs[ql * SP + w * C::KW + c32] = __builtin_bit_cast(uint16_t, h);
      }
    }
    __syncthreads();

    // dQ rows q0 .. q0+63 += dS K over the block's 128 keys (scale applied
    // when converting).  Tasks: (query sub-block, 32-column slice of d).
    constexpr int TASKS = (BRQ / 32) * (D / 32);
#pragma unroll
    for (int t = w; t < TASKS; t += C::NW) {
      const int qs = t / (D / 32), db = t % (D / 32);
      f32x16 acc = zero16();
#pragma unroll
      for (int kc = 0; kc < BCK / 16; ++kc) {
        const bf16x8 sa = *reinterpret_cast<const bf16x8*>(dSs + (qs * 32 + c32) * SP + kc * 16 + g * 8);
        const bf16x8 kb_ = *reinterpret_cast<const bf16x8*>(Kt + (db * 32 + c32) * KTP + kc * 16 + g * 8);
        acc = mfma32(sa, kb_, acc);
      }
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int q = q0 + qs * 32 + 8 * (idx >> 2) + 4 * g + (idx & 3);
        if (q < N) atomicAdd(dQh + (int64_t)q * D + db * 32 + c32, acc[idx]);
      }
    }
  }

  // dK = scale * (dS^T Q), dV = P^T dO, rows of this lane's key.
  if (key < N) {
    uint16_t* dKrow = a.dk + hoff + (int64_t)key * D;
    uint16_t* dVrow = a.dv + hoff + (int64_t)key * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = db * 32 + 8 * r4 + 4 * g;
        u32x2 kv, vv;
        kv.x = pack2(dk[db][4 * r4 + 0] * sc, dk[db][4 * r4 + 1] * sc);
        kv.y = pack2(dk[db][4 * r4 + 2] * sc, dk[db][4 * r4 + 3] * sc);
        vv.x = pack2(dv[db][4 * r4 + 0], dv[db][4 * r4 + 1]);
        vv.y = pack2(dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]);
        *reinterpret_cast<u32x2*>(dKrow + col) = kv;
        *reinterpret_cast<u32x2*>(dVrow + col) = vv;
      }
  }
}

// ------------------------------------------------------------------ dQ convert
__global__ void __launch_bounds__(256) fa_bwd_dq_kernel(BwdArgs a, int64_t n8) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(a.dq_acc + t * 8);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(a.dq_acc + t * 8 + 4);
  const float sc = a.scale;
  u32x4 r;
  r.x = pack2(x0.x * sc, x0.y * sc);
  r.y = pack2(x0.z * sc, x0.w * sc);
  r.z = pack2(x1.x * sc, x1.y * sc);
  r.w = pack2(x1.z * sc, x1.w * sc);
  *reinterpret_cast<u32x4*>(a.dq + t * 8) = r;
}

template <int D>
static hipError_t launch_pre_t(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.N;
  const int64_t rpb = 256 / (D / 8);
  hipLaunchKernelGGL((fa_bwd_pre_kernel<D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_main_t(const BwdArgs& a, hipStream_t stream) {
  using C = BwdCfg<D>;
  const int64_t nkb = (a.N + C::BCK - 1) / C::BCK;
  hipLaunchKernelGGL((fa_bwd_main_kernel<D, CAUSAL>), dim3((unsigned)(nkb * a.BH)), dim3(C::NT), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdArgs& a, int d, hipStream_t stream) {
  return d == 64 ? launch_pre_t<64>(a, stream) : launch_pre_t<128>(a, stream);
}

hipError_t launch_bwd_main(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_main_t<64, true>(a, stream) : launch_main_t<64, false>(a, stream);
  return causal ? launch_main_t<128, true>(a, stream) : launch_main_t<128, false>(a, stream);
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, hipStream_t stream) {
  const int64_t n8 = (int64_t)a.BH * a.N * d / 8;
  hipLaunchKernelGGL(fa_bwd_dq_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, a,
                     n8);
  return hipGetLastError();
}

}  // namespace fa
