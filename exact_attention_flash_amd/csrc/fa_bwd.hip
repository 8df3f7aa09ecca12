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
// Row pass over [B*H, Npad] rows (Npad = N rounded up to the query block):
// D = rowsum(dO o O) and LSE * log2(e) for real rows, D = 0 and +inf for the
// padding rows (so a padded query gets P = 0 in the main pass), and the dQ
// accumulator rows cleared.
template <int D>
__global__ void __launch_bounds__(256) fa_bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;       // threads per row (16-byte chunks)
  constexpr int RPB = 256 / TPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const int64_t rr = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int ch = tid % TPR;
  const int64_t rows = (int64_t)a.BH * a.Npad;
  const int64_t bh = rr / a.Npad;
  const int q = (int)(rr - bh * a.Npad);
  const bool real = rr < rows && q < a.N;
  const int64_t row = bh * a.N + q;  // row of the [B*H, N] tensors
  float acc = 0.f;
  if (real) {
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
  if (rr < rows && ch == 0) {
    a.delta[rr] = acc;
    a.lse2[rr] = real ? a.lse[row] * kLog2e : INFINITY;
  }
}

// ------------------------------------------------------------------ main pass
template <int D>
struct BwdCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int KW = 32;            // keys per wave
  static constexpr int BCK = NW * KW;      // keys per workgroup
  static constexpr int BRQ = kBwdQueryBlock;  // queries per iteration
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int QT = BRQ * D;       // elements of a Q or dO tile
  static constexpr int KT = BCK * D;       // elements of the K tile
  static constexpr int ST = BCK * BRQ;     // elements of a dS^T tile
};

// Asynchronous copy of query block [q0, q0 + BRQ) of Q and dO (natural row
// order, swizzled chunks) and of its LSE*log2(e) and D rows into one stage.
// Rows past N copy row N - 1 (their LSE is +inf, so they get P = 0).
template <int D>
__device__ __forceinline__ void issue_q_tile(const uint16_t* Qh, const uint16_t* dOh,
                                             const float* lse2h, const float* delh,
                                             uint16_t* Qs, uint16_t* dOs, float* vec, int q0,
                                             int N, int w, int lane) {
  using C = BwdCfg<D>;
  constexpr int COPIES = C::BRQ * C::CPR / C::NT;
#pragma unroll
  for (int t = 0; t < COPIES; ++t) {
    const int slot = (t * C::NW + w) * 64 + lane;
    const int row = slot / C::CPR;
    const int lc = (slot % C::CPR) ^ chunk_swizzle<D>(row);
    const int qq = min(q0 + row, N - 1);
    const int base = (t * C::NW + w) * 64 * 8;
    load_lds16(Qh + (int64_t)qq * D + lc * 8, Qs + base);
    load_lds16(dOh + (int64_t)qq * D + lc * 8, dOs + base);
  }
  // LSE*log2(e) then D: 2 x BRQ floats = BRQ / 2 lanes of 16 bytes (padded rows)
  if (w == 0 && lane < C::BRQ / 2) {
    const int half = C::BRQ / 4;  // lanes per vector
    const float* src = lane < half ? lse2h + q0 + 4 * lane : delh + q0 + 4 * (lane - half);
    load_lds16(src, vec);
  }
}

// Shared memory of the key-block pass: the K block (for the K^T operand of
// dS K), double-buffered Q / dO tiles with their LSE*log2(e) and D rows, and
// double-buffered dS^T tiles ([key][query], bf16).
template <int D>
struct BwdSmem {
  using C = BwdCfg<D>;
  uint16_t k[C::KT];
  uint16_t q[2][C::QT];
  uint16_t dout[2][C::QT];
  uint16_t dst[2][C::ST];
  float vec[2][2 * C::BRQ];
};

// One workgroup of the key-block pass: per-lane state and the steps of one
// query block.  Stage indices are template parameters so every LDS offset
// that does not depend on the lane is a compile-time immediate.
template <int D, bool CAUSAL>
struct BwdBlock {
  using C = BwdCfg<D>;
  static constexpr int BRQ = C::BRQ, BCK = C::BCK;

  BwdSmem<D>& sm;
  const BwdArgs& a;
  int w, lane, c32, g, N, bh, kb0, kw0, key, nqb;
  int64_t hoff;
  const uint16_t* Qh;
  const uint16_t* dOh;
  const float* lse2h;
  const float* delh;
  float* dQh;
  float sl2;
  TrLane<D> trd;       // transposed reads of the Q, dO and K tiles
  TrLane<BRQ> trs;     // transposed reads of the dS^T tile
  RowLane<D> rowd;     // row reads of the Q and dO tiles
  int dsw_base, dsw_u; // dS^T row writes
  int kr_base, kr_u;   // row reads of this lane's key in the K block
  bf16x8 vf[D / 16];
  f32x16 dk[D / 32], dv[D / 32];  // dK^T, dV^T: lane holds [32 db + 8(i/4) + 4g + i%4][key]

  __device__ __forceinline__ BwdBlock(BwdSmem<D>& sm_, const BwdArgs& a_, int bh_, int kb0_)
      : sm(sm_), a(a_), trd(threadIdx.x & 63), trs(threadIdx.x & 63), rowd(threadIdx.x & 63) {
    const int tid = threadIdx.x;
    w = tid >> 6;
    lane = tid & 63;
    c32 = lane & 31;
    g = lane >> 5;
    N = a.N;
    bh = bh_;
    kb0 = kb0_;
    kw0 = kb0 + w * C::KW;
    key = kw0 + c32;
    nqb = (N + BRQ - 1) / BRQ;
    hoff = (int64_t)bh * N * D;
    Qh = a.q + hoff;
    dOh = a.dout + hoff;
    lse2h = a.lse2 + (int64_t)bh * a.Npad;
    delh = a.delta + (int64_t)bh * a.Npad;
    dQh = a.dq_acc + hoff;
    sl2 = a.scale_log2;
    dsw_base = (w * C::KW + c32) * BRQ;
    dsw_u = g ^ chunk_swizzle<BRQ>(c32);
    kr_base = (w * C::KW + c32) * D;
    kr_u = g ^ chunk_swizzle<D>(c32);
  }

  __device__ __forceinline__ void issue_k_block() {
    constexpr int COPIES = BCK * C::CPR / C::NT;
#pragma unroll
    for (int t = 0; t < COPIES; ++t) {
      const int slot = (t * C::NW + w) * 64 + lane;
      const int row = slot / C::CPR;
      const int lc = (slot % C::CPR) ^ chunk_swizzle<D>(row);
      const int kk = min(kb0 + row, N - 1);
      load_lds16(a.k + hoff + (int64_t)kk * D + lc * 8, sm.k + (t * C::NW + w) * 64 * 8);
    }
  }

  __device__ __forceinline__ void load_kv_operands() {
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const int64_t off = hoff + (int64_t)key * D + kc * 16 + g * 8;
      vf[kc] = key < N ? load_global<bf16x8>(a.v + off) : zero_bf16x8();
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) { dk[db] = zero16(); dv[db] = zero16(); }
  }

  template <int ST>
  __device__ __forceinline__ void issue_q(int i) {
    issue_q_tile<D>(Qh, dOh, lse2h, delh, sm.q[ST], sm.dout[ST], sm.vec[ST], i * BRQ, N, w, lane);
  }

  // dQ rows of query block ib += dS K over the block's keys, from dS^T stage
  // ST.  Wave w computes 32-column slices: db = w (d = 128) or
  // (qs, db) = (w / 2, w % 2) (d = 64).
  template <int ST>
  __device__ __forceinline__ void dq_block(int ib) {
    const uint16_t* sd = sm.dst[ST];
    const TrLane<D> trd = this->trd.fresh();
    const TrLane<BRQ> trs = this->trs.fresh();
    constexpr int TASKS = (BRQ / 32) * (D / 32);
#pragma unroll
    for (int t0 = 0; t0 < TASKS; t0 += C::NW) {
      const int t = t0 + w;
      const int qs = t / (D / 32), db = t % (D / 32);
      f32x16 acc = zero16();
#pragma unroll
      for (int kc = 0; kc < BCK / 16; ++kc) {
        const bf16x8 sa = join_tr(lds_read_tr(sd + trs.off(16 * kc, 32 * qs, 0)),
                                  lds_read_tr(sd + trs.off(16 * kc, 32 * qs, 1)));
        const bf16x8 kt = join_tr(lds_read_tr(sm.k + trd.off(16 * kc, 32 * db, 0)),
                                  lds_read_tr(sm.k + trd.off(16 * kc, 32 * db, 1)));
        acc = mfma32(sa, kt, acc);
      }
      // rows qb0 + 8 (idx/4) + 4 g + idx%4, column 32 db + c32
      const int qb0 = ib * BRQ + 32 * qs;
      float* base = dQh + (int64_t)(qb0 + 4 * g) * D + db * 32 + c32;
      if (qb0 + 32 <= N) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx)
          atomicAdd(base + (8 * (idx >> 2) + (idx & 3)) * D, acc[idx]);
      } else {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx)
          if (qb0 + 4 * g + 8 * (idx >> 2) + (idx & 3) < N)
            atomicAdd(base + (8 * (idx >> 2) + (idx & 3)) * D, acc[idx]);
      }
    }
  }

  // S, P, dP, dS for query block i (stage ST): dV^T, dK^T accumulate; dS^T
  // goes to LDS stage ST for the dQ product.
  template <int ST>
  __device__ __forceinline__ void kv_block(int i) {
    const uint16_t* Qt = sm.q[ST];
    const uint16_t* dOt = sm.dout[ST];
    const float* lv = sm.vec[ST];
    uint16_t* sd = sm.dst[ST];
    const int q0 = i * BRQ;
    const TrLane<D> trd = this->trd.fresh();
    const RowLane<D> rowd = this->rowd.fresh();
    const int kr_base = opaque(this->kr_base), kr_u = opaque(this->kr_u);
    const int dsw_base = opaque(this->dsw_base), dsw_u = opaque(this->dsw_u);
#pragma unroll
    for (int qs = 0; qs < BRQ / 32; ++qs) {
      // value idx <-> query q0 + 32 qs + 16 (idx/8) + 8 g + idx%8, key `key`
      const bool skip = CAUSAL && (kw0 > q0 + 32 * qs + 31);
      float p[16], ds[16];
      if (!skip) {
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          const int o = rowd.off(32 * qs, kc);
          const bf16x8 kb = *reinterpret_cast<const bf16x8*>(sm.k + kr_base + (((2 * kc) ^ kr_u) << 3));
          s = mfma32(*reinterpret_cast<const bf16x8*>(Qt + o), kb, s);
          dp = mfma32(*reinterpret_cast<const bf16x8*>(dOt + o), vf[kc], dp);
        }
        const bool need_mask = (kb0 + BCK > N) || (CAUSAL && kw0 + C::KW - 1 > q0 + 32 * qs);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int ql = 32 * qs + 16 * c + 8 * g;
          const f32x4 l0 = *reinterpret_cast<const f32x4*>(lv + ql);
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(lv + ql + 4);
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(lv + BRQ + ql);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(lv + BRQ + ql + 4);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int idx = 8 * c + jj;
            const float lse = jj < 4 ? l0[jj] : l1[jj - 4];
            const float dlt = jj < 4 ? d0[jj] : d1[jj - 4];
            float pv = exp2_fast(fmaf(s[idx], sl2, -lse));
            if (need_mask) {
              const int q = q0 + ql + jj;
              if (key >= N || (CAUSAL && key > q)) pv = 0.f;
            }
            p[idx] = pv;
            ds[idx] = pv * (dp[idx] - dlt);
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the sub-block's 32 queries.
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 pb = pack8(p + 8 * c);
          const bf16x8 sb = pack8(ds + 8 * c);
          const int R0 = 32 * qs + 16 * c;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int o0 = trd.off(R0, 32 * db, 0), o1 = trd.off(R0, 32 * db, 1);
            const bf16x8 oa = join_tr(lds_read_tr(dOt + o0), lds_read_tr(dOt + o1));
            const bf16x8 qa = join_tr(lds_read_tr(Qt + o0), lds_read_tr(Qt + o1));
            dv[db] = mfma32(oa, pb, dv[db]);
            dk[db] = mfma32(qa, sb, dk[db]);
          }
          // dS^T row `key`, 8 consecutive queries (16 bytes)
          *reinterpret_cast<bf16x8*>(sd + dsw_base + (((4 * qs + 2 * c) ^ dsw_u) << 3)) = sb;
        }
      } else {
        const bf16x8 z = zero_bf16x8();
#pragma unroll
        for (int c = 0; c < 2; ++c)
          *reinterpret_cast<bf16x8*>(sd + dsw_base + (((4 * qs + 2 * c) ^ dsw_u) << 3)) = z;
      }
    }
  }

  // One iteration of the steady state: prefetch block i + 1, dQ of block
  // i - 1, then block i.
  template <int ST>
  __device__ __forceinline__ void step(int i) {
    if (i + 1 < nqb) issue_q<ST ^ 1>(i + 1);
    dq_block<ST ^ 1>(i - 1);
    kv_block<ST>(i);
    wait_vmem();
    __syncthreads();
  }

  __device__ __forceinline__ void store_dkdv() {
    if (key >= N) return;
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
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) fa_bwd_main_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  static_assert(C::BRQ == 64, "two 32-query sub-blocks per iteration");
  __shared__ __attribute__((aligned(1024))) BwdSmem<D> sm;

  const int N = a.N;
  const int nkb = (N + C::BCK - 1) / C::BCK;
  // Workgroup -> (head, key block), XCD-contiguous like the forward pass.
  // Causal key blocks near the start see the most query blocks, so the
  // natural order is already heaviest first.
  const int total = gridDim.x;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int bh = L / nkb;
  const int kb = L - bh * nkb;

  BwdBlock<D, CAUSAL> blk(sm, a, bh, kb * C::BCK);
  const int nqb = blk.nqb;
  const int i0 = CAUSAL ? blk.kb0 / C::BRQ : 0;
  blk.issue_k_block();
  blk.template issue_q<0>(i0);
  blk.load_kv_operands();
  wait_vmem();
  __syncthreads();

  // block i0 (stage 0) has no previous dQ to do
  if (i0 + 1 < nqb) blk.template issue_q<1>(i0 + 1);
  blk.template kv_block<0>(i0);
  wait_vmem();
  __syncthreads();
  int i = i0 + 1;
  for (; i + 1 < nqb; i += 2) {
    blk.template step<1>(i);
    blk.template step<0>(i + 1);
  }
  if (i < nqb) {
    blk.template step<1>(i);
    blk.template dq_block<1>(nqb - 1);
  } else {
    blk.template dq_block<0>(nqb - 1);
  }
  blk.store_dkdv();
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
  const int64_t rows = (int64_t)a.BH * a.Npad;
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
