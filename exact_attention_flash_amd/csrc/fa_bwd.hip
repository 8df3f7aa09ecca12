// Fused attention backward for gfx950 (recompute from the stored LSE).
//
// Method ("FlashAttention 的基本原理", section 2.4; "FlashAttention 系列技术
// 详解", section "反向传播步骤"): the scores are recomputed block by block, and
// because LSE is known the probabilities P = exp(scale*S - LSE) are final at
// once, with no running max.  Then
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   D_i = sum_c dO_ic O_ic,
//   dK = scale * dS^T Q,   dQ = scale * dS K.
// The CMU 15-442/642 notes (section "为什么前向和反向的并行化策略不同")
// parallelise the backward pass over key blocks and accumulate dQ across
// key blocks with atomic adds in device memory.  On MI355X that accumulation
// is the bottleneck: fp32 atomics retire at about one 4-byte add per clock
// per L2 channel, and the dQ adds alone would take longer than the whole
// rest of the pass.  So dQ gets its own pass, parallel over query blocks
// like the forward pass, which recomputes S and dP for its rows (two more
// GEMMs per block pair) and needs no atomics: dQ is deterministic.
//
// Three kernels on the caller's stream:
//   fa_bwd_pre   D = rowsum(dO o O) and LSE * log2(e), padded to whole
//                64-row query blocks (D = 0, LSE = +inf on padding rows)
//   fa_bwd_kv    persistent: one workgroup per CU walks its share of the
//                (batch, head, 128-key block) items: dK, dV
//   fa_bwd_q     one workgroup per (batch, head, 128-query block): dQ
#include <algorithm>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// ------------------------------------------------------------------ pre pass
// Row pass over [B*H, Npad] rows (Npad = N rounded up to the query block):
// D = rowsum(dO o O) and LSE * log2(e) for real rows, D = 0 and +inf for the
// padding rows (so a padded query gets P = 0 in the key-block pass).
// Each thread takes 16 bytes of PRE_ROWS rows, RPB rows apart, and issues
// all of its loads before any arithmetic.
constexpr int PRE_ROWS = 4;

template <int D>
__global__ void __launch_bounds__(256) fa_bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;       // threads per row (16-byte chunks)
  constexpr int RPB = 256 / TPR;   // rows per pass of the workgroup
  const int tid = threadIdx.x;
  const int ch = tid % TPR;
  const int64_t rows = (int64_t)a.BH * a.Npad;
  const int64_t r0 = (int64_t)blockIdx.x * RPB * PRE_ROWS + tid / TPR;
  u32x4 o[PRE_ROWS], d[PRE_ROWS];
  float lv[PRE_ROWS];
  bool real[PRE_ROWS];
#pragma unroll
  for (int k = 0; k < PRE_ROWS; ++k) {
    const int64_t rr = r0 + k * RPB;
    const int64_t bh = rr / a.Npad;
    const int q = (int)(rr - bh * a.Npad);
    real[k] = rr < rows && q < a.N;
    const int64_t row = bh * a.N + q;  // row of the [B*H, N] tensors
    o[k] = real[k] ? load_global<u32x4>(a.o + row * D + ch * 8) : u32x4{0u, 0u, 0u, 0u};
    d[k] = real[k] ? load_global<u32x4>(a.dout + row * D + ch * 8) : u32x4{0u, 0u, 0u, 0u};
    lv[k] = real[k] && ch == 0 ? a.lse[row] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < PRE_ROWS; ++k) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(bf16_to_f32((uint16_t)(o[k][j] & 0xffffu)), bf16_to_f32((uint16_t)(d[k][j] & 0xffffu)), acc);
      acc = fmaf(bf16_to_f32((uint16_t)(o[k][j] >> 16)), bf16_to_f32((uint16_t)(d[k][j] >> 16)), acc);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    const int64_t rr = r0 + k * RPB;
    if (rr < rows && ch == 0) {
      a.delta[rr] = -acc;  // stored negated: the passes start dP from it
      a.lse2[rr] = real[k] ? lv[k] * kLog2e : INFINITY;
    }
  }
}

// ------------------------------------------------------------------ key-block pass
// Steps by which the key-block pass reads its LDS operands ahead of the
// MFMAs that use them.  Measured on causal B=4 H=16 N=4096 d=128 (medians,
// alternating processes): 2 ahead in both loops 0.568 ms, 3 0.574, 4 0.590,
// 1 in the score loop 0.599; the compiler's own schedule 0.599.
constexpr int kKvReadAhead = 2;

template <int D>
struct KvCfg {
  static constexpr int NW = 8;             // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int KW = 16;            // keys per wave
  static constexpr int BCK = NW * KW;      // keys per workgroup
  static constexpr int BRQ = kBwdQueryBlock;  // queries per iteration
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int QT = BRQ * D;       // elements of a Q or dO tile
};

// Asynchronous copies of query block [q0, q0 + BRQ) of Q and dO (natural
// row order, qtile_swizzle chunks) into one stage.  Copy t of thread
// (w, lane) fills 16-byte slot (t * NW + w) * 64 + lane of a tile; its source
// byte offset within the block is the same for every block and is computed
// once.  Rows past N copy row N - 1 (their LSE is +inf, so they get P = 0).
template <int D>
struct QTileCopy {
  using C = KvCfg<D>;
  static constexpr int COPIES = C::BRQ * C::CPR / C::NT;
  uint32_t off[COPIES];

  __device__ __forceinline__ static int slot_row(int t, int w, int lane) {
    return ((t * C::NW + w) * 64 + lane) / C::CPR;
  }
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int t = 0; t < COPIES; ++t) {
      const int slot = (t * C::NW + w) * 64 + lane;
      const int r = slot / C::CPR;
      off[t] = 2 * (r * D + (((slot % C::CPR) ^ qtile_swizzle<D>(r)) << 3));
    }
  }
  __device__ __forceinline__ void issue(const uint16_t* Qh, const uint16_t* dOh, uint16_t* Qs,
                                        uint16_t* dOs, int q0, int N, int w, int lane) const {
    constexpr uint32_t kBytes = C::BRQ * D * 2;
    const buf_rsrc qr = make_rsrc(Qh + (int64_t)q0 * D, kBytes);
    const buf_rsrc dr = make_rsrc(dOh + (int64_t)q0 * D, kBytes);
    if (q0 + C::BRQ <= N) {
#pragma unroll
      for (int t = 0; t < COPIES; ++t) {
        const int base = (t * C::NW + w) * 64 * 8;
        buffer_load_lds16(qr, off[t], Qs + base);
        buffer_load_lds16(dr, off[t], dOs + base);
      }
    } else {
#pragma unroll
      for (int t = 0; t < COPIES; ++t) {
        const int base = (t * C::NW + w) * 64 * 8;
        const int r = slot_row(t, w, lane);
        const int shift = (min(q0 + r, N - 1) - (q0 + r)) * D * 2;
        buffer_load_lds16(qr, off[t] + shift, Qs + base);
        buffer_load_lds16(dr, off[t] + shift, dOs + base);
      }
    }
  }
};

// LDS of the key-block pass: double-buffered Q / dO tiles with their
// LSE*log2(e) and D rows.  Every buffer is its own LDS object, so the
// compiler can tell that the copies into one stage never overlap reads of
// the other and does not wait for them.
struct KvSmem {
  uint16_t* q[2];
  uint16_t* dout[2];
  float* vec[2];
  uint8_t* drop;  // dropout bytes, 1 KiB per wave (DROP only)
};

// One workgroup of the key-block pass (8 waves, 16 keys each).  S = Q K^T,
// dP = dO V^T, dV^T += dO^T P and dK^T += Q^T dS use v_mfma_f32_16x16x32_bf16
// with a lane owning one key; the 16 queries of an S tile are fed in the
// order that gives each lane 8 consecutive queries per 32-query group, so P
// and dS are directly the B operands of the dV and dK products.
template <int D, bool CAUSAL, bool DROP>
struct KvBlock {
  using C = KvCfg<D>;
  static constexpr int BRQ = C::BRQ, BCK = C::BCK;

  const KvSmem sm;
  const BwdArgs& a;
  int w, lane, c16, kg, N, nqb;
  int bh, kb0, kw0, key;  // the current item: head, first key, this wave's keys, lane's key
  int64_t hoff;
  int nbh, nkb0;          // the next item of this workgroup (nbh < 0: none)
  int round;              // index of the current item in the workgroup's walk
  float sl2;
  int srow_base, srow_u;  // 16-byte row reads of Q / dO for S and dP
  int tq_base, tq_t;      // transposed reads of Q / dO for dK and dV
  QTileCopy<D> cp;                // source offsets of the Q / dO tile copies
  bf16x8 kf[D / 32], vf[D / 32];    // B operands: K, V rows of this lane's key
  bf16x8 kfn[D / 32], vfn[D / 32];  // the same rows of the next item, loaded ahead
  f32x4 dk[D / 16], dv[D / 16];     // dK^T, dV^T: lane holds [16 dt + 4 kg + i][key]

  __device__ __forceinline__ KvBlock(const KvSmem& sm_, const BwdArgs& a_) : sm(sm_), a(a_) {
    const int tid = threadIdx.x;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    lane = tid & 63;
    c16 = lane & 15;
    kg = lane >> 4;
    N = a.N;
    nqb = (N + BRQ - 1) / BRQ;
    sl2 = a.scale_log2;
    // row of S tile t in 32-query group qg fed by lane c16:
    // 32 qg + 8 (c16 / 4) + 4 t + c16 % 4 (t and qg do not change the swizzle)
    const int sr = 8 * (c16 >> 2) + (c16 & 3);
    srow_base = sr * D;
    srow_u = kg ^ qtile_swizzle<D>(sr);
    // transposed reads: lane 16 G + 4 e + q reads row 32 qg + 8 G + e (+4),
    // columns 16 dt + 4 q .. + 3
    const int te = (lane >> 2) & 3, tq = lane & 3;
    const int tr = 8 * kg + te;
    tq_base = tr * D + 4 * (tq & 1);
    tq_t = (tq >> 1) ^ qtile_swizzle<D>(tr);
    cp.init(w, lane);
  }

  // First query block that item (head, key block from kb0_) visits.
  __device__ __forceinline__ int first_block(int kb0_) const { return CAUSAL ? kb0_ / BRQ : 0; }

  __device__ __forceinline__ void set_item(int bh_, int kb0_) {
    bh = bh_;
    kb0 = kb0_;
    kw0 = kb0 + w * C::KW;
    key = kw0 + c16;
    hoff = (int64_t)bh * N * D;
  }

  // Item L of the walk, or nbh = -1 past its end.
  __device__ __forceinline__ void plan_next(const ItemWalk& walk, int nkb) {
    const int L = walk.item(round + 1);
    if (L < 0) {
      nbh = -1;
      return;
    }
    int kb;
    xcd_head_block<kHeadsPerGroup>(L, walk.total, a.BH, nkb, nbh, kb);
    nkb0 = kb * BCK;
  }

  // K and V rows of this lane's key of item (bh_, kb0_) (zero past N).
  __device__ __forceinline__ void load_rows(bf16x8 (&kd)[D / 32], bf16x8 (&vd)[D / 32], int bh_,
                                            int kb0_) const {
    const int ky = kb0_ + w * C::KW + c16;
    const int64_t ho = (int64_t)bh_ * N * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const int64_t off = ho + (int64_t)ky * D + 32 * s + 8 * kg;
      kd[s] = ky < N ? load_global<bf16x8>(a.k + off) : zero_bf16x8();
      vd[s] = ky < N ? load_global<bf16x8>(a.v + off) : zero_bf16x8();
    }
  }

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) { dk[dt] = zero4(); dv[dt] = zero4(); }
  }

  // Copies of query block i of head bh_ into stage ST.
  template <int ST>
  __device__ __forceinline__ void issue_q(int bh_, int i) {
    const int q0 = i * BRQ;
    const int64_t ho = (int64_t)bh_ * N * D;
    cp.issue(a.q + ho, a.dout + ho, sm.q[ST], sm.dout[ST], q0, N, w, lane);
    // LSE*log2(e) then D of the block: 2 x BRQ floats = BRQ / 2 lanes of 16
    // bytes (the rows are padded to whole blocks)
    // (buffer copies, not global_load_lds: the compiler takes a pending
    // global_load_lds for a possible LDS access of unknown order and then
    // waits for every LDS read with lgkmcnt(0))
    if (w == 0 && lane < BRQ / 2) {
      constexpr int half = BRQ / 4;  // lanes per vector
      const int64_t vo = (int64_t)bh_ * a.Npad + q0;
      if (lane < half)
        buffer_load_lds16(make_rsrc(a.lse2 + vo, BRQ * 4), 16 * lane, sm.vec[ST]);
      else
        buffer_load_lds16(make_rsrc(a.delta + vo, BRQ * 4), 16 * (lane - half), sm.vec[ST]);
    }
  }

  // Dropout bytes of this lane's key for the block's queries: byte m of the
  // result belongs to query q0 + 32 (m / 8) + 8 kg + m % 8.  The wave's 16
  // keys are one 16-key group of the Philox layout, so the call for one
  // query gives the bytes of all 16 keys: lane (c16, kg) draws for query
  // m = c16 of its kg group, and the 16 x 16 bytes of the group are
  // transposed through the wave's LDS region (byte b of lane m to row b,
  // column m; row c16 read back).
  __device__ __forceinline__ i32x4 drop_bytes(int q0) const {
    const int m = c16;
    const uint32_t qd = (uint32_t)(q0 + 32 * (m >> 3) + 8 * kg + (m & 7));
    const u32x4 r = philox4x32_10((uint32_t)(kw0 >> 4), qd, (uint32_t)bh, a.drop.offset,
                                  a.drop.k0, a.drop.k1);
    uint8_t* base = sm.drop + (w * 4 + kg) * 256;
#pragma unroll
    for (int b = 0; b < 16; ++b) base[b * 16 + m] = (uint8_t)(r[b >> 2] >> (8 * (b & 3)));
    return *reinterpret_cast<const i32x4*>(base + c16 * 16);
  }

  // S, P, dP, dS for query block i (stage ST); dV^T and dK^T accumulate.
  template <int ST>
  __device__ __forceinline__ void block(int i) {
    const uint16_t* Qt = sm.q[ST];
    const uint16_t* dOt = sm.dout[ST];
    const float* lv = sm.vec[ST];
    const int q0 = i * BRQ;
    i32x4 rb;
    if constexpr (DROP) rb = drop_bytes(q0);
    const int sb = opaque(srow_base), su = opaque(srow_u);
    const int tb = opaque(tq_base), tt = opaque(tq_t);
#pragma unroll
    for (int qg = 0; qg < BRQ / 32; ++qg) {
      // lane (key, kg) gets queries q0 + 32 qg + 8 kg + j, j < 8
      if (CAUSAL && (kw0 > q0 + 32 * qg + 31)) continue;  // every key after every query
      const int ql = 32 * qg + 8 * kg;
      // -D of the lane's 8 queries; without dropout dP starts from it, so
      // the products leave dP - D in the accumulator
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(lv + BRQ + ql);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(lv + BRQ + ql + 4);
      // S and dP in 2 (D / 32) steps (tile t, contraction slice k), each
      // reading its Q and dO operands kKvReadAhead steps ahead of its MFMAs
      // into a rotating set of registers (the compiler's own schedule
      // reuses one set and waits for each read right before its product).
      constexpr int NS = 2 * (D / 32), AS = kKvReadAhead;
      static_assert(AS >= 1 && AS <= NS, "look-ahead within the group's steps");
      f32x4 s[2], dp[2];
      s[0] = s[1] = zero4();
      dp[0] = DROP ? zero4() : d0;
      dp[1] = DROP ? zero4() : d1;
      bf16x8 qo[AS], dop[AS];
      auto srow = [&](int st) {
        return (32 * qg + 4 * (st / (D / 32))) * D + sb + (((4 * (st % (D / 32))) ^ su) << 3);
      };
#pragma unroll
      for (int st = 0; st < AS; ++st) {
        qo[st] = *reinterpret_cast<const bf16x8*>(Qt + srow(st));
        dop[st] = *reinterpret_cast<const bf16x8*>(dOt + srow(st));
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int t = st / (D / 32), k = st % (D / 32);
        s[t] = mfma16(qo[st % AS], kf[k], s[t]);
        dp[t] = mfma16(dop[st % AS], vf[k], dp[t]);
        if (st + AS < NS) {
          qo[st % AS] = *reinterpret_cast<const bf16x8*>(Qt + srow(st + AS));
          dop[st % AS] = *reinterpret_cast<const bf16x8*>(dOt + srow(st + AS));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool need_mask = (kb0 + BCK > N) || (CAUSAL && kw0 + C::KW - 1 > q0 + 32 * qg);
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(lv + ql);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(lv + ql + 4);
      float p[8], ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float sv = j < 4 ? s[0][j] : s[1][j - 4];
        const float dpv = j < 4 ? dp[0][j] : dp[1][j - 4];
        const float lse = j < 4 ? l0[j] : l1[j - 4];
        const float ndlt = j < 4 ? d0[j] : d1[j - 4];  // -D
        float pv = exp2_fast(fmaf(sv, sl2, -lse));
        if (need_mask) {
          const int q = q0 + ql + j;
          if (key >= N || (CAUSAL && key > q)) pv = 0.f;
        }
        if constexpr (DROP) {
          // dV takes the kept probabilities (rescaled at the store); dS the
          // kept dP, rescaled: dS = P (Z s dP - D)
          const int mb = 8 * qg + j;
          const bool keep = drop_keep((uint32_t)rb[mb >> 2], mb & 3, a.drop.t);
          p[j] = keep ? pv : 0.f;
          ds[j] = pv * fmaf(dpv, keep ? a.drop.scale : 0.f, ndlt);
        } else {
          p[j] = pv;
          ds[j] = pv * dpv;  // dpv already holds dP - D
        }
      }
      const bf16x8 pb = pack8(p);
      const bf16x8 sbv = pack8(ds);
      // dV^T += dO^T P, dK^T += Q^T dS over the group's 32 queries; dO^T and
      // Q^T come transposed out of the row-major tiles.
      // (reads kKvReadAhead column blocks ahead, as above)
      constexpr int NT = D / 16, AT = kKvReadAhead;
      static_assert(AT >= 1 && AT <= NT, "look-ahead within the group's steps");
      bf16x8 oa[AT], qa[AT];
      auto trread = [&](const uint16_t* X, int dt) {
        const int o0 = (32 * qg) * D + tb + (((2 * dt) ^ tt) << 3);
        return join_tr(lds_read_tr(X + o0), lds_read_tr(X + o0 + 4 * D));
      };
#pragma unroll
      for (int dt = 0; dt < AT; ++dt) {
        oa[dt] = trread(dOt, dt);
        qa[dt] = trread(Qt, dt);
      }
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        dv[dt] = mfma16(oa[dt % AT], pb, dv[dt]);
        dk[dt] = mfma16(qa[dt % AT], sbv, dk[dt]);
        if (dt + AT < NT) {
          oa[dt % AT] = trread(dOt, dt + AT);
          qa[dt % AT] = trread(Qt, dt + AT);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Block i of the current item from stage ST, with the next block (of this
  // item, else the first of the next item, whose K and V rows are loaded at
  // the same time) prefetched into the other stage.  After an item's last
  // block: dK and dV are stored and the next item takes over.  Returns false
  // once the walk is done.
  template <int ST>
  __device__ __forceinline__ bool step(int& i, const ItemWalk& walk, int nkb) {
    const bool last = i + 1 == nqb;
    if (!last) {
      issue_q<ST ^ 1>(bh, i + 1);
    } else if (nbh >= 0) {
      issue_q<ST ^ 1>(nbh, first_block(nkb0));
      load_rows(kfn, vfn, nbh, nkb0);
    }
    block<ST>(i);
    wait_vmem();
    __syncthreads();
    if (!last) {
      ++i;
      return true;
    }
    store();
    if (nbh < 0) return false;
    set_item(nbh, nkb0);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      kf[s] = kfn[s];
      vf[s] = vfn[s];
    }
    zero_acc();
    i = first_block(kb0);
    ++round;
    plan_next(walk, nkb);
    return true;
  }

  __device__ __forceinline__ void store() {
    if (key >= N) return;
    uint16_t* dKrow = a.dk + hoff + (int64_t)key * D;
    uint16_t* dVrow = a.dv + hoff + (int64_t)key * D;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int col = 16 * dt + 4 * kg;
      u32x2 kv, vv;
      kv.x = pack2(dk[dt][0] * sc, dk[dt][1] * sc);
      kv.y = pack2(dk[dt][2] * sc, dk[dt][3] * sc);
      if constexpr (DROP) {
        const float vs = a.drop.scale;  // the dropout rescale of the kept P
        vv.x = pack2(dv[dt][0] * vs, dv[dt][1] * vs);
        vv.y = pack2(dv[dt][2] * vs, dv[dt][3] * vs);
      } else {
        vv.x = pack2(dv[dt][0], dv[dt][1]);
        vv.y = pack2(dv[dt][2], dv[dt][3]);
      }
      *reinterpret_cast<u32x2*>(dKrow + col) = kv;
      *reinterpret_cast<u32x2*>(dVrow + col) = vv;
    }
  }
};

template <int D, bool CAUSAL, bool DROP = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_bwd_kv_kernel(BwdArgs a) {
  using C = KvCfg<D>;
  static_assert(C::BRQ == 64, "two 32-query groups per iteration");
  __shared__ __attribute__((aligned(1024))) uint16_t q0_s[C::QT];
  __shared__ __attribute__((aligned(1024))) uint16_t q1_s[C::QT];
  __shared__ __attribute__((aligned(1024))) uint16_t do0_s[C::QT];
  __shared__ __attribute__((aligned(1024))) uint16_t do1_s[C::QT];
  __shared__ __attribute__((aligned(16))) float vec0_s[2 * C::BRQ];
  __shared__ __attribute__((aligned(16))) float vec1_s[2 * C::BRQ];
  __shared__ __attribute__((aligned(16))) uint8_t drop_s[DROP ? C::NW * 1024 : 16];
  const KvSmem sm{{q0_s, q1_s}, {do0_s, do1_s}, {vec0_s, vec1_s}, drop_s};

  const int N = a.N;
  const int nkb = (N + C::BCK - 1) / C::BCK;
  // Items (head, key block) in run order: heads grouped per XCD; causal key
  // blocks near the start see the most query blocks, so run order 0 is the
  // heaviest.  The grid (at most one workgroup per CU, never more than the
  // items) walks them.
  const ItemWalk walk{(int)blockIdx.x, (int)gridDim.x, a.BH * nkb};
  KvBlock<D, CAUSAL, DROP> blk(sm, a);
  int bh, kb;
  xcd_head_block<kHeadsPerGroup>(walk.item(0), walk.total, a.BH, nkb, bh, kb);
  blk.set_item(bh, kb * C::BCK);
  blk.round = 0;
  blk.plan_next(walk, nkb);
  int i = blk.first_block(blk.kb0);
  blk.template issue_q<0>(bh, i);
  blk.load_rows(blk.kf, blk.vf, bh, blk.kb0);
  blk.zero_acc();
  wait_vmem();
  __syncthreads();
  while (blk.template step<0>(i, walk, nkb) && blk.template step<1>(i, walk, nkb)) {
  }
}

// ------------------------------------------------------------------ query-block pass
template <int D>
struct QCfg {
  static constexpr int NW = 4;                      // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int QW = 32;                     // query rows per wave
  static constexpr int BR = NW * QW;                // query rows per workgroup
  static constexpr int BC = 64;                     // keys per K/V tile
  static constexpr int CPR = D / 8;
  static constexpr int TILE = BC * D;
  static constexpr int COPIES = BC * CPR / NT;
};

// One workgroup of the query-block pass (4 waves, 32 query rows each), laid
// out like the forward pass: a lane owns one query row, K and V tiles stream
// through a double-buffered LDS, and per tile
//   S^T = K Q^T, dP^T = V dO^T (32x32x16, K / V rows as A operands),
//   P^T = exp2(scale log2(e) S^T - LSE log2(e)), dS^T = P^T o (dP^T - D),
//   dQ^T += K^T dS^T (K^T read transposed from the K tile, dS^T straight
//   from registers as the B operand).
// dQ stays in registers and is written once.
template <int D, bool CAUSAL, bool DROP>
struct QBlock {
  using C = QCfg<D>;
  static constexpr int BC = C::BC;

  DropArgs drop;  // DROP only
  int bh;
  uint16_t* ks[2];
  uint16_t* vs[2];
  const uint16_t* Kh;
  const uint16_t* Vh;
  int w, lane, c32, g, N, qw0, qrow, nt;
  float sl2, lse2, ndlt;  // ndlt = -D of the lane's query
  bf16x8 qf[D / 16], dof[D / 16];  // B operands: Q, dO rows of this lane's query
  f32x16 dq[D / 32];                // dQ^T: lane holds dQ[qrow][32 db + 8(i/4) + 4g + i%4]
  RowLane<D> rowk;                  // row reads of K / V (row swap23(c32) of each block)
  TrLane<D> trk;                    // transposed reads of K

  // Copy t of thread (w, lane) fills 16-byte slot (t * NW + w) * 64 + lane of
  // a K / V tile (natural row order, chunk_swizzle chunks); its source byte
  // offset within the tile is the same for every tile.  Rows past N copy row
  // N - 1 (finite data for keys that are masked anyway).
  __device__ __forceinline__ static int slot_row(int t, int w, int lane) {
    return ((t * C::NW + w) * 64 + lane) / C::CPR;
  }
  // Computed at each use from an opaque lane index (a few integer
  // operations per tile) rather than held in registers all kernel long.
  __device__ __forceinline__ uint32_t copy_off(int t) const {
    const int slot = (t * C::NW + w) * 64 + opaque(lane);
    const int r = slot / C::CPR;
    return 2 * (r * D + (((slot % C::CPR) ^ chunk_swizzle<D>(r)) << 3));
  }

  template <int ST>
  __device__ __forceinline__ void issue(int j) {
    constexpr uint32_t kBytes = BC * D * 2;
    const int k0 = j * BC;
    const buf_rsrc kr = make_rsrc(Kh + (int64_t)k0 * D, kBytes);
    const buf_rsrc vr = make_rsrc(Vh + (int64_t)k0 * D, kBytes);
    if (k0 + BC <= N) {
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t) {
        const int base = (t * C::NW + w) * 64 * 8;
        const uint32_t off = copy_off(t);
        buffer_load_lds16(kr, off, ks[ST] + base);
        buffer_load_lds16(vr, off, vs[ST] + base);
      }
    } else {
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t) {
        const int base = (t * C::NW + w) * 64 * 8;
        const int r = slot_row(t, w, lane);
        const int shift = (min(k0 + r, N - 1) - (k0 + r)) * D * 2;
        const uint32_t off = copy_off(t) + shift;
        buffer_load_lds16(kr, off, ks[ST] + base);
        buffer_load_lds16(vr, off, vs[ST] + base);
      }
    }
  }

  // S^T and dP^T of 32-key block sb of the tile: value i of s[sb] is key
  // k0 + 32 sb + 16 (i/8) + 8 g + i%8.
  template <int ST>
  __device__ __forceinline__ void scores(int sb, f32x16* s, f32x16* dp, const RowLane<D>& rk) {
    const uint16_t* Ks = ks[ST];
    const uint16_t* Vs = vs[ST];
    s[sb] = zero16();
    dp[sb] = zero16();
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const int o = rk.off(32 * sb, kc);
      s[sb] = mfma32(*reinterpret_cast<const bf16x8*>(Ks + o), qf[kc], s[sb]);
      dp[sb] = mfma32(*reinterpret_cast<const bf16x8*>(Vs + o), dof[kc], dp[sb]);
    }
    // keep the K / V reads two slices ahead of the MFMAs that consume them
    sched_pipeline<D / 16, 2, 2, 2>();
  }

  // dS^T = P^T o (dP^T - D) of 32-key block sb, P^T = exp2(scale log2(e) S^T
  // - LSE log2(e)), packed to bf16 as the B operands of 16-key chunks 2 sb
  // and 2 sb + 1.
  template <bool MASK>
  __device__ __forceinline__ void softmax_ds(int sb, int k0, const f32x16* s, const f32x16* dp,
                                             bf16x8* dsb) {
    // dropout bytes of keys 32 sb + 16 h + 8 g + 0..7 (as in the forward pass:
    // the lane draws 16-key group 2 sb + g and swaps half with the other
    // wave half)
    uint32_t rw[2][2];
    if constexpr (DROP) {
      const u32x4 own = philox4x32_10((uint32_t)(k0 >> 4) + 2 * sb + g, (uint32_t)qrow,
                                      (uint32_t)bh, drop.offset, drop.k0, drop.k1);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto r = __builtin_amdgcn_permlane32_swap(own[e], own[2 + e], false, false);
        rw[0][e] = r[0];
        rw[1][e] = r[1];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float t8[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int i = 8 * h + jj;
        float pv = exp2_fast(fmaf(s[sb][i], sl2, -lse2));
        if constexpr (MASK) {
          const int key = k0 + 32 * sb + 16 * h + 8 * g + jj;
          if (key >= N || (CAUSAL && key > qrow)) pv = 0.f;
        }
        if constexpr (DROP) {
          const bool keep = drop_keep(rw[h][jj >> 2], jj & 3, drop.t);
          t8[jj] = pv * fmaf(dp[sb][i], keep ? drop.scale : 0.f, ndlt);
        } else {
          t8[jj] = pv * (dp[sb][i] + ndlt);
        }
      }
      dsb[2 * sb + h] = pack8(t8);
    }
  }

  // dQ^T += K^T dS^T over 16-key chunk kc2 of the tile (K^T read transposed).
  template <int ST>
  __device__ __forceinline__ void dq_chunk(int kc2, const bf16x8* dsb, const TrLane<D>& tr) {
    const uint16_t* Ks = ks[ST];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16x8 ka = join_tr(lds_read_tr(Ks + tr.off(16 * kc2, 32 * db, 0)),
                                lds_read_tr(Ks + tr.off(16 * kc2, 32 * db, 1)));
      dq[db] = mfma32(ka, dsb[kc2], dq[db]);
    }
  }

  // One tile, ordered so that each block's exponentials and dS run beside
  // independent MFMAs of the same wave (an MFMA issues and executes while
  // the wave goes on issuing vector instructions): block 1's S and dP beside
  // block 0's softmax, the dQ products of block 0's chunks beside block 1's.
  // MASK: the tile straddles the diagonal or the end of the sequence.
  // cj: the tile whose copies this one issues into the other stage, or -1.
  template <int ST, bool MASK>
  __device__ __forceinline__ void tile(int j, int cj) {
    static_assert(BC == 64, "two 32-key blocks per tile");
    const int k0 = j * BC;
    const RowLane<D> rk = rowk.fresh();
    const TrLane<D> tr = trk.fresh();
    f32x16 s[2], dp[2];
    bf16x8 dsb[4];
    // scheduling regions; the compiler interleaves within each
    scores<ST>(0, s, dp, rk);
    __builtin_amdgcn_sched_barrier(0);
    // the next tile's copies (cj < 0: none) go out here rather than before
    // the first products: issued beside them they slowed the first block's
    // score MFMAs (C5 query-block pass 0.404 -> 0.395 ms)
    if (cj >= 0) issue<ST ^ 1>(cj);
    scores<ST>(1, s, dp, rk);
    softmax_ds<MASK>(0, k0, s, dp, dsb);
    __builtin_amdgcn_sched_barrier(0);
    softmax_ds<MASK>(1, k0, s, dp, dsb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc2 = 0; kc2 < 4; ++kc2) dq_chunk<ST>(kc2, dsb, tr);
  }

  template <int ST>
  __device__ __forceinline__ void step(int j) {
    const int k0 = j * BC;
    const int cj = j + 1 < nt ? j + 1 : -1;
    if (!(CAUSAL && (k0 > qw0 + C::QW - 1))) {
      const bool need_mask = (k0 + BC > N) || (CAUSAL && (k0 + BC - 1 > qw0));
      if (need_mask) tile<ST, true>(j, cj);
      else tile<ST, false>(j, cj);
    } else if (cj >= 0) {
      issue<ST ^ 1>(cj);
    }
    wait_vmem();
    __syncthreads();
  }
};

template <int D, bool CAUSAL, bool DROP = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_bwd_q_kernel(BwdArgs a) {
  using C = QCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[C::TILE];

  const int tid = threadIdx.x;
  const int N = a.N;
  const int nqb = (N + C::BR - 1) / C::BR;
  // Workgroup -> (head, query block): heads grouped per XCD, heaviest
  // (last) causal query blocks first.
  int bh, qb;
  xcd_head_block<kHeadsPerGroup>(blockIdx.x, gridDim.x, a.BH, nqb, bh, qb);
  if (CAUSAL) qb = nqb - 1 - qb;

  const int64_t hoff = (int64_t)bh * N * D;
  QBlock<D, CAUSAL, DROP> f;
  f.drop = a.drop;
  f.bh = bh;
  f.ks[0] = k0s;
  f.ks[1] = k1s;
  f.vs[0] = v0s;
  f.vs[1] = v1s;
  f.Kh = a.k + hoff;
  f.Vh = a.v + hoff;
  f.w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  f.lane = tid & 63;
  f.c32 = f.lane & 31;
  f.g = f.lane >> 5;
  f.N = N;
  const int q0 = qb * C::BR;
  f.qw0 = q0 + f.w * C::QW;
  f.qrow = f.qw0 + f.c32;
  f.nt = (N + C::BC - 1) / C::BC;
  if (CAUSAL) f.nt = min(f.nt, (q0 + C::BR + C::BC - 1) / C::BC);
  f.sl2 = a.scale_log2;
  f.rowk = RowLane<D>(f.lane);
  f.trk = TrLane<D>(f.lane);

  f.template issue<0>(0);
  const bool real = f.qrow < N;
  const int64_t ro = hoff + (int64_t)f.qrow * D;
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    f.qf[kc] = real ? load_global<bf16x8>(a.q + ro + kc * 16 + f.g * 8) : zero_bf16x8();
    f.dof[kc] = real ? load_global<bf16x8>(a.dout + ro + kc * 16 + f.g * 8) : zero_bf16x8();
  }
  const int64_t vrow = (int64_t)bh * a.Npad + f.qrow;
  f.lse2 = real ? a.lse2[vrow] : INFINITY;  // padded rows get P = 0
  f.ndlt = real ? a.delta[vrow] : 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) f.dq[db] = zero16();
  wait_vmem();
  __syncthreads();

  int j = 0;
  for (; j + 1 < f.nt; j += 2) {
    f.template step<0>(j);
    f.template step<1>(j + 1);
  }
  if (j < f.nt) f.template step<0>(j);

  if (real) {
    uint16_t* row = a.dq + ro;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 val;
        val.x = pack2(f.dq[db][4 * r4 + 0] * sc, f.dq[db][4 * r4 + 1] * sc);
        val.y = pack2(f.dq[db][4 * r4 + 2] * sc, f.dq[db][4 * r4 + 3] * sc);
        *reinterpret_cast<u32x2*>(row + db * 32 + 8 * r4 + 4 * f.g) = val;
      }
  }
}

// ------------------------------------------------------------------ launchers
template <int D>
static hipError_t launch_pre_t(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.Npad;
  const int64_t rpw = 256 / (D / 8) * PRE_ROWS;  // rows per workgroup
  hipLaunchKernelGGL((fa_bwd_pre_kernel<D>), dim3((unsigned)((rows + rpw - 1) / rpw)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool DROP = false>
static hipError_t launch_kv_t(const BwdArgs& a, hipStream_t stream) {
  using C = KvCfg<D>;
  // one workgroup per CU: the kernel's registers allow no more
  const int64_t grid = persistent_grid((int64_t)((a.N + C::BCK - 1) / C::BCK) * a.BH);
  hipLaunchKernelGGL((fa_bwd_kv_kernel<D, CAUSAL, DROP>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool DROP = false>
static hipError_t launch_q_t(const BwdArgs& a, hipStream_t stream) {
  using C = QCfg<D>;
  const int64_t nqb = (a.N + C::BR - 1) / C::BR;
  hipLaunchKernelGGL((fa_bwd_q_kernel<D, CAUSAL, DROP>), dim3((unsigned)(nqb * a.BH)), dim3(C::NT),
                     0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdArgs& a, int d, hipStream_t stream) {
  return d == 64 ? launch_pre_t<64>(a, stream) : launch_pre_t<128>(a, stream);
}

hipError_t launch_bwd_kv(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_kv_t<64, true>(a, stream) : launch_kv_t<64, false>(a, stream);
  return causal ? launch_kv_t<128, true>(a, stream) : launch_kv_t<128, false>(a, stream);
}

hipError_t launch_bwd_q(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_q_t<64, true>(a, stream) : launch_q_t<64, false>(a, stream);
  return causal ? launch_q_t<128, true>(a, stream) : launch_q_t<128, false>(a, stream);
}

hipError_t launch_bwd_kv_dropout(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_kv_t<64, true, true>(a, stream) : launch_kv_t<64, false, true>(a, stream);
  return causal ? launch_kv_t<128, true, true>(a, stream) : launch_kv_t<128, false, true>(a, stream);
}

hipError_t launch_bwd_q_dropout(const BwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_q_t<64, true, true>(a, stream) : launch_q_t<64, false, true>(a, stream);
  return causal ? launch_q_t<128, true, true>(a, stream) : launch_q_t<128, false, true>(a, stream);
}

}  // namespace fa
