// Fused attention forward for gfx950: O = softmax(scale * Q K^T) V and LSE.
//
// Method: the FlashAttention-2 forward outlined in the CMU 15-442/642 notes
// "Transformer、注意力机制与优化" (section "FlashAttention-2 算法"): Q is cut
// into row blocks, one per workgroup; K and V are streamed block by block
// through on-chip memory; a running row max m, row sum l and unnormalised
// output are updated with the notes' two-block merge (section
// "安全 Softmax 与在线 Softmax"); O is divided by l once at the end and only
// LSE = m + ln l is stored ("FlashAttention 系列技术详解", section
// "具体优化策略").  Work is split over (batch, head, query block) and, inside
// a workgroup, over query rows per wave, so no two waves ever combine partial
// results (CMU notes, section "并行化策略").
//
// gfx950 mapping (one workgroup = 8 waves = 256 query rows, 32 per wave; K/V
// tiles of 64 keys; one workgroup per CU, two waves per SIMD):
//  * ping-pong: waves w and w + 4 share a SIMD.  Each wave alternates a
//    matrix phase (S^T = K Q^T for tile t and O^T += V^T P^T for tile t - 1,
//    all MFMA and LDS reads) with a softmax phase (mask, row max, exp2, row
//    sum, bf16 packing: all VALU) for tile t.  Waves 0-3 and 4-7 run these
//    phases half a period apart, with one workgroup barrier per period, so on each
//    SIMD one wave keeps the matrix core busy while the other does the
//    softmax arithmetic.  Measured on gfx950, an MFMA-only wave and a
//    VALU-only wave on one SIMD overlap almost completely; two waves that
//    each mix both kinds of work do not;
//  * K and V tiles go global -> LDS with asynchronous 16-byte buffer loads
//    into three buffers each: tile t + 2 of K and t + 1 of V are in flight
//    while tile t is used.  Tiles are unpadded row-major with an XOR swizzle
//    of the 16-byte chunks, so that operand reads are free of bank conflicts;
//  * each wave computes S^T = K Q^T for its 32 queries with
//    v_mfma_f32_32x32x16_bf16, so a lane owns one query and 32 of the tile's
//    keys: the row max is an in-lane max plus one swap of wave halves, and the
//    row sum needs no cross-lane step until the end;
//  * K rows sit in LDS in swap23 order (bits 2 and 3 of the row swapped),
//    which makes each lane's 16 scores per 32-key block come out as two runs
//    of eight consecutive keys: rounded to bf16 they are directly the B
//    operand of O^T += V^T P^T;
//  * the V^T operand of that product is read from the row-major V tile with
//    the transposing LDS read (ds_read_b64_tr_b16);
//  * exponentials are base 2 with log2(e) folded into the scale; the running
//    max (and with it O and l) is moved only on tiles that raise some row's
//    max by more than 2^8 (kLazyThreshold), a branch the whole wave takes or
//    skips;
//  * causal: key tiles past the block's last query are never loaded, tiles
//    past a wave's last query are skipped by that wave, and only tiles that
//    straddle the diagonal (or the ragged end of the sequence) are masked.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct FwdCfg {
  static constexpr int NW = 8;                      // waves per workgroup
  static constexpr int NT = NW * 64;                // threads per workgroup
  static constexpr int QW = 32;                     // query rows per wave
  static constexpr int BR = NW * QW;                // query rows per workgroup
  static constexpr int BC = 64;                     // keys per K/V tile
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE = BC * D;               // elements per K or V tile
  static constexpr int COPIES = BC * CPR / NT;      // 16-byte copies per thread per tile
  static_assert(COPIES >= 1 && COPIES * NT == BC * CPR, "tile copies must split evenly");
};

// Largest growth of the probabilities (in log2 units) tolerated before the
// running max is moved (and O and the row sums rescaled).
//  * Lazy (the O and LSE outputs): 8, so probabilities stay below 2^8 and the
//    max moves only when a tile raises some row of the wave by more than
//    that; with N(0, 1) inputs that is the first tile of the row.  A stale
//    max makes the dominant probability of a nearly one-hot row some 2^x,
//    whose bf16 rounding (relative error up to 2^-8) would land on O
//    undivided.  So the sum O is divided by also takes, for each tile, the
//    rounding error of the tile's largest probability (the bf16 value the
//    P V product used, minus the fp32 one): a one-hot row then gives its V
//    row exactly, as with an exact max, at six vector operations per tile
//    instead of 64 multiplies of O on most tiles.  LSE keeps the sum of the
//    unrounded probabilities.
//  * Eager (the split-KV partials, whose merge takes one row sum per range):
//    0, the max moves whenever a tile raises it, so the dominant probability
//    is exactly 1 when rounded.
constexpr float kLazyThreshold = 8.f;

// Per-lane source offsets of the asynchronous tile copies.  Copy t of a lane
// fills 16-byte slot (t * NW + w) * 64 + lane of a tile: row r = slot / CPR,
// physical chunk slot % CPR, which holds logical chunk pc ^ swizzle(r).  V row
// r is key r of the tile; K row r is key swap23(r), so that lane c of the
// S^T product reads LDS row c and still gets key swap23(c).  The offsets are
// the same for every tile and are computed once; a tile that runs past the
// end of the sequence clamps its keys to N - 1 (finite data for keys that are
// masked anyway).
template <int D>
struct TileCopy {
  using C = FwdCfg<D>;
  uint32_t koff[C::COPIES];  // byte offsets of the lane's 16 bytes in K and V
  uint32_t voff[C::COPIES];

  __device__ __forceinline__ static int slot_row(int t, int w, int lane) {
    return ((t * C::NW + w) * 64 + lane) / C::CPR;
  }

  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int t = 0; t < C::COPIES; ++t) {
      const int slot = (t * C::NW + w) * 64 + lane;
      const int r = slot / C::CPR;
      const int chunk = ((slot % C::CPR) ^ chunk_swizzle<D>(r)) << 3;
      koff[t] = 2 * (swap23(r) * D + chunk);
      voff[t] = 2 * (r * D + chunk);
    }
  }

  // One tile (rows k0 .. k0 + BC - 1) of K (KEYS) or V (!KEYS) into Ts.
  // UNI: pass the resource words through readfirstlane (all of them are
  // wave-uniform, but in the dropout kernel the compiler loses track of that
  // for some copies and would put the scalar operands in vector registers).
  template <bool KEYS, bool UNI = false>
  __device__ __forceinline__ void issue(const uint16_t* Xh, uint16_t* Ts, int k0, int N, int w,
                                        int lane) const {
    i32x4 rs = make_rsrc_words(Xh + (int64_t)k0 * D, C::BC * D * 2);
    if constexpr (UNI) {
#pragma unroll
      for (int e = 0; e < 2; ++e) rs[e] = __builtin_amdgcn_readfirstlane(rs[e]);
    }
    const int wb = opaque_s(w * 64 * 8);  // this wave's slots
    if (k0 + C::BC <= N) {
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t)
        buffer_load_lds16_unseen(rs, KEYS ? koff[t] : voff[t], Ts + t * C::NW * 64 * 8 + wb);
    } else {
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t) {
        // not worth a register across the loop
        const int r = opaque(KEYS ? swap23(slot_row(t, w, lane)) : slot_row(t, w, lane));
        const int shift = (min(k0 + r, N - 1) - (k0 + r)) * D * 2;
        buffer_load_lds16_unseen(rs, (KEYS ? koff[t] : voff[t]) + shift,
                                 Ts + t * C::NW * 64 * 8 + wb);
      }
    }
  }
};

// LDS of one forward workgroup: three K and three V tile buffers.  The tile
// copies are invisible to the compiler; the period structure orders every
// read of a buffer after the wait and barrier that follow its copy.
struct FwdSmem {
  uint16_t* k[3];
  uint16_t* v[3];
};

template <int D, bool CAUSAL, bool DROP, bool LAZY>
struct FwdWave {
  using C = FwdCfg<D>;
  static constexpr int BC = C::BC;
  static constexpr float kThreshold = LAZY ? kLazyThreshold : 0.f;

  FwdSmem sm;
  DropArgs drop;  // dropout (DROP only)
  int bh;
  const uint16_t* Kh;
  const uint16_t* Vh;
  const uint16_t* Qh;
  int w, grp, lane, c32, g, N, Nk, qw0, qrow;  // N queries, Nk keys per head
  int t0;       // first key tile of this workgroup's key range
  int nt, ntw;  // tiles in the range; of those, tiles this wave sees (causal)
  float sl2;
  float m_run;   // running max of scale*log2(e)*s
  float l_part;  // this lane's share of the running row sum
  float l_corr;  // LAZY: sum over tiles of bf16(p_max) - p_max (the same in both halves)
  bf16x8 qf[D / 16];
  f32x16 oacc[D / 32];  // O^T: lane holds O[qrow][32 db + 8(i/4) + 4g + i%4]
  f32x16 s[BC / 32];    // S^T of the tile between the matrix and softmax phases
  bf16x8 pb[BC / 16];   // P^T of the tile between the softmax and matrix phases
  TrLane<D> trv;        // transposed reads of the V tile
  int kbase, ku;        // row reads of the K tile (row c32 of each 32-key block)
  TileCopy<D> cp;       // per-lane offsets of the tile copies

  // S^T = K Q^T for the tile in K buffer KB.  Value i of s[sb] is the score
  // of key 32 sb + 16 (i / 8) + 8 g + i % 8 of the tile against qrow.
  template <int KB>
  __device__ __forceinline__ void scores() {
    const uint16_t* Ks = sm.k[KB];
    const int kb = opaque(kbase), kx = opaque(ku);
#pragma unroll
    for (int sb = 0; sb < BC / 32; ++sb) s[sb] = zero16();
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
#pragma unroll
      for (int sb = 0; sb < BC / 32; ++sb) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(Ks + sb * 32 * D + kb + (((2 * kc) ^ kx) << 3));
        s[sb] = mfma32(ka, qf[kc], s[sb]);
      }
    // keep the K reads two contraction slices ahead of the MFMAs using them
    sched_pipeline<D / 16, BC / 32, BC / 32, 2>();
  }

  // O^T += V^T P^T for the tile in V buffer VB over its four 16-key chunks.
  // B operand: P^T chunk kc2 (keys 16 kc2 + 8 g + 0..7 of this lane's query).
  // A operand: V^T rows 32 db + c32, read transposed from the V tile.
  template <int VB>
  __device__ __forceinline__ void pv() {
    const uint16_t* Vs = sm.v[VB];
    const TrLane<D> tr = trv.fresh();
#pragma unroll
    for (int kc2 = 0; kc2 < BC / 16; ++kc2)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 va = join_tr(lds_read_tr(Vs + tr.off(16 * kc2, 32 * db, 0)),
                                  lds_read_tr(Vs + tr.off(16 * kc2, 32 * db, 1)));
        oacc[db] = mfma32(va, pb[kc2], oacc[db]);
      }
    // keep the V reads one 16-key chunk ahead of the MFMAs using them
    sched_pipeline<BC / 16, 2 * (D / 32), D / 32, 1>();
  }

  // Matrix phase of period t: S^T of tile t (K buffer KB) and O^T += V^T P^T
  // of tile t - 1 (V buffer VB), each only where this wave has that tile.
  template <int KB, int VB>
  __device__ __forceinline__ void matrix_phase(int t) {
    const bool do_s = t < ntw;
    const bool do_pv = t >= 1 && t - 1 < ntw;
    if (do_s) scores<KB>();
    if (do_pv) pv<VB>();
  }

  // Softmax phase for tile t: P^T = exp2(scale log2(e) S^T - m) into pb,
  // with the lazy move of the running max.
  __device__ __forceinline__ void softmax_phase(int t) {
    if (t < 0 || t >= ntw) return;
    const int k0 = (t0 + t) * BC;
    const bool need_mask = (k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > qw0));
    if (need_mask) {
      // key k0 + 8 g + o is visible iff o <= lim (o is a compile-time offset).
      // The select is bit arithmetic on a sign mask kept opaque, so that it
      // stays in vector registers instead of 32 live compare masks in
      // scalar register pairs.
      const int lim = opaque((CAUSAL ? min(Nk - 1, qrow) : Nk - 1) - k0 - 8 * g);
#pragma unroll
      for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t hide = (uint32_t)opaque((lim - (32 * sb + 16 * (i >> 3) + (i & 7))) >> 31);
          s[sb][i] = __uint_as_float((__float_as_uint(s[sb][i]) & ~hide) | (0xff800000u & hide));
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
    const float mraw = max_halves(mx);  // the row's largest score in the tile (-inf if none)
    mx = mraw * sl2;
    // Move the running max when this tile raises it for some query of the
    // wave (always on the first visible tile, where m = -inf).
    if (__ballot(mx > m_run + kThreshold)) {
      const float m_new = fmaxf(m_run, mx);
      // a query with every key so far masked keeps m = -inf and nothing to rescale
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
      if constexpr (LAZY) l_corr *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    if constexpr (LAZY) {
      // the tile's largest probability exactly as the loop below computes it
      const float pt = exp2_fast(fmaf(mraw, sl2, -m_use));
      l_corr += __uint_as_float(pack2(0.f, pt) & 0xffff0000u) - pt;
    }
    // Dropout bytes of this lane's keys 16 n + 8 g + 0..7 (chunk n): the
    // lane computes the Philox call of 16-key group n = 2 m + g and swaps
    // half of it with the other wave half, which computed group 2 m + 1 - g.
    // After v_permlane32_swap(X = words 0-1, Y = words 2-3) both halves hold
    // group 2 m's words in X and group 2 m + 1's in Y.
    uint32_t rw[BC / 16][2];
    if constexpr (DROP) {
      const uint32_t jg0 = (uint32_t)(((t0 + t) * BC) >> 4);
#pragma unroll
      for (int m = 0; m < BC / 32; ++m) {
        const u32x4 own = philox4x32_10(jg0 + 2 * m + g, (uint32_t)qrow, (uint32_t)bh,
                                        drop.offset, drop.k0, drop.k1);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(own[e], own[2 + e], false, false);
          rw[2 * m][e] = r[0];
          rw[2 * m + 1][e] = r[1];
        }
      }
    }
    float rs = 0.f;
#pragma unroll
    for (int kc2 = 0; kc2 < BC / 16; ++kc2) {
      float p[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        p[jj] = exp2_fast(fmaf(s[kc2 >> 1][(kc2 & 1) * 8 + jj], sl2, -m_use));
        rs += p[jj];
      }
      // the row sums take every probability; the product with V only the kept ones
      if constexpr (DROP) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          p[jj] = drop_keep(rw[kc2][jj >> 2], jj & 3, drop.t) ? p[jj] : 0.f;
      }
      pb[kc2] = pack8(p);
    }
    l_part += rs;
  }

  // Per-item fields for query block qb of head bh and key range `split` of
  // `splits`, with a fresh running max and sum.
  __device__ __forceinline__ void begin_item(const FwdArgs& a, int bh_, int qb, int split,
                                             int splits) {
    bh = bh_;
    const int64_t koff = (int64_t)bh * Nk * D;
    Kh = a.k + koff;
    Vh = a.v + koff;
    Qh = a.q + (int64_t)bh * N * D;
    const int q0 = qb * C::BR;
    qw0 = q0 + (2 * (w & 3) + grp) * C::QW;
    qrow = qw0 + c32;  // the query this lane owns
    // key tiles the block sees, then this workgroup's range of them
    int nt_all = (Nk + BC - 1) / BC;
    if (CAUSAL) nt_all = min(nt_all, (q0 + C::BR + BC - 1) / BC);
    t0 = split * nt_all / splits;
    const int t1 = (split + 1) * nt_all / splits;
    nt = t1 - t0;
    const int ntw_all = CAUSAL ? min(nt_all, (qw0 + C::QW + BC - 1) / BC) : nt_all;
    ntw = max(0, min(nt, ntw_all - t0));
    if (qw0 >= N) ntw = 0;  // no real query in this wave: copies and barriers only
    m_run = -INFINITY;
    l_part = 0.f;
    l_corr = 0.f;
  }

  // K tiles 0 and 1 and V tile 0 of the item's range, before its first
  // period (an empty range, possible only for a split, copies nothing), and
  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16 kc + 8 g + 0..7].
  __device__ __forceinline__ void issue_prologue(const FwdArgs& a) {
    if (nt > 0) {
      cp.template issue<true>(Kh, sm.k[0], t0 * BC, Nk, w, lane);
      if (nt > 1) cp.template issue<true>(Kh, sm.k[1], (t0 + 1) * BC, Nk, w, lane);
      cp.template issue<false>(Vh, sm.v[0], t0 * BC, Nk, w, lane);
    }
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
      qf[kc] = qrow < N ? load_global<bf16x8>(Qh + (int64_t)qrow * D + kc * 16 + g * 8)
                        : zero_bf16x8();
  }

  // The row sum O is divided by: l with the rounding corrections (LAZY).
  __device__ __forceinline__ float lazy_sum(float l) const { return LAZY ? l + l_corr : l; }

  __device__ __forceinline__ void zero_o() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
  }

  // Epilogue of the item with head bh_ whose lane row is row: one division
  // by lo, the row sum O is normalised with (and the dropout rescale),
  // LSE = (m + log2 l) ln 2.
  __device__ __forceinline__ void store_out(const FwdArgs& a, int bh_, int row, float l,
                                            float lo, float m) const {
    if (row >= N) return;
    const float inv = DROP ? drop.scale / lo : 1.f / lo;
    uint16_t* Orow = a.o + (int64_t)bh_ * N * D + (int64_t)row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 val;
        val.x = pack2(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv);
        val.y = pack2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2*>(Orow + db * 32 + 8 * r4 + 4 * g) = val;
      }
    if (g == 0) a.lse[(int64_t)bh_ * N + row] = (m + log2_fast(l)) * kLn2;
  }

  // One period (two slots) of a wave of group GRP.  R = t mod 3 names the
  // buffers: K tile t in K buffer R, V tile t - 1 in V buffer (R + 2) mod 3.
  // The period also starts the copies of K tile t + 2 (into the buffer of K
  // tile t - 1) and V tile t + 1 (into the buffer of V tile t - 2), both last
  // read in the previous period, and ends at a workgroup barrier once K tile
  // t + 1 and V tile t are in LDS for the next one.  Group 0 runs the matrix
  // phase of tile t in the first slot and its softmax phase in the second;
  // group 1 runs the softmax phase of tile t - 1 and then the matrix phase of
  // tile t.  No barrier separates the slots: nothing read in one slot is
  // written in the other, and the two groups' phases are of similar length,
  // so they stay in step on their own (a barrier between the slots cost 1-2%;
  // the FP8 forward, whose softmax phase is the longer one, keeps it).
  template <int R, int GRP>
  __device__ __forceinline__ void period(int t) {
    constexpr int KB = R, VB = (R + 2) % 3, KN = (R + 2) % 3, VN = (R + 1) % 3;
    const bool kn = t + 2 < nt, vn = t + 1 < nt;
    // Each wave starts its share of the copies in the slot that has room for
    // them: the softmax slot without dropout (off the matrix phase's critical
    // path), the matrix slot with dropout, whose softmax slot (with its Philox
    // draws) is the longer one.  Measured on C5: 0.275 against 0.290 ms
    // without dropout, 0.384 against 0.393 with it.
    constexpr bool CP_M = DROP;
    // this wave's share of the copies of K tile t + 2 and V tile t + 1
    auto copies = [&](int t_, bool kn_, bool vn_) {
      if (kn_) cp.template issue<true, DROP>(Kh, sm.k[KN], (t0 + t_ + 2) * BC, Nk, w, lane);
      if (vn_) cp.template issue<false, DROP>(Vh, sm.v[VN], (t0 + t_ + 1) * BC, Nk, w, lane);
    };
    if (GRP == 0) {
      if (CP_M) copies(t, kn, vn);
      matrix_phase<KB, VB>(t);
    } else {
      if (!CP_M) copies(t, kn, vn);
      softmax_phase(t - 1);
    }
    if (GRP == 0) {
      if (!CP_M) copies(t, kn, vn);
      softmax_phase(t);
    } else {
      if (CP_M) copies(t, kn, vn);
      matrix_phase<KB, VB>(t);
    }
    if (kn) wait_vmem_except_last<2 * C::COPIES>();
    else if (vn) wait_vmem_except_last<C::COPIES>();
    else wait_vmem();
    block_barrier();
  }

  // Periods 0 .. nt (the last one only finishes O^T += V^T P^T of the last
  // tile).  Both groups pass the same sequence of barriers.
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

// SPLIT: workgroup = (head, query block, key range); writes the range's
// unnormalised partials (see FwdArgs) instead of O and LSE.
// DROP: dropout on the probabilities (a.drop); never combined with SPLIT.
template <int D, bool CAUSAL, bool SPLIT, bool DROP = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_kernel(FwdArgs a) {
  static_assert(!(SPLIT && DROP), "split-KV forward has no dropout");
  using C = FwdCfg<D>;
  constexpr int TILE = C::TILE;
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k2s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v2s[TILE];

  const int tid = threadIdx.x;
  const int N = a.N;
  const int nqb = (N + C::BR - 1) / C::BR;

  // per-lane constants, the same for every item
  FwdWave<D, CAUSAL, DROP, !SPLIT> f;
  f.sm = FwdSmem{{k0s, k1s, k2s}, {v0s, v1s, v2s}};
  f.drop = a.drop;
  f.w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // Waves w and w + 4 run on the same SIMD: they form a ping-pong pair and
  // take adjacent 32-row chunks, so the pair's causal work is balanced.
  f.grp = f.w >> 2;
  f.lane = tid & 63;
  f.c32 = f.lane & 31;
  f.g = f.lane >> 5;
  f.N = N;
  f.Nk = SPLIT ? a.Nk : N;  // the same value as N outside the split-KV forward
  f.sl2 = a.scale_log2;
  f.trv = TrLane<D>(f.lane);
  f.kbase = f.c32 * D;
  f.ku = f.g ^ chunk_swizzle<D>(f.c32);
  f.cp.init(f.w, f.lane);

  if constexpr (SPLIT) {
    // Workgroup -> (head, query block, key range): heads grouped per XCD,
    // heaviest (last) causal query blocks first.
    const int split = (int)(blockIdx.x % (unsigned)a.splits);
    const int total = (int)(gridDim.x / (unsigned)a.splits);
    int bh, qb;
    xcd_head_block<kHeadsPerGroup>((int)(blockIdx.x / (unsigned)a.splits), total, a.BH, nqb, bh,
                                   qb);
    if (CAUSAL) qb = nqb - 1 - qb;
    f.begin_item(a, bh, qb, split, a.splits);
    f.issue_prologue(a);
    f.zero_o();
    wait_vmem();
    block_barrier();
    if (f.nt > 0) {
      if (f.grp == 0) f.template run<0>();
      else f.template run<1>();
    }
    const float l = sum_halves(f.l_part);
    // the range's partials, relative to its own running max
    if (f.qrow < N) {
      const int64_t row = ((int64_t)split * a.BH + bh) * N + f.qrow;
      float* Orow = a.opart + row * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = f.oacc[db][4 * r4 + e];
          *reinterpret_cast<f32x4*>(Orow + db * 32 + 8 * r4 + 4 * f.g) = val;
        }
      if (f.g == 0) {
        a.mpart[row] = f.m_run;
        a.lpart[row] = l;
      }
    }
  } else {
    // Persistent: the grid walks the (head, query block) items in run order
    // (heads grouped per XCD, heaviest causal query blocks first).  After an
    // item's last period every buffer is free, so the next item's first
    // copies and Q loads are issued before this item's epilogue and overlap
    // it.
    const ItemWalk walk{(int)blockIdx.x, (int)gridDim.x, a.BH * nqb};
    int bh, qb;
    xcd_head_block<kHeadsPerGroup>(walk.item(0), walk.total, a.BH, nqb, bh, qb);
    f.begin_item(a, bh, CAUSAL ? nqb - 1 - qb : qb, 0, 1);
    f.issue_prologue(a);
    f.zero_o();
    wait_vmem();
    block_barrier();
    for (int r = 1;; ++r) {
      // fresh copies of the per-lane constants each item, so that nothing
      // derived from them is hoisted out of the item loop and held across it
      f.kbase = opaque(f.kbase);
      f.ku = opaque(f.ku);
      f.trv = f.trv.fresh();
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t) {
        f.cp.koff[t] = (uint32_t)opaque((int)f.cp.koff[t]);
        f.cp.voff[t] = (uint32_t)opaque((int)f.cp.voff[t]);
      }
      if (f.grp == 0) f.template run<0>();
      else f.template run<1>();
      const float l = sum_halves(f.l_part);
      const float lo = f.lazy_sum(l);
      const float m = f.m_run;
      const int cur_bh = f.bh, cur_row = f.qrow;
      const int L = walk.item(r);
      if (L >= 0) {
        xcd_head_block<kHeadsPerGroup>(L, walk.total, a.BH, nqb, bh, qb);
        f.begin_item(a, bh, CAUSAL ? nqb - 1 - qb : qb, 0, 1);
        f.issue_prologue(a);
      }
      f.store_out(a, cur_bh, cur_row, l, lo, m);
      if (L < 0) break;
      f.zero_o();
      // the previous item's scores and probabilities are dead: say so
#pragma unroll
      for (int sb = 0; sb < C::BC / 32; ++sb) f.s[sb] = zero16();
#pragma unroll
      for (int kc2 = 0; kc2 < C::BC / 16; ++kc2) f.pb[kc2] = zero_bf16x8();
      wait_vmem();
      block_barrier();
    }
  }
}

// Merge of the split-KV partials (Flash-Decoding's combine step, CMU notes
// section "Flash-Decoding"; the two-block merge of section "安全 Softmax 与
// 在线 Softmax" applied over all ranges at once): per row
//   M = max_s m_s,  w_s = 2^(m_s - M),  L = sum_s w_s l_s,
//   O = sum_s w_s O_s / L,  LSE = (M + log2 L) ln 2.
// A range that saw no visible key has m_s = -inf, l_s = 0, O_s = 0 and
// weight 0.  D / 4 threads per row, 4 columns each.
template <int D>
__global__ void __launch_bounds__(256) fa_fwd_merge_kernel(FwdArgs a) {
  constexpr int TPR = D / 4;        // threads per row
  constexpr int RPB = 256 / TPR;    // rows per workgroup
  const int64_t rows = (int64_t)a.BH * a.N;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int col = (threadIdx.x % TPR) * 4;
  if (row >= rows) return;
  const int64_t plane = rows;       // rows per split
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.mpart[s * plane + row]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) {
    const float m = a.mpart[s * plane + row];
    const float wgt = m == -INFINITY ? 0.f : exp2_fast(m - M);
    L = fmaf(wgt, a.lpart[s * plane + row], L);
    const f32x4 o = *reinterpret_cast<const f32x4*>(a.opart + (s * plane + row) * D + col);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, o[e], acc[e]);
  }
  const float inv = 1.f / L;
  u32x2 val;
  val.x = pack2(acc[0] * inv, acc[1] * inv);
  val.y = pack2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(a.o + row * D + col) = val;
  if (col == 0) a.lse[row] = (M + log2_fast(L)) * kLn2;
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int64_t nqb = (a.N + C::BR - 1) / C::BR;
  // persistent: one workgroup per CU (the kernel's registers allow no more)
  const int64_t grid = persistent_grid(nqb * a.BH);
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, false>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_splitkv_t(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int64_t nqb = (a.N + C::BR - 1) / C::BR;
  const int64_t grid = nqb * a.BH * a.splits;
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, true>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPB = 256 / (D / 4);
  const int64_t rows = (int64_t)a.BH * a.N;
  hipLaunchKernelGGL((fa_fwd_merge_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                     0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_fwd_t<64, true>(a, stream) : launch_fwd_t<64, false>(a, stream);
  return causal ? launch_fwd_t<128, true>(a, stream) : launch_fwd_t<128, false>(a, stream);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_dropout_t(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int64_t nqb = (a.N + C::BR - 1) / C::BR;
  const int64_t grid = persistent_grid(nqb * a.BH);
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, false, true>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_dropout(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_fwd_dropout_t<64, true>(a, stream) : launch_fwd_dropout_t<64, false>(a, stream);
  return causal ? launch_fwd_dropout_t<128, true>(a, stream)
                : launch_fwd_dropout_t<128, false>(a, stream);
}

hipError_t launch_fwd_splitkv(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_fwd_splitkv_t<64, true>(a, stream) : launch_fwd_splitkv_t<64, false>(a, stream);
  return causal ? launch_fwd_splitkv_t<128, true>(a, stream)
                : launch_fwd_splitkv_t<128, false>(a, stream);
}

}  // namespace fa
