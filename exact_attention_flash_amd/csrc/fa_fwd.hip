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
// gfx950 mapping (one workgroup = 4 waves = 128 query rows; K/V tiles of 64
// keys; two workgroups per CU):
//  * K and V tiles go global -> LDS with asynchronous 16-byte copies
//    (global_load_lds_dwordx4) into a double buffer: the next tile is in
//    flight while the current one is used, and no register holds staging
//    data.  Tiles are unpadded row-major with an XOR swizzle of the 16-byte
//    chunks, so that operand reads are free of bank conflicts;
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
//  * exponentials are base 2 with log2(e) folded into the scale, and the
//    running max is only moved (and O, l rescaled) when a tile's max exceeds
//    it by more than 2^8: until then the probabilities are taken relative to
//    the stale max, which changes nothing after the final division by l;
//  * causal: key tiles past the block's last query are never loaded, tiles
//    past a wave's last query are skipped by that wave, and only tiles that
//    straddle the diagonal (or the ragged end of the sequence) are masked.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct FwdCfg {
  static constexpr int NW = 4;                      // waves per workgroup
  static constexpr int NT = NW * 64;                // threads per workgroup
  static constexpr int QW = 32;                     // query rows per wave
  static constexpr int BR = NW * QW;                // query rows per workgroup
  static constexpr int BC = 64;                     // keys per K/V tile
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE = BC * D;               // elements per K or V tile
  static constexpr int COPIES = BC * CPR / NT;      // 16-byte copies per thread per tile
};

// Largest growth of the probabilities (in log2 units) tolerated before the
// running max is moved.
constexpr float kRescaleThreshold = 8.f;

// Per-lane source offsets of the asynchronous tile copies.  Copy t of a lane
// fills 16-byte slot (t * NW + w) * 64 + lane of a tile: row r = slot / CPR,
// physical chunk slot % CPR, which holds logical chunk pc ^ swizzle(r).  V row
// r is key r of the tile; K row r is key swap23(r), so that lane c of the
// S^T product reads LDS row c (conflict-free) and still gets key swap23(c).
// The offsets are the same for every tile and are computed once; a tile
// that runs past the end of the sequence clamps its keys to N - 1 (finite
// data for keys that are masked anyway).
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

  __device__ __forceinline__ void issue(const uint16_t* Kh, const uint16_t* Vh, uint16_t* Ks,
                                        uint16_t* Vs, int k0, int N, int w, int lane) const {
    constexpr uint32_t kTileBytes = C::BC * D * 2;
    const buf_rsrc kr = make_rsrc(Kh + (int64_t)k0 * D, kTileBytes);
    const buf_rsrc vr = make_rsrc(Vh + (int64_t)k0 * D, kTileBytes);
    if (k0 + C::BC <= N) {
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t) {
        const int base = (t * C::NW + w) * 64 * 8;
        buffer_load_lds16(kr, koff[t], Ks + base);
        buffer_load_lds16(vr, voff[t], Vs + base);
      }
    } else {
#pragma unroll
      for (int t = 0; t < C::COPIES; ++t) {
        const int base = (t * C::NW + w) * 64 * 8;
        const int r = slot_row(t, w, lane);
        const int kr_row = swap23(r);
        const int kshift = (min(k0 + kr_row, N - 1) - (k0 + kr_row)) * D * 2;
        const int vshift = (min(k0 + r, N - 1) - (k0 + r)) * D * 2;
        buffer_load_lds16(kr, koff[t] + kshift, Ks + base);
        buffer_load_lds16(vr, voff[t] + vshift, Vs + base);
      }
    }
  }
};

// LDS of one forward workgroup: K and V tiles of two stages, each its own
// object.  Separate objects let the compiler see that the copies into one
// stage never overlap reads of the other, so it does not wait for the
// in-flight copies before reading the current tile.
template <int D>
struct FwdSmem {
  uint16_t* k0;
  uint16_t* v0;
  uint16_t* k1;
  uint16_t* v1;
};

template <int D, bool CAUSAL>
struct FwdBlock {
  using C = FwdCfg<D>;
  static constexpr int BC = C::BC;

  FwdSmem<D> sm;
  const uint16_t* Kh;
  const uint16_t* Vh;
  int w, lane, c32, g, N, qw0, qrow, nt;
  float sl2;
  float m_run;   // running max of scale*log2(e)*s (possibly stale)
  float l_part;  // this lane's share of the running row sum
  bf16x8 qf[D / 16];
  f32x16 oacc[D / 32];  // O^T: lane holds O[qrow][32 db + 8(i/4) + 4g + i%4]
  TrLane<D> trv;        // transposed reads of the V tile
  int kbase, ku;        // row reads of the K tile (row c32 of each 32-key block)
  TileCopy<D> cp;       // per-lane offsets of the tile copies

  template <int ST>
  __device__ __forceinline__ uint16_t* ktile() const { return ST ? sm.k1 : sm.k0; }
  template <int ST>
  __device__ __forceinline__ uint16_t* vtile() const { return ST ? sm.v1 : sm.v0; }

  template <int ST>
  __device__ __forceinline__ void issue(int j) {
    cp.issue(Kh, Vh, ktile<ST>(), vtile<ST>(), j * BC, N, w, lane);
  }

  // One key tile from stage ST; prefetches tile j + 1 into the other stage.
  template <int ST>
  __device__ __forceinline__ void step(int j) {
    if (j + 1 < nt) issue<ST ^ 1>(j + 1);
    const uint16_t* Ks = ktile<ST>();
    const uint16_t* Vs = vtile<ST>();
    const int k0 = j * BC;
    const bool skip = CAUSAL && (k0 > qw0 + C::QW - 1);
    if (!skip) {
      const TrLane<D> tr = trv.fresh();
      const int kb = opaque(kbase), kx = opaque(ku);
      // S^T for the tile: two 32-key blocks.  Value i of s[sb] is the score
      // of key k0 + 32 sb + 16 (i / 8) + 8 g + i % 8 against qrow.
      f32x16 s[BC / 32];
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
      // keep the K reads two slices ahead of the MFMAs that consume them
      sched_pipeline<D / 16, BC / 32, BC / 32, 2>();
      const bool need_mask = (k0 + BC > N) || (CAUSAL && (k0 + BC - 1 > qw0));
      if (need_mask) {
#pragma unroll
        for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * sb + 16 * (i >> 3) + 8 * g + (i & 7);
            if (key >= N || (CAUSAL && key > qrow)) s[sb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
      mx = fmaxf(mx, swap_halves(mx)) * sl2;
      // Move the running max only when some query's probabilities would grow
      // past 2^threshold (always on the first visible tile, where m = -inf).
      if (__ballot(mx > m_run + kRescaleThreshold)) {
        const float m_new = fmaxf(m_run, mx);
        // a query with every key so far masked keeps m = -inf and nothing to rescale
        const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_fast(fmaf(s[sb][i], sl2, -m_use));
          s[sb][i] = p;
          rs += p;
        }
      l_part += rs;
      // O^T += V^T P^T over the tile's four 16-key chunks.  B operand: P^T
      // chunk kc2 (keys k0 + 16 kc2 + 8 g + 0..7 of this lane's query).  A
      // operand: V^T rows 32 db + c32, read transposed from the V tile.
#pragma unroll
      for (int kc2 = 0; kc2 < BC / 16; ++kc2) {
        float t[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) t[jj] = s[kc2 >> 1][(kc2 & 1) * 8 + jj];
        const bf16x8 pb = pack8(t);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 va = join_tr(lds_read_tr(Vs + tr.off(16 * kc2, 32 * db, 0)),
                                    lds_read_tr(Vs + tr.off(16 * kc2, 32 * db, 1)));
          oacc[db] = mfma32(va, pb, oacc[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  constexpr int TILE = C::TILE;
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[TILE];

  const int tid = threadIdx.x;
  const int N = a.N;
  const int nqb = (N + C::BR - 1) / C::BR;

  // Workgroup -> (head, query block).  Consecutive workgroup ids land on
  // different XCDs (round robin over 8); give each XCD a contiguous run of
  // work so the query blocks of one head share that XCD's L2.  Within a head
  // the heaviest (last) causal blocks go first.
  const int total = gridDim.x;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int bh = L / nqb;
  int qb = L - bh * nqb;
  if (CAUSAL) qb = nqb - 1 - qb;

  const int64_t hoff = (int64_t)bh * N * D;
  FwdBlock<D, CAUSAL> f;
  f.sm = FwdSmem<D>{k0s, v0s, k1s, v1s};
  f.Kh = a.k + hoff;
  f.Vh = a.v + hoff;
  f.w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  f.lane = tid & 63;
  f.c32 = f.lane & 31;
  f.g = f.lane >> 5;
  f.N = N;
  const int q0 = qb * C::BR;
  f.qw0 = q0 + f.w * C::QW;
  f.qrow = f.qw0 + f.c32;  // the query this lane owns
  f.nt = (N + C::BC - 1) / C::BC;
  if (CAUSAL) f.nt = min(f.nt, (q0 + C::BR + C::BC - 1) / C::BC);
  f.sl2 = a.scale_log2;
  f.m_run = -INFINITY;
  f.l_part = 0.f;
  f.trv = TrLane<D>(f.lane);
  f.kbase = f.c32 * D;
  f.ku = f.g ^ chunk_swizzle<D>(f.c32);
  f.cp.init(f.w, f.lane);

  f.template issue<0>(0);
  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16 kc + 8 g + 0..7].
  const uint16_t* Qh = a.q + hoff;
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc)
    f.qf[kc] = f.qrow < N ? load_global<bf16x8>(Qh + (int64_t)f.qrow * D + kc * 16 + f.g * 8)
                          : zero_bf16x8();
#pragma unroll
  for (int db = 0; db < D / 32; ++db) f.oacc[db] = zero16();
  wait_vmem();
  __syncthreads();

  int j = 0;
  for (; j + 1 < f.nt; j += 2) {
    f.template step<0>(j);
    f.template step<1>(j + 1);
  }
  if (j < f.nt) f.template step<0>(j);

  // Epilogue: one division by l, LSE = (m + log2 l) ln 2.
  const float l = f.l_part + swap_halves(f.l_part);
  if (f.qrow < N) {
    const float inv = 1.f / l;
    uint16_t* Orow = a.o + hoff + (int64_t)f.qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 val;
        val.x = pack2(f.oacc[db][4 * r4 + 0] * inv, f.oacc[db][4 * r4 + 1] * inv);
        val.y = pack2(f.oacc[db][4 * r4 + 2] * inv, f.oacc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2*>(Orow + db * 32 + 8 * r4 + 4 * f.g) = val;
      }
    if (f.g == 0) a.lse[(int64_t)bh * N + f.qrow] = (f.m_run + log2_fast(l)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int64_t nqb = (a.N + C::BR - 1) / C::BR;
  const int64_t grid = nqb * a.BH;
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_fwd_t<64, true>(a, stream) : launch_fwd_t<64, false>(a, stream);
  return causal ? launch_fwd_t<128, true>(a, stream) : launch_fwd_t<128, false>(a, stream);
}

}  // namespace fa
