// Device-side building blocks shared by the forward and backward kernels:
// vector types, the gfx950 bf16 MFMA, bf16 packing and small cross-lane ops.
//
// MFMA 32x32x16 (v_mfma_f32_32x32x16_bf16) register layout, for a wave of 64
// lanes, lane = 32 * g + c with c in [0, 32) and g in {0, 1}:
//   A (32 x 16, row-major view): lane holds A[c][8g .. 8g+7]
//   B (16 x 32):                 lane holds B[8g .. 8g+7][c]
//   C (32 x 32, fp32):           lane holds C[8(i/4) + 4g + i%4][c], i < 16
// so a lane owns one output column and 16 of its rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

// fp32 -> bf16, round to nearest even (gfx950 has a native converter).
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
  return r;
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// 2^x on the transcendental unit; exact 0 for -inf.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// log2 on the transcendental unit, for positive normal inputs.
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// max(x[lane], x[lane ^ 32]) and x[lane] + x[lane ^ 32] with one
// v_permlane32_swap (gfx950): swapping one wave half of x against the other
// leaves the two values of each lane pair in the two results.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup id -> (head, block-in-run-order) for a grid of BH * nblk
// workgroups.  Consecutive workgroup ids land on different XCDs (round robin
// over 8).  When the heads split evenly over the XCDs, XCD x takes heads
// x * BH/8 .. x * BH/8 + BH/8 - 1 in groups of G and walks each group block
// by block (run order 0 for every head of the group first, then 1, ...).
// A group's K and V (or Q and dO) are shared by the XCD's L2 and the
// device-wide last-level cache while it runs, and callers that map run
// order 0 to their heaviest block start the longest work first; the light
// blocks that end a group overlap the heavy blocks that start the next.  Otherwise each XCD takes a contiguous run of
// (head, block) pairs.
template <int G>
__device__ __forceinline__ void xcd_head_block(int wg, int total, int BH, int nblk, int& bh,
                                               int& blk) {
  if ((BH & 7) == 0) {
    const int hpx = BH >> 3;
    const int j = wg >> 3;
    const int gsz = min(G, hpx);
    const int grp = j / (gsz * nblk);
    const int g0 = grp * gsz;
    const int gs = min(gsz, hpx - g0);  // the last group may be smaller
    const int r = j - grp * gsz * nblk;
    bh = (wg & 7) * hpx + g0 + r % gs;
    blk = r / gs;
  } else {
    int L = wg;
    if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
    bh = L / nblk;
    blk = L - bh * nblk;
  }
}

// The items (head, block) of a persistent kernel: round r of workgroup b
// takes item(r), an index in the run order of xcd_head_block.  With the item
// count and the grid both multiples of 8, workgroup b stays on the XCD of its
// items (b mod 8, as consecutive workgroups are placed round robin over the
// 8 XCDs) and walks that XCD's list in snake order (forward in even rounds,
// backward in odd ones), which pairs the heavy early causal blocks with light
// late ones; otherwise round robin over all items.
struct ItemWalk {
  int b, G, total;
  __device__ __forceinline__ int item(int r) const {
    if (((total | G) & 7) == 0) {
      const int g = G >> 3, c = b >> 3;
      const int j = r * g + ((r & 1) ? g - 1 - c : c);
      return j < (total >> 3) ? 8 * j + (b & 7) : -1;
    }
    const int L = b + r * G;
    return L < total ? L : -1;
  }
};

// Heads per group in xcd_head_block.  Measured on causal B=4 H=16 N=4096
// d=128 (forward + both backward passes): 4 heads per group beat 1 (which
// ends every group with a long tail) by 8% and 2 by 3%; 8 was within noise
// of 4 but fetched more from HBM.
constexpr int kHeadsPerGroup = 4;

// Workgroup barrier without a memory fence: unlike __syncthreads() it does
// not wait for this wave's outstanding global -> LDS copies.  The compiler
// may not move memory operations across it.  Callers wait for the copies a
// barrier must cover themselves (wait_vmem*).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename T>
__device__ __forceinline__ T load_global(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

}  // namespace fa

namespace fa {

// Row order used for tiles that feed the A operand of a 32x32 MFMA whose C
// rows must come out in runs of eight consecutive indices per lane: storing
// row r at LDS row swap23(r) (bits 2 and 3 exchanged, an involution) makes
// C value i of lane half g hold row 16 * (i / 8) + 8 * g + i % 8.
__device__ __forceinline__ int swap23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

}  // namespace fa

namespace fa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over `bytes` bytes from `base` (raw addressing, stride 0;
// the last word is the gfx9 data-format setting for plain 32-bit access).
// `base` must be wave-uniform.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Asynchronous 16-byte copy global -> LDS through a buffer resource: lane
// i's 16 bytes come from byte offset voff (per lane, 32-bit) of the resource
// and land at lds_wave_base + 16 * i (lds_wave_base the same for every lane
// of the wave); completion is tracked by the wave's vmcnt.  (The
// global_load_lds form of this copy is not used: while one is pending the
// compiler treats LDS reads as completing out of order and waits for each
// with lgkmcnt(0).)  The resource and the LDS base live in scalar registers,
// so an address costs one VGPR and no per-copy vector arithmetic.
__device__ __forceinline__ void buffer_load_lds16(buf_rsrc r, uint32_t voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, (int)voff, 0, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only:
// vmcnt in bits 3:0 and 15:14, expcnt (bits 6:4) and lgkmcnt (bits 11:8)
// left at their maximum.
constexpr int waitcnt_vm_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | 0x70 | 0xF00; }

// Buffer resource as four 32-bit words for inline assembly: base address
// (48 bits, stride 0), size in bytes, gfx9 data-format word.  `base` must be
// wave-uniform.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// The copy of buffer_load_lds16, issued from inline assembly so that the
// compiler neither sees the LDS write nor adds waits for it: the caller
// orders every read of the destination after the copy with its own
// wait_vmem* and block_barrier.  The instruction has no register result;
// its VGPR offset, resource and M0 (the LDS destination of lane 0) are read
// when it issues.  M0 is declared clobbered.
__device__ __forceinline__ void buffer_load_lds16_unseen(const i32x4& r, uint32_t voff,
                                                         const void* lds_wave_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :
               : "v"(voff), "s"(lds), "s"(r)
               : "memory", "m0");
}

// Wait until every global load (including global -> LDS copies) of this wave
// has completed.  Issued through the builtin, so the compiler's own waitcnt
// bookkeeping sees it and does not add a second, later wait.
__device__ __forceinline__ void wait_vmem() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_imm(0));
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector memory operations are still in
// flight.  The counter retires operations in issue order, so this waits for
// everything issued before the last N operations (used to wait for older
// tile copies while the newest ones stay in flight).
template <int N>
__device__ __forceinline__ void wait_vmem_except_last() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_imm(N));
  asm volatile("" ::: "memory");
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane 4e + q supplies the address of 4 consecutive 16-bit values;
// lane i of the group receives element i % 4 of the run supplied by lane
// 4e + i / 4, for e = 0..3.  With lane 4e + q pointing at M[r0 + e][c0 + 4q],
// lane i receives M[r0 .. r0+3][c0 + i]: a column of four rows.
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

typedef short i16x8 __attribute__((ext_vector_type(8)));

// Two transposed reads joined into one bf16x8 MFMA operand (lo = elements
// 0..3, hi = 4..7).  Joined as a 16-bit integer shuffle and bit-cast once:
// inserting bit-cast bf16 elements one at a time is miscompiled by this
// toolchain (the upper half of each read is dropped).
__device__ __forceinline__ bf16x8 join_tr(const i16x4& lo, const i16x4& hi) {
  const i16x8 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// XOR swizzle of the 16-byte chunks of an unpadded row-major LDS tile whose
// rows hold D bf16 values (D = 128: 16 chunks; D = 64: 8 chunks), so that the
// MFMA operand reads (16 consecutive rows at one chunk; 4 rows at 2-4 chunks
// for the transposed reads) hit distinct banks.  It is linear over the low 4
// bits of the row (period 16), so rows that differ by a multiple of 16 share
// it, and rows r and r + 4 (r % 8 < 4) differ by chunk bit 0.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 128) {
    return ((row & 1) ? 0x6 : 0) ^ ((row & 2) ? 0xC : 0) ^ ((row & 4) ? 0x1 : 0) ^
           ((row & 8) ? 0x8 : 0);
  } else {
    return ((row & 1) ? 0x2 : 0) ^ ((row & 2) ? 0x4 : 0) ^ ((row & 4) ? 0x1 : 0) ^
           ((row & 8) ? 0x2 : 0);
  }
}

}  // namespace fa

namespace fa {

// Make the compiler forget what it knows about a per-lane value.  Used on
// address constants at the top of each loop iteration: without it every LDS
// address (all loop invariant once the double-buffer stage is a template
// parameter) is hoisted out of the loop into its own register.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The same for a wave-uniform value in a scalar register: sums built on it
// at each use (an LDS destination per copy, say) cost one scalar add there
// instead of a scalar register each for the whole kernel.
__device__ __forceinline__ int opaque_s(int x) {
  asm volatile("" : "+s"(x));
  return x;
}
template <typename T>
__device__ __forceinline__ const T* opaque_s(const T* p) {
  uint32_t lo = (uint32_t)(uintptr_t)p, hi = (uint32_t)((uintptr_t)p >> 32);
  asm volatile("" : "+s"(lo), "+s"(hi));
  return reinterpret_cast<const T*>((uintptr_t)lo | ((uintptr_t)hi << 32));
}

// Per-lane constants for transposed reads (lds_read_tr) of a swizzled
// row-major [rows][D] tile, as MFMA operands with rows = contraction index:
// the read for row block R0 (a multiple of 16), column block C0 (a multiple
// of 32) and half `hi` gives lane (c, g) the column C0 + c of rows
// R0 + 8g + 4hi + 0..3.  Only the XOR with (C0 / 8) ^ hi depends on the
// compile-time indices, so each read costs two integer operations.
template <int D>
struct TrLane {
  int base;  // lane's row and 8-byte half, in elements
  int t;     // lane's chunk bits XOR its rows' swizzle
  TrLane() = default;
  __device__ __forceinline__ explicit TrLane(int lane) {
    const int g = lane >> 5, e = (lane >> 2) & 3, q = lane & 3, half = (lane >> 4) & 1;
    const int r = 8 * g + e;
    base = r * D + 4 * (q & 1);
    t = (2 * half + (q >> 1)) ^ chunk_swizzle<D>(r);
  }
  __device__ __forceinline__ int off(int R0, int C0, int hi) const {
    return (R0 + 4 * hi) * D + base + ((((C0 >> 3) ^ hi) ^ t) << 3);
  }
  __device__ __forceinline__ TrLane fresh() const {
    TrLane r = *this;
    r.base = opaque(base);
    r.t = opaque(t);
    return r;
  }
};

// Per-lane constants for the row reads of a swizzled [rows][D] tile as the
// A operand of a 32x32x16 MFMA whose lane c reads row swap23(c) (so its C
// rows come out in runs of eight): the read for row block R0 (a multiple of
// 32) and contraction slice kc gives the lane 8 values of row
// R0 + swap23(c), columns 16 kc + 8 g + 0..7.
template <int D>
struct RowLane {
  int base;
  int u;
  RowLane() = default;
  __device__ __forceinline__ explicit RowLane(int lane) {
    const int r = swap23(lane & 31);
    base = r * D;
    u = (lane >> 5) ^ chunk_swizzle<D>(r);
  }
  __device__ __forceinline__ int off(int R0, int kc) const {
    return R0 * D + base + (((2 * kc) ^ u) << 3);
  }
  __device__ __forceinline__ RowLane fresh() const {
    RowLane r = *this;
    r.base = opaque(base);
    r.u = opaque(u);
    return r;
  }
};

}  // namespace fa

namespace fa {

// Instruction-group scheduling hints for a software-pipelined loop of STEPS
// steps, each with R LDS reads feeding M MFMAs: the reads of the first AHEAD
// steps go first, then every step's MFMAs are followed by the reads of the
// step AHEAD later.  Applies to the scheduling region it is placed in.
template <int STEPS, int R, int M, int AHEAD>
__device__ __forceinline__ void sched_pipeline() {
  constexpr int kMfma = 0x008, kDsRead = 0x100;
#pragma unroll
  for (int s = 0; s < AHEAD; ++s) __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    __builtin_amdgcn_sched_group_barrier(kMfma, M, 0);
    if (s + AHEAD < STEPS) __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
  }
}

}  // namespace fa

namespace fa {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16.  Lane l = 16 kg + c, c < 16, kg < 4:
//   A (16 x 32): lane holds A[c][8 kg .. 8 kg + 7]
//   B (32 x 16): lane holds B[8 kg .. 8 kg + 7][c]
//   C (16 x 16): lane holds C[4 kg + i][c], i < 4
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// XOR swizzle of the 16-byte chunks of the backward pass's Q and dO tiles
// ([query][D] bf16), linear over row bits 0, 1 and 3.  gfx950's LDS has 64
// banks of 4 bytes; measured with SQ_LDS_BANK_CONFLICT on single reads, it
// serves a ds_read_b128 in four cycles of 16 lanes (lanes with the same bit
// 5 and the same parity of bits 2..4) and a ds_read_b64_tr_b16 in two cycles
// of 32 consecutive lanes.  With that grouping this swizzle leaves both reads
// of these tiles free of conflicts: 16-byte row reads where lane (c, kg) of
// a 16x16x32 operand takes row 8 (c / 4) + c % 4 (+ 4 t) and chunk 4 k + kg,
// and transposed reads where lane 16 G + 4 e + q takes row 8 G + e.
template <int D>
__device__ __forceinline__ int qtile_swizzle(int row) {
  constexpr int m0 = D == 128 ? 6 : 4, m1 = D == 128 ? 4 : 2, m3 = D == 128 ? 9 : 5;
  return ((row & 1) ? m0 : 0) ^ ((row & 2) ? m1 : 0) ^ ((row & 8) ? m3 : 0);
}

}  // namespace fa

namespace fa {

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of
//   (x0, x1, x2, x3) -> (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0))
// with the key advanced by the Weyl increments after every round.  The key
// is wave-uniform, so its schedule stays in scalar registers; each 32 x 32-bit
// product is one v_mad_u64_u32.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                               uint32_t k0, uint32_t k1) {
  // recompute the round keys at each call instead of keeping all twenty
  // hoisted in scalar registers
  asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
    x0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
    x1 = (uint32_t)p1;
    x2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
    x3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  u32x4 r = {x0, x1, x2, x3};
  return r;
}

// Byte b (0..3) of word w, compared with the dropout threshold: kept iff >= t.
__device__ __forceinline__ bool drop_keep(uint32_t w, int b, uint32_t t) {
  return ((w >> (8 * b)) & 0xFFu) >= t;
}

}  // namespace fa
