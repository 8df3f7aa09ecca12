// Kernel argument blocks and launchers, shared by the C ABI layer (api.cpp)
// and the kernel translation units.  Plain data only: the ABI layer has
// already validated every field when these are filled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

namespace fa {

// Dropout on the attention probabilities (inactive unless a kernel is
// instantiated for it).  Element (query i, key j) of head bh is kept iff byte
// j mod 16 of Philox4x32-10(counter (j / 16, i, bh, offset), key (k0, k1)) is
// >= t; kept values are multiplied by scale = 256 / (256 - t).
struct DropArgs {
  uint32_t t = 0;
  float scale = 1.f;
  uint32_t k0 = 0, k1 = 0;  // seed, low and high words
  uint32_t offset = 0;
};

struct FwdArgs {
  const uint16_t* q;  // bf16 [B, H, N, d]
  const uint16_t* k;  // bf16 [B, H, Nk, d]
  const uint16_t* v;
  uint16_t* o;        // bf16 [B, H, N, d]
  float* lse;         // fp32 [B, H, N], natural log
  int N;              // queries per head
  int Nk;             // keys per head (= N except in the split-KV forward)
  int BH;             // B * H
  float scale_log2;   // softmax_scale * log2(e), > 0
  // Split-KV forward only (splits > 1 or partials requested): each query
  // block's key tiles are cut into `splits` contiguous ranges, one
  // workgroup per range, whose unnormalised partial results go to
  // Only this path allows Nk != N (without the causal mask).
  //   opart  fp32 [splits, B*H, N, d]  (sum of 2^(s - m) V over the range)
  //   mpart  fp32 [splits, B*H, N]     running max m, log2 units, scaled
  //   lpart  fp32 [splits, B*H, N]     sum of 2^(s - m) over the range
  // and a merge kernel writes O and LSE.
  int splits = 1;
  float* opart = nullptr;
  float* mpart = nullptr;
  float* lpart = nullptr;
  DropArgs drop;
};

// FP8 forward: Q, K, V are OCP E4M3 codes, each tensor with one dequantisation
// factor (real value = descale * e4m3(code)).
struct Fp8FwdArgs {
  const uint8_t* q;   // E4M3 [B, H, N, d]
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;        // bf16 [B, H, N, d]
  float* lse;         // fp32 [B, H, N], natural log
  int N;
  int BH;
  float scale_log2;   // softmax_scale * descale_q * descale_k * log2(e), > 0
  float descale_v;    // > 0
};

// FP8 quantisation of a bf16 tensor of `rows` rows of d values, optionally
// rotated by diag(signs) H_d / sqrt(d) first.
struct QuantArgs {
  const uint16_t* x;   // bf16 [rows, d]
  uint8_t* codes;      // E4M3 [rows, d]
  float* descale;      // out: amax / 448 (1 float)
  float* part;         // workspace: one partial amax per workgroup of the amax pass
  const float* signs;  // [d] of +-1, or nullptr (no rotation)
  int64_t rows;
  int parts;           // set by the launcher: workgroups of the amax pass
};

// Largest number of partial maxima of the quantisation (workspace floats).
constexpr int kQuantParts = 512;

// Query rows per block of the backward key-block pass; the row vectors in
// the backward workspace are padded to a multiple of it.
constexpr int kBwdQueryBlock = 64;

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;       // workspace: fp32 [B*H, Npad], -rowsum(dO o O), 0 on padding
  float* lse2;        // workspace: fp32 [B*H, Npad], LSE * log2(e), +inf on padding
  int N;
  int Npad;           // N rounded up to kBwdQueryBlock
  int BH;
  float scale;        // softmax_scale, > 0
  float scale_log2;   // softmax_scale * log2(e)
  DropArgs drop;
};

// Size of the library-owned device scratch of the allocation-free backward
// entry point (one copy per device; it holds the backward pass's two fp32
// row vectors, so at most 1 M padded rows: B * H * Npad <= 2^20).
constexpr size_t kNoallocScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;

// Device address of this device's copy of that scratch (looked up on the
// first call on each device, with the device current, then cached).
hipError_t noalloc_scratch(void** out);

// Compute units of the current device (cached per device; 0 if unknown).
inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Grid of a persistent kernel over `items` work items with one workgroup per
// CU: at most one per CU and never more than the items, a multiple of 8 when
// at least 8 (so that each workgroup stays on the XCD of its items).
inline int64_t persistent_grid(int64_t items) {
  const int cus = cu_count();
  int64_t grid = cus > 0 ? std::min<int64_t>(items, cus) : items;
  if (grid >= 8) grid &= ~int64_t(7);
  return grid;
}

// Enqueue the forward kernel for head dim d (64 or 128).
hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, hipStream_t stream);

// Enqueue the forward kernel with dropout (a.drop) for head dim d.
hipError_t launch_fwd_dropout(const FwdArgs& a, int d, bool causal, hipStream_t stream);

// Enqueue the split-KV forward: the partial kernel over a.splits key ranges
// per query block, then the merge kernel that writes O and LSE.
hipError_t launch_fwd_splitkv(const FwdArgs& a, int d, bool causal, hipStream_t stream);

// Enqueue the FP8 forward kernel for head dim d (64 or 128).
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, int d, bool causal, hipStream_t stream);

// Enqueue the FP8 quantisation (two launches) for head dim d (64 or 128).
hipError_t launch_quant_fp8(const QuantArgs& a, int d, hipStream_t stream);

// The three backward stages, each one kernel launch, for head dim d (64 or
// 128): the row pass, the pass over key blocks (dK, dV) and the pass over
// query blocks (dQ).
hipError_t launch_bwd_pre(const BwdArgs& a, int d, hipStream_t stream);
hipError_t launch_bwd_kv(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_q(const BwdArgs& a, int d, bool causal, hipStream_t stream);
// The key-block and query-block passes with dropout (a.drop); the row pass is
// the same with or without it.
hipError_t launch_bwd_kv_dropout(const BwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_q_dropout(const BwdArgs& a, int d, bool causal, hipStream_t stream);

}  // namespace fa
