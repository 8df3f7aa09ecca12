// C ABI of the fused attention library: argument validation and dispatch.
// Every check runs on the host before any HIP call, so a rejected call has
// no side effect.  The entry points are declared (with their contracts) in
// include/flash_attn.h.
#include "flash_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fa_launch.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;  // keeps every byte count in int64
constexpr size_t kWsAlign = 256;
constexpr int64_t kMaxSplits = 128;              // split-KV ranges per query block

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shape check shared by both passes.  Sets *empty for B*H*N == 0.
int check_shape(int64_t B, int64_t H, int64_t N, int64_t d, bool* empty) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  *empty = (B == 0 || H == 0 || N == 0);
  if (*empty) return FA_OK;
  // sizes must fit the kernels' index arithmetic: N and B*H in int32, the
  // element count well inside int64
  if (N > INT32_MAX / 2 || B > INT32_MAX || H > INT32_MAX) return FA_ERR_BAD_SHAPE;
  const int64_t bh = B * H;
  if (bh > INT32_MAX) return FA_ERR_BAD_SHAPE;
  if (N > kMaxElems / d || bh > kMaxElems / (N * d)) return FA_ERR_BAD_SHAPE;
  // grid sizes: query blocks of 64 rows (smallest tile) times heads must fit
  // a one-dimensional launch
  if (((N + 63) / 64) * bh > INT32_MAX) return FA_ERR_BAD_SHAPE;
  return FA_OK;
}

int check_scale(float s) {
  if (!std::isfinite(s) || !(s > 0.f)) return FA_ERR_BAD_SCALE;
  return FA_OK;
}

// Dropout threshold t = floor(256 p + 1/2), 0 <= t <= 255, and the rescale
// 256 / (256 - t); FA_ERR_BAD_DROPOUT for NaN, negative or too large p.
int prepare_dropout(float p, uint64_t seed, uint32_t offset, fa::DropArgs* d) {
  if (!(p >= 0.f)) return FA_ERR_BAD_DROPOUT;  // also NaN
  const double t = std::floor(256.0 * double(p) + 0.5);
  if (!(t <= 255.0)) return FA_ERR_BAD_DROPOUT;
  d->t = uint32_t(t);
  d->scale = float(256.0 / (256.0 - t));
  d->k0 = uint32_t(seed);
  d->k1 = uint32_t(seed >> 32);
  d->offset = offset;
  return FA_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// True if any output range overlaps an input range or another output range.
bool any_alias(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

int64_t padded_rows(int64_t N) {
  return (N + fa::kBwdQueryBlock - 1) / fa::kBwdQueryBlock * fa::kBwdQueryBlock;
}

// Workspace layout: the fp32 row vectors D and LSE*log2(e), each
// [B*H, Npad], each section 256-byte aligned.
size_t ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  (void)d;
  const size_t prow = size_t(B) * size_t(H) * size_t(padded_rows(N));
  return 2 * round_up(prow * 4, kWsAlign);
}

// Split-KV workspace: fp32 partial O [S, B*H, N, d], then the fp32 running
// max and row sum [S, B*H, N] each, every section 256-byte aligned.
size_t splitkv_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t S) {
  const size_t rows = size_t(S) * size_t(B) * size_t(H) * size_t(N);
  return round_up(rows * size_t(d) * 4, kWsAlign) + 2 * round_up(rows * 4, kWsAlign);
}

// Pointers of the backward pass; `used` selects the ones a stage reads or
// writes (the others may be null and are ignored).
struct BwdPtrs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* ws;
};

enum : unsigned {
  kQ = 1u << 0, kK = 1u << 1, kV = 1u << 2, kO = 1u << 3, kLse = 1u << 4, kDout = 1u << 5,
  kDq = 1u << 6, kDk = 1u << 7, kDv = 1u << 8, kWs = 1u << 9,
  kAllBwd = (1u << 10) - 1
};

// Validate the arguments of a backward stage and fill its kernel arguments.
// Returns FA_OK with a->BH == 0 for an empty problem.
int prepare_bwd(const BwdPtrs& p, unsigned used, size_t workspace_bytes, int64_t B, int64_t H,
                int64_t N, int64_t d, float scale, fa::BwdArgs* a) {
  bool empty = false;
  int st = check_shape(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  a->BH = 0;
  if (empty) return FA_OK;
  const void* ptrs[10] = {p.q, p.k, p.v, p.o, p.lse, p.dout, p.dq, p.dk, p.dv, p.ws};
  for (int i = 0; i < 10; ++i)
    if ((used >> i & 1u) && !ptrs[i]) return FA_ERR_NULL_POINTER;
  for (int i = 0; i < 10; ++i)
    if ((used >> i & 1u) && !aligned(ptrs[i], i == 4 ? 4 : 16)) return FA_ERR_MISALIGNED;
  const size_t need = ws_bytes(B, H, N, d);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;
  const size_t tb = size_t(B * H * N * d) * 2, lb = size_t(B * H * N) * 4;
  Range ins[6], outs[4];
  int n_in = 0, n_out = 0;
  const size_t sizes[10] = {tb, tb, tb, tb, lb, tb, tb, tb, tb, need};
  for (int i = 0; i < 10; ++i) {
    if (!(used >> i & 1u)) continue;
    if (i < 6) ins[n_in++] = range_of(ptrs[i], sizes[i]);
    else outs[n_out++] = range_of(ptrs[i], sizes[i]);
  }
  if (any_alias(outs, n_out, ins, n_in)) return FA_ERR_ALIASING;

  const size_t prow = size_t(B * H) * size_t(padded_rows(N));
  char* ws = static_cast<char*>(p.ws);
  a->q = static_cast<const uint16_t*>(p.q);
  a->k = static_cast<const uint16_t*>(p.k);
  a->v = static_cast<const uint16_t*>(p.v);
  a->o = static_cast<const uint16_t*>(p.o);
  a->lse = p.lse;
  a->dout = static_cast<const uint16_t*>(p.dout);
  a->dq = static_cast<uint16_t*>(p.dq);
  a->dk = static_cast<uint16_t*>(p.dk);
  a->dv = static_cast<uint16_t*>(p.dv);
  a->delta = reinterpret_cast<float*>(ws);
  a->lse2 = reinterpret_cast<float*>(ws + round_up(prow * 4, kWsAlign));
  a->N = int(N);
  a->Npad = int(padded_rows(N));
  a->BH = int(B * H);
  a->scale = scale;
  a->scale_log2 = scale * 1.4426950408889634f;
  return FA_OK;
}

// Shared by flash_attn_fwd and flash_attn_fwd_dropout: validation and the
// argument block.  Returns FA_OK with a->BH == 0 for an empty problem.
int prepare_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t H, int64_t N, int64_t d, float softmax_scale, const fa::DropArgs* drop,
                fa::FwdArgs* a) {
  bool empty = false;
  int st = check_shape(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  a->BH = 0;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_MISALIGNED;
  const size_t tb = size_t(B * H * N * d) * 2, lb = size_t(B * H * N) * 4;
  const Range ins[3] = {range_of(q, tb), range_of(k, tb), range_of(v, tb)};
  const Range outs[2] = {range_of(o, tb), range_of(lse, lb)};
  if (any_alias(outs, 2, ins, 3)) return FA_ERR_ALIASING;
  a->q = static_cast<const uint16_t*>(q);
  a->k = static_cast<const uint16_t*>(k);
  a->v = static_cast<const uint16_t*>(v);
  a->o = static_cast<uint16_t*>(o);
  a->lse = lse;
  a->N = int(N);
  a->Nk = int(N);
  a->BH = int(B * H);
  a->scale_log2 = softmax_scale * 1.4426950408889634f;
  if (drop) a->drop = *drop;
  return FA_OK;
}

}  // namespace

extern "C" {


int flash_attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                           float softmax_scale, float dropout_p, uint64_t seed, uint32_t offset,
                           void* stream) {
  fa::DropArgs drop;
  bool empty = false;
  int st = check_shape(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  if ((st = prepare_dropout(dropout_p, seed, offset, &drop)) != FA_OK) return st;
  fa::FwdArgs a;
  if ((st = prepare_fwd(q, k, v, o, lse, B, H, N, d, softmax_scale, &drop, &a)) != FA_OK ||
      a.BH == 0)
    return st;
  const hipError_t e =
      fa::launch_fwd_dropout(a, int(d), causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                   int64_t H, int64_t N, int64_t d, int causal, float softmax_scale, void* stream) {
  fa::FwdArgs a;
  const int st = prepare_fwd(q, k, v, o, lse, B, H, N, d, softmax_scale, nullptr, &a);
  if (st != FA_OK || a.BH == 0) return st;
  const hipError_t e = fa::launch_fwd(a, int(d), causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t flash_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  bool empty = false;
  if (check_shape(B, H, N, d, &empty) != FA_OK || empty) return 0;
  return ws_bytes(B, H, N, d);
}

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                   float softmax_scale, void* stream) {
  const BwdPtrs p{q, k, v, o, lse, dout, dq, dk, dv, workspace};
  fa::BwdArgs a;
  const int st = prepare_bwd(p, kAllBwd, workspace_bytes, B, H, N, d, softmax_scale, &a);
  if (st != FA_OK || a.BH == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (fa::launch_bwd_pre(a, int(d), s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_kv(a, int(d), causal != 0, s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_q(a, int(d), causal != 0, s) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                           float softmax_scale, void* stream) {
  static_assert(FA_BWD_NOALLOC_SCRATCH_BYTES == fa::kNoallocScratchBytes, "scratch size");
  bool empty = false;
  int st = check_shape(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if (!empty && ws_bytes(B, H, N, d) > fa::kNoallocScratchBytes) return FA_ERR_SCRATCH_TOO_SMALL;
  // validate every caller pointer (the workspace is the library's own, so
  // it is left out of the checks), then point the row vectors at it
  const BwdPtrs p{q, k, v, o, lse, dout, dq, dk, dv, nullptr};
  fa::BwdArgs a;
  const size_t need = empty ? 0 : ws_bytes(B, H, N, d);
  st = prepare_bwd(p, kAllBwd & ~unsigned(kWs), need, B, H, N, d, softmax_scale, &a);
  if (st != FA_OK || a.BH == 0) return st;
  void* scratch = nullptr;
  if (fa::noalloc_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
  const size_t prow = size_t(B * H) * size_t(padded_rows(N));
  char* ws = static_cast<char*>(scratch);
  a.delta = reinterpret_cast<float*>(ws);
  a.lse2 = reinterpret_cast<float*>(ws + round_up(prow * 4, kWsAlign));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (fa::launch_bwd_pre(a, int(d), s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_kv(a, int(d), causal != 0, s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_q(a, int(d), causal != 0, s) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int flash_attn_bwd_preprocess(const void* o, const float* lse, const void* dout, void* workspace,
                              size_t workspace_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                              void* stream) {
  const BwdPtrs p{nullptr, nullptr, nullptr, o, lse, dout, nullptr, nullptr, nullptr, workspace};
  fa::BwdArgs a;
  const int st = prepare_bwd(p, kO | kLse | kDout | kWs, workspace_bytes, B, H, N, d, 1.f, &a);
  if (st != FA_OK || a.BH == 0) return st;
  return fa::launch_bwd_pre(a, int(d), static_cast<hipStream_t>(stream)) == hipSuccess
             ? FA_OK : FA_ERR_HIP;
}

int flash_attn_bwd_kv_blocks(const void* q, const void* k, const void* v, const void* dout,
                             void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                             float softmax_scale, void* stream) {
  const BwdPtrs p{q, k, v, nullptr, nullptr, dout, nullptr, dk, dv, workspace};
  fa::BwdArgs a;
  const int st = prepare_bwd(p, kQ | kK | kV | kDout | kDk | kDv | kWs, workspace_bytes, B, H, N,
                             d, softmax_scale, &a);
  if (st != FA_OK || a.BH == 0) return st;
  return fa::launch_bwd_kv(a, int(d), causal != 0, static_cast<hipStream_t>(stream)) ==
                 hipSuccess ? FA_OK : FA_ERR_HIP;
}

int flash_attn_bwd_q_blocks(const void* q, const void* k, const void* v, const void* dout,
                            void* dq, void* workspace, size_t workspace_bytes, int64_t B,
                            int64_t H, int64_t N, int64_t d, int causal, float softmax_scale,
                            void* stream) {
  const BwdPtrs p{q, k, v, nullptr, nullptr, dout, dq, nullptr, nullptr, workspace};
  fa::BwdArgs a;
  const int st = prepare_bwd(p, kQ | kK | kV | kDout | kDq | kWs, workspace_bytes, B, H, N, d,
                             softmax_scale, &a);
  if (st != FA_OK || a.BH == 0) return st;
  return fa::launch_bwd_q(a, int(d), causal != 0, static_cast<hipStream_t>(stream)) ==
                 hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t flash_attn_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d,
                                              int64_t num_splits) {
  bool empty = false;
  if (check_shape(B, H, N, d, &empty) != FA_OK || empty) return 0;
  if (num_splits < 1 || num_splits > kMaxSplits) return 0;
  return splitkv_ws_bytes(B, H, N, d, num_splits);
}

int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                           int64_t N_q, int64_t N_kv, int64_t d, int causal, float softmax_scale,
                           int64_t num_splits, void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N_q, d, &empty);
  if (st != FA_OK) return st;
  bool no_keys = false;
  if ((st = check_shape(B, H, N_kv, d, &no_keys)) != FA_OK) return st;
  // the causal mask is defined for equal lengths only; and a query needs at
  // least one key
  if ((causal && N_q != N_kv) || (!empty && N_kv == 0)) return FA_ERR_BAD_SHAPE;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_BAD_SPLITS;
  if (empty) return FA_OK;
  // the partial kernel's grid: 256-row query blocks x heads x ranges
  if (((N_q + 255) / 256) * (B * H) * num_splits > INT32_MAX) return FA_ERR_BAD_SHAPE;
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 16))
    return FA_ERR_MISALIGNED;
  const size_t need = splitkv_ws_bytes(B, H, N_q, d, num_splits);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;
  const size_t qb = size_t(B * H * N_q * d) * 2, kb = size_t(B * H * N_kv * d) * 2,
               lb = size_t(B * H * N_q) * 4;
  const Range ins[3] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
  const Range outs[3] = {range_of(o, qb), range_of(lse, lb), range_of(workspace, need)};
  if (any_alias(outs, 3, ins, 3)) return FA_ERR_ALIASING;

  const size_t rows = size_t(num_splits) * size_t(B * H) * size_t(N_q);
  char* ws = static_cast<char*>(workspace);
  fa::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.N = int(N_q);
  a.Nk = int(N_kv);
  a.BH = int(B * H);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.splits = int(num_splits);
  a.opart = reinterpret_cast<float*>(ws);
  a.mpart = reinterpret_cast<float*>(ws + round_up(rows * size_t(d) * 4, kWsAlign));
  a.lpart = reinterpret_cast<float*>(ws + round_up(rows * size_t(d) * 4, kWsAlign) +
                                     round_up(rows * 4, kWsAlign));
  const hipError_t e =
      fa::launch_fwd_splitkv(a, int(d), causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int flash_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                       float softmax_scale, float descale_q, float descale_k, float descale_v,
                       void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  for (const float ds : {descale_q, descale_k, descale_v})
    if (!std::isfinite(ds) || !(ds > 0.f)) return FA_ERR_BAD_DESCALE;
  // the scale the kernel applies to the scores must itself be usable
  const float sl2 = float(double(softmax_scale) * double(descale_q) * double(descale_k) *
                          1.4426950408889634);
  if (!std::isfinite(sl2) || !(sl2 > 0.f)) return FA_ERR_BAD_DESCALE;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_MISALIGNED;
  const size_t nb = size_t(B * H * N * d), lb = size_t(B * H * N) * 4;
  const Range ins[3] = {range_of(q, nb), range_of(k, nb), range_of(v, nb)};
  const Range outs[2] = {range_of(o, 2 * nb), range_of(lse, lb)};
  if (any_alias(outs, 2, ins, 3)) return FA_ERR_ALIASING;

  fa::Fp8FwdArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.N = int(N);
  a.BH = int(B * H);
  a.scale_log2 = sl2;
  a.descale_v = descale_v;
  const hipError_t e = fa::launch_fwd_fp8(a, int(d), causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int flash_attn_quantize_fp8(const void* x, void* codes, float* descale, void* workspace,
                            size_t workspace_bytes, int64_t rows, int64_t d, const float* signs,
                            void* stream) {
  if (rows < 0) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
  if (rows > kMaxElems / d) return FA_ERR_BAD_SHAPE;
  if (rows == 0) return FA_OK;
  // grid: rows / (256 / (d / 8)) workgroups must fit a one-dimensional launch
  if ((rows + 15) / 16 > INT32_MAX) return FA_ERR_BAD_SHAPE;
  if (!x || !codes || !descale || !workspace) return FA_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(descale, 4) || !aligned(workspace, 16) ||
      (signs && !aligned(signs, 16)))
    return FA_ERR_MISALIGNED;
  if (workspace_bytes < FA_QUANT_WORKSPACE_BYTES) return FA_ERR_WORKSPACE_TOO_SMALL;
  const size_t n = size_t(rows) * size_t(d);
  Range ins[2] = {range_of(x, 2 * n), range_of(signs, signs ? size_t(d) * 4 : 0)};
  const Range outs[3] = {range_of(codes, n), range_of(descale, 4),
                          range_of(workspace, FA_QUANT_WORKSPACE_BYTES)};
  if (any_alias(outs, 3, ins, signs ? 2 : 1)) return FA_ERR_ALIASING;
  fa::QuantArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.codes = static_cast<uint8_t*>(codes);
  a.descale = descale;
  a.part = static_cast<float*>(workspace);
  static_assert(FA_QUANT_WORKSPACE_BYTES >= 4 * fa::kQuantParts, "quantise workspace");
  a.signs = signs;
  a.rows = rows;
  return fa::launch_quant_fp8(a, int(d), static_cast<hipStream_t>(stream)) == hipSuccess
             ? FA_OK : FA_ERR_HIP;
}

int flash_attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                           int64_t N, int64_t d, int causal, float softmax_scale, float dropout_p,
                           uint64_t seed, uint32_t offset, void* stream) {
  fa::DropArgs drop;
  bool empty = false;
  int st = check_shape(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  if ((st = prepare_dropout(dropout_p, seed, offset, &drop)) != FA_OK) return st;
  const BwdPtrs p{q, k, v, o, lse, dout, dq, dk, dv, workspace};
  fa::BwdArgs a;
  st = prepare_bwd(p, kAllBwd, workspace_bytes, B, H, N, d, softmax_scale, &a);
  if (st != FA_OK || a.BH == 0) return st;
  a.drop = drop;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (fa::launch_bwd_pre(a, int(d), s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_kv_dropout(a, int(d), causal != 0, s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_q_dropout(a, int(d), causal != 0, s) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

const char* flash_attn_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "bad shape: B, H, N must be >= 0 and the sizes must fit";
    case FA_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dim: d must be 64 or 128";
    case FA_ERR_MISALIGNED: return "misaligned pointer: tensors need 16 bytes, LSE 4 bytes";
    case FA_ERR_BAD_SCALE: return "softmax_scale must be finite and > 0";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than flash_attn_bwd_workspace_bytes()";
    case FA_ERR_ALIASING: return "an output buffer overlaps an input or another output";
    case FA_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case FA_ERR_BAD_SPLITS: return "num_splits must be between 1 and 128";
    case FA_ERR_BAD_DESCALE: return "FP8 descale factors must be finite and > 0";
    case FA_ERR_BAD_DROPOUT: return "dropout_p must be >= 0 and round (in steps of 1/256) below 1";
    case FA_ERR_SCRATCH_TOO_SMALL:
      return "problem too large for the static scratch of flash_attn_bwd_noalloc "
             "(B * H * ceil(N / 64) * 64 must be <= 2^20)";
    default: return "unknown status";
  }
}

}  // extern "C"
