// dit_attn_api.cpp -- the extern "C" boundary: argument checks, workspace
// layout and kernel dispatch.  Every check runs before the first HIP call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/dit_attn.h"
#include "launch.h"

// Scratch of dit_attn_fwd_noalloc: the partial results of the split tail
// blocks (see dit_attn_fwd_ws), in a device array the library owns, so that
// the entry point allocates nothing.  Host code must never take this name's
// address for device use: the device address of each GPU's copy comes from
// hipGetSymbolAddress (scratch_device_ptr below).
static constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

constexpr uint32_t kKnownFlags = DIT_ATTN_FLAG_OUT_F32;
constexpr int64_t kMaxSliceBytes = (int64_t)1 << 31;   // one (b, h) slice, 32-bit buffer offsets
// Row strides up to 2^22 elements keep the 32-bit byte offsets of the key
// tiles staged past the last row (up to 127 rows beyond N) from wrapping.
constexpr int64_t kMaxRowStride = (int64_t)1 << 22;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Bytes spanned by one (b, h) slice of a [.., N, 128] tensor with row stride sn.
int64_t slice_bytes(int64_t N, int64_t sn, int64_t elem) { return ((N - 1) * sn + 128) * elem; }

int check_tensor(const char* name, const void* p, const int64_t* st, int64_t N, int64_t elem_bytes,
                 bool is_output) {
  if (p == nullptr) return fail(DIT_ATTN_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(DIT_ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(DIT_ATTN_ERR_INVALID_ARG, "%s stride[%d] = %lld is negative", name, i, (long long)st[i]);
    if (st[i] % 8 != 0)
      return fail(DIT_ATTN_ERR_INVALID_ARG, "%s stride[%d] = %lld is not a multiple of 8 elements", name, i,
                  (long long)st[i]);
  }
  if (st[2] < 128)
    return fail(DIT_ATTN_ERR_INVALID_ARG, "%s row stride %lld is smaller than head_dim 128 (rows overlap)", name,
                (long long)st[2]);
  if (st[2] > kMaxRowStride)
    return fail(DIT_ATTN_ERR_UNSUPPORTED, "%s row stride %lld is above %lld elements", name, (long long)st[2],
                (long long)kMaxRowStride);
  if (slice_bytes(N, st[2], elem_bytes) >= kMaxSliceBytes)
    return fail(DIT_ATTN_ERR_UNSUPPORTED, "%s: one (batch, head) slice spans more than 2 GiB", name);
  (void)is_output;
  return DIT_ATTN_OK;
}

int check_common(const dit_attn_shape* sh, const void* q, const void* k, const void* v, const void* o,
                 const float* lse) {
  if (sh == nullptr) return fail(DIT_ATTN_ERR_INVALID_ARG, "shape is NULL");
  if (sh->batch < 1 || sh->heads < 1 || sh->seqlen < 1)
    return fail(DIT_ATTN_ERR_INVALID_ARG, "batch=%d heads=%d seqlen=%d must all be >= 1", sh->batch, sh->heads,
                sh->seqlen);
  if (sh->head_dim != 128) return fail(DIT_ATTN_ERR_UNSUPPORTED, "head_dim=%d: only 128 is built", sh->head_dim);
  if (!(std::isfinite(sh->softmax_scale) && sh->softmax_scale > 0.f))
    return fail(DIT_ATTN_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (sh->flags & ~kKnownFlags) return fail(DIT_ATTN_ERR_INVALID_ARG, "unknown flag bits 0x%x", sh->flags);
  if ((int64_t)sh->batch * sh->heads * sh->seqlen > ((int64_t)1 << 40))
    return fail(DIT_ATTN_ERR_UNSUPPORTED, "problem too large");
  const int64_t N = sh->seqlen;
  int rc;
  if ((rc = check_tensor("q", q, sh->q_stride, N, 2, false))) return rc;
  if ((rc = check_tensor("k", k, sh->k_stride, N, 2, false))) return rc;
  if ((rc = check_tensor("v", v, sh->v_stride, N, 2, false))) return rc;
  const int64_t oel = (sh->flags & DIT_ATTN_FLAG_OUT_F32) ? 4 : 2;
  if ((rc = check_tensor("o", o, sh->o_stride, N, oel, true))) return rc;
  if (lse != nullptr && !aligned(lse, 4)) return fail(DIT_ATTN_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  return DIT_ATTN_OK;
}

void fill_common(const dit_attn_shape* sh, const void* q, const void* k, const void* v, void* o, float* lse,
                 dit::AttnArgs& a) {
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = sh->q_stride[i];
    a.ks[i] = sh->k_stride[i];
    a.vs[i] = sh->v_stride[i];
    a.os[i] = sh->o_stride[i];
  }
  a.q_bytes = (uint32_t)slice_bytes(sh->seqlen, sh->q_stride[2], 2);
  a.k_bytes = (uint32_t)slice_bytes(sh->seqlen, sh->k_stride[2], 2);
  a.v_bytes = (uint32_t)slice_bytes(sh->seqlen, sh->v_stride[2], 2);
  a.B = sh->batch;
  a.H = sh->heads;
  a.N = sh->seqlen;
  a.nb = (sh->seqlen + 127) / 128;
  a.c = (float)((double)sh->softmax_scale * 1.4426950408889634);
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DIT_ATTN_OK;
  return fail(DIT_ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device, read once per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64 && cus > 0) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Tail split of a grid of `rows`-row work-groups (one runs per CU at a
// time): B*H*ceil(N/rows) work-groups leave a last partial round of r
// blocks.  Each of those is split into `split` key ranges (as many as fill
// the CUs, at most one per key tile), so the last round costs 1/split of a
// full one.  With `small`, a grid smaller than one round is all partial
// round and is split the same way (the bf16 path; the fp8 path keeps such
// grids whole, so their rows follow the one-pass recipe).  No split when the
// grid is whole rounds, or when more than half the CUs are busy in the last
// round (split < 2).
struct TailPlan {
  int nfull = 0, ntail = 0, split = 1;
  size_t bytes = 0;
};

TailPlan tail_plan(const dit_attn_shape* sh, int cus, int rows, int tile_keys, bool small) {
  TailPlan t;
  const int64_t units = (int64_t)sh->batch * sh->heads * ((sh->seqlen + rows - 1) / rows);
  t.nfull = (int)units;
  if (cus <= 0 || units > 0x7fffffff) return t;
  const int64_t r = units % cus;
  const int64_t tiles = (sh->seqlen + tile_keys - 1) / tile_keys;
  if (r == 0 || (!small && units < cus)) return t;
  const int64_t split = std::min<int64_t>(cus / r, tiles);
  if (split < 2) return t;
  t.nfull = (int)(units - r);
  t.ntail = (int)r;
  t.split = (int)split;
  t.bytes = (size_t)(r * split) * rows * dit::kPartRow * sizeof(float);
  return t;
}

// Device address of `scratch` on the current device.  Each GPU holds its own
// copy of the array; its address is looked up once per device, with that
// device current, and kept.
int scratch_device_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DIT_ATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(DIT_ATTN_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(DIT_ATTN_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return DIT_ATTN_OK;
}

struct Fp8Layout {
  size_t q8, k8, v8t, sq, sk, sv, part, total;
  TailPlan plan;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// `sh` (may be null: no tail split) sizes the partial-result region of the
// attention grid's tail split (128-key tiles) on the current device.
Fp8Layout fp8_layout(int64_t BH, int64_t N, const dit_attn_shape* sh) {
  const int64_t nb = (N + 127) / 128, np = nb * 128;
  Fp8Layout L;
  if (sh != nullptr) L.plan = tail_plan(sh, device_cus(), 256, 128, false);   // 256-row blocks, 128-key tiles
  const size_t codes = (size_t)(BH * np * 128), scales = (size_t)(BH * nb) * 4;
  L.q8 = 0;
  L.k8 = round256(L.q8 + codes);
  L.v8t = round256(L.k8 + codes);
  L.sq = round256(L.v8t + codes);
  L.sk = round256(L.sq + scales);
  L.sv = round256(L.sk + scales);
  L.part = round256(L.sv + scales);
  L.total = round256(L.part + L.plan.bytes);
  return L;
}

int prepare_fp8(const dit_attn_shape* sh, const void* q, const void* k, const void* v, void* o, float* lse,
                void* ws, size_t ws_bytes, bool need_out, dit::Fp8Args& f) {
  int rc;
  if (need_out) {
    if ((rc = check_common(sh, q, k, v, o, lse))) return rc;
  } else {
    // quantise-only: O is not touched, validate the inputs alone
    if (sh == nullptr) return fail(DIT_ATTN_ERR_INVALID_ARG, "shape is NULL");
    dit_attn_shape tmp = *sh;
    for (int i = 0; i < 3; ++i) tmp.o_stride[i] = tmp.q_stride[i];
    tmp.flags = 0;
    if ((rc = check_common(&tmp, q, k, v, q, nullptr))) return rc;
  }
  const int64_t BH = (int64_t)sh->batch * sh->heads, N = sh->seqlen;
  const Fp8Layout L = fp8_layout(BH, N, sh);
  if (ws == nullptr) return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if (!aligned(ws, 256)) return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(DIT_ATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, L.total);
  if ((int64_t)((N + 127) / 128) * 128 * 128 >= kMaxSliceBytes)
    return fail(DIT_ATTN_ERR_UNSUPPORTED, "seqlen too large for the fp8 workspace slices");
  std::memset(&f, 0, sizeof(f));
  f.q = q;
  f.k = k;
  f.v = v;
  f.o = o;
  f.lse = lse;
  for (int i = 0; i < 3; ++i) {
    f.qs[i] = sh->q_stride[i];
    f.ks[i] = sh->k_stride[i];
    f.vs[i] = sh->v_stride[i];
    f.os[i] = sh->o_stride[i];
  }
  f.q_bytes = (uint32_t)slice_bytes(N, sh->q_stride[2], 2);
  f.k_bytes = (uint32_t)slice_bytes(N, sh->k_stride[2], 2);
  f.v_bytes = (uint32_t)slice_bytes(N, sh->v_stride[2], 2);
  f.B = sh->batch;
  f.H = sh->heads;
  f.N = (int)N;
  f.nb = (int)((N + 127) / 128);
  f.np = f.nb * 128;
  uint8_t* base = static_cast<uint8_t*>(ws);
  f.q8 = base + L.q8;
  f.k8 = base + L.k8;
  f.v8t = base + L.v8t;
  f.sq = reinterpret_cast<float*>(base + L.sq);
  f.sk = reinterpret_cast<float*>(base + L.sk);
  f.sv = reinterpret_cast<float*>(base + L.sv);
  f.nfull = L.plan.nfull;
  f.ntail = L.plan.ntail;
  f.split = L.plan.split;
  f.part = L.plan.split > 1 ? reinterpret_cast<float*>(base + L.part) : nullptr;
  f.c = (float)((double)sh->softmax_scale * 1.4426950408889634);
  // 448 w = 2^(x + p_off) with p_off just below log2(448): the margin of
  // 2^-14 covers the rounding of the running max, so the product never
  // exceeds 448 before it is converted to e4m3 (w <= 1).
  float off = (float)(std::log2(448.0) - 1.0 / 16384.0);
  while (std::exp2((double)off) > 448.0) off = std::nextafter(off, 0.f);
  f.p_off = off;
  return DIT_ATTN_OK;
}

}  // namespace

extern "C" {

int dit_attn_fwd(const dit_attn_shape* shape, const void* q, const void* k, const void* v, void* o, float* lse,
                 void* stream) {
  g_err[0] = '\0';
  int rc = check_common(shape, q, k, v, o, lse);
  if (rc) return rc;
  dit::AttnArgs a;
  fill_common(shape, q, k, v, o, lse, a);
  return hip_status(dit::launch_attn_bf16(a, (shape->flags & DIT_ATTN_FLAG_OUT_F32) != 0, false,
                                          static_cast<hipStream_t>(stream)),
                    "dit_attn_fwd launch");
}

size_t dit_attn_fwd_workspace_bytes(const dit_attn_shape* shape) {
  if (shape == nullptr || shape->batch < 1 || shape->heads < 1 || shape->seqlen < 1) return 0;
  return tail_plan(shape, device_cus(), dit::kDenseRows, dit::kDenseTileKeys, true).bytes;
}

int dit_attn_fwd_ws(const dit_attn_shape* shape, const void* q, const void* k, const void* v, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  int rc = check_common(shape, q, k, v, o, lse);
  if (rc) return rc;
  const TailPlan t = tail_plan(shape, device_cus(), dit::kDenseRows, dit::kDenseTileKeys, true);
  dit::AttnArgs a;
  fill_common(shape, q, k, v, o, lse, a);
  if (t.split > 1) {
    if (workspace == nullptr) return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", t.bytes);
    if (!aligned(workspace, 256)) return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < t.bytes)
      return fail(DIT_ATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, t.bytes);
    a.nfull = t.nfull;
    a.ntail = t.ntail;
    a.split = t.split;
    a.part = static_cast<float*>(workspace);
  }
  return hip_status(dit::launch_attn_bf16(a, (shape->flags & DIT_ATTN_FLAG_OUT_F32) != 0, false,
                                          static_cast<hipStream_t>(stream)),
                    "dit_attn_fwd_ws launch");
}

int dit_attn_fwd_noalloc(const dit_attn_shape* shape, const void* q, const void* k, const void* v, void* o,
                         float* lse, void* stream) {
  g_err[0] = '\0';
  int rc = check_common(shape, q, k, v, o, lse);
  if (rc) return rc;
  const TailPlan t = tail_plan(shape, device_cus(), dit::kDenseRows, dit::kDenseTileKeys, true);
  if (t.bytes > kNoallocScratchBytes)
    return fail(DIT_ATTN_ERR_WORKSPACE,
                "the tail split of this shape needs %zu bytes of scratch; the library's static scratch holds %zu",
                t.bytes, kNoallocScratchBytes);
  dit::AttnArgs a;
  fill_common(shape, q, k, v, o, lse, a);
  if (t.split > 1) {
    void* ptr = nullptr;
    if ((rc = scratch_device_ptr(&ptr))) return rc;
    a.nfull = t.nfull;
    a.ntail = t.ntail;
    a.split = t.split;
    a.part = static_cast<float*>(ptr);
  }
  return hip_status(dit::launch_attn_bf16(a, (shape->flags & DIT_ATTN_FLAG_OUT_F32) != 0, false,
                                          static_cast<hipStream_t>(stream)),
                    "dit_attn_fwd_noalloc launch");
}

size_t dit_attn_fwd_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

size_t dit_attn_fwd_blocksparse_workspace_bytes(const dit_attn_shape* shape) {
  (void)shape;
  return 0;   // the block-sparse kernel keeps no cross-work-group state
}

int dit_attn_fwd_blocksparse(const dit_attn_shape* shape, const void* q, const void* k, const void* v, void* o,
                             float* lse, const uint8_t* block_mask, int64_t mask_stride_bh, int32_t block_size,
                             void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  int rc = check_common(shape, q, k, v, o, lse);
  if (rc) return rc;
  if (block_mask == nullptr) return fail(DIT_ATTN_ERR_INVALID_ARG, "block_mask is NULL");
  if (block_size != 128) return fail(DIT_ATTN_ERR_UNSUPPORTED, "block_size=%d: only 128 is built", block_size);
  if (mask_stride_bh < 0) return fail(DIT_ATTN_ERR_INVALID_ARG, "mask_stride_bh is negative");
  const size_t need = dit_attn_fwd_blocksparse_workspace_bytes(shape);
  if (need > 0) {
    if (workspace == nullptr) return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (!aligned(workspace, 256)) return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(DIT_ATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
  } else if (workspace != nullptr && !aligned(workspace, 256)) {
    return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  dit::AttnArgs a;
  fill_common(shape, q, k, v, o, lse, a);
  a.mask = block_mask;
  a.mask_bh = mask_stride_bh;
  return hip_status(dit::launch_attn_bf16(a, (shape->flags & DIT_ATTN_FLAG_OUT_F32) != 0, true,
                                          static_cast<hipStream_t>(stream)),
                    "dit_attn_fwd_blocksparse launch");
}

size_t dit_attn_fwd_fp8_workspace_bytes(const dit_attn_shape* shape) {
  if (shape == nullptr || shape->batch < 1 || shape->heads < 1 || shape->seqlen < 1) return 0;
  return fp8_layout((int64_t)shape->batch * shape->heads, shape->seqlen, shape).total;
}

int dit_attn_fp8_quantize(const dit_attn_shape* shape, const void* q, const void* k, const void* v,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  dit::Fp8Args f;
  int rc = prepare_fp8(shape, q, k, v, nullptr, nullptr, workspace, workspace_bytes, false, f);
  if (rc) return rc;
  return hip_status(dit::launch_fp8_quantize(f, static_cast<hipStream_t>(stream)), "fp8 quantise launch");
}

int dit_attn_fwd_fp8(const dit_attn_shape* shape, const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  dit::Fp8Args f;
  int rc = prepare_fp8(shape, q, k, v, o, lse, workspace, workspace_bytes, true, f);
  if (rc) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  f.first_tensor = 1;   // the attention kernel quantises Q in its prologue
  rc = hip_status(dit::launch_fp8_quantize(f, s), "fp8 quantise launch");
  if (rc) return rc;
  return hip_status(dit::launch_attn_fp8(f, (shape->flags & DIT_ATTN_FLAG_OUT_F32) != 0, s), "fp8 attention launch");
}

size_t dit_attn_select_blocks_workspace_bytes(const dit_attn_shape* shape) {
  if (shape == nullptr || shape->batch < 1 || shape->heads < 1 || shape->seqlen < 1) return 0;
  const int64_t nb = (shape->seqlen + 127) / 128;
  return (size_t)(2 * (int64_t)shape->batch * shape->heads * nb * 128 * 4);
}

int dit_attn_select_blocks(const dit_attn_shape* shape, const void* q, const void* k, float tau,
                           int32_t text_tokens, uint8_t* block_mask, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_err[0] = '\0';
  if (shape == nullptr) return fail(DIT_ATTN_ERR_INVALID_ARG, "shape is NULL");
  // Only q and k are read: validate them with the common checks (v and o
  // stand in as q, with q's strides).
  dit_attn_shape tmp = *shape;
  for (int i = 0; i < 3; ++i) tmp.v_stride[i] = tmp.o_stride[i] = tmp.q_stride[i];
  tmp.flags = 0;
  int rc = check_common(&tmp, q, k, q, q, nullptr);
  if (rc) return rc;
  if (!(std::isfinite(tau) && tau >= 0.f)) return fail(DIT_ATTN_ERR_INVALID_ARG, "tau must be finite and >= 0");
  if (text_tokens < 0 || text_tokens > shape->seqlen)
    return fail(DIT_ATTN_ERR_INVALID_ARG, "text_tokens=%d is outside [0, seqlen=%d]", text_tokens, shape->seqlen);
  if (block_mask == nullptr) return fail(DIT_ATTN_ERR_INVALID_ARG, "block_mask is NULL");
  const int64_t nb = (shape->seqlen + 127) / 128;
  if (nb > dit::kSelectMaxBlocks)
    return fail(DIT_ATTN_ERR_UNSUPPORTED, "seqlen=%d: the selection kernel handles at most %d blocks",
                shape->seqlen, dit::kSelectMaxBlocks);
  const size_t need = dit_attn_select_blocks_workspace_bytes(shape);
  if (workspace == nullptr) return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned(workspace, 256)) return fail(DIT_ATTN_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(DIT_ATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
  dit::SelectArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = shape->q_stride[i];
    a.ks[i] = shape->k_stride[i];
  }
  a.q_bytes = (uint32_t)slice_bytes(shape->seqlen, shape->q_stride[2], 2);
  a.k_bytes = (uint32_t)slice_bytes(shape->seqlen, shape->k_stride[2], 2);
  a.B = shape->batch;
  a.H = shape->heads;
  a.N = shape->seqlen;
  a.nb = (int)nb;
  a.tb = (text_tokens + 127) / 128;
  a.scale = shape->softmax_scale;
  a.tau = tau;
  a.pooled = static_cast<float*>(workspace);
  a.mask = block_mask;
  return hip_status(dit::launch_select_blocks(a, static_cast<hipStream_t>(stream)), "dit_attn_select_blocks launch");
}

const char* dit_attn_status_string(int status) {
  switch (status) {
    case DIT_ATTN_OK: return "ok";
    case DIT_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case DIT_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case DIT_ATTN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DIT_ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dit_attn_last_error(void) { return g_err; }

int dit_attn_version(void) { return 1 * 10000 + 0 * 100 + 0; }

}  // extern "C"
