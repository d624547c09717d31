// launch.h -- internal interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// Arguments of the bf16 attention kernels (dense and block-sparse).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;           // nullable, [B*H][N]
  int64_t qs[3], ks[3], vs[3], os[3];  // element strides of (b, h, n)
  uint32_t q_bytes, k_bytes, v_bytes;  // extent of one (b, h) slice in bytes
  int B, H, N;
  int nqb;              // query blocks per (b, h)
  float c;              // softmax_scale * log2(e)
  const uint8_t* mask;  // block-sparse only: [nb][nb] per (b, h)
  int64_t mask_bh;      // element offset between (b, h) masks
  int nb;               // ceil(N / 128)
  // Dense tail balancing: work-groups [0, nfull) each own one query block
  // and its whole key range; the last ntail query blocks are each split
  // into `split` key ranges whose partial results go to `part` and are
  // combined by the merge kernel.  split == 1: no tail split.
  int nfull, ntail, split;
  float* part;          // [ntail * split][bm rows][kPartRow] fp32
  float lse_off;        // added to log2 of the merged weight sum (0; fp8: -log2 448)
  int bm;               // query rows per block of the split grid (merge)
};

// Dense bf16 kernel: query rows per work-group and keys per LDS tile (the
// host's tail-split plan works in these units).
constexpr int kDenseRows = 384;
constexpr int kDenseTileKeys = 32;

// fp32 words per row of a partial result: 128 unnormalised O, the row's
// reference m c (log2 units), its weight sum l, and two words of padding.
constexpr int kPartRow = 132;

// Arguments of the fp8 quantisation pass and the fp8 attention kernel.
struct Fp8Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs[3], ks[3], vs[3], os[3];
  uint32_t q_bytes, k_bytes, v_bytes;
  int B, H, N, nb, np;  // np = 128 * nb
  uint8_t* q8;          // [BH][np][128]
  uint8_t* k8;          // [BH][np][128]
  uint8_t* v8t;         // [BH][128][np], key-permuted per 64-key group
  float* sq;            // [BH][nb]
  float* sk;
  float* sv;
  float c;              // softmax_scale * log2(e)
  float p_off;          // just below log2(448): w * 448 = exp2(x + p_off) <= 448
  int first_tensor;     // quantisation pass: 0 = Q, K and V; 1 = K and V (the attention quantises Q itself)
  // Tail split of the attention grid, as for AttnArgs (split == 1: none).
  int nfull, ntail, split;
  float* part;          // [ntail * split][bm rows][kPartRow] fp32
};

// Arguments of the block-mask selection passes.
struct SelectArgs {
  const void* q;
  const void* k;
  int64_t qs[3], ks[3];
  uint32_t q_bytes, k_bytes;
  int B, H, N, nb, tb;           // nb = ceil(N / 128), tb = ceil(text tokens / 128)
  float scale, tau;
  float* pooled;                 // fp32 block means: Q [BH][nb][128], then K transposed [BH][128][nb]
  uint8_t* mask;                 // [BH][nb][nb]
};

// Launch `kernel` and return the status of this launch alone: hipLaunchKernel
// reports it directly, whereas hipGetLastError would also return (and clear)
// an error left on the thread by an earlier, unrelated HIP call.
template <typename... P>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, const P&... args) {
  void* argv[] = {const_cast<void*>(static_cast<const void*>(&args))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
}

hipError_t launch_attn_bf16(const AttnArgs& a, bool out_f32, bool sparse, hipStream_t s);
hipError_t launch_attn_merge(const AttnArgs& a, bool out_f32, hipStream_t s);
hipError_t launch_fp8_quantize(const Fp8Args& a, hipStream_t s);
hipError_t launch_attn_fp8(const Fp8Args& a, bool out_f32, hipStream_t s);
hipError_t launch_select_blocks(const SelectArgs& a, hipStream_t s);
constexpr int kSelectMaxBlocks = 4096;   // nb limit of the selection kernel (key-block logits kept in registers)

}  // namespace dit
