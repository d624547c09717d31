// select_blocks.hip -- block-mask selection for block-sparse attention, in the
// manner of Sol-Attention (a tau-controlled block-sparse backend; bpdata.com
// page, section "Részletes optimalizációs lépések és hatásuk").  The pages
// give no rule; the one built here: key block j is kept for query block i iff
// its share of the row's attention, estimated from block-mean-pooled queries
// and keys, is at least tau times the uniform share:
//   qm_i, km_j = means over the valid tokens of the 128-token blocks
//   s_ij = scale <qm_i, km_j>,  p_ij = softmax_j(s_ij),  keep iff p_ij >= tau / nb
// plus the diagonal and the text blocks' rows and columns, always kept.
//
// Two passes:
//   pool_kernel     one work-group per (tensor, b, h, block): fp32 column
//                   means of the block's valid tokens (HBM-bound: Q and K
//                   read once), in a fixed summation order.
//   select_kernel   one work-group per (b, h, four query blocks): the nb
//                   logits of each row, their max and exponential sum
//                   (fixed-order reductions), and the keep decisions
//                   e_j >= tau * sum / nb, written as mask rows.
#include "device_common.h"
#include "launch.h"

#include <math.h>

namespace dit {
namespace {

constexpr int D = kHeadDim;
constexpr int SQB = 4;      // query blocks (mask rows) per selection work-group
constexpr int SMAXT = kSelectMaxBlocks / 256;   // key blocks per thread

// grid: 2 * BH * nb; 256 threads.  Thread (r, c) = (tid / 16, tid % 16) sums
// rows r, r + 16, .., r + 112 of the block over d = 8c .. 8c + 7; the 16 row
// partials of each column are then added in row order.
__global__ __launch_bounds__(256) void pool_kernel(SelectArgs a) {
  __shared__ float part[16][D];
  const int tid = threadIdx.x;
  const int BH = a.B * a.H;
  const int id = blockIdx.x;
  const int tensor = id / (BH * a.nb);
  const int rem = id % (BH * a.nb);
  const int bh = rem / a.nb, blk = rem % a.nb;
  const int b = bh / a.H, hd = bh % a.H;
  const __bf16* src = static_cast<const __bf16*>(tensor == 0 ? a.q : a.k);
  const int64_t* st = tensor == 0 ? a.qs : a.ks;
  src += b * st[0] + hd * st[1];
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, tensor == 0 ? a.q_bytes : a.k_bytes);
  const uint32_t row_bytes = (uint32_t)(st[2] * 2);
  const int r = tid >> 4, c = tid & 15;
  const int j0 = blk * kBlock;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = min(j0 + r + 16 * i, a.N);   // rows >= N read as zero
    const u32x4 x = buf_load_b128(rs, (uint32_t)row * row_bytes + c * 16);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += __builtin_bit_cast(float, x[w] << 16);
      acc[2 * w + 1] += __builtin_bit_cast(float, x[w] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r][8 * c + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s += part[rr][tid];
    const int count = min(kBlock, a.N - j0);
    const float mean = s / (float)count;
    if (tensor == 0)
      a.pooled[((int64_t)bh * a.nb + blk) * D + tid] = mean;                          // Q: [bh][nb][d]
    else
      a.pooled[(int64_t)BH * a.nb * D + ((int64_t)bh * D + tid) * a.nb + blk] = mean;   // K: [bh][d][nb]
  }
}

// Sum (or max) over the work-group's four waves of SQB values per thread,
// in a fixed order: a butterfly inside each wave, then the four wave results
// added in wave order.  Every thread receives the results.
template <bool MAX>
__device__ __forceinline__ void wg_reduce(float (&v)[SQB], float (*red)[SQB]) {
#pragma unroll
  for (int r = 0; r < SQB; ++r)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float o = __shfl_xor(v[r], m, 64);
      v[r] = MAX ? fmaxf(v[r], o) : v[r] + o;
    }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int r = 0; r < SQB; ++r) red[w][r] = v[r];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < SQB; ++r) {
    float x = red[0][r];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) x = MAX ? fmaxf(x, red[ww][r]) : x + red[ww][r];
    v[r] = x;
  }
  __syncthreads();
}

// grid: BH * ceil(nb / SQB); 256 threads.  Work-group (bh, g) decides the
// mask rows of query blocks i = SQB g .. SQB g + SQB - 1; thread t owns key
// blocks j = t + 256 u (u < SMAXT) and keeps their logits in registers.  The
// pooled keys are stored transposed ([d][nb]), so the loads of one d are
// coalesced over the threads' key blocks.
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  __shared__ float qm[SQB][D];
  __shared__ float red[4][SQB];
  const int tid = threadIdx.x;
  const int BH = a.B * a.H;
  const int ng = (a.nb + SQB - 1) / SQB;
  const int bh = blockIdx.x / ng, i0 = (blockIdx.x % ng) * SQB;
  const float* qpool = a.pooled + (int64_t)bh * a.nb * D;
  const float* kpoolT = a.pooled + (int64_t)BH * a.nb * D + (int64_t)bh * D * a.nb;
  for (int e = tid; e < SQB * D; e += 256) {
    const int r = e / D, i = i0 + r;
    qm[r][e % D] = i < a.nb ? qpool[(int64_t)i * D + e % D] : 0.f;
  }
  __syncthreads();
  float s[SQB][SMAXT];
  float mx[SQB];
#pragma unroll
  for (int r = 0; r < SQB; ++r) mx[r] = -INFINITY;
#pragma unroll
  for (int u = 0; u < SMAXT; ++u) {
    const int j = tid + 256 * u;
    float dot[SQB] = {};
    if (j < a.nb) {
#pragma unroll 16
      for (int d = 0; d < D; ++d) {
        const float kv = kpoolT[(int64_t)d * a.nb + j];
#pragma unroll
        for (int r = 0; r < SQB; ++r) dot[r] = __builtin_fmaf(qm[r][d], kv, dot[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < SQB; ++r) {
      s[r][u] = dot[r] * a.scale;
      if (j < a.nb) mx[r] = fmaxf(mx[r], s[r][u]);
    }
  }
  wg_reduce<true>(mx, red);
  float z[SQB];
#pragma unroll
  for (int r = 0; r < SQB; ++r) {
    z[r] = 0.f;
#pragma unroll
    for (int u = 0; u < SMAXT; ++u) {
      const int j = tid + 256 * u;
      s[r][u] = j < a.nb ? __expf(s[r][u] - mx[r]) : 0.f;
      z[r] += s[r][u];
    }
  }
  wg_reduce<false>(z, red);
#pragma unroll
  for (int r = 0; r < SQB; ++r) {
    const int i = i0 + r;
    if (i >= a.nb) break;
    const float thr = a.tau * z[r] / (float)a.nb;
    uint8_t* out = a.mask + ((int64_t)bh * a.nb + i) * a.nb;
#pragma unroll
    for (int u = 0; u < SMAXT; ++u) {
      const int j = tid + 256 * u;
      if (j < a.nb) {
        const bool forced = (j == i) || (i < a.tb) || (j < a.tb);
        out[j] = (uint8_t)((s[r][u] >= thr) || forced);
      }
    }
  }
}

}  // namespace

hipError_t launch_select_blocks(const SelectArgs& a, hipStream_t s) {
  const int64_t npool = 2LL * a.B * a.H * a.nb, nsel = (int64_t)a.B * a.H * ((a.nb + SQB - 1) / SQB);
  if (npool <= 0 || npool > 0x7fffffff || a.nb > kSelectMaxBlocks) return hipErrorInvalidConfiguration;
  hipError_t e = launch_kernel(pool_kernel, dim3((unsigned)npool), dim3(256), s, a);
  if (e != hipSuccess) return e;
  return launch_kernel(select_kernel, dim3((unsigned)nsel), dim3(256), s, a);
}

}  // namespace dit
