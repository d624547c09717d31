// attn_bf16.hip -- bf16 flash-style joint attention forward for gfx950.
//
// One work-group owns BM = 32 * R * NW query rows of one (batch, head); each
// wave owns R blocks of 32 rows (R = 2 dense: 256 rows per work-group; R = 1
// block-sparse: 128 rows, one mask row).  K and V stream through LDS in
// tiles of 64 keys, double-buffered: the global loads of tile t+2 are in
// flight while tile t is computed and tile t+1 waits in the other LDS buffer.
//
// Per tile and wave, with the 32x32x16 bf16 MFMA (fp32 accumulate):
//   S^T = K Q^T      A = K rows from LDS, B = Q held in registers.  In the
//                    transposed product each lane holds 16 keys of one query
//                    row, so the row max and row sum are in-register
//                    reductions plus one exchange with lane l^32.
//   online softmax   P = 2^(S c - m c) with c = scale * log2(e) and m the
//                    running row max; l += sum P.  m is only moved when a
//                    row's max grows by more than 2^8 in P units: then
//                    alpha = 2^((m - m') c), O *= alpha, l *= alpha.  The
//                    result is the same softmax (the factor cancels in O / l).
//   O^T += V^T P^T   A = V^T from LDS, B = P straight from the S registers
//                    rounded to bf16 -- no shuffle: the PV reduction index
//                    is permuted instead, by storing the V^T tile in LDS with
//                    its keys in the order the accumulator hands P out.
// Epilogue: O = O^T / l, stored bf16 (round to nearest even) or fp32, and
// optionally lse = ln2 * (m c + log2 l).
//
// The block-sparse variant runs the same per-tile arithmetic over the active
// 128-key blocks of its query block only (masked blocks are never loaded).
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace dit {
namespace {

constexpr int D = kHeadDim;
constexpr int BN = 64;        // keys per LDS tile
constexpr int KS = D + 8;     // K tile row stride in bf16 (272 B: conflict-free b128 reads)
constexpr int VS = BN + 8;    // V^T tile row stride in bf16 (144 B)
// Lazy rescaling: P = 2^(S c - m c) may reach 2^kLazy before the running max
// m is moved, so O and l are rescaled only on large jumps of the row max.
constexpr float kLazy = 8.f;

// Position (in 4-key groups) of key group g4 inside a 16-key group of the
// V^T tile.  Lane half h of the PV operand reads 8 consecutive keys at 8h:
// the 32x32 accumulator gives half 0 keys {0..3, 8..11} and half 1 keys
// {4..7, 12..15} of every 16, so groups 1 and 2 trade places.
__device__ __forceinline__ int vpos16(int g4) { return ((g4 & 1) << 1) | (g4 >> 1); }

// Global -> register -> LDS staging of one K tile (row-major, padded rows)
// and one V^T tile (d-major, keys permuted per 16 as above).  K moves as
// 16-byte chunks; V as units of 4 keys x 8 d that are transposed in
// registers (16 v_perm-style ops) and written as 8-byte rows of V^T.  With
// 512 threads the first half of the work-group moves V and the second K.
template <int NT>
struct TileLoader {
  static constexpr int KCHUNKS = BN * (D / 8);        // 16-byte K chunks per tile
  static constexpr int VUNITS = (BN / 4) * (D / 8);   // V units per tile
  static constexpr bool SPLIT = NT > VUNITS;          // separate K and V threads
  static constexpr int KCH = SPLIT ? KCHUNKS / (NT - VUNITS) : KCHUNKS / NT;
  static constexpr int VUN = SPLIT ? 1 : VUNITS / NT;
  static_assert(SPLIT ? (KCH * (NT - VUNITS) == KCHUNKS && NT - VUNITS > 0)
                      : (KCH * NT == KCHUNKS && VUN * NT == VUNITS), "tile split");
  u32x4 kr[KCH];
  u32x4 vr[VUN][4];

  __device__ __forceinline__ bool does_k(int tid) const { return !SPLIT || tid >= VUNITS; }
  __device__ __forceinline__ bool does_v(int tid) const { return !SPLIT || tid < VUNITS; }
  __device__ __forceinline__ int ktid(int tid) const { return SPLIT ? tid - VUNITS : tid; }
  static constexpr int KSTRIDE = SPLIT ? NT - VUNITS : NT;

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                       uint32_t krow, uint32_t vrow, int key0, int tid) {
    if (does_k(tid)) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int id = ktid(tid) + i * KSTRIDE, key = id >> 4, c = id & 15;
        kr[i] = buf_load_b128(rk, (uint32_t)(key0 + key) * krow + c * 16);
      }
    }
    if (does_v(tid)) {
#pragma unroll
      for (int u = 0; u < VUN; ++u) {
        const int id = tid + u * NT, g = id & 15, c = id >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vr[u][r] = buf_load_b128(rv, (uint32_t)(key0 + 4 * g + r) * vrow + c * 16);
      }
    }
  }

  __device__ __forceinline__ void store(__bf16* sk, __bf16* sv, int tid) const {
    if (does_k(tid)) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int id = ktid(tid) + i * KSTRIDE, key = id >> 4, c = id & 15;
        *reinterpret_cast<u32x4*>(sk + key * KS + c * 8) = kr[i];
      }
    }
    if (does_v(tid)) {
#pragma unroll
      for (int u = 0; u < VUN; ++u) {
        const int id = tid + u * NT, g = id & 15, c = id >> 4;
        const int pos = 16 * (g >> 2) + 4 * vpos16(g & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int w = j >> 1;
          const uint32_t a0 = vr[u][0][w], a1 = vr[u][1][w], a2 = vr[u][2][w], a3 = vr[u][3][w];
          u32x2 out;
          if ((j & 1) == 0) {
            out[0] = (a0 & 0xffffu) | (a1 << 16);
            out[1] = (a2 & 0xffffu) | (a3 << 16);
          } else {
            out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
            out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
          }
          *reinterpret_cast<u32x2*>(sv + (8 * c + j) * VS + pos) = out;
        }
      }
    }
  }
};

struct DenseTiles {
  int pos, N;
  __device__ __forceinline__ int next() {
    if (pos >= N) return -1;
    const int k = pos;
    pos += BN;
    return k;
  }
};

// Active 128-key blocks of one mask row, found 64 at a time with a ballot;
// every value here is wave-uniform.
struct SparseTiles {
  const uint8_t* row;
  int nb, N, chunk, pend;
  uint64_t bits;
  __device__ __forceinline__ int next_block() {
    while (bits == 0) {
      ++chunk;
      if (chunk * 64 >= nb) return -1;
      const int j = chunk * 64 + (int)(threadIdx.x & 63);
      const int keep = (j < nb) ? (int)row[j] : 0;
      bits = __ballot(keep != 0);
    }
    const int b = __builtin_ctzll(bits);
    bits &= bits - 1;
    return chunk * 64 + b;
  }
  __device__ __forceinline__ int next() {
    if (pend >= 0) {
      const int k = pend;
      pend = -1;
      return k;
    }
    const int blk = next_block();
    if (blk < 0) return -1;
    const int k = blk * kBlock;
    if (k + BN < N) pend = k + BN;
    return k;
  }
};

template <int NW, int R, bool OUT_F32, bool SPARSE>
__global__ __launch_bounds__(NW * 64, (R == 1 ? 2 : 1)) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32 * R;
  static_assert(!SPARSE || BM == kBlock, "block-sparse work-groups cover one 128-row mask block");
  __shared__ __attribute__((aligned(16))) __bf16 smK[2][BN * KS];
  __shared__ __attribute__((aligned(16))) __bf16 smV[2][D * VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / a.nqb, qblk = tile % a.nqb;
  const int b = bh / a.H, hd = bh % a.H;
  const int N = a.N;
  const float c = a.c;

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.qs[0] + hd * a.qs[1];
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.ks[0] + hd * a.ks[1];
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.vs[0] + hd * a.vs[1];
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qp, a.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp, a.k_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp, a.v_bytes);
  const uint32_t qrow = (uint32_t)(a.qs[2] * 2), krow = (uint32_t)(a.ks[2] * 2),
                 vrow = (uint32_t)(a.vs[2] * 2);

  const int q0 = qblk * BM + wave * 32 * R;

  // Q as the B operand of S^T = K Q^T: lane (l32, h) holds row q0 + 32 qi + l32,
  // d = 16 s + 8 h .. +7 for step s.  Rows >= N load as zero.
  bf16x8 qf[R][8];
#pragma unroll
  for (int qi = 0; qi < R; ++qi)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[qi][s] = __builtin_bit_cast(
          bf16x8, buf_load_b128(rq, (uint32_t)(q0 + qi * 32 + l32) * qrow + (16 * s + 8 * h) * 2));

  f32x16 oacc[R][4];
#pragma unroll
  for (int qi = 0; qi < R; ++qi)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qi][db][r] = 0.f;
  // m_run: running max of the raw dot products (the value P is taken
  // against), mc_run = m_run * c (0 until the first tile sets it).
  float m_run[R], mc_run[R], l_run[R];
#pragma unroll
  for (int qi = 0; qi < R; ++qi) {
    m_run[qi] = -INFINITY;
    mc_run[qi] = 0.f;
    l_run[qi] = 0.f;
  }

  typename std::conditional<SPARSE, SparseTiles, DenseTiles>::type tiles;
  if constexpr (SPARSE) {
    tiles.row = a.mask + (int64_t)bh * a.mask_bh + (int64_t)qblk * a.nb;
    tiles.nb = a.nb;
    tiles.N = N;
    tiles.chunk = -1;
    tiles.pend = -1;
    tiles.bits = 0;
  } else {
    tiles.pos = 0;
    tiles.N = N;
  }

  TileLoader<NT> ld;
  int k_cur = tiles.next();
  if (k_cur >= 0) {
    ld.load(rk, rv, krow, vrow, k_cur, tid);
    ld.store(smK[0], smV[0], tid);
  }
  int k_nxt = tiles.next();
  if (k_nxt >= 0) ld.load(rk, rv, krow, vrow, k_nxt, tid);
  __syncthreads();

  // One key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  MASK is set
  // only for the ragged last tile, so full tiles carry no key compares.
  auto tile_body = [&](auto mask_tag, const __bf16* sK, const __bf16* sV, int k_cur) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 sacc[R][2];
#pragma unroll
    for (int qi = 0; qi < R; ++qi)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qi][kb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (kb * 32 + l32) * KS + 16 * s + 8 * h);
#pragma unroll
        for (int qi = 0; qi < R; ++qi)
          sacc[qi][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qi][s], sacc[qi][kb], 0, 0, 0);
      }
    }

    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k_cur + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          if (key >= N) {
#pragma unroll
            for (int qi = 0; qi < R; ++qi) sacc[qi][kb][r] = -INFINITY;
          }
        }
    }

    // Row max of the tile; the running max moves (and O, l are rescaled)
    // only when some row of the wave gains more than 2^kLazy, so most
    // tiles skip the rescale of the 64 x 128 accumulator.
    float mx[R];
    bool grow = false;
#pragma unroll
    for (int qi = 0; qi < R; ++qi) {
      float t = sacc[qi][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) t = fmaxf(t, sacc[qi][kb][r]);
      t = fmaxf(t, swap_halves(t));
      mx[qi] = t;
      grow |= (t - m_run[qi]) * c > kLazy;
    }
    if (__any(grow)) {
#pragma unroll
      for (int qi = 0; qi < R; ++qi) {
        const float mnew = fmaxf(m_run[qi], mx[qi]);
        const float alpha = fast_exp2((m_run[qi] - mnew) * c);
        l_run[qi] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qi][db][r] *= alpha;
        m_run[qi] = mnew;
        mc_run[qi] = mnew * c;
      }
    }

    // P rounded to bf16 (round to nearest even) feeds the PV product, and the
    // row sum is taken over those same rounded weights (one v_dot2 with
    // (1, 1) per pair), so the normalised weights stay a convex combination
    // even when a single key dominates the row.
    uint32_t pk[R][2][8];   // P as packed bf16 pairs, [qi][kb][pair]
#pragma unroll
    for (int qi = 0; qi < R; ++qi) {
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(sacc[qi][kb][r], c, -mc_run[qi]));
          const float p1 = fast_exp2(__builtin_fmaf(sacc[qi][kb][r + 1], c, -mc_run[qi]));
          pk[qi][kb][r >> 1] = pack_bf16x2(p0, p1);
          ls[(r >> 1) & 3] = sum_bf16x2(pk[qi][kb][r >> 1], ls[(r >> 1) & 3]);
        }
      l_run[qi] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }

#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      bf16x8 pf[R];
#pragma unroll
      for (int qi = 0; qi < R; ++qi) {
        u32x4 t;
#pragma unroll
        for (int w = 0; w < 4; ++w) t[w] = pk[qi][s4 >> 1][4 * (s4 & 1) + w];
        pf[qi] = __builtin_bit_cast(bf16x8, t);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + (db * 32 + l32) * VS + 16 * s4 + 8 * h);
#pragma unroll
        for (int qi = 0; qi < R; ++qi)
          oacc[qi][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qi], oacc[qi][db], 0, 0, 0);
      }
    }
  };

  // Full tiles; the ragged tile (if any) holds key N - 1 and so comes last
  // in both the dense and the block-sparse order: it runs after the loop.
  int buf = 0;
  while (k_cur >= 0 && k_cur + BN <= N) {
    tile_body(std::false_type{}, smK[buf], smV[buf], k_cur);

    int k_nn = -1;
    if (k_nxt >= 0) {
      ld.store(smK[buf ^ 1], smV[buf ^ 1], tid);
      k_nn = tiles.next();
      if (k_nn >= 0) ld.load(rk, rv, krow, vrow, k_nn, tid);
    }
    __syncthreads();
    k_cur = k_nxt;
    k_nxt = k_nn;
    buf ^= 1;
  }
  if (k_cur >= 0) tile_body(std::true_type{}, smK[buf], smV[buf], k_cur);

  // ---- epilogue ----
  const int64_t ob = b * a.os[0] + hd * a.os[1];
#pragma unroll
  for (int qi = 0; qi < R; ++qi) {
    const float lt = l_run[qi] + swap_halves(l_run[qi]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int row = q0 + qi * 32 + l32;
    if (row < N) {
      const int64_t orow = ob + (int64_t)row * a.os[2];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = db * 32 + r4 * 8 + h * 4;
          const float v0 = oacc[qi][db][4 * r4 + 0] * inv, v1 = oacc[qi][db][4 * r4 + 1] * inv;
          const float v2 = oacc[qi][db][4 * r4 + 2] * inv, v3 = oacc[qi][db][4 * r4 + 3] * inv;
          if constexpr (OUT_F32) {
            f32x4 t = {v0, v1, v2, v3};
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d0) = t;
          } else {
            u32x2 t = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
            *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.o) + orow + d0) = t;
          }
        }
      if (a.lse != nullptr && h == 0)
        a.lse[(int64_t)bh * N + row] =
            lt > 0.f ? (m_run[qi] * c + __builtin_log2f(lt)) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& args, bool out_f32, bool sparse, hipStream_t s) {
  AttnArgs a = args;
  a.nqb = sparse ? a.nb : (a.N + 255) / 256;   // work-group rows: 128 (sparse) or 256 (dense)
  const int64_t nwg = (int64_t)a.B * a.H * a.nqb;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nwg);
  if (sparse) {
    if (out_f32) hipLaunchKernelGGL((attn_bf16_kernel<4, 1, true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<4, 1, false, true>), grid, dim3(256), 0, s, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((attn_bf16_kernel<8, 1, true, false>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<8, 1, false, false>), grid, dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dit
