// attn_bf16.hip -- bf16 flash-style joint attention forward for gfx950.
//
// Both kernels follow one recipe per key tile (fp32 accumulate):
//   S^T = K Q^T      A = K rows from LDS, B = Q held in registers for the
//                    whole kernel.
//   online softmax   P = 2^(S c - m c) with c = scale * log2(e) and m a
//                    running reference: the row max of the first tile.  Later
//                    tiles take their exponentials against it directly; only
//                    when a lane's weights would pass 2^64 (a row max that
//                    grew by more than 64 bits) is m moved to the new max,
//                    O and l rescaled and the tile redone.  The factor
//                    cancels in O / l, so the result is unchanged.
//   O^T += V^T P^T   A = V^T, read from the row-major V tile with the gfx950
//                    transposing LDS read (ds_read_b64_tr_b16: 16 lanes
//                    fetch a 4-key x 16-d block and each lane receives one d
//                    column of it), B = P straight from the S registers
//                    rounded to bf16 -- no shuffle: the PV reduction index is
//                    permuted instead, by choosing which 4 keys each
//                    transposing read fetches to match the order in which
//                    the accumulator hands P out.  l accumulates the same
//                    rounded P (v_dot2 with (1, 1)).
// Epilogue: O = O^T / l, stored bf16 (round to nearest even) or fp32, and
// optionally lse = ln2 * (m c + log2 l).
//
// Dense kernel (attn_dense_kernel): 8 waves x 48 query rows = 384 rows of
// one (batch, head) per work-group, two waves per SIMD.  Each wave's rows are
// three 16-row blocks on the 16x16x32 bf16 MFMA, so every K fragment and V
// operand read from LDS feeds three MFMAs (a third less LDS traffic per flop
// than 32-row waves).  K and V stream through LDS in 32-key tiles in three
// rotating buffers.  Step t issues the QK^T MFMAs of tile t+1 and the PV
// MFMAs of tile t as one stream with their LDS operands read ahead; the LDS
// stores of tile t+2 and the global loads of tile t+3 ride on the PV MFMAs;
// then one barrier, then the softmax of tile t+1.
//
// Tail split (dense, with a caller workspace): one 384-row work-group runs
// per compute unit at a time, so the query blocks of a last, partial round
// would leave most units idle.  Each of those blocks is instead split into
// `split` consecutive key ranges run by separate work-groups (launched after
// the full blocks); each range stores its unnormalised O, reference m c and
// weight sum l, and attn_merge_kernel combines them in key order with the
// exact rescaling 2^(m_p c - max m c).
//
// Block-sparse kernel (attn_sparse_kernel): 4 waves x 32 rows = one 128-row
// mask block per work-group (two per CU), 32x32x16 MFMAs, 64-key tiles over
// the kept 128-key blocks of its mask row only (masked blocks are never
// loaded), two LDS buffers, and its global loads issued two steps ahead in
// two alternating register sets.

#include "device_common.h"
#include "launch.h"

namespace dit {
namespace {

constexpr int D = kHeadDim;
constexpr int BN = 64;        // keys per LDS tile (block-sparse kernel)
constexpr int KS = D + 8;     // K tile row stride in bf16 (272 B: conflict-free b128 reads)
constexpr int VSR = D + 32;   // V tile row stride in bf16 (320 B: 4 consecutive rows of a
                              // transposing read land in disjoint bank quarters)
// When the reference max is recomputed (first tile, or a redo after a huge
// jump), it only moves if some row of the wave grew by more than 2^kLazy.
constexpr float kLazy = 8.f;

// Global -> register -> LDS staging of one tile: K and V both row-major
// (padded rows), moved as 16-byte chunks; the tile's 2048 chunks are dealt
// round-robin over the work-group, K first.
template <int NT>
struct TileLoader {
  static constexpr int KCH = BN * (D / 8) / NT;   // K chunks per thread; V has as many
  static constexpr int CH = 2 * KCH;
  static_assert(KCH * NT == BN * (D / 8), "tile split");
  u32x4 r[CH];

  // Chunk i of this thread: K for i < KCH, else V (compile-time per i, so
  // every load takes a uniform buffer resource).
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                       uint32_t krow, uint32_t vrow, int key0, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool isk = i < KCH;
      const int cid = tid + (isk ? i : i - KCH) * NT, key = cid >> 4, c = cid & 15;
      r[i] = buf_load_b128(isk ? rk : rv, (uint32_t)(key0 + key) * (isk ? krow : vrow) + c * 16);
    }
  }

  template <int I>
  __device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           uint32_t krow, uint32_t vrow, int key0, int tid) {
    constexpr bool isk = I < KCH;
    const int cid = tid + (isk ? I : I - KCH) * NT, key = cid >> 4, c = cid & 15;
    r[I] = buf_load_b128(isk ? rk : rv, (uint32_t)(key0 + key) * (isk ? krow : vrow) + c * 16);
  }
  template <int I>
  __device__ __forceinline__ void store_one(__bf16* sk, __bf16* sv, int tid) const {
    constexpr bool isk = I < KCH;
    const int cid = tid + (isk ? I : I - KCH) * NT, key = cid >> 4, c = cid & 15;
    *reinterpret_cast<u32x4*>((isk ? sk + key * KS : sv + key * VSR) + c * 8) = r[I];
  }

  __device__ __forceinline__ void store(__bf16* sk, __bf16* sv, int tid) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool isk = i < KCH;
      const int cid = tid + (isk ? i : i - KCH) * NT, key = cid >> 4, c = cid & 15;
      *reinterpret_cast<u32x4*>((isk ? sk + key * KS : sv + key * VSR) + c * 8) = r[i];
    }
  }
};

// A operand of O^T += V^T P^T for k-step s4 (16 keys) and d block db: lane
// (l32, h) needs V[key][32 db + l32] for the 8 keys its P registers cover,
// keys 16 s4 + 8 r + 4 h + j (r, j = 0..3).  Each transposing read serves
// one r: lane s of a 16-lane group points at row 16 s4 + 8 r + 4 h + s/4,
// columns 32 db + 16 (group & 1) + 4 (s & 3) .. +3, and receives the column
// 32 db + l32 of those 4 rows.
__device__ __forceinline__ bf16x8 v_operand(const __bf16* sV, int s4, int db, int lane) {
  const int grp = lane >> 4, s = lane & 15;
  const int h = grp >> 1;
  const __bf16* base = sV + (16 * s4 + 4 * h + (s >> 2)) * VSR + 32 * db + 16 * (grp & 1) + 4 * (s & 3);
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + 8 * VSR));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

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

// S^T for one 64-key tile: sacc[kb][r] holds key 32 kb + (r/4)*8 + 4h + r%4
// of query row l32.
__device__ __forceinline__ void qk_tile(f32x16 (&sacc)[2], const __bf16* sK, const bf16x8 (&qf)[8],
                                        int l32, int h) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (kb * 32 + l32) * KS + 16 * s + 8 * h);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kb], 0, 0, 0);
    }
}

struct RowState {
  float m;    // running max of the raw dot products P is taken against
  float mc;   // m * c (0 until the first tile sets it)
  float l;    // this lane's partial sum of the rounded P
};

// Sum over both lane halves of one query row (lanes l and l^32).
__device__ __forceinline__ float row_sum_halves(float x) { return x + swap_halves(x); }

// Move the running max when some row of the wave grew past the lazy bound
// (t is the tile's row max), rescaling O and l.
__device__ __forceinline__ void maybe_rescale(float t, RowState& st, f32x16 (&oacc)[4], float c) {
  const bool grow = (t - st.m) * c > kLazy;
  if (__any(grow)) {
    const float mnew = fmaxf(st.m, t);
    const float alpha = fast_exp2((st.m - mnew) * c);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    st.m = mnew;
    st.mc = mnew * c;
  }
}

// Four independent max chains (folded into v_max3 by the compiler), then
// the lane-half exchange.
__device__ __forceinline__ float tile_max(const f32x16 (&sacc)[2]) {
  float t[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t[j] = sacc[j >> 1][8 * (j & 1)];
#pragma unroll
    for (int r = 1; r < 8; ++r) t[j] = fmaxf(t[j], sacc[j >> 1][8 * (j & 1) + r]);
  }
  return max_halves(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
}

// P = 2^(S c - mc) for the 32 elements, rounded to bf16 pairs in pk; returns
// this lane's sum of the rounded P.  The elements go through each stage
// together (exponent FMAs, exponentials, packing, sums), so dependent
// instructions sit far apart and one wave can keep the vector ALU busy.
__device__ __forceinline__ float exp_tile_sum(const f32x16 (&sacc)[2], float mc, uint32_t (&pk)[2][8], float c) {
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(sacc[i >> 4][i & 15], c, -mc);
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = fast_exp2(x[i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) pk[i >> 3][i & 7] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) ls[i & 3] = sum_bf16x2(pk[i >> 3][i & 7], ls[i & 3]);
  return (ls[0] + ls[1]) + (ls[2] + ls[3]);
}

// Later tiles: take the exponentials against the current reference
// straight away.  Weights far above 1 are harmless in floating point (the
// row sum and O keep their relative precision), so the tile is kept unless a
// lane's weights sum past 2^64 or overflow; only then is the reference moved
// to the tile's max (O and l rescaled) and the tile redone.  This keeps the
// per-tile row max out of the common path.
// `first` (wave-uniform) forces the max pass, for the first tile of a row.
constexpr float kCheck = 0x1p64f;   // 2^64
__device__ __forceinline__ void softmax_next(const f32x16 (&sacc)[2], RowState& st, f32x16 (&oacc)[4],
                                             uint32_t (&pk)[2][8], float c, bool first = false) {
  float ls = exp_tile_sum(sacc, st.mc, pk, c);
  if (first || __any(!(ls <= kCheck))) {
    maybe_rescale(tile_max(sacc), st, oacc, c);
    ls = exp_tile_sum(sacc, st.mc, pk, c);
  }
  st.l += ls;
}

__device__ __forceinline__ bf16x8 p_operand(const uint32_t (&pk)[2][8], int s4) {
  u32x4 t;
#pragma unroll
  for (int w = 0; w < 4; ++w) t[w] = pk[s4 >> 1][4 * (s4 & 1) + w];
  return __builtin_bit_cast(bf16x8, t);
}

__device__ __forceinline__ void pv_tile(f32x16 (&oacc)[4], const uint32_t (&pk)[2][8], const __bf16* sV,
                                        int lane) {
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const bf16x8 pf = p_operand(pk, s4);
#pragma unroll
    for (int db = 0; db < 4; ++db)
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(sV, s4, db, lane), pf, oacc[db], 0, 0, 0);
  }
}

// One MFMA phase of the pipeline: S^T of the next tile (16 MFMAs, A = K
// rows from sK) followed by O^T += V^T P^T of the current tile (16 MFMAs,
// A = V^T from sV).  The 32 A operands are read from LDS as one stream kept
// prefetch_depth MFMAs ahead of their use, and the scheduler is told to keep
// that interleave, so the LDS latency is covered by the matrix core's own
// work.  Riding on the PV half: the four 16-byte chunks of the staged tile
// are stored to LDS (buffers sKs / sVs) and each register is refilled at once
// with the global load of the tile after it (key offset kload).
//
// Depth 4: the kernel's second load register set leaves no room for more
// (6 measured 0.5 % slower).
template <int NT>
constexpr int prefetch_depth() { return 4; }

template <int I>
__device__ __forceinline__ bf16x8 step_operand(const __bf16* sK, const __bf16* sV, int l32, int h, int lane) {
  if constexpr (I < 16) {
    constexpr int s = I >> 1, kb = I & 1;
    return *reinterpret_cast<const bf16x8*>(sK + (kb * 32 + l32) * KS + 16 * s + 8 * h);
  } else {
    constexpr int j = I - 16, s4 = j >> 2, db = j & 3;
    return v_operand(sV, s4, db, lane);
  }
}

template <int NT>
struct StepLoads {
  TileLoader<NT>& ld;
  __bf16* sk;
  __bf16* sv;
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t krow, vrow;
  int kload, tid;
};

// MFMAs [FIRST, LAST) of a step (0-15: QK^T, 16-31: PV).  With LOADS, the
// CH staged chunks are stored to LDS and each register refilled from HBM,
// spread evenly over the PV MFMAs.
template <int I, int FIRST, int LAST, bool LOADS, int NT>
__device__ __forceinline__ void step_body(f32x16 (&sacc)[2], f32x16 (&oacc)[4], const bf16x8 (&qf)[8],
                                          const uint32_t (&pk)[2][8], const __bf16* sK, const __bf16* sV,
                                          int l32, int h, int lane, bf16x8 (&fr)[prefetch_depth<NT>() + 1],
                                          const StepLoads<NT>& sl) {
  constexpr int PF = prefetch_depth<NT>();
  if constexpr (I < LAST) {
    if constexpr (I + PF < LAST)
      fr[(I + PF) % (PF + 1)] = step_operand<I + PF>(sK, sV, l32, h, lane);
    if constexpr (I < 16) {
      constexpr int s = I >> 1, kb = I & 1;
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[I % (PF + 1)], qf[s], sacc[kb], 0, 0, 0);
    } else {
      constexpr int j = I - 16, s4 = j >> 2, db = j & 3;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[I % (PF + 1)], p_operand(pk, s4),
                                                         oacc[db], 0, 0, 0);
      if constexpr (LOADS) {
        constexpr int CH = TileLoader<NT>::CH, every = 16 / CH;
        if constexpr (j % every == 0) {
          sl.ld.template store_one<j / every>(sl.sk, sl.sv, sl.tid);
          sl.ld.template load_one<j / every>(sl.rk, sl.rv, sl.krow, sl.vrow, sl.kload, sl.tid);
        }
      }
    }
    step_body<I + 1, FIRST, LAST, LOADS, NT>(sacc, oacc, qf, pk, sK, sV, l32, h, lane, fr, sl);
  }
}

template <int I, int LAST, bool LOADS, int CH, int PF>
__device__ __forceinline__ void step_schedule() {
  if constexpr (I < LAST) {
    if constexpr (I + PF < LAST)
      __builtin_amdgcn_sched_group_barrier(0x100, I + PF < 16 ? 1 : 2, 0);          // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                             // one MFMA
    if constexpr (LOADS && I >= 16 && ((I - 16) % (16 / CH)) == 0) {
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);                           // LDS store
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                           // global load
    }
    step_schedule<I + 1, LAST, LOADS, CH, PF>();
  }
}

// Operand reads of MFMAs [I, END) before the first MFMA of a range.
template <int I, int END, int PF>
__device__ __forceinline__ void prefetch_operands(bf16x8 (&fr)[PF + 1], const __bf16* sK, const __bf16* sV,
                                                  int l32, int h, int lane) {
  if constexpr (I < END) {
    fr[I % (PF + 1)] = step_operand<I>(sK, sV, l32, h, lane);
    prefetch_operands<I + 1, END, PF>(fr, sK, sV, l32, h, lane);
  }
}

template <int FIRST, int LAST, bool LOADS, int NT>
__device__ __forceinline__ void mfma_range(f32x16 (&sacc)[2], f32x16 (&oacc)[4], const bf16x8 (&qf)[8],
                                           const uint32_t (&pk)[2][8], const __bf16* sK, const __bf16* sV,
                                           int l32, int h, int lane, const StepLoads<NT>& sl) {
  constexpr int PF = prefetch_depth<NT>();
  static_assert(LAST - FIRST >= PF && (FIRST >= 16 || FIRST + PF <= 16), "prologue reads in one half");
  static_assert(16 % TileLoader<NT>::CH == 0, "staged chunks spread over the PV MFMAs");
  if constexpr (FIRST == 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
  }
  bf16x8 fr[PF + 1];
  prefetch_operands<FIRST, FIRST + PF, PF>(fr, sK, sV, l32, h, lane);
  step_body<FIRST, FIRST, LAST, LOADS, NT>(sacc, oacc, qf, pk, sK, sV, l32, h, lane, fr, sl);
  __builtin_amdgcn_sched_group_barrier(0x100, (FIRST < 16 ? 1 : 2) * PF, 0);
  step_schedule<FIRST, LAST, LOADS, TileLoader<NT>::CH, PF>();
}

__device__ __forceinline__ void mask_tail(f32x16 (&sacc)[2], int key0, int N, int h) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
      if (key >= N) sacc[kb][r] = -INFINITY;
    }
}

// Block-sparse kernel: a work-group of 4 waves owns one 128-row mask block
// (each wave 32 rows); two work-groups share a CU.  K and V of the kept key
// blocks pass through two LDS buffers.
template <bool OUT_F32>
__global__ __launch_bounds__(256, 2) void attn_sparse_kernel(AttnArgs a) {
  constexpr int NW = 4;
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  static_assert(BM == kBlock, "block-sparse work-groups cover one 128-row mask block");
  __shared__ __attribute__((aligned(16))) __bf16 smK[2][BN * KS];
  __shared__ __attribute__((aligned(16))) __bf16 smV[2][BN * VSR];

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

  const int q0 = qblk * BM + wave * 32;

  // Q as the B operand of S^T = K Q^T: lane (l32, h) holds row q0 + l32,
  // d = 16 s + 8 h .. +7 for step s.  Rows >= N load as zero.
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load_b128(rq, (uint32_t)(q0 + l32) * qrow + (16 * s + 8 * h) * 2));

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  RowState st = {-INFINITY, 0.f, 0.f};

  SparseTiles tiles;
  tiles.row = a.mask + (int64_t)bh * a.mask_bh + (int64_t)qblk * a.nb;
  tiles.nb = a.nb;
  tiles.N = N;
  tiles.chunk = -1;
  tiles.pend = -1;
  tiles.bits = 0;

  TileLoader<NT> ld;
  const int k0 = tiles.next();
  // ---- prologue: tile 0 into LDS, tiles 1 and 2 into two register sets ----
  // The kept blocks of a mask are scattered, so their loads miss L2 far more
  // often than the dense walk's; each tile's loads are issued two steps
  // before its LDS store, alternating between the two register sets.
  TileLoader<NT> ld2;
  int k1 = -1, k2 = -1;
  if (k0 >= 0) {
    ld.load(rk, rv, krow, vrow, k0, tid);
    ld.store(smK[0], smV[0], tid);
    k1 = tiles.next();
    ld.load(rk, rv, krow, vrow, k1 >= 0 ? k1 : N, tid);
    k2 = k1 >= 0 ? tiles.next() : -1;
    ld2.load(rk, rv, krow, vrow, k2 >= 0 ? k2 : N, tid);
  }
  __syncthreads();

  f32x16 sacc[2];
  uint32_t pk[2][8];
  int kc = k0, kn = k1, kn2 = k2, bc = 0;
  bool first = true;   // wave-uniform
  // One full tile: L holds tile kn, which goes to the other buffer, and L
  // then fetches the tile after kn2. The staged tile goes to the other
  // buffer even when there is none (that buffer is free), and loads past
  // the last tile fetch key offset N, which the buffer bounds turn into
  // zeros.
  auto full_step = [&](TileLoader<NT>& L) {
    const int kn3 = kn2 >= 0 ? tiles.next() : -1;
    const StepLoads<NT> sl = {L, smK[bc ^ 1], smV[bc ^ 1], rk, rv, krow, vrow, kn3 >= 0 ? kn3 : N, tid};
    mfma_range<0, 16, false, NT>(sacc, oacc, qf, pk, smK[bc], smV[bc], l32, h, lane, sl);
    softmax_next(sacc, st, oacc, pk, c, first);
    first = false;
    mfma_range<16, 32, true, NT>(sacc, oacc, qf, pk, smK[bc], smV[bc], l32, h, lane, sl);
    __syncthreads();
    kc = kn;
    kn = kn2;
    kn2 = kn3;
    bc ^= 1;
  };
  while (kc >= 0 && kc + BN <= N) {
    full_step(ld);
    if (!(kc >= 0 && kc + BN <= N)) break;
    full_step(ld2);
  }
  if (kc >= 0) {   // ragged last tile
    qk_tile(sacc, smK[bc], qf, l32, h);
    mask_tail(sacc, kc, N, h);
    softmax_next(sacc, st, oacc, pk, c, first);
    pv_tile(oacc, pk, smV[bc], lane);
  }

  // ---- epilogue ----
  const int64_t ob = b * a.os[0] + hd * a.os[1];
  const float lt = row_sum_halves(st.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int row = q0 + l32;
  if (row < N) {
    const int64_t orow = ob + (int64_t)row * a.os[2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + r4 * 8 + h * 4;
        const float v0 = oacc[db][4 * r4 + 0] * inv, v1 = oacc[db][4 * r4 + 1] * inv;
        const float v2 = oacc[db][4 * r4 + 2] * inv, v3 = oacc[db][4 * r4 + 3] * inv;
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
          lt > 0.f ? (st.mc + __builtin_log2f(lt)) * 0.69314718055994530942f : -INFINITY;
  }
}

// ---- dense kernel: 48 query rows per wave on the 16x16x32 MFMA ----
//
// Per 32-key tile and wave (lane = 16 g + l16):
//   S^T = K Q^T      A = K (16 keys x 32 d) from LDS, B = Q^T (32 d x 16 rows)
//                    in registers; the accumulator gives lane (g, l16) keys
//                    4 g + r of query row l16 of each 16-row block, and each
//                    K fragment feeds the three row blocks.
//   O^T += V^T P^T   A = V^T (16 d x 32 keys) by two transposing LDS reads
//                    (keys 4g..4g+3 and 16+4g..16+4g+3 for lane group g), B =
//                    P packed from the S registers in the same key order;
//                    each V operand feeds the three row blocks.
// A query row's keys are spread over the four lane groups, so its row max
// and sum take two exchanges (lanes l^16, then l^32).

constexpr int RBN = 32;                 // keys per tile
constexpr int RNB = 3;                  // LDS tile buffers
constexpr int RRB = 3;                  // 16-row blocks per wave
constexpr int RNW = 8;                  // waves per work-group
constexpr int RBM = RNW * 16 * RRB;     // 384 query rows per work-group
static_assert(RBM == kDenseRows && RBN == kDenseTileKeys, "the host plans with these sizes");
constexpr int RNT = RNW * 64;
// V tile row stride in bf16: 288 B (72 banks).  A transposing read covers
// rows 4g .. 4g+3 for each lane group g; with 72 r mod 64 = 8 r the rows of
// groups 0 and 1 (and of 2 and 3) use disjoint banks.  Measured: half the
// bank-conflict cycles of 64-bank strides of 68, 76, 80, 84 or 92 (88 ties).
constexpr int RVS = D + 16;

struct RLoader {
  // 32 keys x 16 chunks of 16 bytes, for K (I = 0) and V (I = 1).
  u32x4 r[2];
  template <int I>
  __device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t krow,
                                           uint32_t vrow, int key0, int N, int tid) {
    const int key = tid >> 4, c = tid & 15;
    const int row = min(key0 + key, N);
    r[I] = buf_load_b128(I == 0 ? rk : rv, (uint32_t)row * (I == 0 ? krow : vrow) + c * 16);
  }
  template <int I>
  __device__ __forceinline__ void store_one(__bf16* sk, __bf16* sv, int tid) const {
    const int key = tid >> 4, c = tid & 15;
    *reinterpret_cast<u32x4*>((I == 0 ? sk + key * KS : sv + key * RVS) + c * 8) = r[I];
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t krow,
                                       uint32_t vrow, int key0, int N, int tid) {
    load_one<0>(rk, rv, krow, vrow, key0, N, tid);
    load_one<1>(rk, rv, krow, vrow, key0, N, tid);
  }
  __device__ __forceinline__ void store(__bf16* sk, __bf16* sv, int tid) const {
    store_one<0>(sk, sv, tid);
    store_one<1>(sk, sv, tid);
  }
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A operand J of a step: J < 8 -> K fragment (ds, kb) = (J / 2, J % 2):
// rows 16 kb + l % 16, d 32 ds + 8 g .. +7.  J >= 8 -> V^T operand, d block
// db = J - 8: lane (g, s) reads rows 4g + s/4 (+16), columns 16 db + 4 (s%4).
__device__ __forceinline__ bf16x8 r_v_operand(const __bf16* sV, int db, int g, int s) {
  const __bf16* base = sV + (4 * g + (s >> 2)) * RVS + 16 * db + 4 * (s & 3);
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + 16 * RVS));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int J>
__device__ __forceinline__ bf16x8 r_operand(const __bf16* sK, const __bf16* sV, int l16, int g, int s) {
  if constexpr (J < 8) {
    return *reinterpret_cast<const bf16x8*>(sK + ((J & 1) * 16 + l16) * KS + 32 * (J >> 1) + 8 * g);
  } else {
    return r_v_operand(sV, J - 8, g, s);
  }
}

__device__ __forceinline__ bf16x8 r_p_operand(const uint32_t (&pk)[4]) {
  const u32x4 t = {pk[0], pk[1], pk[2], pk[3]};
  return __builtin_bit_cast(bf16x8, t);
}

constexpr int kRPre = 3;   // operand pairs read this many steps ahead (2-4 measured within 1 %)

// Operand pair I of a step (0..15), three MFMAs each (row blocks).  With
// staging, the K and V chunks of the staged tile are stored at I = 8 and 12
// and the registers refilled with the tile after it.
template <int I>
__device__ __forceinline__ void r_step(f32x4 (&sacc)[2][RRB], f32x4 (&oacc)[8][RRB], const bf16x8 (&qf)[RRB][4],
                                       const uint32_t (&pk)[RRB][4], const __bf16* sK, const __bf16* sV, int l16,
                                       int g, int s, bf16x8 (&fr)[kRPre + 1], RLoader& ld, __bf16* sks, __bf16* svs,
                                       __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t krow,
                                       uint32_t vrow, int kload, int N, int tid) {
  if constexpr (I < 16) {
    if constexpr (I + kRPre < 16) fr[(I + kRPre) % (kRPre + 1)] = r_operand<I + kRPre>(sK, sV, l16, g, s);
    const bf16x8 a = fr[I % (kRPre + 1)];
    if constexpr (I < 8) {
      constexpr int ds = I >> 1, kb = I & 1;
#pragma unroll
      for (int rb = 0; rb < RRB; ++rb) sacc[kb][rb] = mfma16(a, qf[rb][ds], sacc[kb][rb]);
    } else {
      constexpr int db = I - 8;
#pragma unroll
      for (int rb = 0; rb < RRB; ++rb) oacc[db][rb] = mfma16(a, r_p_operand(pk[rb]), oacc[db][rb]);
      if constexpr (I == 8) {
        ld.template store_one<0>(sks, svs, tid);
        ld.template load_one<0>(rk, rv, krow, vrow, kload, N, tid);
      }
      if constexpr (I == 12) {
        ld.template store_one<1>(sks, svs, tid);
        ld.template load_one<1>(rk, rv, krow, vrow, kload, N, tid);
      }
    }
    r_step<I + 1>(sacc, oacc, qf, pk, sK, sV, l16, g, s, fr, ld, sks, svs, rk, rv, krow, vrow, kload, N, tid);
  }
}

template <int I>
__device__ __forceinline__ void r_step_schedule() {
  if constexpr (I < 16) {
    if constexpr (I + kRPre < 16) __builtin_amdgcn_sched_group_barrier(0x100, I + kRPre < 8 ? 1 : 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, RRB, 0);
    if constexpr (I == 8 || I == 12) {
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    r_step_schedule<I + 1>();
  }
}

// Max over the 8 keys a lane holds of row block rb, then over the 4 lane
// groups sharing the query row (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float r_row_max(const f32x4 (&sacc)[2][RRB], int rb) {
  float m = fmaxf(fmaxf(fmaxf(sacc[0][rb][0], sacc[0][rb][1]), fmaxf(sacc[0][rb][2], sacc[0][rb][3])),
                  fmaxf(fmaxf(sacc[1][rb][0], sacc[1][rb][1]), fmaxf(sacc[1][rb][2], sacc[1][rb][3])));
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  return max_halves(m);
}
__device__ __forceinline__ float r_row_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + swap_halves(x);
}

__device__ __forceinline__ void r_rescale(float t, RowState& st, f32x4 (&oacc)[8][RRB], int rb, float c) {
  const bool grow = (t - st.m) * c > kLazy;
  if (__any(grow)) {
    const float mnew = fmaxf(st.m, t);
    const float alpha = fast_exp2((st.m - mnew) * c);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[db][rb][r] *= alpha;
    st.m = mnew;
    st.mc = mnew * c;
  }
}

// P for row block rb: 2^(S c - mc) rounded to bf16 pairs in the B-operand
// order (keys 4g..4g+3, then 16+4g..16+4g+3); returns the lane's sum of the
// rounded P.
__device__ __forceinline__ float r_exp_block(const f32x4 (&sacc)[2][RRB], int rb, float mc, float c,
                                             uint32_t (&pk)[4]) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(sacc[i >> 2][rb][i & 3], c, -mc);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = fast_exp2(x[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
  float ls0 = sum_bf16x2(pk[0], 0.f), ls1 = sum_bf16x2(pk[1], 0.f);
  ls0 = sum_bf16x2(pk[2], ls0);
  ls1 = sum_bf16x2(pk[3], ls1);
  return ls0 + ls1;
}

__device__ __forceinline__ void r_mask(f32x4 (&sacc)[2][RRB], int key0, int N, int g) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + kb * 16 + 4 * g + r;
      if (key >= N) {
#pragma unroll
        for (int rb = 0; rb < RRB; ++rb) sacc[kb][rb][r] = -INFINITY;
      }
    }
}

// Softmax of one tile for the three row blocks (first: take the tile max as
// the reference first; later tiles keep the reference unless a lane's
// weights pass 2^64).
__device__ __forceinline__ void r_softmax(f32x4 (&sacc)[2][RRB], RowState (&st)[RRB], f32x4 (&oacc)[8][RRB],
                                          uint32_t (&pk)[RRB][4], float c, bool first) {
#pragma unroll
  for (int rb = 0; rb < RRB; ++rb) {
    float ls = 0.f;
    if (!first) ls = r_exp_block(sacc, rb, st[rb].mc, c, pk[rb]);
    if (first || __any(!(ls <= kCheck))) {
      r_rescale(r_row_max(sacc, rb), st[rb], oacc, rb, c);
      ls = r_exp_block(sacc, rb, st[rb].mc, c, pk[rb]);
    }
    st[rb].l += ls;
  }
}

__device__ __forceinline__ void r_qk_tile(f32x4 (&sacc)[2][RRB], const __bf16* sK, const bf16x8 (&qf)[RRB][4],
                                          int l16, int g) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int rb = 0; rb < RRB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[kb][rb][r] = 0.f;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (kb * 16 + l16) * KS + 32 * ds + 8 * g);
#pragma unroll
      for (int rb = 0; rb < RRB; ++rb) sacc[kb][rb] = mfma16(kf, qf[rb][ds], sacc[kb][rb]);
    }
}


// Dense kernel.  A work-group of 8 waves owns 384 query rows of one (b, h);
// a tail work-group (with a caller workspace) gets one of the `split` key
// ranges of its block and stores a partial result instead of O.
template <int I, int END>
__device__ __forceinline__ void r_prefetch(bf16x8 (&fr)[kRPre + 1], const __bf16* sK, const __bf16* sV, int l16,
                                          int g, int s) {
  if constexpr (I < END) {
    fr[I % (kRPre + 1)] = r_operand<I>(sK, sV, l16, g, s);
    r_prefetch<I + 1, END>(fr, sK, sV, l16, g, s);
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(RNT, 2) void attn_dense_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 smK[RNB][RBN * KS];
  __shared__ __attribute__((aligned(16))) __bf16 smV[RNB][RBN * RVS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4, s = lane & 15;
  int tile, part = -1;
  if ((int)blockIdx.x < a.nfull) {
    tile = xcd_remap(blockIdx.x, a.nfull);
  } else {
    const int j = blockIdx.x - a.nfull;
    tile = a.nfull + j / a.split;
    part = j % a.split;
  }
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

  // Q as the B operand: lane (g, l16) holds row q0 + 16 rb + l16, d = 32 ds
  // + 8 g .. +7.  Rows >= N load as zero (row N is past the buffer).
  const int q0 = qblk * RBM + wave * (16 * RRB);
  bf16x8 qf[RRB][4];
#pragma unroll
  for (int rb = 0; rb < RRB; ++rb)
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const int row = min(q0 + 16 * rb + l16, N);
      qf[rb][ds] = __builtin_bit_cast(bf16x8, buf_load_b128(rq, (uint32_t)row * qrow + (32 * ds + 8 * g) * 2));
    }

  f32x4 oacc[8][RRB];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rb = 0; rb < RRB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[db][rb][r] = 0.f;
  RowState st[RRB];
#pragma unroll
  for (int rb = 0; rb < RRB; ++rb) st[rb] = {-INFINITY, 0.f, 0.f};

  // Key tiles [t0, t1) of T; part p of `split` takes t = p T / split ..
  // (p + 1) T / split (never empty: split <= T).
  const int T = (N + RBN - 1) / RBN;
  int t0 = 0, t1 = T;
  if (part >= 0) {
    t0 = part * T / a.split;
    t1 = (part + 1) * T / a.split;
  }

  // ---- prologue: tiles t0 and t0+1 into LDS, t0+2 into registers (loads
  // past N read as zero; tiles past t1 are never used) ----
  RLoader ld;
  ld.load(rk, rv, krow, vrow, t0 * RBN, N, tid);
  ld.store(smK[0], smV[0], tid);
  ld.load(rk, rv, krow, vrow, (t0 + 1) * RBN, N, tid);
  ld.store(smK[1], smV[1], tid);
  ld.load(rk, rv, krow, vrow, (t0 + 2) * RBN, N, tid);
  __syncthreads();

  f32x4 sacc[2][RRB];
  uint32_t pk[RRB][4];
  r_qk_tile(sacc, smK[0], qf, l16, g);
  if ((t0 + 1) * RBN > N) r_mask(sacc, t0 * RBN, N, g);
  r_softmax(sacc, st, oacc, pk, c, true);

  // ---- step t: QK^T of tile t+1 and PV of tile t, barrier, softmax of t+1 ----
  int bc = 0;
  for (int t = t0; t + 1 < t1; ++t) {
    const int bn = (bc + 1 == RNB) ? 0 : bc + 1;
    const int bn2 = (bn + 1 == RNB) ? 0 : bn + 1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < RRB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[kb][rb][r] = 0.f;
    bf16x8 fr[kRPre + 1];
    r_prefetch<0, kRPre>(fr, smK[bn], smV[bc], l16, g, s);
    r_step<0>(sacc, oacc, qf, pk, smK[bn], smV[bc], l16, g, s, fr, ld, smK[bn2], smV[bn2], rk, rv, krow, vrow,
              (t + 3) * RBN, N, tid);
    __builtin_amdgcn_sched_group_barrier(0x100, kRPre, 0);
    r_step_schedule<0>();
    __syncthreads();
    const int key1 = (t + 1) * RBN;
    if (key1 + RBN > N) r_mask(sacc, key1, N, g);
    r_softmax(sacc, st, oacc, pk, c, false);
    bc = bn;
  }
  // ---- drain: PV of the last tile ----
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const bf16x8 vf = r_v_operand(smV[bc], db, g, s);
#pragma unroll
    for (int rb = 0; rb < RRB; ++rb) oacc[db][rb] = mfma16(vf, r_p_operand(pk[rb]), oacc[db][rb]);
  }

  // ---- epilogue: lane (g, l16) holds d = 16 db + 4 g + r of row q0 + 16 rb + l16 ----
  const int64_t ob = b * a.os[0] + hd * a.os[1];
#pragma unroll
  for (int rb = 0; rb < RRB; ++rb) {
    const float lt = r_row_sum(st[rb].l);
    const int row = q0 + 16 * rb + l16;
    if (row >= N) continue;
    if (part >= 0) {
      // Partial result of one key range: unnormalised O, m c and l.
      float* pr = a.part + ((int64_t)(blockIdx.x - a.nfull) * RBM + wave * (16 * RRB) + 16 * rb + l16) * kPartRow;
#pragma unroll
      for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(pr + 16 * db + 4 * g) = oacc[db][rb];
      if (g == 0) {
        pr[128] = st[rb].mc;
        pr[129] = lt;
      }
      continue;
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t orow = ob + (int64_t)row * a.os[2];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d0 = 16 * db + 4 * g;
      const float v0 = oacc[db][rb][0] * inv, v1 = oacc[db][rb][1] * inv;
      const float v2 = oacc[db][rb][2] * inv, v3 = oacc[db][rb][3] * inv;
      if constexpr (OUT_F32) {
        const f32x4 t4 = {v0, v1, v2, v3};
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d0) = t4;
      } else {
        const u32x2 t2 = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.o) + orow + d0) = t2;
      }
    }
    if (a.lse != nullptr && g == 0)
      a.lse[(int64_t)bh * N + row] =
          lt > 0.f ? (st[rb].mc + __builtin_log2f(lt)) * 0.69314718055994530942f : -INFINITY;
  }
}

// Combine the partial results of the split tail blocks, one wave per row:
// M = max_p m_p, w_p = 2^(m_p - M), O = sum_p w_p O_p / sum_p w_p l_p,
// lse = ln2 (M + log2 l + lse_off), the parts taken in key order (m in log2
// units; the fp8 kernel's weights are in units of 1/448, lse_off = -log2 448).
template <bool OUT_F32>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int rid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tail = rid / a.bm, rr = rid % a.bm;
  const int tile = a.nfull + tail;
  const int bh = tile / a.nqb, qblk = tile % a.nqb;
  const int b = bh / a.H, hd = bh % a.H;
  const int row = qblk * a.bm + rr;
  if (row >= a.N) return;
  const float* base = a.part + ((int64_t)tail * a.split * a.bm + rr) * kPartRow;
  const int64_t pstride = (int64_t)a.bm * kPartRow;
  float M = -INFINITY;
  for (int p = 0; p < a.split; ++p) M = fmaxf(M, base[p * pstride + 128]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int p = 0; p < a.split; ++p) {
    const float* pr = base + p * pstride;
    const float w = fast_exp2(pr[128] - M);
    L = __builtin_fmaf(w, pr[129], L);
    const f32x2 ov = *reinterpret_cast<const f32x2*>(pr + 2 * lane);
    o0 = __builtin_fmaf(w, ov[0], o0);
    o1 = __builtin_fmaf(w, ov[1], o1);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t orow = b * a.os[0] + hd * a.os[1] + (int64_t)row * a.os[2] + 2 * lane;
  if constexpr (OUT_F32) {
    const f32x2 t = {o0 * inv, o1 * inv};
    *reinterpret_cast<f32x2*>(static_cast<float*>(a.o) + orow) = t;
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<__bf16*>(a.o) + orow) = pack_bf16x2(o0 * inv, o1 * inv);
  }
  if (a.lse != nullptr && lane == 0)
    a.lse[(int64_t)bh * a.N + row] = L > 0.f ? (M + __builtin_log2f(L) + a.lse_off) * 0.69314718055994530942f
                                           : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(const AttnArgs& a, bool out_f32, hipStream_t s) {
  if (a.split <= 1 || a.ntail <= 0) return hipSuccess;
  const dim3 grid((unsigned)(a.ntail * a.bm / 4));   // one wave per row, 4 waves per work-group
  if (out_f32) hipLaunchKernelGGL((attn_merge_kernel<true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((attn_merge_kernel<false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& args, bool out_f32, bool sparse, hipStream_t s) {
  AttnArgs a = args;
  if (sparse) {
    a.nqb = a.nb;   // one work-group per 128-row mask block
    const int64_t nwg = (int64_t)a.B * a.H * a.nqb;
    if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (out_f32) hipLaunchKernelGGL((attn_sparse_kernel<true>), dim3((unsigned)nwg), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_sparse_kernel<false>), dim3((unsigned)nwg), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  a.nqb = (a.N + kDenseRows - 1) / kDenseRows;
  a.bm = kDenseRows;
  int64_t nwg = (int64_t)a.B * a.H * a.nqb;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.split <= 1 || a.part == nullptr) {
    a.nfull = (int)nwg;
    a.ntail = 0;
    a.split = 1;
  } else {
    if (a.nfull + a.ntail != nwg) return hipErrorInvalidConfiguration;
    nwg = (int64_t)a.nfull + (int64_t)a.ntail * a.split;
  }
  const dim3 grid((unsigned)nwg);
  if (out_f32) hipLaunchKernelGGL((attn_dense_kernel<true>), grid, dim3(RNT), 0, s, a);
  else hipLaunchKernelGGL((attn_dense_kernel<false>), grid, dim3(RNT), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_merge(a, out_f32, s);
}

}  // namespace dit
