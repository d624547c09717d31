// attn_bf16.hip -- bf16 flash-style joint attention forward for gfx950.
//
// Both kernels follow one recipe per key tile (fp32 accumulate):
//   S^T = K Q^T      A = K rows from LDS, B = Q held in registers for the
//                    whole kernel.
//   online softmax   P = 2^(S c - m c) with c = scale * log2(e) and m a
//                    running reference: the row max of the first tile.  Later
//                    tiles take their exponentials against it directly: P
//                    far above 1 is harmless in fp32 (l and O keep their
//                    relative precision), and the reference is moved to a
//                    new max (O and l rescaled, the work redone) only when
//                    the weights grow past a bound -- per tile (2^64, the
//                    block-sparse kernel) or per row at the end (2^80, the
//                    dense kernel).  The factor cancels in O / l.
//   O^T += V^T P^T   A = V^T, read from the row-major V tile with the gfx950
//                    transposing LDS read (ds_read_b64_tr_b16: 16 lanes
//                    fetch a 4-key x 16-d block and each lane receives one d
//                    column of it), B = P straight from the S registers
//                    rounded to bf16 -- no shuffle: the PV reduction index is
//                    permuted instead, by choosing which 4 keys each
//                    transposing read fetches to match the order in which
//                    the accumulator hands P out.  l accumulates the same
//                    rounded P: v_dot2 with (1, 1) in the block-sparse
//                    kernel, one extra MFMA per 32-key tile and row block
//                    with an all-ones A operand in the dense kernel (every
//                    row of its result is the column sum of P^T).
// Epilogue: O = O^T / l, stored bf16 (round to nearest even) or fp32, and
// optionally lse = ln2 * (m c + log2 l).
//
// Dense kernel (attn_dense_kernel): 8 waves x 48 query rows = 384 rows of
// one (batch, head) per work-group, two waves per SIMD.  Each wave's rows are
// three 16-row blocks on the 16x16x32 bf16 MFMA, so every K fragment and V
// operand read from LDS feeds three MFMAs (a third less LDS traffic per flop
// than 32-row waves).  K and V stream through LDS in 32-key tiles in four
// rotating buffers, loaded straight from global memory into LDS.  Step t
// issues the QK^T MFMAs of tile t+1 and the PV MFMAs of tile t as one stream
// with their LDS operands read ahead, and the loads of tile t+3 beside its
// first MFMAs; then the softmax of tile t+1.  Waves 4-7 run half a step behind waves 0-3
// (two barriers per step), so on each SIMD one wave's MFMA stream runs while
// the other wave does its softmax.
//
// Tail split (dense, with a caller workspace): one 384-row work-group runs
// per compute unit at a time, so the query blocks of a last, partial round
// would leave most units idle.  Each of those blocks is instead split into
// `split` consecutive key ranges run by separate work-groups (launched after
// the full blocks); each range stores its unnormalised O, reference m c and
// weight sum l, and attn_merge_kernel combines them in key order with the
// exact rescaling 2^(m_p c - max m c).
//
// Block-sparse kernel (attn_sparse_kernel): 4 waves x 32 rows (two 16-row
// blocks each) = one 128-row mask block per work-group, two work-groups per
// CU; the 32-key tiles of the kept 128-key blocks of its mask row (masked
// blocks are never loaded) go through the dense kernel's pipeline.

#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace dit {
namespace {

constexpr int D = kHeadDim;
// K tile row stride in bf16: 272 B.  The QK^T operand reads (lane (g, l16)
// takes 16 bytes of row l16 at chunk 4 ds + g) cost 4 LDS bank-conflict
// cycles each at this stride (SQ_LDS_BANK_CONFLICT), none at 288 or 352 B or
// with 256-byte rows whose 16-byte chunks are XOR-ed with the row; but with
// those layouts the dense kernel measured 6-10 % slower (its matrix cores
// idled more), so the padded 272-byte rows stay.
constexpr int KS = D + 8;
// When the reference max is recomputed (first tile, or a redo after a huge
// jump), it only moves if some row of the wave grew by more than 2^kLazy.
constexpr float kLazy = 8.f;

struct RowState {
  float m;    // reference the weights are taken against (a raw dot product)
  float mc;   // m * c (0 until the first tile sets it)
};

// The kernels check each row's whole weight sum once, at the end.
constexpr float kEndCheck = 0x1p80f;

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
constexpr int RNB = 4;                  // LDS tile buffers
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

// Direct global -> LDS staging of one 32-key tile (buffer_load ... lds): a
// tile buffer holds the 32 K rows at the 272-byte stride and the 32 V rows
// at 288 bytes, each in a region of 576 16-byte slots, then a 1 KB junk
// area.  One such instruction writes 64 consecutive slots (lane i -> slot
// i), so a region takes 9 instructions and a tile 18.  They are dealt to the
// waves round-robin (instruction i to wave i % NW); the PER * NW - 18 left
// over load into the junk area, so that every wave issues exactly PER per
// tile.  A slot in a row's padding or past the 32 K rows gets some chunk of
// row 31 of the tile: those slots are never read.  Rows at or past N lie
// beyond the buffer resource and load zeros.
constexpr int kRegion = 576 * 8;               // bf16 per tensor region (9216 B)
constexpr int kTileBuf = 2 * kRegion + 512;    // bf16 per tile buffer: K, V, junk

template <int NW>
struct TileDma {
  static constexpr int NI = 18;
  static constexpr int PER = (NI + NW - 1) / NW;
  uint32_t off[PER];    // this lane's byte offset inside the tile, per instruction
  i32x4 rsrc[PER];      // buffer resource (K or V slice), wave-uniform
  uint32_t dst[PER];    // LDS byte offset inside a tile buffer, wave-uniform
  uint32_t srow[PER];   // row stride in bytes of that tensor, wave-uniform
  __device__ __forceinline__ void init(int wave, int lane, const void* kp, uint32_t kbytes, uint32_t krow,
                                       const void* vp, uint32_t vbytes, uint32_t vrow) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = wave + j * NW;
      const bool isv = i >= NI / 2;
      const int slot = 64 * (isv ? i - NI / 2 : i) + lane;
      const int per_row = isv ? RVS / 8 : KS / 8;   // 18 or 17 slots
      const int row = min(slot / per_row, RBN - 1), c = min(slot % per_row, 15);
      const uint32_t rstride = isv ? vrow : krow;
      off[j] = (uint32_t)row * rstride + 16u * (uint32_t)c;
      const uint64_t base = reinterpret_cast<uint64_t>(isv ? vp : kp);
      rsrc[j] = i32x4{(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xffffu), (int)(isv ? vbytes : kbytes),
                      0x00020000};
      dst[j] = i >= NI ? 2u * 2u * kRegion : 2u * (uint32_t)(isv ? kRegion + 512 * (i - NI / 2) : 512 * i);
      srow[j] = rstride;
    }
  }
  // Instruction J of this wave for the tile whose first key row is `key0`,
  // into the tile buffer at LDS byte address `buf`.  Issued from inline
  // assembly: the compiler would otherwise order every later LDS read of
  // the work-group after it (it cannot tell the buffers apart).  The only
  // register it reads is the address, at issue; completion is awaited by
  // dma_barrier / dma_wait_all.
  template <int J>
  __device__ __forceinline__ void issue(uint32_t buf, uint32_t key0) const {
    const uint32_t voff = off[J] + key0 * srow[J];
    // The LDS address goes in through M0 as an operand, so the compiler
    // writes M0 itself and knows it was changed.
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc[J]), "{m0}"(buf + dst[J])
                 : "memory");
  }
  template <int J = 0>
  __device__ __forceinline__ void issue_all(uint32_t buf, uint32_t key0) const {
    if constexpr (J < PER) {
      issue<J>(buf, key0);
      issue_all<J + 1>(buf, key0);
    }
  }
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}

// The barrier after a step's MFMA stream.  Each wave first waits until at
// most its PER newest staging loads (the tile it issued in this step) are in
// flight: the tile issued in the step before, which the next step reads, is
// then in LDS for every wave.  The compiler does not order these loads
// against the barrier by itself, hence the explicit wait.
template <int PER>
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(PER) : "memory");
}
__device__ __forceinline__ void dma_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// Operand pair I of a step (0..15), NRB MFMAs each (row blocks), plus the
// NRB row-sum MFMAs at I = 8.  The wave's PER staging loads of the tile
// three ahead go out at I = 1, 3, 5, ...

template <int I, int NT, int NRB>
__device__ __forceinline__ void r_step(f32x4 (&sacc)[2][NRB], f32x4 (&oacc)[8][NRB], f32x4 (&lacc)[NRB],
                                       const bf16x8& ones, const bf16x8 (&qf)[NRB][4],
                                       const uint32_t (&pk)[NRB][4], const __bf16* sK, const __bf16* sV, int l16,
                                       int g, int s, bf16x8 (&fr)[kRPre + 1], const TileDma<NT / 64>& dma,
                                       uint32_t dbuf, uint32_t dkey) {
  if constexpr (I < 16) {
    if constexpr (I + kRPre < 16) fr[(I + kRPre) % (kRPre + 1)] = r_operand<I + kRPre>(sK, sV, l16, g, s);
    const bf16x8 a = fr[I % (kRPre + 1)];
    if constexpr (I < 8) {
      constexpr int ds = I >> 1, kb = I & 1;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) sacc[kb][rb] = mfma16(a, qf[rb][ds], sacc[kb][rb]);
    } else {
      constexpr int db = I - 8;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) oacc[db][rb] = mfma16(a, r_p_operand(pk[rb]), oacc[db][rb]);
      if constexpr (I == 8) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) lacc[rb] = mfma16(ones, r_p_operand(pk[rb]), lacc[rb]);
      }
    }
    if constexpr ((I & 1) == 1 && (I >> 1) < TileDma<NT / 64>::PER)
      dma.template issue<(I >> 1)>(dbuf, dkey);
    r_step<I + 1, NT, NRB>(sacc, oacc, lacc, ones, qf, pk, sK, sV, l16, g, s, fr, dma, dbuf, dkey);
  }
}

template <int I, int NT, int NRB>
__device__ __forceinline__ void r_step_schedule() {
  if constexpr (I < 16) {
    if constexpr (I + kRPre < 16) __builtin_amdgcn_sched_group_barrier(0x100, I + kRPre < 8 ? 1 : 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, I == 8 ? 2 * NRB : NRB, 0);
    if constexpr ((I & 1) == 1 && (I >> 1) < TileDma<NT / 64>::PER) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    r_step_schedule<I + 1, NT, NRB>();
  }
}

// Max over the 8 keys a lane holds of row block rb, then over the 4 lane
// groups sharing the query row (lanes l, l^16, l^32, l^48).
template <int NRB>
__device__ __forceinline__ float r_row_max(const f32x4 (&sacc)[2][NRB], int rb) {
  float m = fmaxf(fmaxf(fmaxf(sacc[0][rb][0], sacc[0][rb][1]), fmaxf(sacc[0][rb][2], sacc[0][rb][3])),
                  fmaxf(fmaxf(sacc[1][rb][0], sacc[1][rb][1]), fmaxf(sacc[1][rb][2], sacc[1][rb][3])));
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  return max_halves(m);
}

template <int NRB>
__device__ __forceinline__ void r_rescale(float t, RowState& st, f32x4 (&oacc)[8][NRB], f32x4 (&lacc)[NRB], int rb,
                                          float c) {
  const bool grow = (t - st.m) * c > kLazy;
  if (__any(grow)) {
    const float mnew = fmaxf(st.m, t);
    const float alpha = fast_exp2((st.m - mnew) * c);
#pragma unroll
    for (int r = 0; r < 4; ++r) lacc[rb][r] *= alpha;
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
template <int NRB>
__device__ __forceinline__ void r_exp_block(const f32x4 (&sacc)[2][NRB], int rb, float mc, float c,
                                            uint32_t (&pk)[4]) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(sacc[i >> 2][rb][i & 3], c, -mc);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = fast_exp2(x[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
}

template <int NRB>
__device__ __forceinline__ void r_mask(f32x4 (&sacc)[2][NRB], int key0, int N, int g) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + kb * 16 + 4 * g + r;
      if (key >= N) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) sacc[kb][rb][r] = -INFINITY;
      }
    }
}

// Softmax of one tile for the three row blocks (first: take the tile max as
// the reference first; later tiles keep the reference unless a lane's
// weights pass 2^64).
template <int NRB>
__device__ __forceinline__ void r_softmax(f32x4 (&sacc)[2][NRB], RowState (&st)[NRB], f32x4 (&oacc)[8][NRB],
                                          f32x4 (&lacc)[NRB], uint32_t (&pk)[NRB][4], float c, bool exact) {
  if (exact) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) r_rescale(r_row_max(sacc, rb), st[rb], oacc, lacc, rb, c);
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) r_exp_block(sacc, rb, st[rb].mc, c, pk[rb]);
}

template <int NRB>
__device__ __forceinline__ void r_qk_tile(f32x4 (&sacc)[2][NRB], const __bf16* sK, const bf16x8 (&qf)[NRB][4],
                                          int l16, int g) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[kb][rb][r] = 0.f;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (kb * 16 + l16) * KS + 32 * ds + 8 * g);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) sacc[kb][rb] = mfma16(kf, qf[rb][ds], sacc[kb][rb]);
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
  __shared__ __attribute__((aligned(16))) __bf16 smT[RNB][kTileBuf];

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

  // Key tiles [t0, t1) of T; part p of `split` takes t = p T / split ..
  // (p + 1) T / split (never empty: split <= T).
  const int T = (N + RBN - 1) / RBN;
  int t0 = 0, t1 = T;
  if (part >= 0) {
    t0 = part * T / a.split;
    t1 = (part + 1) * T / a.split;
  }
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  TileDma<RNW> dma;
  dma.init(__builtin_amdgcn_readfirstlane(wave), lane, kp, a.k_bytes, krow, vp, a.v_bytes, vrow);
  constexpr int PER = TileDma<RNW>::PER;

  f32x4 oacc[8][RRB];
  f32x4 lacc[RRB];   // row sums of the rounded P (every element of a row block's C holds its row's sum)
  RowState st[RRB];
  int bc = 0;
  // Pass 0 takes every tile after the first against the first tile's row max
  // (no per-tile max, no per-tile check).  Weights far above 1 are harmless
  // in fp32 as long as nothing overflows: if some row's weight sum ends at
  // most 2^80, every weight was at most 2^80 and the row's unnormalised O is
  // at most 2^80 max|V| (finite for |V| below 2.8e14), and the result is
  // kept.  Otherwise (the reference lagged the row max by more than about
  // 80 bits somewhere, or a weight overflowed) the work-group runs its key
  // range again (EXACT pass) with the row max taken on every tile, so that
  // no weight exceeds 2^8.  Two copies of the loop, so that the common one
  // carries no per-tile max code.
  auto run_pass = [&](auto exact_tag) {
    constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int rb = 0; rb < RRB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][rb][r] = 0.f;
#pragma unroll
    for (int rb = 0; rb < RRB; ++rb) {
      st[rb] = {-INFINITY, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) lacc[rb][r] = 0.f;
    }

    // ---- prologue: tiles t0 .. t0+2 into LDS buffers 0 .. 2 ----
#pragma unroll
    for (int j = 0; j < 3; ++j) dma.issue_all(lds_addr(smT[j]), (uint32_t)((t0 + j) * RBN));
    dma_wait_all();
    __syncthreads();

    f32x4 sacc[2][RRB];
    uint32_t pk[RRB][4];
    r_qk_tile(sacc, smT[0], qf, l16, g);
    if ((t0 + 1) * RBN > N) r_mask(sacc, t0 * RBN, N, g);
    r_softmax(sacc, st, oacc, lacc, pk, c, true);

    if (grp == 1) __syncthreads();
    bc = 0;
    for (int t = t0; t + 1 < t1; ++t) {
      const int bn = (bc + 1) & (RNB - 1);
      const int b3 = (bc + 3) & (RNB - 1);
      const uint32_t kload = (uint32_t)((t + 3) * RBN);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rb = 0; rb < RRB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[kb][rb][r] = 0.f;
      bf16x8 fr[kRPre + 1];
      r_prefetch<0, kRPre>(fr, smT[bn], smT[bc] + kRegion, l16, g, s);
      r_step<0, RNT, RRB>(sacc, oacc, lacc, ones, qf, pk, smT[bn], smT[bc] + kRegion, l16, g, s, fr, dma,
                          lds_addr(smT[b3]), kload);
      __builtin_amdgcn_sched_group_barrier(0x100, kRPre, 0);
      r_step_schedule<0, RNT, RRB>();
      dma_barrier<PER>();
      const int key1 = (t + 1) * RBN;
      if (key1 + RBN > N) r_mask(sacc, key1, N, g);
      r_softmax(sacc, st, oacc, lacc, pk, c, EXACT);
      plain_barrier();
      bc = bn;
    }
    dma_wait_all();
    if (grp == 0) __syncthreads();
    // ---- drain: PV of the last tile ----
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 vf = r_v_operand(smT[bc] + kRegion, db, g, s);
#pragma unroll
      for (int rb = 0; rb < RRB; ++rb) oacc[db][rb] = mfma16(vf, r_p_operand(pk[rb]), oacc[db][rb]);
    }
#pragma unroll
    for (int rb = 0; rb < RRB; ++rb) lacc[rb] = mfma16(ones, r_p_operand(pk[rb]), lacc[rb]);
  };
  run_pass(std::false_type{});
  bool ok = true;
#pragma unroll
  for (int rb = 0; rb < RRB; ++rb) ok = ok && (lacc[rb][0] <= kEndCheck);
  if (__syncthreads_or(!ok)) run_pass(std::true_type{});

  // ---- epilogue: lane (g, l16) holds d = 16 db + 4 g + r of row q0 + 16 rb + l16 ----
  const int64_t ob = b * a.os[0] + hd * a.os[1];
#pragma unroll
  for (int rb = 0; rb < RRB; ++rb) {
    const float lt = lacc[rb][0];
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

// ---- block-sparse kernel: the dense pipeline on the kept key blocks ----
//
// One 128-row mask block per work-group: 4 waves x 32 rows (two 16-row
// blocks each, on the 16x16x32 MFMA), two work-groups per CU.  The key
// tiles are the 32-key tiles of the row's kept 128-key blocks, in order
// (masked blocks are never loaded); they flow through the dense kernel's
// pipeline: four LDS buffers, step t = QK^T of tile t+1 and PV of tile t
// with tile t+3 loaded into LDS beside them, a barrier, then the softmax of
// tile t+1; row sums on the matrix core; the
// lazy reference with the end-of-row 2^80 check and an exact second pass.

// Key offsets of the successive 32-key tiles of the kept 128-key blocks of
// one mask row; the row is scanned 64 entries at a time with a ballot, so
// every value here is wave-uniform.  -1 when the row is exhausted.  The
// first 32 chunks' entries are read at init (bit c of `pre`: this lane's
// entry of chunk c is kept): a mask read inside the key loop would wait for
// every outstanding load of the wave, the tile staging loads included.
struct SparseTileQueue {
  const uint8_t* row;
  int nb, N, chunk, blk, sub;
  uint64_t bits;
  uint32_t pre;
  static constexpr int kPreChunks = 32;
  __device__ __forceinline__ void init(const uint8_t* r, int nb_, int N_) {
    row = r;
    nb = nb_;
    N = N_;
    chunk = -1;
    blk = -1;
    sub = 0;
    bits = 0;
    pre = 0;
    const int lane = (int)(threadIdx.x & 63);
    // four chunks per round, their loads issued together (index clamped to
    // the row), one wait per round
    for (int c0 = 0; c0 < kPreChunks && c0 * 64 < nb; c0 += 4) {
      uint32_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = row[min((c0 + u) * 64 + lane, nb - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pre |= ((c0 + u) * 64 + lane < nb && v[u] != 0) ? (1u << (c0 + u)) : 0u;
    }
  }
  __device__ __forceinline__ int next() {
    if (blk >= 0) {
      ++sub;
      const int k = blk * kBlock + sub * RBN;
      if (sub < kBlock / RBN && k < N) return k;
    }
    while (bits == 0) {
      ++chunk;
      if (chunk * 64 >= nb) {
        blk = -1;
        return -1;
      }
      if (chunk < kPreChunks) {
        bits = __ballot(((pre >> chunk) & 1u) != 0);
      } else {
        const int j = chunk * 64 + (int)(threadIdx.x & 63);
        const int keep = (j < nb) ? (int)row[j] : 0;
        bits = __ballot(keep != 0);
      }
    }
    const int b = __builtin_ctzll(bits);
    bits &= bits - 1;
    blk = chunk * 64 + b;
    sub = 0;
    return blk * kBlock;
  }
};

constexpr int SNW = 4;                  // waves per block-sparse work-group
constexpr int SRB = 2;                  // 16-row blocks per wave
constexpr int SNT = SNW * 64;
static_assert(SNW * 16 * SRB == kBlock, "a block-sparse work-group covers one 128-row mask block");

template <bool OUT_F32>
__global__ __launch_bounds__(SNT, 2) void attn_sparse_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 smT[RNB][kTileBuf];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4, s = lane & 15;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / a.nqb, qblk = tile % a.nqb;
  const int b = bh / a.H, hd = bh % a.H;
  const int N = a.N;
  const float c = a.c;

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.qs[0] + hd * a.qs[1];
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.ks[0] + hd * a.ks[1];
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.vs[0] + hd * a.vs[1];
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qp, a.q_bytes);
  const uint32_t qrow = (uint32_t)(a.qs[2] * 2), krow = (uint32_t)(a.ks[2] * 2),
                 vrow = (uint32_t)(a.vs[2] * 2);
  const uint8_t* mrow = a.mask + (int64_t)bh * a.mask_bh + (int64_t)qblk * a.nb;

  const int q0 = qblk * kBlock + wave * (16 * SRB);
  bf16x8 qf[SRB][4];
#pragma unroll
  for (int rb = 0; rb < SRB; ++rb)
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const int row = min(q0 + 16 * rb + l16, N);
      qf[rb][ds] = __builtin_bit_cast(bf16x8, buf_load_b128(rq, (uint32_t)row * qrow + (32 * ds + 8 * g) * 2));
    }
  const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  TileDma<SNW> dma;
  dma.init(__builtin_amdgcn_readfirstlane(wave), lane, kp, a.k_bytes, krow, vp, a.v_bytes, vrow);
  constexpr int PER = TileDma<SNW>::PER;

  f32x4 oacc[8][SRB];
  f32x4 lacc[SRB];
  RowState st[SRB];
  auto run_pass = [&](auto exact_tag) {
    constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int rb = 0; rb < SRB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][rb][r] = 0.f;
#pragma unroll
    for (int rb = 0; rb < SRB; ++rb) {
      st[rb] = {-INFINITY, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) lacc[rb][r] = 0.f;
    }
    SparseTileQueue tq;
    tq.init(mrow, a.nb, N);
    int k0 = tq.next();
    if (k0 < 0) return;   // no kept key: O = 0, l = 0 (same for every wave)
    int k1 = tq.next();
    int k2 = (k1 >= 0) ? tq.next() : -1;

    // ---- prologue: tiles k0, k1, k2 into LDS buffers 0 .. 2 (a missing
    // tile loads key offset N, i.e. zeros, into a buffer nobody reads) ----
    {
      const uint32_t kk[3] = {(uint32_t)k0, (uint32_t)(k1 >= 0 ? k1 : N), (uint32_t)(k2 >= 0 ? k2 : N)};
#pragma unroll
      for (int j = 0; j < 3; ++j) dma.issue_all(lds_addr(smT[j]), kk[j]);
    }
    dma_wait_all();
    __syncthreads();

    f32x4 sacc[2][SRB];
    uint32_t pk[SRB][4];
    r_qk_tile(sacc, smT[0], qf, l16, g);
    if (k0 + RBN > N) r_mask(sacc, k0, N, g);
    r_softmax(sacc, st, oacc, lacc, pk, c, true);

    int bc = 0;
    while (k1 >= 0) {
      const int bn = (bc + 1) & (RNB - 1);
      const int b3 = (bc + 3) & (RNB - 1);
      const int k3 = (k2 >= 0) ? tq.next() : -1;
      const uint32_t kload = (uint32_t)(k3 >= 0 ? k3 : N);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rb = 0; rb < SRB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[kb][rb][r] = 0.f;
      bf16x8 fr[kRPre + 1];
      r_prefetch<0, kRPre>(fr, smT[bn], smT[bc] + kRegion, l16, g, s);
      r_step<0, SNT, SRB>(sacc, oacc, lacc, ones, qf, pk, smT[bn], smT[bc] + kRegion, l16, g, s, fr, dma,
                          lds_addr(smT[b3]), kload);
      __builtin_amdgcn_sched_group_barrier(0x100, kRPre, 0);
      r_step_schedule<0, SNT, SRB>();
      dma_barrier<PER>();
      if (k1 + RBN > N) r_mask(sacc, k1, N, g);
      r_softmax(sacc, st, oacc, lacc, pk, c, EXACT);
      bc = bn;
      k1 = k2;
      k2 = k3;
    }
    dma_wait_all();
    // ---- drain: PV of the last tile ----
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 vf = r_v_operand(smT[bc] + kRegion, db, g, s);
#pragma unroll
      for (int rb = 0; rb < SRB; ++rb) oacc[db][rb] = mfma16(vf, r_p_operand(pk[rb]), oacc[db][rb]);
    }
#pragma unroll
    for (int rb = 0; rb < SRB; ++rb) lacc[rb] = mfma16(ones, r_p_operand(pk[rb]), lacc[rb]);
  };
  run_pass(std::false_type{});
  bool ok = true;
#pragma unroll
  for (int rb = 0; rb < SRB; ++rb) ok = ok && (lacc[rb][0] <= kEndCheck);
  if (__syncthreads_or(!ok)) {
    __syncthreads();   // every wave is past its last LDS read before the buffers are refilled
    run_pass(std::true_type{});
  }

  // ---- epilogue ----
  const int64_t ob = b * a.os[0] + hd * a.os[1];
#pragma unroll
  for (int rb = 0; rb < SRB; ++rb) {
    const float lt = lacc[rb][0];
    const int row = q0 + 16 * rb + l16;
    if (row >= N) continue;
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
  return launch_kernel(out_f32 ? attn_merge_kernel<true> : attn_merge_kernel<false>, grid, dim3(256), s, a);
}

hipError_t launch_attn_bf16(const AttnArgs& args, bool out_f32, bool sparse, hipStream_t s) {
  AttnArgs a = args;
  if (sparse) {
    a.nqb = a.nb;   // one work-group per 128-row mask block
    const int64_t nwg = (int64_t)a.B * a.H * a.nqb;
    if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
    return launch_kernel(out_f32 ? attn_sparse_kernel<true> : attn_sparse_kernel<false>, dim3((unsigned)nwg),
                         dim3(256), s, a);
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
  const hipError_t e =
      launch_kernel(out_f32 ? attn_dense_kernel<true> : attn_dense_kernel<false>, grid, dim3(RNT), s, a);
  if (e != hipSuccess) return e;
  return launch_attn_merge(a, out_f32, s);
}

}  // namespace dit
