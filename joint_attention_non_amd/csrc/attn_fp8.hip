// attn_fp8.hip -- fp8 (OCP e4m3) joint attention for gfx950: a quantisation
// pass over Q, K, V and a flash-style attention kernel on the fp8 MFMA.
//
// Quantisation (one work-group per tensor x (b, h) x 128-token block):
//   absmax over the block (fp32), inv = 448 / absmax, s = absmax / 448,
//   code = e4m3_rne(clamp(x * inv, +-448)) via v_cvt_pk_fp8_f32.
//   Q and K codes are stored row-major [BH][Np][128]; V codes transposed
//   [BH][128][Np] with every 64-key group's 4-key groups permuted into the
//   order the PV operand reads them, so the attention kernel copies tiles
//   into LDS without any shuffle.
//
// Attention (work-group = 8 waves x 32 query rows, two waves per SIMD; key
// tiles of 128 = one scale block, in three rotating LDS buffers; the QK^T
// MFMAs of tile t+1 and the PV MFMAs of tile t form one stream with their
// LDS operands read ahead, then one barrier, then the softmax of tile t+1),
// per tile with the 32x32x64 f8f6f4 MFMA:
//   S^T = K8 Q8^T                    raw integer-grid dot products (fp32)
//   t = S * (sQ sK scale log2 e)     logits in log2 units
//   m' = max(m, rowmax t), alpha = 2^(m - m')
//   y = 2^(t - m' + log2 448)        = 448 w with w in [0, 1]
//   l = alpha l + sum e4m3(y)        (row sum of the quantised weights, on
//                                     the MFMA with an all-ones operand)
//   A = A * alpha * sV_prev / sV + V8^T e4m3(y)^T
// and at the end O = A * sV_last / l, lse = ln2 (m + log2(l / 448)).
#include "device_common.h"
#include "launch.h"

namespace dit {
namespace {

constexpr int D = kHeadDim;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Position group (4 keys) inside a 64-key group of V8t for key group kg.
__device__ __forceinline__ int v8_pos_group(int kg) {
  return 8 * (kg & 1) + 4 * (kg >> 3) + ((kg >> 1) & 3);
}

// Four floats -> four e4m3 codes (a in the low byte).  The first convert
// writes the low 16 bits and keeps the high half of its third operand, which
// the second convert then overwrites, so any register serves as that
// operand: a's own (dead after it), so no zeroed register or copy is needed.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// grid: (3 * BH * nb); 256 threads.  Work-group -> (tensor, bh, kb).
__global__ __launch_bounds__(256) void fp8_quantize_kernel(Fp8Args a) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int BH = a.B * a.H;
  const int id = blockIdx.x;
  const int tensor = id / (BH * a.nb);
  const int rem = id % (BH * a.nb);
  const int bh = rem / a.nb, kb = rem % a.nb;
  const int b = bh / a.H, hd = bh % a.H;

  const __bf16* src;
  const int64_t* st;
  uint32_t bytes;
  float* scales;
  if (tensor == 0) { src = (const __bf16*)a.q; st = a.qs; bytes = a.q_bytes; scales = a.sq; }
  else if (tensor == 1) { src = (const __bf16*)a.k; st = a.ks; bytes = a.k_bytes; scales = a.sk; }
  else { src = (const __bf16*)a.v; st = a.vs; bytes = a.v_bytes; scales = a.sv; }
  src += b * st[0] + hd * st[1];
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, bytes);
  const uint32_t row_bytes = (uint32_t)(st[2] * 2);
  const bool is_v = (tensor == 2);

  // Two units of 4 keys x 8 d per thread.  Q/K: lanes run along d (8-byte
  // row-major stores); V: lanes run along key groups (4-byte transposed
  // stores that fill 64 contiguous bytes per 16 lanes).
  int kg[2], cc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (is_v) { kg[i] = 16 * i + (tid & 15); cc[i] = tid >> 4; }
    else { cc[i] = tid & 15; kg[i] = (tid >> 4) + 16 * i; }
  }
  u32x4 x[2][4];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kb * kBlock + 4 * kg[i] + r;
      x[i][r] = buf_load_b128(rs, (uint32_t)key * row_bytes + cc[i] * 16);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(x[i][r][w])), fabsf(bf16_hi(x[i][r][w]))));
    }
  amax = wave_max(amax);
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = (amax > 0.f) ? 448.0f / amax : 0.f;
  if (tid == 0) scales[(int64_t)bh * a.nb + kb] = (amax > 0.f) ? amax / 448.0f : 1.0f;

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t codes[4][2];   // [key r][d half]: 4 codes each
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t w = x[i][r][2 * hf + e];
          y[2 * e] = fminf(fmaxf(bf16_lo(w) * inv, -448.f), 448.f);
          y[2 * e + 1] = fminf(fmaxf(bf16_hi(w) * inv, -448.f), 448.f);
        }
        codes[r][hf] = cvt4_e4m3(y[0], y[1], y[2], y[3]);
      }
    if (!is_v) {
      uint8_t* dst = (tensor == 0 ? a.q8 : a.k8) + ((int64_t)bh * a.np + kb * kBlock + 4 * kg[i]) * D + 8 * cc[i];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 t = {codes[r][0], codes[r][1]};
        *reinterpret_cast<u32x2*>(dst + r * D) = t;
      }
    } else {
      // byte transpose: for each d (8 of them) gather the 4 keys' codes
      const int g64 = kg[i] >> 4, kgl = kg[i] & 15;
      uint8_t* dst = a.v8t + ((int64_t)bh * D + 8 * cc[i]) * a.np + kb * kBlock + 64 * g64 + 4 * v8_pos_group(kgl);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int hf = j >> 2, sh = 8 * (j & 3);
        const uint32_t w = ((codes[0][hf] >> sh) & 0xffu) | (((codes[1][hf] >> sh) & 0xffu) << 8) |
                           (((codes[2][hf] >> sh) & 0xffu) << 16) | (((codes[3][hf] >> sh) & 0xffu) << 24);
        *reinterpret_cast<uint32_t*>(dst + (int64_t)j * a.np) = w;
      }
    }
  }
}

constexpr int BN8 = 128;        // keys per tile = one scale block
constexpr int RS8 = 128 + 16;   // LDS row stride in bytes (conflict-free 16-byte reads)
constexpr int NB8 = 3;          // rotating LDS tile buffers
constexpr int kPre8 = 2;        // MFMA operands read this many MFMAs ahead

__device__ __forceinline__ i32x8 lds_frag8(const uint8_t* p) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p), hi = *reinterpret_cast<const u32x4*>(p + 16);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// A operand J of a step's MFMA stream.  J < 8: K8 fragment (s, kb) =
// (J / 4, J % 4) of the next tile: rows 32 kb + l32, bytes 64 s + 32 h ..
// +31.  J >= 8: V8t fragment (s, db) = ((J-8) / 4, (J-8) % 4) of the current
// tile: d rows 32 db + l32, key bytes 64 s + 32 h .. +31.
template <int J>
__device__ __forceinline__ i32x8 op8(const uint8_t* sK, const uint8_t* sV, int l32, int h) {
  if constexpr (J < 8) return lds_frag8(sK + ((J & 3) * 32 + l32) * RS8 + 64 * (J >> 2) + 32 * h);
  else return lds_frag8(sV + (((J - 8) & 3) * 32 + l32) * RS8 + 64 * ((J - 8) >> 2) + 32 * h);
}

// Operands [I, kPre8) of a step, read before its first MFMA.
template <int I>
__device__ __forceinline__ void prefetch8(i32x8 (&fr)[kPre8 + 1], const uint8_t* sK, const uint8_t* sV, int l32,
                                          int h) {
  if constexpr (I < kPre8) {
    fr[I] = op8<I>(sK, sV, l32, h);
    prefetch8<I + 1>(fr, sK, sV, l32, h);
  }
}

__device__ __forceinline__ i32x8 p_frag8(const uint32_t (&p8)[2][8], int s) {
  return i32x8{(int)p8[s][0], (int)p8[s][1], (int)p8[s][2], (int)p8[s][3],
               (int)p8[s][4], (int)p8[s][5], (int)p8[s][6], (int)p8[s][7]};
}

// Global -> register -> LDS staging of one 128-key tile of K8 (row-major)
// and V8t (d-major), 16-byte chunks, KCH of each per thread.
template <int NT>
struct Loader8 {
  static constexpr int KCH = BN8 * (D / 16) / NT;
  static_assert(KCH * NT == BN8 * (D / 16), "tile split");
  u32x4 r[2 * KCH];
  template <int I>
  __device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int t, int np,
                                           int tid) {
    const int id = tid + (I % KCH) * NT, row = id >> 3, c = id & 7;
    if constexpr (I < KCH) r[I] = buf_load_b128(rk, (uint32_t)(t * BN8 + row) * D + c * 16);
    else r[I] = buf_load_b128(rv, (uint32_t)row * np + t * BN8 + c * 16);
  }
  template <int I>
  __device__ __forceinline__ void store_one(uint8_t* sk, uint8_t* sv, int tid) const {
    const int id = tid + (I % KCH) * NT, row = id >> 3, c = id & 7;
    *reinterpret_cast<u32x4*>((I < KCH ? sk : sv) + row * RS8 + c * 16) = r[I];
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int t, int np, int tid) {
    if constexpr (KCH == 2) {
      load_one<0>(rk, rv, t, np, tid); load_one<1>(rk, rv, t, np, tid);
      load_one<2>(rk, rv, t, np, tid); load_one<3>(rk, rv, t, np, tid);
    } else {
      static_assert(KCH == 2, "loader unrolled for 512 threads");
    }
  }
  __device__ __forceinline__ void store(uint8_t* sk, uint8_t* sv, int tid) const {
    store_one<0>(sk, sv, tid); store_one<1>(sk, sv, tid);
    store_one<2>(sk, sv, tid); store_one<3>(sk, sv, tid);
  }
};

// MFMA I (0..15) of a step: 0-7 QK^T of the next tile, 8-15 PV of the
// current one (plus, at I = 8 and 12, the row-sum MFMA of that 64-key step
// with an all-ones A operand: every row of its result is the column sum of
// P8, so each lane gets its query row's sum).  The four staged chunks are
// stored to LDS and refilled from memory beside the PV MFMAs.
template <int I, int NT>
__device__ __forceinline__ void step8(f32x16 (&sacc)[4], f32x16 (&oacc)[4], f32x16& lacc, const i32x8 (&qf)[2],
                                      const uint32_t (&p8)[2][8], const uint8_t* sK, const uint8_t* sV, int l32,
                                      int h, i32x8 (&fr)[kPre8 + 1], Loader8<NT>& ld, uint8_t* sks, uint8_t* svs,
                                      __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int tload, int np,
                                      int tid) {
  if constexpr (I < 16) {
    if constexpr (I + kPre8 < 16) fr[(I + kPre8) % (kPre8 + 1)] = op8<I + kPre8>(sK, sV, l32, h);
    const i32x8 a = fr[I % (kPre8 + 1)];
    if constexpr (I < 8) {
      constexpr int s = I >> 2, kb = I & 3;
      sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[s], sacc[kb], 0, 0, 0, 0, 0, 0);
    } else {
      constexpr int s = (I - 8) >> 2, db = (I - 8) & 3;
      const i32x8 pf = p_frag8(p8, s);
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, oacc[db], 0, 0, 0, 0, 0, 0);
      if constexpr (db == 0) {
        const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                            0x38383838, 0x38383838, 0x38383838, 0x38383838};   // e4m3 1.0
        lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, 0, 0, 0);
      }
      if constexpr ((I & 1) == 0) {
        ld.template store_one<((I - 8) >> 1)>(sks, svs, tid);
        ld.template load_one<((I - 8) >> 1)>(rk, rv, tload, np, tid);
      }
    }
    step8<I + 1, NT>(sacc, oacc, lacc, qf, p8, sK, sV, l32, h, fr, ld, sks, svs, rk, rv, tload, np, tid);
  }
}

template <int I>
__device__ __forceinline__ void step8_schedule() {
  if constexpr (I < 16) {
    if constexpr (I + kPre8 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, ((I >= 8) && ((I - 8) & 3) == 0) ? 2 : 1, 0);
    if constexpr (I >= 8 && (I & 1) == 0) {
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS store
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
    }
    step8_schedule<I + 1>();
  }
}

__device__ __forceinline__ void qk8_tile(f32x16 (&sacc)[4], const uint8_t* sK, const i32x8 (&qf)[2], int l32, int h) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          lds_frag8(sK + (kb * 32 + l32) * RS8 + 64 * s + 32 * h), qf[s], sacc[kb], 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ void pv8_tile(f32x16 (&oacc)[4], f32x16& lacc, const uint32_t (&p8)[2][8],
                                         const uint8_t* sV, int l32, int h) {
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const i32x8 pf = p_frag8(p8, s);
#pragma unroll
    for (int db = 0; db < 4; ++db)
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          lds_frag8(sV + (db * 32 + l32) * RS8 + 64 * s + 32 * h), pf, oacc[db], 0, 0, 0, 0, 0, 0);
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, 0, 0, 0);
  }
}

// Softmax of one tile (keys key0 ..): t = S f, new running max, quantised
// weights e4m3(2^(t - m + log2 448)) into p8, and the running accumulator
// and row sum brought to the new max and to this tile's V scale.
__device__ __forceinline__ void softmax8(f32x16 (&sacc)[4], f32x16 (&oacc)[4], f32x16& lacc, uint32_t (&p8)[2][8],
                                         float& m_run, float& sv_prev, float f, float svt, float p_off, int key0,
                                         int N, int h) {
  if (key0 + BN8 > N) {
    // Keys past N get -inf.  Element (kb, r) of this lane is key key0 + off
    // + 4h with off = 32 kb + 8 (r/4) + r%4; each select uses its compare at
    // once (the schedule barriers keep 64 compare masks from being live
    // together in scalar registers).
    const int rem = N - key0 - 4 * h;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
        sacc[kb][r] = off < rem ? sacc[kb][r] : -INFINITY;
        __builtin_amdgcn_sched_barrier(0);
      }
  }
  const float vratio = sv_prev / svt;
  sv_prev = svt;
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
  mx = fmaxf(mx, swap_halves(mx));
  const float mnew = fmaxf(m_run, mx * f);
  const float alpha = fast_exp2(m_run - mnew);
  const float moff = mnew - p_off;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int slot = 4 * w + e, kb = 2 * s + (slot >> 4), r = slot & 15;
        y[e] = fast_exp2(__builtin_fmaf(sacc[kb][r], f, -moff));
      }
      p8[s][w] = cvt4_e4m3(y[0], y[1], y[2], y[3]);
    }
  // Only element 0 of the row-sum accumulator is read at the end.
  lacc[0] *= alpha;
  m_run = mnew;
  const float g = alpha * vratio;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] *= g;
}

// Work-group: NW waves x 32 query rows.  Step t issues the QK^T MFMAs of
// tile t+1 and the PV MFMAs of tile t as one stream, their A operands read
// from LDS kPre8 MFMAs ahead, with tile t+2 stored to LDS and tile t+3
// loaded into registers beside the PV half; one barrier; then the softmax of
// tile t+1.  Tiles rotate through NB8 LDS buffers.
template <int NW, bool OUT_F32>
__global__ __launch_bounds__(NW * 64, 2) void attn_fp8_kernel(Fp8Args a, int nqb) {
  constexpr int BM = NW * 32, NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t smK[NB8][BN8 * RS8];
  __shared__ __attribute__((aligned(16))) uint8_t smV[NB8][D * RS8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  // Work-group -> query block; a tail work-group also gets one of the
  // `split` key-tile ranges [t0, t1) of its block.
  int tile, part = -1;
  if ((int)blockIdx.x < a.nfull) {
    tile = xcd_remap(blockIdx.x, a.nfull);
  } else {
    const int j = blockIdx.x - a.nfull;
    tile = a.nfull + j / a.split;
    part = j % a.split;
  }
  const int bh = tile / nqb, qblk = tile % nqb;
  const int b = bh / a.H, hd = bh % a.H;
  const int N = a.N, np = a.np, nb = a.nb;
  const int t0 = part < 0 ? 0 : part * nb / a.split;
  const int t1 = part < 0 ? nb : (part + 1) * nb / a.split;

  const uint8_t* q8 = a.q8 + (int64_t)bh * np * D;
  const uint8_t* k8 = a.k8 + (int64_t)bh * np * D;
  const uint8_t* v8 = a.v8t + (int64_t)bh * D * np;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q8, (uint32_t)(np * D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k8, (uint32_t)(np * D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v8, (uint32_t)(np * D));

  const int q0 = qblk * BM + wave * 32;
  const float sqw = (q0 < np) ? a.sq[(int64_t)bh * nb + q0 / kBlock] : 1.f;
  const float fq = sqw * a.c;
  const float* skp = a.sk + (int64_t)bh * nb;
  const float* svp = a.sv + (int64_t)bh * nb;

  // Q8 as the B operand: lane (l32, h) holds row q0 + l32, d = 64 s + 32 h .. +31.
  i32x8 qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint32_t off = (uint32_t)(q0 + l32) * D + 64 * s + 32 * h;
    const u32x4 lo = buf_load_b128(rq, off), hi = buf_load_b128(rq, off + 16);
    qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  f32x16 oacc[4];
  f32x16 lacc;   // row sums of the quantised weights (448 units), element 0 used
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    lacc[r] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db][r] = 0.f;
  }
  float m_run = -INFINITY, sv_prev = 1.f;

  // ---- prologue: tiles t0 and t0+1 into LDS, t0+2 into registers ----
  Loader8<NT> ld;
  ld.load(rk, rv, t0, np, tid);
  ld.store(smK[0], smV[0], tid);
  ld.load(rk, rv, min(t0 + 1, t1 - 1), np, tid);
  ld.store(smK[1], smV[1], tid);
  ld.load(rk, rv, min(t0 + 2, t1 - 1), np, tid);
  __syncthreads();

  f32x16 sacc[4];
  uint32_t p8[2][8];
  qk8_tile(sacc, smK[0], qf, l32, h);
  softmax8(sacc, oacc, lacc, p8, m_run, sv_prev, fq * skp[t0], svp[t0], a.p_off, t0 * BN8, N, h);

  int bc = 0;   // LDS buffer of tile t; tile t+1 is in bc+1, tile t+2 goes to bc+2 (mod 3)
  for (int t = t0; t + 1 < t1; ++t) {
    const int bn = (bc + 1 == NB8) ? 0 : bc + 1;
    const int bn2 = (bn + 1 == NB8) ? 0 : bn + 1;
    // Past the last tile the staged buffer is free and never read, and the
    // load repeats the last tile.
    const int tload = min(t + 3, t1 - 1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
    i32x8 fr[kPre8 + 1];
    prefetch8<0>(fr, smK[bn], smV[bc], l32, h);
    step8<0, NT>(sacc, oacc, lacc, qf, p8, smK[bn], smV[bc], l32, h, fr, ld, smK[bn2], smV[bn2], rk, rv, tload,
                 np, tid);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre8, 0);
    step8_schedule<0>();
    __syncthreads();
    softmax8(sacc, oacc, lacc, p8, m_run, sv_prev, fq * skp[t + 1], svp[t + 1], a.p_off, (t + 1) * BN8, N, h);
    bc = bn;
  }
  pv8_tile(oacc, lacc, p8, smV[bc], l32, h);

  // ---- epilogue: O = A * sV_last / l ----
  const int64_t ob = b * a.os[0] + hd * a.os[1];
  const float lt = lacc[0];
  const float inv = lt > 0.f ? sv_prev / lt : 0.f;
  const int row = q0 + l32;
  if (part >= 0) {
    // Partial result of one key range: A * sV_last (unnormalised O), m, l.
    float* pr = a.part + ((int64_t)(blockIdx.x - a.nfull) * BM + wave * 32 + l32) * kPartRow;
    if (row < N) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 t4 = {oacc[db][4 * r4 + 0] * sv_prev, oacc[db][4 * r4 + 1] * sv_prev,
                            oacc[db][4 * r4 + 2] * sv_prev, oacc[db][4 * r4 + 3] * sv_prev};
          *reinterpret_cast<f32x4*>(pr + db * 32 + r4 * 8 + h * 4) = t4;
        }
      if (h == 0) {
        pr[128] = m_run;
        pr[129] = lt;
      }
    }
    return;
  }
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
          f32x4 t4 = {v0, v1, v2, v3};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d0) = t4;
        } else {
          u32x2 t2 = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.o) + orow + d0) = t2;
        }
      }
    if (a.lse != nullptr && h == 0)
      a.lse[(int64_t)bh * N + row] =
          lt > 0.f ? (m_run + __builtin_log2f(lt) - 8.8073549220576041f) * 0.69314718055994530942f : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8Args& a, hipStream_t s) {
  const int64_t nwg = 3LL * a.B * a.H * a.nb;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fp8_quantize_kernel, dim3((unsigned)nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const Fp8Args& args, bool out_f32, hipStream_t s) {
  Fp8Args a = args;
  const int nqb = (a.N + 255) / 256;   // 8 waves x 32 query rows per work-group
  int64_t nwg = (int64_t)a.B * a.H * nqb;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool split = a.split > 1 && a.part != nullptr;
  if (split) {
    if (a.nfull + a.ntail != nwg) return hipErrorInvalidConfiguration;
    nwg = (int64_t)a.nfull + (int64_t)a.ntail * a.split;
  } else {
    a.nfull = (int)nwg;
    a.ntail = 0;
    a.split = 1;
  }
  if (out_f32) hipLaunchKernelGGL((attn_fp8_kernel<8, true>), dim3((unsigned)nwg), dim3(512), 0, s, a, nqb);
  else hipLaunchKernelGGL((attn_fp8_kernel<8, false>), dim3((unsigned)nwg), dim3(512), 0, s, a, nqb);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  // Merge the split key ranges (the weights are in units of 1/448).
  AttnArgs m = {};
  m.o = a.o;
  m.lse = a.lse;
  for (int i = 0; i < 3; ++i) m.os[i] = a.os[i];
  m.B = a.B;
  m.H = a.H;
  m.N = a.N;
  m.nqb = nqb;
  m.nfull = a.nfull;
  m.ntail = a.ntail;
  m.split = a.split;
  m.part = a.part;
  m.lse_off = -8.8073549220576041f;   // -log2(448)
  m.bm = 256;                          // 8 waves x 32 query rows
  return launch_attn_merge(m, out_f32, s);
}

}  // namespace dit
