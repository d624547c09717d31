// attn_fp8.hip -- fp8 (OCP e4m3) joint attention for gfx950: a quantisation
// pass over K and V (and Q, for the quantise-only entry point) and a
// flash-style attention kernel on the fp8 MFMA that quantises its own Q
// rows in its prologue.
//
// Quantisation (one work-group per tensor x (b, h) x 128-token block):
//   absmax over the block (fp32), inv = 448 / absmax, s = absmax / 448,
//   code = e4m3_rne(clamp(x * inv, +-448)) via v_cvt_pk_fp8_f32; a block
//   with absmax = 0 or 448 / absmax = inf gets s = 1 and zero codes.
//   Q and K codes are stored row-major [BH][Np][128]; V codes transposed
//   [BH][128][Np] with every 64-key group's 4-key groups permuted into the
//   order the PV operand reads them, so the attention kernel copies tiles
//   into LDS without any shuffle.
//
// Attention (work-group = 8 waves x 32 query rows, two waves per SIMD; key
// tiles of 128 = one scale block, in four rotating LDS buffers; the QK^T
// MFMAs of tile t+1 and the PV MFMAs of tile t form one stream with their
// LDS operands read ahead, then the softmax of tile t+1; waves 4-7 run half
// a step behind waves 0-3, two barriers per step),
// per tile with the 32x32x64 f8f6f4 MFMA:
//   S^T = K8 Q8^T                    raw integer-grid dot products (fp32)
//   t = S * (sQ sK scale log2 e)     logits in log2 units
//   m' = max(m, rowmax t), alpha = 2^(m - m')
//   y = 2^(t - m' + log2 448)        = 448 w with w in [0, 1]
//   l = alpha l + sum e4m3(y)        (row sum of the quantised weights, on
//                                     the MFMA with an all-ones operand)
//   A = A * alpha * sV_prev / sV + V8^T e4m3(y)^T
// and at the end O = A * sV_last / l, lse = ln2 (m + log2(l / 448)).  (A V
// block whose scale is below 2^-64 of the largest one added so far is left
// out of A, which keeps A finite whatever the spread of V scales; see VUnit.)
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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, 64));
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
  const int tensor = a.first_tensor + id / (BH * a.nb);
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
  // A block whose absmax is 0, or so small that 448 / absmax is not a finite
  // fp32 number (absmax below 448 / FLT_MAX, about 1.3e-36), is stored as a
  // zero block: scale 1 and all codes 0 (+0), whatever the signs of its zeros.
  const float inv = 448.0f / amax;
  const bool zero_block = !(inv <= 3.40282347e38f);
  if (tid == 0) scales[(int64_t)bh * a.nb + kb] = zero_block ? 1.0f : amax / 448.0f;

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
        codes[r][hf] = zero_block ? 0u : cvt4_e4m3(y[0], y[1], y[2], y[3]);
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
constexpr int NB8 = 4;          // rotating LDS tile buffers
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

// Direct global -> LDS staging of one 128-key tile (buffer_load ... lds): a
// tile buffer holds the tile's 128 K8 rows and its 128 V8t rows (d-major),
// each at the 144-byte stride in a region of 1152 16-byte slots, then a 1 KB
// junk area.  One such instruction writes 64 consecutive slots (lane i ->
// slot i): 18 per region, 36 per tile, dealt to the 8 waves round-robin
// (instruction i to wave i % 8), the 4 left over loading into the junk area
// so that every wave issues PER = 5 per tile.  A row's padding slot gets a
// copy of its chunk 7 (never read).
constexpr int kRegion8 = BN8 * RS8;            // bytes per tensor region (18432)
constexpr int kTileBuf8 = 2 * kRegion8 + 1024;

template <int NW>
struct TileDma8 {
  static constexpr int NI = 2 * kRegion8 / 1024;   // 36
  static constexpr int PER = (NI + NW - 1) / NW;
  uint32_t off[PER];    // this lane's byte offset inside the tile, per instruction
  i32x4 rsrc[PER];      // K8 or V8t slice, wave-uniform
  uint32_t dst[PER];    // LDS byte offset inside a tile buffer, wave-uniform
  uint32_t step[PER];   // bytes between consecutive tiles in that tensor, wave-uniform
  __device__ __forceinline__ void init(int wave, int lane, const uint8_t* k8, const uint8_t* v8, int np) {
    const uint32_t bytes = (uint32_t)(np * D);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = wave + j * NW;
      const bool isv = i >= NI / 2;
      const int slot = 64 * (isv ? i - NI / 2 : i) + lane;
      const int row = slot / (RS8 / 16), c = min(slot % (RS8 / 16), 7);
      // K8 rows are 128 bytes apart and a tile is 128 rows; V8t rows (d)
      // are np bytes apart and a tile is 128 bytes of each.
      off[j] = (uint32_t)row * (isv ? (uint32_t)np : 128u) + 16u * (uint32_t)c;
      const uint64_t base = reinterpret_cast<uint64_t>(isv ? v8 : k8);
      rsrc[j] = i32x4{(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xffffu), (int)bytes, 0x00020000};
      dst[j] = i >= NI ? 2u * kRegion8 : (uint32_t)(isv ? kRegion8 + 1024 * (i - NI / 2) : 1024 * i);
      step[j] = isv ? (uint32_t)BN8 : (uint32_t)(BN8 * D);
    }
  }
  // Instruction J of this wave for tile t into the tile buffer at LDS byte
  // address `buf` (inline assembly, for the reason given with the bf16
  // kernels' staging: the compiler would order later LDS reads after it).
  template <int J>
  __device__ __forceinline__ void issue(uint32_t buf, uint32_t t) const {
    const uint32_t voff = off[J] + t * step[J];
    // The LDS address goes in through M0 as an operand, so the compiler
    // writes M0 itself and knows it was changed.
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc[J]), "{m0}"(buf + dst[J])
                 : "memory");
  }
  template <int J = 0>
  __device__ __forceinline__ void issue_all(uint32_t buf, uint32_t t) const {
    if constexpr (J < PER) {
      issue<J>(buf, t);
      issue_all<J + 1>(buf, t);
    }
  }
};

__device__ __forceinline__ uint32_t lds_addr8(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}

// After a step's MFMA stream: wait until at most this wave's PER newest
// staging loads (this step's tile) are in flight, then the barrier.
template <int PER>
__device__ __forceinline__ void dma8_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(PER) : "memory");
}
__device__ __forceinline__ void dma8_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void plain_barrier8() { asm volatile("s_barrier" ::: "memory"); }

// MFMA I (0..15) of a step: 0-7 QK^T of the next tile, 8-15 PV of the
// current one (plus, at I = 8 and 12, the row-sum MFMA of that 64-key step
// with an all-ones A operand: every row of its result is the column sum of
// P8, so each lane gets its query row's sum).  The wave's PER staging loads
// of the tile three ahead go out at I = 1, 3, 5, ...
template <int I, int NT>
__device__ __forceinline__ void step8(f32x16 (&sacc)[4], f32x16 (&oacc)[4], f32x16& lacc, const i32x8 (&qf)[2],
                                      const uint32_t (&p8)[2][8], const uint8_t* sK, const uint8_t* sV, int l32,
                                      int h, i32x8 (&fr)[kPre8 + 1], const TileDma8<NT / 64>& dma, uint32_t dbuf,
                                      uint32_t tload) {
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
    }
    if constexpr ((I & 1) == 1 && (I >> 1) < TileDma8<NT / 64>::PER) dma.template issue<(I >> 1)>(dbuf, tload);
    step8<I + 1, NT>(sacc, oacc, lacc, qf, p8, sK, sV, l32, h, fr, dma, dbuf, tload);
  }
}

template <int I>
__device__ __forceinline__ void step8_schedule() {
  if constexpr (I < 16) {
    if constexpr (I + kPre8 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, ((I >= 8) && ((I - 8) & 3) == 0) ? 2 : 1, 0);
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

// The PV accumulator A is carried in the dequantisation scale of the V block
// last added to it (sv): moving to the next block's scale svt multiplies A by
// sv / svt (with the softmax's alpha).  A V block whose scale is below 2^-64
// times the largest scale added so far (vmax) is not added at all -- its
// values are below 2^-64 of the largest V magnitude among the row's keys, so
// leaving them out changes O by less than that -- while its weights still
// count in the row sum: the row-sum MFMAs of that tile run at once and its
// quantised weights are then zeroed, so the PV and row-sum MFMAs of the
// pipeline add nothing for it.  That bounds the factor by 2^64 and A by about
// 448^2 * keys * 2^64, far inside fp32, whatever the spread of V scales.  No
// V block is left out of inputs whose V scales stay within 2^64 of each
// other (every ordinary input).
struct VUnit {
  float sv;     // scale of the last V block added to A
  float vmax;   // largest scale of the V blocks added to A
};

// Softmax of one tile (keys key0 ..): t = S f, new running max, quantised
// weights e4m3(2^(t - m + log2 448)) into p8, and the running accumulator
// and row sum brought to the new max and to this tile's V scale (or the
// tile's V left out, see VUnit).
__device__ __forceinline__ void softmax8(f32x16 (&sacc)[4], f32x16 (&oacc)[4], f32x16& lacc, uint32_t (&p8)[2][8],
                                         float& m_run, VUnit& unit, float f, float svt, float p_off, int key0,
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
  const bool add_v = svt >= unit.vmax * 0x1p-64f;   // wave-uniform
  const float vratio = add_v ? unit.sv / svt : 1.f;
  if (add_v) {
    unit.sv = svt;
    unit.vmax = fmaxf(unit.vmax, svt);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
  mx = max_halves(mx);
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
  if (!add_v) {
    // V block left out (see VUnit): count its weights now, then zero them.
    const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, p_frag8(p8, s), lacc, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int w = 0; w < 8; ++w) p8[s][w] = 0u;
    }
  }
}

// Work-group: NW waves x 32 query rows.  Step t issues the QK^T MFMAs of
// tile t+1 and the PV MFMAs of tile t as one stream, their A operands read
// from LDS kPre8 MFMAs ahead, with tile t+3 loaded straight into LDS beside
// them; a barrier; then the softmax of tile t+1 and a second barrier, with
// waves 4-7 half a step behind waves 0-3.  Tiles rotate through NB8 LDS
// buffers.
template <int NW, bool OUT_F32>
__global__ __launch_bounds__(NW * 64, 2) void attn_fp8_kernel(Fp8Args a, int nqb) {
  constexpr int BM = NW * 32, NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t smT[NB8][kTileBuf8];
  __shared__ uint32_t qmax_lds[NW];

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

  const uint8_t* k8 = a.k8 + (int64_t)bh * np * D;
  const uint8_t* v8 = a.v8t + (int64_t)bh * D * np;
  TileDma8<NW> dma;
  dma.init(__builtin_amdgcn_readfirstlane(wave), lane, k8, v8, np);
  constexpr int PER = TileDma8<NW>::PER;
  // The K and V scales are read through the scalar cache (constant address
  // space; the quantisation pass wrote them before this kernel started): a
  // vector load here would make the compiler wait for every outstanding
  // vector memory operation, the in-flight tile staging included.
  typedef const __attribute__((address_space(4))) float* cfloat_ptr;
  const cfloat_ptr skp = (cfloat_ptr)(a.sk + (int64_t)bh * nb);
  const cfloat_ptr svp = (cfloat_ptr)(a.sv + (int64_t)bh * nb);

  // Q is quantised here, in the prologue, rather than by the quantisation
  // pass: the work-group's 256 rows are exactly two 128-token scale blocks
  // (waves 0-3 and 4-7), so each block's absmax is a reduction inside the
  // work-group.  Same arithmetic as the pass, hence the same codes and
  // scale.  Lane (l32, h) loads row q0 + l32, d = 64 s + 32 h .. +31 (bf16;
  // rows >= N read as zero and leave the absmax alone), which is exactly
  // the part of Q8 it needs as the B operand.
  const int q0 = qblk * BM + wave * 32;
  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.qs[0] + hd * a.qs[1];
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qp, a.q_bytes);
  const uint32_t qoff = (uint32_t)min(q0 + l32, N) * (uint32_t)(a.qs[2] * 2);

  f32x16 oacc[4];
  f32x16 lacc;   // row sums of the quantised weights (448 units), element 0 used
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    lacc[r] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db][r] = 0.f;
  }
  float m_run = -INFINITY;
  VUnit unit = {svp[t0], svp[t0]};

  // ---- prologue: tiles t0 .. t0+2 into LDS buffers 0 .. 2 (past the last
  // tile the load repeats it into a buffer nobody reads) ----
  dma.issue_all(lds_addr8(smT[0]), (uint32_t)t0);
  u32x4 qx[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) qx[s][c4] = buf_load_b128(rq, qoff + (64 * s + 32 * h + 8 * c4) * 2);
  dma.issue_all(lds_addr8(smT[1]), (uint32_t)min(t0 + 1, t1 - 1));
  dma.issue_all(lds_addr8(smT[2]), (uint32_t)min(t0 + 2, t1 - 1));
  uint32_t qabs = 0;   // max of |x| over this lane's elements, as bf16 bits (ordered like the values)
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t m = qx[s][c4][w] & 0x7fff7fffu;
        qabs = max(qabs, max(m & 0xffffu, m >> 16));
      }
  qabs = wave_max_u32(qabs);
  if (lane == 0) qmax_lds[wave] = qabs;
  dma8_wait_all();
  __syncthreads();

  // The Q scale block of this wave: absmax over its four waves, then the
  // quantisation pass's rule (448 / absmax in fp32, codes e4m3(clamp(x *
  // inv)), a block whose 448 / absmax is not finite stored as zero codes
  // with scale 1).
  const int w0 = wave & 4;
  const uint32_t qbits = max(max(qmax_lds[w0], qmax_lds[w0 + 1]), max(qmax_lds[w0 + 2], qmax_lds[w0 + 3]));
  const float qamax = __builtin_bit_cast(float, qbits << 16);
  const float qinv = 448.0f / qamax;
  const bool qzero = !(qinv <= 3.40282347e38f);
  const float fq = (qzero ? 1.0f : qamax / 448.0f) * a.c;
  i32x8 qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t w = qx[s][c4][2 * hf + e];
          y[2 * e] = fminf(fmaxf(bf16_lo(w) * qinv, -448.f), 448.f);
          y[2 * e + 1] = fminf(fmaxf(bf16_hi(w) * qinv, -448.f), 448.f);
        }
        qf[s][2 * c4 + hf] = qzero ? 0 : (int)cvt4_e4m3(y[0], y[1], y[2], y[3]);
      }

  f32x16 sacc[4];
  uint32_t p8[2][8];
  qk8_tile(sacc, smT[0], qf, l32, h);
  softmax8(sacc, oacc, lacc, p8, m_run, unit, fq * skp[t0], svp[t0], a.p_off, t0 * BN8, N, h);

  // Ping-pong, as in the bf16 dense kernel: waves 4-7 run half a step behind
  // waves 0-3 (two barriers per step, one extra for each group outside the
  // loop), so on every SIMD one wave's MFMAs overlap the other's softmax.
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  if (grp == 1) __syncthreads();
  int bc = 0;   // LDS buffer of tile t; tile t+1 is in bc+1, tile t+3 goes to bc+3 (mod 4)
  float sk_next = skp[min(t0 + 1, t1 - 1)], sv_next = svp[min(t0 + 1, t1 - 1)];   // scales of tile t+1
  for (int t = t0; t + 1 < t1; ++t) {
    const int bn = (bc + 1) & (NB8 - 1);
    const int b3 = (bc + 3) & (NB8 - 1);
    // Past the last tile the staged buffer is free and never read, and the
    // load repeats the last tile.
    const int tload = min(t + 3, t1 - 1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
    i32x8 fr[kPre8 + 1];
    prefetch8<0>(fr, smT[bn], smT[bc] + kRegion8, l32, h);
    step8<0, NT>(sacc, oacc, lacc, qf, p8, smT[bn], smT[bc] + kRegion8, l32, h, fr, dma, lds_addr8(smT[b3]),
                 (uint32_t)tload);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre8, 0);
    step8_schedule<0>();
    __builtin_amdgcn_sched_barrier(0);   // the whole MFMA stream before the barrier
    dma8_barrier<PER>();
    // The scales of the tile after next, read at the start of the softmax,
    // which makes no LDS access: a scalar load shares its wait counter with
    // the LDS operand reads, so one still in flight during the MFMA stream
    // would hold up its first read.  The empty asm keeps the loads here.
    const int t2 = min(t + 2, t1 - 1);
    const float sk_nn = skp[t2], sv_nn = svp[t2];
    asm volatile("" ::: "memory");
    softmax8(sacc, oacc, lacc, p8, m_run, unit, fq * sk_next, sv_next, a.p_off, (t + 1) * BN8, N, h);
    sk_next = sk_nn;
    sv_next = sv_nn;
    plain_barrier8();
    bc = bn;
  }
  dma8_wait_all();
  if (grp == 0) __syncthreads();
  pv8_tile(oacc, lacc, p8, smT[bc] + kRegion8, l32, h);

  // ---- epilogue: O = A * sV_last / l ----
  const int64_t ob = b * a.os[0] + hd * a.os[1];
  const float lt = lacc[0];
  const float inv = lt > 0.f ? unit.sv / lt : 0.f;
  const float ounit = unit.sv;
  const int row = q0 + l32;
  if (part >= 0) {
    // Partial result of one key range: A * sV_last (unnormalised O), m, l.
    float* pr = a.part + ((int64_t)(blockIdx.x - a.nfull) * BM + wave * 32 + l32) * kPartRow;
    if (row < N) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 t4 = {oacc[db][4 * r4 + 0] * ounit, oacc[db][4 * r4 + 1] * ounit,
                            oacc[db][4 * r4 + 2] * ounit, oacc[db][4 * r4 + 3] * ounit};
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
  const int64_t nwg = (3LL - a.first_tensor) * a.B * a.H * a.nb;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  return launch_kernel(fp8_quantize_kernel, dim3((unsigned)nwg), dim3(256), s, a);
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
  const hipError_t e = launch_kernel(out_f32 ? attn_fp8_kernel<8, true> : attn_fp8_kernel<8, false>,
                                     dim3((unsigned)nwg), dim3(512), s, a, nqb);
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
