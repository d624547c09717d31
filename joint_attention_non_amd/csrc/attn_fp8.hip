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
// tiles of 128 = one scale block), per tile with the 32x32x64 f8f6f4 MFMA:
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

__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
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

template <int NW, int R, bool OUT_F32>
__global__ __launch_bounds__(NW * 64, (R == 1 ? 2 : 1)) void attn_fp8_kernel(Fp8Args a, int nqb) {
  constexpr int BM = NW * 32 * R, NT = NW * 64;
  constexpr int KCH = BN8 * (D / 16) / NT;   // 16-byte chunks of each of K8 and V8t per thread
  static_assert(KCH * NT == BN8 * (D / 16), "tile split");
  __shared__ __attribute__((aligned(16))) uint8_t smK[2][BN8 * RS8];
  __shared__ __attribute__((aligned(16))) uint8_t smV[2][D * RS8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / nqb, qblk = tile % nqb;
  const int b = bh / a.H, hd = bh % a.H;
  const int N = a.N, np = a.np, nb = a.nb;

  const uint8_t* q8 = a.q8 + (int64_t)bh * np * D;
  const uint8_t* k8 = a.k8 + (int64_t)bh * np * D;
  const uint8_t* v8 = a.v8t + (int64_t)bh * D * np;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q8, (uint32_t)(np * D));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k8, (uint32_t)(np * D));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v8, (uint32_t)(np * D));

  const int q0 = qblk * BM + wave * 32 * R;
  const float sqw = (q0 < np) ? a.sq[(int64_t)bh * nb + q0 / kBlock] : 1.f;
  const float fq = sqw * a.c;

  // Q8 as the B operand: lane (l32, h) holds row q0 + 32 qi + l32, d = 64 s + 32 h .. +31.
  i32x8 qf[R][2];
#pragma unroll
  for (int qi = 0; qi < R; ++qi)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t off = (uint32_t)(q0 + qi * 32 + l32) * D + 64 * s + 32 * h;
      const u32x4 lo = buf_load_b128(rq, off), hi = buf_load_b128(rq, off + 16);
      qf[qi][s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }

  f32x16 oacc[R][4];
#pragma unroll
  for (int qi = 0; qi < R; ++qi)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qi][db][r] = 0.f;
  float m_run[R];
  f32x16 lacc[R];   // row sums of the quantised weights (448 units), element 0 used
#pragma unroll
  for (int qi = 0; qi < R; ++qi) {
    m_run[qi] = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[qi][r] = 0.f;
  }
  const i32x8 kOnes = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                       0x38383838, 0x38383838, 0x38383838, 0x38383838};   // e4m3 1.0
  float sv_prev = 1.f;

  // tile loader: KCH x 16 B of K8 and of V8t per thread
  u32x4 kr[KCH], vr[KCH];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + i * NT, row = id >> 3, c = id & 7;
      kr[i] = buf_load_b128(rk, (uint32_t)(t * BN8 + row) * D + c * 16);
      vr[i] = buf_load_b128(rv, (uint32_t)row * np + t * BN8 + c * 16);
    }
  };
  auto store_tile = [&](int bf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + i * NT, row = id >> 3, c = id & 7;
      *reinterpret_cast<u32x4*>(&smK[bf][row * RS8 + c * 16]) = kr[i];
      *reinterpret_cast<u32x4*>(&smV[bf][row * RS8 + c * 16]) = vr[i];
    }
  };

  load_tile(0);
  store_tile(0);
  if (nb > 1) load_tile(1);
  __syncthreads();

  for (int t = 0; t < nb; ++t) {
    const int bf = t & 1;
    const uint8_t* sK = smK[bf];
    const uint8_t* sV = smV[bf];
    const int key0 = t * BN8;

    // ---- S^T = K8 Q8^T ----
    f32x16 sacc[R][4];
#pragma unroll
    for (int qi = 0; qi < R; ++qi)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qi][kb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint8_t* p = sK + (kb * 32 + l32) * RS8 + 64 * s + 32 * h;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(p), hi = *reinterpret_cast<const u32x4*>(p + 16);
        const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
        for (int qi = 0; qi < R; ++qi)
          sacc[qi][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[qi][s], sacc[qi][kb], 0, 0, 0, 0, 0, 0);
      }

    if (key0 + BN8 > N) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          if (key >= N) {
#pragma unroll
            for (int qi = 0; qi < R; ++qi) sacc[qi][kb][r] = -INFINITY;
          }
        }
    }

    const float f = fq * a.sk[(int64_t)bh * nb + t];
    const float svt = a.sv[(int64_t)bh * nb + t];
    const float vratio = sv_prev / svt;
    sv_prev = svt;

    uint32_t p8[R][2][8];   // [qi][k-step of 64 keys][dword]
#pragma unroll
    for (int qi = 0; qi < R; ++qi) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qi][kb][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mnew = fmaxf(m_run[qi], mx * f);
      const float alpha = fast_exp2(m_run[qi] - mnew);
      const float moff = mnew - a.p_off;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int slot = 4 * w + e, kb = 2 * s + (slot >> 4), r = slot & 15;
            y[e] = fast_exp2(__builtin_fmaf(sacc[qi][kb][r], f, -moff));
          }
          p8[qi][s][w] = cvt4_e4m3(y[0], y[1], y[2], y[3]);
        }
      // Only element 0 of the row-sum accumulator is read (see below).
      lacc[qi][0] *= alpha;
      m_run[qi] = mnew;
      const float g = alpha * vratio;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qi][db][r] *= g;
    }

    // ---- A += V8^T P8^T ----
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint8_t* p = sV + (db * 32 + l32) * RS8 + 64 * s + 32 * h;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(p), hi = *reinterpret_cast<const u32x4*>(p + 16);
        const i32x8 vf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
        for (int qi = 0; qi < R; ++qi) {
          const i32x8 pf = {(int)p8[qi][s][0], (int)p8[qi][s][1], (int)p8[qi][s][2], (int)p8[qi][s][3],
                            (int)p8[qi][s][4], (int)p8[qi][s][5], (int)p8[qi][s][6], (int)p8[qi][s][7]};
          oacc[qi][db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, oacc[qi][db], 0, 0, 0, 0, 0, 0);
          // Row sum of the quantised weights on the matrix core: an all-ones
          // A operand makes every row of the 32x32 result the column sum of
          // P8, so each lane gets its query row's sum in every register.
          if (db == 0)
            lacc[qi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kOnes, pf, lacc[qi], 0, 0, 0, 0, 0, 0);
        }
      }

    if (t + 1 < nb) {
      store_tile(bf ^ 1);
      if (t + 2 < nb) load_tile(t + 2);
    }
    __syncthreads();
  }

  // ---- epilogue: O = A * sV_last / l ----
  const int64_t ob = b * a.os[0] + hd * a.os[1];
#pragma unroll
  for (int qi = 0; qi < R; ++qi) {
    const float lt = lacc[qi][0];
    const float inv = lt > 0.f ? sv_prev / lt : 0.f;
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
            f32x4 t4 = {v0, v1, v2, v3};
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d0) = t4;
          } else {
            u32x2 t2 = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
            *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.o) + orow + d0) = t2;
          }
        }
      if (a.lse != nullptr && h == 0)
        a.lse[(int64_t)bh * N + row] =
            lt > 0.f ? (m_run[qi] + __builtin_log2f(lt) - 8.8073549220576041f) * 0.69314718055994530942f
                     : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8Args& a, hipStream_t s) {
  const int64_t nwg = 3LL * a.B * a.H * a.nb;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fp8_quantize_kernel, dim3((unsigned)nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const Fp8Args& a, bool out_f32, hipStream_t s) {
  const int nqb = (a.N + 255) / 256;   // 8 waves x 32 query rows per work-group
  const int64_t nwg = (int64_t)a.B * a.H * nqb;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (out_f32) hipLaunchKernelGGL((attn_fp8_kernel<8, 1, true>), dim3((unsigned)nwg), dim3(512), 0, s, a, nqb);
  else hipLaunchKernelGGL((attn_fp8_kernel<8, 1, false>), dim3((unsigned)nwg), dim3(512), 0, s, a, nqb);
  return hipGetLastError();
}

}  // namespace dit
