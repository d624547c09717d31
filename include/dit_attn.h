/*
 * dit_attn.h -- C ABI of the dit_attn library: non-causal joint attention
 * forward for diffusion transformers on one AMD Instinct MI355X (gfx950).
 *
 * What is computed.  FLUX-family DiTs embed text tokens, noisy target-image
 * latent tokens and an optional reference image separately and then unite
 * them in one shared attention layer (bpdata.com "FLUX 3 Image Klein
 * optimalizálása", section "Modellezés és pipeline jellemzők").  That layer
 * is plain bidirectional softmax attention over the concatenated sequence:
 *
 *     O[b,h,i,:] = sum_j softmax_j(scale * <Q[b,h,i,:], K[b,h,j,:]>) V[b,h,j,:]
 *
 * with no causal mask.  The pages select among a "VANILLA" BF16 attention,
 * quantised FP8 attention, and block-sparse attention backends (scopeai.cc
 * page, section "各项优化的效果与质量代价"; bpdata.com page, section "Mi
 * szerepel az optimalizálásban"); the three attention calls below are this
 * library's versions of those three, and dit_attn_select_blocks chooses the
 * block mask for the block-sparse one.
 *
 * Conventions shared by every call.
 *  - Tensors.  Q, K, V and O are [B, H, N, D] with element strides given per
 *    tensor for (b, h, n); the d stride is 1.  Q, K, V are bfloat16.  O is
 *    bfloat16 (round to nearest even), or fp32 when DIT_ATTN_FLAG_OUT_F32 is
 *    set.  D must be 128.
 *  - Optional lse output: fp32 [B, H, N] contiguous, lse = ln sum_j
 *    exp(scale * <q_i, k_j>) over the keys the row attends to.  Pass NULL to
 *    skip it.  A row that attends to no key gets O = 0 and lse = -inf.
 *  - Pointers are device pointers.  Q, K, V, O must be 16-byte aligned; every
 *    (b, h, n) stride of Q, K, V and O must be a multiple of 8 elements, a
 *    row stride at most 2^22 elements, and one (b, h) slice must span less
 *    than 2 GiB (DIT_ATTN_ERR_UNSUPPORTED otherwise).
 *  - Ownership.  The caller owns every buffer and the stream; the library
 *    never allocates or frees memory.
 *  - Asynchrony.  Calls enqueue work on `stream` (a hipStream_t; NULL is the
 *    default stream) and return without waiting; they never read device
 *    memory from the host, so they may be captured into a HIP graph.
 *  - Errors.  All arguments are checked before any HIP call; on a bad
 *    argument nothing is launched and a nonzero dit_attn_status is returned.
 *    dit_attn_last_error() then gives a per-thread description.
 *  - Determinism.  For a fixed build, device and arguments the output is
 *    bitwise reproducible: reductions use no atomics and a fixed key order.
 *  - Thread safety.  Calls are re-entrant.  Global state: the per-thread
 *    error string, per-device caches filled once (compute-unit count, the
 *    address of dit_attn_fwd_noalloc's array) and that array itself.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dit_attn_status {
    DIT_ATTN_OK = 0,
    DIT_ATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size/stride/alignment */
    DIT_ATTN_ERR_UNSUPPORTED = 2, /* valid request this build does not cover (e.g. D != 128) */
    DIT_ATTN_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
    DIT_ATTN_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} dit_attn_status;

/* Store O as fp32 instead of bfloat16 (the arithmetic is unchanged, so the
 * bf16 output equals the round-to-nearest-even image of the fp32 output). */
#define DIT_ATTN_FLAG_OUT_F32 1u

/* Problem description.  Strides are in elements, for (b, h, n). */
typedef struct dit_attn_shape {
    int32_t batch;       /* B >= 1 */
    int32_t heads;       /* H >= 1 */
    int32_t seqlen;      /* N >= 1: text + image (+ reference) tokens */
    int32_t head_dim;    /* D, must be 128 */
    int64_t q_stride[3];
    int64_t k_stride[3];
    int64_t v_stride[3];
    int64_t o_stride[3];
    float softmax_scale; /* > 0 and finite; 1/sqrt(D) for the DiT workloads */
    uint32_t flags;      /* DIT_ATTN_FLAG_* */
} dit_attn_shape;

/* Dense bf16 joint attention (the "VANILLA BF16 attention" backend).
 * Flash-style: QK^T and PV on bf16 MFMA with fp32 accumulation, online
 * softmax in fp32, P rounded to bf16 for the PV product.  Query blocks of
 * 384 rows run one per compute unit; when their count leaves a partial last
 * round, dit_attn_fwd_ws (same result within rounding, caller workspace) is
 * faster: 4.66-4.76 against 4.98-5.01 ms at B2 H24 N16896 on 256 CUs. */
int dit_attn_fwd(const dit_attn_shape* shape,
                 const void* q, const void* k, const void* v,
                 void* o, float* lse, void* stream);

/* Workspace bytes dit_attn_fwd_ws needs for `shape` on the current device
 * (0: no split applies, the workspace may be NULL; also 0 for an invalid
 * shape).  Layout: fp32 [P][384][132], one row per query row of each of the
 * P = ntail * split tail work-groups: 128 unnormalised O values, m * scale
 * * log2(e), the row's weight sum, 2 words of padding. */
size_t dit_attn_fwd_workspace_bytes(const dit_attn_shape* shape);

/* The same attention as dit_attn_fwd (same operation, same arguments and
 * errors), with a caller workspace for load balancing: the query blocks of
 * 384 rows run one per compute unit, and those of the last, partial round
 * (the whole grid, if it is smaller than one round) are each split into key
 * ranges whose partial results (own running max,
 * unnormalised O and weight sum) are combined by a second kernel in key
 * order: O = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p with M = max m_p.
 * The workspace (device memory, 256-byte aligned, caller-owned, at least
 * dit_attn_fwd_workspace_bytes) is scratch: nothing is read from it before
 * it is written in the same call; calls that share one workspace must not
 * overlap.  Output is deterministic per device; rows of split blocks can
 * differ from dit_attn_fwd's in the last bits (P is rounded against a
 * different reference max). */
int dit_attn_fwd_ws(const dit_attn_shape* shape,
                    const void* q, const void* k, const void* v,
                    void* o, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * attention as dit_attn_fwd_ws (same arguments and errors, same kernels, same
 * split plan, bit-identical output), with the partial results of the split
 * tail blocks kept in a device array the library itself holds instead of a
 * caller workspace.  The array holds dit_attn_fwd_noalloc_scratch_bytes()
 * bytes (64 MiB) on every GPU the library runs on, until the process ends;
 * a shape whose split needs more (dit_attn_fwd_workspace_bytes(shape) above
 * that: more than about 330 compute units) is refused with
 * DIT_ATTN_ERR_WORKSPACE before anything is launched.  Nothing in the array
 * needs to start at any value (every partial result is written before it is
 * read, in the same call).  All calls on one GPU share its array: calls that
 * may overlap on one GPU (several streams, several host threads) race and
 * must be serialised by the caller.  The call allocates and frees nothing;
 * its first call on a device looks up that device's copy of the array. */
int dit_attn_fwd_noalloc(const dit_attn_shape* shape,
                         const void* q, const void* k, const void* v,
                         void* o, float* lse, void* stream);

/* Size in bytes of the device array dit_attn_fwd_noalloc uses. */
size_t dit_attn_fwd_noalloc_scratch_bytes(void);

/* Workspace bytes dit_attn_fwd_fp8 / dit_attn_fp8_quantize need for `shape`
 * (0 if the shape is invalid).  Layout, with BH = B*H, nb = ceil(N/128),
 * Np = 128*nb, each region starting at a 256-byte boundary in this order:
 *   Q8  uint8 [BH][Np][128]  e4m3 codes of Q, rows >= N are 0
 *   K8  uint8 [BH][Np][128]  e4m3 codes of K, rows >= N are 0
 *   V8t uint8 [BH][128][Np]  e4m3 codes of V transposed (d-major); within
 *       every 64-key group the 4-key groups are stored in the order the PV
 *       operand is read: position group pg holds key group
 *       8*((pg>>2)&1) + 2*(pg&3) + (pg>>3); keys >= N are 0
 *   sQ, sK, sV  fp32 [BH][nb]  dequantisation scales (absmax / 448)
 *   part  fp32 [P][256][132]  scratch of the attention's tail split (see
 *       dit_attn_fwd_ws; here in 128-key tiles, O already in V units, m in
 *       log2 units, weights in units of 1/448); present only when the grid
 *       leaves a partial round on the current device, so the size depends
 *       on that device. */
size_t dit_attn_fwd_fp8_workspace_bytes(const dit_attn_shape* shape);

/* Quantised attention with on-device dynamic scaling.  FP8 dynamic
 * quantisation of activations (wavespeed.ai FLUX.1-dev page, section "FP8
 * Dynamische Quantisierung") applied to attention: Q, K and V are quantised
 * to OCP e4m3 with one scale per (b, h, 128-token block):
 *     s = absmax / 448,  code = e4m3_rne(clamp(x * (448 / absmax), +-448))
 * (a block whose 448 / absmax is not a finite fp32 number -- absmax 0, or
 * below 448 / FLT_MAX -- gets s = 1 and zero codes).  QK^T runs on fp8
 * MFMA; the
 * online softmax keeps a running max per 128-key block; the unnormalised
 * probabilities w in [0, 1] are quantised as e4m3(448 w) for the fp8 PV
 * product, and the row sum is taken over the same quantised weights (so the
 * normalised weights sum to one); output is bf16 (or fp32).
 * The quantisation pass writes the K and V regions of the workspace (layout
 * above), then the attention pass reads them, both on `stream`; Q is
 * quantised inside the attention kernel (each of its 256-row work-groups
 * owns two whole 128-token scale blocks), with the same arithmetic and
 * codes, so the Q8 and sQ regions are left untouched (dit_attn_fp8_quantize
 * fills them).  As in dit_attn_fwd_ws, the
 * 256-row query blocks of a last partial round are split over key ranges,
 * each with its own running max, and merged with exact rescaling; their P
 * is therefore rounded against a different running max than in one pass. */
int dit_attn_fwd_fp8(const dit_attn_shape* shape,
                     const void* q, const void* k, const void* v,
                     void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The quantisation of dit_attn_fwd_fp8 alone, for Q, K and V: fills every
 * region of the workspace but the tail-split scratch (same layout) so a
 * caller can inspect or reuse the e4m3 codes and scales. */
int dit_attn_fp8_quantize(const dit_attn_shape* shape,
                          const void* q, const void* k, const void* v,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes dit_attn_fwd_blocksparse needs for `shape` on the current
 * device.  This build's block-sparse kernel keeps no state between its
 * work-groups, so the answer is 0 for every shape (the workspace may then be
 * NULL); callers should still ask, so that a later build can use the
 * workspace (for an active-block list, for instance) without an ABI change. */
size_t dit_attn_fwd_blocksparse_workspace_bytes(const dit_attn_shape* shape);

/* Block-sparse bf16 attention over 128x128 (query block, key block) tiles
 * (the "blokksparse" attention backend, bpdata.com page, section "Mi
 * szerepel az optimalizálásban").  block_mask is a device uint8 array
 * [ceil(N/128)][ceil(N/128)], row = query block, column = key block, nonzero
 * = attend.  Masked blocks act as -inf logits: they are skipped and their K
 * and V are never read.  mask_stride_bh is the element offset between the
 * masks of consecutive (b, h) slices (b-major); 0 shares one mask.  The
 * mask's size cannot be checked here: the caller guarantees that
 * (B*H - 1) * mask_stride_bh + nb * nb bytes are readable.
 * block_size must be 128.  workspace / workspace_bytes: device memory of at
 * least dit_attn_fwd_blocksparse_workspace_bytes(shape) bytes, 256-byte
 * aligned (NULL when that is 0); ERR_WORKSPACE otherwise.
 * The per-tile arithmetic is that of dit_attn_fwd (fp32 scores, P rounded
 * to bf16, row sums over the rounded P, 32-key tiles) on 128-row blocks, so
 * an all-ones mask reproduces dit_attn_fwd within the same tolerance, not
 * bit for bit (the first-tile reference differs: the two kernels group rows
 * differently). */
int dit_attn_fwd_blocksparse(const dit_attn_shape* shape,
                             const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             const uint8_t* block_mask, int64_t mask_stride_bh,
                             int32_t block_size,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes dit_attn_select_blocks needs for `shape`: the fp32
 * block means of Q and K, 2 * B * H * ceil(N/128) * 128 * 4 bytes. */
size_t dit_attn_select_blocks_workspace_bytes(const dit_attn_shape* shape);

/* Block-mask selection for dit_attn_fwd_blocksparse, in the manner of
 * Sol-Attention (a block-sparse backend whose sparsity a threshold tau
 * controls: bpdata.com page, section "Részletes optimalizációs lépések és
 * hatásuk").  The pages give no rule; the one built here estimates, for each
 * (b, h) and query block i, the share of attention each key block j draws,
 * from block-mean-pooled queries and keys:
 *     qm_i, km_j = means of q, k over the valid tokens of 128-token blocks
 *     s_ij = softmax_scale * <qm_i, km_j>,   p_ij = softmax over j of s_ij
 * and keeps block j iff p_ij >= tau / nb (at least tau times the uniform
 * share), or j == i, or i < tb, or j < tb, with nb = ceil(N/128) and
 * tb = ceil(text_tokens/128): the diagonal and the rows and columns of the
 * text blocks (the first text_tokens tokens of the joint sequence) are
 * always kept.  tau = 0 keeps every block; larger tau keeps fewer.
 * Reads q and k ([B, H, N, 128] bf16, strides from `shape`; v, o, lse and
 * the flags are not used) and writes block_mask, a device uint8 array
 * [B*H][nb][nb] (b-major, row = query block, 1 = keep), ready for
 * dit_attn_fwd_blocksparse with mask_stride_bh = nb * nb.  The shares are
 * computed in fp32 with fixed-order reductions, so a call is deterministic;
 * a share within about 1e-5 relative of tau / nb may be decided either way
 * compared with exact arithmetic.
 * tau must be finite and >= 0, text_tokens in [0, N], nb <= 4096
 * (ERR_UNSUPPORTED beyond).  workspace: device memory of at least
 * dit_attn_select_blocks_workspace_bytes(shape) bytes, 256-byte aligned
 * (ERR_WORKSPACE otherwise), overwritten.  Two kernels run on `stream`; the
 * mask is ready when the stream reaches that point. */
int dit_attn_select_blocks(const dit_attn_shape* shape,
                           const void* q, const void* k,
                           float tau, int32_t text_tokens,
                           uint8_t* block_mask,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* dit_attn_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* dit_attn_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int dit_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
