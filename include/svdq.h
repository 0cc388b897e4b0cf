/*
 * svdq.h -- C ABI of libsvdq.so, the MI355X (gfx950) hot path of the SVDQuant
 * 4-bit linear layer.
 *
 * The layer (SVDQuant notes page, hoonably.github.io/blog/svdquant, section 4.2,
 * the low-rank decomposition identity; section 4.3, Nunchaku kernel fusion):
 *
 *     Y = act( deQ(Q4(X_hat)) . deQ(Q4(R))^T  +  (X_hat L1) L2  +  b ),
 *     X_hat = X diag(lambda)^-1,
 *
 * with lambda the per-input-channel smoothing factor, L1 (K x r) and L2 (r x N)
 * the 16-bit low-rank branch, R (N x K here, nn.Linear orientation) the residual
 * quantized to 4 bits, b the bias and act the identity or GELU.  Q4 is the
 * max-scaled quantizer of section 3 applied per group of g consecutive elements
 * along K:
 *   SVDQ_MXFP4    : E2M1 codes, one E8M0 (power of two) scale per 32;
 *                   scale 2^e, e = floor(log2 amax) - 2 clamped to [-127, 127],
 *                   codes = nearest E2M1 of x / 2^e, ties to even, saturating at 6.
 *   SVDQ_INT4_G64 : two's complement codes, one fp16 scale per 64;
 *                   s = fp16(fp32(amax / 7)) (clamped to 65504),
 *                   q = clamp(rint(fp32(x / s)), -8, 7), 0 when s == 0.
 *   SVDQ_NVFP4    : the NVFP4-style format the Nunchaku in Diffusers page names
 *                   for its Blackwell kernels: E2M1 codes, one E4M3 scale per 16,
 *                   and a float32 tensor scale gs (R: gs = fp32(max|R| / 2688),
 *                   computed at packing; X_hat: gs = 1).  Group scale byte =
 *                   nearest E4M3 of fp32(fp32(amax / 6) / gs) (ties to even,
 *                   saturating at 448), S = fp32(E4M3 * gs), codes = nearest E2M1
 *                   of fp32(x / S) (ties to even, saturating at 6); signed zeros
 *                   when S == 0.  Value = E2M1 * E4M3 * gs.
 * All float32 decision arithmetic is IEEE (correctly rounded divisions).
 *
 * Two steps per layer, as section 4.3 describes: svdq_quantize_act (smooth,
 * group amax, scale, encode, pack, and the down projection X_hat L1 in the same
 * pass over X) and svdq_gemm (the block-scaled 4-bit GEMM whose epilogue adds
 * (X_hat L1) L2, the bias and the activation).  svdq_linear runs both.  The
 * quantize step is one kernel when it keeps K whole; when it splits K over
 * workgroups to fill the GPU (every FLUX shape: 12 splits at K = 3072 and at
 * K = 12288 for 4608 rows) a second small kernel sums the fp32 partials of the
 * down projection in split order, so a layer is then three launches (the sum
 * takes about 5 us at those shapes).  svdq_gemm_quant likewise ends with the
 * sum of one partial per output tile column.
 *
 * Conventions for every entry point:
 *   - Pointers named as device buffers are device pointers owned by the caller;
 *     the library never allocates, frees or synchronizes the host.
 *   - Every call enqueues its work on `stream` (a hipStream_t; NULL is the null
 *     stream) and returns without waiting for it.
 *   - Validation is synchronous and happens before any launch: on an error the
 *     outputs are untouched and nothing is enqueued.  Checks, in this order:
 *     NULL pointers, shapes, formats/flags, alignment, workspace size, then the
 *     device (the current device must be gfx950; otherwise SVDQ_ERR_DEVICE, the
 *     load-time capability check the Diffusers integration page describes).
 *   - No C++ exception crosses the ABI.  Calls that overlap on one stream are
 *     ordered; the library holds no mutable state (apart from a per-device
 *     cache of the architecture check, and svdq_linear_noalloc's static device
 *     workspace, see there) and is re-entrant.
 *
 * Shapes: K % 512 == 0, 16 <= N, N % 16 == 0, 0 <= rank <= 256, M >= 0,
 * K <= 65536, N <= 65536.  Row strides (ldx, ldy) are in elements and
 * multiples of 8 (16-byte rows); ldx <= 2^24 (the kernels address 16 rows of X
 * with 32-bit offsets), else SVDQ_ERR_SHAPE.  Device buffers must be 16-byte aligned;
 * packed weights and activation workspaces 256-byte aligned.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_NULL = 1,      /* a required pointer is NULL                         */
  SVDQ_ERR_SHAPE = 2,     /* K, N, rank, M, ldx or ldy outside the stated set    */
  SVDQ_ERR_FORMAT = 3,    /* unknown format or epilogue flag                     */
  SVDQ_ERR_ALIGN = 4,     /* a pointer or stride is not aligned as required      */
  SVDQ_ERR_WORKSPACE = 5, /* workspace smaller than svdq_act_bytes               */
  SVDQ_ERR_DEVICE = 6,    /* no device, or the current device is not gfx950      */
  SVDQ_ERR_LAUNCH = 7,    /* a kernel launch failed                              */
  SVDQ_ERR_TOO_LARGE = 8  /* svdq_linear_noalloc: the layer's workspace exceeds its static scratch */
} svdq_status;

typedef enum {
  SVDQ_MXFP4 = 1,         /* E2M1 codes, E8M0 scale per 32 along K   */
  SVDQ_INT4_G64 = 2,      /* int4 codes, fp16 scale per 64 along K   */
  SVDQ_NVFP4 = 3          /* E2M1 codes, E4M3 scale per 16 along K, fp32 tensor scale */
} svdq_format;

/* Epilogue flags of svdq_gemm / svdq_linear. */
enum {
  SVDQ_EPI_LOWRANK = 1u,  /* add (X_hat L1) L2 (ignored when rank == 0)          */
  SVDQ_EPI_BIAS = 2u,     /* add b                                              */
  SVDQ_EPI_GELU = 4u,     /* apply GELU, erf form y * Phi(y), last              */
  SVDQ_EPI_OUT_F32 = 8u   /* Y is float32 (default: bf16, round to nearest even) */
};

/* One layer: format, input features K, output features N, low-rank rank. */
typedef struct {
  int32_t fmt;
  int32_t K;
  int32_t N;
  int32_t rank;
} svdq_layer_desc;

/* Bytes of the packed weight blob for this layer; 0 if the descriptor is invalid.
 * Host-only query, no device access. */
size_t svdq_weight_bytes(const svdq_layer_desc* d);

/* Bytes of the activation workspace for M rows (packed codes, scales and the
 * down projection X_hat L1); 0 if the descriptor or M is invalid. Host-only. */
size_t svdq_act_bytes(const svdq_layer_desc* d, int64_t M);

/* Quantize and pack one layer's weights once (load time).
 * Definition: section 4.2 of the SVDQuant notes page -- R is the residual
 * diag(lambda) W - L1 L2 that is quantized to 4 bits; L1, L2 stay 16-bit.
 *   R       device, float32, N x K row-major (row n = output channel n)
 *   L1      device, bf16 bits, K x rank row-major (may be NULL iff rank == 0)
 *   L2      device, bf16 bits, rank x N row-major (may be NULL iff rank == 0)
 *   lambda  device, float32[K], smoothing factors (finite, > 0)
 *   bias    device, bf16 bits [N], or NULL for a zero bias
 *   w_packed device, svdq_weight_bytes(d) bytes, 256-byte aligned; opaque layout
 * R's codes and scales are computed on the device with the Q4 rule above.
 * Repacking with adapter factors concatenated onto L1/L2 (rank grows) leaves the
 * 4-bit residual section byte-identical (SVDQuant abstract: adapters need no
 * re-quantization). */
svdq_status svdq_pack_weight(const svdq_layer_desc* d, const float* R, const uint16_t* L1,
                             const uint16_t* L2, const float* lambda, const uint16_t* bias,
                             void* w_packed, void* stream);

/* Launch 1 (section 4.3: the down projection fused into the quantization kernel).
 *   X        device, bf16 bits, M x K with row stride ldx
 *   a_packed device, svdq_act_bytes(d, M) bytes, 256-byte aligned; receives the
 *            packed codes and scales of X_hat = X / lambda and D = X_hat L1. */
svdq_status svdq_quantize_act(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X,
                              int64_t M, int64_t ldx, void* a_packed, void* stream);

/* Launch 2 (section 4.3: the up projection fused into the 4-bit GEMM kernel).
 *   Y  device, M x N with row stride ldy; bf16 bits, or float32 with
 *      SVDQ_EPI_OUT_F32.  epi: OR of SVDQ_EPI_* flags. */
svdq_status svdq_gemm(const svdq_layer_desc* d, const void* w_packed, const void* a_packed,
                      int64_t M, void* Y, int64_t ldy, uint32_t epi, void* stream);

/* Fused MLP step: launch 2 of layer d, whose output feeds layer dn (dn->K == d->N),
 * with that output quantized for dn instead of stored.  The Nunchaku in Diffusers
 * page (section "Background: SVDQuant and Nunchaku") names fused GELU/MLP kernels
 * among the original engine's model-specific paths; this is that fusion for the
 * 4-bit layer.  The epilogue forms H = bf16(act(acc + (X_hat L1) L2 + b)) exactly
 * as svdq_gemm would store it, then smooths, quantizes and packs H for dn into
 * an_packed as svdq_quantize_act(dn, wn_packed, H, M, ...) would: the same codes
 * and scales bit for bit, and D' = H_hat L1' summed in a different (fixed) order
 * (one fp32 partial per output tile column of H, 128 or 256 columns, added in
 * column order by a second launch).  svdq_gemm(dn, wn_packed, an_packed, ...) then completes dn.  H itself
 * is never written.  The Diffusers page's kernels are INT4 (and NVFP4 on Blackwell):
 * INT4 pairs are served as well as MXFP4 ones.
 *   d, w_packed, a_packed  layer d as for svdq_gemm (a_packed from svdq_quantize_act)
 *   epi       SVDQ_EPI_LOWRANK | SVDQ_EPI_BIAS | SVDQ_EPI_GELU (no SVDQ_EPI_OUT_F32)
 *   dn, wn_packed  the next layer and its packed weights
 *   an_packed device, svdq_act_bytes(dn, M) bytes, 256-byte aligned
 * Both layers MXFP4 or both INT4 (else SVDQ_ERR_FORMAT); dn->K != d->N or dn->rank > 64 give
 * SVDQ_ERR_SHAPE; other checks and errors as svdq_gemm. */
svdq_status svdq_gemm_quant(const svdq_layer_desc* d, const void* w_packed, const void* a_packed, int64_t M,
                            uint32_t epi, const svdq_layer_desc* dn, const void* wn_packed, void* an_packed,
                            void* stream);

/* Fused QKV step: launch 2 of a layer whose N = 3 H head_dim outputs are [Q | K | V]
 * (the Nunchaku in Diffusers page, section "Quantizing your own model": the FLUX.1
 * to_qkv projection feeds one operator that also applies the Q/K normalization
 * modules and the rotary embedding).  With y = acc + (X_hat L1) L2 + b in fp32
 * (epi: SVDQ_EPI_LOWRANK and / or SVDQ_EPI_BIAS only), for every token m and every
 * Q head (weight norm_q) and K head (weight norm_k):
 *     z = y / sqrt(mean over the head's features of y^2 + eps) * w,
 *     (z[2p], z[2p+1]) -> (z[2p] c - z[2p+1] s, z[2p] s + z[2p+1] c),
 *     c = rope_cos[m][p], s = rope_sin[m][p];
 * V heads are y.  Y receives the bf16 (nearest even) result, M x N, row stride ldy.
 *   head_dim  must be 128; N a multiple of 384; any of the three formats (the
 *             Diffusers page names INT4 and NVFP4 kernels; the epilogue is the same)
 *   norm_q, norm_k  device, bf16 bits [128], 16-byte aligned
 *   eps       in [0, 1]
 *   rope_cos, rope_sin  device, float32, M x 64 row-major (angle of pair p of token m),
 *             16-byte aligned
 * Other checks and errors as svdq_gemm. */
svdq_status svdq_gemm_qkv(const svdq_layer_desc* d, const void* w_packed, const void* a_packed, int64_t M,
                          uint32_t epi, int32_t head_dim, const uint16_t* norm_q, const uint16_t* norm_k, float eps,
                          const float* rope_cos, const float* rope_sin, void* Y, int64_t ldy, void* stream);

/* 4-bit weights with 16-bit activations (W4A16), the Nunchaku in Diffusers page,
 * section "Introducing Nunchaku Lite": the memory-bound modulation projections
 * keep bf16 inputs and read INT4 weights.  One launch computes
 *     Y = X deQ(Q4(W))^T (+ b),  fp32 sums of exact bf16 products,
 * Y written as bf16 (nearest even), or float32 with SVDQ_EPI_OUT_F32.  The weights
 * are an INT4-g64, rank-0 blob from svdq_pack_weight with R = W; its lambda is not
 * applied (an AWQ-style per-channel scale is folded into W and the previous
 * operation, so pack with lambda = 1).  The kernel is built for few tokens (it
 * streams all weights once per 16 tokens); any M is computed correctly.
 *   X  device, bf16 bits, M x K, row stride ldx (K <= ldx <= 2^24, multiple of 8),
 *      16-byte aligned
 *   Y  device, M x N, row stride ldy (>= N, multiple of 8), 16-byte aligned
 *   epi  SVDQ_EPI_BIAS and / or SVDQ_EPI_OUT_F32
 * d->fmt other than SVDQ_INT4_G64, d->rank != 0 or other epilogue flags give
 * SVDQ_ERR_FORMAT; other checks and errors as svdq_gemm. */
svdq_status svdq_gemm_w4a16(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X, int64_t M,
                            int64_t ldx, void* Y, int64_t ldy, uint32_t epi, void* stream);

/* Both launches; workspace >= svdq_act_bytes(d, M) bytes (device, 256-aligned). */
svdq_status svdq_linear(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X,
                        int64_t M, int64_t ldx, void* Y, int64_t ldy, uint32_t epi,
                        void* workspace, size_t ws_bytes, void* stream);

/* svdq_linear for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments as svdq_linear minus the workspace, same kernels and the same
 * result bits; the activation workspace instead lives in a static device array
 * of 64 MiB inside the library (one per GPU, allocated with the library's code
 * on that GPU and held until the process ends; no call allocates or frees
 * anything).  A layer whose workspace (codes, scales, the down projection and
 * its K-split partials: about M (K/2 + K/32 + 4 r) bytes plus the partials)
 * exceeds 64 MiB gives SVDQ_ERR_TOO_LARGE before anything is enqueued; the FLUX
 * shapes need at most 38 MiB (M = 4608, K = 12288).  Every call on a GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialized by the caller.  Each call
 * overwrites every byte it reads, so the previous call's contents never matter. */
svdq_status svdq_linear_noalloc(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X,
                                int64_t M, int64_t ldx, void* Y, int64_t ldy, uint32_t epi, void* stream);

/* Test access to the opaque layouts, in canonical form (device outputs, any may be NULL):
 *   codes   uint8 rows x K/2: two 4-bit codes per byte, element 2j in the low nibble
 *           of byte j (INT4 codes as 4-bit two's complement)
 *   scales  rows x K/32 uint8 E8M0 bytes (MXFP4), rows x K/64 uint16 fp16 bits (INT4)
 *           or rows x K/16 uint8 E4M3 bytes (NVFP4)
 *   weight: L1 (K x rank bf16), L2 (rank x N bf16), lambda (float32[K]), bias (bf16[N])
 *   act:    D (M x rank float32, the down projection as the GEMM epilogue consumes it) */
svdq_status svdq_unpack_weight(const svdq_layer_desc* d, const void* w_packed, uint8_t* codes,
                               void* scales, uint16_t* L1, uint16_t* L2, float* lambda,
                               uint16_t* bias, void* stream);
svdq_status svdq_unpack_act(const svdq_layer_desc* d, const void* a_packed, int64_t M,
                            uint8_t* codes, void* scales, float* D, void* stream);

/* Static string for a status code (never NULL). */
const char* svdq_status_str(svdq_status s);

/* SVDQ_OK if the current device is gfx950, else SVDQ_ERR_DEVICE. */
svdq_status svdq_device_check(void);

/* ABI version of this header (major * 100 + minor). */
int svdq_version(void);

/* Test hook: with a nonzero argument every later device check reports
 * SVDQ_ERR_DEVICE (until called again with 0), so that error path can be
 * exercised on a machine whose GPU would pass the check.  Process-wide. */
void svdq_test_force_device_error(int on);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
