// Launch 2 of the layer: the 4-bit GEMM with the low-rank up projection, the
// bias and the activation folded into its epilogue (section 4.3 of the SVDQuant
// notes page: the up projection is fused into the 4-bit computation kernel, so
// the low-rank branch adds no extra pass over the output).
//
//   acc[n, m] = sum_g sW[n, g] sX[m, g] sum_{k in g} qW[n, k] qX[m, k]   (section 3's
//               scaled product, one scale pair per group along K)
//   acc      += sum_i L2[i, n] D[m, i]          (D = X_hat L1, bf16 hi + lo)
//   Y[m, n]   = act(acc + b[n])
//
// Orientation: the MFMA A operand is the weight (rows n), B the activation (columns
// m); a lane's 4 accumulators are 4 consecutive n of one m, i.e. one 8-byte
// (bf16) or 16-byte (fp32) store into row-major Y.
//
// MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands and the E8M0
// scales applied by the instruction (scale byte of the K step picked by op_sel).
// INT4: codes unpacked to int8 in registers, v_mfma_i32_16x16x64_i8 per 64-group,
// then int32 -> fp32 times sW * sX accumulated in fp32.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "svdq.h"
#include "common.h"

namespace svdq {

struct GemmArgs {
  const uint8_t* wblob;
  const uint8_t* act;
  size_t w_codes, w_scales, w_L2, w_bias, w_amax;
  size_t a_codes, a_scales, a_D;
  int64_t N_pad, M_pad, M, ldy;
  int K, N, r_pad;
  uint32_t epi;
  void* Y;
  // Fused QKV epilogue: Q/K normalization weights (bf16[128]), eps, and the
  // rotary cos / sin per token and pair (fp32, M x 64).
  const uint16_t* norm_q;
  const uint16_t* norm_k;
  const float* rope_cos;
  const float* rope_sin;
  float eps;
  // Output quantized for the next layer instead of Y (its K is N): that layer's
  // packed weights (lambda, 1/lambda, the correction, L1, flags) and activation
  // workspace (codes, scales, down-projection partials).
  const uint8_t* nblob;
  uint8_t* nact;
  size_t n_lam, n_rlam, n_rlo, n_L1, n_flags;
  size_t n_codes, n_scales, n_part;
  int nr_pad;
};

// ------------------------------------------------------------------ epilogue pieces

// bf16 output staging: one row of a wave tile (WN * 16 outputs) plus 16 bytes of padding
// against LDS bank conflicts; 32 rows per wave at a time.
template <int WN>
constexpr int stage_row_bytes() { return WN * 32 + 16; }

// acc += (X_hat L1) L2 over the wave tile: bf16 MFMAs of L2 (A) against D hi and lo (B).
// ROWCHECK (short tiles only): skip the blocks past the padded rows.
template <int WN, int WM, bool ROWCHECK = false>
__device__ __forceinline__ void add_lowrank(const GemmArgs& g, v4f (&acc)[WN][WM], int64_t n0, int64_t m0,
                                            int lane) {
  if (!(g.epi & SVDQ_EPI_LOWRANK) || g.r_pad == 0) return;
  const int R32 = g.r_pad / 32;
  const uint4* L2f = reinterpret_cast<const uint4*>(g.wblob + g.w_L2) + (n0 / 16) * R32 * 64 + lane;
  const uint4* Df = reinterpret_cast<const uint4*>(g.act + g.a_D) + (m0 / 16) * R32 * 128 + lane;
  const int64_t jend = g.M_pad / 16 - m0 / 16;   // blocks of this wave inside the padded rows
  for (int r32 = 0; r32 < R32; ++r32) {
    uint4 l2[WN];
#pragma unroll
    for (int i = 0; i < WN; ++i) l2[i] = L2f[(i * R32 + r32) * 64];
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      if (ROWCHECK && j >= jend) break;
      const uint4 dh = Df[(j * R32 + r32) * 128];
      const uint4 dl = Df[(j * R32 + r32) * 128 + 64];
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        acc[i][j] = mfma_bf16(l2[i], dh, acc[i][j]);
        acc[i][j] = mfma_bf16(l2[i], dl, acc[i][j]);
      }
    }
  }
}

// Bias of the lane's 4 consecutive outputs in each of the WN blocks (zero without BIAS).
template <int WN>
__device__ __forceinline__ void load_bias(const GemmArgs& g, int64_t n0, int lane, float (&bv)[WN][4]) {
  const uint16_t* bias = reinterpret_cast<const uint16_t*>(g.wblob + g.w_bias);
  const bool use_bias = (g.epi & SVDQ_EPI_BIAS) != 0;
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    uint2 braw = make_uint2(0u, 0u);
    if (use_bias) braw = *reinterpret_cast<const uint2*>(bias + n0 + i * 16 + (lane >> 4) * 4);
    bv[i][0] = bf_lo(braw.x); bv[i][1] = bf_hi(braw.x); bv[i][2] = bf_lo(braw.y); bv[i][3] = bf_hi(braw.y);
  }
}

// Y = act(acc (+ bias)) for the wave tile.  fp32 output: one 16-byte store per
// lane and block.  bf16 output: each pair of 16-row blocks (the last block alone
// when their number is odd) goes through the wave's LDS staging area, so that
// every store instruction writes whole 256-byte row segments.
template <int WN, int WM, bool OUT_F32, bool GELU, bool ADD_BIAS>
__device__ __forceinline__ void store_out(const GemmArgs& g, v4f (&acc)[WN][WM], const float (&bv)[WN][4],
                                          int64_t n0, int64_t m0, int lane, uint8_t* stage) {
  auto act = [&](int i, int j, float (&y)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = ADD_BIAS ? acc[i][j][e] + bv[i][e] : acc[i][j][e];
      if (GELU) y[e] = gelu_erf(y[e]);
    }
  };
  if constexpr (OUT_F32) {
    const bool full = (m0 + WM * 16 <= g.M) && (n0 + WN * 16 <= g.N);
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int64_t n = n0 + i * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        const int64_t m = m0 + j * 16 + (lane & 15);
        float y[4];
        act(i, j, y);
        if (full || (m < g.M && n < g.N))
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(g.Y) + m * g.ldy + n) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
  } else {
    constexpr int RB = stage_row_bytes<WN>();
    constexpr int LPR = WN * 2;          // lanes per row (16 bytes each)
    constexpr int RPI = 64 / LPR;        // rows per store instruction
    static_assert(16 % RPI == 0, "wave tile shape");
#pragma unroll
    for (int jp = 0; jp < (WM + 1) / 2; ++jp) {
      const int nj = 2 * jp + 2 <= WM ? 2 : 1;   // blocks in this pair (1 for the last of an odd count)
#pragma unroll
      for (int jj = 0; jj < nj; ++jj) {
        const int j = 2 * jp + jj;
        uint8_t* row = stage + (jj * 16 + (lane & 15)) * RB + (lane >> 4) * 8;
#pragma unroll
        for (int i = 0; i < WN; ++i) {
          float y[4];
          act(i, j, y);
          *reinterpret_cast<uint2*>(row + i * 32) = make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]));
        }
      }
#pragma unroll
      for (int r = 0; r < nj * 16 / RPI; ++r) {
        const int rr = r * RPI + lane / LPR;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + rr * RB + (lane % LPR) * 16);
        const int64_t m = m0 + jp * 32 + rr;
        const int64_t n = n0 + (lane % LPR) * 8;
        if (m < g.M && n < g.N)
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(g.Y) + m * g.ldy + n) = v;
      }
    }
  }
}

// Output quantized for the next layer (the fused MLP step: the next row after
// the layer itself; the Nunchaku in Diffusers page, section "Background:
// SVDQuant and Nunchaku", names fused GELU/MLP kernels among the original
// engine's model-specific paths).  H = bf16(act(acc + b)) is the next layer's
// input X (its K is this layer's N).  Instead of storing H, the workgroup
// quantizes its tile of H (256 x 256 or 128 x 128) for the next layer exactly
// as the activation kernel does with H read from memory (same rounding of H,
// same quotients, group maxima, scales and codes), and writes its tile's share
// of the next layer's down projection H_hat L1' as one fp32 partial per tile
// column (summed in column order by a second launch).
//
// Phase 1: each wave writes its block of H (bf16) into LDS, the workgroup's
// TC = 32 WN columns of each row in 64-row ring slots (TC * 2 bytes per row,
// 16-byte chunks swizzled by the row against bank conflicts).  Phase 2: wave
// w quantizes rows 8 WM w .. 8 WM w + 8 WM - 1 of the tile from LDS in the
// activation kernel's lane layout (lane = row % 16 + 16 c holds 8 consecutive
// elements of each 32-block), 64 columns per step.

// Byte offset of bf16 element (row % 64, column k) of the tile in its slot.
template <int WN>
__device__ __forceinline__ uint32_t htile_off(int row, int k) {
  constexpr int CH = 4 * WN;                        // 16-byte chunks per row
  return uint32_t((row & 63) * (CH * 16) + (((k >> 3) ^ (row & (CH - 1))) << 4) + (k & 7) * 2);
}

template <int WN, int WM, bool GELU>
__device__ __forceinline__ void stage_h(v4f (&acc)[WN][WM], const float (&bv)[WN][4], int lane, int wn, int wm,
                                        uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3) {
  const int q = lane >> 4, r = lane & 15;
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const int row0 = wm * 16 * WM + j * 16;          // first row of the block within the workgroup tile
    const int si = row0 >> 6;                        // its slot
    uint8_t* const sl = si == 0 ? s0 : si == 1 ? s1 : si == 2 ? s2 : s3;
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = acc[i][j][e] + bv[i][e];
        if (GELU) y[e] = gelu_erf(y[e]);
      }
      *reinterpret_cast<uint2*>(sl + htile_off<WN>(row0 + r, wn * 16 * WN + i * 16 + q * 4)) =
          make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]));
    }
  }
}

// The next layer's L1' fragments (B operands of its down projection) for the
// tile's NB 32-blocks and R16 rank tiles, into registers ahead of phase 2 (so
// that no global load, which would also wait for the stores before it, sits
// inside phase 2).
template <int R16, int NB>
__device__ __forceinline__ void load_l1_next(const GemmArgs& g, int k0, int lane, uint4 (&l1r)[NB][R16 > 0 ? R16 : 1]) {
  const uint4* const l1f = reinterpret_cast<const uint4*>(g.nblob + g.n_L1);
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int cb = 0; cb < R16; ++cb) l1r[kb][cb] = l1f[(size_t(k0 / 32 + kb) * R16 + cb) * 64 + lane];
}

// Phase 2 loop for wave w: rows mrow0 .. mrow0 + 8 WN - 1 of the output, rows
// rbase .. of the slot.  lamv holds lambda, 1/lambda and the correction term of
// the tile's TC columns (the next layer's K range k0 .. k0 + TC - 1).  FAST:
// every quotient by the two-operation form fma(x, r, x rl); otherwise by IEEE
// division.  Both give the correctly rounded quotient wherever FAST is chosen
// (see quant_h).
template <int WN, int R16, bool FAST, int NFMT>
__device__ __forceinline__ void quant_rows(const GemmArgs& g, const uint8_t* slot, int rbase, const float* lamv,
                                           int lane, int64_t mrow0, int k0, int tn,
                                           const uint4 (&l1r)[WN][R16 > 0 ? R16 : 1]) {
  constexpr int TC = 32 * WN;                       // columns of the tile
  constexpr int RT = WN / 2;                        // 16-row tiles per wave (8 WN rows)
  constexpr int ST = TC / 64;                       // 64-column steps
  const int r = lane & 15, c = lane >> 4;
  const int K2 = g.N;
  uint8_t* const codes = g.nact + g.n_codes;
  uint8_t* const scales = g.nact + g.n_scales;
  float* const part = reinterpret_cast<float*>(g.nact + g.n_part);
  const float* const slam = lamv;
  const float* const srl = lamv + TC;
  const float* const srlo = lamv + 2 * TC;

  for (int t = 0; t < RT; ++t) {                    // the wave's 16-row tiles
    const int row = rbase + t * 16 + r;              // row within the slot
    const int64_t m = mrow0 + t * 16 + r;
    v4f dacc[R16 > 0 ? R16 : 1];
#pragma unroll
    for (int cb = 0; cb < R16; ++cb) dacc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < ST; ++s) {                   // 64 columns per step
      float ah[2][8], x[16];
      unpack_bf8(*reinterpret_cast<const uint4*>(slot + htile_off<WN>(row, s * 64 + c * 8)), ah[0]);
      unpack_bf8(*reinterpret_cast<const uint4*>(slot + htile_off<WN>(row, s * 64 + 32 + c * 8)), ah[1]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kl = s * 64 + (e >> 3) * 32 + c * 8 + (e & 7);
        const float a = ah[e >> 3][e & 7];
        x[e] = FAST ? fmaf(a, srl[kl], a * srlo[kl]) : a / slam[kl];
      }
      if constexpr (NFMT == kFmtMXFP4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kb = (k0 + s * 64 + h * 32) / 32;  // block index in the next layer's K
          float amax = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[8 * h + e]));
          amax = rowgroup_max(amax);
          const uint32_t sb = e8m0_of_amax(amax);
          const float so = scale_operand(sb);
          uint32_t cw = 0;
          cw = cvt_fp4x2_div<0>(cw, x[8 * h + 0], x[8 * h + 1], so);
          cw = cvt_fp4x2_div<1>(cw, x[8 * h + 2], x[8 * h + 3], so);
          cw = cvt_fp4x2_div<2>(cw, x[8 * h + 4], x[8 * h + 5], so);
          cw = cvt_fp4x2_div<3>(cw, x[8 * h + 6], x[8 * h + 7], so);
          // lane chunk (kb & 3) * 16 + row of the 128-K step, bytes 4c .. 4c+3
          *reinterpret_cast<uint32_t*>(codes + code_chunk(m / 16, kb / 4, K2, (kb & 3) * 16 + r) + c * 4) = cw;
          if (c == (kb & 3)) scales[mx_scale_byte(m, kb, K2)] = uint8_t(sb);
        }
      } else {
        // INT4: the step is one 64-group, the activation kernel's rule: fp16
        // scale amax / 7, codes rint(x / s) clamped to [-8, 7] (0 when s is 0)
        const int kg = (k0 + s * 64) / 64;             // group index in the next layer's K
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
        amax = rowgroup_max(amax);
        const _Float16 h16 = (_Float16)fminf(amax / 7.0f, 65504.0f);
        const float sc = (float)h16;
        const float rs = 1.0f / sc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = FAST ? div_refined(x[8 * h + e], sc, rs) : x[8 * h + e] / sc;
          uint32_t cw = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float tq = __builtin_rintf(fminf(fmaxf(t[e], -8.0f), 7.0f));
            const int q = (sc == 0.0f) ? 0 : int(tq);
            cw |= (uint32_t(q) & 0xFu) << (8 * (e & 3) + 4 * (e >> 2));  // INT4 dword order
          }
          // group offset o = 32h + 8c: lane chunk (o / 16) * 16 + row, bytes 8 (g % 2) + (o % 16) / 2
          *reinterpret_cast<uint32_t*>(codes + code_chunk(m / 16, kg / 2, K2, (2 * h + c / 2) * 16 + r) +
                                       (kg & 1) * 8 + (c & 1) * 4) = cw;
        }
        if (c == 0) *reinterpret_cast<_Float16*>(scales + i4_scale_byte(m, kg, g.M_pad)) = h16;
      }
      if (R16 > 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // down projection: x_hat as a bf16 hi + lo pair against the next layer's L1 fragments
          uint4 hi, lo;
          hi.x = cvt_bf2(x[8 * h + 0], x[8 * h + 1]);
          hi.y = cvt_bf2(x[8 * h + 2], x[8 * h + 3]);
          hi.z = cvt_bf2(x[8 * h + 4], x[8 * h + 5]);
          hi.w = cvt_bf2(x[8 * h + 6], x[8 * h + 7]);
          lo.x = cvt_bf2(x[8 * h + 0] - bf_lo(hi.x), x[8 * h + 1] - bf_hi(hi.x));
          lo.y = cvt_bf2(x[8 * h + 2] - bf_lo(hi.y), x[8 * h + 3] - bf_hi(hi.y));
          lo.z = cvt_bf2(x[8 * h + 4] - bf_lo(hi.z), x[8 * h + 5] - bf_hi(hi.z));
          lo.w = cvt_bf2(x[8 * h + 6] - bf_lo(hi.w), x[8 * h + 7] - bf_hi(hi.w));
#pragma unroll
          for (int cb = 0; cb < R16; ++cb) {
            dacc[cb] = mfma_bf16(hi, l1r[2 * s + h][cb], dacc[cb]);
            dacc[cb] = mfma_bf16(lo, l1r[2 * s + h][cb], dacc[cb]);
          }
        }
      }
    }
    // lane holds rows (lane / 16) * 4 + e, rank column cb * 16 + lane % 16 of the tile
#pragma unroll
    for (int cb = 0; cb < R16; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t mm = mrow0 + t * 16 + (lane >> 4) * 4 + e;
        part[(size_t(tn) * g.M_pad + mm) * g.nr_pad + cb * 16 + r] = dacc[cb][e];
      }
  }
}

// Phase 2 for wave w.  The smoothing quotients must be the IEEE ones.  The
// two-operation form gives them when every lambda is in [2^-32, 2^32] and passed
// the packing-time check, and every value of H is +0 or in [2^-40, 2^60) in
// magnitude (the activation kernel's conditions); a first pass over the wave's
// rows checks the values, and a wave with any value outside takes IEEE division
// for all of its rows (same quotients, slower).
template <int WN, int R16, int NFMT = kFmtMXFP4>
__device__ __forceinline__ void quant_h(const GemmArgs& g, const uint8_t* slot, int rbase, const float* lamv, int lane,
                                        int64_t mrow0, int k0, int tn, const uint4 (&l1r)[WN][R16 > 0 ? R16 : 1]) {
  const int r = lane & 15, c = lane >> 4;
  const uint32_t wf = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(g.nblob + g.n_flags));
  bool oor = false;
#pragma unroll
  for (int t = 0; t < WN / 2; ++t)
#pragma unroll
    for (int s = 0; s < WN / 2; ++s)
      oor = oor || exp_out_of_range(
                       *reinterpret_cast<const uint4*>(slot + htile_off<WN>(rbase + t * 16 + r, s * 64 + c * 8)),
                       *reinterpret_cast<const uint4*>(slot + htile_off<WN>(rbase + t * 16 + r, s * 64 + 32 + c * 8)));
  const bool fast = (wf & (kLamRangeBit | kDivSlowBit)) == 0 && !__any(oor);
  if (__builtin_expect(fast, 1))
    quant_rows<WN, R16, true, NFMT>(g, slot, rbase, lamv, lane, mrow0, k0, tn, l1r);
  else
    quant_rows<WN, R16, false, NFMT>(g, slot, rbase, lamv, lane, mrow0, k0, tn, l1r);
}

// Fused QKV epilogue (the next row after the layer: the Nunchaku in Diffusers
// page, section "Quantizing your own model", describes the grouped to_qkv
// projection whose output one fused operator normalizes (norm_q, norm_k) and
// rotates (rotary embedding)).  The N = 3 H 128 outputs are [Q | K | V] and a
// wave's 128 columns are one head.  For a Q or K head each row is
// RMS-normalized over the head, y / sqrt(mean(y^2) + eps) * w, and each pair of
// consecutive features (2p, 2p + 1) is rotated by the row token's angle for p:
// (a, b) -> (a cos - b sin, a sin + b cos).  All in fp32 from the accumulators
// (bias included), one bf16 rounding at the store; V heads are stored as is.
template <int WN, int WM>
__device__ __forceinline__ void store_qkv(const GemmArgs& g, v4f (&acc)[WN][WM], const float (&bv)[WN][4],
                                          int64_t n0, int64_t m0, int lane, int w, uint8_t* stage) {
  // WN == 8: a wave's 128 columns are one head.  WN == 4: a head is the 128
  // columns of the workgroup, split between waves w and w ^ 1, whose partial
  // sums of squares meet in LDS.
  static_assert(WN == 8 || WN == 4, "a head is one wave's or two waves' columns");
  const int q = lane >> 4;
  const int64_t hd = g.N / 3;
  const int seg = int(n0 / hd);                 // 0: Q, 1: K, 2: V (uniform for the workgroup)
  const int fo = int(n0 % 128);                 // the wave's first feature within its head
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] += bv[i][e];
  if (seg < 2) {
    const uint16_t* const wnorm = seg == 0 ? g.norm_q : g.norm_k;
    float wv[WN][4];
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const uint2 u = *reinterpret_cast<const uint2*>(wnorm + fo + 16 * i + 4 * q);
      wv[i][0] = bf_lo(u.x); wv[i][1] = bf_hi(u.x); wv[i][2] = bf_lo(u.y); wv[i][3] = bf_hi(u.y);
    }
    // cos / sin of the lane's row in 16-row tile j: features fo + 16 i + 4 q + e
    // are pairs p = fo / 2 + 8 i + 2 q (e = 0, 1) and p + 1 (e = 2, 3); loaded one
    // tile ahead
    float2 cb[2][WN], sbuf[2][WN];
    auto load_rot = [&](int j, float2 (&c)[WN], float2 (&sn)[WN]) {
      const int64_t m = m0 + 16 * j + (lane & 15);
      const int64_t mc = m < g.M ? m : g.M - 1;  // rows past M are not stored
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        c[i] = *reinterpret_cast<const float2*>(g.rope_cos + mc * 64 + fo / 2 + 8 * i + 2 * q);
        sn[i] = *reinterpret_cast<const float2*>(g.rope_sin + mc * 64 + fo / 2 + 8 * i + 2 * q);
      }
    };
    // sum of squares of each token's features in this wave
    auto sumsq = [&](int j) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(acc[i][j][e], acc[i][j][e], ss);
      return rowgroup_sum(ss);
    };
    // WN == 4: plus the partner wave's half of the head, through LDS
    float ssum[WN == 4 ? WM : 1];
    if constexpr (WN == 4) {
      __shared__ float part_ss[4][WM][16];
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        ssum[j] = sumsq(j);
        if (q == 0) part_ss[w][j][lane & 15] = ssum[j];
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < WM; ++j) ssum[j] += part_ss[w ^ 1][j][lane & 15];
    }
    load_rot(0, cb[0], sbuf[0]);
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      if (j + 1 < WM) load_rot(j + 1, cb[(j + 1) & 1], sbuf[(j + 1) & 1]);
      float ss;
      if constexpr (WN == 4)
        ss = ssum[j];
      else
        ss = sumsq(j);
      const float inv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + g.eps);
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        const float2 c = cb[j & 1][i], sn = sbuf[j & 1][i];
        const float y0 = acc[i][j][0] * inv * wv[i][0], y1 = acc[i][j][1] * inv * wv[i][1];
        const float y2 = acc[i][j][2] * inv * wv[i][2], y3 = acc[i][j][3] * inv * wv[i][3];
        acc[i][j][0] = y0 * c.x - y1 * sn.x;
        acc[i][j][1] = y0 * sn.x + y1 * c.x;
        acc[i][j][2] = y2 * c.y - y3 * sn.y;
        acc[i][j][3] = y2 * sn.y + y3 * c.y;
      }
    }
  }
  store_out<WN, WM, false, false, false>(g, acc, bv, n0, m0, lane, stage);
}

// Whole epilogue after the main loop: low-rank MFMAs first (their operand loads
// come before any store; LOWRANK false when the kernel started from them), then
// every bias value, then bias + activation + conversion + stores with no loads
// in between (the vector-memory counter also counts stores, so a load waited on
// among the stores would wait for them).
template <int WN, int WM, bool OUT_F32, bool GELU, bool LOWRANK = true, bool ROWCHECK = false>
__device__ __forceinline__ void epilogue(const GemmArgs& g, v4f (&acc)[WN][WM], int64_t n0, int64_t m0, int lane,
                                         uint8_t* stage) {
  if (LOWRANK) add_lowrank<WN, WM, ROWCHECK>(g, acc, n0, m0, lane);
  float bv[WN][4];
  load_bias<WN>(g, n0, lane, bv);
  store_out<WN, WM, OUT_F32, GELU, true>(g, acc, bv, n0, m0, lane, stage);
}

// ------------------------------------------------------------------ MXFP4
//
// 256 threads = 4 waves (1 per SIMD, so each has the full register file), workgroup
// tile 256 (n) x 256 (m), wave tile 128 (n) x 128 (m) = 8 x 8 MFMA blocks with the
// accumulators in AGPRs.  A stage (one 128-K step) is 16 weight and 16 activation
// fragments, 32 KiB.  LDS holds a ring of four stages, filled by buffer loads
// that write LDS directly (no staging registers), so a fetch has two steps to
// land.  In step t a wave
//   - issues its 8 fragment loads of stage t+3 into ring slot (t+3) % 4,
//   - runs the 64 MFMAs of stage t from registers, and reads each of its 16
//     fragments of stage t+1 from slot (t+1) % 4 into the register that the
//     finished MFMAs no longer need,
//   - waits for its loads issued before this step (stage t+2) and for its LDS
//     reads, then joins the workgroup barrier.
// Slot (t+3) % 4 last held stage t-1, read during step t-2; slot (t+1) % 4 was
// loaded during step t-2 and every wave waited for its share before the
// barrier of step t-1.  Slots are separate LDS arrays indexed by compile-time
// constants, so the compiler can tell the loads into one slot from the reads
// of another and adds no waits of its own.  The E8M0 scales of a 512-K
// superfragment (one dword per lane and 16-row tile) are loaded one
// superfragment ahead; the MFMA of step u of the superfragment picks byte u.
// The 128 x 128 tiles also come with a three-slot ring (NS = 3, 48 KiB, three
// workgroups per CU): there step t reads its own fragments first and loads
// stage t+2 into the slot of stage t-1.  The same ring serves 256 (n) x 128 (m)
// tiles of 8 x 4 blocks per wave (a stage of 16 weight and 8 activation
// fragments, 72 KiB, two workgroups per CU).


__device__ __forceinline__ uint4 load_frag(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const v4i v = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  return make_uint4(uint32_t(v[0]), uint32_t(v[1]), uint32_t(v[2]), uint32_t(v[3]));
}

// One fragment (64 lanes x 16 bytes) from global memory straight into LDS at
// `dst` (wave-uniform).
__device__ __forceinline__ void load_frag_lds(__amdgpu_buffer_rsrc_t r, uint4* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst), 16, voff, soff, 0, 0);
}

// Wait until at most VM vector-memory operations of this wave are in flight and
// its LDS operations are done, then a workgroup barrier without a memory fence
// (a fence would wait for every load in flight); the empty asm keeps the
// compiler from moving memory accesses across it.
template <int VM>
__device__ __forceinline__ void wait_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Tile order of a grid that covers the whole output (tiles_n x tiles_m tiles):
// groups of kRasterCols output columns, consecutive tiles walking a group's
// columns first, then its rows, so the workgroups an XCD runs at once (t from
// xcd_remap: a contiguous range per XCD) share a few weight and activation
// panels in that XCD's L2.
constexpr int kRasterCols = 8;
__device__ __forceinline__ void raster_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int grp = t / (kRasterCols * tiles_m), in = t % (kRasterCols * tiles_m);
  const int gcols = tiles_n - grp * kRasterCols < kRasterCols ? tiles_n - grp * kRasterCols : kRasterCols;
  tn = grp * kRasterCols + in % gcols;
  tm = in / gcols;
}

template <int WN, int WM, bool OUT_F32, bool GELU, int QOUT = -1, bool QKV = false, int WMA = WM, int NS = 4>
__global__ void __launch_bounds__(256, WN == 8 ? (NS == 3 ? 2 : 1) : (NS == 3 ? 3 : 2)) gemm_mxfp4_kernel(GemmArgs g) {
  // NS = 3: a three-slot ring (48 KiB) so that three workgroups share a CU;
  // each step reads its own fragments at its start (128 x 128 tiles; the fused
  // output quantization up to a next-layer rank of 32, the fused QKV epilogue).
  // 256 x 128 tiles (8 x 4 blocks per wave) take a three-slot ring of 72 KiB,
  // two workgroups per CU.
  constexpr bool RECT = WN == 8 && WM == 4;
  static_assert(NS == 4 || (NS == 3 && WN == 4 && QOUT <= 2) || (NS == 3 && RECT && QOUT < 0 && !QKV),
                "three-slot ring: 128 x 128 or 256 x 128 tiles");
  static_assert((WN == WM && (WN == 8 || WN == 4)) || (RECT && NS == 3), "wave tiles of 8 x 8, 4 x 4 or 8 x 4 blocks");
  static_assert(!QKV || (QOUT < 0 && !OUT_F32 && !GELU), "the QKV epilogue stores bf16 with no activation");
  // Short tiles: WMA < WM active activation blocks per wave, a 256 x 32 WMA tile.
  static_assert(WMA == WM || (WN == 8 && QOUT < 0 && !QKV && WMA > WM / 2 && WMA < WM), "short tiles");
  constexpr int SF = 2 * WN;            // weight fragments per stage
  constexpr int SFB = 2 * WM;           // activation fragments per stage
  constexpr int PW = SF / 4;            // weight fragments that each wave fetches per stage
  constexpr int PWB = SFB / 4;          // activation fragments that each wave fetches per stage
  constexpr int FW = PW + PWB;          // fragment loads per wave and stage
  constexpr int SU4 = (SF + SFB) * 64;  // uint4 per stage (weights, then activations)
  static_assert(FW <= WN, "each wave row issues at most one fragment load per step");
  __shared__ uint4 ring0[SU4], ring1[SU4], ring2[SU4], ring3[NS == 4 ? SU4 : 1];   // 4 x 32 KiB (8 x 8) or 4 x 16 KiB
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = w & 1, wm = w >> 1;               // 2 x 2 waves
  constexpr int BN = 32 * WN, BM = 32 * WMA;
  const int tiles_m = int((g.M_pad + BM - 1) / BM);
  int tm, tn;
  {
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    raster_tile(t, tiles_m, int(g.N_pad / BN), tm, tn);
  }
  const int64_t nt0 = int64_t(tn) * (BN / 16);    // first 16-row weight tile of the workgroup
  const int64_t mt0 = int64_t(tm) * (BM / 16);
  const int KS = g.K / kKStep, KSUP = g.K / kKSuper;
  const int64_t n0 = (nt0 + wn * WN) * 16;
  const int64_t m0 = (mt0 + wm * WMA) * 16;
  auto slot = [&](int u) -> uint4* {
    if constexpr (NS == 3)
      return u == 0 ? ring0 : u == 1 ? ring1 : ring2;
    else
      return u == 0 ? ring0 : u == 1 ? ring1 : u == 2 ? ring2 : ring3;
  };

  // Per-workgroup views of the operands: SF row tiles of codes and of scales each.
  // A stage always holds SF activation fragments; with short tiles the last
  // 2 (WM - WMA) are not read, and the view stops at the padded rows (loads
  // past it return zeros; those rows are never stored).
  const int64_t act_rt = g.M_pad / 16 - mt0 < SFB ? g.M_pad / 16 - mt0 : SFB;
  const uint32_t code_bytes = uint32_t(SF) * KS * 1024, scale_bytes = uint32_t(SF) * KSUP * 256;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.wblob + g.w_codes + size_t(nt0) * KS * 1024, code_bytes);
  const __amdgpu_buffer_rsrc_t rB =
      make_rsrc(g.act + g.a_codes + size_t(mt0) * KS * 1024, uint32_t(act_rt) * KS * 1024);
  const __amdgpu_buffer_rsrc_t rSA = make_rsrc(g.wblob + g.w_scales + size_t(nt0) * KSUP * 256, scale_bytes);
  const __amdgpu_buffer_rsrc_t rSB =
      make_rsrc(g.act + g.a_scales + size_t(mt0) * KSUP * 256, uint32_t(act_rt) * KSUP * 256);
  const uint32_t voff16 = uint32_t(lane) * 16, voff4 = uint32_t(lane) * 4;

  // E8M0 scales of this wave's 8 weight tiles and 8 activation tiles, one superfragment
  uint32_t sa[WN], sb[WMA], san[WN], sbn[WMA];
  auto load_scales = [&](uint32_t (&x)[WN], uint32_t (&y)[WMA], int sup) {
#pragma unroll
    for (int i = 0; i < WN; ++i)
      x[i] = __builtin_amdgcn_raw_buffer_load_b32(rSA, voff4, uint32_t((wn * WN + i) * KSUP + sup) * 256, 0);
#pragma unroll
    for (int j = 0; j < WMA; ++j)
      y[j] = __builtin_amdgcn_raw_buffer_load_b32(rSB, voff4, uint32_t((wm * WMA + j) * KSUP + sup) * 256, 0);
  };
  // This wave's share of a stage: weight fragments PW w .. PW w + PW-1 (f < PW)
  // and the activation fragments of the same numbers (PW <= f < 2 PW).
  auto fetch1 = [&](uint4* dst_stage, int step, int f) {
    const bool wt = f < PW;
    const int fi = wt ? f : f - PW;
    const int fr = (wt ? PW : PWB) * w + fi;     // the fragment's row tile in its operand
    const uint32_t so = uint32_t(fr * KS + step) * 1024;
    load_frag_lds(wt ? rA : rB, dst_stage + ((wt ? 0 : SF) + fr) * 64, voff16, so);
  };
  // The same, or (!valid) the same load through a buffer resource of zero
  // bytes: every lane is out of range, so it writes zeros and reads no memory.
  const __amdgpu_buffer_rsrc_t rZ = make_rsrc(g.wblob, 0u);
  auto fetch1x = [&](uint4* dst_stage, int step, int f, bool valid) {
    const bool wt = f < PW;
    const int fi = wt ? f : f - PW;
    const int fr = (wt ? PW : PWB) * w + fi;
    const uint32_t so = uint32_t(fr * KS + step) * 1024;
    load_frag_lds(valid ? (wt ? rA : rB) : rZ, dst_stage + ((wt ? 0 : SF) + fr) * 64, voff16, so);
  };
  auto frag_a = [&](const uint4* st, int i) { return st[(wn * WN + i) * 64 + lane]; };
  auto frag_b = [&](const uint4* st, int j) { return st[(SF + wm * WMA + j) * 64 + lane]; };

  // Prologue.  128 x 128 tiles: the accumulators start from the low-rank term
  // (X_hat L1) L2 (bf16 MFMAs of L2 against D hi and lo).  The operands of its
  // first 32 ranks are loaded ahead of the scales of superfragment 0 and of
  // stages 0..2 (into slots 0..2), and its MFMAs run while those land; further
  // 32-rank chunks follow in order.  256-wide tiles (no registers to spare
  // here) add the low-rank term after the main loop instead.
  constexpr bool LR_FIRST = WN == 4 || RECT;
  v4f acc[WN][WMA];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WMA; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const bool lowrank = LR_FIRST && (g.epi & SVDQ_EPI_LOWRANK) && g.r_pad > 0;
  const int R32 = g.r_pad / 32;
  const uint4* const L2f = reinterpret_cast<const uint4*>(g.wblob + g.w_L2) + (n0 / 16) * R32 * 64 + lane;
  const uint4* const Df = reinterpret_cast<const uint4*>(g.act + g.a_D) + (m0 / 16) * R32 * 128 + lane;
  auto lowrank_operands = [&](int r32, uint4 (&l2)[WN], uint4 (&dh)[WMA], uint4 (&dl)[WMA]) {
#pragma unroll
    for (int i = 0; i < WN; ++i) l2[i] = L2f[(i * R32 + r32) * 64];
#pragma unroll
    for (int j = 0; j < WMA; ++j) {
      dh[j] = Df[(j * R32 + r32) * 128];
      dl[j] = Df[(j * R32 + r32) * 128 + 64];
    }
  };
  auto lowrank_mfma = [&](const uint4 (&l2)[WN], const uint4 (&dh)[WMA], const uint4 (&dl)[WMA]) {
#pragma unroll
    for (int j = 0; j < WMA; ++j)
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        acc[i][j] = mfma_bf16(l2[i], dh[j], acc[i][j]);
        acc[i][j] = mfma_bf16(l2[i], dl[j], acc[i][j]);
      }
  };
  {
    uint4 l2[WN], dh[WMA], dl[WMA];
    if (lowrank) lowrank_operands(0, l2, dh, dl);
    load_scales(sa, sb, 0);
#pragma unroll
    for (int f = 0; f < FW; ++f) fetch1(ring0, 0, f);
#pragma unroll
    for (int f = 0; f < FW; ++f) fetch1(ring1, 1, f);
    if constexpr (NS == 4) {
#pragma unroll
      for (int f = 0; f < FW; ++f) fetch1(ring2, 2, f);
    }
    if (lowrank) {
      lowrank_mfma(l2, dh, dl);
      for (int r32 = 1; r32 < R32; ++r32) {
        lowrank_operands(r32, l2, dh, dl);
        lowrank_mfma(l2, dh, dl);
      }
    }
  }
  wait_barrier<FW>();                              // stages 0 and 1 (three slots: stage 0) are in LDS
  // Fragments in registers, reloaded in place.  A step runs its 8 x 8 MFMAs in
  // two halves by activation fragment: half 0 uses fb[0..3] and meanwhile reads
  // fb[4..7] of the same stage; half 1 uses fb[4..7] and meanwhile reads the
  // next stage's fb[0..3] and, after row i, fa[i].  So every fragment is read
  // while the MFMAs of another one run, and the reads spread over the step.
  uint4 fa[WN], fb[WMA];
  if constexpr (NS == 4) {
#pragma unroll
    for (int j = 0; j < WM / 2; ++j) fb[j] = frag_b(ring0, j);
#pragma unroll
    for (int i = 0; i < WN; ++i) fa[i] = frag_a(ring0, i);
  }

  // Step U of a superfragment.  Row i also issues one fragment load of stage
  // step+3 (2 PW = WN loads per step).  The flags drop the loads / reads of stages past the end in the
  // peeled last superfragment (peeling keeps the loop body free of branches);
  // VM is the number of vector-memory operations the step itself issues.  The
  // scheduling barriers keep each row's memory operations between its MFMAs
  // and stop the scheduler from interleaving rows, which would make the
  // register allocator move accumulators around.
#define SVDQ_FP4_STEP(U, FETCH, READ, SCALES, VM)                                                     \
  {                                                                                                   \
    const int step = t0 + (U);                                                                        \
    uint4* const s3 = slot(((U) + 3) & 3);                                                            \
    const uint4* const s0 = slot((U) & 3);                                                            \
    const uint4* const s1 = slot(((U) + 1) & 3);                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                                \
    _Pragma("unroll") for (int i = 0; i < WN; ++i) {                                                  \
      if (FETCH) fetch1(s3, step + 3, i);                                                             \
      _Pragma("unroll") for (int j = 0; j < WM / 2; ++j)                                              \
        acc[i][j] = mfma_fp4_sel<(U)>(fa[i], fb[j], acc[i][j], sa[i], sb[j]);                         \
      if (i % 2 == 1 && WM / 2 + i / 2 < WMA) fb[WM / 2 + i / 2] = frag_b(s0, WM / 2 + i / 2);        \
      __builtin_amdgcn_sched_barrier(0);                                                              \
    }                                                                                                 \
    _Pragma("unroll") for (int i = 0; i < WN; ++i) {                                                  \
      _Pragma("unroll") for (int j = WM / 2; j < WMA; ++j)                                            \
        acc[i][j] = mfma_fp4_sel<(U)>(fa[i], fb[j], acc[i][j], sa[i], sb[j]);                         \
      if (READ) {                                                                                     \
        fa[i] = frag_a(s1, i);                                                                        \
        if (i % 2 == 1) fb[i / 2] = frag_b(s1, i / 2);                                                \
      }                                                                                               \
      __builtin_amdgcn_sched_barrier(0);                                                              \
    }                                                                                                 \
    if (SCALES) load_scales(san, sbn, sup + 1);                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                                \
    wait_barrier<(VM)>();                                                                             \
  }
  // Three slots: step U (of twelve, three superfragments) reads its own
  // fragments from slot U % 3 first, runs its MFMAs while issuing the loads of
  // stage step+2 into slot (U+2) % 3 (which held stage step-1, read during the
  // previous step), and at its end waits for stage step+1: what may still be in
  // flight is stage step+2 and the scale loads issued after stage step+1's.
  // Every block of twelve steps goes through the loop (a straight-line copy of
  // the last block, or a branch around its loads, made the register allocator
  // spill accumulators): in the last two steps the stage loads go through a
  // buffer resource of zero bytes (they write zeros into slots already consumed
  // and read no memory), and the last scale load repeats the last
  // superfragment, so that the wait counts hold throughout.  The loop is
  // followed by a wait for every load of every wave (a barrier), so that those
  // zeros have landed before the epilogue writes its LDS staging.
#define SVDQ_FP4_STEP3(U, SCALES, VM)                                                                 \
  {                                                                                                   \
    const int step = t0 + (U);                                                                        \
    const bool fv = step + 2 < KS;                                                                    \
    uint4* const sf = slot(((U) + 2) % 3);                                                            \
    const uint4* const sc = slot((U) % 3);                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                                \
    _Pragma("unroll") for (int j = 0; j < WM; ++j) fb[j] = frag_b(sc, j);                             \
    _Pragma("unroll") for (int i = 0; i < WN; ++i) fa[i] = frag_a(sc, i);                             \
    _Pragma("unroll") for (int i = 0; i < WN; ++i) {                                                  \
      if (i < FW) fetch1x(sf, step + 2, i, fv);                                                       \
      _Pragma("unroll") for (int j = 0; j < WM; ++j)                                                  \
        acc[i][j] = mfma_fp4_sel<((U) & 3)>(fa[i], fb[j], acc[i][j], sa[i], sb[j]);                   \
      __builtin_amdgcn_sched_barrier(0);                                                              \
    }                                                                                                 \
    if (SCALES) load_scales(san, sbn, (step >> 2) + 1 < KSUP ? (step >> 2) + 1 : KSUP - 1);           \
    __builtin_amdgcn_sched_barrier(0);                                                                \
    wait_barrier<(VM)>();                                                                             \
    if (((U) & 3) == 3) {                                                                             \
      _Pragma("unroll") for (int i = 0; i < WN; ++i) sa[i] = san[i];                                  \
      _Pragma("unroll") for (int j = 0; j < WMA; ++j) sb[j] = sbn[j];                                 \
    }                                                                                                 \
  }
  if constexpr (NS == 3) {
    constexpr int F = FW, S = WN + WMA;            // loads per stage, per superfragment's scales
    for (int t0 = 0; t0 < KS; t0 += 12) {
      SVDQ_FP4_STEP3(0, false, F)
      SVDQ_FP4_STEP3(1, true, F + S)
      SVDQ_FP4_STEP3(2, false, F + S)
      SVDQ_FP4_STEP3(3, false, F)
      SVDQ_FP4_STEP3(4, false, F)
      SVDQ_FP4_STEP3(5, true, F + S)
      SVDQ_FP4_STEP3(6, false, F + S)
      SVDQ_FP4_STEP3(7, false, F)
      SVDQ_FP4_STEP3(8, false, F)
      SVDQ_FP4_STEP3(9, true, F + S)
      SVDQ_FP4_STEP3(10, false, F + S)
      SVDQ_FP4_STEP3(11, false, F)
    }
    // every wave's loads have landed (the zeros included: another wave's
    // fragments share the slots this wave stages its output in) before any
    // wave writes the ring again
    wait_barrier<0>();
  } else {
    int sup = 0;
    for (; sup + 1 < KSUP; ++sup) {
      const int t0 = sup * 4;
      SVDQ_FP4_STEP(0, true, true, false, 2 * PW)
      SVDQ_FP4_STEP(1, true, true, true, 2 * PW + WN + WMA)
      SVDQ_FP4_STEP(2, true, true, false, 2 * PW)
      SVDQ_FP4_STEP(3, true, true, false, 2 * PW)
#pragma unroll
      for (int i = 0; i < WN; ++i) sa[i] = san[i];
#pragma unroll
      for (int j = 0; j < WMA; ++j) sb[j] = sbn[j];
    }
    {
      const int t0 = sup * 4;
      SVDQ_FP4_STEP(0, true, true, false, 2 * PW)
      SVDQ_FP4_STEP(1, false, true, false, 0)
      SVDQ_FP4_STEP(2, false, true, false, 0)
      SVDQ_FP4_STEP(3, false, false, false, 0)
    }
  }
#undef SVDQ_FP4_STEP3
#undef SVDQ_FP4_STEP
  // every wave passed the last barrier with no load in flight: the ring is free
  // for the output staging (one slot per wave)
  if constexpr (QOUT >= 0) {                        // QOUT = the next layer's rank tiles of 16
    // lambda, 1/lambda and the correction of the next layer for this tile's BN columns
    __shared__ float lamv[3 * BN];
    if (int(threadIdx.x) < BN) {
      const int k = int(threadIdx.x);
      const int64_t kn = nt0 * 16 + k;
      lamv[k] = reinterpret_cast<const float*>(g.nblob + g.n_lam)[kn];
      lamv[BN + k] = reinterpret_cast<const float*>(g.nblob + g.n_rlam)[kn];
      lamv[2 * BN + k] = reinterpret_cast<const float*>(g.nblob + g.n_rlo)[kn];
    }
    if (!LR_FIRST) add_lowrank<WN, WM>(g, acc, n0, m0, lane);
    float bv[WN][4];
    load_bias<WN>(g, n0, lane, bv);
    uint4 l1r[WN][QOUT > 0 ? QOUT : 1];
    load_l1_next<QOUT, WN>(g, int(nt0 * 16), lane, l1r);
    stage_h<WN, WM, GELU>(acc, bv, lane, wn, wm, reinterpret_cast<uint8_t*>(ring0), reinterpret_cast<uint8_t*>(ring1),
                          reinterpret_cast<uint8_t*>(ring2), reinterpret_cast<uint8_t*>(ring3));
    __syncthreads();
    const int prow = w * 8 * WM;                     // the wave's first row of the tile
    quant_h<WN, QOUT>(g, reinterpret_cast<const uint8_t*>(slot(prow >> 6)), prow & 63, lamv, lane, mt0 * 16 + prow,
                      int(nt0 * 16), tn, l1r);
  } else if constexpr (QKV) {
    if (!LR_FIRST) add_lowrank<WN, WM>(g, acc, n0, m0, lane);
    float bv[WN][4];
    load_bias<WN>(g, n0, lane, bv);
    store_qkv<WN, WM>(g, acc, bv, n0, m0, lane, w,
                      NS == 3 ? reinterpret_cast<uint8_t*>(slot(w >> 1)) + (w & 1) * 32 * stage_row_bytes<WN>()
                              : reinterpret_cast<uint8_t*>(slot(w)));
  } else {
    // bf16 staging: 32 rows of stage_row_bytes per wave; two waves per slot with three slots
    uint8_t* const stage = NS == 3 ? reinterpret_cast<uint8_t*>(slot(w >> 1)) + (w & 1) * 32 * stage_row_bytes<WN>()
                                   : reinterpret_cast<uint8_t*>(slot(w));
    epilogue<WN, WMA, OUT_F32, GELU, !LR_FIRST, (WMA < WM)>(g, acc, n0, m0, lane, stage);
  }
}

// ------------------------------------------------------------------ INT4

__device__ __forceinline__ float h2f(uint32_t bits) { return float(__builtin_bit_cast(_Float16, uint16_t(bits))); }

// A fragment's 32 codes as int8 operands of two 64-K MFMAs, each code times 16.
__device__ __forceinline__ void unpack_frag(const uint4& q, v4i& g0, v4i& g1) {
  int e0, o0, e1, o1;
  unpack_i4x8_x16(q.x, e0, o0);
  unpack_i4x8_x16(q.y, e1, o1);
  g0 = v4i{e0, o0, e1, o1};
  unpack_i4x8_x16(q.z, e0, o0);
  unpack_i4x8_x16(q.w, e1, o1);
  g1 = v4i{e0, o0, e1, o1};
}

// 256 threads = 4 waves in 2 x 2; workgroup tile 2 WN x 2 WM blocks of 16 x 16,
// wave tile WN x WM.  Per 128-K step a wave needs its WN weight and WM activation
// fragments (one coalesced 1 KiB load each) and their fp16 scales; these are
// loaded one step ahead into a second register set, so their latency hides
// behind the current step.  The nibbles are unpacked to int8,
// v_mfma_i32_16x16x64_i8 gives each 64-group's exact int32 sum, and sW sX times
// that sum is added to the fp32 accumulators.  That rescale (int -> float, the
// scale product, a fused multiply-add per output and group) is VALU work no
// matrix instruction takes over, so this kernel is bound by the VALU rather than
// the MFMA rate: 3 M N K / 64 lane operations.
template <int WN, int WM>
struct Int4Stage {
  uint4 cw[WN], cx[WM];   // raw codes: weight and activation fragments
  uint4 sw[WN];           // weight scales: the lane's 4 rows x 2 groups (fp16)
  uint32_t sx[WM];        // activation scales: the lane's row x 2 groups (fp16)
};

// QOUT >= 0: the fused MLP step (the output quantized for an INT4 next layer with
// QOUT rank tiles of 16), as in the MXFP4 kernel's 128 x 128 tiles.
template <int WN, int WM, bool OUT_F32, bool GELU, bool QKV = false, int QOUT = -1>
__global__ void __launch_bounds__(256, 2) gemm_int4_kernel(GemmArgs g) {
  static_assert(QOUT < 0 || (WN == 4 && WM == 4 && !OUT_F32 && !QKV), "fused MLP epilogue on 128 x 128 tiles");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  constexpr int BN = 2 * WN * 16, BM = 2 * WM * 16;
  const int tiles_m = int(g.M_pad / BM);
  int tm, tn;
  raster_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, int(g.N_pad / BN), tm, tn);
  const int64_t n0 = int64_t(tn) * BN + (w & 1) * (WN * 16);
  const int64_t m0 = int64_t(tm) * BM + (w >> 1) * (WM * 16);
  const int KS = g.K / kKStep;

  // Buffer views: the wave's WN weight and WM activation row tiles of codes,
  // and the scales ([ks][rows_pad][2] fp16); lane offsets in the vector
  // operand, the step's offsets in the scalar one (no per-load address math).
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(g.wblob + g.w_codes + size_t(n0 / 16) * KS * 1024, uint32_t(WN) * KS * 1024);
  const __amdgpu_buffer_rsrc_t rX =
      make_rsrc(g.act + g.a_codes + size_t(m0 / 16) * KS * 1024, uint32_t(WM) * KS * 1024);
  // (weight scales: at most 512 steps x 65536 rows x 4 bytes, within 32 bits;
  // activation scales, with up to 2^26 rows: one view per step)
  const __amdgpu_buffer_rsrc_t rWs = make_rsrc(g.wblob + g.w_scales, uint32_t(KS * g.N_pad * 4));
  const uint32_t voff16 = uint32_t(lane) * 16;
  const uint32_t wsoff = uint32_t(n0 + (lane >> 4) * 4) * 4;   // the lane's 4 weight rows in block 0
  const uint32_t xsoff = uint32_t(m0 + (lane & 15)) * 4;

  auto load = [&](int ks, Int4Stage<WN, WM>& st) {
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      st.cw[i] = load_frag(rW, voff16, uint32_t(i * KS + ks) * 1024);
      const v4i sv = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(rWs, wsoff, uint32_t(ks * g.N_pad + i * 16) * 4, 0));
      st.sw[i] = make_uint4(uint32_t(sv[0]), uint32_t(sv[1]), uint32_t(sv[2]), uint32_t(sv[3]));
    }
    const __amdgpu_buffer_rsrc_t rXs = make_rsrc(g.act + g.a_scales + size_t(ks) * g.M_pad * 4, uint32_t(g.M_pad * 4));
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      st.cx[j] = load_frag(rX, voff16, uint32_t(j * KS + ks) * 1024);
      st.sx[j] = __builtin_amdgcn_raw_buffer_load_b32(rXs, xsoff, uint32_t(j * 16) * 4, 0);
    }
  };

  v4f acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Int4Stage<WN, WM>& st) {
    v4i b0[WM], b1[WM];
    float sx0[WM], sx1[WM];
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      unpack_frag(st.cx[j], b0[j], b1[j]);
      sx0[j] = h2f(st.sx[j]);
      sx1[j] = h2f(st.sx[j] >> 16);
    }
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      v4i a0, a1;
      unpack_frag(st.cw[i], a0, a1);
      const uint32_t swv[4] = {st.sw[i].x, st.sw[i].y, st.sw[i].z, st.sw[i].w};
      float sw0[4], sw1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sw0[e] = h2f(swv[e]);
        sw1[e] = h2f(swv[e] >> 16);
      }
      // The MFMAs of block j + 1 are issued before the rescale of block j reads
      // its sums, so the VALU does not stall on a result just issued.
      v4i p0 = mfma_i8(a0, b0[0]), p1 = mfma_i8(a1, b1[0]);
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        v4i q0 = p0, q1 = p1;
        if (j + 1 < WM) {
          q0 = mfma_i8(a0, b0[j + 1]);
          q1 = mfma_i8(a1, b1[j + 1]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][j][e] = fmaf(float(p0[e]), sw0[e] * sx0[j], acc[i][j][e]);
          acc[i][j][e] = fmaf(float(p1[e]), sw1[e] * sx1[j], acc[i][j][e]);
        }
        p0 = q0;
        p1 = q1;
      }
    }
  };

  // KS is a multiple of 4 (K % 512 == 0): two steps per iteration, each
  // computing one register set while the other fills; the final load repeats
  // the last step (in bounds, unused).
  Int4Stage<WN, WM> s0, s1;
  load(0, s0);
  for (int ks = 0; ks < KS; ks += 2) {
    load(ks + 1, s1);
    compute(s0);
    load(ks + 2 < KS ? ks + 2 : KS - 1, s0);
    compute(s1);
  }
  // Both MFMA operands carry a factor 16 (unpack_frag), so every int32 sum is
  // 256 times the codes' sum (|sum| <= 2^20, exact as a float) and so is every
  // accumulator: each FMA adds 256 times the term to 256 times the sum, which
  // rounds to exactly 256 times the unscaled result (every nonzero partial sum
  // is at least 2^-48, a product of two fp16 scales, far from fp32 underflow).
  // One exact scaling by 2^-8 gives the same bits as unscaled operands.
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] *= 0x1p-8f;
  if constexpr (QOUT >= 0) {
    // H = bf16(act(acc + b)) into LDS (two 64-row slots of the tile's 128
    // columns), then each wave quantizes 32 of its rows for the next layer
    __shared__ uint4 hs0[64 * 16], hs1[64 * 16];
    __shared__ float lamv[3 * BN];
    const int wn = w & 1, wm = w >> 1;
    if (int(threadIdx.x) < BN) {
      const int k = int(threadIdx.x);
      const int64_t kn = int64_t(tn) * BN + k;
      lamv[k] = reinterpret_cast<const float*>(g.nblob + g.n_lam)[kn];
      lamv[BN + k] = reinterpret_cast<const float*>(g.nblob + g.n_rlam)[kn];
      lamv[2 * BN + k] = reinterpret_cast<const float*>(g.nblob + g.n_rlo)[kn];
    }
    add_lowrank<WN, WM>(g, acc, n0, m0, lane);
    float bv[WN][4];
    load_bias<WN>(g, n0, lane, bv);
    uint4 l1r[WN][QOUT > 0 ? QOUT : 1];
    load_l1_next<QOUT, WN>(g, tn * BN, lane, l1r);
    stage_h<WN, WM, GELU>(acc, bv, lane, wn, wm, reinterpret_cast<uint8_t*>(hs0), reinterpret_cast<uint8_t*>(hs1),
                          nullptr, nullptr);
    __syncthreads();
    const int prow = w * 8 * WM;                     // the wave's first row of the tile
    quant_h<WN, QOUT, kFmtINT4>(g, reinterpret_cast<const uint8_t*>(prow < 64 ? hs0 : hs1), prow & 63, lamv, lane,
                                int64_t(tm) * BM + prow, tn * BN, tn, l1r);
  } else {
    __shared__ uint8_t stage[4 * 32 * stage_row_bytes<WN>()];     // 32 rows per wave (store_out)
    if constexpr (QKV) {
      static_assert(!OUT_F32 && !GELU, "the QKV epilogue stores bf16 with no activation");
      add_lowrank<WN, WM>(g, acc, n0, m0, lane);
      float bv[WN][4];
      load_bias<WN>(g, n0, lane, bv);
      store_qkv<WN, WM>(g, acc, bv, n0, m0, lane, w, stage + w * 32 * stage_row_bytes<WN>());
    } else {
      epilogue<WN, WM, OUT_F32, GELU>(g, acc, n0, m0, lane, stage + w * 32 * stage_row_bytes<WN>());
    }
  }
}

// ------------------------------------------------------------------ NVFP4
//
// The NVFP4-style format (E2M1 codes, an E4M3 scale per 16, a float32 tensor
// scale) has no matrix instruction on gfx950: the scaled FP4 MFMA takes one
// power-of-two scale per 32.  Both operands are therefore dequantized in
// registers to fp16 and multiplied on the fp16 MFMA (16 x 16 x 32): the gfx950
// FP4 convert applies the power of two 2^floor(log2 S) of the group scale S,
// then a packed fp16 multiply applies S's mantissa (1.xxx).  The value
// code * S has at most 6 significant bits and lies in [2^-10, 2880], so it is
// exact in fp16, every product is exact in fp32, and the fp32 sums round like
// any other accumulation.  The tensor scale multiplies the sum before the
// epilogue.  Tiles, prefetch and epilogue follow the INT4 kernel.

// 8 E2M1 codes of one dword (code e in byte e / 2, low nibble for even e) -> 4
// dwords of fp16 pairs code * S, in code order; sf = S as fp32, m2 = S's
// mantissa as fp16 in both halves.
__device__ __forceinline__ uint4 nv_dequant8(uint32_t d, float sf, uint32_t m2) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 mm = __builtin_bit_cast(h2, m2);
  const h2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, sf, 0) * mm;
  const h2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, sf, 1) * mm;
  const h2 r2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, sf, 2) * mm;
  const h2 r3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, sf, 3) * mm;
  return make_uint4(__builtin_bit_cast(uint32_t, r0), __builtin_bit_cast(uint32_t, r1),
                    __builtin_bit_cast(uint32_t, r2), __builtin_bit_cast(uint32_t, r3));
}

// The group scale S of half h of a lane's 32-element block (byte h of the
// lane's two E4M3 bytes) as fp32, and its mantissa 1.xxx as fp16 in both halves
// of a dword (1.0 when S == 0).
struct NvScale { float sf; uint32_t m2; };
__device__ __forceinline__ NvScale nv_scale(uint32_t s2, int h) {
  const float sf = e4m3_value((s2 >> (8 * h)) & 0xFFu);
  const uint32_t m16 = 0x3C00u | ((__float_as_uint(sf) >> 13) & 0x3FFu);
  return NvScale{sf, m16 | (m16 << 16)};
}

template <int WN, int WM>
struct Nv4Stage {
  uint4 cw[WN], cx[WM];       // codes of the weight and activation fragments
  uint32_t sw[WN], sx[WM];    // the lane's two E4M3 group scales per fragment
};

template <int WN, int WM, bool OUT_F32, bool GELU, bool QKV = false>
__global__ void __launch_bounds__(256, 2) gemm_nvfp4_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  constexpr int BN = 2 * WN * 16, BM = 2 * WM * 16;
  const int tiles_m = int(g.M_pad / BM);
  int tm, tn;
  raster_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, int(g.N_pad / BN), tm, tn);
  const int64_t n0 = int64_t(tn) * BN + (w & 1) * (WN * 16);
  const int64_t m0 = int64_t(tm) * BM + (w >> 1) * (WM * 16);
  const int KS = g.K / kKStep;

  // Buffer views of the wave's WN weight and WM activation row tiles: codes
  // (1 KiB per tile and step) and scales (per tile and step, lane L's two bytes
  // at 2 L); lane offsets in the vector operand, step offsets in the scalar one.
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(g.wblob + g.w_codes + size_t(n0 / 16) * KS * 1024, uint32_t(WN) * KS * 1024);
  const __amdgpu_buffer_rsrc_t rX =
      make_rsrc(g.act + g.a_codes + size_t(m0 / 16) * KS * 1024, uint32_t(WM) * KS * 1024);
  const __amdgpu_buffer_rsrc_t rWs =
      make_rsrc(g.wblob + g.w_scales + size_t(n0 / 16) * KS * 128, uint32_t(WN) * KS * 128);
  const __amdgpu_buffer_rsrc_t rXs =
      make_rsrc(g.act + g.a_scales + size_t(m0 / 16) * KS * 128, uint32_t(WM) * KS * 128);
  const uint32_t voff16 = uint32_t(lane) * 16, voff2 = uint32_t(lane) * 2;

  auto load = [&](int ks, Nv4Stage<WN, WM>& st) {
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      st.cw[i] = load_frag(rW, voff16, uint32_t(i * KS + ks) * 1024);
      st.sw[i] = __builtin_amdgcn_raw_buffer_load_b16(rWs, voff2, uint32_t(i * KS + ks) * 128, 0);
    }
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      st.cx[j] = load_frag(rX, voff16, uint32_t(j * KS + ks) * 1024);
      st.sx[j] = __builtin_amdgcn_raw_buffer_load_b16(rXs, voff2, uint32_t(j * KS + ks) * 128, 0);
    }
  };

  v4f acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // MFMA chunk u of a step takes elements 8u .. 8u + 7 of every lane's
  // 32-element block (dword u of its codes, group half u / 2), on both operands
  auto compute = [&](const Nv4Stage<WN, WM>& st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      NvScale sa[WN], sb[WM];
#pragma unroll
      for (int i = 0; i < WN; ++i) sa[i] = nv_scale(st.sw[i], h);
#pragma unroll
      for (int j = 0; j < WM; ++j) sb[j] = nv_scale(st.sx[j], h);
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int u = 2 * h + uu;
        uint4 a[WN], b[WM];
#pragma unroll
        for (int j = 0; j < WM; ++j) {
          const uint32_t q = u == 0 ? st.cx[j].x : u == 1 ? st.cx[j].y : u == 2 ? st.cx[j].z : st.cx[j].w;
          b[j] = nv_dequant8(q, sb[j].sf, sb[j].m2);
        }
#pragma unroll
        for (int i = 0; i < WN; ++i) {
          const uint32_t q = u == 0 ? st.cw[i].x : u == 1 ? st.cw[i].y : u == 2 ? st.cw[i].z : st.cw[i].w;
          a[i] = nv_dequant8(q, sa[i].sf, sa[i].m2);
        }
#pragma unroll
        for (int i = 0; i < WN; ++i)
#pragma unroll
          for (int j = 0; j < WM; ++j) acc[i][j] = mfma_f16(a[i], b[j], acc[i][j]);
      }
    }
  };

  // two register sets, one computing while the other fills (KS is a multiple
  // of 4; the final load repeats the last step, in bounds and unused)
  Nv4Stage<WN, WM> s0, s1;
  load(0, s0);
  for (int ks = 0; ks < KS; ks += 2) {
    load(ks + 1, s1);
    compute(s0);
    load(ks + 2 < KS ? ks + 2 : KS - 1, s0);
    compute(s1);
  }
  // the weight tensor scale gs = fp32(max|R| / 2688); the activations' is 1
  const float gs = __uint_as_float(*reinterpret_cast<const uint32_t*>(g.wblob + g.w_amax)) / kNvfp4GlobalDiv;
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = acc[i][j] * gs;
  __shared__ uint8_t stage[4 * 32 * stage_row_bytes<WN>()];     // 32 rows per wave (store_out)
  if constexpr (QKV) {
    static_assert(!OUT_F32 && !GELU, "the QKV epilogue stores bf16 with no activation");
    add_lowrank<WN, WM>(g, acc, n0, m0, lane);
    float bv[WN][4];
    load_bias<WN>(g, n0, lane, bv);
    store_qkv<WN, WM>(g, acc, bv, n0, m0, lane, w, stage + w * 32 * stage_row_bytes<WN>());
  } else {
    epilogue<WN, WM, OUT_F32, GELU>(g, acc, n0, m0, lane, stage + w * 32 * stage_row_bytes<WN>());
  }
}

// ------------------------------------------------------------------ W4A16
//
// The second kernel family of the Nunchaku in Diffusers page (section
// "Introducing Nunchaku Lite"): 4-bit weights with 16-bit activations for the
// memory-bound modulation projections, Y = X deQ(Q4(W))^T + b with X in bf16.
// The weights use the INT4-g64 packing of the W4A4 layer.  A workgroup computes
// T 16-row weight tiles on the bf16 MFMA (16 x 16 x 32, weights as A, up to 16
// tokens as B); its four waves take every fourth 128-K step and their fp32
// sums are added in wave order through LDS.  A code q becomes the bf16
// 128 + u with u = q + 8 (the offset nibble in the mantissa of 128, one byte
// permute per two codes); a second product of the same X with the bf16
// constant -136 goes into the same accumulator, so each 64-group's sum is the
// exact sum of q x in fp32 before its scale is applied.  Each wave keeps the
// codes and scales of its next kW4A16Depth steps in flight (buffer loads: a
// scalar base and step offset, one per-lane offset).
//
// X: with XL, all M rows of X are copied once into LDS (direct-to-LDS loads,
// issued before the first weights) and the B fragments are read from there;
// otherwise each 16-token block's fragments are loaded from global memory two
// steps ahead.  Token columns past M hold the last token's values (MFMA output
// columns are independent, and those columns are never stored).
struct W4A16Args {
  const uint8_t* wblob;
  size_t w_codes, w_scales, w_bias;
  const uint16_t* X;
  int64_t ldx, M, N_pad, ldy;
  int K;
  uint32_t epi;
  void* Y;
};

// 8 INT4 codes in the packed dword order (code e in byte e % 4, high nibble for
// e >= 4) -> 4 dwords of bf16 pairs 128 + q + 8 in code order.  k43 holds 0x43
// in every byte (the high byte of bf16 128).
__device__ __forceinline__ uint4 w4_to_bf16(uint32_t d, uint32_t k43) {
  d ^= 0x88888888u;                                // offset nibbles u = q + 8
  const uint32_t lo = d & 0x0F0F0F0Fu;             // codes 0..3, one per byte
  const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;      // codes 4..7
  // selector bytes 0..3 pick bytes of the code word, 4 picks 0x43
  return make_uint4(__builtin_amdgcn_perm(k43, lo, 0x04010400u), __builtin_amdgcn_perm(k43, lo, 0x04030402u),
                    __builtin_amdgcn_perm(k43, hi, 0x04010400u), __builtin_amdgcn_perm(k43, hi, 0x04030402u));
}

constexpr int kW4A16Depth = 3;        // 128-K steps of codes and scales in flight per wave
constexpr int kW4A16XLds = 40960;     // LDS for X rows (XL form): M (K * 2 + 16) bytes at most
constexpr int kW4A16Tiles = 2;        // 16-row tiles per workgroup (when N allows)

__host__ __device__ inline int w4a16_xstride(int K) { return K * 2 + 16; }   // bytes; 16 skews the banks

template <int T, bool XL, bool OUT_F32>
__global__ void __launch_bounds__(256, 3) gemm_w4a16_kernel(W4A16Args a) {
  __shared__ v4f red[3][T][64];
  extern __shared__ uint4 xlds[];                  // XL: M rows of X, stride w4a16_xstride(K) bytes
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KS = a.K / kKStep, n = KS / 4;         // this wave's steps: ks = w + 4 i
  const int c = lane >> 4, tl = lane & 15;
  const int64_t row0 = int64_t(blockIdx.x) * 16 * T;
  // codes of the T tiles (contiguous, KS KiB each), scales of rows row0 .. row0 + 16 T - 1
  const __amdgpu_buffer_rsrc_t rW =
      make_rsrc(a.wblob + a.w_codes + size_t(row0 / 16) * KS * 1024, uint32_t(T * KS * 1024));
  const __amdgpu_buffer_rsrc_t rS =
      make_rsrc(a.wblob + a.w_scales + size_t(row0) * 4, uint32_t((size_t(KS - 1) * a.N_pad + 16 * T) * 4));
  const uint32_t wvoff = uint32_t(lane) * 16, svoff = uint32_t(c) * 16;
  const uint4 m136 = make_uint4(0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u);  // bf16 -136
  // an opaque copy keeps the constant in a register for the byte permutes
  uint32_t k43 = 0x43434343u;
  asm volatile("" : "+v"(k43));

  // bias bits first: every later wait on the vector-memory counter covers this load
  uint2 bias_bits[T];
#pragma unroll
  for (int t = 0; t < T; ++t)
    bias_bits[t] = (a.epi & SVDQ_EPI_BIAS)
                       ? *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.wblob + a.w_bias) +
                                                         row0 + t * 16 + c * 4)
                       : make_uint2(0u, 0u);
  struct WStage { uint4 q[T], s[T]; };
  // loads past the last step repeat it (cache hits, never used)
  auto loadw = [&](int i, WStage& st) {
    i = i < n ? i : n - 1;
    const int ks = w + 4 * i;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      st.q[t] = load_frag(rW, wvoff, uint32_t((t * KS + ks) * 1024));
      st.s[t] = load_frag(rS, svoff, uint32_t((size_t(ks) * a.N_pad + t * 16) * 4));
    }
  };
  v4f acc[T];
  auto compute = [&](const WStage& st, const uint4 (&x)[4]) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t q0 = g == 0 ? st.q[t].x : st.q[t].z, q1 = g == 0 ? st.q[t].y : st.q[t].w;
        v4f p = {0.f, 0.f, 0.f, 0.f};
        p = mfma_bf16(w4_to_bf16(q0, k43), x[2 * g], p);
        p = mfma_bf16(w4_to_bf16(q1, k43), x[2 * g + 1], p);
        p = mfma_bf16(m136, x[2 * g], p);
        p = mfma_bf16(m136, x[2 * g + 1], p);
        const uint32_t sd[4] = {st.s[t].x, st.s[t].y, st.s[t].z, st.s[t].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(h2f(g == 0 ? sd[e] : sd[e] >> 16), p[e], acc[t][e]);
      }
    }
  };
  WStage ws[kW4A16Depth];

  if constexpr (XL) {
    // copy X (M rows, K * 2 bytes each) into LDS: 1 KiB pieces, wave w takes w, w + 4, ...
    const int per_row = a.K / 512, pieces = int(a.M) * per_row, xs_b = w4a16_xstride(a.K);
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.X, uint32_t(a.M * a.ldx * 2));
    for (int pc = w; pc < pieces; pc += 4) {
      const int r = pc / per_row, q = pc % per_row;
      load_frag_lds(rX, reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(xlds) + r * xs_b + q * 1024), wvoff,
                    uint32_t(r * a.ldx * 2 + q * 1024));
    }
    // keep every X copy ahead of the weight loads (the wait below counts on it)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kW4A16Depth; ++j) loadw(j, ws[j]);
    // the X copies were issued before the 2 T kW4A16Depth weight loads
    wait_barrier<2 * T * kW4A16Depth>();
    const int tr = tl < a.M ? tl : int(a.M) - 1;
    const uint8_t* const xb = reinterpret_cast<const uint8_t*>(xlds) + tr * xs_b + (w * kKStep + c * 16) * 2;
    auto readx = [&](int i, uint4 (&x)[4]) {
      const uint8_t* const p = xb + i * 4 * kKStep * 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = *reinterpret_cast<const uint4*>(p + (j >> 1) * 128 + (j & 1) * 16);
    };
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < n; i0 += kW4A16Depth) {
#pragma unroll
      for (int j = 0; j < kW4A16Depth; ++j) {
        if (i0 + j < n) {
          uint4 x[4];
          readx(i0 + j, x);
          compute(ws[j], x);
        }
        loadw(i0 + j + kW4A16Depth, ws[j]);
      }
    }
  }

  // wave sums in order 0 + 1 + 2 + 3; lane holds rows row0 + 16 t + 4 c .. + 3 of token m0 + tl
  auto finish = [&](int64_t m0, int64_t rows) {
    if (w > 0) {
#pragma unroll
      for (int t = 0; t < T; ++t) red[w - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (w == 0 && tl < rows) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const v4f a1 = red[0][t][lane], a2 = red[1][t][lane], a3 = red[2][t][lane];
        float y[4];
        const float b[4] = {bf_lo(bias_bits[t].x), bf_hi(bias_bits[t].x), bf_lo(bias_bits[t].y),
                            bf_hi(bias_bits[t].y)};
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = ((acc[t][e] + a1[e]) + a2[e]) + a3[e] + b[e];
        const int64_t o = (m0 + tl) * a.ldy + row0 + t * 16 + c * 4;
        if (OUT_F32)
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.Y) + o) = make_float4(y[0], y[1], y[2], y[3]);
        else
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.Y) + o) =
              make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]));
      }
    }
    __syncthreads();
  };

  if constexpr (XL) {
    finish(0, a.M);
  } else {
    for (int64_t m0 = 0; m0 < a.M; m0 += 16) {
      const int64_t rows = a.M - m0 < 16 ? a.M - m0 : 16;
      // rows past M fall outside the X range and read 0
      const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.X + m0 * a.ldx, uint32_t(rows * a.ldx * 2));
      const uint32_t xvoff = (uint32_t(tl) * uint32_t(a.ldx) + uint32_t(c) * 16) * 2;
      auto loadx = [&](int i, uint4 (&x)[4]) {
        i = i < n ? i : n - 1;
        const uint32_t so = uint32_t(w + 4 * i) * kKStep * 2;
        // MFMA j covers group j / 2, half j % 2 of the lane's 16 codes per group
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = load_frag(rX, xvoff + (j >> 1) * 128 + (j & 1) * 16, so);
      };
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
      uint4 xs[2][4];
#pragma unroll
      for (int j = 0; j < kW4A16Depth; ++j) loadw(j, ws[j]);
      loadx(0, xs[0]);
      loadx(1, xs[1]);
      for (int i0 = 0; i0 < n; i0 += 2 * kW4A16Depth) {
#pragma unroll
        for (int j = 0; j < 2 * kW4A16Depth; ++j) {
          if (i0 + j < n) compute(ws[j % kW4A16Depth], xs[j & 1]);
          loadw(i0 + j + kW4A16Depth, ws[j % kW4A16Depth]);
          loadx(i0 + j + 2, xs[j & 1]);
        }
      }
      finish(m0, rows);
    }
  }
}

// Requires K % 512 == 0, N % 16 == 0, X rows 16-byte aligned with M ldx * 2
// bytes (XL form) or 16 ldx * 2 bytes below 2^32, Y rows 16-byte aligned.
hipError_t launch_gemm_w4a16(const uint8_t* wblob, const WeightLayout& wl, int K, int N, const uint16_t* X,
                             int64_t ldx, int64_t M, void* Y, int64_t ldy, uint32_t epi, hipStream_t s) {
  W4A16Args a{};
  a.wblob = wblob;
  a.w_codes = wl.codes; a.w_scales = wl.scales; a.w_bias = wl.bias;
  a.X = X; a.ldx = ldx; a.M = M; a.N_pad = wl.N_pad; a.ldy = ldy;
  a.K = K; a.epi = epi; a.Y = Y;
  const bool f32 = (epi & SVDQ_EPI_OUT_F32) != 0;
  const bool xl = M <= 16 && M * w4a16_xstride(K) <= kW4A16XLds && M * ldx * 2 < (int64_t(1) << 32);
  const size_t lds = xl ? size_t(M) * w4a16_xstride(K) : 0;
  const dim3 block(256);
#define SVDQ_W4A16(T_, XL_)                                                                        \
  {                                                                                                \
    const dim3 grid(unsigned(N / (16 * T_)));                                                      \
    if (f32)                                                                                       \
      hipLaunchKernelGGL((gemm_w4a16_kernel<T_, XL_, true>), grid, block, lds, s, a);              \
    else                                                                                           \
      hipLaunchKernelGGL((gemm_w4a16_kernel<T_, XL_, false>), grid, block, lds, s, a);             \
  }
  // X from LDS: one 16-row tile per workgroup (the most workgroups in flight).
  // X from global memory: two tiles share each X fragment, when that still
  // leaves at least two workgroups per CU.
  if (xl)
    SVDQ_W4A16(1, true)
  else if (N % (16 * kW4A16Tiles) == 0 && N / (16 * kW4A16Tiles) >= 512)
    SVDQ_W4A16(kW4A16Tiles, false)
  else
    SVDQ_W4A16(1, false)
#undef SVDQ_W4A16
  return hipGetLastError();
}

// ------------------------------------------------------------------ launcher

constexpr unsigned kMinBigTiles = 128;   // MXFP4: fewer 256 x 256 tiles than this -> 128 x 128 tiles

static int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// The MXFP4 tile choice (see launch_gemm): 256 x 256 tiles for kMinBigTiles up
// to one round of them on this device's CUs, else 128 x 128 tiles.
static bool use_big_tiles(unsigned big) { return big >= kMinBigTiles && big < unsigned(device_cus()); }

// MXFP4 128 x 128 tiles with the three-slot ring (three workgroups per CU) when
// the grid is more than two workgroups per CU; its loop takes blocks of twelve
// 128-K steps.
static bool use_three_slots(unsigned tiles, int K) { return tiles > 2u * unsigned(device_cus()) && K % 1536 == 0; }

// Height of the 256-wide tiles, as activation blocks of 16 rows per wave (the
// tile is 32 wma rows): the fewest rounds of workgroups on the CUs times the
// rows per tile, the taller tile on a tie.  FLUX fc2 (4608 rows, 12 tile
// columns): 216 tiles of 256 rows leave 40 of 256 CUs idle, 252 tiles of 224
// rows fill them, each with 7/8 of the work.
static int short_tile_blocks(int64_t tiles_n, int64_t M_pad) {
  const int64_t cus = device_cus();
  int best = 8;
  int64_t best_cost = 0;
  for (int w = 8; w >= 6; --w) {
    const int64_t tiles = tiles_n * ((M_pad + 32 * w - 1) / (32 * w));
    const int64_t cost = (tiles + cus - 1) / cus * w;
    if (w == 8 || cost < best_cost) {
      best = w;
      best_cost = cost;
    }
  }
  return best;
}

// The 256-wide kernel with WMA activation blocks per wave.
// INT4 / NVFP4 grids with fewer 128 x 128 tiles than this (the CU count) take 64 x 64 tiles.
constexpr unsigned kSmallGridTiles = 256;

template <int WMA>
static void launch_big(bool f32, bool gelu, unsigned nb, hipStream_t s, const GemmArgs& g) {
  if (f32 && gelu)
    hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 8, true, true, -1, false, WMA>), dim3(nb), dim3(256), 0, s, g);
  else if (f32)
    hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 8, true, false, -1, false, WMA>), dim3(nb), dim3(256), 0, s, g);
  else if (gelu)
    hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 8, false, true, -1, false, WMA>), dim3(nb), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 8, false, false, -1, false, WMA>), dim3(nb), dim3(256), 0, s, g);
}

hipError_t launch_gemm(int fmt, const uint8_t* wblob, const WeightLayout& wl, const uint8_t* act, const ActLayout& al,
                       int K, int N, int64_t M, void* Y, int64_t ldy, uint32_t epi, hipStream_t s) {
  GemmArgs g{};
  g.wblob = wblob;
  g.act = act;
  g.w_codes = wl.codes; g.w_scales = wl.scales; g.w_L2 = wl.L2; g.w_bias = wl.bias; g.w_amax = wl.amax;
  g.a_codes = al.codes; g.a_scales = al.scales; g.a_D = al.D;
  g.N_pad = wl.N_pad; g.M_pad = al.M_pad; g.M = M; g.ldy = ldy;
  g.K = K; g.N = N; g.r_pad = int(wl.r_pad);
  g.epi = epi;
  g.Y = Y;
  const bool f32 = (epi & SVDQ_EPI_OUT_F32) != 0;
  const bool gelu = (epi & SVDQ_EPI_GELU) != 0;
#define SVDQ_LAUNCH(KERNEL, WN, WM, THREADS, NB)                                                           \
  do {                                                                                                     \
    if (f32 && gelu) hipLaunchKernelGGL((KERNEL<WN, WM, true, true>), dim3(NB), dim3(THREADS), 0, s, g);    \
    else if (f32) hipLaunchKernelGGL((KERNEL<WN, WM, true, false>), dim3(NB), dim3(THREADS), 0, s, g);      \
    else if (gelu) hipLaunchKernelGGL((KERNEL<WN, WM, false, true>), dim3(NB), dim3(THREADS), 0, s, g);     \
    else hipLaunchKernelGGL((KERNEL<WN, WM, false, false>), dim3(NB), dim3(THREADS), 0, s, g);              \
  } while (0)
  if (fmt == kFmtMXFP4) {
    // 256 x 256 tiles (one workgroup per CU) when there are between kMinBigTiles
    // and one round of them: fewer, larger tiles then keep more of the chip busy
    // per byte staged.  Otherwise 128 x 128 tiles, two workgroups per CU: with
    // the grouped raster their operand panels stay in L2, the last round is half
    // as coarse, and one workgroup's epilogue (the VALU-bound GELU) overlaps the
    // other's main loop.  Measured back to back on one device (us, big / small
    // tiles): fc1 4608 x 3072 -> 12288 with GELU 125 / 121, QKV 4608 x 3072 ->
    // 9216 90 / 84, fc2 4608 x 12288 -> 3072 (216 big tiles) 88 / 100.
    //
    // 256-wide tiles may be shorter than 256 rows (short_tile_blocks), so that
    // one round fills more CUs: fc2 on 252 tiles of 224 rows takes 89 us
    // against 94 on 216 tiles of 256 (alternating runs on one device).
    const unsigned big = unsigned((wl.N_pad / 256) * (al.M_pad / 256));
    if (use_big_tiles(big)) {
      const int wma = short_tile_blocks(wl.N_pad / 256, al.M_pad);
      const unsigned nb = unsigned((wl.N_pad / 256) * ((al.M_pad + 32 * wma - 1) / (32 * wma)));
      if (wma == 8) launch_big<8>(f32, gelu, nb, s, g);
      else if (wma == 7) launch_big<7>(f32, gelu, nb, s, g);
      else launch_big<6>(f32, gelu, nb, s, g);
    } else if (!gelu && use_three_slots(big * 4, K)) {
      // 256 x 128 tiles, 8 x 4 blocks per wave and two workgroups per CU on a
      // 72 KiB three-slot ring: 12 fragment reads per 32 MFMAs instead of 8 per
      // 16, and the same operations per output as the 128 x 128 tiles (the
      // same bits).  Without GELU only: with it, the 128 x 128 tiles at three
      // per CU hide more of the VALU-heavy epilogue (measured level at FLUX fc1;
      // the LoRA layer 103.5 -> 97.6 us).
      const dim3 grid(big * 2);
      if (f32) hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 4, true, false, -1, false, 4, 3>), grid, dim3(256), 0, s, g);
      else hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 4, false, false, -1, false, 4, 3>), grid, dim3(256), 0, s, g);
    } else if (use_three_slots(big * 4, K)) {
      const dim3 grid(big * 4);
      if (f32 && gelu) hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, true, true, -1, false, 4, 3>), grid, dim3(256), 0, s, g);
      else if (f32) hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, true, false, -1, false, 4, 3>), grid, dim3(256), 0, s, g);
      else if (gelu) hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, false, true, -1, false, 4, 3>), grid, dim3(256), 0, s, g);
      else hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, false, false, -1, false, 4, 3>), grid, dim3(256), 0, s, g);
    } else {
      SVDQ_LAUNCH(gemm_mxfp4_kernel, 4, 4, 256, big * 4);
    }
  } else {
    // INT4 and NVFP4 are bound by the VALU work of each wave (the per-group
    // rescale, the dequantization), which grows with the wave tile.  A grid of
    // fewer 128 x 128 tiles than CUs takes 64 x 64 tiles instead (2 x 2 blocks
    // per wave): four times the workgroups, a quarter of the work per wave and
    // step, and for every output the same operations in the same order.
    const unsigned nb = unsigned((wl.N_pad / 128) * (al.M_pad / 128));
    if (nb < kSmallGridTiles) {
      if (fmt == kFmtNVFP4) SVDQ_LAUNCH(gemm_nvfp4_kernel, 2, 2, 256, nb * 4);
      else SVDQ_LAUNCH(gemm_int4_kernel, 2, 2, 256, nb * 4);
    } else if (fmt == kFmtNVFP4) {
      SVDQ_LAUNCH(gemm_nvfp4_kernel, 4, 4, 256, nb);
    } else {
      SVDQ_LAUNCH(gemm_int4_kernel, 4, 4, 256, nb);
    }
  }
#undef SVDQ_LAUNCH
  return hipGetLastError();
}

hipError_t launch_reduce_down(const float* part, int splits, int64_t rows_pad, int r_pad, uint16_t* Dout, hipStream_t s);

// The GEMM of a fused QKV layer (head dim 128) with the Q/K normalization and
// rotary embedding in its epilogue; bf16 output.  Every format: the INT4 and
// NVFP4 kernels (128 x 128 tiles, a head split between two waves) take the same
// epilogue as the MXFP4 kernel's 128 x 128 tiles.
hipError_t launch_gemm_qkv(int fmt, const uint8_t* wblob, const WeightLayout& wl, const uint8_t* act,
                           const ActLayout& al, int K, int N, int64_t M, void* Y, int64_t ldy, uint32_t epi,
                           const uint16_t* norm_q,
                           const uint16_t* norm_k, float eps, const float* rope_cos, const float* rope_sin,
                           hipStream_t s) {
  GemmArgs g{};
  g.wblob = wblob;
  g.act = act;
  g.w_codes = wl.codes; g.w_scales = wl.scales; g.w_L2 = wl.L2; g.w_bias = wl.bias;
  g.a_codes = al.codes; g.a_scales = al.scales; g.a_D = al.D;
  g.N_pad = wl.N_pad; g.M_pad = al.M_pad; g.M = M; g.ldy = ldy;
  g.K = K; g.N = N; g.r_pad = int(wl.r_pad);
  g.epi = epi;
  g.Y = Y;
  g.norm_q = norm_q; g.norm_k = norm_k; g.rope_cos = rope_cos; g.rope_sin = rope_sin; g.eps = eps;
  g.w_amax = wl.amax;
  const unsigned big = unsigned((wl.N_pad / 256) * (al.M_pad / 256));
  if (fmt == kFmtINT4)
    hipLaunchKernelGGL((gemm_int4_kernel<4, 4, false, false, true>), dim3(big * 4), dim3(256), 0, s, g);
  else if (fmt == kFmtNVFP4)
    hipLaunchKernelGGL((gemm_nvfp4_kernel<4, 4, false, false, true>), dim3(big * 4), dim3(256), 0, s, g);
  else if (use_big_tiles(big))
    hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 8, false, false, -1, true>), dim3(big), dim3(256), 0, s, g);
  else if (use_three_slots(big * 4, K))
    hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, false, false, -1, true, 4, 3>), dim3(big * 4), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, false, false, -1, true>), dim3(big * 4), dim3(256), 0, s, g);
  return hipGetLastError();
}

// The GEMM of one layer with its bf16 output quantized for the next layer (both
// MXFP4 or both INT4), then the sum of the down-projection partials into that
// layer's D.
hipError_t launch_gemm_quant(int fmt, const uint8_t* wblob, const WeightLayout& wl, const uint8_t* act,
                             const ActLayout& al, int K, int N, int64_t M, uint32_t epi, const uint8_t* nblob,
                             const WeightLayout& nwl, uint8_t* nact, const ActLayout& nal, hipStream_t s) {
  GemmArgs g{};
  g.wblob = wblob;
  g.act = act;
  g.w_codes = wl.codes; g.w_scales = wl.scales; g.w_L2 = wl.L2; g.w_bias = wl.bias;
  g.a_codes = al.codes; g.a_scales = al.scales; g.a_D = al.D;
  g.N_pad = wl.N_pad; g.M_pad = al.M_pad; g.M = M; g.ldy = 0;
  g.K = K; g.N = N; g.r_pad = int(wl.r_pad);
  g.epi = epi;
  g.Y = nullptr;
  g.nblob = nblob;
  g.nact = nact;
  g.n_lam = nwl.lam; g.n_rlam = nwl.rlam; g.n_rlo = nwl.rlo; g.n_L1 = nwl.L1; g.n_flags = nwl.flags;
  g.n_codes = nal.codes; g.n_scales = nal.scales; g.n_part = nal.part;
  g.nr_pad = int(nwl.r_pad);
  // The plain GEMM's tile choice: 256 x 256 tiles for 128 up to one round of
  // them, else 128 x 128 tiles (two workgroups per CU, so that one's
  // quantization overlaps the other's main loop).
  const unsigned big = unsigned((wl.N_pad / 256) * (al.M_pad / 256));
  const bool int4 = fmt == kFmtINT4;                // the INT4 GEMM: 128 x 128 tiles only
  const bool bigt = !int4 && use_big_tiles(big);
  const unsigned nb = bigt ? big : big * 4;
  const int tile_cols = bigt ? 256 : 128;
  const bool gelu = (epi & SVDQ_EPI_GELU) != 0;
  // three 128 x 128 workgroups per CU as for the plain GEMM, up to a next-layer
  // rank of 32 (a rank of 64 leaves too few registers)
  const bool three = !int4 && !bigt && nwl.r_pad <= 32 && use_three_slots(nb, K);
#define SVDQ_QLAUNCH(R16)                                                                                        \
  if (three && gelu) hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, false, true, (R16 <= 2 ? R16 : 0), false, 4, 3>), dim3(nb), dim3(256), 0, s, g); \
  else if (three) hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, false, false, (R16 <= 2 ? R16 : 0), false, 4, 3>), dim3(nb), dim3(256), 0, s, g); \
  else if (int4 && gelu) hipLaunchKernelGGL((gemm_int4_kernel<4, 4, false, true, false, R16>), dim3(nb), dim3(256), 0, s, g); \
  else if (int4) hipLaunchKernelGGL((gemm_int4_kernel<4, 4, false, false, false, R16>), dim3(nb), dim3(256), 0, s, g); \
  else if (bigt && gelu) hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 8, false, true, R16>), dim3(nb), dim3(256), 0, s, g); \
  else if (bigt) hipLaunchKernelGGL((gemm_mxfp4_kernel<8, 8, false, false, R16>), dim3(nb), dim3(256), 0, s, g);  \
  else if (gelu) hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, false, true, R16>), dim3(nb), dim3(256), 0, s, g);   \
  else hipLaunchKernelGGL((gemm_mxfp4_kernel<4, 4, false, false, R16>), dim3(nb), dim3(256), 0, s, g)
  switch (nwl.r_pad / 16) {
    case 0: SVDQ_QLAUNCH(0); break;
    case 2: SVDQ_QLAUNCH(2); break;
    case 4: SVDQ_QLAUNCH(4); break;
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_QLAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nwl.r_pad == 0) return e;
  return launch_reduce_down(reinterpret_cast<const float*>(nact + nal.part), N / tile_cols, nal.M_pad,
                            int(nwl.r_pad), reinterpret_cast<uint16_t*>(nact + nal.D), s);
}

}  // namespace svdq
