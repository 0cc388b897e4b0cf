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

#include "../../include/svdq.h"
#include "common.h"

namespace svdq {

struct GemmArgs {
  const uint8_t* wblob;
  const uint8_t* act;
  size_t w_codes, w_scales, w_L2, w_bias;
  size_t a_codes, a_scales, a_D;
  int64_t N_pad, M_pad, M, ldy;
  int K, N, r_pad;
  uint32_t epi;
  void* Y;
};

// ------------------------------------------------------------------ epilogue

template <int WN, int WM, bool OUT_F32>
__device__ __forceinline__ void epilogue(const GemmArgs& g, v4f (&acc)[WN][WM], int64_t n0, int64_t m0, int lane) {
  if ((g.epi & SVDQ_EPI_LOWRANK) && g.r_pad > 0) {
    const int R32 = g.r_pad / 32;
    const uint4* L2f = reinterpret_cast<const uint4*>(g.wblob + g.w_L2) + (n0 / 16) * R32 * 64 + lane;
    const uint4* Df = reinterpret_cast<const uint4*>(g.act + g.a_D) + (m0 / 16) * R32 * 128 + lane;
    for (int r32 = 0; r32 < R32; ++r32) {
      uint4 l2[WN];
#pragma unroll
      for (int i = 0; i < WN; ++i) l2[i] = L2f[(i * R32 + r32) * 64];
#pragma unroll
      for (int j = 0; j < WM; ++j) {
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
  const uint16_t* bias = reinterpret_cast<const uint16_t*>(g.wblob + g.w_bias);
  const bool use_bias = (g.epi & SVDQ_EPI_BIAS) != 0;
  const bool use_gelu = (g.epi & SVDQ_EPI_GELU) != 0;
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    const int64_t n = n0 + i * 16 + (lane >> 4) * 4;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (use_bias) {
      const uint2 braw = *reinterpret_cast<const uint2*>(bias + n);
      bv[0] = bf_lo(braw.x); bv[1] = bf_hi(braw.x); bv[2] = bf_lo(braw.y); bv[3] = bf_hi(braw.y);
    }
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const int64_t m = m0 + j * 16 + (lane & 15);
      if (m < g.M && n < g.N) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = acc[i][j][e] + bv[e];
          if (use_gelu) y[e] = gelu_erf(y[e]);
        }
        if (OUT_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(g.Y) + m * g.ldy + n) = make_float4(y[0], y[1], y[2], y[3]);
        } else {
          uint2 o;
          o.x = pack_bf2(y[0], y[1]);
          o.y = pack_bf2(y[2], y[3]);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.Y) + m * g.ldy + n) = o;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ MXFP4

template <int TT, int WN, int WM>
__device__ __forceinline__ void fp4_kstep(v4f (&acc)[WN][WM], uint4 (&a)[2][WN], uint4 (&b)[2][WM],
                                          const uint32_t (&sa)[WN], const uint32_t (&sb)[WM], const uint4* Wc,
                                          const uint4* Ac, int KS, int ks) {
  constexpr int cur = TT & 1, nxt = cur ^ 1;
  if (ks + 1 < KS) {
#pragma unroll
    for (int i = 0; i < WN; ++i) a[nxt][i] = Wc[(size_t(i) * KS + ks + 1) * 64];
#pragma unroll
    for (int j = 0; j < WM; ++j) b[nxt][j] = Ac[(size_t(j) * KS + ks + 1) * 64];
  }
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = mfma_fp4_sel<TT>(a[cur][i], b[cur][j], acc[i][j], sa[i], sb[j]);
}

template <int WN, int WM, bool OUT_F32>
__global__ void __launch_bounds__(256) gemm_mxfp4_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int BN = 2 * WN * 16, BM = 2 * WM * 16;
  const int tiles_m = int(g.M_pad / BM);
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int64_t n0 = int64_t(tn) * BN + (w & 1) * (WN * 16);
  const int64_t m0 = int64_t(tm) * BM + (w >> 1) * (WM * 16);
  const int KS = g.K / kKStep, KSUP = g.K / kKSuper;

  const uint4* Wc = reinterpret_cast<const uint4*>(g.wblob + g.w_codes) + (n0 / 16) * KS * 64 + lane;
  const uint4* Ac = reinterpret_cast<const uint4*>(g.act + g.a_codes) + (m0 / 16) * KS * 64 + lane;
  const uint32_t* Ws = reinterpret_cast<const uint32_t*>(g.wblob + g.w_scales) + (n0 / 16) * KSUP * 64 + lane;
  const uint32_t* As = reinterpret_cast<const uint32_t*>(g.act + g.a_scales) + (m0 / 16) * KSUP * 64 + lane;

  v4f acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 a[2][WN], b[2][WM];
  uint32_t sa[WN], sb[WM], san[WN], sbn[WM];
#pragma unroll
  for (int i = 0; i < WN; ++i) { a[0][i] = Wc[size_t(i) * KS * 64]; sa[i] = Ws[size_t(i) * KSUP * 64]; }
#pragma unroll
  for (int j = 0; j < WM; ++j) { b[0][j] = Ac[size_t(j) * KS * 64]; sb[j] = As[size_t(j) * KSUP * 64]; }

  for (int sup = 0; sup < KSUP; ++sup) {
    const int ks = sup * 4;
    if (sup + 1 < KSUP) {
#pragma unroll
      for (int i = 0; i < WN; ++i) san[i] = Ws[(size_t(i) * KSUP + sup + 1) * 64];
#pragma unroll
      for (int j = 0; j < WM; ++j) sbn[j] = As[(size_t(j) * KSUP + sup + 1) * 64];
    }
    fp4_kstep<0>(acc, a, b, sa, sb, Wc, Ac, KS, ks + 0);
    fp4_kstep<1>(acc, a, b, sa, sb, Wc, Ac, KS, ks + 1);
    fp4_kstep<2>(acc, a, b, sa, sb, Wc, Ac, KS, ks + 2);
    fp4_kstep<3>(acc, a, b, sa, sb, Wc, Ac, KS, ks + 3);
#pragma unroll
    for (int i = 0; i < WN; ++i) sa[i] = san[i];
#pragma unroll
    for (int j = 0; j < WM; ++j) sb[j] = sbn[j];
  }
  epilogue<WN, WM, OUT_F32>(g, acc, n0, m0, lane);
}

// ------------------------------------------------------------------ INT4

__device__ __forceinline__ float h2f(uint32_t bits) { return float(__builtin_bit_cast(_Float16, uint16_t(bits))); }

__device__ __forceinline__ void unpack_frag(const uint4& q, v4i& g0, v4i& g1) {
  int e0, o0, e1, o1;
  unpack_i4x8(q.x, e0, o0);
  unpack_i4x8(q.y, e1, o1);
  g0 = v4i{e0, o0, e1, o1};
  unpack_i4x8(q.z, e0, o0);
  unpack_i4x8(q.w, e1, o1);
  g1 = v4i{e0, o0, e1, o1};
}

template <int WN, int WM, bool OUT_F32>
__global__ void __launch_bounds__(256) gemm_int4_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int BN = 2 * WN * 16, BM = 2 * WM * 16;
  const int tiles_m = int(g.M_pad / BM);
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int64_t n0 = int64_t(tn) * BN + (w & 1) * (WN * 16);
  const int64_t m0 = int64_t(tm) * BM + (w >> 1) * (WM * 16);
  const int KS = g.K / kKStep;

  const uint4* Wc = reinterpret_cast<const uint4*>(g.wblob + g.w_codes) + (n0 / 16) * KS * 64 + lane;
  const uint4* Ac = reinterpret_cast<const uint4*>(g.act + g.a_codes) + (m0 / 16) * KS * 64 + lane;
  // scales: [ks][rows_pad][2] fp16
  const uint4* Wsc = reinterpret_cast<const uint4*>(g.wblob + g.w_scales);
  const uint32_t* Asc = reinterpret_cast<const uint32_t*>(g.act + g.a_scales);
  const int64_t wrow = n0 + (lane >> 4) * 4;  // first of the lane's 4 weight rows in block 0
  const int64_t arow = m0 + (lane & 15);

  v4f acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int ks = 0; ks < KS; ++ks) {
    v4i A0[WN], A1[WN], B0[WM], B1[WM];
    float sw0[WN][4], sw1[WN][4], sx0[WM], sx1[WM];
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      unpack_frag(Wc[(size_t(i) * KS + ks) * 64], A0[i], A1[i]);
      const uint4 s = Wsc[(size_t(ks) * g.N_pad + wrow + i * 16) / 4];  // 4 rows x 2 fp16 per 16 B
      sw0[i][0] = h2f(s.x); sw1[i][0] = h2f(s.x >> 16);
      sw0[i][1] = h2f(s.y); sw1[i][1] = h2f(s.y >> 16);
      sw0[i][2] = h2f(s.z); sw1[i][2] = h2f(s.z >> 16);
      sw0[i][3] = h2f(s.w); sw1[i][3] = h2f(s.w >> 16);
    }
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      unpack_frag(Ac[(size_t(j) * KS + ks) * 64], B0[j], B1[j]);
      const uint32_t s = Asc[size_t(ks) * g.M_pad + arow + j * 16];
      sx0[j] = h2f(s);
      sx1[j] = h2f(s >> 16);
    }
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        const v4i p0 = mfma_i8(A0[i], B0[j]);
        const v4i p1 = mfma_i8(A1[i], B1[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][j][e] = fmaf(float(p0[e]), sw0[i][e] * sx0[j], acc[i][j][e]);
          acc[i][j][e] = fmaf(float(p1[e]), sw1[i][e] * sx1[j], acc[i][j][e]);
        }
      }
  }
  epilogue<WN, WM, OUT_F32>(g, acc, n0, m0, lane);
}

// ------------------------------------------------------------------ launcher

hipError_t launch_gemm(int fmt, const uint8_t* wblob, const WeightLayout& wl, const uint8_t* act, const ActLayout& al,
                       int K, int N, int64_t M, void* Y, int64_t ldy, uint32_t epi, hipStream_t s) {
  GemmArgs g;
  g.wblob = wblob;
  g.act = act;
  g.w_codes = wl.codes; g.w_scales = wl.scales; g.w_L2 = wl.L2; g.w_bias = wl.bias;
  g.a_codes = al.codes; g.a_scales = al.scales; g.a_D = al.D;
  g.N_pad = wl.N_pad; g.M_pad = al.M_pad; g.M = M; g.ldy = ldy;
  g.K = K; g.N = N; g.r_pad = int(wl.r_pad);
  g.epi = epi;
  g.Y = Y;
  const bool f32 = (epi & SVDQ_EPI_OUT_F32) != 0;
  if (fmt == kFmtMXFP4) {
    constexpr int WN = 8, WM = 4;
    const unsigned nb = unsigned((wl.N_pad / (2 * WN * 16)) * (al.M_pad / (2 * WM * 16)));
    if (f32)
      hipLaunchKernelGGL((gemm_mxfp4_kernel<WN, WM, true>), dim3(nb), dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_mxfp4_kernel<WN, WM, false>), dim3(nb), dim3(256), 0, s, g);
  } else {
    constexpr int WN = 4, WM = 4;
    const unsigned nb = unsigned((wl.N_pad / (2 * WN * 16)) * (al.M_pad / (2 * WM * 16)));
    if (f32)
      hipLaunchKernelGGL((gemm_int4_kernel<WN, WM, true>), dim3(nb), dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_int4_kernel<WN, WM, false>), dim3(nb), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace svdq
