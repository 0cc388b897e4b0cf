// Launch 1 of the layer and the weight packer.
//
// quantize_rows: one pass over a 16-row tile of X (activations, bf16) or R
// (weights, fp32).  For activations it divides by lambda (the smoothing step of
// section 4.2 of the SVDQuant notes page), and in the same pass computes the
// down projection D = X_hat L1 on bf16 MFMA (section 4.3: the down projection is
// fused into the quantization kernel).  Per group of g elements along K it takes
// amax, the scale and the 4-bit codes (section 3's max-scaled quantizer; MXFP4:
// E8M0 power of two with e = floor(log2 amax) - 2; INT4: fp16(amax / 7)), and
// writes codes and scales straight into the GEMM's fragment layout.
//
// Work split: workgroup = one 16-row tile; its NW waves stride over the K/512
// superchunks; lane (row = lane % 16, c = lane / 16) holds 8 consecutive
// elements of each 32-element block, i.e. exactly the A fragment of the bf16
// 16x16x32 MFMA, so the down projection needs no data movement.
#include <hip/hip_runtime.h>

#include "common.h"

namespace svdq {

template <int FMT, bool ACT, int R16>
__global__ void __launch_bounds__(512) quantize_rows_kernel(
    const void* __restrict__ src, int64_t rows, int64_t ld, int K, const float* __restrict__ lam,
    const uint4* __restrict__ L1f, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    int64_t rows_pad, uint16_t* __restrict__ Dout, int r_pad) {
  extern __shared__ float dred[];  // [NW][16][r_pad] partial down projections
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int row = lane & 15, c = lane >> 4;
  const int64_t rt = blockIdx.x;
  const int64_t m = rt * 16 + row;
  const bool valid = m < rows;
  const int nsuper = K / kKSuper;

  v4f dacc[R16 > 0 ? R16 : 1];
#pragma unroll
  for (int i = 0; i < (R16 > 0 ? R16 : 1); ++i) dacc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kc = w; kc < nsuper; kc += nw) {
    uint32_t sdw = 0;  // MXFP4: this lane's scale dword of the superfragment
#pragma unroll 2
    for (int p = 0; p < 8; ++p) {  // 64-element units of the 512 chunk
      float x[16];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = kc * kKSuper + (2 * p + h) * 32 + c * 8;
        if (ACT) {
          uint4 raw = make_uint4(0u, 0u, 0u, 0u);
          if (valid) raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + m * ld + k);
          const float4 l0 = *reinterpret_cast<const float4*>(lam + k);
          const float4 l1 = *reinterpret_cast<const float4*>(lam + k + 4);
          x[8 * h + 0] = bf_lo(raw.x) / l0.x;
          x[8 * h + 1] = bf_hi(raw.x) / l0.y;
          x[8 * h + 2] = bf_lo(raw.y) / l0.z;
          x[8 * h + 3] = bf_hi(raw.y) / l0.w;
          x[8 * h + 4] = bf_lo(raw.z) / l1.x;
          x[8 * h + 5] = bf_hi(raw.z) / l1.y;
          x[8 * h + 6] = bf_lo(raw.w) / l1.z;
          x[8 * h + 7] = bf_hi(raw.w) / l1.w;
        } else {
          float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
          if (valid) {
            const float* s = reinterpret_cast<const float*>(src) + m * ld + k;
            a = *reinterpret_cast<const float4*>(s);
            b = *reinterpret_cast<const float4*>(s + 4);
          }
          x[8 * h + 0] = a.x; x[8 * h + 1] = a.y; x[8 * h + 2] = a.z; x[8 * h + 3] = a.w;
          x[8 * h + 4] = b.x; x[8 * h + 5] = b.y; x[8 * h + 6] = b.z; x[8 * h + 7] = b.w;
        }
      }

      if (FMT == kFmtMXFP4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jb = 2 * p + h;  // 32-block within the superchunk
          float amax = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[8 * h + e]));
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          const uint32_t sb = e8m0_of_amax(amax);
          const float inv = inv_scale_of_e8m0(sb);
          uint32_t cw = 0;
          cw = cvt_fp4x2<0>(cw, x[8 * h + 0] * inv, x[8 * h + 1] * inv);
          cw = cvt_fp4x2<1>(cw, x[8 * h + 2] * inv, x[8 * h + 3] * inv);
          cw = cvt_fp4x2<2>(cw, x[8 * h + 4] * inv, x[8 * h + 5] * inv);
          cw = cvt_fp4x2<3>(cw, x[8 * h + 6] * inv, x[8 * h + 7] * inv);
          const int ks = kc * 4 + jb / 4;
          *reinterpret_cast<uint32_t*>(codes + code_chunk(rt, ks, K, (jb & 3) * 16 + row) + c * 4) = cw;
          if ((jb & 3) == c) sdw |= sb << (8 * (jb >> 2));
        }
      } else {
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const float s32 = amax / 7.0f;
        const _Float16 h16 = (_Float16)fminf(s32, 65504.0f);
        const float s = (float)h16;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t cw = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float t = x[8 * h + e] / s;
            t = __builtin_rintf(fminf(fmaxf(t, -8.0f), 7.0f));
            const int q = (s == 0.0f) ? 0 : int(t);
            cw |= (uint32_t(q) & 0xFu) << (4 * e);
          }
          const int jb = 2 * p + h;
          const int kk = (jb & 3) * 32 + c * 8;  // offset inside the 128-K step
          const int gi = kk / 64, o = kk % 64;
          const int ks = kc * 4 + jb / 4;
          *reinterpret_cast<uint32_t*>(codes + code_chunk(rt, ks, K, (o / 16) * 16 + row) + gi * 8 + (o % 16) / 2) = cw;
        }
        if (c == 0) {
          const int g = kc * 8 + p;
          *reinterpret_cast<_Float16*>(scales + i4_scale_byte(m, g, rows_pad)) = h16;
        }
      }

      if (ACT && R16 > 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jb = 2 * p + h;
          uint4 hi, lo;
          float r[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) r[e] = x[8 * h + e] - bf_lo(f2bf(x[8 * h + e]));
          hi.x = pack_bf2(x[8 * h + 0], x[8 * h + 1]);
          hi.y = pack_bf2(x[8 * h + 2], x[8 * h + 3]);
          hi.z = pack_bf2(x[8 * h + 4], x[8 * h + 5]);
          hi.w = pack_bf2(x[8 * h + 6], x[8 * h + 7]);
          lo.x = pack_bf2(r[0], r[1]);
          lo.y = pack_bf2(r[2], r[3]);
          lo.z = pack_bf2(r[4], r[5]);
          lo.w = pack_bf2(r[6], r[7]);
          const uint4* bf = L1f + (size_t(kc * 16 + jb) * R16) * 64 + lane;
#pragma unroll
          for (int ib = 0; ib < (R16 > 0 ? R16 : 1); ++ib) {
            const uint4 b = bf[ib * 64];
            dacc[ib] = mfma_bf16(hi, b, dacc[ib]);
            dacc[ib] = mfma_bf16(lo, b, dacc[ib]);
          }
        }
      }
    }
    if (FMT == kFmtMXFP4)
      *reinterpret_cast<uint32_t*>(scales + (size_t(rt) * nsuper + kc) * 256 + lane * 4) = sdw;
  }

  if (ACT && R16 > 0) {
    // Reduce the waves' partial sums in a fixed order (deterministic), then store
    // D as bf16 hi + lo in the up projection's B-fragment layout.
#pragma unroll
    for (int ib = 0; ib < (R16 > 0 ? R16 : 1); ++ib)
#pragma unroll
      for (int e = 0; e < 4; ++e) dred[(w * 16 + (lane >> 4) * 4 + e) * r_pad + ib * 16 + (lane & 15)] = dacc[ib][e];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * r_pad; idx += blockDim.x) {
      const int rr = idx / r_pad, col = idx % r_pad;
      float s = 0.f;
      for (int ww = 0; ww < nw; ++ww) s += dred[(ww * 16 + rr) * r_pad + col];
      const uint32_t hb = f2bf(s);
      const uint32_t lb = f2bf(s - bf_lo(hb));
      const int64_t mm = rt * 16 + rr;
      Dout[d_elem(mm, col, 0, r_pad)] = uint16_t(hb);
      Dout[d_elem(mm, col, 1, r_pad)] = uint16_t(lb);
    }
  }
}

// ---- packing of the small operands (load time) ----

__global__ void pack_l1_kernel(const uint16_t* __restrict__ L1, int K, int rank, int r_pad, uint16_t* __restrict__ out) {
  const size_t total = size_t(K) * r_pad;
  for (size_t d = size_t(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += size_t(gridDim.x) * blockDim.x) {
    const int e = int(d % 8);
    const int L = int((d / 8) % 64);
    const size_t t = d / 512;
    const int i16 = int(t % (r_pad / 16));
    const int k32 = int(t / (r_pad / 16));
    const int k = k32 * 32 + (L / 16) * 8 + e;
    const int i = i16 * 16 + (L % 16);
    out[d] = (i < rank) ? L1[size_t(k) * rank + i] : uint16_t(0);
  }
}

__global__ void pack_l2_kernel(const uint16_t* __restrict__ L2, int N, int64_t N_pad, int rank, int r_pad,
                               uint16_t* __restrict__ out) {
  const size_t total = size_t(N_pad) * r_pad;
  for (size_t d = size_t(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += size_t(gridDim.x) * blockDim.x) {
    const int e = int(d % 8);
    const int L = int((d / 8) % 64);
    const size_t t = d / 512;
    const int r32 = int(t % (r_pad / 32));
    const int64_t n16 = int64_t(t / (r_pad / 32));
    const int64_t n = n16 * 16 + (L % 16);
    const int rk = r32 * 32 + (L / 16) * 8 + e;
    out[d] = (rk < rank && n < N) ? L2[size_t(rk) * N + n] : uint16_t(0);
  }
}

__global__ void pack_vec_kernel(const float* __restrict__ lam, int K, const uint16_t* __restrict__ bias, int N,
                                int64_t N_pad, float* __restrict__ lam_out, float* __restrict__ rlam_out,
                                uint16_t* __restrict__ bias_out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < K) {
    lam_out[i] = lam[i];
    rlam_out[i] = 1.0f / lam[i];
  }
  if (i < N_pad) bias_out[i] = (bias != nullptr && i < N) ? bias[i] : uint16_t(0);
}

// ---- test-only unpackers to the canonical layout ----

__global__ void unpack_codes_kernel(int fmt, const uint8_t* __restrict__ codes, int64_t rows, int K,
                                    uint8_t* __restrict__ out) {
  const int64_t total = rows * (K / 2);
  for (int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = d / (K / 2);
    const int j = int(d % (K / 2));
    int h0, h1;
    const size_t b0 = code_byte(fmt, r, 2 * j, K, &h0);
    const size_t b1 = code_byte(fmt, r, 2 * j + 1, K, &h1);
    const uint32_t n0 = (codes[b0] >> (4 * h0)) & 0xFu;
    const uint32_t n1 = (codes[b1] >> (4 * h1)) & 0xFu;
    out[d] = uint8_t(n0 | (n1 << 4));
  }
}

__global__ void unpack_scales_kernel(int fmt, const uint8_t* __restrict__ scales, int64_t rows, int64_t rows_pad, int K,
                                     void* __restrict__ out) {
  const int ng = (fmt == kFmtMXFP4) ? K / 32 : K / 64;
  const int64_t total = rows * ng;
  for (int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = d / ng;
    const int g = int(d % ng);
    if (fmt == kFmtMXFP4)
      reinterpret_cast<uint8_t*>(out)[d] = scales[mx_scale_byte(r, g, K)];
    else
      reinterpret_cast<uint16_t*>(out)[d] = *reinterpret_cast<const uint16_t*>(scales + i4_scale_byte(r, g, rows_pad));
  }
}

__global__ void unpack_lowrank_kernel(const uint16_t* __restrict__ L1f, const uint16_t* __restrict__ L2f, int K, int N,
                                      int rank, int r_pad, uint16_t* __restrict__ L1, uint16_t* __restrict__ L2) {
  const int64_t n1 = int64_t(K) * rank, n2 = int64_t(rank) * N;
  for (int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; d < n1 + n2; d += int64_t(gridDim.x) * blockDim.x) {
    if (d < n1) {
      if (L1) L1[d] = L1f[l1_elem(int(d / rank), int(d % rank), r_pad)];
    } else {
      const int64_t e = d - n1;
      if (L2) L2[e] = L2f[l2_elem(e % N, int(e / N), r_pad)];
    }
  }
}

__global__ void unpack_d_kernel(const uint16_t* __restrict__ Df, int64_t M, int rank, int r_pad, float* __restrict__ D) {
  const int64_t total = M * rank;
  for (int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += int64_t(gridDim.x) * blockDim.x) {
    const int64_t m = d / rank;
    const int i = int(d % rank);
    D[d] = bf_lo(Df[d_elem(m, i, 0, r_pad)]) + bf_lo(Df[d_elem(m, i, 1, r_pad)]);
  }
}

// ---- host launchers ----

static int pick_waves(int K) {
  const int n = K / kKSuper;
  return n < 8 ? n : 8;
}

template <int FMT, bool ACT>
static hipError_t launch_quantize_fmt(const void* src, int64_t rows, int64_t ld, int K, const float* lam,
                                      const void* L1f, uint8_t* codes, uint8_t* scales, int64_t rows_pad,
                                      uint16_t* Dout, int r_pad, hipStream_t s) {
  const int nw = pick_waves(K);
  const dim3 grid(unsigned(rows_pad / 16)), block(unsigned(64 * nw));
  const size_t shm = ACT ? size_t(nw) * 16 * r_pad * 4 : 0;
  const uint4* l1 = reinterpret_cast<const uint4*>(L1f);
#define SVDQ_Q(R16)                                                                                         \
  hipLaunchKernelGGL((quantize_rows_kernel<FMT, ACT, R16>), grid, block, shm, s, src, rows, ld, K, lam, l1, \
                     codes, scales, rows_pad, Dout, r_pad)
  if constexpr (!ACT) {
    SVDQ_Q(0);
  } else {
    switch (r_pad / 16) {
      case 0: SVDQ_Q(0); break;
      case 2: SVDQ_Q(2); break;
      case 4: SVDQ_Q(4); break;
      case 6: SVDQ_Q(6); break;
      case 8: SVDQ_Q(8); break;
      case 10: SVDQ_Q(10); break;
      case 12: SVDQ_Q(12); break;
      case 14: SVDQ_Q(14); break;
      case 16: SVDQ_Q(16); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef SVDQ_Q
  return hipGetLastError();
}

hipError_t launch_quantize(int fmt, bool act, const void* src, int64_t rows, int64_t ld, int K, const float* lam,
                           const void* L1f, uint8_t* codes, uint8_t* scales, int64_t rows_pad, uint16_t* Dout,
                           int r_pad, hipStream_t s) {
  if (fmt == kFmtMXFP4)
    return act ? launch_quantize_fmt<kFmtMXFP4, true>(src, rows, ld, K, lam, L1f, codes, scales, rows_pad, Dout, r_pad, s)
               : launch_quantize_fmt<kFmtMXFP4, false>(src, rows, ld, K, lam, L1f, codes, scales, rows_pad, Dout, r_pad, s);
  return act ? launch_quantize_fmt<kFmtINT4, true>(src, rows, ld, K, lam, L1f, codes, scales, rows_pad, Dout, r_pad, s)
             : launch_quantize_fmt<kFmtINT4, false>(src, rows, ld, K, lam, L1f, codes, scales, rows_pad, Dout, r_pad, s);
}

static unsigned grid_for(int64_t total, int block) {
  int64_t g = (total + block - 1) / block;
  if (g > 65536) g = 65536;
  return unsigned(g < 1 ? 1 : g);
}

hipError_t launch_pack_aux(const uint16_t* L1, const uint16_t* L2, const float* lam, const uint16_t* bias, int K,
                           int N, int rank, const WeightLayout& wl, uint8_t* blob, hipStream_t s) {
  if (wl.r_pad > 0) {
    hipLaunchKernelGGL(pack_l1_kernel, dim3(grid_for(int64_t(K) * wl.r_pad, 256)), dim3(256), 0, s,
                       rank > 0 ? L1 : nullptr, K, rank, int(wl.r_pad), reinterpret_cast<uint16_t*>(blob + wl.L1));
    hipLaunchKernelGGL(pack_l2_kernel, dim3(grid_for(wl.N_pad * wl.r_pad, 256)), dim3(256), 0, s,
                       rank > 0 ? L2 : nullptr, N, wl.N_pad, rank, int(wl.r_pad),
                       reinterpret_cast<uint16_t*>(blob + wl.L2));
  }
  const int64_t n = wl.N_pad > K ? wl.N_pad : K;
  hipLaunchKernelGGL(pack_vec_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, lam, K, bias, N, wl.N_pad,
                     reinterpret_cast<float*>(blob + wl.lam), reinterpret_cast<float*>(blob + wl.rlam),
                     reinterpret_cast<uint16_t*>(blob + wl.bias));
  return hipGetLastError();
}

hipError_t launch_unpack_weight(int fmt, int K, int N, int rank, const WeightLayout& wl, const uint8_t* blob,
                                uint8_t* codes, void* scales, uint16_t* L1, uint16_t* L2, float* lam, uint16_t* bias,
                                hipStream_t s) {
  if (codes)
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(grid_for(int64_t(N) * K / 2, 256)), dim3(256), 0, s, fmt,
                       blob + wl.codes, int64_t(N), K, codes);
  if (scales)
    hipLaunchKernelGGL(unpack_scales_kernel, dim3(grid_for(int64_t(N) * K / 32, 256)), dim3(256), 0, s, fmt,
                       blob + wl.scales, int64_t(N), wl.N_pad, K, scales);
  if (rank > 0 && (L1 || L2))
    hipLaunchKernelGGL(unpack_lowrank_kernel, dim3(grid_for(int64_t(K) * rank + int64_t(rank) * N, 256)), dim3(256), 0,
                       s, reinterpret_cast<const uint16_t*>(blob + wl.L1), reinterpret_cast<const uint16_t*>(blob + wl.L2),
                       K, N, rank, int(wl.r_pad), L1, L2);
  if (lam) {
    hipError_t e = hipMemcpyAsync(lam, blob + wl.lam, size_t(K) * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  if (bias) {
    hipError_t e = hipMemcpyAsync(bias, blob + wl.bias, size_t(N) * 2, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_unpack_act(int fmt, int K, int rank, int64_t M, const ActLayout& al, const uint8_t* ws,
                             uint8_t* codes, void* scales, float* D, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (codes)
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(grid_for(M * K / 2, 256)), dim3(256), 0, s, fmt, ws + al.codes, M, K,
                       codes);
  if (scales)
    hipLaunchKernelGGL(unpack_scales_kernel, dim3(grid_for(M * K / 32, 256)), dim3(256), 0, s, fmt, ws + al.scales, M,
                       al.M_pad, K, scales);
  if (D && rank > 0)
    hipLaunchKernelGGL(unpack_d_kernel, dim3(grid_for(M * rank, 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(ws + al.D), M, rank, int(al.r_pad), D);
  return hipGetLastError();
}

}  // namespace svdq
