// Launch 1 of the layer (quantize_act_kernel) and the weight packer.
//
// Both quantizers apply section 3's max-scaled quantizer of the SVDQuant notes
// page per group of g elements along K (MXFP4: E8M0 power of two with
// e = floor(log2 amax) - 2, g = 32; INT4: fp16(amax / 7), g = 64) and write the
// codes and scales straight into the GEMM's fragment layout.  The activation
// kernel also divides by lambda (the smoothing step of section 4.2) and computes
// the down projection D = X_hat L1 in the same pass over X (section 4.3: the
// down projection is fused into the quantization kernel).
#include <hip/hip_runtime.h>

#include "common.h"

namespace svdq {

// ---- weights (load time): R, fp32, one 16-row tile per workgroup ----
//
// Lane (row = lane % 16, c = lane / 16) holds 8 consecutive elements of each
// 32-element block; the workgroup's NW waves stride over K/512 superchunks.
template <int FMT>
__global__ void __launch_bounds__(512) quantize_weight_kernel(const float* __restrict__ src, int64_t rows,
                                                              int64_t ld, int K, uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales, int64_t rows_pad,
                                                              const uint32_t* __restrict__ amax_bits) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int row = lane & 15, c = lane >> 4;
  const int64_t rt = blockIdx.x;
  const int64_t m = rt * 16 + row;
  const bool valid = m < rows;
  const int nsuper = K / kKSuper;
  // NVFP4: the tensor scale gs = fp32(max|R| / 2688)
  const float gs = FMT == kFmtNVFP4 ? __uint_as_float(*amax_bits) / kNvfp4GlobalDiv : 1.0f;

  for (int kc = w; kc < nsuper; kc += nw) {
    uint32_t sdw = 0;  // MXFP4: this lane's scale dword of the superfragment
#pragma unroll 2
    for (int p = 0; p < 8; ++p) {  // 64-element units of the 512 chunk
      float x[16];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = kc * kKSuper + (2 * p + h) * 32 + c * 8;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (valid) {
          const float* s = src + m * ld + k;
          a = *reinterpret_cast<const float4*>(s);
          b = *reinterpret_cast<const float4*>(s + 4);
        }
        x[8 * h + 0] = a.x; x[8 * h + 1] = a.y; x[8 * h + 2] = a.z; x[8 * h + 3] = a.w;
        x[8 * h + 4] = b.x; x[8 * h + 5] = b.y; x[8 * h + 6] = b.z; x[8 * h + 7] = b.w;
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
          const float so = scale_operand(sb);
          uint32_t cw = 0;
          cw = cvt_fp4x2_div<0>(cw, x[8 * h + 0], x[8 * h + 1], so);
          cw = cvt_fp4x2_div<1>(cw, x[8 * h + 2], x[8 * h + 3], so);
          cw = cvt_fp4x2_div<2>(cw, x[8 * h + 4], x[8 * h + 5], so);
          cw = cvt_fp4x2_div<3>(cw, x[8 * h + 6], x[8 * h + 7], so);
          const int ks = kc * 4 + jb / 4;
          *reinterpret_cast<uint32_t*>(codes + code_chunk(rt, ks, K, (jb & 3) * 16 + row) + c * 4) = cw;
          if ((jb & 3) == c) sdw |= sb << (8 * (jb >> 2));
        }
      } else if (FMT == kFmtNVFP4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jb = 2 * p + h;  // 32-block within the superchunk
          // this lane's 8 elements are half c / 2 of the 32-block: a 16-group
          // shared with lane ^ 16
          float amax = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[8 * h + e]));
          amax = rowpair_max(amax);
          const float a6 = amax / 6.0f;
          const uint32_t sb = e4m3_rne(gs != 0.0f ? a6 / gs : 0.0f);
          const float S = e4m3_value(sb) * gs;
          float t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = S != 0.0f ? x[8 * h + e] / S : x[8 * h + e] * 0.0f;
          uint32_t cw = 0;
          cw = cvt_fp4x2<0>(cw, t[0], t[1]);
          cw = cvt_fp4x2<1>(cw, t[2], t[3]);
          cw = cvt_fp4x2<2>(cw, t[4], t[5]);
          cw = cvt_fp4x2<3>(cw, t[6], t[7]);
          const int ks = kc * 4 + jb / 4;
          *reinterpret_cast<uint32_t*>(codes + code_chunk(rt, ks, K, (jb & 3) * 16 + row) + c * 4) = cw;
          if ((c & 1) == 0) {
            const int kg = (kc * kKSuper + jb * 32) / 16 + c / 2;
            scales[nv_scale_byte(m, kg, K)] = uint8_t(sb);
          }
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
            cw |= (uint32_t(q) & 0xFu) << (8 * (e & 3) + 4 * (e >> 2));  // INT4 dword order
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
    }
    if (FMT == kFmtMXFP4)
      *reinterpret_cast<uint32_t*>(scales + (size_t(rt) * nsuper + kc) * 256 + lane * 4) = sdw;
  }
}

// ---- launch 1 for activations ----
//
// Workgroup = kActRowTiles waves, one 16-row tile each, over one K range of kr
// (a split of K).  The workgroup first stages lambda, 1/lambda and the L1
// fragments of its K range in LDS; the only global loads in the main loop are
// then the wave's own X, issued kActDepth steps ahead (loads complete in issue
// order, so no other load ever waits behind the X prefetch).  Lane
// (row = lane % 16, c = lane / 16) holds 8 consecutive elements of each
// 32-element block: the A fragment of the bf16 16x16x32 MFMA, so the down
// projection runs on the same registers.  The smoothing divide is the refined
// reciprocal division (same result as IEEE division, far fewer operations); the
// group maximum over the 4 lanes of a row uses the VALU lane swaps.


constexpr int kActStep = 64;   // K per pipeline step: two 32-blocks (one INT4 group)
constexpr int kActDepth = 3;   // steps of X in flight ahead of the one being computed

// Register budget by down-projection width: waves per SIMD the compiler must
// leave room for (the L1 fragments and accumulators grow with the rank).
__host__ __device__ constexpr int act_min_waves(int r16) { return r16 <= 2 ? 4 : (r16 <= 8 ? 2 : 1); }

// Grid: (row tiles / kActRowTiles, K splits); block: kActRowTiles waves;
// dynamic LDS: kr * (8 + 2 r_pad) bytes.  With one split the waves write D;
// otherwise their fp32 partials go to `part` and reduce_down_kernel sums them.
// Loads and stores go through buffer resources with a per-wave base, so the
// per-step addressing is a scalar offset (no 64-bit vector address math).
template <int FMT, int R16>
__global__ void __launch_bounds__(64 * kActRowTiles, act_min_waves(R16)) quantize_act_kernel(
    const uint16_t* __restrict__ X, int64_t rows, int64_t ld, int K, const float* __restrict__ lam,
    const float* __restrict__ rlam, const float* __restrict__ rlo, const uint4* __restrict__ L1f,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t rows_pad, uint16_t* __restrict__ Dout,
    float* __restrict__ part, int r_pad, int kr, const uint32_t* __restrict__ wflags) {
  extern __shared__ uint4 smem[];  // lambda[kr], r[kr], rl[kr] (fp32), then L1 fragments [kr/32][R16][64]
  float* const slam = reinterpret_cast<float*>(smem);
  float* const srlam = slam + kr;
  float* const srlo = srlam + kr;
  uint4* const sl1 = smem + 3 * kr / 4;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, c = lane >> 4;
  const int64_t rt = int64_t(blockIdx.x) * kActRowTiles + w;
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int k_beg = split * kr;
  const int64_t m = rt * 16 + row;
  const int KS = K / kKStep, nsuper = K / kKSuper;
  const int nsteps = kr / kActStep;

  // Per-wave buffer views.  X: the tile's 16 rows from k_beg on; rows past the
  // end read the last row (their codes are never read back: the GEMM drops
  // those outputs and the unpacking stops at M).
  const int64_t row0 = rt * 16 < rows ? rt * 16 : rows - 1;
  const int64_t my_row = m < rows ? m : rows - 1;
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(X + row0 * ld + k_beg, uint32_t((16 * ld) * 2));
  const uint32_t xoff = uint32_t((my_row - row0) * ld * 2 + c * 16);
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(codes + size_t(rt) * KS * 1024, uint32_t(KS) * 1024);
  // scales of the tile: MXFP4 nsuper superfragments of 256 B; NVFP4 KS steps of 128 B
  const __amdgpu_buffer_rsrc_t rS =
      FMT == kFmtNVFP4 ? make_rsrc(scales + size_t(rt) * KS * 128, uint32_t(KS) * 128)
                       : make_rsrc(scales + size_t(rt) * nsuper * 256, uint32_t(nsuper) * 256);
  auto load_x = [&](int p, uint4& lo, uint4& hi) {
    const int q = p < nsteps ? p : nsteps - 1;   // past the end: an in-bounds load that is never used
    lo = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rX, xoff, uint32_t(q) * 128, 0));
    hi = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rX, xoff, uint32_t(q) * 128 + 64, 0));
  };

  // X of the first kActDepth steps, then the LDS staging of this K range.
  uint4 xs[kActDepth + 1][2];
#pragma unroll
  for (int j = 0; j < kActDepth; ++j) load_x(j, xs[j][0], xs[j][1]);
  // The staging is done by loads that write LDS directly: no register round
  // trip, every chunk in flight at once (a copy through registers waits for
  // each load in turn); the barrier's wait covers them.  lambda, 1/lambda and
  // the correction: kr / 64 chunks of 256 bytes each.
  {
    const int nl = kr / 64;
    const __amdgpu_buffer_rsrc_t rl0 = make_rsrc(lam + k_beg, uint32_t(kr) * 4);
    const __amdgpu_buffer_rsrc_t rl1 = make_rsrc(rlam + k_beg, uint32_t(kr) * 4);
    const __amdgpu_buffer_rsrc_t rl2 = make_rsrc(rlo + k_beg, uint32_t(kr) * 4);
    for (int ci = w; ci < 3 * nl; ci += kActRowTiles) {
      const int a = ci / nl, o = ci % nl;
      float* const dst = (a == 0 ? slam : a == 1 ? srlam : srlo) + o * 64;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a == 0 ? rl0 : a == 1 ? rl1 : rl2,
                                               (__attribute__((address_space(3))) void*)(dst), 4,
                                               uint32_t(lane) * 4, uint32_t(o) * 256, 0, 0);
    }
  }
  if (R16 > 0) {
    // the L1 fragments of this K range: (kr / 32) R16 chunks of 1 KiB
    const int nchunk = (kr / 32) * R16;
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(L1f + size_t(k_beg / 32) * R16 * 64, uint32_t(nchunk) * 1024);
    for (int ci = w; ci < nchunk; ci += kActRowTiles)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (__attribute__((address_space(3))) void*)(sl1 + ci * 64), 16,
                                               uint32_t(lane) * 16, uint32_t(ci) * 1024, 0, 0);
  }
  __syncthreads();

  v4f dacc[R16 > 0 ? R16 : 1];
#pragma unroll
  for (int i = 0; i < (R16 > 0 ? R16 : 1); ++i) dacc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  // Division path of the layer (uniform for the launch): with every lambda in
  // [2^-32, 2^32], the two-operation quotient fma(x, r, x rl) when the weight
  // packing verified it exact for every lambda, else the refined division;
  // with some lambda outside that range, IEEE division everywhere.
  const uint32_t wf = __builtin_amdgcn_readfirstlane(*wflags);
  const bool ieee_only = (wf & kLamRangeBit) != 0;
  const bool div2 = (wf & kDivSlowBit) == 0;

  // One 64-K step on the X held in (xa, xb).
  auto step = [&](int p, const uint4& xa, const uint4& xb) {
    const int kl = p * kActStep;                  // K offset inside the range
    // The fast divisions (and, for INT4, the refined division by the group
    // scale) equal the IEEE quotient when |x| is in [2^-40, 2^60) and lambda in
    // [2^-32, 2^32]: every product, quotient and remainder then stays far inside
    // the normal range.  Checked on the bf16 exponent fields, two per dword: the
    // biased exponent must lie in [87, 187) (+0 passes; -0 and subnormals fail).
    const bool fast = !ieee_only && !__any(exp_out_of_range(xa, xb));
    float x[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ko = kl + h * 32 + c * 8;
      auto ld8 = [&](const float* v, float (&o)[8]) {
        const float4 u0 = *reinterpret_cast<const float4*>(v + ko), u1 = *reinterpret_cast<const float4*>(v + ko + 4);
        o[0] = u0.x; o[1] = u0.y; o[2] = u0.z; o[3] = u0.w; o[4] = u1.x; o[5] = u1.y; o[6] = u1.z; o[7] = u1.w;
      };
      float a[8], r[8];
      unpack_bf8(h == 0 ? xa : xb, a);
      ld8(srlam, r);
      if (__builtin_expect(fast && div2, 1)) {
        float rl[8];
        ld8(srlo, rl);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * h + e] = fmaf(a[e], r[e], a[e] * rl[e]);
      } else if (fast) {
        float lv[8];
        ld8(slam, lv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * h + e] = div_refined(a[e], lv[e], r[e]);
      } else {
        float lv[8];
        ld8(slam, lv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * h + e] = a[e] / lv[e];
      }
    }

    const int kb0 = (k_beg + kl) / 32;            // global 32-block index of the step's first block
    const int ks = kb0 / 4;                       // 128-K step
    if (FMT == kFmtMXFP4) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = kb0 + h;
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
        __builtin_amdgcn_raw_buffer_store_b32(cw, rC, uint32_t(row * 16 + c * 4),
                                              uint32_t(ks * 1024 + (kb & 3) * 256), 0);
        // the scale of (row, block kb & 3 of its 128-K step) is byte ks % 4 of
        // that lane's superfragment dword: this lane when c == kb & 3
        if (c == (kb & 3))
          __builtin_amdgcn_raw_buffer_store_b8(uint8_t(sb), rS, uint32_t(lane * 4), uint32_t((kb / 16) * 256 + ks % 4),
                                               0);
      }
    } else if (FMT == kFmtNVFP4) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = kb0 + h;
        // the lane's 8 elements are half c / 2 of the 32-block, a 16-group shared with lane ^ 16;
        // the activations' tensor scale is 1, so the group scale is E4M3(amax / 6)
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[8 * h + e]));
        amax = rowpair_max(amax);
        const uint32_t sb = e4m3_rne(amax / 6.0f);
        const float S = e4m3_value(sb);
        const float rs = 1.0f / S;
        float t[8];
        if (__builtin_expect(fast, 1)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = div_refined(x[8 * h + e], S, rs);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = x[8 * h + e] / S;
        }
        // a zero scale (the whole group rounds it to 0): signed zeros
        if (S == 0.0f) {
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = x[8 * h + e] * 0.0f;
        }
        uint32_t cw = 0;
        cw = cvt_fp4x2<0>(cw, t[0], t[1]);
        cw = cvt_fp4x2<1>(cw, t[2], t[3]);
        cw = cvt_fp4x2<2>(cw, t[4], t[5]);
        cw = cvt_fp4x2<3>(cw, t[6], t[7]);
        __builtin_amdgcn_raw_buffer_store_b32(cw, rC, uint32_t(row * 16 + c * 4),
                                              uint32_t(ks * 1024 + (kb & 3) * 256), 0);
        // scale byte of (row, 16-group): GEMM lane (kb & 3) * 16 + row, half c / 2
        if ((c & 1) == 0)
          __builtin_amdgcn_raw_buffer_store_b8(uint8_t(sb), rS, uint32_t(((kb & 3) * 16 + row) * 2 + c / 2),
                                               uint32_t(ks * 128), 0);
      }
    } else {
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
      amax = rowgroup_max(amax);
      const float s32 = amax / 7.0f;
      const _Float16 h16 = (_Float16)fminf(s32, 65504.0f);
      const float sc = (float)h16;
      const float rs = 1.0f / sc;
      const int g = kb0 / 2, gi = g & 1;          // 64-group and its index in the 128-K step
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // a zero scale (every x of the group rounds it to 0) gives codes 0
        // whatever t is, so the quotient only matters for a positive scale
        float t[8];
        if (__builtin_expect(fast, 1)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = div_refined(x[8 * h + e], sc, rs);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = x[8 * h + e] / sc;
        }
        uint32_t cw = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float tq = __builtin_rintf(fminf(fmaxf(t[e], -8.0f), 7.0f));
          const int q = (sc == 0.0f) ? 0 : int(tq);
          cw |= (uint32_t(q) & 0xFu) << (8 * (e & 3) + 4 * (e >> 2));  // INT4 dword order
        }
        // group offset o = 32h + 8c: lane chunk (o / 16) * 16 + row, bytes 8 gi + (o % 16) / 2
        __builtin_amdgcn_raw_buffer_store_b32(cw, rC, uint32_t((c / 2) * 256 + row * 16 + (c % 2) * 4),
                                              uint32_t(ks * 1024 + h * 512 + gi * 8), 0);
      }
      if (c == 0) *reinterpret_cast<_Float16*>(scales + i4_scale_byte(m, g, rows_pad)) = h16;
    }

    if (R16 > 0) {
      // Down projection: x_hat as a bf16 hi + lo pair (about 16 significant
      // bits) against the bf16 L1, accumulated in fp32.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 hi, lo;
        hi.x = cvt_bf2(x[8 * h + 0], x[8 * h + 1]);
        hi.y = cvt_bf2(x[8 * h + 2], x[8 * h + 3]);
        hi.z = cvt_bf2(x[8 * h + 4], x[8 * h + 5]);
        hi.w = cvt_bf2(x[8 * h + 6], x[8 * h + 7]);
        lo.x = cvt_bf2(x[8 * h + 0] - bf_lo(hi.x), x[8 * h + 1] - bf_hi(hi.x));
        lo.y = cvt_bf2(x[8 * h + 2] - bf_lo(hi.y), x[8 * h + 3] - bf_hi(hi.y));
        lo.z = cvt_bf2(x[8 * h + 4] - bf_lo(hi.z), x[8 * h + 5] - bf_hi(hi.z));
        lo.w = cvt_bf2(x[8 * h + 6] - bf_lo(hi.w), x[8 * h + 7] - bf_hi(hi.w));
        const uint4* bf = sl1 + size_t((2 * p + h) * R16) * 64 + lane;
#pragma unroll
        for (int ib = 0; ib < (R16 > 0 ? R16 : 1); ++ib) {
          const uint4 b = bf[ib * 64];
          dacc[ib] = mfma_bf16(hi, b, dacc[ib]);
          dacc[ib] = mfma_bf16(lo, b, dacc[ib]);
        }
      }
    }
  };

  // X stages form a ring of kActDepth + 1 register sets: step p uses set p % 4
  // and refills the set of step p - 1 with step p + 3.  Four steps per
  // iteration keep the set indices compile-time; a range of 1 or 2 steps
  // (large ranks) takes the short loop that rotates the sets instead.
  static_assert(kActDepth == 3, "ring of four register sets");
  if (nsteps % 4 == 0) {
    for (int p = 0; p < nsteps; p += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        load_x(p + j + 3, xs[(j + 3) & 3][0], xs[(j + 3) & 3][1]);
        step(p + j, xs[j][0], xs[j][1]);
      }
    }
  } else {
    for (int p = 0; p < nsteps; ++p) {
      load_x(p + 3, xs[3][0], xs[3][1]);
      step(p, xs[0][0], xs[0][1]);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        xs[j][0] = xs[j + 1][0];
        xs[j][1] = xs[j + 1][1];
      }
    }
  }

  if (R16 > 0) {
    // Lane holds rows (lane / 16) * 4 + e, column ib * 16 + lane % 16 of its tile.
#pragma unroll
    for (int ib = 0; ib < (R16 > 0 ? R16 : 1); ++ib)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t mm = rt * 16 + (lane >> 4) * 4 + e;
        const int col = ib * 16 + (lane & 15);
        const float v = dacc[ib][e];
        if (nsplit > 1) {
          part[(size_t(split) * rows_pad + mm) * r_pad + col] = v;
        } else {
          const uint32_t hb = f2bf(v);
          const uint32_t lb = f2bf(v - bf_lo(hb));
          Dout[d_elem(mm, col, 0, r_pad)] = uint16_t(hb);
          Dout[d_elem(mm, col, 1, r_pad)] = uint16_t(lb);
        }
      }
  }
}

// Sum of the K splits' partial down projections, in split order, stored as
// the bf16 hi + lo pair the GEMM epilogue reads.  Each thread takes 4
// consecutive columns; the loads of 4 splits go out before their sums.
__global__ void reduce_down_kernel(const float* __restrict__ part, int splits, int64_t rows_pad, int r_pad,
                                   uint16_t* __restrict__ Dout) {
  const int64_t total = rows_pad * r_pad;
  const int64_t i4 = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i4 >= total) return;
  const float4* src = reinterpret_cast<const float4*>(part + i4);
  const int64_t stride = total / 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  int sp = 0;
  for (; sp + 4 <= splits; sp += 4) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[(sp + u) * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
    }
  }
  for (; sp < splits; ++sp) {
    const float4 v = src[sp * stride];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  const float vals[4] = {s.x, s.y, s.z, s.w};
  const int64_t mm = i4 / r_pad;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int col = int(i4 % r_pad) + e;
    const uint32_t hb = f2bf(vals[e]);
    const uint32_t lb = f2bf(vals[e] - bf_lo(hb));
    Dout[d_elem(mm, col, 0, r_pad)] = uint16_t(hb);
    Dout[d_elem(mm, col, 1, r_pad)] = uint16_t(lb);
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
                                float* __restrict__ rlo_out, uint16_t* __restrict__ bias_out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < K) {
    const float v = lam[i];
    const float r = 1.0f / v;                    // RN(1/lambda)
    lam_out[i] = v;
    rlam_out[i] = r;
    rlo_out[i] = fmaf(-r, v, 1.0f) * r;          // (1 - r lambda) is exact; rl ~ 1/lambda - r
  }
  if (i < N_pad) bias_out[i] = (bias != nullptr && i < N) ? bias[i] : uint16_t(0);
}

// Flags word of the packed weights, for the activation kernel's smoothing divide
// x / lambda of bf16 x:
//   kLamRangeBit: some lambda outside [2^-32, 2^32] (or not finite); the layer
//     then takes the IEEE division throughout.
//   kDivSlowBit: for some lambda the two-operation quotient fma(x, r, x rl)
//     differs from the IEEE quotient for some bf16 x; the layer then takes the
//     refined division (five operations) instead.  The check covers every bf16
//     mantissa (x = m / 128, m in [128, 256)); scaling x by a power of two
//     scales every step exactly while nothing under- or overflows, which the
//     kernel's exponent range check ensures, and the sign is symmetric.
// One workgroup; a fixed-order reduction, so no prior zeroing is needed.
__global__ void __launch_bounds__(1024) check_lambda_kernel(const float* __restrict__ lam,
                                                            const float* __restrict__ rlam,
                                                            const float* __restrict__ rlo, int K,
                                                            uint32_t* __restrict__ flags) {
  __shared__ uint32_t red[1024];
  uint32_t bad = 0;
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    const float v = lam[i];
    if (!(v >= 0x1p-32f && v <= 0x1p32f)) {      // false for NaN too
      bad |= kLamRangeBit;
      continue;
    }
    const float r = rlam[i], rl = rlo[i];
    for (int mnt = 128; mnt < 256; ++mnt) {
      const float x = float(mnt) * 0x1p-7f;
      if (fmaf(x, r, x * rl) != x / v) bad |= kDivSlowBit;
    }
  }
  red[threadIdx.x] = bad;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w /= 2) {
    if (int(threadIdx.x) < w) red[threadIdx.x] |= red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *flags = red[0];
}

// ---- NVFP4 tensor maximum (load time) ----

__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

// max |R| over rows x K (row stride ld) into *out as fp32 bits: non-negative
// floats order like their bit patterns, so an unsigned atomic max suffices.
__global__ void __launch_bounds__(256) abs_max_kernel(const float* __restrict__ src, int64_t rows, int64_t ld, int K,
                                                      uint32_t* __restrict__ out) {
  const int64_t total = rows * (K / 4);
  float m = 0.f;
  for (int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = d / (K / 4);
    const int j = int(d % (K / 4));
    const float4 v = *reinterpret_cast<const float4*>(src + r * ld + 4 * j);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  // one atomic per workgroup (a few hundred in all: many on one address serialize)
  __shared__ float wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(out, __float_as_uint(fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]))));
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
  const int ng = (fmt == kFmtMXFP4) ? K / 32 : (fmt == kFmtNVFP4 ? K / 16 : K / 64);
  const int64_t total = rows * ng;
  for (int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = d / ng;
    const int g = int(d % ng);
    if (fmt == kFmtMXFP4)
      reinterpret_cast<uint8_t*>(out)[d] = scales[mx_scale_byte(r, g, K)];
    else if (fmt == kFmtNVFP4)
      reinterpret_cast<uint8_t*>(out)[d] = scales[nv_scale_byte(r, g, K)];
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

// D = the sum of `splits` fp32 partials (splits x rows_pad x r_pad), in order, as bf16 hi + lo.
hipError_t launch_reduce_down(const float* part, int splits, int64_t rows_pad, int r_pad, uint16_t* Dout,
                              hipStream_t s) {
  const int64_t total = rows_pad * r_pad;   // a multiple of 4 (r_pad is a multiple of 32)
  hipLaunchKernelGGL(reduce_down_kernel, dim3(unsigned((total / 4 + 255) / 256)), dim3(256), 0, s, part, splits,
                     rows_pad, r_pad, Dout);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_quantize_act_fmt(const uint16_t* X, int64_t rows, int64_t ld, int K, const float* lam,
                                          const float* rlam, const float* rlo, const void* L1f, uint8_t* codes,
                                          uint8_t* scales,
                                          int64_t rows_pad, uint16_t* Dout, float* part, int r_pad, int kr,
                                          int splits, const uint32_t* wflags, hipStream_t s) {
  const dim3 grid(unsigned(rows_pad / (16 * kActRowTiles)), unsigned(splits)), block(64 * kActRowTiles);
  const size_t shm = size_t(kr) * (12 + 2 * r_pad);
  const uint4* l1 = reinterpret_cast<const uint4*>(L1f);
#define SVDQ_QA(R16)                                                                                      \
  hipLaunchKernelGGL((quantize_act_kernel<FMT, R16>), grid, block, shm, s, X, rows, ld, K, lam, rlam, rlo, l1, \
                     codes, scales, rows_pad, Dout, part, r_pad, kr, wflags)
  switch (r_pad / 16) {
    case 0: SVDQ_QA(0); break;
    case 2: SVDQ_QA(2); break;
    case 4: SVDQ_QA(4); break;
    case 6: SVDQ_QA(6); break;
    case 8: SVDQ_QA(8); break;
    case 10: SVDQ_QA(10); break;
    case 12: SVDQ_QA(12); break;
    case 14: SVDQ_QA(14); break;
    case 16: SVDQ_QA(16); break;
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_QA
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1 || r_pad == 0) return e;
  return launch_reduce_down(part, splits, rows_pad, r_pad, Dout, s);
}

hipError_t launch_quantize_act(int fmt, const uint16_t* X, int64_t rows, int64_t ld, int K, const float* lam,
                               const float* rlam, const float* rlo, const void* L1f, uint8_t* codes, uint8_t* scales,
                               int64_t rows_pad,
                               uint16_t* Dout, float* part, int r_pad, int kr, int splits, const uint32_t* wflags,
                               hipStream_t s) {
  if (fmt == kFmtMXFP4)
    return launch_quantize_act_fmt<kFmtMXFP4>(X, rows, ld, K, lam, rlam, rlo, L1f, codes, scales, rows_pad, Dout, part,
                                              r_pad, kr, splits, wflags, s);
  if (fmt == kFmtNVFP4)
    return launch_quantize_act_fmt<kFmtNVFP4>(X, rows, ld, K, lam, rlam, rlo, L1f, codes, scales, rows_pad, Dout, part,
                                              r_pad, kr, splits, wflags, s);
  return launch_quantize_act_fmt<kFmtINT4>(X, rows, ld, K, lam, rlam, rlo, L1f, codes, scales, rows_pad, Dout, part,
                                           r_pad, kr, splits, wflags, s);
}

static unsigned grid_for(int64_t total, int block);

// NVFP4 first writes max |R| to amax_bits (the tensor scale's source).
hipError_t launch_quantize_weight(int fmt, const float* R, int64_t rows, int64_t ld, int K, uint8_t* codes,
                                  uint8_t* scales, int64_t rows_pad, uint32_t* amax_bits, hipStream_t s) {
  const int nw = pick_waves(K);
  const dim3 grid(unsigned(rows_pad / 16)), block(unsigned(64 * nw));
  if (fmt == kFmtMXFP4) {
    hipLaunchKernelGGL((quantize_weight_kernel<kFmtMXFP4>), grid, block, 0, s, R, rows, ld, K, codes, scales, rows_pad,
                       amax_bits);
  } else if (fmt == kFmtNVFP4) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, s, amax_bits);
    const unsigned gm = grid_for(rows * (K / 4), 256);
    hipLaunchKernelGGL(abs_max_kernel, dim3(gm < 512 ? gm : 512), dim3(256), 0, s, R, rows, ld, K, amax_bits);
    hipLaunchKernelGGL((quantize_weight_kernel<kFmtNVFP4>), grid, block, 0, s, R, rows, ld, K, codes, scales, rows_pad,
                       amax_bits);
  } else {
    hipLaunchKernelGGL((quantize_weight_kernel<kFmtINT4>), grid, block, 0, s, R, rows, ld, K, codes, scales, rows_pad,
                       amax_bits);
  }
  return hipGetLastError();
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
                     reinterpret_cast<float*>(blob + wl.rlo), reinterpret_cast<uint16_t*>(blob + wl.bias));
  hipLaunchKernelGGL(check_lambda_kernel, dim3(1), dim3(1024), 0, s, reinterpret_cast<const float*>(blob + wl.lam),
                     reinterpret_cast<const float*>(blob + wl.rlam), reinterpret_cast<const float*>(blob + wl.rlo), K,
                     reinterpret_cast<uint32_t*>(blob + wl.flags));
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
