// Physical layouts of the packed weight blob and the activation workspace.
//
// Everything the GEMM reads is stored in the order one MFMA operand fragment is
// consumed, so each fragment is one fully coalesced 1 KiB load (64 lanes x 16 B)
// and no shuffling happens in the hot loop.
//
// Scaled FP4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4), per 16-row x 128-K tile:
//   lane L holds row (L % 16) and the 32-element K block (L / 16): 16 bytes,
//   element t of the block in byte t/2 (low nibble for even t).  The E8M0 scale
//   of that (row, block) is one byte of a per-lane 32-bit scale register.
//   Scale "superfragment" per 16 rows x 512 K: lane L's dword holds, in byte j,
//   the scale of row L%16, block L/16 of the 128-K step j.
// INT8 MFMA (v_mfma_i32_16x16x64_i8) for INT4: per 16-row x 128-K tile, lane L
//   holds row L%16 and, for both 64-element groups g of the tile, the 16 codes
//   at group offset (L/16)*16: bytes [8g, 8g+8) = 16 nibbles, two dwords of 8
//   codes each.  Inside a dword, code e (0..7) is in byte e%4, low nibble for
//   e < 4: masking the low (high) nibbles gives codes 0-3 (4-7) one per byte, in
//   order, which is what both the int8 expansion and the bf16 conversion of the
//   W4A16 kernel want.  Scales: per 128-K step and row, two fp16 (groups 0 and
//   1) in 4 bytes, rows contiguous.
// NVFP4-style (E2M1 codes, an E4M3 scale per 16): the codes use the MXFP4
//   fragment layout (lane L: row L%16, 32-element block L/16, 16 B).  Scales:
//   per 16-row tile and 128-K step, lane L's two E4M3 bytes (its block's halves
//   0 and 1) at 2 L, 128 B per tile-step.  The weight blob also holds the
//   residual's max |R| (fp32 bits), from which the tensor scale is derived.
// bf16 MFMA (v_mfma_f32_16x16x32_bf16) fragments for the low-rank branch: lane
//   L holds row/column L%16 and 8 consecutive K (rank) elements at (L/16)*8.
//
// Both operands use the same in-lane element order, so the product is the dot
// product over each K block regardless of that order.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace svdq {

constexpr int kTileRows = 256;     // rows of N (weights) and M (activations) are padded to this
constexpr int kFusedTileCols = 128; // narrowest output tile of a GEMM that quantizes its output
constexpr int kKStep = 128;        // K per MFMA step
constexpr int kKSuper = 512;       // K per scale superfragment; K must be a multiple
constexpr int kRankAlign = 32;     // rank padded to the bf16 MFMA K
constexpr int kFmtMXFP4 = 1;
constexpr int kFmtINT4 = 2;
constexpr int kFmtNVFP4 = 3;
constexpr float kNvfp4GlobalDiv = 2688.0f;   // E2M1 max 6 times E4M3 max 448

// Scale bytes per row: K/32 (E8M0 per 32, or fp16 per 64), K/16 for NVFP4 (E4M3 per 16).
__host__ __device__ inline size_t scale_row_bytes(int fmt, int K) { return fmt == kFmtNVFP4 ? K / 16 : K / 32; }
constexpr uint32_t kLamRangeBit = 1;   // weight flags: a lambda outside [2^-32, 2^32]
constexpr uint32_t kDivSlowBit = 2;    // weight flags: the two-operation division is not exact for some lambda

__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ inline size_t align256(size_t a) { return (a + 255) & ~size_t(255); }

struct WeightLayout {
  int64_t N_pad, r_pad;
  size_t codes, scales, L1, L2, lam, rlam, rlo, bias, flags, amax, total;
};

struct ActLayout {
  int64_t M_pad, r_pad;
  int kr, splits;                  // activation kernel: K per workgroup, K splits (K / kr)
  size_t codes, scales, D, part, total;
};

// Codes: N_pad x K/2 bytes.  Scales: N_pad x scale_row_bytes(fmt, K) bytes.
// L1: K x r_pad bf16 (B fragments of the down projection).  L2: N_pad x r_pad bf16
// (A fragments of the up projection).  lambda, r = RN(1/lambda) and the correction
// rl = RN((1 - r lambda) r): fp32[K] each.  bias: bf16[N_pad].  flags: uint32
// (kLamRangeBit, kDivSlowBit).  amax: the NVFP4 residual's max |R| as fp32 bits.
__host__ __device__ inline WeightLayout weight_layout(int fmt, int K, int N, int rank) {
  WeightLayout w;
  w.N_pad = round_up(N, kTileRows);
  w.r_pad = round_up(rank, kRankAlign);
  size_t o = 0;
  w.codes = o;  o = align256(o + size_t(w.N_pad) * K / 2);
  w.scales = o; o = align256(o + size_t(w.N_pad) * scale_row_bytes(fmt, K));
  w.L1 = o;     o = align256(o + size_t(K) * w.r_pad * 2);
  w.L2 = o;     o = align256(o + size_t(w.N_pad) * w.r_pad * 2);
  w.lam = o;    o = align256(o + size_t(K) * 4);
  w.rlam = o;   o = align256(o + size_t(K) * 4);
  w.rlo = o;    o = align256(o + size_t(K) * 4);
  w.bias = o;   o = align256(o + size_t(w.N_pad) * 2);
  w.flags = o;  o = align256(o + 4);
  w.amax = o;   o = align256(o + 4);
  w.total = o;
  return w;
}

constexpr int kActRowTiles = 8;        // 16-row tiles (one per wave) per activation workgroup
constexpr int kActLdsBytes = 81920;    // LDS for one workgroup's lambda, r, rl and L1 fragments (two fit a CU)
constexpr int kActMinWorkgroups = 384; // fewer leave CUs idle

// Work split of the activation kernel: a workgroup takes kActRowTiles 16-row
// tiles and one K range of kr (its lambda, r, rl and L1 fragments staged in
// LDS, kr * (12 + 2 r_pad) bytes).  kr is the largest power of two dividing K
// within the LDS budget, halved (down to 128) while the grid has fewer than
// kActMinWorkgroups workgroups.  With more than one split, each workgroup
// writes an fp32 partial of the down projection, summed in split order by a
// second small kernel.
__host__ __device__ inline void act_split(int K, int r_pad, int64_t M_pad, int* kr_out, int* splits) {
  const int64_t groups = M_pad / (16 * kActRowTiles);
  int kr = 64;
  for (int c = 4096; c >= 64; c /= 2)
    if (K % c == 0 && int64_t(c) * (12 + 2 * r_pad) <= kActLdsBytes) {
      kr = c;
      break;
    }
  while (kr > 128 && groups * (K / kr) < kActMinWorkgroups) kr /= 2;
  *kr_out = kr;
  *splits = K / kr;
}

// Codes: M_pad x K/2.  Scales: M_pad x scale_row_bytes(fmt, K).  D: M_pad x r_pad x {hi, lo} bf16.
// part: fp32 partial down projections, P x M_pad x r_pad, for the larger of the two
// producers: the activation kernel's K splits (when it splits K), and the GEMM of a
// previous layer that quantizes its output for this layer (one partial per tile
// column of that output: K / 128 of them with 128-wide tiles, K / 256 with 256-wide).
__host__ __device__ inline ActLayout act_layout(int fmt, int K, int rank, int64_t M) {
  ActLayout a;
  a.M_pad = round_up(M > 0 ? M : 1, kTileRows);
  a.r_pad = round_up(rank, kRankAlign);
  act_split(K, int(a.r_pad), a.M_pad, &a.kr, &a.splits);
  size_t o = 0;
  a.codes = o;  o = align256(o + size_t(a.M_pad) * K / 2);
  a.scales = o; o = align256(o + size_t(a.M_pad) * scale_row_bytes(fmt, K));
  a.D = o;      o = align256(o + size_t(a.M_pad) * a.r_pad * 4);
  const int nparts = (a.splits > 1 && a.splits > K / kFusedTileCols) ? a.splits : K / kFusedTileCols;
  a.part = o;   o = align256(o + size_t(nparts) * a.M_pad * a.r_pad * 4);
  a.total = o;
  return a;
}

// Bytes of the workspace that the two launches of one layer touch: codes,
// scales, D and the activation kernel's K-split partials (without the room a
// fused producer's partials take).
__host__ __device__ inline size_t act_linear_bytes(const ActLayout& a) {
  return a.part + (a.splits > 1 ? size_t(a.splits) * a.M_pad * a.r_pad * 4 : 0);
}

// ---- codes: byte offset of the 16-byte lane chunk of tile (rt, ks), lane L ----
__host__ __device__ inline size_t code_chunk(int64_t rt, int ks, int K, int L) {
  return (size_t(rt) * (K / kKStep) + ks) * 1024 + size_t(L) * 16;
}

// Canonical (row, k) -> (byte offset, high-nibble?) in the code section.
__host__ __device__ inline size_t code_byte(int fmt, int64_t row, int k, int K, int* hi) {
  const int64_t rt = row / 16;
  const int r = int(row % 16);
  const int ks = k / kKStep;
  const int kk = k % kKStep;
  if (fmt != kFmtINT4) {                         // MXFP4 and NVFP4
    const int blk = kk / 32, t = kk % 32;
    *hi = t & 1;
    return code_chunk(rt, ks, K, blk * 16 + r) + t / 2;
  }
  const int g = kk / 64, o = kk % 64, c = o / 16, t = o % 16, e = t % 8;
  *hi = e >> 2;
  return code_chunk(rt, ks, K, c * 16 + r) + g * 8 + (t / 8) * 4 + (e & 3);
}

// ---- scales ----
// MXFP4: byte offset of the scale of (row, 32-block index kb) (kb = k / 32).
__host__ __device__ inline size_t mx_scale_byte(int64_t row, int kb, int K) {
  const int64_t rt = row / 16;
  const int r = int(row % 16);
  const int ks = kb / 4, blk = kb % 4;          // 128-K step and block within it
  const int sup = ks / 4, j = ks % 4;           // superfragment and byte within the dword
  return ((size_t(rt) * (K / kKSuper) + sup) * 64 + (blk * 16 + r)) * 4 + j;
}
// NVFP4: byte offset of the E4M3 scale of (row, 16-group index kg) (kg = k / 16).
__host__ __device__ inline size_t nv_scale_byte(int64_t row, int kg, int K) {
  const int64_t rt = row / 16;
  const int r = int(row % 16);
  const int ks = kg / 8, blk = (kg / 2) % 4, half = kg % 2;
  return ((size_t(rt) * (K / kKStep) + ks) * 64 + (blk * 16 + r)) * 2 + half;
}
// INT4: byte offset of the fp16 scale of (row, 64-group index g) with rows padded to rows_pad.
__host__ __device__ inline size_t i4_scale_byte(int64_t row, int g, int64_t rows_pad) {
  const int ks = g / 2, h = g % 2;
  return ((size_t(ks) * rows_pad + row) * 2 + h) * 2;
}

// ---- low-rank fragments (bf16 element offsets) ----
// L1 (K x r_pad): B fragment of the down projection, tile (k32, i16), lane L, element e:
//   k = k32*32 + (L/16)*8 + e, i = i16*16 + L%16.
__host__ __device__ inline size_t l1_elem(int k, int i, int r_pad) {
  const int k32 = k / 32, kk = k % 32, i16 = i / 16, L = (kk / 8) * 16 + (i % 16), e = kk % 8;
  return ((size_t(k32) * (r_pad / 16) + i16) * 64 + L) * 8 + e;
}
// L2 (N_pad x r_pad): A fragment of the up projection, tile (n16, r32), lane L, element e:
//   n = n16*16 + L%16, rank = r32*32 + (L/16)*8 + e.
__host__ __device__ inline size_t l2_elem(int64_t n, int rk, int r_pad) {
  const int64_t n16 = n / 16;
  const int r32 = rk / 32, kk = rk % 32, L = (kk / 8) * 16 + int(n % 16), e = kk % 8;
  return ((size_t(n16) * (r_pad / 32) + r32) * 64 + L) * 8 + e;
}
// D (M_pad x r_pad, hi/lo bf16): B fragment of the up projection, tile (m16, r32), part h.
__host__ __device__ inline size_t d_elem(int64_t m, int rk, int h, int r_pad) {
  const int64_t m16 = m / 16;
  const int r32 = rk / 32, kk = rk % 32, L = (kk / 8) * 16 + int(m % 16), e = kk % 8;
  return (((size_t(m16) * (r_pad / 32) + r32) * 2 + h) * 64 + L) * 8 + e;
}

}  // namespace svdq
