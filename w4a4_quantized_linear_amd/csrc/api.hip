// C ABI of libsvdq.so: argument validation, size queries and launches.
// Every check runs on the host before anything is enqueued; see include/svdq.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "svdq.h"
#include "layout.h"

namespace svdq {
hipError_t launch_quantize_weight(int fmt, const float* R, int64_t rows, int64_t ld, int K, uint8_t* codes,
                                  uint8_t* scales, int64_t rows_pad, uint32_t* amax_bits, hipStream_t s);
hipError_t launch_quantize_act(int fmt, const uint16_t* X, int64_t rows, int64_t ld, int K, const float* lam,
                               const float* rlam, const float* rlo, const void* L1f, uint8_t* codes, uint8_t* scales,
                               int64_t rows_pad,
                               uint16_t* Dout, float* part, int r_pad, int kr, int splits, const uint32_t* wflags,
                               hipStream_t s);
hipError_t launch_pack_aux(const uint16_t* L1, const uint16_t* L2, const float* lam, const uint16_t* bias, int K,
                           int N, int rank, const WeightLayout& wl, uint8_t* blob, hipStream_t s);
hipError_t launch_gemm(int fmt, const uint8_t* wblob, const WeightLayout& wl, const uint8_t* act, const ActLayout& al,
                       int K, int N, int64_t M, void* Y, int64_t ldy, uint32_t epi, hipStream_t s);
hipError_t launch_gemm_quant(int fmt, const uint8_t* wblob, const WeightLayout& wl, const uint8_t* act,
                             const ActLayout& al, int K, int N, int64_t M, uint32_t epi, const uint8_t* nblob,
                             const WeightLayout& nwl, uint8_t* nact, const ActLayout& nal, hipStream_t s);
hipError_t launch_gemm_qkv(int fmt, const uint8_t* wblob, const WeightLayout& wl, const uint8_t* act,
                           const ActLayout& al, int K, int N, int64_t M, void* Y, int64_t ldy, uint32_t epi,
                           const uint16_t* norm_q,
                           const uint16_t* norm_k, float eps, const float* rope_cos, const float* rope_sin,
                           hipStream_t s);
hipError_t launch_gemm_w4a16(const uint8_t* wblob, const WeightLayout& wl, int K, int N, const uint16_t* X,
                             int64_t ldx, int64_t M, void* Y, int64_t ldy, uint32_t epi, hipStream_t s);
hipError_t launch_unpack_weight(int fmt, int K, int N, int rank, const WeightLayout& wl, const uint8_t* blob,
                                uint8_t* codes, void* scales, uint16_t* L1, uint16_t* L2, float* lam, uint16_t* bias,
                                hipStream_t s);
hipError_t launch_unpack_act(int fmt, int K, int rank, int64_t M, const ActLayout& al, const uint8_t* ws,
                             uint8_t* codes, void* scales, float* D, hipStream_t s);
}  // namespace svdq

using namespace svdq;

// Scratch of svdq_linear_noalloc: the layer's activation workspace (codes,
// scales, D, K-split partials) in a static device array, one copy per GPU the
// library runs on, held until the process ends.  Host code never uses the
// array's name as an address: each device's address comes from
// hipGetSymbolAddress, taken once with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int64_t kMaxRows = int64_t(1) << 26;
constexpr int kGemmQuantMaxRank = 64;   // next layer's rank in svdq_gemm_quant (4 rank tiles of 16)
constexpr int kQkvHeadDim = 128;        // svdq_gemm_qkv: one head per 128 output columns of a wave
constexpr int64_t kMaxLdx = int64_t(1) << 24;   // 16 rows of X within a kernel's 32-bit buffer range
constexpr uint32_t kEpiAll = SVDQ_EPI_LOWRANK | SVDQ_EPI_BIAS | SVDQ_EPI_GELU | SVDQ_EPI_OUT_F32;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

svdq_status check_shape(const svdq_layer_desc* d) {
  if (d->K <= 0 || d->K % kKSuper != 0 || d->K > 65536) return SVDQ_ERR_SHAPE;
  if (d->N < 16 || d->N % 16 != 0 || d->N > 65536) return SVDQ_ERR_SHAPE;
  if (d->rank < 0 || d->rank > 256) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

svdq_status check_fmt(const svdq_layer_desc* d) {
  return (d->fmt == SVDQ_MXFP4 || d->fmt == SVDQ_INT4_G64 || d->fmt == SVDQ_NVFP4) ? SVDQ_OK : SVDQ_ERR_FORMAT;
}

// Architecture check, cached per device: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_cache[64];
std::atomic<int> g_force_device_fail{0};

svdq_status device_check() {
  if (g_force_device_fail.load()) return SVDQ_ERR_DEVICE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SVDQ_ERR_DEVICE;
  if (dev < 64) {
    const int c = g_arch_cache[dev].load();
    if (c == 1) return SVDQ_OK;
    if (c == 2) return SVDQ_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SVDQ_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch_cache[dev].store(ok ? 1 : 2);
  return ok ? SVDQ_OK : SVDQ_ERR_DEVICE;
}

svdq_status launched(hipError_t e) { return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_LAUNCH; }

// Per-device address of `scratch` (nullptr until the first svdq_linear_noalloc on that device).
std::atomic<uint8_t*> g_scratch_addr[64];

// Device address of this device's scratch array, looked up on the first call
// per device (SVDQ_ERR_DEVICE if the lookup fails).
svdq_status scratch_address(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SVDQ_ERR_DEVICE;
  uint8_t* p = g_scratch_addr[dev].load();
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return SVDQ_ERR_DEVICE;
    p = static_cast<uint8_t*>(q);
    g_scratch_addr[dev].store(p);
  }
  *out = p;
  return SVDQ_OK;
}

svdq_status check_act_args(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X, int64_t M, int64_t ldx,
                           const void* a_packed) {
  if (!d || !w_packed || !a_packed || (M > 0 && !X)) return SVDQ_ERR_NULL;
  svdq_status s = check_shape(d);
  if (s != SVDQ_OK) return s;
  if (M < 0 || M > kMaxRows || ldx < d->K || ldx > kMaxLdx) return SVDQ_ERR_SHAPE;
  if ((s = check_fmt(d)) != SVDQ_OK) return s;
  if (!aligned(w_packed, 256) || !aligned(a_packed, 256) || (M > 0 && !aligned(X, 16)) || ldx % 8 != 0)
    return SVDQ_ERR_ALIGN;
  return SVDQ_OK;
}

svdq_status check_gemm_args(const svdq_layer_desc* d, const void* w_packed, const void* a_packed, int64_t M, void* Y,
                            int64_t ldy, uint32_t epi) {
  if (!d || !w_packed || !a_packed || (M > 0 && !Y)) return SVDQ_ERR_NULL;
  svdq_status s = check_shape(d);
  if (s != SVDQ_OK) return s;
  if (M < 0 || M > kMaxRows || ldy < d->N) return SVDQ_ERR_SHAPE;
  if ((s = check_fmt(d)) != SVDQ_OK) return s;
  if ((epi & ~kEpiAll) != 0) return SVDQ_ERR_FORMAT;
  if (!aligned(w_packed, 256) || !aligned(a_packed, 256) || (M > 0 && !aligned(Y, 16)) || ldy % 8 != 0)
    return SVDQ_ERR_ALIGN;
  return SVDQ_OK;
}

}  // namespace

extern "C" {

int svdq_version(void) { return 107; }

const char* svdq_status_str(svdq_status s) {
  switch (s) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_NULL: return "a required pointer is NULL";
    case SVDQ_ERR_SHAPE: return "unsupported shape (K % 512, N % 16, 0 <= rank <= 256, M, ldx/ldy)";
    case SVDQ_ERR_FORMAT: return "unknown format or epilogue flag";
    case SVDQ_ERR_ALIGN: return "misaligned pointer or row stride";
    case SVDQ_ERR_WORKSPACE: return "workspace smaller than svdq_act_bytes";
    case SVDQ_ERR_DEVICE: return "no device, or the current device is not gfx950 (MI355X)";
    case SVDQ_ERR_LAUNCH: return "kernel launch failed";
    case SVDQ_ERR_TOO_LARGE: return "layer needs more than the 64 MiB static scratch of svdq_linear_noalloc";
  }
  return "unknown status";
}

svdq_status svdq_device_check(void) { return device_check(); }

// Test hook: nonzero makes every device check fail, so the device error path
// can be exercised on a machine that has the right GPU.
void svdq_test_force_device_error(int on) { g_force_device_fail.store(on ? 1 : 0); }

size_t svdq_weight_bytes(const svdq_layer_desc* d) {
  if (!d || check_shape(d) != SVDQ_OK || check_fmt(d) != SVDQ_OK) return 0;
  return weight_layout(d->fmt, d->K, d->N, d->rank).total;
}

size_t svdq_act_bytes(const svdq_layer_desc* d, int64_t M) {
  if (!d || check_shape(d) != SVDQ_OK || check_fmt(d) != SVDQ_OK || M < 0 || M > kMaxRows) return 0;
  return act_layout(d->fmt, d->K, d->rank, M).total;
}

svdq_status svdq_pack_weight(const svdq_layer_desc* d, const float* R, const uint16_t* L1, const uint16_t* L2,
                             const float* lambda, const uint16_t* bias, void* w_packed, void* stream) {
  if (!d || !R || !lambda || !w_packed) return SVDQ_ERR_NULL;
  if (d->rank > 0 && (!L1 || !L2)) return SVDQ_ERR_NULL;
  svdq_status s = check_shape(d);
  if (s != SVDQ_OK) return s;
  if ((s = check_fmt(d)) != SVDQ_OK) return s;
  if (!aligned(R, 16) || !aligned(lambda, 4) || !aligned(w_packed, 256) || (L1 && !aligned(L1, 2)) ||
      (L2 && !aligned(L2, 2)) || (bias && !aligned(bias, 2)))
    return SVDQ_ERR_ALIGN;
  if ((s = device_check()) != SVDQ_OK) return s;
  const WeightLayout wl = weight_layout(d->fmt, d->K, d->N, d->rank);
  uint8_t* blob = static_cast<uint8_t*>(w_packed);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_quantize_weight(d->fmt, R, d->N, d->K, d->K, blob + wl.codes, blob + wl.scales, wl.N_pad,
                                        reinterpret_cast<uint32_t*>(blob + wl.amax), st);
  if (e != hipSuccess) return SVDQ_ERR_LAUNCH;
  return launched(launch_pack_aux(L1, L2, lambda, bias, d->K, d->N, d->rank, wl, blob, st));
}

svdq_status svdq_quantize_act(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X, int64_t M,
                              int64_t ldx, void* a_packed, void* stream) {
  svdq_status s = check_act_args(d, w_packed, X, M, ldx, a_packed);
  if (s != SVDQ_OK) return s;
  if ((s = device_check()) != SVDQ_OK) return s;
  if (M == 0) return SVDQ_OK;
  const WeightLayout wl = weight_layout(d->fmt, d->K, d->N, d->rank);
  const ActLayout al = act_layout(d->fmt, d->K, d->rank, M);
  const uint8_t* blob = static_cast<const uint8_t*>(w_packed);
  uint8_t* ws = static_cast<uint8_t*>(a_packed);
  return launched(launch_quantize_act(d->fmt, X, M, ldx, d->K, reinterpret_cast<const float*>(blob + wl.lam),
                                      reinterpret_cast<const float*>(blob + wl.rlam),
                                      reinterpret_cast<const float*>(blob + wl.rlo), blob + wl.L1, ws + al.codes,
                                      ws + al.scales, al.M_pad, reinterpret_cast<uint16_t*>(ws + al.D),
                                      reinterpret_cast<float*>(ws + al.part), int(al.r_pad), al.kr, al.splits,
                                      reinterpret_cast<const uint32_t*>(blob + wl.flags),
                                      static_cast<hipStream_t>(stream)));
}

svdq_status svdq_gemm(const svdq_layer_desc* d, const void* w_packed, const void* a_packed, int64_t M, void* Y,
                      int64_t ldy, uint32_t epi, void* stream) {
  svdq_status s = check_gemm_args(d, w_packed, a_packed, M, Y, ldy, epi);
  if (s != SVDQ_OK) return s;
  if ((s = device_check()) != SVDQ_OK) return s;
  if (M == 0) return SVDQ_OK;
  const WeightLayout wl = weight_layout(d->fmt, d->K, d->N, d->rank);
  const ActLayout al = act_layout(d->fmt, d->K, d->rank, M);
  return launched(launch_gemm(d->fmt, static_cast<const uint8_t*>(w_packed), wl, static_cast<const uint8_t*>(a_packed),
                              al, d->K, d->N, M, Y, ldy, epi, static_cast<hipStream_t>(stream)));
}

svdq_status svdq_gemm_quant(const svdq_layer_desc* d, const void* w_packed, const void* a_packed, int64_t M,
                            uint32_t epi, const svdq_layer_desc* dn, const void* wn_packed, void* an_packed,
                            void* stream) {
  if (!d || !dn || !w_packed || !a_packed || !wn_packed || !an_packed) return SVDQ_ERR_NULL;
  svdq_status s = check_shape(d);
  if (s != SVDQ_OK || (s = check_shape(dn)) != SVDQ_OK) return s;
  if (M < 0 || M > kMaxRows || dn->K != d->N || dn->rank > kGemmQuantMaxRank) return SVDQ_ERR_SHAPE;
  if ((s = check_fmt(d)) != SVDQ_OK || (s = check_fmt(dn)) != SVDQ_OK) return s;
  if (d->fmt != dn->fmt || (d->fmt != SVDQ_MXFP4 && d->fmt != SVDQ_INT4_G64)) return SVDQ_ERR_FORMAT;
  if ((epi & ~(SVDQ_EPI_LOWRANK | SVDQ_EPI_BIAS | SVDQ_EPI_GELU)) != 0) return SVDQ_ERR_FORMAT;
  if (!aligned(w_packed, 256) || !aligned(a_packed, 256) || !aligned(wn_packed, 256) || !aligned(an_packed, 256))
    return SVDQ_ERR_ALIGN;
  if ((s = device_check()) != SVDQ_OK) return s;
  if (M == 0) return SVDQ_OK;
  const WeightLayout wl = weight_layout(d->fmt, d->K, d->N, d->rank);
  const ActLayout al = act_layout(d->fmt, d->K, d->rank, M);
  const WeightLayout nwl = weight_layout(dn->fmt, dn->K, dn->N, dn->rank);
  const ActLayout nal = act_layout(dn->fmt, dn->K, dn->rank, M);
  return launched(launch_gemm_quant(d->fmt, static_cast<const uint8_t*>(w_packed), wl, static_cast<const uint8_t*>(a_packed),
                                    al, d->K, d->N, M, epi, static_cast<const uint8_t*>(wn_packed), nwl,
                                    static_cast<uint8_t*>(an_packed), nal, static_cast<hipStream_t>(stream)));
}

svdq_status svdq_gemm_qkv(const svdq_layer_desc* d, const void* w_packed, const void* a_packed, int64_t M,
                          uint32_t epi, int32_t head_dim, const uint16_t* norm_q, const uint16_t* norm_k, float eps,
                          const float* rope_cos, const float* rope_sin, void* Y, int64_t ldy, void* stream) {
  if (!d || !w_packed || !a_packed || !norm_q || !norm_k || (M > 0 && (!Y || !rope_cos || !rope_sin)))
    return SVDQ_ERR_NULL;
  svdq_status s = check_shape(d);
  if (s != SVDQ_OK) return s;
  if (M < 0 || M > kMaxRows || ldy < d->N || head_dim != kQkvHeadDim || d->N % (3 * kQkvHeadDim) != 0 ||
      !(eps >= 0.0f && eps <= 1.0f))
    return SVDQ_ERR_SHAPE;
  if ((s = check_fmt(d)) != SVDQ_OK) return s;
  if ((epi & ~(SVDQ_EPI_LOWRANK | SVDQ_EPI_BIAS)) != 0) return SVDQ_ERR_FORMAT;
  if (!aligned(w_packed, 256) || !aligned(a_packed, 256) || !aligned(norm_q, 16) || !aligned(norm_k, 16) ||
      (M > 0 && (!aligned(Y, 16) || !aligned(rope_cos, 16) || !aligned(rope_sin, 16))) || ldy % 8 != 0)
    return SVDQ_ERR_ALIGN;
  if ((s = device_check()) != SVDQ_OK) return s;
  if (M == 0) return SVDQ_OK;
  const WeightLayout wl = weight_layout(d->fmt, d->K, d->N, d->rank);
  const ActLayout al = act_layout(d->fmt, d->K, d->rank, M);
  return launched(launch_gemm_qkv(d->fmt, static_cast<const uint8_t*>(w_packed), wl, static_cast<const uint8_t*>(a_packed),
                                  al, d->K, d->N, M, Y, ldy, epi, norm_q, norm_k, eps, rope_cos, rope_sin,
                                  static_cast<hipStream_t>(stream)));
}

svdq_status svdq_gemm_w4a16(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X, int64_t M,
                            int64_t ldx, void* Y, int64_t ldy, uint32_t epi, void* stream) {
  if (!d || !w_packed || (M > 0 && (!X || !Y))) return SVDQ_ERR_NULL;
  svdq_status s = check_shape(d);
  if (s != SVDQ_OK) return s;
  if (M < 0 || M > kMaxRows || ldx < d->K || ldx > kMaxLdx || ldy < d->N) return SVDQ_ERR_SHAPE;
  if ((s = check_fmt(d)) != SVDQ_OK) return s;
  if (d->fmt != SVDQ_INT4_G64 || d->rank != 0 || (epi & ~(SVDQ_EPI_BIAS | SVDQ_EPI_OUT_F32)) != 0)
    return SVDQ_ERR_FORMAT;
  if (!aligned(w_packed, 256) || (M > 0 && (!aligned(X, 16) || !aligned(Y, 16))) || ldx % 8 != 0 || ldy % 8 != 0)
    return SVDQ_ERR_ALIGN;
  if ((s = device_check()) != SVDQ_OK) return s;
  if (M == 0) return SVDQ_OK;
  const WeightLayout wl = weight_layout(d->fmt, d->K, d->N, d->rank);
  return launched(launch_gemm_w4a16(static_cast<const uint8_t*>(w_packed), wl, d->K, d->N, X, ldx, M, Y, ldy, epi,
                                    static_cast<hipStream_t>(stream)));
}

svdq_status svdq_linear(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X, int64_t M, int64_t ldx,
                        void* Y, int64_t ldy, uint32_t epi, void* workspace, size_t ws_bytes, void* stream) {
  svdq_status s = check_act_args(d, w_packed, X, M, ldx, workspace);
  if (s != SVDQ_OK) return s;
  if ((s = check_gemm_args(d, w_packed, workspace, M, Y, ldy, epi)) != SVDQ_OK) return s;
  if (ws_bytes < act_layout(d->fmt, d->K, d->rank, M).total) return SVDQ_ERR_WORKSPACE;
  if ((s = device_check()) != SVDQ_OK) return s;
  if (M == 0) return SVDQ_OK;
  if ((s = svdq_quantize_act(d, w_packed, X, M, ldx, workspace, stream)) != SVDQ_OK) return s;
  return svdq_gemm(d, w_packed, workspace, M, Y, ldy, epi, stream);
}

svdq_status svdq_linear_noalloc(const svdq_layer_desc* d, const void* w_packed, const uint16_t* X, int64_t M,
                                int64_t ldx, void* Y, int64_t ldy, uint32_t epi, void* stream) {
  // w_packed stands in for the workspace pointer the checks expect (non-NULL, 256-aligned)
  svdq_status s = check_act_args(d, w_packed, X, M, ldx, w_packed);
  if (s != SVDQ_OK) return s;
  if ((s = check_gemm_args(d, w_packed, w_packed, M, Y, ldy, epi)) != SVDQ_OK) return s;
  const ActLayout al = act_layout(d->fmt, d->K, d->rank, M);
  if (act_linear_bytes(al) > kScratchBytes) return SVDQ_ERR_TOO_LARGE;
  if ((s = device_check()) != SVDQ_OK) return s;
  if (M == 0) return SVDQ_OK;
  uint8_t* ws = nullptr;
  if ((s = scratch_address(&ws)) != SVDQ_OK) return s;
  const WeightLayout wl = weight_layout(d->fmt, d->K, d->N, d->rank);
  const uint8_t* blob = static_cast<const uint8_t*>(w_packed);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_quantize_act(d->fmt, X, M, ldx, d->K, reinterpret_cast<const float*>(blob + wl.lam),
                                     reinterpret_cast<const float*>(blob + wl.rlam),
                                     reinterpret_cast<const float*>(blob + wl.rlo), blob + wl.L1, ws + al.codes,
                                     ws + al.scales, al.M_pad, reinterpret_cast<uint16_t*>(ws + al.D),
                                     reinterpret_cast<float*>(ws + al.part), int(al.r_pad), al.kr, al.splits,
                                     reinterpret_cast<const uint32_t*>(blob + wl.flags), st);
  if (e != hipSuccess) return SVDQ_ERR_LAUNCH;
  return launched(launch_gemm(d->fmt, blob, wl, ws, al, d->K, d->N, M, Y, ldy, epi, st));
}

svdq_status svdq_unpack_weight(const svdq_layer_desc* d, const void* w_packed, uint8_t* codes, void* scales,
                               uint16_t* L1, uint16_t* L2, float* lambda, uint16_t* bias, void* stream) {
  if (!d || !w_packed) return SVDQ_ERR_NULL;
  svdq_status s = check_shape(d);
  if (s != SVDQ_OK) return s;
  if ((s = check_fmt(d)) != SVDQ_OK) return s;
  if (!aligned(w_packed, 256)) return SVDQ_ERR_ALIGN;
  if ((s = device_check()) != SVDQ_OK) return s;
  const WeightLayout wl = weight_layout(d->fmt, d->K, d->N, d->rank);
  return launched(launch_unpack_weight(d->fmt, d->K, d->N, d->rank, wl, static_cast<const uint8_t*>(w_packed), codes,
                                       scales, L1, L2, lambda, bias, static_cast<hipStream_t>(stream)));
}

svdq_status svdq_unpack_act(const svdq_layer_desc* d, const void* a_packed, int64_t M, uint8_t* codes, void* scales,
                            float* D, void* stream) {
  if (!d || !a_packed) return SVDQ_ERR_NULL;
  svdq_status s = check_shape(d);
  if (s != SVDQ_OK) return s;
  if (M < 0 || M > kMaxRows) return SVDQ_ERR_SHAPE;
  if ((s = check_fmt(d)) != SVDQ_OK) return s;
  if (!aligned(a_packed, 256)) return SVDQ_ERR_ALIGN;
  if ((s = device_check()) != SVDQ_OK) return s;
  const ActLayout al = act_layout(d->fmt, d->K, d->rank, M);
  return launched(launch_unpack_act(d->fmt, d->K, d->rank, M, al, static_cast<const uint8_t*>(a_packed), codes, scales,
                                    D, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
