// C ABI of the attention library: argument checks, launches, status codes,
// and the two debug exports (the device mask predicate and the tile plan).
//
// Argument errors are reported as status codes before anything is enqueued,
// in the spirit of vllm_mlx.attention's validate_configuration returning its
// errors rather than raising; the calls write their outputs in place and
// return no tensor (Tylo.jl "Primitives", attention! "Returns nothing").
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/attn.h"
#include "attn_common.h"
#include "attn_host.h"

namespace attn {

template <int D>
hipError_t launch_fwd_bf16(void*, const void*, const void*, const void*,
                           float*, int, int, int, int, int, int, int, int,
                           const int32_t*, hipStream_t);
template <int D>
hipError_t launch_fwd_flex(void*, const void*, const void*, const void*,
                           float*, int, int, int, int, int, int, int, int,
                           const int32_t*, const attn_flex_t*, hipStream_t);
hipError_t launch_build_block_mask(uint8_t*, int, int, int, int, int, int,
                                   const int32_t*, const attn_flex_t*, hipStream_t);
template <int D>
hipError_t launch_fwd_f32(void*, const void*, const void*, const void*,
                          float*, int, int, int, int, int, int, int, int,
                          const int32_t*, hipStream_t);
hipError_t launch_decode(void*, const void*, const void*, const void*,
                         const int32_t*, int, int, int, int, int, int, void*,
                         hipStream_t);
size_t decode_workspace_bytes(int B, int H, int n_splits, int D);
template <int D>
hipError_t launch_fwd_sparse(void*, const void*, const void*, const void*,
                             float*, int, int, int, int, int, int, int, int,
                             const int32_t*, const uint8_t*, hipStream_t);
size_t block_scores_workspace_bytes(int B, int Hkv, int Sk, int D);
hipError_t launch_block_scores(float*, float*, const void*, const void*, int,
                               int, int, int, int, int, int, float, float,
                               void*, hipStream_t);
hipError_t launch_block_mask(uint8_t*, const float*, long long, int, int, int,
                             float, int, int, int, hipStream_t);
hipError_t launch_bwd(void*, void*, void*, const void*, const void*,
                      const void*, const void*, const void*, const float*, int,
                      int, int, int, int, int, int, int, int, const int32_t*,
                      void*, hipStream_t);
size_t bwd_workspace_bytes(int B, int H, int Sq);
hipError_t launch_decode_paged(void*, const void*, const void*, const void*,
                               const int32_t*, const int32_t*, int, int, int,
                               int, int, int, int, int, void*, hipStream_t);

__global__ void mask_dump_kernel(uint8_t* __restrict__ M, int Sq, int Sk,
                                 int causal, int window, int input_pos,
                                 int kl) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)Sq * Sk) return;
  const int i = (int)(idx / Sk), j = (int)(idx % Sk);
  const RowRange r = row_range(i, kl, causal, window, input_pos);
  M[idx] = (j >= r.lo && j < r.hi) ? 1 : 0;
}

__global__ void tile_plan_kernel(int8_t* __restrict__ P, int Sq, int Sk,
                                 int causal, int window, int input_pos,
                                 int kl, int nqt, int nkt, int tp) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)nqt * nkt) return;
  const int qt = (int)(idx / nkt), kt = (int)(idx % nkt);
  const int i0 = qt * tp;
  const int i1 = min(i0 + tp, Sq);
  const KvGeometry g = kv_geometry(i0, i1, kl, causal, window, input_pos);
  P[idx] = (int8_t)tile_class(g, kt * ATTN_FWD_TILE_N, ATTN_FWD_TILE_N);
}

static int hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  (void)hipGetLastError();  // clear the sticky launch error
  return ATTN_EHIP;
}

constexpr int kMaxDevices = 64;
static std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not looked up yet

int device_cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    // every thread that races here stores the same value
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        n < 1) {
      (void)hipGetLastError();
      n = -1;
    }
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n > 0 ? n : 0;
}

bool log_enabled() {
  static const bool on = [] {
    const char* v = getenv("ATTN_LOG");
    return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
  }();
  return on;
}

void log_line(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[attn] %s\n", buf);
}

// One log line per entry-point call: its sizes and the status it returns.
static int logged(int rc, const char* name, int B, int H, int Hkv, int Sq, int Sk,
                  int D, const char* extra_fmt = "", ...) {
  if (!log_enabled()) return rc;
  char extra[256] = "";
  va_list ap;
  va_start(ap, extra_fmt);
  vsnprintf(extra, sizeof extra, extra_fmt, ap);
  va_end(ap);
  log_line("%s B=%d H=%d Hkv=%d Sq=%d Sk=%d D=%d%s%s -> %s", name, B, H, Hkv, Sq, Sk, D,
           extra[0] ? " " : "", extra,
           rc == ATTN_OK ? "ok" : rc == ATTN_EINVAL ? "invalid argument"
           : rc == ATTN_EUNSUPPORTED ? "unsupported" : "HIP error");
  return rc;
}

// Checks shared by the prefill entry points.  Sizes must keep every key and
// row index (plus one tile of overshoot) inside int32.
static int check_fwd(const void* O, const void* Q, const void* K,
                     const void* V, int B, int H, int Hkv, int Sq, int Sk,
                     int D, int causal, int window) {
  if (B < 1 || H < 1 || Hkv < 1 || Sq < 0 || Sk < 0) return ATTN_EINVAL;
  if (H % Hkv != 0) return ATTN_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_EINVAL;
  if (window > 0 && !causal) return ATTN_EINVAL;
  if (D != 64 && D != 128) return ATTN_EUNSUPPORTED;
  if (Sq > INT_MAX - 256 || Sk > INT_MAX - 256) return ATTN_EUNSUPPORTED;
  // K/V rows of one KV head are addressed through 32-bit buffer offsets
  if ((long long)Sk * D * 4 + 65536 > INT_MAX) return ATTN_EUNSUPPORTED;
  const long long nqt = ((long long)Sq + 127) / 64;  // finest row tiling used
  if (nqt * H * B > INT_MAX) return ATTN_EUNSUPPORTED;
  if ((long long)B * H > INT_MAX / 2 || (long long)B * Hkv > INT_MAX / 2)
    return ATTN_EUNSUPPORTED;
  if (Sq > 0 && (!O || !Q)) return ATTN_EINVAL;
  if (Sq > 0 && Sk > 0 && (!K || !V)) return ATTN_EINVAL;
  return ATTN_OK;
}

static int check_decode(const void* O, const void* Q, const void* K,
                        const void* V, const int32_t* lengths, int n_splits,
                        int B, int H, int Hkv, int Smax, int D) {
  if (B < 1 || H < 1 || Hkv < 1 || Smax < 1 || n_splits < 1)
    return ATTN_EINVAL;
  if (H % Hkv != 0) return ATTN_EINVAL;
  if (D != 64 && D != 128) return ATTN_EUNSUPPORTED;
  if (Smax > INT_MAX - 256) return ATTN_EUNSUPPORTED;
  // K/V rows of one KV head are addressed through 32-bit buffer offsets
  if ((long long)Smax * D * 2 + 65536 > INT_MAX) return ATTN_EUNSUPPORTED;
  if ((long long)B * H * n_splits > INT_MAX / 2) return ATTN_EUNSUPPORTED;
  if ((long long)B * Hkv * H * n_splits > INT_MAX) return ATTN_EUNSUPPORTED;
  if (!O || !Q || !K || !V || !lengths) return ATTN_EINVAL;
  return ATTN_OK;
}

// Checks of the paged decode; on success *bs_log2 = log2(block_size).
static int check_decode_paged(const void* O, const void* Q, const void* Kc,
                              const void* Vc, const int32_t* tables,
                              const int32_t* lengths, int n_splits, int B,
                              int H, int Hkv, int num_blocks, int block_size,
                              int max_blocks, int D, int* bs_log2) {
  if (B < 1 || H < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1 ||
      n_splits < 1 || block_size < 1)
    return ATTN_EINVAL;
  if (block_size & (block_size - 1)) return ATTN_EINVAL;  // power of two
  if (H % Hkv != 0) return ATTN_EINVAL;
  if (D != 64 && D != 128) return ATTN_EUNSUPPORTED;
  if (block_size > 1024) return ATTN_EUNSUPPORTED;
  if ((long long)max_blocks * block_size > INT_MAX - 256) return ATTN_EUNSUPPORTED;
  if ((long long)B * H * n_splits > INT_MAX / 2) return ATTN_EUNSUPPORTED;
  if ((long long)B * Hkv * H * n_splits > INT_MAX) return ATTN_EUNSUPPORTED;
  if (!O || !Q || !Kc || !Vc || !tables || !lengths) return ATTN_EINVAL;
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  *bs_log2 = lg;
  return ATTN_OK;
}

// ---- scratch of attn_decode_static ----
// The decode's slice partials (O_s and LSE_s of every (sequence, head,
// slice)) live in this file-scope device array instead of an allocation, for
// callers that cannot allocate.  Each GPU holds its own copy from the time
// the library's code is loaded on it until the process ends.  In host code
// `scratch` is only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) char scratch[ATTN_DECODE_STATIC_SCRATCH_BYTES];

static std::atomic<void*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (set up on the first
// call on each device, under a lock).
static int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return ATTN_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_EUNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return ATTN_EHIP;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ATTN_OK;
}

}  // namespace attn

using namespace attn;

extern "C" {

int attn_fwd(void* O, const void* Q, const void* K, const void* V, float* LSE,
             int B, int H, int Hkv, int Sq, int Sk, int D, int causal,
             int window, int input_pos, const int32_t* k_lengths,
             hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int rc = check_fwd(O, Q, K, V, B, H, Hkv, Sq, Sk, D, causal, window);
    if (rc != ATTN_OK || Sq == 0) return rc;
    hipError_t e =
        D == 64 ? launch_fwd_bf16<64>(O, Q, K, V, LSE, B, H, Hkv, Sq, Sk, causal,
                                      window, input_pos, k_lengths, stream)
                : launch_fwd_bf16<128>(O, Q, K, V, LSE, B, H, Hkv, Sq, Sk,
                                       causal, window, input_pos, k_lengths,
                                       stream);
    return hip_status(e);
  }();
  return logged(rc_, "attn_fwd", B, H, Hkv, Sq, Sk, D,
                "causal=%d window=%d input_pos=%d k_lengths=%s lse=%s",
                causal, window, input_pos, k_lengths ? "yes" : "no", LSE ? "yes" : "no");
}

int attn_fwd_flex(void* O, const void* Q, const void* K, const void* V,
                  float* LSE, int B, int H, int Hkv, int Sq, int Sk, int D,
                  int causal, int window, int input_pos,
                  const int32_t* k_lengths, const attn_flex_t* flex,
                  hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int rc = check_fwd(O, Q, K, V, B, H, Hkv, Sq, Sk, D, causal, window);
    if (rc != ATTN_OK) return rc;
    attn_flex_t none = {};
    const attn_flex_t* f = flex ? flex : &none;
    if (f->softcap < 0.f || f->qk_scale < 0.f || f->prefix < 0) return ATTN_EINVAL;
    if ((f->doc_q == nullptr) != (f->doc_kv == nullptr)) return ATTN_EINVAL;
    if (f->bias) {
      if ((f->bias_B != 1 && f->bias_B != B) || (f->bias_H != 1 && f->bias_H != H))
        return ATTN_EINVAL;
      if (((long long)Sq * Sk + Sk) * 4 + 256 > INT_MAX) return ATTN_EUNSUPPORTED;
    }
    if (f->block_mask) {
      if (f->block_mask_B != 1 && f->block_mask_B != B) return ATTN_EINVAL;
      if (((long long)Sk + ATTN_BLOCK - 1) / ATTN_BLOCK > ATTN_SPARSE_MAX_KEY_BLOCKS)
        return ATTN_EUNSUPPORTED;
    }
    if (Sq == 0) return ATTN_OK;
    hipError_t e =
        D == 64 ? launch_fwd_flex<64>(O, Q, K, V, LSE, B, H, Hkv, Sq, Sk, causal,
                                      window, input_pos, k_lengths, f, stream)
                : launch_fwd_flex<128>(O, Q, K, V, LSE, B, H, Hkv, Sq, Sk, causal,
                                       window, input_pos, k_lengths, f, stream);
    return hip_status(e);
  }();
  return logged(rc_, "attn_fwd_flex", B, H, Hkv, Sq, Sk, D,
                "causal=%d window=%d input_pos=%d block_mask=%s",
                causal, window, input_pos, flex && flex->block_mask ? "yes" : "no");
}

int attn_build_block_mask(uint8_t* block_mask, int B, int Sq, int Sk, int causal,
                          int window, int input_pos, const int32_t* k_lengths,
                          const attn_flex_t* flex, hipStream_t stream) {
  const int rc_ = [&]() -> int {
    if (B < 1 || Sq < 0 || Sk < 0) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (window < 0 || (window > 0 && !causal)) return ATTN_EINVAL;
    attn_flex_t none = {};
    const attn_flex_t* f = flex ? flex : &none;
    if (f->prefix < 0) return ATTN_EINVAL;
    if ((f->doc_q == nullptr) != (f->doc_kv == nullptr)) return ATTN_EINVAL;
    if (((long long)Sk + ATTN_BLOCK - 1) / ATTN_BLOCK > ATTN_SPARSE_MAX_KEY_BLOCKS)
      return ATTN_EUNSUPPORTED;
    if ((long long)B * ((Sq + ATTN_BLOCK - 1) / ATTN_BLOCK) *
            ((Sk + ATTN_BLOCK - 1) / ATTN_BLOCK) > INT_MAX)
      return ATTN_EUNSUPPORTED;
    if (Sq == 0 || Sk == 0) return ATTN_OK;
    if (!block_mask) return ATTN_EINVAL;
    return hip_status(launch_build_block_mask(block_mask, B, Sq, Sk, causal, window,
                                              input_pos, k_lengths, f, stream));
  }();
  return logged(rc_, "attn_build_block_mask", B, 0, 0, Sq, Sk, 0,
                "causal=%d window=%d input_pos=%d", causal, window, input_pos);
}

int attn_fwd_f32(void* O, const void* Q, const void* K, const void* V,
                 float* LSE, int B, int H, int Hkv, int Sq, int Sk, int D,
                 int causal, int window, int input_pos,
                 const int32_t* k_lengths, hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int rc = check_fwd(O, Q, K, V, B, H, Hkv, Sq, Sk, D, causal, window);
    if (rc != ATTN_OK || Sq == 0) return rc;
    hipError_t e =
        D == 64 ? launch_fwd_f32<64>(O, Q, K, V, LSE, B, H, Hkv, Sq, Sk, causal,
                                     window, input_pos, k_lengths, stream)
                : launch_fwd_f32<128>(O, Q, K, V, LSE, B, H, Hkv, Sq, Sk, causal,
                                      window, input_pos, k_lengths, stream);
    return hip_status(e);
  }();
  return logged(rc_, "attn_fwd_f32", B, H, Hkv, Sq, Sk, D,
                "causal=%d window=%d input_pos=%d",
                causal, window, input_pos);
}

size_t attn_decode_workspace_bytes(int B, int H, int n_splits, int D) {
  if (B < 1 || H < 1 || n_splits < 1 || (D != 64 && D != 128)) return 0;
  return decode_workspace_bytes(B, H, n_splits, D);
}

int attn_decode_ws(void* O, const void* Q, const void* K, const void* V,
                   const int32_t* lengths, int n_splits, int B, int H, int Hkv,
                   int Smax, int D, void* workspace, size_t ws_bytes,
                   hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int rc = check_decode(O, Q, K, V, lengths, n_splits, B, H, Hkv, Smax, D);
    if (rc != ATTN_OK) return rc;
    if (n_splits > 1) {
      if (!workspace || ((uintptr_t)workspace & 255) != 0) return ATTN_EINVAL;
      if (ws_bytes < decode_workspace_bytes(B, H, n_splits, D))
        return ATTN_EINVAL;
    }
    return hip_status(launch_decode(O, Q, K, V, lengths, n_splits, B, H, Hkv,
                                    Smax, D, workspace, stream));
  }();
  return logged(rc_, "attn_decode_ws", B, H, Hkv, 1, Smax, D,
                "n_splits=%d ws_bytes=%zu",
                n_splits, ws_bytes);
}

int attn_decode(void* O, const void* Q, const void* K, const void* V,
                const int32_t* lengths, int n_splits, int B, int H, int Hkv,
                int Smax, int D, hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int rc = check_decode(O, Q, K, V, lengths, n_splits, B, H, Hkv, Smax, D);
    if (rc != ATTN_OK) return rc;
    void* ws = nullptr;
    if (n_splits > 1) {
      const size_t bytes = decode_workspace_bytes(B, H, n_splits, D);
      if (hipMallocAsync(&ws, bytes, stream) != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_EHIP;
      }
    }
    rc = hip_status(launch_decode(O, Q, K, V, lengths, n_splits, B, H, Hkv, Smax,
                                  D, ws, stream));
    if (ws && hipFreeAsync(ws, stream) != hipSuccess) {
      (void)hipGetLastError();
      rc = ATTN_EHIP;
    }
    return rc;
  }();
  return logged(rc_, "attn_decode", B, H, Hkv, 1, Smax, D,
                "n_splits=%d",
                n_splits);
}

int attn_decode_static(void* O, const void* Q, const void* K, const void* V,
                       const int32_t* lengths, int n_splits, int B, int H,
                       int Hkv, int Smax, int D, hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int rc = check_decode(O, Q, K, V, lengths, n_splits, B, H, Hkv, Smax, D);
    if (rc != ATTN_OK) return rc;
    void* ws = nullptr;
    if (n_splits > 1) {
      // every slice writes its partial row (zeros and LSE = -inf when empty),
      // so nothing in the scratch has to start at zero
      if (decode_workspace_bytes(B, H, n_splits, D) > ATTN_DECODE_STATIC_SCRATCH_BYTES)
        return ATTN_EUNSUPPORTED;
      rc = static_scratch(&ws);
      if (rc != ATTN_OK) return rc;
    }
    return hip_status(launch_decode(O, Q, K, V, lengths, n_splits, B, H, Hkv,
                                    Smax, D, ws, stream));
  }();
  return logged(rc_, "attn_decode_static", B, H, Hkv, 1, Smax, D,
                "n_splits=%d",
                n_splits);
}

int attn_fwd_block_sparse(void* O, const void* Q, const void* K, const void* V,
                          float* LSE, int B, int H, int Hkv, int Sq, int Sk,
                          int D, int causal, int window, int input_pos,
                          const int32_t* k_lengths, const uint8_t* keep,
                          hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int rc = check_fwd(O, Q, K, V, B, H, Hkv, Sq, Sk, D, causal, window);
    if (rc != ATTN_OK || Sq == 0) return rc;
    if (!keep) return ATTN_EINVAL;
    if ((Sk + ATTN_BLOCK - 1) / ATTN_BLOCK > ATTN_SPARSE_MAX_KEY_BLOCKS)
      return ATTN_EUNSUPPORTED;
    hipError_t e =
        D == 64 ? launch_fwd_sparse<64>(O, Q, K, V, LSE, B, H, Hkv, Sq, Sk, causal,
                                        window, input_pos, k_lengths, keep, stream)
                : launch_fwd_sparse<128>(O, Q, K, V, LSE, B, H, Hkv, Sq, Sk,
                                         causal, window, input_pos, k_lengths,
                                         keep, stream);
    return hip_status(e);
  }();
  return logged(rc_, "attn_fwd_block_sparse", B, H, Hkv, Sq, Sk, D,
                "causal=%d window=%d input_pos=%d",
                causal, window, input_pos);
}

size_t attn_block_scores_workspace_bytes(int B, int Hkv, int Sk, int D) {
  if (B < 1 || Hkv < 1 || Sk < 1 || (D != 64 && D != 128)) return 0;
  return block_scores_workspace_bytes(B, Hkv, Sk, D);
}

int attn_block_scores(float* base, float* rescue, const void* Q, const void* K,
                      int B, int H, int Hkv, int Sq, int Sk, int D, int kind,
                      float low, float high, void* workspace, size_t ws_bytes,
                      hipStream_t stream) {
  const int rc_ = [&]() -> int {
    if (B < 1 || H < 1 || Hkv < 1 || Sq < 1 || Sk < 1) return ATTN_EINVAL;
    if (H % Hkv != 0) return ATTN_EINVAL;
    if (kind != ATTN_BLOCK_SCORES_RBS && kind != ATTN_BLOCK_SCORES_MINMAX)
      return ATTN_EINVAL;
    if (!(low >= 0.f && low <= 1.f && high >= 0.f && high <= 1.f)) return ATTN_EINVAL;
    if (D != 64 && D != 128) return ATTN_EUNSUPPORTED;
    if (Sq > INT_MAX - 256 || Sk > INT_MAX - 256) return ATTN_EUNSUPPORTED;
    if ((Sk + ATTN_BLOCK - 1) / ATTN_BLOCK > 4096) return ATTN_EUNSUPPORTED;
    if (!base || !Q || !K) return ATTN_EINVAL;
    void* ws = workspace;
    bool owned = false;
    const size_t need = block_scores_workspace_bytes(B, Hkv, Sk, D);
    if (ws) {
      if (((uintptr_t)ws & 255) != 0 || ws_bytes < need) return ATTN_EINVAL;
    } else {
      if (hipMallocAsync(&ws, need, stream) != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_EHIP;
      }
      owned = true;
    }
    int rc = hip_status(launch_block_scores(base, rescue, Q, K, B, H, Hkv, Sq, Sk,
                                            D, kind, low, high, ws, stream));
    if (owned && hipFreeAsync(ws, stream) != hipSuccess) {
      (void)hipGetLastError();
      rc = ATTN_EHIP;
    }
    return rc;
  }();
  return logged(rc_, "attn_block_scores", B, H, Hkv, Sq, Sk, D,
                "kind=%d",
                kind);
}

int attn_block_mask(uint8_t* keep, const float* scores, int rows, int nqb,
                    int nkb, int mode, float alpha, int k, int diagonal,
                    int accumulate, hipStream_t stream) {
  const int rc_ = [&]() -> int {
    if (rows < 0 || nqb < 1 || nkb < 1 || !keep) return ATTN_EINVAL;
    if (mode < ATTN_BLOCK_MASK_RELATIVE || mode > ATTN_BLOCK_MASK_BAND) return ATTN_EINVAL;
    if (mode != ATTN_BLOCK_MASK_BAND && !scores) return ATTN_EINVAL;
    if (mode == ATTN_BLOCK_MASK_RELATIVE && !(alpha > 0.f && alpha <= 1.f)) return ATTN_EINVAL;
    if (mode == ATTN_BLOCK_MASK_TOPK && k < 0) return ATTN_EINVAL;
    if (rows == 0) return ATTN_OK;
    const float ln_alpha = mode == ATTN_BLOCK_MASK_RELATIVE ? (float)log((double)alpha) : 0.f;
    return hip_status(launch_block_mask(keep, scores, rows, nqb, nkb, mode, ln_alpha,
                                        k, diagonal, accumulate != 0, stream));
  }();
  return logged(rc_, "attn_block_mask", 0, 0, 0, nqb, nkb, 0,
                "rows=%d mode=%d",
                rows, mode);
}

size_t attn_bwd_workspace_bytes(int B, int H, int Sq, int D) {
  if (B < 1 || H < 1 || Sq < 1 || (D != 64 && D != 128)) return 0;
  return bwd_workspace_bytes(B, H, Sq);
}

int attn_bwd(void* dQ, void* dK, void* dV, const void* dO, const void* Q,
             const void* K, const void* V, const void* O, const float* LSE,
             int B, int H, int Hkv, int Sq, int Sk, int D, int causal,
             int window, int input_pos, const int32_t* k_lengths,
             void* workspace, size_t ws_bytes, hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int rc = check_fwd(O, Q, K, V, B, H, Hkv, Sq, Sk, D, causal, window);
    if (rc != ATTN_OK) return rc;
    if (Sq == 0 && Sk == 0) return ATTN_OK;
    if (Sk > 0 && (!dK || !dV || !K || !V)) return ATTN_EINVAL;
    if (Sq > 0 && (!dQ || !dO || !LSE)) return ATTN_EINVAL;
    if ((long long)B * H * Sq > INT_MAX / 2) return ATTN_EUNSUPPORTED;
    // the Q and dO rows of one head are addressed through 32-bit buffer offsets
    if ((long long)Sq * D * 4 + 65536 > INT_MAX) return ATTN_EUNSUPPORTED;
    if (Sq == 0)  // no query: the key gradients are zero, no scratch needed
      return hip_status(launch_bwd(dQ, dK, dV, dO, Q, K, V, O, LSE, B, H, Hkv,
                                   Sq, Sk, D, causal, window, input_pos,
                                   k_lengths, nullptr, stream));
    void* ws = workspace;
    bool owned = false;
    const size_t need = bwd_workspace_bytes(B, H, Sq);
    if (ws) {
      if (((uintptr_t)ws & 255) != 0 || ws_bytes < need) return ATTN_EINVAL;
    } else {
      if (hipMallocAsync(&ws, need, stream) != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_EHIP;
      }
      owned = true;
    }
    rc = hip_status(launch_bwd(dQ, dK, dV, dO, Q, K, V, O, LSE, B, H, Hkv, Sq, Sk,
                               D, causal, window, input_pos, k_lengths, ws,
                               stream));
    if (owned && hipFreeAsync(ws, stream) != hipSuccess) {
      (void)hipGetLastError();
      rc = ATTN_EHIP;
    }
    return rc;
  }();
  return logged(rc_, "attn_bwd", B, H, Hkv, Sq, Sk, D,
                "causal=%d window=%d input_pos=%d",
                causal, window, input_pos);
}

int attn_decode_paged(void* O, const void* Q, const void* K_cache,
                      const void* V_cache, const int32_t* block_tables,
                      const int32_t* lengths, int n_splits, int B, int H,
                      int Hkv, int num_blocks, int block_size, int max_blocks,
                      int D, void* workspace, size_t ws_bytes,
                      hipStream_t stream) {
  const int rc_ = [&]() -> int {
    int bs_log2 = 0;
    int rc = check_decode_paged(O, Q, K_cache, V_cache, block_tables, lengths,
                                n_splits, B, H, Hkv, num_blocks, block_size,
                                max_blocks, D, &bs_log2);
    if (rc != ATTN_OK) return rc;
    void* ws = workspace;
    bool owned = false;
    if (n_splits > 1) {
      const size_t need = decode_workspace_bytes(B, H, n_splits, D);
      if (ws) {
        if (((uintptr_t)ws & 255) != 0 || ws_bytes < need) return ATTN_EINVAL;
      } else {
        if (hipMallocAsync(&ws, need, stream) != hipSuccess) {
          (void)hipGetLastError();
          return ATTN_EHIP;
        }
        owned = true;
      }
    }
    rc = hip_status(launch_decode_paged(O, Q, K_cache, V_cache, block_tables,
                                        lengths, n_splits, B, H, Hkv, num_blocks,
                                        bs_log2, max_blocks, D, ws, stream));
    if (owned && hipFreeAsync(ws, stream) != hipSuccess) {
      (void)hipGetLastError();
      rc = ATTN_EHIP;
    }
    return rc;
  }();
  return logged(rc_, "attn_decode_paged", B, H, Hkv, 1, max_blocks * block_size, D,
                "n_splits=%d block_size=%d num_blocks=%d",
                n_splits, block_size, num_blocks);
}

int attn_mask_dump(uint8_t* M, int Sq, int Sk, int causal, int window,
                   int input_pos, int k_len, hipStream_t stream) {
  if (Sq < 0 || Sk < 0 || (causal != 0 && causal != 1)) return ATTN_EINVAL;
  if (window > 0 && !causal) return ATTN_EINVAL;
  if ((long long)Sq * Sk > (long long)INT_MAX * 256) return ATTN_EUNSUPPORTED;
  if ((long long)Sq * Sk == 0) return ATTN_OK;
  if (!M) return ATTN_EINVAL;
  const int kl = k_len < 0 ? 0 : (k_len > Sk ? Sk : k_len);
  const long long n = (long long)Sq * Sk;
  hipLaunchKernelGGL(mask_dump_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream, M, Sq, Sk, causal, window,
                     input_pos, kl);
  return hip_status(hipGetLastError());
}

int attn_tile_plan(int8_t* P, int Sq, int Sk, int causal, int window,
                   int input_pos, int k_len, int group, hipStream_t stream) {
  if (Sq < 0 || Sk < 0 || (causal != 0 && causal != 1) || group < 1) return ATTN_EINVAL;
  if (window > 0 && !causal) return ATTN_EINVAL;
  if (Sq > INT_MAX - 256 || Sk > INT_MAX - 256) return ATTN_EUNSUPPORTED;
  const int tp = ATTN_FWD_TILE_M >> fwd_heads_log2(group);
  const int nqt = (Sq + tp - 1) / tp;
  const int nkt = (Sk + ATTN_FWD_TILE_N - 1) / ATTN_FWD_TILE_N;
  const long long n = (long long)nqt * nkt;
  if (n == 0) return ATTN_OK;
  if (!P) return ATTN_EINVAL;
  const int kl = k_len < 0 ? 0 : (k_len > Sk ? Sk : k_len);
  hipLaunchKernelGGL(tile_plan_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream, P, Sq, Sk, causal, window,
                     input_pos, kl, nqt, nkt, tp);
  return hip_status(hipGetLastError());
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported size or head dimension";
    case ATTN_EHIP: return "HIP launch or allocation error";
    default: return "unknown status";
  }
}

int attn_version(void) { return 10000; }

}  // extern "C"
