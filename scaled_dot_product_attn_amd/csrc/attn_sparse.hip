// Block-score estimators and block masks for block-sparse prefill on gfx950.
//
// mlx-arsenal "Radius-bounded block scores (RBS)": block-sparse attention
// scores each (query block, key block) pair from a summary of the key block.
//   base    per query token q.c_b / sqrt(D)   (c_b the block's centroid)
//   rescue  (q.c_b + ||q|| r_b beta_b) / sqrt(D), r_b = max ||k - c_b||,
//           beta_b = clip((r_b - r_low) / (r_high - r_low), 0, 1) from the
//           median / 90th percentile of the head's block radii (beta_b = [r_b >
//           r_low] when the two coincide)
//   min/max sum_d max(q_d lo_bd, q_d hi_bd) / sqrt(D), the element-wise box
//           bound (lo / hi the block's per-dimension min / max)
// and a block score is the log of the sum of exp over the query block's tokens.
// Block masks: keep the blocks within alpha of the row maximum (relative),
// the k best of a row (top-k, ties to the lower index), or a diagonal band.
//
// These are small, HBM/latency-bound kernels (float32 vector ALU, no matrix
// cores): one pass over K for the block statistics, one over Q for the scores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

namespace sparse {

constexpr int kBlock = 64;       // tokens per query / key block
constexpr int kMaxBlocks = 4096; // key blocks per head the quantile sort holds

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace sparse

using namespace sparse;

// Per (key block, KV head, batch): centroid, per-dimension min / max, radius.
// stats layout per (b, g): c (nk, D), lo (nk, D), hi (nk, D), r (nk).
template <int D>
__global__ __launch_bounds__(256) void attn_block_stats_kernel(
    const __bf16* __restrict__ K, float* __restrict__ stats, int Hkv, int Sk,
    int nk) {
  __shared__ float s_part[3][256 / D][D];
  __shared__ float s_c[D];
  __shared__ float s_r[256 / 64];
  const int kb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int d = tid % D, part = tid / D;       // 256 / D threads per dimension
  constexpr int PARTS = 256 / D;
  const int j0 = kb * kBlock;
  const int n = min(kBlock, Sk - j0);
  const __bf16* kp = K + ((size_t)(b * Hkv + g) * Sk + j0) * D;
  float sum = 0.f, lo = INFINITY, hi = -INFINITY;
  for (int j = part; j < n; j += PARTS) {
    const float x = (float)kp[(size_t)j * D + d];
    sum += x;
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  }
  s_part[0][part][d] = sum;
  s_part[1][part][d] = lo;
  s_part[2][part][d] = hi;
  __syncthreads();
  float* base = stats + (size_t)(b * Hkv + g) * nk * (3 * D + 1);
  if (tid < D) {
    float su = 0.f, l = INFINITY, h = -INFINITY;
#pragma unroll
    for (int p = 0; p < PARTS; ++p) {
      su += s_part[0][p][tid];
      l = fminf(l, s_part[1][p][tid]);
      h = fmaxf(h, s_part[2][p][tid]);
    }
    const float c = su / (float)n;
    s_c[tid] = c;
    base[(size_t)kb * D + tid] = c;
    base[(size_t)nk * D + (size_t)kb * D + tid] = l;
    base[(size_t)2 * nk * D + (size_t)kb * D + tid] = h;
  }
  __syncthreads();
  // radius: one thread per key, squared distance to the centroid
  float dist = 0.f;
  if (tid < n) {
    const __bf16* row = kp + (size_t)tid * D;
    for (int e = 0; e < D; ++e) {
      const float t = (float)row[e] - s_c[e];
      dist = __builtin_fmaf(t, t, dist);
    }
  }
  const float m = wave_max(tid < n ? dist : 0.f);
  if ((tid & 63) == 0) s_r[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    float r = fmaxf(fmaxf(s_r[0], s_r[1]), fmaxf(s_r[2], s_r[3]));
    base[(size_t)3 * nk * D + kb] = sqrtf(r);
  }
}

// Per (KV head, batch): the `low` / `high` quantiles of the nk block radii
// (linear interpolation between order statistics), by a bitonic sort in LDS.
__global__ __launch_bounds__(256) void attn_block_quantile_kernel(
    float* __restrict__ stats, float* __restrict__ qout, int Hkv, int nk, int D,
    float low, float high) {
  __shared__ float s[kMaxBlocks];
  const int g = blockIdx.x, b = blockIdx.y;
  const float* r = stats + (size_t)(b * Hkv + g) * nk * (3 * D + 1) + (size_t)3 * nk * D;
  int n2 = 1;
  while (n2 < nk) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += 256) s[i] = i < nk ? r[i] : INFINITY;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n2; i += 256) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const float a = s[i], c = s[j];
          if ((a > c) == up) {
            s[i] = c;
            s[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x < 2) {
    const float q = threadIdx.x == 0 ? low : high;
    const float pos = q * (float)(nk - 1);
    const int i = min((int)floorf(pos), nk - 1);
    const int j = min(i + 1, nk - 1);
    const float f = pos - (float)i;
    qout[(size_t)(b * Hkv + g) * 2 + threadIdx.x] = s[i] + f * (s[j] - s[i]);
  }
}

// Centroid (RBS) scores per (query block, query head, batch), one wave:
// block scores against every key block.  Lane = key block (blocks lane, lane + 64, ...), holding the
// block's summary in registers; the query block (float32, with its row norms)
// sits in LDS and every lane reads the same row (broadcast).  The log-sum-exp
// over the block's query tokens is an online update inside each lane, so no
// cross-lane reduction is needed.
template <int D>
__global__ __launch_bounds__(64) void attn_block_scores_kernel(
    float* __restrict__ base_out, float* __restrict__ rescue_out,
    const __bf16* __restrict__ Q, const float* __restrict__ stats,
    const float* __restrict__ quant, int H, int Hkv, int Sq, int nq, int nk,
    float scale) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) float s_q[kBlock][D];
  __shared__ float s_qn[kBlock];
  const int a = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int g = h / (H / Hkv);
  const int i0 = a * kBlock;
  const int nrows = min(kBlock, Sq - i0);
  // stage the query block as float32 and its row norms
  {
    const __bf16* qb = Q + ((size_t)(b * H + h) * Sq + i0) * D;
    for (int x = lane; x < nrows * (D / 8); x += 64) {
      const int r = x / (D / 8), c = x % (D / 8);
      const u32x4_t w = *(const u32x4_t*)(qb + (size_t)r * D + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_q[r][c * 8 + 2 * e] = bf16_lo(w[e]);
        s_q[r][c * 8 + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
    __syncthreads();
    if (lane < nrows) {
      float n2 = 0.f;
      for (int d = 0; d < D; ++d) n2 = __builtin_fmaf(s_q[lane][d], s_q[lane][d], n2);
      s_qn[lane] = sqrtf(n2);
    }
    __syncthreads();
  }
  const float* st = stats + (size_t)(b * Hkv + g) * nk * (3 * D + 1);
  const float r_low = quant[(size_t)(b * Hkv + g) * 2];
  const float r_high = quant[(size_t)(b * Hkv + g) * 2 + 1];
  const size_t row = ((size_t)(b * H + h) * nq + a) * nk;
  for (int kb = lane; kb < nk; kb += 64) {
    float v0[D];
#pragma unroll
    for (int d = 0; d < D; ++d) v0[d] = st[(size_t)kb * D + d];
    const float r = st[(size_t)3 * nk * D + kb];
    const float beta = r_high == r_low
                           ? (r > r_low ? 1.f : 0.f)
                           : fminf(fmaxf((r - r_low) / (r_high - r_low), 0.f), 1.f);
    const float w = r * beta;
    float m1 = -INFINITY, s1 = 0.f, m2 = -INFINITY, s2 = 0.f;
    for (int r = 0; r < nrows; ++r) {
      float part[8] = {};
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const f32x4_t x = *(const f32x4_t*)&s_q[r][d4 * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = d4 * 4 + e;
          part[d & 7] = __builtin_fmaf(x[e], v0[d], part[d & 7]);
        }
      }
      float acc = 0.f;
#pragma unroll
      for (int p = 0; p < 8; ++p) acc += part[p];
      const float e1 = acc * scale;
      const float n1 = fmaxf(m1, e1);
      s1 = s1 * __expf(m1 - n1) + __expf(e1 - n1);
      m1 = n1;
      const float e2 = __builtin_fmaf(s_qn[r], w, acc) * scale;
      const float n2 = fmaxf(m2, e2);
      s2 = s2 * __expf(m2 - n2) + __expf(e2 - n2);
      m2 = n2;
    }
    base_out[row + kb] = m1 + __logf(s1);
    if (rescue_out) rescue_out[row + kb] = m2 + __logf(s2);
  }
}

// Min/max box-bound scores per (query block, query head, batch).  Lane = query
// token of the block; wave w takes key blocks w, w + 4, ...; the block's lo /
// hi rows are wave-uniform (scalar loads), the log-sum-exp over the block's
// tokens is a wave reduction.  (The lane-per-key-block layout of the centroid
// kernel would need both 2 x D summaries in registers.)
template <int D>
__global__ __launch_bounds__(256) void attn_block_minmax_kernel(
    float* __restrict__ base_out, const __bf16* __restrict__ Q,
    const float* __restrict__ stats, int H, int Hkv, int Sq, int nq, int nk,
    float scale) {
  const int a = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loads
  const int g = h / (H / Hkv);
  const int i = a * kBlock + lane;
  const bool live = i < Sq;
  float q[D];
  {
    const u32x4_t* qp = (const u32x4_t*)(Q + ((size_t)(b * H + h) * Sq + (live ? i : 0)) * D);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4_t w = qp[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q[c * 8 + 2 * e] = bf16_lo(w[e]);
        q[c * 8 + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
  }
  const float* st = stats + (size_t)(b * Hkv + g) * nk * (3 * D + 1);
  const size_t row = ((size_t)(b * H + h) * nq + a) * nk;
  for (int kb = wave; kb < nk; kb += 4) {
    float ell;
    {
      const float* lo = st + (size_t)nk * D + (size_t)kb * D;
      const float* hi = st + (size_t)2 * nk * D + (size_t)kb * D;
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc += fmaxf(q[d] * lo[d], q[d] * hi[d]);
      ell = acc * scale;
    }
    // log-sum-exp over the block's live query tokens
    const float e1 = live ? ell : -INFINITY;
    const float m1 = wave_max(e1);
    const float s1 = wave_sum(live ? __expf(e1 - m1) : 0.f);
    if (lane == 0) base_out[row + kb] = m1 + __logf(s1);
  }
}

// One wave per block-mask row (a query block of one head): relative (mode 0),
// top-k (mode 1) or diagonal band (mode 2); with `accumulate` the result is
// ORed into keep.
__global__ __launch_bounds__(256) void attn_block_mask_kernel(
    uint8_t* __restrict__ keep, const float* __restrict__ scores, long long rows,
    int nq, int nk, int mode, float ln_alpha, int k, int diagonal, int accumulate) {
  const long long rw = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rw >= rows) return;
  const float* s = scores ? scores + rw * nk : nullptr;
  uint8_t* out = keep + rw * nk;
  float thr = 0.f;
  if (mode == 0) {
    float m = -INFINITY;
    for (int j = lane; j < nk; j += 64) m = fmaxf(m, s[j]);
    thr = wave_max(m) + ln_alpha;
  }
  const int a = (int)(rw % nq);
  for (int j = lane; j < nk; j += 64) {
    bool on;
    if (mode == 0) {
      on = s[j] >= thr;
    } else if (mode == 1) {
      const float x = s[j];
      int rank = 0;
      for (int t = 0; t < nk; ++t) {
        const float y = s[t];
        rank += (y > x) || (y == x && t < j);
      }
      on = rank < k;
    } else {
      on = (a - j < diagonal) && (j - a < diagonal);
    }
    out[j] = (uint8_t)((accumulate && out[j]) || on);
  }
}

size_t block_scores_workspace_bytes(int B, int Hkv, int Sk, int D) {
  const size_t nk = (size_t)(Sk + kBlock - 1) / kBlock;
  const size_t stats = (size_t)B * Hkv * nk * (3 * D + 1) * sizeof(float);
  return (stats + 255) / 256 * 256 + ((size_t)B * Hkv * 2 * sizeof(float) + 255) / 256 * 256;
}

template <int D>
static hipError_t launch_scores_d(float* base, float* rescue, const void* Q,
                                  const void* K, int B, int H, int Hkv, int Sq,
                                  int Sk, int kind, float low, float high,
                                  void* ws, hipStream_t stream) {
  const int nq = (Sq + kBlock - 1) / kBlock, nk = (Sk + kBlock - 1) / kBlock;
  float* stats = (float*)ws;
  const size_t sbytes = ((size_t)B * Hkv * nk * (3 * D + 1) * sizeof(float) + 255) / 256 * 256;
  float* quant = (float*)((char*)ws + sbytes);
  hipLaunchKernelGGL(attn_block_stats_kernel<D>, dim3(nk, Hkv, B), dim3(256), 0, stream,
                     (const __bf16*)K, stats, Hkv, Sk, nk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale = 1.f / sqrtf((float)D);
  if (kind == 1) {
    hipLaunchKernelGGL(attn_block_minmax_kernel<D>, dim3(nq, H, B), dim3(256), 0, stream,
                       base, (const __bf16*)Q, (const float*)stats, H, Hkv, Sq, nq, nk,
                       scale);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(attn_block_quantile_kernel, dim3(Hkv, B), dim3(256), 0, stream,
                     stats, quant, Hkv, nk, D, low, high);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_block_scores_kernel<D>, dim3(nq, H, B), dim3(64), 0,
                     stream, base, rescue, (const __bf16*)Q, (const float*)stats,
                     (const float*)quant, H, Hkv, Sq, nq, nk, scale);
  return hipGetLastError();
}

hipError_t launch_block_scores(float* base, float* rescue, const void* Q,
                               const void* K, int B, int H, int Hkv, int Sq,
                               int Sk, int D, int kind, float low, float high,
                               void* ws, hipStream_t stream) {
  if (D == 64)
    return launch_scores_d<64>(base, rescue, Q, K, B, H, Hkv, Sq, Sk, kind, low, high, ws,
                               stream);
  return launch_scores_d<128>(base, rescue, Q, K, B, H, Hkv, Sq, Sk, kind, low, high, ws,
                              stream);
}

hipError_t launch_block_mask(uint8_t* keep, const float* scores, long long rows,
                             int nq, int nk, int mode, float ln_alpha, int k,
                             int diagonal, int accumulate, hipStream_t stream) {
  hipLaunchKernelGGL(attn_block_mask_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, keep, scores, rows, nq, nk, mode, ln_alpha, k, diagonal,
                     accumulate);
  return hipGetLastError();
}

}  // namespace attn
