// Block-score estimators and block masks for block-sparse prefill on gfx950.
//
// mlx-arsenal "Radius-bounded block scores (RBS)": a block score estimates how
// much a query block attends to a key block from a few statistics of the
// key block, without the token-level scores.
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
// The block statistics and masks are small float32 vector-ALU kernels (one
// pass over K); the centroid scores, a Q C^T contraction, run on the matrix
// cores.
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
// One pass over the block: 16-byte loads with 16 (D = 128) or 8 (D = 64)
// consecutive threads per row, each thread holding RPT rows x 8 d-values in
// registers; per-dimension sums / min / max reduce over the rows by lane
// shuffles and then across the four waves in LDS, row distances to the
// centroid over the row's threads by shuffles.
template <int D>
__global__ __launch_bounds__(256) void attn_block_stats_kernel(
    const __bf16* __restrict__ K, float* __restrict__ stats, int Hkv, int Sk,
    int nk) {
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;       // rows one pass of the workgroup covers
  constexpr int RPT = kBlock / RPP;    // rows per thread
  __shared__ float s_part[3][4][D];
  __shared__ float s_c[D];
  __shared__ float s_r[4];
  const int kb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % CPR;             // this thread's chunk: d = 8 c .. 8 c + 7
  const int j0 = kb * kBlock;
  const int n = min(kBlock, Sk - j0);
  const __bf16* kp = K + ((size_t)(b * Hkv + g) * Sk + j0) * D;
  float x[RPT][8];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = tid / CPR + i * RPP;
    u32x4_t v = {0, 0, 0, 0};
    if (r < n) v = *(const u32x4_t*)(kp + (size_t)r * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[i][2 * w] = bf16_lo(v[w]);
      x[i][2 * w + 1] = bf16_hi(v[w]);
    }
  }
  // per-dimension partials over this thread's rows, then over the wave's rows
  float su[8], lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    su[e] = 0.f;
    lo[e] = INFINITY;
    hi[e] = -INFINITY;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if (tid / CPR + i * RPP < n) {
        su[e] += x[i][e];
        lo[e] = fminf(lo[e], x[i][e]);
        hi[e] = fmaxf(hi[e], x[i][e]);
      }
    }
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1) {
      su[e] += __shfl_xor(su[e], o);
      lo[e] = fminf(lo[e], __shfl_xor(lo[e], o));
      hi[e] = fmaxf(hi[e], __shfl_xor(hi[e], o));
    }
  }
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_part[0][wave][c * 8 + e] = su[e];
      s_part[1][wave][c * 8 + e] = lo[e];
      s_part[2][wave][c * 8 + e] = hi[e];
    }
  }
  __syncthreads();
  float* base = stats + (size_t)(b * Hkv + g) * nk * (3 * D + 1);
  if (tid < D) {
    float sm = 0.f, l = INFINITY, h = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sm += s_part[0][w][tid];
      l = fminf(l, s_part[1][w][tid]);
      h = fmaxf(h, s_part[2][w][tid]);
    }
    const float cen = sm / (float)n;
    s_c[tid] = cen;
    base[(size_t)kb * D + tid] = cen;
    base[(size_t)nk * D + (size_t)kb * D + tid] = l;
    base[(size_t)2 * nk * D + (size_t)kb * D + tid] = h;
  }
  __syncthreads();
  // radius: the largest squared distance of a row to the centroid
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    float dist = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = x[i][e] - s_c[c * 8 + e];
      dist = __builtin_fmaf(t, t, dist);
    }
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) dist += __shfl_xor(dist, o);
    if (tid / CPR + i * RPP < n) m = fmaxf(m, dist);
  }
  m = wave_max(m);
  if (lane == 0) s_r[wave] = m;
  __syncthreads();
  if (tid == 0) {
    const float r = fmaxf(fmaxf(s_r[0], s_r[1]), fmaxf(s_r[2], s_r[3]));
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

// Block scores on the matrix cores.  A workgroup of four waves takes
// four query blocks of one (query head, batch); wave w scores block 4x + w
// against every key block.  Per chunk of 64 key blocks the workgroup stages
// the centroids in LDS split into three bf16 planes, c = c0 + c1 + c2 (each
// the bf16 rounding of what the previous ones leave), so that the bf16 MFMA
// products q.c0 + q.c1 + q.c2 with exact bf16 q and float32 accumulation give
// q.c to within 2^-27 |q||c| per term, float32 quality.  S = Q C^T comes out
// in the accumulator layout (lane: one key block, 16 query rows per 32 x 32
// tile), so the log-sum-exp over the 64 query rows is in-lane plus one
// exchange with lane ^ 32; the rescue term adds ||q_i|| r_b beta_b before
// the exponential.
// BOX: the min/max box bound instead of the centroid.  With m = (lo + hi) / 2
// and r = (hi - lo) / 2 per dimension, max(q lo, q hi) = q m + |q| r for
// either sign of q, so the bound is the contraction [q, |q|] . [m; r]: six
// planes (m and r, three each) and |q| by clearing the sign bits.
template <int D, bool BOX>
__global__ __launch_bounds__(256) void attn_block_scores_kernel(
    float* __restrict__ base_out, float* __restrict__ rescue_out,
    const __bf16* __restrict__ Q, const float* __restrict__ stats,
    const float* __restrict__ quant, int H, int Hkv, int Sq, int nq, int nk,
    float scale) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  constexpr int KSTEPS = D / 16;
  constexpr int ROW = D * 2 + 16;     // padded bf16 centroid row in LDS
  constexpr int PLANE = kBlock * ROW;
  constexpr int NPL = BOX ? 6 : 3;    // bf16 planes staged per chunk
  __shared__ __attribute__((aligned(16))) char s_c[NPL * PLANE];
  __shared__ float s_qn[4][kBlock];
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int lcol = lane & 31, half = lane >> 5;
  const int a = blockIdx.x * 4 + wave;  // this wave's query block
  const bool live = a < nq;
  const int g = h / (H / Hkv);
  const int i0 = a * kBlock;

  // Q rows as A operands: qa[rt][ks] = row rt*32 + lcol, d = 16 ks + 8 half..
  bf16x8_t qa[2][KSTEPS];
  float qn2[2] = {0.f, 0.f};
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int i = i0 + rt * 32 + lcol;
    const bool ok = live && i < Sq;
    const __bf16* qp = Q + ((size_t)(b * H + h) * Sq + (ok ? i : 0)) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4_t w = ok ? *(const u32x4_t*)(qp + ks * 16) : u32x4_t{0, 0, 0, 0};
      qa[rt][ks] = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
        qn2[rt] = __builtin_fmaf(x0, x0, __builtin_fmaf(x1, x1, qn2[rt]));
      }
    }
  }
  // ||q|| of the wave's 64 rows into LDS (the two halves of a row sit in lanes l, l ^ 32)
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float t = qn2[rt] + __shfl_xor(qn2[rt], 32);
    if (half == 0) s_qn[wave][rt * 32 + lcol] = sqrtf(t);
  }
  __syncthreads();
  // query rows of the block below Sq; the lane's rows of the accumulator
  // layout are rt*32 + 8 (r/4) + 4 half + r%4
  const int nrows = live ? min(kBlock, Sq - i0) : 0;
  auto row_of = [&](int rt, int r) { return rt * 32 + (r >> 2) * 8 + half * 4 + (r & 3); };

  const float* st = stats + (size_t)(b * Hkv + g) * nk * (3 * D + 1);
  // radius quantiles of the head (centroid scores only; the box bound has none)
  const float r_low = BOX ? 0.f : quant[(size_t)(b * Hkv + g) * 2];
  const float r_high = BOX ? 0.f : quant[(size_t)(b * Hkv + g) * 2 + 1];
  const size_t orow = ((size_t)(b * H + h) * nq + (live ? a : 0)) * nk;

  for (int c0 = 0; c0 < nk; c0 += kBlock) {
    // stage centroids c0 .. c0 + 63 (zeros past nk) as three bf16 planes
    __syncthreads();  // the previous chunk's reads are done
    auto split3 = [&](const f32x4_t c, char* dst) {
      bf16x4_t p0, p1, p2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 h0 = (__bf16)c[e];
        const float r1 = c[e] - (float)h0;
        const __bf16 h1 = (__bf16)r1;
        const float r2 = r1 - (float)h1;
        p0[e] = h0;
        p1[e] = h1;
        p2[e] = (__bf16)r2;
      }
      *(bf16x4_t*)(dst) = p0;
      *(bf16x4_t*)(dst + PLANE) = p1;
      *(bf16x4_t*)(dst + 2 * PLANE) = p2;
    };
    for (int x = tid; x < kBlock * (D / 4); x += 256) {
      const int kb = x / (D / 4), d4 = x % (D / 4);
      const bool in = c0 + kb < nk;
      char* dst = s_c + kb * ROW + d4 * 8;
      const size_t off = (size_t)(c0 + kb) * D + d4 * 4;
      if constexpr (BOX) {
        const f32x4_t lo = in ? *(const f32x4_t*)(st + (size_t)nk * D + off) : f32x4_t{};
        const f32x4_t hi = in ? *(const f32x4_t*)(st + (size_t)2 * nk * D + off) : f32x4_t{};
        split3((lo + hi) * 0.5f, dst);
        split3((hi - lo) * 0.5f, dst + 3 * PLANE);
      } else {
        split3(in ? *(const f32x4_t*)(st + off) : f32x4_t{}, dst);
      }
    }
    __syncthreads();
    if (!live) continue;
    // S = Q C^T in tiles of 32 rows x 32 key blocks, one column tile at a time
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          const bf16x8_t bop = *(const bf16x8_t*)(s_c + pl * PLANE + (ct * 32 + lcol) * ROW +
                                                 ks * 32 + half * 16);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            bf16x8_t x = qa[rt][ks];
            if (BOX && pl >= 3)  // |q|
              x = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, x) & 0x7fff7fffu);
            acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, bop, acc[rt], 0, 0, 0);
          }
        }
      // log-sum-exp over the query rows, per key block (the lane's column)
      const int kb = c0 + ct * 32 + lcol;
      float w = 0.f;
      if (!BOX && rescue_out && kb < nk) {
        const float r = st[(size_t)3 * nk * D + kb];
        const float beta = r_high == r_low
                               ? (r > r_low ? 1.f : 0.f)
                               : fminf(fmaxf((r - r_low) / (r_high - r_low), 0.f), 1.f);
        w = r * beta;
      }
      float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_of(rt, r);
          if (row >= nrows) continue;
          m1 = fmaxf(m1, acc[rt][r] * scale);
          m2 = fmaxf(m2, __builtin_fmaf(s_qn[wave][row], w, acc[rt][r]) * scale);
        }
      m1 = fmaxf(m1, __shfl_xor(m1, 32));
      m2 = fmaxf(m2, __shfl_xor(m2, 32));
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_of(rt, r);
          if (row >= nrows) continue;
          s1 += __expf(acc[rt][r] * scale - m1);
          s2 += __expf(__builtin_fmaf(s_qn[wave][row], w, acc[rt][r]) * scale - m2);
        }
      s1 += __shfl_xor(s1, 32);
      s2 += __shfl_xor(s2, 32);
      if (half == 0 && kb < nk) {
        base_out[orow + kb] = m1 + __logf(s1);
        if (!BOX && rescue_out) rescue_out[orow + kb] = m2 + __logf(s2);
      }
    }
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
    hipLaunchKernelGGL((attn_block_scores_kernel<D, true>), dim3((nq + 3) / 4, H, B), dim3(256),
                       0, stream, base, nullptr, (const __bf16*)Q, (const float*)stats,
                       (const float*)nullptr, H, Hkv, Sq, nq, nk, scale);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(attn_block_quantile_kernel, dim3(Hkv, B), dim3(256), 0, stream,
                     stats, quant, Hkv, nk, D, low, high);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_block_scores_kernel<D, false>), dim3((nq + 3) / 4, H, B), dim3(256), 0,
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
