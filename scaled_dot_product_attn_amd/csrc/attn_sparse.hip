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

#include <type_traits>

namespace attn {

namespace sparse {

constexpr int kBlock = 64;       // tokens per query / key block
constexpr int kMaxBlocks = 4096; // key blocks per head the quantile sort holds

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

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

// One exchange step of the radius reduction (see attn_block_stats_kernel):
// over lane bit O, keep CNT of the 2 CNT partials and add the partner's.
template <int CNT, int O>
__device__ inline void halve_sum(float* dist, int lane) {
  if constexpr (O >= 1) {
    const bool upper = (lane & O) != 0;
#pragma unroll
    for (int k = 0; k < CNT; ++k) {
      const float keep = upper ? dist[k + CNT] : dist[k];
      const float send = upper ? dist[k] : dist[k + CNT];
      dist[k] = keep + __shfl_xor(send, O);
    }
    halve_sum<CNT / 2, O / 2>(dist, lane);
  }
}

}  // namespace sparse

using namespace sparse;

// Per (key block, KV head, batch): centroid, per-dimension min / max, radius.
// stats layout per (b, g): c (nk, D), lo (nk, D), hi (nk, D), r (nk).
// One wave per key block, four blocks per workgroup: lane l holds the 16-byte
// chunk l % CPR (8 d-values) of rows l / CPR + RPW i, all NI loads issued
// before any arithmetic; per-dimension sums / min / max reduce over the
// lanes of a chunk by shuffles, row distances to the centroid over a row's
// lanes.  The wave also writes the bf16 operand planes of the score kernel
// (the centroid, or for the box bound its midpoint and half-width, each as
// three bf16 planes whose sum is the float32 value), once per block instead
// of once per query-block workgroup.
template <int D>
__global__ __launch_bounds__(256) void attn_block_stats_kernel(
    const __bf16* __restrict__ K, float* __restrict__ stats, __bf16* __restrict__ planes,
    int B, int Hkv, int Sk, int nk, int box) {
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPW = 64 / CPR;     // rows one load instruction of the wave covers
  constexpr int NI = kBlock / RPW;  // loads per lane
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long long)B * Hkv * nk) return;
  const int kb = (int)(w % nk);
  const long long bg = w / nk;      // b * Hkv + g
  const int c = lane % CPR, r0 = lane / CPR;
  const int j0 = kb * kBlock;
  const int n = min(kBlock, Sk - j0);
  const __bf16* kp = K + ((size_t)bg * Sk + j0) * D + c * 8;
  u32x4_t v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = r0 + i * RPW;
    v[i] = r < n ? *(const u32x4_t*)(kp + (size_t)r * D) : u32x4_t{0, 0, 0, 0};
  }
  auto elem = [&](int i, int e) {
    return (e & 1) ? bf16_hi(v[i][e >> 1]) : bf16_lo(v[i][e >> 1]);
  };
  // rows past n load as zeros: they add nothing to the sums and are kept out
  // of the minima / maxima and the radius by selects (no branches)
  float su[8], lo[8], hi[8], cen[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    su[e] = 0.f;
    lo[e] = INFINITY;
    hi[e] = -INFINITY;
  }
  auto accumulate = [&](auto whole) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool ok = whole || r0 + i * RPW < n;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = elem(i, e);
        su[e] += x;
        lo[e] = fminf(lo[e], ok ? x : INFINITY);
        hi[e] = fmaxf(hi[e], ok ? x : -INFINITY);
      }
    }
  };
  if (n == kBlock)
    accumulate(std::true_type{});
  else
    accumulate(false);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1) {
      su[e] += __shfl_xor(su[e], o);
      lo[e] = fminf(lo[e], __shfl_xor(lo[e], o));
      hi[e] = fmaxf(hi[e], __shfl_xor(hi[e], o));
    }
    cen[e] = su[e] / (float)n;
  }
  float* base = stats + (size_t)bg * nk * (3 * D + 1);
  if (lane < CPR) {
    float* cp = base + (size_t)kb * D + c * 8;
    *(float4*)cp = make_float4(cen[0], cen[1], cen[2], cen[3]);
    *(float4*)(cp + 4) = make_float4(cen[4], cen[5], cen[6], cen[7]);
    float* lp = cp + (size_t)nk * D;
    *(float4*)lp = make_float4(lo[0], lo[1], lo[2], lo[3]);
    *(float4*)(lp + 4) = make_float4(lo[4], lo[5], lo[6], lo[7]);
    float* hp = lp + (size_t)nk * D;
    *(float4*)hp = make_float4(hi[0], hi[1], hi[2], hi[3]);
    *(float4*)(hp + 4) = make_float4(hi[4], hi[5], hi[6], hi[7]);
  }
  // radius: the largest squared distance of a row to the centroid.  Row i's
  // distance is the sum of its CPR lanes' partials; the NI partials of a
  // lane reduce over those lanes by halving exchanges (at the step over lane
  // bit o the lane keeps the half of its rows it is responsible for and adds
  // the partner's partials of the same rows), so each lane ends with the
  // whole distance of one row (NI >= CPR).
  static_assert(NI >= CPR, "a row per lane after the exchanges");
  float dist[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float t2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = elem(i, e) - cen[e];
      t2 = __builtin_fmaf(t, t, t2);
    }
    dist[i] = r0 + i * RPW < n ? t2 : 0.f;
  }
  halve_sum<NI / 2, CPR / 2>(dist, lane);
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < NI / CPR; ++k) m = fmaxf(m, dist[k]);
  m = wave_max(m);
  if (lane == 0) base[(size_t)3 * nk * D + kb] = sqrtf(m);
  // operand planes: plane p of (b, g) is (nk, D) bf16 at planes + (bg * 6 + p) * nk * D
  if (lane < CPR) {
    __bf16* pp = planes + ((size_t)bg * 6 * nk + kb) * D + c * 8;
    auto split3 = [&](const float (&x)[8], int p0) {
      bf16x8_t q0, q1, q2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 h0 = (__bf16)x[e];
        const float r1 = x[e] - (float)h0;
        const __bf16 h1 = (__bf16)r1;
        q0[e] = h0;
        q1[e] = h1;
        q2[e] = (__bf16)(r1 - (float)h1);
      }
      *(bf16x8_t*)(pp + (size_t)p0 * nk * D) = q0;
      *(bf16x8_t*)(pp + (size_t)(p0 + 1) * nk * D) = q1;
      *(bf16x8_t*)(pp + (size_t)(p0 + 2) * nk * D) = q2;
    };
    if (!box) {
      split3(cen, 0);
    } else {
      float mid[8], rad[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mid[e] = (lo[e] + hi[e]) * 0.5f;
        rad[e] = (hi[e] - lo[e]) * 0.5f;
      }
      split3(mid, 0);
      split3(rad, 3);
    }
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
// against every key block.  Per chunk of 64 key blocks the workgroup copies
// into LDS the centroids as three bf16 planes, c = c0 + c1 + c2 (each the
// bf16 rounding of what the previous ones leave, written by the statistics
// kernel), so that the bf16 MFMA products q.c0 + q.c1 + q.c2 with exact bf16
// q and float32 accumulation give q.c to within 2^-27 |q||c| per term,
// float32 quality.  S = Q C^T comes out
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
    const __bf16* __restrict__ planes, const float* __restrict__ quant, int H, int Hkv,
    int Sq, int nq, int nk, float scale) {
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
  const __bf16* pls = planes + (size_t)(b * Hkv + g) * 6 * nk * D;
  // radius quantiles of the head (the rescue scores only)
  const float r_low = !BOX && rescue_out ? quant[(size_t)(b * Hkv + g) * 2] : 0.f;
  const float r_high = !BOX && rescue_out ? quant[(size_t)(b * Hkv + g) * 2 + 1] : 0.f;
  const size_t orow = ((size_t)(b * H + h) * nq + (live ? a : 0)) * nk;

  for (int c0 = 0; c0 < nk; c0 += kBlock) {
    // copy the planes of key blocks c0 .. c0 + 63 (zeros past nk) into LDS
    __syncthreads();  // the previous chunk's reads are done
    // (in batches of three planes: a thread's loads of a batch are all in
    // flight before its stores)
    constexpr int CH = D / 8;                    // 16-byte chunks per row
    constexpr int PER = 3 * kBlock * CH / 256;   // chunks per thread per batch
#pragma unroll
    for (int p0 = 0; p0 < NPL; p0 += 3) {
      u32x4_t v[PER];
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int x = tid + t * 256;
        const int pl = p0 + x / (kBlock * CH), rem = x % (kBlock * CH);
        const int kb = rem / CH, ch = rem % CH;
        v[t] = c0 + kb < nk ? *(const u32x4_t*)(pls + ((size_t)pl * nk + c0 + kb) * D + ch * 8)
                            : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int x = tid + t * 256;
        const int pl = p0 + x / (kBlock * CH), rem = x % (kBlock * CH);
        const int kb = rem / CH, ch = rem % CH;
        *(u32x4_t*)(s_c + pl * PLANE + kb * ROW + ch * 16) = v[t];
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
      // log-sum-exp over the block's rows (rows past its end count as -inf),
      // in base 2: exp2 and log2 are single instructions
      constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.69314718055994531f;
      const float sc = scale * kLog2e;
      auto lse = [&](auto with_rescue) {
        float t[2][16];
        float mx = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row_of(rt, r);
            float x = acc[rt][r];
            if constexpr (decltype(with_rescue)::value) x = __builtin_fmaf(s_qn[wave][row], w, x);
            t[rt][r] = row < nrows ? x * sc : -INFINITY;
            mx = fmaxf(mx, t[rt][r]);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        float sm = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int r = 0; r < 16; ++r) sm += __builtin_amdgcn_exp2f(t[rt][r] - mx);
        sm += __shfl_xor(sm, 32);
        return (mx + __builtin_amdgcn_logf(sm)) * kLn2;
      };
      const float l1 = lse(std::false_type{});
      if (half == 0 && kb < nk) base_out[orow + kb] = l1;
      if (!BOX && rescue_out) {
        const float l2 = lse(std::true_type{});
        if (half == 0 && kb < nk) rescue_out[orow + kb] = l2;
      }
    }
  }
}

// One wave per block-mask row (a query block of one head): relative (mode 0),
// top-k (mode 1) or diagonal band (mode 2); with `accumulate` the result is
// ORed into keep.  Top-k ranks each entry against the whole row, which the
// wave first copies into its own LDS (rows up to kMaskRow entries).
constexpr int kMaskRow = 1024;
__global__ __launch_bounds__(256) void attn_block_mask_kernel(
    uint8_t* __restrict__ keep, const float* __restrict__ scores, long long rows,
    int nq, int nk, int mode, float ln_alpha, int k, int diagonal, int accumulate) {
  __shared__ float s_row[4][kMaskRow];
  const long long rw = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rw >= rows) return;
  const float* s = scores ? scores + rw * nk : nullptr;
  // (the wave reads back only what it wrote; a wave's LDS accesses run in
  // program order)
  const bool staged = mode == 1 && nk <= kMaskRow;
  float* row = s_row[threadIdx.x >> 6];
  if (staged)
    for (int j = lane; j < nk; j += 64) row[j] = s[j];
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
      if (staged) {
        for (int t = 0; t < nk; ++t) {
          const float y = row[t];
          rank += (y > x) || (y == x && t < j);
        }
      } else {
        for (int t = 0; t < nk; ++t) {
          const float y = s[t];
          rank += (y > x) || (y == x && t < j);
        }
      }
      on = rank < k;
    } else {
      on = (a - j < diagonal) && (j - a < diagonal);
    }
    out[j] = (uint8_t)((accumulate && out[j]) || on);
  }
}

// Workspace: the block statistics (float32), the radius quantiles, the bf16
// operand planes (six per (b, g): enough for the box bound's two values).
static size_t ws_stats_bytes(int B, int Hkv, size_t nk, int D) {
  return ((size_t)B * Hkv * nk * (3 * D + 1) * sizeof(float) + 255) / 256 * 256;
}
static size_t ws_quant_bytes(int B, int Hkv) {
  return ((size_t)B * Hkv * 2 * sizeof(float) + 255) / 256 * 256;
}

size_t block_scores_workspace_bytes(int B, int Hkv, int Sk, int D) {
  const size_t nk = (size_t)(Sk + kBlock - 1) / kBlock;
  return ws_stats_bytes(B, Hkv, nk, D) + ws_quant_bytes(B, Hkv) +
         ((size_t)B * Hkv * 6 * nk * D * 2 + 255) / 256 * 256;
}

template <int D>
static hipError_t launch_scores_d(float* base, float* rescue, const void* Q,
                                  const void* K, int B, int H, int Hkv, int Sq,
                                  int Sk, int kind, float low, float high,
                                  void* ws, hipStream_t stream) {
  const int nq = (Sq + kBlock - 1) / kBlock, nk = (Sk + kBlock - 1) / kBlock;
  float* stats = (float*)ws;
  float* quant = (float*)((char*)ws + ws_stats_bytes(B, Hkv, nk, D));
  __bf16* planes = (__bf16*)((char*)quant + ws_quant_bytes(B, Hkv));
  const long long nblk = (long long)B * Hkv * nk;
  hipLaunchKernelGGL(attn_block_stats_kernel<D>, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0,
                     stream, (const __bf16*)K, stats, planes, B, Hkv, Sk, nk, kind == 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale = 1.f / sqrtf((float)D);
  if (kind == 1) {
    hipLaunchKernelGGL((attn_block_scores_kernel<D, true>), dim3((nq + 3) / 4, H, B), dim3(256),
                       0, stream, base, nullptr, (const __bf16*)Q, (const float*)stats,
                       (const __bf16*)planes, (const float*)nullptr, H, Hkv, Sq, nq, nk, scale);
    return hipGetLastError();
  }
  // the radius quantiles only weigh the rescue scores
  if (rescue) {
    hipLaunchKernelGGL(attn_block_quantile_kernel, dim3(Hkv, B), dim3(256), 0, stream,
                       stats, quant, Hkv, nk, D, low, high);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_block_scores_kernel<D, false>), dim3((nq + 3) / 4, H, B), dim3(256), 0,
                     stream, base, rescue, (const __bf16*)Q, (const float*)stats,
                     (const __bf16*)planes, (const float*)quant, H, Hkv, Sq, nq, nk, scale);
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
