// Split-KV (Flash-Decoding) single-query decode for bf16 on gfx950.
//
// Tylo.jl "Primitives", decode_attention!: one query vector per head and
// sequence, valid KV length per sequence, the KV cache processed in n_splits
// parallel slices (TILE_N = 64), then combined.  The combination weighs each
// slice's normalised partial output by exp(LSE_s - max LSE), which is the
// softmax over the union of the slices.
//
// The work is HBM-bound (about 4 flop per byte of K/V), so the split kernel is
// built for streaming, not for the matrix cores:
//   * one workgroup = (sequence, KV head, slice[, head chunk]); it serves every
//     query head of the GQA group, so each K/V byte is read from HBM once;
//   * D/16 lanes share a key, each holding 16 of its d values (32 contiguous
//     bytes of K and of V); a wave reads whole 256-byte key rows;
//   * dot products with v_dot2c_f32_bf16 straight from the bf16 words, the
//     per-key sum by butterfly exchanges across the D/16 lanes;
//   * two key tiles in flight per thread (register double buffer);
//   * nothing past lengths[b] is ever read;
//   * the longest sequences are dealt first (rank by length) so the long
//     slices do not form the tail.
// A second small kernel merges the slices; with n_splits = 1 the split kernel
// writes the bf16 output itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;
constexpr int kDecTileN = 64;
constexpr float kDecLazy = 8.0f;
constexpr int kDecSortMaxB = 256;

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

__device__ inline uint16_t f32_to_bf16_rne(float x) {
  const bf16x2_t r = __builtin_convertvector(
      (float __attribute__((ext_vector_type(2)))){x, 0.f}, bf16x2_t);
  return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xffffu);
}

// Keys [k_begin, k_end) of slice s of a sequence with `len` valid keys.
__device__ inline void split_range(int len, int n_splits, int s, int* k_begin,
                                   int* k_end) {
  const int tiles = (len + kDecTileN - 1) / kDecTileN;
  const int per = ((tiles + n_splits - 1) / n_splits) * kDecTileN;
  const long long lo = (long long)s * per;
  *k_begin = (int)(lo < len ? lo : len);
  const long long hi = lo + per;
  *k_end = (int)(hi < len ? hi : len);
}

template <int D, int GM>
__global__ __launch_bounds__(kDecThreads) void attn_decode_split_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, const int32_t* __restrict__ lengths,
    float* __restrict__ Opart, float* __restrict__ Lpart,
    __bf16* __restrict__ O, int B, int H, int Hkv, int Smax, int n_splits,
    int n_hchunks, float scale_log2) {
  constexpr int LPK = D / 16;                 // lanes per key
  constexpr int NG = kDecThreads / LPK;       // keys per pass
  constexpr int KPT = kDecTileN / NG;         // keys per thread per tile
  constexpr int NGW = 64 / LPK;               // key groups per wave
  static_assert(KPT >= 1, "tile smaller than a pass");

  __shared__ int s_b;
  __shared__ float s_m[4][GM];
  __shared__ float s_acc[4][GM][D];
  __shared__ float s_l[4][GM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = tid % LPK;  // which 16-wide d slice
  const int gi = tid / LPK;  // key group within the workgroup

  // ---- work item: (rank, kv head, head chunk, slice) ----
  const int lid = blockIdx.x;
  const int s = lid % n_splits;
  int t = lid / n_splits;
  const int hc = t % n_hchunks;
  t /= n_hchunks;
  const int g = t % Hkv;
  const int rank = t / Hkv;

  int b = rank;
  if (B <= kDecSortMaxB) {
    // b = the sequence whose length ranks `rank`-th (longest first, ties by
    // index), so long slices start early.
    if (tid < B) {
      const int my = lengths[tid];
      int r = 0;
      for (int j = 0; j < B; ++j) {
        const int lj = lengths[j];
        r += (lj > my) || (lj == my && j < tid);
      }
      if (r == rank) s_b = tid;
    }
    __syncthreads();
    b = s_b;
  }

  const int len = min(max(lengths[b], 0), Smax);
  int k_begin, k_end;
  split_range(len, n_splits, s, &k_begin, &k_end);

  const int G = H / Hkv;
  const int h0 = g * G + hc * GM;
  const int nh = min(GM, G - hc * GM);

  // query slices, bf16 pairs
  uint32_t q[GM][8];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    const int hq = h0 + (hh < nh ? hh : 0);
    const u32x4_t* qp =
        (const u32x4_t*)(Q + ((size_t)b * H + hq) * D + li * 16);
    const u32x4_t a = qp[0], c = qp[1];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      q[hh][w] = a[w];
      q[hh][4 + w] = c[w];
    }
  }

  float m[GM], l[GM], acc[GM][16];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[hh][e] = 0.f;
  }

  const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)Smax * D;
  const __bf16* Kp = K + kv_base + li * 16;
  const __bf16* Vp = V + kv_base + li * 16;

  u32x4_t kr[2][KPT][2], vr[2][KPT][2];
  auto fetch = [&](int slot, int base) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int key = base + gi + NG * u;
      if (key < k_end) {
        const u32x4_t* kp = (const u32x4_t*)(Kp + (size_t)key * D);
        const u32x4_t* vp = (const u32x4_t*)(Vp + (size_t)key * D);
        kr[slot][u][0] = kp[0];
        kr[slot][u][1] = kp[1];
        vr[slot][u][0] = vp[0];
        vr[slot][u][1] = vp[1];
      } else {
        kr[slot][u][0] = kr[slot][u][1] = u32x4_t{0, 0, 0, 0};
        vr[slot][u][0] = vr[slot][u][1] = u32x4_t{0, 0, 0, 0};
      }
    }
  };

  const int ntiles = (k_end - k_begin + kDecTileN - 1) / kDecTileN;
  if (ntiles > 0) fetch(0, k_begin);
  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int base = k_begin + it * kDecTileN;
    if (it + 1 < ntiles) fetch(cur ^ 1, base + kDecTileN);

    float tsc[KPT][GM];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool valid = base + gi + NG * u < k_end;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          a = dot2_bf16(q[hh][w], kr[cur][u][0][w], a);
          a = dot2_bf16(q[hh][4 + w], kr[cur][u][1][w], a);
        }
#pragma unroll
        for (int x = 1; x < LPK; x <<= 1) a += __shfl_xor(a, x);
        tsc[u][hh] = valid ? a * scale_log2 : -INFINITY;
      }
    }

    bool need_any = false;
    float tmax[GM];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      tmax[hh] = tsc[0][hh];
#pragma unroll
      for (int u = 1; u < KPT; ++u) tmax[hh] = fmaxf(tmax[hh], tsc[u][hh]);
      need_any |= tmax[hh] > m[hh] + kDecLazy;
    }
    if (__builtin_amdgcn_ballot_w64(need_any)) {
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        const bool need = tmax[hh] > m[hh] + kDecLazy;
        const float alpha = need ? __builtin_amdgcn_exp2f(m[hh] - tmax[hh]) : 1.f;
        m[hh] = need ? tmax[hh] : m[hh];
        l[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[hh][e] *= alpha;
      }
    }

#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      float vf[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vf[2 * w] = bf16_lo(vr[cur][u][0][w]);
        vf[2 * w + 1] = bf16_hi(vr[cur][u][0][w]);
        vf[8 + 2 * w] = bf16_lo(vr[cur][u][1][w]);
        vf[8 + 2 * w + 1] = bf16_hi(vr[cur][u][1][w]);
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        const float mref = m[hh] == -INFINITY ? 0.f : m[hh];
        const float p = __builtin_amdgcn_exp2f(tsc[u][hh] - mref);
        l[hh] += p;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[hh][e] = __builtin_fmaf(p, vf[e], acc[hh][e]);
      }
    }
  }

  // ---- merge the key groups of the workgroup ----
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    float mw = m[hh];
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) mw = fmaxf(mw, __shfl_xor(mw, x));
    if (lane == 0) s_m[wave][hh] = mw;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    const float M = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]),
                          fmaxf(s_m[2][hh], s_m[3][hh]));
    const float f = m[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh] - M);
    float lw = l[hh] * f;
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) lw += __shfl_xor(lw, x);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float a = acc[hh][e] * f;
#pragma unroll
      for (int x = LPK; x < 64; x <<= 1) a += __shfl_xor(a, x);
      acc[hh][e] = a;
    }
    if (lane < LPK) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s_acc[wave][hh][li * 16 + e] = acc[hh][e];
      if (li == 0) s_l[wave][hh] = lw;
    }
  }
  __syncthreads();

  for (int idx = tid; idx < GM * D; idx += kDecThreads) {
    const int hh = idx / D, d = idx % D;
    if (hh >= nh) continue;
    const float M = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]),
                          fmaxf(s_m[2][hh], s_m[3][hh]));
    const float lt = s_l[0][hh] + s_l[1][hh] + s_l[2][hh] + s_l[3][hh];
    const float at = s_acc[0][hh][d] + s_acc[1][hh][d] + s_acc[2][hh][d] +
                     s_acc[3][hh][d];
    const float o = lt > 0.f ? at / lt : 0.f;
    const size_t bh = (size_t)b * H + h0 + hh;
    if (n_splits == 1) {
      ((uint16_t*)O)[bh * D + d] = f32_to_bf16_rne(o);
    } else {
      Opart[(bh * n_splits + s) * D + d] = o;
      if (d == 0) Lpart[bh * n_splits + s] = lt > 0.f ? M + __builtin_log2f(lt) : -INFINITY;
    }
  }
}

// One wave per (sequence, head): O = sum_s w_s O_s / sum_s w_s with
// w_s = 2^(L_s - max L) (L_s in base-2 units); O = 0 when every slice is empty.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(
    const float* __restrict__ Opart, const float* __restrict__ Lpart,
    __bf16* __restrict__ O, int BH, int n_splits) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (bh >= BH) return;
  const float* lp = Lpart + (size_t)bh * n_splits;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, lp[s]);
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float ls = lp[s];
      if (ls == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(ls - M);
      wsum += w;
      const float* op = Opart + ((size_t)bh * n_splits + s) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(w, op[lane + 64 * e], o[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    ((uint16_t*)O)[(size_t)bh * D + lane + 64 * e] = f32_to_bf16_rne(o[e] * inv);
}

size_t decode_workspace_bytes(int B, int H, int n_splits, int D) {
  const size_t bhs = (size_t)B * H * n_splits;
  const size_t o_bytes = (bhs * D * sizeof(float) + 255) / 256 * 256;
  const size_t l_bytes = (bhs * sizeof(float) + 255) / 256 * 256;
  return o_bytes + l_bytes;
}

template <int D, int GM>
static hipError_t launch_split(const void* Q, const void* K, const void* V,
                               const int32_t* lengths, float* Opart,
                               float* Lpart, void* O, int B, int H, int Hkv,
                               int Smax, int n_splits, hipStream_t stream) {
  const int G = H / Hkv;
  const int n_hchunks = (G + GM - 1) / GM;
  const long long grid = (long long)B * Hkv * n_hchunks * n_splits;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  hipLaunchKernelGGL((attn_decode_split_kernel<D, GM>), dim3((unsigned)grid),
                     dim3(kDecThreads), 0, stream, (const __bf16*)Q,
                     (const __bf16*)K, (const __bf16*)V, lengths, Opart, Lpart,
                     (__bf16*)O, B, H, Hkv, Smax, n_splits, n_hchunks,
                     scale_log2);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(void* O, const void* Q, const void* K,
                                  const void* V, const int32_t* lengths,
                                  int n_splits, int B, int H, int Hkv,
                                  int Smax, void* ws, hipStream_t stream) {
  const size_t bhs = (size_t)B * H * n_splits;
  float* Opart = (float*)ws;
  float* Lpart =
      (float*)((char*)ws + (bhs * D * sizeof(float) + 255) / 256 * 256);
  const int G = H / Hkv;
  hipError_t e;
  if (G <= 1)
    e = launch_split<D, 1>(Q, K, V, lengths, Opart, Lpart, O, B, H, Hkv, Smax, n_splits, stream);
  else if (G <= 2)
    e = launch_split<D, 2>(Q, K, V, lengths, Opart, Lpart, O, B, H, Hkv, Smax, n_splits, stream);
  else if (G <= 4)
    e = launch_split<D, 4>(Q, K, V, lengths, Opart, Lpart, O, B, H, Hkv, Smax, n_splits, stream);
  else
    e = launch_split<D, 8>(Q, K, V, lengths, Opart, Lpart, O, B, H, Hkv, Smax, n_splits, stream);
  if (e != hipSuccess || n_splits == 1) return e;
  const int BH = B * H;
  hipLaunchKernelGGL(attn_decode_merge_kernel<D>, dim3((BH + 3) / 4), dim3(256),
                     0, stream, (const float*)Opart, (const float*)Lpart,
                     (__bf16*)O, BH, n_splits);
  return hipGetLastError();
}

hipError_t launch_decode(void* O, const void* Q, const void* K, const void* V,
                         const int32_t* lengths, int n_splits, int B, int H,
                         int Hkv, int Smax, int D, void* ws,
                         hipStream_t stream) {
  if (D == 64)
    return launch_decode_d<64>(O, Q, K, V, lengths, n_splits, B, H, Hkv, Smax, ws, stream);
  return launch_decode_d<128>(O, Q, K, V, lengths, n_splits, B, H, Hkv, Smax, ws, stream);
}

}  // namespace attn
