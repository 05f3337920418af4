// Fused attention forward for float32 Q/K/V/O: exact float32 products and
// sums, no reduced-precision contraction inside (Tylo.jl "Primitives",
// attention!: compute precision follows the element type of Q, Float32
// accumulation).  Same mask and LSE semantics as the bf16 kernel.
//
// One workgroup = 256 threads = 64 query rows x 4 lanes.  Each lane holds a
// quarter of its row's query and output vectors (16-byte d chunks
// 16*c + 4*part .. +3).  K and V tiles of 32 keys are staged in LDS; every
// lane of a row reads the same K/V words, so the LDS reads are broadcasts.
// The score of a key is the sum of the four lanes' partial dot products
// (two butterfly exchanges), followed by a per-tile online softmax.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_common.h"

namespace attn {

constexpr int kF32Rows = 64;
constexpr int kF32Threads = 256;
constexpr int kF32TileN = 32;

template <int D>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32_kernel(
    float* __restrict__ O, const float* __restrict__ Q,
    const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ LSE, int B, int H, int Hkv, int Sq, int Sk, int causal,
    int window, int input_pos, const int32_t* __restrict__ k_lengths,
    float scale_log2) {
  constexpr int C = D / 16;  // float4 chunks per lane
  __shared__ float4 ks[kF32TileN * D / 4];
  __shared__ float4 vs[kF32TileN * D / 4];

  const int tid = threadIdx.x;
  const int part = tid & 3;
  const int row = tid >> 2;
  const int nqt = (Sq + kF32Rows - 1) / kF32Rows;
  const int qt = blockIdx.x % nqt;
  const int bh = blockIdx.x / nqt;
  const int b = bh / H, h = bh % H;
  const int g = h / (H / Hkv);

  const int i0 = qt * kF32Rows;
  const int i1 = min(i0 + kF32Rows, Sq);
  const int kl = k_lengths ? min(max(k_lengths[b], 0), Sk) : Sk;
  const KvGeometry geo = kv_geometry(i0, i1, kl, causal, window, input_pos);
  const int qi = i0 + row;
  const RowRange rr = row_range(qi, kl, causal, window, input_pos);

  const float* Kp = K + ((size_t)(b * Hkv + g) * Sk) * D;
  const float* Vp = V + ((size_t)(b * Hkv + g) * Sk) * D;
  const size_t qrow = ((size_t)(b * H + h) * Sq + (qi < Sq ? qi : 0)) * D;

  float4 q[C], acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    q[c] = qi < Sq ? *(const float4*)(Q + qrow + 16 * c + 4 * part)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m_run = -INFINITY, l_run = 0.f;

  int kt_first = 0, kt_last = -1;
  if (geo.any) {
    kt_first = geo.union_lo / kF32TileN;
    kt_last = (geo.union_hi - 1) / kF32TileN;
  }
  for (int kt = kt_first; kt <= kt_last; ++kt) {
    const int j0 = kt * kF32TileN;
    __syncthreads();
    for (int e = tid; e < kF32TileN * D / 4; e += kF32Threads) {
      const int key = j0 + e / (D / 4);
      const bool ok = key >= geo.union_lo && key < geo.union_hi;
      const size_t off = (size_t)key * D + (e % (D / 4)) * 4;
      ks[e] = ok ? *(const float4*)(Kp + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      vs[e] = ok ? *(const float4*)(Vp + off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    float s[kF32TileN];
#pragma unroll
    for (int j = 0; j < kF32TileN; ++j) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float4 k4 = ks[j * (D / 4) + 4 * c + part];
        a = fmaf(q[c].x, k4.x, a);
        a = fmaf(q[c].y, k4.y, a);
        a = fmaf(q[c].z, k4.z, a);
        a = fmaf(q[c].w, k4.w, a);
      }
      a += __shfl_xor(a, 1);
      a += __shfl_xor(a, 2);
      const int key = j0 + j;
      s[j] = (key >= rr.lo && key < rr.hi) ? a * scale_log2 : -INFINITY;
    }
    float mx = m_run;
#pragma unroll
    for (int j = 0; j < kF32TileN; ++j) mx = fmaxf(mx, s[j]);
    const float mref = mx == -INFINITY ? 0.f : mx;
    const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - mref);
    m_run = mx;
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      acc[c].x *= alpha; acc[c].y *= alpha; acc[c].z *= alpha; acc[c].w *= alpha;
    }
#pragma unroll
    for (int j = 0; j < kF32TileN; ++j) {
      const float p = exp2f(s[j] - mref);
      psum += p;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float4 v4 = vs[j * (D / 4) + 4 * c + part];
        acc[c].x = fmaf(p, v4.x, acc[c].x);
        acc[c].y = fmaf(p, v4.y, acc[c].y);
        acc[c].z = fmaf(p, v4.z, acc[c].z);
        acc[c].w = fmaf(p, v4.w, acc[c].w);
      }
    }
    l_run = l_run * alpha + psum;
  }

  if (qi < Sq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float4 o = acc[c];
      o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
      *(float4*)(O + qrow + 16 * c + 4 * part) = o;
    }
    if (LSE && part == 0)
      LSE[(size_t)(b * H + h) * Sq + qi] =
          l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f
                      : -INFINITY;
  }
}

template <int D>
hipError_t launch_fwd_f32(void* O, const void* Q, const void* K, const void* V,
                          float* LSE, int B, int H, int Hkv, int Sq, int Sk,
                          int causal, int window, int input_pos,
                          const int32_t* k_lengths, hipStream_t stream) {
  const int nqt = (Sq + kF32Rows - 1) / kF32Rows;
  const long long total = (long long)nqt * H * B;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  hipLaunchKernelGGL(attn_fwd_f32_kernel<D>, dim3((unsigned)total),
                     dim3(kF32Threads), 0, stream, (float*)O, (const float*)Q,
                     (const float*)K, (const float*)V, LSE, B, H, Hkv, Sq, Sk,
                     causal, window, input_pos, k_lengths, scale_log2);
  return hipGetLastError();
}

template hipError_t launch_fwd_f32<64>(void*, const void*, const void*,
                                       const void*, float*, int, int, int, int,
                                       int, int, int, int, const int32_t*,
                                       hipStream_t);
template hipError_t launch_fwd_f32<128>(void*, const void*, const void*,
                                        const void*, float*, int, int, int,
                                        int, int, int, int, int,
                                        const int32_t*, hipStream_t);

}  // namespace attn
