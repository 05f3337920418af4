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
//   * D/8 lanes share a key, each holding one 16-byte chunk (8 d values) of
//     K and of V; a wave reads whole 256-byte key rows;
//   * dot products with v_dot2c_f32_bf16 straight from the bf16 words, the
//     per-key sum by butterfly exchanges across the D/8 lanes;
//   * a ring of four key passes in flight per thread, loaded through buffer
//     resources that cover exactly the slice's keys, and about 100 VGPRs so
//     four waves share each SIMD: enough bytes in flight to cover HBM latency;
//   * nothing past lengths[b] is ever read;
//   * the longest sequences are dealt first (rank by length) so the long
//     slices do not form the tail.
// A second small kernel merges the slices; with n_splits = 1 the split kernel
// writes the bf16 output itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_host.h"

namespace attn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;
constexpr int kDecTileN = 64;
constexpr float kDecLazy = 8.0f;
constexpr int kDecSortMaxB = 256;
constexpr int kDecStages = 4;              // key passes in flight per thread
// Word 3 of a gfx9-family raw buffer resource: out-of-range reads return 0.
constexpr int kDecRsrcWord3 = 0x00020000;
// Cache policy of the K/V stream: non-temporal (every byte is read once;
// measured 5.76 -> 6.41 TB/s on the contiguous decode workload)
constexpr int kDecNT = 2;

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Sum over aligned groups of LPK lanes (LPK in {2, 4, 8, 16}) with DPP moves:
// swap neighbours, swap pairs, mirror within 8 lanes, mirror within 16 lanes.
template <int CTRL>
__device__ inline float dpp_mov(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int LPK>
__device__ inline float group_sum(float x) {
  static_assert(LPK == 2 || LPK == 4 || LPK == 8 || LPK == 16, "group size");
  x += dpp_mov<0xB1>(x);                  // quad_perm [1,0,3,2]
  if (LPK >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  if (LPK >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
  if (LPK >= 16) x += dpp_mov<0x140>(x);  // row_mirror
  return x;
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

// b = the sequence whose length ranks `rank`-th (longest first, ties by
// index), so long slices start early; identity when B is too large to rank.
__device__ inline int batch_of_rank(const int32_t* __restrict__ lengths, int B,
                                    int rank, int tid, int& s_b) {
  if (B > kDecSortMaxB) return rank;
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
  return s_b;
}

// Merge the key slots of the workgroup (per-slot running max m, sum l and
// unnormalised accumulators) and write the slice's result: the bf16 output
// when there is a single slice, else the normalised partial output and its
// base-2 LSE.
template <int D, int GM>
__device__ inline void slice_epilogue(
    float (&m)[GM], float (&l)[GM], float (&acc)[GM][8], float (&s_m)[4][GM],
    float (&s_acc)[4][GM][D], float (&s_l)[4][GM], int tid, int b, int H,
    int h0, int nh, int s, int n_splits, float* __restrict__ Opart,
    float* __restrict__ Lpart, __bf16* __restrict__ O) {
  constexpr int LPK = D / 8;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = tid % LPK;
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
    for (int e = 0; e < 8; ++e) {
      float a = acc[hh][e] * f;
#pragma unroll
      for (int x = LPK; x < 64; x <<= 1) a += __shfl_xor(a, x);
      acc[hh][e] = a;
    }
    if (lane < LPK) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][hh][li * 8 + e] = acc[hh][e];
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


template <int D, int GM>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4)))
void attn_decode_split_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, const int32_t* __restrict__ lengths,
    float* __restrict__ Opart, float* __restrict__ Lpart,
    __bf16* __restrict__ O, int B, int H, int Hkv, int Smax, int n_splits,
    int n_hchunks, float scale_log2) {
  constexpr int LPK = D / 8;               // lanes per key, 8 d (16 bytes) each
  constexpr int KPP = kDecThreads / LPK;   // keys per pass of the workgroup
  constexpr int NS = kDecStages;           // passes in flight per thread

  __shared__ int s_b;
  __shared__ float s_m[4][GM];
  __shared__ float s_acc[4][GM][D];
  __shared__ float s_l[4][GM];

  const int tid = threadIdx.x;
  const int li = tid % LPK;  // which 8-wide d chunk
  const int gi = tid / LPK;  // key slot within a pass

  // ---- work item: (rank, kv head, head chunk, slice) ----
  const int lid = blockIdx.x;
  const int s = lid % n_splits;
  int t = lid / n_splits;
  const int hc = t % n_hchunks;
  t /= n_hchunks;
  const int g = t % Hkv;
  const int rank = t / Hkv;

  const int b = batch_of_rank(lengths, B, rank, tid, s_b);

  const int len = min(max(lengths[b], 0), Smax);
  int k_begin, k_end;
  split_range(len, n_splits, s, &k_begin, &k_end);

  const int G = H / Hkv;
  const int h0 = g * G + hc * GM;
  const int nh = min(GM, G - hc * GM);

  // query chunks, bf16 pairs
  uint32_t q[GM][4];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    const int hq = h0 + (hh < nh ? hh : 0);
    const u32x4_t a = *(const u32x4_t*)(Q + ((size_t)b * H + hq) * D + li * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) q[hh][w] = a[w];
  }

  float m[GM], l[GM], acc[GM][8];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  }

  // Buffer resources covering exactly this slice's keys: reads past k_end
  // (the padded part of the cache included) return zeros without a branch.
  const size_t kv_base =
      ((size_t)b * Hkv + g) * (size_t)Smax * D + (size_t)k_begin * D;
  const int nbytes = (k_end - k_begin) * D * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(K + kv_base), (short)0, nbytes, kDecRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(V + kv_base), (short)0, nbytes, kDecRsrcWord3);
  const int lane_off = (gi * D + li * 8) * 2;

  const int nkeys = k_end - k_begin;
  const int npass = (nkeys + KPP - 1) / KPP;
  const int nround = (npass + NS - 1) / NS;
  // Ring of NS passes in flight, refilled one round (NS passes) ahead.  Round
  // -1 runs on zeros and only issues the first loads, and the body has no
  // branch, so the wait before each use counts exactly the loads issued after
  // it.  K for round r+1 is requested once round r's scores are done, V once
  // round r's P.V is done.
  u32x4_t kr[NS], vr[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) kr[st] = vr[st] = u32x4_t{0, 0, 0, 0};

  for (int rd = -1; rd < nround; ++rd) {
    float tsc[NS][GM];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bool valid = rd >= 0 && (rd * NS + st) * KPP + gi < nkeys;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) a = dot2_bf16(q[hh][w], kr[st][w], a);
        a = group_sum<LPK>(a);
        tsc[st][hh] = valid ? a * scale_log2 : -INFINITY;
      }
    }
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int off = lane_off + ((rd + 1) * NS + st) * KPP * D * 2;
      kr[st] = __builtin_bit_cast(u32x4_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kDecNT));
    }
    // keep the refills here: the scheduler would otherwise sink them next to
    // their use a round later and expose the memory latency
    __builtin_amdgcn_sched_barrier(0);
    // Lazy running max, once per round and without a branch: m moves only
    // when the round's max exceeds it by more than 2^8.
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      float mx = tsc[0][hh];
#pragma unroll
      for (int st = 1; st < NS; ++st) mx = fmaxf(mx, tsc[st][hh]);
      const bool need = mx > m[hh] + kDecLazy;
      const float alpha = need ? __builtin_amdgcn_exp2f(m[hh] - mx) : 1.f;
      m[hh] = need ? mx : m[hh];
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
    }
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      float vf[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vf[2 * w] = bf16_lo(vr[st][w]);
        vf[2 * w + 1] = bf16_hi(vr[st][w]);
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        const float mref = m[hh] == -INFINITY ? 0.f : m[hh];
        const float pr = __builtin_amdgcn_exp2f(tsc[st][hh] - mref);
        l[hh] += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = __builtin_fmaf(pr, vf[e], acc[hh][e]);
      }
    }
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int off = lane_off + ((rd + 1) * NS + st) * KPP * D * 2;
      vr[st] = __builtin_bit_cast(u32x4_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kDecNT));
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  slice_epilogue<D, GM>(m, l, acc, s_m, s_acc, s_l, tid, b, H, h0, nh, s,
                        n_splits, Opart, Lpart, O);
}

// Split-KV decode over a paged KV cache (vllm_mlx.attention: a
// (num_blocks, block_size, num_kv_heads, head_size) cache, per-sequence block
// tables and seq_lens).  Same work decomposition, key slicing, ring of loads
// and merge as the contiguous kernel; only the addressing differs: token t of
// sequence b sits in physical block tables[b][t / block_size] at slot
// t % block_size, and one key row of one KV head is D contiguous bf16 inside
// a token's (Hkv, D) row.  Block-table entries are fetched one round ahead of
// the K/V loads that need them, so the gather adds no dependent latency to the
// ring.  Keys past the slice read block 0 (always in bounds) and are masked:
// their score is -inf and their V chunk is replaced by zeros, so neither
// padding nor stale cache contents can reach the result.  Table entries are
// clamped to [0, num_blocks) so a corrupt table cannot address outside the
// cache.
template <int D, int GM, bool WAVE_BLOCK>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4)))
void attn_decode_paged_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc,
    const __bf16* __restrict__ Vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lengths, float* __restrict__ Opart,
    float* __restrict__ Lpart, __bf16* __restrict__ O, int B, int H, int Hkv,
    int num_blocks, int bs_log2, int max_blocks, int n_splits, int n_hchunks,
    float scale_log2) {
  constexpr int LPK = D / 8;
  constexpr int KPP = kDecThreads / LPK;
  constexpr int NS = kDecStages;

  __shared__ int s_b;
  __shared__ float s_m[4][GM];
  __shared__ float s_acc[4][GM][D];
  __shared__ float s_l[4][GM];

  const int tid = threadIdx.x;
  const int li = tid % LPK;
  const int gi = tid / LPK;

  const int lid = blockIdx.x;
  const int s = lid % n_splits;
  int t = lid / n_splits;
  const int hc = t % n_hchunks;
  t /= n_hchunks;
  const int g = t % Hkv;
  const int rank = t / Hkv;
  const int b = batch_of_rank(lengths, B, rank, tid, s_b);

  const int cap = max_blocks << bs_log2;
  const int len = min(max(lengths[b], 0), cap);
  int k_begin, k_end;
  split_range(len, n_splits, s, &k_begin, &k_end);

  const int G = H / Hkv;
  const int h0 = g * G + hc * GM;
  const int nh = min(GM, G - hc * GM);

  uint32_t q[GM][4];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    const int hq = h0 + (hh < nh ? hh : 0);
    const u32x4_t a = *(const u32x4_t*)(Q + ((size_t)b * H + hq) * D + li * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) q[hh][w] = a[w];
  }

  float m[GM], l[GM], acc[GM][8];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  }

  const int32_t* trow = tables + (size_t)b * max_blocks;
  const int token_row = Hkv * D;                 // elements per cache token
  const size_t block_elems = (size_t)token_row << bs_log2;
  const int head_off = g * D + li * 8;
  const int slot_mask = (1 << bs_log2) - 1;
  const int nkeys = k_end - k_begin;
  const int npass = (nkeys + KPP - 1) / KPP;
  const int nround = (npass + NS - 1) / NS;
  // The keys of one wave in one pass are KPW consecutive keys starting at a
  // multiple of KPW (slices start at multiples of 64).  With WAVE_BLOCK
  // (block_size >= KPW) they share one cache block, so the block-table entry
  // is wave-uniform: a scalar load, and the block base a scalar address.
  constexpr int KPW = 64 / LPK;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto key_of = [&](int rd, int st) { return k_begin + (rd * NS + st) * KPP + gi; };
  auto wave_key = [&](int rd, int st) {
    return k_begin + (rd * NS + st) * KPP + wave * KPW;
  };
  auto table_entry = [&](int rd, int st) {
    const int key = WAVE_BLOCK ? wave_key(rd, st) : key_of(rd, st);
    return trow[key < k_end ? key >> bs_log2 : 0];
  };
  // Address of this lane's 16-byte chunk of key (rd, st) in `cache`, whose
  // block-table entry is `entry`; keys past the slice read block 0.  With
  // WAVE_BLOCK the block base is wave-uniform (a scalar 64-bit address) and
  // the lane adds a 32-bit byte offset.
  auto chunk = [&](const __bf16* cache, int rd, int st, int entry) {
    const int key = key_of(rd, st);
    const int lead = WAVE_BLOCK ? wave_key(rd, st) : key;
    const int phys = lead < k_end ? min(max(entry, 0), num_blocks - 1) : 0;
    const char* base = (const char*)(cache + (size_t)phys * block_elems);
    const uint32_t off = (uint32_t)((key & slot_mask) * token_row + head_off) * 2u;
    return __builtin_nontemporal_load((const u32x4_t*)(base + off));
  };

  // tcur: table entries of the keys loaded in this round (round rd + 1);
  // tnext: those of round rd + 2, requested at the top of the round.
  int tcur[NS], tnext[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) tcur[st] = table_entry(0, st);
  u32x4_t kr[NS], vr[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) kr[st] = vr[st] = u32x4_t{0, 0, 0, 0};

  for (int rd = -1; rd < nround; ++rd) {
#pragma unroll
    for (int st = 0; st < NS; ++st) tnext[st] = table_entry(rd + 2, st);
    float tsc[NS][GM];
    bool valid[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      valid[st] = rd >= 0 && (rd * NS + st) * KPP + gi < nkeys;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) a = dot2_bf16(q[hh][w], kr[st][w], a);
        a = group_sum<LPK>(a);
        tsc[st][hh] = valid[st] ? a * scale_log2 : -INFINITY;
      }
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
      kr[st] = chunk(Kc, rd + 1, st, tcur[st]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      float mx = tsc[0][hh];
#pragma unroll
      for (int st = 1; st < NS; ++st) mx = fmaxf(mx, tsc[st][hh]);
      const bool need = mx > m[hh] + kDecLazy;
      const float alpha = need ? __builtin_amdgcn_exp2f(m[hh] - mx) : 1.f;
      m[hh] = need ? mx : m[hh];
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
    }
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      float vf[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = valid[st] ? vr[st][w] : 0u;
        vf[2 * w] = bf16_lo(x);
        vf[2 * w + 1] = bf16_hi(x);
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        const float mref = m[hh] == -INFINITY ? 0.f : m[hh];
        const float pr = __builtin_amdgcn_exp2f(tsc[st][hh] - mref);
        l[hh] += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = __builtin_fmaf(pr, vf[e], acc[hh][e]);
      }
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
      vr[st] = chunk(Vc, rd + 1, st, tcur[st]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NS; ++st) tcur[st] = tnext[st];
  }

  slice_epilogue<D, GM>(m, l, acc, s_m, s_acc, s_l, tid, b, H, h0, nh, s,
                        n_splits, Opart, Lpart, O);
}

// One wave per (sequence, head): O = sum_s w_s O_s / sum_s w_s with
// w_s = 2^(L_s - max L) (L_s in base-2 units); O = 0 when every slice is empty.
// Every slice writes its partial row (zeros and L = -inf when it is empty),
// so an empty slice enters with w_s = 2^-inf = 0.  The kernel is bound by
// load latency, not bytes: the slice maxima come from one load per lane and
// a butterfly, and the partial rows of kMergeBatch slices are all loaded
// before the first of them is used.
constexpr int kMergeBatch = 8;

template <int D>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(
    const float* __restrict__ Opart, const float* __restrict__ Lpart,
    __bf16* __restrict__ O, int BH, int n_splits) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (bh >= BH) return;
  const float* lp = Lpart + (size_t)bh * n_splits;
  const float* op = Opart + (size_t)bh * n_splits * D + lane;
  float M = -INFINITY;
  for (int s = lane; s < n_splits; s += 64) M = fmaxf(M, lp[s]);
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < n_splits; s0 += kMergeBatch) {
      float ls[kMergeBatch], x[kMergeBatch][PER];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int s = min(s0 + u, n_splits - 1);  // past the end: weight 0
        ls[u] = s0 + u < n_splits ? lp[s] : -INFINITY;
#pragma unroll
        for (int e = 0; e < PER; ++e) x[u][e] = op[(size_t)s * D + 64 * e];
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float w = __builtin_amdgcn_exp2f(ls[u] - M);
        wsum += w;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(w, x[u][e], o[e]);
      }
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
  if (log_enabled())
    log_line("  attn_decode_split_kernel<D=%d, GM=%d> grid=%lld threads=%d", D, GM, grid,
             kDecThreads);
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
  else  // larger groups run as chunks of four heads (an eight-head chunk spills)
    e = launch_split<D, 4>(Q, K, V, lengths, Opart, Lpart, O, B, H, Hkv, Smax, n_splits, stream);
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

template <int D, int GM, bool WAVE_BLOCK>
static hipError_t launch_paged_split(const void* Q, const void* Kc,
                                     const void* Vc, const int32_t* tables,
                                     const int32_t* lengths, float* Opart,
                                     float* Lpart, void* O, int B, int H,
                                     int Hkv, int num_blocks, int bs_log2,
                                     int max_blocks, int n_splits,
                                     hipStream_t stream) {
  const int G = H / Hkv;
  const int n_hchunks = (G + GM - 1) / GM;
  const long long grid = (long long)B * Hkv * n_hchunks * n_splits;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  if (log_enabled())
    log_line("  attn_decode_paged_kernel<D=%d, GM=%d, WAVE_BLOCK=%d> grid=%lld threads=%d", D,
             GM, (int)WAVE_BLOCK, grid, kDecThreads);
  hipLaunchKernelGGL((attn_decode_paged_kernel<D, GM, WAVE_BLOCK>), dim3((unsigned)grid),
                     dim3(kDecThreads), 0, stream, (const __bf16*)Q,
                     (const __bf16*)Kc, (const __bf16*)Vc, tables, lengths,
                     Opart, Lpart, (__bf16*)O, B, H, Hkv, num_blocks, bs_log2,
                     max_blocks, n_splits, n_hchunks, scale_log2);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_paged_d(void* O, const void* Q, const void* Kc,
                                 const void* Vc, const int32_t* tables,
                                 const int32_t* lengths, int n_splits, int B,
                                 int H, int Hkv, int num_blocks, int bs_log2,
                                 int max_blocks, void* ws, hipStream_t stream) {
  const size_t bhs = (size_t)B * H * n_splits;
  float* Opart = (float*)ws;
  float* Lpart =
      (float*)((char*)ws + (bhs * D * sizeof(float) + 255) / 256 * 256);
  const int G = H / Hkv;
  hipError_t e;
  // One wave covers 64 / (D / 8) consecutive keys per pass; when a cache
  // block holds at least that many, the block lookup is wave-uniform.
  // At most four query heads per workgroup (two with per-lane lookups): more
  // would push the kernel past the 128 registers of four waves per SIMD;
  // larger groups run as several head chunks that read the same K/V through L2.
  const bool wave_block = (1 << bs_log2) >= 64 / (D / 8);
#define ATTN_PAGED(GM, WB)                                                     \
  launch_paged_split<D, GM, WB>(Q, Kc, Vc, tables, lengths, Opart, Lpart, O,  \
                                B, H, Hkv, num_blocks, bs_log2, max_blocks,   \
                                n_splits, stream)
  if (G <= 1) e = wave_block ? ATTN_PAGED(1, true) : ATTN_PAGED(1, false);
  else if (G <= 2 || !wave_block)
    e = wave_block ? ATTN_PAGED(2, true) : ATTN_PAGED(2, false);
  else e = ATTN_PAGED(4, true);
#undef ATTN_PAGED
  if (e != hipSuccess || n_splits == 1) return e;
  const int BH = B * H;
  hipLaunchKernelGGL(attn_decode_merge_kernel<D>, dim3((BH + 3) / 4), dim3(256),
                     0, stream, (const float*)Opart, (const float*)Lpart,
                     (__bf16*)O, BH, n_splits);
  return hipGetLastError();
}

hipError_t launch_decode_paged(void* O, const void* Q, const void* Kc,
                               const void* Vc, const int32_t* tables,
                               const int32_t* lengths, int n_splits, int B,
                               int H, int Hkv, int num_blocks, int bs_log2,
                               int max_blocks, int D, void* ws,
                               hipStream_t stream) {
  if (D == 64)
    return launch_paged_d<64>(O, Q, Kc, Vc, tables, lengths, n_splits, B, H,
                              Hkv, num_blocks, bs_log2, max_blocks, ws, stream);
  return launch_paged_d<128>(O, Q, Kc, Vc, tables, lengths, n_splits, B, H,
                             Hkv, num_blocks, bs_log2, max_blocks, ws, stream);
}

}  // namespace attn
