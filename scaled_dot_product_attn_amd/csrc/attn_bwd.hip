// Backward of the bf16 attention forward on gfx950 (MI355X).
//
// Tylo.jl "Primitives", ∇attention!: from the output gradient dO, the primals
// Q, K, V, the forward output O and its saved softmax statistics (here the row
// LSE), the input gradients.  With S = scale * Q K^T + mask, P = exp(S - LSE):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),  delta_i = sum_d dO O,
//   dQ = scale * dS K,  dK = scale * dS^T Q
// (delta_i equals sum_j P_ij dP_ij because O = P V).  With GQA a KV head's
// dK / dV sum over the query heads of its group.
//
// Three kernels:
//   attn_bwd_delta_kernel  delta and the base-2 LSE per query row (HBM-bound);
//   attn_bwd_dkdv8_kernel  one workgroup per (128-key tile, KV head, batch),
//                          eight waves: two per 32 keys, each taking one
//                          32-row half of every 64-row query tile; it walks
//                          every query head of the group and every query tile
//                          that can see its keys, keeping partial dK^T and
//                          dV^T in registers (summed through LDS at the end);
//   attn_bwd_dq_kernel     one workgroup per (128-row query tile, head,
//                          batch), one wave per 32 rows, walking the 32-key
//                          tiles its rows can see (the forward's structure),
//                          two workgroups per compute unit.
// Both stage their LDS tiles with direct global-to-LDS loads.
// dQ is computed by its own kernel rather than by atomics from the dK/dV
// kernel: it costs two more contractions per pair but no read-modify-write
// traffic and gives deterministic results.
//
// Contractions on v_mfma_f32_32x32x16_bf16 with the forward's conventions:
// A operands are rows read from LDS, B operands are per-lane registers or
// rows read from LDS, and a product whose result feeds the next contraction
// as a B operand is formed transposed so that the accumulator already has the
// B layout.  The A
// operands of those second contractions (dO^T, Q^T, K^T) are transposing LDS
// reads (ds_read_b64_tr_b16) of the row-major tiles, which deliver the inner
// index in the permuted order the accumulator registers hold it in; no
// transposed copy is staged.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.h"
#include "attn_host.h"

namespace attn {

namespace bwd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;      // four waves (dQ)
constexpr int kKeysPerWave = 32;
constexpr int kKvTile = 128;       // keys per dK/dV workgroup
constexpr int kQTile = 64;         // query rows per step of the dK/dV kernel
constexpr int kDqRows = 128;       // query rows per dQ workgroup
constexpr int kDqKeys = 32;        // keys per step of the dQ kernel
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, out-of-range reads = 0

// Direct global-to-LDS 16-byte load issued from inline assembly: lane l of
// the wave fills the 16 bytes at LDS address lds_addr + 16 l from byte
// voffset of the buffer.  With the compiler's builtin for this instruction the
// compiler, which cannot tell these LDS writes from the kernel's LDS reads,
// waits for every outstanding load before the next LDS read, i.e. for the
// whole next stage in the middle of a step; here the kernels wait themselves,
// before the barrier that publishes the stage.  Five wait states first: the
// descriptor may have just been written by a vector instruction, which a
// memory instruction may read only five wait states later, and no wait is
// inserted before an instruction inside inline assembly (M0, written just
// before, needs one).
__device__ inline void lds_load16(u32x4_t rsrc, uint32_t lds_addr, int voffset) {
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "{m0}"(lds_addr)
      : "memory");
}

// A raw buffer descriptor (no stride, num_records bytes, out-of-range reads
// return zero) in four scalar registers, for lds_load16.
__device__ inline u32x4_t buffer_desc_s(const void* base, int num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4_t d;
  d[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
  d[2] = __builtin_amdgcn_readfirstlane((uint32_t)num_records);
  d[3] = (uint32_t)kRsrcWord3;
  return d;
}

__device__ inline uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
#ifndef KBWD_OP_DEPTH
#define KBWD_OP_DEPTH 4
#endif
constexpr int kBwdOpDepth = KBWD_OP_DEPTH;  // LDS operand reads in flight per wave
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// Tiles in LDS are row-major, rows of D bf16 unpadded, with the 16-byte
// chunk c of row r stored at chunk c ^ bwd_swizzle<D>(r).  The swizzle keeps
// both read patterns free of bank conflicts: 16 lanes reading one chunk of 16
// consecutive rows (row operands), and 32 lanes of a transposing read covering
// 4 consecutive rows (from a multiple of 4) x 4 aligned consecutive chunks.
// D = 128: a bijection of r % 16 whose values for 4 consecutive rows differ
// in bits 2-3.  D = 64 (8 chunks, two rows per 256 bytes): a bijection on the
// rows of one parity whose bit 2 differs for rows r and r + 2.
template <int D>
__device__ inline int bwd_swizzle(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// A operand (32 rows x 16 k) of the transpose of a row-major tile: rows are
// d = 32 db + (l % 32), the k-slice of lane l is tile rows 16 ks + 4 (l / 32)
// + {0..3} and 16 ks + 8 + 4 (l / 32) + {0..3} (the permuted order in which
// an accumulator holds its rows).  Two ds_read_b64_tr_b16: within 16 lanes,
// lane i points at 4 d-values of tile row kb + i / 4 and lane j receives
// d-value j of tile rows kb .. kb + 3.
template <int D>
__device__ inline bf16x8_t tr_operand(const char* tile, int row_bytes, int ks, int db, int lane) {
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  const int grp = lane >> 4, j = lane & 15;
  const int d = db * 32 + (grp & 1) * 16 + (j & 3) * 4;
  i16x4_t part[2];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int r = ks * 16 + h8 * 8 + (grp >> 1) * 4 + (j >> 2);
    const char* a = tile + r * row_bytes + (((d >> 3) ^ bwd_swizzle<D>(r)) << 4) + (d & 7) * 2;
    part[h8] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)a);
  }
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace bwd

using namespace bwd;

// ---------------------------------------------------------------------------
// delta_i = sum_d dO_id O_id and L2_i = LSE_i * log2(e) (+inf for a row with
// no allowed key, so that exp2(s - L2) = 0 there)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(
    const __bf16* __restrict__ dO, const __bf16* __restrict__ O,
    const float* __restrict__ LSE, float* __restrict__ delta,
    float* __restrict__ L2, long long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 d each
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4_t a = *(const u32x4_t*)(dO + row * D + c * 8);
    const u32x4_t o = *(const u32x4_t*)(O + row * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += __uint_as_float(a[w] << 16) * __uint_as_float(o[w] << 16);
      acc += __uint_as_float(a[w] & 0xffff0000u) * __uint_as_float(o[w] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int x = 1; x < TPR; x <<= 1) acc += __shfl_xor(acc, x);
  if (row < rows && c == 0) {
    delta[row] = acc;
    const float l = LSE[row];
    L2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV with eight waves: the two waves on a SIMD share a 32-key block and
// take the two 32-row halves of every 64-row query tile, each accumulating a
// partial dK^T and dV^T that are summed through LDS at the end.  K and V of
// the workgroup's 128 keys stay in LDS and are read as B operands, so a wave
// holds its two accumulators, one 32 x 32 S/dP pair and its operands in
// fewer than 256 registers and two waves share each SIMD.
// ---------------------------------------------------------------------------
constexpr int kThreads8 = 512;

template <int D>
struct Dkdv8Lds {
  static constexpr int kRow = D * 2;
  static constexpr int kOffK = 0;                   // K rows of the key tile
  static constexpr int kOffV = kKvTile * kRow;      // V rows of the key tile
  static constexpr int kOffStage = 2 * kKvTile * kRow;
  // per stage: Q, dO, L2 and delta of one 64-row query tile
  static constexpr int kOffQ = 0;
  static constexpr int kOffO = kQTile * kRow;
  static constexpr int kOffL = 2 * kQTile * kRow;
  static constexpr int kOffDel = kOffL + kQTile * 4;
  static constexpr int kStage = kOffDel + kQTile * 4;
  static constexpr int kTotal = kOffStage + 2 * kStage;
  // final reduction: per key block the partial dK^T and dV^T of the
  // second-half wave, 16 DBLK floats per lane, aliasing everything above
  static constexpr int kRed = 4 * 2 * 64 * 16 * (D / 32) * 4;
  static_assert(kRed <= kTotal, "reduction area fits");
};

template <int D>
__global__ __launch_bounds__(kThreads8) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv8_kernel(
    __bf16* __restrict__ dK, __bf16* __restrict__ dV,
    const __bf16* __restrict__ dO, const __bf16* __restrict__ Q,
    const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const float* __restrict__ delta, const float* __restrict__ L2,
    int B, int H, int Hkv, int Sq, int Sk, int causal, int window,
    int input_pos, const int32_t* __restrict__ k_lengths, float scale) {
  using L = Dkdv8Lds<D>;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int kb = wave & 3;     // 32-key block of the tile
  const int qh = wave >> 2;    // which 32-row half of each query tile
  const int lcol = lane & 31;  // key column this lane owns
  const int half = lane >> 5;

  const int kt = blockIdx.x;  // low keys (the most rows under causal masking) first
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int G = H / Hkv;
  const int j0 = kt * kKvTile;
  const int j1 = min(j0 + kKvTile, Sk);
  const int kl = k_lengths ? min(max(k_lengths[b], 0), Sk) : Sk;
  const int kj = j0 + kb * kKeysPerWave + lcol;  // this lane's key

  // the tile's K and V rows into LDS (direct loads, swizzled; keys past Sk read zeros)
  {
    const size_t kvb = ((size_t)(b * Hkv + g) * Sk + j0) * D;
    const int nbytes = (Sk - j0) * D * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(K + kvb), (short)0, nbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(V + kvb), (short)0, nbytes, kRsrcWord3);
    constexpr int NKV = kKvTile * CPR / kThreads8;
#pragma unroll
    for (int n = 0; n < NKV; ++n) {
      const int slot = (n * 8 + wave_u) * 64 + lane;
      const int r = slot / CPR;
      const int c = (slot % CPR) ^ bwd_swizzle<D>(r);
      const int off = (r * D + c * 8) * 2;
      const int at = (n * 8 + wave_u) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krs, (__attribute__((address_space(3))) void*)(smem + L::kOffK + at), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrs, (__attribute__((address_space(3))) void*)(smem + L::kOffV + at), 16, off, 0, 0, 0);
    }
  }

  f32x16_t dkT[DBLK], dvT[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dkT[db] = dvT[db] = f32x16_t{};

  // query rows that may see keys [j0, min(j1, kl)): causal needs p >= j0, a
  // window needs p - window + 1 <= j_last
  int i_lo = 0, i_hi = Sq;
  const int jl = min(j1, kl);
  if (jl <= j0) i_hi = 0;
  if (causal) i_lo = max(i_lo, j0 - input_pos);
  if (window > 0) i_hi = min(i_hi, (int)min((long long)jl - 1 + window - input_pos, (long long)Sq));
  i_lo = max(i_lo, 0);
  const int qt_lo = i_lo / kQTile;
  const int qt_hi = i_hi > i_lo ? (i_hi + kQTile - 1) / kQTile : qt_lo;
  const int nq = qt_hi - qt_lo;
  const int n_items = nq * G;

  // staging: the Q and dO rows of a tile go from global memory straight into
  // LDS (buffer_load ... lds: lane l of an instruction fills the 16 bytes at
  // the wave's LDS address + 16 l, from any global address), so a stage costs
  // no registers and no wait until the barrier that publishes it.  LDS slot s
  // (in 16-byte chunks) of a tensor is written by instruction s / 512, wave
  // (s / 64) % 8, lane s % 64, and holds row s / CPR at chunk s % CPR: the
  // lane loads the logical chunk that the swizzle puts there.  Rows past Sq
  // read zeros through the resource's range check.  L2 and delta (64 floats
  // each) come the same way, by 16 lanes of the last wave; rows past Sq read
  // zeros there too, and contribute nothing (their Q and dO rows are zero, so
  // dP = 0, dS = P (0 - 0) = 0 and dO^T P = 0).
  constexpr int NCH = kQTile * CPR / kThreads8;
  static_assert(NCH * kThreads8 == kQTile * CPR, "whole tiles per stage");
  auto advance = [&](int& hh, int& q) {
    if (++q == nq) {
      q = 0;
      ++hh;
    }
  };
  auto fetch = [&](int hh, int q, int buf) {
    const int h = g * G + hh;
    const int i0 = (qt_lo + q) * kQTile;
    const size_t rb = (size_t)(b * H + h) * Sq;
    const u32x4_t qrs = buffer_desc_s(Q + rb * D, Sq * D * 2);
    const u32x4_t ors = buffer_desc_s(dO + rb * D, Sq * D * 2);
    char* st = smem + L::kOffStage + buf * L::kStage;
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int slot = (n * 8 + wave_u) * 64 + lane;
      const int r = slot / CPR;
      const int c = (slot % CPR) ^ bwd_swizzle<D>(r);
      const int off = ((i0 + r) * D + c * 8) * 2;
      const int at = (n * 8 + wave_u) * 1024;
      lds_load16(qrs, lds_addr_of(st + L::kOffQ + at), off);
      lds_load16(ors, lds_addr_of(st + L::kOffO + at), off);
    }
    if (wave_u == kThreads8 / 64 - 1 && lane < kQTile / 4) {
      const u32x4_t lrs = buffer_desc_s(L2 + rb, Sq * 4);
      const u32x4_t drs = buffer_desc_s(delta + rb, Sq * 4);
      lds_load16(lrs, lds_addr_of(st + L::kOffL), (i0 + lane * 4) * 4);
      lds_load16(drs, lds_addr_of(st + L::kOffDel), (i0 + lane * 4) * 4);
    }
  };
  // this thread's loads of the stage complete (the barrier that follows
  // publishes it)
  auto stash = [&](int) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  const float sl2 = scale * kLog2e;
  if (n_items > 0) fetch(0, 0, 0);
  stash(0);  // also completes the K/V tile loads
  __syncthreads();
  // query rows my key may be seen by: [r_lo, r_hi) (none past k_lengths)
  int r_lo = 0, r_hi = 0;
  if (kj < kl) {
    const long long lo = causal ? (long long)kj - input_pos : 0;            // p >= j
    const long long hi = window > 0 ? (long long)kj + window - input_pos : Sq;  // p < j + w
    r_lo = clamp_i64(lo, 0, Sq);
    r_hi = clamp_i64(hi, 0, Sq);
  }
  const unsigned r_width = (unsigned)max(r_hi - r_lo, 0);
  const char* krow = smem + L::kOffK + (kb * 32 + lcol) * L::kRow;
  const char* vrow = smem + L::kOffV + (kb * 32 + lcol) * L::kRow;
  const int ksw = bwd_swizzle<D>(kb * 32 + lcol);

  int cur_hh = 0, cur_q = 0;  // the item of iteration it
  for (int it = 0; it < n_items; ++it) {
    const char* st = smem + L::kOffStage + (it & 1) * L::kStage;
    const int i0 = (qt_lo + cur_q) * kQTile;
    int nxt_hh = cur_hh, nxt_q = cur_q;
    advance(nxt_hh, nxt_q);
    const int i1 = min(i0 + kQTile, Sq);
    const RowRange first = row_range(i0, kl, causal, window, input_pos);
    const RowRange last = row_range(i1 - 1, kl, causal, window, input_pos);
    const bool partial =
        i1 - i0 < kQTile || !(last.lo <= j0 && j0 + kKvTile <= first.hi);

    // S and dP (this wave's 32 queries x its 32 keys): operand pair i: k-step
    // i / 2, (Q row, K row) for even i and (dO row, V row) for odd i
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
    {
      constexpr int NOP = 2 * KSTEPS;
      const int qr = qh * 32 + lcol;
      const int qsw = bwd_swizzle<D>(qr);
      auto opa = [&](int i) -> bf16x8_t {
        const int ks = i / 2;
        const int off = (i & 1) ? L::kOffO : L::kOffQ;
        return *(const bf16x8_t*)(st + off + qr * L::kRow + (((2 * ks + half) ^ qsw) << 4));
      };
      auto opb = [&](int i) -> bf16x8_t {
        const int ks = i / 2;
        return *(const bf16x8_t*)(((i & 1) ? vrow : krow) + (((2 * ks + half) ^ ksw) << 4));
      };
      bf16x8_t ra[kBwdOpDepth], rb[kBwdOpDepth];
#pragma unroll
      for (int i = 0; i < kBwdOpDepth; ++i) {
        ra[i] = opa(i);
        rb[i] = opb(i);
      }
#pragma unroll
      for (int i = 0; i < NOP; ++i) {
        const bf16x8_t a = ra[i % kBwdOpDepth], bb = rb[i % kBwdOpDepth];
        if (i + kBwdOpDepth < NOP) {
          ra[i % kBwdOpDepth] = opa(i + kBwdOpDepth);
          rb[i % kBwdOpDepth] = opb(i + kBwdOpDepth);
        }
        if (i & 1)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, dp, 0, 0, 0);
        else
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, s, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kBwdOpDepth, 0);
#pragma unroll
      for (int i = 0; i < NOP - kBwdOpDepth; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kBwdOpDepth, 0);
    }
    // P = exp2(s * scale * log2e - L2), dS = P (dP - delta); lane's queries are
    // i0 + 32 qh + 8*(r/4) + 4*half + r%4
    u32x4_t pk[2], dsk[2];  // packed bf16, one 16-query k-step each
    // (a separate copy for the steps that mask, so that the others carry no
    // compare and select per element)
    auto p_and_ds = [&](auto masked) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qo = qh * 32 + r4 * 8 + half * 4;
        const f32x4_t l4 = *(const f32x4_t*)(st + L::kOffL + qo * 4);
        const f32x4_t d4 = *(const f32x4_t*)(st + L::kOffDel + qo * 4);
        const int t0 = i0 + qo - r_lo;
        float pv[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = r4 * 4 + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -l4[e]));
          if constexpr (decltype(masked)::value) p = (unsigned)(t0 + e) < r_width ? p : 0.f;
          pv[e] = p;
          dv[e] = p * (dp[r] - d4[e]);
        }
        const int kq = r4 >> 1;
        const int w = (r4 & 1) * 2;
        pk[kq][w] = pack_bf16x2(pv[0], pv[1]);
        pk[kq][w + 1] = pack_bf16x2(pv[2], pv[3]);
        dsk[kq][w] = pack_bf16x2(dv[0], dv[1]);
        dsk[kq][w + 1] = pack_bf16x2(dv[2], dv[3]);
      }
    };
    if (partial)
      p_and_ds(std::true_type{});
    else
      p_and_ds(std::false_type{});
    // the next tile's rows stream into the other stage during the rest
    if (it + 1 < n_items) fetch(nxt_hh, nxt_q, (it + 1) & 1);
    // dV^T += dO^T P, dK^T += Q^T dS (d x keys), k over this wave's 32
    // queries: operand i: d block i / 4, query k-step (i / 2) % 2, dO^T for
    // even i and Q^T for odd i (transposing reads of the half's rows)
    {
      constexpr int NOP = DBLK * 4;
      auto op = [&](int i) -> bf16x8_t {
        const int db = i / 4, kq = (i / 2) % 2;
        const int off = (i & 1) ? L::kOffQ : L::kOffO;
        return tr_operand<D>(st + off + qh * 32 * L::kRow, L::kRow, kq, db, lane);
      };
      bf16x8_t ring[kBwdOpDepth];
#pragma unroll
      for (int i = 0; i < kBwdOpDepth; ++i) ring[i] = op(i);
#pragma unroll
      for (int i = 0; i < NOP; ++i) {
        const bf16x8_t a = ring[i % kBwdOpDepth];
        if (i + kBwdOpDepth < NOP) ring[i % kBwdOpDepth] = op(i + kBwdOpDepth);
        const int db = i / 4, kq = (i / 2) % 2;
        if (i & 1)
          dkT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, __builtin_bit_cast(bf16x8_t, dsk[kq]), dkT[db], 0, 0, 0);
        else
          dvT[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, __builtin_bit_cast(bf16x8_t, pk[kq]), dvT[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kBwdOpDepth, 0);
#pragma unroll
      for (int i = 0; i < NOP - kBwdOpDepth; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kBwdOpDepth, 0);
    }
    if (it + 1 < n_items) stash((it + 1) & 1);
    __syncthreads();
    cur_hh = nxt_hh;
    cur_q = nxt_q;
  }

  // ---- the second-half waves hand their partial sums to the first-half ones ----
  // (every LDS read of the loop is behind its closing barrier)
  f32x4_t* red = (f32x4_t*)smem + (kb * 2) * (DBLK * 4) * 64 + lane;
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        red[(db * 4 + q4) * 64] = f32x4_t{dkT[db][q4 * 4], dkT[db][q4 * 4 + 1],
                                          dkT[db][q4 * 4 + 2], dkT[db][q4 * 4 + 3]};
        red[(DBLK * 4 + db * 4 + q4) * 64] = f32x4_t{dvT[db][q4 * 4], dvT[db][q4 * 4 + 1],
                                                     dvT[db][q4 * 4 + 2], dvT[db][q4 * 4 + 3]};
      }
  }
  __syncthreads();
  if (qh == 1) return;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4_t a = red[(db * 4 + q4) * 64];
      const f32x4_t c = red[(DBLK * 4 + db * 4 + q4) * 64];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dkT[db][q4 * 4 + e] += a[e];
        dvT[db][q4 * 4 + e] += c[e];
      }
    }

  // ---- store: lane owns key kj, holds d = db*32 + 8*(r/4) + 4*half + r%4 ----
  if (kj < Sk) {
    const size_t base = ((size_t)(b * Hkv + g) * Sk + kj) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + half * 4;
        u32x2_t wk = {pack_bf16x2(dkT[db][r4 * 4] * scale, dkT[db][r4 * 4 + 1] * scale),
                      pack_bf16x2(dkT[db][r4 * 4 + 2] * scale, dkT[db][r4 * 4 + 3] * scale)};
        u32x2_t wv = {pack_bf16x2(dvT[db][r4 * 4], dvT[db][r4 * 4 + 1]),
                      pack_bf16x2(dvT[db][r4 * 4 + 2], dvT[db][r4 * 4 + 3])};
        *(u32x2_t*)(dK + base + d) = wk;
        *(u32x2_t*)(dV + base + d) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (128-row query tile, head, batch)
// ---------------------------------------------------------------------------
// Per stage the K and V rows of one kDqKeys-key tile, unpadded and swizzled
// (bwd_swizzle); K^T operands of dQ are transposing reads of the K rows.
template <int D>
struct DqLds {
  static constexpr int kRow = D * 2;
  static constexpr int kOffK = 0;
  static constexpr int kOffV = kDqKeys * kRow;
  static constexpr int kStage = 2 * kDqKeys * kRow;
  static constexpr int kTotal = 2 * kStage;
};

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(
    __bf16* __restrict__ dQ, const __bf16* __restrict__ dO,
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, const float* __restrict__ delta,
    const float* __restrict__ L2, int B, int H, int Hkv, int Sq, int Sk,
    int causal, int window, int input_pos, const int32_t* __restrict__ k_lengths,
    float scale) {
  using L = DqLds<D>;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  const int nqt = (Sq + kDqRows - 1) / kDqRows;
  const int qtr = blockIdx.x;
  const int qt = causal ? nqt - 1 - qtr : qtr;  // heaviest first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / (H / Hkv);
  const int i0 = qt * kDqRows;
  const int i1 = min(i0 + kDqRows, Sq);
  const int kl = k_lengths ? min(max(k_lengths[b], 0), Sk) : Sk;
  const KvGeometry geo = kv_geometry(i0, i1, kl, causal, window, input_pos);

  const int qi = i0 + wave * 32 + lrow;
  const RowRange rr = row_range(qi, kl, causal, window, input_pos);
  const size_t rowbase = (size_t)(b * H + h) * Sq;
  bf16x8_t qreg[KSTEPS], oreg[KSTEPS];
  {
    const bool ok = qi < Sq;
    const size_t off = (rowbase + (ok ? qi : 0)) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t q4 = ok ? *(const u32x4_t*)(Q + off + ks * 16) : u32x4_t{0, 0, 0, 0};
      u32x4_t o4 = ok ? *(const u32x4_t*)(dO + off + ks * 16) : u32x4_t{0, 0, 0, 0};
      qreg[ks] = __builtin_bit_cast(bf16x8_t, q4);
      oreg[ks] = __builtin_bit_cast(bf16x8_t, o4);
    }
  }
  const float l2 = qi < Sq ? L2[rowbase + qi] : INFINITY;
  const float del = qi < Sq ? delta[rowbase + qi] : 0.f;

  f32x16_t dqT[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dqT[db] = f32x16_t{};

  int kt_first = 0, kt_last = -1;
  if (geo.any) {
    kt_first = geo.union_lo / kDqKeys;
    kt_last = (geo.union_hi - 1) / kDqKeys;
  }
  const int nvalid = geo.union_hi - geo.union_lo;
  const size_t valid_base = ((size_t)(b * Hkv + g) * Sk + geo.union_lo) * D;
  // staging: K and V rows go from global memory straight into LDS
  // (buffer_load ... lds, as in the dK/dV kernel): slot s of a tensor is
  // written by instruction s / 256, wave (s / 64) % 4, lane s % 64 and holds
  // row s / CPR at chunk s % CPR; keys outside [union_lo, union_hi) read zeros
  constexpr int NCH = kDqKeys * CPR / kThreads;
  static_assert(NCH * kThreads == kDqKeys * CPR, "whole tiles per stage");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const u32x4_t kds = buffer_desc_s(K + valid_base, nvalid * D * 2);
  const u32x4_t vds = buffer_desc_s(V + valid_base, nvalid * D * 2);
  auto fetch = [&](int kt, int buf) {
    const int rel0 = kt * kDqKeys - geo.union_lo;
    char* st = smem + buf * L::kStage;
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int slot = (n * 4 + wave_u) * 64 + lane;
      const int r = slot / CPR;
      const int c = (slot % CPR) ^ bwd_swizzle<D>(r);
      const int off = ((rel0 + r) * D + c * 8) * 2;
      const int at = (n * 4 + wave_u) * 1024;
      lds_load16(kds, lds_addr_of(st + L::kOffK + at), off);
      lds_load16(vds, lds_addr_of(st + L::kOffV + at), off);
    }
  };
  // this thread's direct loads complete (the barrier that follows publishes the stage)
  auto stage_done = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  const float sl2 = scale * kLog2e;
  constexpr int KB = kDqKeys / 32;  // 32-key blocks per step
  if (kt_first <= kt_last) {
    fetch(kt_first, 0);
    stage_done();
    __syncthreads();
  }
  for (int kt = kt_first; kt <= kt_last; ++kt) {
    const int it = kt - kt_first;
    const char* st = smem + (it & 1) * L::kStage;
    const int j0 = kt * kDqKeys;
    // S^T and dP^T (kDqKeys keys x 32 queries) in 32-key blocks; operand i:
    // key block i / (2 KSTEPS), k-step (i / 2) % KSTEPS, K rows for even i and
    // V rows for odd i, through a ring kBwdOpDepth reads ahead of the MFMAs
    f32x16_t s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = dp[kb] = f32x16_t{};
    {
      constexpr int NOP = 2 * KB * KSTEPS;
      auto op = [&](int i) -> const bf16x8_t* {
        const int kb = i / (2 * KSTEPS), ks = (i / 2) % KSTEPS;
        const int off = (i & 1) ? L::kOffV : L::kOffK;
        const int r = kb * 32 + lrow;
        return (const bf16x8_t*)(st + off + r * L::kRow + (((2 * ks + half) ^ bwd_swizzle<D>(r)) << 4));
      };
      bf16x8_t ring[kBwdOpDepth];
#pragma unroll
      for (int i = 0; i < kBwdOpDepth; ++i) ring[i] = *op(i);
#pragma unroll
      for (int i = 0; i < NOP; ++i) {
        const bf16x8_t a = ring[i % kBwdOpDepth];
        if (i + kBwdOpDepth < NOP) ring[i % kBwdOpDepth] = *op(i + kBwdOpDepth);
        const int kb = i / (2 * KSTEPS), ks = (i / 2) % KSTEPS;
        if (i & 1)
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, oreg[ks], dp[kb], 0, 0, 0);
        else
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kBwdOpDepth, 0);
#pragma unroll
      for (int i = 0; i < NOP - kBwdOpDepth; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kBwdOpDepth, 0);
    }
    // the next tile's keys are requested now and land during the rest
    if (kt + 1 <= kt_last) fetch(kt + 1, (it + 1) & 1);
    // lane's keys: j0 + kb*32 + 8*(r/4) + 4*half + r%4
    const bool partial = tile_class(geo, j0, kDqKeys) == kTilePartial;
    const int t_lo = rr.lo - (j0 + half * 4);
    const unsigned width = (unsigned)max(rr.hi - rr.lo, 0);
    u32x4_t dsk[2 * KB];
    // (a separate copy for the tiles that mask)
    auto ds_of = [&](auto masked) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float dv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + e], sl2, -l2));
            if constexpr (decltype(masked)::value) {
              const int c = kb * 32 + ((r + e) >> 2) * 8 + ((r + e) & 3);
              p = (unsigned)(c - t_lo) < width ? p : 0.f;
            }
            dv[e] = p * (dp[kb][r + e] - del);
          }
          dsk[kb * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(dv[0], dv[1]);
        }
    };
    if (partial)
      ds_of(std::true_type{});
    else
      ds_of(std::false_type{});
    // dQ^T (d x queries) += K^T (d x keys) dS^T (keys x queries); operand i:
    // d block i / (2 KB), key k-step i % (2 KB).  K^T comes from the K rows by
    // transposing reads (tr_operand), in the key order dS^T has in the S^T
    // registers.
    {
      constexpr int KST = 2 * KB;
      constexpr int NOP = DBLK * KST;
      auto op = [&](int i) -> bf16x8_t {
        return tr_operand<D>(st + L::kOffK, L::kRow, i % KST, i / KST, lane);
      };
      bf16x8_t ring[kBwdOpDepth];
#pragma unroll
      for (int i = 0; i < kBwdOpDepth; ++i) ring[i] = op(i);
#pragma unroll
      for (int i = 0; i < NOP; ++i) {
        const bf16x8_t a = ring[i % kBwdOpDepth];
        if (i + kBwdOpDepth < NOP) ring[i % kBwdOpDepth] = op(i + kBwdOpDepth);
        dqT[i / KST] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, __builtin_bit_cast(bf16x8_t, dsk[i % KST]), dqT[i / KST], 0, 0, 0);
      }
      // (two transposing reads per operand)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kBwdOpDepth, 0);
#pragma unroll
      for (int i = 0; i < NOP - kBwdOpDepth; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kBwdOpDepth, 0);
    }
    if (kt + 1 <= kt_last) stage_done();
    __syncthreads();
  }

  if (qi < Sq) {
    __bf16* op = dQ + (rowbase + qi) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + half * 4;
        u32x2_t w = {pack_bf16x2(dqT[db][r4 * 4] * scale, dqT[db][r4 * 4 + 1] * scale),
                     pack_bf16x2(dqT[db][r4 * 4 + 2] * scale, dqT[db][r4 * 4 + 3] * scale)};
        *(u32x2_t*)(op + d) = w;
      }
  }
}

size_t bwd_workspace_bytes(int B, int H, int Sq) {
  const size_t rows = (size_t)B * H * Sq;
  return 2 * ((rows * sizeof(float) + 255) / 256 * 256);
}

template <int D>
static hipError_t launch_bwd_d(void* dQ, void* dK, void* dV, const void* dO,
                               const void* Q, const void* K, const void* V,
                               const void* O, const float* LSE, int B, int H,
                               int Hkv, int Sq, int Sk, int causal, int window,
                               int input_pos, const int32_t* k_lengths,
                               void* ws, hipStream_t stream) {
  const long long rows = (long long)B * H * Sq;
  float* delta = (float*)ws;
  float* L2 = (float*)((char*)ws + ((size_t)rows * sizeof(float) + 255) / 256 * 256);
  const float scale = 1.f / sqrtf((float)D);
  constexpr int RPB = 256 / (D / 8);
  hipError_t e = hipSuccess;
  if (rows > 0) {
    hipLaunchKernelGGL(attn_bwd_delta_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(256), 0, stream, (const __bf16*)dO, (const __bf16*)O, LSE,
                       delta, L2, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (Sk > 0) {
    const int nkt = (Sk + kKvTile - 1) / kKvTile;
    if (log_enabled())
      log_line("  attn_bwd_dkdv8_kernel<D=%d> grid=(%d, %d, %d) threads=%d", D, nkt, Hkv, B,
               kThreads8);
    hipLaunchKernelGGL(attn_bwd_dkdv8_kernel<D>, dim3(nkt, Hkv, B), dim3(kThreads8), 0,
                       stream, (__bf16*)dK, (__bf16*)dV, (const __bf16*)dO,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V,
                       (const float*)delta, (const float*)L2, B, H, Hkv, Sq, Sk,
                       causal, window, input_pos, k_lengths, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows == 0) return hipSuccess;
  const int nqt = (Sq + kDqRows - 1) / kDqRows;
  if (log_enabled())
    log_line("  attn_bwd_dq_kernel<D=%d> grid=(%d, %d, %d) threads=%d", D, nqt, H, B, kThreads);
  hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3(nqt, H, B), dim3(kThreads), 0,
                     stream, (__bf16*)dQ, (const __bf16*)dO, (const __bf16*)Q,
                     (const __bf16*)K, (const __bf16*)V, (const float*)delta,
                     (const float*)L2, B, H, Hkv, Sq, Sk, causal, window,
                     input_pos, k_lengths, scale);
  return hipGetLastError();
}

hipError_t launch_bwd(void* dQ, void* dK, void* dV, const void* dO,
                      const void* Q, const void* K, const void* V,
                      const void* O, const float* LSE, int B, int H, int Hkv,
                      int Sq, int Sk, int D, int causal, int window,
                      int input_pos, const int32_t* k_lengths, void* ws,
                      hipStream_t stream) {
  if (D == 64)
    return launch_bwd_d<64>(dQ, dK, dV, dO, Q, K, V, O, LSE, B, H, Hkv, Sq, Sk,
                            causal, window, input_pos, k_lengths, ws, stream);
  return launch_bwd_d<128>(dQ, dK, dV, dO, Q, K, V, O, LSE, B, H, Hkv, Sq, Sk,
                           causal, window, input_pos, k_lengths, ws, stream);
}

}  // namespace attn
