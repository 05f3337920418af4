// Fused attention forward for bf16 Q/K/V/O on gfx950 (MI355X).
//
// O = softmax(scale * Q K^T + mask) V with Float32 accumulation and the row
// logsumexp saved (Tylo.jl "Primitives", attention!: GQA, causal, input_pos,
// k_lengths, checkpoints M/L; flex_attention!: qk_scale = 1/sqrt(Dk), in-kernel
// block skipping for analytic masks; mlx-arsenal "Attention": causal_mask /
// sliding_window_mask with -inf at blocked positions).
//
// Work decomposition
//   One workgroup = 8 waves = 256 query rows of one (batch, head); each wave
//   owns 32 rows.  The workgroup walks the 64-key tiles its rows can see
//   (empty tiles are never visited).
//
// Ping-pong between two wave groups.  Waves 0-3 (group A) and 4-7 (group B)
// sit one per SIMD each, so every SIMD holds one wave of each group.  Each
// wave alternates two phases, separated by workgroup barriers:
//   M-phase k: O += P(k-1) V(k-1) and S(k) = K(k) Q^T   (32 MFMAs)
//   V-phase k: mask and online softmax of S(k) -> P(k), plus staging
// and group B runs one phase behind group A, so while one wave of a SIMD
// feeds the matrix core the other works on the vector ALU.
//
// Staging: K and V^T each have a two-tile LDS ring.  In V-phase k group A
// stores K(k+1) and group B stores V(k+1) (transposed), from registers loaded
// by buffer loads issued one V-phase earlier.  Reads of K(k) happen in the
// M-phases k of both groups, reads of V(k) in the M-phases k+1, so no buffer
// is rewritten while a group may still read it.
//
// Contractions on the matrix cores (v_mfma_f32_32x32x16_bf16), transposed so
// that one lane owns one query row:
//   S^T (32 keys x 32 queries) = K (32 x 16 d) * Q^T (16 d x 32 queries)
//     -> lane l holds query l%32 and 16 of the 32 keys, so the row max and
//        row sum are in-lane reductions plus one exchange with lane l^32.
//   O^T (32 d x 32 queries) += V^T (32 d x 16 keys) * P^T (16 keys x 32 q)
//     -> P^T is the S^T accumulator itself, rounded to bf16: no shuffle.
//   The key order inside V^T's LDS rows is permuted to match the order in
//   which the S^T accumulator registers hold the keys.
//
// Flex variants (FLEX = true; Tylo.jl "Primitives", flex_attention! and its
// mods): the same kernel with the score rewritten before the softmax, in this
// order: qk_scale * s, plus an additive bias tile (BiasScore), plus
// slope_h * (q - kv) (AliBiScore), then cap * tanh(. / cap) (SoftCapScore);
// and the mask extended by a prefix (prefix_lm = CausalMask | PrefixMask),
// per-batch query lengths (q_lengths) and document ids (DocumentMask).  The
// bias tile of a lane's row is loaded at the start of the M-phase that computes
// the tile's scores, document ids of the keys are staged in LDS with K.
//
// Online softmax in base 2: t = s * log2(e) / sqrt(D), p = exp2(t - m).  The
// running max m is only raised when a tile's max exceeds it by more than
// 2^8 (p <= 256 otherwise), so the O rescale is skipped on almost all tiles;
// O / l and m + log2 l are unchanged by which m is used.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "attn_common.h"

#ifndef KFWD_OP_DEPTH
#define KFWD_OP_DEPTH 6
#endif

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kFwdWaves = 8;               // two groups of four
constexpr int kFwdThreads = kFwdWaves * 64;
constexpr int kFwdTileM = kFwdWaves * 32;  // query rows per workgroup
constexpr int kFwdTileN = 64;              // keys per tile
constexpr float kLazyRescale = 8.0f;       // log2 headroom before m is raised
constexpr int kFwdOpDepth = KFWD_OP_DEPTH; // LDS operand reads in flight per wave
// Word 3 of a gfx9-family buffer resource (32-bit data format, no swizzle):
// a raw buffer whose out-of-range reads return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;
static_assert(kFwdTileM == ATTN_FWD_TILE_M && kFwdTileN == ATTN_FWD_TILE_N,
              "the exported tile plan must use the kernel's tile sizes");
// block-sparse prefill: 64 x 64 blocks, at most this many key tiles per row
constexpr int kSparseBlock = 64;
constexpr int kSparseMaxTiles = ATTN_SPARSE_MAX_KEY_BLOCKS;
static_assert(kSparseBlock == kFwdTileN && kFwdTileM % kSparseBlock == 0,
              "a key tile is one block; a workgroup holds whole row blocks");

// Kernel-side copy of attn_flex_t (see include/attn.h); strides in elements.
struct FlexArgs {
  const int32_t* q_lengths;
  const float* alibi;
  const float* bias;
  const int32_t* doc_q;
  const int32_t* doc_kv;
  long long bias_bstride, bias_hstride;
  int prefix;
  float softcap;
  float qk_scale;
};

template <int D>
struct FwdLds {
  // K tile: kFwdTileN rows of D bf16, each row padded by 16 bytes so that the
  // 16-byte operand reads of 16 consecutive rows fall on distinct banks.
  static constexpr int kRowK = D * 2 + 16;
  static constexpr int kBytesK = kFwdTileN * kRowK;
  // V^T tile: D rows of kFwdTileN bf16 keys (permuted order), padded likewise.
  static constexpr int kRowV = kFwdTileN * 2 + 16;
  static constexpr int kBytesV = D * kRowV;
  // two K buffers, then two V^T buffers
  static constexpr int kOffV = 2 * kBytesK;
  static constexpr int kTotal = 2 * kBytesK + 2 * kBytesV;
  // flex: two buffers of the tile's kFwdTileN document ids
  static constexpr int kOffDoc = kTotal;
  static constexpr int kBytesDoc = kFwdTileN * 4;
  static constexpr int kTotalFlex = kTotal + 2 * kBytesDoc;
  // output staging: per wave its 32 rows of D bf16, padded like K
  static constexpr int kRowO = D * 2 + 16;
  static constexpr int kBytesOWave = 32 * kRowO;
  static constexpr int kOffO = kTotalFlex;
  static constexpr int kTotalAll = kOffO + (kFwdThreads / 64) * kBytesOWave;
};

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);  // v_cvt_pk_bf16_f32, RNE
  return __builtin_bit_cast(uint32_t, r);
}

// Reductions over the lane pair (l, l ^ 32): v_permlane32_swap hands each lane
// both values (in some order), so combining its two results is symmetric.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of a key inside its 16-key group in the V^T rows: keys 4..7 and
// 8..11 swap places, which is the order the S^T accumulator holds them in.
__device__ inline int vt_group_pos(int quad_in_group) {
  return ((quad_in_group & 1) << 3) | ((quad_in_group >> 1) << 2);
}

// Threads of a workgroup: eight waves in two ping-pong groups, or for the
// block-sparse instantiation four waves (128 rows, two 64-row blocks) without
// groups, two workgroups per CU (see the block-sparse notes below).
template <bool SPARSE>
constexpr int fwd_threads() { return SPARSE ? 256 : kFwdThreads; }

template <int D, bool FLEX, bool BIAS, bool SPARSE>
__global__ __launch_bounds__(fwd_threads<SPARSE>())
__attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_bf16_kernel(
    __bf16* __restrict__ O, const __bf16* __restrict__ Q,
    const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    float* __restrict__ LSE, int B, int H, int Hkv, int Sq, int Sk, int causal,
    int window, int input_pos, const int32_t* __restrict__ k_lengths,
    float scale_log2, FlexArgs fx, const uint8_t* __restrict__ keep,
    int n_wg) {
  using L = FwdLds<D>;
  constexpr int KSTEPS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int DBLK = D / 32;     // 32-wide blocks of the head dimension
  // Block-sparse workgroups are four waves, 128 rows: a 256-row workgroup
  // walks the union of the tiles its four 64-row blocks keep, and those sets
  // overlap little (on the image workload the union is 3.4x each block's
  // set, 1.9x for two blocks), so most of its steps would keep one block's
  // two waves busy while the rest wait at the barriers.  Without the second
  // group both K and V are staged by every thread, the phases are separated
  // by plain barriers, and two workgroups share a CU.
  constexpr bool PP = !SPARSE;                 // ping-pong between two groups
  constexpr int NT = fwd_threads<SPARSE>();
  constexpr int TM = NT / 2;                   // query rows per workgroup
  constexpr int GT = PP ? NT / 2 : NT;         // threads staging each of K, V
  constexpr int KLOADS = kFwdTileN * D / 8 / GT;       // K loads/thread
  constexpr int VTHREADS = (kFwdTileN / 4) * (D / 8);  // threads staging V
  static_assert(TM % kSparseBlock == 0, "row blocks per workgroup");

  // (the block-sparse kernel stages O in the K/V rings, after a barrier)
  __shared__ __attribute__((aligned(16))) char smem[SPARSE ? L::kTotal : L::kTotalAll];
  // block-sparse: the key tiles some row block of this workgroup keeps, and
  // per listed tile the keep bits of its 64-row blocks
  __shared__ int16_t s_list[SPARSE ? kSparseMaxTiles : 1];
  __shared__ uint8_t s_kbits[SPARSE ? kSparseMaxTiles : 1];
  __shared__ int s_ntiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = PP ? wave >> 2 : 0;     // 0: group A, 1: group B
  const int gtid = tid & (GT - 1);        // thread index within the group
  const int lrow = lane & 31;  // query row (within the wave) this lane owns
  const int half = lane >> 5;  // which half of each MFMA k-slice this lane feeds

  // ---- work items: heaviest query tiles first, XCD-grouped by KV head ----
  const int G = H / Hkv;
  const int nqt = (Sq + TM - 1) / TM;
  const int total = nqt * H * B;
  // Persistent launch (n_wg > 0 workgroups, a multiple of 8, one per CU): the
  // workgroup on XCD x (= blockIdx % 8) walks that XCD's item positions in a
  // snake order (c, 2C-1-c, 2C+c, ...), which pairs heavy and light causal
  // tiles; the few items past 8 * (total / 8) come in a last round.
  // Otherwise one workgroup per item.
  const bool persistent = n_wg > 0;
  const int per_xcd = total >> 3;
  const int wg_x = n_wg >> 3;
  const int rounds = persistent ? (per_xcd + wg_x - 1) / wg_x + 1 : 1;
  for (int round = 0; round < rounds; ++round) {
  int lid = blockIdx.x;
  if (persistent) {
    const int c = (int)blockIdx.x >> 3;
    if (round < rounds - 1) {
      const int pos = (round & 1) ? (round + 1) * wg_x - 1 - c : round * wg_x + c;
      if (pos >= per_xcd) continue;
      lid = (pos << 3) | ((int)blockIdx.x & 7);
    } else {
      lid = (per_xcd << 3) + (int)blockIdx.x;
      if (lid >= total) continue;
    }
  }
  int wid = lid;
  {
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous range of work so the query heads sharing a KV head (and
    // their K/V tiles) stay in one L2.
    const int per = total >> 3;
    if (lid < (per << 3)) wid = (lid & 7) * per + (lid >> 3);
  }
  const int per_pair = nqt * G;
  const int pair = wid / per_pair;
  const int rem = wid - pair * per_pair;
  const int qt_rank = rem / G;
  const int hg = rem - qt_rank * G;
  const int b = pair / Hkv;
  const int g = pair - b * Hkv;
  const int h = g * G + hg;
  const int qt = causal ? (nqt - 1 - qt_rank) : qt_rank;

  const int i0 = qt * TM;
  const int i1 = min(i0 + TM, Sq);
  const int kl = k_lengths ? min(max(k_lengths[b], 0), Sk) : Sk;
  // flex: rows at or past q_lengths[b] attend to nothing; the geometry covers
  // the live rows, and a workgroup with dead rows (or a document mask) masks
  // every tile element by element
  int prefix = 0, ql = Sq;
  bool force_partial = false;
  if constexpr (FLEX) {
    prefix = fx.prefix;
    if (fx.q_lengths) ql = min(max(fx.q_lengths[b], 0), Sq);
    force_partial = fx.doc_q != nullptr || ql < i1;
  }
  const int i1g = FLEX ? max(min(i1, ql), i0) : i1;
  KvGeometry geo = {0, 0, 0, 0, 0};
  if (i1g > i0) geo = kv_geometry(i0, i1g, kl, causal, window, input_pos, prefix);

  const size_t q_base = ((size_t)(b * H + h) * Sq) * D;
  const size_t kv_base = ((size_t)(b * Hkv + g) * Sk) * D;

  // ---- my query row ----
  const int qi = i0 + wave * 32 + lrow;  // global query row of this lane
  RowRange rr = row_range(qi, kl, causal, window, input_pos, prefix);
  if (FLEX && qi >= ql) rr.lo = rr.hi = 0;

  bf16x8_t qreg[KSTEPS];
  {
    const bool ok = qi < Sq;
    const __bf16* qp = Q + q_base + (size_t)(ok ? qi : 0) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = ok ? *(const u32x4_t*)(qp + ks * 16) : u32x4_t{0, 0, 0, 0};
      qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x16_t oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16_t{};
  float m_run = -INFINITY;  // running max (base-2 scaled domain)
  float l_run = 0.f;        // this lane's half of the running row sum

  int kt_first = 0, kt_last = -1;
  if (geo.any) {
    kt_first = geo.union_lo / kFwdTileN;
    kt_last = (geo.union_hi - 1) / kFwdTileN;
  }
  // The tiles walked, in order: every tile of the union, or (block-sparse)
  // those that some row block of the workgroup keeps, listed by wave 0.
  int n_tiles = kt_last - kt_first + 1;
  if constexpr (SPARSE) {
    const int nqb = (Sq + kSparseBlock - 1) / kSparseBlock;
    const int nkb = (Sk + kSparseBlock - 1) / kSparseBlock;
    const int qb0 = i0 / kSparseBlock;
    const uint8_t* krow = keep + ((size_t)(b * H + h) * nqb + qb0) * nkb;
    if (wave == 0) {
      int base = 0;
      for (int c0 = kt_first; c0 <= kt_last; c0 += 64) {
        const int kt = c0 + lane;
        unsigned bits = 0;
        if (kt <= kt_last) {
#pragma unroll
          for (int q = 0; q < TM / kSparseBlock; ++q)
            if (qb0 + q < nqb && krow[(size_t)q * nkb + kt]) bits |= 1u << q;
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(bits != 0);
        if (bits) {
          const int at = base + __builtin_popcountll(m & ((1ull << lane) - 1));
          s_list[at] = (int16_t)kt;
          s_kbits[at] = (uint8_t)bits;
        }
        base += __builtin_popcountll(m);
      }
      if (lane == 0) s_ntiles = base;
    }
    __syncthreads();
    n_tiles = s_ntiles;
  }
  auto tile_at = [&](int idx) { return SPARSE ? (int)s_list[idx] : kt_first + idx; };
  // block-sparse: does this wave's 64-row block keep the idx-th walked tile?
  // (uniform per wave; a wave skips the products and softmax of a tile it
  // drops, and still takes part in the staging and the barriers)
  auto wave_keeps = [&](int idx) {
    return !SPARSE || ((s_kbits[idx] >> (wave >> 1)) & 1) != 0;
  };

  // ---- staging: global -> registers -> LDS ----
  // K/V are read through buffer resources whose range is exactly the keys
  // some row of this workgroup may attend, [union_lo, union_hi): the hardware
  // range check returns zeros for any other key, so keys that no row may see
  // (past k_lengths, past the causal frontier, before the window) are never
  // read and the loads need no branches.  Group A stages K, group B stages V.
  const int nvalid = geo.union_hi - geo.union_lo;
  const size_t valid_base = kv_base + (size_t)geo.union_lo * D;
  // one resource per tensor, both uniform: selecting between them per group
  // would make the resource divergent
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(K + valid_base), (short)0, nvalid * D * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(V + valid_base), (short)0, nvalid * D * 2, kBufferRsrcWord3);

  // ---- flex per-lane state ----
  const bool has_bias = FLEX && BIAS;
  const bool has_alibi = FLEX && fx.alibi != nullptr;
  const bool has_doc = FLEX && fx.doc_q != nullptr;
  const bool has_cap = FLEX && fx.softcap > 0.f;
  float alibi_slope = 0.f;
  int doc_row = 0;
  int bias_row = 0;
  if constexpr (FLEX) {
    if (has_alibi) alibi_slope = fx.alibi[h];
    if (has_doc) doc_row = qi < Sq ? fx.doc_q[(size_t)b * Sq + qi] : 0;
    // rows past Sq read zeros
    if (has_bias) bias_row = qi < Sq ? qi * Sk : Sq * Sk;
  }
  // document ids of the workgroup's key union; the (batch, head) bias plane
  const __amdgpu_buffer_rsrc_t doc_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      has_doc ? (void*)(fx.doc_kv + (size_t)b * Sk + geo.union_lo) : nullptr,
      (short)0, has_doc ? nvalid * 4 : 0, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t bias_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      has_bias ? (void*)(fx.bias + b * fx.bias_bstride + h * fx.bias_hstride)
               : nullptr,
      (short)0, has_bias ? Sq * Sk * 4 : 0, kBufferRsrcWord3);
  f32x16_t bias_t[2];  // bias of this lane's row for the tile being scored
  u32x4_t stg_doc = {0, 0, 0, 0};

  u32x4_t stg[4];
  u32x4_t stgv[PP ? 1 : 4];   // V staged alongside K (no groups)
  const int vkq = gtid & 15;  // key quad within the tile (V staging)
  const int vdc = gtid >> 4;  // 8-wide d chunk (V staging)
  const bool v_stager = VTHREADS == GT || gtid < VTHREADS;

  auto fetch = [&](int kt) {
    const int rel0 = kt * kFwdTileN - geo.union_lo;  // tile start, in valid keys
    auto fetch_v = [&](u32x4_t (&dst)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = rel0 + vkq * 4 + i;
        dst[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         vrsrc, (key * D + vdc * 8) * 2, 0, 0));
      }
    };
    if constexpr (!PP) {
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) {
        const int c = i * GT + gtid;
        stg[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         krsrc, ((rel0 + c / (D / 8)) * D + (c % (D / 8)) * 8) * 2, 0, 0));
      }
      if (v_stager) fetch_v(stgv);
      return;
    }
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) {
        const int c = i * GT + gtid;
        const int key = rel0 + c / (D / 8);
        const int dch = c % (D / 8);
        stg[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         krsrc, (key * D + dch * 8) * 2, 0, 0));
      }
      if (FLEX && has_doc && gtid < kFwdTileN / 4)
        stg_doc = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         doc_rsrc, (rel0 + gtid * 4) * 4, 0, 0));
    } else if (v_stager) {
      fetch_v(stg);
    }
  };

  auto stash = [&](int buf) {
    auto stash_v = [&](const u32x4_t (&src)[4]) {
      // 4 keys x 8 d  ->  8 rows of V^T, 4 keys (8 bytes) each
      char* vb = smem + L::kOffV + buf * L::kBytesV;
      const int grp16 = vkq >> 2;
      const int pos = grp16 * 16 + vt_group_pos(vkq & 3);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t r0 = src[0][m], r1 = src[1][m], r2 = src[2][m],
                       r3 = src[3][m];
        u32x2_t even = {__builtin_amdgcn_perm(r1, r0, 0x05040100u),
                        __builtin_amdgcn_perm(r3, r2, 0x05040100u)};
        u32x2_t odd = {__builtin_amdgcn_perm(r1, r0, 0x07060302u),
                       __builtin_amdgcn_perm(r3, r2, 0x07060302u)};
        const int d = vdc * 8 + 2 * m;
        *(u32x2_t*)(vb + d * L::kRowV + pos * 2) = even;
        *(u32x2_t*)(vb + (d + 1) * L::kRowV + pos * 2) = odd;
      }
    };
    if (!PP || grp == 0) {
      char* kb = smem + buf * L::kBytesK;
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) {
        const int c = i * GT + gtid;
        const int key = c / (D / 8);
        const int dch = c % (D / 8);
        *(u32x4_t*)(kb + key * L::kRowK + dch * 16) = stg[i];
      }
      if (FLEX && has_doc && gtid < kFwdTileN / 4)
        *(u32x4_t*)(smem + L::kOffDoc + buf * L::kBytesDoc + gtid * 16) = stg_doc;
    }
    if constexpr (!PP) {
      if (v_stager) stash_v(stgv);
    } else if (grp == 1 && v_stager) {
      stash_v(stg);
    }
  };

  f32x16_t s[2];           // S^T of the current tile (two 32-key blocks)
  u32x4_t pb[2][2];        // P^T of the previous tile, packed bf16 (MFMA B operands)

  // flex: the bias of this lane's row for the keys of the idx-th walked tile:
  // j0 + kb2*32 + q4*8 + half*4 + e, held in register q4*4 + e of block kb2
  // (the S^T accumulator order)
  auto bias_loads = [&](int idx) {
    const int jb = tile_at(idx) * kFwdTileN + half * 4;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jb + kb2 * 32 + (r >> 2) * 8 + (r & 3);
        bias_t[kb2][r] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(bias_rsrc, (bias_row + j) * 4, 0, 0));
      }
  };

  // M-phase of the idx-th walked tile: O += P V of the previous one, then
  // S = K Q^T of this one; tile idx sits in LDS buffer idx & 1
  auto m_phase = [&](int idx, bool do_pv, bool do_s) {
    if constexpr (SPARSE) {
      do_pv = do_pv && wave_keeps(idx - 1);
      do_s = do_s && wave_keeps(idx);
    }
    if (!FLEX && do_pv && do_s) {
      // Steady state: the 32 products of the phase with their LDS operand
      // reads kept kFwdOpDepth ahead (left to itself the compiler keeps only
      // one or two in flight and each MFMA waits for its read).  Consecutive
      // products go to different accumulators.  (The flex kernels keep the
      // plain order: their extra registers leave no room for the ring.)
      const char* vb = smem + L::kOffV + ((idx - 1) & 1) * L::kBytesV;
      const char* kb = smem + (idx & 1) * L::kBytesK;
      constexpr int NPV = DBLK * 4;
      constexpr int NOP = NPV + 2 * KSTEPS;
      auto op_addr = [&](int i) -> const char* {
        if (i < NPV) {
          const int pr = i / DBLK, db = i % DBLK;  // pr = kb2 * 2 + st
          return vb + (db * 32 + lrow) * L::kRowV + half * 16 + pr * 32;
        }
        const int j = i - NPV, ks = j >> 1, kb2 = j & 1;
        return kb + (kb2 * 32 + lrow) * L::kRowK + half * 16 + ks * 32;
      };
      bf16x8_t ring[kFwdOpDepth];
#pragma unroll
      for (int i = 0; i < kFwdOpDepth; ++i) ring[i] = *(const bf16x8_t*)op_addr(i);
      s[0] = s[1] = f32x16_t{};
#pragma unroll
      for (int i = 0; i < NOP; ++i) {
        const bf16x8_t a = ring[i % kFwdOpDepth];
        if (i + kFwdOpDepth < NOP)
          ring[i % kFwdOpDepth] = *(const bf16x8_t*)op_addr(i + kFwdOpDepth);
        if (i < NPV) {
          const int pr = i / DBLK, db = i % DBLK;
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, __builtin_bit_cast(bf16x8_t, pb[pr >> 1][pr & 1]), oacc[db], 0, 0, 0);
        } else {
          const int j = i - NPV, ks = j >> 1, kb2 = j & 1;
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[kb2], 0, 0, 0);
        }
      }
      // hold the scheduler to that order: kFwdOpDepth reads, then one MFMA
      // and one read alternately, then the last MFMAs (0x100 = LDS read,
      // 0x008 = MFMA)
      __builtin_amdgcn_sched_group_barrier(0x100, kFwdOpDepth, 0);
#pragma unroll
      for (int i = 0; i < NOP - kFwdOpDepth; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kFwdOpDepth, 0);
      // and keep the last products ahead of the barrier that ends the phase
      asm volatile("" : "+v"(s[0]), "+v"(s[1]));
      return;
    }
    if (do_pv) {
      const char* vb = smem + L::kOffV + ((idx - 1) & 1) * L::kBytesV;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const char* arow = vb + (db * 32 + lrow) * L::kRowV + half * 16;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            bf16x8_t a = *(const bf16x8_t*)(arow + (kb2 * 2 + st) * 32);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, __builtin_bit_cast(bf16x8_t, pb[kb2][st]), oacc[db], 0, 0, 0);
          }
      }
    }
    if (FLEX && do_s && has_bias) bias_loads(idx);
    if (do_s) {
      const char* kb = smem + (idx & 1) * L::kBytesK;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[kb2] = f32x16_t{};
        const char* arow = kb + (kb2 * 32 + lrow) * L::kRowK + half * 16;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          bf16x8_t a = *(const bf16x8_t*)(arow + ks * 32);
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[kb2],
                                                           0, 0, 0);
        }
      }
    }
  };

  // V-phase: softmax of S(kt) into P(kt); stage tile kt+1 and fetch kt+2
  // flex: scores into base-2 units of the modified score, in place.  With y =
  // qk_scale * s + bias + alibi (natural units), the base-2 score is
  //   y * log2(e)                                  without a cap, and
  //   log2(e) * cap * tanh(y / cap) = A - B / (exp2(y * 2 log2(e) / cap) + 1)
  // with A = log2(e) * cap, B = 2 A; the factor in front of y (u) is folded
  // into the per-element FMAs.  Without bias, ALiBi and cap the factor goes
  // into the exponent instead (no pass over the scores).
  constexpr float kLog2e = 1.4426950408889634f;
  const bool transform = has_bias || has_alibi || has_cap;
  const float u = has_cap ? 2.f * kLog2e / fx.softcap : kLog2e;
  const float k_s = fx.qk_scale * u;
  const float cap_a = kLog2e * fx.softcap, cap_b = 2.f * cap_a;
  auto flex_scores = [&](int j0) {
    if (has_alibi) {
      // u * slope * (p - j) with j = j0 + half*4 + c, c constant per register
      const float su = alibi_slope * u;
      const float a0 = su * (float)(input_pos + qi - j0 - half * 4);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float c = (float)(kb2 * 32 + (r >> 2) * 8 + (r & 3));
          s[kb2][r] = __builtin_fmaf(s[kb2][r], k_s, __builtin_fmaf(-su, c, a0));
        }
    } else {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb2][r] *= k_s;
    }
    if (has_bias) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb2][r] = __builtin_fmaf(bias_t[kb2][r], u, s[kb2][r]);
    }
    if (has_cap) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(s[kb2][r]);
          s[kb2][r] = __builtin_fmaf(-cap_b, __builtin_amdgcn_rcpf(e + 1.f), cap_a);
        }
    }
  };
  // flex: a key whose document differs from the row's is blocked
  auto doc_mask = [&](int idx) {
    const char* db = smem + L::kOffDoc + (idx & 1) * L::kBytesDoc + half * 16;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x4_t ids = *(const u32x4_t*)(db + (kb2 * 32 + q4 * 8) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((int)ids[e] != doc_row) s[kb2][q4 * 4 + e] = -INFINITY;
      }
  };
  // base-2 factor of the exponent: the plain path scales here, transformed
  // flex scores are already in base-2 units
  const float sl2 = FLEX ? (transform ? 1.f : fx.qk_scale * kLog2e) : scale_log2;

  auto v_phase = [&](int idx) {
    const int kt = tile_at(idx);
    const int j0 = kt * kFwdTileN;
    if constexpr (FLEX) {
      if (transform) flex_scores(j0);
      if (has_doc) doc_mask(idx);
    }
    if constexpr (SPARSE) {
      // this wave's 64-row block drops the tile: no score, only the staging
      if (!wave_keeps(idx)) {
        if (idx + 1 < n_tiles) stash((idx + 1) & 1);
        if (idx + 2 < n_tiles) fetch(tile_at(idx + 2));
        return;
      }
    }
    if (tile_class(geo, j0, kFwdTileN) == kTilePartial || (FLEX && force_partial)) {
      // key j0 + half*4 + c is allowed iff c lies in [t_lo, t_lo + width);
      // c is a compile-time constant per register, so one subtract, one
      // unsigned compare and one select per score
      const int t_lo = rr.lo - (j0 + half * 4);
      const unsigned width = (unsigned)max(rr.hi - rr.lo, 0);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb2 * 32 + (r >> 2) * 8 + (r & 3);
          if ((unsigned)(c - t_lo) >= width) s[kb2][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    const float mt = pair_max(mx) * sl2;
    const bool need = mt > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // need == false leaves the lane unchanged (and avoids -inf - -inf)
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
      m_run = need ? mt : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 =
            __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][r], sl2, -mref));
        const float p1 = __builtin_amdgcn_exp2f(
            __builtin_fmaf(s[kb2][r + 1], sl2, -mref));
        psum += p0 + p1;
        pb[kb2][r >> 3][(r & 7) >> 1] = pack_bf16x2(p0, p1);
      }
    l_run += psum;
    // Pin P here: left alone, the compiler sinks the exponentials past the
    // barrier into the next MFMA phase (their only user), which serialises
    // them with that phase's products instead of overlapping them with the
    // other group's.
    asm volatile("" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]),
                 "+v"(l_run));
    if (idx + 1 < n_tiles) stash((idx + 1) & 1);
    if (idx + 2 < n_tiles) fetch(tile_at(idx + 2));
  };

  if (n_tiles > 0) {
    // prologue: the first tile in LDS, the second in flight
    fetch(tile_at(0));
    stash(0);
    if (n_tiles > 1) fetch(tile_at(1));
    __syncthreads();
    if (PP && grp == 1) __syncthreads();  // group B runs one phase behind
    for (int idx = 0; idx < n_tiles; ++idx) {
      m_phase(idx, idx > 0, true);
      __syncthreads();
      v_phase(idx);
      __syncthreads();
    }
    m_phase(n_tiles, true, false);
    if (PP && grp == 0) __syncthreads();  // matches group B's extra barrier
  }

  // ---- epilogue ----
  const float l_tot = pair_sum(l_run);
  {
    // O goes out through LDS: a lane holds 4-element pieces of its own row,
    // so storing them directly writes 8 bytes into each of 64 rows per
    // instruction; staged in the wave's own LDS rows and read back as 16-byte
    // chunks, each 16 lanes write one whole row.  The wave only reads what it
    // wrote, so no barrier is needed.
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // (without groups the staging area is the K/V rings, free once every
    // wave is past its last products)
    if constexpr (!PP) __syncthreads();
    char* ost = smem + (PP ? L::kOffO : 0) + wave * L::kBytesOWave;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + half * 4;
        u32x2_t w = {pack_bf16x2(oacc[db][r4 * 4 + 0] * inv,
                                 oacc[db][r4 * 4 + 1] * inv),
                     pack_bf16x2(oacc[db][r4 * 4 + 2] * inv,
                                 oacc[db][r4 * 4 + 3] * inv)};
        *(u32x2_t*)(ost + lrow * L::kRowO + d * 2) = w;
      }
    __builtin_amdgcn_wave_barrier();
    constexpr int CHUNKS = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < 32 * CHUNKS / 64; ++i) {
      const int c = i * 64 + lane;
      const int row = c / CHUNKS, ch = c - row * CHUNKS;
      const u32x4_t v = *(const u32x4_t*)(ost + row * L::kRowO + ch * 16);
      const int qrow = i0 + wave * 32 + row;
      if (qrow < Sq) *(u32x4_t*)(O + q_base + (size_t)qrow * D + ch * 8) = v;
    }
  }
  if (LSE && qi < Sq && half == 0) {
    const float lse = l_tot > 0.f
                          ? (m_run + __builtin_log2f(l_tot)) * 0.69314718055994530942f
                          : -INFINITY;
    LSE[(size_t)(b * H + h) * Sq + qi] = lse;
  }
  __syncthreads();  // LDS is reused by the next item
  }
}

// Number of persistent workgroups for `total` items (one per CU, a multiple
// of 8), or 0 for a launch of one workgroup per item when there are too few
// items to pair up.
static int persistent_workgroups(long long total, int per_cu = 1) {
  static int cu_count[64];  // per device; 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n = -1;
    cu_count[dev] = n > 0 ? n : -1;
  }
  const int n_wg = (cu_count[dev] / 8) * 8 * per_cu;
  if (n_wg < 8 || total < 2LL * n_wg) return 0;
  return n_wg;
}

template <int D>
hipError_t launch_fwd_bf16(void* O, const void* Q, const void* K,
                           const void* V, float* LSE, int B, int H, int Hkv,
                           int Sq, int Sk, int causal, int window,
                           int input_pos, const int32_t* k_lengths,
                           hipStream_t stream) {
  const int nqt = (Sq + kFwdTileM - 1) / kFwdTileM;
  const long long total = (long long)nqt * H * B;
  const int n_wg = persistent_workgroups(total);
  const unsigned grid = n_wg > 0 ? (unsigned)n_wg : (unsigned)total;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, false, false>), dim3(grid),
                     dim3(kFwdThreads), 0, stream, (__bf16*)O,
                     (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, LSE,
                     B, H, Hkv, Sq, Sk, causal, window, input_pos, k_lengths,
                     scale_log2, FlexArgs{}, (const uint8_t*)nullptr, n_wg);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_flex(void* O, const void* Q, const void* K,
                           const void* V, float* LSE, int B, int H, int Hkv,
                           int Sq, int Sk, int causal, int window,
                           int input_pos, const int32_t* k_lengths,
                           const attn_flex_t* f, hipStream_t stream) {
  const int nqt = (Sq + kFwdTileM - 1) / kFwdTileM;
  const long long total = (long long)nqt * H * B;
  const int n_wg = persistent_workgroups(total);
  const unsigned grid = n_wg > 0 ? (unsigned)n_wg : (unsigned)total;
  FlexArgs fx{};
  fx.q_lengths = f->q_lengths;
  fx.alibi = f->alibi_slopes;
  fx.bias = f->bias;
  fx.doc_q = f->doc_q;
  fx.doc_kv = f->doc_kv;
  const long long plane = (long long)Sq * Sk;
  fx.bias_hstride = f->bias && f->bias_H > 1 ? plane : 0;
  fx.bias_bstride = f->bias && f->bias_B > 1 ? plane * f->bias_H : 0;
  fx.prefix = f->prefix;
  fx.softcap = f->softcap;
  fx.qk_scale = f->qk_scale > 0.f ? f->qk_scale : 1.f / sqrtf((float)D);
  // the bias tile costs 32 registers per lane: a kernel of its own
  if (fx.bias)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, true, false>), dim3(grid),
                       dim3(kFwdThreads), 0, stream, (__bf16*)O,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, LSE,
                       B, H, Hkv, Sq, Sk, causal, window, input_pos, k_lengths,
                       0.f, fx, (const uint8_t*)nullptr, n_wg);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true, false, false>), dim3(grid),
                       dim3(kFwdThreads), 0, stream, (__bf16*)O,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, LSE,
                       B, H, Hkv, Sq, Sk, causal, window, input_pos, k_lengths,
                       0.f, fx, (const uint8_t*)nullptr, n_wg);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_sparse(void* O, const void* Q, const void* K,
                             const void* V, float* LSE, int B, int H, int Hkv,
                             int Sq, int Sk, int causal, int window,
                             int input_pos, const int32_t* k_lengths,
                             const uint8_t* keep, hipStream_t stream) {
  constexpr int NT = fwd_threads<true>();
  const int nqt = (Sq + NT / 2 - 1) / (NT / 2);
  const long long total = (long long)nqt * H * B;
  const int n_wg = persistent_workgroups(total, 2);  // two workgroups per CU
  const unsigned grid = n_wg > 0 ? (unsigned)n_wg : (unsigned)total;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, false, true>), dim3(grid),
                     dim3(NT), 0, stream, (__bf16*)O,
                     (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, LSE,
                     B, H, Hkv, Sq, Sk, causal, window, input_pos, k_lengths,
                     scale_log2, FlexArgs{}, keep, n_wg);
  return hipGetLastError();
}

#define ATTN_INST(D)                                                          \
  template hipError_t launch_fwd_bf16<D>(void*, const void*, const void*,     \
                                         const void*, float*, int, int, int,  \
                                         int, int, int, int, int,             \
                                         const int32_t*, hipStream_t);        \
  template hipError_t launch_fwd_flex<D>(void*, const void*, const void*,     \
                                         const void*, float*, int, int, int,  \
                                         int, int, int, int, int,             \
                                         const int32_t*, const attn_flex_t*,  \
                                         hipStream_t);                        \
  template hipError_t launch_fwd_sparse<D>(void*, const void*, const void*,   \
                                           const void*, float*, int, int,     \
                                           int, int, int, int, int, int,      \
                                           const int32_t*, const uint8_t*,    \
                                           hipStream_t);
ATTN_INST(64)
ATTN_INST(128)
#undef ATTN_INST

}  // namespace attn
