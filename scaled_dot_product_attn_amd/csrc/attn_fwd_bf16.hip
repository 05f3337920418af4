// Fused attention forward for bf16 Q/K/V/O on gfx950 (MI355X).
//
// O = softmax(scale * Q K^T + mask) V with Float32 accumulation and the row
// logsumexp saved (Tylo.jl "Primitives", attention!: GQA, causal, input_pos,
// k_lengths, checkpoints M/L; flex_attention!: qk_scale = 1/sqrt(Dk), in-kernel
// block skipping for analytic masks; mlx-arsenal "Attention": causal_mask /
// sliding_window_mask with -inf at blocked positions).
//
// Work decomposition
//   One workgroup = 8 waves = 256 query rows; each wave owns 32 rows.  With
//   grouped-query attention the rows are hp query heads (the largest power
//   of two up to 8 dividing H / Hkv) of one KV head at 256 / hp positions, so
//   the heads share every K/V tile.  The workgroup walks the 64-key tiles its
//   rows can see (empty tiles are never visited); a persistent workgroup
//   loads the next item's queries and first tiles during its last product.
//
// Ping-pong between two wave groups.  Waves 0-3 (group A) and 4-7 (group B)
// sit one per SIMD each, so every SIMD holds one wave of each group.  Each
// wave alternates two phases:
//   M-phase k: O += P(k-1) V(k-1) and S(k) = K(k) Q^T   (32 MFMAs)
//   V-phase k: mask and online softmax of S(k) -> P(k)
// with one workgroup barrier per tile: window k is M(k) then V(k) for group
// A and V(k-1) then M(k) for group B, so at the start of a window one wave of
// each SIMD feeds the matrix core while the other runs the softmax, and they
// swap halfway (the M-phase runs at raised wave priority).
//
// Staging: K and V tiles go from HBM straight into LDS (buffer loads with the
// LDS bit, issued by all eight waves two windows ahead of their use, at the
// start of a V-phase, each wave a fixed sequence without branches), K into a
// three-slot ring of padded rows, V into a
// four-slot ring of row-major rows read as V^T by transposing LDS reads.  K(k)
// is read in window k, V(k) in window k+1, so a slot is rewritten only after
// the barrier that ends its last reader's window; each wave waits for its own
// loads of the next window's tiles just before the barrier.
//
// Contractions on the matrix cores (v_mfma_f32_32x32x16_bf16), transposed so
// that one lane owns one query row:
//   S^T (32 keys x 32 queries) = K (32 x 16 d) * Q^T (16 d x 32 queries)
//     -> lane l holds query l%32 and 16 of the 32 keys, so the row max and
//        row sum are in-lane reductions plus one exchange with lane l^32.
//   O^T (32 d x 32 queries) += V^T (32 d x 16 keys) * P^T (16 keys x 32 q)
//     -> P^T is the S^T accumulator itself, rounded to bf16: no shuffle.
//   The transposing reads (ds_read_b64_tr_b16) deliver V^T's keys in the
//   order in which the S^T accumulator registers hold them.
//
// Flex variants (FLEX = true; Tylo.jl "Primitives", flex_attention! and its
// mods): the same kernel with the score rewritten before the softmax, in this
// order: qk_scale * s, plus an additive bias tile (BiasScore), plus
// slope_h * (q - kv) (AliBiScore), then cap * tanh(. / cap) (SoftCapScore);
// and the mask extended by a prefix (prefix_lm = CausalMask | PrefixMask),
// per-batch query lengths (q_lengths) and document ids (DocumentMask).  The
// bias tile of a lane's row is loaded at the start of the M-phase that computes
// the tile's scores, document ids of the keys are loaded into LDS with K.  The
// mask extensions (XM) have an instantiation of their own: a precomputed
// BlockMask (Tylo.jl "Primitives", BlockMask / build_block_mask: empty key
// blocks are skipped, fully unmasked ones need no document mask) and a prefix
// beside a sliding window (two key intervals per row).
//
// The block-sparse instantiation (SPARSE) keeps register staging: four waves
// without groups, K and V^T written to two-tile rings by the threads.
//
// Online softmax in base 2: t = s * log2(e) / sqrt(D), p = exp2(t - m); O / l
// and m + log2 l are unchanged by which m is used, as long as no p overflows
// or all of a row's underflow.  Optimistic steps: a row takes its first tile
// max as m and keeps it, so the tile max is computed only while some row of
// the wave has none; an item on which a half row's sum of p passes 2^16 (or
// is not a number) is walked again with exact steps, which raise m whenever a
// tile max exceeds it by more than 2^8.  Under a soft-cap of at most
// 60 / log2(e) the cap itself bounds every score and serves as m.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

#include "../../include/attn.h"
#include "attn_common.h"
#include "attn_host.h"

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
constexpr float kOptSum = 65536.0f;        // largest half-row sum of P the optimistic step keeps
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
  const uint8_t* bmask;   // block classes (ATTN_BLOCK_*), or null
  long long bm_bstride;   // elements between batches of bmask (0: shared)
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
  static_assert((kFwdThreads / 64) * kBytesOWave <= kTotal, "O staging fits the buffers");
  // Direct-to-LDS staging (the ping-pong kernels): K in a ring of kRingK
  // padded tiles as above; V in a ring of kRingV unpadded row-major tiles
  // whose 16-byte chunks are XOR-swizzled (v_swizzle) for the transposing
  // reads that deliver V^T operands; document ids beside K.
  static constexpr int kRingK = 3, kRingV = 4;
  static constexpr int kRowVd = D * 2;
  static constexpr int kBytesVd = kFwdTileN * kRowVd;
  static constexpr int kOffVd = kRingK * kBytesK;
  static constexpr int kOffDocD = kOffVd + kRingV * kBytesVd;
  // (document ids are read in V-phases, which group B runs a window after
  // group A: their ring is as deep as V's)
  static constexpr int kTotalDma = kOffDocD + kRingV * kBytesDoc;
  // ping-pong kernels: O staged in an area of its own, half the head
  // dimension at a time (the rings may already hold the next item's tiles)
  static constexpr int kRowOh = D + 16;
  static constexpr int kBytesOWaveH = 32 * kRowOh;
  static constexpr int kOffOs = kTotalDma;
  static constexpr int kTotalPP = kOffOs + (kFwdThreads / 64) * kBytesOWaveH;
  // DMA instructions per tile: 64 lanes x 16 bytes each
  static constexpr int kChunksK = kRowK / 16;                 // incl. the pad chunk
  static constexpr int kInstrK = kFwdTileN * kChunksK / 64;
  static constexpr int kInstrV = kFwdTileN * (D / 8) / 64;
  static_assert(kFwdTileN * kChunksK % 64 == 0, "whole K instructions");
};

// One 16-byte-per-lane load from a buffer straight into LDS: lane l's chunk
// lands at lds_addr + 16 l.  Written as inline assembly so that the compiler
// does not treat the loads still in flight as pending LDS writes (it would
// wait for them before every LDS read and barrier); the kernel waits for them
// itself (s_waitcnt vmcnt) before the barrier that precedes their readers.
// The instruction writes no vector register.
__device__ inline void lds_load16(u32x4_t rsrc, uint32_t lds_addr, int voffset) {
  // Five wait states first: the descriptor registers may have just been
  // written by a vector instruction (v_readlane / v_readfirstlane), which a
  // memory instruction may read only five wait states later, and the
  // compiler inserts no such wait for an instruction inside inline assembly
  // (M0, written just before, needs one).
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "{m0}"(lds_addr)
      : "memory");
}

// The same load when the descriptor registers were written long before (by
// the time of the item's first loads): only M0, written by a scalar
// instruction just before, needs its one wait state.
__device__ inline void lds_load16_m0(u32x4_t rsrc, uint32_t lds_addr, int voffset) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "{m0}"(lds_addr)
      : "memory");
}

// A raw buffer descriptor (as for __builtin_amdgcn_make_buffer_rsrc: no
// stride, num_records bytes, out-of-range reads return zero) in four scalar
// registers, for the inline-assembly loads above.
__device__ inline u32x4_t buffer_desc_s(const void* base, int num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4_t d;
  d[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
  d[2] = __builtin_amdgcn_readfirstlane((uint32_t)num_records);
  d[3] = (uint32_t)kBufferRsrcWord3;
  return d;
}

__device__ inline uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Chunk swizzle of the row-major V tiles: chunk c of row r is stored at
// c ^ v_swizzle(r).  A transposing read covers 4 consecutive rows (from a
// multiple of 4) x 4 aligned chunks with 32 lanes; the swizzle spreads those
// 16 (row, chunk) pairs over distinct 16-byte bank groups.
template <int D>
__device__ inline int v_swizzle(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

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

// XM (flex only): the mask extensions — a BlockMask, or a prefix beside a
// window (two key intervals per row) — in an instantiation of their own, so
// the other flex launches carry none of their registers.
template <int D, bool FLEX, bool BIAS, bool SPARSE, bool XM = false>
__global__ __launch_bounds__(fwd_threads<SPARSE>())
__attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_bf16_kernel(
    __bf16* __restrict__ O, const __bf16* __restrict__ Q,
    const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    float* __restrict__ LSE, int B, int H, int Hkv, int Sq, int Sk, int causal,
    int window, int input_pos, const int32_t* __restrict__ k_lengths,
    float scale_log2, FlexArgs fx, const uint8_t* __restrict__ keep,
    int n_wg, int hp_log2) {
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
  __shared__ __attribute__((aligned(16))) char smem[SPARSE ? L::kTotal : L::kTotalPP];
  // block-sparse: the key tiles some row block of this workgroup keeps, and
  // per listed tile the keep bits of its 64-row blocks
  __shared__ int16_t s_list[SPARSE ? kSparseMaxTiles : 1];
  __shared__ uint8_t s_kbits[SPARSE ? kSparseMaxTiles : 1];
  // flex with a block mask: the key tiles of the item whose class is not
  // empty, bit 15 set for FULL
  __shared__ int16_t s_blist[XM ? kSparseMaxTiles : 1];
  __shared__ int s_ntiles;
  // per item parity: the sequence number of an item on which some wave's
  // optimistic softmax step failed
  __shared__ int s_fail[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // (uniform per wave; the block-sparse kernel keeps the plain form, whose
  // registers the compiler allocates better there)
  const int wave = PP ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int grp = PP ? wave >> 2 : 0;     // 0: group A, 1: group B
  const int gtid = tid & (GT - 1);        // thread index within the group
  const int lrow = lane & 31;  // query row (within the wave) this lane owns
  const int half = lane >> 5;  // which half of each MFMA k-slice this lane feeds

  // ---- work items: heaviest query tiles first, XCD-grouped by KV head ----
  // A workgroup serves hp = 2^hp_log2 query heads of one KV head (they read
  // the same K/V tiles) at TP = TM / hp query positions: with grouped-query
  // attention the causal diagonal and window edges cut TP x TP blocks instead
  // of TM x TM, so fewer tile elements are masked away.
  const int G = H / Hkv;
  const int hp = 1 << hp_log2;
  const int TP = TM >> hp_log2;           // query positions per workgroup
  const int nch = G >> hp_log2;           // head chunks per KV head
  const int nqt = (Sq + TP - 1) / TP;
  const int total = nqt * nch * Hkv * B;
  // Persistent launch (n_wg > 0 workgroups, a multiple of 8, one per CU): the
  // workgroup on XCD x (= blockIdx % 8) walks that XCD's item positions in a
  // snake order (c, 2C-1-c, 2C+c, ...), which pairs heavy and light causal
  // tiles; the few items past 8 * (total / 8) come in a last round.
  // Otherwise one workgroup per item.
  const bool persistent = n_wg > 0;
  const int per_xcd = total >> 3;
  const int wg_x = n_wg >> 3;
  const int rounds = persistent ? (per_xcd + wg_x - 1) / wg_x + 1 : 1;
  // the item (workgroup-level work unit) of a round, or -1 for none
  auto lid_of = [&](int rd) -> int {
    int lid = blockIdx.x;
    if (persistent) {
      const int c = (int)blockIdx.x >> 3;
      if (rd < rounds - 1) {
        const int pos = (rd & 1) ? (rd + 1) * wg_x - 1 - c : rd * wg_x + c;
        if (pos >= per_xcd) return -1;
        lid = (pos << 3) | ((int)blockIdx.x & 7);
      } else {
        lid = (per_xcd << 3) + (int)blockIdx.x;
        if (lid >= total) return -1;
      }
    } else if (rd > 0) {
      return -1;
    }
    return lid;
  };
  // An item's keys: the interval geometry `geo` of its live rows and, with a
  // prefix beside a window, the keys [0, pe) every live row sees as well.
  // The tiles walked are kt0, kt0 + 1, ... for the first n1, then the rest
  // after a jump of `gap` tiles (over the keys between the prefix and the
  // window); K/V are read from the key range [vlo, vhi).
  struct ItemGeo {
    int b, g, ch, i0, i1, kl, ql, prefix, pe;
    bool force_partial;
    KvGeometry geo;
    int kt0, n1, gap, nwalk, vlo, vhi;
  };
  auto item_geo = [&](int lid) -> ItemGeo {
    ItemGeo it;
    int wid = lid;
    {
      // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
      // contiguous range of work so the query heads sharing a KV head (and
      // their K/V tiles) stay in one L2.
      const int per = total >> 3;
      if (lid < (per << 3)) wid = (lid & 7) * per + (lid >> 3);
    }
    const int per_pair = nqt * nch;
    const int pair = wid / per_pair;
    const int rem = wid - pair * per_pair;
    const int qt_rank = rem / nch;
    it.ch = rem - qt_rank * nch;
    it.b = pair / Hkv;
    it.g = pair - it.b * Hkv;
    const int qt = causal ? (nqt - 1 - qt_rank) : qt_rank;
    it.i0 = qt * TP;
    it.i1 = min(it.i0 + TP, Sq);
    it.kl = k_lengths ? min(max(k_lengths[it.b], 0), Sk) : Sk;
    // flex: rows at or past q_lengths[b] attend to nothing; the geometry
    // covers the live rows, and a workgroup with dead rows masks every tile
    // element by element
    it.prefix = 0;
    it.pe = 0;
    it.ql = Sq;
    it.force_partial = false;
    if constexpr (FLEX) {
      if (fx.q_lengths) it.ql = min(max(fx.q_lengths[it.b], 0), Sq);
      it.force_partial = it.ql < it.i1;
      // without a window the prefix widens each row's one interval; beside a
      // window it is a second interval
      if (XM && window > 0) it.pe = min(fx.prefix, it.kl);
      else it.prefix = fx.prefix;
    }
    const int i1g = FLEX ? max(min(it.i1, it.ql), it.i0) : it.i1;
    it.geo = KvGeometry{0, 0, 0, 0, 0};
    if (i1g > it.i0)
      it.geo = kv_geometry(it.i0, i1g, it.kl, causal, window, input_pos, it.prefix);
    else
      it.pe = 0;
    it.kt0 = 0;
    it.gap = 0;
    it.nwalk = 0;
    it.vlo = it.vhi = 0;
    if (it.geo.any) {
      it.kt0 = it.geo.union_lo / kFwdTileN;
      it.nwalk = (it.geo.union_hi - 1) / kFwdTileN - it.kt0 + 1;
      it.vlo = it.geo.union_lo;
      it.vhi = it.geo.union_hi;
    }
    if (it.pe > 0) {
      const int pt = (it.pe + kFwdTileN - 1) / kFwdTileN;  // tiles of [0, pe)
      if (!it.geo.any) {
        it.nwalk = pt;
        it.vhi = it.pe;
      } else if (it.kt0 <= pt) {
        it.nwalk = max(pt, it.kt0 + it.nwalk);
        it.vhi = max(it.pe, it.vhi);
      } else {
        it.gap = it.kt0 - pt;
        it.nwalk += pt;
        it.n1 = pt;
      }
      if (!it.geo.any || it.kt0 <= pt) it.n1 = it.nwalk;
      it.kt0 = 0;
      it.vlo = 0;
    } else {
      it.n1 = it.nwalk;
    }
    return it;
  };
  // the t-th tile of an item's walk
  auto walk_tile = [&](const ItemGeo& it, int t) {
    if constexpr (!XM) return it.kt0 + t;
    return it.kt0 + t + (t >= it.n1 ? it.gap : 0);
  };
  const int rb = wave >> hp_log2;         // this wave's 32-row block of the positions
  auto head_of = [&](const ItemGeo& it) { return it.g * G + it.ch * hp + (wave & (hp - 1)); };
  auto load_q = [&](bf16x8_t (&qr)[KSTEPS], const ItemGeo& it) {
    const int qrow = it.i0 + rb * 32 + lrow;
    const bool ok = qrow < Sq;
    const __bf16* qp = Q + ((size_t)(it.b * H + head_of(it)) * Sq + (ok ? qrow : 0)) * D +
                       half * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = ok ? *(const u32x4_t*)(qp + ks * 16) : u32x4_t{0, 0, 0, 0};
      qr[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  bf16x8_t qreg[KSTEPS];
  int pf_round = -1;  // the round whose Q and first tiles are already loaded
  int t0 = 0;         // tiles walked so far: ring slot of tile idx is t0 + idx
  // Optimistic softmax bookkeeping (ping-pong kernels): items are numbered
  // in the order they are walked (seq); a wave whose optimistic step fails
  // on an item records its number in s_fail, read by every wave after the
  // next barrier that follows the item (the next item's prologue, or the
  // end).  A failed item is walked again with exact steps only, as is every
  // later item of the workgroup (opt_ok).
  bool opt_ok = true;
  int seq = 0;
  int pending = -1, pending_round = 0;  // the item not yet checked, if any
  if (tid == 0) s_fail[0] = s_fail[1] = -1;
  auto pending_failed = [&]() -> bool {
    const bool f = pending >= 0 &&
                   __builtin_amdgcn_readfirstlane(s_fail[pending & 1]) == pending;
    pending = -1;
    return f;
  };
  for (int round = 0;; ++round) {
  if (round >= rounds) {
    // the last item's check; walk it again if it failed
    if (PP && pending >= 0) {
      const int pr = pending_round;
      __syncthreads();
      if (pending_failed()) {
        opt_ok = false;
        pf_round = -1;
        round = pr - 1;
        continue;
      }
    }
    break;
  }
  const int lid = lid_of(round);
  if (lid < 0) continue;
  const ItemGeo itg = item_geo(lid);
  const int b = itg.b, g = itg.g;
  const int h = head_of(itg);
  const int i0 = itg.i0, i1 = itg.i1, kl = itg.kl;
  const int prefix = itg.prefix, ql = itg.ql;
  const bool force_partial = itg.force_partial;
  const KvGeometry geo = itg.geo;
  const int pe = itg.pe;

  const size_t q_base = ((size_t)(b * H + h) * Sq) * D;
  const size_t kv_base = ((size_t)(b * Hkv + g) * Sk) * D;

  // ---- my query row ----
  const int qi = i0 + rb * 32 + lrow;  // global query row of this lane
  RowRange rr = row_range(qi, kl, causal, window, input_pos, prefix);
  int pe_row = pe;  // the row also sees the keys [0, pe_row)
  if (FLEX && qi >= ql) rr.lo = rr.hi = pe_row = 0;

  // the queries (and, without a block mask, the first tiles) are loaded
  const bool prefetched = PP && round == pf_round;
  if (!prefetched) load_q(qreg, itg);

  f32x16_t oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16_t{};
  float m_run = -INFINITY;  // running max (base-2 scaled domain)
  float l_run = 0.f;        // this lane's half of the running row sum

  // The tiles walked, in order: the item's walk, or (block-sparse) those
  // that some row block of the workgroup keeps, listed by wave 0, or (flex
  // with a block mask) those whose class is not empty for some row block of
  // the workgroup, listed by wave 0.
  int n_tiles = itg.nwalk;
  if constexpr (SPARSE) {
    const int nqb = (Sq + kSparseBlock - 1) / kSparseBlock;
    const int nkb = (Sk + kSparseBlock - 1) / kSparseBlock;
    const int qb0 = i0 / kSparseBlock;
    const uint8_t* krow = keep + ((size_t)(b * H + h) * nqb + qb0) * nkb;
    if (wave == 0) {
      int base = 0;
      for (int c0 = 0; c0 < n_tiles; c0 += 64) {
        const int t = c0 + lane;
        const int kt = itg.kt0 + t;
        unsigned bits = 0;
        if (t < n_tiles) {
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
  const bool use_bm = XM && fx.bmask != nullptr;
  if (XM && use_bm) {
    // (the first barrier: every wave is past its reads of the last list)
    __syncthreads();
    if (wave == 0) {
      const int nkb = (Sk + kFwdTileN - 1) / kFwdTileN;
      const int qb0 = i0 / kFwdTileN;
      const int nq = n_tiles > 0 ? (max(min(i1, ql), i0 + 1) - 1) / kFwdTileN - qb0 + 1 : 0;
      const uint8_t* brow = fx.bmask + b * fx.bm_bstride + (size_t)qb0 * nkb;
      int base = 0;
      for (int c0 = 0; c0 < n_tiles; c0 += 64) {
        const int t = c0 + lane;
        const int kt = walk_tile(itg, t);
        bool some = false, every = true;
        if (t < n_tiles) {
          for (int q = 0; q < nq; ++q) {
            const int c = brow[(size_t)q * nkb + kt];
            some |= c != ATTN_BLOCK_EMPTY;
            every &= c == ATTN_BLOCK_FULL;
          }
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(some);
        if (some) {
          const int at = base + __builtin_popcountll(m & ((1ull << lane) - 1));
          s_blist[at] = (int16_t)(kt | (every ? 0x8000 : 0));
        }
        base += __builtin_popcountll(m);
      }
      if (lane == 0) s_ntiles = base;
    }
    __syncthreads();
    n_tiles = s_ntiles;
  }
  auto tile_at = [&](int idx) -> int {
    if constexpr (SPARSE) return s_list[idx];
    if (XM && use_bm) return __builtin_amdgcn_readfirstlane((int)s_blist[idx]) & 0x7fff;
    return walk_tile(itg, idx);
  };
  // flex with a block mask: every pair of the idx-th walked tile is in the
  // same document
  auto bm_full = [&](int idx) {
    return XM && use_bm && __builtin_amdgcn_readfirstlane((int)s_blist[idx]) < 0;
  };
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
  const int nvalid = itg.vhi - itg.vlo;
  const size_t valid_base = kv_base + (size_t)itg.vlo * D;
  // one resource per tensor, both uniform: selecting between them per group
  // would make the resource divergent
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(K + valid_base), (short)0, nvalid * D * 2, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(V + valid_base), (short)0, nvalid * D * 2, kBufferRsrcWord3);

  // ---- direct-to-LDS staging (ping-pong kernels) ----
  // A tile's K rows are kInstrK instructions, its V rows kInstrV = kInstrK - 1.
  // Wave w issues the K instructions w + 8 t and the V instructions w + 8 t
  // (t < DMA_KV), and wave 0 also the last K instruction, so the sequence of
  // each wave is fixed and needs no branch.  Lane l of an instruction fills
  // the 16 bytes at the instruction's LDS address + 16 l, so each lane
  // fetches the chunk the layout puts in that slot: for K, slot s holds row
  // s / kChunksK, chunk s % kChunksK (the pad chunk re-reads the row's last
  // chunk); for V, row s / (D / 8) and the chunk the swizzle stores there.
  constexpr int NDMA = L::kInstrK + L::kInstrV;
  constexpr int DMA_KV = L::kInstrV / kFwdWaves;
  static_assert(L::kInstrV % kFwdWaves == 0 && L::kInstrK == L::kInstrV + 1,
                "every wave issues DMA_KV K and DMA_KV V instructions, wave 0 one more");
  auto k_off = [&](int n) {
    const int sl = n * 64 + lane;
    const int r = sl / L::kChunksK;
    const int c = min(sl % L::kChunksK, L::kChunksK - 2);
    return (r * D + c * 8) * 2;
  };
  auto v_off = [&](int n) {
    const int sl = n * 64 + lane;
    const int r = sl / (D / 8);
    const int c = (sl % (D / 8)) ^ v_swizzle<D>(r);
    return (r * D + c * 8) * 2;
  };
  int dma_koff[DMA_KV], dma_voff[DMA_KV];
#pragma unroll
  for (int t = 0; t < DMA_KV; ++t) {
    dma_koff[t] = k_off(wave + kFwdWaves * t);
    dma_voff[t] = v_off(wave + kFwdWaves * t);
  }
  const int dma_klast = k_off(L::kInstrK - 1);
  // V^T operand reads: lane l of a transposing read points at 4 d-values of
  // one row; per 32-wide d block db its offset inside a 16-row slice
  int vt_off[DBLK];
  {
    const int g4 = lane >> 4, j = lane & 15;
    const int rr = (g4 >> 1) * 4 + (j >> 2);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int d = db * 32 + (g4 & 1) * 16 + (j & 3) * 4;
      vt_off[db] = rr * L::kRowVd + (((d >> 3) ^ v_swizzle<D>(rr)) << 4) + (d & 7) * 2;
    }
  }

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
      has_doc ? (void*)(fx.doc_kv + (size_t)b * Sk + itg.vlo) : nullptr,
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
    const int rel0 = kt * kFwdTileN - itg.vlo;  // tile start, in valid keys
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

  // Direct-to-LDS loads of the idx-th walked tile into ring slots idx % kRingK
  // (K, document ids) and idx % kRingV (V).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const u32x4_t kdesc = buffer_desc_s(K + valid_base, nvalid * D * 2);
  const u32x4_t vdesc = buffer_desc_s(V + valid_base, nvalid * D * 2);
  const u32x4_t ddesc = buffer_desc_s(has_doc ? (const void*)(fx.doc_kv + (size_t)b * Sk + itg.vlo)
                                              : nullptr,
                                      has_doc ? nvalid * 4 : 0);
  // (kt: the key tile; slot: its place in the rings; ulo: the first key of
  // the range the descriptors cover)
  auto dma_issue = [&](const u32x4_t& kd, const u32x4_t& vd, const u32x4_t& dd, bool doc,
                       int ulo, int kt, int slot, bool fresh) {
    const int rel = (kt * kFwdTileN - ulo) * D * 2;  // in the valid range
    const uint32_t kdst = lds_addr_of(smem + (slot % L::kRingK) * L::kBytesK);
    const uint32_t vdst = lds_addr_of(smem + L::kOffVd + (slot % L::kRingV) * L::kBytesVd);
    // Descriptors built just before (the next item's first tiles) need the
    // full wait before the first load; in the mask-extension kernels the
    // compiler reloads descriptors spilled to vector lanes before each load.
    auto load = [&](bool full, const u32x4_t& d, uint32_t dst, int off) {
      if (full || XM) lds_load16(d, dst, off);
      else lds_load16_m0(d, dst, off);
    };
    load(fresh, kd, kdst + wave_u * 1024, dma_koff[0] + rel);
#pragma unroll
    for (int t = 1; t < DMA_KV; ++t)
      load(false, kd, kdst + (wave_u + kFwdWaves * t) * 1024, dma_koff[t] + rel);
#pragma unroll
    for (int t = 0; t < DMA_KV; ++t)
      load(false, vd, vdst + (wave_u + kFwdWaves * t) * 1024, dma_voff[t] + rel);
    if (wave_u == 0) load(false, kd, kdst + (L::kInstrK - 1) * 1024, dma_klast + rel);
    if (FLEX && doc && wave_u == kFwdWaves - 1 && lane < kFwdTileN / 4)
      lds_load16(dd, lds_addr_of(smem + L::kOffDocD + (slot % L::kRingV) * L::kBytesDoc),
                 (kt * kFwdTileN - ulo + lane * 4) * 4);
  };
  auto dma_tile = [&](int idx) {
    dma_issue(kdesc, vdesc, ddesc, has_doc, itg.vlo, tile_at(idx), t0 + idx, false);
  };
  // Wait until this wave's loads of the tile after the current one have
  // landed, leaving those of the tile after that in flight (loads complete in
  // order; every wave issues at least NDMA / 8 loads per tile; the flex
  // kernel's later bias loads only make the wait longer).
  auto dma_wait = [&](bool more_in_flight) {
    static_assert(NDMA / kFwdWaves == 4 || NDMA / kFwdWaves == 2, "wait counts");
    if (more_in_flight) {
      if constexpr (NDMA / kFwdWaves == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    // V^T operand i (< NPV) of the previous tile: two transposing reads, rows
    // kb2 * 32 + st * 16 + 8 h8 + the lane's row of its 16-row slice
    auto vt_operand = [&](const char* vb, int i) -> bf16x8_t {
      const int pr = i / DBLK, db = i % DBLK;
      i16x4_t part[2];
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8)
        part[h8] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(vb + vt_off[db] +
                                                        (pr * 16 + h8 * 8) * L::kRowVd));
      return __builtin_bit_cast(bf16x8_t,
                                __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    if (PP && !FLEX && do_pv && do_s) {
      const char* vb = smem + L::kOffVd + ((t0 + idx - 1) % L::kRingV) * L::kBytesVd;
      const char* kb = smem + ((t0 + idx) % L::kRingK) * L::kBytesK;
      constexpr int NPV = DBLK * 4;
      constexpr int NOP = NPV + 2 * KSTEPS;
      auto load_op = [&](int i) -> bf16x8_t {
        if (i < NPV) return vt_operand(vb, i);
        const int j = i - NPV, ks = j >> 1, kb2 = j & 1;
        return *(const bf16x8_t*)(kb + (kb2 * 32 + lrow) * L::kRowK + half * 16 + ks * 32);
      };
      bf16x8_t ring[kFwdOpDepth];
#pragma unroll
      for (int i = 0; i < kFwdOpDepth; ++i) ring[i] = load_op(i);
      s[0] = s[1] = f32x16_t{};
#pragma unroll
      for (int i = 0; i < NOP; ++i) {
        const bf16x8_t a = ring[i % kFwdOpDepth];
        if (i + kFwdOpDepth < NOP) ring[i % kFwdOpDepth] = load_op(i + kFwdOpDepth);
        if (i < NPV) {
          const int pr = i / DBLK, db = i % DBLK;
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, __builtin_bit_cast(bf16x8_t, pb[pr >> 1][pr & 1]), oacc[db], 0, 0, 0);
        } else {
          const int j = i - NPV, ks = j >> 1, kb2 = j & 1;
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[kb2], 0, 0, 0);
        }
      }
      // the LDS reads of the first operands, then one MFMA and the reads of
      // the operand kFwdOpDepth ahead alternately (two transposing reads per
      // V^T operand), then the last MFMAs (0x100 = LDS read, 0x008 = MFMA)
      {
        constexpr int first = (kFwdOpDepth < NPV ? kFwdOpDepth : NPV) * 2 +
                              (kFwdOpDepth > NPV ? kFwdOpDepth - NPV : 0);
        __builtin_amdgcn_sched_group_barrier(0x100, first, 0);
      }
#pragma unroll
      for (int i = 0; i < NOP - kFwdOpDepth; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kFwdOpDepth < NPV)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kFwdOpDepth, 0);
      asm volatile("" : "+v"(s[0]), "+v"(s[1]));
      return;
    }
    if (!PP && !FLEX && do_pv && do_s) {
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
      if constexpr (PP) {
        const char* vb = smem + L::kOffVd + ((t0 + idx - 1) % L::kRingV) * L::kBytesVd;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr)
#pragma unroll
          for (int db = 0; db < DBLK; ++db) {
            const bf16x8_t a = vt_operand(vb, pr * DBLK + db);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, __builtin_bit_cast(bf16x8_t, pb[pr >> 1][pr & 1]), oacc[db], 0, 0, 0);
          }
      } else {
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
    }
    if (FLEX && do_s && has_bias) bias_loads(idx);
    if (do_s) {
      const char* kb = smem + (PP ? (t0 + idx) % L::kRingK : idx & 1) * L::kBytesK;
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
  // With a soft-cap of at most 60 / log2(e) every base-2 score lies in
  // [-C, C], C = cap log2(e), and C serves as every row's running max from
  // the start: P <= 1, and P >= 2^-2C is still a normal number.
  const bool fixed_ref = FLEX && has_cap && fx.softcap * kLog2e <= 60.f;
  // optimistic softmax steps on this item (ALiBi raises the scores tile
  // after tile towards the diagonal: exact steps only, unless capped)
  const bool opt_item = opt_ok && (!(FLEX && has_alibi) || fixed_ref);
  // With C as the reference the transform yields the exponent's argument
  // directly: A - B / (e + 1) - C = -B / (e + 1), one product instead of an
  // FMA here and another in the softmax step.
  const bool pre_shift = opt_item && fixed_ref;
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
    if (has_cap && pre_shift) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(s[kb2][r]);
          s[kb2][r] = -cap_b * __builtin_amdgcn_rcpf(e + 1.f);
        }
    } else if (has_cap) {
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
    const char* db = smem + (PP ? L::kOffDocD + ((t0 + idx) % L::kRingV) * L::kBytesDoc
                                : L::kOffDoc + (idx & 1) * L::kBytesDoc) + half * 16;
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

  if (opt_item && fixed_ref) m_run = fx.softcap * kLog2e;
  // lanes of this wave whose P exceeded the optimistic bound (or was not a
  // number) on some tile of the item
  uint64_t fail_bits = 0;
  // m is raised when the tile max exceeds it by more than this (exact steps:
  // 2^8; optimistic steps: only a row without one takes its first max)
  const float raise_above = opt_item ? 1e30f : kLazyRescale;
  auto v_phase = [&](int idx) {
    if constexpr (PP) {
      // group A's V(idx) runs in window idx, group B's in window idx + 1:
      // both load the tile two windows ahead, first thing in the phase
      const int ahead = idx + 2 + grp;
      if (ahead < n_tiles) dma_tile(ahead);
    }
    const int kt = tile_at(idx);
    const int j0 = kt * kFwdTileN;
    if constexpr (FLEX) {
      if (transform) flex_scores(j0);
      if (has_doc && !bm_full(idx)) doc_mask(idx);
    }
    if constexpr (SPARSE) {
      // this wave's 64-row block drops the tile: no score, only the staging
      if (!wave_keeps(idx)) {
        if (idx + 1 < n_tiles) stash((idx + 1) & 1);
        if (idx + 2 < n_tiles) fetch(tile_at(idx + 2));
        return;
      }
    }
    int cls = tile_class(geo, j0, kFwdTileN);
    // beside a window, a tile inside the prefix is seen whole by every row
    if (XM && pe > 0)
      cls = j0 + kFwdTileN <= pe || cls == kTileFull ? kTileFull : kTilePartial;
    if (cls == kTilePartial || (FLEX && force_partial)) {
      // key j0 + half*4 + c is allowed iff c lies in [t_lo, t_lo + width);
      // c is a compile-time constant per register, so one subtract, one
      // unsigned compare and one select per score
      const int t_lo = rr.lo - (j0 + half * 4);
      const unsigned width = (unsigned)max(rr.hi - rr.lo, 0);
      if (XM && pe > 0) {
        // ... or c < t_pe (the prefix)
        const int t_pe = pe_row - (j0 + half * 4);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = kb2 * 32 + (r >> 2) * 8 + (r & 3);
            if ((unsigned)(c - t_lo) >= width && c >= t_pe) s[kb2][r] = -INFINITY;
          }
      } else {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = kb2 * 32 + (r >> 2) * 8 + (r & 3);
            if ((unsigned)(c - t_lo) >= width) s[kb2][r] = -INFINITY;
          }
      }
    }
    // The running max m.  Optimistic step (opt_item): a row takes its first
    // tile max as m and keeps it; the tile max is taken only while some row
    // of the wave has none yet.  Each row's result then depends only on its
    // own scores (tiles it sees nothing of change nothing), whichever tiles
    // the walk visits.  A P of a half row above kOptSum (checked below) makes
    // the item fail; it is walked again with exact steps: m raised whenever
    // the tile max exceeds it by more than 2^8 (P <= 256).
    // (with a fixed reference there is no max to take and nothing to rescale)
    if (!(FLEX && pre_shift)) {
      float mt = m_run;
      if (!opt_item || __builtin_amdgcn_ballot_w64(m_run == -INFINITY)) {
        // row max as a tree of three-input maxima (v_max3_f32)
        float m16[11];
#pragma unroll
        for (int t = 0; t < 10; ++t) {
          const int a = 3 * t, b = a + 1, c = a + 2;
          m16[t] = __builtin_fmaxf(__builtin_fmaxf(s[a >> 4][a & 15], s[b >> 4][b & 15]),
                                   s[c >> 4][c & 15]);
        }
        m16[10] = __builtin_fmaxf(s[1][14], s[1][15]);
        float mx = __builtin_fmaxf(__builtin_fmaxf(m16[0], m16[1]), m16[2]);
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, m16[3]), m16[4]);
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, m16[5]), m16[6]);
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, m16[7]), m16[8]);
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, m16[9]), m16[10]);
        mt = pair_max(mx) * sl2;
      }
      const bool need = mt > m_run + raise_above;
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
    }
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    // Wide schedule: only this wave of its SIMD runs vector work now, so the
    // latency of each dependent step must be covered by independent work:
    // all 32 exponents' arguments, then the 32 exponentials, then packing and
    // a tree of partial sums.
    // (scores already relative to a fixed reference need no shift)
    if (!(FLEX && pre_shift)) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb2][r] = __builtin_fmaf(s[kb2][r], sl2, -mref);
    }
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb2][r] = __builtin_amdgcn_exp2f(s[kb2][r]);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        pb[kb2][r >> 3][(r & 7) >> 1] = pack_bf16x2(s[kb2][r], s[kb2][r + 1]);
    float q16[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) q16[r] = s[0][r] + s[1][r];
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) q16[r] = q16[r] + q16[r + w];
    const float psum = q16[0];
    fail_bits |= __builtin_amdgcn_ballot_w64(!(psum <= kOptSum));
    l_run += psum;
    // Pin P here: left alone, the compiler sinks the exponentials past the
    // barrier into the next MFMA phase (their only user), which serialises
    // them with that phase's products instead of overlapping them with the
    // other group's.
    asm volatile("" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]),
                 "+v"(l_run));
    if constexpr (PP) {
    } else {
      if (idx + 1 < n_tiles) stash((idx + 1) & 1);
      if (idx + 2 < n_tiles) fetch(tile_at(idx + 2));
    }
  };

  if (PP && n_tiles == 0 && pending >= 0) {
    // (an item without tiles has no prologue barrier: one for the check)
    const int pr = pending_round;
    __syncthreads();
    if (pending_failed()) {
      opt_ok = false;
      pf_round = -1;
      round = pr - 1;
      continue;
    }
  }
  if (n_tiles > 0) {
    if constexpr (PP) {
      // prologue: the first two tiles (group B also the third) in LDS,
      // unless the previous item already loaded them
      const bool gb = __builtin_amdgcn_readfirstlane(tid >> 8) != 0;
      if (!prefetched || use_bm) {
        dma_tile(0);
        if (n_tiles > 1) dma_tile(1);
        if (gb && n_tiles > 2) dma_tile(2);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      // (a prefetched item's loads were waited for before the previous
      // item's stores, which need no wait)
      __syncthreads();
      // the previous item's check: if it failed, walk it again (this item's
      // loads have landed and nothing else of it has started)
      {
        const int pr = pending_round;
        if (pending_failed()) {
          opt_ok = false;
          pf_round = -1;
          round = pr - 1;
          continue;
        }
      }
    } else {
      // prologue: the first tile in LDS, the second in flight
      fetch(tile_at(0));
      stash(0);
      if (n_tiles > 1) fetch(tile_at(1));
      __syncthreads();
    }
    if constexpr (PP) {
      // One barrier per tile.  Both groups run M(0) V(0) M(1) V(1) ...;
      // group A ends window k with V(k), group B with M(k), so in window k
      // group A runs M(k) then V(k) while group B runs V(k-1) then M(k): at
      // the start of a window one wave of each SIMD feeds the matrix core
      // while the other runs the softmax, and they swap halfway.  Every LDS
      // buffer written in window k (K(k+1) by A, V(k) by B) was last read in
      // window k-1.
      const bool group_b = __builtin_amdgcn_readfirstlane(tid >> 8) != 0;
      for (int idx = 0; idx < n_tiles; ++idx) {
        __builtin_amdgcn_s_setprio(3);
        m_phase(idx, idx > 0, true);
        __builtin_amdgcn_s_setprio(0);
        // before a barrier, this wave's loads of the tile read in the next
        // window have landed
        if (group_b) {
          dma_wait(idx + 2 < n_tiles);
          __syncthreads();
        }
        v_phase(idx);
        if (!group_b) {
          dma_wait(idx + 2 < n_tiles);
          __syncthreads();
        }
      }
      // Start the next item: its queries into registers and its first tiles
      // into the ring slots after this item's.  Past the last barrier no wave
      // reads those slots again (the last product below reads only the slot
      // of this item's last V tile), and the next item's prologue barrier
      // orders them before the slots come round again.
      int nr = round + 1;
      while (nr < rounds && lid_of(nr) < 0) ++nr;
      ItemGeo nx;
      if (nr < rounds) {
        nx = item_geo(lid_of(nr));
        // (with a block mask the next item's tiles are known only once its
        // list is built)
        if (nx.nwalk > 0 && !use_bm) {
          const int nval = nx.vhi - nx.vlo;
          const size_t nbase = ((size_t)(nx.b * Hkv + nx.g) * Sk + nx.vlo) * D;
          const u32x4_t kd = buffer_desc_s(K + nbase, nval * D * 2);
          const u32x4_t vd = buffer_desc_s(V + nbase, nval * D * 2);
          const u32x4_t dd = buffer_desc_s(
              has_doc ? (const void*)(fx.doc_kv + (size_t)nx.b * Sk + nx.vlo) : nullptr,
              has_doc ? nval * 4 : 0);
          const int cnt = min(group_b ? 3 : 2, nx.nwalk);
          for (int t = 0; t < cnt; ++t)
            dma_issue(kd, vd, dd, has_doc, nx.vlo, walk_tile(nx, t), t0 + n_tiles + t, t == 0);
        }
        pf_round = nr;
        // (the queries: the last products below take none)
        load_q(qreg, nx);
      }
      m_phase(n_tiles, true, false);
    } else {
      for (int idx = 0; idx < n_tiles; ++idx) {
        m_phase(idx, idx > 0, true);
        __syncthreads();
        v_phase(idx);
        __syncthreads();
      }
      m_phase(n_tiles, true, false);
    }
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
    if constexpr (PP) {
      // The ping-pong kernels stage in an area of their own, half the head
      // dimension per pass, so neither the staging nor the next item's loads
      // into the rings wait for the other waves.
      char* ost = smem + L::kOffOs + wave * L::kBytesOWaveH;
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        if (hd) __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int dbh = 0; dbh < DBLK / 2; ++dbh)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int db = hd * (DBLK / 2) + dbh;
            const int d = dbh * 32 + r4 * 8 + half * 4;  // within the half
            u32x2_t w = {pack_bf16x2(oacc[db][r4 * 4 + 0] * inv,
                                     oacc[db][r4 * 4 + 1] * inv),
                         pack_bf16x2(oacc[db][r4 * 4 + 2] * inv,
                                     oacc[db][r4 * 4 + 3] * inv)};
            *(u32x2_t*)(ost + lrow * L::kRowOh + d * 2) = w;
          }
        __builtin_amdgcn_wave_barrier();
        // The next item's loads have landed before this item's stores go out
        // (the staging above overlapped them): a wait for them later would
        // wait for the stores as well (one counter for both on this
        // architecture).
        if (hd == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        constexpr int CHUNKS = D / 16;  // 16-byte chunks per half row
#pragma unroll
        for (int i = 0; i < 32 * CHUNKS / 64; ++i) {
          const int c = i * 64 + lane;
          const int row = c / CHUNKS, ch = c - row * CHUNKS;
          const u32x4_t v = *(const u32x4_t*)(ost + row * L::kRowOh + ch * 16);
          const int qrow = i0 + rb * 32 + row;
          if (qrow < Sq)
            *(u32x4_t*)(O + q_base + (size_t)qrow * D + hd * (D / 2) + ch * 8) = v;
        }
      }
    } else {
    // (without groups the staging area is the K/V rings, free once every
    // wave is past its last products)
    __syncthreads();
    char* ost = smem + wave * L::kBytesOWave;
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
      const int qrow = i0 + rb * 32 + row;
      if (qrow < Sq) *(u32x4_t*)(O + q_base + (size_t)qrow * D + ch * 8) = v;
    }
    }
  }
  if (LSE && qi < Sq && half == 0) {
    const float lse = l_tot > 0.f
                          ? (m_run + __builtin_log2f(l_tot)) * 0.69314718055994530942f
                          : -INFINITY;
    LSE[(size_t)(b * H + h) * Sq + qi] = lse;
  }
  // (a P above the optimistic bound, or not a number: the item fails)
  if (opt_item && fail_bits != 0 && lane == 0) s_fail[seq & 1] = seq;
  if constexpr (PP) {
    // (checked after the next barrier)
    if (opt_item && n_tiles > 0) {
      pending = seq;
      pending_round = round;
    }
    ++seq;
    t0 = __builtin_amdgcn_readfirstlane(t0 + n_tiles);
  } else {
    __syncthreads();  // LDS is reused by the next item
    // (the item's check: every wave is past its softmax steps)
    if (opt_item) {
      pending = seq++;
      if (pending_failed()) {
        opt_ok = false;
        --round;
        continue;
      }
    }
  }
  }
}

// Number of persistent workgroups for `total` items (per_cu per CU, a
// multiple of 8), or 0 for a launch of one workgroup per item when there are
// too few items to pair up.
static int persistent_workgroups(long long total, int per_cu = 1) {
  const int n_wg = (device_cu_count() / 8) * 8 * per_cu;
  if (n_wg < 8 || total < 2LL * n_wg) return 0;
  return n_wg;
}

static void log_fwd_grid(const char* kernel, int D, unsigned grid, int threads,
                         long long items, int n_wg) {
  if (log_enabled())
    log_line("  %s<D=%d> grid=%u threads=%d items=%lld %s", kernel, D, grid, threads,
             items, n_wg > 0 ? "persistent" : "one workgroup per item");
}

template <int D>
hipError_t launch_fwd_bf16(void* O, const void* Q, const void* K,
                           const void* V, float* LSE, int B, int H, int Hkv,
                           int Sq, int Sk, int causal, int window,
                           int input_pos, const int32_t* k_lengths,
                           hipStream_t stream) {
  const int hl = fwd_heads_log2(H / Hkv);
  const int nqt = (Sq + (kFwdTileM >> hl) - 1) / (kFwdTileM >> hl);
  const long long total = (long long)nqt * (H >> hl) * B;
  const int n_wg = persistent_workgroups(total);
  const unsigned grid = n_wg > 0 ? (unsigned)n_wg : (unsigned)total;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  log_fwd_grid("attn_fwd_bf16_kernel", D, grid, kFwdThreads, total, n_wg);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, false, false>), dim3(grid),
                     dim3(kFwdThreads), 0, stream, (__bf16*)O,
                     (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, LSE,
                     B, H, Hkv, Sq, Sk, causal, window, input_pos, k_lengths,
                     scale_log2, FlexArgs{}, (const uint8_t*)nullptr, n_wg, hl);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_flex(void* O, const void* Q, const void* K,
                           const void* V, float* LSE, int B, int H, int Hkv,
                           int Sq, int Sk, int causal, int window,
                           int input_pos, const int32_t* k_lengths,
                           const attn_flex_t* f, hipStream_t stream) {
  const int hl = fwd_heads_log2(H / Hkv);
  const int nqt = (Sq + (kFwdTileM >> hl) - 1) / (kFwdTileM >> hl);
  const long long total = (long long)nqt * (H >> hl) * B;
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
  fx.bmask = f->block_mask;
  fx.bm_bstride = f->block_mask && f->block_mask_B > 1
                      ? (long long)((Sq + kFwdTileN - 1) / kFwdTileN) *
                            ((Sk + kFwdTileN - 1) / kFwdTileN)
                      : 0;
  fx.softcap = f->softcap;
  fx.qk_scale = f->qk_scale > 0.f ? f->qk_scale : 1.f / sqrtf((float)D);
  log_fwd_grid(fx.bias ? "attn_fwd_bf16_kernel[flex+bias]" : "attn_fwd_bf16_kernel[flex]", D,
               grid, kFwdThreads, total, n_wg);
  if (log_enabled() && (fx.bmask || (fx.prefix > 0 && window > 0)))
    log_line("  (mask extensions: %s)", fx.bmask ? "block mask" : "prefix beside a window");
  // the bias tile costs 32 registers per lane, the mask extensions some
  // more: kernels of their own
  const bool xm = fx.bmask != nullptr || (fx.prefix > 0 && window > 0);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kFwdThreads), 0, stream, (__bf16*)O,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, LSE,
                       B, H, Hkv, Sq, Sk, causal, window, input_pos, k_lengths,
                       0.f, fx, (const uint8_t*)nullptr, n_wg, hl);
  };
  if (fx.bias)
    xm ? go(attn_fwd_bf16_kernel<D, true, true, false, true>)
       : go(attn_fwd_bf16_kernel<D, true, true, false, false>);
  else
    xm ? go(attn_fwd_bf16_kernel<D, true, false, false, true>)
       : go(attn_fwd_bf16_kernel<D, true, false, false, false>);
  return hipGetLastError();
}

// ---- BlockMask of a flex mask (Tylo.jl "Primitives", BlockMask /
// build_block_mask) ----
// One wave per (batch, query block, key block): lane l holds key kb * 64 + l
// and the wave walks the block's rows, testing every pair with the flex
// mask's own predicate (causal / window at absolute positions, OR the
// prefix, AND the key and query lengths, AND equal document ids).
__global__ __launch_bounds__(256) void attn_build_block_mask_kernel(
    uint8_t* __restrict__ out, int B, int Sq, int Sk, int causal, int window,
    int input_pos, const int32_t* __restrict__ k_lengths,
    const int32_t* __restrict__ q_lengths, const int32_t* __restrict__ doc_q,
    const int32_t* __restrict__ doc_kv, int prefix) {
  const int nqb = (Sq + kFwdTileN - 1) / kFwdTileN;
  const int nkb = (Sk + kFwdTileN - 1) / kFwdTileN;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long long)B * nqb * nkb) return;
  const int lane = threadIdx.x & 63;
  const int kb = (int)(w % nkb);
  const int qb = (int)((w / nkb) % nqb);
  const int b = (int)(w / ((long long)nkb * nqb));
  const int kl = k_lengths ? min(max(k_lengths[b], 0), Sk) : Sk;
  const int ql = q_lengths ? min(max(q_lengths[b], 0), Sq) : Sq;
  const int j = kb * kFwdTileN + lane;
  const bool key_exists = j < Sk;
  const uint64_t exists = __builtin_amdgcn_ballot_w64(key_exists);
  const int r_end = min(kFwdTileN, Sq - qb * kFwdTileN);
  const int i_lane = qb * kFwdTileN + lane;  // this lane's row, for the row-side loads
  const int dkv = doc_kv && key_exists ? doc_kv[(size_t)b * Sk + j] : 0;
  const int dq_lane = doc_q && lane < r_end ? doc_q[(size_t)b * Sq + i_lane] : 0;
  // Quick rejections, each a sufficient condition for no attending pair: no
  // live row or key, or (documents) disjoint ranges of document ids.
  bool empty = qb * kFwdTileN >= ql || kb * kFwdTileN >= kl;
  if (doc_q && !empty) {
    int qmin = lane < r_end ? dq_lane : INT_MAX, qmax = lane < r_end ? dq_lane : INT_MIN;
    int kmin = key_exists ? dkv : INT_MAX, kmax = key_exists ? dkv : INT_MIN;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      qmin = min(qmin, __shfl_xor(qmin, o));
      qmax = max(qmax, __shfl_xor(qmax, o));
      kmin = min(kmin, __shfl_xor(kmin, o));
      kmax = max(kmax, __shfl_xor(kmax, o));
    }
    empty = qmax < kmin || kmax < qmin;
  }
  bool some = false, every = !empty;
  for (int r = 0; r < r_end && !empty; ++r) {
    const int i = qb * kFwdTileN + r;
    const long long p = (long long)input_pos + i;
    bool ok = (!causal || j <= p) && (window <= 0 || j >= p - window + 1);
    ok = (ok || j < prefix) && j < kl && i < ql;
    if (doc_q) ok = ok && __builtin_amdgcn_readlane(dq_lane, r) == dkv;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ok && key_exists);
    some |= m != 0;
    every &= m == exists;
    if (some && !every) break;
  }
  if (lane == 0)
    out[w] = some ? (every ? ATTN_BLOCK_FULL : ATTN_BLOCK_PARTIAL) : ATTN_BLOCK_EMPTY;
}

hipError_t launch_build_block_mask(uint8_t* out, int B, int Sq, int Sk, int causal,
                                   int window, int input_pos, const int32_t* k_lengths,
                                   const attn_flex_t* f, hipStream_t stream) {
  const long long n = (long long)B * ((Sq + kFwdTileN - 1) / kFwdTileN) *
                      ((Sk + kFwdTileN - 1) / kFwdTileN);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 3) / 4);
  if (log_enabled())
    log_line("  attn_build_block_mask_kernel grid=%u threads=256 blocks=%lld", grid, n);
  hipLaunchKernelGGL(attn_build_block_mask_kernel, dim3(grid), dim3(256), 0, stream, out, B,
                     Sq, Sk, causal, window, input_pos, k_lengths, f->q_lengths, f->doc_q,
                     f->doc_kv, f->prefix);
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
  log_fwd_grid("attn_fwd_bf16_kernel[block-sparse]", D, grid, NT, total, n_wg);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false, false, true>), dim3(grid),
                     dim3(NT), 0, stream, (__bf16*)O,
                     (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, LSE,
                     B, H, Hkv, Sq, Sk, causal, window, input_pos, k_lengths,
                     scale_log2, FlexArgs{}, keep, n_wg, 0);
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
