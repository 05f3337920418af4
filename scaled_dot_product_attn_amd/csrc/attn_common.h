// Device-side helpers shared by the attention kernels: the mask predicate in
// interval form, the per-workgroup key geometry and the tile classifier.
//
// Mask (mlx-arsenal "Attention": causal_mask / sliding_window_mask;
// Tylo.jl "Primitives": CausalMask, attention! keywords input_pos and
// k_lengths): query row i at absolute position p = input_pos + i may attend to
// key j iff j < kl, (causal => j <= p) and (window > 0 => j >= p - window + 1).
// For one row that is the half-open interval [lo, hi) with
//   lo = clamp(p - window + 1, 0, kl)   (0 without a window)
//   hi = clamp(p + 1, 0, kl)            (kl without causal masking)
// and both ends are non-decreasing in i.  The flex prefix (Tylo.jl
// "Primitives", PrefixMask / prefix_lm = CausalMask | PrefixMask) ORs keys
// j < prefix into a causal row without a window, which keeps the row one
// interval: hi = clamp(max(p + 1, prefix), 0, kl).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

enum TileClass : int8_t { kTileEmpty = 0, kTilePartial = 1, kTileFull = 2 };

struct RowRange {
  int lo;  // first allowed key
  int hi;  // one past the last allowed key; the row is empty when lo >= hi
};

__host__ __device__ inline int clamp_i64(long long x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : (int)x);
}

__host__ __device__ inline RowRange row_range(int i, int kl, int causal,
                                              int window, int input_pos,
                                              int prefix = 0) {
  long long p = (long long)input_pos + i;
  RowRange r;
  const long long reach = p + 1 > prefix ? p + 1 : (long long)prefix;
  r.hi = causal ? clamp_i64(reach, 0, kl) : kl;
  r.lo = window > 0 ? clamp_i64(p - window + 1, 0, kl) : 0;
  return r;
}

// Key geometry of the query rows [i0, i1) of one workgroup.
//   any       : some row has an allowed key
//   union_lo/hi: allowed keys of the rows, together, are exactly
//               [union_lo, union_hi).  (Per-row intervals have non-decreasing
//               ends moving by at most one per row, and empty rows only occur
//               before or after the non-empty ones, so the union has no gap.)
//   all_lo/hi : keys every row allows are [all_lo, all_hi) (empty if
//               all_lo >= all_hi); all_lo = lo of the last row, all_hi = hi of
//               the first row.
struct KvGeometry {
  int any;
  int union_lo, union_hi;
  int all_lo, all_hi;
};

// Closed form from the monotone row ends.  A row is non-empty iff kl > 0,
// p >= 0 when causal without a prefix (earlier rows have hi = 0) and
// p <= kl + window - 2 when windowed (later rows have lo = kl).  So the
// non-empty rows are [a, b] with
//   a = max(i0, -input_pos) (causal, no prefix) and b = min(i1 - 1, kl +
//   window - 2 - input_pos) (window),
// and the union of their intervals runs from lo(a) to hi(b).  (A prefix is
// only taken without a window.)
__host__ __device__ inline KvGeometry kv_geometry(int i0, int i1, int kl,
                                                  int causal, int window,
                                                  int input_pos,
                                                  int prefix = 0) {
  KvGeometry g;
  RowRange first = row_range(i0, kl, causal, window, input_pos, prefix);
  RowRange last = row_range(i1 - 1, kl, causal, window, input_pos, prefix);
  g.all_lo = last.lo;
  g.all_hi = first.hi;
  long long a = i0, b = (long long)i1 - 1;
  if (causal && prefix <= 0 && -(long long)input_pos > a)
    a = -(long long)input_pos;
  if (window > 0) {
    long long lb = (long long)kl + window - 2 - input_pos;
    if (lb < b) b = lb;
  }
  if (kl <= 0 || a > b) {
    g.any = 0;
    g.union_lo = g.union_hi = 0;
    return g;
  }
  g.any = 1;
  g.union_lo = row_range((int)a, kl, causal, window, input_pos, prefix).lo;
  g.union_hi = row_range((int)b, kl, causal, window, input_pos, prefix).hi;
  return g;
}

// Query heads a prefill workgroup serves, as log2: the largest power of two
// up to 8 that divides the group size G = H / Hkv.  The workgroup's 256 rows
// are then 256 >> log2 query positions of that many heads of one KV head,
// which read the same K/V tiles.
__host__ __device__ inline int fwd_heads_log2(int G) {
  int l = 0;
  while (l < 3 && G % (2 << l) == 0) ++l;
  return l;
}

// Class of the key tile [j0, j0 + tile_n) for the rows described by g.
__host__ __device__ inline int tile_class(const KvGeometry& g, int j0,
                                          int tile_n) {
  if (!g.any || j0 >= g.union_hi || j0 + tile_n <= g.union_lo)
    return kTileEmpty;
  if (j0 >= g.all_lo && j0 + tile_n <= g.all_hi) return kTileFull;
  return kTilePartial;
}

}  // namespace attn
