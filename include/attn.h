/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention library
 * (libattn_mi355x.so).
 *
 * Operations, as the pages define them:
 *
 *   O = softmax(scale * Q K^T + mask) V,  scale = 1/sqrt(D)
 *
 * (Tylo.jl "Primitives": attention! -- fused multi-head attention with GQA,
 * causal, input_pos, k_lengths, saved softmax statistics M/L, Float32
 * accumulation; flex_attention! -- qk_scale = 1/sqrt(Dk) and "Heads must be a
 * multiple of Heads_KV"; decode_attention! -- split-KV single-query decode;
 * mlx-arsenal "Attention": causal_mask / sliding_window_mask, additive masks
 * with -inf at blocked positions; vllm_mlx.attention: MLXAttentionImpl.forward
 * computing scaled_dot_product_attention(q, k, v, scale).)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts: all tensors are contiguous, row-major.
 *   prefill  Q, O : (B, H,   Sq, D)      K, V : (B, Hkv, Sk, D)
 *            LSE  : (B, H, Sq) float32
 *   decode   Q, O : (B, H, D)            K, V : (B, Hkv, Smax, D)
 * (Tylo's column-major (D, S, H, B) read in row-major order.)
 *
 * Heads: H must be a multiple of Hkv; query head h reads KV head
 *   h / (H / Hkv) (contiguous groups).
 *
 * Mask: query row i sits at absolute position p = input_pos + i and may attend
 *   to key j iff   j < kl                                (k_lengths)
 *             and (causal == 0 or j <= p)                (CausalMask: q >= kv)
 *             and (window <= 0 or j >= p - window + 1)   (at most `window`
 *                                           previous positions, itself included)
 *   where kl = clamp(k_lengths[b], 0, Sk), or Sk when k_lengths is NULL.
 *   A window requires causal = 1.  Blocked pairs contribute exactly nothing
 *   (masked K/V values are never multiplied into the result).
 *   A row with no allowed key gets O = 0 and LSE = -inf.
 *
 * LSE: natural-log row logsumexp of the masked scaled scores (M + ln L in
 *   the pages' M/L terms), float32.  Pass NULL to skip it.
 *
 * Ownership: every pointer is a caller-owned DEVICE pointer (except where
 *   stated); the library keeps none after the call returns.  Work is enqueued
 *   asynchronously on `stream` (0 = the null stream); inputs and outputs must
 *   stay alive until the stream has passed it.  No entry point synchronises,
 *   and the host never reads device arrays (k_lengths, lengths).  Calls from
 *   several host threads are safe, except overlapping attn_decode_static
 *   calls on one GPU (they share its static scratch).
 *
 * Errors: every int-returning entry point returns
 *   ATTN_OK (0), ATTN_EINVAL (1, a bad argument: shape, H % Hkv, window
 *   without causal, n_splits < 1, a NULL required pointer, too small a
 *   workspace), ATTN_EUNSUPPORTED (2, D not in {64, 128}, or sizes beyond the
 *   32-bit index range), or ATTN_EHIP (3, a HIP launch or allocation error;
 *   the HIP error is cleared).  Nothing is enqueued when an argument check
 *   fails.  attn_status_string() names a code.
 *
 * Logging: off by default, nothing is printed.  With ATTN_LOG=1 in the
 *   environment (read once, at the first call) every entry point prints one
 *   line to stderr with its sizes, flags and returned status, and each kernel
 *   launch prints its grid, in the spirit of the debug logging the
 *   vllm_mlx.attention backend does through its module logger.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_EINVAL 1
#define ATTN_EUNSUPPORTED 2
#define ATTN_EHIP 3

/* Prefill tile sizes used by attn_fwd (query rows per workgroup, counted
 * over the query heads it serves, and keys per K/V tile); attn_tile_plan
 * reports the plan at these sizes. */
#define ATTN_FWD_TILE_M 256
#define ATTN_FWD_TILE_N 64

/* Prefill forward, bfloat16 Q/K/V/O, float32 accumulation and LSE.
 *   O         out (B, H, Sq, D) bf16
 *   Q         in  (B, H, Sq, D) bf16
 *   K, V      in  (B, Hkv, Sk, D) bf16
 *   LSE       out (B, H, Sq) float32, or NULL
 *   B, H, Hkv, Sq, Sk   >= 1 (Sq or Sk = 0 is a no-op returning ATTN_OK)
 *   D         64 or 128
 *   causal    0 or 1
 *   window    <= 0: none; > 0: sliding window (requires causal = 1)
 *   input_pos absolute position of query row 0 (any int)
 *   k_lengths device int32 (B,), or NULL (= Sk for every batch)
 * Defined by: Tylo.jl "Primitives", attention! (layouts, GQA, input_pos,
 * k_lengths, checkpoints M/L, Float32 accumulation); mlx-arsenal "Attention",
 * causal_mask and sliding_window_mask (offset, window, -inf masking). */
int attn_fwd(void* O, const void* Q, const void* K, const void* V, float* LSE,
             int B, int H, int Hkv, int Sq, int Sk, int D, int causal,
             int window, int input_pos, const int32_t* k_lengths,
             hipStream_t stream);

/* Prefill forward, float32 Q/K/V/O, exact float32 products (no reduced
 * precision inside).  Same arguments and semantics as attn_fwd; the element
 * type is carried by the symbol.  Defined by: Tylo.jl "Primitives",
 * attention! (compute precision follows the element type of Q). */
int attn_fwd_f32(void* O, const void* Q, const void* K, const void* V,
                 float* LSE, int B, int H, int Hkv, int Sq, int Sk, int D,
                 int causal, int window, int input_pos,
                 const int32_t* k_lengths, hipStream_t stream);

/* Flex variants of the bf16 prefill (Tylo.jl "Primitives", flex_attention!
 * and its mods).  Every pointer is a caller-owned device pointer or NULL (mod
 * off); a zeroed struct is plain attention.
 *   q_lengths     int32 (B,): query rows i >= q_lengths[b] (clamped to
 *                 [0, Sq]) attend to nothing: O = 0, LSE = -inf (q_lengths)
 *   alibi_slopes  float32 (H,): adds slopes[h] * (q - kv) to the score, q the
 *                 absolute query position input_pos + i, kv the key position
 *                 (AliBiScore)
 *   bias          float32 (bias_B, bias_H, Sq, Sk) row-major, added to the
 *                 score; bias_B in {1, B} and bias_H in {1, H}, a size of 1
 *                 broadcasting; indexed by the local query row (BiasScore).
 *                 Requires (Sq * Sk + Sk) * 4 + 256 <= INT_MAX.
 *   doc_q, doc_kv int32 (B, Sq) and (B, Sk): a pair attends only if
 *                 doc_q[b][i] == doc_kv[b][j] (DocumentMask(doc_q, doc_kv));
 *                 both or neither
 *   prefix        >= 0: keys j < prefix are visible to every query in addition
 *                 to the causal / window set (PrefixMask; causal + prefix is
 *                 prefix_lm; with a window a row sees the prefix and its
 *                 window, two key intervals: PrefixMask | SlidingWindowMask)
 *   softcap       0: off; > 0: score -> softcap * tanh(score / softcap),
 *                 applied after bias and ALiBi (SoftCapScore)
 *   qk_scale      0: 1/sqrt(D); > 0: the scale applied to q.k (qk_scale)
 *   block_mask    uint8 (block_mask_B, ceil(Sq / ATTN_BLOCK), ceil(Sk /
 *                 ATTN_BLOCK)) row-major, block_mask_B in {1, B}: the coarse
 *                 class of each (query block, key block) under the whole mask
 *                 (BlockMask): ATTN_BLOCK_EMPTY blocks are skipped,
 *                 ATTN_BLOCK_FULL blocks take no document mask, other values
 *                 are masked element by element.  Query block qb is the local
 *                 rows [qb * ATTN_BLOCK, (qb + 1) * ATTN_BLOCK).  The classes
 *                 must agree with the mask (an EMPTY block with an attending
 *                 pair, or a FULL one with a blocked document pair, gives
 *                 wrong results); attn_build_block_mask writes them.  Needs
 *                 ceil(Sk / ATTN_BLOCK) <= ATTN_SPARSE_MAX_KEY_BLOCKS.
 * The score is qk_scale * q.k, plus bias, plus ALiBi, then soft-capped; blocked
 * pairs (causal / window / k_lengths / q_lengths / documents, OR the prefix)
 * contribute nothing. */
typedef struct attn_flex {
  const int32_t* q_lengths;
  const float* alibi_slopes;
  const float* bias;
  const int32_t* doc_q;
  const int32_t* doc_kv;
  int bias_B, bias_H;
  int prefix;
  float softcap;
  float qk_scale;
  const uint8_t* block_mask;
  int block_mask_B;
} attn_flex_t;

/* Classes of a BlockMask entry (Tylo.jl "Primitives", BlockMask): no pair
 * of the (query block, key block) attends, some do, or all do. */
#define ATTN_BLOCK_EMPTY 0
#define ATTN_BLOCK_PARTIAL 1
#define ATTN_BLOCK_FULL 2

/* attn_fwd with the flex mods of *flex (NULL = none), bf16 only.  Same
 * arguments, layouts and errors as attn_fwd, plus ATTN_EINVAL for a bad
 * flex field (softcap or qk_scale < 0, prefix < 0, bias_B / bias_H not 1 or
 * B / H, doc_q without doc_kv or the reverse, block_mask_B not 1 or B) and
 * ATTN_EUNSUPPORTED for a block mask past ATTN_SPARSE_MAX_KEY_BLOCKS key
 * blocks.  Defined by: Tylo.jl
 * "Primitives", flex_attention! (score_mod, mask_mod, qk_scale, q_lengths),
 * SoftCapScore, AliBiScore, BiasScore, PrefixMask, prefix_lm, DocumentMask. */
int attn_fwd_flex(void* O, const void* Q, const void* K, const void* V,
                  float* LSE, int B, int H, int Hkv, int Sq, int Sk, int D,
                  int causal, int window, int input_pos,
                  const int32_t* k_lengths, const attn_flex_t* flex,
                  hipStream_t stream);

/* BlockMask of the flex mask of these arguments, on the device (the
 * predicate build_block_mask takes, evaluated at every pair): writes
 * block_mask, uint8 (B, ceil(Sq / ATTN_BLOCK), ceil(Sk / ATTN_BLOCK)), with
 * ATTN_BLOCK_EMPTY where no pair of the block attends, ATTN_BLOCK_FULL where
 * every existing pair does (rows < Sq, keys < Sk) and ATTN_BLOCK_PARTIAL
 * otherwise.  The pair mask is that of attn_fwd_flex: causal / window at
 * absolute query positions input_pos + i, OR keys j < prefix, AND j <
 * k_lengths[b], AND i < q_lengths[b], AND doc_q[b][i] == doc_kv[b][j]; the
 * score fields and block_mask of *flex are ignored.  The output can be
 * passed as flex->block_mask (block_mask_B = B) with the same arguments.
 * Errors: ATTN_EINVAL for a NULL block_mask with Sq, Sk > 0 or a bad
 * argument (as attn_fwd_flex), ATTN_EUNSUPPORTED past
 * ATTN_SPARSE_MAX_KEY_BLOCKS key blocks.  Defined by: Tylo.jl "Primitives",
 * BlockMask and build_block_mask (block classes from a keep predicate that
 * agrees with the device mask_mod; TILE_M = TILE_N = 64). */
int attn_build_block_mask(uint8_t* block_mask, int B, int Sq, int Sk,
                          int causal, int window, int input_pos,
                          const int32_t* k_lengths, const attn_flex_t* flex,
                          hipStream_t stream);

/* Bytes of scratch attn_bwd needs (two float32 values per query row),
 * host-only; 0 for invalid sizes. */
size_t attn_bwd_workspace_bytes(int B, int H, int Sq, int D);

/* Backward of attn_fwd (bf16): input gradients from the output gradient.
 *   dQ        out (B, H, Sq, D) bf16
 *   dK, dV    out (B, Hkv, Sk, D) bf16 (overwritten; keys no query may see
 *             get 0)
 *   dO        in  (B, H, Sq, D) bf16, the output gradient
 *   Q, K, V   in  the forward's inputs
 *   O, LSE    in  the forward's output and its float32 row LSE (attn_fwd with
 *             LSE != NULL); rows with LSE = -inf contribute nothing
 *   B .. k_lengths: as attn_fwd and equal to the forward's
 *   workspace NULL: allocated stream-ordered on `stream`; else a caller buffer
 *             of ws_bytes >= attn_bwd_workspace_bytes(B, H, Sq, D), 256-byte
 *             aligned, not shared by concurrent calls
 * With S = Q K^T / sqrt(D) + mask and P = exp(S - LSE):
 *   dV = P^T dO, dS = P * (dO V^T - rowsum(dO * O)), dQ = dS K / sqrt(D),
 *   dK = dS^T Q / sqrt(D); a KV head's dK / dV sum over its query heads.
 * Float32 accumulation; P and dS are rounded to bf16 as matrix-core operands.
 * Errors as attn_fwd, plus ATTN_EINVAL for a NULL gradient, dO or LSE, or too
 * small / misaligned a workspace.  Defined by: Tylo.jl "Primitives",
 * ∇attention! (gradients from Ō, the primals, O and the checkpoints M/L;
 * scratch workspace; causal / input_pos matching the forward). */
int attn_bwd(void* dQ, void* dK, void* dV, const void* dO, const void* Q,
             const void* K, const void* V, const void* O, const float* LSE,
             int B, int H, int Hkv, int Sq, int Sk, int D, int causal,
             int window, int input_pos, const int32_t* k_lengths,
             void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- block-sparse prefill (mlx-arsenal "Radius-bounded block scores (RBS)")
 * Blocks are ATTN_BLOCK tokens on both sides; a block mask is uint8
 * (B, H, nqb, nkb) with nqb = ceil(Sq / ATTN_BLOCK), nkb = ceil(Sk /
 * ATTN_BLOCK), nonzero = keep. */
#define ATTN_BLOCK 64
#define ATTN_SPARSE_MAX_KEY_BLOCKS 2048
#define ATTN_BLOCK_SCORES_RBS 0
#define ATTN_BLOCK_SCORES_MINMAX 1
#define ATTN_BLOCK_MASK_RELATIVE 0
#define ATTN_BLOCK_MASK_TOPK 1
#define ATTN_BLOCK_MASK_BAND 2

/* Scratch bytes attn_block_scores needs (host-only); 0 for invalid sizes. */
size_t attn_block_scores_workspace_bytes(int B, int Hkv, int Sk, int D);

/* Block scores from bf16 Q (B, H, Sq, D) and K (B, Hkv, Sk, D), float32 out
 * (B, H, nqb, nkb): for each query token and key block a logit, then the log
 * of the sum of exp over the query block's tokens.
 *   kind ATTN_BLOCK_SCORES_RBS: base = q.c / sqrt(D) (c the key block's
 *     centroid) and, if `rescue` is not NULL, rescue = (q.c + ||q|| r beta) /
 *     sqrt(D) with r the block radius max ||k - c|| and beta = clip((r - r_lo)
 *     / (r_hi - r_lo), 0, 1), r_lo / r_hi the `low` / `high` quantiles (linear
 *     interpolation) of the KV head's block radii (beta = [r > r_lo] when they
 *     coincide); the page uses low = 0.5, high = 0.9;
 *   kind ATTN_BLOCK_SCORES_MINMAX: base = sum_d max(q_d lo_d, q_d hi_d) /
 *     sqrt(D) (element-wise min / max of the key block), rescue unused.
 * workspace: NULL = allocated stream-ordered, else >=
 * attn_block_scores_workspace_bytes bytes, 256-byte aligned.  Errors as
 * attn_fwd; ATTN_EUNSUPPORTED past 4096 key blocks.  Defined by:
 * mlx-arsenal "Radius-bounded block scores (RBS)" (the idea, the formulas,
 * radius_bounded_block_scores, the min/max box bound). */
int attn_block_scores(float* base, float* rescue, const void* Q, const void* K,
                      int B, int H, int Hkv, int Sq, int Sk, int D, int kind,
                      float low, float high, void* workspace, size_t ws_bytes,
                      hipStream_t stream);

/* Block mask rows from block scores: `rows` = B * H * nqb rows of nkb entries.
 *   mode ATTN_BLOCK_MASK_RELATIVE: keep score >= row max + ln(alpha), alpha in
 *     (0, 1] (relative_block_mask: within alpha of the row maximum);
 *   mode ATTN_BLOCK_MASK_TOPK: keep the k best of each row, ties to the lower
 *     block index (top_k_block_mask);
 *   mode ATTN_BLOCK_MASK_BAND: keep |row block - key block| < diagonal (the
 *     recipe's forced band; `scores` may be NULL);
 * accumulate != 0 ORs into `keep` instead of overwriting (the recipe's union
 * of branches).  Defined by: mlx-arsenal "Radius-bounded block scores (RBS)",
 * relative_block_mask, top_k_block_mask and the rbs_block_mask recipe. */
int attn_block_mask(uint8_t* keep, const float* scores, int rows, int nqb,
                    int nkb, int mode, float alpha, int k, int diagonal,
                    int accumulate, hipStream_t stream);

/* attn_fwd restricted to the kept blocks of `keep` (B, H, nqb, nkb) uint8, on
 * top of the causal / window / k_lengths mask (a pair counts iff both allow
 * it).  Key tiles no row block of a 256-row workgroup keeps are never read.
 * A row whose blocks keep nothing gets O = 0, LSE = -inf.  ATTN_EUNSUPPORTED
 * past ATTN_SPARSE_MAX_KEY_BLOCKS key blocks.  Defined by: mlx-arsenal
 * "Radius-bounded block scores (RBS)" (the block mask expanded to tokens);
 * Tylo.jl "Primitives", flex_attention! block_mask (precomputed block
 * sparsity). */
int attn_fwd_block_sparse(void* O, const void* Q, const void* K, const void* V,
                          float* LSE, int B, int H, int Hkv, int Sq, int Sk,
                          int D, int causal, int window, int input_pos,
                          const int32_t* k_lengths, const uint8_t* keep,
                          hipStream_t stream);

/* Split-KV (Flash-Decoding) single-query decode, bf16 Q/K/V/O.
 *   O        out (B, H, D) bf16
 *   Q        in  (B, H, D) bf16
 *   K, V     in  (B, Hkv, Smax, D) bf16; slots at or past lengths[b] are
 *            never read
 *   lengths  device int32 (B,): valid KV length per sequence, clamped to
 *            [0, Smax]; a zero length gives O = 0
 *   n_splits >= 1: the valid keys of each (sequence, KV head) are cut into
 *            n_splits slices of C = ceil(ceil(len/64)/n_splits)*64 keys that
 *            run in parallel; their partial results are merged with LSE
 *            weights.  The result does not depend on n_splits beyond rounding.
 *   B, H, Hkv, Smax >= 1, D in {64, 128}
 * Allocates its partial-result scratch stream-ordered on `stream`
 * (hipMallocAsync / hipFreeAsync).  Defined by: Tylo.jl "Primitives",
 * decode_attention! (layouts, lengths, n_splits = 8, TILE_N = 64). */
int attn_decode(void* O, const void* Q, const void* K, const void* V,
                const int32_t* lengths, int n_splits, int B, int H, int Hkv,
                int Smax, int D, hipStream_t stream);

/* Bytes of scratch attn_decode_ws needs for these sizes (host-only, no HIP
 * call).  Returns 0 for invalid sizes. */
size_t attn_decode_workspace_bytes(int B, int H, int n_splits, int D);

/* attn_decode with a caller-provided device scratch buffer `workspace` of
 * `ws_bytes` >= attn_decode_workspace_bytes(B, H, n_splits, D) bytes,
 * 256-byte aligned.  Allocates nothing.  Concurrent calls must not share a
 * workspace. */
int attn_decode_ws(void* O, const void* Q, const void* K, const void* V,
                   const int32_t* lengths, int n_splits, int B, int H, int Hkv,
                   int Smax, int D, void* workspace, size_t ws_bytes,
                   hipStream_t stream);

/* Maximum scratch of attn_decode_static: 32 MiB per GPU, i.e.
 * attn_decode_workspace_bytes(B, H, n_splits, D) must not exceed it
 * (B * H * n_splits up to about 65,000 at D = 128). */
#define ATTN_DECODE_STATIC_SCRATCH_BYTES (32u << 20)

/* attn_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, semantics and kernels as attn_decode, with the slice
 * partials in a static device array of ATTN_DECODE_STATIC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends.  Calls no
 * allocating routine.  Returns ATTN_EUNSUPPORTED, before anything is
 * enqueued, when attn_decode_workspace_bytes(B, H, n_splits, D) exceeds that
 * size (n_splits = 1 needs no scratch).  Every call on one GPU shares its
 * array and leaves its partials there: calls that overlap on one GPU (two
 * streams, two host threads) race and must be serialised by the caller.  The
 * array's device address is looked up on the first call on each device. */
int attn_decode_static(void* O, const void* Q, const void* K, const void* V,
                       const int32_t* lengths, int n_splits, int B, int H,
                       int Hkv, int Smax, int D, hipStream_t stream);

/* Split-KV decode over a paged KV cache, bf16 Q/K/V/O.
 *   O, Q          (B, H, D) bf16, as attn_decode
 *   K_cache,
 *   V_cache       in (num_blocks, block_size, Hkv, D) bf16: token slot
 *                 `slot` of physical block `blk` holds the K (V) rows of all
 *                 KV heads of one token
 *   block_tables  device int32 (B, max_blocks): entry i of row b names the
 *                 physical block holding tokens [i*block_size, (i+1)*block_size)
 *                 of sequence b; entries past the sequence's last block are
 *                 never read; entries outside [0, num_blocks) are clamped into
 *                 range (no fault, meaningless result)
 *   lengths       device int32 (B,): tokens of each sequence (seq_lens),
 *                 clamped to [0, max_blocks * block_size]; zero gives O = 0
 *   n_splits      >= 1, the same key slicing and merge as attn_decode
 *   block_size    a power of two, 1..1024 (8, 16 and 32 are the serving sizes)
 *   D             64 or 128
 *   workspace     NULL: the library allocates its partial-result scratch
 *                 stream-ordered (hipMallocAsync / hipFreeAsync on `stream`);
 *                 else a caller buffer of ws_bytes >=
 *                 attn_decode_workspace_bytes(B, H, n_splits, D), 256-byte
 *                 aligned, not shared by concurrent calls.
 * Defined by: vllm_mlx.attention, MLXAttentionBackend.get_kv_cache_shape
 * (cache layout), supports_block_size (8/16/32), MLXAttentionMetadata
 * (seq_lens, block_tables); Tylo.jl "Primitives", decode_attention! (the
 * split-KV decode itself). */
int attn_decode_paged(void* O, const void* Q, const void* K_cache,
                      const void* V_cache, const int32_t* block_tables,
                      const int32_t* lengths, int n_splits, int B, int H,
                      int Hkv, int num_blocks, int block_size, int max_blocks,
                      int D, void* workspace, size_t ws_bytes,
                      hipStream_t stream);

/* Debug export: evaluates the kernels' own mask predicate into M (device,
 * uint8 (Sq, Sk), 1 = attend, 0 = blocked) for one batch with valid key
 * length k_len (clamped to [0, Sk]).  Tylo.jl "Primitives", hmask: host and
 * device masks must agree. */
int attn_mask_dump(uint8_t* M, int Sq, int Sk, int causal, int window,
                   int input_pos, int k_len, hipStream_t stream);

/* Debug export: the tile plan attn_fwd uses for group = H / Hkv query heads
 * per KV head.  A workgroup serves hp query heads of one KV head, hp the
 * largest power of two up to 8 dividing group, at TP = ATTN_FWD_TILE_M / hp
 * query positions; P (device) is int8 (ceil(Sq/TP), ceil(Sk/ATTN_FWD_TILE_N)):
 * 0 = empty (skipped), 1 = partial (masked per element), 2 = full (no
 * per-element mask).  ATTN_EINVAL for group < 1.  Tylo.jl "Primitives",
 * BlockMask / build_block_mask. */
int attn_tile_plan(int8_t* P, int Sq, int Sk, int causal, int window,
                   int input_pos, int k_len, int group, hipStream_t stream);

/* Static string naming a status code (never NULL). */
const char* attn_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
