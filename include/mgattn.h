/*
 * mgattn: segmented multi-head softmax attention for AMD Instinct MI355X (gfx950).
 *
 * The operation is the perception-encoder attention of the Muse Glimmer vision
 * tower as described in vllm.cpp issue #1545 ("Muse Glimmer's vision tower runs 50
 * layers on the naive attention kernel"):
 *   - section "Why this one is bad": non-causal, 16 heads, head_dim 96, 50 layers;
 *   - section "The fix": the block-diagonal window mask is a set of per-segment row
 *     slices, each attended on its own, and the flash rung honours a causal flag;
 *   - second comment, "Two of the three labelled uncertainties are now resolved":
 *     13 full-attention layers (one segment per image) and 37 window layers whose
 *     segments are 32x32 = 1024-patch windows.
 * For every segment [a, b) of cu_seqlens, every head h and every query i in [a, b):
 *     out[i,h,:] = sum_j softmax_j(scale * <q[i,h,:], k[j,h,:]>) * v[j,h,:]
 * with j over [a, b) (causal: j over [a, i]).
 *
 * Refusal conventions follow vllm.cpp PR #1578 ("a model on the naive attention
 * kernel now says why, and AttentionDenseFlash advertises the head_dim it can
 * launch"), section "AttentionDenseFlash advertises the head_dim it can launch": the
 * supported domain and the on-chip memory a launch asks for are pure host queries
 * that need no GPU, bounds are inclusive, and an unsupported request is refused by
 * name before any launch instead of surfacing as a bare launch error.
 *
 * Every function is callable from C; no C++ type or exception crosses this boundary.
 */
#ifndef MGATTN_H
#define MGATTN_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out (one type for all four). */
typedef enum {
  MGATTN_F32 = 0,  /* IEEE binary32 */
  MGATTN_BF16 = 1  /* bfloat16 (upper half of a binary32) */
} mgattn_dtype;

/* Return codes.  Every negative status means nothing was enqueued. */
typedef enum {
  MGATTN_OK = 0,
  MGATTN_ERR_NULL = -1,      /* a required pointer is NULL */
  MGATTN_ERR_DTYPE = -2,     /* dtype is not an mgattn_dtype */
  MGATTN_ERR_HEAD_DIM = -3,  /* head_dim outside mgattn_dense_supported's domain */
  MGATTN_ERR_HEADS = -4,     /* H < 1 (mgattn_attention_kv: Hkv < 1 or Hq % Hkv != 0) */
  MGATTN_ERR_SEQLENS = -5,   /* cu_seqlens malformed (see mgattn_dense) */
  MGATTN_ERR_SEGMENTS = -6,  /* n_seg < 1 */
  MGATTN_ERR_ALIAS = -7,     /* out overlaps q, k or v */
  MGATTN_ERR_ALIGN = -8,     /* a tensor pointer is not 16-byte aligned */
  MGATTN_ERR_SCALE = -9,     /* scale is NaN or infinite, or causal is not 0 or 1 */
  MGATTN_ERR_LAUNCH = -10,   /* the HIP runtime reported an error for the launch */
  MGATTN_ERR_DEVICE = -11,   /* the current device is not a gfx950 GPU */
  MGATTN_ERR_SIZE = -12,     /* a segment spans >= 2^31 bytes (len*ld*element size),
                                or a launch would need more than 2^31-1 workgroups */
  MGATTN_ERR_STRIDE = -13,   /* a leading dimension is below H*d, above 2^31-1, or not
                                a multiple of 16 bytes (also: a bad row_bytes) */
  MGATTN_ERR_GRID = -14,     /* a patch grid is empty, more than 64 images, a window
                                below its minimum, or a flag is not 0 or 1 */
  MGATTN_ERR_WINDOW = -15,   /* mgattn_attention_kv: window < 0 */
  MGATTN_ERR_SCRATCH = -16   /* mgattn_attention_kv_noalloc: more scratch than it holds */
} mgattn_status;

/*
 * mgattn_dense: enqueue segmented attention on `stream` and return.
 *
 *   q, k, v    device pointers, each [T, H, d] contiguous row-major in `dtype`
 *              (element (t, h, c) at offset (t*H + h)*d + c), T = cu_seqlens[n_seg].
 *              Caller-owned; read only.  16-byte aligned.
 *   out        device pointer, [T, H, d] in `dtype`, caller-owned, written in full
 *              (every token of every segment, every head).  Must not overlap q, k or v.
 *              16-byte aligned.
 *   cu_seqlens HOST pointer to n_seg+1 int32 values: cu_seqlens[0] == 0, non-decreasing,
 *              cu_seqlens[n_seg] == T > 0.  Segment g is tokens [cu[g], cu[g+1]);
 *              empty segments are allowed and do nothing.  Read during the call only.
 *   n_seg      number of segments, >= 1.  No upper limit: large counts are split
 *              over several launches on the same stream.
 *   H          heads, >= 1.
 *   d          head_dim; see mgattn_dense_supported (96 is always supported).
 *   scale      logit multiplier (for the tower, 1/sqrt(d)); any finite value, 0 included.
 *   causal     0: every query sees its whole segment.  1: query i sees keys [a, i].
 *   dtype      an mgattn_dtype.  Accumulation is f32 in both cases; bf16 results are
 *              rounded to nearest even.
 *   stream     a hipStream_t (NULL = the default stream).
 *
 * Returns MGATTN_OK once the work is enqueued (no host synchronisation), or a
 * negative mgattn_status.  All argument checks run before anything is enqueued.
 * MGATTN_ERR_LAUNCH reports an error from the HIP runtime at launch time; errors that
 * surface later during execution belong to the stream, as for any kernel.
 * The library allocates no device memory and keeps no pointer after returning; calls
 * on different streams may overlap.  NaN or infinite input values are not checked:
 * their rows of out are unspecified.
 */
int mgattn_dense(const void* q, const void* k, const void* v, void* out,
                 const int32_t* cu_seqlens, int n_seg, int H, int d, float scale,
                 int causal, int dtype, void* stream);

/*
 * mgattn_dense_strided: mgattn_dense on tensors whose consecutive tokens are ld
 * elements apart (row-major [T, ld], head h of token t at offset t*ld + h*d).  The
 * motivating layout is the merged projection output the perception encoder carries
 * (vllm.cpp PR #279: the vision tower's q|k|v projections folded into one qkv
 * matrix at load time): a [T, 3*H*d] buffer qkv is consumed as
 *     q = qkv, k = qkv + H*d, v = qkv + 2*H*d, ldq = ldk = ldv = 3*H*d
 * without splitting it first.  out may be strided too (its other elements are not
 * written).
 *
 *   ldq, ldk, ldv, ldo  leading dimensions in elements: >= H*d, <= 2^31-1, and a
 *                       multiple of 16 bytes (8 bf16 or 4 f32 elements).
 *   q, k, v             may overlap each other (they are only read).  out must not
 *                       overlap the span [x, x + ((T-1)*ldx + H*d) elements) of any input.
 * Every other argument, the return value and the stream semantics are those of
 * mgattn_dense; mgattn_dense(...) is mgattn_dense_strided with all four = H*d.
 */
int mgattn_dense_strided(const void* q, const void* k, const void* v, void* out,
                         int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                         const int32_t* cu_seqlens, int n_seg, int H, int d, float scale,
                         int causal, int dtype, void* stream);

/*
 * mgattn_attention_kv: causal sliding-window attention with grouped key/value heads
 * over a key/value cache -- the attention of the Muse Glimmer text decoder (mbext
 * next-steps page, "Architecture / Text decoder": 32 query heads, 2 key/value heads,
 * head size 128, a repeating [sliding, sliding, sliding, full] pattern with a local
 * window of 2048 tokens; prefill and incremental decoding with a KV cache).
 *
 * n_seq sequences.  Sequence s has Lq = cu_seqlens_q[s+1] - cu_seqlens_q[s] new
 * queries (rows of q and out) and Lk = cu_seqlens_k[s+1] - cu_seqlens_k[s] >= Lq keys
 * and values (rows of k and v: the cache, ending with the new tokens' own entries).
 * Query i of the sequence sits at position p = Lk - Lq + i; for query head h and key
 * /value head g = h / (Hq / Hkv),
 *     out[i,h,:] = sum_j softmax_j(scale * <q[i,h,:], k[j,g,:]>) * v[j,g,:]
 * with j over [max(0, p - window + 1), p] (window == 0: over [0, p]).  The local window
 * thus holds the query's own key and the window-1 before it; prefill is Lq == Lk,
 * one-token decoding Lq == 1.
 *
 *   q, out   device, [Tq rows, leading dimension ldq / ldo], Hq heads of d channels
 *            (Tq = cu_seqlens_q[n_seq]); ldq, ldo >= Hq*d.
 *   k, v     device, [Tk rows, leading dimension ldk / ldv], Hkv heads of d channels
 *            (Tk = cu_seqlens_k[n_seq]); ldk, ldv >= Hkv*d.
 *   cu_seqlens_q, cu_seqlens_k   HOST arrays of n_seq+1 int32 (prefix sums as in
 *            mgattn_dense); a sequence with Lq == 0 does nothing.
 *   Hq, Hkv  query and key/value heads, Hkv >= 1, Hq a multiple of Hkv.
 *   window   >= 0 (0: no window, plain causal).
 * Every other argument, alignment, aliasing rule, return value and the stream
 * semantics are those of mgattn_dense_strided.
 */
int mgattn_attention_kv(const void* q, const void* k, const void* v, void* out,
                        int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seq,
                        int Hq, int Hkv, int d, float scale, int window, int dtype, void* stream);

/*
 * mgattn_attention_kv_ws: mgattn_attention_kv with a caller-provided device workspace.
 * One-token decoding (bf16, every sequence with Lq <= 1, Hq / Hkv <= 32) runs one
 * workgroup per (sequence, key/value head) in mgattn_attention_kv; with few sequences
 * that leaves most of the 256 CUs idle while the cache is streamed from HBM.  Given a
 * workspace, the visible keys of each (sequence, key/value head) are split over up to
 * 16 workgroups (as many as workspace_bytes holds, toward one workgroup per CU); each
 * writes its partial result (running maximum, denominator and normalised output, in
 * f32) to the workspace and a second kernel merges them into out.  The result equals
 * mgattn_attention_kv's up to the f32 rounding of that merge.  Calls that are not
 * one-token decoding ignore the workspace.
 *
 *   workspace        device, 256-byte aligned, workspace_bytes bytes, overlapping none
 *                    of q, k, v, out.  Scratch: written and read by the call's kernels
 *                    in stream order; calls that may overlap in time need distinct
 *                    workspaces.  The library still allocates no device memory.
 *   workspace_bytes  0 (workspace may be NULL): exactly mgattn_attention_kv.  A size
 *                    from mgattn_attention_kv_workspace gives the full split.
 * Other arguments, checks and return values: mgattn_attention_kv; a misaligned
 * workspace is MGATTN_ERR_ALIGN, an overlapping one MGATTN_ERR_ALIAS, NULL with
 * workspace_bytes > 0 MGATTN_ERR_NULL.
 */
int mgattn_attention_kv_ws(const void* q, const void* k, const void* v, void* out,
                           int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seq,
                           int Hq, int Hkv, int d, float scale, int window, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace with which mgattn_attention_kv_ws splits these arguments fully:
 * 0 when they are not one-token decoding in bf16 or no split would help.  Pure host
 * arithmetic, no GPU needed; a negative mgattn_status for malformed arguments (the
 * host array and shape checks of mgattn_attention_kv). */
long mgattn_attention_kv_workspace(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seq,
                                   int Hq, int Hkv, int d, int window, int dtype);

/* mgattn_attention_kv_noalloc: mgattn_attention_kv_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and result as mgattn_attention_kv without the
 * workspace: the partial results of the decode key splits go to a scratch array the
 * library holds in each GPU's memory (a static device array of
 * mgattn_attention_kv_noalloc_scratch_bytes() = 4,259,840 bytes, the most any call
 * needs under the split rule, resolved once per device), so
 * the call allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * A call that needs more than that is refused with MGATTN_ERR_SCRATCH before anything
 * is launched (mgattn_attention_kv_workspace gives the need).  Every call on one GPU
 * shares that GPU's scratch and leaves its contents behind (nothing in it needs to
 * start at zero): calls that overlap on one GPU (different streams without ordering)
 * race; calls in stream order do not. */
int mgattn_attention_kv_noalloc(const void* q, const void* k, const void* v, void* out,
                                int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int n_seq, int Hq, int Hkv, int d, float scale, int window,
                                int dtype, void* stream);

/* Bytes of the per-device scratch of mgattn_attention_kv_noalloc (its size limit). */
long mgattn_attention_kv_noalloc_scratch_bytes(void);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* mgattn_strerror(int status);

/* 1 if (H, d, dtype) can be launched, else 0.  Pure host arithmetic, no GPU needed.
 * The head_dim domain is {64, 96, 128}; H >= 1; dtype an mgattn_dtype. */
int mgattn_dense_supported(int H, int d, int dtype);

/* Bytes of LDS (on-chip shared memory) one workgroup of the (d, dtype) kernel asks
 * for, or a negative mgattn_status if (d, dtype) is not supported.  Pure host
 * arithmetic, no GPU needed; equals the static LDS footprint of the kernel's largest
 * workgroup shape (bf16 head_dim 96: the 256-query tile; f32: the key-split 32-query
 * block at head_dim 64 and 96, the 128-query tile at 128; the key-split 16-query block
 * asks for less at every head_dim). */
long mgattn_dense_lds_bytes(int d, int dtype);

/* Queries per workgroup of the (d, dtype) kernel (the tallest q-tile it uses), or a
 * negative mgattn_status.  Pure host arithmetic. */
int mgattn_dense_block_m(int d, int dtype);

/* Queries per workgroup mgattn_dense uses for this segment table (same arguments and
 * refusals as mgattn_dense_plan), or a negative mgattn_status.  Pure host arithmetic.
 * The bf16 head_dim-96 kernel takes 256 when the (segment, head, q-tile) units of 256
 * give at least 256 workgroups (one per CU).  Otherwise a non-causal call splits each
 * tile's keys between wave groups and takes 128 (two groups) if the units of 128 give
 * 256 workgroups, else 64 (four groups; one 1024-token segment of 16 heads: 64 units
 * of 256, 256 of 64); a causal call takes 128.  f32 takes 128, or for a non-causal
 * call whose 128-query units give fewer than 256 workgroups 32 (the keys of each
 * 32-query block split over the workgroup's waves), or 16 if the 32-query blocks too
 * give fewer than 256 (a 256-token segment of 16 heads: 128 blocks of 32, 256 of 16).
 * Every other (d, dtype) has the single height of mgattn_dense_block_m. */
int mgattn_dense_plan_block_m(const int32_t* cu_seqlens, int n_seg, int H, int d, int dtype, int causal);

/* Introspection of the work split (pure host arithmetic, no GPU needed).
 *
 * mgattn_dense_plan: number of kernel launches mgattn_dense makes for these
 * arguments (segments are ordered longest first and packed up to 120 per launch),
 * or a negative mgattn_status.  If grids is not NULL, grids[i] receives the
 * workgroup count of launch i for i < max_launches.
 *
 * mgattn_dense_tile: what workgroup `block` of launch `launch` computes.  Returns 1
 * and writes {segment index in cu_seqlens, head, first query of the tile relative
 * to the segment start} to seg_head_q0[0..2]; returns 0 for an idle workgroup; or a
 * negative mgattn_status.  Every (segment, head, q-tile) of the call appears exactly
 * once over all launches and blocks. */
int mgattn_dense_plan(const int32_t* cu_seqlens, int n_seg, int H, int d, int dtype, int causal,
                      int64_t* grids, int max_launches);
int mgattn_dense_tile(const int32_t* cu_seqlens, int n_seg, int H, int d, int dtype, int causal,
                      int launch, int64_t block, int32_t* seg_head_q0);

/*
 * Token order of the perception encoder's patch grids.
 *
 * A batch is n_img images; grids[2i], grids[2i+1] are image i's patch-grid height
 * and width (gh, gw >= 1, 1 <= n_img <= 64).  In raster order, image i's tokens
 * follow those of images < i, row-major (token y*gw + x).  Window layers attend
 * within win x win blocks of patches (vllm.cpp issue #1545, second comment: the
 * vision tower's sparse permutation cuts 32x32 = 1024-patch windows); in window
 * order each image's tokens are regrouped block by block so that every block is a
 * contiguous segment.  The pages do not state the block walk order or the order
 * inside a block; this library takes row-major over the blocks (blocks at the right
 * and bottom edges clipped to the grid) and row-major inside a block.  The order
 * inside a block does not change the attention output; the block order fixes the
 * sequence of segments.
 */

/* Segments of the window layers: writes the n_seg+1 prefix sums of the window
 * sizes, in window order, to cu_seqlens (host) and returns n_seg.  With cu_seqlens
 * NULL, only returns n_seg; if max_seg < n_seg, returns MGATTN_ERR_SIZE.  A window at
 * least as large as every grid gives one segment per image (the full-attention
 * layers).  Pure host arithmetic. */
int mgattn_window_segments(const int32_t* grids, int n_img, int win, int32_t* cu_seqlens, int max_seg);

/* Enqueue on `stream` the permutation of T = sum(gh*gw) rows of row_bytes bytes
 * (row_bytes a multiple of 16): inverse == 0 gathers src (raster order) into dst
 * (window order of window win); inverse == 1 scatters src (window order) back into
 * dst (raster order), as the tower does before its final LayerNorm (vllm.cpp PR
 * #279, vision-tower commit).  src and dst are caller-owned device buffers of
 * T*row_bytes bytes, 16-byte aligned, not overlapping.  Any element type: rows are
 * moved as bytes. */
int mgattn_window_permute(const void* src, void* dst, int64_t row_bytes, const int32_t* grids, int n_img,
                          int win, int inverse, void* stream);

/* Enqueue on `stream` the 2D rotary position embedding of the vision tower (vllm.cpp
 * PR #279, vision-tower commits: width-first order, 1-based positions), in place on
 * x: T = sum(gh*gw) token rows with leading dimension ldx elements, each holding H
 * heads of d channels (head h of token t at t*ldx + h*d), in `dtype`.  Tokens are in
 * raster order if win == 0, in the window order of window win (as produced by
 * mgattn_window_permute) if win > 0; the position of a token is that of its patch.
 * The pages name the convention without a formula; the reading taken:
 *   for a patch at row y, column x, and each head:
 *     channels [0, d/2) rotate with position x + 1, channels [d/2, d) with y + 1;
 *     inside a half, pair (2i, 2i+1) is multiplied, as the complex number
 *     c_2i + i*c_2i+1, by exp(i * pos * theta^(-4i/d)),  i = 0 .. d/4 - 1.
 * Angles are formed in f32 (pos * f32(theta^(-4i/d)), theta^(-4i/d) computed in
 * double on the host) and rotated with f32 sincos; bf16 results are rounded to
 * nearest even.  d is a multiple of 16 in [16, 128]; theta > 1 and finite (the
 * tower's value is not on the pages; 10000 is the customary base). */
int mgattn_rope2d(void* x, int64_t ldx, const int32_t* grids, int n_img, int win, int H, int d, float theta,
                  int dtype, void* stream);

/* mgattn_dense_strided over 2D-RoPE-rotated queries and keys, the rotation of q fused
 * into the attention's loads (vllm.cpp PR #279, vision-tower commits: the tower
 * rotates q and k before attention; width-first, 1-based positions, as in
 * mgattn_rope2d).  k is rotated in place by the RoPE pass (mgattn_rope2d on k); q is
 * read-only and each workgroup rotates its query rows in registers as it loads them,
 * rounding exactly as mgattn_rope2d does, so `out` equals, bit for bit, that of
 * mgattn_rope2d on q and on k followed by mgattn_dense_strided -- with one read and
 * one write of q fewer.  The images of (grids, n_img) in token order `win` (0: raster,
 * > 0: window order, as mgattn_rope2d) must hold exactly the call's tokens
 * (cu_seqlens[n_seg]), else MGATTN_ERR_GRID.  The fused path is the tower's: bf16 and
 * head_dim 96; other (dtype, d) are refused (MGATTN_ERR_DTYPE, MGATTN_ERR_HEAD_DIM)
 * before anything is launched -- use mgattn_rope2d and mgattn_dense_strided.  Other
 * arguments, refusals and ownership as mgattn_dense_strided and mgattn_rope2d. */
int mgattn_dense_rope2d(const void* q, void* k, const void* v, void* out, int64_t ldq, int64_t ldk, int64_t ldv,
                        int64_t ldo, const int32_t* cu_seqlens, int n_seg, int H, int d, float scale, int causal,
                        int dtype, const int32_t* grids, int n_img, int win, float theta, void* stream);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int mgattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MGATTN_H */
