/*
 * mrope.h — C ABI of the MI355X (gfx950) multimodal rotary position embedding
 * library: RMSNorm + MRoPE over query/key heads, as used by Qwen3-VL,
 * Qwen3.5 and Qwen3-Omni style attention.
 *
 * Sources (web pages, cited by title and section):
 *  [RoPE]  "Interleaved Rotary Position Embedding" (RoPE post): the inv_freq
 *          listing, rotate_half / apply_rotary_pos_emb with partial rotary,
 *          the interleaved axis selection, get_rope_index.
 *  [M01]   "M01 · RMSNorm and multimodal RoPE (interleaved / chunked)": the
 *          function list and shapes, RMSNorm numeric conventions, the
 *          interleaved rule and the chunked layout, the shape trace.
 *  [QVL]   "Qwen3-VL" annotated source: the text rotary embedding (fp32
 *          angles, cat(f, f), cos/sin) and the vision 2-D rotary
 *          (rot_pos_emb, apply_rotary_pos_emb_vision).
 *  [Q3V]   cortiq-engine qwen3vis.rs: rope_angles and the split-half
 *          rotation over the whole vision head.
 *
 * Conventions shared by every entry point
 *  - Tensors are token-major, x[T][heads][D] ([M01] shape list: q/k as
 *    [T, heads, D]).  Heads of one token are contiguous (head stride D); the
 *    token stride is an argument (in elements, >= heads*D) so views into
 *    packed buffers work.
 *  - dtype: MROPE_DTYPE_F32 (binary32) or MROPE_DTYPE_BF16 (bfloat16).
 *    RMSNorm weights have the dtype of x.  cos/sin tables are binary32.
 *  - Positions are int32 [n_axes][T] with axis stride pos_axis_stride (in
 *    elements; 0 broadcasts one 1-D position row to every axis).  |p| must
 *    be below 2^24 so float(p) is exact.
 *  - Device buffers are owned by the caller.  The library allocates nothing
 *    and keeps no state between calls beyond two thread-local diagnostics
 *    (mrope_last_error, mrope_last_kernel) and the static device workspace of
 *    mrope_rope_index_noalloc (1 MiB per GPU, in the code object); small
 *    tables (section, inv_freq) are host pointers copied into kernel
 *    arguments.
 *  - Kernels address a token's rows of a tensor (or, for per-head planes, the
 *    rows of a few tokens across all planes) with 32-bit byte offsets: a
 *    span of 2^31 bytes or more is MROPE_EUNSUPPORTED, and so are more than
 *    2^20 heads in one tensor.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without synchronising.
 *  - Outputs may alias their own input exactly (in place).  Any other overlap
 *    between an output and any input or the other output is MROPE_EINVAL.
 *  - T == 0 (or no heads) is a valid no-op returning MROPE_OK.
 *  - Arguments are checked before any HIP call; on a non-zero return nothing
 *    has been enqueued and mrope_last_error() describes the failure.  There is
 *    no host fallback.
 */
#ifndef MROPE_H_
#define MROPE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes */
#define MROPE_OK            0
#define MROPE_EINVAL       (-1)  /* bad argument: null pointer, shape, section, overlap */
#define MROPE_EUNSUPPORTED (-2)  /* valid but unsupported: dtype, alignment, size limits */
#define MROPE_EHIP         (-3)  /* a HIP call failed (launch error, no device) */

/* Frequency-column layouts ([M01] layout table) */
#define MROPE_LAYOUT_CHUNKED     0  /* TTTT..HHH..WWW: consecutive ranges of section[a] columns */
#define MROPE_LAYOUT_INTERLEAVED 1  /* THWTHW..TT: j%3==1 && j<3*s_h -> H, j%3==2 && j<3*s_w -> W */
#define MROPE_LAYOUT_VISION_2D   2  /* first half/2 columns read the row, the rest the column */

#define MROPE_DTYPE_F32  0
#define MROPE_DTYPE_BF16 1

/* Rotation precision (argument `precision` of the rotating entry points).
 *  EXACT: the products of the stored value and the binary32 cos/sin and
 *         their sum are evaluated in double (the products are exact), rounded
 *         to binary32 and then (bf16) to bfloat16: the binary32 result of
 *         the rotation, rounded to the tensor's dtype.
 *  DTYPE: the rotation as tensor operations in the tensor's dtype ([M01]
 *         shape trace, apply_rotary row, and its broadcast note: cos/sin are
 *         cast to x.dtype before the multiplies, as HF's text rotary does):
 *         c = dt(cos), s = dt(sin); out = dt(dt(x*c) + dt(rotate_half(x)*s)),
 *         where dt() rounds to the dtype and each bf16 operation is computed
 *         in binary32 before it rounds.
 *  FP32:  the rotation as binary32 tensor operations with one cast at the
 *         end ([QVL] apply_rotary_pos_emb_vision): out = dt(f(f(x*cos) +
 *         f(rotate_half(x)*sin))) with f() rounding to binary32.
 * For MROPE_DTYPE_F32, DTYPE and FP32 are the same arithmetic.  No mode fuses
 * a product into the sum. */
#define MROPE_PRECISION_EXACT 0
#define MROPE_PRECISION_DTYPE 1
#define MROPE_PRECISION_FP32  2

/* Largest rotary_dim the kernels accept (the per-column table travels as a
 * kernel argument). */
#define MROPE_MAX_ROTARY_DIM 512

/*
 * mrope_inv_freq — inv[i] = theta^(-2i/dim) for i < dim/2, evaluated in
 * double and rounded once to binary32 ([RoPE] inv_freq listing; [M01]
 * rope_inv_freq).  Text layouts use dim = rotary_dim (frequencies of the
 * rotated slice only, [RoPE] partial rotary); the vision layout uses
 * dim = head_dim/2 ([Q3V] rope_angles: 18 frequencies for a 72-dim head).
 *   out: host array of dim/2 floats, written.
 * Host-only: makes no HIP call.  EINVAL if dim <= 0, dim odd, theta <= 0 or
 * not finite, or out == NULL.
 */
int mrope_inv_freq(int dim, double theta, float* out);

/*
 * mrope_axis_table — the axis each frequency column j < half reads
 * (0 = T / row, 1 = H / column, 2 = W), per `layout` ([M01] interleaved rule
 * and chunked table; [QVL] apply_interleaved_mrope; [Q3V] rope_angles).
 *   section: host array of n_sections ints (chunked: 1..3 entries summing to
 *            half; interleaved: exactly 3 entries summing to half; vision:
 *            ignored, may be NULL).
 *   axis_out: host array of half bytes, written.
 * Host-only.  EINVAL if half <= 0 or > MROPE_MAX_ROTARY_DIM/2, a section entry
 * is negative, the section does not sum to half, the interleaved rule cannot
 * give an axis its section count (3*(s_h-1)+1 >= half or 3*(s_w-1)+2 >= half),
 * the vision half is odd, or a pointer is NULL.
 */
int mrope_axis_table(int half, const int* section, int n_sections, int layout,
                     uint8_t* axis_out);

/*
 * mrope_cos_sin — cos/sin tables of shape [T][rotary_dim], binary32
 * ([M01] mrope_cos_sin(inv_freq, positions[3,T], section, interleaved) and
 * shape-trace rows 4-7): for column j < half, angle = fl32(float(p) * inv),
 * p = pos[axis[j]][t]; cos = fl32(cos(angle)), sin = fl32(sin(angle)) with
 * cos/sin evaluated in double; columns j and j+half hold the same values
 * (cat(f, f)).
 *   pos:       device int32, [n_axes][T] with axis stride pos_axis_stride.
 *   n_axes:    3 (interleaved), 2 (vision), or len(section) (chunked).
 *   inv_freq:  host binary32, half entries (text layouts) or half/2 entries
 *              (vision), taken as given (inv = ones runs the axis probe).
 *   cos_out, sin_out: device binary32, [T][rotary_dim] with token stride
 *              cs_tok_stride (elements, >= rotary_dim).
 * EINVAL on a bad section/layout/axes combination, rotary_dim odd or <= 0
 * or > MROPE_MAX_ROTARY_DIM, null pointers, or overlapping outputs.
 */
int mrope_cos_sin(const int32_t* pos, int64_t pos_axis_stride, int n_axes, int64_t T,
                  const float* inv_freq, const int* section, int n_sections, int layout,
                  int rotary_dim, float* cos_out, float* sin_out, int64_t cs_tok_stride,
                  void* stream);

/*
 * rms_norm — per-head RMSNorm over the last dimension ([M01] numeric
 * conventions): r = fl32(1/sqrt(sum(x^2)/D + eps)) with the sum of squares
 * accumulated in double; n = fl32(x*r); cast n to the dtype of x; multiply by
 * w (one weight vector [D] shared by all heads); cast to the dtype of x.
 *   x:   device, [T][heads][D], token stride x_tok_stride.
 *   w:   device, [D], dtype of x.
 *   out: device, [T][heads][D], token stride out_tok_stride (may equal x).
 * EINVAL on null pointers, D <= 0 or odd, strides below heads*D, overlap.
 * EUNSUPPORTED if D is too large for one wavefront per row or the buffers are
 * not element-aligned.
 */
int rms_norm(const void* x, int64_t x_tok_stride, int64_t T, int heads, int D,
             const void* w, float eps, int dtype, void* out, int64_t out_tok_stride,
             void* stream);

/*
 * apply_rotary_qk — split-half rotation of q and k with given cos/sin
 * ([RoPE] rotate_half / apply_rotary_pos_emb; [M01] apply_rotary with cos/sin
 * broadcast over heads as [T, 1, D]):
 *   out[j]      = x[j]*cos[j]      - x[j+h]*sin[j]        (j < h = rotary_dim/2)
 *   out[j+h]    = x[j+h]*cos[j+h]  + x[j]*sin[j+h]
 *   out[j]      = x[j]                                    (rotary_dim <= j < D)
 * evaluated with the rounding points `precision` names (MROPE_PRECISION_*;
 * EXACT: in double from the stored inputs and the binary32 tables, rounded
 * once to binary32 and then (bf16) to bfloat16).
 *   q: device [T][hq][D], token stride q_tok_stride; k likewise with hk heads
 *      (k may be NULL when hk == 0).
 *   cos, sin: device binary32 [T][rotary_dim], token stride cs_tok_stride.
 *   q_out, k_out: device, same shapes, own token strides (may equal q / k).
 * EINVAL on bad shapes (rotary_dim odd, <= 0 or > D), null pointers, overlap,
 * or an unknown precision.
 */
int apply_rotary_qk(const void* q, int64_t q_tok_stride, int hq,
                    const void* k, int64_t k_tok_stride, int hk,
                    int64_t T, int D, int rotary_dim,
                    const float* cos, const float* sin, int64_t cs_tok_stride,
                    int dtype, int precision,
                    void* q_out, int64_t q_out_tok_stride,
                    void* k_out, int64_t k_out_tok_stride,
                    void* stream);

/*
 * rmsnorm_mrope_qk — the fused hot path: optional per-head RMSNorm (as
 * rms_norm, with wq for q heads and wk for k heads), then MRoPE on the first
 * rotary_dim dims of every q and k head with cos/sin computed in the kernel
 * from the positions (as mrope_cos_sin with inv_freq = mrope_inv_freq(
 * rotary_dim, theta) for text layouts, mrope_inv_freq(rotary_dim/2, theta)
 * reused for row and column for the vision layout), and the rest of each head
 * passed through ([RoPE] Qwen3.5 attention: q/k norm, then
 * apply_rotary_pos_emb; [M01] "Where it sits"; [QVL] the vision rotary).
 * cos/sin are formed once per (token, column) and shared by all hq + hk heads.
 * The result is bit-identical to rms_norm followed by mrope_cos_sin and
 * apply_rotary_qk with the same precision.
 *   wq, wk: device [D] weights of the dtype; both NULL = no normalisation.
 *   precision: MROPE_PRECISION_* (rotation only; the RMSNorm is the same in
 *              every mode).
 *   Other arguments as in the functions above.
 * EINVAL as above, or if exactly one of wq / wk is NULL.
 */
int rmsnorm_mrope_qk(const void* q, int64_t q_tok_stride, int hq,
                     const void* k, int64_t k_tok_stride, int hk,
                     int64_t T, int D, int rotary_dim,
                     const int32_t* pos, int64_t pos_axis_stride, int n_axes,
                     const int* section, int n_sections, int layout, double theta,
                     const void* wq, const void* wk, float eps, int dtype, int precision,
                     void* q_out, int64_t q_out_tok_stride,
                     void* k_out, int64_t k_out_tok_stride,
                     void* stream);

/*
 * mrope_cos_sin_cache — a cos/sin table by position value ([RoPE] the
 * "method 2" listing: the outer product of arange(max + 1) and inv_freq,
 * gathered by position afterwards):
 *   cache[2*(p*(dim/2) + i)]     = fl32(cos(fl32(float(p) * inv[i])))
 *   cache[2*(p*(dim/2) + i) + 1] = fl32(sin(...)),   0 <= p < rows,
 * with inv = mrope_inv_freq(dim, theta): the values mrope_cos_sin computes
 * for position p, bit for bit.  dim = rotary_dim for the text layouts,
 * rotary_dim/2 for the vision layout.  The table depends on (dim, theta,
 * rows) only, so a model builds it once and reuses it for every layer.
 *   cache: device binary32 [rows][dim/2][2], 8-byte aligned.
 * EINVAL on dim odd, <= 0 or > MROPE_MAX_ROTARY_DIM, theta <= 0, rows < 0,
 * NULL or misaligned cache.
 */
int mrope_cos_sin_cache(int dim, double theta, int rows, float* cache, void* stream);

/*
 * rmsnorm_mrope_qk_cached — rmsnorm_mrope_qk taking cos/sin from a cache by
 * position (mrope_cos_sin_cache with the matching dim and theta, rows
 * cache_rows) for positions in [0, cache_rows), and computing them as
 * rmsnorm_mrope_qk does for any other position: the result is bit-identical
 * to rmsnorm_mrope_qk whenever the cache was built with the same theta.
 * cs_cache NULL (and cache_rows 0) is rmsnorm_mrope_qk.  The cache may not
 * overlap an output.
 */
int rmsnorm_mrope_qk_cached(const void* q, int64_t q_tok_stride, int hq,
                            const void* k, int64_t k_tok_stride, int hk,
                            int64_t T, int D, int rotary_dim,
                            const int32_t* pos, int64_t pos_axis_stride, int n_axes,
                            const int* section, int n_sections, int layout, double theta,
                            const void* wq, const void* wk, float eps, int dtype, int precision,
                            void* q_out, int64_t q_out_tok_stride,
                            void* k_out, int64_t k_out_tok_stride,
                            const float* cs_cache, int cache_rows, void* stream);

/*
 * mrope_decode_qk — one decode step of the fused path ([RoPE] Qwen3.5 call
 * chain, compute_3d_position_ids: with rope_deltas stored and a non-empty
 * cache, positions are recovered from the sequence index counted from the
 * cache length, the same on all three axes, plus each sample's rope_deltas).
 * Token i of sequence b is row b*new_tokens + i of q and k; its position is
 * p = cache_len[b] + i + rope_delta[b] (rope_delta NULL = 0) on every axis,
 * so the rotation is 1-D RoPE with inv_freq = mrope_inv_freq(rotary_dim,
 * theta) whatever the model's section.  Optional per-head RMSNorm and the
 * rotation precision as in rmsnorm_mrope_qk.  Rotated q goes to q_out;
 * rotated k of token (b, i) is
 * written into the KV cache row
 *     k_cache + b*k_cache_seq_stride + (cache_len[b] + i)*k_cache_tok_stride
 * (hk*D contiguous elements); a row at or past k_cache_capacity (or below 0)
 * is not written.
 *   q: device [batch*new_tokens][hq][D]; k likewise with hk heads.
 *   cache_len, rope_delta: device int32 [batch] (rope_delta may be NULL).
 *   k_cache: device, batch sequences of k_cache_capacity rows; strides in
 *            elements (k_cache_tok_stride >= hk*D, k_cache_seq_stride >=
 *            k_cache_capacity*k_cache_tok_stride when batch > 1).
 * Positions must stay below 2^24 in magnitude.  EINVAL on bad shapes, null
 * pointers, or a cache that overlaps q, k, q_out, the weights or cache_len /
 * rope_delta.
 */
int mrope_decode_qk(const void* q, int64_t q_tok_stride, int hq,
                    const void* k, int64_t k_tok_stride, int hk,
                    int batch, int new_tokens, int D, int rotary_dim,
                    const int32_t* cache_len, const int32_t* rope_delta, double theta,
                    const void* wq, const void* wk, float eps, int dtype, int precision,
                    void* q_out, int64_t q_out_tok_stride,
                    void* k_cache, int64_t k_cache_seq_stride, int64_t k_cache_tok_stride,
                    int k_cache_capacity, void* stream);

/*
 * mrope_vision_qkv — the vision tower's rotary step on a packed qkv in one
 * pass ([Q3V] attention: the packed projection is [n, 3, heads, hd] with the
 * head axis innermost; q and k are rotated split-half over the head and
 * written, with v copied, to per-head planes for the attention kernel;
 * [QVL] apply_rotary_pos_emb_vision for the rotation and its precision):
 *   q_out[h][t][j] = rotate(qkv[t][0][h][:])[j], k_out likewise from
 *   qkv[t][1], v_out[h][t][j] = qkv[t][2][h][j],
 * with the rotation and cos/sin of rmsnorm_mrope_qk for the vision 2-D
 * layout (positions [2][n]: row, col; inv_freq = mrope_inv_freq(
 * rotary_dim/2, theta) for both), dims past rotary_dim passed through, and
 * the precision argument as there.
 *   qkv:        device [n][3][heads][D], token stride qkv_tok_stride
 *               (elements, >= 3*heads*D).
 *   q_out, k_out, v_out: device; element (h, t, j) at
 *               h*out_head_stride + t*out_tok_stride + j.  Head-major planes:
 *               out_head_stride = n*D, out_tok_stride = D; token-major rows:
 *               out_head_stride = D, out_tok_stride >= heads*D.  v_out may be
 *               NULL (v not written).
 *   cs_cache, cache_rows: optional cos/sin cache by position
 *               (mrope_cos_sin_cache(rotary_dim/2, theta, cache_rows));
 *               positions outside [0, cache_rows) are computed.  NULL, 0 =
 *               compute all.
 * The outputs may not overlap the input, the cache or each other.  EINVAL
 * on bad shapes or strides (rows that would overlap), null pointers,
 * overlap; EUNSUPPORTED when one token's output rows span 2^31 bytes or
 * more.
 */
int mrope_vision_qkv(const void* qkv, int64_t qkv_tok_stride, int64_t n, int heads, int D,
                     int rotary_dim, const int32_t* pos, int64_t pos_axis_stride, double theta,
                     int dtype, int precision, void* q_out, void* k_out, void* v_out,
                     int64_t out_head_stride, int64_t out_tok_stride, const float* cs_cache,
                     int cache_rows, void* stream);

/* Status bits written by the position builders into their device `status`
 * word (0 = the inputs describe a sequence the walkthrough can build). */
#define MROPE_POS_BAD_TYPE      1   /* a valid token's type is not 0, 1 or 2 (taken as text) */
#define MROPE_POS_NO_GRID       2   /* a visual segment has no (usable) grid left: text positions */
#define MROPE_POS_LENGTH        4   /* a visual segment's token count differs from its grid */
#define MROPE_POS_NOT_DIVISIBLE 8   /* a vision grid's h or w is not a multiple of the merge size */
#define MROPE_POS_COUNT        16   /* the grids' patch total differs from n_tokens */

/*
 * mrope_rope_index_workspace_size — bytes of device workspace
 * mrope_rope_index needs for these sizes (0 on invalid sizes).
 */
size_t mrope_rope_index_workspace_size(int batch, int64_t seq_len, int n_images, int n_videos);

/*
 * mrope_rope_index — the 3-axis position table and rope_deltas of a batch of
 * mixed text / image / video token sequences ([RoPE] get_rope_index
 * walkthrough and its single-batch L = 10 table):
 *  - padding (attention_mask 0) is removed first; it keeps position 0;
 *  - the remaining tokens of a sample are split into runs of equal type
 *    (0 text, 1 image, 2 video);
 *  - a text run of n tokens takes p, p+1, ..., p+n-1 on all three axes and
 *    advances p by n;
 *  - an image run takes the next image grid (t, h, w) of the batch (one
 *    iterator shared by all samples, in sample order); a video run takes the
 *    next single-slice grid (1, h, w), each video of t slices giving t of
 *    them; its slots (t, h/merge, w/merge), flattened width fastest, get
 *    (p + ti, p + row, p + col); p then advances by max(h, w) / merge;
 *  - rope_delta[b] = max position + 1 - valid token count (0 when none).
 *   mm_token_type:   device int32 [batch][seq_len] (contiguous).
 *   attention_mask:  device int32 [batch][seq_len], nonzero = valid; NULL =
 *                    all valid.
 *   image_grid_thw:  device int32 [n_images][3]; video_grid_thw likewise
 *                    (NULL when the count is 0).
 *   pos:             device int32 [3][batch*seq_len], axis stride
 *                    pos_axis_stride (>= batch*seq_len): the layout the
 *                    rotating entry points read (token b*seq_len + l).
 *   rope_delta:      device int32 [batch].
 *   status:          device int32, set to the OR of MROPE_POS_* conditions.
 *   workspace:       device scratch of mrope_rope_index_workspace_size bytes,
 *                    owned by the caller; its contents on entry do not matter.
 * Two or three kernels on `stream` (mrope_last_kernel names the form of
 * passes 2 and 3); the host does not wait.  Positions are computed
 * in 64-bit integers and stored as int32.  EINVAL on negative sizes, a merge
 * size outside [1, 1024], null pointers, a short or misaligned (8-byte)
 * workspace, or overlapping outputs.
 */
int mrope_rope_index(const int32_t* mm_token_type, const int32_t* attention_mask, int batch,
                     int64_t seq_len, const int32_t* image_grid_thw, int n_images,
                     const int32_t* video_grid_thw, int n_videos, int spatial_merge,
                     int32_t* pos, int64_t pos_axis_stride, int32_t* rope_delta,
                     int32_t* status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mrope_rope_index_noalloc — mrope_rope_index without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that allocate nothing per step, harnesses that forbid
 * hipMalloc).  The workspace is a static device array of
 * MROPE_ROPE_INDEX_SCRATCH_BYTES in the library's code object: each GPU
 * holds its own copy until the process ends, and the first call on a GPU
 * takes its address there (hipGetSymbolAddress, no allocation).  Arguments,
 * results, status bits and errors are mrope_rope_index's, and so are the
 * kernels; sizes whose workspace (mrope_rope_index_workspace_size) exceeds
 * the static array are MROPE_EUNSUPPORTED, with nothing enqueued.  Calls on
 * one GPU share its array: two calls whose work overlaps in time on that GPU
 * (different streams, or host threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe.  Nothing needs clearing
 * between calls: every pass writes the workspace before it reads it.
 */
#define MROPE_ROPE_INDEX_SCRATCH_BYTES (1 << 20)
int mrope_rope_index_noalloc(const int32_t* mm_token_type, const int32_t* attention_mask,
                             int batch, int64_t seq_len, const int32_t* image_grid_thw,
                             int n_images, const int32_t* video_grid_thw, int n_videos,
                             int spatial_merge, int32_t* pos, int64_t pos_axis_stride,
                             int32_t* rope_delta, int32_t* status, void* stream);

/*
 * mrope_vision_pos_ids — the (row, col) position of every vision patch
 * ([QVL] rot_pos_emb): images in order; within an image, patches in
 * merge x merge block order (block row, block col, row in block, col in
 * block), row = block_row*merge + row_in_block, col likewise; the t frames of
 * an image repeat its coordinates.
 *   grid_thw: device int32 [n_images][3] (t, h, w), n_images <= 4096.
 *   pos:      device int32 [2][n_tokens], axis stride pos_axis_stride: the
 *             layout of the vision-2D rotating entry points.
 *   status:   device int32: MROPE_POS_NOT_DIVISIBLE, MROPE_POS_COUNT (patches
 *             past the grids' total are written as (0, 0)).
 * EINVAL on bad sizes, a merge size outside [1, 1024], null pointers or
 * overlapping buffers.
 */
int mrope_vision_pos_ids(const int32_t* grid_thw, int n_images, int spatial_merge,
                         int64_t n_tokens, int32_t* pos, int64_t pos_axis_stride,
                         int32_t* status, void* stream);

/*
 * mrope_stream_copy — copy `bytes` from src to dst with a plain streaming
 * kernel (16-byte loads of whole contiguous spans, then non-temporal 16-byte
 * stores; no arithmetic).  A measurement aid, not a step of the rotary path:
 * it gives the copy rate of a given number of bytes on this device, the
 * achievable ceiling that the benchmark reports beside each kernel's rate.
 *   src, dst: device buffers, 16-byte aligned, not overlapping.
 *   bytes:    a multiple of 16, at most 2^40.
 * EINVAL on a misaligned or overlapping buffer, a null pointer or a size
 * that is negative or not a multiple of 16; bytes == 0 is a no-op.
 */
int mrope_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * mrope_last_error — message for the last non-zero return on this thread
 * (empty string if none).  The pointer stays valid until the next call on
 * the same thread.
 */
const char* mrope_last_error(void);

/*
 * mrope_last_kernel — name of the kernel that the last q/k launch on this
 * thread (rms_norm, apply_rotary_qk, rmsnorm_mrope_qk[_cached],
 * mrope_decode_qk, mrope_vision_qkv) enqueued: "qk_kernel" (rows spread over
 * lane groups, the general path), "qk_pipe_kernel" (one token per wavefront,
 * its row-steps pipelined: launches of 2048 tokens or more on the positions
 * path with 16-byte chunks), "flat_kernel" (a token's block of rows lane
 * after lane), "planes_kernel" (a few tokens x every per-head plane per
 * block, chunks in output order: full rotary into planes) or "stage_kernel"
 * (rows staged through LDS, written in output order); after
 * mrope_rope_index, the kernels of its passes 2 and 3:
 * "rope_index_fused" (one kernel; up to 1024 chunks of 1024 tokens and 256
 * grids per type) or "rope_index_carry+apply" (two kernels, any size); empty
 * string before the first launch.  A diagnostic for profiles, benchmarks and
 * tests: the choice depends on the shapes, dtype, layout and grid counts
 * only, never on the values.  Static storage; no ownership.
 */
const char* mrope_last_kernel(void);

#ifdef __cplusplus
}
#endif

#endif /* MROPE_H_ */
