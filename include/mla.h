/*
 * mla.h - C ABI of an MI355X (gfx950) library for absorbed-weight Multi-head
 * Latent Attention (MLA) decode over a paged latent KV cache.
 *
 * The method (DeepSeek-V2 MLA) as the source pages define it:
 *   - keybo.xyz, "MLA 之后，KV cache 确实得重新理解一遍":
 *       section "第一步，训练时"      c_kv(t) = W_DKV x(t); k = W_UK c_kv; v = W_UV c_kv
 *       section "第二步，推理时的吸收"  score = (W_UK^T q)^T c_kv;  o = W_UV (sum_j a_j c_kv(j))
 *       section "RoPE 为什么必须解耦"  k_R(t) = RoPE(W_KR x(t)) (64 dims, shared by all
 *                                    heads); score = q_C^T k_C + q_R^T k_R
 *       section "所以 cache 逻辑到底哪里要重写"  the cache is paged by token latent
 *   - dgblog.top, "MLA 是什么 | dg's Blog", section "一组真实数字": n_h = 128,
 *       d_h = 128, d_c = 512, d_h^R = 64, so a cached token holds 512 + 64 values.
 *   - algomooc.com MLA interview page, section "先区分 KV Cache 与 MLA": a decode
 *       step appends the new token, then attends over history plus current.
 *
 * One decode step of one layer is four calls, in this order:
 *   mla_absorb_q      q_abs = [W_UK^T q_C || RoPE(q_R)]          (per head)
 *   mla_cache_append  cache[slot] = [c_kv || RoPE(k_R)]           (per new token)
 *   mla_decode        o_lat = softmax(scale * q_abs . rows) . rows[:, :d_c]
 *                     (split over KV chunks, merged by log-sum-exp)
 *   mla_up_v          out = W_UV o_lat                            (per head)
 *
 * Conventions shared by every call
 *   - Every pointer argument except `dims` is device memory owned by the
 *     caller.  The library allocates nothing, frees nothing, and keeps no
 *     pointer after the call returns.  Kernels run asynchronously on `stream`
 *     (a hipStream_t; NULL is the default stream); buffers must stay alive
 *     until the stream has executed them.  No call synchronises the stream.
 *   - All tensors are dense and row-major (last index fastest).
 *   - `dims` and every host-visible argument are validated before anything is
 *     launched; on any error nothing is launched.  Values that live in device
 *     memory (positions, slots, page ids, sequence lengths) are preconditions
 *     the library does not read on the host; violating them is undefined.
 *   - Floating-point arithmetic is done in float32 with float32 accumulation;
 *     RoPE angles, cosines and sines are computed in float64.
 *   - The functions are stateless and may be called from several host threads
 *     (mla_last_hip_error is per thread).
 *   - `stream` is a hipStream_t passed as void* so that this header needs no
 *     HIP include; the caller casts.
 *   - Decode calls take no maximum-length hint: the split-KV plan (how many
 *     chunks, how much workspace) depends only on the batch size, the head
 *     count, num_splits and the current device's compute-unit count (asked
 *     of the runtime once per device; 256 when no device answers), and the
 *     kernels read the lengths themselves, so the same workspace serves any
 *     lengths within the block table.  Query the workspace size with the
 *     device current that will run the call.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = -2,       /* a size is out of range or unsupported */
  MLA_ERR_DTYPE = -3,       /* unknown dtype or unsupported combination */
  MLA_ERR_WORKSPACE = -4,   /* workspace smaller than mla_decode_workspace_bytes */
  MLA_ERR_UNSUPPORTED = -5, /* valid request the library has no kernel for */
  MLA_ERR_HIP = -6          /* a HIP launch failed; see mla_last_hip_error() */
} mla_status;

typedef enum {
  MLA_F32 = 0,   /* IEEE binary32 */
  MLA_BF16 = 1,  /* bfloat16 */
  MLA_E4M3 = 2   /* OCP 8-bit float E4M3 (bias 7, no infinities, max 448); cache only */
} mla_dtype;

/* Model shape.  Field order and types are part of the ABI (40 bytes). */
typedef struct mla_dims {
  int32_t n_heads;       /* n_h: query heads                                   */
  int32_t d_head;        /* d_h: per-head width of q_C, k_C, v and the output   */
  int32_t d_latent;      /* d_c: width of the cached latent c_kv                */
  int32_t d_rope;        /* d_R: width of the decoupled RoPE key (even, may be 0) */
  int32_t block_size;    /* tokens per cache page                               */
  int32_t act_dtype;     /* mla_dtype of q_c, q_r, c_kv, k_r, w_uk, w_uv, q_abs,
                            o_lat and out: MLA_F32 or MLA_BF16                  */
  int32_t kv_dtype;      /* cache element type: MLA_F32, MLA_BF16 or MLA_E4M3   */
  float softmax_scale;   /* multiplies q_abs . row; normally 1/sqrt(d_h + d_R);
                            finite and > 0 (else MLA_ERR_SHAPE)               */
  double rope_base;      /* RoPE base b: theta_i = b^(-2i/d_R), pairs (2i, 2i+1) */
} mla_dims;

/*
 * mla_absorb_q - absorb W_UK into the query and rotate its RoPE part.
 *   Source: keybo.xyz page, section "第二步，推理时的吸收" (score identity) and
 *   section "RoPE 为什么必须解耦" (q_R is rotated by the query position).
 *
 *   q_abs[b,h,0:d_c]   = sum_i W_UK[h,i,:] * q_c[b,h,i]     (= W_UK[h]^T q_C)
 *   q_abs[b,h,d_c:D]   = RoPE(q_r[b,h,:], q_pos[b])         D = d_c + d_R
 *
 *   q_c   [batch, n_h, d_h]      act_dtype
 *   q_r   [batch, n_h, d_R]      act_dtype (not yet rotated); may be NULL if d_R = 0
 *   q_pos [batch]                int32, the query token's 0-based position
 *   w_uk  [n_h, d_h, d_c]        act_dtype
 *   q_abs [batch, n_h, D]        act_dtype, written (no scaling applied)
 *   Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (batch < 1 or bad dims), MLA_ERR_DTYPE.
 */
mla_status mla_absorb_q(const mla_dims* dims, int32_t batch, const void* q_c, const void* q_r,
                        const int32_t* q_pos, const void* w_uk, void* q_abs, void* stream);

/*
 * mla_cache_append - write new tokens' latent rows into the paged cache.
 *   Source: keybo.xyz page, sections "RoPE 为什么必须解耦" (k_R is rotated
 *   before caching) and "所以 cache 逻辑到底哪里要重写" (rows paged per token
 *   latent; quantising c_kv spreads its error over all heads, and K and V
 *   share it, so a row is quantised as one unit).
 *
 *   row_t = [c_kv[t,:] || RoPE(k_r[t,:], pos[t])]  (rotation in float64, the
 *   result rounded to float32 and then to the cache type, nearest-even)
 *   page = slot[t] / block_size, offset = slot[t] % block_size
 *   kv_cache[page, offset, :] = row_t
 *   E4M3 cache: s = max|row_t| / 448 in float32 (s = 1 for an all-zero row);
 *   kv_cache holds e4m3(row_t / s) (float32 division, nearest-even, saturating
 *   at +-448) and kv_scale[page, offset] = s.
 *
 *   c_kv     [n_tokens, d_c]                 act_dtype
 *   k_r      [n_tokens, d_R]                 act_dtype (not yet rotated)
 *   pos      [n_tokens]                      int32 positions
 *   slot     [n_tokens]                      int64, 0 <= slot < num_pages * block_size,
 *                                            distinct within one call
 *   kv_cache [num_pages, block_size, D]      kv_dtype, rows written in place
 *   kv_scale [num_pages, block_size]         float32; required for E4M3, else ignored
 *   n_tokens = 0 is a no-op.  Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE.
 */
mla_status mla_cache_append(const mla_dims* dims, int32_t n_tokens, const void* c_kv,
                            const void* k_r, const int32_t* pos, const int64_t* slot,
                            int64_t num_pages, void* kv_cache, float* kv_scale, void* stream);

/*
 * mla_absorb_q_append - mla_absorb_q and mla_cache_append in one call (they
 * are independent: the query of step t and the row of token t), so that a
 * decode step pays one kernel launch for both where the shapes allow.
 *   Sources: as mla_absorb_q and mla_cache_append.
 *
 *   Exactly mla_absorb_q(dims, batch, q_c, q_r, q_pos, w_uk, q_abs) and
 *   mla_cache_append(dims, n_tokens, c_kv, k_r, pos, slot, num_pages,
 *   kv_cache, kv_scale): the same results bit for bit.  n_tokens = 0 appends
 *   nothing.  Arguments, layouts and errors: as the two calls.
 */
mla_status mla_absorb_q_append(const mla_dims* dims, int32_t batch, const void* q_c, const void* q_r,
                               const int32_t* q_pos, const void* w_uk, void* q_abs, int32_t n_tokens,
                               const void* c_kv, const void* k_r, const int32_t* pos, const int64_t* slot,
                               int64_t num_pages, void* kv_cache, float* kv_scale, void* stream);

/*
 * mla_kv_project_workspace_bytes - device workspace mla_kv_project_append
 * needs for n_tokens tokens of width d_model.  Pure host computation;
 * returns 0 when the arguments are invalid.
 */
size_t mla_kv_project_workspace_bytes(const mla_dims* dims, int32_t n_tokens, int32_t d_model);

/*
 * mla_kv_project_append - the down-projection of new tokens fused with their
 * append: the latent and the RoPE key are computed from the hidden states
 * and written straight into the paged cache.
 *   Source: keybo.xyz page, section "第一步，训练时" (c_kv = W_DKV x; only the
 *   latent is cached) and section "RoPE 为什么必须解耦" (k_R = RoPE(W_KR x),
 *   rotated before it is cached); dgblog.top page, section "1. 下采样（压缩）".
 *
 *   c_kv[t,:] = W_DKV h[t,:],  k_r[t,:] = W_KR h[t,:]   (float32 accumulation,
 *   each result rounded once to act_dtype, nearest-even), then exactly
 *   mla_cache_append(c_kv, k_r, pos, slot): the result is the same as
 *   projecting into act_dtype buffers and appending them.
 *
 *   h         [n_tokens, d_model]     act_dtype hidden states
 *   w_dkv     [d_c, d_model]          act_dtype
 *   w_kr      [d_R, d_model]          act_dtype; may be NULL if d_R = 0
 *   pos, slot, num_pages, kv_cache, kv_scale: as mla_cache_append
 *   workspace >= mla_kv_project_workspace_bytes(dims, n_tokens, d_model)
 *             bytes, device memory, 256-byte aligned; clobbered
 *   n_tokens = 0 is a no-op.  1 <= d_model <= 2^20.
 *   Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE, MLA_ERR_WORKSPACE.
 */
mla_status mla_kv_project_append(const mla_dims* dims, int32_t n_tokens, int32_t d_model, const void* h,
                                 const void* w_dkv, const void* w_kr, const int32_t* pos, const int64_t* slot,
                                 int64_t num_pages, void* kv_cache, float* kv_scale, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * mla_decode_workspace_bytes - device workspace mla_decode needs for this
 * batch and split count (num_splits = 0 means the automatic choice).  Pure
 * host computation; returns 0 when the arguments are invalid.
 */
size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t num_splits);

/*
 * mla_decode - attention of one absorbed query per sequence over its cached
 * latent rows (history plus the current token), split over KV chunks and
 * merged exactly.
 *   Source: keybo.xyz page, section "第二步，推理时的吸收" (score over the
 *   latent; latent-space weighted sum), section "RoPE 为什么必须解耦" (the
 *   two score terms), section "所以 cache 逻辑到底哪里要重写" (pages; a
 *   dedicated kernel for head width 576).  The split over KV chunks and its
 *   log-sum-exp merge are an exact re-association of the softmax sum.
 *
 *   For sequence b with L = seq_lens[b] rows r_0..r_{L-1} (row j of b lives at
 *   kv_cache[block_table[b, j / block_size], j % block_size]; E4M3 rows are
 *   kv_scale * e4m3 value) and every head h:
 *     s_j = softmax_scale * (q_abs[b,h,:] . r_j)
 *     o_lat[b,h,:] = sum_j softmax(s)_j * r_j[0:d_c]
 *     lse[b,h]     = log sum_j exp(s_j)
 *   L = 0 gives o_lat = 0 and lse = -inf.
 *
 *   q_abs       [batch, n_h, D]          act_dtype (from mla_absorb_q)
 *   kv_cache    [num_pages, block_size, D]  kv_dtype
 *   kv_scale    [num_pages, block_size]  float32, E4M3 only (else may be NULL)
 *   block_table [batch, max_pages]       int32 physical page ids; entries past
 *                                        ceil(L/block_size) are not read
 *   seq_lens    [batch]                  int32, 0 <= L <= max_pages * block_size
 *   num_splits  number of KV chunks the whole batch's pages are cut into
 *               (0 = automatic, >= 1 explicit, <= 65536); the result does not
 *               depend on it beyond float rounding
 *   workspace   >= mla_decode_workspace_bytes(dims, batch, num_splits) bytes,
 *               device memory, 256-byte aligned; clobbered
 *   o_lat       [batch, n_h, d_c]        act_dtype, written
 *   lse         [batch, n_h]             float32, written (may be NULL)
 *   Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE, MLA_ERR_WORKSPACE.
 */
mla_status mla_decode(const mla_dims* dims, int32_t batch, const void* q_abs, const void* kv_cache,
                      const float* kv_scale, const int32_t* block_table, int32_t max_pages,
                      const int32_t* seq_lens, int32_t num_splits, void* workspace,
                      size_t workspace_bytes, void* o_lat, float* lse, void* stream);

/*
 * mla_decode_window - mla_decode over a window of each sequence's rows.
 *   Source: keybo.xyz page, section "所以 cache 逻辑到底哪里要重写": with the
 *   cache paged by token latent, eviction policies such as a sliding window
 *   or dropping tokens work as before, and several requests that share a
 *   prefix share its latent pages.
 *
 *   Sequence b attends to its rows j with seq_starts[b] <= j < L (L =
 *   seq_lens[b]); everything else is as in mla_decode, which is this call
 *   with every start 0.  Only the block-table entries from
 *   seq_starts[b] / block_size to ceil(L / block_size) - 1 are read, so the
 *   pages wholly before the window may already be freed or reused (their
 *   entries are ignored); rows of the first page that lie before the window
 *   are read but carry weight zero, whatever they hold.  Several sequences
 *   may name the same physical page (a shared prefix): pages are only read.
 *   A window with seq_starts[b] >= L is empty: o_lat = 0, lse = -inf.
 *
 *   seq_starts  [batch]   int32, 0 <= seq_starts[b] (device memory); NULL
 *                         means all zero
 *   Other arguments, workspace size and errors: as mla_decode.
 */
mla_status mla_decode_window(const mla_dims* dims, int32_t batch, const void* q_abs, const void* kv_cache,
                             const float* kv_scale, const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, const int32_t* seq_starts, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, void* o_lat, float* lse, void* stream);

/*
 * mla_decode_noalloc - mla_decode_window without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 *   Computes exactly what mla_decode_window computes with the same arguments
 *   (the same kernels; seq_starts may be NULL, which is mla_decode), keeping
 *   the split-KV partials in a scratch array built into the library:
 *   MLA_NOALLOC_SCRATCH_BYTES of device memory per GPU, held from the moment
 *   the library's device code is loaded on that GPU until the process ends.
 *   The call allocates and frees nothing; the caller still provides every
 *   input and output.
 *
 *   Limit: mla_decode_workspace_bytes(dims, batch, num_splits) must not
 *   exceed MLA_NOALLOC_SCRATCH_BYTES, else MLA_ERR_WORKSPACE and nothing is
 *   launched.  (At 128 heads and automatic splits that covers batches of 96 sequences.)
 *   No part of the scratch needs to start at any value: the kernels write
 *   every byte they read within the call.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap on
 *   one GPU (different streams, or different host threads without ordering)
 *   race and must be serialised by the caller.
 *   Errors: as mla_decode_window, with MLA_ERR_WORKSPACE for the limit.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_decode_noalloc(const mla_dims* dims, int32_t batch, const void* q_abs, const void* kv_cache,
                              const float* kv_scale, const int32_t* block_table, int32_t max_pages,
                              const int32_t* seq_lens, const int32_t* seq_starts, int32_t num_splits, void* o_lat,
                              float* lse, void* stream);

/*
 * mla_decode_multi_workspace_bytes - device workspace mla_decode_multi needs.
 * Pure host computation; returns 0 when the arguments are invalid.
 */
size_t mla_decode_multi_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t num_splits);

/*
 * mla_decode_multi - several new query tokens per sequence (a chunk of new
 * tokens, as in chunked prefill or when checking drafted tokens), each
 * attending causally.
 *   Source: algomooc.com MLA interview page, section "先区分 KV Cache 与 MLA"
 *   (new tokens are appended, then attend over history plus current) and
 *   keybo.xyz page, section "第一步，训练时" (every token attends over the
 *   tokens up to itself); the absorbed score and latent sum as in mla_decode.
 *
 *   The last q_len rows of sequence b (positions L - q_len .. L - 1, L =
 *   seq_lens[b], already appended) are its queries; query i attends to the
 *   rows j with seq_starts[b] <= j <= L - q_len + i:
 *     o_lat[b, i] and lse[b, i] = mla_decode_window of that query over those rows.
 *   If L < q_len, the queries with no row of their own (i < q_len - L) get
 *   o_lat = 0, lse = -inf.
 *
 *   q_abs  [batch, q_len, n_h, D]     act_dtype (mla_absorb_q with
 *                                     batch * q_len rows, positions L - q_len + i)
 *   o_lat  [batch, q_len, n_h, d_c]   act_dtype, written
 *   lse    [batch, q_len, n_h]        float32, written (may be NULL)
 *   seq_starts may be NULL (every start 0); other arguments as
 *   mla_decode_window.  1 <= q_len; batch * q_len <= 2^24.  The rows of a
 *   sequence's pages are read once per query token.
 *   Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE, MLA_ERR_WORKSPACE.
 */
mla_status mla_decode_multi(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_abs,
                            const void* kv_cache, const float* kv_scale, const int32_t* block_table,
                            int32_t max_pages, const int32_t* seq_lens, const int32_t* seq_starts,
                            int32_t num_splits, void* workspace, size_t workspace_bytes, void* o_lat, float* lse,
                            void* stream);

/*
 * mla_up_v - the single W_UV up-projection after the latent weighted sum.
 *   Source: keybo.xyz page, section "第二步，推理时的吸收" (output identity).
 *
 *   out[b,h,i] = sum_c W_UV[h,i,c] * o_lat[b,h,c]
 *   o_lat [batch, n_h, d_c]   act_dtype
 *   w_uv  [n_h, d_h, d_c]     act_dtype
 *   out   [batch, n_h, d_h]   act_dtype, written
 *   Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE.
 */
mla_status mla_up_v(const mla_dims* dims, int32_t batch, const void* o_lat, const void* w_uv,
                    void* out, void* stream);

/* Text for a status code (static storage). */
const char* mla_status_string(mla_status status);

/* hipError_t of the last MLA_ERR_HIP returned on this thread (0 if none). */
int32_t mla_last_hip_error(void);

/* Version of this ABI; bumped on any incompatible change. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
