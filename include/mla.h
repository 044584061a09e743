/*
 * mla.h - C ABI of the latent-KV chunk-attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * The library implements one layer's streaming chunk-attention step of
 * VideoMLA ("VideoMLA: Low-Rank Latent KV Cache for Minute-Scale
 * Autoregressive Video Diffusion"):
 *   - every token x_t is compressed to a shared content latent
 *     c_t = W_dkv x_t and one head-shared, unrotated positional key
 *     kR_t = W_kR x_t, and only those d_c + d_rope scalars are cached
 *     (hyper.ai summary, Method section; 192 + 32 = 224 instead of 3072 at
 *     the Wan2.1-1.3B shape: ai-papers.net explainer, paragraph under Fig. 1);
 *   - the cache is a fixed-size sliding window of frames (chatpaper.ai,
 *     English abstract);
 *   - at attention time the positional key is rotated by 3D-RoPE over
 *     (t, y, x), and head h's score is the content part q_nope . (W_uk[h] c)
 *     plus the positional part R(p_q) qR . R(p_k) kR; the value is
 *     W_uv[h] c (hyper.ai summary, Method section).
 * The library evaluates the content score and the value through the latent
 * (the "absorbed" form: (W_uk[h]^T q_nope) . c, and W_uv[h] (sum_j p_j c_j)),
 * which is the same value re-associated.
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are HIP device memory; (host) are host memory
 *     read only during the call. The caller owns every buffer; the library
 *     keeps no pointer after returning and allocates nothing.
 *   - stream is a hipStream_t (NULL = the default stream). Every call is
 *     asynchronous on that stream: it validates on the host, enqueues its
 *     kernels and returns. Calls are reentrant; calls that write the same
 *     buffers must be ordered by the caller.
 *   - Arrays are row-major and contiguous. Element type of x, weights,
 *     cache, queries and outputs is shape->dtype: MLA_BF16 (bfloat16) or
 *     MLA_F32 (float). Accumulation is fp32 in both cases. RoPE tables are
 *     always float.
 *   - Every device pointer must be 16-byte aligned.
 *   - The *_workspace_bytes queries return 0 for any shape, chunk size or
 *     split that the matching call rejects.
 *   - Errors are reported by return value before anything is enqueued
 *     (MLA_ERR_NULL, _SHAPE, _DTYPE, _ALIGN, _WORKSPACE, _UNSUPPORTED,
 *     _RANGE), or MLA_ERR_HIP if a launch fails. No C++ exception crosses
 *     this boundary.
 *   - Supported latent widths (d_c, d_rope): (192, 32) (the Wan2.1 split),
 *     (128, 32), (160, 64), (192, 64) and (16, 8), either dtype. d_head must be a multiple of 8 and at most 256; hidden a
 *     multiple of 8; window_frames at most 64; each RoPE axis width even;
 *     and window_frames * grid_y * grid_x at most 2^22 keys. Shapes
 *     outside these limits return MLA_ERR_SHAPE.
 *
 * Token positions: a frame has grid_y * grid_x tokens in row-major order;
 * token k of frame f sits at (t, y, x) = (f, k / grid_x, k % grid_x).
 * RoPE: the d_rope dims are three contiguous blocks [t | y | x] of widths
 * d_rope_t, d_rope_y, d_rope_x; inside each block the interleaved pair
 * (2i, 2i+1) is rotated by pos * rope_base^(-2i/d_axis).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,       /* dimensions inconsistent or out of range */
  MLA_ERR_DTYPE = 3,       /* dtype is neither MLA_BF16 nor MLA_F32 */
  MLA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  MLA_ERR_WORKSPACE = 5,   /* workspace smaller than the *_workspace_bytes query */
  MLA_ERR_UNSUPPORTED = 6, /* (d_c, d_rope) has no kernel instantiation */
  MLA_ERR_HIP = 7,         /* a HIP launch failed */
  MLA_ERR_RANGE = 8,       /* frame or table index arguments out of range */
  MLA_ERR_SCRATCH = 9      /* needs more than the fixed scratch of mla_flash_attend_noalloc */
} mla_status;

typedef enum mla_dtype { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

/* Layer and stream geometry (host memory). */
typedef struct mla_shape {
  int32_t batch;         /* B independent streams, each with its own window */
  int32_t hidden;        /* token width (input of the down-projections) */
  int32_t n_heads;       /* H */
  int32_t d_head;        /* per-head key / value width */
  int32_t d_c;           /* content latent width */
  int32_t d_rope;        /* positional key width = d_rope_t + d_rope_y + d_rope_x */
  int32_t d_rope_t;      /* rotary dims driven by the frame index t */
  int32_t d_rope_y;      /* rotary dims driven by the grid row y */
  int32_t d_rope_x;      /* rotary dims driven by the grid column x */
  int32_t grid_y;        /* tokens per frame = grid_y * grid_x */
  int32_t grid_x;
  int32_t window_frames; /* W: ring slots; frame f lives in slot f mod W */
  int32_t dtype;         /* mla_dtype */
  float rope_base;       /* RoPE base (10000 for the Wan shapes) */
  float softmax_scale;   /* <= 0 selects 1/sqrt(d_head + d_rope) */
} mla_shape;

/* Library version; equals MLA_ABI_VERSION of the header it was built from. */
int32_t mla_abi_version(void);

/* Static text for a status code (never NULL). */
const char* mla_status_string(int32_t status);

/* Host-only validation of a shape; enqueues nothing. */
mla_status mla_shape_check(const mla_shape* shape);

/* Width of one absorbed-query row: d_c + d_rope rounded up to 32 (padding
 * columns are zero). 0 if the shape is invalid. */
int32_t mla_qabs_dim(const mla_shape* shape);

/* ---------------------------------------------------------------- a1
 * 3D-RoPE tables (hyper.ai summary, Method: the positional key is rotated
 * by 3D-RoPE at attention time; axes (t, h, w) = (t, y, x)).
 * Fills `tables` (device, float) with, in order:
 *   cos_t[n_t][d_rope_t/2], sin_t[n_t][d_rope_t/2]   positions t_first + i
 *   cos_y[grid_y][d_rope_y/2], sin_y[grid_y][d_rope_y/2]
 *   cos_x[grid_x][d_rope_x/2], sin_x[grid_x][d_rope_x/2]
 * Angles are formed in double precision and rounded to float.
 * mla_rope3d_table_floats gives the element count (0 if invalid). */
size_t mla_rope3d_table_floats(const mla_shape* shape, int32_t n_t);
mla_status mla_rope3d_tables(const mla_shape* shape, int32_t t_first, int32_t n_t, float* tables,
                             void* stream);

/* ---------------------------------------------------------------- a2 + a6
 * Cache write (hyper.ai summary, Method: c = W_dkv x is written to the
 * compressed cache; kR = W_kR x is stored unrotated; chatpaper.ai abstract:
 * fixed-size sliding window).
 *   x          (device) [B][n_frames * T][hidden]   tokens of frames
 *                       frame_first .. frame_first + n_frames - 1, T = grid_y*grid_x
 *   w_dkv      (device) [d_c][hidden]
 *   w_kr       (device) [d_rope][hidden]
 *   cache      (device) [B][W][T][d_c + d_rope]   row = [c | kR], rounded to dtype
 *   slot_frame (device) [B][W] int32               frame held by each slot, -1 = empty
 * Frame f goes to slot f mod W (evicting what the slot held) and
 * slot_frame[b][f mod W] = f. Requires 0 <= frame_first, 1 <= n_frames <= W
 * (else MLA_ERR_RANGE). Writing the same frame again is idempotent. The
 * caller initialises slot_frame to -1 before the first write. */
mla_status mla_cache_write(const mla_shape* shape, const void* x, const void* w_dkv, const void* w_kr,
                           int32_t frame_first, int32_t n_frames, void* cache, int32_t* slot_frame,
                           void* stream);

/* ---------------------------------------------------------------- a3
 * Query absorb and rotate (hyper.ai summary, Method: score = content part
 * + positional part). For query token i of the chunk (frame
 * q_frame_first + i / T) and head h, with g = softmax_scale * log2(e) (the
 * temperature folded in, so scores come out in log2 units):
 *   q_abs[b][i][h][0:d_c]            = g W_uk[h]^T q_nope[b][i][h]
 *   q_abs[b][i][h][d_c:d_c+d_rope]   = g R(t, y, x) q_r[b][i][h]
 *   q_abs[b][i][h][d_c+d_rope:Q]     = 0,    Q = mla_qabs_dim(shape)
 *   q_nope (device) [B][N_q][H][d_head], q_r (device) [B][N_q][H][d_rope]
 *   (unrotated), w_uk (device) [H][d_head][d_c], N_q = q_n_frames * T.
 *   rope_tables (device) from mla_rope3d_tables(shape, rope_t_first,
 *   rope_n_t, ...); the chunk's frames must lie in
 *   [rope_t_first, rope_t_first + rope_n_t) (else MLA_ERR_RANGE).
 *   q_abs (device) [B][N_q][H][Q], dtype. */
mla_status mla_absorb_q(const mla_shape* shape, const void* q_nope, const void* q_r, int32_t q_frame_first,
                        int32_t q_n_frames, const void* w_uk, const float* rope_tables, int32_t rope_t_first,
                        int32_t rope_n_t, void* q_abs, void* stream);

/* ---------------------------------------------------------------- a4
 * Latent flash attention (hyper.ai summary, Method; chatpaper.ai abstract:
 * softmax over the sliding window). For every row (b, i, h), with q_abs as
 * mla_absorb_q writes it (temperature and log2 e already folded in):
 *   s_j   = q_abs[b][i][h] . [c_j | R(t_j, y_j, x_j) kR_j]
 *   o_lat = sum_j 2^(s_j) c_j / sum_j 2^(s_j)            -> [d_c]
 * over every key j of every slot of stream b with slot_frame[b][s] >= 0
 * (no intra-chunk mask); rows with no valid key get zeros.
 *   q_abs (device) [B][N_q][H][Q] from mla_absorb_q; cache, slot_frame as
 *   written by mla_cache_write; rope_tables from mla_rope3d_tables (any
 *   rope_t_first >= 0, rope_n_t >= 1): the keys' spatial angles are read from
 *   them, while the temporal angles of the frames held in the window are
 *   formed during the call by the same computation the tables use, so window
 *   frames need not lie in the table's range.
 *   o_lat (device) [B][N_q][H][d_c], dtype.
 *   workspace (device) of at least mla_flash_workspace_bytes(shape,
 *   q_n_frames, kv_splits) bytes; its contents on entry do not matter. The
 *   call keeps there the window's positional keys after 3D-RoPE (rotated
 *   once per call, d_rope values per key), the list of rows for the exact
 *   fallback and, when row blocks are shared, the partial results.
 *   kv_splits: how the (row block, key tile) work is split between
 *   work-groups. 0 (recommended): one work-group per compute unit of the
 *   current device, each taking an equal share; row blocks shared by
 *   several work-groups are finished by a merge pass over their partial
 *   (output, reference, sum). s in 1..16: every row block gets s equal key
 *   ranges (1 = no merge). The result is the same up to rounding. With 0
 *   the workspace size depends on the compute-unit count of the current
 *   device: query it with the device that will run the call current.
 *   Returns MLA_ERR_SHAPE if the work grid is too large to index
 *   (more than 2^40 units). */
size_t mla_flash_workspace_bytes(const mla_shape* shape, int32_t q_n_frames, int32_t kv_splits);
mla_status mla_flash_attend(const mla_shape* shape, const void* q_abs, int32_t q_n_frames, const void* cache,
                            const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                            int32_t rope_n_t, void* o_lat, int32_t kv_splits, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- a4, no allocation
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mla_flash_attend with its workspace replaced by a fixed scratch array of
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each GPU it
 * runs on, from the first call with that GPU current until the process ends.
 * The call itself allocates nothing. Same arguments, result and errors as
 * mla_flash_attend without workspace / workspace_bytes; a problem whose
 * mla_flash_workspace_bytes exceeds the scratch returns MLA_ERR_SCRATCH
 * before anything is enqueued (the Wan2.1 chunk, 3 frames over a 21-frame
 * window, needs about 53 MB at one stream with kv_splits = 0). Every call on
 * one GPU uses that GPU's single array: calls that may overlap on one GPU
 * (several streams, several host threads) race on it and must be ordered by
 * the caller. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_flash_attend_noalloc(const mla_shape* shape, const void* q_abs, int32_t q_n_frames, const void* cache,
                                    const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                                    int32_t rope_n_t, void* o_lat, int32_t kv_splits, void* stream);

/* ---------------------------------------------------------------- a4, frame-causal
 * mla_flash_attend under the frame-causal mask inside the chunk (the
 * chunk-wise autoregressive reading of the hyper.ai summary, Method, and the
 * chatpaper.ai abstract): the row of query token i (frame
 * q_frame_first + i / T) takes only the keys of slots holding frames
 * <= that frame; a row with no such key gets zeros. Same arguments,
 * workspace (mla_flash_workspace_bytes) and errors as mla_flash_attend,
 * plus q_frame_first >= 0 (else MLA_ERR_RANGE). */
mla_status mla_flash_attend_frame_causal(const mla_shape* shape, const void* q_abs, int32_t q_frame_first,
                                         int32_t q_n_frames, const void* cache, const int32_t* slot_frame,
                                         const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                                         void* o_lat, int32_t kv_splits, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* ---------------------------------------------------------------- a5
 * Value up-projection (hyper.ai summary, Method: v = W_uv[h] c, so
 * sum_j p_j v_j = W_uv[h] sum_j p_j c_j):
 *   out[b][i][h][:] = W_uv[h] o_lat[b][i][h][:]
 *   o_lat (device) [B][N_q][H][d_c], w_uv (device) [H][d_head][d_c],
 *   out (device) [B][N_q][H][d_head], dtype. */
mla_status mla_up_v(const mla_shape* shape, const void* o_lat, int32_t q_n_frames, const void* w_uv, void* out,
                    void* stream);

/* ---------------------------------------------------------------- a3..a5
 * The whole attention side of the step (hyper.ai summary, Method: the score
 * and value through the shared latent), in one of two forms that give the
 * same result up to rounding:
 *   - the latent form, mla_chunk_attend_latent: mla_absorb_q,
 *     mla_flash_attend and mla_up_v in sequence on `stream`, with q_abs and
 *     o_lat carved from `workspace`;
 *   - the per-head form, mla_chunk_attend_heads (below).
 * mla_chunk_attend takes the form mla_chunk_attend_form names for the shape
 * and chunk size: the per-head form where it is supported (bf16,
 * d_head = 128), does at least 20% fewer products per (query, key, head)
 * (2 d_head + d_rope against 2 d_c + d_rope) and the chunk has at least 2048
 * query tokens per stream to repay its per-call expansion of the window's
 * keys and values; else the latent form. At the Wan2.1 shape (d_c 192,
 * 3-frame chunks of 4680 tokens) that is the per-head form.
 * mla_chunk_attend_workspace_bytes covers both the latent form and, where
 * mla_chunk_attend takes it, the per-head form (so one workspace serves
 * mla_chunk_attend, mla_chunk_attend_latent and
 * mla_chunk_attend_frame_causal).
 * Arguments as above; out (device) [B][N_q][H][d_head]. */
#define MLA_FORM_LATENT 0
#define MLA_FORM_HEADS 1
int32_t mla_chunk_attend_form(const mla_shape* shape, int32_t q_n_frames); /* -1 if invalid */
size_t mla_chunk_attend_workspace_bytes(const mla_shape* shape, int32_t q_n_frames);
mla_status mla_chunk_attend(const mla_shape* shape, const void* q_nope, const void* q_r, int32_t q_frame_first,
                            int32_t q_n_frames, const void* w_uk, const void* w_uv, const void* cache,
                            const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                            int32_t rope_n_t, void* out, void* workspace, size_t workspace_bytes,
                            void* stream);
mla_status mla_chunk_attend_latent(const mla_shape* shape, const void* q_nope, const void* q_r,
                                   int32_t q_frame_first, int32_t q_n_frames, const void* w_uk, const void* w_uv,
                                   const void* cache, const int32_t* slot_frame, const float* rope_tables,
                                   int32_t rope_t_first, int32_t rope_n_t, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- a3..a5, frame-causal
 * mla_chunk_attend with a frame-causal mask inside the chunk (the
 * chunk-wise autoregressive reading of the hyper.ai summary, Method, and the
 * chatpaper.ai abstract): a query of frame f = q_frame_first + i / T attends
 * only the keys of frames <= f. Keys of earlier chunks are all visible and
 * a query always sees its own frame's keys (when they are in the window).
 * Same arguments, workspace (mla_chunk_attend_workspace_bytes) and errors as
 * mla_chunk_attend, and the same choice of form (mla_chunk_attend_form):
 * mla_chunk_attend_latent_frame_causal and
 * mla_chunk_attend_heads_frame_causal (below, with the per-head form's
 * workspace) force one. Only the key tiles a row block may see are visited;
 * tiles that every row of a block sees run unmasked. */
mla_status mla_chunk_attend_frame_causal(const mla_shape* shape, const void* q_nope, const void* q_r,
                                         int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                         const void* w_uv, const void* cache, const int32_t* slot_frame,
                                         const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                                         void* out, void* workspace, size_t workspace_bytes, void* stream);
mla_status mla_chunk_attend_latent_frame_causal(const mla_shape* shape, const void* q_nope, const void* q_r,
                                                int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                                const void* w_uv, const void* cache, const int32_t* slot_frame,
                                                const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                                                void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- a3'..a5'
 * Per-head form of the same step (hyper.ai summary, Method: per-head keys
 * and values are reconstructed from the shared latent when needed). Same
 * arguments and result as mla_chunk_attend, up to rounding: the window's
 * keys and values are expanded once per call for every head,
 *   k[h][j] = W_uk[h] c_j,  v[h][j] = W_uv[h] c_j   (bf16, in the workspace),
 * and each head attends with the score
 *   scale * (q_nope . k[h][j] + R(p_i) qR . R(p_j) kR_j)
 * over every key of every valid slot. It does
 * 2 N_q N_k H (d_head + d_rope + d_head) products in the attention against
 * the latent form's 2 N_q N_k H (d_c + d_rope + d_c), plus the expansion
 * (4 N_k H d_head d_c products and 4 N_k H d_head bytes). Only bf16 with
 * d_head = 128 and a latent width the library instantiates; other shapes
 * return MLA_ERR_UNSUPPORTED (and a workspace size of 0).
 *   workspace (device) of at least mla_chunk_attend_heads_workspace_bytes
 *   bytes (about 4 B H W T d_head bytes: 201 MB at the Wan2.1 shape);
 *   contents on entry do not matter. */
size_t mla_chunk_attend_heads_workspace_bytes(const mla_shape* shape, int32_t q_n_frames);
mla_status mla_chunk_attend_heads(const mla_shape* shape, const void* q_nope, const void* q_r,
                                  int32_t q_frame_first, int32_t q_n_frames, const void* w_uk, const void* w_uv,
                                  const void* cache, const int32_t* slot_frame, const float* rope_tables,
                                  int32_t rope_t_first, int32_t rope_n_t, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);
/* The per-head form with the frame-causal mask of
 * mla_chunk_attend_frame_causal; arguments, workspace and errors as
 * mla_chunk_attend_heads. */
mla_status mla_chunk_attend_heads_frame_causal(const mla_shape* shape, const void* q_nope, const void* q_r,
                                               int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                               const void* w_uv, const void* cache, const int32_t* slot_frame,
                                               const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                                               void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- query path
 * Queries of the chunk's tokens (hyper.ai summary, Method: a query latent is
 * derived from each token, and the per-head positional query is computed
 * from that latent and rotated at attention time; the per-head content query
 * is read as the query latent's own per-head up-projection):
 *   c_q[r]        = W_dq x[r]                 (rounded to dtype)
 *   q_nope[r][h]  = W_uq[h] c_q[r]
 *   q_r[r][h]     = W_qr[h] c_q[r]            (unrotated; mla_absorb_q and the
 *                                               chunk_attend calls rotate it)
 *   d_cq          query latent width: a multiple of 8, at most 65536 (the
 *                 pages leave it open)
 *   x      (device) [B][n_frames * T][hidden]  the chunk's tokens (the same
 *                   rows mla_cache_write takes)
 *   w_dq   (device) [d_cq][hidden]
 *   w_uq   (device) [H][d_head][d_cq]
 *   w_qr   (device) [H][d_rope][d_cq]
 *   c_q    (device) [B][n_frames * T][d_cq]      output (the query latent)
 *   q_nope (device) [B][n_frames * T][H][d_head] output
 *   q_r    (device) [B][n_frames * T][H][d_rope] output
 * Three matrix products on `stream`; fp32 accumulation. d_rope must be a
 * multiple of 8. n_frames < 1 returns MLA_ERR_RANGE. */
mla_status mla_query_project(const mla_shape* shape, int32_t d_cq, const void* x, int32_t n_frames,
                             const void* w_dq, const void* w_uq, const void* w_qr, void* c_q, void* q_nope,
                             void* q_r, void* stream);

/* ---------------------------------------------------------------- absorbed query path
 * The query path with the key up-projection folded in (the re-association
 * of the hyper.ai summary's content score, applied to the query path as
 * well): W_uk[h]^T q_nope[h] = (W_uk[h]^T W_uq[h]) c_q, so one product of
 * the query latent with per-head absorbed weights gives the attention's
 * query directly.
 * mla_query_absorb_weights (once per layer, when the weights change):
 *   w_qabs[h][j][:] = (W_uk[h]^T W_uq[h])[j][:]  for j < d_c   (fp32 sums, rounded to dtype)
 *                   = W_qr[h][j - d_c][:]        for d_c <= j < d_c + d_rope
 *                   = 0                          up to Q = mla_qabs_dim
 *   w_uq (device) [H][d_head][d_cq], w_qr [H][d_rope][d_cq], w_uk [H][d_head][d_c],
 *   w_qabs (device) [H][Q][d_cq] output.
 * mla_query_project_absorbed: c_q = W_dq x (rounded), then
 *   q_abs[r][h] = g [ (w_qabs c_q)[h][0..d_c) | R(t, y, x) (w_qabs c_q)[h][d_c..) | 0 ]
 * with g = softmax scale * log2(e) and (t, y, x) the position of token r
 * (frame q_frame_first + r / T within its stream), rounded once: the input
 * of mla_flash_attend, equal to mla_query_project + mla_absorb_q up to
 * rounding.
 *   x (device) [B][n_frames * T][hidden]; w_dq [d_cq][hidden];
 *   rope_tables as for mla_absorb_q (must cover the query frames);
 *   c_q (device) [B][n_frames * T][d_cq] output; q_abs (device)
 *   [B][n_frames * T][H][Q] output. */
mla_status mla_query_absorb_weights(const mla_shape* shape, int32_t d_cq, const void* w_uq, const void* w_qr,
                                    const void* w_uk, void* w_qabs, void* stream);
mla_status mla_query_project_absorbed(const mla_shape* shape, int32_t d_cq, const void* x, int32_t q_frame_first,
                                      int32_t n_frames, const void* w_dq, const void* w_qabs,
                                      const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t, void* c_q,
                                      void* q_abs, void* stream);

/* ---------------------------------------------------------------- output projection
 * u[r] = W_o [o[r][0]; ...; o[r][H-1]]: the concatenated heads projected back
 * to the token width (the output projection of multi-head attention; the
 * pages do not describe it).
 *   o   (device) [B][n_frames * T][H][d_head]  (out of the chunk_attend calls)
 *   w_o (device) [hidden][H * d_head]
 *   u   (device) [B][n_frames * T][hidden]      output
 * One matrix product on `stream`; fp32 accumulation. */
mla_status mla_output_project(const mla_shape* shape, const void* o, int32_t n_frames, const void* w_o, void* u,
                              void* stream);

/* ---------------------------------------------------------------- whole layer
 * One layer's chunk step in one call, on `stream`, in this order:
 * mla_query_project (queries from the chunk's tokens x) together with
 * mla_cache_write (the same tokens into the ring): the query latent and the
 * cached rows [c | kR] come from one product of x with
 * [W_dq ; W_dkv ; W_kR], so x is read once (the cached rows equal
 * mla_cache_write's up to the order of the fp32 sums); then
 * mla_chunk_attend in the form
 * mla_chunk_attend_form names or, with frame_causal != 0,
 * mla_chunk_attend_frame_causal (the chunk's queries over the window),
 * mla_output_project (u = W_o of the heads' outputs). The query
 * latent, the queries, the heads' outputs and the attention's workspace are
 * carved from `workspace` (at least mla_layer_step_workspace_bytes bytes;
 * its contents on entry do not matter). Every part's arguments are checked
 * before the first launch, with the statuses the parts document.
 *   weights (host) struct of device pointers, the layouts of the parts;
 *   x (device) [B][n_frames * T][hidden]; frames frame_first ..
 *   frame_first + n_frames - 1 (n_frames <= window_frames), which are also
 *   the query frames (rope tables must cover them); cache, slot_frame as
 *   for mla_cache_write; u (device) [B][n_frames * T][hidden] output. */
typedef struct mla_layer_weights {
  const void* w_dkv; /* [d_c][hidden] */
  const void* w_kr;  /* [d_rope][hidden] */
  const void* w_dq;  /* [d_cq][hidden] */
  const void* w_uq;  /* [H][d_head][d_cq] */
  const void* w_qr;  /* [H][d_rope][d_cq] */
  const void* w_uk;  /* [H][d_head][d_c] */
  const void* w_uv;  /* [H][d_head][d_c] */
  const void* w_o;   /* [hidden][H * d_head] */
  const void* w_qabs; /* optional, [H][Q][d_cq] from mla_query_absorb_weights: when set and
                         the latent form runs, the queries go through
                         mla_query_project_absorbed. The per-head form needs w_uq, w_qr
                         and w_uk; where any of them is NULL the latent form runs */
} mla_layer_weights;

size_t mla_layer_step_workspace_bytes(const mla_shape* shape, int32_t d_cq, int32_t n_frames);
mla_status mla_layer_step(const mla_shape* shape, int32_t d_cq, const mla_layer_weights* weights, const void* x,
                          int32_t frame_first, int32_t n_frames, void* cache, int32_t* slot_frame,
                          const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t, int32_t frame_causal,
                          void* u, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
