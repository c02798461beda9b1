/*
 * qwen3_prefill.h — C ABI of the MI355X (gfx950) Qwen3/Qwen3-VL text decoder-layer prefill.
 *
 * The library computes the full-sequence causal prefill of one Qwen3/Qwen3-VL text
 * decoder layer (every token at once):
 *
 *   xn = RMSNorm(x, attn_norm)                                 plain weight, eps inside the sqrt
 *   q, k, v = xn Wq^T, xn Wk^T, xn Wv^T                        no biases
 *   q, k = per-head RMSNorm (q_norm / k_norm), then interleaved three-axis MRoPE
 *   o = causal GQA softmax(q k^T / sqrt(head_dim)) v
 *   y1 = x + o Wo^T
 *   y2 = y1 + (silu(RMSNorm(y1, ffn_norm) Wg^T) * (RMSNorm(y1, ffn_norm) Wu^T)) Wd^T
 *   y2[rows[i]] += deepstack[i]                                 optional, image-token rows only
 *
 * Around it: the whole-model text prefill to the last position's logits, the KV cache a prefill
 * can leave and one-token decode steps over it, bidirectional attention and rotary tables for
 * vision-tower blocks, and weight-only quantized (Q4_0, int8-row) projections (sections below).
 *
 * Sources (web pages, cited by title and item):
 *   hf2q 0.1.1, qwen3vl_text/forward.rs — module doc (the per-layer graph of the peer
 *     reference), Phase D (position-gated DeepStack residual add), argument validation of
 *     `forward_text_prefill_logits_last`.
 *   cortiq-engine 0.8.21, qwen3te.rs — module doc (q/k RMSNorm before the rotation, GQA,
 *     split-half RoPE, plain-w RMSNorm, no final norm), `rms_norm_into`, `silu`, `norm_rope`,
 *     `attention_gemm`, the per-pair causal loop and `encode_with_images`.
 *   inferencelayer 0.2.3, vision.rs — `mrope_positions` (what the three position axes hold).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library never allocates
 *     or frees device memory inside these calls and keeps no pointer after a call returns.
 *     Tensor pointers must be 16-byte aligned (rows move in 16-byte vectors); a misaligned one
 *     returns QWEN3_ERR_INVALID_ARG. Allocator-returned buffers (hipMalloc, torch) satisfy this.
 *   - Matrices are row-major. Weights use the torch nn.Linear layout [out_features, in_features].
 *     Activations are token-major: [seq_len, ...]; q/k/v/attention outputs are [seq_len, heads,
 *     head_dim] contiguous.
 *   - bf16 / f16 tensors hold IEEE bfloat16 / binary16 bit patterns (uint16_t); f32 tensors hold
 *     IEEE binary32.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default stream).
 *     No call synchronizes the device.
 *   - Arguments are checked on the host before anything is enqueued. A failed check returns a
 *     nonzero qwen3_status, enqueues nothing, and sets a message readable through
 *     qwen3_last_error(). There is no fallback path: an unsupported shape is an error.
 *   - A HIP launch error returns QWEN3_ERR_HIP with the HIP error text.
 */
#ifndef QWEN3_PREFILL_H
#define QWEN3_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. QWEN3_F16_TILED is a weight storage format only (cfg.wdtype): fp16 values
 * with each projection matrix in the tiled layout that qwen3_tile_weights writes. */
typedef enum { QWEN3_F32 = 0, QWEN3_BF16 = 1, QWEN3_F16 = 2, QWEN3_F16_TILED = 3 } qwen3_dtype;

typedef enum {
  QWEN3_OK = 0,
  QWEN3_ERR_INVALID_ARG = 1,  /* a pointer, size or relation among sizes is invalid      */
  QWEN3_ERR_UNSUPPORTED = 2,  /* valid, but a shape or dtype this library does not run   */
  QWEN3_ERR_WORKSPACE = 3,    /* workspace pointer NULL or smaller than required         */
  QWEN3_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed              */
} qwen3_status;

/* Shape and numerics of one decoder layer.
 *   hidden      H; multiple of 256, at most 16384.
 *   n_heads     query heads nh; n_heads % n_kv_heads == 0 and n_heads / n_kv_heads in {1,2,4,8}
 *               (16-bit operands); any divisor for f32.
 *   n_kv_heads  KV heads nkv (GQA: query head h reads KV head h / (nh / nkv), cortiq-engine
 *               qwen3te.rs, `attention_gemm`).
 *   head_dim    hd: 64 or 128 (16-bit operands and f32 alike).
 *   ffn         F, the SwiGLU width; multiple of 128.
 *   rms_eps     eps added to the mean of squares inside the square root (`rms_norm_into`).
 *   rope_theta  RoPE base: pair i < hd/2 turns at theta^(-2i/hd) per position (`norm_rope`).
 *   mrope_section  (t, h, w) pair counts: sum == hd/2, 3*h <= hd/2 and 3*w <= hd/2. Pair i
 *               follows the h axis when i % 3 == 1 and i < 3*h, the w axis when i % 3 == 2 and
 *               i < 3*w, and the t axis otherwise (Qwen3-VL interleaved MRoPE, `norm_rope`).
 *   wdtype      dtype of the weights: QWEN3_BF16, QWEN3_F16 or QWEN3_F32; or QWEN3_F16_TILED:
 *               fp16 weights whose seven projection matrices (wq, wk, wv, wo, w_gate, w_up,
 *               w_down) are stored in the tiled layout (qwen3_tile_weights) while the norm
 *               vectors, DeepStack slabs, embeddings and LM head stay plain row-major fp16.
 *               Same values and same results as QWEN3_F16; each 32-wide K step of 16 weight
 *               rows is then one contiguous 1 KiB block, which the products load faster
 *               (requires act_dtype QWEN3_F16).
 *   act_dtype   dtype of the intermediate matrix-product operands (normalized activations,
 *               q, k, v, attention probabilities and output, the SwiGLU activation):
 *                 QWEN3_F16  fp16 operands, fp32 accumulation and softmax (with bf16 weights,
 *                            each weight tile is converted to fp16 on its way into LDS: exact
 *                            for |w| in [2^-17, 65504]);
 *                 QWEN3_BF16 bf16 operands (bf16 weights only);
 *                 QWEN3_F32  fp32 end to end (requires wdtype QWEN3_F32).
 *               fp16 and bf16 run at the same MFMA rate; fp16 keeps 3 more mantissa bits
 *               but holds magnitudes only up to 65504. With fp16 operands the SwiGLU
 *               activation is stored as 2^-4 * a and the down product scales its sum back by
 *               2^4 (both exact), so activations up to 65504 * 16 (about 1.05e6) stay
 *               finite; the other fp16 operands (normalized rows, q, k, v, probabilities,
 *               attention output) hold up to 65504 and become infinite beyond (such a model
 *               needs QWEN3_BF16). Measured agreement of the layer output with an exact (float64)
 *               reference, max |error| / RMS over the output, on synthetic N(0, 0.02)
 *               weights:
 *                 QWEN3_F16   2e-3 .. 5e-3 at every shape measured (2048-hidden layers at
 *                             1024/2048 tokens, the 4096-hidden 4-layer stack at 4096
 *                             tokens, the 5120-hidden layer at 8192 tokens);
 *                 QWEN3_BF16  about 1.2e-2 on the 2048-hidden layers; 1.8e-2 .. 3.4e-2 on the
 *                             4096- and 5120-hidden layers, i.e. ABOVE a 2e-2 bound there: the
 *                             down projection sums 12k-26k products of bf16-rounded operands.
 *   resid_dtype dtype of the residual stream x_in/x_out; must be QWEN3_F32.
 */
typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, ffn;
  float rms_eps, rope_theta;
  int32_t mrope_section[3];
  qwen3_dtype wdtype;
  qwen3_dtype act_dtype;
  qwen3_dtype resid_dtype;
} qwen3_layer_cfg;

/* Device pointers to one layer's weights, all of dtype cfg.wdtype, layout [out, in]
 * (QWEN3_F16_TILED: the seven matrices in the tiled layout, the four vectors plain fp16). */
typedef struct {
  const void *attn_norm;   /* [H]                 input RMSNorm weight                    */
  const void *wq;          /* [nh*hd, H]                                                  */
  const void *wk;          /* [nkv*hd, H]                                                 */
  const void *wv;          /* [nkv*hd, H]                                                 */
  const void *q_norm;      /* [hd]                per-head RMSNorm weight on q            */
  const void *k_norm;      /* [hd]                per-head RMSNorm weight on k            */
  const void *wo;          /* [H, nh*hd]                                                  */
  const void *ffn_norm;    /* [H]                 post-attention RMSNorm weight           */
  const void *w_gate;      /* [F, H]                                                      */
  const void *w_up;        /* [F, H]                                                      */
  const void *w_down;      /* [H, F]                                                      */
} qwen3_layer_weights;

/* Bytes of device workspace qwen3_layer_prefill needs for `seq_len` tokens (0 if cfg is
 * NULL or seq_len < 1). The workspace holds the normalized activations, q/k/v, the attention
 * output, the SwiGLU activation and the device copy of the DeepStack row list; its contents
 * on entry do not matter. The normalized activations, attention output and SwiGLU activation
 * (the A operands of the products) take seq_len rounded up to a multiple of 16 rows: with
 * 16-bit operands they are kept in the tiled layout. */
size_t qwen3_layer_workspace_bytes(const qwen3_layer_cfg *cfg, int32_t seq_len);

/* One decoder layer over all `seq_len` tokens (the recipe at the top of this file).
 *   x_in, x_out   [S, H] f32 residual stream in and out; x_out may equal x_in (in place),
 *                 other overlaps are not allowed.
 *   positions     [3, S] int32: the t row, then the h row, then the w row. A text token has
 *                 t = h = w; an image token has one t per image and h, w on its merged grid
 *                 (inferencelayer vision.rs, `mrope_positions`). Values must be >= 0.
 *   ds_rows, n_ds DeepStack rows: a HOST array of n_ds >= 0 strictly increasing row indices in
 *                 [0, S), or NULL/0 (hf2q forward.rs, Phase D: the slab is added on image-token
 *                 rows only; `forward_text_prefill_logits_last` rejects an image-token position
 *                 outside the sequence). The list is checked on the host and copied into the
 *                 workspace on `stream` during the call; the caller may reuse it on return.
 *   ds            device [n_ds, H] of cfg.wdtype (plain fp16 for QWEN3_F16_TILED): ds[i] is
 *                 added to output row ds_rows[i]
 *                 after the FFN residual; must be NULL when n_ds == 0 and non-NULL otherwise.
 *   workspace     at least qwen3_layer_workspace_bytes(cfg, S) bytes, 256-byte aligned.
 * Errors: seq_len < 1, NULL pointers, unsupported shapes, a DeepStack row outside [0, S) or
 * not above its predecessor, a slab without rows (or rows without a slab), or a small
 * workspace return QWEN3_ERR_INVALID_ARG / _UNSUPPORTED / _WORKSPACE before anything is
 * enqueued. */
int qwen3_layer_prefill(const qwen3_layer_cfg *cfg, const qwen3_layer_weights *w,
                        const void *x_in, void *x_out, int32_t seq_len,
                        const int32_t *positions, const int32_t *ds_rows, int32_t n_ds,
                        const void *ds, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Per-head RMSNorm then interleaved-MRoPE rotation of q and k, in place
 * (cortiq-engine qwen3te.rs, `norm_rope`).
 *   q [S, n_heads, head_dim], k [S, n_kv_heads, head_dim] of `dtype`, contiguous; n_heads and
 *   n_kv_heads >= 1, and q, k, q_norm, k_norm all non-NULL.
 *   q_norm, k_norm [head_dim] of `norm_dtype`. Each (token, head) row x is replaced by
 *   r = x / sqrt(mean(x^2) + eps) * norm_w, then for i < hd/2 the pair (r_i, r_{i+hd/2}) is
 *   rotated by phi = positions[axis(i)][s] * theta^(-2i/hd) (axis rule under qwen3_layer_cfg).
 *   positions [3, S] int32 as for qwen3_layer_prefill. head_dim 64 or 128; any dtypes. The
 *   norm and rotation run in fp32 (the angle is formed and range-reduced in fp64). */
int qk_norm_mrope(void *q, void *k, int32_t seq_len, int32_t n_heads, int32_t n_kv_heads,
                  int32_t head_dim, const void *q_norm, const void *k_norm, float eps,
                  const int32_t *positions, float theta, const int32_t mrope_section[3],
                  qwen3_dtype dtype, qwen3_dtype norm_dtype, void *stream);

/* Causal grouped-query attention (cortiq-engine qwen3te.rs, per-pair loop / `attention_gemm`):
 *   out[s, h] = sum_{j<=s} softmax_j(scale * q[s,h] . k[j,g]) v[j,g],  g = h / (nh / nkv).
 *   q, out [S, n_heads, head_dim]; k, v [S, n_kv_heads, head_dim]; all `dtype`, contiguous.
 *   scale is normally 1/sqrt(head_dim). head_dim 64 or 128. bf16 / f16: nh/nkv in {1,2,4,8},
 *   16-bit products with fp32 accumulation and fp32 online softmax. f32: fp32 throughout.
 *   out must not overlap q, k or v. */
int gqa_causal_attention(const void *q, const void *k, const void *v, void *out,
                         int32_t seq_len, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, float scale, qwen3_dtype dtype, void *stream);

/* Bidirectional (non-causal) attention of a vision-tower block (inferencelayer 0.2.3 vision.rs,
 * the block's `attention`; cortiq-engine 0.8.51 onevision2.rs, `attend`): as
 * gqa_causal_attention with every key visible to every query,
 *   out[s, h] = sum_{j<S} softmax_j(scale * q[s,h] . k[j,g]) v[j,g].
 *   Same layouts, types, limits and errors. */
int gqa_bidirectional_attention(const void *q, const void *k, const void *v, void *out,
                                int32_t seq_len, int32_t n_heads, int32_t n_kv_heads,
                                int32_t head_dim, float scale, qwen3_dtype dtype, void *stream);

/* Rotary tables of a vision-tower patch grid (frames x grid_h x grid_w patches, merge x merge
 * merge blocks): cos_out, sin_out device fp32 [frames*grid_h*grid_w, head_dim], patches in
 * merge-block order (frames in order; within a frame the blocks row-major, each block's patches
 * row-major), entries j and j + head_dim/2 equal.
 *   layout 0 (inferencelayer 0.2.3 vision.rs, `rope_tables_2d`): with half = head_dim/2 and
 *     nf = half/2, angle j < nf = row * theta^(-2j/half), angle nf + j = col * theta^(-2j/half);
 *     head_dim a multiple of 4.
 *   layout 1 (cortiq-engine 0.8.51 onevision2.rs, `rope_tables`): the half angles split 4:6:6
 *     between frame, row and column (unit = half/16), an axis with n slots turning by
 *     theta^(-i/n); head_dim a multiple of 32.
 * Angles are formed in fp64. grid_h and grid_w must be multiples of merge. */
int vision_rope_tables(int32_t frames, int32_t grid_h, int32_t grid_w, int32_t merge, int32_t head_dim,
                       float theta, int32_t layout, float *cos_out, float *sin_out, void *stream);

/* Applies rotary tables in place to x [n, heads, head_dim] of `dtype` (row r of head h at
 * x + r*row_stride + h*head_dim), cos_tab / sin_tab fp32 [n, head_dim], fp32 arithmetic:
 *   pairing 0 (inferencelayer vision.rs, the block's `attention`): rotate_half on split halves,
 *     y_i = x_i c_i - x_{i+half} s_i, y_{i+half} = x_{i+half} c_{i+half} + x_i s_{i+half};
 *   pairing 1 (onevision2.rs, `split_rope`): adjacent lanes,
 *     y_2i = x_2i c_2i - x_2i+1 s_2i, y_2i+1 = x_2i+1 c_2i+1 + x_2i s_2i+1 (each lane takes its
 *     own table entry, so the two lanes of a pair turn by different angles). */
int apply_rope_tables(void *x, int32_t n, int32_t heads, int32_t head_dim, int64_t row_stride,
                      const float *cos_tab, const float *sin_tab, int32_t pairing, qwen3_dtype dtype,
                      void *stream);

/* SwiGLU feed-forward with optional residual (cortiq-engine qwen3te.rs, gate/up/act/down):
 *   out = [residual +] (silu(x W_gate^T) * (x W_up^T)) W_down^T,  silu(z) = z / (1 + e^-z).
 *   W_gate, W_up [ffn, hidden] and W_down [hidden, ffn] of `wdtype`; x_normed [S, hidden] of
 *   `x_dtype`, which is also the product operand format (the (wdtype, x_dtype) pairs allowed
 *   are those of (wdtype, act_dtype) in qwen3_layer_cfg). residual [S, hidden] f32 or NULL.
 *   out [S, hidden] of `out_dtype`: f32, or x_dtype when residual is NULL; out may equal
 *   residual. wdtype QWEN3_F16_TILED: the three matrices in the tiled layout. workspace holds
 *   the [S, ffn] activation (with fp16 operands scaled by 2^-4, undone exactly in the down
 *   product, as for qwen3_layer_prefill): swiglu_ffn_workspace_bytes() bytes. */
int swiglu_ffn(const void *x_normed, const void *w_gate, const void *w_up, const void *w_down,
               const void *residual, void *out, int32_t seq_len, int32_t hidden, int32_t ffn,
               qwen3_dtype wdtype, qwen3_dtype x_dtype, qwen3_dtype out_dtype, void *workspace,
               size_t workspace_bytes, void *stream);
size_t swiglu_ffn_workspace_bytes(int32_t seq_len, int32_t ffn, qwen3_dtype x_dtype);

/* Weight preparation for QWEN3_F16_TILED (for callers that load weights once and run many
 * prefills; the layer computes the same products either way).
 *   src   device [rows, cols] row-major of src_dtype (QWEN3_F32, QWEN3_BF16 or QWEN3_F16).
 *   dst   device rows * cols fp16 values (2 * rows * cols bytes, 16-byte aligned), written
 *         in the tiled layout: 16-row x 32-column tiles of 1 KiB, row-major inside a tile,
 *         tiles ordered by row group and then by column, i.e. element (r, c) at
 *         ((r / 16) * (cols / 32) + c / 32) * 512 + (r % 16) * 32 + c % 32.
 *   Each value is rounded to the nearest fp16 (ties to even): exact for bf16 and f32 values
 *   representable in fp16 (bf16 values of magnitude in [2^-14, 65504]); magnitudes beyond
 *   65504 become infinite, as in any fp16 conversion. rows must be a positive multiple of 16,
 *   cols of 32; dst must not overlap src. Errors (QWEN3_ERR_INVALID_ARG /
 *   QWEN3_ERR_UNSUPPORTED) are returned before anything is enqueued. */
int qwen3_tile_weights(const void *src, qwen3_dtype src_dtype, int32_t rows, int32_t cols, void *dst,
                       void *stream);

/* Row RMSNorm with a plain weight (cortiq-engine qwen3te.rs, `rms_norm_into`):
 *   y[s] = x[s] / sqrt(mean_j x[s,j]^2 + eps) * w.
 *   x [rows, hidden] f32; w [hidden] of w_dtype; y [rows, hidden] of y_dtype.
 *   hidden a multiple of 256. y must not overlap x. */
int rms_norm_rows(const float *x, const void *w, void *y, int32_t rows, int32_t hidden,
                  float eps, qwen3_dtype w_dtype, qwen3_dtype y_dtype, void *stream);

/* Thread-local text of the last nonzero status returned on this thread ("" if none). */
const char *qwen3_last_error(void);

/* ---- Measurement aid -------------------------------------------------------------------
 * When enabled, every kernel launched by the calls above is bracketed by a pair of hipEvents
 * recorded on the call's stream. qwen3_timing_collect() waits for the recorded events, sums
 * the elapsed time per kernel name (and takes the median launch), writes up to `max_entries`
 * entries and clears the record. At most 65536 launches are recorded between collects; later
 * ones are not timed. */
typedef struct {
  char name[48];
  int32_t launches;
  double total_ms;
  double median_ms;   /* median of the launches' times (mean of the two middle ones if even) */
} qwen3_kernel_time;

int qwen3_timing_enable(int enable);
int qwen3_timing_collect(qwen3_kernel_time *out, int32_t max_entries, int32_t *n_out);

/* MFMA throughput probe: `workgroups` workgroups of 4 waves, each wave issuing iters x 8
 * independent 32x32x16 fp16 MFMAs (32768 FLOP each) with no memory traffic, so the launch time
 * measures the matrix cores' rate at the clock the chip holds under that load. clocks (device,
 * 2 x uint64) receives the shader-clock cycles (s_memtime) and the 100 MHz real-time ticks
 * (s_memrealtime) that one wave spent in its loop: their ratio times 100 MHz is that clock.
 * sink (device, 1 float) is never written in practice (it keeps the products alive). */
int qwen3_mfma_probe(int32_t workgroups, int32_t iters, float *sink, unsigned long long *clocks, void *stream);

/* ---- Whole-model text prefill: last position's logits --------------------------------------
 *
 * hf2q 0.1.1, qwen3vl_text/forward.rs: the module doc (per-layer graph; "Final": output RMSNorm,
 * then the LM head, which is the token embedding table when the embeddings are tied) and
 * `forward_text_prefill_logits_last` (embedding lookup, the layers in order with DeepStack slab
 * il added after layer il for il < n_deepstack_layers, final RMSNorm and LM head on the last
 * position only; an empty prompt and out-of-range token ids are errors).
 */
typedef struct {
  qwen3_layer_cfg layer;        /* shared by every decoder layer                                */
  int32_t n_layers;             /* >= 0                                                         */
  int32_t vocab;                /* rows of the embedding table and of the LM head, >= 1         */
  int32_t n_deepstack_layers;   /* layers 0 .. n-1 receive DeepStack slab il; 0 <= n <= n_layers */
} qwen3_model_cfg;

typedef struct {
  const void* token_embd;              /* device [vocab, hidden], layer.wdtype                  */
  const qwen3_layer_weights* layers;   /* HOST array of n_layers entries (device pointers)      */
  const void* output_norm;             /* device [hidden], layer.wdtype                         */
  const void* lm_head;                 /* device [vocab, hidden], layer.wdtype; NULL = tied      */
} qwen3_model_weights;                 /* (QWEN3_F16_TILED: these three plain row-major fp16)   */

/* Workspace for qwen3_model_prefill_logits_last: the token ids, the fp32 residual stream
 * [S, hidden], the last row's normalized state and one layer's workspace. 0 for invalid input. */
size_t qwen3_model_workspace_bytes(const qwen3_model_cfg* cfg, int32_t seq_len);

/* logits[v] for v < vocab: the LM head applied to RMSNorm(output_norm) of the last position's
 * hidden state after all layers.
 *   tokens     HOST array [seq_len] of ids in [0, vocab), checked on the host before anything is
 *              enqueued and copied into the workspace during the call.
 *   positions  device [3][seq_len] int32 (t, h, w rows), as for qwen3_layer_prefill.
 *   ds_rows, n_ds  HOST DeepStack row list shared by the first n_deepstack_layers layers (rules
 *              and errors as for qwen3_layer_prefill); ds is a HOST array of n_deepstack_layers
 *              device slabs [n_ds, hidden] (layer.wdtype), or NULL when n_ds == 0.
 *   logits     device [vocab] fp32, written.
 * Every layer uses the same workspace region in turn; the residual stream stays in fp32. */
int qwen3_model_prefill_logits_last(const qwen3_model_cfg* cfg, const qwen3_model_weights* w,
                                    const int32_t* tokens, int32_t seq_len, const int32_t* positions,
                                    const int32_t* ds_rows, int32_t n_ds, const void* const* ds,
                                    float* logits, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ---- KV cache and one decode step -------------------------------------------------------------
 *
 * hf2q 0.1.1, qwen3vl_text/forward.rs: the module doc's note on why the prefill keeps no KV cache
 * yet (a generation loop would prefill prompt + decoded tokens again per new token; keeping the
 * keys and values for incremental decode is the later step) and point 4 of the notes on
 * `forward_text_prefill_logits_last`. Reading taken here: per layer the cache keeps, for every
 * position and KV head, k' (k after the per-head RMSNorm and the rotation) and v, exactly as the
 * causal layer forms them; a decode step runs the layer on one new token whose query attends to
 * every cached key and to its own, so its output equals the last row of a prefill over the longer
 * sequence.
 *
 * Cache layout: K and V are separate device buffers, each [n_kv_heads][capacity][head_dim]
 * (head-major: one KV head's rows are contiguous), of the layer's act_dtype (f16 by default).
 * Row r of head g lives at cache + (g * capacity + r) * head_dim elements. The caller owns both
 * buffers and the count of live rows.
 */

/* Copies n token rows of k and v into cache rows row0 .. row0+n-1, converting src_dtype to
 * cache_dtype (round to nearest even; the same type copies bit for bit).
 *   k, v        [n, n_kv_heads, head_dim] of src_dtype, token t of head g at k + t*k_stride +
 *               g*head_dim (strides in elements, multiples of 8, >= n_kv_heads*head_dim).
 *   head_dim    a multiple of 8. row0 >= 0, row0 + n <= capacity.
 * The caches must not overlap k or v. */
int kv_cache_write(const void *k, const void *v, int64_t k_stride, int64_t v_stride, int32_t n,
                   int32_t n_kv_heads, int32_t head_dim, qwen3_dtype src_dtype, void *k_cache,
                   void *v_cache, qwen3_dtype cache_dtype, int32_t capacity, int32_t row0, void *stream);

/* qwen3_layer_prefill that also leaves the layer's cache: k' and v of positions 0 .. seq_len-1
 * are written to rows 0 .. seq_len-1 of k_cache / v_cache (act_dtype, capacity >= seq_len rows
 * per KV head). The output is the same as qwen3_layer_prefill's, bit for bit. The caches must
 * not overlap the workspace, x_in or x_out. */
int qwen3_layer_prefill_kv(const qwen3_layer_cfg *cfg, const qwen3_layer_weights *w,
                           const void *x_in, void *x_out, int32_t seq_len,
                           const int32_t *positions, const int32_t *ds_rows, int32_t n_ds,
                           const void *ds, void *k_cache, void *v_cache, int32_t capacity,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Attention of one query row per head over the first `len` rows of the caches:
 *   out[h] = sum_{j<len} softmax_j(scale * q[h] . K[g][j]) V[g][j],  g = h / (nh / nkv).
 *   q, out      [n_heads, head_dim] fp32 (the query is rounded to cache_dtype before the
 *               products, which accumulate in fp32; softmax and output in fp32).
 *   k_cache, v_cache  [n_kv_heads][capacity][head_dim] of cache_dtype; 1 <= len <= capacity.
 *   head_dim 64 or 128; n_heads / n_kv_heads <= 16; scale finite and > 0.
 *   workspace   gqa_decode_attention_workspace_bytes(n_heads, n_kv_heads, head_dim, len) bytes,
 *               256-byte aligned (per-split partial results; contents on entry do not matter). */
int gqa_decode_attention(const float *q, const void *k_cache, const void *v_cache, int32_t capacity,
                         int32_t len, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                         qwen3_dtype cache_dtype, float *out, void *workspace, size_t workspace_bytes,
                         void *stream);
/* Workspace for gqa_decode_attention; also enough for every smaller len. 0 for invalid input. */
size_t gqa_decode_attention_workspace_bytes(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t len);

/* gqa_decode_attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same checks, kernels and
 * results, with the per-split partial results in a fixed array of the library's device code
 * (QWEN3_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends) instead of a workspace.
 * Calls whose gqa_decode_attention_workspace_bytes() exceeds that size return
 * QWEN3_ERR_UNSUPPORTED (the 8B shape, 32 query / 8 KV heads of 128, needs 1 MiB at any length).
 * Every call on one GPU uses that GPU's one array: calls that overlap on one GPU (several host
 * threads, or several streams) race and must be ordered by the caller. Allocates nothing. */
#define QWEN3_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int gqa_decode_attention_noalloc(const float *q, const void *k_cache, const void *v_cache, int32_t capacity,
                                 int32_t len, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                                 qwen3_dtype cache_dtype, float *out, void *stream);

/* One new token through the layer, reading positions 0 .. len-1 from the caches and appending
 * its own k' and v at row len:
 *   xn = RMSNorm(x); q, k, v = xn W^T; per-head RMSNorm + interleaved MRoPE at `position`;
 *   K[g][len] = k', V[g][len] = v; o = attention of q over rows 0 .. len; y1 = x + o Wo^T;
 *   x_out = y1 + SwiGLU FFN(RMSNorm(y1)).
 *   x_in, x_out [hidden] f32 (x_out may equal x_in); position device int32 [3] (t, h, w);
 *   0 <= len < capacity. The new token's vectors stay in fp32 (matrix-vector products with
 *   fp32 accumulation); the cache rows are stored in act_dtype. The same shape limits as
 *   qwen3_layer_prefill, plus head_dim 64 or 128 and n_heads / n_kv_heads <= 16.
 *   workspace   qwen3_layer_decode_workspace_bytes(cfg, capacity) bytes, 256-byte aligned.
 * No DeepStack: decoded tokens are text. */
int qwen3_layer_decode(const qwen3_layer_cfg *cfg, const qwen3_layer_weights *w, const float *x_in,
                       float *x_out, const int32_t *position, void *k_cache, void *v_cache,
                       int32_t capacity, int32_t len, void *workspace, size_t workspace_bytes,
                       void *stream);
size_t qwen3_layer_decode_workspace_bytes(const qwen3_layer_cfg *cfg, int32_t capacity);

/* Whole-model forms of the cache and the decode step.
 * qwen3_model_prefill_logits_last_kv: qwen3_model_prefill_logits_last that also leaves every
 *   layer's cache; k_caches, v_caches are HOST arrays of n_layers device pointers (layer l's
 *   caches as for qwen3_layer_prefill_kv), capacity >= seq_len. Same workspace.
 * qwen3_model_decode_logits: logits [vocab] fp32 of one new token (host id in [0, vocab)) at
 *   `position` (device int32 [3]) after len tokens: the embedding row, every layer's decode step
 *   (each appends its cache row len), final RMSNorm and the LM head. Equals the last position's
 *   logits of a prefill over the len + 1 tokens. workspace: qwen3_model_decode_workspace_bytes. */
int qwen3_model_prefill_logits_last_kv(const qwen3_model_cfg* cfg, const qwen3_model_weights* w,
                                       const int32_t* tokens, int32_t seq_len, const int32_t* positions,
                                       const int32_t* ds_rows, int32_t n_ds, const void* const* ds,
                                       void* const* k_caches, void* const* v_caches, int32_t capacity,
                                       float* logits, void* workspace, size_t workspace_bytes, void* stream);
size_t qwen3_model_decode_workspace_bytes(const qwen3_model_cfg* cfg, int32_t capacity);
int qwen3_model_decode_logits(const qwen3_model_cfg* cfg, const qwen3_model_weights* w, int32_t token,
                              const int32_t* position, void* const* k_caches, void* const* v_caches,
                              int32_t capacity, int32_t len, float* logits, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ---- Weight-only quantized projections ---------------------------------------------------------
 *
 * hf2q 0.1.1, qwen3vl_text/forward.rs, the dense FFN step: the converted Qwen3-VL checkpoints hold
 * their projections as GGML Q4_0 tensors. The page names the type only; the layout read here is
 * GGML's published Q4_0 block: 32 consecutive weights of a row per 18-byte block, a little-endian
 * binary16 scale d then 16 bytes of codes, byte j holding weight j's code in its low nibble and
 * weight j + 16's in its high nibble; weight = d * (code - 8). A row of K weights is K/32 blocks
 * back to back, rows back to back.
 * cortiq-engine 0.8.21, qwen3te.rs, `q8_exact_matmat`: int8 rows with a per-row scale, weight[o, j]
 * = row_scale[o] * q[o, j], activations not quantized.
 *
 * Projections with quantized weights compute x W^T with the dequantized W, each weight rounded
 * once to the operand type (f16 or bf16, round to nearest even: d * (code - 8) and
 * row_scale * q). In a prefill, a product group whose matrices are all Q4_0 (q|k|v, o, gate|up,
 * down) reads the blocks inside the MFMA product, decoding them in its weight-tile path, with
 * the same bits as the product over expanded weights; other quantized groups (int8 rows, or
 * Q4_0 mixed with int8 rows) are expanded into the workspace just before their product. A decode
 * step reads the quantized bytes directly (Q4_0: the activations are rounded to binary16 for
 * v_dot2 products with fp32 sums; int8 rows: fp32 activations).
 * Norm weights stay in cfg.wdtype; dense projections use cfg.wdtype as in qwen3_layer_weights.
 */
typedef enum { QWEN3_W_DENSE = 0, QWEN3_W_Q4_0 = 1, QWEN3_W_Q8_ROW = 2 } qwen3_wformat;

typedef struct {
  qwen3_wformat format;
  const void *data;       /* DENSE: [rows, cols] of cfg.wdtype (16-byte aligned); Q4_0: rows*cols/32
                             blocks of 18 bytes (4-byte aligned); Q8_ROW: int8 [rows, cols] (16-byte aligned) */
  const float *row_scale; /* Q8_ROW: fp32 [rows]; otherwise ignored                                        */
} qwen3_qmatrix;

typedef struct {
  const void *attn_norm;   /* [H] of cfg.wdtype */
  qwen3_qmatrix wq;        /* [nh*hd, H]        */
  qwen3_qmatrix wk;        /* [nkv*hd, H]       */
  qwen3_qmatrix wv;        /* [nkv*hd, H]       */
  const void *q_norm;      /* [hd]              */
  const void *k_norm;      /* [hd]              */
  qwen3_qmatrix wo;        /* [H, nh*hd]        */
  const void *ffn_norm;    /* [H]               */
  qwen3_qmatrix w_gate;    /* [F, H]            */
  qwen3_qmatrix w_up;      /* [F, H]            */
  qwen3_qmatrix w_down;    /* [H, F]            */
} qwen3_layer_qweights;

/* out [rows, cols] of out_dtype (f16 or bf16) = the dequantized matrix m (Q4_0 or Q8_ROW);
 * cols a multiple of 64. */
int dequantize_matrix(const qwen3_qmatrix *m, int32_t rows, int32_t cols, qwen3_dtype out_dtype, void *out,
                      void *stream);

/* Workspace of qwen3_layer_prefill_quant: the layer workspace plus room for the largest product
 * group expanded to 16 bits. */
size_t qwen3_layer_quant_workspace_bytes(const qwen3_layer_cfg *cfg, int32_t seq_len);

/* qwen3_layer_prefill (and, with non-NULL caches, qwen3_layer_prefill_kv) with per-projection
 * formats. Rules: act_dtype f16 or bf16 when any projection is quantized; wq, wk, wv all dense or
 * all quantized (Q4_0 and Q8_ROW may be mixed); w_gate and w_up share one format. k_cache and
 * v_cache are both NULL or both given (then capacity >= seq_len). */
int qwen3_layer_prefill_quant(const qwen3_layer_cfg *cfg, const qwen3_layer_qweights *w, const void *x_in,
                              void *x_out, int32_t seq_len, const int32_t *positions, const int32_t *ds_rows,
                              int32_t n_ds, const void *ds, void *k_cache, void *v_cache, int32_t capacity,
                              void *workspace, size_t workspace_bytes, void *stream);

/* qwen3_layer_decode with per-projection formats (same rules); the workspace is
 * qwen3_layer_decode_workspace_bytes(cfg, capacity). */
int qwen3_layer_decode_quant(const qwen3_layer_cfg *cfg, const qwen3_layer_qweights *w, const float *x_in,
                             float *x_out, const int32_t *position, void *k_cache, void *v_cache,
                             int32_t capacity, int32_t len, void *workspace, size_t workspace_bytes,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QWEN3_PREFILL_H */
