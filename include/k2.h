/*
 * k2.h — C ABI of the MI355X (gfx950) Krea 2 single-stream MMDiT library (libk2.so).
 *
 * What is computed follows, by page title and section:
 *   [API]      diffusers v0.43.0 model page "Krea2Transformer2DModel": constructor defaults and the
 *              forward() contract (hidden_states, encoder_hidden_states, timestep, position_ids,
 *              encoder_attention_mask; image-token velocity out).
 *   [ARTICLE]  article "Diffusers 中的 Krea2Transformer2DModel：Krea 2 单流 MMDiT 流匹配 Transformer
 *              架构全解": §二 (I/O contract and its ValueErrors), §三 (defaults and the axes check),
 *              §四 data flow, §四.1 TextFusion, §四.2 TransformerBlock, §四.3 Attention, §四.4 RMSNorm,
 *              §四.5 TimestepEmbedding, §四.6 FinalLayer.
 *   [PIPELINE] diffusers v0.43.0 pipeline page "Krea 2": Krea2Pipeline parameters (scheduler,
 *              is_distilled) and __call__ parameters (num_inference_steps, sigmas, guidance_scale).
 *   [QWEN21]   diffusers model page "QwenImage21Transformer2DModel": the block-causal attention
 *              item and build_token_metadata (image_ids), for k2_block_forward_block_causal.
 *
 * Conventions shared by every entry point
 *   - Pointers named *_w, *_b, tables, activations, outputs and workspace are DEVICE pointers owned by
 *     the caller; the library allocates no device memory and keeps no per-call state (the timing
 *     diagnostics at the end of this header are its only process-wide state).
 *   - Config and weight-table structs are HOST memory, read during the call only.
 *   - nn.Linear weights use PyTorch's (out_features, in_features) row-major layout, element type
 *     `dtype` (K2_F32: float, K2_BF16: bfloat16). Norm weights, modulation tables, biases, the
 *     residual stream, timesteps and position ids are float32 in both modes.
 *   - RMSNorm weights are zero-centred: the multiplier is (1 + w); NULL means w = 0.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream). The library never
 *     synchronises; the caller does. Inputs must stay valid until the stream has run the work.
 *   - Every function validates its arguments on the host before any launch and returns a k2_status.
 *     On error nothing is enqueued and k2_last_error() describes the failure (thread-local string).
 *     A launch failure returns K2_ERR_HIP; a fault inside a kernel surfaces at the caller's next sync.
 *   - Workspace: at least *_workspace_bytes() bytes of device memory, 256-byte aligned. Its contents
 *     on entry are ignored; it is clobbered.
 *   - Every other device pointer (weights, biases, norm weights, tables, activations, outputs) must be
 *     16-byte aligned: the kernels move 16 bytes per lane. Violations return K2_ERR_ALIGN.
 */
#ifndef K2_H
#define K2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  K2_OK = 0,
  K2_ERR_NULL = -1,      /* a required pointer is NULL */
  K2_ERR_SHAPE = -2,     /* sizes inconsistent (e.g. position_ids not (T+N, 3)) */
  K2_ERR_CONFIG = -3,    /* unsupported or inconsistent configuration */
  K2_ERR_DTYPE = -4,     /* unknown dtype */
  K2_ERR_WORKSPACE = -5, /* workspace too small or misaligned */
  K2_ERR_HIP = -6,       /* a HIP launch failed */
  K2_ERR_ALIGN = -7      /* a device pointer is not 16-byte aligned */
} k2_status;

typedef enum { K2_F32 = 0, K2_BF16 = 1 } k2_dtype;

/* ------------------------------------------------------------------------------------------------
 * One single-stream block ([ARTICLE] §四.2 block, §四.3 attention, §四.4 norm; defaults [API]).
 * Requirements checked by k2_block_forward: hidden == num_heads * head_dim ([API]: hidden size is
 * head dim times heads); num_heads % num_kv_heads == 0 with num_heads / num_kv_heads in {1, 2, 4};
 * head_dim in {64, 128}; axes_dims even and summing to head_dim ([ARTICLE] §三); hidden and
 * intermediate multiples of 8; B <= 65535; T <= 16384 text tokens.
 * --------------------------------------------------------------------------------------------- */
typedef struct {
  int hidden;        /* 6144 */
  int num_heads;     /* 48 query heads */
  int num_kv_heads;  /* 12 key/value heads (GQA) */
  int head_dim;      /* 128 */
  int intermediate;  /* 16384, SwiGLU hidden size */
  int axes_dims[3];  /* (32, 48, 48): head-dim split among the (t, h, w) rotary axes */
  float rope_theta;  /* 1000 */
  float eps;         /* 1e-5, every RMSNorm */
  int dtype;         /* k2_dtype of weights and of matrix operands between kernels */
} k2_block_cfg;

typedef struct {
  const float* scale_shift_table; /* (6, hidden) added to temb's 6 chunks; NULL = unmodulated block
                                     (text fusion: no modulation, gates of 1) */
  const float* norm1_w;           /* (hidden) */
  const float* norm2_w;           /* (hidden) */
  const float* norm_q_w;          /* (head_dim), shared by all query heads */
  const float* norm_k_w;          /* (head_dim), shared by all key heads */
  const void* to_q;               /* (num_heads*head_dim, hidden) */
  const void* to_k;               /* (num_kv_heads*head_dim, hidden) */
  const void* to_v;               /* (num_kv_heads*head_dim, hidden) */
  const void* to_gate;            /* (num_heads*head_dim, hidden), sigmoid output gate */
  const void* to_out;             /* (hidden, num_heads*head_dim) */
  const void* ff_gate;            /* (intermediate, hidden) */
  const void* ff_up;              /* (intermediate, hidden) */
  const void* ff_down;            /* (hidden, intermediate) */
} k2_block_weights;

/* Fills *cfg with the [API] constructor defaults (bf16). */
void k2_block_cfg_default(k2_block_cfg* cfg);

/* Workspace bytes k2_block_forward needs for B batch rows of T text + N image tokens;
   0 if cfg is NULL or sizes are negative. */
size_t k2_block_workspace_bytes(const k2_block_cfg* cfg, int B, int T, int N);

/* Byte offsets of the intermediate tensors inside the block workspace (valid after a call on the
   same sizes): x1/x2 (B*L, hidden) modulated norms, q (B*L, nh*hd) and k (B*L, nkv*hd) after q/k norm
   and RoPE, vt (B, nkv, hd, ldvt) values transposed (ldvt = 32 when L <= 32, else L rounded up to
   64), g (B*L, nh*hd) raw gate, og (B*L, nh*hd) gated attention output, a (B*L, intermediate)
   SwiGLU activation — all of element type dtype — mod (B, 6, hidden) float32 modulation, and reach
   (L) int32, the block-causal reach of k2_block_forward_block_causal. Intended for tests and
   debugging. */
typedef struct {
  size_t x1, q, k, vt, g, og, x2, a, rope, mod, reach, total;
  int ldvt;
} k2_block_workspace_layout;
int k2_block_workspace_layout_query(const k2_block_cfg* cfg, int B, int T, int N,
                                    k2_block_workspace_layout* out);

/* One block forward over the concatenated [text, image] sequence, L = T + N tokens per batch row:
     mod = temb (B, 6, hidden) + scale_shift_table          -> prescale, preshift, pregate,
                                                               postscale, postshift, postgate
     x1  = (1 + prescale) * RMSNorm(h; norm1_w) + preshift
     q,k = RMSNorm per head (norm_q_w / norm_k_w), then 3-axis RoPE from position_ids
     o   = softmax(q k^T / sqrt(head_dim) + key mask) v       (query head i reads kv head i / G)
     h  += pregate * to_out(o * sigmoid(to_gate(x1)))
     x2  = (1 + postscale) * RMSNorm(h; norm2_w) + postshift
     h  += postgate * ff_down(silu(ff_gate(x2)) * ff_up(x2))
   hidden_in / hidden_out: (B, L, hidden) float32 residual stream, row b*L + l; may alias.
   temb: (B, 6*hidden) float32 shared modulation; NULL iff scale_shift_table is NULL.
   position_ids: (pos_rows, pos_cols) float32 with pos_rows == T + N and pos_cols == 3 ([ARTICLE] §二
   ValueError); text rows are normally zero, image rows (0, h, w). NULL = no RoPE (text fusion).
   encoder_attention_mask: (B, T) bytes, nonzero = valid text token; NULL = all valid. Padded text
   tokens are masked as keys only; image keys are always valid; every query row is computed. */
int k2_block_forward(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N,
                     const float* hidden_in, float* hidden_out, const float* temb,
                     const float* position_ids, int pos_rows, int pos_cols,
                     const uint8_t* encoder_attention_mask,
                     void* workspace, size_t workspace_bytes, void* stream);

/* k2_block_forward for callers that cannot allocate device memory (code under HIP graph capture,
   tight serving loops, harnesses that forbid allocation): the same computation and kernels, with no
   workspace argument. The library's scratch is a static device array of
   k2_block_forward_static_ws_max_bytes() bytes (128 MiB: the full-size block at 512^2, B = 1, needs
   123.3 MiB), held on each device the library runs on until the process ends; its address is looked
   up once per device on the first call made with that device current, and `stream` must belong to
   the current device. The call allocates nothing (keep the timing diagnostics below off: they create
   events). Every call on one device shares that device's scratch: calls that overlap on one device
   (concurrent streams, or host threads) race and must be serialised by the caller. Its contents
   need not be cleared between calls: every byte read is written first in the same call.
   Arguments as k2_block_forward. Returns K2_ERR_WORKSPACE when k2_block_workspace_bytes(cfg, B, T, N)
   exceeds the static size, K2_ERR_HIP if the scratch's address cannot be obtained, else as
   k2_block_forward. */
size_t k2_block_forward_static_ws_max_bytes(void);
int k2_block_forward_static_ws(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N,
                               const float* hidden_in, float* hidden_out, const float* temb,
                               const float* position_ids, int pos_rows, int pos_cols,
                               const uint8_t* encoder_attention_mask, void* stream);

/* Backward pass of one block ([ARTICLE] §四 data flow; §六: the model's test matrix trains it, with
   gradient checkpointing): the gradients of a loss with respect to the block's input, its
   modulation input and its weights, given the gradient grad_out of the block's output
   hidden_out. The forward is recomputed from hidden_in (checkpointing), then the chain rule runs
   through its steps in reverse. Matrix products use the block's dtype for their operands with
   float32 accumulation; gradients come out in float32.
   hidden_in, temb, position_ids, mask: exactly as given to k2_block_forward (attention over every
   allowed key; the block-causal variant has no backward here).
   grad_out: (B, L, hidden) float32 gradient of hidden_out.  grad_in: (B, L, hidden) float32,
   written (not accumulated); must not alias hidden_in or grad_out.
   grad_temb: (B, 6*hidden) float32 or NULL; NULL is required when the block has no
   scale_shift_table.  grads: one float32 device pointer per weight, same shapes as
   k2_block_weights' tensors, each written (not accumulated), or NULL to skip that gradient (the
   product it needs is then not run). Requires hidden <= 8192, text tokens T <= 16384 and
   (T + N) * num_heads * head_dim * element size <= 2^31 - 16 bytes (K2_ERR_SHAPE above it).
   Workspace: k2_block_backward_workspace_bytes(cfg, B, T, N). */
typedef struct {
  float* scale_shift_table; /* (6, hidden) */
  float* norm1_w;           /* (hidden) */
  float* norm2_w;           /* (hidden) */
  float* norm_q_w;          /* (head_dim) */
  float* norm_k_w;          /* (head_dim) */
  float* to_q;              /* (num_heads*head_dim, hidden) */
  float* to_k;              /* (num_kv_heads*head_dim, hidden) */
  float* to_v;              /* (num_kv_heads*head_dim, hidden) */
  float* to_gate;           /* (num_heads*head_dim, hidden) */
  float* to_out;            /* (hidden, num_heads*head_dim) */
  float* ff_gate;           /* (intermediate, hidden) */
  float* ff_up;             /* (intermediate, hidden) */
  float* ff_down;           /* (hidden, intermediate) */
} k2_block_grads;
size_t k2_block_backward_workspace_bytes(const k2_block_cfg* cfg, int B, int T, int N);
int k2_block_backward(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N,
                      const float* hidden_in, const float* temb, const float* position_ids, int pos_rows,
                      int pos_cols, const uint8_t* encoder_attention_mask, const float* grad_out, float* grad_in,
                      float* grad_temb, const k2_block_grads* grads, void* workspace, size_t workspace_bytes,
                      void* stream);

/* The same block with block-causal attention ([QWEN21] model page "QwenImage21Transformer2DModel":
   block-causal attention item; build_token_metadata): query i attends key j only if j <= i or both
   tokens lie in the same image block, on top of the key-padding mask. The sequence is causal while
   every image block stays bidirectional inside.
   image_ids: (T + N) int32 device array, 4-byte aligned, shared by all batch rows: -1 for tokens
   outside every image block, one id >= 0 per block. A block is a contiguous run of equal ids;
   two adjacent blocks must carry different ids (runs are what the kernels see).
   A query left with no key it may attend (text queries whose earlier text is all padding) gets a
   zero attention output. Workspace: k2_block_workspace_bytes. */
int k2_block_forward_block_causal(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N,
                                  const float* hidden_in, float* hidden_out, const float* temb,
                                  const float* position_ids, int pos_rows, int pos_cols,
                                  const uint8_t* encoder_attention_mask, const int32_t* image_ids,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Time path ([ARTICLE] §四.5 and §四 data flow): emb = [cos(1000 t f_k)] ++ [sin(1000 t f_k)],
 * f_k = 10000^(-k/half), half = timestep_embed_dim / 2; e = lin2(gelu_tanh(lin1(emb)));
 * temb = mod_proj(gelu_tanh(e)).
 * --------------------------------------------------------------------------------------------- */
typedef struct {
  int hidden;             /* 6144 */
  int timestep_embed_dim; /* 256; even, multiple of 64 */
  int dtype;
} k2_time_cfg;

typedef struct {
  const void* lin1_w; const float* lin1_b; /* (hidden, timestep_embed_dim), (hidden) */
  const void* lin2_w; const float* lin2_b; /* (hidden, hidden), (hidden) */
  const void* mod_w;  const float* mod_b;  /* (6*hidden, hidden), (6*hidden) */
} k2_time_weights;

size_t k2_timestep_modulation_workspace_bytes(const k2_time_cfg* cfg, int B);
/* timestep: (B,) float32 in [0, 1] (1 = noise). temb: (B, 6*hidden) float32 out.
   emb_out: (B, hidden) float32 out (time embedding before the GELU, used by the final layer) or NULL. */
int k2_timestep_modulation_forward(const k2_time_cfg* cfg, const k2_time_weights* w, int B,
                                   const float* timestep, float* temb, float* emb_out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Text fusion ([ARTICLE] §四.1): (B, T, num_layers, D) -> layerwise blocks over the layer axis of every
 * token (no mask, no RoPE) -> Linear(num_layers, 1, bias=False) over the layer axis -> refiner blocks
 * over the tokens with the key mask. Blocks are unmodulated pre-norm blocks (scale_shift_table NULL).
 * --------------------------------------------------------------------------------------------- */
typedef struct {
  k2_block_cfg block;       /* hidden 2560, 20/20 heads, head_dim 128, intermediate 6912 */
  int num_layers;           /* 12 */
  int num_layerwise_blocks; /* 2 */
  int num_refiner_blocks;   /* 2 */
} k2_text_cfg;

typedef struct {
  const k2_block_weights* layerwise; /* host array of num_layerwise_blocks */
  const float* compress_w;           /* (num_layers) float32 */
  const k2_block_weights* refiner;   /* host array of num_refiner_blocks */
} k2_text_weights;

void k2_text_cfg_default(k2_text_cfg* cfg);
size_t k2_text_fusion_workspace_bytes(const k2_text_cfg* cfg, int B, int T);
/* encoder_hidden_states: (B, T, num_layers, D) of dtype; mask (B, T) or NULL; out: (B, T, D) float32. */
int k2_text_fusion_forward(const k2_text_cfg* cfg, const k2_text_weights* w, int B, int T,
                           const void* encoder_hidden_states, const uint8_t* encoder_attention_mask,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Backbone ([API] forward; [ARTICLE] §四 data flow): time path; text fusion then txt_in; img_in;
 * concat [text, image]; RoPE table once; num_layers blocks; image rows only; final layer
 * ((scale, shift) = final_table + e; Linear to in_channels). Output: velocity (B, N, in_channels).
 * --------------------------------------------------------------------------------------------- */
typedef struct {
  k2_block_cfg block;
  k2_text_cfg text;
  int num_layers;         /* 28 */
  int in_channels;        /* 64 */
  int timestep_embed_dim; /* 256 */
} k2_model_cfg;

typedef struct {
  const void* img_in_w; const float* img_in_b; /* (hidden, in_channels), (hidden) */
  const void* txt_in_w; const float* txt_in_b; /* (hidden, text hidden), (hidden) */
  k2_time_weights time;
  k2_text_weights text;
  const k2_block_weights* blocks;              /* host array of num_layers */
  const float* final_table;                    /* (2, hidden): scale row, shift row */
  const float* final_norm_w;                   /* (hidden) or NULL */
  const void* final_w; const float* final_b;   /* (in_channels, hidden), (in_channels) */
} k2_model_weights;

void k2_model_cfg_default(k2_model_cfg* cfg);
size_t k2_backbone_workspace_bytes(const k2_model_cfg* cfg, int B, int T, int N);
/* hidden_states: (B, N, in_channels) of dtype (packed noisy latents);
   encoder_hidden_states: (B, T, num_text_layers, text hidden) of dtype; timestep (B,) float32;
   position_ids (pos_rows == T + N, pos_cols == 3) float32; mask (B, T) or NULL;
   out: (B, N, in_channels) float32 velocity. */
int k2_backbone_forward(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, int N,
                        const void* hidden_states, const void* encoder_hidden_states,
                        const float* timestep, const float* position_ids, int pos_rows, int pos_cols,
                        const uint8_t* encoder_attention_mask, float* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Text-path cache ([ARTICLE] §四 data flow, §五: the text stack enters only through text fusion and
   txt_in, which do not depend on the timestep or the latents, so a sampler computes them once per
   prompt). k2_text_embed writes txt_in(text_fusion(encoder_hidden_states)) to txt_h, (B, T, hidden)
   float32: exactly the rows [0, T) that k2_backbone_forward builds before its first block.
   k2_backbone_forward_cached is k2_backbone_forward with those rows taken from txt_h (B, T, hidden)
   float32 instead of being computed: given txt_h from k2_text_embed on the same inputs its output is
   bit-identical. The mask is still required for the blocks' attention; the text-fusion weights
   (w->text, w->txt_in_*) are not read. Workspaces: k2_text_embed_workspace_bytes and
   k2_backbone_cached_workspace_bytes (no text-fusion buffers). txt_h must be 16-byte aligned. */
size_t k2_text_embed_workspace_bytes(const k2_model_cfg* cfg, int B, int T);
int k2_text_embed(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T,
                  const void* encoder_hidden_states, const uint8_t* encoder_attention_mask, float* txt_h,
                  void* workspace, size_t workspace_bytes, void* stream);
size_t k2_backbone_cached_workspace_bytes(const k2_model_cfg* cfg, int B, int T, int N);
int k2_backbone_forward_cached(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, int N,
                               const void* hidden_states, const float* txt_h,
                               const float* timestep, const float* position_ids, int pos_rows, int pos_cols,
                               const uint8_t* encoder_attention_mask, float* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Sampler ([PIPELINE] Krea2Pipeline: FlowMatchEulerDiscreteScheduler with dynamic shifting and
 * Krea 2's shift parameters, is_distilled; __call__: sigmas, guidance_scale, num_inference_steps).
 *   sigma grid: linspace(1, 1/N, N) under the exponential time shift e^mu / (e^mu + 1/sigma - 1),
 *   mu on the line through (base_image_seq_len, base_shift) and (max_image_seq_len, max_shift) at
 *   the image token count (distilled checkpoint: mu = distilled_mu), then a terminal 0;
 *   velocity v = cond + g (cond - uncond), the unconditional pass skipped when g <= 0;
 *   Euler update x <- x + (sigma_next - sigma) v; the transformer runs at timestep t = sigma.
 * The latent state is float32 between steps.
 * --------------------------------------------------------------------------------------------- */
typedef struct {
  float base_shift;       /* 0.5 */
  float max_shift;        /* 1.15 */
  int base_image_seq_len; /* 256 */
  int max_image_seq_len;  /* 6400 */
  float distilled_mu;     /* 1.15 */
} k2_shift_cfg;
void k2_shift_cfg_default(k2_shift_cfg* cfg);

/* HOST function (no device work): the num_steps + 1 noise levels into the host array sigmas_out.
   cfg NULL = the defaults above. K2_ERR_SHAPE if num_steps < 1 or image_seq_len < 1. */
int k2_flow_sigmas(const k2_shift_cfg* cfg, int num_steps, int image_seq_len, int distilled, float* sigmas_out);

/* x_out = x + (sigma_next - sigma) * (v_cond + guidance (v_cond - v_uncond)) over n device floats
   (v_uncond unused, may be NULL, when guidance <= 0). x_out may alias x. One fused kernel. */
int k2_cfg_euler_update(const float* x, float* x_out, const float* v_cond, const float* v_uncond, size_t n,
                        float guidance, float sigma, float sigma_next, void* stream);

/* One sampler step of ONE image: the transformer (k2_backbone_forward semantics) on the batch
   (prompt, negative prompt) when guidance > 0, else on the prompt alone, at timestep sigma; then the
   guidance combine and Euler update into `latents`.
   latents: (1, N, in_channels) float32, read and updated in place.
   enc: (G, T, text layers, text hidden) in dtype, G = 2 (prompt, then negative prompt) when
   guidance > 0, else 1; mask: (G, T) or NULL; position_ids: (T + N, 3) float32.
   Workspace: k2_denoise_workspace_bytes(cfg, T, N, guidance > 0). */
size_t k2_denoise_workspace_bytes(const k2_model_cfg* cfg, int T, int N, int guided);
int k2_denoise_step(const k2_model_cfg* cfg, const k2_model_weights* w, int T, int N, float* latents, const void* enc,
                    const uint8_t* mask, const float* position_ids, int pos_rows, int pos_cols, float sigma,
                    float sigma_next, float guidance, void* workspace, size_t workspace_bytes, void* stream);
/* The same step with the text rows from k2_text_embed: txt_h (G, T, hidden) float32 for the G
   sequences above, computed once per prompt pair and reused at every step. Bit-identical to
   k2_denoise_step on the encoder states txt_h was computed from.
   Workspace: k2_denoise_cached_workspace_bytes(cfg, T, N, guidance > 0). */
size_t k2_denoise_cached_workspace_bytes(const k2_model_cfg* cfg, int T, int N, int guided);
int k2_denoise_step_cached(const k2_model_cfg* cfg, const k2_model_weights* w, int T, int N, float* latents,
                           const float* txt_h, const uint8_t* mask, const float* position_ids, int pos_rows,
                           int pos_cols, float sigma, float sigma_next, float guidance, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Diagnostics
 * --------------------------------------------------------------------------------------------- */
/* Message for the last non-OK status returned on this thread ("" if none). */
const char* k2_last_error(void);

/* Matrix-core rate probe (hardware calibration, not part of the method): `blocks` workgroups of four
   waves, each wave issuing iters x 4 independent bf16 32x32x16 matrix products on registers with no
   memory traffic, on `stream`: blocks * iters * 524288 FLOP in one launch. Time it with events on the
   stream to obtain the bf16 rate the part sustains (512 blocks = two waves per SIMD on 256 CUs).
   out: device float, 16-byte aligned (one value written, never meaningful). Returns K2_ERR_NULL,
   K2_ERR_SHAPE (iters < 1, blocks outside 1..65535), K2_ERR_ALIGN or K2_ERR_HIP. */
int k2_mfma_rate_probe(int iters, int blocks, float* out, void* stream);

/* Kernel timing with HIP events recorded on the launch stream around every kernel the library
   launches while enabled. This facility is the library's only process-wide state: the switch, the
   filter and the recorded events are shared by every thread (guarded by a mutex); timing one
   stream while another thread enables or resets it mixes their records. k2_profile_query synchronises on the recorded events and returns the
   total milliseconds and launch count of kernels whose name equals `kernel` (names: "modnorm",
   "gemm_qkvg", "attention", "gemm_out", "gemm_swiglu", "gemm_down", "rope", "modulation",
   "gemm_plain", "time_embed", "layer_compress", "convert", "fill", "cfg_euler", ...). Returns K2_OK or
   K2_ERR_HIP. */
void k2_profile_enable(int enable);
/* Record only kernels named `kernel` while enabled (NULL or "" = every kernel): two events per
   launch of that kernel alone, so that timing one kernel disturbs the rest as little as possible. */
void k2_profile_filter(const char* kernel);
void k2_profile_reset(void);
int k2_profile_query(const char* kernel, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif

#endif /* K2_H */
