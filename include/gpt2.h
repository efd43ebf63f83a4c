/*
 * gpt2.h -- C ABI of one GPT-2 training step (forward, backward, global-norm
 * clip, AdamW) on one MI355X (gfx950), implemented with hand-written HIP
 * kernels.  No C++ or PyTorch types cross this boundary: plain pointers
 * (host or device, as stated per argument), sizes and status codes.
 *
 * What the step computes (pages cited by title and section):
 *  - "Let's reproduce GPT-2 (124M)" key takeaways, bullet "GPT-2
 *    Architecture Specifics": decoder-only stack, LayerNorm before attention
 *    and before the MLP, one more LayerNorm before the classifier, GELU.
 *  - "From Scratch: Building GPT-2 for Efficient Language Modeling", Key
 *    Features: token + position embeddings, multi-head self-attention,
 *    residual connections, GELU MLP.
 *  - "Let's reproduce GPT-2 (124M)" key takeaways, bullet "Weight Tying &
 *    Numerical Padding": the classifier weight is the token embedding; the
 *    embedding may have more rows than the vocabulary (50257 -> 50304).
 *  - chapter list of the same video: cross entropy loss; "model
 *    initialization: std 0.02, residual init".
 *  - key takeaways, bullets "Optimization Hyperparameters" and "Scaling
 *    Training with Gradient Accumulation & DDP": AdamW (0.9, 0.95, 1e-8),
 *    clip the global gradient norm at 1.0, weight decay 0.1 on 2-D tensors
 *    only, loss divided by the number of accumulation micro-steps.
 *
 * Conventions (readings where the pages are silent): tanh-GELU; LayerNorm
 * eps 1e-5 with the biased variance; attention scale 1/sqrt(head_dim),
 * query i attends to keys j <= i; weights stored [out, in] row-major; q, k,
 * v are the three contiguous thirds of the qkv projection; the softmax runs
 * over all padded_vocab logits (pad rows are ordinary rows that never occur
 * as ids or targets); clip coefficient min(1, clip / (norm + 1e-6));
 * decoupled weight decay lr * wd * p.
 *
 * Memory.  The caller owns all device memory: one arena of
 * gpt2_arena_bytes(cfg) bytes (256-byte aligned), the int32 token and
 * target buffers and the HIP stream.  The library never allocates or frees
 * device memory; it owns only the host-side context.  The arena must
 * outlive the context.  All work is enqueued on the given stream.
 *
 * Errors.  Every call returns a gpt2_status; nothing throws or aborts
 * across the ABI.  gpt2_last_error() gives a message.  After GPT2_E_HIP the
 * context is poisoned and every later call returns GPT2_E_STATE.
 */
#ifndef GPT2_MI_H
#define GPT2_MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT2_OK = 0,
  GPT2_E_ARG = -1,        /* NULL pointer, bad enum, bad config value */
  GPT2_E_SHAPE = -2,      /* B*T beyond the arena, T > max_seq, ... */
  GPT2_E_STATE = -3,      /* call out of order, or context poisoned */
  GPT2_E_HIP = -4,        /* a HIP runtime error (message has the HIP text) */
  GPT2_E_TOKEN = -5,      /* an id or target outside [0, vocab_size) */
  GPT2_E_NONFINITE = -6,  /* non-finite loss, or non-finite gradient norm */
  GPT2_E_ARENA = -7       /* arena too small or misaligned */
} gpt2_status;

typedef enum {
  GPT2_FP32 = 0,  /* fp32 storage and arithmetic throughout (GEMMs of 2^27
                     multiply-adds or more on the fp32 matrix cores) */
  GPT2_BF16 = 1,  /* bf16 GEMM/attention operands, fp32 accumulation,
                     fp32 residual stream, master weights and optimizer */
  GPT2_FP16 = 2   /* as GPT2_BF16 with fp16 (IEEE half) operands, plus dynamic
                     loss scaling ("Let's reproduce GPT-2 (124M)" chapter
                     "float16, gradient scalers, bfloat16"): see
                     gpt2_get_loss_scale */
} gpt2_compute;

typedef struct {
  int32_t n_layer;       /* L */
  int32_t n_head;        /* H, n_embd % n_head == 0 */
  int32_t n_embd;        /* C, multiple of 64, <= 1024 */
  int32_t block_size;    /* rows of the position embedding */
  int32_t vocab_size;    /* V: ids and targets must lie in [0, V) */
  int32_t padded_vocab;  /* Vp >= V, <= 65536: rows of wte = width of the logits */
  int32_t max_batch;     /* arena sizing: B * T <= max_batch * max_seq <= 32768,
                            and the logits buffer (max_batch * max_seq rows of
                            Vp rounded up to 64, 2 or 4 bytes each) < 4 GiB */
  int32_t max_seq;       /* T <= max_seq <= block_size */
  int32_t compute;       /* gpt2_compute */
  float ln_eps;          /* 1e-5 */
  float beta1, beta2;    /* 0.9, 0.95 */
  float adam_eps;        /* 1e-8 */
  float weight_decay;    /* 0.1, applied to 2-D tensors only */
} gpt2_config;

typedef struct gpt2_ctx gpt2_ctx;

/* Tensor kinds and dtypes reported by gpt2_tensor_info. */
enum { GPT2_K_PARAM = 0, GPT2_K_GRAD = 1, GPT2_K_ADAM_M = 2, GPT2_K_ADAM_V = 3,
       GPT2_K_SHADOW = 4, GPT2_K_ACT = 5, GPT2_K_LOGITS = 6, GPT2_K_SCALAR = 7 };
enum { GPT2_DT_F32 = 0, GPT2_DT_BF16 = 1, GPT2_DT_I32 = 2, GPT2_DT_F64 = 3, GPT2_DT_F16 = 4 };

typedef struct {
  char name[48];
  int32_t kind;      /* GPT2_K_* */
  int32_t dtype;     /* GPT2_DT_* */
  int32_t ndim;
  int32_t decay;     /* 1 for parameters that receive weight decay */
  int64_t shape[4];  /* activations: leading dim is the maximum B*T */
  uint64_t offset;   /* byte offset inside the arena */
  uint64_t bytes;
} gpt2_tensor_desc;

/* Fills *cfg with the GPT-2 124M shape and the optimizer constants above,
 * with the given batch limits (padded vocabulary 50304, bf16 compute). */
void gpt2_default_config(gpt2_config* cfg, int32_t max_batch, int32_t max_seq);

/* Bytes of device memory the caller must provide for cfg (0 if cfg is
 * invalid).  Host-only; makes no HIP call. */
size_t gpt2_arena_bytes(const gpt2_config* cfg);

/* Writes the initial parameters (float32, canonical order, concatenated)
 * into the host buffer out_params of gpt2_num_params(cfg) floats.
 * Initialization: tensor j in canonical order draws from its own SplitMix64
 * stream (Steele, Lea & Flood 2014) seeded with seed ^ (j << 32); pair q
 * uses outputs 2q, 2q+1 through Box-Muller; std 0.02 for wte, wpe, qkv.w and
 * fc.w, 0.02 / sqrt(2 n_layer) for proj.w and mproj.w; biases 0; LayerNorm
 * gain 1, bias 0.  Canonical order: wte[Vp,C], wpe[block_size,C], then per
 * layer ln1.w, ln1.b, qkv.w[3C,C], qkv.b, proj.w[C,C], proj.b, ln2.w, ln2.b,
 * fc.w[4C,C], fc.b, mproj.w[C,4C], mproj.b; then lnf.w, lnf.b.
 * Host-only; makes no HIP call. */
int64_t gpt2_num_params(const gpt2_config* cfg);
gpt2_status gpt2_init_host(const gpt2_config* cfg, uint64_t seed, float* out_params);

/* Creates a context on the current HIP device.  d_arena: device pointer to
 * arena_bytes >= gpt2_arena_bytes(cfg) bytes, 256-byte aligned; hip_stream:
 * a hipStream_t (NULL = default stream).  Initializes parameters (as
 * gpt2_init_host), zeroes gradients and AdamW state, writes the bf16 weight
 * copies.  Synchronizes the stream once. */
gpt2_status gpt2_create(const gpt2_config* cfg, uint64_t seed, void* d_arena, size_t arena_bytes,
                        void* hip_stream, gpt2_ctx** out);
void gpt2_destroy(gpt2_ctx* c);
const char* gpt2_last_error(const gpt2_ctx* c);

/* Forward pass on device int32 [B,T] ids.  With d_targets (device int32
 * [B,T]) it also computes the mean cross-entropy and overwrites the logits
 * in place by d(loss)/d(logits) (scaled by 1/(B*T)), arming backward.  With
 * d_targets NULL it stops at the logits (readable through the tensor
 * table).  h_loss (host, nullable): if given, the stream is synchronized
 * once and the loss written; GPT2_E_TOKEN / GPT2_E_NONFINITE are reported
 * then.  Out-of-range ids are clamped on the device before use. */
gpt2_status gpt2_forward(gpt2_ctx* c, const int32_t* d_tokens, const int32_t* d_targets,
                         int32_t B, int32_t T, float* h_loss);

/* Forward-only loss ("Let's reproduce GPT-2 (124M)" chapter "validation
 * data split, validation loss, sampling revive"): the same forward and
 * per-position cross-entropy as gpt2_forward with targets (d_targets is
 * required), but the logits are left in place (no gradient is written) and
 * backward is not armed; a backward armed by an earlier forward is
 * disarmed, since its activations are overwritten.  h_loss as in
 * gpt2_forward. */
gpt2_status gpt2_eval_loss(gpt2_ctx* c, const int32_t* d_tokens, const int32_t* d_targets,
                           int32_t B, int32_t T, float* h_loss);

/* Autoregressive sampling with a key/value cache (same video, chapters
 * "sampling init, prefix tokens" and "sampling loop").
 * d_tokens: device int32 [B, T_total] row-major; positions [0, T0) hold the
 * prefix on entry, positions [T0, T_total) receive the sampled tokens.
 * d_uniform: device float [B, T_total - T0], the uniform draw in [0, 1) for
 * each new token (the caller supplies the randomness; values outside are
 * clamped).  Token t is the smallest id v < vocab_size whose cumulative
 * softmax probability (ids in increasing order, over the vocab_size real
 * ids: padding ids are never sampled, temperature 1, no truncation) exceeds
 * the draw.  d_logprob (device float [B, T_total - T0], nullable) receives
 * each sampled token's log-probability under that softmax.
 * d_kv_cache: caller-owned device memory of gpt2_kv_cache_bytes(cfg) bytes
 * (per layer [max_batch][max_seq][2][C] keys and values in the activation
 * type); kv_bytes its size.  Needs 1 <= B <= max_batch and
 * 1 <= T0 < T_total <= max_seq.  The prefix runs through the ordinary
 * forward (its keys and values are then copied to the cache); each later
 * position runs one row per sequence through the blocks, appending its
 * keys and values and attending over the cache.  Overwrites the
 * activations (a pending backward is disarmed); does not touch gradients or
 * optimizer state.  Synchronizes the stream once at the end;
 * GPT2_E_TOKEN if a prefix id is outside [0, vocab_size). */
size_t gpt2_kv_cache_bytes(const gpt2_config* cfg);
gpt2_status gpt2_generate(gpt2_ctx* c, void* d_kv_cache, size_t kv_bytes, int32_t* d_tokens, int32_t B,
                          int32_t T0, int32_t T_total, const float* d_uniform, float* d_logprob);

/* Backward of grad_scale * loss (grad_scale 1, or 1/k for k accumulation
 * micro-steps).  The first backward after create / step / zero_grad writes
 * the gradients; later ones add to them. */
gpt2_status gpt2_backward(gpt2_ctx* c, float grad_scale);

/* Makes the next backward overwrite the gradients. */
gpt2_status gpt2_zero_grad(gpt2_ctx* c);

/* Global-norm clip then AdamW at learning rate lr.  The norm, the clip
 * coefficient and the bias corrections stay on the device; if the norm is
 * not finite the update is skipped on the device (parameters and state
 * unchanged, step count not advanced).  h_grad_norm (host, nullable): if
 * given, synchronizes once and returns the pre-clip norm; a non-finite norm
 * is then reported as GPT2_E_NONFINITE. */
gpt2_status gpt2_step(gpt2_ctx* c, float lr, float clip, float* h_grad_norm);

/* Dynamic loss scaling (GPT2_FP16 only).  The logits gradient is multiplied
 * by the loss scale S (device-resident, 65536 after gpt2_create), so the
 * fp16 gradients of backward carry S; gpt2_step divides it out of the norm
 * (the reported norm is the unscaled one) and out of the AdamW update.  If
 * the scaled gradients overflow (non-finite norm), the step is skipped on
 * the device (parameters, moments and step count unchanged), S is halved,
 * and gpt2_step returns GPT2_OK with *h_grad_norm = +inf.  After
 * growth_interval (2000 after create) consecutive finite steps S doubles.
 * get: synchronizes and reads S (1 for the other compute modes).
 * set: sets S and growth_interval and restarts the interval count; fp16
 * only (GPT2_E_ARG otherwise); S finite and > 0, growth_interval >= 1. */
gpt2_status gpt2_get_loss_scale(gpt2_ctx* c, float* scale);
gpt2_status gpt2_set_loss_scale(gpt2_ctx* c, float scale, int32_t growth_interval);

/* Learning rate at optimizer iteration it (0-based), "Let's reproduce GPT-2
 * (124M)" key takeaways, bullet "Optimization Hyperparameters" (linear
 * warm-up, then cosine decay to 10 % of the maximum) with the iteration
 * counts of "From Scratch: Building GPT-2 for Efficient Language Modeling",
 * Training Setup table (132 warm-up, 3400 iterations):
 *   it < warmup:                 max_lr * (it + 1) / warmup
 *   warmup <= it <= decay_end:   min_lr + (max_lr - min_lr) * (1 + cos(pi f)) / 2,
 *                                f = (it - warmup) / (decay_end - warmup)
 *   it > decay_end:              min_lr
 * so lr(warmup) = max_lr and lr(decay_end) = min_lr.  Host arithmetic in
 * double precision; makes no HIP call.  Returns NaN when it < 0,
 * warmup < 1, decay_end <= warmup, or not 0 <= min_lr <= max_lr. */
double gpt2_lr_at(int64_t it, double max_lr, double min_lr, int64_t warmup, int64_t decay_end);

/* One transformer block in isolation: y = block_layer(x) and dx, with the
 * block's parameter gradients written (overwritten) in the arena, for
 * upstream gradient dy.  d_x, d_dy, d_y, d_dx: device float32 [B,T,C]. */
gpt2_status gpt2_block_fwd_bwd(gpt2_ctx* c, int32_t layer, const float* d_x, const float* d_dy,
                               float* d_y, float* d_dx, int32_t B, int32_t T);

/* Checkpoint and resume.  A checkpoint is the fp32 parameters, both AdamW
 * moments (tensor kinds GPT2_K_PARAM, GPT2_K_ADAM_M, GPT2_K_ADAM_V, read and
 * written through the tensor table's views) and the optimizer step count.
 * After writing parameters into a context, gpt2_sync_weight_copies rewrites
 * the 16-bit weight copies that the GEMMs read from the
 * fp32 parameters; a context resumed this way continues bitwise like the
 * one that was saved.  The step count t (AdamW's bias corrections use t + 1
 * at the next step) lives on the device: get synchronizes the stream and
 * reads it, set (0 <= t <= 2^24) writes it and synchronizes. */
gpt2_status gpt2_sync_weight_copies(gpt2_ctx* c);
gpt2_status gpt2_get_step_count(gpt2_ctx* c, int64_t* t);
gpt2_status gpt2_set_step_count(gpt2_ctx* c, int64_t t);

/* Arena guards: the layout leaves 64 bytes of 0xA5 after every region
 * (tensor or workspace), written by gpt2_create.  gpt2_check_arena
 * synchronizes the stream and reads them back.  GPT2_OK if every guard is
 * intact; otherwise GPT2_E_ARENA, gpt2_last_error names the region before
 * the first damaged guard, and *n_bad (host, nullable) counts the damaged
 * guards.  A debugging aid for kernels that write past their region; not
 * needed for normal use. */
gpt2_status gpt2_check_arena(gpt2_ctx* c, int32_t* n_bad);

/* Introspection: zero-copy views into the arena. */
int32_t gpt2_num_tensors(const gpt2_ctx* c);
gpt2_status gpt2_tensor_info(const gpt2_ctx* c, int32_t i, gpt2_tensor_desc* out);

/* Kernel timing with HIP events on the library stream.  kernel_class
 * selects which launches are bracketed (GPT2_T_*); 0 turns timing off.
 * One bracket covers one library operation of that class (a GEMM with its
 * split-K reduction, a LayerNorm backward with its parameter-gradient
 * reduction, ...).  Classes: the classifier forward GEMM alone; every GEMM
 * (the classifier forward included); attention forward; attention backward;
 * LayerNorm forward; LayerNorm backward; cross-entropy; AdamW; gradient
 * norm; embedding forward and backward.  The bias gradients are formed
 * inside the weight-gradient GEMMs and time with the GEMM class.
 * gpt2_timing_read synchronizes, returns the summed milliseconds and the
 * bracket count since the last read, and resets them. */
enum { GPT2_T_NONE = 0, GPT2_T_LMHEAD_FWD = 1, GPT2_T_GEMM = 2, GPT2_T_ATTN_FWD = 3,
       GPT2_T_ATTN_BWD = 4, GPT2_T_LN_FWD = 5, GPT2_T_LN_BWD = 6, GPT2_T_XENT = 7,
       GPT2_T_ADAMW = 8, GPT2_T_NORM = 9, GPT2_T_EMBED = 10 };
gpt2_status gpt2_timing_enable(gpt2_ctx* c, int32_t kernel_class);
gpt2_status gpt2_timing_read(gpt2_ctx* c, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_MI_H */
