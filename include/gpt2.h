/*
 * gpt2.h -- C ABI of the GPT-2 training-step library for AMD MI355X (gfx950).
 *
 * One training step of a decoder-only GPT-2 on one GPU: forward, backward, AdamW update.
 * The model and what each call computes follow the pages on llm.c:
 *   - layer order (encoder, LayerNorm, QKV matmul, attention, ..., classifier) and a hand-ordered
 *     backward starting from the logits: "Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现",
 *     section 代码解剖 (code walk-through);
 *   - attention softmax(Q K^T / sqrt(d_k)) V: the LLM primer page ("从Andrej Karpathy
 *     《深入了解ChatGPT之类的大语言模型》入门LLMs"), attention formula; causal for GPT-2;
 *   - a model built from scratch at a given depth, memory allocated once at start-up, bitwise
 *     determinism, gradient accumulation to a total batch, AdamW with weight decay on 2-D tensors,
 *     fp32 master weights with bf16 compute: "Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672",
 *     sections 训练 (training), 参数指南 (flags -d -c -e -y) and 代码 (code);
 *   - vocabulary padded (50257 -> 50304) for efficiency only: same post, section PyTorch 对比.
 *
 * Conventions
 *   - One model per process; the library is not thread-safe.
 *   - Device pointers are HIP device memory owned by the caller (e.g. torch tensors). The library
 *     never allocates device memory: everything it needs lives in the caller's workspace, carved
 *     once by gpt2_init. Host pointers are owned by the caller and only read/written inside a call.
 *   - All work is enqueued on cfg.stream (0 = the null stream).
 *   - Status codes: GPT2_OK (0) or a negative GPT2_E*; gpt2_last_error() describes the last one.
 *
 * Parameter layout (flat, float32 master, in this order; weights are [out, in], y = x W^T):
 *   wte [Vp, C], wpe [max_seq, C], then per layer l = 0..L-1:
 *   ln1w [C], ln1b [C], qkvw [3C, C], qkvb [3C], attprojw [C, C], attprojb [C], ln2w [C], ln2b [C],
 *   fcw [4C, C], fcb [4C], fcprojw [C, 4C], fcprojb [C]; then lnfw [C], lnfb [C].
 *   Linear biases are absent when linear_bias == 0, LayerNorm biases when ln_bias == 0.
 *   qkvw rows: Q (head h at rows h*hs..), then K, then V. wte is also the classifier (tied).
 */
#ifndef GPT2_H
#define GPT2_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPT2_OK 0
#define GPT2_EINVAL (-1)     /* bad configuration or argument */
#define GPT2_ENOMEM (-2)     /* workspace smaller than gpt2_workspace_bytes() */
#define GPT2_EHIP (-3)       /* HIP runtime error */
#define GPT2_ESTATE (-4)     /* call out of order (e.g. backward without a forward with targets) */
#define GPT2_ERANGE (-5)     /* token not in [0, V) or target not in [-1, V) */
#define GPT2_ENONFINITE (-6) /* gradient norm not finite: the update was skipped */
#define GPT2_EIO (-7)        /* checkpoint file could not be written or read, or does not match */

#define GPT2_FP32 0 /* fp32 everywhere */
#define GPT2_BF16 1 /* bf16 activations and matmul inputs, fp32 accumulation, fp32 master/grads/m/v */

typedef struct {
  int32_t n_layer, n_head, n_embd; /* L, H, C; C % H == 0, C % 8 == 0 */
  int32_t vocab, padded_vocab;     /* V (softmax width), Vp >= V rows of wte; Vp <= 65536 */
  int32_t max_seq;                 /* rows of wpe */
  int32_t batch, seq;              /* micro-batch B x T, T <= max_seq, B*T <= 32768 */
  int32_t precision;               /* GPT2_FP32 or GPT2_BF16 (bf16 needs C / H == 64) */
  int32_t linear_bias, ln_bias;    /* 1/1 for GPT-2; 0/1 for the BabyGPT toy */
  int32_t grad_accum;              /* micro-steps per update, >= 1 */
  float grad_clip;                 /* global-norm clip; <= 0 disables */
  int32_t recompute;               /* activation recompute ("Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672",
                                      section 参数指南, flag -r): 0 keeps every activation the
                                      backward reads; 1 keeps the MLP pre-activation only and
                                      recomputes GELU in the backward; 2 also recomputes the
                                      outputs of the two LayerNorms of each layer from their
                                      inputs and saved statistics. Same results up to the bf16
                                      rounding of the recomputed GELU input; less memory. */
  int32_t no_master;               /* 1: no fp32 master parameters (same post, flag -w 0); the
                                      bf16 parameters are updated in fp32 and rounded back
                                      stochastically (seeded SplitMix64 bits, see
                                      gpt2_adamw_step). GPT2_BF16 only. 0: fp32 master. */
  void* stream;                    /* hipStream_t */
  void* workspace;                 /* device memory, >= gpt2_workspace_bytes(cfg), 256-byte aligned */
  uint64_t workspace_bytes;
} gpt2_config;

/* Bytes of device workspace the configuration needs (0 if the configuration is invalid). */
uint64_t gpt2_workspace_bytes(const gpt2_config* cfg);

/* Validate cfg, carve the workspace, initialise the parameters, zero m and v.
 * Defined by "Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section 参数指南 (flag -e: a GPT-2 of a
 * given depth initialised from scratch; flags -b -t: the micro-batch B x T) and section 代码 (all GPU
 * memory is allocated once at start-up and stays fixed for the run). The pages give no init recipe;
 * the one below is the plain reading of a seeded normal(0, 0.02) init.
 * Init: every 2-D tensor in layout order draws N(0, 0.02^2) from one stream (SplitMix64 seeded
 * with `seed`, Box-Muller in double, rounded to fp32); biases 0; LayerNorm weights 1.
 * Synchronous. Replaces any previous model. */
int gpt2_init(const gpt2_config* cfg, uint64_t seed);

/* Forward pass on device int32 tokens [B*T] (row-major [B][T]) and targets [B*T].
 * Defined by "Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖 (the layer
 * order: encoder, L x [LayerNorm, QKV matmul, attention, projection, LayerNorm, MLP], final
 * LayerNorm, classifier, then the loss), with the attention softmax(Q K^T / sqrt(d_k)) V of the LLM
 * primer page, causal.
 * Errors: GPT2_ERANGE when a token is outside [0, V) or a target outside [-1, V) (the step is not
 * usable; call gpt2_forward again with valid ids).
 * targets == NULL: logits only (kept for gpt2_get_logits), returns NaN with status OK.
 * target < 0 is ignored; the loss is the mean of -log softmax(logits)[target] over valid targets
 * (0 when there is none). Synchronous: returns the loss, or NaN on error (see gpt2_last_status). */
float gpt2_forward(const int32_t* tokens, const int32_t* targets);

/* Backward pass of the last forward (which must have had targets), written in the reverse order
 * of the forward starting from the gradient at the logits ("Karpathy 的 llm.c：从零理解大模型训练的
 * C/CUDA 实现", section 代码解剖), with gradient accumulation over micro-steps to the total batch
 * ("Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section 参数指南, flag -d). The first backward after
 * gpt2_init or an update overwrites the gradients, later ones add (gradient accumulation; each
 * micro-step's loss is scaled by 1 / grad_accum). Asynchronous. */
int gpt2_backward(void);

/* AdamW update ("Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672": section 训练 allocates AdamW's m and
 * v and an fp32 master copy; section 参数指南, flag -c: decay on 2-D weights only; one kernel for all
 * parameters: "Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 性能对比).
 * t >= 1 (bias correction), decoupled weight decay `wd` on 2-D tensors only,
 * after scaling the gradients by min(1, grad_clip / ||g||) when grad_clip > 0.
 * In GPT2_BF16 mode also rewrites the bf16 parameter copy: rounded to nearest even from the fp32
 * master, or, with no_master, rounded stochastically: element i (flat layout index) of update t
 * takes r = the low 16 bits of output number (t << 32 | i) of SplitMix64 seeded with
 * gpt2_init's seed XOR 0xD1B54A32D192ED03, adds r to the fp32 result's magnitude bits and keeps
 * the upper 16 (rounds away from zero with probability discarded bits / 2^16). If ||g|| is not finite the update is
 * skipped on the device; gpt2_grad_norm() then returns a non-finite value. Asynchronous. */
int gpt2_adamw_step(float lr, float b1, float b2, float eps, float wd, int32_t t);

/* Discard the gradients accumulated since the last update without applying them (the update is
 * skipped, e.g. after a loss or gradient-norm spike); the next gpt2_backward overwrites them.
 * Host-side state only. */
int gpt2_skip_update(void);

/* One data-parallel rank's share of a sharded update, as ZeRO-1 runs it ("Karpathy 用 C 复现 GPT-2：
 * 单卡 24 小时 $672", section 参数指南, flag -z: the optimizer state split over the ranks, each rank
 * updating its own slice of the parameters): on one GPU, a contiguous slice [begin, end) of the
 * flat parameter vector (the layout of gpt2_get_params), whose ends may cut through tensors; weight
 * decay still follows the tensor each element belongs to. begin and end must be multiples of 4
 * with begin <= end <= gpt2_num_params(), else GPT2_EINVAL. Both calls are synchronous.
 *
 * gpt2_grad_sumsq_range: *sumsq = the sum of g^2 over the slice (double, the kernels and fixed
 * summation order of the full update's norm; over [0, N) it is exactly the squared norm the full
 * update uses). The sum of all ranks' values is the squared global norm a rank would get from an
 * all-reduce.
 *
 * gpt2_adamw_step_range: the update of gpt2_adamw_step restricted to the slice, with the clip
 * scale formed from global_sumsq (the squared global gradient norm) exactly as the full update
 * forms it from its own norm; writes the fp32 master, m, v and the bf16 copy of the slice (bit for
 * bit what gpt2_adamw_step writes there, given the same global_sumsq). The transposed bf16 weight
 * copies the backward reads are rewritten from the bf16 copy at the next gpt2_forward. finish != 0
 * ends the update as gpt2_adamw_step does (the next gpt2_backward overwrites the gradients); a
 * sharded update is one call per slice with finish set on the last. Needs a gpt2_backward since
 * the last update (GPT2_ESTATE). */
int gpt2_grad_sumsq_range(uint64_t begin, uint64_t end, double* sumsq);
int gpt2_adamw_step_range(float lr, float b1, float b2, float eps, float wd, int32_t t, uint64_t begin, uint64_t end,
                          double global_sumsq, int finish);

/* Checkpoint and bitwise resume ("Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section 参数指南:
 * -n checkpoints every n steps, -y 1 resumes, and determinism makes a resumed run continue
 * exactly). gpt2_save writes the fp32 master parameters, AdamW's m and v, the caller's update
 * count t and an opaque data cursor (e.g. the index of the next batch) to the host file `path`;
 * it must be called between updates (no gradients pending: GPT2_ESTATE otherwise). gpt2_load
 * reads such a file into the current model, whose architecture (n_layer, n_head, n_embd, vocab,
 * padded_vocab, max_seq, linear_bias, ln_bias) must match the file's (precision, batch and seq
 * may differ), refreshes the bf16 copies, discards pending gradients, and returns t and the
 * cursor, and takes over the file's gpt2_init seed (the stream the no_master stochastic rounding
 * draws from). Continuing from a loaded checkpoint reproduces the uninterrupted run bit for bit.
 * File: the 8 bytes "GPT2CKPT", uint32 version 1, the 8 int32 architecture fields above, uint64
 * N, int32 t, uint64 cursor, uint64 seed, then N floats each of parameters, m and v
 * (little-endian).
 * Synchronous. GPT2_EIO on a file error, a short file or a mismatch; the file's length is checked
 * before anything on the device is overwritten, so then the model is unchanged. Only a read or
 * runtime error after that check (e.g. the file shrinking underneath) leaves the model half
 * restored: it is then marked not ready and must be initialised again. */
int gpt2_save(const char* path, int32_t t, uint64_t cursor);
int gpt2_load(const char* path, int32_t* t, uint64_t* cursor);

/* Host-side training-loop helpers (no device work, callable before gpt2_init).
 * Learning rate of update `step` (1-based): linear warmup from 0 to lr_max over `warmup` updates
 * (lr_max * step / warmup), then a cosine decay from lr_max to final_frac * lr_max reached at
 * update `total`, constant after that: "Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section
 * 参数指南 (flags -k cosine, -l, -q, -u, -x) and the lr column printed in section 训练. The shape of
 * the decay between the two ends is half a cosine period. warmup >= 0, total > warmup. */
float gpt2_lr_schedule(int32_t step, float lr_max, int32_t warmup, int32_t total, float final_frac);

/* Spike detector for the update-skip of the same post (flags -sl / -sg, section 400B token 运行):
 * gpt2_outlier_update returns the z-score (x - mean) / std of x against the previous
 * GPT2_OUTLIER_WINDOW values it was given (population standard deviation), or NaN while fewer than
 * that many have been seen or the window has zero spread, and then adds x to the window. The caller
 * skips the update when the loss or gradient-norm z-score exceeds its threshold (5.0 on the page).
 * The state is caller-owned host memory; gpt2_outlier_reset empties it. */
#define GPT2_OUTLIER_WINDOW 128
typedef struct {
  double values[GPT2_OUTLIER_WINDOW];
  int32_t count; /* values seen, saturating at GPT2_OUTLIER_WINDOW */
  int32_t next;  /* slot the next value goes to */
} gpt2_outlier;
void gpt2_outlier_reset(gpt2_outlier* d);
double gpt2_outlier_update(gpt2_outlier* d, double x);

/* Diagnostics and parity (synchronous; host buffers owned by the caller). */
float gpt2_grad_norm(void);     /* pre-clip global L2 norm of the last update's gradients */
int gpt2_last_status(void);     /* status of the most recent call */
const char* gpt2_last_error(void);
uint64_t gpt2_num_params(void);
int gpt2_get_params(float* dst, uint64_t n);      /* fp32 master (no_master: the bf16 values), layout order */
int gpt2_set_params(const float* src, uint64_t n); /* also refreshes the bf16 copy (no_master: RNE) */
int gpt2_get_grads(float* dst, uint64_t n);
int gpt2_get_adam_state(float* m, float* v, uint64_t n);
/* Logits [B*T, V] as float (real vocabulary only) of the last gpt2_forward, which must have had
 * targets == NULL (with targets the logit buffer is overwritten by its gradient). */
int gpt2_get_logits(float* dst, uint64_t n);
/* Kernel timing (diagnostics). Each enabled class gets a pair of HIP events recorded on
 * cfg.stream around every launch of that class; gpt2_profile_read synchronises the stream and
 * returns, per class, the summed milliseconds and the number of launches since the last
 * enable/read. mask = 0 turns timing off. Classes (bit index): */
#define GPT2_K_ENCODER_FWD 0
#define GPT2_K_LAYERNORM_FWD 1
#define GPT2_K_GEMM_QKV 2           /* [BT,C] x [3C,C]^T + bias              */
#define GPT2_K_ATTENTION_FWD 3
#define GPT2_K_GEMM_ATTPROJ 4       /* [BT,C] x [C,C]^T + bias + residual    */
#define GPT2_K_GEMM_FC 5            /* [BT,C] x [4C,C]^T + bias, GELU        */
#define GPT2_K_GEMM_FCPROJ 6        /* [BT,4C] x [C,4C]^T + bias + residual  */
#define GPT2_K_GEMM_CLASSIFIER 7    /* [BT,C] x [Vp,C]^T                     */
#define GPT2_K_CROSS_ENTROPY 8
#define GPT2_K_GEMM_CLASSIFIER_DX 9
#define GPT2_K_GEMM_CLASSIFIER_DW 10
#define GPT2_K_LAYERNORM_BWD 11
#define GPT2_K_GEMM_FCPROJ_DX 12
#define GPT2_K_GEMM_FCPROJ_DW 13
#define GPT2_K_BIAS_GRAD 14           /* qkv bias gradient outside the batched finish (fp32 runs) */
#define GPT2_K_GEMM_FC_DX 15
#define GPT2_K_GEMM_FC_DW 16
#define GPT2_K_GEMM_ATTPROJ_DX 17
#define GPT2_K_GEMM_ATTPROJ_DW 18     /* no launches: taken with GPT2_K_GEMM_QKV_DW */
#define GPT2_K_ATTENTION_BWD 19      /* dK, dV                                */
#define GPT2_K_GEMM_QKV_DX 20
#define GPT2_K_GEMM_QKV_DW 21         /* qkv and attproj weight gradients, one launch */
#define GPT2_K_ENCODER_BWD 22
#define GPT2_K_GRAD_NORM 23
#define GPT2_K_ADAMW 24
#define GPT2_K_ATTENTION_BWD_Q 25    /* dQ (bf16: also D = rowsum(dO * O))    */
#define GPT2_K_ATTENTION_BWD_PRE 26  /* D = rowsum(dO * O) per query (fp32)   */
#define GPT2_K_WEIGHT_TRANSPOSE 27  /* bf16 weight matrices -> transposed copies */
#define GPT2_K_RECOMPUTE 28          /* activation recompute in the backward (recompute >= 1) */
#define GPT2_K_GRAD_FINISH 29        /* second stage of the backward's column sums, one batched launch */
#define GPT2_K_COUNT 30
int gpt2_profile_enable(uint32_t mask);
int gpt2_profile_read(float* ms, int32_t* launches, int32_t n);

void gpt2_free(void);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_H */
