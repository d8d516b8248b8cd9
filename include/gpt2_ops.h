/*
 * gpt2_ops.h -- per-kernel entry points of the GPT-2 training-step library.
 *
 * Each call enqueues one step of the training step on raw device pointers (caller-owned HIP
 * device memory) so that it can be checked on its own against the CPU oracle. `dtype` is
 * GPT2_FP32 (float buffers) or GPT2_BF16 (bf16 buffers, 16-bit storage); fp32 statistics and
 * gradients of parameters are always float. `stream` is a hipStream_t. Every call returns
 * GPT2_OK or GPT2_EINVAL (unsupported shape or argument) / GPT2_EHIP (launch failure).
 * Row-major layouts throughout; leading dimensions must be multiples of 16 bytes (8 bf16 or 4
 * fp32 elements) and pointers 16-byte aligned (the GEMM ops check this and return GPT2_EINVAL).
 */
#ifndef GPT2_OPS_H
#define GPT2_OPS_H

#include <stdint.h>

#include "gpt2.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of gpt2op_gemm */
#define GPT2_EPI_BIAS 0     /* C = acc + bias                        (C in dtype)       */
#define GPT2_EPI_GELU 1     /* C = acc + bias ; C2 = gelu_tanh(C)    (forward MLP)      */
#define GPT2_EPI_RESID 2    /* C = aux + acc + bias                  (residual add)     */
#define GPT2_EPI_GELU_BWD 3 /* C = acc * gelu_tanh'(aux)             (MLP backward)     */
#define GPT2_EPI_F32 4      /* C(float) = acc, or += acc when accumulate (weight grads)  */
#define GPT2_EPI_GELU_GRAD 5 /* z = acc + bias ; C = gelu_tanh'(z) ; C2 = gelu_tanh(z)       */
#define GPT2_EPI_MUL 6      /* C = acc * aux                          (elementwise)      */

/* C[M,N] = sum_k A(m,k) B(n,k) then the epilogue.
 * A(m,k) = A[m*lda + k] if a_kcontig else A[k*lda + m]; B(n,k) = B[n*ldb + k] if b_kcontig
 * else B[k*ldb + n]. bias [N] (dtype) may be NULL. aux has leading dimension ldaux.
 * scratch (float, scratch_floats) enables deterministic split-K for GPT2_EPI_F32; may be NULL.
 * Linear layer forward is (a_kcontig=1, b_kcontig=1), input-gradient (1, 0), weight-gradient (0, 0).
 * Checked before any launch (else GPT2_EINVAL): M, N, K >= 0; A, B, C non-null when M, N > 0;
 * lda >= (a_kcontig ? K : M), ldb >= (b_kcontig ? K : N), ldc >= N; lda, ldb, ldaux multiples of 16
 * bytes of dtype, ldc of its output type (float for GPT2_EPI_F32); aux (and ldaux >= N) present for
 * RESID / GELU_BWD / MUL, C2 for GELU / GELU_GRAD; A, B, C, bias, aux, C2 16-byte aligned. */
int gpt2op_gemm(int dtype, int a_kcontig, int b_kcontig, int epilogue, int M, int N, int K, const void* A,
                int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, const void* bias, const void* aux,
                int64_t ldaux, void* C2, int accumulate, float* scratch, uint64_t scratch_floats, void* stream);
/* gpt2op_gemm with an epilogue other than GPT2_EPI_F32 that also sums the stored C over its rows:
 * colsum[n] = (or += when colsum_accumulate) sum_m C[m][n], the values as stored in dtype: the
 * bias gradient of the linear layer whose output gradient this product writes (the hand-ordered
 * backward of "Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖).
 * Deterministic: fixed-order partial sums through scratch, which must hold ceil(M/128) * 2 * N
 * floats (else GPT2_EINVAL). colsum (float [N]) is caller-owned device memory. */
int gpt2op_gemm_colsum(int dtype, int a_kcontig, int b_kcontig, int epilogue, int M, int N, int K, const void* A,
                       int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, const void* bias,
                       const void* aux, int64_t ldaux, void* C2, float* colsum, int colsum_accumulate,
                       float* scratch, uint64_t scratch_floats, void* stream);

/* Stochastic rounding fp32 -> bf16 as the no_master update does it (gpt2.h, gpt2_adamw_step):
 * y[i] = SR(x[i]) with the random bits of element index0 + i at update t of the stream seeded
 * with `seed` (the update uses gpt2_init's seed XOR 0xD1B54A32D192ED03). x, y device buffers of
 * n elements (y: bf16 bits). */
int gpt2op_stochastic_round(const float* x, uint16_t* y, uint64_t n, uint64_t seed, int32_t t, uint64_t index0,
                            void* stream);

/* LayerNorm over rows of width C (eps 1e-5, biased variance): y, mean[rows], rstd[rows]. b may be NULL.
 * C must be a positive multiple of 8 (bf16) or 4 (fp32), at most 4096 in bf16 and 2048 in fp32
 * (one row is held in one wave's registers: up to 8 16-byte vectors per lane), else GPT2_EINVAL
 * (both directions). */
int gpt2op_layernorm_forward(int dtype, int rows, int C, const void* x, const void* w, const void* b, void* y,
                             float* mean, float* rstd, void* stream);
/* dres += dx; dw, db (float [C]) = or += column sums (accumulate). db may be NULL.
 * dsum (float [C], may be NULL) = or += the column sums of the updated dres (the bias gradient of
 * the linear layer whose output is added to this residual stream).
 * partial: float scratch of gpt2op_layernorm_backward_scratch(rows, C) elements. */
int gpt2op_layernorm_backward(int dtype, int rows, int C, const void* dy, const void* x, const void* w,
                              const float* mean, const float* rstd, void* dres, float* dw, float* db, float* dsum,
                              int accumulate, float* partial, void* stream);
uint64_t gpt2op_layernorm_backward_scratch(int rows, int C);

/* Causal attention of qkv [B,T,3C] (Q|K|V, head h at columns h*hs of each third) into
 * out [B,T,C] and lse [B,H,T] (natural log of the softmax denominators). bf16 requires hs == 64;
 * fp32 supports hs in {4, 8, 16, 32, 64}. B, T >= 0 (0: nothing to do) and H >= 1, else
 * GPT2_EINVAL (all attention ops). */
int gpt2op_attention_forward(int dtype, int B, int T, int H, int hs, const void* qkv, void* out, float* lse,
                             void* stream);
/* dqkv [B,T,3C] (fully written) from qkv, out, dout, lse; dvec: float scratch [B*H*T]. */
int gpt2op_attention_backward(int dtype, int B, int T, int H, int hs, const void* qkv, const void* out,
                              const void* dout, const float* lse, void* dqkv, float* dvec, void* stream);
/* gpt2op_attention_backward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and results,
 * with the dvec scratch taken from a fixed array the library holds on each GPU (4 MiB, kept until
 * the process ends) instead of from the caller. Needs B*T*H <= GPT2_NOALLOC_ATTN_SCRATCH_FLOATS,
 * else GPT2_EINVAL; calls no allocator. Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from several threads) race and must be serialised
 * by the caller. Each call writes every entry it reads, so no clearing is needed between calls. */
#define GPT2_NOALLOC_ATTN_SCRATCH_FLOATS (1 << 20)
int gpt2op_attention_backward_noalloc(int dtype, int B, int T, int H, int hs, const void* qkv, const void* out,
                                      const void* dout, const float* lse, void* dqkv, void* stream);
/* gpt2op_attention_backward that also sums dqkv over its B*T rows: dbias[3C] = (or += when
 * accumulate) sum over rows of dqkv as stored, the gradient of the qkv bias (the hand-ordered
 * backward of "Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖).
 * bf16: the backward kernels leave per-tile column partials; fp32: a separate column-sum pass.
 * Deterministic. scratch (float) must hold B * ceil(T/128) * 3C floats (else GPT2_EINVAL). */
int gpt2op_attention_backward_colsum(int dtype, int B, int T, int H, int hs, const void* qkv, const void* out,
                                     const void* dout, const float* lse, void* dqkv, float* dvec, float* dbias,
                                     int accumulate, float* scratch, uint64_t scratch_floats, void* stream);

/* Softmax cross-entropy over the first V of ld columns of each row. losses[rows] (float).
 * When dloss != NULL (device float scalar), logits are overwritten by (softmax - onehot)*dloss,
 * with 0 in padded columns and on rows whose target is < 0. Requires 1 <= V <= ld and ld a
 * multiple of 8 (bf16) or 4 (fp32), else GPT2_EINVAL. */
int gpt2op_cross_entropy(int dtype, int rows, int V, int ld, void* logits, const int32_t* targets,
                         const float* dloss, float* losses, void* stream);

/* out[b,t,:] = wte[tok[b,t],:] + wpe[t,:]; err (device int) gets bit 0 set on an id outside [0, V). */
int gpt2op_encoder_forward(int dtype, int B, int T, int C, int V, const int32_t* tok, const void* wte,
                           const void* wpe, void* out, int* err, void* stream);
/* dwte[tok[p]] += dout[p] for every position p (deterministic order); dwpe[t] = or += sum_b dout[b,t]
 * (rows t >= T of the max_seq rows are set to 0 / left). keys: uint32 scratch [B*T];
 * partial: float scratch of gpt2op_encoder_backward_scratch(B*T, C) elements. Both directions
 * require C to be a positive multiple of 8 (bf16) or 4 (fp32), the backward T <= max_seq, else
 * GPT2_EINVAL; the backward checks its shapes before the sort writes `keys`. */
int gpt2op_encoder_backward(int dtype, int B, int T, int max_seq, int C, int V, const int32_t* tok,
                            const void* dout, float* dwte, float* dwpe, int accumulate_wpe, uint32_t* keys,
                            float* partial, void* stream);
uint64_t gpt2op_encoder_backward_scratch(int BT, int C);

/* Measurement utility, not part of the training step: dst[0, bytes) = src[0, bytes) with one
 * streaming kernel (16-byte loads and stores; bytes and both pointers 16-byte aligned, else
 * GPT2_EINVAL). Reads and writes exactly `bytes` each, so its HBM traffic counters give the scale
 * that converts the counters of any other kernel into bytes. */
int gpt2op_copy(void* dst, const void* src, uint64_t bytes, void* stream);

/* Measurement utility, not part of the training step: the matrix-core work of the GEMM main loop
 * without its global traffic. Each of `blocks` blocks (8 waves) copies the 65536 bytes at
 * `operands` (device, 16-byte aligned: two 256 x 64 bf16 operand tiles) into LDS, then every wave
 * runs `iters` rounds of 4 k-steps, each of 6 LDS fragment reads and 8 v_mfma_f32_32x32x16_bf16:
 * blocks * 8 * iters * 32 * 32768 FLOP in all, timed by the caller. out (device float [blocks])
 * receives one checksum per block. The rate depends on the operand bits: the matrix cores draw
 * more power on random bits than on zeros, and the clock follows the power. blocks in
 * [1, 1 << 20], iters >= 0, else GPT2_EINVAL. */
int gpt2op_mfma_rate(const void* operands, float* out, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_OPS_H */
