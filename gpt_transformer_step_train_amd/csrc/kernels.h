// Internal launchers of the gfx950 kernels (host-callable; enqueue on `stream`).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g2 {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

// Column sums taken in two stages (per-block partial rows, then a fixed-order sum over them) may
// leave their second stage for later: a launcher given a ColsumDefer writes its partial rows into
// [part, part + cap) floats and sets `rows` to their number (0: it finished the sums itself, as
// without a ColsumDefer). The caller then lists FinishBlocks for one batched launch.
struct ColsumDefer {
  float* part;
  size_t cap;
  int rows;
};
// One block of the batched second stage:
//   out[32 chunk + c] (+)= sum_{y < ny} part[y ld + 32 chunk + c],  c < 32, 32 chunk + c < ncols
struct FinishBlock {
  const float* part;
  float* out;
  long ld;
  int ny, ncols, chunk, pad;
};
// All blocks' sums in one launch (accumulate: add to out instead of storing). Two blocks must not
// share an output column.
hipError_t launch_finish_batch(const FinishBlock* blocks, int nblocks, int accumulate, hipStream_t s);

// GEMM  C[M,N] = sum_k A(m,k) * B(n,k)
//   A(m,k) = A[m*lda + k] when a_kc (K-contiguous) else A[k*lda + m]
//   B(n,k) = B[n*ldb + k] when b_kc (K-contiguous) else B[k*ldb + n]
enum Epi {
  EPI_BIAS = 0,      // C(T) = acc + bias
  EPI_GELU = 1,      // C(T) = pre = acc + bias ; C2(T) = gelu(pre)
  EPI_RESID = 2,     // C(T) = aux + acc + bias        (residual add)
  EPI_GELU_BWD = 3,  // C(T) = acc * gelu'(aux)
  EPI_F32 = 4,       // C(f32) = acc  (or += acc when accumulate)
  EPI_GELU_GRAD = 5, // z = acc + bias ; C(T) = gelu'(z) ; C2(T) = gelu(z)
  EPI_MUL = 6,       // C(T) = acc * aux
};

struct GemmArgs {
  int M, N, K;
  const void* A;
  long lda;
  const void* B;
  long ldb;
  void* C;
  long ldc;
  const void* bias;  // [N] in the compute dtype, or null
  const void* aux;   // residual / pre-activation input (compute dtype)
  long ldaux;
  void* C2;          // second output (EPI_GELU), same ldc
  int accumulate;    // EPI_F32 only
  // non-EPI_F32 epilogues: when set, colsum[n] (+)= sum over m of the stored C[m][n] (the bias
  // gradient of a layer whose input gradient this product writes); partials go through scratch
  float* colsum;
  int colsum_accumulate;
  ColsumDefer* colsum_defer;  // when set, the column-sum partials may be left for a batched finish
};

// split-K: for EPI_F32 only; `scratch` must hold splits*M*N floats (nullptr => no split).
// Column sums (GemmArgs::colsum): `scratch` must hold (M/128 rounded up) * 2 * N floats.
hipError_t launch_gemm(DType dt, bool a_kc, bool b_kc, Epi epi, const GemmArgs& a, float* scratch,
                       size_t scratch_floats, hipStream_t s);
// Two EPI_F32 products with the same K (weight gradients of two layers) in one split-K launch;
// scratch as for launch_gemm, for the partials of both. Falls back to two launches when the
// shapes do not allow it (K differs, ldc != N, fp32).
hipError_t launch_gemm_f32_pair(DType dt, bool a_kc, bool b_kc, const GemmArgs& a0, const GemmArgs& a1,
                                float* scratch, size_t scratch_floats, hipStream_t s);
// Choose the number of K splits for an EPI_F32 GEMM (1 = none).
int gemm_splits(int M, int N, int K, size_t scratch_floats);

// out[n] (+)= sum_{y < ny} partial[y * N + n], summed in a fixed order
hipError_t launch_colsum_finish(const float* partial, int ny, int N, float* out, int accumulate, hipStream_t s);
// Upper bound of the fused column-sum partials of an M-row product: rows * N floats.
int gemm_colsum_rows_max(int M);
// db[n] (+)= sum_m dY[m*ld + n]; deterministic, two stages through `partial` (rows_split*N floats)
hipError_t launch_colsum(DType dt, const void* dY, long ld, int M, int N, float* db, int accumulate,
                         float* partial, size_t partial_floats, hipStream_t s);

// LayerNorm
hipError_t launch_layernorm_fwd(DType dt, int rows, int C, const void* x, const void* w, const void* b,
                                void* y, float* mean, float* rstd, hipStream_t s);
// dres[row] += dx (add = 1) or = dx (add = 0); dw/db (+)= column sums (two-stage, deterministic)
// dsum (may be null): column sums of the updated dres rows (= or += per accumulate)
hipError_t launch_layernorm_bwd(DType dt, int rows, int C, const void* dy, const void* x, const void* w,
                                const float* mean, const float* rstd, void* dres, int add, float* dw, float* db,
                                float* dsum, int accumulate, float* partial, size_t partial_floats, hipStream_t s,
                                ColsumDefer* defer = nullptr);
// partial floats of one backward; with a ColsumDefer the partial rows are [rows][3][C] (dw, db, dsum)
size_t layernorm_bwd_partial_floats(int rows, int C);

// Encoder
hipError_t launch_encoder_fwd(DType dt, int B, int T, int C, int V, const int32_t* tok, const void* wte,
                              const void* wpe, void* out, int* err, hipStream_t s);
// Sort (token, position) keys for the deterministic embedding-gradient scatter; needs BT <= 32768.
hipError_t launch_encoder_sort(int BT, int V, const int32_t* tok, uint32_t* keys, hipStream_t s);
hipError_t launch_encoder_bwd(DType dt, int B, int T, int maxT, int C, const uint32_t* sorted_keys, const void* dout,
                              float* dwte, float* dwpe, int accumulate_wpe, float* partial,
                              size_t partial_floats, hipStream_t s);
size_t encoder_bwd_partial_floats(int BT, int C);

// Attention (causal). qkv [B,T,3C], out [B,T,C], lse [B,H,T] (natural log).
hipError_t launch_attention_fwd(DType dt, int B, int T, int H, int hs, const void* qkv, void* out,
                                float* lse, hipStream_t s);
// dqkv [B,T,3C] is fully written. `dvec` holds B*H*T floats of scratch.
// parts: any of ATT_BWD_PRE (D = rowsum(dO * O)), ATT_BWD_KV (dK, dV), ATT_BWD_Q (dQ). fp32: PRE, then
// the other two in any order. bf16: the dQ kernel forms D itself and writes it to dvec, so PRE
// launches nothing and Q must run before KV (ATT_BWD_ALL does so).
constexpr int ATT_BWD_PRE = 1, ATT_BWD_KV = 2, ATT_BWD_Q = 4, ATT_BWD_ALL = 7;
// cs (bf16 only, may be null): the KV and Q kernels also write the column sums of the dqkv rows
// they store, one partial row of 3C floats per (sequence, 128-row tile):
// attention_bias_partial_rows(B, T) rows in all; launch_colsum_finish turns them into the qkv
// bias gradient.
hipError_t launch_attention_bwd(DType dt, int B, int T, int H, int hs, const void* qkv, const void* out,
                                const void* dout, const float* lse, void* dqkv, float* dvec, int parts,
                                hipStream_t s, float* cs = nullptr);
int attention_bias_partial_rows(int B, int T);

// Softmax cross-entropy over the first V columns of each row (row stride ld).
// targets < 0 are ignored. When dloss != nullptr the logits are overwritten by
// (softmax - onehot) * (*dloss) (0 in padded columns and ignored rows).
// losses[row] = lse - logit[target] (0 when ignored).
hipError_t launch_count_targets(const int32_t* targets, int rows, int V, int accum, float* dloss, int* nvalid,
                                int* err, hipStream_t s);
hipError_t launch_cross_entropy(DType dt, int rows, int V, int ld, void* logits, const int32_t* targets,
                                const float* dloss, float* losses, hipStream_t s);
hipError_t launch_loss_mean(const float* losses, int rows, const int* nvalid, float* out, hipStream_t s);

// Deterministic sum of squares: per-block partials (double), fixed grid.
hipError_t launch_sumsq_partial(const float* x, size_t n, double* partial, int nparts, hipStream_t s);

// Optimizer / init work items: contiguous runs of the flat parameter vector.
struct WorkItem {
  uint64_t off;      // first element
  uint32_t len;      // elements (<= ITEM_LEN)
  uint32_t kind;     // 0: 1-D, no decay, init const ; 1: 2-D, decay, init normal
  uint64_t normal0;  // index of the first element in the normal stream (kind 1)
  float init_val;    // constant init (kind 0)
  float pad_;
};
constexpr uint32_t ITEM_LEN = 8192;

struct AdamArgs {
  float lr, b1, b2, eps, wd;
  float bc1, bc2;    // 1/(1-b1^t), 1/(1-b2^t)
  float clip;        // <= 0: off
  // bf16 parameters only (no fp32 master): p is read from and written back to the bf16 copy,
  // rounded stochastically with the bits of sr_random(sr_seed, t, index)
  int no_master;
  int t;
  uint64_t sr_seed;
};
// Stochastic rounding fp32 -> bf16 of element `index` at update t: r = the low 16 bits of the
// SplitMix64 output number (t << 32 | index) of the stream seeded with `seed`; the magnitude is
// truncated to bf16 after adding r to it, so it rounds away from zero exactly when r plus the 16
// discarded bits reach 2^16, i.e. with probability (discarded bits) / 2^16 (unbiased).
// Inf and NaN round to nearest.
hipError_t launch_stochastic_round(const float* x, uint16_t* y, size_t n, uint64_t seed, int t, uint64_t index0,
                                   hipStream_t s);
// norm: partials -> norm2 (double) ; scale = clip / ||g|| when above the clip
hipError_t launch_grad_norm_finish(const double* partial, int nparts, double* norm2, float* scale, float clip,
                                   hipStream_t s);
hipError_t launch_adamw(const WorkItem* items, int nitems, float* p, const float* g, float* m, float* v,
                        uint16_t* shadow, const float* scale, const double* norm2, AdamArgs a,
                        hipStream_t s);
// AdamW over ADAM_TR x ADAM_TC tiles of the weight matrices that also have a transposed bf16 copy:
// the update of launch_adamw, plus the transposed copy written from the same registers through LDS.
constexpr int ADAM_TR = 64, ADAM_TC = 64;
struct AdamTile {
  uint64_t off;      // first element of the tile in the flat parameter vector
  uint64_t dst_off;  // element (c0, r0) of the transposed copy
  int32_t rows, cols;  // tile extent (<= ADAM_TR, ADAM_TC)
  int32_t ld, ldd;     // row pitch of the matrix, row pitch of its transposed copy
};
hipError_t launch_adamw_tiles(const AdamTile* tiles, int ntiles, float* p, const float* g, float* m, float* v,
                              uint16_t* shadow, uint16_t* shadow_t, const float* scale, const double* norm2,
                              AdamArgs a, hipStream_t s);
hipError_t launch_init_params(const WorkItem* items, int nitems, float* p, uint64_t seed, double std_,
                              hipStream_t s);
hipError_t launch_to_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t s);
// out[i] = gelu(in[i]) (tanh form) in the compute dtype; n a multiple of 8
hipError_t launch_gelu(DType dt, const void* in, void* out, size_t n, hipStream_t s);
// Transposed bf16 copy of a weight matrix: dst[dst_off + c * ldd + r] = src[src_off + r * cols + c],
// r < rows, c < cols. tile0: the first 64 x 64 tile of this matrix in the launch's tile numbering.
struct TransItem {
  uint64_t src_off, dst_off;
  int32_t rows, cols, ldd, tile0;
};
inline int trans_tiles(int rows, int cols) { return ((rows + 63) / 64) * ((cols + 63) / 64); }
hipError_t launch_transpose_bf16(const TransItem* items, int nitems, int ntiles, const uint16_t* src, uint16_t* dst,
                                 hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
// measurement utility: blocks x 8 waves x iters x 32 MFMAs (32x32x16 bf16) on the 64 KiB of operand
// bits at `operands`, read through LDS; out[block] receives a checksum
hipError_t launch_mfma_rate(const void* operands, float* out, int blocks, int iters, hipStream_t s);
hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s);

}  // namespace g2
