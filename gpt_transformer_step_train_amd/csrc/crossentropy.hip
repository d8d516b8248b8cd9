// Fused softmax cross-entropy + logit gradient, and the deterministic loss mean.
//
// The llm.c tour ("Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖)
// says the backward starts from the gradient of the loss w.r.t. the logits; the GPT-2
// reproduction post ("Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section PyTorch 对比)
// credits a fused classifier. Here one block per row reads the row once into registers, takes
// its max and sum of exponentials over the V real classes (fp32, wave64 DPP reductions), writes
// the row loss lse - logit[target], and overwrites the logits in place with
// (softmax - onehot(target)) * dloss; padded columns v >= V and ignored rows get 0.
// dloss = 1 / (number of valid targets * micro-steps per update) is read from device memory,
// computed by count_targets, so no host round trip is needed.
#include "common.h"
#include "kernels.h"

namespace g2 {

constexpr int CE_THREADS = 1024;
constexpr int CE_WAVES = CE_THREADS / 64;

// dloss_out = 1/(n_valid * accum) (0 when n_valid == 0); nvalid_out = n_valid; err |= 2 on bad target
__global__ __launch_bounds__(1024) void count_targets_kernel(const int32_t* __restrict__ targets, int rows, int V,
                                                             int accum, float* dloss_out, int* nvalid_out, int* err) {
  __shared__ float red[16];  // count_targets runs with 1024 threads
  float c = 0.f;
  bool bad = false;
  for (int i = threadIdx.x; i < rows; i += 1024) {
    const int t = targets[i];
    if (t >= 0 && t < V) c += 1.f;
    if (t >= V || t < -1) bad = true;  // -1 marks an ignored position; anything else outside [0, V) is an error
  }
  if (bad) atomicOr(err, 2);
  const float n = block_sum<16>(c, red);
  if (threadIdx.x == 0) {
    *nvalid_out = (int)n;
    *dloss_out = n > 0.f ? (float)(1.0 / ((double)n * accum)) : 0.f;
  }
}

// (m, s) pairs in log2 units: s = sum 2^(y - m) over the values seen; m = -inf while empty
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float a = m == -INFINITY ? 0.f : s * fast_exp2(m - M);
  const float b = m2 == -INFINITY ? 0.f : s2 * fast_exp2(m2 - M);
  m = M;
  s = a + b;
}

// One block of 1024 threads per row. The row is loaded once into registers (packed), the max and
// the sum of exponentials are accumulated in one online pass per thread (rescaled once per 8 or 4
// values), merged across the wave and the 16 waves in a fixed order, then the gradient is written.
// Blocks of 1024 threads with ~7 packed vectors each leave room for two rows per CU, so the
// loads of one row overlap the arithmetic and stores of another.
template <typename T, int NVT>
__global__ __launch_bounds__(CE_THREADS) void ce_kernel(int V, int ld, T* __restrict__ logits,
                                                        const int32_t* __restrict__ targets,
                                                        const float* __restrict__ dloss_p, float* __restrict__ losses) {
  constexpr int VEC = Elt<T>::VEC;
  __shared__ float red_m[CE_WAVES], red_s[CE_WAVES];
  __shared__ float xt_sh;
  const int row = blockIdx.x;
  T* x = logits + (size_t)row * ld;
  int tgt = targets ? targets[row] : -1;
  if (tgt >= V) tgt = -1;  // reported by count_targets
  const int nvec = ld / VEC;

  u32x4 raw[NVT];
#pragma unroll
  for (int j = 0; j < NVT; ++j) {
    const int v = threadIdx.x + j * CE_THREADS;
    raw[j] = v < nvec ? *reinterpret_cast<const u32x4*>(x + (size_t)v * VEC) : u32x4{0u, 0u, 0u, 0u};
  }
  // (after the row's loads are issued, so that wave 0 does not wait for this one first)
  if (threadIdx.x == 0) xt_sh = tgt >= 0 ? ld1(x, tgt) : 0.f;
  // values in log2 units; columns >= V are -inf
  auto unpack = [&](int j, float (&y)[VEC]) {
    V16<T> t;
    t.unpack(raw[j]);
    const int c0 = (threadIdx.x + j * CE_THREADS) * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[e] = c0 + e < V ? t.v[e] * LOG2E : -INFINITY;
  };
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int j = 0; j < NVT; ++j) {
    if (threadIdx.x + j * CE_THREADS < nvec) {
      float y[VEC];
      unpack(j, y);
      float vm = y[0];
#pragma unroll
      for (int e = 1; e < VEC; ++e) vm = fmaxf(vm, y[e]);
      if (vm != -INFINITY) {
        const float mn = fmaxf(m, vm);
        float acc = m == -INFINITY ? 0.f : s * fast_exp2(m - mn);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc += fast_exp2(y[e] - mn);
        m = mn;
        s = acc;
      }
    }
  }
  // merge over the wave: common max, then the rescaled sums
  const float wm = wave_max(m);
  float ws = wave_sum(m == -INFINITY ? 0.f : s * fast_exp2(m - wm));
  if ((threadIdx.x & 63) == 0) {
    red_m[threadIdx.x >> 6] = wm;
    red_s[threadIdx.x >> 6] = ws;
  }
  __syncthreads();  // also publishes xt_sh
  float M = red_m[0], S = red_s[0];
#pragma unroll
  for (int w = 1; w < CE_WAVES; ++w) lse_merge(M, S, red_m[w], red_s[w]);
  const float lse2 = M + __log2f(S);  // log2 units
  if (threadIdx.x == 0) losses[row] = tgt >= 0 ? lse2 / LOG2E - xt_sh : 0.f;
  if (!dloss_p) return;
  const float dl = tgt >= 0 ? *dloss_p : 0.f;
#pragma unroll
  for (int j = 0; j < NVT; ++j) {
    const int v = threadIdx.x + j * CE_THREADS;
    if (v < nvec) {
      float y[VEC];
      unpack(j, y);
      V16<T> o;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int col = v * VEC + e;
        o.v[e] = fast_exp2(y[e] - lse2) * dl - (col == tgt ? dl : 0.f);
      }
      o.store(x + (size_t)v * VEC);
    }
  }
}

template <typename T>
static hipError_t ce_t(int rows, int V, int ld, void* logits, const int32_t* targets, const float* dloss,
                       float* losses, hipStream_t s) {
  constexpr int VEC = Elt<T>::VEC;
  const int nvt = cdiv(ld / VEC, CE_THREADS);
  T* L = reinterpret_cast<T*>(logits);
#define CE_CASE(n) \
  if (nvt <= n) { \
    ce_kernel<T, n><<<rows, CE_THREADS, 0, s>>>(V, ld, L, targets, dloss, losses); \
    return hipGetLastError(); \
  }
  CE_CASE(1) CE_CASE(2) CE_CASE(4) CE_CASE(8) CE_CASE(13) CE_CASE(16) CE_CASE(25) CE_CASE(32)
#undef CE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_count_targets(const int32_t* targets, int rows, int V, int accum, float* dloss, int* nvalid,
                                int* err, hipStream_t s) {
  count_targets_kernel<<<1, 1024, 0, s>>>(targets, rows, V, accum, dloss, nvalid, err);
  return hipGetLastError();
}

hipError_t launch_cross_entropy(DType dt, int rows, int V, int ld, void* logits, const int32_t* targets,
                                const float* dloss, float* losses, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (V <= 0 || ld < V || ld % (dt == DT_BF16 ? 8 : 4)) return hipErrorInvalidValue;
  return dt == DT_BF16 ? ce_t<bf16>(rows, V, ld, logits, targets, dloss, losses, s)
                       : ce_t<float>(rows, V, ld, logits, targets, dloss, losses, s);
}

// mean = sum(losses) / n_valid in double, fixed order (one block); writes float and double
__global__ __launch_bounds__(1024) void loss_mean_kernel(const float* __restrict__ losses, int rows,
                                                         const int* __restrict__ nvalid, float* out) {
  __shared__ double sh[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < rows; i += 1024) s += (double)losses[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = *nvalid;
    out[0] = n > 0 ? (float)(sh[0] / n) : 0.f;
  }
}

hipError_t launch_loss_mean(const float* losses, int rows, const int* nvalid, float* out, hipStream_t s) {
  loss_mean_kernel<<<1, 1024, 0, s>>>(losses, rows, nvalid, out);
  return hipGetLastError();
}

}  // namespace g2
