// LayerNorm forward and backward (eps = 1e-5, biased variance), HBM-bound.
//
// The llm.c tour ("Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖)
// lists layernorm_forward among the forward layers and describes the backward as written by hand
// in reverse order; the formulas here are the standard ones:
//   y = (x - mu) * rstd * w + b,   rstd = 1/sqrt(var + eps)
//   dx = rstd * (g - mean(g) - xhat * mean(g * xhat)),  g = dy * w
//   dw = sum_rows dy * xhat,  db = sum_rows dy
// One wave64 owns a row; 16-byte loads; row statistics with DPP reductions (fp32).
// Weight/bias gradients: per-block column partials in registers, then a fixed-order sum.
#include "common.h"
#include "kernels.h"

namespace g2 {

constexpr float LN_EPS = 1e-5f;

template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_fwd_kernel(int rows, int C, const T* __restrict__ x,
                                                     const T* __restrict__ w, const T* __restrict__ b,
                                                     T* __restrict__ y, float* __restrict__ mean,
                                                     float* __restrict__ rstd) {
  constexpr int VEC = Elt<T>::VEC;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int nvec = C / VEC;
  const T* xr = x + (size_t)row * C;
  V16<T> xv[NV];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = lane + 64 * j;
    if (v < nvec) {
      xv[j].load(xr + v * VEC);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s += xv[j].v[e];
    }
  }
  const float mu = wave_sum(s) / (float)C;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = lane + 64 * j;
    if (v < nvec) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = xv[j].v[e] - mu;
        ss += d * d;
      }
    }
  }
  const float var = wave_sum(ss) / (float)C;
  const float rs = 1.0f / sqrtf(var + LN_EPS);
  T* yr = y + (size_t)row * C;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = lane + 64 * j;
    if (v < nvec) {
      V16<T> wv, bv, o;
      wv.load(w + v * VEC);
      if (b) bv.load(b + v * VEC);
#pragma unroll
      for (int e = 0; e < VEC; ++e) o.v[e] = (xv[j].v[e] - mu) * rs * wv.v[e] + (b ? bv.v[e] : 0.f);
      o.store(yr + v * VEC);
    }
  }
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

constexpr int LNB_BLOCKS = 1024;

template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_bwd_kernel(int rows, int C, int rows_per_block,
                                                     const T* __restrict__ dy, const T* __restrict__ x,
                                                     const T* __restrict__ w, const float* __restrict__ mean,
                                                     const float* __restrict__ rstd, T* __restrict__ dres,
                                                     int add, float* __restrict__ partial) {
  constexpr int VEC = Elt<T>::VEC;
  extern __shared__ float red[];  // [4][2*C]
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nvec = C / VEC;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(rows, r0 + rows_per_block);

  float dw_acc[NV][VEC], db_acc[NV][VEC];
  V16<T> wvec[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) dw_acc[j][e] = db_acc[j][e] = 0.f;
    const int v = lane + 64 * j;
    if (v < nvec) wvec[j].load(w + v * VEC);
  }

  for (int row = r0 + wv; row < r1; row += 4) {
    const float mu = mean[row], rs = rstd[row];
    V16<T> dyv[NV], xv[NV];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = lane + 64 * j;
      if (v < nvec) {
        dyv[j].load(dy + (size_t)row * C + v * VEC);
        xv[j].load(x + (size_t)row * C + v * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float xh = (xv[j].v[e] - mu) * rs;
          xv[j].v[e] = xh;  // keep xhat
          const float g = dyv[j].v[e] * wvec[j].v[e];
          sg += g;
          sgx += g * xh;
          dw_acc[j][e] += dyv[j].v[e] * xh;
          db_acc[j][e] += dyv[j].v[e];
        }
      }
    }
    const float mg = wave_sum(sg) / (float)C;
    const float mgx = wave_sum(sgx) / (float)C;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = lane + 64 * j;
      if (v < nvec) {
        T* dr = dres + (size_t)row * C + v * VEC;
        V16<T> o;
        if (add) o.load(dr);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float g = dyv[j].v[e] * wvec[j].v[e];
          const float dx = rs * (g - mg - xv[j].v[e] * mgx);
          o.v[e] = add ? o.v[e] + dx : dx;
        }
        o.store(dr);
      }
    }
  }
  // combine the 4 waves' column partials in LDS, then write this block's partial row
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = lane + 64 * j;
    if (v < nvec) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        red[wv * 2 * C + v * VEC + e] = dw_acc[j][e];
        red[wv * 2 * C + C + v * VEC + e] = db_acc[j][e];
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 2 * C; c += 256) {
    const float s = (red[c] + red[2 * C + c]) + (red[4 * C + c] + red[6 * C + c]);
    partial[(size_t)blockIdx.x * 2 * C + c] = s;
  }
}

// grid (cdiv(C, 32), 2): y = 0 -> dw, y = 1 -> db
__global__ __launch_bounds__(RP_THREADS) void ln_bwd_finish(const float* __restrict__ partial, int nblocks, int C,
                                                     float* __restrict__ dw, float* __restrict__ db,
                                                     int accumulate) {
  float* out = blockIdx.y == 0 ? dw : db;
  if (!out) return;
  reduce_partials_block(partial + (size_t)blockIdx.y * C, nblocks, 2L * C, C, out, accumulate);
}

size_t layernorm_bwd_partial_floats(int rows, int C) { return (size_t)LNB_BLOCKS * 2 * C; }

template <typename T>
static hipError_t ln_fwd_t(int rows, int C, const void* x, const void* w, const void* b, void* y, float* mean,
                           float* rstd, hipStream_t s) {
  constexpr int VEC = Elt<T>::VEC;
  const int nv = cdiv(C / VEC, 64);
  dim3 grid(cdiv(rows, 4));
  auto X = reinterpret_cast<const T*>(x);
  auto W = reinterpret_cast<const T*>(w);
  auto Bb = reinterpret_cast<const T*>(b);
  auto Y = reinterpret_cast<T*>(y);
  if (nv <= 1) ln_fwd_kernel<T, 1><<<grid, 256, 0, s>>>(rows, C, X, W, Bb, Y, mean, rstd);
  else if (nv <= 2) ln_fwd_kernel<T, 2><<<grid, 256, 0, s>>>(rows, C, X, W, Bb, Y, mean, rstd);
  else if (nv <= 4) ln_fwd_kernel<T, 4><<<grid, 256, 0, s>>>(rows, C, X, W, Bb, Y, mean, rstd);
  else if (nv <= 8) ln_fwd_kernel<T, 8><<<grid, 256, 0, s>>>(rows, C, X, W, Bb, Y, mean, rstd);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_layernorm_fwd(DType dt, int rows, int C, const void* x, const void* w, const void* b, void* y,
                                float* mean, float* rstd, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return dt == DT_BF16 ? ln_fwd_t<bf16>(rows, C, x, w, b, y, mean, rstd, s)
                       : ln_fwd_t<float>(rows, C, x, w, b, y, mean, rstd, s);
}

template <typename T>
static hipError_t ln_bwd_t(int rows, int C, const void* dy, const void* x, const void* w, const float* mean,
                           const float* rstd, void* dres, int add, float* dw, float* db, int accumulate,
                           float* partial, hipStream_t s) {
  constexpr int VEC = Elt<T>::VEC;
  const int nv = cdiv(C / VEC, 64);
  const int rpb = cdiv(rows, LNB_BLOCKS);
  const int nb = rows > 0 ? cdiv(rows, rpb) : 0;
  const size_t shm = (size_t)4 * 2 * C * sizeof(float);
  auto DY = reinterpret_cast<const T*>(dy);
  auto X = reinterpret_cast<const T*>(x);
  auto W = reinterpret_cast<const T*>(w);
  auto DR = reinterpret_cast<T*>(dres);
  if (nb > 0) {
    if (nv <= 1) ln_bwd_kernel<T, 1><<<nb, 256, shm, s>>>(rows, C, rpb, DY, X, W, mean, rstd, DR, add, partial);
    else if (nv <= 2) ln_bwd_kernel<T, 2><<<nb, 256, shm, s>>>(rows, C, rpb, DY, X, W, mean, rstd, DR, add, partial);
    else if (nv <= 4) ln_bwd_kernel<T, 4><<<nb, 256, shm, s>>>(rows, C, rpb, DY, X, W, mean, rstd, DR, add, partial);
    else if (nv <= 8) ln_bwd_kernel<T, 8><<<nb, 256, shm, s>>>(rows, C, rpb, DY, X, W, mean, rstd, DR, add, partial);
    else return hipErrorInvalidValue;
  }
  ln_bwd_finish<<<dim3(cdiv(C, 32), 2), RP_THREADS, 0, s>>>(partial, nb, C, dw, db, accumulate);
  return hipGetLastError();
}

hipError_t launch_layernorm_bwd(DType dt, int rows, int C, const void* dy, const void* x, const void* w,
                                const float* mean, const float* rstd, void* dres, int add, float* dw, float* db,
                                int accumulate, float* partial, size_t partial_floats, hipStream_t s) {
  if ((size_t)LNB_BLOCKS * 2 * C > partial_floats) return hipErrorInvalidValue;
  if ((size_t)4 * 2 * C * sizeof(float) > 64 * 1024) return hipErrorInvalidValue;
  return dt == DT_BF16 ? ln_bwd_t<bf16>(rows, C, dy, x, w, mean, rstd, dres, add, dw, db, accumulate, partial, s)
                       : ln_bwd_t<float>(rows, C, dy, x, w, mean, rstd, dres, add, dw, db, accumulate, partial, s);
}

}  // namespace g2
