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
  // the row, the weight and the bias are all requested before the first reduction
  u32x4 xraw[NV], wraw[NV], braw[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = lane + 64 * j;
    if (v < nvec) {
      xraw[j] = *reinterpret_cast<const u32x4*>(xr + v * VEC);
      wraw[j] = *reinterpret_cast<const u32x4*>(w + v * VEC);
      if (b) braw[j] = *reinterpret_cast<const u32x4*>(b + v * VEC);
    }
  }
  V16<T> xv[NV];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = lane + 64 * j;
    if (v < nvec) {
      xv[j].unpack(xraw[j]);
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
      wv.unpack(wraw[j]);
      if (b) bv.unpack(braw[j]);
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

constexpr int LNB_BLOCKS = 512;

// Raw (packed) inputs of one row of the backward, held in registers so that the loads of the next
// row are in flight while this one is processed.
template <typename T, int NV> struct LnRow {
  u32x4 dy[NV], x[NV], dr[NV];
  float mu, rs;
};

// dx of every row (into dres: = or += dx), and per-block column partials of
//   dw = sum dy * xhat,  db = sum dy,  and (when dsum) the sum of the updated dres rows
// (the bias gradient of the linear layer whose output feeds this residual stream).
// Block = 4 waves; wave wv takes rows r0 + wv, r0 + wv + 4, ...; partial layout [block][3][C].
template <typename T, int NV, bool PF>
__global__ __launch_bounds__(256) void ln_bwd_kernel(int rows, int C, int rows_per_block,
                                                     const T* __restrict__ dy, const T* __restrict__ x,
                                                     const T* __restrict__ w, const float* __restrict__ mean,
                                                     const float* __restrict__ rstd, T* __restrict__ dres,
                                                     int add, int dsum, float* __restrict__ partial) {
  constexpr int VEC = Elt<T>::VEC;
  extern __shared__ float red[];  // [4][C]
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nvec = C / VEC;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(rows, r0 + rows_per_block);

  float acc[3][NV][VEC];  // dw, db, dres sums
  float wf[NV][VEC];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = lane + 64 * j;
    V16<T> t;
    if (v < nvec) t.load(w + v * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      wf[j][e] = v < nvec ? t.v[e] : 0.f;
      acc[0][j][e] = acc[1][j][e] = acc[2][j][e] = 0.f;
    }
  }
  auto load_row = [&](int row, LnRow<T, NV>& d) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = lane + 64 * j;
      if (v < nvec) {
        const size_t o = (size_t)row * C + v * VEC;
        d.dy[j] = *reinterpret_cast<const u32x4*>(dy + o);
        d.x[j] = *reinterpret_cast<const u32x4*>(x + o);
        if (add) d.dr[j] = *reinterpret_cast<const u32x4*>(dres + o);
      }
    }
    d.mu = mean[row];
    d.rs = rstd[row];
  };
  auto process = [&](int row, const LnRow<T, NV>& d) {
    float dyf[NV][VEC], xh[NV][VEC];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (lane + 64 * j < nvec) {
        V16<T> a, b;
        a.unpack(d.dy[j]);
        b.unpack(d.x[j]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          dyf[j][e] = a.v[e];
          xh[j][e] = (b.v[e] - d.mu) * d.rs;
          const float g = a.v[e] * wf[j][e];
          sg += g;
          sgx += g * xh[j][e];
          acc[0][j][e] += a.v[e] * xh[j][e];
          acc[1][j][e] += a.v[e];
        }
      }
    }
    const float mg = wave_sum(sg) / (float)C;
    const float mgx = wave_sum(sgx) / (float)C;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = lane + 64 * j;
      if (v < nvec) {
        V16<T> o;
        if (add) o.unpack(d.dr[j]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float dx = d.rs * (dyf[j][e] * wf[j][e] - mg - xh[j][e] * mgx);
          o.v[e] = add ? o.v[e] + dx : dx;
          acc[2][j][e] += o.v[e];
        }
        o.store(dres + (size_t)row * C + v * VEC);
      }
    }
  };
  int row = r0 + wv;
  if constexpr (PF) {
    LnRow<T, NV> cur, nxt;
    if (row < r1) load_row(row, cur);
    for (; row < r1; row += 4) {
      if (row + 4 < r1) load_row(row + 4, nxt);
      process(row, cur);
      cur = nxt;
    }
  } else {
    for (; row < r1; row += 4) {
      LnRow<T, NV> cur;
      load_row(row, cur);
      process(row, cur);
    }
  }
  // combine the 4 waves' column partials in LDS, one quantity at a time, and write this
  // block's partial rows
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    if (q == 2 && !dsum) break;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = lane + 64 * j;
      if (v < nvec) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) red[wv * C + v * VEC + e] = acc[q][j][e];
      }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < C; c += 256) {
      const float sum = (red[c] + red[C + c]) + (red[2 * C + c] + red[3 * C + c]);
      partial[((size_t)blockIdx.x * 3 + q) * C + c] = sum;
    }
    __syncthreads();
  }
}

// grid (cdiv(C, 32), 3): y = 0 -> dw, 1 -> db, 2 -> dres column sums
__global__ __launch_bounds__(RP_THREADS) void ln_bwd_finish(const float* __restrict__ partial, int nblocks, int C,
                                                     float* __restrict__ dw, float* __restrict__ db,
                                                     float* __restrict__ dsum, int accumulate) {
  float* out = blockIdx.y == 0 ? dw : blockIdx.y == 1 ? db : dsum;
  if (!out) return;
  reduce_partials_block(partial + (size_t)blockIdx.y * C, nblocks, 3L * C, C, out, accumulate);
}

size_t layernorm_bwd_partial_floats(int rows, int C) { return (size_t)LNB_BLOCKS * 3 * C; }

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
                           const float* rstd, void* dres, int add, float* dw, float* db, float* dsum,
                           int accumulate, float* partial, hipStream_t s) {
  constexpr int VEC = Elt<T>::VEC;
  const int nv = cdiv(C / VEC, 64);
  const int rpb = cdiv(rows, LNB_BLOCKS);
  const int nb = rows > 0 ? cdiv(rows, rpb) : 0;
  const size_t shm = (size_t)4 * C * sizeof(float);
  auto DY = reinterpret_cast<const T*>(dy);
  auto X = reinterpret_cast<const T*>(x);
  auto W = reinterpret_cast<const T*>(w);
  auto DR = reinterpret_cast<T*>(dres);
  const int ds = dsum != nullptr;
  if (nb > 0) {
#define LNB(n, pf) ln_bwd_kernel<T, n, pf><<<nb, 256, shm, s>>>(rows, C, rpb, DY, X, W, mean, rstd, DR, add, ds, partial)
    if (nv <= 1) LNB(1, true);
    else if (nv <= 2) LNB(2, true);
    else if (nv <= 4) LNB(4, false);
    else if (nv <= 8) LNB(8, false);
    else return hipErrorInvalidValue;
#undef LNB
  }
  ln_bwd_finish<<<dim3(cdiv(C, 32), 3), RP_THREADS, 0, s>>>(partial, nb, C, dw, db, dsum, accumulate);
  return hipGetLastError();
}

hipError_t launch_layernorm_bwd(DType dt, int rows, int C, const void* dy, const void* x, const void* w,
                                const float* mean, const float* rstd, void* dres, int add, float* dw, float* db,
                                float* dsum, int accumulate, float* partial, size_t partial_floats, hipStream_t s) {
  if ((size_t)LNB_BLOCKS * 3 * C > partial_floats) return hipErrorInvalidValue;
  if ((size_t)4 * C * sizeof(float) > 64 * 1024) return hipErrorInvalidValue;
  return dt == DT_BF16
             ? ln_bwd_t<bf16>(rows, C, dy, x, w, mean, rstd, dres, add, dw, db, dsum, accumulate, partial, s)
             : ln_bwd_t<float>(rows, C, dy, x, w, mean, rstd, dres, add, dw, db, dsum, accumulate, partial, s);
}

}  // namespace g2
