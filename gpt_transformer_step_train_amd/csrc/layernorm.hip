// LayerNorm forward and backward (eps = 1e-5, biased variance), HBM-bound.
//
// The llm.c tour ("Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖)
// lists layernorm_forward among the forward layers and describes the backward as written by hand
// in reverse order; the formulas here are the standard ones:
//   y = (x - mu) * rstd * w + b,   rstd = 1/sqrt(var + eps)
//   dx = rstd * (g - mean(g) - xhat * mean(g * xhat)),  g = dy * w
//   dw = sum_rows dy * xhat,  db = sum_rows dy
// Forward: a row belongs to one wave64 or to one half-wave (whichever idles fewer lanes); backward:
// one wave64 per row, two rows per wave at a time. 16-byte loads, row statistics with DPP
// reductions (fp32).
// Weight/bias gradients: per-block column partials in registers, then a fixed-order sum over the
// blocks (here, or in a batched launch with the other column sums of the backward).
#include "common.h"
#include "kernels.h"

namespace g2 {

constexpr float LN_EPS = 1e-5f;

// Sum over the L lanes that share a row (L = 64: the whole wave, in wave_sum's order; L = 32:
// each half-wave, every lane receiving its own half's sum).
template <int L> __device__ __forceinline__ float row_sum(float v) {
  if constexpr (L == 64) {
    return wave_sum(v);
  } else {
    v = row16_sum(v);
    const float lo = readlane(v, 0) + readlane(v, 16), hi = readlane(v, 32) + readlane(v, 48);
    return (threadIdx.x & 32) ? hi : lo;
  }
}

// L lanes per row (64, or 32 when that leaves fewer lanes idle: a wave then takes two rows at
// once), NV 16-byte vectors per lane.
template <typename T, int NV, int L>
__global__ __launch_bounds__(256) void ln_fwd_kernel(int rows, int C, const T* __restrict__ x,
                                                     const T* __restrict__ w, const T* __restrict__ b,
                                                     T* __restrict__ y, float* __restrict__ mean,
                                                     float* __restrict__ rstd) {
  constexpr int VEC = Elt<T>::VEC;
  const int row = blockIdx.x * (256 / L) + (int)threadIdx.x / L;
  const int li = threadIdx.x & (L - 1);
  if (row >= rows) return;
  const int nvec = C / VEC;
  const T* xr = x + (size_t)row * C;
  // the row, the weight and the bias are all requested before the first reduction, as straight-line
  // loads (lanes past the row end read its last vector, unused; no bias: the weight again): a
  // guarded load makes the compiler wait for it at the branch join
  u32x4 xraw[NV], wraw[NV], braw[NV];
  const T* bsrc = b ? b : w;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vc = min(li + L * j, nvec - 1);
    xraw[j] = *reinterpret_cast<const u32x4*>(xr + vc * VEC);
    wraw[j] = *reinterpret_cast<const u32x4*>(w + vc * VEC);
    braw[j] = *reinterpret_cast<const u32x4*>(bsrc + vc * VEC);
  }
  V16<T> xv[NV];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = li + L * j;
    if (v < nvec) {
      xv[j].unpack(xraw[j]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s += xv[j].v[e];
    }
  }
  const float mu = row_sum<L>(s) / (float)C;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = li + L * j;
    if (v < nvec) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = xv[j].v[e] - mu;
        ss += d * d;
      }
    }
  }
  const float var = row_sum<L>(ss) / (float)C;
  const float rs = 1.0f / sqrtf(var + LN_EPS);
  T* yr = y + (size_t)row * C;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = li + L * j;
    if (v < nvec) {
      V16<T> wv, bv, o;
      wv.unpack(wraw[j]);
      if (b) bv.unpack(braw[j]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) o.v[e] = (xv[j].v[e] - mu) * rs * wv.v[e] + (b ? bv.v[e] : 0.f);
      o.store(yr + v * VEC);
    }
  }
  if (li == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

// Backward grid: at most LNB_BLOCKS blocks, each taking cdiv(rows, LNB_BLOCKS) consecutive rows, of
// 8 waves (4 when a lane holds more than two 16-byte vectors of a row: one wave per SIMD then
// keeps the wider rows' registers without spills).
constexpr int LNB_BLOCKS = 256;

// dx of every row (into dres: = or += dx), and per-block column partials of
//   dw = sum dy * xhat,  db = sum dy,  and (when dsum) the sum of the updated dres rows
// (the bias gradient of the linear layer whose output feeds this residual stream).
// Block = NW waves: wave wv takes rows r0 + wv, r0 + wv + NW, ...; the waves' column partials are
// added in wave order through LDS; partial layout [block][3][C].
template <typename T, int NV, int NW>
__global__ __launch_bounds__(64 * NW) void ln_bwd_kernel(int rows, int C, int rows_per_block,
                                                         const T* __restrict__ dy, const T* __restrict__ x,
                                                         const T* __restrict__ w, const float* __restrict__ mean,
                                                         const float* __restrict__ rstd, T* __restrict__ dres,
                                                         int add, int dsum, float* __restrict__ partial) {
  constexpr int VEC = Elt<T>::VEC;
  extern __shared__ float red[];  // [NW][C]
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nvec = C / VEC;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(rows, r0 + rows_per_block);

  float acc[3][NV][VEC];  // dw, db, dres sums
  // the weight as straight-line loads (clamped index, masked after), all in flight together
  float wf[NV][VEC];
  u32x4 wraw[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) wraw[j] = *reinterpret_cast<const u32x4*>(w + min(lane + 64 * j, nvec - 1) * VEC);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = lane + 64 * j;
    V16<T> t;
    t.unpack(wraw[j]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      wf[j][e] = v < nvec ? t.v[e] : 0.f;
      acc[0][j][e] = acc[1][j][e] = acc[2][j][e] = 0.f;
    }
  }
  // R rows per wave at a time, their loads issued together (at C = 768, bf16, two rows measured
  // faster than one, three, four, or one row with a register prefetch of the next); one row for
  // the wider rows, whose registers would spill
  constexpr int R = NV <= 2 ? 2 : 1;
  for (int row0 = r0 + wv; row0 < r1; row0 += R * NW) {
    u32x4 dyr[R][NV], xr[R][NV], drr[R][NV];
    float mu[R], rs[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r * NW;
      mu[r] = 0.f;
      rs[r] = 0.f;
      if (row < r1) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int v = lane + 64 * j;
          if (v < nvec) {
            const size_t o = (size_t)row * C + v * VEC;
            dyr[r][j] = *reinterpret_cast<const u32x4*>(dy + o);
            xr[r][j] = *reinterpret_cast<const u32x4*>(x + o);
            if (add) drr[r][j] = *reinterpret_cast<const u32x4*>(dres + o);
          }
        }
        mu[r] = mean[row];
        rs[r] = rstd[row];
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r * NW;
      if (row >= r1) break;
      float dyf[NV][VEC], xh[NV][VEC];
      float sg = 0.f, sgx = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if (lane + 64 * j < nvec) {
          V16<T> a, bx;
          a.unpack(dyr[r][j]);
          bx.unpack(xr[r][j]);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            dyf[j][e] = a.v[e];
            xh[j][e] = (bx.v[e] - mu[r]) * rs[r];
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
          if (add) o.unpack(drr[r][j]);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float dx = rs[r] * (dyf[j][e] * wf[j][e] - mg - xh[j][e] * mgx);
            o.v[e] = add ? o.v[e] + dx : dx;
            acc[2][j][e] += o.v[e];
          }
          o.store(dres + (size_t)row * C + v * VEC);
        }
      }
    }
  }
  // combine the waves' column partials in LDS, one quantity at a time, and write this block's
  // partial rows
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
    for (int c = threadIdx.x; c < C; c += 64 * NW) {
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < NW; ++k) sum += red[k * C + c];
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
  reduce_partials_block(partial + (size_t)blockIdx.y * C, nblocks, 3L * C, C, out, accumulate, blockIdx.x);
}

size_t layernorm_bwd_partial_floats(int rows, int C) { return (size_t)LNB_BLOCKS * 3 * C; }
// blocks of the backward (at most LNB_BLOCKS, each taking cdiv(rows, LNB_BLOCKS) rows)
static int ln_bwd_blocks(int rows) { return rows > 0 ? cdiv(rows, cdiv(rows, LNB_BLOCKS)) : 0; }

// Lanes per row of the forward: 32 when the row's 16-byte vectors leave an odd number of
// half-waves (then a full wave would idle half its lanes on the last vector) and that fits 8
// vectors per lane; else 64. Returns the vectors per lane in *nv. (The backward keeps 64: with
// two rows per wave it measured slower at C = 768, bf16.)
// elements per 16-byte vector
static int Elt16(DType dt) { return dt == DT_BF16 ? 8 : 4; }

static int ln_fwd_lanes(int nvec, int* nv) {
  const int h = cdiv(nvec, 32);
  if ((h & 1) && h <= 8) {
    *nv = h;
    return 32;
  }
  *nv = cdiv(nvec, 64);
  return 64;
}

template <typename T>
static hipError_t ln_fwd_t(int rows, int C, const void* x, const void* w, const void* b, void* y, float* mean,
                           float* rstd, hipStream_t s) {
  constexpr int VEC = Elt<T>::VEC;
  int nv;
  const int L = ln_fwd_lanes(C / VEC, &nv);
  dim3 grid(cdiv(rows, 256 / L));
  auto X = reinterpret_cast<const T*>(x);
  auto W = reinterpret_cast<const T*>(w);
  auto Bb = reinterpret_cast<const T*>(b);
  auto Y = reinterpret_cast<T*>(y);
#define LNF(n, l) ln_fwd_kernel<T, n, l><<<grid, 256, 0, s>>>(rows, C, X, W, Bb, Y, mean, rstd)
  if (L == 32) {
    if (nv == 1) LNF(1, 32);
    else if (nv == 3) LNF(3, 32);
    else if (nv == 5) LNF(5, 32);
    else LNF(7, 32);
  } else if (nv <= 1) LNF(1, 64);
  else if (nv <= 2) LNF(2, 64);
  else if (nv <= 4) LNF(4, 64);
  else if (nv <= 8) LNF(8, 64);
  else return hipErrorInvalidValue;
#undef LNF
  return hipGetLastError();
}

hipError_t launch_layernorm_fwd(DType dt, int rows, int C, const void* x, const void* w, const void* b, void* y,
                                float* mean, float* rstd, hipStream_t s) {
  if (C <= 0 || C % Elt16(dt)) return hipErrorInvalidValue;  // rows move as 16-byte vectors
  if (rows <= 0) return hipSuccess;
  return dt == DT_BF16 ? ln_fwd_t<bf16>(rows, C, x, w, b, y, mean, rstd, s)
                       : ln_fwd_t<float>(rows, C, x, w, b, y, mean, rstd, s);
}

template <typename T>
static hipError_t ln_bwd_t(int rows, int C, const void* dy, const void* x, const void* w, const float* mean,
                           const float* rstd, void* dres, int add, float* dw, float* db, float* dsum,
                           int accumulate, float* partial, hipStream_t s, bool finish) {
  constexpr int VEC = Elt<T>::VEC;
  const int nv = cdiv(C / VEC, 64);
  const int rpb = cdiv(rows, LNB_BLOCKS);
  const int nb = ln_bwd_blocks(rows);
  auto DY = reinterpret_cast<const T*>(dy);
  auto X = reinterpret_cast<const T*>(x);
  auto W = reinterpret_cast<const T*>(w);
  auto DR = reinterpret_cast<T*>(dres);
  const int ds = dsum != nullptr;
  if (nb > 0) {
#define LNB(n, nw)                                                                                      \
  ln_bwd_kernel<T, n, nw><<<nb, 64 * nw, (size_t)nw * C * sizeof(float), s>>>(rows, C, rpb, DY, X, W, mean, \
                                                                              rstd, DR, add, ds, partial)
    if (nv <= 1) LNB(1, 8);
    else if (nv <= 2) LNB(2, 8);
    else if (nv <= 4) LNB(4, 4);
    else if (nv <= 8) LNB(8, 4);
    else return hipErrorInvalidValue;
#undef LNB
  }
  if (finish) ln_bwd_finish<<<dim3(cdiv(C, 32), 3), RP_THREADS, 0, s>>>(partial, nb, C, dw, db, dsum, accumulate);
  return hipGetLastError();
}

hipError_t launch_layernorm_bwd(DType dt, int rows, int C, const void* dy, const void* x, const void* w,
                                const float* mean, const float* rstd, void* dres, int add, float* dw, float* db,
                                float* dsum, int accumulate, float* partial, size_t partial_floats, hipStream_t s,
                                ColsumDefer* defer) {
  const size_t pf = layernorm_bwd_partial_floats(rows, C);
  if (C <= 0 || C % Elt16(dt) || (size_t)4 * C * sizeof(float) > 64 * 1024) return hipErrorInvalidValue;
  // partials left for a batched finish when the caller offers room for them
  bool finish = true;
  if (defer) {
    defer->rows = 0;
    if (rows > 0 && pf <= defer->cap) {
      partial = defer->part;
      finish = false;
      defer->rows = ln_bwd_blocks(rows);
    }
  }
  if (finish && pf > partial_floats) return hipErrorInvalidValue;
  return dt == DT_BF16
             ? ln_bwd_t<bf16>(rows, C, dy, x, w, mean, rstd, dres, add, dw, db, dsum, accumulate, partial, s, finish)
             : ln_bwd_t<float>(rows, C, dy, x, w, mean, rstd, dres, add, dw, db, dsum, accumulate, partial, s, finish);
}

}  // namespace g2
