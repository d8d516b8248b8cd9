// Global gradient norm + clip scale, the single-launch AdamW update (which also refreshes the
// bf16 parameter shadow), and the seeded parameter initialisation.
//
// Pages: the llm.c tour ("Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 性能对比)
// contrasts one update kernel for all parameters with an optimizer that launches several; the
// GPT-2 reproduction post ("Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section 训练) shows
// AdamW state m, v and an fp32 master copy next to bf16 parameters, and (section 参数指南, -c)
// weight decay on 2-D tensors only.
//
// Without an fp32 master copy ("Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section 参数指南: -w 0
// keeps no fp32 parameters and relies on stochastic rounding) the update reads the bf16
// parameters, computes in fp32, and rounds the result back stochastically.
//
// AdamW, decoupled decay on the pre-update value:
//   g = s * grad;  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2
//   p = p - lr * ( (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps) + wd_i * p ),  wd_i = wd on 2-D tensors
// s = clip / ||g|| when clipping is on and ||g|| > clip, else 1. If ||g|| is not finite the
// update is skipped (p, m, v unchanged).
// The parameter vector is cut into work items (<= 8192 elements, never straddling a tensor), so one
// launch covers every tensor and each block knows its tensor's decay flag.
#include "common.h"
#include "kernels.h"

namespace g2 {

// ---------------------------------------------------------------- sum of squares (double)
__global__ __launch_bounds__(256) void sumsq_partial_kernel(const float* __restrict__ x, size_t n,
                                                            double* __restrict__ partial) {
  __shared__ double sh[256];
  double s = 0.0;
  const size_t n4 = n / 4;
  const size_t stride = (size_t)gridDim.x * 256;
  // four 16-byte loads in flight per thread (straight-line: an index past the end reads the last
  // vector, which is then dropped), so that enough bytes are requested to cover the memory latency
  constexpr int U = 4;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n4; i += U * stride) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = reinterpret_cast<const f32x4*>(x)[min(i + u * stride, n4 - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i + u * stride < n4) {
        const double a0 = v[u][0], a1 = v[u][1], a2 = v[u][2], a3 = v[u][3];
        s += a0 * a0 + a1 * a1 + a2 * a2 + a3 * a3;
      }
    }
  }
  for (size_t i = n4 * 4 + blockIdx.x * 256ull + threadIdx.x; i < n; i += stride) s += (double)x[i] * (double)x[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = sh[0];
}

hipError_t launch_sumsq_partial(const float* x, size_t n, double* partial, int nparts, hipStream_t s) {
  sumsq_partial_kernel<<<nparts, 256, 0, s>>>(x, n, partial);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void norm_finish_kernel(const double* __restrict__ partial, int nparts,
                                                          double* norm2, float* scale, float clip) {
  __shared__ double sh[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 256) s += partial[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double n2 = sh[0];
    const double nrm = sqrt(n2);
    *norm2 = n2;
    *scale = (clip > 0.f && nrm > (double)clip) ? (float)((double)clip / nrm) : 1.0f;
  }
}

hipError_t launch_grad_norm_finish(const double* partial, int nparts, double* norm2, float* scale, float clip,
                                   hipStream_t s) {
  norm_finish_kernel<<<1, 256, 0, s>>>(partial, nparts, norm2, scale, clip);
  return hipGetLastError();
}

// SplitMix64 (Steele, Lea & Flood 2014): output n of the stream seeded with s is
// mix(s + (n+1) * 0x9E3779B97F4A7C15). Uniform in (0,1): ((x >> 11) + 0.5) * 2^-53.
// Box-Muller (1958) on outputs (2p, 2p+1): normals 2p = r cos(2 pi u2), 2p+1 = r sin(2 pi u2),
// r = sqrt(-2 ln u1), in double; parameter = float(std * z).
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ double u01(uint64_t x) { return ((double)(x >> 11) + 0.5) * 0x1.0p-53; }

// stochastic rounding to bf16 (see kernels.h)
__device__ __forceinline__ uint16_t sr_bf16(float x, uint64_t seed, int t, uint64_t index) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u) return f2bf(x);
  const uint32_t r = (uint32_t)splitmix64(seed, ((uint64_t)(uint32_t)t << 32) | index) & 0xffffu;
  // adding r to the magnitude carries into the kept bits exactly when r + discarded >= 2^16
  return (uint16_t)((u + r) >> 16);
}

__global__ __launch_bounds__(256) void sr_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, size_t n,
                                                 uint64_t seed, int t, uint64_t index0) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    y[i] = sr_bf16(x[i], seed, t, index0 + i);
}
hipError_t launch_stochastic_round(const float* x, uint16_t* y, size_t n, uint64_t seed, int t, uint64_t index0,
                                   hipStream_t s) {
  if (!n) return hipSuccess;
  sr_kernel<<<(int)std::min<size_t>(8192, (n + 255) / 256), 256, 0, s>>>(x, y, n, seed, t, index0);
  return hipGetLastError();
}

// ---------------------------------------------------------------- AdamW
constexpr int ADAM_T = 256;

// NOMASTER: the parameters are the bf16 copy (p unused), read, updated in fp32 and rounded back
// stochastically; else p is the fp32 master and the bf16 copy (when present) is its RNE rounding.
template <bool NOMASTER>
__global__ __launch_bounds__(ADAM_T) void adamw_kernel(const WorkItem* __restrict__ items, float* __restrict__ p,
                                                       const float* __restrict__ g, float* __restrict__ m,
                                                       float* __restrict__ v, uint16_t* __restrict__ shadow,
                                                       const float* __restrict__ scale_p,
                                                       const double* __restrict__ norm2_p, AdamArgs a) {
  const double n2 = *norm2_p;
  if (!(n2 <= 1.0e300)) return;  // non-finite norm: skip the update (NaN fails the compare)
  const WorkItem it = items[blockIdx.x];
  const float sc = *scale_p;
  const float wd = it.kind == 1 ? a.wd : 0.f;
  const size_t base = it.off;
  auto upd = [&](float pp, float gg, float& mm, float& vv) {
    gg *= sc;
    mm = a.b1 * mm + (1.f - a.b1) * gg;
    vv = a.b2 * vv + (1.f - a.b2) * gg * gg;
    const float mh = mm * a.bc1;
    const float vh = vv * a.bc2;
    return pp - a.lr * (mh / (sqrtf(vh) + a.eps) + wd * pp);
  };
  // 4 consecutive elements from index i
  auto load_p = [&](size_t i) {
    if constexpr (NOMASTER) {
      const u32x2 r = *reinterpret_cast<const u32x2*>(shadow + i);
      return f32x4{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u), __uint_as_float(r[1] << 16),
                   __uint_as_float(r[1] & 0xffff0000u)};
    } else {
      return *reinterpret_cast<const f32x4*>(p + i);
    }
  };
  auto store_p = [&](size_t i, const f32x4& pv) {
    if constexpr (NOMASTER) {
      u32x2 r;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        r[h] = (uint32_t)sr_bf16(pv[2 * h], a.sr_seed, a.t, i + 2 * h) |
               ((uint32_t)sr_bf16(pv[2 * h + 1], a.sr_seed, a.t, i + 2 * h + 1) << 16);
      *reinterpret_cast<u32x2*>(shadow + i) = r;
    } else {
      *reinterpret_cast<f32x4*>(p + i) = pv;
      if (shadow) {
        const u32x2 sv = {pack2bf(pv[0], pv[1]), pack2bf(pv[2], pv[3])};
        *reinterpret_cast<u32x2*>(shadow + i) = sv;
      }
    }
  };
  // U vectors of 4 per thread and pass: all U x 4 loads are in flight before any arithmetic
  constexpr int U = 4;
  const int full = (int)it.len / (ADAM_T * 4 * U) * (ADAM_T * 4 * U);
  for (int j0 = 0; j0 < full; j0 += ADAM_T * 4 * U) {
    f32x4 pv[U], gv[U], mv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + j0 + (u * ADAM_T + threadIdx.x) * 4;
      pv[u] = load_p(i);
      gv[u] = *reinterpret_cast<const f32x4*>(g + i);
      mv[u] = *reinterpret_cast<const f32x4*>(m + i);
      vv[u] = *reinterpret_cast<const f32x4*>(v + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + j0 + (u * ADAM_T + threadIdx.x) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float mm = mv[u][e], vq = vv[u][e];
        pv[u][e] = upd(pv[u][e], gv[u][e], mm, vq);
        mv[u][e] = mm;
        vv[u][e] = vq;
      }
      store_p(i, pv[u]);
      *reinterpret_cast<f32x4*>(m + i) = mv[u];
      *reinterpret_cast<f32x4*>(v + i) = vv[u];
    }
  }
  for (int j = full + threadIdx.x * 4; j < (int)it.len; j += ADAM_T * 4) {
    const size_t i = base + j;
    if (j + 4 <= (int)it.len) {
      f32x4 pv = load_p(i);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(g + i);
      f32x4 mv = *reinterpret_cast<const f32x4*>(m + i);
      f32x4 vv = *reinterpret_cast<const f32x4*>(v + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float mm = mv[e], vq = vv[e];
        pv[e] = upd(pv[e], gv[e], mm, vq);
        mv[e] = mm;
        vv[e] = vq;
      }
      store_p(i, pv);
      *reinterpret_cast<f32x4*>(m + i) = mv;
      *reinterpret_cast<f32x4*>(v + i) = vv;
    } else {
      for (int e = 0; j + e < (int)it.len; ++e) {
        const size_t k = i + e;
        float mm = m[k], vv2 = v[k];
        const float p0 = NOMASTER ? bf2f(shadow[k]) : p[k];
        const float pp = upd(p0, g[k], mm, vv2);
        m[k] = mm;
        v[k] = vv2;
        if constexpr (NOMASTER) {
          shadow[k] = sr_bf16(pp, a.sr_seed, a.t, k);
        } else {
          p[k] = pp;
          if (shadow) shadow[k] = f2bf(pp);
        }
      }
    }
  }
}

hipError_t launch_adamw(const WorkItem* items, int nitems, float* p, const float* g, float* m, float* v,
                        uint16_t* shadow, const float* scale, const double* norm2, AdamArgs a, hipStream_t s) {
  if (nitems <= 0) return hipSuccess;
  if (a.no_master) {
    if (!shadow) return hipErrorInvalidValue;
    adamw_kernel<true><<<nitems, ADAM_T, 0, s>>>(items, p, g, m, v, shadow, scale, norm2, a);
  } else {
    adamw_kernel<false><<<nitems, ADAM_T, 0, s>>>(items, p, g, m, v, shadow, scale, norm2, a);
  }
  return hipGetLastError();
}

// ADAM_TR x ADAM_TC tiles of the transposed matrices (decay on: they are all 2-D). With TPR =
// ADAM_TC / 4 threads per row, thread t owns columns 4 (t % TPR) .. +3 of rows t / TPR + RPP k
// (RPP = 256 / TPR rows per pass), so every row segment is read and written as 16-byte vectors;
// the new bf16 values also go to LDS transposed, and come out as 16-byte rows of the transposed
// copy.
template <bool NOMASTER>
__global__ __launch_bounds__(256) void adamw_tile_kernel(const AdamTile* __restrict__ tiles, float* __restrict__ p,
                                                         const float* __restrict__ g, float* __restrict__ m,
                                                         float* __restrict__ v, uint16_t* __restrict__ shadow,
                                                         uint16_t* __restrict__ shadow_t,
                                                         const float* __restrict__ scale_p,
                                                         const double* __restrict__ norm2_p, AdamArgs a) {
  constexpr int TR = ADAM_TR, TC = ADAM_TC, TPR = TC / 4, RPP = 256 / TPR, NP = TR / RPP;
  static_assert(TC % 4 == 0 && 256 % TPR == 0 && TR % RPP == 0 && TR % 8 == 0, "AdamW tile shape");
  constexpr int P = TR + 8;  // LDS pitch (bf16 elements) of the transposed tile
  __shared__ __attribute__((aligned(16))) uint16_t tt[TC * P];
  const double n2 = *norm2_p;
  if (!(n2 <= 1.0e300)) return;
  const AdamTile T = tiles[blockIdx.x];
  const float sc = *scale_p;
  const int cq = threadIdx.x % TPR, rg = threadIdx.x / TPR;
  const bool full = T.rows == TR && T.cols == TC;
  auto upd = [&](float pp, float gg, float& mm, float& vv) {
    gg *= sc;
    mm = a.b1 * mm + (1.f - a.b1) * gg;
    vv = a.b2 * vv + (1.f - a.b2) * gg * gg;
    const float mh = mm * a.bc1;
    const float vh = vv * a.bc2;
    return pp - a.lr * (mh / (sqrtf(vh) + a.eps) + a.wd * pp);
  };
  if (full) {
    f32x4 pv[NP], gv[NP], mv[NP], vv[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const size_t i = T.off + (size_t)(rg + RPP * k) * T.ld + 4 * cq;
      if constexpr (NOMASTER) {
        const u32x2 r = *reinterpret_cast<const u32x2*>(shadow + i);
        pv[k] = f32x4{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u),
                      __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xffff0000u)};
      } else {
        pv[k] = *reinterpret_cast<const f32x4*>(p + i);
      }
      gv[k] = *reinterpret_cast<const f32x4*>(g + i);
      mv[k] = *reinterpret_cast<const f32x4*>(m + i);
      vv[k] = *reinterpret_cast<const f32x4*>(v + i);
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int r = rg + RPP * k;
      const size_t i = T.off + (size_t)r * T.ld + 4 * cq;
      uint16_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float mm = mv[k][e], vq = vv[k][e];
        pv[k][e] = upd(pv[k][e], gv[k][e], mm, vq);
        mv[k][e] = mm;
        vv[k][e] = vq;
        b[e] = NOMASTER ? sr_bf16(pv[k][e], a.sr_seed, a.t, i + e) : f2bf(pv[k][e]);
      }
      if constexpr (!NOMASTER) *reinterpret_cast<f32x4*>(p + i) = pv[k];
      *reinterpret_cast<f32x4*>(m + i) = mv[k];
      *reinterpret_cast<f32x4*>(v + i) = vv[k];
      const u32x2 sv = {(uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16)};
      *reinterpret_cast<u32x2*>(shadow + i) = sv;
#pragma unroll
      for (int e = 0; e < 4; ++e) tt[(4 * cq + e) * P + r] = b[e];
    }
  } else {
    for (int k = 0; k < NP; ++k) {
      const int r = rg + RPP * k;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 4 * cq + e;
        if (r >= T.rows || c >= T.cols) continue;
        const size_t i = T.off + (size_t)r * T.ld + c;
        float mm = m[i], vq = v[i];
        const float p0 = NOMASTER ? bf2f(shadow[i]) : p[i];
        const float pn = upd(p0, g[i], mm, vq);
        m[i] = mm;
        v[i] = vq;
        const uint16_t b = NOMASTER ? sr_bf16(pn, a.sr_seed, a.t, i) : f2bf(pn);
        if constexpr (!NOMASTER) p[i] = pn;
        shadow[i] = b;
        tt[c * P + r] = b;
      }
    }
  }
  __syncthreads();
  // row c of the transposed copy: rows r0 .. r0 + rows - 1 of the tile, 8 at a time
  for (int w = threadIdx.x; w < TC * (TR / 8); w += 256) {
    const int c = w / (TR / 8), r = (w % (TR / 8)) * 8;
    if (c >= T.cols || r >= T.rows) continue;
    uint16_t* out = shadow_t + T.dst_off + (size_t)c * T.ldd + r;
    if (full) {
      *reinterpret_cast<u32x4*>(out) = *reinterpret_cast<const u32x4*>(tt + c * P + r);
    } else {
      for (int e = 0; e < 8 && r + e < T.rows; ++e) out[e] = tt[c * P + r + e];
    }
  }
}

hipError_t launch_adamw_tiles(const AdamTile* tiles, int ntiles, float* p, const float* g, float* m, float* v,
                              uint16_t* shadow, uint16_t* shadow_t, const float* scale, const double* norm2,
                              AdamArgs a, hipStream_t s) {
  if (ntiles <= 0) return hipSuccess;
  if (a.no_master)
    adamw_tile_kernel<true><<<ntiles, 256, 0, s>>>(tiles, p, g, m, v, shadow, shadow_t, scale, norm2, a);
  else
    adamw_tile_kernel<false><<<ntiles, 256, 0, s>>>(tiles, p, g, m, v, shadow, shadow_t, scale, norm2, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- init

__global__ __launch_bounds__(256) void init_kernel(const WorkItem* __restrict__ items, float* __restrict__ p,
                                                   uint64_t seed, double std_) {
  const WorkItem it = items[blockIdx.x];
  for (int j = threadIdx.x; j < (int)it.len; j += 256) {
    float val;
    if (it.kind == 1) {
      const uint64_t idx = it.normal0 + j;
      const uint64_t pr = idx >> 1;
      const double u1 = u01(splitmix64(seed, 2 * pr));
      const double u2 = u01(splitmix64(seed, 2 * pr + 1));
      const double r = sqrt(-2.0 * log(u1));
      const double ang = (2.0 * M_PI) * u2;
      const double z = (idx & 1) ? r * sin(ang) : r * cos(ang);
      val = (float)(std_ * z);
    } else {
      val = it.init_val;
    }
    p[it.off + j] = val;
  }
}

hipError_t launch_init_params(const WorkItem* items, int nitems, float* p, uint64_t seed, double std_,
                              hipStream_t s) {
  if (nitems <= 0) return hipSuccess;
  init_kernel<<<nitems, 256, 0, s>>>(items, p, seed, std_);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                      size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = f2bf(src[i]);
}
hipError_t launch_to_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  to_bf16_kernel<<<(int)std::min<size_t>(8192, (n + 255) / 256), 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

// One block per 64 x 64 tile: 16-byte row vectors of the source into LDS, 16-byte row vectors of
// the copy out of it (each gathered from 8 LDS rows).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const TransItem* __restrict__ items, int nitems,
                                                             const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst) {
  constexpr int P = 72;  // LDS row pitch (elements): 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * P];
  int i = nitems - 1;
  while (i > 0 && items[i].tile0 > (int)blockIdx.x) --i;
  const TransItem it = items[i];
  const int t = (int)blockIdx.x - it.tile0;
  const int tcols = (it.cols + 63) / 64;
  const int r0 = (t / tcols) * 64, c0 = (t % tcols) * 64;
  const uint16_t* s = src + it.src_off;
  uint16_t* d = dst + it.dst_off;
  const bool svec = ((it.src_off | (uint64_t)it.cols) & 7) == 0;
  const bool dvec = ((it.dst_off | (uint64_t)it.ldd) & 7) == 0;
  for (int v = threadIdx.x; v < 512; v += 256) {
    const int r = v >> 3, c = (v & 7) * 8;
    const int gr = r0 + r, gc = c0 + c;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (gr < it.rows) {
      const uint16_t* row = s + (size_t)gr * it.cols;
      if (svec && gc + 8 <= it.cols) {
        x = *reinterpret_cast<const u32x4*>(row + gc);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = gc + k < it.cols ? row[gc + k] : (uint16_t)0;
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = (uint32_t)e[2 * k] | ((uint32_t)e[2 * k + 1] << 16);
      }
    }
    *reinterpret_cast<u32x4*>(tile + r * P + c) = x;
  }
  __syncthreads();
  for (int v = threadIdx.x; v < 512; v += 256) {
    const int c = v >> 3, r = (v & 7) * 8;  // row c of the copy, source rows r .. r + 7
    const int gc = c0 + c, gr = r0 + r;
    if (gc >= it.cols || gr >= it.rows) continue;
    uint16_t e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = tile[(r + k) * P + c];
    uint16_t* out = d + (size_t)gc * it.ldd + gr;
    if (dvec && gr + 8 <= it.rows) {
      u32x4 x;
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = (uint32_t)e[2 * k] | ((uint32_t)e[2 * k + 1] << 16);
      *reinterpret_cast<u32x4*>(out) = x;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (gr + k < it.rows) out[k] = e[k];
    }
  }
}
hipError_t launch_transpose_bf16(const TransItem* items, int nitems, int ntiles, const uint16_t* src, uint16_t* dst,
                                 hipStream_t s) {
  if (nitems <= 0 || ntiles <= 0) return hipSuccess;
  transpose_bf16_kernel<<<ntiles, 256, 0, s>>>(items, nitems, src, dst);
  return hipGetLastError();
}

// out = gelu(in), 8 elements (16 or 32 bytes) per thread and step
template <typename T>
__global__ __launch_bounds__(256) void gelu_kernel(const T* __restrict__ in, T* __restrict__ out, size_t n8) {
  constexpr int VEC = Elt<T>::VEC;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
#pragma unroll
    for (int h = 0; h < 8 / VEC; ++h) {
      V16<T> v;
      v.load(in + i * 8 + h * VEC);
#pragma unroll
      for (int e = 0; e < VEC; ++e) v.v[e] = gelu_fwd(v.v[e]);
      v.store(out + i * 8 + h * VEC);
    }
  }
}
hipError_t launch_gelu(DType dt, const void* in, void* out, size_t n, hipStream_t s) {
  if (n % 8) return hipErrorInvalidValue;
  const size_t n8 = n / 8;
  if (!n8) return hipSuccess;
  const int blocks = (int)std::min<size_t>(8192, (n8 + 255) / 256);
  if (dt == DT_BF16)
    gelu_kernel<bf16><<<blocks, 256, 0, s>>>(reinterpret_cast<const bf16*>(in), reinterpret_cast<bf16*>(out), n8);
  else
    gelu_kernel<float><<<blocks, 256, 0, s>>>(reinterpret_cast<const float*>(in), reinterpret_cast<float*>(out), n8);
  return hipGetLastError();
}

// A plain streaming copy, the reference for what this part sustains on a read-and-write stream:
// 1024 blocks striding over the buffer, each thread with four 16-byte loads in flight (straight-
// line: an index past the end reads the last vector and is not stored).
__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                   size_t n16) {
  constexpr int U = 4;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[min(i + u * stride, n16 - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + u * stride < n16) dst[i + u * stride] = v[u];
  }
}
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  copy_kernel<<<(int)std::min<size_t>(1024, (n16 + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), n16);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, size_t n, float v) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}
hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s) {
  if (!n) return hipSuccess;
  fill_kernel<<<(int)std::min<size_t>(8192, (n + 255) / 256), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace g2
