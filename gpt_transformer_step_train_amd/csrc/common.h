// Device-side building blocks shared by the gfx950 kernels: storage types, 128-bit vector
// access, bf16 conversion, wave64 reductions, and the fp32 math used in the epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g2 {

// bf16 is stored as its 16 raw bits; arithmetic is always done in fp32.
struct bf16 {
  uint16_t u;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two at once: one v_cvt_pk_bf16_f32 (the scalar conversions above would take two, plus the
// shift and or that join them).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int VEC = 4;  // elements per 16-byte vector
  __device__ static float get(const float* p, size_t i) { return p[i]; }
  __device__ static void put(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elt<bf16> {
  static constexpr int VEC = 8;
  __device__ static float get(const bf16* p, size_t i) { return bf2f(p[i].u); }
  __device__ static void put(bf16* p, size_t i, float v) { p[i].u = f2bf(v); }
};
template <typename T> __device__ __forceinline__ float ld1(const T* p, size_t i) { return Elt<T>::get(p, i); }
template <typename T> __device__ __forceinline__ void st1(T* p, size_t i, float v) { Elt<T>::put(p, i, v); }

// 16-byte vector <-> VEC floats
template <typename T> struct V16 {
  static constexpr int N = Elt<T>::VEC;
  float v[N];
  __device__ __forceinline__ void load(const T* p) {
    u32x4 r = *reinterpret_cast<const u32x4*>(p);
    unpack(r);
  }
  __device__ __forceinline__ void unpack(u32x4 r);
  __device__ __forceinline__ u32x4 pack() const;
  __device__ __forceinline__ void store(T* p) const { *reinterpret_cast<u32x4*>(p) = pack(); }
};
template <> __device__ __forceinline__ void V16<float>::unpack(u32x4 r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
}
template <> __device__ __forceinline__ u32x4 V16<float>::pack() const {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(v[i]);
  return r;
}
template <> __device__ __forceinline__ void V16<bf16>::unpack(u32x4 r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r[i] << 16);
    v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ u32x4 V16<bf16>::pack() const {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack2bf(v[2 * i], v[2 * i + 1]);
  return r;
}

// ---------------------------------------------------------------------------------------
// Wave64 reductions. Within each 16-lane row DPP moves combine quads, then half-rows, then
// rows; the four row results are read with v_readlane and combined in a fixed order, so every
// lane gets the same, deterministic value.
// ---------------------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<DPP_QUAD_XOR1>(v);
  v += dpp<DPP_QUAD_XOR2>(v);
  v += dpp<DPP_ROW_HALF_MIRROR>(v);
  v += dpp<DPP_ROW_MIRROR>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  return v;
}
__device__ __forceinline__ float readlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}
// Combine a value with the one held by lane (l ^ 32), using v_permlane32_swap (gfx950). With
// both operands = v, the swap returns {v for lanes < 32, v[l-32] above} and {v[l+32] below, v
// above}, so the two results hold this lane's value and its partner's in some order.
__device__ __forceinline__ float pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Block-wide sum for blockDim.x = 64 * NW; deterministic order. `red` holds >= NW floats.
template <int NW> __device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += red[i];
  return s;
}
template <int NW> __device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = -INFINITY;
#pragma unroll
  for (int i = 0; i < NW; ++i) s = fmaxf(s, red[i]);
  return s;
}

// ---------------------------------------------------------------------------------------
// fp32 math
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E = 1.4426950408889634f;
constexpr float GELU_K = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float GELU_C = 0.044715f;

// GELU, tanh form, written as x * sigmoid(2u) with u = sqrt(2/pi)(x + 0.044715 x^3);
// 0.5(1 + tanh u) equals sigmoid(2u) exactly. The constants are folded so that the exponent is
// x (a + b x^2) in base 2 (two VALU ops) and the derivative
//   s + 2 x s (1 - s) sqrt(2/pi) (1 + 3 * 0.044715 x^2) = s + g (1 - s) (p + q x^2), g = x s,
// costs three more fused multiply-adds: these run in GEMM epilogues, where VALU time counts.
constexpr float GELU_EA = -2.0f * LOG2E * GELU_K;           // exponent: x (EA + EB x^2)
constexpr float GELU_EB = -2.0f * LOG2E * GELU_K * GELU_C;
constexpr float GELU_DP = 2.0f * GELU_K;                    // derivative polynomial p + q x^2
constexpr float GELU_DQ = 6.0f * GELU_K * GELU_C;
__device__ __forceinline__ float gelu_sig2(float x, float x2) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(x * fmaf(x2, GELU_EB, GELU_EA)));
}
__device__ __forceinline__ float gelu_fwd(float x) { return x * gelu_sig2(x, x * x); }
__device__ __forceinline__ float gelu_bwd(float x) {
  const float x2 = x * x;
  const float s = gelu_sig2(x, x2);
  const float g = x * s;
  return fmaf(fmaf(-g, s, g), fmaf(x2, GELU_DQ, GELU_DP), s);
}
// gelu(x) and gelu'(x) sharing one sigmoid
__device__ __forceinline__ void gelu_both(float x, float& g, float& dg) {
  const float x2 = x * x;
  const float s = gelu_sig2(x, x2);
  g = x * s;
  dg = fmaf(fmaf(-g, s, g), fmaf(x2, GELU_DQ, GELU_DP), s);
}

__host__ __device__ constexpr int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// out[c] (+)= sum_{y < ny} part[y * ld + c] for c < ncols, summed in a fixed order.
// Block of 1024 threads handles 32 columns: 32 row-groups stride over y, each thread issuing the
// loads of 16 rows (y, y + 32, ...) before adding any of them, so that up to 512 rows cost one
// memory round trip; then the 32 group sums of a column are added in order. Columns
// [32 chunk, 32 chunk + 32).
constexpr int RP_THREADS = 1024;
__device__ __forceinline__ void reduce_partials_block(const float* __restrict__ part, int ny, long ld, int ncols,
                                                      float* __restrict__ out, int accumulate, int chunk) {
  constexpr int U = 16;
  __shared__ float sh[32][33];
  const int cl = threadIdx.x & 31, yg = threadIdx.x >> 5;
  const int c = chunk * 32 + cl;
  float s = 0.f;
  if (c < ncols) {
    for (int y0 = yg; y0 < ny; y0 += U * 32) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int y = y0 + u * 32;
        v[u] = y < ny ? part[(size_t)y * ld + c] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) s += v[u];
    }
  }
  sh[yg][cl] = s;
  __syncthreads();
  if (yg == 0 && c < ncols) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) t += sh[i][cl];
    out[c] = accumulate ? out[c] + t : t;
  }
}

}  // namespace g2
