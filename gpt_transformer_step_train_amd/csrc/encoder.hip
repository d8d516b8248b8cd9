// Token + position encoder, forward and backward.
//
// The llm.c tour ("Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖)
// names encoder_forward first and encoder_backward among the backward layers: the forward adds
// the token row of wte and the position row of wpe; the backward adds the output gradient of each
// position into the wte row of its token and the wpe row of its position.
//
// The wte scatter is made deterministic without atomics: the (token, position) pairs are sorted
// once (bitonic sort of unique 31-bit keys in LDS), every run of equal tokens is then summed in
// position order. Runs are cut into fixed 32-entry chunks; a run that crosses a chunk boundary
// leaves per-chunk pieces that its first chunk adds up in chunk order.
#include "common.h"
#include "kernels.h"

namespace g2 {

template <typename T>
__global__ __launch_bounds__(256) void encoder_fwd_kernel(int BT, int T_, int C, int V, const int32_t* __restrict__ tok,
                                                          const T* __restrict__ wte, const T* __restrict__ wpe,
                                                          T* __restrict__ out, int* err) {
  constexpr int VEC = Elt<T>::VEC;
  const int nv = C / VEC;
  const size_t total = (size_t)BT * nv;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const int row = (int)(i / nv);
    const int cv = (int)(i % nv);
    int t = tok[row];
    if (t < 0 || t >= V) {
      if (cv == 0) atomicOr(err, 1);
      t = 0;
    }
    V16<T> a, b;
    a.load(wte + (size_t)t * C + cv * VEC);
    b.load(wpe + (size_t)(row % T_) * C + cv * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) a.v[e] += b.v[e];
    a.store(out + (size_t)row * C + cv * VEC);
  }
}

hipError_t launch_encoder_fwd(DType dt, int B, int T, int C, int V, const int32_t* tok, const void* wte,
                              const void* wpe, void* out, int* err, hipStream_t s) {
  const int BT = B * T;
  if (BT <= 0) return hipSuccess;
  const int vec = dt == DT_BF16 ? 8 : 4;
  if (C <= 0 || C % vec) return hipErrorInvalidValue;  // rows move as 16-byte vectors
  const int blocks = std::min(cdiv((long)BT * (C / vec), 256), 8192);
  if (dt == DT_BF16)
    encoder_fwd_kernel<bf16><<<blocks, 256, 0, s>>>(BT, T, C, V, tok, reinterpret_cast<const bf16*>(wte),
                                                   reinterpret_cast<const bf16*>(wpe), reinterpret_cast<bf16*>(out), err);
  else
    encoder_fwd_kernel<float><<<blocks, 256, 0, s>>>(BT, T, C, V, tok, reinterpret_cast<const float*>(wte),
                                                    reinterpret_cast<const float*>(wpe), reinterpret_cast<float*>(out), err);
  return hipGetLastError();
}

// ------------------------------------------------------------------ sort of (token, position)
constexpr int POS_BITS = 15;  // BT <= 32768
constexpr uint32_t POS_MASK = (1u << POS_BITS) - 1u;
__device__ __forceinline__ int key_tok(uint32_t k) { return (int)(k >> POS_BITS); }
__device__ __forceinline__ int key_pos(uint32_t k) { return (int)(k & POS_MASK); }

__global__ __launch_bounds__(1024) void encoder_sort_kernel(int BT, int n2, int V, const int32_t* __restrict__ tok,
                                                            uint32_t* __restrict__ keys) {
  extern __shared__ uint32_t sk[];
  for (int i = threadIdx.x; i < n2; i += 1024) {
    uint32_t k = 0xffffffffu;
    if (i < BT) {
      int t = tok[i];
      t = (t < 0 || t >= V) ? 0 : t;  // out-of-range ids were reported by the forward
      k = ((uint32_t)t << POS_BITS) | (uint32_t)i;
    }
    sk[i] = k;
  }
  __syncthreads();
  const int npairs = n2 >> 1;
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int pr = threadIdx.x; pr < npairs; pr += 1024) {
        const int i = 2 * j * (pr / j) + (pr % j);
        const int l = i + j;
        const uint32_t a = sk[i], b = sk[l];
        const bool up = (i & k) == 0;
        if ((a > b) == up) {
          sk[i] = b;
          sk[l] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < BT; i += 1024) keys[i] = sk[i];
}

hipError_t launch_encoder_sort(int BT, int V, const int32_t* tok, uint32_t* keys, hipStream_t s) {
  if (BT <= 0) return hipSuccess;
  if (BT > (1 << POS_BITS) || V > (1 << (32 - POS_BITS - 1))) return hipErrorInvalidValue;
  int n2 = 1;
  while (n2 < BT) n2 <<= 1;
  n2 = std::max(n2, 2);
  if ((size_t)n2 * 4 > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&encoder_sort_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, n2 * 4);
    if (e != hipSuccess) return e;
  }
  encoder_sort_kernel<<<1, 1024, (size_t)n2 * 4, s>>>(BT, n2, V, tok, keys);
  return hipGetLastError();
}

// ------------------------------------------------------------------ backward
constexpr int CH = 32;  // sorted entries per chunk

// dwpe[t] (+)= sum_b dout[b, t]: one thread per 16-byte column vector of one position; the rows of
// 8 batch entries are requested at a time (straight-line loads), then added in batch order.
template <typename T>
__global__ __launch_bounds__(256) void wpe_bwd_kernel(int B, int T_, int maxT, int C, const T* __restrict__ dout,
                                                      float* __restrict__ dwpe, int accumulate) {
  constexpr int VEC = Elt<T>::VEC;
  const int nv = C / VEC;
  const int i = blockIdx.x * 256 + threadIdx.x;  // over maxT * nv; rows t >= T get no gradient
  if (i >= maxT * nv) return;
  const int t = i / nv, c = (i % nv) * VEC;
  float s[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = 0.f;
  if (t < T_) {
    for (int b0 = 0; b0 < B; b0 += 8) {
      u32x4 r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = min(b0 + u, B - 1);
        r[u] = *reinterpret_cast<const u32x4*>(dout + ((size_t)b * T_ + t) * C + c);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < B) {
          V16<T> v;
          v.unpack(r[u]);
#pragma unroll
          for (int e = 0; e < VEC; ++e) s[e] += v.v[e];
        }
      }
    }
  }
  float* dst = dwpe + (size_t)t * C + c;
#pragma unroll
  for (int e = 0; e < VEC; ++e) dst[e] = accumulate ? dst[e] + s[e] : s[e];
}

struct ChunkInfo {
  int start, end;
  bool head_cont, tail_cont, single;
};
__device__ __forceinline__ ChunkInfo chunk_info(const uint32_t* keys, int BT, int ch) {
  ChunkInfo c;
  c.start = ch * CH;
  c.end = min(BT, c.start + CH);
  c.head_cont = ch > 0 && key_tok(keys[c.start]) == key_tok(keys[c.start - 1]);
  c.tail_cont = c.end < BT && key_tok(keys[c.end - 1]) == key_tok(keys[c.end]);
  c.single = key_tok(keys[c.start]) == key_tok(keys[c.end - 1]);
  return c;
}

// 4 consecutive elements of a row of the output gradient (8 bytes in bf16, 16 in fp32), as floats
template <typename T> __device__ __forceinline__ f32x4 load4(const T* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
template <> __device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  const u32x2 r = *reinterpret_cast<const u32x2*>(p);
  return f32x4{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u), __uint_as_float(r[1] << 16),
               __uint_as_float(r[1] & 0xffff0000u)};
}

// grid: (nchunks, cdiv(C/4, 64)), block 64: 4 consecutive columns per thread. Everything a chunk
// reads is requested before the first value is used, so a chunk costs one memory round trip
// instead of one per entry and one per token it adds into: the keys with one vector load (lane i
// holds entry i) broadcast with readlane, then, as straight-line loads, the output-gradient row of
// every entry and the dwte row of every entry's token (the old value a run adds to; each dwte row
// is added to by at most one chunk here, the one holding its whole run). Entries past the chunk
// end repeat its last one and lanes past the last column read the last one; both are unused.
// (A guarded load would make the compiler wait for it at the branch join.)
template <typename T>
__global__ __launch_bounds__(64) void wte_bwd_chunks(int BT, int C, const uint32_t* __restrict__ keys,
                                                     const T* __restrict__ dout, float* __restrict__ dwte,
                                                     float* __restrict__ part_head, float* __restrict__ part_tail) {
  const int lane = threadIdx.x;
  const int c4 = blockIdx.y * 64 + lane;  // column group of 4
  const bool active = c4 * 4 < C;
  const int col = (active ? c4 : C / 4 - 1) * 4;
  const int ch = blockIdx.x;
  const ChunkInfo ci = chunk_info(keys, BT, ch);
  const int n = ci.end - ci.start;
  const uint32_t kl = keys[ci.start + min(lane, n - 1)];
  uint32_t kk[CH];
  f32x4 d[CH], old[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    kk[i] = __builtin_amdgcn_readlane(kl, i);
    d[i] = load4<T>(dout + (size_t)key_pos(kk[i]) * C + col);
    old[i] = *reinterpret_cast<const f32x4*>(dwte + (size_t)key_tok(kk[i]) * C + col);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int cur = key_tok(kk[0]);
  bool first = true;
  // the run of token cur ends at entry i (whose prefetched dwte row is old[i])
  auto flush = [&](int i, bool last) {
    if (!active) return;
    float* dst;
    f32x4 v = acc;
    if (first && ci.head_cont) dst = part_head + (size_t)ch * C;
    else if (last && ci.tail_cont) dst = part_tail + (size_t)ch * C;
    else {
      dst = dwte + (size_t)cur * C;
      v = old[i] + acc;
    }
    *reinterpret_cast<f32x4*>(dst + col) = v;
  };
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (i < n) {
      const int v = key_tok(kk[i]);
      if (v != cur) {
        flush(i - 1, false);
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        cur = v;
        first = false;
      }
      acc += d[i];
      if (i == n - 1) flush(i, true);
    }
  }
}

// Runs that cross chunk boundaries: the chunk where the run starts adds the pieces of the chunks
// the run reaches, in chunk order. The run's end is found by binary search over the sorted keys
// (a few dependent loads, where walking the chunks one by one cost two per chunk), then the pieces
// are loaded 8 at a time.
__global__ __launch_bounds__(256) void wte_bwd_fixup(int BT, int C, int nch, const uint32_t* __restrict__ keys,
                                                     float* __restrict__ dwte, const float* __restrict__ part_head,
                                                     const float* __restrict__ part_tail) {
  const int ch = blockIdx.x;
  const ChunkInfo ci = chunk_info(keys, BT, ch);
  if (!ci.tail_cont || (ci.single && ci.head_cont)) return;
  const int v = key_tok(keys[ci.end - 1]);
  // first sorted index past the run: entries of token v form a prefix of [ci.end, BT)
  int lo = ci.end, hi = BT;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (key_tok(keys[mid]) == v) lo = mid + 1;
    else hi = mid;
  }
  const int last = (lo - 1) / CH;  // the chunk holding the run's last entry
  for (int c = threadIdx.x; c < C; c += 256) {
    float s = part_tail[(size_t)ch * C + c];
    for (int n0 = ch + 1; n0 <= last; n0 += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = n0 + u <= last ? part_head[(size_t)(n0 + u) * C + c] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (n0 + u <= last) s += t[u];
    }
    dwte[(size_t)v * C + c] += s;
  }
}

size_t encoder_bwd_partial_floats(int BT, int C) { return (size_t)2 * cdiv(BT, CH) * C; }

hipError_t launch_encoder_bwd(DType dt, int B, int T, int maxT, int C, const uint32_t* keys, const void* dout, float* dwte,
                              float* dwpe, int accumulate_wpe, float* partial, size_t partial_floats,
                              hipStream_t s) {
  const int BT = B * T;
  if (BT <= 0) return hipSuccess;
  if (T > maxT) return hipErrorInvalidValue;  // positions past the position table
  const int nch = cdiv(BT, CH);
  if (encoder_bwd_partial_floats(BT, C) > partial_floats) return hipErrorInvalidValue;
  float* ph = partial;
  float* pt = partial + (size_t)nch * C;
  const int vec = dt == DT_BF16 ? 8 : 4;
  if (C <= 0 || C % vec) return hipErrorInvalidValue;  // rows move as 16-byte vectors
  dim3 g1(nch, cdiv(C / 4, 64));
  if (dt == DT_BF16) {
    auto D = reinterpret_cast<const bf16*>(dout);
    wpe_bwd_kernel<bf16><<<cdiv((long)maxT * (C / 8), 256), 256, 0, s>>>(B, T, maxT, C, D, dwpe, accumulate_wpe);
    wte_bwd_chunks<bf16><<<g1, 64, 0, s>>>(BT, C, keys, D, dwte, ph, pt);
  } else {
    auto D = reinterpret_cast<const float*>(dout);
    wpe_bwd_kernel<float><<<cdiv((long)maxT * (C / 4), 256), 256, 0, s>>>(B, T, maxT, C, D, dwpe, accumulate_wpe);
    wte_bwd_chunks<float><<<g1, 64, 0, s>>>(BT, C, keys, D, dwte, ph, pt);
  }
  wte_bwd_fixup<<<nch, 256, 0, s>>>(BT, C, nch, keys, dwte, ph, pt);
  return hipGetLastError();
}

}  // namespace g2
