// MFMA GEMMs for gfx950: C[M,N] = sum_k A(m,k) B(n,k) with fused epilogues.
//
// Every dense contraction of the training step (QKV, attention projection, MLP, tied
// classifier; their input- and weight-gradients) goes through this one template. The llm.c
// code tour ("Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖) names
// operator fusion as the main lever; here bias, GELU (and its derivative) and the residual add
// run in the GEMM epilogue instead of separate passes over HBM.
//
// Design (CDNA4, wave64):
//  * 128x128 block tile, 4 waves in a 2x2 grid, 64x64 per wave = 2x2 MFMA 32x32 blocks.
//    bf16: v_mfma_f32_32x32x16_bf16, BK = 64.  fp32: v_mfma_f32_32x32x2f32, BK = 32.
//  * LDS holds both operands as [row][k] (k contiguous, +16 B pad), so every MFMA operand is one
//    LDS read per lane. Operands whose memory layout is K-contiguous are copied 16 B at a time;
//    M/N-contiguous operands (the transposed side of NN / TN products) are loaded as 4 x 16 B
//    row pieces and transposed in registers on the way into LDS.
//  * Double-buffered LDS with register staging: the global loads of tile k+1 are in flight while
//    tile k is multiplied; one barrier per K tile.
//  * Block ids are remapped so that each XCD (blocks are dealt round-robin to the 8 XCDs) gets a
//    contiguous run of tiles, and tiles are ordered in groups of 8 tile-rows for L2 reuse.
//  * Split-K (weight gradients, K = B*T) writes fp32 partials that a second kernel sums in a
//    fixed order: deterministic, no atomics.
#include "common.h"
#include "kernels.h"

namespace g2 {

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KSTEP = 16;  // k per instruction
  static constexpr int KPL = 8;     // k elements supplied by one lane
  static constexpr int BK = 64;
  typedef bf16x8 frag;
  __device__ static frag load(const bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KSTEP = 2;
  static constexpr int KPL = 1;
  static constexpr int BK = 32;
  typedef float frag;
  __device__ static frag load(const float* p) { return *p; }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

constexpr int BM = 128, BN = 128, NTHR = 256, WGN = 2;
constexpr int TM = 64, TN = 64, FM = 2, FN = 2;
constexpr int GROUP_M = 8;

// Transposed piece: TKR k-rows x VEC m-columns per thread.
constexpr int TKR = 4;

template <typename T> struct Tile {
  static constexpr int VEC = Elt<T>::VEC;
  static constexpr int BK = Mma<T>::BK;
  static constexpr int LD = BK + VEC;  // LDS row pitch in elements (16 B pad)
  // K-contiguous copy: vectors per thread
  static constexpr int NV_K = (BM * BK / VEC) / NTHR;
  // transposed copy: pieces per thread
  static constexpr int NV_T = ((BK / TKR) * (BM / VEC)) / NTHR;
};

// Load one operand tile (ROWS=128 rows of the M or N side, BK of K) into registers.
// kc: operand is K-contiguous (ptr[row*ld + k]) else row-contiguous (ptr[k*ld + row]).
template <typename T, bool KC> struct Loader {
  using TL = Tile<T>;
  static constexpr int VEC = TL::VEC;
  static constexpr int NREG = KC ? TL::NV_K : TL::NV_T * TKR;
  u32x4 r[NREG];

  __device__ __forceinline__ void load(const T* __restrict__ ptr, long ld, int row0, int nrows, int k0, int K) {
    const int tid = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < TL::NV_K; ++i) {
        const int v = i * NTHR + tid;
        const int row = v / (TL::BK / VEC);
        const int kc = (v % (TL::BK / VEC)) * VEC;
        const int k = k0 + kc;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row0 + row < nrows && k < K) {
          x = *reinterpret_cast<const u32x4*>(ptr + (size_t)(row0 + row) * ld + k);
          if (k + VEC > K) mask_tail(x, K - k);
        }
        r[i] = x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < TL::NV_T; ++i) {
        const int pc = i * NTHR + tid;
        const int mc = (pc % (BM / VEC)) * VEC;
        const int kr = (pc / (BM / VEC)) * TKR;
#pragma unroll
        for (int j = 0; j < TKR; ++j) {
          const int k = k0 + kr + j;
          const int m = row0 + mc;
          u32x4 x = {0u, 0u, 0u, 0u};
          if (k < K && m < nrows) {
            x = *reinterpret_cast<const u32x4*>(ptr + (size_t)k * ld + m);
            if (m + VEC > nrows) mask_tail(x, nrows - m);
          }
          r[i * TKR + j] = x;
        }
      }
    }
  }

  // zero elements [keep, VEC) of a 16-byte vector
  __device__ __forceinline__ static void mask_tail(u32x4& x, int keep) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e >= keep) x[e] = 0u;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (2 * e >= keep) x[e] = 0u;
        else if (2 * e + 1 >= keep) x[e] &= 0xffffu;
      }
    }
  }

  __device__ __forceinline__ void store(T* __restrict__ lds) const {
    const int tid = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < TL::NV_K; ++i) {
        const int v = i * NTHR + tid;
        const int row = v / (TL::BK / VEC);
        const int kc = (v % (TL::BK / VEC)) * VEC;
        *reinterpret_cast<u32x4*>(lds + row * TL::LD + kc) = r[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < TL::NV_T; ++i) {
        const int pc = i * NTHR + tid;
        const int mc = (pc % (BM / VEC)) * VEC;
        const int kr = (pc / (BM / VEC)) * TKR;
        const u32x4* in = &r[i * TKR];
        if constexpr (sizeof(T) == 4) {
          // 4x4 floats: column c of the 4 k-rows becomes one 16-byte LDS row piece
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x4 o = {in[0][c], in[1][c], in[2][c], in[3][c]};
            *reinterpret_cast<u32x4*>(lds + (mc + c) * TL::LD + kr) = o;
          }
        } else {
          // 4 k-rows x 8 bf16 columns -> 8 LDS rows of 4 bf16 (8 bytes)
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int d = c >> 1;
            u32x2 o;
            if ((c & 1) == 0) {
              o[0] = (in[0][d] & 0xffffu) | (in[1][d] << 16);
              o[1] = (in[2][d] & 0xffffu) | (in[3][d] << 16);
            } else {
              o[0] = (in[0][d] >> 16) | (in[1][d] & 0xffff0000u);
              o[1] = (in[2][d] >> 16) | (in[3][d] & 0xffff0000u);
            }
            *reinterpret_cast<u32x2*>(lds + (mc + c) * TL::LD + kr) = o;
          }
        }
      }
    }
  }
};

template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const f32x16 (&acc)[FM][FN], int m_base, int n_base) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const T* bias = reinterpret_cast<const T*>(p.bias);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n_base + j * 32 + (lane & 31);
    if (col >= p.N) continue;
    float bv = 0.f;
    if constexpr (EPI == EPI_BIAS || EPI == EPI_GELU || EPI == EPI_RESID)
      if (bias) bv = ld1(bias, col);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m_base + i * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
        if (row >= p.M) continue;
        const float a = acc[i][j][r];
        const size_t idx = (size_t)row * p.ldc + col;
        if constexpr (EPI == EPI_BIAS) {
          st1(reinterpret_cast<T*>(p.C), idx, a + bv);
        } else if constexpr (EPI == EPI_GELU) {
          const float pre = a + bv;
          st1(reinterpret_cast<T*>(p.C), idx, pre);
          st1(reinterpret_cast<T*>(p.C2), idx, gelu_fwd(pre));
        } else if constexpr (EPI == EPI_RESID) {
          const float res = ld1(reinterpret_cast<const T*>(p.aux), (size_t)row * p.ldaux + col);
          st1(reinterpret_cast<T*>(p.C), idx, res + (a + bv));
        } else if constexpr (EPI == EPI_GELU_BWD) {
          const float pre = ld1(reinterpret_cast<const T*>(p.aux), (size_t)row * p.ldaux + col);
          st1(reinterpret_cast<T*>(p.C), idx, a * gelu_bwd(pre));
        } else {  // EPI_F32 ; split partials use ldc = N and a pre-offset C
          float* C = reinterpret_cast<float*>(p.C);
          C[idx] = p.accumulate ? C[idx] + a : a;
        }
      }
    }
  }
}

template <typename T, bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(GemmArgs p, int k_split, float* split_out) {
  using TL = Tile<T>;
  using MM = Mma<T>;
  __shared__ __attribute__((aligned(16))) T As[2][BM * TL::LD];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * TL::LD];

  // tile mapping: XCD-contiguous runs, then grouped row-major order
  const int tiles_m = cdiv(p.M, BM), tiles_n = cdiv(p.N, BN);
  const int nt = gridDim.x;
  int b = blockIdx.x;
  if ((nt & 7) == 0) b = (b & 7) * (nt >> 3) + (b >> 3);
  const int group = GROUP_M * tiles_n;
  const int first_m = (b / group) * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (b % group) % gsz;
  const int tn = (b % group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = blockIdx.z * k_split;
  const int kend = min(p.K, kbeg + k_split);
  const int nkt = cdiv(kend - kbeg, TL::BK);

  const T* A = reinterpret_cast<const T*>(p.A);
  const T* B = reinterpret_cast<const T*>(p.B);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w / WGN, wn = w % WGN;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Loader<T, AKC> la;
  Loader<T, BKC> lb;
  if (nkt > 0) {
    la.load(A, p.lda, m0, p.M, kbeg, kend);
    lb.load(B, p.ldb, n0, p.N, kbeg, kend);
    la.store(As[0]);
    lb.store(Bs[0]);
  }
  __syncthreads();

  const int arow = wm * TM + (lane & 31);
  const int brow = wn * TN + (lane & 31);
  const int kofs = (lane >> 5) * MM::KPL;

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
      const int k0 = kbeg + (kt + 1) * TL::BK;
      la.load(A, p.lda, m0, p.M, k0, kend);
      lb.load(B, p.ldb, n0, p.N, k0, kend);
    }
    const T* as = As[cur];
    const T* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < TL::BK; kk += MM::KSTEP) {
      typename MM::frag fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = MM::load(as + (arow + i * 32) * TL::LD + kk + kofs);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = MM::load(bs + (brow + j * 32) * TL::LD + kk + kofs);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = MM::mma(fa[i], fb[j], acc[i][j]);
    }
    if (more) {
      la.store(As[cur ^ 1]);
      lb.store(Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  if constexpr (EPI == EPI_F32) {
    if (split_out) {
      GemmArgs q = p;
      q.C = split_out + (size_t)blockIdx.z * p.M * p.N;
      q.ldc = p.N;
      q.accumulate = 0;
      epilogue<T, EPI>(q, acc, m0 + wm * TM, n0 + wn * TN);
      return;
    }
  }
  epilogue<T, EPI>(p, acc, m0 + wm * TM, n0 + wn * TN);
}

// dst[i] (+)= sum_z part[z][i], z in order
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ part, int splits, size_t n,
                                                     float* __restrict__ dst, int accumulate) {
  const size_t n4 = n / 4;
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    f32x4 s = accumulate ? reinterpret_cast<const f32x4*>(dst)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z) s += reinterpret_cast<const f32x4*>(part + (size_t)z * n)[i];
    reinterpret_cast<f32x4*>(dst)[i] = s;
  }
  for (size_t i = n4 * 4 + blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float s = accumulate ? dst[i] : 0.f;
    for (int z = 0; z < splits; ++z) s += part[(size_t)z * n + i];
    dst[i] = s;
  }
}

int gemm_splits(int M, int N, int K, size_t scratch_floats) {
  const long tiles = (long)cdiv(M, BM) * cdiv(N, BN);
  int s = 1;
  // aim for >= ~2 waves of 256 CUs x 2 blocks; each split keeps >= 1024 of K
  while (tiles * s < 1024 && K / (s * 2) >= 1024 && (size_t)(s * 2) * M * N <= scratch_floats) s *= 2;
  return s;
}

template <typename T, bool AKC, bool BKC>
static hipError_t launch_t(Epi epi, const GemmArgs& a, float* scratch, size_t scratch_floats, hipStream_t s) {
  const int tiles = cdiv(a.M, BM) * cdiv(a.N, BN);
  int splits = 1;
  if (epi == EPI_F32 && scratch) splits = gemm_splits(a.M, a.N, a.K, scratch_floats);
  int k_split = a.K;
  if (splits > 1) {
    k_split = cdiv(cdiv(a.K, splits), Tile<T>::BK) * Tile<T>::BK;
    splits = cdiv(a.K, k_split);
  }
  dim3 grid(tiles, 1, splits);
  switch (epi) {
    case EPI_BIAS: gemm_kernel<T, AKC, BKC, EPI_BIAS><<<grid, NTHR, 0, s>>>(a, k_split, nullptr); break;
    case EPI_GELU: gemm_kernel<T, AKC, BKC, EPI_GELU><<<grid, NTHR, 0, s>>>(a, k_split, nullptr); break;
    case EPI_RESID: gemm_kernel<T, AKC, BKC, EPI_RESID><<<grid, NTHR, 0, s>>>(a, k_split, nullptr); break;
    case EPI_GELU_BWD: gemm_kernel<T, AKC, BKC, EPI_GELU_BWD><<<grid, NTHR, 0, s>>>(a, k_split, nullptr); break;
    case EPI_F32:
      gemm_kernel<T, AKC, BKC, EPI_F32><<<grid, NTHR, 0, s>>>(a, k_split, splits > 1 ? scratch : nullptr);
      if (splits > 1) {
        const size_t n = (size_t)a.M * a.N;
        const int blocks = (int)std::min<size_t>(4096, (n / 4 + 255) / 256 + 1);
        // C must be dense (ldc == N) for the reduction
        splitk_reduce<<<blocks, 256, 0, s>>>(scratch, splits, n, reinterpret_cast<float*>(a.C), a.accumulate);
      }
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(DType dt, bool a_kc, bool b_kc, Epi epi, const GemmArgs& a, float* scratch,
                       size_t scratch_floats, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (epi == EPI_F32 && scratch && a.ldc != a.N) scratch = nullptr;
  if (dt == DT_BF16) {
    if (a_kc && b_kc) return launch_t<bf16, true, true>(epi, a, scratch, scratch_floats, s);
    if (a_kc && !b_kc) return launch_t<bf16, true, false>(epi, a, scratch, scratch_floats, s);
    if (!a_kc && !b_kc) return launch_t<bf16, false, false>(epi, a, scratch, scratch_floats, s);
    return launch_t<bf16, false, true>(epi, a, scratch, scratch_floats, s);
  }
  if (a_kc && b_kc) return launch_t<float, true, true>(epi, a, scratch, scratch_floats, s);
  if (a_kc && !b_kc) return launch_t<float, true, false>(epi, a, scratch, scratch_floats, s);
  if (!a_kc && !b_kc) return launch_t<float, false, false>(epi, a, scratch, scratch_floats, s);
  return launch_t<float, false, true>(epi, a, scratch, scratch_floats, s);
}

// ----------------------------------------------------------------------------------------
// Column sums (bias gradients): partial[y][n] = sum over rows of chunk y; then db (+)= sum_y.
// ----------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void colsum_partial(const T* __restrict__ x, long ld, int M, int N, int rows_per,
                                                      float* __restrict__ partial) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= N) return;
  const int r0 = blockIdx.y * rows_per;
  const int r1 = min(M, r0 + rows_per);
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += ld1(x, (size_t)r * ld + col);
  partial[(size_t)blockIdx.y * N + col] = s;
}

__global__ __launch_bounds__(256) void colsum_finish(const float* __restrict__ partial, int ny, int N,
                                                     float* __restrict__ out, int accumulate) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= N) return;
  float s = 0.f;
  for (int y = 0; y < ny; ++y) s += partial[(size_t)y * N + col];
  out[col] = accumulate ? out[col] + s : s;
}

hipError_t launch_colsum(DType dt, const void* dY, long ld, int M, int N, float* db, int accumulate,
                         float* partial, size_t partial_floats, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  int ny = std::max(1, std::min(cdiv(M, 64), 256));
  while ((size_t)ny * N > partial_floats && ny > 1) ny /= 2;
  const int rows_per = cdiv(M, ny);
  ny = cdiv(M, rows_per);
  if (M <= 0) ny = 0;
  dim3 grid(cdiv(N, 256), std::max(ny, 1));
  if (ny > 0) {
    if (dt == DT_BF16)
      colsum_partial<bf16><<<grid, 256, 0, s>>>(reinterpret_cast<const bf16*>(dY), ld, M, N, rows_per, partial);
    else
      colsum_partial<float><<<grid, 256, 0, s>>>(reinterpret_cast<const float*>(dY), ld, M, N, rows_per, partial);
  }
  colsum_finish<<<cdiv(N, 256), 256, 0, s>>>(partial, ny, N, db, accumulate);
  return hipGetLastError();
}

}  // namespace g2
