// MFMA GEMMs for gfx950: C[M,N] = sum_k A(m,k) B(n,k) with fused epilogues.
//
// Every dense contraction of the training step (QKV, attention projection, MLP, tied
// classifier; their input- and weight-gradients) goes through this one template. The llm.c
// code tour ("Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖) names
// operator fusion as the main lever; here bias, GELU (and its derivative) and the residual add
// run in the GEMM epilogue instead of separate passes over HBM.
//
// Design (CDNA4, wave64):
//  * Block tiles: 256x256 with 8 waves (2 per SIMD, 128x64 each = 4x2 MFMA 32x32 blocks) for
//    the large bf16 products and the split-K weight gradients; 256x192 with 8 waves (64x96 each)
//    where 192-wide column tiles fill the rounds of 256 CUs better (N = 768, 2304); 128x128 with
//    4 waves (64x64 each) for small grids and fp32. bf16: v_mfma_f32_32x32x16_bf16; fp32:
//    v_mfma_f32_32x32x2f32.
//  * bf16 products stage 64 of K per tile; interior tiles are copied global -> LDS directly
//    (global_load_lds_dwordx4: no staging registers, no LDS write instructions). A K-contiguous
//    operand lands as [row][k] rows whose 16-byte chunks are XOR-swizzled so that the MFMA
//    fragment reads are free of bank conflicts; a row-contiguous one (the weight gradients) stays
//    [k][row] and its MFMA fragments are read with the gfx950 transpose load ds_read_b64_tr_b16.
//    The copies into one stage and the reads of another are issued through distinct restrict
//    pointers: without that the compiler makes every transpose read wait for all copies in
//    flight. Edge tiles and fp32 go through registers.
//  * Double-buffered LDS, one barrier per tile; operand fragments double-buffered in registers
//    so the LDS reads of one k-step overlap the MFMAs of the previous one.
//  * Epilogue through LDS: each wave parks 32 rows of fp32 accumulators in LDS and reads them back
//    row-contiguous, so bias / residual / GELU inputs are read and results written as 16-byte
//    coalesced vectors.
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
  typedef float frag;
  __device__ static frag load(const float* p) { return *p; }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

constexpr int GROUP_M = 8;
constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int TKR = 4;  // transposed piece: TKR k-rows x VEC row-contiguous elements

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One operand (ROWS rows of the M or N side, BK of K per stage).
// KC: the operand is K-contiguous in memory (ptr[row*ld + k]); else row-contiguous (ptr[k*ld + row]).
// Three LDS layouts (MODE):
//  0 (K-contiguous): unpadded [row][k], BK elements per row (128 bytes), the 16-byte chunk c of
//    row r stored at chunk position c ^ (r & 7): a fragment read (32 consecutive rows, one chunk)
//    touches every bank once.
//  2 (bf16 row-contiguous): [k][row] as in memory, so interior tiles can be copied directly too;
//    the MFMA fragments (8 consecutive k of one row per lane) come out of ds_read_b64_tr_b16,
//    which hands lane 16g+i the element (i & 3) of the 8 bytes addressed by lane 16g+4j+(i>>2)
//    as its element j. The k-rows are packed RB = 512/ROWS to a 1024-byte block (one wave-wide
//    direct copy); block b holds the rows k = (b/4)*4*RB + 4q + (b & 3), q < RB, and blocks are
//    1088 bytes apart, so the four k-rows one transpose read touches fall in four different
//    64-byte bank groups.
//  1 (fp32 row-contiguous): loaded as 4 x 16 B row pieces, transposed in registers and stored as
//    [row][k] with rows padded by 16 bytes.
// Interior tiles of modes 0 and 2 are copied global -> LDS with global_load_lds_dwordx4 (lane l
// of a wave lands at LDS base + 16 l, so each lane fetches the global chunk that belongs there);
// edge tiles and mode 1 go through registers, with out-of-range elements zeroed.
template <typename T, bool KC, int ROWS, int BK_, int NTHR> struct Operand {
  static constexpr int VEC = Elt<T>::VEC;
  static constexpr int BK = BK_;
  static constexpr int MODE = KC ? 0 : (sizeof(T) == 2 ? 2 : 1);
  // interior tiles can be copied global -> LDS
  static constexpr bool DIRECT = MODE == 0 || MODE == 2;
  static constexpr int LD = MODE == 0 ? BK : BK + VEC;  // [row][k] pitch (elements), modes 0 / 1
  // mode 2 geometry
  static constexpr int RB = 512 / ROWS;             // k-rows per 1024-byte block
  static constexpr int BLK = (1024 + 64) / 2;       // block pitch (elements)
  static constexpr int NBLK = BK / RB;              // blocks per stage
  static constexpr int ELEMS = MODE == 2 ? NBLK * BLK : ROWS * LD;  // one stage
  static constexpr int CPK = BK / VEC;  // 16-byte chunks per [row][k] row, mode 0
  static_assert(MODE != 0 || CPK == 4 || CPK == 8, "the swizzle assumes 4 or 8 chunks per row");
  static_assert(MODE != 2 || ((ROWS == 128 || ROWS == 256) && NBLK % 4 == 0), "mode 2 tile shape");
  static constexpr int NV_K = (ROWS * BK / VEC) / NTHR;           // 16-byte vectors per thread
  static constexpr int NV_T = ((BK / TKR) * (ROWS / VEC)) / NTHR;  // transposed pieces per thread
  static constexpr int NREG = MODE == 1 ? NV_T * TKR : NV_K;
  static_assert(NREG > 0, "tile too small for the thread count");
  u32x4 r[NREG];

  // mode 0: chunk c of row r sits at chunk position c ^ swz(r). The LDS serves a 16-byte read
  // for 16 consecutive lanes per clock over 64 banks; the fragment read of 16 consecutive rows at
  // one chunk then touches every bank once.
  __device__ __forceinline__ static int swz(int row) {
    if constexpr (CPK == 8) return (row >> 1) & 7;
    else return (row >> 2) & 3;
  }
  // element offset of (row, k) inside one stage, modes 0 and 1
  __device__ __forceinline__ static int idx(int row, int k) {
    if constexpr (MODE == 0) return row * BK + ((((k / VEC) ^ swz(row)) * VEC) | (k % VEC));
    else return row * LD + k;
  }
  // direct copies per wave per tile
  static constexpr int NDIRECT = MODE == 0 ? (ROWS / (NTHR / 64)) / (64 / CPK) : NBLK / (NTHR / 64);

  // mode 2: block j of wave w; lane l holds (k-row, first row element) of its 16 bytes
  __device__ __forceinline__ static void tr_slot(int b, int lane, int& k, int& m) {
    constexpr int LPR = ROWS / 8;  // lanes per k-row
    const int q = lane / LPR;
    m = (lane % LPR) * 8;
    k = (b >> 2) * 4 * RB + q * 4 + (b & 3);
  }

  // mode 2: per-lane part of the transpose-read address for the wave whose rows start at wrow
  __device__ __forceinline__ static int tr_lane_off(int wrow, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int kh = g >> 1, j = s >> 2;
    const int mq = (g & 1) * 16 + 4 * (s & 3);
    return j * BLK + (RB == 2 ? kh * 4 * BLK : kh * 2 * ROWS) + wrow + mq;
  }
  // mode 2: the fragment of 32-row block i at k-step st (k = 16 st .. 16 st + 15)
  __device__ __forceinline__ static bf16x8 tr_frag(const T* stage, int lane_off, int i, int st) {
    typedef __attribute__((address_space(3))) bf16x4 lds_v4;
    const int c0 = (RB == 2 ? st * 8 : st * 4) * BLK + i * 32;
    const T* p0 = stage + lane_off + c0;
    const T* p1 = p0 + ROWS;  // k + 4
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(p0)));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(p1)));
    const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, v);
  }

  // zero the elements [keep, VEC) of a 16-byte vector (keep <= 0: all), branch-free
  __device__ __forceinline__ static u32x4 keep_first(u32x4 x, int keep) {
    u32x4 o;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = e < keep ? x[e] : 0u;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t m = 2 * e + 1 < keep ? 0xffffffffu : (2 * e < keep ? 0x0000ffffu : 0u);
        o[e] = x[e] & m;
      }
    }
    return o;
  }

  __device__ __forceinline__ static bool interior(int row0, int nrows, int k0, int K) {
    return row0 + ROWS <= nrows && k0 + BK <= K;
  }

  // interior tile, modes 0 and 2: global -> LDS without registers
  __device__ __forceinline__ static void issue_direct(const T* __restrict__ ptr, long ld, int row0, int k0,
                                                      T* lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if constexpr (MODE == 0) {
      constexpr int RPW = ROWS / (NTHR / 64);  // rows per wave
      constexpr int RPI = 64 / CPK;            // rows per wave-wide copy
#pragma unroll
      for (int j = 0; j < RPW / RPI; ++j) {
        const int rb = w * RPW + j * RPI;
        const int rr = rb + lane / CPK;
        const int c = (lane % CPK) ^ swz(rr);
        const T* g = ptr + (size_t)(row0 + rr) * ld + k0 + c * VEC;
        __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(lds + rb * BK), 16, 0, 0);
      }
    } else {
      constexpr int BPW = NBLK / (NTHR / 64);  // blocks per wave
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int b = w * BPW + j;
        int k, m;
        tr_slot(b, lane, k, m);
        const T* g = ptr + (size_t)(k0 + k) * ld + row0 + m;
        __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(lds + b * BLK), 16, 0, 0);
      }
    }
  }

  // Register path. load() only issues the loads (straight-line; out-of-range addresses are
  // replaced by a valid one); store() zeroes the out-of-range elements of edge tiles and writes
  // LDS, so no instruction between the two waits for the loads.
  // Per vector i of this thread: its row (M/N side) and k, relative to the tile.
  __device__ __forceinline__ static void coords(int i, int& row, int& k) {
    const int tid = threadIdx.x;
    if constexpr (MODE == 2) {
      constexpr int BPW = NBLK / (NTHR / 64);
      tr_slot((tid >> 6) * BPW + i, tid & 63, k, row);  // 8 consecutive rows at one k
    } else if constexpr (MODE == 0) {
      const int v = i * NTHR + tid;
      row = v / CPK;
      k = (v % CPK) * VEC;  // VEC consecutive k of one row
    } else {
      const int pc = (i / TKR) * NTHR + tid;
      k = (pc % (BK / TKR)) * TKR + i % TKR;
      row = (pc / (BK / TKR)) * VEC;  // VEC consecutive rows at one k
    }
  }
  // elements of vector i that are in range (0 when it is out of range altogether)
  __device__ __forceinline__ static int keep_count(int i, int row0, int nrows, int k0, int K) {
    int row, k;
    coords(i, row, k);
    row += row0;
    k += k0;
    if constexpr (MODE == 0) return row < nrows && k < K ? K - k : 0;
    else return k < K && row < nrows ? nrows - row : 0;
  }

  __device__ __forceinline__ void load(const T* __restrict__ ptr, long ld, int row0, int nrows, int k0, int K) {
    // one straight-line path for interior and edge tiles: a branch between two load sequences
    // makes the compiler wait for the loads at the join, right after issuing them
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      int row, k;
      coords(i, row, k);
      row += row0;
      k += k0;
      const size_t off = MODE == 0 ? (size_t)row * ld + k : (size_t)k * ld + row;
      const bool ok = row < nrows && k < K;
      r[i] = *reinterpret_cast<const u32x4*>(ok ? ptr + off : ptr);
    }
  }

  __device__ __forceinline__ void store(T* __restrict__ lds, int row0, int nrows, int k0, int K) {
    if (!interior(row0, nrows, k0, K)) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) r[i] = keep_first(r[i], keep_count(i, row0, nrows, k0, K));
    }
    const int tid = threadIdx.x;
    if constexpr (MODE == 2) {
      const int lane = tid & 63, w = tid >> 6;
      constexpr int BPW = NBLK / (NTHR / 64);
#pragma unroll
      for (int j = 0; j < BPW; ++j) *reinterpret_cast<u32x4*>(lds + (w * BPW + j) * BLK + lane * 8) = r[j];
    } else if constexpr (MODE == 0) {
#pragma unroll
      for (int i = 0; i < NV_K; ++i) {
        int row, k;
        coords(i, row, k);
        *reinterpret_cast<u32x4*>(lds + idx(row, k)) = r[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NV_T; ++i) {
        const int pc = i * NTHR + tid;
        const int kr = (pc % (BK / TKR)) * TKR;
        const int mc = (pc / (BK / TKR)) * VEC;
        const u32x4* in = &r[i * TKR];
        if constexpr (sizeof(T) == 4) {
          // 4x4 floats: column c of the 4 k-rows becomes one 16-byte LDS row piece
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x4 o = {in[0][c], in[1][c], in[2][c], in[3][c]};
            *reinterpret_cast<u32x4*>(lds + (mc + c) * LD + kr) = o;
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
            *reinterpret_cast<u32x2*>(lds + (mc + c) * LD + kr) = o;
          }
        }
      }
    }
  }
};

template <typename T, int BM_, int BN_, bool AKC, bool BKC> struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  // waves per block, in a WGM x WGN grid over the tile: 2 x (NW/2), except 256 x 192 (4 x 2,
  // 64 x 96 per wave)
  static constexpr bool BIG = sizeof(T) == 2 && BM == 256 && (BN == 256 || BN == 192);
  static constexpr int NW = BIG ? 8 : 4;
  static constexpr int NTHR = 64 * NW, WGM = BN == 192 ? 4 : 2, WGN = NW / WGM;
  static constexpr int TM = BM / WGM, TN = BN / WGN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  // k per LDS stage: 64 for bf16 (direct copies, 4 k-steps of MFMAs per wave between barriers),
  // 32 for fp32 (register staging)
  static constexpr int BK = sizeof(T) == 2 ? 64 : 32;
  using OA = Operand<T, AKC, BM, BK, NTHR>;
  using OB = Operand<T, BKC, BN, BK, NTHR>;
  static constexpr int STAGE = OA::ELEMS + OB::ELEMS;  // elements per LDS stage
  static constexpr int NS = 2;  // LDS stages
  static constexpr int EPI_LD = TN + 4;                 // epilogue staging pitch (floats)
  static constexpr size_t OPS_BYTES = (size_t)NS * STAGE * sizeof(T);
  static constexpr size_t EPI_BYTES = (size_t)NW * 32 * EPI_LD * 4;
  static constexpr size_t LDS_BYTES = OPS_BYTES > EPI_BYTES ? OPS_BYTES : EPI_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Per 8-column chunk, the epilogue inputs besides the accumulators: the residual / GELU input
// (aux) or, for fp32 accumulation, the old C. They are fetched for a whole slab before any of
// its results is stored, so the loads are in flight together.
template <typename T, int EPI> struct EpiX {
  static constexpr bool AUX = EPI == EPI_RESID || EPI == EPI_GELU_BWD || EPI == EPI_MUL;
  static constexpr bool USED = AUX || EPI == EPI_F32;
  static constexpr int NW = EPI == EPI_F32 ? 2 : 8 / Elt<T>::VEC;  // 16-byte words per chunk
  u32x4 w[NW];
};

template <typename T, int EPI>
__device__ __forceinline__ void epi_fetch8(const GemmArgs& p, const float* C_f32, long ldc, int row, int col,
                                           EpiX<T, EPI>& x) {
  const bool full = col + 8 <= p.N;
  if constexpr (EPI == EPI_F32) {
    if (!p.accumulate) return;
    const float* src = C_f32 + (size_t)row * ldc + col;
    if (full) {
      x.w[0] = reinterpret_cast<const u32x4*>(src)[0];
      x.w[1] = reinterpret_cast<const u32x4*>(src)[1];
    } else {
      V16<float> t[2];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e / 4].v[e % 4] = col + e < p.N ? src[e] : 0.f;
      x.w[0] = t[0].pack();
      x.w[1] = t[1].pack();
    }
  } else if constexpr (EpiX<T, EPI>::AUX) {
    constexpr int VEC = Elt<T>::VEC;
    const T* src = reinterpret_cast<const T*>(p.aux) + (size_t)row * p.ldaux + col;
    if (full) {
#pragma unroll
      for (int h = 0; h < 8 / VEC; ++h) x.w[h] = reinterpret_cast<const u32x4*>(src)[h];
    } else {
#pragma unroll
      for (int h = 0; h < 8 / VEC; ++h) {
        V16<T> t;
#pragma unroll
        for (int e = 0; e < VEC; ++e) t.v[e] = col + h * VEC + e < p.N ? ld1(src, h * VEC + e) : 0.f;
        x.w[h] = t.pack();
      }
    }
  }
}

// Apply the epilogue to 8 consecutive columns of one row and store them (16-byte vectors when
// the chunk is whole, element by element at the right edge). bv: bias of the 8 columns.
template <typename T, int EPI>
__device__ __forceinline__ void epi_store8(const GemmArgs& p, float* C_f32, long ldc, int row, int col,
                                           const float (&a)[8], const float (&bv)[8], const EpiX<T, EPI>& x,
                                           bool csum, float (&cs)[8]) {
  const bool full = col + 8 <= p.N;
  if constexpr (EPI == EPI_F32) {
    float* dst = C_f32 + (size_t)row * ldc + col;
    V16<float> v[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e / 4].v[e % 4] = a[e];
    if (p.accumulate) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        V16<float> o;
        o.unpack(x.w[h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[h].v[e] += o.v[e];
      }
    }
    if (full) {
      v[0].store(dst);
      v[1].store(dst + 4);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < p.N) dst[e] = v[e / 4].v[e % 4];
    }
  } else {
    constexpr int VEC = Elt<T>::VEC;
    float xv[8], o[8], o2[8];
    if constexpr (EpiX<T, EPI>::AUX) {
#pragma unroll
      for (int h = 0; h < 8 / VEC; ++h) {
        V16<T> t;
        t.unpack(x.w[h]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) xv[h * VEC + e] = t.v[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (EPI == EPI_BIAS) o[e] = a[e] + bv[e];
      else if constexpr (EPI == EPI_GELU) {
        o[e] = a[e] + bv[e];
        o2[e] = gelu_fwd(o[e]);
      } else if constexpr (EPI == EPI_GELU_GRAD) gelu_both(a[e] + bv[e], o2[e], o[e]);
      else if constexpr (EPI == EPI_RESID) o[e] = xv[e] + (a[e] + bv[e]);
      else if constexpr (EPI == EPI_MUL) o[e] = a[e] * xv[e];
      else o[e] = a[e] * gelu_bwd(xv[e]);
    }
    if (csum) {  // column sums of the values as stored
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < p.N) cs[e] += sizeof(T) == 2 ? bf2f(f2bf(o[e])) : o[e];
    }
    T* dst = reinterpret_cast<T*>(p.C) + (size_t)row * ldc + col;
    if (full) {
#pragma unroll
      for (int h = 0; h < 8 / VEC; ++h) {
        V16<T> t;
#pragma unroll
        for (int e = 0; e < VEC; ++e) t.v[e] = o[h * VEC + e];
        t.store(dst + h * VEC);
      }
      if constexpr (EPI == EPI_GELU || EPI == EPI_GELU_GRAD) {
        T* dst2 = reinterpret_cast<T*>(p.C2) + (size_t)row * ldc + col;
#pragma unroll
        for (int h = 0; h < 8 / VEC; ++h) {
          V16<T> t;
#pragma unroll
          for (int e = 0; e < VEC; ++e) t.v[e] = o2[h * VEC + e];
          t.store(dst2 + h * VEC);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (col + e < p.N) {
          st1(dst, e, o[e]);
          if constexpr (EPI == EPI_GELU || EPI == EPI_GELU_GRAD)
            st1(reinterpret_cast<T*>(p.C2) + (size_t)row * ldc + col, e, o2[e]);
        }
      }
    }
  }
}

// The K loop of one block. DIRECT: every tile of both operands is interior and K-contiguous and
// is copied global -> LDS directly, NS - 1 tiles ahead through NS LDS stages (one barrier per
// tile). Otherwise the tiles go through registers.
template <typename T, int BM, int BN, bool AKC, bool BKC, bool DIRECT>
__device__ __forceinline__ void gemm_mainloop(const GemmArgs& p, int m0, int n0, int kbeg, int kend, T* st0,
                                              f32x16 (&acc)[Cfg<T, BM, BN, AKC, BKC>::FM][Cfg<T, BM, BN, AKC, BKC>::FN]) {
  using CF = Cfg<T, BM, BN, AKC, BKC>;
  using MM = Mma<T>;
  using OA = typename CF::OA;
  using OB = typename CF::OB;
  constexpr int BK = CF::BK, TM = CF::TM, TN = CF::TN, FM = CF::FM, FN = CF::FN;
  auto Abuf = [&](int stg) { return st0 + stg * CF::STAGE; };
  auto Bbuf = [&](int stg) { return st0 + stg * CF::STAGE + OA::ELEMS; };
  const T* A = reinterpret_cast<const T*>(p.A);
  const T* B = reinterpret_cast<const T*>(p.B);
  const int nkt = cdiv(kend - kbeg, BK);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w / CF::WGN, wn = w % CF::WGN;

  const int arow = wm * TM + (lane & 31);
  const int brow = wn * TN + (lane & 31);
  const int kofs = (lane >> 5) * MM::KPL;
  int atr = 0, btr = 0;
  if constexpr (OA::MODE == 2) atr = OA::tr_lane_off(wm * TM, lane);
  if constexpr (OB::MODE == 2) btr = OB::tr_lane_off(wn * TN, lane);
  // operand fragments of 32-row block i at k-step st
  auto fragA = [&](const T* as, int i, int st) {
    if constexpr (OA::MODE == 2) return OA::tr_frag(as, atr, i, st);
    else return MM::load(as + OA::idx(arow + i * 32, st * MM::KSTEP + kofs));
  };
  auto fragB = [&](const T* bs, int j, int st) {
    if constexpr (OB::MODE == 2) return OB::tr_frag(bs, btr, j, st);
    else return MM::load(bs + OB::idx(brow + j * 32, st * MM::KSTEP + kofs));
  };
  // all MFMAs of one staged tile; operand fragments are double-buffered: the LDS reads of k-step
  // s+1 are issued before the MFMAs of k-step s, so their latency hides behind FM*FN MFMAs
  auto compute = [&](const T* as, const T* bs) {
    constexpr int KS = BK / MM::KSTEP;
    typename MM::frag fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = fragA(as, i, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = fragB(bs, j, 0);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const int cb = st & 1, nb = cb ^ 1;
      if (st + 1 < KS) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[nb][i] = fragA(as, i, st + 1);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[nb][j] = fragB(bs, j, st + 1);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = MM::mma(fa[cb][i], fb[cb][j], acc[i][j]);
    }
    {
      // issue order: the reads of step 0, then within each step one read of the next step after
      // each MFMA (the rest at the end), so no MFMA waits for a read issued in its own step
      constexpr int NR = FM * (OA::MODE == 2 ? 2 : 1) + FN * (OB::MODE == 2 ? 2 : 1);
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
      for (int st = 0; st + 1 < KS; ++st) {
#pragma unroll
        for (int r = 0; r < NR && r < FM * FN; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NR > FM * FN) __builtin_amdgcn_sched_group_barrier(0x100, NR - FM * FN, 0);
        if (FM * FN > NR) __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - NR, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
    }
  };

  if constexpr (DIRECT) {
    constexpr int NS = CF::NS;
    static_assert(NS >= 2, "stages");
    // copies in flight per wave while tile kt is consumed: those of tiles kt+1 .. kt+NS-2
    constexpr int WAIT_N = (NS - 2) * (OA::NDIRECT + OB::NDIRECT);
    static_assert(WAIT_N < 64, "vmcnt range");
    constexpr int WAIT_IMM = (WAIT_N & 15) | (7 << 4) | (15 << 8) | ((WAIT_N >> 4) << 14);
    auto issue = [&](int t) {
      OA::issue_direct(A, p.lda, m0, kbeg + t * BK, Abuf(t % NS));
      OB::issue_direct(B, p.ldb, n0, kbeg + t * BK, Bbuf(t % NS));
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < nkt) issue(t);
    for (int kt = 0; kt < nkt; ++kt) {
      // loads return in order: this wave's copies of tile kt have landed once at most WAIT_N remain
      if (kt + NS - 2 < nkt) __builtin_amdgcn_s_waitcnt(WAIT_IMM);
      else __builtin_amdgcn_s_waitcnt(0);
      // Every wave's copies of tile kt have landed and every wave is done with stage (kt-1) % NS
      // (its fragments fed MFMAs already issued). A bare s_barrier: a workgroup fence here would
      // make the compiler wait for all copies in flight.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // the copies into one stage and the fragment reads of another go through distinct restrict
      // pointers, so the compiler's wait analysis can tell them apart
      auto body = [&](const T* __restrict__ ra, const T* __restrict__ rb, T* __restrict__ da, T* __restrict__ db,
                      int t) {
        if (t < nkt) {
          OA::issue_direct(A, p.lda, m0, kbeg + t * BK, da);
          OB::issue_direct(B, p.ldb, n0, kbeg + t * BK, db);
        }
        compute(ra, rb);
      };
      const int tn = kt + NS - 1;
      body(Abuf(kt % NS), Bbuf(kt % NS), Abuf(tn % NS), Bbuf(tn % NS), tn);

    }
    __syncthreads();  // the epilogue reuses the LDS
  } else {
    OA la;
    OB lb;
    if (nkt > 0) {
      la.load(A, p.lda, m0, p.M, kbeg, kend);
      lb.load(B, p.ldb, n0, p.N, kbeg, kend);
      la.store(Abuf(0), m0, p.M, kbeg, kend);
      lb.store(Bbuf(0), n0, p.N, kbeg, kend);
    }
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nkt;
      if (more) {
        la.load(A, p.lda, m0, p.M, kbeg + (kt + 1) * BK, kend);
        lb.load(B, p.ldb, n0, p.N, kbeg + (kt + 1) * BK, kend);
      }
      compute(Abuf(cur), Bbuf(cur));

      if (more) {
        la.store(Abuf(cur ^ 1), m0, p.M, kbeg + (kt + 1) * BK, kend);
        lb.store(Bbuf(cur ^ 1), n0, p.N, kbeg + (kt + 1) * BK, kend);
      }
      __syncthreads();
    }
  }
}

// 32 zero bytes in global memory: the stand-in source of the bias prefetch when there is no bias
static __device__ __attribute__((aligned(16))) uint32_t g_zero_chunk[8];

template <typename T, int BM, int BN, bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__((Cfg<T, BM, BN, AKC, BKC>::NTHR)) void gemm_kernel(GemmArgs p0, int k_split,
                                                                               float* split_out0, GemmArgs p1,
                                                                               float* split_out1, int nblk0) {
  using CF = Cfg<T, BM, BN, AKC, BKC>;
  constexpr int BK = CF::BK, TM = CF::TM, TN = CF::TN, FM = CF::FM, FN = CF::FN;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* const st0 = reinterpret_cast<T*>(smem);

  // Block -> (problem, split, tile). The 1-D grid holds splits x tiles blocks of problem 0, then
  // (grouped weight gradients) those of problem 1, padded to a multiple of 8; blocks are dealt
  // round-robin to the 8 XCDs, so block L is renumbered to give each XCD a contiguous run of
  // (split, tile) pairs (tiles of one split that share operand rows or columns then share an L2);
  // padding blocks exit. Inside a split, tiles go in groups of GROUP_M tile-rows.
  int bb = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const bool second = bb >= nblk0;
  const GemmArgs p = second ? p1 : p0;
  float* const split_out = second ? split_out1 : split_out0;
  if (second) bb -= nblk0;
  const int tiles_m = cdiv(p.M, BM), tiles_n = cdiv(p.N, BN);
  const int ntiles = tiles_m * tiles_n;
  const int nsplit = cdiv(p.K, k_split);
  if (bb >= ntiles * nsplit) return;
  const int zs = bb / ntiles, b = bb % ntiles;
  const int group = GROUP_M * tiles_n;
  const int first_m = (b / group) * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (b % group) % gsz;
  const int tn = (b % group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = zs * k_split;
  const int kend = min(p.K, kbeg + k_split);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w / CF::WGN, wn = w % CF::WGN;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // The epilogue's 8-column chunks of this lane: chunk it * 64 + lane of a 32-row slab is row
  // (it * 64 + lane) / CPR, column chunk % CPR; a lane's column chunk repeats every BP chunks
  // (1 when CPR divides 64).
  constexpr int CPR = TN / 8;
  constexpr int BP = CPR / gcd_c(64, CPR);
  auto ccol = [&](int it) { return ((it * 64 + lane) % CPR) * 8; };
  // The bias of those chunks is requested before the main loop (whose first wait covers it) from an
  // unguarded address, since a load behind a branch is waited for at the branch join; without a
  // bias, or with N not a whole number of chunks, the loads read a zero chunk instead.
  constexpr bool BIAS_EPI = EPI == EPI_BIAS || EPI == EPI_GELU || EPI == EPI_RESID || EPI == EPI_GELU_GRAD;
  constexpr int BVEC = Elt<T>::VEC;
  const bool bias_pf = BIAS_EPI && p.bias != nullptr && p.N % 8 == 0;
  u32x4 braw[BP][8 / BVEC];
  if constexpr (BIAS_EPI) {
#pragma unroll
    for (int bp = 0; bp < BP; ++bp) {
      const int col = min(n0 + wn * TN + ccol(bp), p.N - 8);
      const T* src = bias_pf ? reinterpret_cast<const T*>(p.bias) + col : reinterpret_cast<const T*>(g_zero_chunk);
#pragma unroll
      for (int h = 0; h < 8 / BVEC; ++h) braw[bp][h] = *reinterpret_cast<const u32x4*>(src + h * BVEC);
    }
  }

  const bool kfull = (kend - kbeg) % BK == 0;
  if constexpr (CF::OA::DIRECT && CF::OB::DIRECT) {
    if (kfull && m0 + BM <= p.M && n0 + BN <= p.N)
      gemm_mainloop<T, BM, BN, AKC, BKC, true>(p, m0, n0, kbeg, kend, st0, acc);
    else
      gemm_mainloop<T, BM, BN, AKC, BKC, false>(p, m0, n0, kbeg, kend, st0, acc);
  } else {
    gemm_mainloop<T, BM, BN, AKC, BKC, false>(p, m0, n0, kbeg, kend, st0, acc);
  }

  // ---- epilogue: 32-row slabs of each wave go through LDS, then 16-byte row chunks out
  float* C_f32 = reinterpret_cast<float*>(p.C);
  long ldc = p.ldc;
  GemmArgs q = p;
  if constexpr (EPI == EPI_F32) {
    if (split_out) {
      C_f32 = split_out + (size_t)zs * p.M * p.N;
      ldc = p.N;
      q.accumulate = 0;
    }
  }
  // column sums of the output (non-fp32 epilogues): split_out then holds the partial sums, one row
  // per (tile row, wave row); a lane's column chunk must be the same for all of its rows
  constexpr bool CSUM_OK = EPI != EPI_F32 && 64 % (TN / 8) == 0;
  const bool csum = CSUM_OK && split_out != nullptr;
  float cs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = 0.f;
  float* stage = reinterpret_cast<float*>(smem) + w * 32 * CF::EPI_LD;
  const int g = lane >> 5, l32 = lane & 31;
  constexpr int NIT = (32 * CPR) / 64;    // chunks per lane per slab (CPR: chunks per staged row)
  static_assert((32 * CPR) % 64 == 0, "whole chunks per lane");
  float bv[BP][8];
#pragma unroll
  for (int bp = 0; bp < BP; ++bp) {
#pragma unroll
    for (int e = 0; e < 8; ++e) bv[bp][e] = 0.f;
    if constexpr (BIAS_EPI) {
      if (bias_pf) {
#pragma unroll
        for (int h = 0; h < 8 / BVEC; ++h) {
          V16<T> t;
          t.unpack(braw[bp][h]);
#pragma unroll
          for (int e = 0; e < BVEC; ++e) bv[bp][h * BVEC + e] = t.v[e];
        }
      } else if (p.bias) {  // N not a whole number of chunks: element loads
        const int col = n0 + wn * TN + ccol(bp);
        const T* bias = reinterpret_cast<const T*>(p.bias) + col;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < p.N) bv[bp][e] = ld1(bias, e);
      }
    }
  }
  // the staging area is private to the wave: wave-level ordering is enough
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // residual / derivative inputs of all slabs are fetched up front (one memory round trip);
  // the old C of fp32 accumulation (twice the registers) is fetched slab by slab
  constexpr bool ALL_AT_ONCE = EpiX<T, EPI>::AUX;
  constexpr int NXS = ALL_AT_ONCE ? FM : 1;
  EpiX<T, EPI> xs[NXS][NIT];
  auto fetch_slab = [&](int i, EpiX<T, EPI>(&xo)[NIT]) {
    const int row0 = m0 + wm * TM + i * 32;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int row = row0 + (it * 64 + lane) / CPR;
      const int col = n0 + wn * TN + ccol(it);
      if (row < p.M && col < p.N) epi_fetch8<T, EPI>(q, C_f32, ldc, row, col, xo[it]);
    }
  };
  if constexpr (ALL_AT_ONCE) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fetch_slab(i, xs[i]);
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row0 = m0 + wm * TM + i * 32;
    if constexpr (EpiX<T, EPI>::USED && !ALL_AT_ONCE) fetch_slab(i, xs[0]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[((r >> 2) * 8 + g * 4 + (r & 3)) * CF::EPI_LD + j * 32 + l32] = acc[i][j][r];
    wave_sync();
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rr = (it * 64 + lane) / CPR;
      const int row = row0 + rr;
      const int cc = ccol(it), col = n0 + wn * TN + cc;
      if (row < p.M && col < p.N) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(stage + rr * CF::EPI_LD + cc);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(stage + rr * CF::EPI_LD + cc + 4);
        const float a8[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        epi_store8<T, EPI>(q, C_f32, ldc, row, col, a8, bv[it % BP], xs[ALL_AT_ONCE ? i : 0][it], csum, cs);
      }
    }
    wave_sync();
  }
  if constexpr (CSUM_OK) {
    if (csum) {
      // lanes l, l + CPR, l + 2 CPR, ... hold the same columns: fixed-order butterfly over them
#pragma unroll
      for (int msk = CPR; msk < 64; msk <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] += __shfl_xor(cs[e], msk);
      const int col = n0 + wn * TN + ccol(0);
      if (lane < CPR && col < p.N) {
        float* dst = split_out + (size_t)(tm * CF::WGM + wm) * p.N + col;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < p.N) dst[e] = cs[e];
      }
    }
  }
}

// dst[i] (+)= sum_z part[z][i], z in order
__device__ __forceinline__ void splitk_reduce_seg(const float* __restrict__ part, int splits, size_t n,
                                                  float* __restrict__ dst, int accumulate, size_t first,
                                                  size_t stride) {
  const size_t n4 = n / 4;
  // straight-line loads, 8 splits at a time (split indices past the last read the last one, and
  // without accumulation the old value is read from the first partial instead of dst: both are
  // dropped by a select after the loads), so that they are all in flight together: a load in a
  // loop of unknown count, or under a guard, is waited for before the next is issued
  const float* base0 = accumulate ? dst : part;
  for (size_t i = first; i < n4; i += stride) {
    const f32x4 d0 = reinterpret_cast<const f32x4*>(base0)[i];
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = reinterpret_cast<const f32x4*>(part + (size_t)min(u, splits - 1) * n)[i];
    f32x4 s = accumulate ? d0 : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < splits) s += v[u];
    for (int z0 = 8; z0 < splits; z0 += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = reinterpret_cast<const f32x4*>(part + (size_t)min(z0 + u, splits - 1) * n)[i];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < splits) s += v[u];
    }
    reinterpret_cast<f32x4*>(dst)[i] = s;
  }
  for (size_t i = n4 * 4 + first; i < n; i += stride) {
    float s = accumulate ? dst[i] : 0.f;
    for (int z = 0; z < splits; ++z) s += part[(size_t)z * n + i];
    dst[i] = s;
  }
}
// one or two products' partials (n1 = 0: one)
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ part0, size_t n0,
                                                     float* __restrict__ dst0, const float* __restrict__ part1,
                                                     size_t n1, float* __restrict__ dst1, int splits,
                                                     int accumulate0, int accumulate1) {
  const size_t first = blockIdx.x * 256ull + threadIdx.x, stride = (size_t)gridDim.x * 256;
  splitk_reduce_seg(part0, splits, n0, dst0, accumulate0, first, stride);
  if (n1) splitk_reduce_seg(part1, splits, n1, dst1, accumulate1, first, stride);
}
static int splitk_reduce_blocks(size_t n) { return (int)std::min<size_t>(4096, (n / 4 + 255) / 256 + 1); }

// ----------------------------------------------------------------------------------------
// Column sums (bias gradients): partial[y][n] over a chunk of rows, 16-byte loads, then a
// fixed-order sum over the chunks. Block: 32 column vectors x 8 row groups.
// ----------------------------------------------------------------------------------------
constexpr int CS_ROWS = 128;  // rows per partial

template <typename T>
__global__ __launch_bounds__(256) void colsum_partial(const T* __restrict__ x, long ld, int M, int N,
                                                      float* __restrict__ partial) {
  constexpr int VEC = Elt<T>::VEC;
  __shared__ float sh[8][32 * VEC + 1];
  const int cv = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int col = (blockIdx.x * 32 + cv) * VEC;
  const int r0 = blockIdx.y * CS_ROWS;
  float s[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = 0.f;
  if (col < N) {
    const int r1 = min(M, r0 + CS_ROWS);
#pragma unroll 4
    for (int r = r0 + rg; r < r1; r += 8) {
      V16<T> v;
      v.load(x + (size_t)r * ld + col);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[e] += v.v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) sh[rg][cv * VEC + e] = s[e];
  __syncthreads();
  for (int c = threadIdx.x; c < 32 * VEC; c += 256) {
    const int gc = blockIdx.x * 32 * VEC + c;
    if (gc < N) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) t += sh[i][c];
      partial[(size_t)blockIdx.y * N + gc] = t;
    }
  }
}

__global__ __launch_bounds__(RP_THREADS) void colsum_finish(const float* __restrict__ partial, int ny, int N,
                                                     float* __restrict__ out, int accumulate) {
  reduce_partials_block(partial, ny, N, N, out, accumulate, blockIdx.x);
}

hipError_t launch_colsum_finish(const float* partial, int ny, int N, float* out, int accumulate, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  colsum_finish<<<cdiv(N, 32), RP_THREADS, 0, s>>>(partial, ny, N, out, accumulate);
  return hipGetLastError();
}

int gemm_colsum_rows_max(int M) { return std::max(cdiv(M, 128) * 2, cdiv(M, 256) * 4); }

// The second stages of many column sums in one launch: block b takes FinishBlock b.
__global__ __launch_bounds__(RP_THREADS) void finish_batch(const FinishBlock* __restrict__ blocks, int accumulate) {
  const FinishBlock f = blocks[blockIdx.x];
  reduce_partials_block(f.part, f.ny, f.ld, f.ncols, f.out, accumulate, f.chunk);
}

hipError_t launch_finish_batch(const FinishBlock* blocks, int nblocks, int accumulate, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  finish_batch<<<nblocks, RP_THREADS, 0, s>>>(blocks, accumulate);
  return hipGetLastError();
}

hipError_t launch_colsum(DType dt, const void* dY, long ld, int M, int N, float* db, int accumulate,
                         float* partial, size_t partial_floats, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int ny = std::max(1, cdiv(M, CS_ROWS));
  if ((size_t)ny * N > partial_floats) return hipErrorInvalidValue;
  const int vec = dt == DT_BF16 ? 8 : 4;
  if (N % vec || ld % vec) return hipErrorInvalidValue;
  dim3 grid(cdiv(N / vec, 32), ny);
  if (M > 0) {
    if (dt == DT_BF16)
      colsum_partial<bf16><<<grid, 256, 0, s>>>(reinterpret_cast<const bf16*>(dY), ld, M, N, partial);
    else
      colsum_partial<float><<<grid, 256, 0, s>>>(reinterpret_cast<const float*>(dY), ld, M, N, partial);
  }
  colsum_finish<<<cdiv(N, 32), RP_THREADS, 0, s>>>(partial, M > 0 ? ny : 0, N, db, accumulate);
  return hipGetLastError();
}


constexpr int NCU = 256;

// The 256x256 tile (8 waves) wins once the grid fills at least half of the CUs for the
// K-contiguous products (direct copies); with a row-contiguous operand the 128x128 tile (several
// blocks per CU) stays ahead until about 1.5 rounds of the CUs.
static bool use_big(DType dt, bool kc_both, int M, int N) {
  if (dt != DT_BF16) return false;
  const long t = (long)cdiv(M, 256) * cdiv(N, 256);
  return t >= (kc_both ? 128 : 384);
}

// Split-K factor for the fp32 weight-gradient products. The blocks run in ceil(tiles s / NCU)
// rounds of K / s each, and every split adds an fp32 partial of M x N that is written and read
// back once; pick the s that minimises that time (K per split >= 512, partials within scratch).
static int splits_for(long tiles, long mn, int K, size_t scratch_floats, int tile) {
  // per-CU MFMA rate and HBM rate as seen by these kernels (order of magnitude is enough)
  const double cu_flops = 1.8e12, hbm = 5.0e12;
  const double tile_flops_per_k = 2.0 * tile * tile;
  int best = 1;
  double best_t = 1e30;
  for (int s = 1; s <= 32; ++s) {
    if (s > 1 && ((long)K / s < 512 || (size_t)s * mn > scratch_floats)) break;
    const double rounds = (double)((tiles * s + NCU - 1) / NCU);
    const double t = rounds * tile_flops_per_k * ((double)K / s) / cu_flops + (s > 1 ? s * 8.0 * mn / hbm : 0.0);
    if (t < best_t * 0.995) {
      best_t = t;
      best = s;
    }
  }
  return best;
}
int gemm_splits_t(int M, int N, int K, size_t scratch_floats, int tile) {
  return splits_for((long)cdiv(M, tile) * cdiv(N, tile), (long)M * N, K, scratch_floats, tile);
}
int gemm_splits(int M, int N, int K, size_t scratch_floats) { return gemm_splits_t(M, N, K, scratch_floats, 128); }

template <typename T, int BM, int BN, bool AKC, bool BKC, int EPI>
static void launch_cfg(dim3 grid, const GemmArgs& a, int k_split, float* split, hipStream_t s) {
  using CF = Cfg<T, BM, BN, AKC, BKC>;
  static bool attr = false;
  auto kern = gemm_kernel<T, BM, BN, AKC, BKC, EPI>;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)CF::LDS_BYTES);
    attr = true;
  }
  kern<<<grid, CF::NTHR, CF::LDS_BYTES, s>>>(a, k_split, split, a, nullptr, INT_MAX);
}

template <typename T, int BM, int BN, bool AKC, bool BKC>
static hipError_t launch_t(Epi epi, const GemmArgs& a, float* scratch, size_t scratch_floats, hipStream_t s) {
  const int tiles = cdiv(a.M, BM) * cdiv(a.N, BN);
  int splits = 1;
  if (epi == EPI_F32 && scratch) splits = gemm_splits_t(a.M, a.N, a.K, scratch_floats, BM);
  int k_split = a.K;
  if (splits > 1) {
    constexpr int BK = Cfg<T, BM, BN, AKC, BKC>::BK;
    k_split = cdiv(cdiv(a.K, splits), BK) * BK;
    splits = cdiv(a.K, k_split);
  }
  dim3 grid(((long)tiles * splits + 7) & ~7L);
  // column sums fused into the epilogue when a lane keeps one column chunk (and the partials fit);
  // otherwise a separate pass over the stored C
  using CF = Cfg<T, BM, BN, AKC, BKC>;
  const int cs_rows = cdiv(a.M, BM) * CF::WGM;
  const bool cs_ok = epi != EPI_F32 && a.colsum && 64 % (CF::TN / 8) == 0;
  // partials left for a batched finish when the caller offers room for them
  ColsumDefer* dfr = a.colsum_defer;
  if (dfr) dfr->rows = 0;
  const bool cs_defer = cs_ok && dfr && (size_t)cs_rows * a.N <= dfr->cap;
  const bool cs_fused = cs_ok && (cs_defer || (scratch && (size_t)cs_rows * a.N <= scratch_floats));
  float* csp = cs_defer ? dfr->part : cs_fused ? scratch : nullptr;
  switch (epi) {
    case EPI_BIAS: launch_cfg<T, BM, BN, AKC, BKC, EPI_BIAS>(grid, a, k_split, csp, s); break;
    case EPI_GELU: launch_cfg<T, BM, BN, AKC, BKC, EPI_GELU>(grid, a, k_split, csp, s); break;
    case EPI_RESID: launch_cfg<T, BM, BN, AKC, BKC, EPI_RESID>(grid, a, k_split, csp, s); break;
    case EPI_GELU_BWD: launch_cfg<T, BM, BN, AKC, BKC, EPI_GELU_BWD>(grid, a, k_split, csp, s); break;
    case EPI_GELU_GRAD: launch_cfg<T, BM, BN, AKC, BKC, EPI_GELU_GRAD>(grid, a, k_split, csp, s); break;
    case EPI_MUL: launch_cfg<T, BM, BN, AKC, BKC, EPI_MUL>(grid, a, k_split, csp, s); break;
    case EPI_F32:
      launch_cfg<T, BM, BN, AKC, BKC, EPI_F32>(grid, a, k_split, splits > 1 ? scratch : nullptr, s);
      if (splits > 1) {
        const size_t n = (size_t)a.M * a.N;
        splitk_reduce<<<splitk_reduce_blocks(n), 256, 0, s>>>(scratch, n, reinterpret_cast<float*>(a.C), nullptr, 0,
                                                              nullptr, splits, a.accumulate, 0);
      }
      break;
  }
  if (cs_defer) {
    dfr->rows = cs_rows;
  } else if (epi != EPI_F32 && a.colsum) {
    if (cs_fused)
      colsum_finish<<<cdiv(a.N, 32), RP_THREADS, 0, s>>>(scratch, cs_rows, a.N, a.colsum, a.colsum_accumulate);
    else
      return launch_colsum(sizeof(T) == 2 ? DT_BF16 : DT_F32, a.C, a.ldc, a.M, a.N, a.colsum, a.colsum_accumulate,
                           scratch, scratch_floats, s);
  }
  return hipGetLastError();
}

// Fraction of the CU slots busy over the rounds a grid of this many single-block-per-CU tiles takes.
static double round_fill(long tiles) { return (double)tiles / (double)(cdiv((int)tiles, NCU) * NCU); }

template <typename T, bool AKC, bool BKC>
static hipError_t launch_sel(Epi epi, const GemmArgs& a, float* scratch, size_t sf, hipStream_t s) {
  // split-K weight gradients (their M x N is small): 256 x 256 tiles unless there are fewer than
  // 16 of them (C x C), where the 128 x 128 tile's smaller partials win
  if (epi == EPI_F32 && scratch && sizeof(T) == 2 && (long)cdiv(a.M, 256) * cdiv(a.N, 256) >= 16)
    return launch_t<T, 256, 256, AKC, BKC>(epi, a, scratch, sf, s);
  if (epi != EPI_F32 && use_big(sizeof(T) == 2 ? DT_BF16 : DT_F32, AKC && BKC, a.M, a.N)) {
    // K-contiguous products whose 256-wide column tiles leave CUs idle in the last round
    // (N = 768: 192 tiles per 16384 rows) take 192-wide column tiles when those fill the rounds
    // clearly better
    if constexpr (AKC && BKC && sizeof(T) == 2) {
      const long t256 = (long)cdiv(a.M, 256) * cdiv(a.N, 256), t192 = (long)cdiv(a.M, 256) * cdiv(a.N, 192);
      if (round_fill(t192) > round_fill(t256) + 0.05) return launch_t<T, 256, 192, AKC, BKC>(epi, a, scratch, sf, s);
    }
    return launch_t<T, 256, 256, AKC, BKC>(epi, a, scratch, sf, s);
  }
  if (epi == EPI_F32 && use_big(sizeof(T) == 2 ? DT_BF16 : DT_F32, AKC && BKC, a.M, a.N))
    return launch_t<T, 256, 256, AKC, BKC>(epi, a, nullptr, 0, s);
  return launch_t<T, 128, 128, AKC, BKC>(epi, a, scratch, sf, s);
}

hipError_t launch_gemm(DType dt, bool a_kc, bool b_kc, Epi epi, const GemmArgs& a, float* scratch,
                       size_t scratch_floats, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (epi == EPI_F32 && scratch && a.ldc != a.N) scratch = nullptr;
  if (dt == DT_BF16) {
    if (a_kc && b_kc) return launch_sel<bf16, true, true>(epi, a, scratch, scratch_floats, s);
    if (a_kc && !b_kc) return launch_sel<bf16, true, false>(epi, a, scratch, scratch_floats, s);
    if (!a_kc && !b_kc) return launch_sel<bf16, false, false>(epi, a, scratch, scratch_floats, s);
    return launch_sel<bf16, false, true>(epi, a, scratch, scratch_floats, s);
  }
  if (a_kc && b_kc) return launch_t<float, 128, 128, true, true>(epi, a, scratch, scratch_floats, s);
  if (a_kc && !b_kc) return launch_t<float, 128, 128, true, false>(epi, a, scratch, scratch_floats, s);
  if (!a_kc && !b_kc) return launch_t<float, 128, 128, false, false>(epi, a, scratch, scratch_floats, s);
  return launch_t<float, 128, 128, false, true>(epi, a, scratch, scratch_floats, s);
}

// Two fp32-output (weight-gradient) products with the same K and operand layouts in one split-K
// launch of 256 x 256 tiles: the splits are chosen for the tiles of both, so two small products
// fill the CUs with fewer, larger partials than each would alone; then one reduction for both.
template <bool AKC, bool BKC>
static hipError_t launch_pair_t(const GemmArgs& a0, const GemmArgs& a1, float* scratch, size_t sf, hipStream_t s) {
  using CF = Cfg<bf16, 256, 256, AKC, BKC>;
  const long t0 = (long)cdiv(a0.M, 256) * cdiv(a0.N, 256), t1 = (long)cdiv(a1.M, 256) * cdiv(a1.N, 256);
  const size_t n0 = (size_t)a0.M * a0.N, n1 = (size_t)a1.M * a1.N;
  int splits = splits_for(t0 + t1, (long)(n0 + n1), a0.K, sf, 256);
  int k_split = a0.K;
  if (splits > 1) {
    k_split = cdiv(cdiv(a0.K, splits), CF::BK) * CF::BK;
    splits = cdiv(a0.K, k_split);
  }
  float* part0 = splits > 1 ? scratch : nullptr;
  float* part1 = splits > 1 ? scratch + (size_t)splits * n0 : nullptr;
  const int nblk0 = (int)(t0 * splits);
  dim3 grid(((t0 + t1) * splits + 7) & ~7L);
  static bool attr = false;
  auto kern = gemm_kernel<bf16, 256, 256, AKC, BKC, EPI_F32>;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)CF::LDS_BYTES);
    attr = true;
  }
  kern<<<grid, CF::NTHR, CF::LDS_BYTES, s>>>(a0, k_split, part0, a1, part1, nblk0);
  if (splits > 1)
    splitk_reduce<<<splitk_reduce_blocks(n0 + n1), 256, 0, s>>>(part0, n0, reinterpret_cast<float*>(a0.C), part1, n1,
                                                                 reinterpret_cast<float*>(a1.C), splits,
                                                                 a0.accumulate, a1.accumulate);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Measurement utility (not part of the training step): the GEMM main loop's MFMA work without
// its global traffic. Each 8-wave block copies 64 KiB of operand bits into LDS (two 256-row x
// 64-k bf16 operand tiles, swizzled as the GEMM stores them), then every wave runs `iters`
// rounds of the GEMM's k-loop over them: per round 4 k-steps of 4 + 2 fragment reads and 8
// v_mfma_f32_32x32x16_bf16 (a 128 x 64 wave tile). Timed by the caller, it gives the MFMA rate
// the part sustains for a given kind of operand data (the matrix cores draw more power on
// random bits than on zeros, and the clock follows the power).
__global__ __launch_bounds__(512) void mfma_rate_kernel(const u32x4* __restrict__ operands, int iters,
                                                        float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16 tile[2 * 256 * 64];
  for (int i = threadIdx.x; i < 2 * 256 * 64 / 8; i += 512) reinterpret_cast<u32x4*>(tile)[i] = operands[i];
  __syncthreads();
  using OP = Operand<bf16, true, 256, 64, 512>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int arow = (w >> 2) * 128 + (lane & 31), brow = (w & 3) * 64 + (lane & 31), kofs = (lane >> 5) * 8;
  const bf16* As = tile;
  const bf16* Bs = tile + 256 * 64;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = Mma<bf16>::load(As + OP::idx(arow + 32 * i, st * 16 + kofs));
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = Mma<bf16>::load(Bs + OP::idx(brow + 32 * j, st * 16 + kofs));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = Mma<bf16>::mma(fa[i], fb[j], acc[i][j]);
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  sum = wave_sum(sum);
  __syncthreads();  // the operand tiles are read no more: their first 32 bytes hold the wave sums
  float* ws = reinterpret_cast<float*>(tile);
  if (lane == 0) ws[w] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int i = 0; i < 8; ++i) t += ws[i];
    out[blockIdx.x] = t;
  }
}

hipError_t launch_mfma_rate(const void* operands, float* out, int blocks, int iters, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  mfma_rate_kernel<<<blocks, 512, 0, s>>>(reinterpret_cast<const u32x4*>(operands), iters, out);
  return hipGetLastError();
}

hipError_t launch_gemm_f32_pair(DType dt, bool a_kc, bool b_kc, const GemmArgs& a0, const GemmArgs& a1,
                                float* scratch, size_t scratch_floats, hipStream_t s) {
  const bool ok = dt == DT_BF16 && a0.K == a1.K && a0.M > 0 && a0.N > 0 && a1.M > 0 && a1.N > 0 && a0.K > 0 &&
                  a0.ldc == a0.N && a1.ldc == a1.N && scratch;
  if (!ok) {  // one after the other
    hipError_t e = launch_gemm(dt, a_kc, b_kc, EPI_F32, a0, scratch, scratch_floats, s);
    if (e != hipSuccess) return e;
    return launch_gemm(dt, a_kc, b_kc, EPI_F32, a1, scratch, scratch_floats, s);
  }
  if (a_kc && b_kc) return launch_pair_t<true, true>(a0, a1, scratch, scratch_floats, s);
  if (a_kc && !b_kc) return launch_pair_t<true, false>(a0, a1, scratch, scratch_floats, s);
  if (!a_kc && !b_kc) return launch_pair_t<false, false>(a0, a1, scratch, scratch_floats, s);
  return launch_pair_t<false, true>(a0, a1, scratch, scratch_floats, s);
}

}  // namespace g2
