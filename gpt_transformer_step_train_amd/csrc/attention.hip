// Causal multi-head attention, forward and backward, without materialising T x T.
//
// What is computed: per (batch, head), out = softmax(Q K^T / sqrt(hs)) V over keys u <= t
// (the LLM primer page "从Andrej Karpathy《深入了解ChatGPT之类的大语言模型》入门LLMs" gives
// softmax(QK^T/sqrt(d_k))V; GPT-2 masks the future). The llm.c tour ("Karpathy 的 llm.c：从零理解
// 大模型训练的 C/CUDA 实现", sections 代码解剖 and 性能对比) describes hand-written warp
// reductions for the softmax and an attention fused into two kernels; here the whole forward is
// one kernel with an online softmax (running max and sum), which keeps nothing T x T in HBM, and
// the backward recomputes the probabilities from the saved log-sum-exp.
//
// Layout: qkv [B, T, 3C] with Q | K | V thirds, head h at columns h*hs .. h*hs+hs-1 of each
// third; out [B, T, C]; lse [B, H, T] (natural log). dqkv uses the qkv layout.
//
// Backward (D = rowsum(dO * O)):  P = exp(S - lse);  dV = P^T dO;  dP = dO V^T;
//   dS = P * (dP - D);  dQ = dS K / sqrt(hs);  dK = dS^T Q / sqrt(hs).
// dK, dV are owned by key blocks and dQ by query blocks (two kernels), so no float atomics are
// needed and results are bitwise reproducible.
//
// Two implementations:
//  * bf16, hs = 64: MFMA 32x32x16 kernels. The softmax runs on S^T tiles (keys as MFMA rows,
//    queries as columns) so each lane owns one query: the row max/sum over keys is a register
//    reduction plus one v_permlane32_swap with the other half-wave. The fp32 accumulator of one
//    MFMA is fed, converted to bf16, straight into the next MFMA as an operand; the operand it
//    meets is read from an LDS tile stored transposed, in the same key order.
//  * fp32 (any hs <= 64): one thread per query (forward, dQ) or per key (dK/dV), K/V or Q/dO
//    tiles staged in LDS; exact fp32 math for the fp32 training configurations.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace g2 {

// =====================================================================================
// fp32 reference-precision kernels (vector ALU)
// =====================================================================================
constexpr int AT = 64;  // tile of queries / keys per block

template <int HS>
__global__ __launch_bounds__(AT) void attn_fwd_f32(int T, int H, const float* __restrict__ qkv,
                                                   float* __restrict__ out, float* __restrict__ lse, float scale) {
  __shared__ float Ks[AT][HS + 1], Vs[AT][HS + 1];
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HS, C3 = 3 * C;
  const int q0 = blockIdx.x * AT;
  const int qi = q0 + threadIdx.x;
  const float* base = qkv + (size_t)b * T * C3;
  float q[HS], o[HS];
  for (int d = 0; d < HS; ++d) {
    q[d] = qi < T ? base[(size_t)qi * C3 + h * HS + d] * scale : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kend = min(T, q0 + AT);
  for (int k0 = 0; k0 < kend; k0 += AT) {
    __syncthreads();
    for (int i = threadIdx.x; i < AT * HS; i += AT) {
      const int r = i / HS, d = i % HS;
      const int kr = k0 + r;
      Ks[r][d] = kr < T ? base[(size_t)kr * C3 + C + h * HS + d] : 0.f;
      Vs[r][d] = kr < T ? base[(size_t)kr * C3 + 2 * C + h * HS + d] : 0.f;
    }
    __syncthreads();
    if (qi < T) {
      const int jn = min(AT, qi - k0 + 1);
      for (int j = 0; j < jn; ++j) {
        float s = 0.f;
        for (int d = 0; d < HS; ++d) s += q[d] * Ks[j][d];
        const float mn = fmaxf(m, s);
        const float corr = expf(m - mn);
        const float pj = expf(s - mn);
        l = l * corr + pj;
        for (int d = 0; d < HS; ++d) o[d] = o[d] * corr + pj * Vs[j][d];
        m = mn;
      }
    }
  }
  if (qi < T) {
    const float inv = 1.f / l;
    for (int d = 0; d < HS; ++d) out[((size_t)b * T + qi) * C + h * HS + d] = o[d] * inv;
    lse[(size_t)bh * T + qi] = m + logf(l);
  }
}

// D[b,h,t] = sum_d dO * O  (fp32 or bf16 inputs); one thread per (row, head), HS unrolled
template <typename T, int HS>
__global__ __launch_bounds__(256) void attn_bwd_dvec(int BT, int T_, int H, const T* __restrict__ out,
                                                     const T* __restrict__ dout, float* __restrict__ dvec) {
  constexpr int VEC = Elt<T>::VEC;
  const int i = blockIdx.x * 256 + threadIdx.x;  // over B*T*H
  if (i >= BT * H) return;
  const int row = i / H, h = i % H;
  const size_t o = (size_t)row * H * HS + h * HS;
  V16<T> a[HS / VEC], c[HS / VEC];
#pragma unroll
  for (int j = 0; j < HS / VEC; ++j) {
    a[j].load(out + o + j * VEC);
    c[j].load(dout + o + j * VEC);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < HS / VEC; ++j)
#pragma unroll
    for (int e = 0; e < VEC; ++e) s += a[j].v[e] * c[j].v[e];
  const int b = row / T_, t = row % T_;
  dvec[((size_t)b * H + h) * T_ + t] = s;
}

// dK, dV: one thread per key
template <int HS>
__global__ __launch_bounds__(AT) void attn_bwd_kv_f32(int T, int H, const float* __restrict__ qkv,
                                                      const float* __restrict__ dout, const float* __restrict__ lse,
                                                      const float* __restrict__ dvec, float* __restrict__ dqkv,
                                                      float scale) {
  __shared__ float Qs[AT][HS + 1], dOs[AT][HS + 1], Ls[AT], Ds[AT];
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HS, C3 = 3 * C;
  const int k0 = blockIdx.x * AT;
  const int kj = k0 + threadIdx.x;
  const float* base = qkv + (size_t)b * T * C3;
  float k[HS], v[HS], dk[HS], dv[HS];
  for (int d = 0; d < HS; ++d) {
    k[d] = kj < T ? base[(size_t)kj * C3 + C + h * HS + d] : 0.f;
    v[d] = kj < T ? base[(size_t)kj * C3 + 2 * C + h * HS + d] : 0.f;
    dk[d] = dv[d] = 0.f;
  }
  for (int q0 = k0; q0 < T; q0 += AT) {
    __syncthreads();
    for (int i = threadIdx.x; i < AT * HS; i += AT) {
      const int r = i / HS, d = i % HS;
      const int qr = q0 + r;
      Qs[r][d] = qr < T ? base[(size_t)qr * C3 + h * HS + d] : 0.f;
      dOs[r][d] = qr < T ? dout[((size_t)b * T + qr) * C + h * HS + d] : 0.f;
    }
    if (threadIdx.x < AT) {
      const int qr = q0 + threadIdx.x;
      Ls[threadIdx.x] = qr < T ? lse[(size_t)bh * T + qr] : 0.f;
      Ds[threadIdx.x] = qr < T ? dvec[(size_t)bh * T + qr] : 0.f;
    }
    __syncthreads();
    if (kj < T) {
      for (int i = 0; i < AT; ++i) {
        const int qi = q0 + i;
        if (qi >= T) break;
        if (qi < kj) continue;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < HS; ++d) {
          s += Qs[i][d] * k[d];
          dp += dOs[i][d] * v[d];
        }
        const float p = expf(s * scale - Ls[i]);
        const float ds = p * (dp - Ds[i]);
        for (int d = 0; d < HS; ++d) {
          dv[d] += p * dOs[i][d];
          dk[d] += ds * Qs[i][d];
        }
      }
    }
  }
  if (kj < T) {
    float* dst = dqkv + ((size_t)b * T + kj) * C3 + h * HS;
    for (int d = 0; d < HS; ++d) {
      dst[C + d] = dk[d] * scale;
      dst[2 * C + d] = dv[d];
    }
  }
}

// dQ: one thread per query
template <int HS>
__global__ __launch_bounds__(AT) void attn_bwd_q_f32(int T, int H, const float* __restrict__ qkv,
                                                     const float* __restrict__ dout, const float* __restrict__ lse,
                                                     const float* __restrict__ dvec, float* __restrict__ dqkv,
                                                     float scale) {
  __shared__ float Ks[AT][HS + 1], Vs[AT][HS + 1];
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int C = H * HS, C3 = 3 * C;
  const int q0 = blockIdx.x * AT;
  const int qi = q0 + threadIdx.x;
  const float* base = qkv + (size_t)b * T * C3;
  float q[HS], dO[HS], dq[HS];
  for (int d = 0; d < HS; ++d) {
    q[d] = qi < T ? base[(size_t)qi * C3 + h * HS + d] : 0.f;
    dO[d] = qi < T ? dout[((size_t)b * T + qi) * C + h * HS + d] : 0.f;
    dq[d] = 0.f;
  }
  const float L = qi < T ? lse[(size_t)bh * T + qi] : 0.f;
  const float Dq = qi < T ? dvec[(size_t)bh * T + qi] : 0.f;
  const int kend = min(T, q0 + AT);
  for (int k0 = 0; k0 < kend; k0 += AT) {
    __syncthreads();
    for (int i = threadIdx.x; i < AT * HS; i += AT) {
      const int r = i / HS, d = i % HS;
      const int kr = k0 + r;
      Ks[r][d] = kr < T ? base[(size_t)kr * C3 + C + h * HS + d] : 0.f;
      Vs[r][d] = kr < T ? base[(size_t)kr * C3 + 2 * C + h * HS + d] : 0.f;
    }
    __syncthreads();
    if (qi < T) {
      const int jn = min(AT, qi - k0 + 1);
      for (int j = 0; j < jn; ++j) {
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < HS; ++d) {
          s += q[d] * Ks[j][d];
          dp += dO[d] * Vs[j][d];
        }
        const float p = expf(s * scale - L);
        const float ds = p * (dp - Dq);
        for (int d = 0; d < HS; ++d) dq[d] += ds * Ks[j][d];
      }
    }
  }
  if (qi < T) {
    float* dst = dqkv + ((size_t)b * T + qi) * C3 + h * HS;
    for (int d = 0; d < HS; ++d) dst[d] = dq[d] * scale;
  }
}

template <int HS>
static void f32_fwd(int B, int T, int H, const float* qkv, float* out, float* lse, hipStream_t s) {
  dim3 grid(cdiv(T, AT), B * H);
  attn_fwd_f32<HS><<<grid, AT, 0, s>>>(T, H, qkv, out, lse, 1.0f / sqrtf((float)HS));
}
template <int HS>
static void f32_bwd(int B, int T, int H, const float* qkv, const float* dout, const float* lse, const float* dvec,
                    float* dqkv, int parts, hipStream_t s) {
  dim3 grid(cdiv(T, AT), B * H);
  if (parts & ATT_BWD_KV)
    attn_bwd_kv_f32<HS><<<grid, AT, 0, s>>>(T, H, qkv, dout, lse, dvec, dqkv, 1.0f / sqrtf((float)HS));
  if (parts & ATT_BWD_Q)
    attn_bwd_q_f32<HS><<<grid, AT, 0, s>>>(T, H, qkv, dout, lse, dvec, dqkv, 1.0f / sqrtf((float)HS));
}

// =====================================================================================
// bf16 MFMA kernels, hs = 64
// =====================================================================================
constexpr int HD = 64;          // head size
constexpr int KT = 64;          // keys (or queries) per LDS tile
constexpr int LDP = HD + 8;     // LDS pitch (elements) of a 64-wide bf16 tile, 16-byte pad
constexpr int BQ = 128;         // rows owned by a block (4 waves x 32)

__device__ __forceinline__ bf16x8 lds_frag16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
// MFMA operand whose k index runs down the rows of a [k][n] LDS tile (pitch LDP), read with
// the gfx950 transpose load ds_read_b64_tr_b16 (lane 16G+i receives as element j the element
// i & 3 of the 8 bytes addressed by lane 16G+4j+(i>>2)). Lane l gets column n = nb + l % 32 and
// k-slots 0..3 = rows kb + 4(l / 32) + 0..3, slots 4..7 = rows kb + 8 + 4(l / 32) + 0..3: the
// k order in which pack_frag lays out accumulator rows, so the two operands agree.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int kb, int nb, int lane) {
  typedef __attribute__((address_space(3))) bf16x4 lds_v4;
  const int G = lane >> 4, t = lane & 15;
  const uint16_t* p = tile + (kb + 4 * (G >> 1) + (t >> 2)) * LDP + nb + (G & 1) * 16 + 4 * (t & 3);
  const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)p));
  const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(p + 8 * LDP)));
  const u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ bf16x8 pack_frag(const float* x) {  // 8 fp32 -> bf16x8
  const u32x4 r = {pack2bf(x[0], x[1]), pack2bf(x[2], x[3]), pack2bf(x[4], x[5]), pack2bf(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}
// row (M index) of accumulator element i for lane group g (= lane / 32)
__device__ __forceinline__ int acc_row(int i, int g) { return (i >> 2) * 8 + g * 4 + (i & 3); }

// Grid (tiles, B*H) -> (b*h, work rank). Blocks are dealt round-robin to the 8 XCDs in linear
// order; here XCD x takes the b*h range [x nbh/8, (x+1) nbh/8) whole (the tiles of one head
// share its L2), and inside it the blocks run in order of decreasing causal work, so every XCD
// gets the same share of heavy and light tiles. rank 0 = the heaviest tile.
__device__ __forceinline__ void attn_block_map(int& bh, int& rank) {
  const int ntile = gridDim.x, nbh = gridDim.y;
  const int L = blockIdx.x + ntile * blockIdx.y;
  if (nbh % 8 == 0) {
    const int per = nbh / 8, xcd = L % 8, j = L / 8;
    bh = xcd * per + j % per;
    rank = j / per;
  } else {
    bh = L / ntile;
    rank = L % ntile;
  }
}

// Buffer resource over rows row0 .. nrows - 1 of a row-major bf16 matrix with ld elements per row,
// starting at m: a load at a byte offset past those rows returns zeros and a store there is
// dropped, so tiles that run past T need no clamping, selects or branches. All arguments must be
// uniform over the wave (the resource lives in scalar registers). The launchers keep
// T * 3C * 2 bytes below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* m, long ld, int row0, int nrows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(m) + (size_t)row0 * ld, (short)0,
                                           (int)(max(nrows - row0, 0) * ld * 2), 0x00020000);
}

// A 64 x 64 bf16 tile piece: rows r, r + 16, r + 32, r + 48 (r = p % 16) x 8 columns per thread
// (128 pieces per tile). The 16 lanes of one 16-byte LDS store cycle write 16 consecutive rows of
// one column chunk, which the 144-byte row pitch spreads over distinct banks (rows 4 apart, as in
// a 4-row piece, would put every fourth lane on the same banks).
// Rows past nrows read as zeros (buffer range check). The per-thread byte offsets are fixed; a
// tile moves only the resource's base, which is scalar work.
struct Piece {
  u32x4 r[4];
  int off[4];  // byte offsets of this thread's rows rg + 16 j, columns cg .. cg + 7, from the tile's row 0
  __device__ __forceinline__ static int rgrp(int p) { return p & 15; }
  __device__ __forceinline__ static int cgrp(int p) { return (p >> 4) * 8; }
  __device__ __forceinline__ void init(long ld, int p) {
#pragma unroll
    for (int j = 0; j < 4; ++j) off[j] = (int)(((rgrp(p) + 16 * j) * ld + cgrp(p)) * 2);
  }
  __device__ __forceinline__ void load(const uint16_t* src, long ld, int row0, int nrows) {
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(src, ld, row0, nrows);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[j], 0, 0));
  }
  __device__ __forceinline__ void store_rows(uint16_t* lds, int p) const {  // lds[row][col]
    const int rg = rgrp(p), cg = cgrp(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(lds + (rg + 16 * j) * LDP + cg) = r[j];
  }
};

// ---------------------------------------------------------------- forward
// grid (T/128, B*H), 256 threads. Wave w owns queries q0 + 32w .. +31.
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16(int T, int H, const uint16_t* __restrict__ qkv,
                                                        uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t Ksb[2][KT * LDP];  // [key][d], two stages
  __shared__ __attribute__((aligned(16))) uint16_t Vsb[2][KT * LDP];  // [key][d]
  int bh, rank;
  attn_block_map(bh, rank);
  const int qt = gridDim.x - 1 - rank;  // the last query tiles see the most keys
  const int b = bh / H, h = bh % H;
  const int C = H * HD;
  const long C3 = 3L * C;
  const uint16_t* base = qkv + (size_t)b * T * C3;
  // the wave index through readfirstlane: the compiler then keeps every per-wave bound below in
  // scalar registers and branches on it instead of masking lanes
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 5,
            l32 = lane & 31;
  const int q0 = qt * BQ;
  const int qw0 = q0 + 32 * w;
  const int myq = qw0 + l32;

  // Q as the B operand of S^T = K Q^T: lane holds Q[myq][16s + 8g .. +8]
  bf16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (myq < T) x = *reinterpret_cast<const u32x4*>(base + (size_t)myq * C3 + h * HD + 16 * s + 8 * g);
    qf[s] = __builtin_bit_cast(bf16x8, x);
  }
  const float c2 = LOG2E / sqrtf((float)HD);  // scale folded into base-2 exponent
  f32x16 o[2] = {zero16(), zero16()};         // O^T: rows d (2 x 32), columns = queries
  float m_run = -INFINITY;
  // The softmax denominators come out of the matrix cores: an A operand whose row 0 is all ones
  // (lanes 0 and 32 supply row 0) times P^T adds the row sums of P, in row 0 of lsum (register 0
  // of lanes 0..31). They sum the bf16 probabilities that also enter P V.
  f32x16 lsum = zero16();
  const bf16x8 ones = __builtin_bit_cast(bf16x8, l32 == 0 ? u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}
                                                          : u32x4{0u, 0u, 0u, 0u});

  const int kend = min(T, q0 + BQ);
  const int ntiles = cdiv(kend, KT);
  Piece pc;
  const int p = tid & 127;
  const bool is_k = w < 2;  // waves 0, 1 stage K, waves 2, 3 stage V (uniform per wave)
  pc.init(C3, p);
  const uint16_t* src = base + (is_k ? C : 2 * C) + h * HD;
  pc.load(src, C3, 0, T);
  pc.store_rows(is_k ? Ksb[0] : Vsb[0], p);
  __syncthreads();
  // one 64-key tile; only the last two tiles (keys from q0 on) hold keys after some query of the
  // block, so the others are compiled without the mask
  auto tile = [&](int kt, auto diag) {
    const uint16_t* Ks = Ksb[kt & 1];
    const uint16_t* Vs = Vsb[kt & 1];
    if (kt + 1 < ntiles) pc.load(src, C3, (kt + 1) * KT, T);
    // both 32-key halves of the tile at once: two independent S chains, one max, one rescale
    const int kb0 = kt * KT;
    if (kb0 <= qw0 + 31) {  // else the whole tile is in the future of this wave's queries
      f32x16 st[2] = {zero16(), zero16()};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
          st[sb] = mfma(lds_frag16(Ks + (sb * 32 + l32) * LDP + 16 * s + 8 * g), qf[s], st[sb]);
      float sc[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] = st[0][i];
        sc[16 + i] = st[1][i];
      }
      if constexpr (decltype(diag)::value) {
        if (kb0 + 63 > qw0) {  // mask keys after the query
          // key = kb0 + 32 (i >> 4) + acc_row(i & 15, g) > myq: one compare with a constant per entry
          const int lim = myq - kb0 - 4 * g;
#pragma unroll
          for (int i = 0; i < 32; ++i)
            if ((i >> 4) * 32 + ((i & 15) >> 2) * 8 + (i & 3) > lim) sc[i] = -INFINITY;
        }
      }
      float mloc = sc[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) mloc = fmaxf(mloc, sc[i]);
      mloc = pair_max(mloc);
      const float m_new = fmaxf(m_run, mloc * c2);  // scaled, log2 units
#pragma unroll
      for (int i = 0; i < 32; ++i) sc[i] = fast_exp2(fmaf(sc[i], c2, -m_new));
      // rescale only when some query of the wave has a new running max (corr is exactly 1 for
      // the others, and for all of them once the maxima settle)
      if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
        const float corr = fast_exp2(m_run - m_new);
        lsum[0] *= corr;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= corr;
      }
      m_run = m_new;
      // O^T += V^T P^T : A = V^T (rows d, k = keys), B = P^T (k = keys, columns = queries)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 pf = pack_frag(sc + 16 * sb + 8 * ks);
#pragma unroll
          for (int db = 0; db < 2; ++db)
            o[db] = mfma(tr_frag(Vs, sb * 32 + 16 * ks, db * 32, lane), pf, o[db]);
          lsum = mfma(ones, pf, lsum);
        }
    }
    // the next tile goes to the other stage (last read in the previous iteration, before the
    // barrier that ended it): one barrier per tile
    if (kt + 1 < ntiles) pc.store_rows(is_k ? Ksb[(kt + 1) & 1] : Vsb[(kt + 1) & 1], p);
    __syncthreads();
  };
  const int nplain = min(ntiles, 2 * qt);  // tiles wholly before the block's first query
  for (int kt = 0; kt < nplain; ++kt) tile(kt, std::false_type{});
  for (int kt = nplain; kt < ntiles; ++kt) tile(kt, std::true_type{});
  const float l_tot = pair_sum(g == 0 ? lsum[0] : 0.f);
  if (myq < T) {
    const float inv = 1.f / l_tot;
    uint16_t* dst = out + ((size_t)b * T + myq) * C + h * HD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + 4 * g;
        const u32x2 v = {pack2bf(o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv),
                         pack2bf(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(dst + d) = v;
      }
    if (g == 0) lse[(size_t)bh * T + myq] = (m_run + __log2f(l_tot)) / LOG2E;
  }
}

// Bias-gradient partials of one block's 128 rows of dqkv: lane sums a[db] (and b[db]) cover
// column db * 32 + (lane & 31) of the head over the lane's 16 rows; lanes l and l ^ 32 hold the
// other 16 rows of the wave, the 4 waves the other 96. Written in a fixed order to
// cs[row][col0 + c] (a) and cs[row][col0 + C + c] (b), c < 64, with C = C3 / 3. red: 2 KB of the
// block's LDS, free once every wave has passed the last barrier of the main loop.
__device__ __forceinline__ void bias_partial(float* __restrict__ cs, int row, long C3, int col0, float (&a)[2],
                                             const float* b, float* red, int w, int lane) {
  const int nq = b ? 2 : 1;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const float ta = a[db] + __shfl_xor(a[db], 32);
    if (lane < 32) red[w * 128 + db * 32 + lane] = ta;
    if (b) {
      const float tb = b[db] + __shfl_xor(b[db], 32);
      if (lane < 32) red[w * 128 + 64 + db * 32 + lane] = tb;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 64 * nq) {
    const float v = (red[t] + red[128 + t]) + (red[256 + t] + red[384 + t]);
    cs[(size_t)row * C3 + col0 + (t >> 6) * (C3 / 3) + (t & 63)] = v;
  }
}

// ---------------------------------------------------------------- backward: dK, dV
// grid (T/128, B*H): block owns 128 keys (wave w: 32 keys), loops over 64-query tiles.
__global__ __launch_bounds__(256, 2) void attn_bwd_kv_bf16(int T, int H, const uint16_t* __restrict__ qkv,
                                                           const uint16_t* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ dvec,
                                                           uint16_t* __restrict__ dqkv,
                                                           float* __restrict__ cs) {
  __shared__ __attribute__((aligned(16))) uint16_t Qs[KT * LDP];   // [q][d]
  __shared__ __attribute__((aligned(16))) uint16_t dOs[KT * LDP];  // [q][d]
  __shared__ __attribute__((aligned(16))) float Ls[KT];
  __shared__ __attribute__((aligned(16))) float Dsh[KT];
  int bh, rank;
  attn_block_map(bh, rank);
  const int kt_blk = rank;  // the first keys see the most queries
  const int b = bh / H, h = bh % H;
  const int C = H * HD;
  const long C3 = 3L * C;
  const uint16_t* base = qkv + (size_t)b * T * C3;
  const uint16_t* dbase = dout + (size_t)b * T * C;
  // the wave index through readfirstlane: the compiler then keeps every per-wave bound below in
  // scalar registers and branches on it instead of masking lanes
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 5,
            l32 = lane & 31;
  const int k0 = kt_blk * BQ;
  const int kw0 = k0 + 32 * w;
  const int mykey = kw0 + l32;
  const int kdiag = mykey - 4 * g;
  const float c2 = LOG2E / sqrtf((float)HD);

  // K and V of this lane's key as B operands (S = Q K^T, dP = dO V^T)
  // unguarded loads: a key past T reads the last row; its probabilities are masked (every query
  // precedes it) and its dK, dV are not stored
  bf16x8 kf[4], vf[4];
  const int krow = min(mykey, T - 1);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + (size_t)krow * C3 + C + h * HD + 16 * s + 8 * g));
    vf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + (size_t)krow * C3 + 2 * C + h * HD + 16 * s + 8 * g));
  }
  f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};  // rows = keys, cols = d

  const int qstart = (k0 / KT) * KT;
  const int ntiles = cdiv(T - qstart, KT);
  Piece pc;
  const int p = tid & 127;
  const bool is_q = w < 2;  // waves 0, 1 stage Q, waves 2, 3 stage dO (uniform per wave)
  const uint16_t* src = (is_q ? base : dbase) + h * HD;
  const long lds_ld = is_q ? C3 : (long)C;
  pc.init(lds_ld, p);
  float lnext = 0.f, dnext = 0.f;  // LSE and D of query tid of the next tile (tid < 64)
  // LSE / D of query qt0 + tid % 64 from a clamped index (straight-line; replaced for rows past T
  // when stored)
  int lrow = 0;
  auto load_tile = [&](int it) {
    const int qt0 = qstart + it * KT;
    pc.load(src, lds_ld, qt0, T);
    lrow = qt0 + (tid & (KT - 1));
    const size_t li = (size_t)bh * T + min(lrow, T - 1);
    lnext = lse[li];
    dnext = dvec[li];
  };
  // one 64-query tile; only the first two tiles (queries below k0 + 128) hold queries before
  // some key of the block, so the others are compiled without the mask
  auto tile = [&](int it, auto diag) {
    const int qt0 = qstart + it * KT;
    pc.store_rows(is_q ? Qs : dOs, p);
    if (tid < KT) {
      Ls[tid] = lrow < T ? lnext * LOG2E : INFINITY;  // a query past T: probability exp2(-inf) = 0
      Dsh[tid] = lrow < T ? dnext : 0.f;
    }
    __syncthreads();
    if (it + 1 < ntiles) load_tile(it + 1);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qq0 = qt0 + 32 * qb;
      // sub-blocks whose queries all precede this wave's keys are not skipped but fully masked
      // below: a skip here puts the dK/dV accumulators on two control paths, and the register
      // copies the compiler then makes on every tile cost more than the few extra MFMAs
      f32x16 sacc = zero16(), dpacc = zero16();  // rows = queries, cols = keys
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 qa = lds_frag16(Qs + (32 * qb + l32) * LDP + 16 * s + 8 * g);
        const bf16x8 da = lds_frag16(dOs + (32 * qb + l32) * LDP + 16 * s + 8 * g);
        sacc = mfma(qa, kf[s], sacc);
        dpacc = mfma(da, vf[s], dpacc);
      }
      // LSE (log2 units) and D of this lane's 16 accumulator rows: rows 32qb + 8*r4 + 4g + 0..3
      float pr[16], ds[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + 32 * qb + 8 * r4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[4 * r4 + e] = fast_exp2(sacc[4 * r4 + e] * c2 - l4[e]);
      }
      if constexpr (decltype(diag)::value) {
        // some keys of the wave follow some queries of the sub-block (uniform over the wave);
        // queries past T already have probability 0 from their infinite LSE.
        // key <= q = qq0 + acc_row(i, g)  <=>  8 (i >> 2) + (i & 3) >= mykey - qq0 - 4g
        if (qq0 < kw0 + 31) {
          const int lim = kdiag - qq0;
#pragma unroll
          for (int i = 0; i < 16; ++i) pr[i] = (i >> 2) * 8 + (i & 3) >= lim ? pr[i] : 0.f;
        }
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dsh + 32 * qb + 8 * r4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) ds[4 * r4 + e] = pr[4 * r4 + e] * (dpacc[4 * r4 + e] - d4[e]);
      }
      // dV += P^T dO ; dK += dS^T Q  (A = accumulator as [key][q], B from transposed tiles)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pa = pack_frag(pr + 8 * ks);
        const bf16x8 sa = pack_frag(ds + 8 * ks);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          dv[db] = mfma(pa, tr_frag(dOs, 32 * qb + 16 * ks, db * 32, lane), dv[db]);
          dk[db] = mfma(sa, tr_frag(Qs, 32 * qb + 16 * ks, db * 32, lane), dk[db]);
        }
      }
    }
    __syncthreads();
  };
  if (ntiles > 0) load_tile(0);
  const int ndiag = min(ntiles, 2);
  for (int it = 0; it < ndiag; ++it) tile(it, std::true_type{});
  for (int it = ndiag; it < ntiles; ++it) tile(it, std::false_type{});
  // store: accumulator rows = keys, columns = d. Keys past T have dK = dV = 0 (every probability
  // of theirs is masked), so they add nothing to the column sums, and their stores fall outside
  // the resource and are dropped.
  const float sc = 1.0f / sqrtf((float)HD);
  float sk[2] = {0.f, 0.f}, sv[2] = {0.f, 0.f};  // column sums over this lane's keys (as stored)
  const __amdgpu_buffer_rsrc_t ors = rows_rsrc(dqkv + (size_t)b * T * C3 + h * HD, C3, kw0, T);
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int d = db * 32 + l32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int o = (int)((acc_row(i, g) * C3 + C + d) * 2);
      const uint16_t k16 = f2bf(dk[db][i] * sc), v16 = f2bf(dv[db][i]);
      __builtin_amdgcn_raw_buffer_store_b16(k16, ors, o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(v16, ors, o + 2 * C, 0, 0);
      sk[db] += bf2f(k16);
      sv[db] += bf2f(v16);
    }
  }
  if (cs) bias_partial(cs, b * gridDim.x + kt_blk, C3, C + h * HD, sk, sv, reinterpret_cast<float*>(Qs), w, lane);
}

// ---------------------------------------------------------------- backward: dQ
// grid (T/128, B*H): block owns 128 queries (wave w: 32), loops over 64-key tiles. Every query is
// owned by exactly one block, which also forms its D = rowsum(dO * O) (from the dO row it holds and
// the O row) and writes it to dvec for the dK/dV kernel, launched after this one.
__global__ __launch_bounds__(256, 2) void attn_bwd_q_bf16(int T, int H, const uint16_t* __restrict__ qkv,
                                                          const uint16_t* __restrict__ out,
                                                          const uint16_t* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ dvec,
                                                          uint16_t* __restrict__ dqkv,
                                                          float* __restrict__ cs) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * LDP];  // [key][d]
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KT * LDP];  // [key][d]
  int bh, rank;
  attn_block_map(bh, rank);
  const int qt = gridDim.x - 1 - rank;
  const int b = bh / H, h = bh % H;
  const int C = H * HD;
  const long C3 = 3L * C;
  const uint16_t* base = qkv + (size_t)b * T * C3;
  const uint16_t* dbase = dout + (size_t)b * T * C;
  // the wave index through readfirstlane: the compiler then keeps every per-wave bound below in
  // scalar registers and branches on it instead of masking lanes
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 5,
            l32 = lane & 31;
  const int q0 = qt * BQ;
  const int qw0 = q0 + 32 * w;
  const int myq = qw0 + l32;
  const float c2 = LOG2E / sqrtf((float)HD);

  // B operands Q[myq], dO[myq] by unguarded loads (a query past T reads the last row; its dS is
  // masked and its dQ not stored)
  bf16x8 qf[4], df[4];
  u32x4 orow[4];
  const int qrow = min(myq, T - 1);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + (size_t)qrow * C3 + h * HD + 16 * s + 8 * g));
    df[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dbase + (size_t)qrow * C + h * HD + 16 * s + 8 * g));
    orow[s] = *reinterpret_cast<const u32x4*>(out + ((size_t)b * T + qrow) * C + h * HD + 16 * s + 8 * g);
  }
  const size_t qi = (size_t)bh * T + qrow;
  const float L2 = myq < T ? lse[qi] * LOG2E : INFINITY;  // a query past T: probabilities exp2(-inf) = 0
  // D of this query: the lane holds 32 of the row's 64 (dO, O) pairs, lane ^ 32 the other 32
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4 dw = __builtin_bit_cast(u32x4, df[s]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dpart += __uint_as_float(dw[e] << 16) * __uint_as_float(orow[s][e] << 16);
      dpart += __uint_as_float(dw[e] & 0xffff0000u) * __uint_as_float(orow[s][e] & 0xffff0000u);
    }
  }
  const float Dq = pair_sum(dpart);
  if (g == 0 && myq < T) dvec[qi] = Dq;
  f32x16 dq[2] = {zero16(), zero16()};  // rows = queries, cols = d

  const int kend = min(T, q0 + BQ);
  const int ntiles = cdiv(kend, KT);
  Piece pc;
  const int p = tid & 127;
  const bool is_k = w < 2;  // waves 0, 1 stage K, waves 2, 3 stage V (uniform per wave)
  const uint16_t* src = base + (is_k ? C : 2 * C) + h * HD;
  pc.init(C3, p);
  // one 64-key tile; only the last two tiles (keys from q0 on) hold keys after some query of the
  // block, so the others are compiled without the mask
  auto tile = [&](int kt, auto diag) {
    pc.store_rows(is_k ? Ks : Vs, p);
    __syncthreads();
    if (kt + 1 < ntiles) pc.load(src, C3, (kt + 1) * KT, T);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int kb = kt * KT + sb * 32;
      if (decltype(diag)::value && kb > qw0 + 31) continue;
      f32x16 st = zero16(), dpt = zero16();  // rows = keys, cols = queries
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        st = mfma(lds_frag16(Ks + (sb * 32 + l32) * LDP + 16 * s + 8 * g), qf[s], st);
        dpt = mfma(lds_frag16(Vs + (sb * 32 + l32) * LDP + 16 * s + 8 * g), df[s], dpt);
      }
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = fast_exp2(st[i] * c2 - L2);
      if constexpr (decltype(diag)::value) {
        // some keys of the sub-block follow some queries of the wave (uniform); queries past T
        // already have probability 0. key = kb + acc_row(i, g) <= myq  <=>  8 (i >> 2) + (i & 3) <= lim
        if (kb + 31 > qw0) {
          const int lim = myq - kb - 4 * g;
#pragma unroll
          for (int i = 0; i < 16; ++i) ds[i] = (i >> 2) * 8 + (i & 3) <= lim ? ds[i] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] *= dpt[i] - Dq;
      // dQ += dS K : A = dS (rows q, k = keys) from the accumulator, B = K read transposed
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 sa = pack_frag(ds + 8 * ks);
#pragma unroll
        for (int db = 0; db < 2; ++db) dq[db] = mfma(sa, tr_frag(Ks, sb * 32 + 16 * ks, db * 32, lane), dq[db]);
      }
    }
    __syncthreads();
  };
  pc.load(src, C3, 0, T);
  const int nplain = min(ntiles, 2 * qt);  // tiles wholly before the block's first query
  for (int kt = 0; kt < nplain; ++kt) tile(kt, std::false_type{});
  for (int kt = nplain; kt < ntiles; ++kt) tile(kt, std::true_type{});
  // queries past T have dQ = 0 (all their probabilities are 0): they add nothing to the column
  // sums, and their stores fall outside the resource and are dropped
  const float sc = 1.0f / sqrtf((float)HD);
  float sq[2] = {0.f, 0.f};  // column sums over this lane's queries (as stored)
  const __amdgpu_buffer_rsrc_t ors = rows_rsrc(dqkv + (size_t)b * T * C3 + h * HD, C3, qw0, T);
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int d = db * 32 + l32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint16_t q16 = f2bf(dq[db][i] * sc);
      __builtin_amdgcn_raw_buffer_store_b16(q16, ors, (int)((acc_row(i, g) * C3 + d) * 2), 0, 0);
      sq[db] += bf2f(q16);
    }
  }
  if (cs) bias_partial(cs, b * gridDim.x + qt, C3, h * HD, sq, nullptr, reinterpret_cast<float*>(Ks), w, lane);
}

// =====================================================================================
// The bf16 kernels address one sequence's [T, 3C] rows through buffer resources with 32-bit byte
// counts and offsets.
static bool bf16_rows_fit(int T, int H) { return (long)T * 3 * H * HD * 2 < (1L << 31); }

hipError_t launch_attention_fwd(DType dt, int B, int T, int H, int hs, const void* qkv, void* out, float* lse,
                                hipStream_t s) {
  if (B < 0 || T < 0 || H < 1) return hipErrorInvalidValue;
  if (B == 0 || T == 0) return hipSuccess;
  if (dt == DT_BF16) {
    if (hs != HD || !bf16_rows_fit(T, H)) return hipErrorInvalidValue;
    dim3 grid(cdiv(T, BQ), B * H);
    attn_fwd_bf16<<<grid, 256, 0, s>>>(T, H, reinterpret_cast<const uint16_t*>(qkv),
                                       reinterpret_cast<uint16_t*>(out), lse);
    return hipGetLastError();
  }
  auto Q = reinterpret_cast<const float*>(qkv);
  auto O = reinterpret_cast<float*>(out);
  switch (hs) {
    case 4: f32_fwd<4>(B, T, H, Q, O, lse, s); break;
    case 8: f32_fwd<8>(B, T, H, Q, O, lse, s); break;
    case 16: f32_fwd<16>(B, T, H, Q, O, lse, s); break;
    case 32: f32_fwd<32>(B, T, H, Q, O, lse, s); break;
    case 64: f32_fwd<64>(B, T, H, Q, O, lse, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int attention_bias_partial_rows(int B, int T) { return B * cdiv(T, BQ); }

hipError_t launch_attention_bwd(DType dt, int B, int T, int H, int hs, const void* qkv, const void* out,
                                const void* dout, const float* lse, void* dqkv, float* dvec, int parts,
                                hipStream_t s, float* cs) {
  if (B < 0 || T < 0 || H < 1) return hipErrorInvalidValue;
  if (B == 0 || T == 0) return hipSuccess;
  const int BT = B * T;
  if (dt == DT_BF16) {
    if (hs != HD || !bf16_rows_fit(T, H)) return hipErrorInvalidValue;
    // D = rowsum(dO * O) comes out of the dQ kernel, which therefore runs first; ATT_BWD_PRE alone
    // has nothing left to do
    dim3 grid(cdiv(T, BQ), B * H);
    auto Q = reinterpret_cast<const uint16_t*>(qkv);
    auto O_ = reinterpret_cast<const uint16_t*>(out);
    auto dO = reinterpret_cast<const uint16_t*>(dout);
    auto dQ = reinterpret_cast<uint16_t*>(dqkv);
    if (parts & ATT_BWD_Q) attn_bwd_q_bf16<<<grid, 256, 0, s>>>(T, H, Q, O_, dO, lse, dvec, dQ, cs);
    if (parts & ATT_BWD_KV) attn_bwd_kv_bf16<<<grid, 256, 0, s>>>(T, H, Q, dO, lse, dvec, dQ, cs);
    (void)BT;
    return hipGetLastError();
  }
  if (parts & ATT_BWD_PRE) {
    auto O_ = reinterpret_cast<const float*>(out);
    auto dO_ = reinterpret_cast<const float*>(dout);
    const int nb = cdiv((long)BT * H, 256);
    switch (hs) {
      case 4: attn_bwd_dvec<float, 4><<<nb, 256, 0, s>>>(BT, T, H, O_, dO_, dvec); break;
      case 8: attn_bwd_dvec<float, 8><<<nb, 256, 0, s>>>(BT, T, H, O_, dO_, dvec); break;
      case 16: attn_bwd_dvec<float, 16><<<nb, 256, 0, s>>>(BT, T, H, O_, dO_, dvec); break;
      case 32: attn_bwd_dvec<float, 32><<<nb, 256, 0, s>>>(BT, T, H, O_, dO_, dvec); break;
      case 64: attn_bwd_dvec<float, 64><<<nb, 256, 0, s>>>(BT, T, H, O_, dO_, dvec); break;
      default: return hipErrorInvalidValue;
    }
  }
  auto Q = reinterpret_cast<const float*>(qkv);
  auto dO = reinterpret_cast<const float*>(dout);
  auto dQ = reinterpret_cast<float*>(dqkv);
  switch (hs) {
    case 4: f32_bwd<4>(B, T, H, Q, dO, lse, dvec, dQ, parts, s); break;
    case 8: f32_bwd<8>(B, T, H, Q, dO, lse, dvec, dQ, parts, s); break;
    case 16: f32_bwd<16>(B, T, H, Q, dO, lse, dvec, dQ, parts, s); break;
    case 32: f32_bwd<32>(B, T, H, Q, dO, lse, dvec, dQ, parts, s); break;
    case 64: f32_bwd<64>(B, T, H, Q, dO, lse, dvec, dQ, parts, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace g2
