// Host runtime behind the C ABI of include/gpt2.h and include/gpt2_ops.h.
//
// Owns no device memory: the caller's workspace is carved once at gpt2_init (the GPT-2
// reproduction post, "Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section 代码, notes that
// all GPU memory is allocated once at start-up so the footprint never changes). Enqueues the
// forward (encoder -> L x [LN, QKV, attention, proj + residual, LN, fc + GELU, proj + residual]
// -> final LN -> tied classifier -> fused cross-entropy) and the backward in the reverse order
// the llm.c tour describes ("Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section
// 代码解剖), then the single-launch AdamW update.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/gpt2.h"
#include "../../include/gpt2_ops.h"
#include "common.h"
#include "kernels.h"

using namespace g2;

namespace {

constexpr size_t NONE = ~(size_t)0;
constexpr int NORM_PARTS = 1024;

struct LayerOff {
  size_t ln1w, ln1b, qkvw, qkvb, attprojw, attprojb, ln2w, ln2b, fcw, fcb, fcprojw, fcprojb;
};
struct LayerAct {
  // recompute 0: fch holds gelu'(z) of the MLP pre-activation z (all the backward needs of z),
  // fchg gelu(z). recompute >= 1: fch holds z and fchg is the buffer all layers share, refilled
  // with gelu(z) in the backward. recompute 2: ln1 and ln2 are one shared buffer as well,
  // refilled from the LayerNorm inputs and saved statistics in the backward.
  char *ln1, *qkv, *atty, *res1, *ln2, *fch, *fchg, *res2;
  float *ln1_mean, *ln1_rstd, *ln2_mean, *ln2_rstd, *lse;
};

struct Model {
  bool ready = false;
  gpt2_config cfg{};
  DType dt = DT_F32;
  size_t es = 4;  // bytes per activation element
  int L = 0, H = 0, C = 0, V = 0, Vp = 0, maxT = 0, B = 0, T = 0, BT = 0, ldl = 0;
  size_t N = 0;
  size_t o_wte = 0, o_wpe = 0, o_lnfw = 0, o_lnfb = NONE;
  uint64_t seed = 0;
  std::vector<LayerOff> lo;
  std::vector<WorkItem> items_host;
  // bf16 mode: AdamW takes the matrices with transposed copies as tiles (updating the copies in
  // the same pass) and everything else as flat items
  std::vector<WorkItem> adam_items_host;
  std::vector<AdamTile> adam_tiles_host;
  WorkItem* adam_items = nullptr;
  AdamTile* adam_tiles = nullptr;

  // device pointers inside the workspace
  float *params = nullptr, *grads = nullptr, *m = nullptr, *v = nullptr;
  uint16_t* shadow = nullptr;
  // bf16 runs: transposed copies of the weight matrices (layer matrices at their parameter
  // offsets in shadow_t, the token embedding as C x ldl in wte_t) for the input-gradient products,
  // which then read both operands K-contiguous
  uint16_t *shadow_t = nullptr, *wte_t = nullptr;
  std::vector<TransItem> tr_host;
  TransItem* tr_items = nullptr;
  int tr_tiles = 0;
  WorkItem* items = nullptr;
  char* encoded = nullptr;
  std::vector<LayerAct> la;
  char* lnf = nullptr;
  float *lnf_mean = nullptr, *lnf_rstd = nullptr;
  char* logits = nullptr;
  float* losses = nullptr;
  char *dres = nullptr, *dbuf1 = nullptr, *dbuf2 = nullptr;
  float* dvec = nullptr;
  uint32_t* keys = nullptr;
  float* scratch = nullptr;
  size_t scratch_floats = 0;
  // column-sum partials of the backward (LayerNorm weight / bias gradients, linear-layer bias
  // gradients) whose second stage runs once, batched, at the end of the backward: the region they
  // are written to, the device table of the batched launch, and the host lists (this backward's
  // and the one in the device table)
  float* defer = nullptr;
  size_t defer_floats = 0, defer_used = 0;
  FinishBlock* fin_dev = nullptr;
  size_t fin_cap = 0;
  std::vector<FinishBlock> fin_host, fin_up;
  double* norm_partial = nullptr;
  double* norm2 = nullptr;
  float* clip_scale = nullptr;
  // one rank's share of a sharded update (gpt2_adamw_step_range): the flat work items cut to the
  // range, and the device copies of the caller's squared global norm and the clip scale from it
  std::vector<WorkItem> range_host;
  WorkItem* range_items = nullptr;
  double* range_norm2 = nullptr;
  float* range_scale = nullptr;
  struct {
    double n2;
    float scale;
  } range_vals{};
  bool transposed_stale = false;  // a range update changed weights whose transposed copies it does not write
  float* loss_dev = nullptr;
  float* dloss_dev = nullptr;
  int* nvalid_dev = nullptr;
  int* err_dev = nullptr;

  // host state
  float* pinned = nullptr;  // [0] loss, [1] error word (as int)
  int micro = 0;            // backward passes since the last update
  bool fwd_targets = false; // last forward had targets and its backward has not run yet
  bool fwd_logits = false;  // last forward had no targets: logits are readable
  hipStream_t stream = nullptr;
  // side stream: the (token, position) sort for the embedding gradient overlaps the forward
  hipStream_t side = nullptr;
  hipEvent_t ev_tokens = nullptr, ev_sorted = nullptr;
};

Model g;
int g_status = GPT2_OK;
std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  g_status = code;
  return code;
}
int ok() {
  g_status = GPT2_OK;
  return GPT2_OK;
}
#define HIPCHK(x)                                                                      \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) return fail(GPT2_EHIP, "%s: %s", #x, hipGetErrorString(e_)); \
  } while (0)

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------------ configuration + layout
const char* check_config(const gpt2_config* c) {
  if (!c) return "null config";
  if (c->n_layer < 1 || c->n_head < 1 || c->n_embd < 8) return "n_layer, n_head >= 1 and n_embd >= 8 required";
  if (c->n_embd % c->n_head) return "n_embd must be a multiple of n_head";
  if (c->n_embd % 8) return "n_embd must be a multiple of 8";
  if (c->vocab < 1 || c->padded_vocab < c->vocab || c->padded_vocab > 65536) return "need 1 <= vocab <= padded_vocab <= 65536";
  if (c->max_seq < 1 || c->seq < 1 || c->seq > c->max_seq) return "need 1 <= seq <= max_seq";
  if (c->batch < 1 || (long)c->batch * c->seq > 32768) return "need batch >= 1 and batch*seq <= 32768";
  if (c->precision != GPT2_FP32 && c->precision != GPT2_BF16) return "precision must be GPT2_FP32 or GPT2_BF16";
  const int hs = c->n_embd / c->n_head;
  if (c->precision == GPT2_BF16 && hs != 64) return "GPT2_BF16 needs head size 64";
  if (c->precision == GPT2_FP32 && hs != 4 && hs != 8 && hs != 16 && hs != 32 && hs != 64)
    return "GPT2_FP32 needs head size in {4, 8, 16, 32, 64}";
  if (c->n_embd > 2048) return "n_embd must be <= 2048";
  if (c->grad_accum < 1) return "grad_accum must be >= 1";
  if (c->recompute < 0 || c->recompute > 2) return "recompute must be 0, 1 or 2";
  if (c->no_master != 0 && c->no_master != 1) return "no_master must be 0 or 1";
  if (c->no_master && c->precision != GPT2_BF16) return "no_master needs GPT2_BF16";
  if (c->linear_bias != 0 && c->linear_bias != 1) return "linear_bias must be 0 or 1";
  if (c->ln_bias != 0 && c->ln_bias != 1) return "ln_bias must be 0 or 1";
  return nullptr;
}

// Walk the layout; returns the number of parameters. Fills offsets when m != nullptr.
size_t layout(const gpt2_config* c, Model* m) {
  const size_t C = c->n_embd;
  size_t off = 0;
  auto take = [&](size_t n) {
    size_t o = off;
    off += n;
    return o;
  };
  size_t wte = take((size_t)c->padded_vocab * C), wpe = take((size_t)c->max_seq * C);
  std::vector<LayerOff> lo(c->n_layer);
  for (int l = 0; l < c->n_layer; ++l) {
    LayerOff& L = lo[l];
    L.ln1w = take(C);
    L.ln1b = c->ln_bias ? take(C) : NONE;
    L.qkvw = take(3 * C * C);
    L.qkvb = c->linear_bias ? take(3 * C) : NONE;
    L.attprojw = take(C * C);
    L.attprojb = c->linear_bias ? take(C) : NONE;
    L.ln2w = take(C);
    L.ln2b = c->ln_bias ? take(C) : NONE;
    L.fcw = take(4 * C * C);
    L.fcb = c->linear_bias ? take(4 * C) : NONE;
    L.fcprojw = take(4 * C * C);
    L.fcprojb = c->linear_bias ? take(C) : NONE;
  }
  size_t lnfw = take(C), lnfb = c->ln_bias ? take(C) : NONE;
  if (m) {
    m->o_wte = wte;
    m->o_wpe = wpe;
    m->o_lnfw = lnfw;
    m->o_lnfb = lnfb;
    m->lo = lo;
  }
  return off;
}

// The tensors in layout order: size, kind (0 LN weight, 1 2-D, 2 bias) and, for the matrices
// that get a transposed bf16 copy, their rows and columns (else 0).
struct TensorDesc {
  size_t size;
  int kind;
  int rows, cols;
};
std::vector<TensorDesc> tensor_list(const gpt2_config* c) {
  const int C = c->n_embd;
  const size_t Cs = C;
  std::vector<TensorDesc> t;
  t.push_back({(size_t)c->padded_vocab * Cs, 1, c->padded_vocab, C});
  t.push_back({(size_t)c->max_seq * Cs, 1, 0, 0});
  for (int l = 0; l < c->n_layer; ++l) {
    t.push_back({Cs, 0, 0, 0});
    if (c->ln_bias) t.push_back({Cs, 2, 0, 0});
    t.push_back({3 * Cs * Cs, 1, 3 * C, C});
    if (c->linear_bias) t.push_back({3 * Cs, 2, 0, 0});
    t.push_back({Cs * Cs, 1, C, C});
    if (c->linear_bias) t.push_back({Cs, 2, 0, 0});
    t.push_back({Cs, 0, 0, 0});
    if (c->ln_bias) t.push_back({Cs, 2, 0, 0});
    t.push_back({4 * Cs * Cs, 1, 4 * C, C});
    if (c->linear_bias) t.push_back({4 * Cs, 2, 0, 0});
    t.push_back({4 * Cs * Cs, 1, C, 4 * C});
    if (c->linear_bias) t.push_back({Cs, 2, 0, 0});
  }
  t.push_back({Cs, 0, 0, 0});
  if (c->ln_bias) t.push_back({Cs, 2, 0, 0});
  return t;
}

// Work items: tensors cut into runs of <= ITEM_LEN elements; 2-D tensors draw normals.
// skip_transposed: leave out the matrices with a transposed copy (the AdamW tiles cover them).
std::vector<WorkItem> make_items(const gpt2_config* c, bool skip_transposed = false) {
  std::vector<WorkItem> items;
  size_t off = 0, normal = 0;
  for (const TensorDesc& t : tensor_list(c)) {
    if (!(skip_transposed && t.rows > 0)) {
      for (size_t s = 0; s < t.size; s += ITEM_LEN) {
        WorkItem it{};
        it.off = off + s;
        it.len = (uint32_t)std::min<size_t>(ITEM_LEN, t.size - s);
        it.kind = t.kind == 1 ? 1u : 0u;
        it.normal0 = normal + s;
        it.init_val = t.kind == 0 ? 1.0f : 0.0f;  // LN weights 1, biases 0
        items.push_back(it);
      }
    }
    off += t.size;
    if (t.kind == 1) normal += t.size;
  }
  return items;
}

// AdamW tiles of the matrices with a transposed copy. dst offsets are relative to shadow_t; the
// token embedding's copy ([C, ldl]) starts at wte_off_t.
std::vector<AdamTile> make_adam_tiles(const gpt2_config* c, size_t wte_off_t, int ldl) {
  std::vector<AdamTile> tiles;
  size_t off = 0;
  bool first = true;
  for (const TensorDesc& t : tensor_list(c)) {
    if (t.rows > 0) {
      const size_t base_t = first ? wte_off_t : off;  // the copy of a layer matrix sits at its offset
      const int ldd = first ? ldl : t.rows;
      for (int r0 = 0; r0 < t.rows; r0 += ADAM_TR)
        for (int c0 = 0; c0 < t.cols; c0 += ADAM_TC) {
          AdamTile a{};
          a.off = off + (size_t)r0 * t.cols + c0;
          a.dst_off = base_t + (size_t)c0 * ldd + r0;
          a.rows = std::min(ADAM_TR, t.rows - r0);
          a.cols = std::min(ADAM_TC, t.cols - c0);
          a.ld = t.cols;
          a.ldd = ldd;
          tiles.push_back(a);
        }
    }
    first = false;
    off += t.size;
  }
  return tiles;
}

// Carve the arena. With base == nullptr only the size is computed.
size_t plan(const gpt2_config* c, Model* m, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    off = round_up(off, 256);
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  const size_t N = layout(c, nullptr);
  const size_t es = c->precision == GPT2_BF16 ? 2 : 4;
  const size_t B = c->batch, T = c->seq, BT = B * T, C = c->n_embd, H = c->n_head, L = c->n_layer;
  const size_t ldl = round_up(c->padded_vocab, 8);
  const size_t nitems = make_items(c).size();

  Model tmp;
  Model* M = m ? m : &tmp;
  M->params = c->no_master ? nullptr : (float*)take(N * 4);
  M->grads = (float*)take(N * 4);
  M->m = (float*)take(N * 4);
  M->v = (float*)take(N * 4);
  M->shadow = c->precision == GPT2_BF16 ? (uint16_t*)take(N * 2) : nullptr;
  if (c->precision == GPT2_BF16) {
    M->shadow_t = (uint16_t*)take(N * 2);
    M->wte_t = (uint16_t*)take(C * ldl * 2);
    M->tr_items = (TransItem*)take((1 + 4 * L) * sizeof(TransItem));
  }
  M->items = (WorkItem*)take(nitems * sizeof(WorkItem));
  if (c->precision == GPT2_BF16) {
    M->adam_items = (WorkItem*)take(make_items(c, true).size() * sizeof(WorkItem));
    M->adam_tiles = (AdamTile*)take(make_adam_tiles(c, 0, (int)ldl).size() * sizeof(AdamTile));
  }
  M->encoded = take(BT * C * es);
  M->la.resize(L);
  const int rc = c->recompute;
  char* gelu_shared = rc >= 1 ? take(BT * 4 * C * es) : nullptr;
  char* ln_shared = rc >= 2 ? take(BT * C * es) : nullptr;
  for (size_t l = 0; l < L; ++l) {
    LayerAct& a = M->la[l];
    a.ln1 = rc >= 2 ? ln_shared : take(BT * C * es);
    a.ln1_mean = (float*)take(BT * 4);
    a.ln1_rstd = (float*)take(BT * 4);
    a.qkv = take(BT * 3 * C * es);
    a.atty = take(BT * C * es);
    a.lse = (float*)take(B * H * T * 4);
    a.res1 = take(BT * C * es);
    a.ln2 = rc >= 2 ? ln_shared : take(BT * C * es);
    a.ln2_mean = (float*)take(BT * 4);
    a.ln2_rstd = (float*)take(BT * 4);
    a.fch = take(BT * 4 * C * es);
    a.fchg = rc >= 1 ? gelu_shared : take(BT * 4 * C * es);
    a.res2 = take(BT * C * es);
  }
  M->lnf = take(BT * C * es);
  M->lnf_mean = (float*)take(BT * 4);
  M->lnf_rstd = (float*)take(BT * 4);
  M->logits = take(BT * ldl * es);
  M->losses = (float*)take(BT * 4);
  M->dres = take(BT * C * es);
  M->dbuf1 = take(BT * 4 * C * es);
  M->dbuf2 = take(BT * C * es);
  M->dvec = (float*)take(B * H * T * 4);
  M->keys = (uint32_t*)take(BT * 4);
  size_t sf = std::max<size_t>(8 * 4 * C * C, (size_t)ldl * C * 3);  // split-K partials of the dW GEMMs
  sf = std::max(sf, layernorm_bwd_partial_floats((int)BT, (int)C));
  sf = std::max(sf, encoder_bwd_partial_floats((int)BT, (int)C));
  sf = std::max<size_t>(sf, (size_t)512 * 4 * C);  // column-sum partials (separate or in a GEMM epilogue)
  M->scratch_floats = sf;
  M->scratch = (float*)take(sf * 4);
  // deferred column-sum partials: 2L + 1 LayerNorm backwards, L fused fc bias sums (fcproj input
  // gradient epilogue), L qkv bias sums (attention backward), and the batch table (32 columns a block)
  const size_t nln = 2 * L + 1;
  M->defer_floats = nln * layernorm_bwd_partial_floats((int)BT, (int)C) +
                    L * (size_t)gemm_colsum_rows_max((int)BT) * 4 * C +
                    L * (size_t)attention_bias_partial_rows((int)B, (int)T) * 3 * C;
  M->defer = (float*)take(M->defer_floats * 4);
  M->fin_cap = nln * 3 * cdiv(C, 32) + L * cdiv(4 * C, 32) + L * cdiv(3 * C, 32);
  M->fin_dev = (FinishBlock*)take(M->fin_cap * sizeof(FinishBlock));
  M->norm_partial = (double*)take(NORM_PARTS * 8);
  M->norm2 = (double*)take(8);
  M->clip_scale = (float*)take(4);
  M->range_items = (WorkItem*)take(nitems * sizeof(WorkItem));  // a range cuts each item to at most one piece
  M->range_norm2 = (double*)take(8);
  M->range_scale = (float*)take(4);
  M->loss_dev = (float*)take(4);
  M->dloss_dev = (float*)take(4);
  M->nvalid_dev = (int*)take(4);
  M->err_dev = (int*)take(4);
  return round_up(off, 256);
}



// ------------------------------------------------------------------ per-class kernel timing
// HIP events recorded on the model's stream around every launch of an enabled class.
struct Prof {
  uint32_t mask = 0;
  std::vector<hipEvent_t> pool;
  std::vector<std::pair<int, int>> recs;  // (class, first event index)
  int used = 0;
};
Prof prof;

struct ProfScope {
  int cls, idx = -1;
  explicit ProfScope(int c) : cls(c) {
    if (!(prof.mask >> c & 1u)) return;
    if (prof.used + 2 > (int)prof.pool.size()) {
      for (int i = 0; i < 512; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        prof.pool.push_back(e);
      }
    }
    idx = prof.used;
    prof.used += 2;
    (void)hipEventRecord(prof.pool[idx], g.stream);
  }
  ~ProfScope() {
    if (idx < 0) return;
    (void)hipEventRecord(prof.pool[idx + 1], g.stream);
    prof.recs.push_back({cls, idx});
  }
};

// weight pointer in the compute dtype (bf16 shadow or fp32 master)
const void* W(size_t off) {
  if (off == NONE) return nullptr;
  if (g.dt == DT_BF16) return g.shadow + off;
  return g.params + off;
}
float* G(size_t off) { return off == NONE ? nullptr : g.grads + off; }
// transposed bf16 copy of a layer weight matrix (bf16 runs only)
const void* WT(size_t off) { return g.shadow_t + off; }

// The transposed copies: the token embedding [Vp, C] -> [C, ldl], each layer's qkvw [3C, C],
// attprojw [C, C], fcw [4C, C] and fcprojw [C, 4C] -> their transposes at the same offsets.
void make_trans_items() {
  g.tr_host.clear();
  g.tr_tiles = 0;
  auto add = [&](size_t src_off, size_t dst_off, int rows, int cols, int ldd) {
    TransItem t{};
    t.src_off = src_off;
    t.dst_off = dst_off;
    t.rows = rows;
    t.cols = cols;
    t.ldd = ldd;
    t.tile0 = g.tr_tiles;
    g.tr_tiles += trans_tiles(rows, cols);
    g.tr_host.push_back(t);
  };
  const int C = g.C;
  add(g.o_wte, (size_t)(g.wte_t - g.shadow_t), g.Vp, C, g.ldl);
  for (int l = 0; l < g.L; ++l) {
    const LayerOff& o = g.lo[l];
    add(o.qkvw, o.qkvw, 3 * C, C, 3 * C);
    add(o.attprojw, o.attprojw, C, C, C);
    add(o.fcw, o.fcw, 4 * C, C, 4 * C);
    add(o.fcprojw, o.fcprojw, C, 4 * C, C);
  }
}
hipError_t refresh_transposed() {
  if (!g.shadow_t) return hipSuccess;
  ProfScope ps_(GPT2_K_WEIGHT_TRANSPOSE);
  return launch_transpose_bf16(g.tr_items, (int)g.tr_host.size(), g.tr_tiles, g.shadow, g.shadow_t, g.stream);
}

int gemm(bool akc, bool bkc, Epi epi, int M, int N, int K, const void* A, long lda, const void* Bp, long ldb,
         void* Cp, long ldc, const void* bias = nullptr, const void* aux = nullptr, long ldaux = 0,
         void* C2 = nullptr, int accumulate = 0, bool split = false, float* colsum = nullptr, int colsum_acc = 0,
         ColsumDefer* colsum_defer = nullptr) {
  GemmArgs a{};
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = A;
  a.lda = lda;
  a.B = Bp;
  a.ldb = ldb;
  a.C = Cp;
  a.ldc = ldc;
  a.bias = bias;
  a.aux = aux;
  a.ldaux = ldaux;
  a.C2 = C2;
  a.accumulate = accumulate;
  a.colsum = colsum;
  a.colsum_accumulate = colsum_acc;
  a.colsum_defer = colsum_defer;
  const bool scr = split || colsum;
  HIPCHK(launch_gemm(g.dt, akc, bkc, epi, a, scr ? g.scratch : nullptr, scr ? g.scratch_floats : 0, g.stream));
  return GPT2_OK;
}

#define RUN(x)                   \
  do {                           \
    int r_ = (x);                \
    if (r_ != GPT2_OK) return r_; \
  } while (0)

__global__ void set_scalars_kernel(int* err) { *err = 0; }

int forward_impl(const int32_t* tokens, const int32_t* targets) {
  const int BT = g.BT, C = g.C, L = g.L;
  const size_t es = g.es;
  hipStream_t s = g.stream;
  if (g.transposed_stale) {  // after range updates: the backward reads the transposed copies
    HIPCHK(refresh_transposed());
    g.transposed_stale = false;
  }
  set_scalars_kernel<<<1, 1, 0, s>>>(g.err_dev);
  {
      ProfScope ps_(GPT2_K_ENCODER_FWD);
      HIPCHK(launch_encoder_fwd(g.dt, g.B, g.T, C, g.V, tokens, W(g.o_wte), W(g.o_wpe), g.encoded, g.err_dev, s));
    }
  if (targets) {
    HIPCHK(hipEventRecord(g.ev_tokens, s));
    HIPCHK(hipStreamWaitEvent(g.side, g.ev_tokens, 0));
    HIPCHK(launch_encoder_sort(BT, g.V, tokens, g.keys, g.side));
    HIPCHK(hipEventRecord(g.ev_sorted, g.side));
  }
  const char* x = g.encoded;
  for (int l = 0; l < L; ++l) {
    const LayerOff& o = g.lo[l];
    LayerAct& a = g.la[l];
    {
      ProfScope ps_(GPT2_K_LAYERNORM_FWD);
      HIPCHK(launch_layernorm_fwd(g.dt, BT, C, x, W(o.ln1w), W(o.ln1b), a.ln1, a.ln1_mean, a.ln1_rstd, s));
    }
    {
      ProfScope ps_(GPT2_K_GEMM_QKV);
      RUN(gemm(true, true, EPI_BIAS, BT, 3 * C, C, a.ln1, C, W(o.qkvw), C, a.qkv, 3 * C, W(o.qkvb)));
    }
    {
      ProfScope ps_(GPT2_K_ATTENTION_FWD);
      HIPCHK(launch_attention_fwd(g.dt, g.B, g.T, g.H, C / g.H, a.qkv, a.atty, a.lse, s));
    }
    {
      ProfScope ps_(GPT2_K_GEMM_ATTPROJ);
      RUN(gemm(true, true, EPI_RESID, BT, C, C, a.atty, C, W(o.attprojw), C, a.res1, C, W(o.attprojb), x, C));
    }
    {
      ProfScope ps_(GPT2_K_LAYERNORM_FWD);
      HIPCHK(launch_layernorm_fwd(g.dt, BT, C, a.res1, W(o.ln2w), W(o.ln2b), a.ln2, a.ln2_mean, a.ln2_rstd, s));
    }
    {
      ProfScope ps_(GPT2_K_GEMM_FC);
      // fch = gelu'(z), fchg = gelu(z); with recompute fch = z
      RUN(gemm(true, true, g.cfg.recompute >= 1 ? EPI_GELU : EPI_GELU_GRAD, BT, 4 * C, C, a.ln2, C, W(o.fcw), C,
               a.fch, 4 * C, W(o.fcb), nullptr, 0, a.fchg));
    }
    {
      ProfScope ps_(GPT2_K_GEMM_FCPROJ);
      RUN(gemm(true, true, EPI_RESID, BT, C, 4 * C, a.fchg, 4 * C, W(o.fcprojw), 4 * C, a.res2, C, W(o.fcprojb),
             a.res1, C));
    }
    x = a.res2;
  }
  {
      ProfScope ps_(GPT2_K_LAYERNORM_FWD);
      HIPCHK(launch_layernorm_fwd(g.dt, BT, C, x, W(g.o_lnfw), W(g.o_lnfb), g.lnf, g.lnf_mean, g.lnf_rstd, s));
    }
  {
      ProfScope ps_(GPT2_K_GEMM_CLASSIFIER);
      RUN(gemm(true, true, EPI_BIAS, BT, g.Vp, C, g.lnf, C, W(g.o_wte), C, g.logits, g.ldl));
    }
  if (targets) {
    HIPCHK(launch_count_targets(targets, BT, g.V, g.cfg.grad_accum, g.dloss_dev, g.nvalid_dev, g.err_dev, s));
    {
      ProfScope ps_(GPT2_K_CROSS_ENTROPY);
      HIPCHK(launch_cross_entropy(g.dt, BT, g.V, g.ldl, g.logits, targets, g.dloss_dev, g.losses, s));
    }
    HIPCHK(launch_loss_mean(g.losses, BT, g.nvalid_dev, g.loss_dev, s));
    HIPCHK(hipMemcpyAsync(g.pinned, g.loss_dev, 4, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamWaitEvent(s, g.ev_sorted, 0));  // tokens are no longer read after this call
  }
  HIPCHK(hipMemcpyAsync(g.pinned + 1, g.err_dev, 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  (void)es;
  return GPT2_OK;
}

// Room in the deferred-partials region for the next launcher.
ColsumDefer defer_slot() { return ColsumDefer{g.defer + g.defer_used, g.defer_floats - g.defer_used, 0}; }
// List the blocks of one deferred column sum: out[c] (+)= sum_{y < rows} part[y ld + c], c < ncols.
int defer_sum(const float* part, long ld, int rows, int ncols, float* out) {
  const int nch = cdiv(ncols, 32);
  if (!out) return GPT2_OK;
  if (g.fin_host.size() + nch > g.fin_cap) return fail(GPT2_ESTATE, "internal: deferred column sums exceed their table");
  for (int ch = 0; ch < nch; ++ch) g.fin_host.push_back(FinishBlock{part, out, ld, rows, ncols, ch, 0});
  return GPT2_OK;
}

int backward_impl() {
  const int BT = g.BT, C = g.C, L = g.L;
  const int acc = g.micro > 0 ? 1 : 0;
  const bool lb = g.cfg.linear_bias != 0;
  hipStream_t s = g.stream;
  float* sc = g.scratch;
  const size_t sf = g.scratch_floats;
  g.fin_host.clear();
  g.defer_used = 0;
  // LayerNorm backward into dres; its column sums (dw, db, and dsum when set) go to the batched finish
  auto ln_bwd = [&](const void* dy, const void* x, const void* w, const float* mean, const float* rstd, int add,
                    float* dw, float* db, float* dsum) -> int {
    ColsumDefer d = defer_slot();
    HIPCHK(launch_layernorm_bwd(g.dt, BT, C, dy, x, w, mean, rstd, g.dres, add, dw, db, dsum, acc, sc, sf, s, &d));
    if (d.rows > 0) {
      RUN(defer_sum(d.part, 3L * C, d.rows, C, dw));
      RUN(defer_sum(d.part + C, 3L * C, d.rows, C, db));
      if (dsum) RUN(defer_sum(d.part + 2 * C, 3L * C, d.rows, C, dsum));
      g.defer_used += (size_t)d.rows * 3 * C;
    }
    return GPT2_OK;
  };
  // classifier (tied wte): dz = dlogits wte ; dwte (+)= dlogits^T z
  {
      ProfScope ps_(GPT2_K_GEMM_CLASSIFIER_DX);
      if (g.wte_t) RUN(gemm(true, true, EPI_BIAS, BT, C, g.Vp, g.logits, g.ldl, g.wte_t, g.ldl, g.dbuf2, C));
      else RUN(gemm(true, false, EPI_BIAS, BT, C, g.Vp, g.logits, g.ldl, W(g.o_wte), C, g.dbuf2, C));
    }
  {
      ProfScope ps_(GPT2_K_GEMM_CLASSIFIER_DW);
      RUN(gemm(false, false, EPI_F32, g.Vp, C, BT, g.logits, g.ldl, g.lnf, C, G(g.o_wte), C, nullptr, nullptr, 0,
           nullptr, acc, true));
    }
  const char* xlast = L > 0 ? g.la[L - 1].res2 : g.encoded;
  {
      ProfScope ps_(GPT2_K_LAYERNORM_BWD);
      // the column sums of the dres it writes are the bias gradient of the last fcproj
      float* dsum = (lb && L > 0) ? G(g.lo[L - 1].fcprojb) : nullptr;
      RUN(ln_bwd(g.dbuf2, xlast, W(g.o_lnfw), g.lnf_mean, g.lnf_rstd, 0, G(g.o_lnfw), G(g.o_lnfb), dsum));
    }
  for (int l = L - 1; l >= 0; --l) {
    const LayerOff& o = g.lo[l];
    LayerAct& a = g.la[l];
    const char* xin = l > 0 ? g.la[l - 1].res2 : g.encoded;
    // fcproj: res2 = res1 + gelu(z) Wfcproj^T + b ; dz = (dres Wfcproj) * gelu'(z)
    {
      ProfScope ps_(GPT2_K_GEMM_FCPROJ_DX);
      // dz = (dres Wfcproj) * gelu'(z) (gelu'(z) stored, or from z with recompute); its column sums
      // are the fc bias gradient
      float* dfcb = lb ? G(o.fcb) : nullptr;
      const Epi ep = g.cfg.recompute >= 1 ? EPI_GELU_BWD : EPI_MUL;
      ColsumDefer d = defer_slot();
      if (g.shadow_t)
        RUN(gemm(true, true, ep, BT, 4 * C, C, g.dres, C, WT(o.fcprojw), C, g.dbuf1, 4 * C, nullptr, a.fch, 4 * C,
                 nullptr, 0, false, dfcb, acc, &d));
      else
        RUN(gemm(true, false, ep, BT, 4 * C, C, g.dres, C, W(o.fcprojw), 4 * C, g.dbuf1, 4 * C, nullptr, a.fch,
                 4 * C, nullptr, 0, false, dfcb, acc, &d));
      if (d.rows > 0) {
        RUN(defer_sum(d.part, 4L * C, d.rows, 4 * C, dfcb));
        g.defer_used += (size_t)d.rows * 4 * C;
      }
    }
    if (g.cfg.recompute >= 1) {  // gelu(z) again, for the fcproj weight gradient
      ProfScope ps_(GPT2_K_RECOMPUTE);
      HIPCHK(launch_gelu(g.dt, a.fch, a.fchg, (size_t)BT * 4 * C, s));
    }
    {
      ProfScope ps_(GPT2_K_GEMM_FCPROJ_DW);
      RUN(gemm(false, false, EPI_F32, C, 4 * C, BT, g.dres, C, a.fchg, 4 * C, G(o.fcprojw), 4 * C, nullptr, nullptr,
             0, nullptr, acc, true));
    }
    // (the fcproj bias gradient, the column sums of dres, came with the LayerNorm backward above)
    // fc: z = ln2 Wfc^T + b (fch = gelu'(z), fchg = gelu(z))
    {
      ProfScope ps_(GPT2_K_GEMM_FC_DX);
      if (g.shadow_t) RUN(gemm(true, true, EPI_BIAS, BT, C, 4 * C, g.dbuf1, 4 * C, WT(o.fcw), 4 * C, g.dbuf2, C));
      else RUN(gemm(true, false, EPI_BIAS, BT, C, 4 * C, g.dbuf1, 4 * C, W(o.fcw), C, g.dbuf2, C));
    }
    if (g.cfg.recompute >= 2) {  // ln2 again, for the fc weight gradient
      ProfScope ps_(GPT2_K_RECOMPUTE);
      HIPCHK(launch_layernorm_fwd(g.dt, BT, C, a.res1, W(o.ln2w), W(o.ln2b), a.ln2, a.ln2_mean, a.ln2_rstd, s));
    }
    {
      ProfScope ps_(GPT2_K_GEMM_FC_DW);
      RUN(gemm(false, false, EPI_F32, 4 * C, C, BT, g.dbuf1, 4 * C, a.ln2, C, G(o.fcw), C, nullptr, nullptr, 0,
             nullptr, acc, true));
    }
    {
      ProfScope ps_(GPT2_K_LAYERNORM_BWD);
      // + column sums of the updated dres = the attproj bias gradient
      RUN(ln_bwd(g.dbuf2, a.res1, W(o.ln2w), a.ln2_mean, a.ln2_rstd, 1, G(o.ln2w), G(o.ln2b),
                 lb ? G(o.attprojb) : nullptr));
    }
    // attproj: res1 = xin + atty Wproj^T + b
    {
      ProfScope ps_(GPT2_K_GEMM_ATTPROJ_DX);
      if (g.shadow_t) RUN(gemm(true, true, EPI_BIAS, BT, C, C, g.dres, C, WT(o.attprojw), C, g.dbuf2, C));
      else RUN(gemm(true, false, EPI_BIAS, BT, C, C, g.dres, C, W(o.attprojw), C, g.dbuf2, C));
    }
    // (the attproj weight gradient, dres^T atty, is taken together with the qkv one below)
    if (g.dt != DT_BF16) {  // bf16: D comes out of the dQ kernel
      ProfScope ps_(GPT2_K_ATTENTION_BWD_PRE);
      HIPCHK(launch_attention_bwd(g.dt, g.B, g.T, g.H, C / g.H, a.qkv, a.atty, g.dbuf2, a.lse, g.dbuf1, g.dvec,
                                  ATT_BWD_PRE, s));
    }
    // bf16: the attention kernels also leave the column partials of dqkv (the qkv bias gradient),
    // summed in the batched finish
    const int arows = attention_bias_partial_rows(g.B, g.T);
    const ColsumDefer ad = defer_slot();
    const bool adefer = (size_t)arows * 3 * C <= ad.cap;
    float* csa = (lb && g.dt == DT_BF16) ? (adefer ? ad.part : sc) : nullptr;
    {  // (first: it also forms D = rowsum(dO * O) for the dK/dV kernel)
      ProfScope ps_(GPT2_K_ATTENTION_BWD_Q);
      HIPCHK(launch_attention_bwd(g.dt, g.B, g.T, g.H, C / g.H, a.qkv, a.atty, g.dbuf2, a.lse, g.dbuf1, g.dvec,
                                  ATT_BWD_Q, s, csa));
    }
    {
      ProfScope ps_(GPT2_K_ATTENTION_BWD);
      HIPCHK(launch_attention_bwd(g.dt, g.B, g.T, g.H, C / g.H, a.qkv, a.atty, g.dbuf2, a.lse, g.dbuf1, g.dvec,
                                  ATT_BWD_KV, s, csa));
    }
    if (csa && adefer) {
      RUN(defer_sum(csa, 3L * C, arows, 3 * C, G(o.qkvb)));
      g.defer_used += (size_t)arows * 3 * C;
    } else if (csa) {
      ProfScope ps_(GPT2_K_BIAS_GRAD);
      HIPCHK(launch_colsum_finish(csa, arows, 3 * C, G(o.qkvb), acc, s));
    } else if (lb) {
      ProfScope ps_(GPT2_K_BIAS_GRAD);
      HIPCHK(launch_colsum(g.dt, g.dbuf1, 3 * C, BT, 3 * C, G(o.qkvb), acc, sc, sf, s));
    }
    // qkv = ln1 Wqkv^T + b
    {
      ProfScope ps_(GPT2_K_GEMM_QKV_DX);
      if (g.shadow_t) RUN(gemm(true, true, EPI_BIAS, BT, C, 3 * C, g.dbuf1, 3 * C, WT(o.qkvw), 3 * C, g.dbuf2, C));
      else RUN(gemm(true, false, EPI_BIAS, BT, C, 3 * C, g.dbuf1, 3 * C, W(o.qkvw), C, g.dbuf2, C));
    }
    if (g.cfg.recompute >= 2) {  // ln1 again, for the qkv weight gradient
      ProfScope ps_(GPT2_K_RECOMPUTE);
      HIPCHK(launch_layernorm_fwd(g.dt, BT, C, xin, W(o.ln1w), W(o.ln1b), a.ln1, a.ln1_mean, a.ln1_rstd, s));
    }
    {
      // the qkv and attproj weight gradients in one split-K launch (dres still holds the gradient
      // at the attention block's output: nothing above touched it)
      ProfScope ps_(GPT2_K_GEMM_QKV_DW);
      GemmArgs q{}, pj{};
      q.M = 3 * C;
      q.N = C;
      q.K = BT;
      q.A = g.dbuf1;
      q.lda = 3 * C;
      q.B = a.ln1;
      q.ldb = C;
      q.C = G(o.qkvw);
      q.ldc = C;
      q.accumulate = acc;
      pj = q;
      pj.M = C;
      pj.A = g.dres;
      pj.lda = C;
      pj.B = a.atty;
      pj.C = G(o.attprojw);
      HIPCHK(launch_gemm_f32_pair(g.dt, false, false, q, pj, g.scratch, g.scratch_floats, s));
    }
    {
      ProfScope ps_(GPT2_K_LAYERNORM_BWD);
      // + column sums of the updated dres = the fcproj bias gradient of the layer below
      float* dsum = (lb && l > 0) ? G(g.lo[l - 1].fcprojb) : nullptr;
      RUN(ln_bwd(g.dbuf2, xin, W(o.ln1w), a.ln1_mean, a.ln1_rstd, 1, G(o.ln1w), G(o.ln1b), dsum));
    }
  }
  if (!g.fin_host.empty()) {
    ProfScope ps_(GPT2_K_GRAD_FINISH);
    const size_t nb = g.fin_host.size();
    if (g.fin_up.size() != nb || memcmp(g.fin_up.data(), g.fin_host.data(), nb * sizeof(FinishBlock)) != 0) {
      // a new table (the first backward: it stays the same while the configuration does); wait
      // for an earlier copy out of the host list before replacing it
      HIPCHK(hipStreamSynchronize(s));
      g.fin_up = g.fin_host;
      HIPCHK(hipMemcpyAsync(g.fin_dev, g.fin_up.data(), nb * sizeof(FinishBlock), hipMemcpyHostToDevice, s));
    }
    HIPCHK(launch_finish_batch(g.fin_dev, (int)nb, acc, s));
  }
  HIPCHK(hipStreamWaitEvent(s, g.ev_sorted, 0));
  {
      ProfScope ps_(GPT2_K_ENCODER_BWD);
      HIPCHK(launch_encoder_bwd(g.dt, g.B, g.T, g.maxT, C, g.keys, g.dres, G(g.o_wte), G(g.o_wpe), acc, sc, sf, s));
    }
  return GPT2_OK;
}

int check_ready() {
  if (!g.ready) return fail(GPT2_ESTATE, "gpt2_init has not succeeded");
  return GPT2_OK;
}

}  // namespace

// ===================================================================================== C ABI
extern "C" {

uint64_t gpt2_workspace_bytes(const gpt2_config* cfg) {
  if (const char* e = check_config(cfg)) {
    fail(GPT2_EINVAL, "%s", e);
    return 0;
  }
  ok();
  return plan(cfg, nullptr, nullptr);
}

void gpt2_free(void) {
  if (g.stream) (void)hipStreamSynchronize(g.stream);
  if (g.side) (void)hipStreamSynchronize(g.side);
  if (g.pinned) (void)hipHostFree(g.pinned);
  if (g.ev_tokens) (void)hipEventDestroy(g.ev_tokens);
  if (g.ev_sorted) (void)hipEventDestroy(g.ev_sorted);
  if (g.side) (void)hipStreamDestroy(g.side);
  g = Model();
}

int gpt2_init(const gpt2_config* cfg, uint64_t seed) {
  gpt2_free();
  if (const char* e = check_config(cfg)) return fail(GPT2_EINVAL, "%s", e);
  const size_t need = plan(cfg, nullptr, nullptr);
  if (!cfg->workspace || cfg->workspace_bytes < need)
    return fail(GPT2_ENOMEM, "workspace of %llu bytes < %llu needed", (unsigned long long)cfg->workspace_bytes,
                (unsigned long long)need);
  if (reinterpret_cast<uintptr_t>(cfg->workspace) % 256) return fail(GPT2_EINVAL, "workspace must be 256-byte aligned");
  g.cfg = *cfg;
  g.dt = cfg->precision == GPT2_BF16 ? DT_BF16 : DT_F32;
  g.es = g.dt == DT_BF16 ? 2 : 4;
  g.L = cfg->n_layer;
  g.H = cfg->n_head;
  g.C = cfg->n_embd;
  g.V = cfg->vocab;
  g.Vp = cfg->padded_vocab;
  g.maxT = cfg->max_seq;
  g.B = cfg->batch;
  g.T = cfg->seq;
  g.BT = g.B * g.T;
  g.ldl = (int)round_up(g.Vp, 8);
  g.N = layout(cfg, &g);
  g.items_host = make_items(cfg);
  plan(cfg, &g, reinterpret_cast<char*>(cfg->workspace));
  g.stream = reinterpret_cast<hipStream_t>(cfg->stream);
  HIPCHK(hipHostMalloc((void**)&g.pinned, 16, hipHostMallocDefault));
  HIPCHK(hipStreamCreateWithFlags(&g.side, hipStreamNonBlocking));
  HIPCHK(hipEventCreateWithFlags(&g.ev_tokens, hipEventDisableTiming));
  HIPCHK(hipEventCreateWithFlags(&g.ev_sorted, hipEventDisableTiming));
  HIPCHK(hipMemcpyAsync(g.items, g.items_host.data(), g.items_host.size() * sizeof(WorkItem), hipMemcpyHostToDevice,
                        g.stream));
  g.seed = seed;
  // without an fp32 master the fp32 initial values pass through the gradient buffer
  float* p0 = g.params ? g.params : g.grads;
  HIPCHK(launch_init_params(g.items, (int)g.items_host.size(), p0, seed, 0.02, g.stream));
  if (g.shadow) HIPCHK(launch_to_bf16(p0, g.shadow, g.N, g.stream));
  HIPCHK(launch_fill_f32(g.m, g.N, 0.f, g.stream));
  HIPCHK(launch_fill_f32(g.v, g.N, 0.f, g.stream));
  HIPCHK(launch_fill_f32(g.grads, g.N, 0.f, g.stream));
  if (g.shadow_t) {
    make_trans_items();
    HIPCHK(hipMemcpyAsync(g.tr_items, g.tr_host.data(), g.tr_host.size() * sizeof(TransItem), hipMemcpyHostToDevice,
                          g.stream));
    HIPCHK(refresh_transposed());
    g.adam_items_host = make_items(cfg, true);
    g.adam_tiles_host = make_adam_tiles(cfg, (size_t)(g.wte_t - g.shadow_t), g.ldl);
    HIPCHK(hipMemcpyAsync(g.adam_items, g.adam_items_host.data(), g.adam_items_host.size() * sizeof(WorkItem),
                          hipMemcpyHostToDevice, g.stream));
    HIPCHK(hipMemcpyAsync(g.adam_tiles, g.adam_tiles_host.data(), g.adam_tiles_host.size() * sizeof(AdamTile),
                          hipMemcpyHostToDevice, g.stream));
  }
  HIPCHK(hipStreamSynchronize(g.stream));
  g.ready = true;
  return ok();
}

float gpt2_forward(const int32_t* tokens, const int32_t* targets) {
  if (check_ready() != GPT2_OK) return NAN;
  if (!tokens) {
    fail(GPT2_EINVAL, "tokens is NULL");
    return NAN;
  }
  g.fwd_targets = false;
  g.fwd_logits = false;
  if (forward_impl(tokens, targets) != GPT2_OK) return NAN;
  const int err = *reinterpret_cast<int*>(g.pinned + 1);
  if (err) {
    fail(GPT2_ERANGE, "%s", (err & 1) ? "token id outside [0, vocab)" : "target outside [-1, vocab)");
    return NAN;
  }
  ok();
  if (!targets) {
    g.fwd_logits = true;
    return NAN;
  }
  g.fwd_targets = true;
  return g.pinned[0];
}

int gpt2_backward(void) {
  RUN(check_ready());
  if (!g.fwd_targets) return fail(GPT2_ESTATE, "gpt2_backward needs a preceding gpt2_forward with targets");
  RUN(backward_impl());
  g.fwd_targets = false;
  g.micro++;
  return ok();
}

static AdamArgs adam_args(float lr, float b1, float b2, float eps, float wd, int32_t t) {
  AdamArgs a;
  a.lr = lr;
  a.b1 = b1;
  a.b2 = b2;
  a.eps = eps;
  a.wd = wd;
  a.bc1 = (float)(1.0 / (1.0 - pow((double)b1, (double)t)));
  a.bc2 = (float)(1.0 / (1.0 - pow((double)b2, (double)t)));
  a.clip = g.cfg.grad_clip;
  a.no_master = g.cfg.no_master;
  a.t = t;
  a.sr_seed = g.seed ^ 0xD1B54A32D192ED03ull;
  return a;
}

int gpt2_adamw_step(float lr, float b1, float b2, float eps, float wd, int32_t t) {
  RUN(check_ready());
  if (t < 1) return fail(GPT2_EINVAL, "t must be >= 1");
  if (g.micro == 0) return fail(GPT2_ESTATE, "gpt2_adamw_step needs at least one gpt2_backward since the last update");
  hipStream_t s = g.stream;
  {
      ProfScope ps_(GPT2_K_GRAD_NORM);
      HIPCHK(launch_sumsq_partial(g.grads, g.N, g.norm_partial, NORM_PARTS, s));
    }
  HIPCHK(launch_grad_norm_finish(g.norm_partial, NORM_PARTS, g.norm2, g.clip_scale, g.cfg.grad_clip, s));
  const AdamArgs a = adam_args(lr, b1, b2, eps, wd, t);
  {
      ProfScope ps_(GPT2_K_ADAMW);
      if (g.shadow_t) {  // flat items for the small tensors, tiles (with their transposed copies) for the matrices
        HIPCHK(launch_adamw(g.adam_items, (int)g.adam_items_host.size(), g.params, g.grads, g.m, g.v, g.shadow,
                            g.clip_scale, g.norm2, a, s));
        HIPCHK(launch_adamw_tiles(g.adam_tiles, (int)g.adam_tiles_host.size(), g.params, g.grads, g.m, g.v, g.shadow,
                                  g.shadow_t, g.clip_scale, g.norm2, a, s));
        g.transposed_stale = false;  // the tiles rewrote every transposed copy
      } else {
        HIPCHK(launch_adamw(g.items, (int)g.items_host.size(), g.params, g.grads, g.m, g.v, g.shadow, g.clip_scale,
                            g.norm2, a, s));
      }
    }
  g.micro = 0;
  return ok();
}

float gpt2_grad_norm(void) {
  if (check_ready() != GPT2_OK) return NAN;
  double n2 = 0;
  hipError_t e = hipMemcpyAsync(&n2, g.norm2, 8, hipMemcpyDeviceToHost, g.stream);
  if (e == hipSuccess) e = hipStreamSynchronize(g.stream);
  if (e != hipSuccess) {
    fail(GPT2_EHIP, "gpt2_grad_norm: %s", hipGetErrorString(e));
    return NAN;
  }
  ok();
  return (float)sqrt(n2);
}


// ------------------------------------------------------------------ one rank's share of a sharded update
static int range_check(uint64_t begin, uint64_t end) {
  if (begin > end || end > g.N || begin % 4 || end % 4)
    return fail(GPT2_EINVAL, "need 0 <= begin <= end <= num_params (%zu), both multiples of 4", g.N);
  return GPT2_OK;
}

int gpt2_grad_sumsq_range(uint64_t begin, uint64_t end, double* sumsq) {
  RUN(check_ready());
  if (!sumsq) return fail(GPT2_EINVAL, "sumsq is NULL");
  RUN(range_check(begin, end));
  hipStream_t s = g.stream;
  // the partial sums and their fixed-order finish of the full norm, over the range
  HIPCHK(launch_sumsq_partial(g.grads + begin, end - begin, g.norm_partial, NORM_PARTS, s));
  HIPCHK(launch_grad_norm_finish(g.norm_partial, NORM_PARTS, g.range_norm2, g.range_scale, 0.f, s));
  HIPCHK(hipMemcpyAsync(&g.range_vals.n2, g.range_norm2, 8, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  *sumsq = g.range_vals.n2;
  return ok();
}

int gpt2_adamw_step_range(float lr, float b1, float b2, float eps, float wd, int32_t t, uint64_t begin, uint64_t end,
                          double global_sumsq, int finish) {
  RUN(check_ready());
  if (t < 1) return fail(GPT2_EINVAL, "t must be >= 1");
  if (g.micro == 0)
    return fail(GPT2_ESTATE, "gpt2_adamw_step_range needs at least one gpt2_backward since the last update");
  RUN(range_check(begin, end));
  hipStream_t s = g.stream;
  HIPCHK(hipStreamSynchronize(s));  // the host copies below are free to change
  // the clip scale from the caller's global norm, as the norm kernel forms it for the full update
  const double nrm = sqrt(global_sumsq);
  const float clip = g.cfg.grad_clip;
  g.range_vals.n2 = global_sumsq;
  g.range_vals.scale = (clip > 0.f && nrm > (double)clip) ? (float)((double)clip / nrm) : 1.0f;
  HIPCHK(hipMemcpyAsync(g.range_norm2, &g.range_vals.n2, 8, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(g.range_scale, &g.range_vals.scale, 4, hipMemcpyHostToDevice, s));
  // the flat work items (runs of one tensor, each with its tensor's decay flag) cut to the range
  g.range_host.clear();
  for (const WorkItem& it : g.items_host) {
    const uint64_t lo = std::max<uint64_t>(it.off, begin), hi = std::min<uint64_t>(it.off + it.len, end);
    if (lo >= hi) continue;
    WorkItem r = it;
    r.off = lo;
    r.len = (uint32_t)(hi - lo);
    r.normal0 = it.normal0 + (lo - it.off);
    g.range_host.push_back(r);
  }
  if (!g.range_host.empty()) {
    HIPCHK(hipMemcpyAsync(g.range_items, g.range_host.data(), g.range_host.size() * sizeof(WorkItem),
                          hipMemcpyHostToDevice, s));
    ProfScope ps_(GPT2_K_ADAMW);
    HIPCHK(launch_adamw(g.range_items, (int)g.range_host.size(), g.params, g.grads, g.m, g.v, g.shadow,
                        g.range_scale, g.range_norm2, adam_args(lr, b1, b2, eps, wd, t), s));
    if (g.shadow_t) g.transposed_stale = true;
  }
  HIPCHK(hipStreamSynchronize(s));
  if (finish) g.micro = 0;
  return ok();
}

int gpt2_profile_enable(uint32_t mask) {
  RUN(check_ready());
  HIPCHK(hipStreamSynchronize(g.stream));
  prof.mask = mask;
  prof.recs.clear();
  prof.used = 0;
  return ok();
}

int gpt2_profile_read(float* ms, int32_t* launches, int32_t n) {
  RUN(check_ready());
  if (!ms || !launches || n < 0) return fail(GPT2_EINVAL, "null output");
  HIPCHK(hipStreamSynchronize(g.stream));
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.f;
    launches[i] = 0;
  }
  for (auto& r : prof.recs) {
    float t = 0.f;
    HIPCHK(hipEventElapsedTime(&t, prof.pool[r.second], prof.pool[r.second + 1]));
    if (r.first < n) {
      ms[r.first] += t;
      launches[r.first] += 1;
    }
  }
  prof.recs.clear();
  prof.used = 0;
  return ok();
}

int gpt2_last_status(void) { return g_status; }

int gpt2_skip_update(void) {
  RUN(check_ready());
  g.micro = 0;
  return ok();
}

float gpt2_lr_schedule(int32_t step, float lr_max, int32_t warmup, int32_t total, float final_frac) {
  if (step < 1 || warmup < 0 || total <= warmup) return NAN;
  if (step <= warmup) return (float)((double)lr_max * step / warmup);
  const double lr_min = (double)final_frac * lr_max;
  if (step >= total) return (float)lr_min;
  const double ratio = (double)(step - warmup) / (double)(total - warmup);
  const double coeff = 0.5 * (1.0 + cos(M_PI * ratio));
  return (float)(lr_min + coeff * ((double)lr_max - lr_min));
}

void gpt2_outlier_reset(gpt2_outlier* d) {
  if (!d) return;
  memset(d, 0, sizeof(*d));
}

double gpt2_outlier_update(gpt2_outlier* d, double x) {
  if (!d) return NAN;
  double z = NAN;
  if (d->count >= GPT2_OUTLIER_WINDOW) {
    double mean = 0.0;
    for (int i = 0; i < GPT2_OUTLIER_WINDOW; ++i) mean += d->values[i];
    mean /= GPT2_OUTLIER_WINDOW;
    double var = 0.0;
    for (int i = 0; i < GPT2_OUTLIER_WINDOW; ++i) var += (d->values[i] - mean) * (d->values[i] - mean);
    var /= GPT2_OUTLIER_WINDOW;
    if (var > 0.0) z = (x - mean) / sqrt(var);
  }
  d->values[d->next] = x;
  d->next = (d->next + 1) % GPT2_OUTLIER_WINDOW;
  if (d->count < GPT2_OUTLIER_WINDOW) d->count++;
  return z;
}
const char* gpt2_last_error(void) { return g_err.c_str(); }
uint64_t gpt2_num_params(void) { return g.ready ? g.N : 0; }

static int copy_d2h(void* dst, const void* src, size_t bytes) {
  HIPCHK(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, g.stream));
  HIPCHK(hipStreamSynchronize(g.stream));
  return ok();
}

// host round-to-nearest-even fp32 -> bf16 (the device conversion's rule; NaN stays NaN)
static uint16_t host_f2bf(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float host_bf2f(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
// parameters [i0, i0 + k) as fp32 on the host (from the master, or the bf16 parameters)
static int params_to_host(float* dst, size_t i0, size_t k, std::vector<uint16_t>& tmp) {
  if (g.params) {
    HIPCHK(hipMemcpyAsync(dst, g.params + i0, k * 4, hipMemcpyDeviceToHost, g.stream));
    HIPCHK(hipStreamSynchronize(g.stream));
    return GPT2_OK;
  }
  tmp.resize(k);
  HIPCHK(hipMemcpyAsync(tmp.data(), g.shadow + i0, k * 2, hipMemcpyDeviceToHost, g.stream));
  HIPCHK(hipStreamSynchronize(g.stream));
  for (size_t i = 0; i < k; ++i) dst[i] = host_bf2f(tmp[i]);
  return GPT2_OK;
}
static int params_from_host(const float* src, size_t i0, size_t k, std::vector<uint16_t>& tmp) {
  if (g.params) {
    HIPCHK(hipMemcpyAsync(g.params + i0, src, k * 4, hipMemcpyHostToDevice, g.stream));
    HIPCHK(hipStreamSynchronize(g.stream));
    return GPT2_OK;
  }
  tmp.resize(k);
  for (size_t i = 0; i < k; ++i) tmp[i] = host_f2bf(src[i]);
  HIPCHK(hipMemcpyAsync(g.shadow + i0, tmp.data(), k * 2, hipMemcpyHostToDevice, g.stream));
  HIPCHK(hipStreamSynchronize(g.stream));
  return GPT2_OK;
}
// after the parameters changed: the bf16 copy (from the master) and the transposed copies
static int params_changed() {
  if (g.params && g.shadow) HIPCHK(launch_to_bf16(g.params, g.shadow, g.N, g.stream));
  HIPCHK(refresh_transposed());
  HIPCHK(hipStreamSynchronize(g.stream));
  return GPT2_OK;
}

int gpt2_get_params(float* dst, uint64_t n) {
  RUN(check_ready());
  if (!dst || n != g.N) return fail(GPT2_EINVAL, "need n == num_params (%zu)", g.N);
  std::vector<uint16_t> tmp;
  RUN(params_to_host(dst, 0, g.N, tmp));
  return ok();
}

int gpt2_set_params(const float* src, uint64_t n) {
  RUN(check_ready());
  if (!src || n != g.N) return fail(GPT2_EINVAL, "need n == num_params (%zu)", g.N);
  std::vector<uint16_t> tmp;
  RUN(params_from_host(src, 0, g.N, tmp));
  RUN(params_changed());
  return ok();
}

// ------------------------------------------------------------------ checkpoint
namespace {
constexpr char CKPT_MAGIC[8] = {'G', 'P', 'T', '2', 'C', 'K', 'P', 'T'};
constexpr uint32_t CKPT_VERSION = 1;
constexpr size_t CKPT_CHUNK = (size_t)16 << 20;  // floats per host staging chunk (64 MiB)

void ckpt_arch(int32_t (&a)[8]) {
  const gpt2_config& c = g.cfg;
  const int32_t v[8] = {c.n_layer, c.n_head, c.n_embd, c.vocab, c.padded_vocab, c.max_seq, c.linear_bias, c.ln_bias};
  for (int i = 0; i < 8; ++i) a[i] = v[i];
}

struct File {
  FILE* f = nullptr;
  ~File() {
    if (f) fclose(f);
  }
};

// device fp32 array <-> file, through a host chunk
int write_dev(FILE* f, const float* dev, size_t n, std::vector<float>& buf) {
  for (size_t i = 0; i < n; i += CKPT_CHUNK) {
    const size_t k = std::min(CKPT_CHUNK, n - i);
    HIPCHK(hipMemcpyAsync(buf.data(), dev + i, k * 4, hipMemcpyDeviceToHost, g.stream));
    HIPCHK(hipStreamSynchronize(g.stream));
    if (fwrite(buf.data(), 4, k, f) != k) return fail(GPT2_EIO, "checkpoint: write failed");
  }
  return GPT2_OK;
}
int read_dev(FILE* f, float* dev, size_t n, std::vector<float>& buf) {
  for (size_t i = 0; i < n; i += CKPT_CHUNK) {
    const size_t k = std::min(CKPT_CHUNK, n - i);
    if (fread(buf.data(), 4, k, f) != k) return fail(GPT2_EIO, "checkpoint: file too short");
    HIPCHK(hipMemcpyAsync(dev + i, buf.data(), k * 4, hipMemcpyHostToDevice, g.stream));
    HIPCHK(hipStreamSynchronize(g.stream));
  }
  return GPT2_OK;
}
}  // namespace

int gpt2_save(const char* path, int32_t t, uint64_t cursor) {
  RUN(check_ready());
  if (!path) return fail(GPT2_EINVAL, "gpt2_save: null path");
  if (g.micro != 0) return fail(GPT2_ESTATE, "gpt2_save: gradients pending; save between updates");
  HIPCHK(hipStreamSynchronize(g.stream));
  File file;
  file.f = fopen(path, "wb");
  if (!file.f) return fail(GPT2_EIO, "gpt2_save: cannot open %s", path);
  int32_t arch[8];
  ckpt_arch(arch);
  const uint64_t n = g.N;
  bool okw = fwrite(CKPT_MAGIC, 1, 8, file.f) == 8 && fwrite(&CKPT_VERSION, 4, 1, file.f) == 1 &&
             fwrite(arch, 4, 8, file.f) == 8 && fwrite(&n, 8, 1, file.f) == 1 && fwrite(&t, 4, 1, file.f) == 1 &&
             fwrite(&cursor, 8, 1, file.f) == 1 && fwrite(&g.seed, 8, 1, file.f) == 1;
  if (!okw) return fail(GPT2_EIO, "gpt2_save: write failed");
  std::vector<float> buf(std::min<size_t>(CKPT_CHUNK, g.N));
  std::vector<uint16_t> tmp;
  for (size_t i = 0; i < g.N; i += CKPT_CHUNK) {  // parameters as fp32 (exact from bf16 too)
    const size_t k = std::min(CKPT_CHUNK, g.N - i);
    RUN(params_to_host(buf.data(), i, k, tmp));
    if (fwrite(buf.data(), 4, k, file.f) != k) return fail(GPT2_EIO, "gpt2_save: write failed");
  }
  RUN(write_dev(file.f, g.m, g.N, buf));
  RUN(write_dev(file.f, g.v, g.N, buf));
  if (fflush(file.f) != 0) return fail(GPT2_EIO, "gpt2_save: write failed");
  return ok();
}

int gpt2_load(const char* path, int32_t* t, uint64_t* cursor) {
  RUN(check_ready());
  if (!path || !t || !cursor) return fail(GPT2_EINVAL, "gpt2_load: null argument");
  File file;
  file.f = fopen(path, "rb");
  if (!file.f) return fail(GPT2_EIO, "gpt2_load: cannot open %s", path);
  char magic[8];
  uint32_t version = 0;
  int32_t arch[8], want[8], tt = 0;
  uint64_t n = 0, cur = 0, seed = 0;
  bool okr = fread(magic, 1, 8, file.f) == 8 && fread(&version, 4, 1, file.f) == 1 &&
             fread(arch, 4, 8, file.f) == 8 && fread(&n, 8, 1, file.f) == 1 && fread(&tt, 4, 1, file.f) == 1 &&
             fread(&cur, 8, 1, file.f) == 1 && fread(&seed, 8, 1, file.f) == 1;
  if (!okr || memcmp(magic, CKPT_MAGIC, 8) != 0 || version != CKPT_VERSION)
    return fail(GPT2_EIO, "gpt2_load: %s is not a version-%u checkpoint", path, CKPT_VERSION);
  ckpt_arch(want);
  if (memcmp(arch, want, sizeof arch) != 0 || n != g.N)
    return fail(GPT2_EIO, "gpt2_load: %s holds a different architecture", path);
  // the whole file must be there before anything on the device is overwritten
  const long body = ftell(file.f);
  if (body < 0 || fseek(file.f, 0, SEEK_END) != 0) return fail(GPT2_EIO, "gpt2_load: cannot seek in %s", path);
  const long end = ftell(file.f);
  if (end < 0 || (uint64_t)(end - body) < (uint64_t)3 * g.N * 4 || fseek(file.f, body, SEEK_SET) != 0)
    return fail(GPT2_EIO, "gpt2_load: %s is shorter than its header says", path);
  // from here a failure leaves the model half restored: it is marked not ready
  auto load_body = [&]() -> int {
    std::vector<float> buf(std::min<size_t>(CKPT_CHUNK, g.N));
    std::vector<uint16_t> tmp;
    for (size_t i = 0; i < g.N; i += CKPT_CHUNK) {
      const size_t k = std::min(CKPT_CHUNK, g.N - i);
      if (fread(buf.data(), 4, k, file.f) != k) return fail(GPT2_EIO, "checkpoint: file too short");
      RUN(params_from_host(buf.data(), i, k, tmp));
    }
    RUN(read_dev(file.f, g.m, g.N, buf));
    RUN(read_dev(file.f, g.v, g.N, buf));
    RUN(params_changed());
    return GPT2_OK;
  };
  if (load_body() != GPT2_OK) {
    g.ready = false;
    g_err += " (the model is no longer usable: gpt2_init again)";
    return g_status;
  }
  g.seed = seed;
  g.micro = 0;
  g.fwd_targets = false;
  g.fwd_logits = false;
  *t = tt;
  *cursor = cur;
  return ok();
}

int gpt2_get_grads(float* dst, uint64_t n) {
  RUN(check_ready());
  if (!dst || n != g.N) return fail(GPT2_EINVAL, "need n == num_params (%zu)", g.N);
  return copy_d2h(dst, g.grads, n * 4);
}

int gpt2_get_adam_state(float* m, float* v, uint64_t n) {
  RUN(check_ready());
  if (!m || !v || n != g.N) return fail(GPT2_EINVAL, "need n == num_params (%zu)", g.N);
  RUN(copy_d2h(m, g.m, n * 4));
  return copy_d2h(v, g.v, n * 4);
}

int gpt2_get_logits(float* dst, uint64_t n) {
  RUN(check_ready());
  if (!g.fwd_logits) return fail(GPT2_ESTATE, "logits are kept only by a gpt2_forward with targets == NULL");
  if (!dst || n != (uint64_t)g.BT * g.V) return fail(GPT2_EINVAL, "need n == B*T*vocab");
  std::vector<char> raw((size_t)g.BT * g.ldl * g.es);
  RUN(copy_d2h(raw.data(), g.logits, raw.size()));
  for (size_t r = 0; r < (size_t)g.BT; ++r)
    for (size_t c = 0; c < (size_t)g.V; ++c) {
      const size_t i = r * g.ldl + c;
      float f;
      if (g.es == 2) {
        const uint32_t u = (uint32_t)reinterpret_cast<const uint16_t*>(raw.data())[i] << 16;
        memcpy(&f, &u, 4);
      } else {
        f = reinterpret_cast<const float*>(raw.data())[i];
      }
      dst[r * g.V + c] = f;
    }
  return ok();
}

// ===================================================================================== per-op ABI
static DType to_dt(int dtype) { return dtype == GPT2_BF16 ? DT_BF16 : DT_F32; }
static int op_ret(hipError_t e) {
  if (e == hipErrorInvalidValue) return fail(GPT2_EINVAL, "unsupported shape or argument");
  if (e != hipSuccess) return fail(GPT2_EHIP, "%s", hipGetErrorString(e));
  return ok();
}

// Operand checks of the GEMM ops: the tiles move 16-byte vectors, so every leading dimension must be a
// whole number of them (8 bf16 or 4 fp32 elements; the EPI_F32 output is fp32) and every pointer
// 16-byte aligned; a leading dimension must also cover the row it strides over.
static const char* gemm_op_check(int dtype, int a_kc, int b_kc, int epilogue, int M, int N, int K, const void* A,
                                 int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                                 const void* bias, const void* aux, int64_t ldaux, const void* C2) {
  if (dtype != GPT2_FP32 && dtype != GPT2_BF16) return "dtype must be GPT2_FP32 or GPT2_BF16";
  if (epilogue < 0 || epilogue > 6 || M < 0 || N < 0 || K < 0) return "bad epilogue or negative size";
  if (M == 0 || N == 0) return nullptr;
  const int64_t vin = dtype == GPT2_BF16 ? 8 : 4, vout = epilogue == EPI_F32 ? 4 : vin;
  if (!A || !B || !C) return "null operand";
  if (lda % vin || ldb % vin || ldc % vout) return "leading dimensions must be multiples of 16 bytes";
  if (lda < (a_kc ? K : M) || ldb < (b_kc ? K : N) || ldc < N) return "leading dimension smaller than the row";
  const bool needs_aux = epilogue == EPI_RESID || epilogue == EPI_GELU_BWD || epilogue == EPI_MUL;
  const bool needs_c2 = epilogue == EPI_GELU || epilogue == EPI_GELU_GRAD;
  if (needs_aux && (!aux || ldaux % vin || ldaux < N)) return "this epilogue needs aux with a valid leading dimension";
  if (needs_c2 && !C2) return "this epilogue needs C2";
  for (const void* ptr : {A, B, C, bias, aux, C2})
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return "pointers must be 16-byte aligned";
  return nullptr;
}

int gpt2op_gemm(int dtype, int a_kcontig, int b_kcontig, int epilogue, int M, int N, int K, const void* A,
                int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, const void* bias, const void* aux,
                int64_t ldaux, void* C2, int accumulate, float* scratch, uint64_t scratch_floats, void* stream) {
  if (const char* e = gemm_op_check(dtype, a_kcontig, b_kcontig, epilogue, M, N, K, A, lda, B, ldb, C, ldc, bias, aux,
                                    ldaux, C2))
    return fail(GPT2_EINVAL, "gemm: %s", e);
  GemmArgs a{};
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = A;
  a.lda = lda;
  a.B = B;
  a.ldb = ldb;
  a.C = C;
  a.ldc = ldc;
  a.bias = bias;
  a.aux = aux;
  a.ldaux = ldaux;
  a.C2 = C2;
  a.accumulate = accumulate;
  return op_ret(launch_gemm(to_dt(dtype), a_kcontig != 0, b_kcontig != 0, (Epi)epilogue, a, scratch, scratch_floats,
                            reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_gemm_colsum(int dtype, int a_kcontig, int b_kcontig, int epilogue, int M, int N, int K, const void* A,
                       int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, const void* bias,
                       const void* aux, int64_t ldaux, void* C2, float* colsum, int colsum_accumulate,
                       float* scratch, uint64_t scratch_floats, void* stream) {
  if (epilogue == EPI_F32 || !colsum) return fail(GPT2_EINVAL, "bad gemm_colsum arguments");
  if (const char* e = gemm_op_check(dtype, a_kcontig, b_kcontig, epilogue, M, N, K, A, lda, B, ldb, C, ldc, bias, aux,
                                    ldaux, C2))
    return fail(GPT2_EINVAL, "gemm_colsum: %s", e);
  if (!scratch || (uint64_t)cdiv(M, 128) * 2 * N > scratch_floats)
    return fail(GPT2_EINVAL, "gemm_colsum needs scratch of ceil(M/128)*2*N floats");
  GemmArgs a{};
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = A;
  a.lda = lda;
  a.B = B;
  a.ldb = ldb;
  a.C = C;
  a.ldc = ldc;
  a.bias = bias;
  a.aux = aux;
  a.ldaux = ldaux;
  a.C2 = C2;
  a.colsum = colsum;
  a.colsum_accumulate = colsum_accumulate;
  return op_ret(launch_gemm(to_dt(dtype), a_kcontig != 0, b_kcontig != 0, (Epi)epilogue, a, scratch, scratch_floats,
                            reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_layernorm_forward(int dtype, int rows, int C, const void* x, const void* w, const void* b, void* y,
                             float* mean, float* rstd, void* stream) {
  return op_ret(launch_layernorm_fwd(to_dt(dtype), rows, C, x, w, b, y, mean, rstd, reinterpret_cast<hipStream_t>(stream)));
}

uint64_t gpt2op_layernorm_backward_scratch(int rows, int C) { return layernorm_bwd_partial_floats(rows, C); }

int gpt2op_layernorm_backward(int dtype, int rows, int C, const void* dy, const void* x, const void* w,
                              const float* mean, const float* rstd, void* dres, float* dw, float* db, float* dsum,
                              int accumulate, float* partial, void* stream) {
  return op_ret(launch_layernorm_bwd(to_dt(dtype), rows, C, dy, x, w, mean, rstd, dres, 1, dw, db, dsum, accumulate,
                                     partial, layernorm_bwd_partial_floats(rows, C),
                                     reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_stochastic_round(const float* x, uint16_t* y, uint64_t n, uint64_t seed, int32_t t, uint64_t index0,
                            void* stream) {
  if ((n && (!x || !y)) || t < 0) return fail(GPT2_EINVAL, "bad stochastic_round arguments");
  return op_ret(launch_stochastic_round(x, y, n, seed, t, index0, reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_attention_forward(int dtype, int B, int T, int H, int hs, const void* qkv, void* out, float* lse,
                             void* stream) {
  return op_ret(launch_attention_fwd(to_dt(dtype), B, T, H, hs, qkv, out, lse, reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_attention_backward(int dtype, int B, int T, int H, int hs, const void* qkv, const void* out,
                              const void* dout, const float* lse, void* dqkv, float* dvec, void* stream) {
  return op_ret(launch_attention_bwd(to_dt(dtype), B, T, H, hs, qkv, out, dout, lse, dqkv, dvec, ATT_BWD_ALL,
                                     reinterpret_cast<hipStream_t>(stream)));
}

// ---- the attention backward that allocates nothing: its scratch (D = rowsum(dO * O), one float per
// query row and head) lives in this file-scope device array, one copy per GPU. In host code the
// name `scratch` is only a host-side stand-in: its device address on the current GPU is looked up
// once per device with hipGetSymbolAddress and only that address is handed to the kernels.
static __device__ __align__(256) float scratch[GPT2_NOALLOC_ATTN_SCRATCH_FLOATS];
static constexpr int NOALLOC_MAX_DEVICES = 64;
static float* g_noalloc_scratch[NOALLOC_MAX_DEVICES];
static std::mutex g_noalloc_mu;

int gpt2op_attention_backward_noalloc(int dtype, int B, int T, int H, int hs, const void* qkv, const void* out,
                                      const void* dout, const float* lse, void* dqkv, void* stream) {
  if (B < 0 || T < 0 || H < 1) return fail(GPT2_EINVAL, "attention_backward_noalloc: need B, T >= 0 and H >= 1");
  if ((uint64_t)B * T * H > (uint64_t)GPT2_NOALLOC_ATTN_SCRATCH_FLOATS)
    return fail(GPT2_EINVAL, "attention_backward_noalloc: B*T*H = %llu exceeds the %d floats of its scratch",
                (unsigned long long)B * T * H, GPT2_NOALLOC_ATTN_SCRATCH_FLOATS);
  int dev = -1;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(GPT2_EINVAL, "attention_backward_noalloc: device %d", dev);
  float* dvec = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    if (!g_noalloc_scratch[dev]) {
      void* p = nullptr;
      HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      if (!p) return fail(GPT2_EHIP, "attention_backward_noalloc: no device address for the scratch array");
      g_noalloc_scratch[dev] = static_cast<float*>(p);
    }
    dvec = g_noalloc_scratch[dev];
  }
  // every scratch entry the kernels read is written first by the D kernel of the same call: nothing
  // needs clearing
  return op_ret(launch_attention_bwd(to_dt(dtype), B, T, H, hs, qkv, out, dout, lse, dqkv, dvec, ATT_BWD_ALL,
                                     reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_attention_backward_colsum(int dtype, int B, int T, int H, int hs, const void* qkv, const void* out,
                                     const void* dout, const float* lse, void* dqkv, float* dvec, float* dbias,
                                     int accumulate, float* scratch, uint64_t scratch_floats, void* stream) {
  if (B < 0 || T < 0 || H < 1 || hs < 1 || !dbias) return fail(GPT2_EINVAL, "bad attention_backward_colsum arguments");
  const long C3 = 3L * H * hs;
  if (!scratch || (uint64_t)cdiv((long)B * T, 128) * C3 > scratch_floats ||
      (uint64_t)attention_bias_partial_rows(B, T) * C3 > scratch_floats)
    return fail(GPT2_EINVAL, "attention_backward_colsum needs scratch of B*ceil(T/128)*3*H*hs floats");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const DType dt = to_dt(dtype);
  if (dt == DT_BF16) {
    int rc = op_ret(launch_attention_bwd(dt, B, T, H, hs, qkv, out, dout, lse, dqkv, dvec, ATT_BWD_ALL, s, scratch));
    if (rc != GPT2_OK || B * T == 0) return rc;
    return op_ret(launch_colsum_finish(scratch, attention_bias_partial_rows(B, T), (int)C3, dbias, accumulate, s));
  }
  int rc = op_ret(launch_attention_bwd(dt, B, T, H, hs, qkv, out, dout, lse, dqkv, dvec, ATT_BWD_ALL, s));
  if (rc != GPT2_OK) return rc;
  return op_ret(launch_colsum(dt, dqkv, C3, B * T, (int)C3, dbias, accumulate, scratch, scratch_floats, s));
}

int gpt2op_cross_entropy(int dtype, int rows, int V, int ld, void* logits, const int32_t* targets, const float* dloss,
                         float* losses, void* stream) {
  return op_ret(launch_cross_entropy(to_dt(dtype), rows, V, ld, logits, targets, dloss, losses,
                                     reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_encoder_forward(int dtype, int B, int T, int C, int V, const int32_t* tok, const void* wte, const void* wpe,
                           void* out, int* err, void* stream) {
  return op_ret(launch_encoder_fwd(to_dt(dtype), B, T, C, V, tok, wte, wpe, out, err, reinterpret_cast<hipStream_t>(stream)));
}

uint64_t gpt2op_encoder_backward_scratch(int BT, int C) { return encoder_bwd_partial_floats(BT, C); }

int gpt2op_copy(void* dst, const void* src, uint64_t bytes, void* stream) {
  if ((bytes % 16) || ((uintptr_t)dst % 16) || ((uintptr_t)src % 16) || (bytes && (!dst || !src)))
    return fail(GPT2_EINVAL, "copy: pointers and size must be 16-byte aligned");
  return op_ret(launch_copy(dst, src, bytes, reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_mfma_rate(const void* operands, float* out, int blocks, int iters, void* stream) {
  if (!operands || !out || (uintptr_t)operands % 16 || blocks < 1 || blocks > (1 << 20) || iters < 0)
    return fail(GPT2_EINVAL, "mfma_rate: need 16-byte aligned operands, out, 1 <= blocks <= 2^20, iters >= 0");
  return op_ret(launch_mfma_rate(operands, out, blocks, iters, reinterpret_cast<hipStream_t>(stream)));
}

int gpt2op_encoder_backward(int dtype, int B, int T, int max_seq, int C, int V, const int32_t* tok, const void* dout,
                            float* dwte, float* dwpe, int accumulate_wpe, uint32_t* keys, float* partial, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the shapes the scatter refuses are refused before the sort writes the keys
  const int vec = dtype == GPT2_BF16 ? 8 : 4;
  if (B < 0 || T < 0 || V < 1 || C <= 0 || C % vec || T > max_seq)
    return fail(GPT2_EINVAL, "encoder_backward: need B, T >= 0, V >= 1, C a positive multiple of 16 bytes, T <= max_seq");
  hipError_t e = launch_encoder_sort(B * T, V, tok, keys, s);
  if (e != hipSuccess) return op_ret(e);
  return op_ret(launch_encoder_bwd(to_dt(dtype), B, T, max_seq, C, keys, dout, dwte, dwpe, accumulate_wpe, partial,
                                   encoder_bwd_partial_floats(B * T, C), s));
}

}  // extern "C"
