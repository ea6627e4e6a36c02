// libgpt2 runtime: workspace layout, the launch plan of one training step,
// and the C ABI declared in include/gpt2.h.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/gpt2.h"
#include "kernels.h"

namespace {

struct LayerOff {  // element offsets of one block's parameters in the flat vector
  long ln1w, ln1b, attnw, attnb, projw, projb, ln2w, ln2b, fcw, fcb, fc2w, fc2b;
};

struct LayerAct {  // saved activations of one block
  float* x_in;
  float *mean1, *rstd1;
  void* u1;
  void* qkv;
  void* y;
  float* lse;
  float* x_mid;
  float *mean2, *rstd2;
  void* u2;
  void* h;
  void* g;
};

struct Layout {
  long P = 0;
  long wte = 0, wpe = 0, lnfw = 0, lnfb = 0;
  std::vector<LayerOff> layer;
  // (offset, length, decay, init) of every tensor in canonical order, and
  // whether the input-gradient products also read it transposed (bf16 mode
  // keeps a transposed bf16 copy of those matrices)
  std::vector<long> t_off, t_len;
  std::vector<int> t_decay;
  std::vector<int> t_init;
  std::vector<int> t_trans;
};

// How a tensor starts ("GPT-2 from Scratch", Initialization: 0.02, and the
// residual scaling): weights and embeddings N(0, 0.02); the two c_proj
// weights of a block N(0, 0.02 / sqrt(2 n_layer)); biases and LayerNorm
// shifts 0; LayerNorm gains 1.
enum { INIT_ZERO = 0, INIT_ONE = 1, INIT_NORMAL = 2, INIT_NORMAL_RESID = 3 };

bool valid_config(const gpt2_config* c, std::string* why) {
  auto fail = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (!c) return fail("config is NULL");
  if (c->n_layer < 1 || c->n_head < 1 || c->n_embd < 1) return fail("n_layer, n_head, n_embd must be >= 1");
  if (c->n_embd % c->n_head) return fail("n_embd must be a multiple of n_head");
  if (c->n_embd % 64 || c->n_embd > 2048) return fail("n_embd must be a multiple of 64 and <= 2048");
  int hd = c->n_embd / c->n_head;
  if (c->precision == GPT2_BF16) {
    if (hd != 64) return fail("bf16 precision needs head width n_embd/n_head == 64");
  } else if (c->precision == GPT2_FP32) {
    if (hd != 32 && hd != 64) return fail("fp32 precision needs head width 32 or 64");
  } else {
    return fail("precision must be GPT2_FP32 or GPT2_BF16");
  }
  if (c->vocab_size < 1 || c->padded_vocab_size < c->vocab_size)
    return fail("need 1 <= vocab_size <= padded_vocab_size");
  if (c->padded_vocab_size % 64 || c->padded_vocab_size > 51200)
    return fail("padded_vocab_size must be a multiple of 64 and <= 51200");
  if (c->block_size < 1 || c->max_batch < 1) return fail("block_size and max_batch must be >= 1");
  if (c->head_chunk < 0 || c->head_chunk % 64)
    return fail("head_chunk must be 0 or a positive multiple of 64");
  return true;
}

Layout make_layout(const gpt2_config* c) {
  Layout L;
  const long C = c->n_embd, Vp = c->padded_vocab_size;
  // matrices and embeddings (dim 2) are decayed, vectors are not
  auto add = [&](long n, int init, int trans = 0) {
    long o = L.P;
    L.t_off.push_back(o);
    L.t_len.push_back(n);
    L.t_decay.push_back(init >= INIT_NORMAL ? 1 : 0);
    L.t_init.push_back(init);
    L.t_trans.push_back(trans);
    L.P += n;
    return o;
  };
  L.wte = add(Vp * C, INIT_NORMAL, 1);
  L.wpe = add((long)c->block_size * C, INIT_NORMAL);
  for (int l = 0; l < c->n_layer; ++l) {
    LayerOff o;
    o.ln1w = add(C, INIT_ONE);
    o.ln1b = add(C, INIT_ZERO);
    o.attnw = add(3 * C * C, INIT_NORMAL, 1);
    o.attnb = add(3 * C, INIT_ZERO);
    o.projw = add(C * C, INIT_NORMAL_RESID, 1);
    o.projb = add(C, INIT_ZERO);
    o.ln2w = add(C, INIT_ONE);
    o.ln2b = add(C, INIT_ZERO);
    o.fcw = add(4 * C * C, INIT_NORMAL, 1);
    o.fcb = add(4 * C, INIT_ZERO);
    o.fc2w = add(4 * C * C, INIT_NORMAL_RESID, 1);
    o.fc2b = add(C, INIT_ZERO);
    L.layer.push_back(o);
  }
  L.lnfw = add(C, INIT_ONE);
  L.lnfb = add(C, INIT_ZERO);
  return L;
}

// elements per AdamW workgroup: 4096 keeps the bf16 step's few vector and wpe
// chunks spread over more CUs (10 us per step faster than 16384)
constexpr long ADAM_CHUNK = 4096;

// Chunks of the flat AdamW pass; skip_trans: leave out the matrices that
// the tiled pass (which also writes their transposed copy) updates.
std::vector<AdamChunk> make_chunks(const Layout& L, bool skip_trans) {
  std::vector<AdamChunk> v;
  for (size_t t = 0; t < L.t_off.size(); ++t) {
    if (skip_trans && L.t_trans[t]) continue;
    for (long s = 0; s < L.t_len[t]; s += ADAM_CHUNK) {
      AdamChunk ck;
      ck.start = L.t_off[t] + s;
      ck.len = (int)std::min(ADAM_CHUNK, L.t_len[t] - s);
      ck.flags = L.t_decay[t];
      v.push_back(ck);
    }
  }
  return v;
}

// 64 x 64 tiles of every weight matrix that a GEMM also reads transposed (the
// input-gradient products dx = dy W): wte and, per block, c_attn, attn
// c_proj, c_fc and mlp c_proj.
std::vector<TTile> make_ttiles(const Layout& L, const gpt2_config* c) {
  std::vector<TTile> v;
  const int C = c->n_embd, Vp = c->padded_vocab_size;
  auto add = [&](long off, int rows, int cols) {
    for (int r = 0; r < rows; r += 64)
      for (int q = 0; q < cols; q += 64) v.push_back(TTile{off, rows, cols, r, q});
  };
  add(L.wte, Vp, C);
  for (const LayerOff& o : L.layer) {
    add(o.attnw, 3 * C, C);
    add(o.projw, C, C);
    add(o.fcw, 4 * C, C);
    add(o.fc2w, C, 4 * C);
  }
  return v;
}

// Bump allocator over the workspace (256-byte aligned pieces).
struct Arena {
  char* base;
  size_t off = 0;
  explicit Arena(char* b) : base(b) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
  template <typename T> T* take_n(size_t n) { return reinterpret_cast<T*>(take(n * sizeof(T))); }
};

}  // namespace

struct gpt2 {
  gpt2_config cfg;
  hipStream_t stream;
  DType act;
  size_t act_size;
  Layout lay;
  int nchunks = 0;
  // persistent state
  float *params, *grads, *m, *v;
  bf16_t* shadow;
  bf16_t* shadow_t;  // transposed bf16 copies of the matrices in ttiles (same offsets)
  TTile* ttiles;
  int nttiles = 0;
  AdamChunk* chunks;
  int* err;
  int* n_valid;
  float *loss, *norm, *clip;
  double* norm_partial;
  int32_t* idx;
  // activations
  std::vector<LayerAct> A;
  float* x_final;
  float *meanf, *rstdf;
  void* z;
  void* logits;           // (B*T, Vp) logits, then d(loss)/d(logits); null with a fused head
  float* row_loss;
  // fused lm_head + cross-entropy (head_chunk > 0)
  int head_chunk = 0;     // vocabulary columns per backward slice (<= Vp)
  void* hslice;           // d(loss)/d(logits) of one slice: (B*T, head_chunk)
  float* hpart;           // (B*T, Vp/64) block partials (max, sum of exp)
  float* hlse;            // (B*T) log-sum-exp
  float* htlogit;         // (B*T) logit of the target
  int32_t* tgt;           // (B*T) copy of the targets, read again by the backward
  // generation
  float* gen_logits;      // (max_batch, Vp) last-position logits
  int32_t* gen_idx;       // (max_batch, block_size) cropped context
  void* kv;               // key/value cache: per block (max_batch, block_size, 2C)
  int kv_len = 0;         // positions 0 .. kv_len-1 of kv_B sequences hold the current
  int kv_B = 0;           // parameters' keys and values (gpt2_prefill / gpt2_decode)
  // backward scratch
  float* dres;
  void* dres_b;           // bf16 mode: 2L slots of the residual gradient (see run_backward)
  float* dxtmp;
  void* dbig;             // bf16 mode: one slot per layer, else one
  void* dqkv;             // bf16 mode: one slot per layer, else one
  // bf16 mode: the weight gradients of all blocks and of the lm_head as one
  // grouped launch at the end of the backward pass
  GemmProblem* wg_probs;
  int wg_n = 0;
  long wg_tiles = 0;
  long wg_elems = 0;  // weight-gradient elements the grouped launch produces
  // the last wg_tail.M rows of the first product, taken out of the group so
  // that it ends on a full round of tiles; run as split-K slices after it
  GemmProblem wg_tail{};
  void* dy;
  float* dbuf;
  // partial column sums, one slot per producing launch, summed by one grouped
  // launch at the end of the backward pass: the 2L+1 LayerNorm backwards (slot
  // 2l: ln_1 of block l, 2l+1: ln_2, 2L: ln_f), and per block the c_fc and
  // c_attn bias gradients
  float* ln_parts;
  float* fcb_parts;
  float* attnb_parts;
  ColsumProblem* cs_probs;
  void* emb_scratch;  // embedding backward: id sort and per-chunk run sums
  int cs_n = 0;
  int cs_chunks = 0;
  float* splitk;
  // state
  int B = 0, T = 0;
  bool have_targets = false;
  bool forward_done = false;
  // gpt2_zero_grad was called and the gradients not yet zeroed: the next
  // backward writes them instead of adding (when every gradient it produces
  // is written whole), anything else that uses them zeroes them first
  bool zero_pending = false;
  int64_t step = 0;
  std::string last_error;
  // kernel timing (gpt2_timing_begin/end)
  uint64_t timing_mask = 0;
  std::vector<hipEvent_t> ev_pool;  // pairs: start, end
  std::vector<int> ev_site;
  size_t ev_used = 0;
  ~gpt2() {
    for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
  }
};

namespace {

// Rows of a c_fc bias-gradient partial slot: per-128-row sums from the
// GEMM epilogue (bf16) or BIAS_SPLITS row slices (fp32), whichever is more.
size_t fcb_part_rows(size_t BT) { return std::max<size_t>((BT + 127) / 128, BIAS_SPLITS); }
// Rows of a c_attn bias-gradient partial slot: per (sequence, 128-position
// block) sums from the attention backward (bf16) or BIAS_SPLITS row slices
// (fp32), whichever is more.
size_t attnb_part_rows(const gpt2_config* c) {
  return std::max<size_t>((size_t)c->max_batch * ((c->block_size + 127) / 128), BIAS_SPLITS);
}

// Lays out the whole workspace; with h == nullptr only measures it.
size_t plan(const gpt2_config* c, char* base, gpt2* h) {
  Arena a(base);
  Layout L = make_layout(c);
  const size_t P = (size_t)L.P;
  const size_t C = c->n_embd, H = c->n_head, Vp = c->padded_vocab_size;
  const size_t BT = (size_t)c->max_batch * c->block_size;
  const size_t es = c->precision == GPT2_BF16 ? 2 : 4;
  std::vector<AdamChunk> ch = make_chunks(L, c->precision == GPT2_BF16);
  float* params = a.take_n<float>(P);
  float* grads = a.take_n<float>(P);
  float* m = a.take_n<float>(P);
  float* v = a.take_n<float>(P);
  bf16_t* shadow = c->precision == GPT2_BF16 ? a.take_n<bf16_t>(P) : nullptr;
  bf16_t* shadow_t = c->precision == GPT2_BF16 ? a.take_n<bf16_t>(P) : nullptr;
  std::vector<TTile> tt = c->precision == GPT2_BF16 ? make_ttiles(L, c) : std::vector<TTile>();
  TTile* ttiles = a.take_n<TTile>(tt.size());
  AdamChunk* chunks = a.take_n<AdamChunk>(ch.size());
  int* err = a.take_n<int>(1);
  int* n_valid = a.take_n<int>(1);
  float* loss = a.take_n<float>(1);
  float* norm = a.take_n<float>(1);
  float* clip = a.take_n<float>(1);
  double* norm_partial = a.take_n<double>(NORM_PARTS);
  int32_t* idx = a.take_n<int32_t>(BT);
  std::vector<LayerAct> acts(c->n_layer);
  for (int l = 0; l < c->n_layer; ++l) {
    LayerAct& x = acts[l];
    x.x_in = a.take_n<float>(BT * C);
    x.mean1 = a.take_n<float>(BT);
    x.rstd1 = a.take_n<float>(BT);
    x.u1 = a.take(BT * C * es);
    x.qkv = a.take(BT * 3 * C * es);
    x.y = a.take(BT * C * es);
    x.lse = a.take_n<float>(BT * H);
    x.x_mid = a.take_n<float>(BT * C);
    x.mean2 = a.take_n<float>(BT);
    x.rstd2 = a.take_n<float>(BT);
    x.u2 = a.take(BT * C * es);
    x.h = a.take(BT * 4 * C * es);
    x.g = a.take(BT * 4 * C * es);
  }
  float* x_final = a.take_n<float>(BT * C);
  float* meanf = a.take_n<float>(BT);
  float* rstdf = a.take_n<float>(BT);
  void* z = a.take(BT * C * es);
  const size_t hc = c->head_chunk > 0 ? std::min<size_t>(c->head_chunk, Vp) : 0;
  void* logits = hc ? nullptr : a.take(BT * Vp * es);
  void* hslice = hc ? a.take(BT * hc * es) : nullptr;
  float* hpart = hc ? a.take_n<float>(BT * (Vp / 64) * 2) : nullptr;
  float* hlse = hc ? a.take_n<float>(BT) : nullptr;
  float* htlogit = hc ? a.take_n<float>(BT) : nullptr;
  int32_t* tgt = hc ? a.take_n<int32_t>(BT) : nullptr;
  float* row_loss = a.take_n<float>(BT);
  float* gen_logits = a.take_n<float>((size_t)c->max_batch * Vp);
  int32_t* gen_idx = a.take_n<int32_t>(BT);
  void* kv = a.take((size_t)c->n_layer * BT * 2 * C * es);
  float* dres = a.take_n<float>(BT * C);
  const bool bf = c->precision == GPT2_BF16;
  const size_t nl = (size_t)c->n_layer;
  void* dres_b = bf ? a.take(2 * nl * BT * C * es) : nullptr;
  float* dxtmp = a.take_n<float>(BT * C);
  void* dbig = a.take((bf ? nl : 1) * BT * 4 * C * es);
  void* dqkv = a.take((bf ? nl : 1) * BT * 3 * C * es);
  GemmProblem* wg_probs = a.take_n<GemmProblem>(bf ? 4 * nl + 1 : 0);
  void* dy = a.take(BT * C * es);
  float* dbuf = a.take_n<float>(BT * H);
  float* ln_parts = a.take_n<float>((2 * nl + 1) * (size_t)ln_bwd_scratch((long)BT, (int)C));
  float* fcb_parts = a.take_n<float>(nl * fcb_part_rows(BT) * 4 * C);
  float* attnb_parts = a.take_n<float>(nl * attnb_part_rows(c) * 3 * C);
  ColsumProblem* cs_probs = a.take_n<ColsumProblem>(4 * nl + 1);
  void* emb_scratch = a.take(embed_bwd_scratch_bytes((long)BT, (int)C));
  float* splitk = a.take_n<float>((size_t)SPLITK_PART_ELEMS);
  size_t total = (a.off + 255) & ~(size_t)255;
  if (h) {
    h->lay = L;
    h->nchunks = (int)ch.size();
    h->params = params; h->grads = grads; h->m = m; h->v = v; h->shadow = shadow;
    h->shadow_t = shadow_t; h->ttiles = ttiles; h->nttiles = (int)tt.size();
    h->chunks = chunks; h->err = err; h->n_valid = n_valid; h->loss = loss; h->norm = norm;
    h->clip = clip; h->norm_partial = norm_partial; h->idx = idx;
    h->A = acts;
    h->x_final = x_final; h->meanf = meanf; h->rstdf = rstdf; h->z = z; h->logits = logits;
    h->row_loss = row_loss;
    h->head_chunk = (int)hc; h->hslice = hslice; h->hpart = hpart; h->hlse = hlse;
    h->htlogit = htlogit; h->tgt = tgt;
    h->gen_logits = gen_logits; h->gen_idx = gen_idx; h->kv = kv;
    h->dres = dres; h->dres_b = dres_b; h->dxtmp = dxtmp; h->dbig = dbig; h->dqkv = dqkv;
    h->wg_probs = wg_probs;
    h->dy = dy; h->dbuf = dbuf;
    h->ln_parts = ln_parts; h->fcb_parts = fcb_parts; h->attnb_parts = attnb_parts;
    h->cs_probs = cs_probs;
    h->emb_scratch = emb_scratch;
    h->splitk = splitk;
  }
  return total;
}

gpt2_status fail(gpt2* h, gpt2_status s, const std::string& msg) {
  if (h) h->last_error = msg;
  return s;
}

#define HIPTRY(h, expr)                                                              \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess)                                                            \
      return fail((h), GPT2_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// bf16 copy of the weights in bf16 mode, the fp32 master otherwise
const void* W(const gpt2* h, long off) {
  return h->act == DT_BF16 ? (const void*)(h->shadow + off) : (const void*)(h->params + off);
}

// B operand of an input-gradient product dx = dy W for the matrix W (rows x
// cols, row-major at `off`), starting at row r0 of W: B(n, k) = W[r0 + k][n].
// bf16 mode reads the transposed copy, k-contiguous; fp32 mode reads the
// master weights transposed.
struct WOp {
  const void* p;
  long ld;
  bool t;
};
WOp w_dx(const gpt2* h, long off, long rows, long cols, long r0 = 0) {
  if (h->act == DT_BF16) return {h->shadow_t + off + r0, rows, false};
  return {h->params + off + r0 * cols, cols, true};
}

// Records an event pair around one launch when its site is being timed.
struct Site {
  gpt2* h;
  long pair = -1;
  Site(gpt2* hh, int site) : h(hh) {
    if (!((h->timing_mask >> site) & 1)) return;
    size_t i = h->ev_used;
    while (h->ev_pool.size() < 2 * (i + 1)) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return;
      h->ev_pool.push_back(e);
    }
    if (h->ev_site.size() < i + 1) h->ev_site.resize(i + 1);
    h->ev_site[i] = site;
    h->ev_used = i + 1;
    pair = (long)i;
    (void)hipEventRecord(h->ev_pool[2 * i], h->stream);
  }
  ~Site() {
    if (pair >= 0) (void)hipEventRecord(h->ev_pool[2 * pair + 1], h->stream);
  }
};

#define TIMED(h, site, expr) \
  do {                       \
    Site ts_((h), (site));   \
    HIPTRY((h), (expr));     \
  } while (0)

EpiArgs epi(void* out, long ldo, float alpha = 1.f) {
  EpiArgs e;
  std::memset(&e, 0, sizeof(e));
  e.out = out;
  e.ldo = ldo;
  e.alpha = alpha;
  return e;
}

gpt2_status check_device_flags(gpt2* h) {
  int f = 0;
  HIPTRY(h, hipMemcpy(&f, h->err, sizeof(int), hipMemcpyDeviceToHost));
  if (f) {
    HIPTRY(h, hipMemset(h->err, 0, sizeof(int)));
    std::string m;
    if (f & ERRF_IDX) m += "token id outside [0, padded_vocab_size); ";
    if (f & ERRF_TARGET) m += "target outside {-1} U [0, padded_vocab_size); ";
    return fail(h, GPT2_E_RANGE, m + "offending values were read as 0");
  }
  return GPT2_OK;
}

gpt2_status sync(gpt2* h) {
  HIPTRY(h, hipStreamSynchronize(h->stream));
  return check_device_flags(h);
}

// last_logits != null: no targets; only the last position of each sequence
// goes through the lm_head, into last_logits (B, Vp) fp32.
gpt2_status run_forward(gpt2* h, const int32_t* d_idx, const int32_t* d_tgt, int B, int T,
                        bool grad, float* last_logits = nullptr) {
  const gpt2_config& c = h->cfg;
  const int C = c.n_embd, H = c.n_head, hd = C / H, Vp = c.padded_vocab_size;
  const long BT = (long)B * T;
  const DType at = h->act;
  hipStream_t s = h->stream;
  float* P = h->params;
  TIMED(h, GPT2_SITE_EMBED_FWD, launch_embed_fwd(d_idx, h->idx, P + h->lay.wte, P + h->lay.wpe, h->A[0].x_in, B, T, C,
                             Vp, h->err, s));
  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& o = h->lay.layer[l];
    LayerAct& a = h->A[l];
    float* x_out = l + 1 < c.n_layer ? h->A[l + 1].x_in : h->x_final;
    TIMED(h, GPT2_SITE_LN_FWD, launch_layernorm_fwd(at, a.x_in, P + o.ln1w, P + o.ln1b, a.u1, a.mean1, a.rstd1, BT,
                                   C, s));
    EpiArgs e = epi(a.qkv, 3 * C);
    e.bias = P + o.attnb;
    TIMED(h, GPT2_SITE_QKV_FWD, launch_gemm_fill(at, (int)BT, 3 * C, C, a.u1, C, false, W(h, o.attnw), C,
                                                 false, EPI_BIAS, at, e, h->splitk, SPLITK_PART_ELEMS, s));
    TIMED(h, GPT2_SITE_ATTN_FWD, launch_attn_fwd(at, a.qkv, a.y, a.lse, B, T, H, hd, s));
    e = epi(a.x_mid, C);
    e.bias = P + o.projb;
    e.resid = a.x_in;
    e.ldr = C;
    TIMED(h, GPT2_SITE_PROJ_FWD, launch_gemm_fill(at, (int)BT, C, C, a.y, C, false, W(h, o.projw), C, false,
                                                  EPI_RESID, DT_F32, e, h->splitk, SPLITK_PART_ELEMS, s));
    TIMED(h, GPT2_SITE_LN_FWD, launch_layernorm_fwd(at, a.x_mid, P + o.ln2w, P + o.ln2b, a.u2, a.mean2, a.rstd2, BT,
                                   C, s));
    e = epi(a.h, 4 * C);
    e.out2 = a.g;
    e.bias = P + o.fcb;
    TIMED(h, GPT2_SITE_FC_FWD, launch_gemm_fill(at, (int)BT, 4 * C, C, a.u2, C, false, W(h, o.fcw), C,
                                                false, EPI_BIAS_GELU, at, e, h->splitk, SPLITK_PART_ELEMS, s));
    e = epi(x_out, C);
    e.bias = P + o.fc2b;
    e.resid = a.x_mid;
    e.ldr = C;
    TIMED(h, GPT2_SITE_FCPROJ_FWD, launch_gemm_fill(at, (int)BT, C, 4 * C, a.g, 4 * C, false, W(h, o.fc2w),
                                                    4 * C, false, EPI_RESID, DT_F32, e, h->splitk,
                                                    SPLITK_PART_ELEMS, s));
  }
  TIMED(h, GPT2_SITE_LN_FWD, launch_layernorm_fwd(at, h->x_final, P + h->lay.lnfw, P + h->lay.lnfb, h->z, h->meanf,
                                 h->rstdf, BT, C, s));
  if (last_logits) {
    // rows T-1, 2T-1, ... of z: a row stride of T*C
    const size_t es = at == DT_BF16 ? 2 : 4;
    const void* zl = static_cast<const char*>(h->z) + (size_t)(T - 1) * C * es;
    TIMED(h, GPT2_SITE_LMHEAD_FWD, launch_gemm(at, B, Vp, C, zl, (long)T * C, false, W(h, h->lay.wte), C,
                                               false, EPI_STORE, DT_F32, epi(last_logits, Vp), 0, s));
    return GPT2_OK;
  }
  if (h->head_chunk) {
    // fused lm_head + cross-entropy: per-row log-sum-exp partials and the
    // target's logit straight from the GEMM's accumulators; no logits kept
    // (and without targets there is nothing to compute)
    if (!d_tgt) return GPT2_OK;
    HIPTRY(h, hipMemcpyAsync(h->tgt, d_tgt, BT * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
    EpiArgs e = epi(nullptr, 0);
    e.tgt = h->tgt;
    e.part = h->hpart;
    e.tlogit = h->htlogit;
    e.nblk = Vp / 64;
    TIMED(h, GPT2_SITE_LMHEAD_FWD, launch_gemm(at, (int)BT, Vp, C, h->z, C, false, W(h, h->lay.wte), C,
                                               false, EPI_LSE, DT_F32, e, 0, s));
    TIMED(h, GPT2_SITE_XENT, launch_head_loss(h->hpart, Vp / 64, h->htlogit, h->tgt, h->n_valid, h->hlse,
                                              h->row_loss, h->loss, BT, Vp, h->err, s));
    return GPT2_OK;
  }
  EpiArgs e = epi(h->logits, Vp);
  TIMED(h, GPT2_SITE_LMHEAD_FWD, launch_gemm(at, (int)BT, Vp, C, h->z, C, false, W(h, h->lay.wte), C, false, EPI_STORE,
                        at, e, 0, s));
  if (d_tgt)
    TIMED(h, GPT2_SITE_XENT, launch_xent(at, h->logits, d_tgt, h->n_valid, h->row_loss, h->loss, BT, Vp, h->err,
                          grad, s));
  return GPT2_OK;
}

// bf16-mode backward buffers.  The residual gradient's bf16 copy has 2L
// slots: 2l holds the gradient at block l's output (read by its mlp c_proj
// products), 2l+1 the gradient at its x_mid (read by its attn c_proj
// products).  dh (dbig) and dqkv have one slot per block.  Keeping every
// slot until the end of the backward pass lets all weight gradients run as
// one grouped launch there.
size_t bt_max(const gpt2* h) { return (size_t)h->cfg.max_batch * h->cfg.block_size; }
bf16_t* dres_slot(const gpt2* h, int i) {
  return reinterpret_cast<bf16_t*>(h->dres_b) + (size_t)i * bt_max(h) * h->cfg.n_embd;
}
void* dbig_slot(const gpt2* h, int l) {
  if (h->act != DT_BF16) return h->dbig;
  return reinterpret_cast<bf16_t*>(h->dbig) + (size_t)l * bt_max(h) * 4 * h->cfg.n_embd;
}
void* dqkv_slot(const gpt2* h, int l) {
  if (h->act != DT_BF16) return h->dqkv;
  return reinterpret_cast<bf16_t*>(h->dqkv) + (size_t)l * bt_max(h) * 3 * h->cfg.n_embd;
}

float* ln_slot(const gpt2* h, int i) {
  return h->ln_parts + (size_t)i * ln_bwd_scratch(bt_max(h), h->cfg.n_embd);
}
float* fcb_slot(const gpt2* h, int l) {
  return h->fcb_parts + (size_t)l * fcb_part_rows(bt_max(h)) * 4 * h->cfg.n_embd;
}
float* attnb_slot(const gpt2* h, int l) {
  return h->attnb_parts + (size_t)l * attnb_part_rows(&h->cfg) * 3 * h->cfg.n_embd;
}

// The column sums the backward defers to its end: LayerNorm weight, bias and
// the residual-gradient sums that are the c_proj bias gradients, the c_fc and
// the c_attn bias gradients.  Every destination appears once.
std::vector<ColsumProblem> colsum_problems(gpt2* h, int* total_chunks) {
  std::vector<ColsumProblem> v;
  const int C = h->cfg.n_embd, L = h->cfg.n_layer;
  float* G = h->grads;
  int chunk0 = 0;
  auto add = [&](const float* part, int ncols, int w, float* d0, float* d1, float* d2, int rpp,
                 int fixed) {
    ColsumProblem q{};
    q.partial = part;
    q.dst[0] = d0; q.dst[1] = d1; q.dst[2] = d2;
    q.ncols = ncols; q.w = w;
    q.rows_per_part = rpp; q.fixed_parts = fixed;
    q.chunk0 = chunk0;
    chunk0 += (ncols + 63) / 64;
    v.push_back(q);
  };
  const bool bf = h->act == DT_BF16;
  add(ln_slot(h, 2 * L), 3 * C, C, G + h->lay.lnfw, G + h->lay.lnfb, G + h->lay.layer[L - 1].fc2b,
      LN_BWD_ROWS, 0);
  for (int l = L - 1; l >= 0; --l) {
    const LayerOff& o = h->lay.layer[l];
    add(fcb_slot(h, l), 4 * C, 4 * C, G + o.fcb, nullptr, nullptr, bf ? 128 : 0, bf ? 0 : BIAS_SPLITS);
    add(ln_slot(h, 2 * l + 1), 3 * C, C, G + o.ln2w, G + o.ln2b, G + o.projb, LN_BWD_ROWS, 0);
    add(attnb_slot(h, l), 3 * C, 3 * C, G + o.attnb, nullptr, nullptr, bf ? -1 : 0,
        bf ? 0 : BIAS_SPLITS);
    add(ln_slot(h, 2 * l), 3 * C, C, G + o.ln1w, G + o.ln1b,
        l > 0 ? G + h->lay.layer[l - 1].fc2b : nullptr, LN_BWD_ROWS, 0);
  }
  *total_chunks = chunk0;
  return v;
}

// The grouped weight-gradient products (bf16 mode): the lm_head's (unless
// the head is fused) and, per block, mlp c_proj, c_fc, attn c_proj, c_attn:
// dW = dY^T X with dY, X the saved (B*T, width) activations.
std::vector<GemmProblem> wgrad_problems(gpt2* h, long* total_tiles) {
  std::vector<GemmProblem> v;
  const int C = h->cfg.n_embd, Vp = h->cfg.padded_vocab_size;
  long item0 = 0;
  auto add = [&](const void* dY, long ldy, const void* X, long ldx, float* out, int Mo, int No,
                 int scaled) {
    GemmProblem p;
    p.A = static_cast<const bf16_t*>(dY);
    p.B = static_cast<const bf16_t*>(X);
    p.out = out;
    p.lda = ldy;
    p.ldb = ldx;
    p.ldo = No;
    p.M = Mo;
    p.N = No;
    p.tiles_m = (Mo + 255) / 256;
    p.tiles_n = (No + 255) / 256;
    p.item0 = item0;
    p.alpha = 1.f;
    p.scaled = scaled;
    item0 += (long)p.tiles_m * p.tiles_n;
    v.push_back(p);
  };
  float* G = h->grads;
  if (!h->head_chunk) add(h->logits, Vp, h->z, C, G + h->lay.wte, Vp, C, 1);
  for (int l = h->cfg.n_layer - 1; l >= 0; --l) {
    const LayerOff& o = h->lay.layer[l];
    const LayerAct& a = h->A[l];
    add(dres_slot(h, 2 * l), C, a.g, 4 * C, G + o.fc2w, C, 4 * C, 0);
    add(dbig_slot(h, l), 4 * C, a.u2, C, G + o.fcw, 4 * C, C, 0);
    add(dres_slot(h, 2 * l + 1), C, a.y, C, G + o.projw, C, C, 0);
    add(dqkv_slot(h, l), 3 * C, a.u1, C, G + o.attnw, 3 * C, C, 0);
  }
  // Whole rounds of tiles: a last round holding rem < slots/2 tiles would
  // leave most CUs idle for a whole tile.  Move the last r tile-rows (r x
  // tiles_n >= rem tiles) of the first product into a tail launch of split-K
  // slices that fills the GPU for a fraction of that time.
  h->wg_tail = GemmProblem{};
  const long slots = gemm_slots();
  const long rem = item0 % slots;
  GemmProblem& p0 = v[0];
  const int r = (int)((rem + p0.tiles_n - 1) / p0.tiles_n);
  if (rem > 0 && rem * 2 < slots && r < p0.tiles_m && (long)r * p0.tiles_n * 2 <= slots) {
    const int M1 = (p0.tiles_m - r) * 256;
    GemmProblem t = p0;
    t.A = p0.A + M1;
    t.out = p0.out + (long)M1 * p0.ldo;
    t.M = p0.M - M1;
    h->wg_tail = t;
    p0.M = M1;
    p0.tiles_m -= r;
    const long moved = (long)r * p0.tiles_n;
    for (size_t i = 1; i < v.size(); ++i) v[i].item0 -= moved;
    item0 -= moved;
  }
  *total_tiles = item0;
  return v;
}

// Carries out a deferred gpt2_zero_grad.
gpt2_status settle_zero(gpt2* h) {
  if (!h->zero_pending) return GPT2_OK;
  h->zero_pending = false;
  TIMED(h, GPT2_SITE_ZERO_GRAD, launch_fill(h->grads, h->lay.P, 0.f, h->stream));
  return GPT2_OK;
}

gpt2_status run_backward(gpt2* h, float scale) {
  const gpt2_config& c = h->cfg;
  const int B = h->B, T = h->T;
  const int C = c.n_embd, H = c.n_head, hd = C / H, Vp = c.padded_vocab_size;
  const long BT = (long)B * T;
  const int M = (int)BT;
  const DType at = h->act;
  hipStream_t s = h->stream;
  float* P = h->params;
  float* G = h->grads;
  const bool bf = at == DT_BF16;
  // bf16: every weight gradient in one grouped launch at the end (whole
  // tiles over the B*T contraction), when B*T is a multiple of 64
  const bool grouped = bf && h->wg_n > 0 && M % 64 == 0;
  // After gpt2_zero_grad, with the grouped weight gradients every gradient
  // element is written by exactly one of: the grouped launch and its tail
  // (every matrix; wte whole with the materialised head), the fused head's
  // slices (wte whole otherwise), the grouped column sums (every vector),
  // the wpe pass (rows < T; rows T.. zeroed here) -- so they store instead
  // of adding, and nothing is zeroed first.  The embedding's rows of dwte
  // are added after the lm_head's are stored.
  const bool store = h->zero_pending && grouped;
  if (store) {
    h->zero_pending = false;
    if (T < c.block_size)
      HIPTRY(h, launch_fill(G + h->lay.wpe + (long)T * C, (long)(c.block_size - T) * C, 0.f, s));
  } else {
    const gpt2_status st = settle_zero(h);
    if (st != GPT2_OK) return st;
  }

  // lm_head (tied): dz = s dlogits wte ; dwte += s dlogits^T z
  if (h->head_chunk) {
    // fused head: per slice of the vocabulary, recompute the logits and turn
    // them into d(loss)/d(logits) in the GEMM epilogue, then the slice's
    // share of dz (accumulated over slices in a fixed order) and its rows of
    // dwte
    for (int v0 = 0; v0 < Vp; v0 += h->head_chunk) {
      const int nc = std::min(h->head_chunk, Vp - v0);
      EpiArgs e = epi(h->hslice, nc);
      e.tgt = h->tgt;
      e.lse = h->hlse;
      e.n_valid = h->n_valid;
      e.col0 = v0;
      TIMED(h, GPT2_SITE_LMHEAD_RECOMP, launch_gemm(at, M, nc, C, h->z, C, false,
                                                    W(h, h->lay.wte + (long)v0 * C), C, false,
                                                    EPI_DLOGITS, at, e, 0, s));
      const WOp ws = w_dx(h, h->lay.wte, Vp, C, v0);
      TIMED(h, GPT2_SITE_LMHEAD_DX, launch_gemm(at, M, C, nc, h->hslice, nc, false, ws.p, ws.ld, ws.t,
                                                v0 == 0 ? EPI_STORE : EPI_ACCUM, DT_F32,
                                                epi(h->dxtmp, C, scale), 0, s));
      TIMED(h, GPT2_SITE_LMHEAD_DW, launch_gemm_wgrad(at, nc, C, M, h->hslice, nc, true, h->z, C, true,
                                                      G + h->lay.wte + (long)v0 * C, C, scale,
                                                      h->splitk, SPLITK_PART_ELEMS, s, store));
    }
  } else {
    const WOp wl = w_dx(h, h->lay.wte, Vp, C);
    TIMED(h, GPT2_SITE_LMHEAD_DX, launch_gemm(at, M, C, Vp, h->logits, Vp, false, wl.p, wl.ld, wl.t,
                                              EPI_STORE, DT_F32, epi(h->dxtmp, C, scale), 0, s));
    if (!grouped)
      TIMED(h, GPT2_SITE_LMHEAD_DW, launch_gemm_wgrad(at, Vp, C, M, h->logits, Vp, true, h->z, C, true,
                                                      G + h->lay.wte, C, scale, h->splitk,
                                                      SPLITK_PART_ELEMS, s));
  }
  // also the bias gradient of the last block's mlp c_proj: sum of dres
  TIMED(h, GPT2_SITE_LN_BWD, launch_layernorm_bwd(at, h->dxtmp, h->x_final, h->meanf, h->rstdf, P + h->lay.lnfw,
                                 h->dres, bf ? dres_slot(h, 2 * (c.n_layer - 1)) : nullptr, 0,
                                 ln_slot(h, 2 * c.n_layer), BT, C, s));
  for (int l = c.n_layer - 1; l >= 0; --l) {
    const LayerOff& o = h->lay.layer[l];
    LayerAct& a = h->A[l];
    // this block's backward buffers (bf16 mode: its own slots)
    const void* dres_out = bf ? (const void*)dres_slot(h, 2 * l) : (const void*)h->dres;
    const void* dres_mid = bf ? (const void*)dres_slot(h, 2 * l + 1) : (const void*)h->dres;
    void* dbig = dbig_slot(h, l);
    void* dqkv = dqkv_slot(h, l);
    // x_out = x_mid + c_proj(gelu(c_fc(ln_2(x_mid))))
    // dh = dg * gelu'(h), the forward having saved gelu'(h); in bf16 mode the
    // same epilogue leaves per-128-row column sums of dh (the c_fc bias
    // gradient) in the block's slot
    EpiArgs e = epi(dbig, 4 * C);
    e.aux = a.h;
    e.ldx = 4 * C;
    if (at == DT_BF16) e.colsum = fcb_slot(h, l);
    const WOp w2 = w_dx(h, o.fc2w, C, 4 * C);
    TIMED(h, GPT2_SITE_FCPROJ_DX, launch_gemm(at, M, 4 * C, C, dres_out, C, false, w2.p, w2.ld, w2.t,
                          EPI_GELU_BWD, at, e, 0, s));
    if (!grouped)
      TIMED(h, GPT2_SITE_FCPROJ_DW, launch_gemm_wgrad(at, C, 4 * C, M, dres_out, C, true, a.g, 4 * C,
                                                      true, G + o.fc2w, 4 * C, 1.f, h->splitk,
                                                      SPLITK_PART_ELEMS, s));
    const WOp w1 = w_dx(h, o.fcw, 4 * C, C);
    TIMED(h, GPT2_SITE_FC_DX, launch_gemm(at, M, C, 4 * C, dbig, 4 * C, false, w1.p, w1.ld, w1.t, EPI_STORE,
                          DT_F32, epi(h->dxtmp, C), 0, s));
    if (!grouped)
      TIMED(h, GPT2_SITE_FC_DW, launch_gemm_wgrad(at, 4 * C, C, M, dbig, 4 * C, true, a.u2, C, true,
                                                  G + o.fcw, C, 1.f, h->splitk, SPLITK_PART_ELEMS, s));
    if (!bf)
      TIMED(h, GPT2_SITE_BIAS_GRAD, launch_colsum_parts(at, dbig, BT, 4 * C, 4 * C, fcb_slot(h, l), s));
    TIMED(h, GPT2_SITE_LN_BWD, launch_layernorm_bwd(at, h->dxtmp, a.x_mid, a.mean2, a.rstd2, P + o.ln2w, h->dres,
                                   bf ? dres_slot(h, 2 * l + 1) : nullptr, 1, ln_slot(h, 2 * l + 1),
                                   BT, C, s));
    // x_mid = x_in + c_proj(attn(ln_1(x_in)))
    const WOp wp = w_dx(h, o.projw, C, C);
    TIMED(h, GPT2_SITE_PROJ_DX, launch_gemm(at, M, C, C, dres_mid, C, false, wp.p, wp.ld, wp.t, EPI_STORE, at,
                          epi(h->dy, C), 0, s));
    if (!grouped)
      TIMED(h, GPT2_SITE_PROJ_DW, launch_gemm_wgrad(at, C, C, M, dres_mid, C, true, a.y, C, true,
                                                    G + o.projw, C, 1.f, h->splitk,
                                                    SPLITK_PART_ELEMS, s));
    // (bf16: the attention backward also leaves the c_attn bias gradient's
    // partial sums in the block's slot)
    TIMED(h, GPT2_SITE_ATTN_BWD, launch_attn_bwd(at, a.qkv, a.y, a.lse, h->dy, dqkv, h->dbuf, B, T, H, hd,
                                                 bf ? attnb_slot(h, l) : nullptr, s));
    const WOp wq = w_dx(h, o.attnw, 3 * C, C);
    TIMED(h, GPT2_SITE_QKV_DX, launch_gemm(at, M, C, 3 * C, dqkv, 3 * C, false, wq.p, wq.ld, wq.t,
                          EPI_STORE, DT_F32, epi(h->dxtmp, C), 0, s));
    if (!grouped)
      TIMED(h, GPT2_SITE_QKV_DW, launch_gemm_wgrad(at, 3 * C, C, M, dqkv, 3 * C, true, a.u1, C, true,
                                                   G + o.attnw, C, 1.f, h->splitk,
                                                   SPLITK_PART_ELEMS, s));
    if (!bf)
      TIMED(h, GPT2_SITE_BIAS_GRAD, launch_colsum_parts(at, dqkv, BT, 3 * C, 3 * C, attnb_slot(h, l), s));
    // the new dres also gives the bias gradient of the previous block's mlp
    // c_proj (its column sums, in the same slot)
    TIMED(h, GPT2_SITE_LN_BWD, launch_layernorm_bwd(at, h->dxtmp, a.x_in, a.mean1, a.rstd1, P + o.ln1w, h->dres,
                                   bf && l > 0 ? dres_slot(h, 2 * (l - 1)) : nullptr, 1,
                                   ln_slot(h, 2 * l), BT, C, s));
  }
  // LayerNorm parameter and bias gradients from every slot of partial sums
  TIMED(h, GPT2_SITE_BIAS_GRAD, launch_colsum_grouped(h->cs_probs, h->cs_n, h->cs_chunks, M,
                                                      B * ((T + 127) / 128), store, s));
  if (grouped) {
    TIMED(h, GPT2_SITE_WGRAD, launch_gemm_grouped_wgrad(h->wg_probs, h->wg_n, h->wg_tiles, M, scale,
                                                        store, s));
    const GemmProblem& t = h->wg_tail;
    if (t.M > 0)
      TIMED(h, GPT2_SITE_WGRAD_TAIL, launch_gemm_wgrad(at, t.M, t.N, M, t.A, t.lda, true, t.B, t.ldb, true,
                                                       t.out, t.ldo, t.scaled ? t.alpha * scale : t.alpha,
                                                       h->splitk, SPLITK_PART_ELEMS, s, store));
  }
  TIMED(h, GPT2_SITE_EMBED_BWD, launch_embed_bwd(h->idx, h->dres, G + h->lay.wte, G + h->lay.wpe, B, T, C,
                                                 c.padded_vocab_size, h->emb_scratch, store, s));
  return GPT2_OK;
}

// The seeded initialisation of every tensor (Layout::t_init), then the bf16
// weight copies the products read.
hipError_t init_params(gpt2* h, uint64_t seed) {
  const Layout& L = h->lay;
  const float std_w = 0.02f;
  const float std_r = (float)(0.02 / std::sqrt(2.0 * h->cfg.n_layer));
  for (size_t t = 0; t < L.t_off.size(); ++t) {
    float* p = h->params + L.t_off[t];
    hipError_t e = hipSuccess;
    switch (L.t_init[t]) {
      case INIT_ZERO: e = launch_fill(p, L.t_len[t], 0.f, h->stream); break;
      case INIT_ONE: e = launch_fill(p, L.t_len[t], 1.f, h->stream); break;
      case INIT_NORMAL:
        e = launch_init_normal(p, L.t_len[t], L.t_off[t], std_w, seed, h->stream);
        break;
      default:
        e = launch_init_normal(p, L.t_len[t], L.t_off[t], std_r, seed, h->stream);
        break;
    }
    if (e != hipSuccess) return e;
  }
  if (h->shadow) {
    hipError_t e = launch_f32_to_bf16(h->params, h->shadow, L.P, h->stream);
    if (e == hipSuccess)
      e = launch_transpose_tiles(h->shadow, h->shadow_t, h->ttiles, h->nttiles, h->stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Key/value cache of block l: (max_batch, block_size, 2C) rows [k | v].
void* kv_slot(const gpt2* h, int l) {
  return static_cast<char*>(h->kv) +
         (size_t)l * bt_max(h) * 2 * h->cfg.n_embd * h->act_size;
}

// One decoding step: the blocks for position p of each sequence only, the
// token ids d_tok (B, device), the keys and values of positions < p read from
// the cache and those of p appended to it; the logits of position p (B, Vp)
// fp32 into `logits`.  The activations of layer 0 serve as scratch.
gpt2_status run_decode(gpt2* h, const int32_t* d_tok, int B, int p, float* logits) {
  const gpt2_config& c = h->cfg;
  const int C = c.n_embd, H = c.n_head, hd = C / H, Vp = c.padded_vocab_size;
  const DType at = h->act;
  hipStream_t s = h->stream;
  float* P = h->params;
  LayerAct& a = h->A[0];
  float* x = a.x_in;      // residual stream, B rows
  float* xm = a.x_mid;
  TIMED(h, GPT2_SITE_EMBED_FWD, launch_embed_fwd(d_tok, h->idx, P + h->lay.wte,
                                                 P + h->lay.wpe + (long)p * C, x, B, 1, C, Vp,
                                                 h->err, s));
  // bf16 with at most 16 sequences: each LayerNorm runs inside the few-rows
  // GEMM that reads it (one launch instead of two)
  const bool ln_fused = at == DT_BF16 && B <= 16 && C % 32 == 0 && C <= LN_SKINNY_MAX_K;
  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& o = h->lay.layer[l];
    EpiArgs e = epi(a.qkv, 3 * C);
    e.bias = P + o.attnb;
    if (ln_fused) {
      TIMED(h, GPT2_SITE_QKV_FWD, launch_gemm_ln_skinny(B, 3 * C, C, x, P + o.ln1w, P + o.ln1b,
                                                        W(h, o.attnw), C, EPI_BIAS, at, e, s));
    } else {
      TIMED(h, GPT2_SITE_LN_FWD, launch_layernorm_fwd(at, x, P + o.ln1w, P + o.ln1b, a.u1, a.mean1,
                                                      a.rstd1, B, C, s));
      TIMED(h, GPT2_SITE_QKV_FWD, launch_gemm_fill(at, B, 3 * C, C, a.u1, C, false, W(h, o.attnw),
                                                   C, false, EPI_BIAS, at, e, h->splitk,
                                                   SPLITK_PART_ELEMS, s));
    }
    // (appends position p's key and value to the cache, then attends)
    TIMED(h, GPT2_SITE_ATTN_FWD, launch_attn_decode(at, a.qkv, kv_slot(h, l), a.y, B, p,
                                                    c.block_size, H, hd, s));
    e = epi(xm, C);
    e.bias = P + o.projb;
    e.resid = x;
    e.ldr = C;
    TIMED(h, GPT2_SITE_PROJ_FWD, launch_gemm_fill(at, B, C, C, a.y, C, false, W(h, o.projw), C,
                                                  false, EPI_RESID, DT_F32, e, h->splitk,
                                                  SPLITK_PART_ELEMS, s));
    e = epi(a.h, 4 * C);
    e.out2 = a.g;
    e.bias = P + o.fcb;
    if (ln_fused) {
      TIMED(h, GPT2_SITE_FC_FWD, launch_gemm_ln_skinny(B, 4 * C, C, xm, P + o.ln2w, P + o.ln2b,
                                                       W(h, o.fcw), C, EPI_BIAS_GELU, at, e, s));
    } else {
      TIMED(h, GPT2_SITE_LN_FWD, launch_layernorm_fwd(at, xm, P + o.ln2w, P + o.ln2b, a.u2, a.mean2,
                                                      a.rstd2, B, C, s));
      TIMED(h, GPT2_SITE_FC_FWD, launch_gemm_fill(at, B, 4 * C, C, a.u2, C, false, W(h, o.fcw), C,
                                                  false, EPI_BIAS_GELU, at, e, h->splitk,
                                                  SPLITK_PART_ELEMS, s));
    }
    e = epi(x, C);
    e.bias = P + o.fc2b;
    e.resid = xm;
    e.ldr = C;
    TIMED(h, GPT2_SITE_FCPROJ_FWD, launch_gemm_fill(at, B, C, 4 * C, a.g, 4 * C, false,
                                                    W(h, o.fc2w), 4 * C, false, EPI_RESID, DT_F32,
                                                    e, h->splitk, SPLITK_PART_ELEMS, s));
  }
  if (ln_fused) {
    TIMED(h, GPT2_SITE_LMHEAD_FWD, launch_gemm_ln_skinny(B, Vp, C, x, P + h->lay.lnfw,
                                                         P + h->lay.lnfb, W(h, h->lay.wte), C,
                                                         EPI_STORE, DT_F32, epi(logits, Vp),
                                                         s));
  } else {
    TIMED(h, GPT2_SITE_LN_FWD, launch_layernorm_fwd(at, x, P + h->lay.lnfw, P + h->lay.lnfb, h->z,
                                                    h->meanf, h->rstdf, B, C, s));
    TIMED(h, GPT2_SITE_LMHEAD_FWD, launch_gemm(at, B, Vp, C, h->z, C, false, W(h, h->lay.wte), C,
                                               false, EPI_STORE, DT_F32, epi(logits, Vp), 0,
                                               s));
  }
  return GPT2_OK;
}

float* state_ptr(gpt2* h, int which) {
  switch (which) {
    case GPT2_PARAMS: return h->params;
    case GPT2_GRADS: return h->grads;
    case GPT2_ADAM_M: return h->m;
    case GPT2_ADAM_V: return h->v;
  }
  return nullptr;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

size_t gpt2_num_params(const gpt2_config* cfg) {
  if (!valid_config(cfg, nullptr)) return 0;
  return (size_t)make_layout(cfg).P;
}

gpt2_status gpt2_workspace_bytes(const gpt2_config* cfg, size_t* bytes) {
  if (!bytes || !valid_config(cfg, nullptr)) return GPT2_E_ARG;
  *bytes = plan(cfg, nullptr, nullptr);
  return GPT2_OK;
}

gpt2_status gpt2_init(const gpt2_config* cfg, void* d_workspace, size_t ws_bytes,
                      void* hip_stream, uint64_t seed, gpt2_t** out) {
  if (!out) return GPT2_E_ARG;
  *out = nullptr;
  if (!valid_config(cfg, nullptr) || !d_workspace) return GPT2_E_ARG;
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256) return GPT2_E_ARG;
  size_t need = plan(cfg, nullptr, nullptr);
  if (ws_bytes < need) return GPT2_E_ARG;
  gpt2* h = new gpt2();
  h->cfg = *cfg;
  h->stream = reinterpret_cast<hipStream_t>(hip_stream);
  h->act = cfg->precision == GPT2_BF16 ? DT_BF16 : DT_F32;
  h->act_size = h->act == DT_BF16 ? 2 : 4;
  plan(cfg, reinterpret_cast<char*>(d_workspace), h);
  std::vector<AdamChunk> ch = make_chunks(h->lay, h->act == DT_BF16);
  hipError_t e = hipMemcpyAsync(h->chunks, ch.data(), ch.size() * sizeof(AdamChunk),
                                hipMemcpyHostToDevice, h->stream);
  std::vector<TTile> tt = h->nttiles ? make_ttiles(h->lay, cfg) : std::vector<TTile>();
  std::vector<GemmProblem> wg;
  if (h->act == DT_BF16) {
    wg = wgrad_problems(h, &h->wg_tiles);
    h->wg_n = (int)wg.size();
    for (const GemmProblem& q : wg) h->wg_elems += (long)q.M * q.N;
    if (e == hipSuccess)
      e = hipMemcpyAsync(h->wg_probs, wg.data(), wg.size() * sizeof(GemmProblem),
                         hipMemcpyHostToDevice, h->stream);
  }
  if (e == hipSuccess && !tt.empty())
    e = hipMemcpyAsync(h->ttiles, tt.data(), tt.size() * sizeof(TTile), hipMemcpyHostToDevice,
                       h->stream);
  std::vector<ColsumProblem> cs = colsum_problems(h, &h->cs_chunks);
  h->cs_n = (int)cs.size();
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->cs_probs, cs.data(), cs.size() * sizeof(ColsumProblem),
                       hipMemcpyHostToDevice, h->stream);
  for (float* t : {h->grads, h->m, h->v})
    if (e == hipSuccess) e = launch_fill(t, h->lay.P, 0.f, h->stream);
  if (e == hipSuccess) e = init_params(h, seed);
  if (e == hipSuccess) e = hipMemsetAsync(h->err, 0, sizeof(int), h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) {
    delete h;
    return GPT2_E_HIP;
  }
  *out = h;
  return GPT2_OK;
}

gpt2_status gpt2_set_params(gpt2_t* h, const float* src, size_t n, int src_on_device) {
  if (!h || !src) return GPT2_E_ARG;
  if (n != (size_t)h->lay.P) return fail(h, GPT2_E_ARG, "n != gpt2_num_params");
  h->kv_len = 0;  // cached keys and values belong to the old parameters
  HIPTRY(h, hipMemcpyAsync(h->params, src, n * 4,
                           src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice,
                           h->stream));
  if (h->shadow) {
    HIPTRY(h, launch_f32_to_bf16(h->params, h->shadow, (long)n, h->stream));
    HIPTRY(h, launch_transpose_tiles(h->shadow, h->shadow_t, h->ttiles, h->nttiles, h->stream));
  }
  for (float* t : {h->grads, h->m, h->v}) HIPTRY(h, launch_fill(t, (long)n, 0.f, h->stream));
  h->zero_pending = false;
  h->step = 0;
  if (!src_on_device) HIPTRY(h, hipStreamSynchronize(h->stream));
  return GPT2_OK;
}

gpt2_status gpt2_get(gpt2_t* h, int which, float* dst, size_t n, int dst_on_device) {
  if (!h || !dst) return GPT2_E_ARG;
  float* p = state_ptr(h, which);
  if (!p) return fail(h, GPT2_E_ARG, "unknown state id");
  if (n != (size_t)h->lay.P) return fail(h, GPT2_E_ARG, "n != gpt2_num_params");
  if (which == GPT2_GRADS) {
    const gpt2_status st = settle_zero(h);
    if (st != GPT2_OK) return st;
  }
  HIPTRY(h, hipMemcpyAsync(dst, p, n * 4,
                           dst_on_device ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost,
                           h->stream));
  if (!dst_on_device) return sync(h);
  return GPT2_OK;
}

gpt2_status gpt2_set_state(gpt2_t* h, int which, const float* src, size_t n, int src_on_device) {
  if (!h || !src) return GPT2_E_ARG;
  if (which == GPT2_PARAMS) return fail(h, GPT2_E_ARG, "use gpt2_set_params for parameters");
  float* p = state_ptr(h, which);
  if (!p) return fail(h, GPT2_E_ARG, "unknown state id");
  if (n != (size_t)h->lay.P) return fail(h, GPT2_E_ARG, "n != gpt2_num_params");
  if (which == GPT2_GRADS) h->zero_pending = false;  // overwritten whole
  HIPTRY(h, hipMemcpyAsync(p, src, n * 4,
                           src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice,
                           h->stream));
  if (!src_on_device) HIPTRY(h, hipStreamSynchronize(h->stream));
  return GPT2_OK;
}

gpt2_status gpt2_get_step(const gpt2_t* h, int64_t* t) {
  if (!h || !t) return GPT2_E_ARG;
  *t = h->step;
  return GPT2_OK;
}

gpt2_status gpt2_wgrad_layout(const gpt2_t* h, int64_t* grouped_elems, int64_t* tail_elems,
                              int64_t* grouped_tiles) {
  if (!h) return GPT2_E_ARG;
  const bool g = h->wg_n > 0;
  if (grouped_elems) *grouped_elems = g ? h->wg_elems : 0;
  if (tail_elems) *tail_elems = g ? (int64_t)h->wg_tail.M * h->wg_tail.N : 0;
  if (grouped_tiles) *grouped_tiles = g ? h->wg_tiles : 0;
  return GPT2_OK;
}

gpt2_status gpt2_set_step(gpt2_t* h, int64_t t) {
  if (!h || t < 0) return GPT2_E_ARG;
  h->step = t;
  return GPT2_OK;
}

gpt2_status gpt2_lr_at(int64_t step, double eta_max, double eta_min, int64_t warmup_steps,
                       int64_t max_steps, double* lr) {
  if (!lr || step < 0 || warmup_steps < 1 || max_steps < warmup_steps) return GPT2_E_ARG;
  // which phase the step is in, and how far through it
  double v;
  if (step >= warmup_steps && step <= max_steps) {
    const double span = (double)(max_steps - warmup_steps);
    const double frac = span > 0 ? (double)(step - warmup_steps) / span : 0.0;
    const double half_cos = 0.5 * (1.0 + std::cos(M_PI * frac));  // 1 at the start, 0 at the end
    v = eta_min + (eta_max - eta_min) * half_cos;
  } else if (step > max_steps) {
    v = eta_min;
  } else {
    v = eta_max * (double)(step + 1) / (double)warmup_steps;
  }
  *lr = v;
  return GPT2_OK;
}

gpt2_status gpt2_forward(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, int B, int T,
                         float* h_loss) {
  if (!h || !d_idx) return GPT2_E_ARG;
  if (B < 1 || B > h->cfg.max_batch || T < 1 || T > h->cfg.block_size)
    return fail(h, GPT2_E_SHAPE, "need 1 <= B <= max_batch and 1 <= T <= block_size");
  h->B = B;
  h->T = T;
  h->have_targets = false;
  h->forward_done = false;
  gpt2_status st = run_forward(h, d_idx, d_targets, B, T, true);
  if (st != GPT2_OK) return st;
  h->forward_done = true;
  h->have_targets = d_targets != nullptr;
  if (h_loss) {
    if (!d_targets) return fail(h, GPT2_E_ARG, "h_loss given without targets");
    return gpt2_get_loss(h, h_loss);
  }
  return GPT2_OK;
}

gpt2_status gpt2_forward_last(gpt2_t* h, const int32_t* d_idx, int B, int T, float* d_logits) {
  if (!h || !d_idx || !d_logits) return GPT2_E_ARG;
  if (B < 1 || B > h->cfg.max_batch || T < 1 || T > h->cfg.block_size)
    return fail(h, GPT2_E_SHAPE, "need 1 <= B <= max_batch and 1 <= T <= block_size");
  h->B = B;
  h->T = T;
  h->have_targets = false;
  h->forward_done = false;
  gpt2_status st = run_forward(h, d_idx, nullptr, B, T, false, d_logits);
  if (st != GPT2_OK) return st;
  h->forward_done = true;
  return GPT2_OK;
}

gpt2_status gpt2_sample(gpt2_t* h, const float* d_logits, long ld, int B, int V, float temperature,
                        int top_k, const float* d_uniform, int32_t* d_tokens) {
  if (!h || !d_logits || !d_uniform || !d_tokens) return GPT2_E_ARG;
  if (B < 1 || V < 1 || V > 53248 || ld < V || ld % 4 ||
      reinterpret_cast<uintptr_t>(d_logits) % 16)
    return fail(h, GPT2_E_ARG, "need B >= 1, 1 <= V <= 53248, ld >= V, ld % 4 == 0, "
                               "16-byte aligned logits");
  if (!(temperature > 0.f)) return fail(h, GPT2_E_ARG, "temperature must be > 0");
  HIPTRY(h, launch_sample(d_logits, ld, B, V, temperature, top_k, d_uniform, 1, d_tokens, 1,
                          h->stream));
  return GPT2_OK;
}

gpt2_status gpt2_generate(gpt2_t* h, const int32_t* d_prompt, int B, int T0, int n_new,
                          float temperature, int top_k, const float* d_uniform, int32_t* d_out) {
  if (!h || !d_prompt || !d_out || (n_new > 0 && !d_uniform)) return GPT2_E_ARG;
  if (B < 1 || B > h->cfg.max_batch || T0 < 1 || n_new < 0)
    return fail(h, GPT2_E_SHAPE, "need 1 <= B <= max_batch, T0 >= 1, n_new >= 0");
  if (!(temperature > 0.f)) return fail(h, GPT2_E_ARG, "temperature must be > 0");
  const int Vp = h->cfg.padded_vocab_size, bs = h->cfg.block_size;
  const long L = (long)T0 + n_new;  // row length of d_out
  hipStream_t s = h->stream;
  h->have_targets = false;
  h->forward_done = false;
  HIPTRY(h, hipMemcpy2DAsync(d_out, L * 4, d_prompt, (size_t)T0 * 4, (size_t)T0 * 4, B,
                             hipMemcpyDeviceToDevice, s));
  for (int step = 0; step < n_new; ++step) {
    const long cur = T0 + step;                 // tokens so far
    const int T = cur < bs ? (int)cur : bs;     // the context: the last block_size of them
    HIPTRY(h, hipMemcpy2DAsync(h->gen_idx, (size_t)T * 4, d_out + (cur - T), L * 4, (size_t)T * 4,
                               B, hipMemcpyDeviceToDevice, s));
    gpt2_status st = run_forward(h, h->gen_idx, nullptr, B, T, false, h->gen_logits);
    if (st != GPT2_OK) return st;
    HIPTRY(h, launch_sample(h->gen_logits, Vp, B, Vp, temperature, top_k, d_uniform + step, n_new,
                            d_out + cur, L, s));
  }
  return GPT2_OK;
}

gpt2_status gpt2_generate_cached(gpt2_t* h, const int32_t* d_prompt, int B, int T0, int n_new,
                                 float temperature, int top_k, const float* d_uniform,
                                 int32_t* d_out) {
  if (!h || !d_prompt || !d_out || (n_new > 0 && !d_uniform)) return GPT2_E_ARG;
  if (B < 1 || B > h->cfg.max_batch || T0 < 1 || n_new < 0)
    return fail(h, GPT2_E_SHAPE, "need 1 <= B <= max_batch, T0 >= 1, n_new >= 0");
  if (!(temperature > 0.f)) return fail(h, GPT2_E_ARG, "temperature must be > 0");
  const int Vp = h->cfg.padded_vocab_size, bs = h->cfg.block_size;
  if (bs > ATTN_DECODE_MAX_POS)
    return fail(h, GPT2_E_ARG, "the key/value cache supports block_size <= 8192");
  const long L = (long)T0 + n_new;  // row length of d_out
  hipStream_t s = h->stream;
  h->have_targets = false;
  h->forward_done = false;
  h->kv_len = 0;  // the loop overwrites the cache
  HIPTRY(h, hipMemcpy2DAsync(d_out, L * 4, d_prompt, (size_t)T0 * 4, (size_t)T0 * 4, B,
                             hipMemcpyDeviceToDevice, s));
  for (int step = 0; step < n_new; ++step) {
    const long cur = T0 + step;  // tokens so far; the next one goes to position cur
    gpt2_status st = GPT2_OK;
    if (cur <= bs && step > 0) {
      // the last drawn token at position cur - 1 against the cached ones
      HIPTRY(h, hipMemcpy2DAsync(h->gen_idx, 4, d_out + (cur - 1), L * 4, 4, B,
                                 hipMemcpyDeviceToDevice, s));
      st = run_decode(h, h->gen_idx, B, (int)(cur - 1), h->gen_logits);
    } else {
      // the prompt (filling the cache), or a window that has shifted: the
      // last block_size tokens at positions 0 .. T-1, recomputed whole
      const int T = cur < bs ? (int)cur : bs;
      HIPTRY(h, hipMemcpy2DAsync(h->gen_idx, (size_t)T * 4, d_out + (cur - T), L * 4,
                                 (size_t)T * 4, B, hipMemcpyDeviceToDevice, s));
      st = run_forward(h, h->gen_idx, nullptr, B, T, false, h->gen_logits);
      if (st == GPT2_OK && step == 0 && cur <= bs)
        for (int l = 0; l < h->cfg.n_layer; ++l)
          HIPTRY(h, launch_kv_append(h->act, h->A[l].qkv, kv_slot(h, l), B, T, 0, bs,
                                     h->cfg.n_embd, s));
    }
    if (st != GPT2_OK) return st;
    HIPTRY(h, launch_sample(h->gen_logits, Vp, B, Vp, temperature, top_k, d_uniform + step, n_new,
                            d_out + cur, L, s));
  }
  return GPT2_OK;
}

gpt2_status gpt2_prefill(gpt2_t* h, const int32_t* d_idx, int B, int T, float* d_logits) {
  if (!h || !d_idx || !d_logits) return GPT2_E_ARG;
  if (reinterpret_cast<uintptr_t>(d_logits) % 16)
    return fail(h, GPT2_E_ARG, "d_logits must be 16-byte aligned");
  if (B < 1 || B > h->cfg.max_batch || T < 1 || T > h->cfg.block_size)
    return fail(h, GPT2_E_SHAPE, "need 1 <= B <= max_batch and 1 <= T <= block_size");
  if (h->cfg.block_size > ATTN_DECODE_MAX_POS)
    return fail(h, GPT2_E_ARG, "the key/value cache supports block_size <= 8192");
  h->kv_len = 0;
  h->have_targets = false;
  h->forward_done = false;
  gpt2_status st = run_forward(h, d_idx, nullptr, B, T, false, d_logits);
  if (st != GPT2_OK) return st;
  for (int l = 0; l < h->cfg.n_layer; ++l)
    HIPTRY(h, launch_kv_append(h->act, h->A[l].qkv, kv_slot(h, l), B, T, 0, h->cfg.block_size,
                               h->cfg.n_embd, h->stream));
  h->kv_B = B;
  h->kv_len = T;
  return GPT2_OK;
}

gpt2_status gpt2_decode(gpt2_t* h, const int32_t* d_tok, int B, int p, float* d_logits) {
  if (!h || !d_tok || !d_logits) return GPT2_E_ARG;
  if (reinterpret_cast<uintptr_t>(d_logits) % 16)
    return fail(h, GPT2_E_ARG, "d_logits must be 16-byte aligned");
  if (h->kv_len < 1 || B != h->kv_B || p != h->kv_len)
    return fail(h, GPT2_E_STATE, "gpt2_decode continues the sequences of the last gpt2_prefill "
                                 "(same B) at the next position");
  if (p >= h->cfg.block_size)
    return fail(h, GPT2_E_SHAPE, "the cache is full (p must be < block_size)");
  h->have_targets = false;
  h->forward_done = false;
  h->kv_len = 0;  // until this step has been issued
  gpt2_status st = run_decode(h, d_tok, B, p, d_logits);
  if (st != GPT2_OK) return st;
  h->kv_len = p + 1;
  return GPT2_OK;
}

gpt2_status gpt2_eval(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, int B, int T,
                      float* d_seq_loss, float* h_loss) {
  if (!h || !d_idx || !d_targets) return GPT2_E_ARG;
  if (B < 1 || B > h->cfg.max_batch || T < 1 || T > h->cfg.block_size)
    return fail(h, GPT2_E_SHAPE, "need 1 <= B <= max_batch and 1 <= T <= block_size");
  h->B = B;
  h->T = T;
  h->have_targets = false;
  h->forward_done = false;
  gpt2_status st = run_forward(h, d_idx, d_targets, B, T, false);
  if (st != GPT2_OK) return st;
  if (d_seq_loss) HIPTRY(h, launch_seq_loss(h->row_loss, d_targets, B, T, d_seq_loss, h->stream));
  h->forward_done = true;  // logits and losses readable; no gradient was formed
  return h_loss ? gpt2_get_loss(h, h_loss) : GPT2_OK;
}

gpt2_status gpt2_get_loss(gpt2_t* h, float* h_loss) {
  if (!h || !h_loss) return GPT2_E_ARG;
  gpt2_status st = sync(h);
  if (st != GPT2_OK) return st;
  HIPTRY(h, hipMemcpy(h_loss, h->loss, sizeof(float), hipMemcpyDeviceToHost));
  return GPT2_OK;
}

gpt2_status gpt2_zero_grad(gpt2_t* h) {
  if (!h) return GPT2_E_ARG;
  h->zero_pending = true;
  return GPT2_OK;
}

gpt2_status gpt2_backward(gpt2_t* h, float loss_scale) {
  if (!h) return GPT2_E_ARG;
  if (!h->forward_done || !h->have_targets)
    return fail(h, GPT2_E_STATE, "backward needs a preceding forward with targets");
  h->have_targets = false;  // the logit gradient is consumed
  return run_backward(h, loss_scale);
}

gpt2_status gpt2_adamw_step(gpt2_t* h, float lr, float beta1, float beta2, float eps,
                            float weight_decay, float max_grad_norm, float* h_grad_norm) {
  if (!h) return GPT2_E_ARG;
  if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f && eps >= 0.f))
    return fail(h, GPT2_E_ARG, "need 0 <= beta < 1 and eps >= 0");
  const gpt2_status st = settle_zero(h);
  if (st != GPT2_OK) return st;
  h->kv_len = 0;  // cached keys and values belong to the old parameters
  h->step += 1;
  const double t = (double)h->step;
  const double bc1 = 1.0 - std::pow((double)beta1, t);
  const double bc2 = 1.0 - std::pow((double)beta2, t);
  const float step_size = (float)(lr / bc1);
  const float inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  TIMED(h, GPT2_SITE_GRAD_NORM, launch_grad_norm(h->grads, h->lay.P, h->norm_partial, max_grad_norm, h->norm, h->clip,
                             h->stream));
  // bf16: the matrices that are also read transposed go tile by tile, writing
  // both bf16 copies; the flat pass takes every other tensor
  if (h->shadow_t)
    TIMED(h, GPT2_SITE_ADAMW, launch_adamw_tiles(h->ttiles, h->nttiles, h->params, h->grads, h->m,
                                                 h->v, h->shadow, h->shadow_t, h->clip, lr, beta1,
                                                 beta2, eps, weight_decay, step_size,
                                                 inv_sqrt_bc2, h->stream));
  TIMED(h, GPT2_SITE_ADAMW, launch_adamw(h->chunks, h->nchunks, h->params, h->grads, h->m, h->v, h->shadow,
                         h->clip, lr, beta1, beta2, eps, weight_decay, step_size, inv_sqrt_bc2,
                         h->stream));
  if (h_grad_norm) return gpt2_get_grad_norm(h, h_grad_norm);
  return GPT2_OK;
}

gpt2_status gpt2_get_grad_norm(gpt2_t* h, float* h_norm) {
  if (!h || !h_norm) return GPT2_E_ARG;
  gpt2_status st = sync(h);
  if (st != GPT2_OK) return st;
  HIPTRY(h, hipMemcpy(h_norm, h->norm, sizeof(float), hipMemcpyDeviceToHost));
  return GPT2_OK;
}

gpt2_status gpt2_sync(gpt2_t* h) {
  if (!h) return GPT2_E_ARG;
  return sync(h);
}

gpt2_status gpt2_timing_begin(gpt2_t* h, uint64_t site_mask) {
  if (!h) return GPT2_E_ARG;
  h->timing_mask = site_mask;
  h->ev_used = 0;
  return GPT2_OK;
}

gpt2_status gpt2_timing_end(gpt2_t* h, double* ms, int32_t* launches) {
  if (!h) return GPT2_E_ARG;
  h->timing_mask = 0;
  HIPTRY(h, hipStreamSynchronize(h->stream));
  std::vector<double> acc(GPT2_NUM_SITES, 0.0);
  std::vector<int32_t> cnt(GPT2_NUM_SITES, 0);
  for (size_t i = 0; i < h->ev_used; ++i) {
    float t = 0.f;
    HIPTRY(h, hipEventElapsedTime(&t, h->ev_pool[2 * i], h->ev_pool[2 * i + 1]));
    acc[h->ev_site[i]] += t;
    cnt[h->ev_site[i]] += 1;
  }
  h->ev_used = 0;
  for (int i = 0; i < GPT2_NUM_SITES; ++i) {
    if (ms) ms[i] = acc[i];
    if (launches) launches[i] = cnt[i];
  }
  return GPT2_OK;
}

const char* gpt2_last_error(const gpt2_t* h) { return h ? h->last_error.c_str() : "null handle"; }

void gpt2_destroy(gpt2_t* h) { delete h; }

gpt2_status gpt2_get_activation(gpt2_t* h, int which, int layer, float* h_dst, size_t n) {
  if (!h || !h_dst) return GPT2_E_ARG;
  if (!h->forward_done) return fail(h, GPT2_E_STATE, "no forward pass has run");
  const gpt2_config& c = h->cfg;
  const size_t BT = (size_t)h->B * h->T, C = c.n_embd;
  const void* src = nullptr;
  size_t count = 0;
  bool f32 = false;
  bool per_layer = which != GPT2_ACT_LNF && which != GPT2_ACT_LOGITS && which != GPT2_ACT_ROW_LOSS;
  int maxl = which == GPT2_ACT_X_IN ? c.n_layer : c.n_layer - 1;
  if (per_layer && (layer < 0 || layer > maxl)) return fail(h, GPT2_E_ARG, "layer out of range");
  const LayerAct* a = per_layer && layer < c.n_layer ? &h->A[layer] : nullptr;
  switch (which) {
    case GPT2_ACT_X_IN: src = layer == c.n_layer ? h->x_final : a->x_in; count = BT * C; f32 = true; break;
    case GPT2_ACT_LN1: src = a->u1; count = BT * C; break;
    case GPT2_ACT_QKV: src = a->qkv; count = BT * 3 * C; break;
    case GPT2_ACT_ATTN_Y: src = a->y; count = BT * C; break;
    case GPT2_ACT_LSE: src = a->lse; count = BT * c.n_head; f32 = true; break;
    case GPT2_ACT_X_MID: src = a->x_mid; count = BT * C; f32 = true; break;
    case GPT2_ACT_LN2: src = a->u2; count = BT * C; break;
    case GPT2_ACT_FC_DGELU: src = a->h; count = BT * 4 * C; break;
    case GPT2_ACT_FC_GELU: src = a->g; count = BT * 4 * C; break;
    case GPT2_ACT_LNF: src = h->z; count = BT * C; break;
    case GPT2_ACT_LOGITS:
      if (!h->logits) return fail(h, GPT2_E_STATE, "a fused lm_head (head_chunk > 0) keeps no logits");
      src = h->logits;
      count = BT * c.padded_vocab_size;
      break;
    case GPT2_ACT_ROW_LOSS: src = h->row_loss; count = BT; f32 = true; break;
    default: return fail(h, GPT2_E_ARG, "unknown activation id");
  }
  if (n > count) return fail(h, GPT2_E_ARG, "n exceeds the activation's element count");
  count = n;
  gpt2_status st = sync(h);
  if (st != GPT2_OK) return st;
  if (f32 || h->act == DT_F32) {
    HIPTRY(h, hipMemcpy(h_dst, src, count * 4, hipMemcpyDeviceToHost));
  } else {
    std::vector<uint16_t> tmp(count);
    HIPTRY(h, hipMemcpy(tmp.data(), src, count * 2, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < count; ++i) {
      uint32_t u = (uint32_t)tmp[i] << 16;
      std::memcpy(h_dst + i, &u, 4);
    }
  }
  return GPT2_OK;
}

}  // extern "C"
