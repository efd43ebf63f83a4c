// Step engine behind the C ABI (include/gpt2.h): arena layout, tensor table,
// host-side seeded initialization, the forward / backward / optimizer
// launch schedules and the call-order state machine.  Host code only; the
// kernels live in elementwise.hip, gemm.hip and attention.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/gpt2.h"
#include "kernels.h"

#define GPT2_API extern "C" __attribute__((visibility("default")))

namespace {

using gk::GemmArgs;

struct Tensor {
  std::string name;
  int kind, dtype, ndim, decay;
  int64_t shape[4];
  size_t offset, bytes;
};

struct ParamSpec {
  std::string name;
  int64_t rows, cols;  // cols = 0 for 1-D
  int init;            // 0 normal(std), 1 ones, 2 zeros
  double std;
  bool decay, gemm_weight;
  size_t numel() const { return (size_t)rows * (cols ? cols : 1); }
};

std::vector<ParamSpec> param_specs(const gpt2_config& c) {
  const int64_t C = c.n_embd;
  const double res = 0.02 / std::sqrt(2.0 * c.n_layer);
  std::vector<ParamSpec> s;
  s.push_back({"wte", c.padded_vocab, C, 0, 0.02, true, true});
  s.push_back({"wpe", c.block_size, C, 0, 0.02, true, false});
  for (int l = 0; l < c.n_layer; ++l) {
    std::string p = "h" + std::to_string(l) + ".";
    s.push_back({p + "ln1.w", C, 0, 1, 0, false, false});
    s.push_back({p + "ln1.b", C, 0, 2, 0, false, false});
    s.push_back({p + "qkv.w", 3 * C, C, 0, 0.02, true, true});
    s.push_back({p + "qkv.b", 3 * C, 0, 2, 0, false, false});
    s.push_back({p + "proj.w", C, C, 0, res, true, true});
    s.push_back({p + "proj.b", C, 0, 2, 0, false, false});
    s.push_back({p + "ln2.w", C, 0, 1, 0, false, false});
    s.push_back({p + "ln2.b", C, 0, 2, 0, false, false});
    s.push_back({p + "fc.w", 4 * C, C, 0, 0.02, true, true});
    s.push_back({p + "fc.b", 4 * C, 0, 2, 0, false, false});
    s.push_back({p + "mproj.w", C, 4 * C, 0, res, true, true});
    s.push_back({p + "mproj.b", C, 0, 2, 0, false, false});
  }
  s.push_back({"lnf.w", C, 0, 1, 0, false, false});
  s.push_back({"lnf.b", C, 0, 2, 0, false, false});
  return s;
}

// ---------------------------------------------------------------- init RNG
// SplitMix64 (Steele, Lea & Flood 2014): output i of the stream started at
// `seed` mixes the state seed + (i + 1) * golden-gamma.
inline uint64_t splitmix_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Box-Muller (1958) on pairs of uniforms: u1 in (0, 1], u2 in [0, 1).
void fill_normal(float* out, size_t n, uint64_t seed, double stdv, size_t q0, size_t q1) {
  const double two_pi = 2.0 * M_PI;
  for (size_t q = q0; q < q1; ++q) {
    uint64_t a = splitmix_at(seed, 2 * q), b = splitmix_at(seed, 2 * q + 1);
    double u1 = ((double)(a >> 11) + 1.0) * 0x1p-53;
    double u2 = (double)(b >> 11) * 0x1p-53;
    double r = std::sqrt(-2.0 * std::log(u1));
    double z0 = r * std::cos(two_pi * u2), z1 = r * std::sin(two_pi * u2);
    out[2 * q] = (float)(z0 * stdv);
    if (2 * q + 1 < n) out[2 * q + 1] = (float)(z1 * stdv);
  }
}

bool config_ok(const gpt2_config* c, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return false; };
  if (!c) return bad("config is NULL");
  if (c->n_layer < 1 || c->n_head < 1 || c->n_embd < 64) return bad("bad layer/head/embd");
  if (c->n_embd % 64 || c->n_embd > 1024) return bad("n_embd must be a multiple of 64, <= 1024");
  if (c->n_embd % c->n_head) return bad("n_embd % n_head != 0");
  if ((c->n_embd / c->n_head) > 128 || (c->n_embd / c->n_head) % 8)
    return bad("head_dim must be a multiple of 8, <= 128");
  if (c->vocab_size < 2 || c->padded_vocab < c->vocab_size) return bad("bad vocab sizes");
  if (c->padded_vocab > 65536) return bad("padded_vocab > 65536");
  if (c->block_size < 1 || c->max_seq < 1 || c->max_seq > c->block_size) return bad("bad seq sizes");
  if (c->max_batch < 1 || (int64_t)c->max_batch * c->max_seq > 32768)
    return bad("max_batch * max_seq must be in [1, 32768]");
  if (c->compute != GPT2_FP32 && c->compute != GPT2_BF16 && c->compute != GPT2_FP16)
    return bad("bad compute mode");
  // the GEMM operand loads address the logits with 32-bit byte offsets
  const uint64_t ldl = ((uint64_t)c->padded_vocab + 63) / 64 * 64;
  if ((uint64_t)c->max_batch * c->max_seq * ldl * (c->compute == GPT2_FP32 ? 4u : 2u) >= (1ull << 32))
    return bad("logits buffer of 4 GiB or more");
  return true;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Every region is followed by a guard of kGuard bytes of kGuardByte,
// written by gpt2_create and checked by gpt2_check_arena: a kernel that
// writes past the end of its region changes them.
constexpr size_t kGuard = 64;
constexpr unsigned char kGuardByte = 0xA5;

struct Guard {
  size_t offset;
  std::string owner;
};


}  // namespace

// ====================================================================== context
struct gpt2_ctx {
  gpt2_config cfg;
  int dev = 0;
  char* arena = nullptr;
  size_t arena_bytes = 0;
  hipStream_t st = nullptr;
  std::vector<Tensor> tensors;
  std::vector<ParamSpec> specs;
  std::vector<size_t> poff;  // element offset of each parameter in the flat arrays
  size_t nflat = 0;          // flat array length (padded)
  int L, H, C, hd, V, Vp, ldl, maxM;
  bool h16;     // 16-bit activations and GEMM operands (bf16 or fp16)
  int dt;       // activation type (gk::ActType)
  bool ls;      // dynamic loss scaling (fp16)
  int ls_interval = 2000;
  float ls_staging[2] = {0.f, 0.f};
  size_t act_es;  // activation element size

  float *params, *grads, *am, *av;
  uint16_t* shadow;
  std::vector<float*> h, mean, rstd, lse;
  std::vector<void*> ln, qkv, att, fcu, fcg;
  void* logits;
  float *losses, *scal;
  int* flag;
  int32_t* tok;
  float* dres;
  void *dres_act, *dA, *dattn, *dqkv, *du;
  float *ln_part, *col_part, *splitk_ws, *attn_ws;
  size_t splitk_elems;
  void* emb_ws;
  double* norm_part;
  gk::AdamChunk* chunks;
  int nchunks;

  int B = 0, T = 0;
  bool armed_bwd = false, armed_step = false, grads_fresh = true, poisoned = false;
  std::string err;

  std::vector<Guard> guards;
  std::vector<unsigned char> guard_host;  // staging for gpt2_check_arena
  float step_staging = 0.f;               // source of gpt2_set_step_count's copy

  int tclass = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  size_t ev_used = 0;

  const float* P(int j) const { return params + poff[j]; }
  float* G(int j) const { return grads + poff[j]; }
  const void* W(int j) const {  // GEMM operand copy of a weight
    return h16 ? (const void*)(shadow + poff[j]) : (const void*)(params + poff[j]);
  }
  int li(int l, int k) const { return 2 + 12 * l + k; }  // parameter index in layer l
  void* act(void* base, size_t elems_off) const { return (char*)base + elems_off * act_es; }
};

namespace {

// ---------------------------------------------------------------- layout
struct Planner {
  size_t off = 0;
  std::vector<Tensor>* out;
  std::vector<Guard>* guards = nullptr;
  size_t close(size_t end, const std::string& owner) {
    if (guards) guards->push_back({end, owner});
    return align256(end + kGuard);
  }
  size_t add(const std::string& name, int kind, int dtype, std::vector<int64_t> shape, int decay = 0) {
    size_t es = dtype == GPT2_DT_BF16 ? 2 : dtype == GPT2_DT_F64 ? 8 : 4;
    size_t n = 1;
    for (auto s : shape) n *= (size_t)s;
    Tensor t;
    t.name = name;
    t.kind = kind;
    t.dtype = dtype;
    t.ndim = (int)shape.size();
    t.decay = decay;
    for (int i = 0; i < 4; ++i) t.shape[i] = i < t.ndim ? shape[i] : 0;
    t.offset = off;
    t.bytes = n * es;
    off = close(off + t.bytes, name);
    if (out) out->push_back(t);
    return t.offset;
  }
  size_t raw(size_t bytes, const std::string& owner) {
    size_t o = off;
    off = close(off + bytes, owner);
    return o;
  }
};

struct Layout {
  size_t total;
};

// Builds the arena layout.  When ctx is non-null its pointers are set.
size_t plan(const gpt2_config& c, gpt2_ctx* x) {
  std::vector<Tensor> tmp;
  Planner pl;
  pl.out = x ? &x->tensors : &tmp;
  pl.guards = x ? &x->guards : nullptr;
  auto specs = param_specs(c);
  const int L = c.n_layer, C = c.n_embd, H = c.n_head;
  const int64_t maxM = (int64_t)c.max_batch * c.max_seq;
  const bool bf = c.compute != GPT2_FP32;  // 16-bit activations
  const int adt = c.compute == GPT2_BF16 ? GPT2_DT_BF16 : c.compute == GPT2_FP16 ? GPT2_DT_F16 : GPT2_DT_F32;
  const size_t aes = bf ? 2 : 4;
  const int ldl = ((c.padded_vocab + 63) / 64) * 64;

  std::vector<size_t> poff;
  size_t n = 0;
  for (auto& s : specs) {
    poff.push_back(n);
    n += s.numel();
  }
  size_t nflat = ((n + 63) / 64) * 64;
  size_t o_par = pl.raw(nflat * 4, "parameters"), o_grad = pl.raw(nflat * 4, "gradients");
  size_t o_m = pl.raw(nflat * 4, "adam_m"), o_v = pl.raw(nflat * 4, "adam_v");
  size_t o_sh = bf ? pl.raw(nflat * 2, "16-bit weight copies") : 0;
  // tensor-table views of the flat arrays
  for (size_t j = 0; j < specs.size(); ++j) {
    auto& s = specs[j];
    std::vector<int64_t> shp = s.cols ? std::vector<int64_t>{s.rows, s.cols} : std::vector<int64_t>{s.rows};
    Tensor t;
    t.ndim = (int)shp.size();
    for (int i = 0; i < 4; ++i) t.shape[i] = i < t.ndim ? shp[i] : 0;
    t.decay = s.decay;
    const char* pre[5] = {"", "grad.", "adam_m.", "adam_v.", "bf16."};
    size_t base[5] = {o_par, o_grad, o_m, o_v, o_sh};
    for (int k = 0; k < 5; ++k) {
      if (k == 4 && (!bf || !s.gemm_weight)) continue;
      t.name = std::string(pre[k]) + s.name;
      t.kind = k;
      t.dtype = k == 4 ? adt : GPT2_DT_F32;
      size_t es = k == 4 ? 2 : 4;
      t.offset = base[k] + poff[j] * es;
      t.bytes = s.numel() * es;
      pl.out->push_back(t);
    }
  }
  std::vector<size_t> o_h, o_ln, o_mean, o_rstd, o_qkv, o_att, o_lse, o_fcu, o_fcg;
  for (int k = 0; k <= 2 * L; ++k) {
    o_h.push_back(pl.add("h." + std::to_string(k), GPT2_K_ACT, GPT2_DT_F32, {maxM, C}));
    o_ln.push_back(pl.add("ln." + std::to_string(k), GPT2_K_ACT, adt, {maxM, C}));
    o_mean.push_back(pl.add("ln_mean." + std::to_string(k), GPT2_K_ACT, GPT2_DT_F32, {maxM}));
    o_rstd.push_back(pl.add("ln_rstd." + std::to_string(k), GPT2_K_ACT, GPT2_DT_F32, {maxM}));
  }
  for (int l = 0; l < L; ++l) {
    o_qkv.push_back(pl.add("qkv." + std::to_string(l), GPT2_K_ACT, adt, {maxM, 3 * C}));
    o_att.push_back(pl.add("attn." + std::to_string(l), GPT2_K_ACT, adt, {maxM, C}));
    o_lse.push_back(pl.add("lse." + std::to_string(l), GPT2_K_ACT, GPT2_DT_F32, {maxM * H}));
    o_fcu.push_back(pl.add("fc_u." + std::to_string(l), GPT2_K_ACT, adt, {maxM, 4 * C}));
    o_fcg.push_back(pl.add("fc_g." + std::to_string(l), GPT2_K_ACT, adt, {maxM, 4 * C}));
  }
  size_t o_logits = pl.add("logits", GPT2_K_LOGITS, adt, {maxM, ldl});
  size_t o_losses = pl.add("losses", GPT2_K_ACT, GPT2_DT_F32, {maxM});
  size_t o_scal = pl.add("scalars", GPT2_K_SCALAR, GPT2_DT_F32, {64});
  size_t o_flag = pl.add("flags", GPT2_K_SCALAR, GPT2_DT_I32, {4});
  size_t o_tok = pl.add("tokens", GPT2_K_ACT, GPT2_DT_I32, {maxM});
  size_t o_dres = pl.add("d_resid", GPT2_K_ACT, GPT2_DT_F32, {maxM, C});
  size_t o_dresa = pl.add("d_resid_act", GPT2_K_ACT, adt, {maxM, C});
  size_t o_dA = pl.add("d_ln_out", GPT2_K_ACT, adt, {maxM, C});
  size_t o_dattn = pl.add("d_attn", GPT2_K_ACT, adt, {maxM, C});
  size_t o_dqkv = pl.add("d_qkv", GPT2_K_ACT, adt, {maxM, 3 * C});
  size_t o_du = pl.add("d_fc_u", GPT2_K_ACT, adt, {maxM, 4 * C});
  size_t o_lnp = pl.raw((size_t)gk::ln_bwd_part_floats((int)maxM, C) * 4, "LayerNorm partials");
  size_t ncolp = 0;  // bias-gradient column sums run over N = C, 3C, 4C
  for (int n : {C, 3 * C, 4 * C}) ncolp = std::max(ncolp, gk::colsum_part_floats((int)maxM, n));
  size_t o_colp = pl.raw(ncolp * 4, "column-sum partials");
  size_t sk = 0;
  {
    const int64_t shapes[5][2] = {{3 * C, C}, {C, C}, {4 * C, C}, {C, 4 * C}, {c.padded_vocab, C}};
    for (auto& s : shapes) sk = std::max(sk, gk::gemm_splitk_ws_elems((int)s[0], (int)s[1], (int)maxM));
  }
  size_t o_sk = pl.raw(sk * 4 + 256, "split-K partials");
  size_t o_emb = pl.raw(gk::embed_bwd_workspace((int)maxM, C), "embedding-backward workspace");
  size_t o_attn = pl.raw(gk::attn_bwd_workspace(1, (int)maxM, H) * 4, "attention workspace");
  size_t o_norm = pl.raw(gk::sumsq_blocks() * 8, "norm partials");
  // AdamW chunk table
  const size_t CH = 16384;
  size_t nchunks = 0;
  for (auto& s : specs) nchunks += (s.numel() + CH - 1) / CH;
  size_t o_chunks = pl.raw(nchunks * sizeof(gk::AdamChunk), "AdamW chunk table");
  size_t total = pl.off;

  if (x) {
    char* a = x->arena;
    x->specs = specs;
    x->poff = poff;
    x->nflat = nflat;
    x->L = L; x->H = H; x->C = C; x->hd = C / H;
    x->V = c.vocab_size; x->Vp = c.padded_vocab; x->ldl = ldl; x->maxM = (int)maxM;
    x->h16 = bf; x->act_es = aes;
    x->dt = c.compute == GPT2_BF16 ? gk::ACT_BF16 : c.compute == GPT2_FP16 ? gk::ACT_F16 : gk::ACT_F32;
    x->ls = c.compute == GPT2_FP16;
    x->params = (float*)(a + o_par); x->grads = (float*)(a + o_grad);
    x->am = (float*)(a + o_m); x->av = (float*)(a + o_v);
    x->shadow = bf ? (uint16_t*)(a + o_sh) : nullptr;
    for (int k = 0; k <= 2 * L; ++k) {
      x->h.push_back((float*)(a + o_h[k]));
      x->ln.push_back(a + o_ln[k]);
      x->mean.push_back((float*)(a + o_mean[k]));
      x->rstd.push_back((float*)(a + o_rstd[k]));
    }
    for (int l = 0; l < L; ++l) {
      x->qkv.push_back(a + o_qkv[l]);
      x->att.push_back(a + o_att[l]);
      x->lse.push_back((float*)(a + o_lse[l]));
      x->fcu.push_back(a + o_fcu[l]);
      x->fcg.push_back(a + o_fcg[l]);
    }
    x->logits = a + o_logits;
    x->losses = (float*)(a + o_losses);
    x->scal = (float*)(a + o_scal);
    x->flag = (int*)(a + o_flag);
    x->tok = (int32_t*)(a + o_tok);
    x->dres = (float*)(a + o_dres);
    x->dres_act = a + o_dresa;
    x->dA = a + o_dA;
    x->dattn = a + o_dattn;
    x->dqkv = a + o_dqkv;
    x->du = a + o_du;
    x->ln_part = (float*)(a + o_lnp);
    x->col_part = (float*)(a + o_colp);
    x->splitk_ws = (float*)(a + o_sk);
    x->splitk_elems = sk;
    x->emb_ws = a + o_emb;
    x->attn_ws = (float*)(a + o_attn);
    x->norm_part = (double*)(a + o_norm);
    x->chunks = (gk::AdamChunk*)(a + o_chunks);
    x->nchunks = (int)nchunks;
  }
  return total;
}

// ---------------------------------------------------------------- errors / timing
#define HIPCHK(ctx, expr)                                                          \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess) {                                                        \
      (ctx)->poisoned = true;                                                      \
      (ctx)->err = std::string(#expr) + ": " + hipGetErrorString(e_);              \
      return GPT2_E_HIP;                                                           \
    }                                                                              \
  } while (0)

gpt2_status fail(gpt2_ctx* c, gpt2_status s, const std::string& m) {
  if (c) c->err = m;
  return s;
}

// Brackets the launches of one kernel class with events when enabled.
struct Timed {
  gpt2_ctx* c;
  bool on;
  Timed(gpt2_ctx* c_, int cls) : c(c_), on(c_->tclass == cls) {
    if (!on) return;
    if (c->ev_used == c->ev.size()) {
      hipEvent_t a, b;
      (void)hipEventCreate(&a);
      (void)hipEventCreate(&b);
      c->ev.push_back({a, b});
    }
    (void)hipEventRecord(c->ev[c->ev_used].first, c->st);
  }
  ~Timed() {
    if (!on) return;
    (void)hipEventRecord(c->ev[c->ev_used].second, c->st);
    ++c->ev_used;
  }
};

GemmArgs gemm_args(gpt2_ctx* c, int M, int N, int K, const void* A, int lda, bool at,
                   const void* B, int ldb, bool bt, int kind, void* out, int ldo) {
  GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.A = A; a.lda = lda; a.a_t = at;
  a.B = B; a.ldb = ldb; a.b_t = bt;
  a.kind = kind; a.out = out; a.ldo = ldo;
  a.out2 = nullptr; a.aux = nullptr; a.bias = nullptr;
  a.alpha = 1.f; a.beta = 0.f;
  a.dt = c->dt;
  a.splitk_ws = c->splitk_ws;
  a.splitk_ws_elems = c->splitk_elems;
  return a;
}

hipError_t run_gemm(gpt2_ctx* c, const GemmArgs& a, int tcls = GPT2_T_GEMM) {
  Timed t(c, tcls);
  Timed t2(c, tcls == GPT2_T_LMHEAD_FWD ? GPT2_T_GEMM : -1);
  return gk::gemm(a, c->st);
}

// ---------------------------------------------------------------- schedules
#define KCHK(expr)                      \
  do {                                  \
    hipError_t e_ = (expr);             \
    if (e_ != hipSuccess) return e_;    \
  } while (0)

// Attention of one decode step: the newest position t of each of B
// sequences against the layer's key/value cache (positions 0..t).
struct DecodeAttn {
  void* cache;  // this layer's [max_batch][max_seq][2][C]
  int t;
};

// One transformer block forward: h[2l] -> h[2l+1] -> h[2l+2].  With `dec`
// the rows are one new position per sequence (M = B) whose keys and values
// are appended to the cache and whose queries attend over it.
hipError_t fwd_layer(gpt2_ctx* c, int l, int M, int B, int T, const DecodeAttn* dec = nullptr) {
  const int C = c->C;
  const float eps = c->cfg.ln_eps;
  {
    Timed t(c, GPT2_T_LN_FWD);
    KCHK(gk::ln_fwd(c->h[2 * l], c->P(c->li(l, 0)), c->P(c->li(l, 1)), c->ln[2 * l], c->dt,
                    c->mean[2 * l], c->rstd[2 * l], M, C, eps, c->st));
  }
  GemmArgs g = gemm_args(c, M, 3 * C, C, c->ln[2 * l], C, false, c->W(c->li(l, 2)), C, false,
                         gk::EPI_STORE, c->qkv[l], 3 * C);
  g.bias = c->P(c->li(l, 3));
  KCHK(run_gemm(c, g));
  if (dec) {
    KCHK(gk::kv_store(c->qkv[l], dec->cache, B, 1, dec->t, c->cfg.max_seq, C, c->dt, c->st));
    KCHK(gk::attn_decode(c->qkv[l], dec->cache, c->att[l], B, c->H, c->hd, c->cfg.max_seq, dec->t + 1, c->dt,
                         c->st));
  } else {
    Timed t(c, GPT2_T_ATTN_FWD);
    KCHK(gk::attn_fwd(c->qkv[l], c->att[l], c->lse[l], B, T, c->H, c->hd, c->dt, c->st));
  }
  g = gemm_args(c, M, C, C, c->att[l], C, false, c->W(c->li(l, 4)), C, false, gk::EPI_RESID,
                c->h[2 * l + 1], C);
  g.aux = c->h[2 * l];
  g.bias = c->P(c->li(l, 5));
  KCHK(run_gemm(c, g));
  {
    Timed t(c, GPT2_T_LN_FWD);
    KCHK(gk::ln_fwd(c->h[2 * l + 1], c->P(c->li(l, 6)), c->P(c->li(l, 7)), c->ln[2 * l + 1], c->dt,
                    c->mean[2 * l + 1], c->rstd[2 * l + 1], M, C, eps, c->st));
  }
  g = gemm_args(c, M, 4 * C, C, c->ln[2 * l + 1], C, false, c->W(c->li(l, 8)), C, false,
                gk::EPI_GELU, c->fcu[l], 4 * C);
  g.out2 = c->fcg[l];
  g.bias = c->P(c->li(l, 9));
  KCHK(run_gemm(c, g));
  g = gemm_args(c, M, C, 4 * C, c->fcg[l], 4 * C, false, c->W(c->li(l, 10)), 4 * C, false,
                gk::EPI_RESID, c->h[2 * l + 2], C);
  g.aux = c->h[2 * l + 1];
  g.bias = c->P(c->li(l, 11));
  KCHK(run_gemm(c, g));
  return hipSuccess;
}

hipError_t ln_backward(gpt2_ctx* c, int k, int wj, const void* dy, bool accum, float beta, int M) {
  Timed t(c, GPT2_T_LN_BWD);
  KCHK(gk::ln_bwd(c->h[k], c->mean[k], c->rstd[k], c->P(wj), dy, c->dt, c->dres, c->dres_act, accum,
                  c->ln_part, M, c->C, c->st));
  return gk::ln_param_grad_reduce(c->ln_part, gk::ln_bwd_blocks(M), c->G(wj), c->G(wj + 1), c->C,
                                  beta, c->st);
}

// Weight gradient dW[out, in] (+)= dY^T X of a linear layer and, with
// bias index bj >= 0, its bias gradient db (+)= column sums of dY, which the
// GEMM forms from the dY tiles it stages.
hipError_t wgrad(gpt2_ctx* c, int M, int n_out, int n_in, const void* dY, const void* X, int wj, int bj,
                 float beta) {
  GemmArgs g = gemm_args(c, n_out, n_in, M, dY, n_out, true, X, n_in, true, gk::EPI_WGRAD, c->G(wj), n_in);
  g.beta = beta;
  if (bj >= 0) {
    g.dbias = c->G(bj);
    g.colsum_ws = c->col_part;
  }
  return run_gemm(c, g);
}

// dX[M, in] = dY[M, out] W[out, in]: the weight (or its 16-bit copy) is read
// in its own [out][in] layout, i.e. as B transposed in memory.
GemmArgs dx_args(gpt2_ctx* c, int M, int n_in, int n_out, const void* dY, int ldy, int wj, int kind,
                 void* out, int ldo) {
  return gemm_args(c, M, n_in, n_out, dY, ldy, false, c->W(wj), n_in, true, kind, out, ldo);
}

// Backward of block l given dres (fp32) / dres_act = dL/d h[2l+2]; leaves
// dL/d h[2l] in dres / dres_act.
hipError_t bwd_layer(gpt2_ctx* c, int l, int M, int B, int T, float beta) {
  const int C = c->C;
  // mlp projection: dg = dr W_mp, du = dg * gelu'(u); dW_mp = dr^T g; db_mp = sum dr
  GemmArgs g = dx_args(c, M, 4 * C, C, c->dres_act, C, c->li(l, 10), gk::EPI_DGELU, c->du, 4 * C);
  g.aux = c->fcu[l];
  KCHK(run_gemm(c, g));
  KCHK(wgrad(c, M, C, 4 * C, c->dres_act, c->fcg[l], c->li(l, 10), c->li(l, 11), beta));
  // fc: da2 = du W_fc; dW_fc = du^T a2; db_fc = sum du
  g = dx_args(c, M, C, 4 * C, c->du, 4 * C, c->li(l, 8), gk::EPI_STORE, c->dA, C);
  KCHK(run_gemm(c, g));
  KCHK(wgrad(c, M, 4 * C, C, c->du, c->ln[2 * l + 1], c->li(l, 8), c->li(l, 9), beta));
  KCHK(ln_backward(c, 2 * l + 1, c->li(l, 6), c->dA, true, beta, M));
  // attention projection: do = dr W_proj; dW_proj = dr^T o; db_proj
  g = dx_args(c, M, C, C, c->dres_act, C, c->li(l, 4), gk::EPI_STORE, c->dattn, C);
  KCHK(run_gemm(c, g));
  KCHK(wgrad(c, M, C, C, c->dres_act, c->att[l], c->li(l, 4), c->li(l, 5), beta));
  {
    Timed t(c, GPT2_T_ATTN_BWD);
    KCHK(gk::attn_bwd(c->qkv[l], c->att[l], c->dattn, c->lse[l], c->dqkv, c->attn_ws, B, T, c->H,
                      c->hd, c->dt, c->st));
  }
  // qkv: da1 = dqkv W_qkv; dW_qkv = dqkv^T a1; db_qkv
  g = dx_args(c, M, C, 3 * C, c->dqkv, 3 * C, c->li(l, 2), gk::EPI_STORE, c->dA, C);
  KCHK(run_gemm(c, g));
  KCHK(wgrad(c, M, 3 * C, C, c->dqkv, c->ln[2 * l], c->li(l, 2), c->li(l, 3), beta));
  KCHK(ln_backward(c, 2 * l, c->li(l, 0), c->dA, true, beta, M));
  return hipSuccess;
}

// The forward schedule over the ids already in c->tok ([B, T] packed):
// embeddings, the L blocks, the final LayerNorm and the classifier; with
// targets also the per-position losses (and, when want_grad, the logits
// gradient in place) and the mean loss in scal[8].
hipError_t run_forward(gpt2_ctx* c, int B, int T, const int32_t* d_targets, bool want_grad) {
  const int M = B * T, C = c->C;
  {
    Timed t(c, GPT2_T_EMBED);
    KCHK(gk::embed_fwd(c->tok, c->P(0), c->P(1), c->h[0], M, T, C, c->V, c->flag, c->st));
  }
  for (int l = 0; l < c->L; ++l) KCHK(fwd_layer(c, l, M, B, T));
  const int lf = 2 + 12 * c->L;
  {
    Timed t(c, GPT2_T_LN_FWD);
    KCHK(gk::ln_fwd(c->h[2 * c->L], c->P(lf), c->P(lf + 1), c->ln[2 * c->L], c->dt, c->mean[2 * c->L],
                    c->rstd[2 * c->L], M, C, c->cfg.ln_eps, c->st));
  }
  GemmArgs g = gemm_args(c, M, c->Vp, C, c->ln[2 * c->L], C, false, c->W(0), C, false, gk::EPI_LOGITS,
                         c->logits, c->ldl);
  KCHK(run_gemm(c, g, GPT2_T_LMHEAD_FWD));
  if (d_targets) {
    {
      Timed t(c, GPT2_T_XENT);
      KCHK(gk::xent(c->logits, c->dt, c->ldl, c->Vp, c->V, d_targets, c->losses, 1.0f / (float)M, want_grad,
                    M, c->flag, c->ls ? c->scal + 10 : nullptr, c->st));
    }
    KCHK(gk::loss_reduce(c->losses, M, c->scal + 8, c->flag, c->st));
  }
  return hipSuccess;
}

gpt2_status check_ctx(gpt2_ctx* c) {
  if (!c) return GPT2_E_ARG;
  if (c->poisoned) return fail(c, GPT2_E_STATE, "context poisoned by an earlier HIP error: " + c->err);
  hipError_t e = hipSetDevice(c->dev);
  if (e != hipSuccess) {
    c->poisoned = true;
    c->err = std::string("hipSetDevice: ") + hipGetErrorString(e);
    return GPT2_E_HIP;
  }
  return GPT2_OK;
}

gpt2_status read_flags(gpt2_ctx* c, int* flags) {
  HIPCHK(c, hipMemcpyAsync(flags, c->flag, sizeof(int), hipMemcpyDeviceToHost, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  return GPT2_OK;
}

}  // namespace

// ====================================================================== ABI
GPT2_API void gpt2_default_config(gpt2_config* cfg, int32_t max_batch, int32_t max_seq) {
  if (!cfg) return;
  cfg->n_layer = 12;
  cfg->n_head = 12;
  cfg->n_embd = 768;
  cfg->block_size = 1024;
  cfg->vocab_size = 50257;
  cfg->padded_vocab = 50304;
  cfg->max_batch = max_batch;
  cfg->max_seq = max_seq;
  cfg->compute = GPT2_BF16;
  cfg->ln_eps = 1e-5f;
  cfg->beta1 = 0.9f;
  cfg->beta2 = 0.95f;
  cfg->adam_eps = 1e-8f;
  cfg->weight_decay = 0.1f;
}

GPT2_API size_t gpt2_arena_bytes(const gpt2_config* cfg) {
  if (!config_ok(cfg, nullptr)) return 0;
  return plan(*cfg, nullptr);
}

GPT2_API int64_t gpt2_num_params(const gpt2_config* cfg) {
  if (!config_ok(cfg, nullptr)) return -1;
  int64_t n = 0;
  for (auto& s : param_specs(*cfg)) n += (int64_t)s.numel();
  return n;
}

GPT2_API gpt2_status gpt2_init_host(const gpt2_config* cfg, uint64_t seed, float* out) {
  if (!out || !config_ok(cfg, nullptr)) return GPT2_E_ARG;
  auto specs = param_specs(*cfg);
  unsigned nt = std::thread::hardware_concurrency();
  nt = nt < 1 ? 1 : (nt > 32 ? 32 : nt);
  size_t off = 0;
  for (size_t j = 0; j < specs.size(); ++j) {
    const auto& s = specs[j];
    size_t n = s.numel();
    float* dst = out + off;
    off += n;
    if (s.init == 1) {
      for (size_t i = 0; i < n; ++i) dst[i] = 1.f;
      continue;
    }
    if (s.init == 2) {
      std::memset(dst, 0, n * 4);
      continue;
    }
    uint64_t ts = seed ^ ((uint64_t)j << 32);
    size_t npair = (n + 1) / 2;
    if (npair < 65536 || nt == 1) {
      fill_normal(dst, n, ts, s.std, 0, npair);
    } else {
      std::vector<std::thread> th;
      size_t per = (npair + nt - 1) / nt;
      for (unsigned t = 0; t < nt; ++t) {
        size_t q0 = t * per, q1 = std::min(npair, q0 + per);
        if (q0 >= q1) break;
        th.emplace_back(fill_normal, dst, n, ts, s.std, q0, q1);
      }
      for (auto& t : th) t.join();
    }
  }
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_create(const gpt2_config* cfg, uint64_t seed, void* d_arena,
                                 size_t arena_bytes, void* hip_stream, gpt2_ctx** out) {
  if (!out) return GPT2_E_ARG;
  *out = nullptr;
  std::string why;
  if (!config_ok(cfg, &why)) return GPT2_E_ARG;
  if (!d_arena || ((uintptr_t)d_arena & 255)) return GPT2_E_ARENA;
  size_t need = plan(*cfg, nullptr);
  if (arena_bytes < need) return GPT2_E_ARENA;
  gpt2_ctx* c = new gpt2_ctx();
  c->cfg = *cfg;
  c->arena = (char*)d_arena;
  c->arena_bytes = arena_bytes;
  c->st = (hipStream_t)hip_stream;
  if (hipGetDevice(&c->dev) != hipSuccess) {
    delete c;
    return GPT2_E_HIP;
  }
  plan(*cfg, c);
  // parameters on the host, then one copy
  int64_t np = gpt2_num_params(cfg);
  std::vector<float> host((size_t)c->nflat, 0.f);
  gpt2_init_host(cfg, seed, host.data());
  auto bail = [&](hipError_t e, const char* what) {
    c->err = std::string(what) + ": " + hipGetErrorString(e);
    gpt2_destroy(c);
    return GPT2_E_HIP;
  };
  hipError_t e;
  if ((e = hipMemcpyAsync(c->params, host.data(), c->nflat * 4, hipMemcpyHostToDevice, c->st)))
    return bail(e, "copy params");
  if ((e = hipMemsetAsync(c->grads, 0, c->nflat * 4, c->st))) return bail(e, "zero grads");
  if ((e = hipMemsetAsync(c->am, 0, c->nflat * 4, c->st))) return bail(e, "zero m");
  if ((e = hipMemsetAsync(c->av, 0, c->nflat * 4, c->st))) return bail(e, "zero v");
  if ((e = hipMemsetAsync(c->scal, 0, 64 * 4, c->st))) return bail(e, "zero scalars");
  if ((e = hipMemsetAsync(c->flag, 0, 16, c->st))) return bail(e, "zero flags");
  // logits columns [Vp, row stride) are never written by the classifier GEMM
  if ((e = hipMemsetAsync(c->logits, 0, (size_t)c->maxM * c->ldl * c->act_es, c->st)))
    return bail(e, "zero logits");
  for (const Guard& g : c->guards)
    if ((e = hipMemsetAsync(c->arena + g.offset, kGuardByte, kGuard, c->st))) return bail(e, "guards");
  if (c->h16 && (e = gk::to_h16(c->params, c->shadow, c->nflat, c->dt, c->st))) return bail(e, "16-bit copy");
  if (c->ls) {  // dynamic loss scale and its step counter
    c->ls_staging[0] = 65536.f;
    c->ls_staging[1] = 0.f;
    if ((e = hipMemcpyAsync(c->scal + 10, c->ls_staging, 8, hipMemcpyHostToDevice, c->st)))
      return bail(e, "loss scale");
  }
  // AdamW chunk table
  std::vector<gk::AdamChunk> ch;
  const size_t CH = 16384;
  for (size_t j = 0; j < c->specs.size(); ++j) {
    const auto& s = c->specs[j];
    size_t n = s.numel();
    for (size_t i = 0; i < n; i += CH) {
      gk::AdamChunk a;
      a.start = c->poff[j] + i;
      a.count = (uint32_t)std::min(CH, n - i);
      a.flags = (s.decay ? 1u : 0u) | ((c->h16 && s.gemm_weight) ? 2u : 0u);
      ch.push_back(a);
    }
  }
  if ((e = hipMemcpyAsync(c->chunks, ch.data(), ch.size() * sizeof(gk::AdamChunk),
                          hipMemcpyHostToDevice, c->st)))
    return bail(e, "copy chunk table");
  if ((e = hipStreamSynchronize(c->st))) return bail(e, "sync");
  (void)np;
  *out = c;
  return GPT2_OK;
}

GPT2_API void gpt2_destroy(gpt2_ctx* c) {
  if (!c) return;
  for (auto& p : c->ev) {
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  delete c;
}

GPT2_API const char* gpt2_last_error(const gpt2_ctx* c) {
  if (!c) return "no context";
  return c->err.c_str();
}

namespace {

// Loss readback shared by forward and evaluation: the flags decide the
// status (ids or targets outside the vocabulary, a non-finite loss).
gpt2_status finish_loss(gpt2_ctx* c, const int32_t* d_targets, float* h_loss) {
  int flags = 0;
  if (d_targets) HIPCHK(c, hipMemcpyAsync(h_loss, c->scal + 8, 4, hipMemcpyDeviceToHost, c->st));
  gpt2_status s = read_flags(c, &flags);
  if (s) return s;
  if (flags & 3) {
    c->armed_bwd = false;
    return fail(c, GPT2_E_TOKEN, "token id or target outside [0, vocab_size)");
  }
  if (flags & 4) return fail(c, GPT2_E_NONFINITE, "non-finite loss");
  return GPT2_OK;
}

gpt2_status start_forward(gpt2_ctx* c, const int32_t* d_tokens, int32_t B, int32_t T) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!d_tokens) return fail(c, GPT2_E_ARG, "tokens is NULL");
  if (B < 1 || T < 1 || T > c->cfg.max_seq || (int64_t)B * T > c->maxM)
    return fail(c, GPT2_E_SHAPE, "B*T exceeds the arena or T > max_seq");
  c->armed_bwd = false;
  c->B = B;
  c->T = T;
  HIPCHK(c, gk::fill_f32((float*)c->flag, 4, 0.f, c->st));  // a kernel, not a memset node, should a caller capture this
  HIPCHK(c, hipMemcpyAsync(c->tok, d_tokens, (size_t)B * T * 4, hipMemcpyDeviceToDevice, c->st));
  return GPT2_OK;
}

}  // namespace

GPT2_API gpt2_status gpt2_forward(gpt2_ctx* c, const int32_t* d_tokens, const int32_t* d_targets,
                                  int32_t B, int32_t T, float* h_loss) {
  gpt2_status s = start_forward(c, d_tokens, B, T);
  if (s) return s;
  HIPCHK(c, run_forward(c, B, T, d_targets, true));
  if (d_targets) c->armed_bwd = true;
  if (h_loss) return finish_loss(c, d_targets, h_loss);
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_eval_loss(gpt2_ctx* c, const int32_t* d_tokens, const int32_t* d_targets,
                                    int32_t B, int32_t T, float* h_loss) {
  if (c && !d_targets) return fail(c, GPT2_E_ARG, "targets is NULL");
  gpt2_status s = start_forward(c, d_tokens, B, T);
  if (s) return s;
  HIPCHK(c, run_forward(c, B, T, d_targets, false));
  if (h_loss) return finish_loss(c, d_targets, h_loss);
  return GPT2_OK;
}

GPT2_API size_t gpt2_kv_cache_bytes(const gpt2_config* cfg) {
  if (!config_ok(cfg, nullptr)) return 0;
  const size_t es = cfg->compute == GPT2_FP32 ? 4 : 2;
  return (size_t)cfg->n_layer * cfg->max_batch * cfg->max_seq * 2 * cfg->n_embd * es;
}

GPT2_API gpt2_status gpt2_generate(gpt2_ctx* c, void* d_kv_cache, size_t kv_bytes, int32_t* d_tokens,
                                   int32_t B, int32_t T0, int32_t T_total, const float* d_uniform,
                                   float* d_logprob) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!d_kv_cache || !d_tokens || !d_uniform) return fail(c, GPT2_E_ARG, "NULL buffer");
  if (kv_bytes < gpt2_kv_cache_bytes(&c->cfg)) return fail(c, GPT2_E_ARENA, "key/value cache too small");
  if (B < 1 || B > c->cfg.max_batch || T0 < 1 || T_total <= T0 || T_total > c->cfg.max_seq)
    return fail(c, GPT2_E_SHAPE, "need 1 <= B <= max_batch and 1 <= T0 < T_total <= max_seq");
  const int C = c->C, L = c->L, n_new = T_total - T0;
  const size_t layer_bytes = (size_t)c->cfg.max_batch * c->cfg.max_seq * 2 * C * c->act_es;
  auto cache = [&](int l) { return (void*)((char*)d_kv_cache + (size_t)l * layer_bytes); };
  c->armed_bwd = false;
  HIPCHK(c, gk::fill_f32((float*)c->flag, 4, 0.f, c->st));  // a kernel, not a memset node, should a caller capture this
  // prefill: the prefix through the ordinary forward, its keys and values
  // into the cache, then the first new token from the last prefix position
  HIPCHK(c, hipMemcpy2DAsync(c->tok, (size_t)T0 * 4, d_tokens, (size_t)T_total * 4, (size_t)T0 * 4, B,
                             hipMemcpyDeviceToDevice, c->st));
  HIPCHK(c, run_forward(c, B, T0, nullptr, false));
  for (int l = 0; l < L; ++l) HIPCHK(c, gk::kv_store(c->qkv[l], cache(l), B, T0, 0, c->cfg.max_seq, C, c->dt, c->st));
  HIPCHK(c, gk::sample(c->logits, c->dt, c->ldl, T0, T0 - 1, c->V, B, d_uniform, n_new, d_tokens + T0, T_total,
                       d_logprob, n_new, c->st));
  // decode: one position per sequence per step, attention over the cache
  const int lf = 2 + 12 * L;
  for (int t = T0; t < T_total - 1; ++t) {
    HIPCHK(c, hipMemcpy2DAsync(c->tok, 4, d_tokens + t, (size_t)T_total * 4, 4, B, hipMemcpyDeviceToDevice,
                               c->st));
    HIPCHK(c, gk::embed_fwd(c->tok, c->P(0), c->P(1), c->h[0], B, 1, C, c->V, c->flag, c->st, t));
    for (int l = 0; l < L; ++l) {
      DecodeAttn d{cache(l), t};
      HIPCHK(c, fwd_layer(c, l, B, B, 1, &d));
    }
    HIPCHK(c, gk::ln_fwd(c->h[2 * L], c->P(lf), c->P(lf + 1), c->ln[2 * L], c->dt, c->mean[2 * L],
                         c->rstd[2 * L], B, C, c->cfg.ln_eps, c->st));
    GemmArgs g = gemm_args(c, B, c->Vp, C, c->ln[2 * L], C, false, c->W(0), C, false, gk::EPI_LOGITS, c->logits,
                           c->ldl);
    HIPCHK(c, run_gemm(c, g));
    const int k = t + 1 - T0;
    HIPCHK(c, gk::sample(c->logits, c->dt, c->ldl, 1, 0, c->V, B, d_uniform + k, n_new, d_tokens + t + 1,
                         T_total, d_logprob ? d_logprob + k : nullptr, n_new, c->st));
  }
  int flags = 0;
  s = read_flags(c, &flags);
  if (s) return s;
  if (flags & 1) return fail(c, GPT2_E_TOKEN, "prefix id outside [0, vocab_size)");
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_backward(gpt2_ctx* c, float grad_scale) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!c->armed_bwd) return fail(c, GPT2_E_STATE, "backward needs a forward with targets first");
  const int B = c->B, T = c->T, M = B * T, C = c->C, L = c->L;
  const float beta = c->grads_fresh ? 0.f : 1.f;
  // classifier (tied): dhf = s dz wte ; dwte = s dz^T hf + beta dwte
  GemmArgs g = dx_args(c, M, C, c->Vp, c->logits, c->ldl, 0, gk::EPI_STORE, c->dA, C);
  g.alpha = grad_scale;
  HIPCHK(c, run_gemm(c, g));
  g = gemm_args(c, c->Vp, C, M, c->logits, c->ldl, true, c->ln[2 * L], C, true, gk::EPI_WGRAD,
                c->G(0), C);
  g.alpha = grad_scale;
  g.beta = beta;
  HIPCHK(c, run_gemm(c, g));
  const int lf = 2 + 12 * L;
  HIPCHK(c, ln_backward(c, 2 * L, lf, c->dA, false, beta, M));
  for (int l = L - 1; l >= 0; --l) HIPCHK(c, bwd_layer(c, l, M, B, T, beta));
  {
    Timed t(c, GPT2_T_EMBED);
    HIPCHK(c, gk::embed_bwd(c->tok, c->dres, c->G(0), c->G(1), B, T, C, c->V, c->cfg.block_size, beta,
                            c->emb_ws, c->st));
  }
  c->armed_bwd = false;
  c->armed_step = true;
  c->grads_fresh = false;
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_zero_grad(gpt2_ctx* c) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  c->grads_fresh = true;
  c->armed_step = false;
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_step(gpt2_ctx* c, float lr, float clip, float* h_grad_norm) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!c->armed_step) return fail(c, GPT2_E_STATE, "step needs a backward first");
  if (!(clip > 0.f) || !(lr >= 0.f)) return fail(c, GPT2_E_ARG, "lr must be >= 0 and clip > 0");
  {
    Timed t(c, GPT2_T_NORM);
    HIPCHK(c, gk::sumsq(c->grads, c->nflat, c->norm_part, c->st));
    HIPCHK(c, gk::norm_finalize(c->norm_part, gk::sumsq_blocks(), clip, c->cfg.beta1, c->cfg.beta2,
                                c->scal, c->flag, c->ls, c->ls_interval, c->st));
  }
  {
    Timed t(c, GPT2_T_ADAMW);
    HIPCHK(c, gk::adamw(c->params, c->grads, c->am, c->av, c->shadow, c->dt, c->chunks, c->nchunks, c->scal,
                        lr, c->cfg.beta1, c->cfg.beta2, c->cfg.adam_eps, c->cfg.weight_decay, c->st));
  }
  c->armed_step = false;
  c->grads_fresh = true;
  if (h_grad_norm) {
    HIPCHK(c, hipMemcpyAsync(h_grad_norm, c->scal, 4, hipMemcpyDeviceToHost, c->st));
    int flags = 0;
    s = read_flags(c, &flags);
    if (s) return s;
    if (flags & 8) return fail(c, GPT2_E_NONFINITE, "non-finite gradient norm; update skipped");
    if (flags & 16) *h_grad_norm = INFINITY;  // fp16 overflow: skipped, loss scale halved
  }
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_get_loss_scale(gpt2_ctx* c, float* scale) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!scale) return fail(c, GPT2_E_ARG, "NULL output");
  if (!c->ls) {
    *scale = 1.f;
    return GPT2_OK;
  }
  HIPCHK(c, hipMemcpyAsync(scale, c->scal + 10, 4, hipMemcpyDeviceToHost, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_set_loss_scale(gpt2_ctx* c, float scale, int32_t growth_interval) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!c->ls) return fail(c, GPT2_E_ARG, "loss scaling is the fp16 compute mode's");
  if (!(scale > 0.f) || !std::isfinite(scale) || growth_interval < 1)
    return fail(c, GPT2_E_ARG, "scale must be finite and > 0, growth_interval >= 1");
  c->ls_interval = growth_interval;
  c->ls_staging[0] = scale;
  c->ls_staging[1] = 0.f;
  HIPCHK(c, hipMemcpyAsync(c->scal + 10, c->ls_staging, 8, hipMemcpyHostToDevice, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  return GPT2_OK;
}

GPT2_API double gpt2_lr_at(int64_t it, double max_lr, double min_lr, int64_t warmup,
                          int64_t decay_end) {
  if (it < 0 || warmup < 1 || decay_end <= warmup || !(min_lr >= 0.0) || !(max_lr >= min_lr))
    return std::nan("");
  if (it < warmup) return max_lr * (double)(it + 1) / (double)warmup;
  if (it > decay_end) return min_lr;
  const double f = (double)(it - warmup) / (double)(decay_end - warmup);
  return min_lr + (max_lr - min_lr) * 0.5 * (1.0 + std::cos(M_PI * f));
}

GPT2_API gpt2_status gpt2_block_fwd_bwd(gpt2_ctx* c, int32_t layer, const float* d_x,
                                        const float* d_dy, float* d_y, float* d_dx, int32_t B,
                                        int32_t T) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!d_x || !d_dy || !d_y || !d_dx) return fail(c, GPT2_E_ARG, "NULL buffer");
  if (layer < 0 || layer >= c->L) return fail(c, GPT2_E_ARG, "layer out of range");
  if (B < 1 || T < 1 || T > c->cfg.max_seq || (int64_t)B * T > c->maxM)
    return fail(c, GPT2_E_SHAPE, "B*T exceeds the arena or T > max_seq");
  const int M = B * T;
  const size_t bytes = (size_t)M * c->C * 4;
  HIPCHK(c, hipMemcpyAsync(c->h[2 * layer], d_x, bytes, hipMemcpyDeviceToDevice, c->st));
  HIPCHK(c, fwd_layer(c, layer, M, B, T));
  HIPCHK(c, hipMemcpyAsync(d_y, c->h[2 * layer + 2], bytes, hipMemcpyDeviceToDevice, c->st));
  HIPCHK(c, hipMemcpyAsync(c->dres, d_dy, bytes, hipMemcpyDeviceToDevice, c->st));
  HIPCHK(c, gk::copy_f32_to_act(c->dres, c->dres_act, c->dt, (size_t)M * c->C, c->st));
  HIPCHK(c, bwd_layer(c, layer, M, B, T, 0.f));
  HIPCHK(c, hipMemcpyAsync(d_dx, c->dres, bytes, hipMemcpyDeviceToDevice, c->st));
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_check_arena(gpt2_ctx* c, int32_t* n_bad) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  const size_t n = c->guards.size();
  c->guard_host.assign(n * kGuard, 0);
  for (size_t i = 0; i < n; ++i)
    HIPCHK(c, hipMemcpyAsync(c->guard_host.data() + i * kGuard, c->arena + c->guards[i].offset, kGuard,
                             hipMemcpyDeviceToHost, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  int32_t bad = 0;
  std::string first;
  for (size_t i = 0; i < n; ++i)
    for (size_t k = 0; k < kGuard; ++k)
      if (c->guard_host[i * kGuard + k] != kGuardByte) {
        if (bad++ == 0) first = c->guards[i].owner;
        break;
      }
  if (n_bad) *n_bad = bad;
  if (bad) return fail(c, GPT2_E_ARENA, "guard after region '" + first + "' overwritten (" +
                                            std::to_string(bad) + " damaged guards)");
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_sync_weight_copies(gpt2_ctx* c) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (c->h16) HIPCHK(c, gk::to_h16(c->params, c->shadow, c->nflat, c->dt, c->st));
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_get_step_count(gpt2_ctx* c, int64_t* t) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!t) return fail(c, GPT2_E_ARG, "NULL output");
  float v = 0.f;
  HIPCHK(c, hipMemcpyAsync(&v, c->scal + 5, 4, hipMemcpyDeviceToHost, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  *t = (int64_t)v;
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_set_step_count(gpt2_ctx* c, int64_t t) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (t < 0 || t > (1 << 24)) return fail(c, GPT2_E_ARG, "step count outside [0, 2^24]");
  c->step_staging = (float)t;
  HIPCHK(c, hipMemcpyAsync(c->scal + 5, &c->step_staging, 4, hipMemcpyHostToDevice, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  return GPT2_OK;
}

GPT2_API int32_t gpt2_num_tensors(const gpt2_ctx* c) { return c ? (int32_t)c->tensors.size() : -1; }

GPT2_API gpt2_status gpt2_tensor_info(const gpt2_ctx* c, int32_t i, gpt2_tensor_desc* out) {
  if (!c || !out || i < 0 || i >= (int32_t)c->tensors.size()) return GPT2_E_ARG;
  const Tensor& t = c->tensors[i];
  std::memset(out, 0, sizeof(*out));
  std::snprintf(out->name, sizeof(out->name), "%s", t.name.c_str());
  out->kind = t.kind;
  out->dtype = t.dtype;
  out->ndim = t.ndim;
  out->decay = t.decay;
  for (int k = 0; k < 4; ++k) out->shape[k] = t.shape[k];
  out->offset = t.offset;
  out->bytes = t.bytes;
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_timing_enable(gpt2_ctx* c, int32_t kernel_class) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (kernel_class < 0 || kernel_class > GPT2_T_EMBED) return fail(c, GPT2_E_ARG, "bad kernel class");
  c->tclass = kernel_class;
  c->ev_used = 0;
  return GPT2_OK;
}

GPT2_API gpt2_status gpt2_timing_read(gpt2_ctx* c, double* total_ms, int64_t* launches) {
  gpt2_status s = check_ctx(c);
  if (s) return s;
  if (!total_ms || !launches) return fail(c, GPT2_E_ARG, "NULL output");
  HIPCHK(c, hipStreamSynchronize(c->st));
  double tot = 0.0;
  for (size_t i = 0; i < c->ev_used; ++i) {
    float ms = 0.f;
    HIPCHK(c, hipEventElapsedTime(&ms, c->ev[i].first, c->ev[i].second));
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)c->ev_used;
  c->ev_used = 0;
  return GPT2_OK;
}
