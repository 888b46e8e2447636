// Host orchestrator and C ABI (include/la.h).
//
// One context = one request.  A round follows "M7.3 - Lookahead Decoding"
// (0x03A lifecycle, 0x06 loop, 0x06A publication plan, 0x07 fail-closed
// publication):
//   la_predict : pool lookup for x_t (after warmup) -> row manifest ->
//                target forward over the packed rows -> fp32 logits of the
//                out / inp / guess rows only;
//   la_verify  : argmax (greedy) or one-hot sampling -> accept record + z;
//   la_commit  : validate the plan, then K/V compaction, pool upsert from
//                the pre-shift window and z, window advance, output append.
// The only host<->device synchronisations of a round are the candidate
// count after the lookup and the accept record after verification.
#include "../../include/la.h"
#include "la_kernels.h"

#include <algorithm>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#define PREFILL_CHUNK 256
#define LA_MAX_DEVICES 64
#define LK_WORDS (1 + 64 * LA_MAX_N)
#define OG_WORDS (LA_MAX_N * LA_MAX_N)   // one round's output n-grams: at most N of N words

static thread_local std::string g_err;

// Packed projection buffer: per layer wqkv, wo, w_gate_up, w_down, then
// lm_head, each in the GEMM's packed layout (element offsets).
struct PackedOffsets { size_t qkv, o, gu, dn, layer, lm, total; };

struct la_ctx {
  la_config cfg;
  la_model_dims dims;
  la_model w;
  PackedOffsets pk;
  hipStream_t st;
  int dtype, esz;
  int L, d, H, Hkv, dh, F, V, qkvdim;
  int R, S;
  int t_cap, q_max, m_max, ws_cap, n_logit_max, nb_max, maxp_max, words_max, parts, wstride, rows_words;
  int rope_rows;      // positions reach kv_len + maxp, beyond the K/V capacity
  int hmax;           // most accepted candidate tokens per round: S, or S - 1 under cap_full_match
  bool rows_fit;      // every round layout fits the row builder's tables
  // device
  char* kc;
  char* vc;
  void *x, *nrm, *qkv, *q, *o, *act, *fin, *kw, *vw;
  float *gemm_p, *attn_po, *attn_pml, *logits;
  float2* rope;
  int32_t* rowbuf;
  int32_t *pf_tok, *pf_pos, *pf_branch, *pf_path, *pf_logit;
  int32_t *pool_cnt, *pool_ent;
  int32_t* win[2];
  int cur;
  int32_t *cand, *ncand, *vcand, *amax, *z, *z2, *tok1;
  LaAcceptDev* acc;
  double* escr;
  // host state
  std::vector<int32_t> out;
  int kv_len = 0;
  int round_id = 0;
  int sizes[LA_MAX_N];
  bool warm = false;
  bool pending = false, verified = false;
  bool paused = false;          // this round runs without the lookahead branch (batch throttle)
  const float* lg = nullptr;    // the pending round's logits (own buffer, or a batch's rows)
  LaLayout lay;
  LaRowsDev rows;
  std::vector<int32_t> cand_host;
  la_accept vacc;
  la_stats_t stats;
  std::string err;
  // opt-in kernel timing
  bool prof = false;
  la_profile_t pr;
  struct Mark { hipEvent_t a, b; int kind; double bytes, flops; };
  std::vector<Mark> marks;      // recorded this round
  std::vector<hipEvent_t> evpool;
  size_t evnext = 0;
  // the next round's pool lookup, started by la_commit: its count and
  // candidates land in pinned host memory (lk_key: the key, -1: none);
  // the verification result follows them in the same allocation
  int32_t* lk_host = nullptr;   // [LK_WORDS] then one LaAcceptDev, then [OG_WORDS]
  LaAcceptDev* acc_host = nullptr;
  int32_t* og_host = nullptr;   // staging of the output n-grams a round inserts
  std::vector<int32_t> ptail;   // the prompt's last N - 1 tokens (n-grams reaching into the prompt)
  int lk_key = -1;
  ~la_ctx() {
    if (lk_host) (void)hipHostFree(lk_host);
  }
};

static hipEvent_t prof_event(la_ctx* c) {
  if (c->evnext == c->evpool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    c->evpool.push_back(e);
  }
  return c->evpool[c->evnext++];
}

// bracket a launch: call with begin=true before it, begin=false after it
static void prof_mark(la_ctx* c, bool begin, int kind, double bytes, double flops) {
  if (!c->prof) return;
  hipEvent_t e = prof_event(c);
  if (!e) return;
  hipEventRecord(e, c->st);
  if (begin) c->marks.push_back({e, nullptr, kind, bytes, flops});
  else c->marks.back().b = e;
}

// called after a stream synchronisation: fold the recorded pairs into the totals
static void prof_collect(la_ctx* c) {
  for (auto& m : c->marks) {
    float ms = 0.f;
    if (m.b && hipEventElapsedTime(&ms, m.a, m.b) == hipSuccess) {
      if (m.kind == 0) { c->pr.gemm_ms += ms; c->pr.gemm_bytes += m.bytes; c->pr.gemm_flops += m.flops; c->pr.gemm_launches++; }
      else { c->pr.attn_ms += ms; c->pr.attn_bytes += m.bytes; c->pr.attn_flops += m.flops; c->pr.attn_launches++; }
    }
  }
  c->marks.clear();
  c->evnext = 0;
}

static int fail(la_ctx* c, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  g_err = buf;
  return code;
}

#define HIPCHK(c, call)                                                                         \
  do {                                                                                          \
    hipError_t _e = (call);                                                                     \
    if (_e != hipSuccess) return fail((c), LA_EDEVICE, "%s: %s", #call, hipGetErrorString(_e)); \
  } while (0)

// ------------------------------------------------------------------ sizing

static int validate_dims(const la_model_dims* d, la_ctx* c) {
  if (d->dtype != LA_DTYPE_F32 && d->dtype != LA_DTYPE_BF16) return fail(c, LA_EINVAL, "dtype %d", d->dtype);
  if (d->n_layers < 1 || d->d_model < 16 || d->n_heads < 1 || d->n_kv_heads < 1 || d->n_heads % d->n_kv_heads)
    return fail(c, LA_EINVAL, "bad model dims");
  const int dh = d->head_dim;
  if (!(d->dtype == LA_DTYPE_BF16 ? (dh == 128 || dh == 64) : (dh == 16 || dh == 64)))
    return fail(c, LA_EINVAL, "head_dim %d unsupported", dh);
  if (d->vocab < 2 || d->vocab > 65536) return fail(c, LA_EINVAL, "vocab %d out of range", d->vocab);
  // the GEMM takes K in whole 128 (bf16) / 64 (fp32) element chunks and N in 16-column tiles
  const int kc = d->dtype == LA_DTYPE_BF16 ? 128 : 64;
  if (d->d_model % kc || (d->n_heads * dh) % kc || d->d_ff % kc || d->vocab % 16 || d->d_ff % 16)
    return fail(c, LA_EINVAL, "d_model, n_heads*head_dim and d_ff must be multiples of %d, vocab of 16", kc);
  // the embedding gather and the residual fold + RMSNorm hold a row in at most
  // 2048 16-byte vectors (256 threads x 8)
  const int esz = d->dtype == LA_DTYPE_BF16 ? 2 : 4;
  if ((long)d->d_model * esz / 16 > 2048)
    return fail(c, LA_EINVAL, "d_model %d exceeds the %d the row kernels hold", d->d_model, 2048 * 16 / esz);
  return LA_OK;
}

static int validate_cfg(const la_config* cfg, const la_model_dims* d, la_ctx* c) {
  if (!cfg || !d) return fail(c, LA_EINVAL, "null config or dims");
  if (cfg->N < 3 || cfg->N > LA_MAX_N) return fail(c, LA_EINVAL, "N=%d not admitted (pinned schedule needs 3 <= N <= %d)", cfg->N, LA_MAX_N);
  if (cfg->W < 1 || cfg->W > 64) return fail(c, LA_EINVAL, "W=%d out of range [1, 64]", cfg->W);
  if (cfg->G < 0 || cfg->G > 64) return fail(c, LA_EINVAL, "G=%d out of range [0, 64]", cfg->G);
  if (cfg->max_new < 1 || cfg->max_prompt < 1) return fail(c, LA_EINVAL, "max_new and max_prompt must be >= 1");
  if (cfg->verify_mode != LA_VERIFY_GREEDY && cfg->verify_mode != LA_VERIFY_SAMPLE)
    return fail(c, LA_EINVAL, "verify_mode %d", cfg->verify_mode);
  if (cfg->verify_mode == LA_VERIFY_SAMPLE && !(cfg->temperature > 0.0)) return fail(c, LA_EINVAL, "temperature must be > 0");
  if (cfg->pool_from_prompt != 0 && cfg->pool_from_prompt != 1)
    return fail(c, LA_EINVAL, "pool_from_prompt %d (0 or 1)", cfg->pool_from_prompt);
  if (cfg->advance_by_accepted != 0 && cfg->advance_by_accepted != 1)
    return fail(c, LA_EINVAL, "advance_by_accepted %d (0 or 1)", cfg->advance_by_accepted);
  if (cfg->cap_full_match != 0 && cfg->cap_full_match != 1)
    return fail(c, LA_EINVAL, "cap_full_match %d (0 or 1)", cfg->cap_full_match);
  if (cfg->pool_from_output != 0 && cfg->pool_from_output != 1)
    return fail(c, LA_EINVAL, "pool_from_output %d (0 or 1)", cfg->pool_from_output);
  return validate_dims(d, c);
}

static PackedOffsets packed_offsets(const la_model_dims& d) {
  const int qkvdim = (d.n_heads + 2 * d.n_kv_heads) * d.head_dim;
  PackedOffsets p{};
  p.qkv = 0;
  const int dt = d.dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32;
  p.o = la_gemm_packed_elems(dt, qkvdim, d.d_model, 0);
  p.gu = p.o + la_gemm_packed_elems(dt, d.d_model, d.n_heads * d.head_dim, 0);
  p.dn = p.gu + la_gemm_packed_elems(dt, d.d_ff, d.d_model, 1);
  p.layer = p.dn + la_gemm_packed_elems(dt, d.d_model, d.d_ff, 0);
  p.lm = p.layer * d.n_layers;
  p.total = p.lm + la_gemm_packed_elems(dt, d.vocab, d.d_model, 0);
  return p;
}

static void setup_dims(la_ctx* c) {
  const la_config& g = c->cfg;
  const la_model_dims& d = c->dims;
  c->dtype = d.dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32;
  c->esz = d.dtype == LA_DTYPE_BF16 ? 2 : 4;
  c->L = d.n_layers; c->d = d.d_model; c->H = d.n_heads; c->Hkv = d.n_kv_heads; c->dh = d.head_dim;
  c->F = d.d_ff; c->V = d.vocab;
  c->qkvdim = (c->H + 2 * c->Hkv) * c->dh;
  c->R = g.N - 1; c->S = g.N - 1;
  c->hmax = c->S - (g.cap_full_match ? 1 : 0);
  // most rows over the warmup schedule and the steady state with G candidates
  int sz[LA_MAX_N] = {0};
  sz[0] = g.W + g.N - 3;
  int qmax = 0, lmax = 0, ncmax = 0, pmax = c->S;
  c->rows_fit = true;
  for (int stage = 0; stage < c->R; ++stage) {
    LaLayout L{};
    L.p = 0; L.R = c->R; L.C = g.G; L.S = c->S;
    for (int r = 0; r < c->R; ++r) { L.sizes[r] = sz[r]; L.starts[r] = r == 0 ? 1 : 0; }
    if (la_layout_finish(&L) == 0) {
      qmax = std::max(qmax, L.Q); lmax = std::max(lmax, L.n_logit);
      ncmax = std::max(ncmax, L.NB); pmax = std::max(pmax, L.maxp);
      c->rows_fit = c->rows_fit && la_build_rows_fits(L);
    }
    int dpt = 0;
    for (int r = 0; r < c->R; ++r) if (sz[r] > 0) dpt = r;
    if (dpt + 1 < c->R) {
      const int ninp = sz[dpt];
      for (int r = 0; r <= dpt; ++r) sz[r] -= 1;
      sz[dpt + 1] = ninp - (dpt >= 1 ? 1 : 0);
    }
  }
  c->q_max = std::max(qmax, 1);
  c->n_logit_max = std::max(lmax, 1);
  c->nb_max = std::max(ncmax, 1);
  c->maxp_max = std::max(pmax, 1);
  c->words_max = (c->q_max + 31) / 32;
  c->m_max = std::max(c->q_max, PREFILL_CHUNK);
  c->ws_cap = c->q_max;
  c->t_cap = g.max_prompt + g.max_new + 16;
  c->parts = la_attention_parts(c->t_cap + c->maxp_max, c->t_cap);   // positions stay below t_cap + maxp
  c->rope_rows = c->t_cap + c->q_max + 1;
  c->wstride = g.W + g.N;
  c->rows_words = 8 * c->q_max + c->nb_max * c->maxp_max + c->nb_max + c->n_logit_max + c->q_max * c->words_max +
                  (c->q_max + 15) / 16 * (64 + 16 * 64);
}

// Admission of the round shapes a config produces, before any state exists
// ("M7.3", 0x01A: unsupported schedules are refused before a round is
// compiled): every kernel of the round must take the largest round.
#define LA_MAX_ROWS 256      // packed rows one GEMM launch holds (16 row tiles)
#define LA_MAX_BRANCH 64     // positions a branch may reach past the committed prefix (attention path table)
static int admit(la_ctx* c) {
  const la_config& g = c->cfg;
  if (c->q_max > LA_MAX_ROWS)
    return fail(c, LA_EINVAL, "W=%d N=%d G=%d needs %d packed rows in a round; at most %d are admitted", g.W, g.N, g.G,
                c->q_max, LA_MAX_ROWS);
  if (c->maxp_max > LA_MAX_BRANCH)
    return fail(c, LA_EINVAL, "W=%d N=%d: a branch reaches %d positions past the committed prefix; at most %d are admitted",
                g.W, g.N, c->maxp_max, LA_MAX_BRANCH);
  if (!c->rows_fit) return fail(c, LA_EINVAL, "W=%d N=%d G=%d: the row builder's tables do not fit", g.W, g.N, g.G);
  if (!la_attention_fits(c->dh, c->esz, c->q_max, c->nb_max, c->maxp_max))
    return fail(c, LA_EINVAL, "W=%d N=%d G=%d needs %d packed rows in a round; the attention's tail stage does not "
                "hold them at head dim %d", g.W, g.N, g.G, c->q_max, c->dh);
  return LA_OK;
}

// fp32 floats of the K-split partials for M projection rows and Ml LM-head rows
static size_t partial_floats(int dt, int d, int qkvdim, int qd, int F, int V, int M, int Ml) {
  struct { int N, K, sw, M; } mats[] = {{qkvdim, d, 0, M}, {d, qd, 0, M}, {F, d, 1, M}, {d, F, 0, M}, {V, d, 0, Ml}};
  size_t mx = 0;
  for (auto& m : mats) {
    const int s = la_gemm_splits(m.N, m.K, dt, m.sw);
    if (s > 1) mx = std::max(mx, (size_t)s * m.M * (m.sw ? 2 * m.N : m.N));
  }
  return mx;
}

static size_t gemm_partial_floats(la_ctx* c) {
  return partial_floats(c->dtype, c->d, c->qkvdim, c->H * c->dh, c->F, c->V, c->m_max, c->n_logit_max);
}

static size_t carve(la_ctx* c, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? (void*)(base + off) : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  const size_t e = c->esz;
  c->x = take((size_t)c->m_max * c->d * e);
  c->nrm = take((size_t)c->m_max * c->d * e);
  c->qkv = take((size_t)c->m_max * c->qkvdim * e);
  c->q = take((size_t)c->m_max * c->H * c->dh * e);
  c->o = take((size_t)c->m_max * c->H * c->dh * e);
  c->act = take((size_t)c->m_max * c->F * e);
  c->fin = take((size_t)c->n_logit_max * c->d * e);
  c->kw = take((size_t)c->L * c->Hkv * c->ws_cap * c->dh * e);
  c->vw = take((size_t)c->L * c->Hkv * c->ws_cap * c->dh * e);
  c->gemm_p = (float*)take(std::max<size_t>(gemm_partial_floats(c), 1) * 4);
  c->attn_po = (float*)take((size_t)c->parts * c->H * c->m_max * c->dh * 4);
  c->attn_pml = (float*)take((size_t)c->parts * c->H * c->m_max * 2 * 4);
  c->logits = (float*)take((size_t)c->n_logit_max * c->V * 4);
  c->rope = (float2*)take((size_t)c->rope_rows * (c->dh / 2) * sizeof(float2));
  c->rowbuf = (int32_t*)take((size_t)c->rows_words * 4);
  c->pf_tok = (int32_t*)take((size_t)c->m_max * 4);
  c->pf_pos = (int32_t*)take((size_t)c->m_max * 4);
  c->pf_branch = (int32_t*)take((size_t)c->m_max * 4);
  c->pf_path = (int32_t*)take(64);
  c->pf_logit = (int32_t*)take(64);
  c->pool_cnt = (int32_t*)take((size_t)c->V * 4);
  c->pool_ent = (int32_t*)take((size_t)c->V * std::max(c->cfg.G, 1) * c->S * 4);
  c->win[0] = (int32_t*)take((size_t)c->R * c->wstride * 4);
  c->win[1] = (int32_t*)take((size_t)c->R * c->wstride * 4);
  c->cand = (int32_t*)take((size_t)64 * LA_MAX_N * 4);
  c->vcand = (int32_t*)take((size_t)64 * LA_MAX_N * 4);
  c->ncand = (int32_t*)take(64);
  c->amax = (int32_t*)take((size_t)std::max(c->n_logit_max, 64) * 4);
  c->acc = (LaAcceptDev*)take(sizeof(LaAcceptDev));
  c->z = (int32_t*)take((size_t)c->wstride * 4);
  c->z2 = (int32_t*)take((size_t)std::max(c->wstride, 64) * 4);
  c->tok1 = (int32_t*)take(64);
  c->escr = (double*)take(((size_t)c->V + 256) * 8);   // a row's masses, then its block sums
  return off;
}

extern "C" int la_query_sizes(const la_config* cfg, const la_model_dims* dims, la_sizes* out) {
  int rc = validate_cfg(cfg, dims, nullptr);
  if (rc) return rc;
  if (!out) return fail(nullptr, LA_EINVAL, "null output");
  la_ctx c{};
  c.cfg = *cfg;
  c.dims = *dims;
  setup_dims(&c);
  if ((rc = admit(&c))) return rc;
  out->kv_bytes = 2ull * c.L * c.Hkv * (size_t)c.t_cap * c.dh * c.esz;
  out->arena_bytes = carve(&c, nullptr);
  out->t_cap = c.t_cap;
  out->q_max = c.q_max;
  out->n_logit_max = c.n_logit_max;
  out->reserved = 0;
  return LA_OK;
}

// ------------------------------------------------------------------ forward

static const char* wptr(const void* base, size_t elems_per_layer, int l, int esz) {
  return (const char*)base + (size_t)l * elems_per_layer * esz;
}

// The fp32 QKV projection writes q, k and v (rotated, placed) from its
// epilogue when its K is not split; its weights are then packed pair-major.
// A function of the shape only, shared by the packer and the forward.  bf16
// stores the projection and rotates / places it with la_qkv_post_launch.
static bool qkv_fused(int qkvdim, int d, int dt, int dh) {
  return dt == LA_DT_F32 && la_gemm_splits(qkvdim, d, dt, 0) == 1 && dh >= 16 && (dh & (dh - 1)) == 0;
}

// Activation buffers of one forward: a context's own (one request) or a
// batch's (several requests whose rows are stacked).
struct FwdBufs {
  void *x, *nrm, *qkv, *q, *o, *act, *fin;
  float *gemm_p, *logits;
};

static FwdBufs own_bufs(la_ctx* c) {
  return FwdBufs{c->x, c->nrm, c->qkv, c->q, c->o, c->act, c->fin, c->gemm_p, c->logits};
}

// One request's rows inside a forward: rows r0 .. r0 + M - 1 of the stacked
// activations, its logit rows at l0 .. l0 + n_logit - 1 of the logits.
// K/V of its rows < n_direct go to cache rows cache_row0 + m, the others to
// workspace rows m - n_direct; keys below shared_end come from the cache.
struct Seg {
  la_ctx* s;
  int r0, M, l0;
  const int32_t *tok, *pos, *branch, *path, *path_len, *tile_meta, *tile_path, *logit_rows;
  int nb, maxp, n_direct, cache_row0, shared_end, max_pos, n_logit;
};

// Device tables of a forward whose per-request passes (rotary placement and
// attention) run as one launch per layer for all requests: entry i is
// request i, with layer 0's cache pointers and the distance between layers.
struct SegTables {
  const LaAttnSeg* attn;
  const LaPostSeg* post;
  LaAttnMulti shape;
};

// One request's attention arguments for layer l (the launcher completes the rest).
static LaAttnArgs seg_attn_args(la_ctx* c, const FwdBufs& B, const Seg& g, int l) {
  la_ctx* s = g.s;
  const int esz = c->esz, qd = c->H * c->dh;
  const size_t skvl = (size_t)s->Hkv * s->t_cap * s->dh;
  const size_t swsl = (size_t)s->Hkv * s->ws_cap * s->dh;
  LaAttnArgs at{};
  at.q = (char*)B.q + (size_t)g.r0 * qd * esz;
  at.o = (char*)B.o + (size_t)g.r0 * qd * esz;
  at.part_o = s->attn_po; at.part_ml = s->attn_pml; at.max_splits = s->parts;
  at.pos = g.pos; at.branch = g.branch; at.path = g.path; at.path_len = g.path_len;
  at.tile_meta = g.tile_meta; at.tile_path = g.tile_path;
  at.Q = g.M; at.H = c->H; at.Hkv = c->Hkv; at.dh = c->dh; at.T_cap = s->t_cap; at.ws_cap = s->ws_cap;
  at.maxp = g.maxp;
  at.shared_end = g.shared_end;
  at.max_pos = g.max_pos;
  at.nb = g.nb;
  at.n_ws = g.M - g.n_direct;
  at.scale = 1.0f / sqrtf((float)c->dh);
  at.kc = s->kc + l * skvl * esz;
  at.vc = s->vc + l * skvl * esz;
  at.kw = (char*)s->kw + l * swsl * esz;
  at.vw = (char*)s->vw + l * swsl * esz;
  return at;
}

// committed K/V read once (positions below shared_end), each packed row's K/V, Q in, O out
static void seg_attn_cost(la_ctx* c, const Seg& g, double* bytes, double* flops) {
  const int qd = c->H * c->dh;
  const double kvrow = 2.0 * c->Hkv * c->dh * c->esz;
  *bytes += g.shared_end * kvrow + (double)(g.M - g.n_direct) * kvrow + 2.0 * g.M * qd * c->esz;
  *flops += 4.0 * g.M * qd * (double)(g.max_pos + 1);
}

static int gemm(la_ctx* c, float* P, int epi, const void* X, const void* W, void* Y, const void* Rr, int M, int N,
                int K, int up_off, bool defer = false, const LaQkvOut* qo = nullptr) {
  LaGemmArgs a{};
  a.X = X; a.W = W; a.Y = Y; a.R = Rr; a.P = P;
  a.M = M; a.N = N; a.K = K; a.ldx = K; a.ldy = N;
  a.splits = la_gemm_splits(N, K, c->dtype, epi == LA_EPI_SWIGLU);
  a.up_off = up_off;
  a.pcols = epi == LA_EPI_SWIGLU ? 2 * N : N;
  a.defer_reduce = defer ? 1 : 0;
  if (qo) a.qo = *qo;
  const double wrows = epi == LA_EPI_SWIGLU ? 2.0 * N : (double)N;
  const double ybytes = epi == LA_EPI_F32 ? 4.0 : (double)c->esz;
  const double bytes = (wrows * K + (double)M * K) * c->esz + (double)M * N * ybytes * (epi == LA_EPI_RESID ? 2 : 1);
  prof_mark(c, true, 0, bytes, 2.0 * M * wrows * K);
  const int rc = la_gemm_launch(c->dtype, epi, a, c->st);
  prof_mark(c, false, 0, 0, 0);
  if (rc) return fail(c, rc == -2 ? LA_EINVAL : LA_EDEVICE, "gemm launch failed (M=%d N=%d K=%d rc=%d)", M, N, K, rc);
  return LA_OK;
}

// A residual projection x += Y W^T.  With a split K its partials stay in
// the partial buffer and the next RMSNorm folds them into x (same sum, same
// rounding); returns the number of pending partials (0 when x was updated in
// place).
static int resid_gemm(la_ctx* c, const FwdBufs& B, const void* X, const void* W, int M, int K, int* pending) {
  const int s = la_gemm_splits(c->d, K, c->dtype, 0);
  *pending = s > 1 ? s : 0;
  return gemm(c, B.gemm_p, LA_EPI_RESID, X, W, B.x, B.x, M, c->d, K, 0, s > 1);
}

// The target forward over the stacked rows of ns requests ("M7.3", 0x04C:
// one causal forward over the packed rows; "Speculative Decoding", Chapter 7:
// concurrent requests share one read of the weights per step).  Every
// projection, RMSNorm and the LM head runs once over all rows; the rotary
// placement of q, k and v and the attention run per request against its own
// cache.  Each row's arithmetic is the same whatever rows share the launch
// (the GEMM's K split depends on the shape only), so a request's logits are
// bitwise those of its own forward.  c supplies the dims, the weights and
// the stream (all requests share them); fp32 logits of request i land in
// B.logits rows sg[i].l0 ...  With tables (entries in the order of sg), the
// per-request passes run as one launch per layer.
static int forward_segs(la_ctx* c, const FwdBufs& B, const Seg* sg, int ns, const SegTables* tab = nullptr) {
  const int esz = c->esz;
  int M = 0, n_logit = 0;
  for (int i = 0; i < ns; ++i) { M += sg[i].M; n_logit += sg[i].n_logit; }
  const int qd = c->H * c->dh;
  for (int i = 0; i < ns; ++i)
    la_embed_launch(c->dtype, c->w.embed, sg[i].tok, (char*)B.x + (size_t)sg[i].r0 * c->d * esz, sg[i].M, c->d, c->st);
  const bool fused = qkv_fused(c->qkvdim, c->d, c->dtype, c->dh);
  const int qs = la_gemm_splits(c->qkvdim, c->d, c->dtype, 0);
  int pend = 0;   // split partials of the last residual projection not yet folded into x
  const size_t pstride = (size_t)M * c->d;
  for (int l = 0; l < c->L; ++l) {
    const char* attn_norm = wptr(c->w.attn_norm, c->d, l, esz);
    const char* mlp_norm = wptr(c->w.mlp_norm, c->d, l, esz);
    const char* wl = (const char*)c->w.packed + c->pk.layer * l * esz;
    const char* wqkv = wl + c->pk.qkv * esz;
    const char* wo = wl + c->pk.o * esz;
    const char* wgu = wl + c->pk.gu * esz;
    const char* wdn = wl + c->pk.dn * esz;
    int rc;
    if (la_addnorm_launch(c->dtype, B.x, B.gemm_p, pend, pstride, 1, attn_norm, B.nrm, nullptr, M, c->d,
                          c->dims.eps, c->st))
      return fail(c, LA_EINVAL, "residual fold of %d split partials exceeds %d", pend, LA_ADDNORM_MAX_SPLITS);
    if (!fused) {
      // split K: the partials go straight to the rotate-and-place pass (one fixed-order sum per value)
      if ((rc = gemm(c, B.gemm_p, LA_EPI_STORE, B.nrm, wqkv, B.qkv, nullptr, M, c->qkvdim, c->d, 0, qs > 1)))
        return rc;
    }
    // rotary placement of q, k and v: each request's k and v go to its own cache
    if (tab && !fused) {
      la_qkv_post_multi_launch(c->dtype, B.gemm_p, qs > 1 ? qs : 0, B.qkv, M, tab->post, ns, l, c->H, c->Hkv, c->dh,
                               B.q, c->st);
    } else {
      for (int i = 0; i < ns; ++i) {
        const Seg& g = sg[i];
        la_ctx* s = g.s;
        const size_t skvl = (size_t)s->Hkv * s->t_cap * s->dh;
        const size_t swsl = (size_t)s->Hkv * s->ws_cap * s->dh;
        char* kc = s->kc + l * skvl * esz;
        char* vc = s->vc + l * skvl * esz;
        char* kw = (char*)s->kw + l * swsl * esz;
        char* vw = (char*)s->vw + l * swsl * esz;
        char* q = (char*)B.q + (size_t)g.r0 * qd * esz;
        if (fused) {
          // the fused epilogue places into one request's cache: one launch per request
          const LaQkvOut qo{s->rope, g.pos, q, kc, vc, kw, vw, c->H, c->Hkv, c->dh, s->t_cap, g.cache_row0,
                            g.n_direct, s->ws_cap};
          if ((rc = gemm(c, B.gemm_p, LA_EPI_QKV, (char*)B.nrm + (size_t)g.r0 * c->d * esz, wqkv, B.qkv, nullptr,
                         g.M, c->qkvdim, c->d, 0, false, &qo)))
            return rc;
        } else if (qs > 1) {
          la_qkv_reduce_post_launch(c->dtype, B.gemm_p + (size_t)g.r0 * c->qkvdim, qs, M, g.M, s->rope, g.pos, c->H,
                                    c->Hkv, c->dh, q, kc, vc, s->t_cap, g.cache_row0, g.n_direct, kw, vw, s->ws_cap,
                                    c->st);
        } else {
          la_qkv_post_launch(c->dtype, (char*)B.qkv + (size_t)g.r0 * c->qkvdim * esz, s->rope, g.pos, g.M, c->H,
                             c->Hkv, c->dh, q, kc, vc, s->t_cap, g.cache_row0, g.n_direct, kw, vw, s->ws_cap, c->st);
        }
      }
    }
    // attention, each request against its own cache
    if (tab) {
      double bytes = 0, flops = 0;
      for (int i = 0; i < ns; ++i) seg_attn_cost(c, sg[i], &bytes, &flops);
      prof_mark(c, true, 1, bytes, flops);
      rc = la_attention_multi_launch(c->dtype, tab->shape, tab->attn, ns, l, c->st);
      prof_mark(c, false, 1, 0, 0);
      if (rc) return fail(c, LA_EDEVICE, "attention launch failed (%d)", rc);
    } else {
      for (int i = 0; i < ns; ++i) {
        double bytes = 0, flops = 0;
        seg_attn_cost(c, sg[i], &bytes, &flops);
        prof_mark(c, true, 1, bytes, flops);
        rc = la_attention_launch(c->dtype, seg_attn_args(c, B, sg[i], l), c->st);
        prof_mark(c, false, 1, 0, 0);
        if (rc) return fail(c, LA_EDEVICE, "attention launch failed (%d)", rc);
      }
    }
    if ((rc = resid_gemm(c, B, B.o, wo, M, qd, &pend))) return rc;
    if (la_addnorm_launch(c->dtype, B.x, B.gemm_p, pend, pstride, 1, mlp_norm, B.nrm, nullptr, M, c->d,
                          c->dims.eps, c->st))
      return fail(c, LA_EINVAL, "residual fold of %d split partials exceeds %d", pend, LA_ADDNORM_MAX_SPLITS);
    if ((rc = gemm(c, B.gemm_p, LA_EPI_SWIGLU, B.nrm, wgu, B.act, nullptr, M, c->F, c->d, c->F))) return rc;
    if ((rc = resid_gemm(c, B, B.act, wdn, M, c->F, &pend))) return rc;
  }
  if (n_logit > 0) {
    for (int i = 0; i < ns; ++i) {
      const Seg& g = sg[i];
      if (g.n_logit <= 0) continue;
      if (la_addnorm_launch(c->dtype, (char*)B.x + (size_t)g.r0 * c->d * esz, B.gemm_p + (size_t)g.r0 * c->d, pend,
                            pstride, 0, c->w.final_norm, (char*)B.fin + (size_t)g.l0 * c->d * esz, g.logit_rows,
                            g.n_logit, c->d, c->dims.eps, c->st))
        return fail(c, LA_EINVAL, "residual fold of %d split partials exceeds %d", pend, LA_ADDNORM_MAX_SPLITS);
    }
    int rc = gemm(c, B.gemm_p, LA_EPI_F32, B.fin, (const char*)c->w.packed + c->pk.lm * esz, B.logits, nullptr,
                  n_logit, c->V, c->d, 0);
    if (rc) return rc;
  }
  HIPCHK(c, hipGetLastError());
  return LA_OK;
}

// Forward M rows of one request into its own buffers.
static int forward(la_ctx* c, int M, const int32_t* tok, const int32_t* pos, const int32_t* branch,
                   const int32_t* path, const int32_t* path_len, const int32_t* tile_meta, const int32_t* tile_path,
                   int nb, int maxp, int n_direct, int cache_row0,
                   int shared_end, int max_pos, const int32_t* logit_rows, int n_logit) {
  Seg g{};
  g.s = c; g.r0 = 0; g.M = M; g.l0 = 0;
  g.tok = tok; g.pos = pos; g.branch = branch; g.path = path; g.path_len = path_len;
  g.tile_meta = tile_meta; g.tile_path = tile_path; g.logit_rows = logit_rows;
  g.nb = nb; g.maxp = maxp; g.n_direct = n_direct; g.cache_row0 = cache_row0; g.shared_end = shared_end;
  g.max_pos = max_pos; g.n_logit = n_logit;
  return forward_segs(c, own_bufs(c), &g, 1);
}

static void rows_layout(const LaLayout& L, int32_t* base, LaRowsDev* r, la_rows_info* info) {
  const int Q = L.Q;
  int off = 0;
  auto take = [&](int n) { int o = off; off += n; return o; };
  const int o_tok = take(Q), o_pos = take(Q), o_role = take(Q), o_level = take(Q), o_col = take(Q),
            o_cand = take(Q), o_off = take(Q), o_branch = take(Q), o_path = take(L.NB * L.maxp),
            o_plen = take(L.NB), o_logit = take(L.n_logit), o_mask = take(Q * L.mask_words);
  const int ntiles = (Q + 15) / 16;
  const int o_tmeta = take(ntiles * 64), o_tpath = take(ntiles * 16 * 64);
  if (r) {
    r->tok = base + o_tok; r->pos = base + o_pos; r->role = base + o_role; r->level = base + o_level;
    r->col = base + o_col; r->cand = base + o_cand; r->off = base + o_off; r->branch = base + o_branch;
    r->path = base + o_path; r->path_len = base + o_plen; r->logit_rows = base + o_logit;
    r->mask = (uint32_t*)(base + o_mask);
    r->tile_meta = base + o_tmeta; r->tile_path = base + o_tpath;
  }
  if (info) {
    info->Q = Q; info->NB = L.NB; info->maxp = L.maxp; info->n_logit = L.n_logit; info->n_inp = L.n_inp;
    info->n_cols = L.n_cols; info->mask_words = L.mask_words; info->total_words = off;
    info->off_tok = o_tok; info->off_pos = o_pos; info->off_role = o_role; info->off_level = o_level;
    info->off_col = o_col; info->off_cand = o_cand; info->off_off = o_off; info->off_branch = o_branch;
    info->off_path = o_path; info->off_path_len = o_plen; info->off_logit_rows = o_logit; info->off_mask = o_mask;
    info->off_tile_meta = o_tmeta; info->off_tile_path = o_tpath;
  }
}

// ------------------------------------------------------------------ lifecycle

// Generated-prefix insertion (pool_from_output; "M7.3", 0x06A pool plan):
// the n-grams that output tokens k0.. (all of c->out from k0 on) complete in
// the text prompt + output, in text order -- key the token N - 1 before,
// suffix the N - 1 tokens up to the new one -- by one wavefront's LRU upsert
// on the stream.  Staged in pinned memory: its previous contents were
// consumed before the caller's last stream synchronisation.
static int insert_output_ngrams(la_ctx* c, int k0) {
  if (!c->cfg.pool_from_output || c->cfg.ar_only || c->cfg.G <= 0) return LA_OK;
  const int S = c->S, np = (int)c->ptail.size(), k1 = (int)c->out.size();
  auto tok = [&](int g) { return g < np ? c->ptail[g] : c->out[g - np]; };   // g: index in ptail ++ out
  if (k1 - k0 > LA_MAX_N) return fail(c, LA_EINVAL, "%d output tokens in one round", k1 - k0);
  int32_t key[LA_MAX_N], suf[LA_MAX_N * LA_MAX_N];
  int n = 0;
  for (int k = k0; k < k1; ++k) {
    const int g = np + k;
    if (g < S) continue;                          // fewer than N tokens of text so far
    key[n] = tok(g - S);
    for (int s = 0; s < S; ++s) suf[n * S + s] = tok(g - S + 1 + s);
    ++n;
  }
  if (n == 0) return LA_OK;
  memcpy(c->og_host, key, (size_t)n * 4);
  memcpy(c->og_host + n, suf, (size_t)n * S * 4);
  HIPCHK(c, hipMemcpyAsync(c->vcand, c->og_host, (size_t)n * (1 + S) * 4, hipMemcpyHostToDevice, c->st));
  la_pool_upsert_launch(c->pool_cnt, c->pool_ent, c->vcand, c->vcand + n, n, c->cfg.G, S, c->st);
  HIPCHK(c, hipGetLastError());
  return LA_OK;
}

extern "C" int la_init(const la_config* cfg, const la_model_dims* dims, const la_model* weights, void* kv,
                       void* arena, const int32_t* prompt, int32_t prompt_len, void* stream, la_ctx** out) {
  if (!out) return fail(nullptr, LA_EINVAL, "null ctx output");
  *out = nullptr;
  int rc = validate_cfg(cfg, dims, nullptr);
  if (rc) return rc;
  if (!weights || !kv || !arena || !prompt) return fail(nullptr, LA_EINVAL, "null weights, buffers or prompt");
  if (!weights->packed || !weights->embed || !weights->final_norm || !weights->attn_norm || !weights->mlp_norm)
    return fail(nullptr, LA_EINVAL, "weights: packed projections (la_pack_weights), embed and norms are required");
  if (prompt_len < 1 || prompt_len > cfg->max_prompt)
    return fail(nullptr, LA_EINVAL, "prompt_len %d outside [1, max_prompt=%d]", prompt_len, cfg->max_prompt);
  for (int i = 0; i < prompt_len; ++i)
    if (prompt[i] < 0 || prompt[i] >= dims->vocab) return fail(nullptr, LA_EINVAL, "prompt token %d out of range", i);
  la_ctx* c = new la_ctx();
  c->cfg = *cfg;
  c->dims = *dims;
  c->w = *weights;
  c->pk = packed_offsets(*dims);
  c->st = (hipStream_t)stream;
  setup_dims(c);
  if ((rc = admit(c))) {
    g_err = c->err;
    delete c;
    return rc;
  }
  const size_t kvb = (size_t)c->L * c->Hkv * c->t_cap * c->dh * c->esz;
  c->kc = (char*)kv;
  c->vc = (char*)kv + kvb;
  carve(c, (char*)arena);
  if (hipHostMalloc((void**)&c->lk_host,
                    LK_WORDS * sizeof(int32_t) + sizeof(LaAcceptDev) + OG_WORDS * sizeof(int32_t),
                    hipHostMallocDefault) != hipSuccess) {
    c->lk_host = nullptr;
    delete c;
    return fail(nullptr, LA_EDEVICE, "pinned host buffer");
  }
  c->acc_host = (LaAcceptDev*)(c->lk_host + LK_WORDS);
  c->og_host = (int32_t*)(c->acc_host + 1);
  c->ptail.assign(prompt + std::max(0, prompt_len - c->S), prompt + prompt_len);
  memset(&c->stats, 0, sizeof c->stats);
  for (int r = 0; r < LA_MAX_N; ++r) c->sizes[r] = 0;
  c->cur = 0;
  auto bail = [&](int code) { delete c; return code; };
#define CK(call)                                                                   \
  do {                                                                             \
    hipError_t _e = (call);                                                        \
    if (_e != hipSuccess) {                                                        \
      fail(nullptr, LA_EDEVICE, "%s: %s", #call, hipGetErrorString(_e));           \
      return bail(LA_EDEVICE);                                                     \
    }                                                                              \
  } while (0)
  la_rope_table_launch(c->rope, c->rope_rows, c->dh, c->dims.rope_theta, c->st);
  la_pool_clear_launch(c->pool_cnt, c->V, c->st);
  // POOL_FROM_PROMPT: the prompt's N-grams in order, through the candidate
  // scratch in chunks (one wavefront upserts them serially, the LRU rule)
  if (c->cfg.pool_from_prompt && !c->cfg.ar_only && c->cfg.G > 0) {
    const int S = c->S, per = (64 * LA_MAX_N) / (1 + S);
    std::vector<int32_t> buf;
    for (int i0 = 0; i0 + S < prompt_len; i0 += per) {
      const int n = std::min(per, prompt_len - S - i0);
      buf.assign((size_t)n * (1 + S), 0);
      for (int i = 0; i < n; ++i) {
        buf[i] = prompt[i0 + i];
        for (int s = 0; s < S; ++s) buf[n + (size_t)i * S + s] = prompt[i0 + i + 1 + s];
      }
      CK(hipMemcpyAsync(c->vcand, buf.data(), buf.size() * 4, hipMemcpyHostToDevice, c->st));
      la_pool_upsert_launch(c->pool_cnt, c->pool_ent, c->vcand, c->vcand + n, n, c->cfg.G, S, c->st);
      CK(hipStreamSynchronize(c->st));      // buf is reused
    }
  }
  // window: level 0 seeded with the last W + N - 3 prompt tokens (cyclic)
  if (!c->cfg.ar_only) {
    const int n0 = c->cfg.W + c->cfg.N - 3;
    std::vector<int32_t> w0((size_t)c->R * c->wstride, 0);
    for (int i = 0; i < n0; ++i) w0[i] = prompt[(((prompt_len - n0 + i) % prompt_len) + prompt_len) % prompt_len];
    CK(hipMemcpyAsync(c->win[0], w0.data(), w0.size() * 4, hipMemcpyHostToDevice, c->st));
    c->sizes[0] = n0;
  }
  // prefill in chunks; every row's K/V goes straight to the cache
  std::vector<int32_t> tok, pos, br;
  for (int c0 = 0; c0 < prompt_len; c0 += PREFILL_CHUNK) {
    const int M = std::min(PREFILL_CHUNK, prompt_len - c0);
    tok.assign(prompt + c0, prompt + c0 + M);
    pos.resize(M);
    br.assign(M, 0);
    for (int i = 0; i < M; ++i) pos[i] = c0 + i;
    const int32_t zero[2] = {0, M - 1};
    CK(hipMemcpyAsync(c->pf_tok, tok.data(), M * 4, hipMemcpyHostToDevice, c->st));
    CK(hipMemcpyAsync(c->pf_pos, pos.data(), M * 4, hipMemcpyHostToDevice, c->st));
    CK(hipMemcpyAsync(c->pf_branch, br.data(), M * 4, hipMemcpyHostToDevice, c->st));
    CK(hipMemcpyAsync(c->pf_path, zero, 4, hipMemcpyHostToDevice, c->st));
    CK(hipMemcpyAsync(c->pf_logit, zero + 1, 4, hipMemcpyHostToDevice, c->st));
    const bool last = c0 + M >= prompt_len;
    rc = forward(c, M, c->pf_tok, c->pf_pos, c->pf_branch, c->pf_path, c->pf_path, nullptr, nullptr, 1, 1, M, c0,
                 c0 + M,
                 c0 + M - 1, c->pf_logit, last ? 1 : 0);
    if (rc) { g_err = c->err; return bail(rc); }
    CK(hipStreamSynchronize(c->st));        // the host-side chunk arrays are reused
  }
  // first output token from the last prompt row
  la_argmax_launch(c->logits, 1, c->V, c->amax, c->st);
  if (c->cfg.verify_mode == LA_VERIFY_SAMPLE)
    la_sample_row_launch(c->logits, c->V, c->cfg.temperature, c->cfg.seed, 0, c->amax, c->escr, c->tok1, c->st);
  int32_t first = 0;
  CK(hipMemcpyAsync(&first, c->cfg.verify_mode == LA_VERIFY_SAMPLE ? c->tok1 : c->amax, 4, hipMemcpyDeviceToHost,
                    c->st));
  CK(hipStreamSynchronize(c->st));
#undef CK
  c->out.push_back(first);
  c->kv_len = prompt_len;
  c->stats.tokens = 1;
  if ((rc = insert_output_ngrams(c, 0))) { g_err = c->err; return bail(rc); }   // the n-gram the first token completes
  *out = c;
  return LA_OK;
}

extern "C" void la_destroy(la_ctx* c) {
  if (!c) return;
  for (auto e : c->evpool) hipEventDestroy(e);
  delete c;
}

extern "C" int la_profile(la_ctx* c, int32_t enable) {
  if (!c) return fail(nullptr, LA_EINVAL, "null ctx");
  if (c->pending) return fail(c, LA_ESTATE, "a predicted round is pending");
  c->prof = enable != 0;
  memset(&c->pr, 0, sizeof c->pr);
  c->marks.clear();
  c->evnext = 0;
  return LA_OK;
}

extern "C" int la_profile_read(const la_ctx* c, la_profile_t* out) {
  if (!c || !out) return fail(nullptr, LA_EINVAL, "null argument");
  *out = c->pr;
  return LA_OK;
}

// ------------------------------------------------------------------ round

static bool is_warm(const la_ctx* c) {
  for (int r = 0; r < c->R; ++r)
    if (c->sizes[r] <= 0) return false;
  return true;
}

// Pool lookup of key into c->cand / c->ncand, with the count and all G
// candidate slots copied to the pinned host buffer (read after a sync).
static int start_lookup(la_ctx* c, int key) {
  la_pool_lookup_launch(c->pool_cnt, c->pool_ent, key, c->cfg.G, c->S, c->cand, c->ncand, c->st);
  HIPCHK(c, hipMemcpyAsync(c->lk_host, c->ncand, 4, hipMemcpyDeviceToHost, c->st));
  HIPCHK(c, hipMemcpyAsync(c->lk_host + 1, c->cand, (size_t)c->cfg.G * c->S * 4, hipMemcpyDeviceToHost, c->st));
  c->lk_key = key;
  return LA_OK;
}

// A round in parts, shared by la_predict / la_verify and la_batch_step.

// Checks before a round is compiled.
static int round_check(la_ctx* c) {
  if (c->pending) return fail(c, LA_ESTATE, "round %d is pending commit", c->round_id + 1);
  if ((int)c->out.size() >= c->cfg.max_new) return fail(c, LA_ESTATE, "max_new tokens already generated");
  if (c->kv_len + 1 + c->S > c->t_cap) return fail(c, LA_EOVERFLOW, "K/V capacity %d exhausted", c->t_cap);
  return LA_OK;
}

// Whether the round reads the pool; if so its lookup for the current token
// is under way after this (usually started by the last commit: same key,
// pool unchanged since).  Its count is read after a stream synchronisation.
static int round_lookup(la_ctx* c, bool* uses_pool) {
  *uses_pool = !c->cfg.ar_only && is_warm(c) && c->cfg.G > 0;
  if (!*uses_pool) {
    c->lk_key = -1;
    return LA_OK;
  }
  if (c->lk_key != c->out.back()) return start_lookup(c, c->out.back());
  return LA_OK;
}

// Candidates the lookup found (its copy has landed).
static int round_found(la_ctx* c, bool uses_pool, int* C) {
  *C = 0;
  if (!uses_pool) return LA_OK;
  const int n = c->lk_host[0];
  if (n < 0 || n > c->cfg.G) return fail(c, LA_EDEVICE, "pool lookup returned %d candidates", n);
  *C = n;
  return LA_OK;
}

// The round's layout with C candidates: the lookahead branch (the window's
// levels), or none when paused or autoregressive.
static int round_layout(const la_ctx* c, int C, bool paused, LaLayout* L) {
  *L = LaLayout{};
  L->p = c->kv_len; L->R = c->R; L->C = C; L->S = c->S;
  for (int r = 0; r < c->R; ++r) {
    L->sizes[r] = c->cfg.ar_only || paused ? 0 : c->sizes[r];
    L->starts[r] = r == 0 ? 1 : 0;
  }
  return la_layout_finish(L);
}

// Compile the round's rows on the stream: the first C of the candidates found
// (pool order: the oldest first, "M7.3" 0x03B), the lookahead branch unless
// paused.
static int round_rows(la_ctx* c, int C, bool paused) {
  const int p = c->kv_len;
  c->lk_key = -1;
  c->cand_host.assign(c->lk_host + 1, c->lk_host + 1 + (size_t)C * c->S);
  LaLayout L;
  if (round_layout(c, C, paused, &L)) return fail(c, LA_EINVAL, "inconsistent window layout");
  if (L.Q > c->q_max) return fail(c, LA_EOVERFLOW, "round needs %d rows > q_max %d", L.Q, c->q_max);
  if (p + L.maxp >= c->rope_rows) return fail(c, LA_EOVERFLOW, "position %d beyond the RoPE table", p + L.maxp);
  rows_layout(L, c->rowbuf, &c->rows, nullptr);
  if (la_build_rows_launch(L, c->out.back(), c->win[c->cur], c->wstride, c->cand, c->rows, c->st))
    return fail(c, LA_EOVERFLOW, "row builder: %d rows exceed its LDS tables", L.Q);
  c->lay = L;
  c->paused = paused;
  return LA_OK;
}

// The round's rows as one segment of a forward: the ordinary row's K/V go to
// the cache at p, the rest to the workspace; the prefix below p + 1 is shared.
static Seg round_seg(la_ctx* c, int r0, int l0) {
  const LaLayout& L = c->lay;
  const int p = c->kv_len;
  Seg g{};
  g.s = c; g.r0 = r0; g.M = L.Q; g.l0 = l0;
  g.tok = c->rows.tok; g.pos = c->rows.pos; g.branch = c->rows.branch; g.path = c->rows.path;
  g.path_len = c->rows.path_len; g.tile_meta = c->rows.tile_meta; g.tile_path = c->rows.tile_path;
  g.logit_rows = c->rows.logit_rows;
  g.nb = L.NB; g.maxp = L.maxp; g.n_direct = 1; g.cache_row0 = p; g.shared_end = p + 1;
  g.max_pos = p + L.maxp;                   // a row's branch path covers its own position
  g.n_logit = L.n_logit;
  return g;
}

static void round_predicted(la_ctx* c, const float* logits) {
  c->lg = logits;
  c->pending = true;
  c->verified = false;
  c->warm = !c->cfg.ar_only && is_warm(c);
}

extern "C" int la_predict(la_ctx* c, la_round_info* info) {
  if (!c) return fail(nullptr, LA_EINVAL, "null ctx");
  int rc = round_check(c);
  if (rc) return rc;
  bool uses_pool;
  if ((rc = round_lookup(c, &uses_pool))) return rc;
  if (uses_pool) HIPCHK(c, hipStreamSynchronize(c->st));
  int C;
  if ((rc = round_found(c, uses_pool, &C))) return rc;
  if ((rc = round_rows(c, C, false))) return rc;
  const Seg g = round_seg(c, 0, 0);
  if ((rc = forward_segs(c, own_bufs(c), &g, 1))) return rc;
  round_predicted(c, c->logits);
  if (info) {
    const LaLayout& L = c->lay;
    info->round_id = c->round_id + 1;
    info->p = c->kv_len; info->Q = L.Q; info->C = L.C; info->n_inp = L.n_inp; info->n_logit = L.n_logit;
    info->warm = c->warm ? 1 : 0;
    info->reserved = 0;
    info->logits = c->lg;
  }
  return LA_OK;
}

// Launch the verification of 1 + n_inp + C * S logit rows and start the copy
// of its result to the pinned host slot (read after a synchronisation).
static int verify_issue(la_ctx* c, const float* logits, int n_inp, const int32_t* cand_dev, int C, int32_t* zdev,
                        int32_t* z_host) {
  const int n_logit = 1 + n_inp + C * c->S;
  const int rid = c->round_id + 1;          // the draws of the round being decided
  la_argmax_launch(logits, n_logit, c->V, c->amax, c->st);
  if (c->cfg.verify_mode == LA_VERIFY_SAMPLE)
    la_sample_accept_launch(logits, c->V, n_inp, c->amax, cand_dev, C, c->S, c->hmax, c->cfg.temperature,
                            c->cfg.seed, rid, c->escr, c->acc, zdev, c->st);
  else
    la_greedy_accept_launch(c->amax, n_inp, cand_dev, C, c->S, c->hmax, c->acc, zdev, c->st);
  HIPCHK(c, hipGetLastError());
  HIPCHK(c, hipMemcpyAsync(c->acc_host, c->acc, sizeof(LaAcceptDev), hipMemcpyDeviceToHost, c->st));
  if (z_host && n_inp > 0) HIPCHK(c, hipMemcpyAsync(z_host, zdev, (size_t)n_inp * 4, hipMemcpyDeviceToHost, c->st));
  return LA_OK;
}

// The verification result, after the stream synchronisation.
static void verify_read(la_ctx* c, la_accept* out, bool own) {
  prof_collect(c);
  const LaAcceptDev& a = *c->acc_host;
  memset(out, 0, sizeof *out);
  out->round_id = c->round_id + 1;
  out->h = a.h;
  out->winner = a.winner;
  out->n_emit = a.n_emit;
  for (int i = 0; i < a.n_emit && i < LA_MAX_EMIT; ++i) out->emitted[i] = a.emitted[i];
  if (own) {
    c->vacc = *out;
    c->verified = true;
  }
}

extern "C" int la_verify(la_ctx* c, const float* logits, int32_t n_inp, const int32_t* cand, int32_t C, la_accept* out,
                         int32_t* z_host) {
  if (!c || !out) return fail(c, LA_EINVAL, "null ctx or output");
  const bool own = logits == nullptr;
  const int32_t* cand_dev;
  int32_t* zdev;
  if (own) {
    if (!c->pending) return fail(c, LA_ESTATE, "no predicted round to verify");
    logits = c->lg;
    n_inp = c->lay.n_inp;
    C = c->lay.C;
    cand_dev = c->cand;
    zdev = c->z;
  } else {
    if (C < 0 || C > 64 || n_inp < 0 || n_inp > c->wstride) return fail(c, LA_EINVAL, "bad C=%d or n_inp=%d", C, n_inp);
    if (C > 0 && !cand) return fail(c, LA_EINVAL, "null candidates");
    if (1 + n_inp + C * c->S > c->n_logit_max) return fail(c, LA_EOVERFLOW, "too many logit rows");
    if (C > 0)
      HIPCHK(c, hipMemcpyAsync(c->vcand, cand, (size_t)C * c->S * 4, hipMemcpyHostToDevice, c->st));
    cand_dev = c->vcand;
    zdev = c->z2;
  }
  int rc = verify_issue(c, logits, n_inp, cand_dev, C, zdev, z_host);
  if (rc) return rc;
  HIPCHK(c, hipStreamSynchronize(c->st));
  verify_read(c, out, own);
  return LA_OK;
}

extern "C" int la_commit(la_ctx* c, const la_accept* a) {
  if (!c || !a) return fail(c, LA_EINVAL, "null ctx or plan");
  if (!c->pending || !c->verified) return fail(c, LA_ESTATE, "no verified round pending");
  const int rid = c->round_id + 1;
  if (a->round_id != rid) return fail(c, LA_ESTATE, "plan for round %d, pending round is %d", a->round_id, rid);
  const LaLayout& L = c->lay;
  const int S = c->S;
  // --- validation: nothing below this block may fail before publication ---
  if (a->h < 0 || a->h > c->hmax) return fail(c, LA_EPLAN, "h=%d outside [0, %d]", a->h, c->hmax);
  if (a->n_emit != a->h + 1) return fail(c, LA_EPLAN, "n_emit=%d != h+1", a->n_emit);
  if (a->h > 0 && (a->winner < 0 || a->winner >= L.C)) return fail(c, LA_EPLAN, "winner %d not a candidate", a->winner);
  if (a->h == 0 && a->winner != -1) return fail(c, LA_EPLAN, "winner %d with h=0", a->winner);
  for (int k = 0; k < a->n_emit; ++k)
    if (a->emitted[k] < 0 || a->emitted[k] >= c->V) return fail(c, LA_EPLAN, "emitted token %d out of range", k);
  for (int k = 0; k < a->h; ++k)
    if (a->emitted[k] != c->cand_host[(size_t)a->winner * S + k])
      return fail(c, LA_EPLAN, "emitted[%d] is not the winner's suffix token", k);
  if (memcmp(a, &c->vacc, sizeof *a) != 0) return fail(c, LA_EPLAN, "plan differs from the verified result");
  if (c->kv_len + 1 + a->h > c->t_cap) return fail(c, LA_EOVERFLOW, "K/V capacity");
  // --- publication ---
  const int cand_start = L.Q - L.C * S;
  if (a->h > 0)
    la_kv_commit_launch(c->dtype, c->kc, c->vc, c->kw, c->vw, c->L, c->Hkv, c->dh, c->t_cap, c->ws_cap,
                        c->kv_len + 1, cand_start - 1 + a->winner * S, a->h, c->st);
  if (!c->cfg.ar_only && !c->paused) {
    if (c->warm && c->cfg.G > 0)
      la_pool_collect_launch(c->pool_cnt, c->pool_ent, c->out.back(), c->win[c->cur], c->wstride, c->R, c->cfg.W,
                             c->z, c->cfg.G, c->st);
    int nsz[LA_MAX_N];
    int deepest = 0;
    for (int r = 0; r < c->R; ++r) if (c->sizes[r] > 0) deepest = r;
    const bool warm = is_warm(c);
    for (int r = 0; r < c->R; ++r) nsz[r] = c->sizes[r];
    if (!warm) {
      for (int r = 0; r <= deepest; ++r) nsz[r] = c->sizes[r] - 1;
      nsz[deepest + 1] = c->sizes[deepest] - (deepest >= 1 ? 1 : 0);
    }
    // ALWAYS_FWD_ONE=False: the h accepted tokens move the live position h further
    const int shift = c->cfg.advance_by_accepted ? a->h : 0;
    la_window_next_launch(c->win[c->cur], c->win[c->cur ^ 1], c->wstride, c->R, c->sizes, nsz, deepest, warm ? 1 : 0,
                          c->z, L.n_inp, shift, a->emitted[a->n_emit - 1], c->st);
    HIPCHK(c, hipGetLastError());
    c->cur ^= 1;
    for (int r = 0; r < c->R; ++r) c->sizes[r] = nsz[r];
  }
  HIPCHK(c, hipGetLastError());
  c->kv_len += 1 + a->h;
  int added = 0;
  const int k0 = (int)c->out.size();
  for (int k = 0; k < a->n_emit && (int)c->out.size() < c->cfg.max_new; ++k, ++added) c->out.push_back(a->emitted[k]);
  // after the trajectory's n-grams, before the next round's lookup (a paused round leaves the pool
  // alone); past publication nothing returns an error -- a failed launch shows at the next call
  if (!c->paused) (void)insert_output_ngrams(c, k0);
  c->round_id = rid;
  c->pending = false;
  c->verified = false;
  c->stats.rounds += 1;
  c->stats.tokens += added;
  c->stats.candidates += L.C;
  c->stats.accepted += a->h;
  c->stats.paused += c->paused ? 1 : 0;
  c->paused = false;
  if (a->n_emit < LA_MAX_EMIT) c->stats.hist[a->n_emit] += 1;
  // the next round's lookup goes out now, so the host's way back to the
  // next la_predict overlaps it
  c->lk_key = -1;
  if (!c->cfg.ar_only && c->cfg.G > 0 && is_warm(c) && (int)c->out.size() < c->cfg.max_new)
    (void)start_lookup(c, c->out.back());   // published already; a failed start is retried by la_predict
  return LA_OK;
}

extern "C" int la_step(la_ctx* c, int32_t* out_tokens, int32_t cap, int32_t* n_out) {
  if (!c || !n_out) return fail(c, LA_EINVAL, "null argument");
  *n_out = 0;
  if ((int)c->out.size() >= c->cfg.max_new) return LA_OK;
  if (cap < c->cfg.N) return fail(c, LA_EOVERFLOW, "cap %d < N=%d", cap, c->cfg.N);
  const size_t before = c->out.size();
  int rc = la_predict(c, nullptr);
  if (rc) return rc;
  la_accept a;
  rc = la_verify(c, nullptr, 0, nullptr, 0, &a, nullptr);
  if (rc) { c->pending = false; return rc; }
  rc = la_commit(c, &a);
  if (rc) { c->pending = false; c->verified = false; return rc; }
  const size_t n = c->out.size() - before;
  if (out_tokens)
    for (size_t i = 0; i < n; ++i) out_tokens[i] = c->out[before + i];
  *n_out = (int32_t)n;
  return LA_OK;
}

extern "C" int la_generate(la_ctx* c, int32_t* out_tokens, int32_t cap, int32_t* n_out) {
  if (!c || !n_out) return fail(c, LA_EINVAL, "null argument");
  if (cap < c->cfg.max_new) return fail(c, LA_EOVERFLOW, "cap %d < max_new %d", cap, c->cfg.max_new);
  int32_t buf[LA_MAX_EMIT];
  while ((int)c->out.size() < c->cfg.max_new) {
    int32_t n = 0;
    int rc = la_step(c, buf, LA_MAX_EMIT, &n);
    if (rc) return rc;
  }
  for (size_t i = 0; i < c->out.size(); ++i) out_tokens[i] = c->out[i];
  *n_out = (int32_t)c->out.size();
  return LA_OK;
}

// ------------------------------------------------------------------ batch

// Several requests, one round each, in one stacked forward ("Speculative
// Decoding", Chapter 7 "Speculation Meets the Batch": concurrent requests
// share one read of the weights per step, and their speculation shares the
// compute left beside it; "M7.3", 0x03B: each request keeps its own pool,
// window and K/V).
// The per-request tables of a step (one entry per request, at most one per
// row): attention entries, then rotary-placement entries.
static size_t tab_bytes(int R) {
  return (size_t)R * sizeof(LaAttnSeg) + (size_t)R * sizeof(LaPostSeg);
}

struct la_batch {
  la_model_dims dims;
  la_model w;
  hipStream_t st;
  int max_rows;
  FwdBufs b;
  char* tab_dev = nullptr;     // the tables in the workspace
  char* tab_host = nullptr;    // pinned staging of the tables
  hipEvent_t tab_ev = nullptr; // recorded after the last upload: the staging is free once it completed
  std::vector<int32_t> base, found, cap, paused;
  ~la_batch() {
    // a step that failed after queuing its table upload may leave the copy in flight
    if (tab_ev) (void)hipEventSynchronize(tab_ev);
    if (tab_ev) (void)hipEventDestroy(tab_ev);
    if (tab_host) (void)hipHostFree(tab_host);
  }
};

static size_t carve_batch(const la_model_dims& d, int R, char* base, FwdBufs* B, char** tab = nullptr) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? (void*)(base + off) : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  const size_t e = d.dtype == LA_DTYPE_BF16 ? 2 : 4;
  const int dt = d.dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32;
  const int qd = d.n_heads * d.head_dim, qkvdim = (d.n_heads + 2 * d.n_kv_heads) * d.head_dim;
  FwdBufs b{};
  b.x = take((size_t)R * d.d_model * e);
  b.nrm = take((size_t)R * d.d_model * e);
  b.qkv = take((size_t)R * qkvdim * e);
  b.q = take((size_t)R * qd * e);
  b.o = take((size_t)R * qd * e);
  b.act = take((size_t)R * d.d_ff * e);
  b.fin = take((size_t)R * d.d_model * e);
  b.gemm_p = (float*)take(std::max<size_t>(partial_floats(dt, d.d_model, qkvdim, qd, d.d_ff, d.vocab, R, R), 1) * 4);
  b.logits = (float*)take((size_t)R * d.vocab * 4);
  char* t = (char*)take(tab_bytes(R));
  if (B) *B = b;
  if (tab) *tab = t;
  return off;
}

extern "C" uint64_t la_batch_bytes(const la_model_dims* dims, int32_t max_rows) {
  if (!dims || validate_dims(dims, nullptr) || max_rows < 1 || max_rows > LA_MAX_ROWS) return 0;
  return carve_batch(*dims, max_rows, nullptr, nullptr);
}

extern "C" int la_batch_init(const la_model_dims* dims, const la_model* weights, int32_t max_rows, void* workspace,
                             uint64_t bytes, void* stream, la_batch** out) {
  if (!out) return fail(nullptr, LA_EINVAL, "null batch output");
  *out = nullptr;
  if (!dims || !weights) return fail(nullptr, LA_EINVAL, "null dims or weights");
  int rc = validate_dims(dims, nullptr);
  if (rc) return rc;
  if (max_rows < 1 || max_rows > LA_MAX_ROWS)
    return fail(nullptr, LA_EINVAL, "max_rows %d outside [1, %d]", max_rows, LA_MAX_ROWS);
  if (!weights->packed || !weights->embed || !weights->final_norm || !weights->attn_norm || !weights->mlp_norm)
    return fail(nullptr, LA_EINVAL, "weights: packed projections (la_pack_weights), embed and norms are required");
  const size_t need = carve_batch(*dims, max_rows, nullptr, nullptr);
  if (!workspace || bytes < need)
    return fail(nullptr, LA_EOVERFLOW, "workspace of %llu bytes, %zu needed", (unsigned long long)bytes, need);
  la_batch* b = new la_batch();
  b->dims = *dims;
  b->w = *weights;
  b->st = (hipStream_t)stream;
  b->max_rows = max_rows;
  carve_batch(*dims, max_rows, (char*)workspace, &b->b, &b->tab_dev);
  if (hipHostMalloc((void**)&b->tab_host, tab_bytes(max_rows), hipHostMallocDefault) != hipSuccess ||
      hipEventCreateWithFlags(&b->tab_ev, hipEventDisableTiming) != hipSuccess) {
    delete b;
    return fail(nullptr, LA_EDEVICE, "batch tables: pinned staging or event");
  }
  *out = b;
  return LA_OK;
}

extern "C" void la_batch_destroy(la_batch* b) { delete b; }

// The occupancy throttle ("Speculative Decoding", Chapter 7: speculation
// spends only the part of the step's row budget that the batch's own rows
// leave free, per request, and is switched off when nothing is left).  Every
// active request (base > 0) first gets its own round's rows without
// candidates (base: its ordinary row plus its lookahead branch).  If that
// exceeds the budget, requests from the last one backwards run without their
// lookahead branch (one row each) until it fits.  The rest of the budget is
// dealt in S-row candidate blocks, one per request in turn (request order),
// among the requests that kept their branch, up to the candidates each found.
static int batch_plan(int n, int budget, int S, const int32_t* base, const int32_t* found, int32_t* cap,
                      int32_t* paused) {
  long rows = 0;
  int act = 0;
  for (int i = 0; i < n; ++i) {
    cap[i] = 0;
    paused[i] = 0;
    if (base[i] > 0) { ++act; rows += base[i]; }
  }
  if (act > budget) return fail(nullptr, LA_EOVERFLOW, "%d active requests exceed the row budget %d", act, budget);
  for (int i = n - 1; i >= 0 && rows > budget; --i)
    if (base[i] > 1) { rows -= base[i] - 1; paused[i] = 1; }
  for (bool more = true; more && rows + S <= budget;) {
    more = false;
    for (int i = 0; i < n && rows + S <= budget; ++i)
      if (base[i] > 0 && !paused[i] && cap[i] < found[i]) { ++cap[i]; rows += S; more = true; }
  }
  return LA_OK;
}

extern "C" int la_batch_plan(int32_t n, int32_t row_budget, int32_t S, const int32_t* base_rows, const int32_t* found,
                             int32_t* cap, int32_t* paused) {
  if (n < 0 || n > LA_MAX_ROWS || row_budget < 1 || S < 1 || S > LA_MAX_N - 1)
    return fail(nullptr, LA_EINVAL, "n=%d, row_budget=%d, S=%d out of range", n, row_budget, S);
  if (n > 0 && (!base_rows || !found || !cap || !paused)) return fail(nullptr, LA_EINVAL, "null array");
  for (int i = 0; i < n; ++i)
    if (base_rows[i] < 0 || found[i] < 0) return fail(nullptr, LA_EINVAL, "negative base_rows or found at %d", i);
  return batch_plan(n, row_budget, S, base_rows, found, cap, paused);
}

extern "C" int la_batch_step(la_batch* b, la_ctx* const* ctx, int32_t n, int32_t row_budget, int32_t* out_tokens,
                             int32_t* n_out, la_batch_round* rinfo) {
  if (!b || !ctx || !out_tokens || !n_out) return fail(nullptr, LA_EINVAL, "null argument");
  if (n < 1 || n > LA_MAX_ROWS) return fail(nullptr, LA_EINVAL, "n=%d outside [1, %d]", n, LA_MAX_ROWS);
  const int budget = row_budget <= 0 ? b->max_rows : row_budget;
  if (budget > b->max_rows) return fail(nullptr, LA_EINVAL, "row budget %d > max_rows %d", budget, b->max_rows);
  for (int i = 0; i < n; ++i) {
    la_ctx* c = ctx[i];
    if (!c) return fail(nullptr, LA_EINVAL, "null context %d", i);
    for (int j = 0; j < i; ++j)
      if (ctx[j] == c) return fail(nullptr, LA_EINVAL, "context %d appears twice", i);
    if (memcmp(&c->dims, &b->dims, sizeof b->dims) || c->w.packed != b->w.packed || c->w.embed != b->w.embed ||
        c->w.final_norm != b->w.final_norm || c->w.attn_norm != b->w.attn_norm || c->w.mlp_norm != b->w.mlp_norm)
      return fail(nullptr, LA_EINVAL, "context %d runs another model than the batch", i);
    if (c->st != b->st) return fail(nullptr, LA_EINVAL, "context %d runs on another stream than the batch", i);
    if (c->cfg.N != ctx[0]->cfg.N)
      return fail(nullptr, LA_EINVAL, "context %d has N=%d, context 0 N=%d: a batch shares N", i, c->cfg.N,
                  ctx[0]->cfg.N);
    n_out[i] = 0;
    if (rinfo) rinfo[i] = la_batch_round{};
  }
  b->base.assign(n, 0); b->found.assign(n, 0); b->cap.assign(n, 0); b->paused.assign(n, 0);
  std::vector<int> act;
  for (int i = 0; i < n; ++i) {
    la_ctx* c = ctx[i];
    if ((int)c->out.size() >= c->cfg.max_new) continue;
    int rc = round_check(c);
    if (rc) return rc;
    LaLayout L;
    if (round_layout(c, 0, false, &L)) return fail(c, LA_EINVAL, "inconsistent window layout");
    b->base[i] = L.Q;
    act.push_back(i);
  }
  if (act.empty()) return LA_OK;
  // the lookups (usually under way since the last commit), one synchronisation
  std::vector<char> uses(n, 0);
  bool any = false;
  for (int i : act) {
    bool u;
    int rc = round_lookup(ctx[i], &u);
    if (rc) return rc;
    uses[i] = u;
    any = any || u;
  }
  if (any) HIPCHK(nullptr, hipStreamSynchronize(b->st));
  for (int i : act) {
    int C, rc = round_found(ctx[i], uses[i], &C);
    if (rc) return rc;
    b->found[i] = C;
  }
  int rc = batch_plan(n, budget, ctx[act[0]]->S, b->base.data(), b->found.data(), b->cap.data(), b->paused.data());
  if (rc) return rc;
  // rows and segments
  std::vector<Seg> seg;
  int r0 = 0, l0 = 0;
  for (int i : act) {
    la_ctx* c = ctx[i];
    if ((rc = round_rows(c, b->cap[i], b->paused[i] != 0))) return rc;
    seg.push_back(round_seg(c, r0, l0));
    r0 += c->lay.Q;
    l0 += c->lay.n_logit;
  }
  if (r0 > b->max_rows) return fail(nullptr, LA_EOVERFLOW, "%d stacked rows > max_rows %d", r0, b->max_rows);
  la_ctx* lead = ctx[act[0]];
  // the per-request tables: built in the pinned staging (free once the last upload completed), one copy each
  const int ns = (int)seg.size();
  HIPCHK(nullptr, hipEventSynchronize(b->tab_ev));
  LaAttnSeg* ah = (LaAttnSeg*)b->tab_host;
  LaPostSeg* ph = (LaPostSeg*)(b->tab_host + (size_t)b->max_rows * sizeof(LaAttnSeg));
  for (int k = 0; k < ns; ++k) {
    const Seg& g = seg[k];
    la_ctx* s = g.s;
    const long long kvl = (long long)s->Hkv * s->t_cap * s->dh * s->esz;
    const long long wsl = (long long)s->Hkv * s->ws_cap * s->dh * s->esz;
    ah[k] = LaAttnSeg{};
    ah[k].a = seg_attn_args(lead, b->b, g, 0);
    ah[k].kv_layer = kvl;
    ah[k].ws_layer = wsl;
    ph[k] = LaPostSeg{g.pos, s->rope, s->kc, s->vc, s->kw, s->vw, kvl, wsl, g.r0, s->t_cap, g.cache_row0,
                      g.n_direct, s->ws_cap, 0};
  }
  SegTables tab{};
  if (la_attention_multi_plan(lead->dtype, ah, ns, &tab.shape))
    return fail(lead, LA_EINVAL, "attention of the stacked requests cannot be planned");
  tab.attn = (const LaAttnSeg*)b->tab_dev;
  tab.post = (const LaPostSeg*)(b->tab_dev + (size_t)b->max_rows * sizeof(LaAttnSeg));
  HIPCHK(nullptr, hipMemcpyAsync((void*)tab.attn, ah, ns * sizeof(LaAttnSeg), hipMemcpyHostToDevice, b->st));
  HIPCHK(nullptr, hipMemcpyAsync((void*)tab.post, ph, ns * sizeof(LaPostSeg), hipMemcpyHostToDevice, b->st));
  HIPCHK(nullptr, hipEventRecord(b->tab_ev, b->st));
  if ((rc = forward_segs(lead, b->b, seg.data(), ns, &tab))) return rc;
  for (size_t k = 0; k < act.size(); ++k) round_predicted(ctx[act[k]], b->b.logits + (size_t)seg[k].l0 * b->dims.vocab);
  auto unwind = [&]() {
    for (int i : act) { ctx[i]->pending = false; ctx[i]->verified = false; }
  };
  for (int i : act) {
    la_ctx* c = ctx[i];
    if ((rc = verify_issue(c, c->lg, c->lay.n_inp, c->cand, c->lay.C, c->z, nullptr))) { unwind(); return rc; }
  }
  if (hipError_t e = hipStreamSynchronize(b->st); e != hipSuccess) {
    unwind();
    return fail(nullptr, LA_EDEVICE, "hipStreamSynchronize: %s", hipGetErrorString(e));
  }
  // publication, request by request (a failure leaves the requests before it published)
  for (int i : act) {
    la_ctx* c = ctx[i];
    la_accept a;
    verify_read(c, &a, true);
    if (rinfo) {
      rinfo[i].Q = c->lay.Q;
      rinfo[i].found = b->found[i];
      rinfo[i].verified = c->lay.C;
      rinfo[i].paused = b->paused[i];
      rinfo[i].h = a.h;
    }
    const size_t before = c->out.size();
    if ((rc = la_commit(c, &a))) {
      for (int j : act) if (ctx[j]->pending) { ctx[j]->pending = false; ctx[j]->verified = false; }
      return rc;
    }
    const size_t k = c->out.size() - before;
    for (size_t t = 0; t < k; ++t) out_tokens[(size_t)i * LA_MAX_EMIT + t] = c->out[before + t];
    n_out[i] = (int32_t)k;
  }
  return LA_OK;
}

// ------------------------------------------------------------------ pool, state

extern "C" int la_pool_lookup(la_ctx* c, int32_t key, int32_t* out, int32_t* n) {
  if (!c || !out || !n) return fail(c, LA_EINVAL, "null argument");
  if (key < 0 || key >= c->V) return fail(c, LA_EINVAL, "key %d out of range", key);
  if (c->cfg.G == 0) { *n = 0; return LA_OK; }
  la_pool_lookup_launch(c->pool_cnt, c->pool_ent, key, c->cfg.G, c->S, c->vcand, c->ncand, c->st);
  int32_t nc = 0;
  HIPCHK(c, hipMemcpyAsync(&nc, c->ncand, 4, hipMemcpyDeviceToHost, c->st));
  HIPCHK(c, hipStreamSynchronize(c->st));
  if (nc > 0) {
    HIPCHK(c, hipMemcpyAsync(out, c->vcand, (size_t)nc * c->S * 4, hipMemcpyDeviceToHost, c->st));
    HIPCHK(c, hipStreamSynchronize(c->st));
  }
  *n = nc;
  return LA_OK;
}

extern "C" int la_pool_insert(la_ctx* c, const int32_t* keys, const int32_t* suffixes, int32_t n) {
  if (c) c->lk_key = -1;   // a lookup started by the last commit no longer sees the pool as it will be
  if (!c || (n > 0 && (!keys || !suffixes))) return fail(c, LA_EINVAL, "null argument");
  if (n < 0 || n > 64) return fail(c, LA_EINVAL, "n=%d outside [0, 64] per call", n);
  if (c->pending) return fail(c, LA_ESTATE, "a predicted round is pending");
  if (c->cfg.G == 0 || n == 0) return LA_OK;
  for (int i = 0; i < n; ++i) {
    if (keys[i] < 0 || keys[i] >= c->V) return fail(c, LA_EINVAL, "key %d out of range", i);
    for (int s = 0; s < c->S; ++s)
      if (suffixes[i * c->S + s] < 0 || suffixes[i * c->S + s] >= c->V) return fail(c, LA_EINVAL, "suffix token out of range");
  }
  // keys then suffixes through the verification candidate scratch
  std::vector<int32_t> buf((size_t)n * (1 + c->S));
  for (int i = 0; i < n; ++i) buf[i] = keys[i];
  memcpy(buf.data() + n, suffixes, (size_t)n * c->S * 4);
  HIPCHK(c, hipMemcpyAsync(c->vcand, buf.data(), buf.size() * 4, hipMemcpyHostToDevice, c->st));
  la_pool_upsert_launch(c->pool_cnt, c->pool_ent, c->vcand, c->vcand + n, n, c->cfg.G, c->S, c->st);
  HIPCHK(c, hipGetLastError());
  HIPCHK(c, hipStreamSynchronize(c->st));
  return LA_OK;
}

extern "C" int la_get_state(la_ctx* c, la_state_t* s, int32_t* window, int32_t* output, int32_t out_cap) {
  if (!c || !s) return fail(c, LA_EINVAL, "null argument");
  memset(s, 0, sizeof *s);
  s->round_id = c->round_id;
  s->kv_len = c->kv_len;
  s->n_out = (int32_t)c->out.size();
  s->R = c->R;
  for (int r = 0; r < c->R; ++r) s->level_sizes[r] = c->sizes[r];
  s->warm = is_warm(c) ? 1 : 0;
  s->win_stride = c->wstride;
  if (window) {
    HIPCHK(c, hipMemcpyAsync(window, c->win[c->cur], (size_t)c->R * c->wstride * 4, hipMemcpyDeviceToHost, c->st));
    HIPCHK(c, hipStreamSynchronize(c->st));
  }
  if (output)
    for (int i = 0; i < (int)c->out.size() && i < out_cap; ++i) output[i] = c->out[i];
  return LA_OK;
}

extern "C" int la_stats(const la_ctx* c, la_stats_t* out) {
  if (!c || !out) return LA_EINVAL;
  *out = c->stats;
  return LA_OK;
}

extern "C" const char* la_last_error(const la_ctx* c) { return c ? c->err.c_str() : g_err.c_str(); }

// ------------------------------------------------------------------ context-free operators

static int desc_layout(const la_rows_desc* d, LaLayout* L) {
  if (!d || d->R < 1 || d->R > LA_MAX_N || d->S < 1 || d->S > LA_MAX_N || d->C < 0 || d->C > 64)
    return fail(nullptr, LA_EINVAL, "bad rows descriptor");
  memset(L, 0, sizeof *L);
  L->p = d->p; L->R = d->R; L->C = d->C; L->S = d->S;
  for (int r = 0; r < d->R; ++r) {
    if (d->sizes[r] < 0 || (r > 0 && d->sizes[r] > 0 && d->sizes[r] > d->win_stride) || d->sizes[0] > d->win_stride)
      return fail(nullptr, LA_EINVAL, "level %d size %d", r, d->sizes[r]);
    L->sizes[r] = d->sizes[r];
    L->starts[r] = r == 0 ? 1 : d->starts[r];
  }
  if (la_layout_finish(L)) return fail(nullptr, LA_EINVAL, "inconsistent level layout");
  if (L->Q > 1024) return fail(nullptr, LA_EINVAL, "too many rows");
  return LA_OK;
}

extern "C" int la_rows_query(const la_rows_desc* desc, la_rows_info* info) {
  LaLayout L;
  int rc = desc_layout(desc, &L);
  if (rc) return rc;
  if (!info) return fail(nullptr, LA_EINVAL, "null info");
  rows_layout(L, nullptr, nullptr, info);
  return LA_OK;
}

extern "C" int la_build_rows(const la_rows_desc* desc, const int32_t* window, const int32_t* cand, int32_t* out,
                             void* stream, la_rows_info* info) {
  LaLayout L;
  int rc = desc_layout(desc, &L);
  if (rc) return rc;
  if (!out || !window || (L.C > 0 && !cand) || !info) return fail(nullptr, LA_EINVAL, "null argument");
  LaRowsDev r;
  rows_layout(L, out, &r, info);
  if (la_build_rows_launch(L, desc->x_t, window, desc->win_stride, cand, r, (hipStream_t)stream))
    return fail(nullptr, LA_EOVERFLOW, "row builder: %d rows exceed its LDS tables", L.Q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(nullptr, LA_EDEVICE, "build rows: %s", hipGetErrorString(e));
  return LA_OK;
}

extern "C" size_t la_attention_workspace(int32_t Q, int32_t H, int32_t dh, int32_t max_pos, int32_t t_cap) {
  const size_t parts = (size_t)la_attention_parts(max_pos, t_cap);
  return parts * H * Q * ((size_t)dh + 2) * 4 + 512;
}

// Argument checks and launch shared by la_attention and la_attention_noalloc.
static int attention_call(int32_t dtype, const void* q, const void* k_cache, const void* v_cache, int32_t t_cap,
                          const void* k_ws, const void* v_ws, int32_t ws_cap, int32_t H, int32_t Hkv, int32_t dh,
                          const int32_t* rows, const la_rows_info* info, int32_t shared_end, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !rows || !info || !out || !workspace) return fail(nullptr, LA_EINVAL, "null argument");
  if (dtype != LA_DTYPE_F32 && dtype != LA_DTYPE_BF16) return fail(nullptr, LA_EINVAL, "dtype");
  if (H < 1 || Hkv < 1 || H % Hkv || shared_end < 1 || shared_end > t_cap) return fail(nullptr, LA_EINVAL, "bad shape");
  if (info->Q > 1 && (!k_ws || !v_ws || ws_cap < info->Q - 1)) return fail(nullptr, LA_EINVAL, "workspace K/V too small");
  // positions never exceed shared_end + maxp (a row's path covers its own position)
  const int max_pos = shared_end - 1 + info->maxp;
  const size_t need = la_attention_workspace(info->Q, H, dh, max_pos, t_cap);
  if (workspace_bytes < need) return fail(nullptr, LA_EOVERFLOW, "workspace %zu < %zu bytes", workspace_bytes, need);
  LaAttnArgs a{};
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.kw = k_ws ? k_ws : k_cache; a.vw = v_ws ? v_ws : v_cache; a.o = out;
  const size_t parts = (size_t)la_attention_parts(max_pos, t_cap);
  a.max_splits = (int)parts;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + parts * H * info->Q * (size_t)dh * 4);
  a.pos = rows + info->off_pos; a.branch = rows + info->off_branch; a.path = rows + info->off_path;
  a.path_len = rows + info->off_path_len;
  a.tile_meta = rows + info->off_tile_meta; a.tile_path = rows + info->off_tile_path;
  a.Q = info->Q; a.H = H; a.Hkv = Hkv; a.dh = dh; a.T_cap = t_cap; a.ws_cap = ws_cap > 0 ? ws_cap : 1;
  a.maxp = info->maxp; a.shared_end = shared_end;
  a.max_pos = max_pos; a.nb = info->NB; a.n_ws = info->Q - 1;
  a.scale = 1.0f / sqrtf((float)dh);
  const int rc = la_attention_launch(dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32, a, (hipStream_t)stream);
  if (rc) return fail(nullptr, rc == -2 ? LA_EINVAL : LA_EDEVICE, "attention launch failed");
  return LA_OK;
}

extern "C" int la_attention(int32_t dtype, const void* q, const void* k_cache, const void* v_cache, int32_t t_cap,
                            const void* k_ws, const void* v_ws, int32_t ws_cap, int32_t H, int32_t Hkv, int32_t dh,
                            const int32_t* rows, const la_rows_info* info, int32_t shared_end, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return attention_call(dtype, q, k_cache, v_cache, t_cap, k_ws, v_ws, ws_cap, H, Hkv, dh, rows, info, shared_end,
                        out, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------------ allocation-free attention
//
// la_attention_noalloc keeps the key splits' softmax states in this
// file-scope device array instead of a caller workspace.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// symbol): its device address is taken once per device with
// hipGetSymbolAddress, with that device current, and kept in g_scratch.
static __device__ __align__(256) char scratch[LA_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch[LA_MAX_DEVICES];

// Device address of `scratch` on the current device (taken on the first call per device).
static int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, LA_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= LA_MAX_DEVICES) return fail(nullptr, LA_EDEVICE, "device %d beyond %d", dev, LA_MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(nullptr, LA_EDEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LA_OK;
}

extern "C" int la_attention_noalloc(int32_t dtype, const void* q, const void* k_cache, const void* v_cache,
                                    int32_t t_cap, const void* k_ws, const void* v_ws, int32_t ws_cap, int32_t H,
                                    int32_t Hkv, int32_t dh, const int32_t* rows, const la_rows_info* info,
                                    int32_t shared_end, void* out, void* stream) {
  if (!info) return fail(nullptr, LA_EINVAL, "null argument");
  if (H < 1 || dh < 1 || shared_end < 1 || shared_end > t_cap) return fail(nullptr, LA_EINVAL, "bad shape");
  const size_t need = la_attention_workspace(info->Q, H, dh, shared_end - 1 + info->maxp, t_cap);
  if (need > LA_NOALLOC_SCRATCH_BYTES)
    return fail(nullptr, LA_EOVERFLOW, "this call needs %zu bytes of split state, beyond the %u the allocation-free "
                "entry point holds; use la_attention with a workspace", need, (unsigned)LA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const int rc = scratch_ptr(&ws);
  if (rc) return rc;
  return attention_call(dtype, q, k_cache, v_cache, t_cap, k_ws, v_ws, ws_cap, H, Hkv, dh, rows, info, shared_end,
                        out, ws, LA_NOALLOC_SCRATCH_BYTES, stream);
}

static int linear_epi(int32_t epilogue) {
  return epilogue == LA_LINEAR_STORE ? LA_EPI_STORE : epilogue == LA_LINEAR_RESIDUAL ? LA_EPI_RESID
         : epilogue == LA_LINEAR_SWIGLU ? LA_EPI_SWIGLU : LA_EPI_F32;
}
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

extern "C" size_t la_packed_linear_bytes(int32_t dtype, int32_t epilogue, int32_t N, int32_t K) {
  if (N <= 0 || K <= 0) return 0;
  return la_gemm_packed_elems(dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32, N, K, epilogue == LA_LINEAR_SWIGLU) *
         (dtype == LA_DTYPE_BF16 ? 2 : 4);
}

extern "C" size_t la_linear_workspace(int32_t dtype, int32_t epilogue, int32_t M, int32_t N, int32_t K) {
  const int dt = dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32;
  const int sw = epilogue == LA_LINEAR_SWIGLU;
  const int splits = la_gemm_splits(N, K, dt, sw);
  const size_t part = splits > 1 ? (size_t)splits * M * (sw ? 2 * N : N) * 4 : 0;
  return align256(la_packed_linear_bytes(dtype, epilogue, N, K)) + part;
}

static int linear_check(int32_t dtype, int32_t epilogue, const void* X, const void* W, const void* Y, const void* R) {
  if (!X || !W || !Y || (epilogue == LA_LINEAR_RESIDUAL && !R)) return fail(nullptr, LA_EINVAL, "null argument");
  if (dtype != LA_DTYPE_F32 && dtype != LA_DTYPE_BF16) return fail(nullptr, LA_EINVAL, "dtype");
  if (epilogue < LA_LINEAR_STORE || epilogue > LA_LINEAR_F32) return fail(nullptr, LA_EINVAL, "epilogue");
  return LA_OK;
}

extern "C" int la_pack_linear(int32_t dtype, int32_t epilogue, const void* W, int32_t N, int32_t K, void* Wp,
                              void* stream) {
  if (!W || !Wp) return fail(nullptr, LA_EINVAL, "null argument");
  if (dtype != LA_DTYPE_F32 && dtype != LA_DTYPE_BF16) return fail(nullptr, LA_EINVAL, "dtype");
  if (epilogue < LA_LINEAR_STORE || epilogue > LA_LINEAR_F32) return fail(nullptr, LA_EINVAL, "epilogue");
  const int rc = la_gemm_pack_launch(dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32, W, Wp, N, K,
                                     epilogue == LA_LINEAR_SWIGLU, (hipStream_t)stream);
  if (rc == -2) return fail(nullptr, LA_EINVAL, "unsupported shape N=%d K=%d", N, K);
  if (rc) return fail(nullptr, LA_EDEVICE, "pack launch failed");
  return LA_OK;
}

extern "C" int la_linear_packed(int32_t dtype, int32_t epilogue, const void* X, const void* Wp, void* Y,
                                const void* R, int32_t M, int32_t N, int32_t K, void* workspace,
                                size_t workspace_bytes, void* stream) {
  int rc = linear_check(dtype, epilogue, X, Wp, Y, R);
  if (rc) return rc;
  const size_t need = la_linear_workspace(dtype, epilogue, M, N, K);
  const size_t skip = align256(la_packed_linear_bytes(dtype, epilogue, N, K));
  if (need > skip && (!workspace || workspace_bytes < need))
    return fail(nullptr, LA_EOVERFLOW, "workspace %zu < %zu bytes", workspace_bytes, need);
  const int dt = dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32;
  const int epi = linear_epi(epilogue);
  LaGemmArgs a{};
  a.X = X; a.W = Wp; a.Y = Y; a.R = R; a.P = need > skip ? (float*)((char*)workspace + skip) : nullptr;
  a.M = M; a.N = N; a.K = K; a.ldx = K; a.ldy = N;
  a.splits = la_gemm_splits(N, K, dt, epi == LA_EPI_SWIGLU);
  a.up_off = N;
  a.pcols = epi == LA_EPI_SWIGLU ? 2 * N : N;
  rc = la_gemm_launch(dt, epi, a, (hipStream_t)stream);
  if (rc == -2) return fail(nullptr, LA_EINVAL, "unsupported shape M=%d N=%d K=%d", M, N, K);
  if (rc) return fail(nullptr, LA_EDEVICE, "linear launch failed");
  return LA_OK;
}

extern "C" int la_linear(int32_t dtype, int32_t epilogue, const void* X, const void* W, void* Y, const void* R,
                         int32_t M, int32_t N, int32_t K, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = linear_check(dtype, epilogue, X, W, Y, R);
  if (rc) return rc;
  const size_t need = la_linear_workspace(dtype, epilogue, M, N, K);
  if (!workspace || workspace_bytes < need)
    return fail(nullptr, LA_EOVERFLOW, "workspace %zu < %zu bytes", workspace_bytes, need);
  if ((rc = la_pack_linear(dtype, epilogue, W, N, K, workspace, stream))) return rc;
  return la_linear_packed(dtype, epilogue, X, workspace, Y, R, M, N, K, workspace, workspace_bytes, stream);
}

extern "C" uint64_t la_packed_weight_bytes(const la_model_dims* dims) {
  if (!dims || dims->n_layers < 1) return 0;
  return (uint64_t)packed_offsets(*dims).total * (dims->dtype == LA_DTYPE_BF16 ? 2 : 4);
}

extern "C" int la_pack_weights(const la_model_dims* dims, const la_model* plain, void* packed, void* stream) {
  if (!dims || !plain || !packed) return fail(nullptr, LA_EINVAL, "null argument");
  la_config probe{};
  probe.W = 1; probe.N = 3; probe.max_new = 1; probe.max_prompt = 1;
  int rc = validate_cfg(&probe, dims, nullptr);
  if (rc) return rc;
  if (!plain->wqkv || !plain->wo || !plain->w_gate_up || !plain->w_down || !plain->lm_head)
    return fail(nullptr, LA_EINVAL, "null projection weights");
  const PackedOffsets pk = packed_offsets(*dims);
  const int dt = dims->dtype == LA_DTYPE_BF16 ? LA_DT_BF16 : LA_DT_F32;
  const size_t esz = dims->dtype == LA_DTYPE_BF16 ? 2 : 4;
  const int d = dims->d_model, F = dims->d_ff, hd = dims->n_heads * dims->head_dim;
  const int qkvdim = (dims->n_heads + 2 * dims->n_kv_heads) * dims->head_dim;
  hipStream_t st = (hipStream_t)stream;
  char* out = (char*)packed;
  for (int l = 0; l < dims->n_layers; ++l) {
    char* pl = out + pk.layer * l * esz;
    rc = la_gemm_pack_launch(dt, (const char*)plain->wqkv + (size_t)l * qkvdim * d * esz, pl + pk.qkv * esz, qkvdim,
                             d, 0, st, qkv_fused(qkvdim, d, dt, dims->head_dim) ? dims->head_dim : 0);
    rc = rc ? rc : la_gemm_pack_launch(dt, (const char*)plain->wo + (size_t)l * d * hd * esz, pl + pk.o * esz, d, hd,
                                       0, st);
    rc = rc ? rc : la_gemm_pack_launch(dt, (const char*)plain->w_gate_up + (size_t)l * 2 * F * d * esz,
                                       pl + pk.gu * esz, F, d, 1, st);
    rc = rc ? rc : la_gemm_pack_launch(dt, (const char*)plain->w_down + (size_t)l * d * F * esz, pl + pk.dn * esz, d,
                                       F, 0, st);
    if (rc) return fail(nullptr, rc == -2 ? LA_EINVAL : LA_EDEVICE, "pack launch failed (layer %d)", l);
  }
  rc = la_gemm_pack_launch(dt, plain->lm_head, out + pk.lm * esz, dims->vocab, d, 0, st);
  if (rc) return fail(nullptr, rc == -2 ? LA_EINVAL : LA_EDEVICE, "pack launch failed (lm_head)");
  return LA_OK;
}
