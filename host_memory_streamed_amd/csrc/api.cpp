// C ABI: context creation (host store and device workspace), parameter
// access, statistics and the schedule trace.
//
// Host store ("MegaTrain: Full Precision Training of 100B+ Parameter LLMs on a
// Single GPU", abstract: parameters and optimizer states live in host memory;
// "Technical Brief: MegaTrain's Single-GPU 120B-Parameter Training
// Breakthrough", section "Core Architecture": host RAM is the warehouse of
// persistent state, GPU memory a constantly refilled cache). Per unit: fp32
// master p, AdamW m and v, the unit's device image (bf16 mode: a pinned bf16
// shadow with fp32 gains; fp32 mode: p itself, pinned), and gradients when
// they are kept. Device memory holds only the layer buffers, two gradient
// buffers, the residual checkpoints and one layer's activations: its size does
// not grow with depth apart from the checkpoints.
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.h"
#include "runtime.h"

namespace mt {

struct StepEvents;
int create_step_events(Ctx& c, StepEvents*& out);
void destroy_step_events(StepEvents* e);
int train_step_impl(Ctx& c, StepEvents& E, const int32_t* tokens, const int32_t* targets, int B,
                     int T, float* loss_out);
int default_threads(int requested);

static thread_local std::string g_create_error;

int set_error(Ctx* c, int code, const std::string& msg) {
  if (c)
    c->err = msg;
  else
    g_create_error = msg;
  return code;
}

static Dims make_dims(const mt_model_cfg& c) {
  Dims D;
  D.L = c.n_layers;
  D.d = c.d_model;
  D.H = c.n_heads;
  D.Hkv = c.n_kv_heads;
  D.hd = c.head_dim;
  D.F = c.ffn_dim;
  D.V = c.vocab;
  D.qd = D.H * D.hd;
  D.kvd = D.Hkv * D.hd;
  D.qkvd = D.qd + 2 * D.kvd;
  return D;
}

static UnitLayout layer_layout(const Dims& D) {
  UnitLayout u;
  const int64_t d = D.d;
  u.off.resize(6);
  u.off[0] = 0;
  u.off[1] = d;
  u.mat_base = align_up(2 * d, kAlign);
  u.off[2] = u.mat_base;                                   // wq | wk | wv
  u.off[3] = align_up(u.off[2] + (int64_t)D.qkvd * d, kAlign);   // wo
  u.off[4] = align_up(u.off[3] + d * D.qd, kAlign);         // w_gate | w_up
  u.off[5] = align_up(u.off[4] + 2 * (int64_t)D.F * d, kAlign);  // w_down
  u.n = align_up(u.off[5] + d * D.F, kAlign);
  return u;
}

static UnitLayout head_layout(const Dims& D) {
  UnitLayout u;
  u.off = {0, align_up(D.d, kAlign)};
  u.mat_base = u.off[1];
  u.n = align_up(u.off[1] + (int64_t)D.V * D.d, kAlign);
  return u;
}

static UnitLayout emb_layout(const Dims& D) {
  UnitLayout u;
  u.off = {0};
  u.n = (int64_t)D.V * D.d;
  u.mat_base = u.n;   // never imaged
  return u;
}

static std::vector<TensorRef> tensor_table(const Dims& D) {
  std::vector<TensorRef> t;
  const UnitLayout ll = layer_layout(D), hl = head_layout(D);
  const int64_t d = D.d;
  t.push_back({-1, 0, (int64_t)D.V * d, D.V, d, "tok_emb"});
  for (int l = 0; l < D.L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    t.push_back({l, ll.off[0], d, d, 1, p + "attn_norm"});
    t.push_back({l, ll.off[2], (int64_t)D.qd * d, D.qd, d, p + "wq"});
    t.push_back({l, ll.off[2] + (int64_t)D.qd * d, (int64_t)D.kvd * d, D.kvd, d, p + "wk"});
    t.push_back({l, ll.off[2] + (int64_t)(D.qd + D.kvd) * d, (int64_t)D.kvd * d, D.kvd, d, p + "wv"});
    t.push_back({l, ll.off[3], d * D.qd, d, D.qd, p + "wo"});
    t.push_back({l, ll.off[1], d, d, 1, p + "mlp_norm"});
    t.push_back({l, ll.off[4], (int64_t)D.F * d, D.F, d, p + "w_gate"});
    t.push_back({l, ll.off[4] + (int64_t)D.F * d, (int64_t)D.F * d, D.F, d, p + "w_up"});
    t.push_back({l, ll.off[5], d * D.F, d, D.F, p + "w_down"});
  }
  t.push_back({D.L, hl.off[0], d, d, 1, "final_norm"});
  t.push_back({D.L, hl.off[1], (int64_t)D.V * d, D.V, d, "lm_head"});
  return t;
}

// Element counts of the pinned gradient staging slots (MT_KEEP_GRADS off).
// Synchronous updates keep up with the gradients: three slots that fit any
// unit. Overlapped updates fall behind during the backward and catch up in
// the next forward: layer-sized slots for as many layers as fit in 16 GiB (3
// to 16), plus one slot kept for the head (the last entry).
// cfg.grad_ring_slots > 0 sets the count (of layer slots, with MT_OVERLAP_OPT).
static std::vector<int64_t> ring_sizes(const mt_model_cfg& cfg, int64_t layer_n, int64_t head_n) {
  std::vector<int64_t> sizes;
  const int k = cfg.grad_ring_slots;
  if (cfg.flags & MT_OVERLAP_OPT) {
    const int r = k > 0 ? k : (int)std::max<int64_t>(3, std::min<int64_t>(16, (16LL << 30) / (layer_n * 4)));
    sizes.assign(r, layer_n);
    sizes.push_back(head_n);
  } else {
    sizes.assign(k > 0 ? k : 3, std::max(layer_n, head_n));
  }
  return sizes;
}

// Gradients pass through the pinned staging slots unless they are kept in
// fp32 host buffers as they come (MT_KEEP_GRADS without MT_BF16_GRADS).
static bool staged_grads(const mt_model_cfg& c) {
  return !(c.flags & MT_KEEP_GRADS) || (c.flags & MT_BF16_GRADS);
}
static int64_t grad_bytes(const mt_model_cfg& c) { return (c.flags & MT_BF16_GRADS) ? 2 : 4; }

static int validate(const mt_model_cfg* c, std::string& why) {
  if (!c) { why = "cfg is NULL"; return MT_EINVAL; }
  auto bad = [&](const char* m) { why = m; return MT_EINVAL; };
  if (c->n_layers < 1) return bad("n_layers must be >= 1");
  if (c->d_model < 4 || c->d_model % 4) return bad("d_model must be a positive multiple of 4");
  if (c->d_model > 16384) return bad("d_model must be <= 16384");
  if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
    return bad("n_kv_heads must divide n_heads");
  if (c->compute_dtype != MT_FP32 && c->compute_dtype != MT_BF16) return bad("compute_dtype must be MT_FP32 or MT_BF16");
  if (!attn_supported(c->compute_dtype, c->head_dim))
    return bad("head_dim must be 16/32/64/128 (fp32) or 64/128 (bf16)");
  if (c->ffn_dim < 1 || c->vocab < 2) return bad("ffn_dim and vocab must be positive");
  if (c->max_batch < 1 || c->max_seq < 1) return bad("max_batch and max_seq must be >= 1");
  if ((int64_t)c->max_batch * c->max_seq >= MAX_BLOCK_ROWS) return bad("max_batch * max_seq must be < 2^24 tokens");
  if ((int64_t)(c->n_heads + 2 * c->n_kv_heads) * c->head_dim >= MAX_ATTN_LD)
    return bad("(n_heads + 2 n_kv_heads) * head_dim must be < 2^24");
  if (c->n_layer_buffers < 2) return bad("n_layer_buffers must be >= 2");
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f) || !(c->lr >= 0.0) || !(c->beta1 >= 0.0 && c->beta1 < 1.0) ||
      !(c->beta2 >= 0.0 && c->beta2 < 1.0) || !(c->adam_eps >= 0.0))
    return bad("invalid eps / rope_base / AdamW hyperparameters");
  if (c->flags & ~(MT_KEEP_GRADS | MT_KERNEL_TIMING | MT_TRACE | MT_OVERLAP_OPT | MT_PROGRESS | MT_CACHE_NO_REFRESH |
                   MT_BF16_GRADS))
    return bad("unknown flags");
  if (c->chunk_rows < 0) return bad("chunk_rows must be >= 0");
  if (c->ckpt_host < 0 || (c->ckpt_host > 0 && c->ckpt_host > c->n_layers - 2))
    return bad("ckpt_host must be 0 or in [1, n_layers - 2]");
  if (c->grad_ring_slots < 0 || c->grad_ring_slots > 64) return bad("grad_ring_slots must be in [0, 64]");
  if (c->wait_timeout_ms < 0) return bad("wait_timeout_ms must be >= 0");
  if (c->micro_batches < 0 || c->micro_batches > c->max_batch) return bad("micro_batches must be in [0, max_batch]");
  return MT_OK;
}

void adam_drain(Ctx& c) {
  std::unique_lock<std::mutex> lk(c.amu);
  c.acv.wait(lk, [&] { return c.adam_pending == 0; });
}

int adam_drain_for(Ctx& c, int64_t ms, const char* what) {
  if (ms <= 0) {
    adam_drain(c);
    return MT_OK;
  }
  std::string busy;
  {
    std::unique_lock<std::mutex> lk(c.amu);
    if (c.acv.wait_for(lk, std::chrono::milliseconds(ms), [&] { return c.adam_pending == 0; })) return MT_OK;
    const int L = c.D.L;
    for (int u = 0; u < (int)c.unit_busy.size(); ++u)
      if (c.unit_busy[u])
        busy += (busy.empty() ? "" : ", ") +
                (u < L ? "layer " + std::to_string(u) : u == L ? std::string("head") : std::string("embedding"));
  }
  return set_error(&c, MT_ETIMEOUT, std::string(what) + ": AdamW updates still running after " +
                                        std::to_string(ms) + " ms (" + busy + ")");
}

static int64_t env_int(const char* name) {
  const char* v = std::getenv(name);
  return v ? std::max<int64_t>(0, std::strtoll(v, nullptr, 10)) : 0;
}

static void free_ctx(Ctx* c) {
  if (!c) return;
  adam_drain(*c);   // no update may still be reading host memory
  if (c->s_comp) hipStreamSynchronize(c->s_comp);
  if (c->s_in) hipStreamSynchronize(c->s_in);
  if (c->s_out) hipStreamSynchronize(c->s_out);
  for (auto& u : c->units) {
    if (u.p) { if (u.p_pinned) hipHostFree(u.p); else host_free_plain(u.p, (size_t)u.lay.n * 4); }
    host_free_plain(u.m, (size_t)u.lay.n * 4);
    host_free_plain(u.v, (size_t)u.lay.n * 4);
    if (u.g) {
      if (&u == &c->units.back()) host_free_plain(u.g, (size_t)u.lay.n * 4);
      else hipHostFree(u.g);
    }
    if (u.shadow) hipHostFree(u.shadow);
  }
  for (auto* p : c->ring_slot) hipHostFree(p);
  for (auto* p : c->ck_host) host_free_plain(p, (size_t)c->M_max * c->D.d * 4);
  for (auto* p : c->bounce)
    if (p) hipHostFree(p);
  for (void* p : {(void*)c->x0_host, (void*)c->tgt_host, (void*)c->loss_host})
    if (p) hipHostFree(p);
  for (void* p : c->dev_allocs) hipFree(p);
  for (auto e : c->kt.ev) hipEventDestroy(e);
  for (int i = 0; i < 3; ++i) {
    hipStream_t s = i == 0 ? c->s_in : i == 1 ? c->s_comp : c->s_out;
    if (s && c->own_streams[i]) hipStreamDestroy(s);
  }
  delete c->pool;
  c->pool = nullptr;
}

}  // namespace mt

using namespace mt;

struct mt_ctx {
  Ctx c;
  StepEvents* ev = nullptr;
};

extern "C" {

int32_t mt_tensor_count(const mt_model_cfg* cfg) { return cfg ? 9 * cfg->n_layers + 3 : 0; }

int mt_tensor_info(const mt_model_cfg* cfg, int32_t id, char* name, int32_t name_cap, int64_t shape[2],
                   int32_t* ndim) {
  if (!cfg || cfg->n_layers < 1 || id < 0 || id >= mt_tensor_count(cfg)) return MT_EINVAL;
  const Dims D = make_dims(*cfg);
  const auto t = tensor_table(D);
  const TensorRef& r = t[id];
  if (name && name_cap > 0) snprintf(name, (size_t)name_cap, "%s", r.name.c_str());
  if (shape) { shape[0] = r.rows; shape[1] = r.cols; }
  if (ndim) *ndim = r.cols == 1 ? 1 : 2;
  return MT_OK;
}

const char* mt_last_error(const mt_ctx* ctx) { return ctx ? ctx->c.err.c_str() : g_create_error.c_str(); }

void mt_destroy(mt_ctx* ctx) {
  if (!ctx) return;
  destroy_step_events(ctx->ev);
  free_ctx(&ctx->c);
  delete ctx;
}

#define HIP_OR(call, code, msg)                                                             \
  do {                                                                                      \
    hipError_t e_ = (call);                                                                 \
    if (e_ != hipSuccess) {                                                                 \
      std::string m_ = std::string(msg) + ": " + hipGetErrorString(e_);                     \
      mt_destroy(h);                                                                        \
      return set_error(nullptr, code, m_);                                                  \
    }                                                                                       \
  } while (0)


// Device memory of a context: malloc (each piece from hipMalloc), region
// (carved in order from a caller's block, 256-byte aligned) or count (sizes
// only, for planning without a device).
struct DevAlloc {
  enum Mode { MALLOC, REGION, COUNT } mode = MALLOC;
  Ctx* c = nullptr;
  char* base = nullptr;
  size_t cap = 0, used = 0;
  bool take(size_t bytes, void** p) {
    bytes = (std::max<size_t>(bytes, 1) + 255) / 256 * 256;
    if (mode == COUNT) {
      *p = nullptr;
      used += bytes;
      return true;
    }
    if (mode == REGION) {
      if (used + bytes > cap) return false;
      *p = base + used;
    } else {
      if (hipMalloc(p, bytes) != hipSuccess) return false;
      c->dev_allocs.push_back(*p);
    }
    used += bytes;
    c->dev_bytes += (int64_t)bytes;
    return true;
  }
};

// Dimensions, buffer assignment, batch and micro-batch rows, unit layouts.
static void setup_layout(Ctx& c, const mt_model_cfg* cfg) {
  c.cfg = *cfg;
  c.D = make_dims(*cfg);
  c.dtype = cfg->compute_dtype;
  if (cfg->n_layer_buffers >= c.D.L + 1) {
    c.nbuf = c.ncache = c.D.L + 1;
  } else {
    c.nbuf = cfg->n_layer_buffers;
    c.ncache = c.nbuf - 2;
  }
  c.M_max = (int64_t)cfg->max_batch * cfg->max_seq;
  const int k = std::max(1, cfg->micro_batches);
  c.mb_seqs = (cfg->max_batch + k - 1) / k;
  c.M_ws = (int64_t)c.mb_seqs * cfg->max_seq;
  c.units.resize(c.D.L + 2);
  for (int l = 0; l < c.D.L; ++l) c.units[l].lay = layer_layout(c.D);
  c.units[c.D.L].lay = head_layout(c.D);
  c.units[c.D.L + 1].lay = emb_layout(c.D);
}

// Layer buffers, gradient buffers and the activation workspace (everything
// on the device but the residual checkpoints).
static bool alloc_device(Ctx& c, DevAlloc& A) {
  const mt_model_cfg* cfg = &c.cfg;
  const Dims& D = c.D;
  const int S = c.dtype;
  const int64_t max_unit = std::max(c.units[0].lay.n, c.units[D.L].lay.n);
  auto dalloc = [&](size_t bytes, void** p) -> bool { return A.take(bytes, p); };
  bool ok = true;
  // streaming buffers fit any unit that streams through them; a cached
  // unit's buffer fits that unit
  std::vector<size_t> bsize(c.nbuf, 0);
  for (int u = 0; u <= D.L; ++u) {
    const int b = c.buf_of(u);
    bsize[b] = std::max(bsize[b], c.units[u].lay.image_bytes(S));
  }
  c.buf.resize(c.nbuf);
  for (int i = 0; i < c.nbuf; ++i) ok &= dalloc(bsize[i], &c.buf[i]);
  ok &= dalloc((size_t)max_unit * 4, (void**)&c.gbuf[0]);
  ok &= dalloc((size_t)max_unit * 4, (void**)&c.gbuf[1]);
  if (cfg->flags & MT_BF16_GRADS) {
    ok &= dalloc((size_t)max_unit * 2, &c.gbuf16[0]);
    ok &= dalloc((size_t)max_unit * 2, &c.gbuf16[1]);
  }
  Workspace& w = c.ws;
  // activations hold one micro-batch (M rows); the residual gradient, the
  // per-token losses and the targets the whole batch (Mb rows)
  const int64_t M = c.M_ws, Mb = c.M_max, d = D.d, F = D.F, V = D.V;
  const size_t es = S ? 2 : 4;
  // token chunk of the QKV projection and the MLP
  {
    const int64_t mlp_row = 2 * F * 4 + F * (int64_t)es + F * 4 + 2 * F * (int64_t)es + d * (int64_t)es;
    int64_t ch = cfg->chunk_rows > 0 ? cfg->chunk_rows : M;
    if (cfg->chunk_rows == 0 && M * mlp_row > (4LL << 30))
      ch = std::max<int64_t>(256, (4LL << 30) / mlp_row / 256 * 256);
    w.chunk = std::min(ch, M);
  }
  const int64_t Q = w.chunk;
  ok &= dalloc(M * d * es, &w.h);
  ok &= dalloc(M * 4, (void**)&w.rstd1);
  ok &= dalloc(M * 4, (void**)&w.rstd2);
  ok &= dalloc(Q * D.qkvd * 4, (void**)&w.qkv_f);
  ok &= dalloc(M * D.qkvd * es, &w.qkv_s);
  ok &= dalloc(M * D.qd * 4, (void**)&w.o_f);
  if (S) ok &= dalloc(M * D.qd * es, &w.o_s); else w.o_s = w.o_f;
  ok &= dalloc(M * D.H * 4, (void**)&w.lse);
  ok &= dalloc(M * d * 4, (void**)&w.x1);
  ok &= dalloc(Q * d * es, &w.h2);
  ok &= dalloc(Q * 2 * F * 4, (void**)&w.gu_f);
  ok &= dalloc(Q * F * es, &w.act);
  ok &= dalloc(Mb * d * 4, (void**)&w.g_f);
  if (S) ok &= dalloc(M * d * es, &w.g_s); else w.g_s = w.g_f;
  ok &= dalloc(Q * F * 4, (void**)&w.dact_f);
  ok &= dalloc(Q * 2 * F * es, &w.dgu_s);
  // dO (consumed by the attention backward) and the projections' input
  // gradients (consumed by the RMSNorm backwards) are never live together
  ok &= dalloc(M * std::max<int64_t>(d, D.qd) * 4, (void**)&w.dh_f);
  w.do_f = w.dh_f;
  ok &= dalloc(M * D.qkvd * es, &w.dqkv_s);
  ok &= dalloc((size_t)mt_op_attn_bwd_ws_bytes(S, c.mb_seqs, cfg->max_seq, D.H, D.hd), &w.attn_ws);
  ok &= dalloc((size_t)rmsnorm_bwd_partials(M) * d * 4, (void**)&w.rms_ws);
  ok &= dalloc((size_t)GEMM_WS_BYTES, &w.gemm_ws);
  w.hf = w.h;   // the head runs between the last forward and the first recompute
  ok &= dalloc(M * 4, (void**)&w.rstdf);
  // logits in token chunks of at most ~4 GiB (multiples of 128 rows)
  int64_t chunk = (int64_t)((4LL << 30) / ((int64_t)V * 4));
  chunk = std::max<int64_t>(128, chunk / 128 * 128);
  w.head_chunk = std::min(chunk, M);
  ok &= dalloc(w.head_chunk * V * 4, (void**)&w.logits);
  if (S) ok &= dalloc(w.head_chunk * V * es, &w.dz_s); else w.dz_s = w.logits;
  ok &= dalloc(Mb * 4, (void**)&w.tok_loss);
  ok &= dalloc(Mb * 4, (void**)&w.targets);
  const int half = D.hd / 2;
  ok &= dalloc((size_t)cfg->max_seq * half * 4, (void**)&w.rope_cos);
  ok &= dalloc((size_t)cfg->max_seq * half * 4, (void**)&w.rope_sin);
  return ok;
}


int mt_create(const mt_model_cfg* cfg, const float* const* host_param_ptrs, const mt_device_env* env,
              mt_ctx** out) {
  if (!out) return set_error(nullptr, MT_EINVAL, "out is NULL");
  *out = nullptr;
  std::string why;
  if (validate(cfg, why)) return set_error(nullptr, MT_EINVAL, why);
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1)
    return set_error(nullptr, MT_EHIP, "no HIP device available");

  if (env && env->workspace && (((uintptr_t)env->workspace & 255) || env->workspace_bytes <= 0))
    return set_error(nullptr, MT_EINVAL, "env workspace must be 256-byte aligned with workspace_bytes > 0");

  mt_ctx* h = new mt_ctx();
  Ctx& c = h->c;
  setup_layout(c, cfg);
  c.dev_current.assign(c.D.L + 1, 0);
  c.tensors = tensor_table(c.D);
  c.pool = new Pool(default_threads(cfg->host_threads));
  c.delay_h2d_us = env_int("MT_TEST_DELAY_H2D_US");
  c.delay_d2h_us = env_int("MT_TEST_DELAY_D2H_US");
  c.delay_adamw_us = env_int("MT_TEST_DELAY_ADAMW_US");
  c.poison = env_int("MT_TEST_POISON") != 0;
  const Dims& D = c.D;
  const bool keep = cfg->flags & MT_KEEP_GRADS;
  const int S = c.dtype;

  // ---- host store ----
  for (int i = 0; i < D.L + 2; ++i) {
    Unit& u = c.units[i];
    const bool streamed = i <= D.L;
    const size_t nb = (size_t)u.lay.n * 4;
    if (streamed && S == 0) {
      HIP_OR(hipHostMalloc((void**)&u.p, nb, hipHostMallocDefault), MT_EHOSTOOM, "pinned master allocation");
      u.p_pinned = true;
    } else {
      u.p = (float*)host_alloc_plain(nb);
    }
    u.m = (float*)host_alloc_plain(nb);
    u.v = (float*)host_alloc_plain(nb);
    if (!u.p || !u.m || !u.v) { mt_destroy(h); return set_error(nullptr, MT_EHOSTOOM, "host allocation failed"); }
    if (streamed && keep) HIP_OR(hipHostMalloc((void**)&u.g, nb, hipHostMallocDefault), MT_EHOSTOOM, "pinned gradient allocation");
    if (!streamed) {
      u.g = (float*)host_alloc_plain(nb);
      if (!u.g) { mt_destroy(h); return set_error(nullptr, MT_EHOSTOOM, "host allocation failed"); }
    }
    if (streamed && S == 1)
      HIP_OR(hipHostMalloc(&u.shadow, u.lay.image_bytes(S), hipHostMallocDefault), MT_EHOSTOOM, "pinned shadow allocation");
  }
  int64_t max_unit = std::max(c.units[0].lay.n, c.units[D.L].lay.n);
  if (staged_grads(*cfg)) {
    const std::vector<int64_t> sizes = ring_sizes(*cfg, c.units[0].lay.n, c.units[D.L].lay.n);
    if (cfg->flags & MT_OVERLAP_OPT) c.head_slot = (int)sizes.size() - 1;
    for (int64_t n : sizes) {
      float* p = nullptr;
      HIP_OR(hipHostMalloc((void**)&p, (size_t)n * grad_bytes(*cfg), hipHostMallocDefault), MT_EHOSTOOM,
             "pinned gradient ring");
      c.ring_slot.push_back(p);
      c.ring_elems.push_back(n);
    }
  }
  c.slot_busy.assign(c.ring_slot.size(), 0);
  c.unit_busy.assign(D.L + 2, 0);
  c.adam_end.assign(D.L + 2, std::chrono::steady_clock::time_point{});
  // x0 (gathered embedding rows, host -> device at the start of the step and,
  // with parked checkpoints, again before layer 0's backward) and dx0 (layer
  // 0's input gradient, device -> host after that backward) are never live
  // together: one pinned slab serves both
  HIP_OR(hipHostMalloc((void**)&c.x0_host, (size_t)c.M_max * D.d * 4, hipHostMallocDefault), MT_EHOSTOOM, "pinned staging");
  c.dx0_host = c.x0_host;
  HIP_OR(hipHostMalloc((void**)&c.tgt_host, (size_t)c.M_max * 4, hipHostMallocDefault), MT_EHOSTOOM, "pinned staging");
  HIP_OR(hipHostMalloc((void**)&c.loss_host, (size_t)c.M_max * 4, hipHostMallocDefault), MT_EHOSTOOM, "pinned staging");
  // pinned memory is not guaranteed to be zero: clear p, images and kept gradients
  for (int i = 0; i <= D.L; ++i) {
    Unit& u = c.units[i];
    auto clear = [&](void* p, size_t bytes) {
      const size_t ch = 64 << 20;
      c.pool->run((int64_t)((bytes + ch - 1) / ch), [&](int64_t j) {
        const size_t a = (size_t)j * ch, b = std::min(bytes, a + ch);
        std::memset(static_cast<char*>(p) + a, 0, b - a);
      });
    };
    if (u.p_pinned) clear(u.p, (size_t)u.lay.n * 4);
    if (u.shadow) clear(u.shadow, u.lay.image_bytes(S));
    if (u.g) clear(u.g, (size_t)u.lay.n * 4);
  }

  // ---- device ----
  DevAlloc A;
  A.c = &c;
  if (env && env->workspace) {
    A.mode = DevAlloc::REGION;
    A.base = static_cast<char*>(env->workspace);
    A.cap = (size_t)env->workspace_bytes;
  }
  if (!alloc_device(c, A)) {
    mt_destroy(h);
    return set_error(nullptr, MT_EDEVOOM, A.mode == DevAlloc::REGION
                                              ? "env workspace smaller than the layer buffers and the workspace "
                                                "(see mt_device_plan)"
                                              : "device allocation failed");
  }
  bool ok = true;
  Workspace& w = c.ws;
  const int64_t Mb = c.M_max, d = D.d;
  const int half = D.hd / 2;

  // ---- residual checkpoints: device slots, parking the rest in host memory ----
  {
    const size_t slot = (size_t)Mb * d * 4;
    int k = cfg->ckpt_host;
    if (k == 0) {
      // free device memory (or what the caller's workspace has left), less a
      // margin for the runtime when allocating
      size_t free_b = 0, total_b = 0, margin = 0;
      if (A.mode == DevAlloc::REGION) {
        free_b = A.cap - A.used;
      } else {
        HIP_OR(hipMemGetInfo(&free_b, &total_b), MT_EHIP, "hipMemGetInfo");
        margin = (size_t)1 << 30;
      }
      const size_t slot_a = (slot + 255) / 256 * 256;
      const int64_t fit = free_b > margin ? (int64_t)((free_b - margin) / slot_a) : 0;
      if (fit < D.L + 1) {
        if (D.L < 3 || fit < 2) {
          mt_destroy(h);
          return set_error(nullptr, MT_EDEVOOM, "device memory cannot hold two residual checkpoints next to the workspace");
        }
        k = (int)(D.L - fit);   // device slots = L - k
      }
    }
    c.ck_nh = k > 0 ? k + 3 : 0;
    const int dev_slots = D.L + 1 - c.ck_nh;
    if (k > 0) {
      ok &= A.take(slot, (void**)&c.stage[0]);
      ok &= A.take(slot, (void**)&c.stage[1]);
    }
    ok &= A.take(slot * (size_t)dev_slots, (void**)&c.ckpt);
    if (!ok) { mt_destroy(h); return set_error(nullptr, MT_EDEVOOM, "device allocation of residual checkpoints failed"); }
    for (int i = 0; i < k; ++i) {
      float* p = (float*)host_alloc_plain(slot);
      if (!p) { mt_destroy(h); return set_error(nullptr, MT_EHOSTOOM, "host checkpoint slab"); }
      c.ck_host.push_back(p);
    }
    if (k > 0)
      for (auto*& b : c.bounce)
        HIP_OR(hipHostMalloc((void**)&b, slot, hipHostMallocDefault), MT_EHOSTOOM, "pinned checkpoint bounce slab");
  }


  // ---- streams (default priority) ----
  hipStream_t* ss[3] = {&c.s_in, &c.s_comp, &c.s_out};
  void* given[3] = {env ? env->copy_in : nullptr, env ? env->compute : nullptr, env ? env->copy_out : nullptr};
  for (int i = 0; i < 3; ++i) {
    if (given[i]) { *ss[i] = (hipStream_t)given[i]; continue; }
    HIP_OR(hipStreamCreateWithFlags(ss[i], hipStreamNonBlocking), MT_EHIP, "hipStreamCreate");
    c.own_streams[i] = true;
  }
  // RoPE table, built in double on the host
  {
    std::vector<float> cs((size_t)cfg->max_seq * half), sn((size_t)cfg->max_seq * half);
    mt_rope_table(cfg->max_seq, D.hd, cfg->rope_base, cs.data(), sn.data());
    HIP_OR(hipMemcpy(w.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice), MT_EHIP, "rope table upload");
    HIP_OR(hipMemcpy(w.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice), MT_EHIP, "rope table upload");
  }
  if (create_step_events(c, h->ev)) {
    std::string m = c.err;
    mt_destroy(h);
    return set_error(nullptr, MT_EHIP, m);
  }
  if (host_param_ptrs) {
    for (int32_t id = 0; id < mt_tensor_count(cfg); ++id) {
      if (!host_param_ptrs[id]) { mt_destroy(h); return set_error(nullptr, MT_EINVAL, "NULL parameter pointer"); }
      int rc = mt_set_param(h, id, host_param_ptrs[id]);
      if (rc) { std::string m = c.err; mt_destroy(h); return set_error(nullptr, rc, m); }
    }
  }
  *out = h;
  return MT_OK;
}

int mt_device_plan(const mt_model_cfg* cfg, int64_t* fixed_bytes, int64_t* ckpt_slot_bytes) {
  std::string why;
  if (validate(cfg, why)) return set_error(nullptr, MT_EINVAL, why);
  Ctx c;
  setup_layout(c, cfg);
  DevAlloc A;
  A.mode = DevAlloc::COUNT;
  A.c = &c;
  alloc_device(c, A);
  if (fixed_bytes) *fixed_bytes = (int64_t)A.used;
  if (ckpt_slot_bytes) *ckpt_slot_bytes = ((int64_t)c.M_max * c.D.d * 4 + 255) / 256 * 256;
  return MT_OK;
}

int mt_host_bytes(const mt_model_cfg* cfg, int64_t* state_bytes, int64_t* pinned_bytes,
                  int64_t* pageable_bytes, int64_t* parked_ckpt_bytes) {
  std::string why;
  if (validate(cfg, why)) return set_error(nullptr, MT_EINVAL, why);
  const Dims D = make_dims(*cfg);
  const UnitLayout ll = layer_layout(D), hl = head_layout(D), el = emb_layout(D);
  const int S = cfg->compute_dtype;
  const bool keep = cfg->flags & MT_KEEP_GRADS;
  const int64_t M = (int64_t)cfg->max_batch * cfg->max_seq;
  int64_t state = 0, pinned = 0, pageable = 0;
  auto unit = [&](const UnitLayout& u, bool streamed) {
    const int64_t nb = u.n * 4;
    state += 3 * nb;                                  // p, m, v
    if (streamed && S == 0) { pinned += nb; pageable += 2 * nb; }
    else pageable += 3 * nb;
    if (streamed && keep) pinned += nb;               // kept gradients
    if (!streamed) pageable += nb;                    // embedding gradient
    if (streamed && S == 1) pinned += (int64_t)u.image_bytes(S);   // bf16 image
  };
  for (int l = 0; l < D.L; ++l) unit(ll, true);
  unit(hl, true);
  unit(el, false);
  if (staged_grads(*cfg))
    for (int64_t n : ring_sizes(*cfg, ll.n, hl.n)) pinned += n * grad_bytes(*cfg);
  pinned += M * D.d * 4 + 2 * M * 4;                 // x0 and dx0 (one slab), targets / losses staging
  if (state_bytes) *state_bytes = state;
  if (pinned_bytes) *pinned_bytes = pinned;
  if (pageable_bytes) *pageable_bytes = pageable;
  if (parked_ckpt_bytes) *parked_ckpt_bytes = M * D.d * 4;
  return MT_OK;
}

int mt_sync(mt_ctx* h) {
  if (!h) return MT_EINVAL;
  return adam_drain_for(h->c, h->c.cfg.wait_timeout_ms, "mt_sync");
}

int mt_set_param(mt_ctx* h, int32_t id, const float* src) {
  if (!h) return MT_EINVAL;
  Ctx& c = h->c;
  adam_drain(c);
  if (id < 0 || id >= (int32_t)c.tensors.size() || !src) return set_error(&c, MT_EINVAL, "bad tensor id or NULL source");
  const TensorRef& r = c.tensors[id];
  Unit& u = r.unit < 0 ? c.emb() : c.units[r.unit];
  if (r.unit >= 0) c.dev_current[r.unit] = 0;
  const int64_t ch = 1 << 20, n = r.numel;
  c.pool->run((n + ch - 1) / ch, [&](int64_t i) {
    const int64_t a = i * ch, b = std::min(n, a + ch);
    std::memcpy(u.p + r.off + a, src + a, (size_t)(b - a) * 4);
    if (u.shadow) {
      const int64_t e = r.off + a;
      if (e < u.lay.mat_base)
        std::memcpy(static_cast<float*>(u.shadow) + e, src + a, (size_t)(b - a) * 4);
      else
        to_bf16_range(src + a,
                      reinterpret_cast<uint16_t*>(static_cast<char*>(u.shadow) + u.lay.mat_base * 4) + (e - u.lay.mat_base),
                      b - a);
    }
  });
  return MT_OK;
}

int mt_train_step(mt_ctx* h, const int32_t* tokens, const int32_t* targets, int32_t B, int32_t T,
                  float* loss_out) {
  if (!h) return MT_EINVAL;
  Ctx& c = h->c;
  if (c.broken) return set_error(&c, MT_ESTATE, "an earlier step exceeded wait_timeout_ms; no further step runs");
  if (!tokens || !targets) return set_error(&c, MT_EINVAL, "NULL tokens or targets");
  if (B < 1 || T < 1 || B > c.cfg.max_batch || T > c.cfg.max_seq)
    return set_error(&c, MT_EINVAL, "B/T outside [1, max_batch] x [1, max_seq]");
  const int64_t M = (int64_t)B * T;
  for (int64_t i = 0; i < M; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.D.V || targets[i] < 0 || targets[i] >= c.D.V)
      return set_error(&c, MT_EINVAL, "token or target id outside [0, vocab) at position " + std::to_string(i));
  try {
    return train_step_impl(c, *h->ev, tokens, targets, B, T, loss_out);
  } catch (const std::exception& e) {
    return set_error(&c, MT_EHOSTOOM, std::string("host exception: ") + e.what());
  }
}

int mt_token_losses(mt_ctx* h, const float** ptr, int64_t* n) {
  if (!h || !ptr || !n) return MT_EINVAL;
  *ptr = h->c.token_loss.data();
  *n = (int64_t)h->c.token_loss.size();
  return MT_OK;
}

static int tensor_ptr(Ctx& c, int32_t id, int which, const float** ptr, int64_t* numel) {
  adam_drain(c);
  if (id < 0 || id >= (int32_t)c.tensors.size() || !ptr) return set_error(&c, MT_EINVAL, "bad tensor id or NULL pointer");
  const TensorRef& r = c.tensors[id];
  Unit& u = r.unit < 0 ? c.emb() : c.units[r.unit];
  const float* base = which == 0 ? u.p : which == 1 ? u.g : which == 2 ? u.m : u.v;
  if (which == 1 && (!(c.cfg.flags & MT_KEEP_GRADS)))
    return set_error(&c, MT_ENOGRADS, "gradients are kept only with MT_KEEP_GRADS");
  *ptr = base + r.off;
  if (numel) *numel = r.numel;
  return MT_OK;
}

int mt_params(mt_ctx* h, int32_t id, const float** ptr, int64_t* numel) {
  return h ? tensor_ptr(h->c, id, 0, ptr, numel) : MT_EINVAL;
}

int mt_grads(mt_ctx* h, int32_t id, const float** ptr, int64_t* numel) {
  return h ? tensor_ptr(h->c, id, 1, ptr, numel) : MT_EINVAL;
}

int mt_opt_state(mt_ctx* h, int32_t id, const float** m, const float** v, int64_t* t) {
  if (!h) return MT_EINVAL;
  int rc = tensor_ptr(h->c, id, 2, m, nullptr);
  if (rc) return rc;
  rc = tensor_ptr(h->c, id, 3, v, nullptr);
  if (rc) return rc;
  if (t) *t = h->c.step;
  return MT_OK;
}

int mt_stats(mt_ctx* h, mt_step_stats* out) {
  if (!h || !out) return MT_EINVAL;
  *out = h->c.stats;
  return MT_OK;
}

int mt_kernel_stats(mt_ctx* h, mt_kernel_stat* out, int32_t cap, int32_t* n) {
  if (!h || !n) return MT_EINVAL;
  const auto& k = h->c.kstats;
  *n = (int32_t)k.size();
  for (int32_t i = 0; i < std::min<int32_t>(cap, *n); ++i) out[i] = k[i];
  return MT_OK;
}

int mt_schedule(mt_ctx* h, mt_sched_entry* out, int32_t cap, int32_t* n) {
  if (!h || !n) return MT_EINVAL;
  const auto& s = h->c.sched;
  *n = (int32_t)s.size();
  for (int32_t i = 0; i < std::min<int32_t>(cap, *n); ++i) out[i] = s[i];
  return MT_OK;
}

int mt_trace_dump(mt_ctx* h, const char* path) {
  if (!h || !path) return MT_EINVAL;
  FILE* f = fopen(path, "w");
  if (!f) return set_error(&h->c, MT_EINVAL, std::string("cannot open ") + path);
  static const char* ph[] = {"load", "fwd", "head", "bwd", "grad", "adamw", "ckpt out", "ckpt in", "refresh"};
  static const char* st[] = {"copy-in", "compute", "copy-out", "host AdamW", "host submit"};
  fprintf(f, "{\"traceEvents\":[\n");
  bool first = true;
  for (int i = 0; i < 5; ++i) {
    fprintf(f, "%s{\"name\":\"thread_name\",\"ph\":\"M\",\"pid\":0,\"tid\":%d,\"args\":{\"name\":\"%s\"}}",
            first ? "" : ",\n", i, st[i]);
    first = false;
  }
  for (const auto& e : h->c.sched) {
    char unit[32];
    if (e.unit == MT_UNIT_HEAD) snprintf(unit, sizeof unit, "head");
    else if (e.unit == MT_UNIT_EMB) snprintf(unit, sizeof unit, "embedding");
    else if (e.phase == MT_PH_CKPT_OUT || e.phase == MT_PH_CKPT_IN) snprintf(unit, sizeof unit, "x_%d", e.unit);
    else snprintf(unit, sizeof unit, "layer %d", e.unit);
    fprintf(f, ",\n{\"name\":\"%s %s\",\"ph\":\"X\",\"pid\":0,\"tid\":%d,\"ts\":%.3f,\"dur\":%.3f,\"args\":{\"buffer\":%d}}",
            ph[e.phase], unit, e.stream, e.t0_ms * 1000.0, (e.t1_ms - e.t0_ms) * 1000.0, e.buffer);
  }
  fprintf(f, "\n]}\n");
  fclose(f);
  return MT_OK;
}

int mt_device_bytes(mt_ctx* h, int64_t* bytes) {
  if (!h || !bytes) return MT_EINVAL;
  *bytes = h->c.dev_bytes;
  return MT_OK;
}

int mt_layout_info(mt_ctx* h, int64_t* chunk_rows, int32_t* ckpt_host, int32_t* ckpt_device_slots) {
  if (!h) return MT_EINVAL;
  const Ctx& c = h->c;
  if (chunk_rows) *chunk_rows = c.ws.chunk;
  if (ckpt_host) *ckpt_host = (int32_t)c.ck_host.size();
  if (ckpt_device_slots) *ckpt_device_slots = c.D.L + 1 - c.ck_nh + (c.ck_nh ? 2 : 0);
  return MT_OK;
}

}  // extern "C"
