// Stateless layer template: the decoder block's forward, recompute and
// backward as kernel sequences on the compute stream, bound at call time to
// whichever device buffer holds the layer's weights ("MegaTrain: Full
// Precision Training of 100B+ Parameter LLMs on a Single GPU", abstract:
// stateless layer templates bind weights dynamically as they stream in, with
// no persistent autograd graph; "Technical Brief: MegaTrain's Single-GPU
// 120B-Parameter Training Breakthrough", section "Checkpointing, Manual
// Gradients, and CPU-Side Optimizer Steps": activation checkpointing and
// manually orchestrated gradients).
//
// Binding is an offset computation over the unit layout: no allocation and no
// per-layer device object. Only the residual stream at layer boundaries is
// kept (checkpoints x_0..x_L); the backward of layer l recomputes the block
// from x_l through the attention output projection, then rebuilds the MLP
// input side chunk by chunk inside the hand-written backward.
#include <cmath>

#include "kernels.h"
#include "runtime.h"

namespace mt {

static inline size_t esz(int dtype) { return dtype ? 2 : 4; }

int timed(Ctx& c, int cls, double flops, double bytes, const std::function<hipError_t()>& fn) {
  KTiming& k = c.kt;
  size_t e0 = 0;
  if (k.on) {
    if (k.used + 2 > k.ev.size()) {
      const size_t grow = k.ev.size() ? k.ev.size() : 4096;
      for (size_t i = 0; i < grow; ++i) {
        hipEvent_t ev;
        if (hipEventCreate(&ev) != hipSuccess) return set_error(&c, MT_EHIP, "hipEventCreate failed");
        k.ev.push_back(ev);
      }
    }
    e0 = k.used;
    k.used += 2;
    if (hipEventRecord(k.ev[e0], c.s_comp) != hipSuccess) return set_error(&c, MT_EHIP, "hipEventRecord failed");
  }
  const hipError_t e = fn();
  if (e != hipSuccess)
    return set_error(&c, MT_EHIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  if (k.on) {
    if (hipEventRecord(k.ev[e0 + 1], c.s_comp) != hipSuccess)
      return set_error(&c, MT_EHIP, "hipEventRecord failed");
    k.recs.push_back({cls, flops, bytes, e0});
  }
  return MT_OK;
}

LayerPtrs bind_layer(const Ctx& c, const void* image) {
  const UnitLayout& L = c.units[0].lay;
  const char* b = static_cast<const char*>(image);
  LayerPtrs W;
  W.attn_norm = reinterpret_cast<const float*>(b + L.image_offset(L.off[0], c.dtype));
  W.mlp_norm = reinterpret_cast<const float*>(b + L.image_offset(L.off[1], c.dtype));
  W.wqkv = b + L.image_offset(L.off[2], c.dtype);
  W.wo = b + L.image_offset(L.off[3], c.dtype);
  W.wgu = b + L.image_offset(L.off[4], c.dtype);
  W.wdown = b + L.image_offset(L.off[5], c.dtype);
  return W;
}

#define RUN(cls, fl, by, call)                            \
  do {                                                    \
    int rc_ = timed(c, cls, fl, by, [&] { return call; }); \
    if (rc_) return rc_;                                  \
  } while (0)

static inline double gemm_bytes(int64_t M, int64_t N, int64_t K, int dt, bool r) {
  return (double)(M * K + K * N) * esz(dt) + (double)M * N * 4 * (r ? 2 : 1);
}

// QKV projection and its rotation, chunk by chunk: qkv_s = rope(h Wqkv^T).
static int qkv_forward(Ctx& c, const LayerPtrs& W, int64_t M, int T) {
  const Dims& D = c.D;
  const int S = c.dtype;
  Workspace& w = c.ws;
  const int64_t d = D.d;
  for (int64_t r0 = 0; r0 < M; r0 += w.chunk) {
    const int64_t mc = std::min(w.chunk, M - r0);
    const void* h = static_cast<const char*>(w.h) + r0 * d * esz(S);
    void* qs = static_cast<char*>(w.qkv_s) + r0 * D.qkvd * esz(S);
    RUN(K_GEMM_NT, 2.0 * mc * D.qkvd * d, gemm_bytes(mc, D.qkvd, d, S, false),
        gemm_ws(S, MT_GEMM_NT, h, d, W.wqkv, d, w.qkv_f, D.qkvd, nullptr, 0, mc, D.qkvd, d, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
    RUN(K_ROPE, 0, (double)mc * D.qkvd * (4 + esz(S)),
        rope(S, 0, w.qkv_f, qs, w.rope_cos, w.rope_sin, r0, mc, T, D.H, D.Hkv, D.hd, c.s_comp));
  }
  return MT_OK;
}

// MLP input side for rows [r0, r0 + mc): h2 = RMSNorm(x1), gu = h2 Wgu^T,
// act = silu(gate) up (chunk buffers).
static int mlp_front(Ctx& c, const LayerPtrs& W, int64_t r0, int64_t mc) {
  const Dims& D = c.D;
  const int S = c.dtype;
  Workspace& w = c.ws;
  const int64_t d = D.d, F = D.F;
  RUN(K_RMS_FWD, 0, (double)mc * d * (4 + esz(S)),
      rmsnorm_fwd(S, w.x1 + r0 * d, W.mlp_norm, w.h2, w.rstd2 + r0, mc, D.d, c.cfg.rms_eps, c.s_comp));
  RUN(K_GEMM_NT, 2.0 * mc * 2 * F * d, gemm_bytes(mc, 2 * F, d, S, false),
      gemm_ws(S, MT_GEMM_NT, w.h2, d, W.wgu, d, w.gu_f, 2 * F, nullptr, 0, mc, 2 * F, d, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  RUN(K_SWIGLU, 0, (double)mc * F * (8 + esz(S)), swiglu_fwd(S, w.gu_f, w.act, mc, D.F, c.s_comp));
  return MT_OK;
}

int layer_forward(Ctx& c, const LayerPtrs& W, int l, int B, int T, bool recompute, int64_t row0) {
  const Dims& D = c.D;
  const int S = c.dtype;
  Workspace& w = c.ws;
  const int64_t M = (int64_t)B * T, d = D.d, F = D.F;
  const float* x = c.ckpt_dev(l) + row0 * d;
  const float eps = c.cfg.rms_eps;
  const double attn_fl = 2.0 * B * (double)T * T * D.H * D.hd;

  RUN(K_RMS_FWD, 0, (double)M * d * (4 + esz(S)), rmsnorm_fwd(S, x, W.attn_norm, w.h, w.rstd1, M, D.d, eps, c.s_comp));
  int rc = qkv_forward(c, W, M, T);
  if (rc) return rc;
  RUN(K_ATTN_FWD, attn_fl, (double)M * D.qkvd * esz(S) + (double)M * D.qd * (4 + (S ? 2 : 0)),
      attn_fwd(S, w.qkv_s, w.o_f, S ? w.o_s : nullptr, w.lse, B, T, D.H, D.Hkv, D.hd, c.s_comp));
  RUN(K_GEMM_NT, 2.0 * M * d * D.qd, gemm_bytes(M, d, D.qd, S, true),
      gemm_ws(S, MT_GEMM_NT, w.o_s, D.qd, W.wo, D.qd, w.x1, d, x, d, M, d, D.qd, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  // the recompute stops here: the backward rebuilds the MLP chunk by chunk
  if (recompute) return MT_OK;
  float* xn = c.ckpt_dev(l + 1) + row0 * d;
  for (int64_t r0 = 0; r0 < M; r0 += w.chunk) {
    const int64_t mc = std::min(w.chunk, M - r0);
    if ((rc = mlp_front(c, W, r0, mc))) return rc;
    RUN(K_GEMM_NT, 2.0 * mc * d * F, gemm_bytes(mc, d, F, S, true),
        gemm_ws(S, MT_GEMM_NT, w.act, F, W.wdown, F, xn + r0 * d, d, w.x1 + r0 * d, d, mc, d, F, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  }
  return MT_OK;
}

int layer_backward(Ctx& c, const LayerPtrs& W, int l, int B, int T, float* gu, int64_t row0, bool first) {
  // gu: this unit's gradient slab on the device (master unit layout); rows
  // [row0, row0 + B T) of the step's batch; the weight gradients are written
  // (first) or added to those of the earlier micro-batches
  const Dims& D = c.D;
  const int S = c.dtype;
  Workspace& w = c.ws;
  const UnitLayout& U = c.units[0].lay;
  const int64_t M = (int64_t)B * T, d = D.d, F = D.F, qd = D.qd, qkvd = D.qkvd;
  const float* x = c.ckpt_dev(l) + row0 * d;
  float* gf = w.g_f + row0 * d;   // the residual gradient of these rows
  // its matrix-product operand: the bf16 cast, or (fp32 mode) itself
  void* gsb = S ? w.g_s : (void*)gf;
  const double attn_fl = 2.0 * B * (double)T * T * D.H * D.hd;
  const float* acc_w = first ? nullptr : gu;   // base of the slab to add to, or none

  int rc = layer_forward(c, W, l, B, T, true, row0);
  if (rc) return rc;

  // MLP, chunk by chunk: recompute h2, gu, act; then
  // down: x_{l+1} = x1 + act Wd^T;  gate/up: gu = h2 Wgu^T.
  // The weight gradients accumulate over the chunks in chunk order.
  if (S) RUN(K_CAST, 0, (double)M * d * 6, cast(S, gf, w.g_s, M * d, c.s_comp));
  for (int64_t r0 = 0; r0 < M; r0 += w.chunk) {
    const int64_t mc = std::min(w.chunk, M - r0);
    const bool acc = r0 > 0 || !first;
    const void* gs = static_cast<const char*>(gsb) + r0 * d * esz(S);
    if ((rc = mlp_front(c, W, r0, mc))) return rc;
    RUN(K_GEMM_NN, 2.0 * mc * F * d, gemm_bytes(mc, F, d, S, false),
        gemm_ws(S, MT_GEMM_NN, gs, d, W.wdown, F, w.dact_f, F, nullptr, 0, mc, F, d, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
    RUN(K_GEMM_TN, 2.0 * d * F * mc, gemm_bytes(d, F, mc, S, acc),
        gemm_ws(S, MT_GEMM_TN, gs, d, w.act, F, gu + U.off[5], F, acc ? gu + U.off[5] : nullptr, F, d, F, mc,
                w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
    RUN(K_SWIGLU, 0, (double)mc * F * (12 + 2 * esz(S)), swiglu_bwd(S, w.gu_f, w.dact_f, w.dgu_s, mc, D.F, c.s_comp));
    RUN(K_GEMM_NN, 2.0 * mc * d * 2 * F, gemm_bytes(mc, d, 2 * F, S, false),
        gemm_ws(S, MT_GEMM_NN, w.dgu_s, 2 * F, W.wgu, d, w.dh_f + r0 * d, d, nullptr, 0, mc, d, 2 * F, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
    RUN(K_GEMM_TN, 2.0 * 2 * F * d * mc, gemm_bytes(2 * F, d, mc, S, acc),
        gemm_ws(S, MT_GEMM_TN, w.dgu_s, 2 * F, w.h2, d, gu + U.off[4], d, acc ? gu + U.off[4] : nullptr, d, 2 * F,
                d, mc, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  }
  RUN(K_RMS_BWD, 0, (double)M * d * 20,
      rmsnorm_bwd(w.x1, W.mlp_norm, w.rstd2, w.dh_f, gf, 1, gu + U.off[1], w.rms_ws, M, D.d, c.s_comp, !first));
  // out projection: x1 = x + o Wo^T
  if (S) RUN(K_CAST, 0, (double)M * d * 6, cast(S, gf, w.g_s, M * d, c.s_comp));
  RUN(K_GEMM_NN, 2.0 * M * qd * d, gemm_bytes(M, qd, d, S, false),
      gemm_ws(S, MT_GEMM_NN, gsb, d, W.wo, qd, w.do_f, qd, nullptr, 0, M, qd, d, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  RUN(K_GEMM_TN, 2.0 * d * qd * M, gemm_bytes(d, qd, M, S, !first),
      gemm_ws(S, MT_GEMM_TN, gsb, d, w.o_s, qd, gu + U.off[3], qd, acc_w ? acc_w + U.off[3] : nullptr, qd, d, qd,
              M, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  // attention, with the rotation's backward applied as the gradients are written
  RUN(K_ATTN_BWD, 2.5 * attn_fl, (double)M * qkvd * 2 * esz(S) + (double)M * qd * 8,
      attn_bwd(S, w.qkv_s, w.o_f, w.do_f, w.lse, w.dqkv_s, S, w.rope_cos, w.rope_sin, w.attn_ws, B, T, D.H,
               D.Hkv, D.hd, c.s_comp));
  // qkv projection
  RUN(K_GEMM_NN, 2.0 * M * d * qkvd, gemm_bytes(M, d, qkvd, S, false),
      gemm_ws(S, MT_GEMM_NN, w.dqkv_s, qkvd, W.wqkv, d, w.dh_f, d, nullptr, 0, M, d, qkvd, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  RUN(K_GEMM_TN, 2.0 * qkvd * d * M, gemm_bytes(qkvd, d, M, S, !first),
      gemm_ws(S, MT_GEMM_TN, w.dqkv_s, qkvd, w.h, d, gu + U.off[2], d, acc_w ? acc_w + U.off[2] : nullptr, d, qkvd,
              d, M, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  RUN(K_RMS_BWD, 0, (double)M * d * 20,
      rmsnorm_bwd(x, W.attn_norm, w.rstd1, w.dh_f, gf, 1, gu + U.off[0], w.rms_ws, M, D.d, c.s_comp, !first));
  return MT_OK;
}

int head_forward_backward(Ctx& c, const void* image, int B, int T, float* gu, int64_t row0, bool first,
                          int64_t M_step) {
  // rows [row0, row0 + B T) of a step of M_step tokens (the loss is the mean
  // over all of them); the head's gradients are written (first) or added to
  const Dims& D = c.D;
  const int S = c.dtype;
  Workspace& w = c.ws;
  const UnitLayout& U = c.head().lay;
  const int64_t M = (int64_t)B * T, d = D.d, V = D.V;
  const char* base = static_cast<const char*>(image);
  const float* w_norm = reinterpret_cast<const float*>(base + U.image_offset(U.off[0], S));
  const void* w_head = base + U.image_offset(U.off[1], S);
  const float* x = c.ckpt_dev(D.L) + row0 * d;
  float* d_head = gu + U.off[1];

  RUN(K_RMS_FWD, 0, (double)M * d * (4 + esz(S)), rmsnorm_fwd(S, x, w_norm, w.hf, w.rstdf, M, D.d, c.cfg.rms_eps, c.s_comp));
  const float scale = 1.f / (float)M_step;
  for (int64_t r0 = 0; r0 < M; r0 += w.head_chunk) {
    const int64_t mc = std::min(w.head_chunk, M - r0);
    const bool acc = r0 > 0 || !first;
    const void* hf = static_cast<const char*>(w.hf) + r0 * d * esz(S);
    RUN(K_GEMM_NT, 2.0 * mc * V * d, gemm_bytes(mc, V, d, S, false),
        gemm_ws(S, MT_GEMM_NT, hf, d, w_head, d, w.logits, V, nullptr, 0, mc, V, d, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
    RUN(K_XENT, 0, (double)mc * V * (4 + esz(S)),
        xent(S, w.logits, w.targets + row0 + r0, w.tok_loss + row0 + r0, w.dz_s, mc, (int)V, scale, c.s_comp));
    RUN(K_GEMM_TN, 2.0 * V * d * mc, gemm_bytes(V, d, mc, S, acc),
        gemm_ws(S, MT_GEMM_TN, w.dz_s, V, hf, d, d_head, d, acc ? d_head : nullptr, d, V, d, mc, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
    RUN(K_GEMM_NN, 2.0 * mc * d * V, gemm_bytes(mc, d, V, S, false),
        gemm_ws(S, MT_GEMM_NN, w.dz_s, V, w_head, d, w.dh_f + r0 * d, d, nullptr, 0, mc, d, V, w.gemm_ws, GEMM_WS_BYTES, c.s_comp));
  }
  RUN(K_RMS_BWD, 0, (double)M * d * 20,
      rmsnorm_bwd(x, w_norm, w.rstdf, w.dh_f, w.g_f + row0 * d, 0, gu + U.off[0], w.rms_ws, M, D.d, c.s_comp,
                  !first));
  return MT_OK;
}

}  // namespace mt
