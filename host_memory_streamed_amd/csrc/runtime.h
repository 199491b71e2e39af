// Internal structures of the streamed training-step library: unit layouts,
// the host store, device workspace, the thread pool and the context.
#pragma once

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdint>
#include <deque>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "mt.h"

namespace mt {

// ----------------------------------------------------------- thread pool ---

class Pool {
 public:
  explicit Pool(int n);
  ~Pool();
  int size() const { return (int)workers_.size(); }
  // Run fn(i) for i in [0, n) on the workers; when all have finished, call
  // done() (on the worker that finished last). Returns immediately. Workers
  // take indices from the job with the lowest priority value first (in
  // submission order among equals), so a later, more urgent job overtakes
  // the rest of an earlier one at index granularity.
  void submit(int64_t n, std::function<void(int64_t)> fn, std::function<void()> done = nullptr,
              int64_t priority = 0);
  // Run fn(i) for i in [0, n) ahead of every queued job and wait for all of them.
  void run(int64_t n, const std::function<void(int64_t)>& fn);

 private:
  struct Job {
    std::function<void(int64_t)> fn;
    std::function<void()> done;
    int64_t n;
    int64_t priority;
    std::atomic<int64_t> next{0};
    std::atomic<int64_t> finished{0};
  };
  void loop();
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::condition_variable cv_;
  std::deque<std::shared_ptr<Job>> jobs_;
  bool stop_ = false;
};

// ------------------------------------------------------------- layouts ---

constexpr int64_t kAlign = 64;   // elements
inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// A unit (embedding, one layer, or the head) is one contiguous slab of fp32
// master values. Norm gains come first ([0, mat_base)), matrices after, each
// matrix group starting on a 64-element boundary. The device image of a unit
// keeps the gains in fp32 and stores the matrices in the compute dtype.
struct UnitLayout {
  int64_t n = 0;          // slab elements, padding included
  int64_t mat_base = 0;   // first matrix element
  // layer: 0 attn_norm, 1 mlp_norm, 2 wqkv, 3 wo, 4 wgu, 5 wdown
  // head : 0 final_norm, 1 lm_head
  std::vector<int64_t> off;
  size_t image_bytes(int dtype) const {
    return (size_t)mat_base * 4 + (size_t)(n - mat_base) * (dtype ? 2 : 4);
  }
  size_t image_offset(int64_t elem, int dtype) const {
    return elem < mat_base ? (size_t)elem * 4
                           : (size_t)mat_base * 4 + (size_t)(elem - mat_base) * (dtype ? 2 : 4);
  }
};

struct Dims {
  int L, d, H, Hkv, hd, F, V;
  int qd, kvd, qkvd;
};

struct TensorRef {
  int unit;        // -1 embedding, 0..L-1 layers, L head
  int64_t off, numel;
  int64_t rows, cols;
  std::string name;
};

struct Unit {
  UnitLayout lay;
  float* p = nullptr;       // fp32 master (pinned when it is the fp32 device image)
  float* m = nullptr;
  float* v = nullptr;
  float* g = nullptr;       // gradients (MT_KEEP_GRADS, and always for the embedding)
  void* shadow = nullptr;   // bf16-mode device image (pinned)
  bool p_pinned = false;
  const void* image() const { return shadow ? shadow : (const void*)p; }
};

// --------------------------------------------------------- kernel timing ---

enum KClass {
  K_GEMM_NT, K_GEMM_NN, K_GEMM_TN, K_ATTN_FWD, K_ATTN_BWD, K_RMS_FWD, K_RMS_BWD,
  K_ROPE, K_SWIGLU, K_XENT, K_CAST, K_OTHER, K_COUNT
};

struct KTiming {
  bool on = false;
  std::vector<hipEvent_t> ev;   // pairs
  size_t used = 0;
  struct Rec { int cls; double flops, bytes; size_t e; };
  std::vector<Rec> recs;
};

// ----------------------------------------------------- device workspace ---

// Full-batch buffers hold M = max_batch * max_seq rows; chunk buffers hold
// `chunk` rows: the QKV projection output before its rotation and the MLP's
// intermediates are produced and consumed chunk by chunk, so their size does
// not grow with the sequence.
struct Workspace {
  int64_t chunk = 0;        // token rows per chunk
  // per-layer activations
  void* h = nullptr;        // RMSNorm out (S)
  float* rstd1 = nullptr;
  float* rstd2 = nullptr;
  float* qkv_f = nullptr;   // projection out [chunk]
  void* qkv_s = nullptr;    // rotated, cast
  float* o_f = nullptr;
  void* o_s = nullptr;      // bf16 mode: cast of o (fp32 mode: o_f)
  float* lse = nullptr;
  float* x1 = nullptr;
  void* h2 = nullptr;       // [chunk]
  float* gu_f = nullptr;    // [chunk]
  void* act = nullptr;      // [chunk]
  // backward
  float* g_f = nullptr;     // running residual gradient
  void* g_s = nullptr;      // its cast (fp32 mode: g_f)
  float* dact_f = nullptr;  // [chunk]
  void* dgu_s = nullptr;    // [chunk]
  float* dh_f = nullptr;
  float* do_f = nullptr;    // shares dh_f's memory (disjoint lifetimes)
  void* dqkv_s = nullptr;   // gradient of the unrotated projection output
  void* attn_ws = nullptr;
  float* rms_ws = nullptr;
  void* gemm_ws = nullptr;  // K-split partials of the GEMMs (GEMM_WS_BYTES)
  // head
  void* hf = nullptr;       // shares h's memory
  float* rstdf = nullptr;
  float* logits = nullptr;  // [head_chunk, V]
  void* dz_s = nullptr;     // bf16 mode cast of dlogits (fp32 mode: logits)
  float* tok_loss = nullptr;
  int32_t* targets = nullptr;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  int64_t head_chunk = 0;
};

// ------------------------------------------------------------- context ---

struct Ctx {
  mt_model_cfg cfg;
  Dims D;
  int dtype;                 // 0 fp32, 1 bf16
  // Layer buffers. Units with a buffer of their own (the device cache) are
  // the head and the layers above L - ncache, i.e. u >= L + 1 - ncache; the
  // other layers stream through buffers 0 and 1 (layer l in l % 2).
  // ncache == L + 1: every unit has its own buffer (unit u in buffer u).
  int nbuf;
  int ncache;
  bool cached(int unit) const { return unit >= D.L + 1 - ncache; }
  int buf_of(int unit) const {
    if (ncache == D.L + 1) return unit;
    return cached(unit) ? 2 + (D.L - unit) : unit % 2;
  }
  // per unit (layers, head): its buffer holds the unit's current image
  // (cached units only; cleared when an update or mt_set_param changes it)
  std::vector<char> dev_current;
  int64_t M_max;
  // sequences per micro-batch (cfg.micro_batches): the layer template runs a
  // step's batch in pieces of at most mb_seqs sequences; the workspace holds
  // one piece (M_ws = mb_seqs * max_seq token rows)
  int mb_seqs = 0;
  int64_t M_ws = 0;
  std::string err;

  std::vector<Unit> units;   // [0, L) layers, L head, L+1 embedding
  Unit& layer(int l) { return units[l]; }
  Unit& head() { return units[D.L]; }
  Unit& emb() { return units[D.L + 1]; }
  std::vector<TensorRef> tensors;

  // Gradient staging (MT_KEEP_GRADS off, or MT_BF16_GRADS): slots of
  // ring_elems[i] gradients (fp32, or bf16 with MT_BF16_GRADS). A slot is
  // busy from its D2H until the AdamW that reads it has finished.
  std::vector<float*> ring_slot;
  std::vector<int64_t> ring_elems;
  int head_slot = -1;              // slot reserved for the head (-1: any slot fits it)

  // Host AdamW jobs in flight, shared with the worker threads. With
  // MT_OVERLAP_OPT they may finish during the next step; a unit is loaded
  // again only when none of its updates is in flight.
  std::mutex amu;
  std::condition_variable acv;
  int adam_pending = 0;
  std::vector<int> unit_busy;      // [L + 2]: layers, head, embedding
  std::vector<char> slot_busy;
  std::vector<std::chrono::steady_clock::time_point> adam_end;   // per unit, last update
  std::atomic<int64_t> adam_ns{0};
  // pinned staging
  float* x0_host = nullptr;      // [M_max, d]
  float* dx0_host = nullptr;     // [M_max, d]
  int32_t* tgt_host = nullptr;   // [M_max]
  float* loss_host = nullptr;    // [M_max]
  std::vector<float> token_loss; // last step
  std::vector<int32_t> prev_rows;  // embedding rows touched by the previous step

  // Residual checkpoints x_0..x_L (x_i is layer i's input, x_L the head's).
  // x_i with i >= ck_nh stays in a device slot from its forward to its
  // backward use. The others pass through two device staging buffers (x_i in
  // stage[i % 2]): x_1..x_{ck_nh-3} are parked in host slabs after their
  // forward and come back before their backward, x_0 comes back from the
  // gathered embedding rows, and the last two fit in the stages throughout.
  // The slabs are pageable (pinned memory is a scarce, capped resource): x_i
  // crosses the link through the pinned bounce slab bounce[i % 2], and the
  // worker pool copies between the bounce slab and the parked slab.
  int ck_nh = 0;                 // 0, or (host slabs) + 3
  std::vector<float*> ck_host;   // pageable slabs for x_1..x_{ck_nh-3}
  float* bounce[2] = {nullptr, nullptr};   // pinned, M_max * d floats each
  float* stage[2] = {nullptr, nullptr};
  float* ckpt_dev(int i) const {
    return i >= ck_nh ? ckpt + (int64_t)(i - ck_nh) * M_max * D.d : stage[i & 1];
  }

  // device
  std::vector<void*> buf;        // layer buffers
  float* gbuf[2] = {nullptr, nullptr};
  void* gbuf16[2] = {nullptr, nullptr};   // MT_BF16_GRADS: the bf16 copy that crosses the link
  float* ckpt = nullptr;         // device slots for x_{ck_nh}..x_L
  Workspace ws;
  std::vector<void*> dev_allocs;
  int64_t dev_bytes = 0;

  hipStream_t s_in = nullptr, s_comp = nullptr, s_out = nullptr;
  bool own_streams[3] = {false, false, false};

  Pool* pool = nullptr;
  int64_t step = 0;
  // Set when a step exceeded cfg.wait_timeout_ms: no further step runs.
  bool broken = false;
  // Schedule test hooks, read from the environment at creation (results must
  // not depend on them): host delays before each layer-image load
  // (MT_TEST_DELAY_H2D_US), before each gradient copy (MT_TEST_DELAY_D2H_US)
  // and at the start of each unit's AdamW (MT_TEST_DELAY_ADAMW_US); and
  // MT_TEST_POISON=1, which fills every tensor of a layer buffer with NaN
  // before it is loaded and of a gradient buffer after its copy has left, so
  // that a read of a released buffer shows up in the results.
  int64_t delay_h2d_us = 0, delay_d2h_us = 0, delay_adamw_us = 0;
  bool poison = false;
  mt_step_stats stats{};
  KTiming kt;
  std::vector<mt_kernel_stat> kstats;
  std::vector<mt_sched_entry> sched;
};

// ----------------------------------------------------------- helpers ---

int set_error(Ctx* c, int code, const std::string& msg);
// Wait until every submitted AdamW job has finished.
void adam_drain(Ctx& c);
// As adam_drain, for at most ms milliseconds (ms <= 0: no limit); MT_ETIMEOUT
// (with an error naming the units still updating) if they have not finished.
int adam_drain_for(Ctx& c, int64_t ms, const char* what);
void* host_alloc_plain(size_t bytes);
void host_free_plain(void* p, size_t bytes);

struct AdamConst {
  float decay, b1, omb1, b2, omb2, step_size, inv_sqrt_bc2, eps;
};
AdamConst adam_const(const mt_model_cfg& c, int64_t t);
// p, m, v, g over [0, n); optional outputs: bf16 image and/or fp32 copy of p.
void adamw_range(float* p, float* m, float* v, const float* g, int64_t n, const AdamConst& k,
                 uint16_t* bf16_out, float* f32_out);
// As adamw_range with the gradient given as bf16 (widened exactly); g32, if
// not NULL, receives the widened gradient.
void adamw_range_g16(float* p, float* m, float* v, const uint16_t* g, int64_t n, const AdamConst& k,
                     uint16_t* bf16_out, float* f32_out, float* g32);
void to_bf16_range(const float* x, uint16_t* y, int64_t n);

// Layer template (layer.cpp)
struct LayerPtrs {
  const float* attn_norm;
  const float* mlp_norm;
  const void* wqkv;
  const void* wo;
  const void* wgu;
  const void* wdown;
};
LayerPtrs bind_layer(const Ctx& c, const void* image);
// B sequences starting at token row row0 of the step's batch (one micro-batch)
int layer_forward(Ctx& c, const LayerPtrs& W, int l, int B, int T, bool recompute, int64_t row0);
int layer_backward(Ctx& c, const LayerPtrs& W, int l, int B, int T, float* grad_unit, int64_t row0, bool first);
int head_forward_backward(Ctx& c, const void* image, int B, int T, float* grad_unit, int64_t row0, bool first,
                          int64_t M_step);

// kernel-timing wrapper: run fn on the compute stream, bracketed by events
int timed(Ctx& c, int cls, double flops, double bytes, const std::function<hipError_t()>& fn);

}  // namespace mt
