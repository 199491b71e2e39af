// One training step: the double-buffered streaming schedule.
//
// "MegaTrain: Full Precision Training of 100B+ Parameter LLMs on a Single
// GPU", abstract: per layer, parameters stream in and gradients stream out; a
// pipelined double-buffered engine overlaps parameter prefetch, computation and
// gradient offload across several streams. "MegaTrain fits 120B LLM training on
// one GPU using CPU RAM", section "Pipelined double buffering": while layer n
// computes, layer n+1 prefetches. "Technical Brief: MegaTrain's Single-GPU
// 120B-Parameter Training Breakthrough", section "Quantifying Host Memory
// Requirements...": gradients are pushed back to the host right after a
// layer's compute.
//
// Three HIP streams: copy-in (unit images host -> layer buffer), compute (the
// layer template's kernels), copy-out (gradients and per-token losses device
// -> host). Compute order: forward of layers 0..L-1, the head (final norm, LM
// head, loss and its backward), then recompute + backward of layers L-1..0.
// Streamed: layer l lives in buffer l % 2 (the head in L % 2), so layer L-1
// is still resident when the backward starts and is not fetched again. A load
// into a buffer waits for the compute that last used it; a gradient item
// waits for the copy-out of the item two before it (two gradient buffers).
//
// Device cache (more than two buffers): "MegaTrain fits 120B LLM training on
// one GPU using CPU RAM", section "Bottom line", and the technical brief's
// "Implementing Host Memory Offloading for Persistent Model State" describe
// device memory as a cache in front of the host store. The head and the top
// layers then keep a buffer each: they are not fetched for their backward,
// and once a unit's AdamW has landed its new image goes into its buffer on
// the copy-in stream (idle in the backward when nothing streams), so the next
// forward does not fetch it. Results are identical to the streamed schedule.
// A host dispatcher loop submits copies only once the compute they depend on
// has completed, enqueues compute with device-side waits on the copies, and
// hands each unit's AdamW to the worker pool as its gradients land; the step
// returns when every update has landed.
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>

#include "kernels.h"
#include "runtime.h"

namespace mt {

namespace {

enum { PH_FWD = MT_PH_FWD, PH_HEAD = MT_PH_HEAD, PH_BWD = MT_PH_BWD };

struct Item {
  int phase;
  int unit;       // layer index, or L for the head
  int buf;
  bool load;
  int prev_user;  // index of the last earlier item using the same buffer, or -1
  int grad_k;     // -1, or the index among gradient-producing items
};

// The step's compute items in order, with their buffers and loads. A
// streamed unit is loaded for its forward, and again for its backward unless
// its buffer's last user was its own forward (layer L-1 at the turn, or the
// last streamed layers below a device cache). A cached unit is loaded for its
// forward only if its buffer does not hold its current image, and never for
// its backward.
std::vector<Item> build_items(const Ctx& c) {
  const int L = c.D.L;
  std::vector<Item> it;
  auto fwd_load = [&](int unit) { return !c.cached(unit) || !c.dev_current[unit]; };
  for (int l = 0; l < L; ++l) it.push_back({PH_FWD, l, c.buf_of(l), fwd_load(l), -1, -1});
  it.push_back({PH_HEAD, L, c.buf_of(L), fwd_load(L), -1, 0});
  for (int l = L - 1; l >= 0; --l) it.push_back({PH_BWD, l, c.buf_of(l), false, -1, L - l});
  for (size_t i = 0; i < it.size(); ++i)
    for (int j = (int)i - 1; j >= 0; --j)
      if (it[j].buf == it[i].buf) { it[i].prev_user = j; break; }
  for (auto& x : it)
    if (x.phase == PH_BWD && !c.cached(x.unit)) x.load = x.prev_user < 0 || it[x.prev_user].unit != x.unit;
  return it;
}

double ms_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

struct StepEvents {
  std::vector<hipEvent_t> loaded, freed, drained;
  std::vector<hipEvent_t> ck_saved, ck_loaded;   // parked checkpoints, by index
  hipEvent_t x0 = nullptr, loss = nullptr, dx0 = nullptr, start = nullptr;
  std::vector<hipEvent_t> trace;   // timing events: per item 6 (load, compute, copy-out)
  std::vector<hipEvent_t> ck_trace;   // per checkpoint index 4 (out, in)
  std::vector<hipEvent_t> refreshed;  // per gradient item: its unit's cache refresh
  std::vector<hipEvent_t> rf_trace;   // per gradient item 2
};

int create_step_events(Ctx& c, StepEvents*& out);
void destroy_step_events(StepEvents* e);

int create_step_events(Ctx& c, StepEvents*& out) {
  auto* e = new StepEvents();
  const int n = 2 * c.D.L + 1;
  auto mk = [&](hipEvent_t& ev, unsigned flags) {
    return hipEventCreateWithFlags(&ev, flags) == hipSuccess;
  };
  bool ok = true;
  const unsigned sync = hipEventDisableTiming;
  const unsigned host = hipEventDisableTiming;
  e->loaded.resize(n);
  e->freed.resize(n);
  e->drained.resize(c.D.L + 1);
  e->ck_saved.resize(c.D.L + 1);
  e->ck_loaded.resize(c.D.L + 1);
  e->refreshed.resize(c.D.L + 1);
  for (auto& ev : e->refreshed) ok &= mk(ev, sync);
  for (auto& ev : e->loaded) ok &= mk(ev, sync);
  for (auto& ev : e->freed) ok &= mk(ev, sync);
  for (auto& ev : e->drained) ok &= mk(ev, host);
  for (auto& ev : e->ck_saved) ok &= mk(ev, sync);
  for (auto& ev : e->ck_loaded) ok &= mk(ev, sync);
  ok &= mk(e->x0, sync);
  ok &= mk(e->loss, host);
  ok &= mk(e->dx0, host);
  ok &= mk(e->start, hipEventBlockingSync);
  if (c.cfg.flags & MT_TRACE) {
    e->trace.resize((size_t)n * 6 + 4);
    for (auto& ev : e->trace) ok &= mk(ev, hipEventDefault);
    e->ck_trace.resize((size_t)(c.D.L + 1) * 4);
    for (auto& ev : e->ck_trace) ok &= mk(ev, hipEventDefault);
    e->rf_trace.resize((size_t)(c.D.L + 1) * 2);
    for (auto& ev : e->rf_trace) ok &= mk(ev, hipEventDefault);
  }
  out = e;
  if (!ok) return set_error(&c, MT_EHIP, "hipEventCreate failed");
  return MT_OK;
}

void destroy_step_events(StepEvents* e) {
  if (!e) return;
  for (auto* v : {&e->loaded, &e->freed, &e->drained, &e->trace, &e->ck_saved, &e->ck_loaded, &e->ck_trace,
                 &e->refreshed, &e->rf_trace})
    for (auto ev : *v)
      if (ev) hipEventDestroy(ev);
  for (auto ev : {e->x0, e->loss, e->dx0, e->start})
    if (ev) hipEventDestroy(ev);
  delete e;
}

#define HIPCK(call)                                                                        \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return set_error(&c, MT_EHIP, std::string(#call ": ") + hipGetErrorString(e_)); \
  } while (0)

// AdamW over element ranges of one unit as a single pool job of chunks of at
// most 1M elements; writes p, m, v and the unit's device image (bf16 mode:
// fp32 gains + bf16 matrices). `uidx` is the unit's index in Ctx::units; the
// unit counts as busy until the job has finished, and the gradient staging
// slot `slot` (or -1) is released then.
static void submit_adamw(Ctx& c, int uidx, const void* g, std::vector<std::pair<int64_t, int64_t>> ranges,
                         const AdamConst& k, int slot, int64_t priority, bool g16 = false, float* g32 = nullptr) {
  constexpr int64_t CH = 1 << 20;
  Unit& u = c.units[uidx];
  auto chunks = std::make_shared<std::vector<std::pair<int64_t, int64_t>>>();
  for (auto& r : ranges)
    for (int64_t a = r.first; a < r.second; a += CH) chunks->push_back({a, std::min(r.second, a + CH)});
  const int dt = c.dtype;
  {
    std::lock_guard<std::mutex> lk(c.amu);
    c.unit_busy[uidx]++;
    c.adam_pending++;
  }
  Ctx* cp = &c;
  c.pool->submit(
      (int64_t)chunks->size(),
      [&u, g, chunks, k, dt, cp, g16, g32](int64_t i) {
        if (i == 0 && cp->delay_adamw_us) std::this_thread::sleep_for(std::chrono::microseconds(cp->delay_adamw_us));
        const auto t0 = std::chrono::steady_clock::now();
        const int64_t a = (*chunks)[i].first, b = (*chunks)[i].second;
        const int64_t mb = u.lay.mat_base;
        // g: fp32, or bf16 widened on the fly (written out to g32 if given)
        auto update = [&](int64_t x, int64_t n, uint16_t* bo, float* f32) {
          if (g16)
            adamw_range_g16(u.p + x, u.m + x, u.v + x, static_cast<const uint16_t*>(g) + x, n, k, bo, f32,
                            g32 ? g32 + x : nullptr);
          else
            adamw_range(u.p + x, u.m + x, u.v + x, static_cast<const float*>(g) + x, n, k, bo, f32);
        };
        if (a < mb) {   // gains region: fp32 in the image
          const int64_t e = std::min(b, mb);
          update(a, e - a, nullptr, (dt && u.shadow) ? static_cast<float*>(u.shadow) + a : nullptr);
        }
        if (b > mb) {   // matrices: bf16 in the image (bf16 mode)
          const int64_t s = std::max(a, mb);
          update(s, b - s,
                 (dt && u.shadow) ? reinterpret_cast<uint16_t*>(static_cast<char*>(u.shadow) + mb * 4) + (s - mb)
                                  : nullptr,
                 nullptr);
        }
        cp->adam_ns.fetch_add((int64_t)(std::chrono::duration<double, std::nano>(
                                            std::chrono::steady_clock::now() - t0).count()));
      },
      [cp, uidx, slot] {
        {
          std::lock_guard<std::mutex> lk(cp->amu);
          cp->unit_busy[uidx]--;
          if (slot >= 0) cp->slot_busy[slot] = 0;
          cp->adam_pending--;
          cp->adam_end[uidx] = std::chrono::steady_clock::now();
        }
        cp->acv.notify_all();
      },
      priority);
}

int train_step_impl(Ctx& c, StepEvents& E, const int32_t* tokens, const int32_t* targets, int B,
                    int T, float* loss_out) {
  const Dims& D = c.D;
  const int L = D.L;
  const int64_t M = (int64_t)B * T;
  const int64_t d = D.d;
  const auto t_begin = std::chrono::steady_clock::now();
  const bool trace = (c.cfg.flags & MT_TRACE) != 0;
  const bool keep = (c.cfg.flags & MT_KEEP_GRADS) != 0;
  const bool overlap = (c.cfg.flags & MT_OVERLAP_OPT) != 0;
  // bf16 gradients cross the link; they (and unkept fp32 ones) go through the staging slots
  const bool g16 = (c.cfg.flags & MT_BF16_GRADS) != 0;
  const bool staged = !keep || g16;
  const size_t gbytes = g16 ? 2 : 4;
  c.kt.on = (c.cfg.flags & MT_KERNEL_TIMING) != 0;
  c.kt.used = 0;
  c.kt.recs.clear();
  c.sched.clear();

  HIPCK(hipEventRecord(E.start, c.s_comp));
  HIPCK(hipEventSynchronize(E.start));
  const auto t_dev0 = std::chrono::steady_clock::now();

  // ---- inputs: targets and the embedding gather x0 = E[tokens] (host) ----
  // (an overlapped update of the embedding from the last step lands first)
  const int64_t limit_ms = c.cfg.wait_timeout_ms;
  {
    std::unique_lock<std::mutex> lk(c.amu);
    auto idle = [&] { return c.unit_busy[L + 1] == 0; };
    if (limit_ms <= 0) {
      c.acv.wait(lk, idle);
    } else if (!c.acv.wait_for(lk, std::chrono::milliseconds(limit_ms), idle)) {
      lk.unlock();
      c.broken = true;
      return set_error(&c, MT_ETIMEOUT, "waited more than " + std::to_string(limit_ms) +
                                            " ms for the previous step's AdamW update of the embedding");
    }
  }
  std::memcpy(c.tgt_host, targets, (size_t)M * 4);
  Unit& emb = c.emb();
  c.pool->run((M + 255) / 256, [&](int64_t i) {
    const int64_t a = i * 256, b = std::min(M, a + 256);
    for (int64_t r = a; r < b; ++r)
      std::memcpy(c.x0_host + r * d, emb.p + (int64_t)tokens[r] * d, (size_t)d * 4);
  });
  HIPCK(hipMemcpyAsync(c.ws.targets, c.tgt_host, (size_t)M * 4, hipMemcpyHostToDevice, c.s_in));
  HIPCK(hipMemcpyAsync(c.ckpt_dev(0), c.x0_host, (size_t)M * d * 4, hipMemcpyHostToDevice, c.s_in));
  HIPCK(hipEventRecord(E.x0, c.s_in));
  double h2d_bytes = (double)M * 4 + (double)M * d * 4, d2h_bytes = 0;

  // rows of the embedding this step touches, with their token positions in
  // (b, t) order (counting sort; deterministic scatter below)
  std::vector<int32_t> cnt(D.V + 1, 0);
  for (int64_t r = 0; r < M; ++r) cnt[tokens[r] + 1]++;
  for (int v = 0; v < D.V; ++v) cnt[v + 1] += cnt[v];
  std::vector<int32_t> pos(M), fill(cnt.begin(), cnt.end() - 1);
  for (int64_t r = 0; r < M; ++r) pos[fill[tokens[r]]++] = (int32_t)r;
  std::vector<int32_t> rows;
  for (int v = 0; v < D.V; ++v)
    if (cnt[v + 1] > cnt[v]) rows.push_back(v);
  // the embedding gradient holds zeros outside the rows written last step
  for (int32_t v : c.prev_rows) std::memset(emb.g + (int64_t)v * d, 0, (size_t)d * 4);
  c.prev_rows = rows;

  const std::vector<Item> items = build_items(c);
  const int n_items = (int)items.size();
  const AdamConst k = adam_const(c.cfg, c.step + 1);

  const int64_t adam_ns0 = c.adam_ns.load();
  std::vector<double> adam_start_ms(L + 2, -1.0);
  bool abort = false;
  double loss_sum = 0.0, forward_ms = 0.0, last_land_ms = 0.0;

  // gradient item kk: 0 = head, kk >= 1 = layer L - kk; units index Ctx::units
  auto grad_uidx = [&](int kk) { return kk == 0 ? L : L - kk; };
  auto grad_unit = [&](int kk) -> Unit& { return c.units[grad_uidx(kk)]; };
  std::vector<int> slot_of(L + 1, -1);
  auto grad_dest = [&](int kk) -> void* { return staged ? (void*)c.ring_slot[slot_of[kk]] : (void*)grad_unit(kk).g; };
  auto unit_id = [&](const Item& it) { return it.phase == PH_HEAD ? MT_UNIT_HEAD : it.unit; };
  // AdamW order: synchronous updates in arrival order (embedding's untouched
  // rows first); overlapped updates in the order the next forward needs them
  auto adam_priority = [&](int uidx) -> int64_t {
    if (overlap) return uidx == L + 1 ? 0 : uidx == L ? L + 1 : 1 + uidx;
    return uidx == L + 1 ? -1 : uidx == L ? 0 : L - uidx;
  };
  auto unit_idle = [&](int uidx) {
    std::lock_guard<std::mutex> lk(c.amu);
    return c.unit_busy[uidx] == 0;
  };
  // a free staging slot that fits gradient item kk (-1: none yet)
  auto take_slot = [&](int kk) -> int {
    std::lock_guard<std::mutex> lk(c.amu);
    const int64_t need = grad_unit(kk).lay.n;
    for (int sidx = 0; sidx < (int)c.ring_slot.size(); ++sidx) {
      if (c.head_slot >= 0 && (sidx == c.head_slot) != (kk == 0)) continue;
      if (!c.slot_busy[sidx] && c.ring_elems[sidx] >= need) {
        c.slot_busy[sidx] = 1;
        return sidx;
      }
    }
    return -1;
  };
  auto free_slot = [&](int sidx) {
    if (sidx < 0) return;
    std::lock_guard<std::mutex> lk(c.amu);
    c.slot_busy[sidx] = 0;
  };

  // ---- host dispatcher ----
  // Copies are submitted only once the compute they depend on has completed
  // (observed by polling its event), so no copy ever waits on the device; the
  // compute stream waits on copy events on the device. Compute therefore runs
  // at most two items ahead of the GPU, which is ample: submitting one layer
  // takes a small fraction of its compute time.
  int rc = MT_OK;
  auto trace_ev = [&](int i, int slot) -> hipEvent_t { return E.trace[(size_t)i * 6 + slot]; };
  struct HostSpan { int phase, unit; double t0, t1; };
  std::vector<HostSpan> host_spans;
  auto span = [&](int phase, int unit, std::chrono::steady_clock::time_point a) {
    if (trace)
      host_spans.push_back({phase, unit, std::chrono::duration<double, std::milli>(a - t_begin).count(),
                            ms_since(t_begin)});
  };
  std::vector<char> computed(n_items, 0), done_seen(n_items, 0), load_issued(n_items, 0);
  std::vector<int> loads, grad_item(L + 1, -1);
  for (int i = 0; i < n_items; ++i) {
    if (items[i].load) loads.push_back(i);
    if (items[i].grad_k >= 0) grad_item[items[i].grad_k] = i;
  }
  const int head_item = L;
  auto item_done = [&](int i) -> int {   // 1 done, 0 not yet, <0 error
    if (!computed[i]) return 0;
    if (done_seen[i]) return 1;
    const hipError_t r = hipEventQuery(E.freed[i]);
    if (r == hipSuccess) { done_seen[i] = 1; return 1; }
    if (r == hipErrorNotReady) return 0;
    return set_error(&c, MT_EHIP, std::string("hipEventQuery: ") + hipGetErrorString(r));
  };
  auto event_done = [&](hipEvent_t e) -> int {
    const hipError_t r = hipEventQuery(e);
    if (r == hipSuccess) return 1;
    if (r == hipErrorNotReady) return 0;
    return set_error(&c, MT_EHIP, std::string("hipEventQuery: ") + hipGetErrorString(r));
  };
  std::vector<char> grad_issued(L + 1, 0);
  const bool show_progress = (c.cfg.flags & MT_PROGRESS) != 0;
  int next_shown = 0;
  size_t next_l = 0;
  int next_c = 0, next_g = 0, next_a = 0;
  bool loss_issued = false, loss_checked = false, dx0_issued = false, dx0_done = false;

  // parked residual checkpoints (see Ctx::ckpt_dev): x_i, i in [1, kpark],
  // goes to the pinned bounce slab bounce[i % 2] once the forward that wrote
  // it has finished (and the pool has copied x_{i-2} out of that slab), then
  // the pool copies it into its pageable host slab. In the backward the pool
  // copies x_j back into bounce[j % 2] (once x_{j+2} has left it), and x_j,
  // j in [0, kpark], comes back into stage[j % 2] once the last reader of
  // x_{j+2} (which shares that stage) has finished; x_0 comes straight from
  // the gathered embedding rows
  const int nh = c.ck_nh, kpark = nh ? nh - 3 : 0;
  const size_t ck_bytes = (size_t)M * d * 4;
  std::vector<char> save_issued(L + 1, 0), reload_issued(L + 1, 0);
  int next_s = 1, next_r = kpark;
  auto ck_ev = [&](int i, int slot) -> hipEvent_t { return E.ck_trace[(size_t)i * 4 + slot]; };
  // host side of parking: the pool copies bounce[i % 2] -> slab after x_i's
  // D2H (cp_out), and slab -> bounce[j % 2] before x_j's H2D (cp_in); the
  // flags are set by the copy jobs, which all finish before the step returns
  std::unique_ptr<std::atomic<char>[]> cp_out(new std::atomic<char>[L + 1]()), cp_in(new std::atomic<char>[L + 1]());
  std::atomic<int> ck_jobs{0};
  int next_co = 1, next_ci = kpark;
  auto host_copy = [&](float* dst, const float* src, std::atomic<char>* flag) {
    const size_t ch = (size_t)64 << 20;
    const int64_t n = (int64_t)((ck_bytes + ch - 1) / ch);
    ck_jobs.fetch_add(1);
    c.pool->submit(
        n,
        [dst, src, ch, bytes = ck_bytes](int64_t t) {
          const size_t a = (size_t)t * ch, b = std::min(bytes, a + ch);
          std::memcpy(reinterpret_cast<char*>(dst) + a, reinterpret_cast<const char*>(src) + a, b - a);
        },
        [flag, &ck_jobs] {
          flag->store(1);
          ck_jobs.fetch_sub(1);
        },
        INT64_MIN + 1);
  };
  auto issue_save = [&](int i) -> int {
    if (trace) HIPCK(hipEventRecord(ck_ev(i, 0), c.s_out));
    HIPCK(hipMemcpyAsync(c.bounce[i & 1], c.stage[i & 1], ck_bytes, hipMemcpyDeviceToHost, c.s_out));
    if (trace) HIPCK(hipEventRecord(ck_ev(i, 1), c.s_out));
    HIPCK(hipEventRecord(E.ck_saved[i], c.s_out));
    save_issued[i] = 1;
    d2h_bytes += (double)ck_bytes;
    return MT_OK;
  };
  auto issue_reload = [&](int j) -> int {
    const float* src = j == 0 ? c.x0_host : c.bounce[j & 1];
    if (trace) HIPCK(hipEventRecord(ck_ev(j, 2), c.s_in));
    HIPCK(hipMemcpyAsync(c.stage[j & 1], src, ck_bytes, hipMemcpyHostToDevice, c.s_in));
    if (trace) HIPCK(hipEventRecord(ck_ev(j, 3), c.s_in));
    HIPCK(hipEventRecord(E.ck_loaded[j], c.s_in));
    reload_issued[j] = 1;
    h2d_bytes += (double)ck_bytes;
    return MT_OK;
  };
  // forward of layer l overwrites stage[(l+1) % 2], which held x_{l-1}
  auto fwd_needs_save = [&](int l) { return nh && l + 1 < nh && l - 1 >= 1 && l - 1 <= kpark; };
  auto bwd_needs_reload = [&](int l) { return nh && l <= kpark; };

  // test hook: NaN over every tensor of a unit-layout buffer (an image, or a
  // gradient slab with elem_bytes 4), leaving the alignment padding alone
  auto poison_unit = [&](void* base, const UnitLayout& lay, int unit, int image_dtype,
                         hipStream_t s) -> int {
    const int64_t dd = d, n_groups = unit == L ? 2 : 6;
    const int64_t len_layer[6] = {dd, dd, (int64_t)D.qkvd * dd, dd * D.qd, 2LL * D.F * dd, dd * D.F};
    const int64_t len_head[2] = {dd, (int64_t)D.V * dd};
    for (int64_t gi = 0; gi < n_groups; ++gi) {
      const int64_t e0 = lay.off[gi], n = unit == L ? len_head[gi] : len_layer[gi];
      const size_t b0 = image_dtype < 0 ? (size_t)e0 * 4 : lay.image_offset(e0, image_dtype);
      const size_t b1 = image_dtype < 0 ? (size_t)(e0 + n) * 4 : lay.image_offset(e0 + n, image_dtype);
      HIPCK(hipMemsetAsync(static_cast<char*>(base) + b0, 0xFF, b1 - b0, s));
    }
    return MT_OK;
  };
  auto issue_load = [&](int j) -> int {
    const Item& it = items[j];
    const Unit& u = it.phase == PH_HEAD ? c.head() : c.layer(it.unit);
    const size_t bytes = u.lay.image_bytes(c.dtype);
    if (c.delay_h2d_us) std::this_thread::sleep_for(std::chrono::microseconds(c.delay_h2d_us));
    if (c.poison) {
      const int rp = poison_unit(c.buf[it.buf], u.lay, it.phase == PH_HEAD ? L : it.unit, c.dtype, c.s_in);
      if (rp) return rp;
    }
    if (trace) HIPCK(hipEventRecord(trace_ev(j, 0), c.s_in));
    const auto hq = std::chrono::steady_clock::now();
    HIPCK(hipMemcpyAsync(c.buf[it.buf], u.image(), bytes, hipMemcpyHostToDevice, c.s_in));
    span(MT_PH_LOAD, unit_id(it), hq);
    if (trace) HIPCK(hipEventRecord(trace_ev(j, 1), c.s_in));
    HIPCK(hipEventRecord(E.loaded[j], c.s_in));
    load_issued[j] = 1;
    h2d_bytes += (double)bytes;
    if (c.cached(it.unit)) c.dev_current[it.unit] = 1;
    return MT_OK;
  };
  // device cache: the updated image of gradient item kk's unit into its own
  // buffer, for the next step
  std::vector<char> rf_issued(L + 1, 0);
  int rf_last = -1;   // the refresh in flight (one at a time, so a load that
                      // becomes ready waits behind at most one)
  auto issue_refresh = [&](int kk) -> int {
    const int ui = grad_uidx(kk);
    const Unit& u = c.units[ui];
    const size_t bytes = u.lay.image_bytes(c.dtype);
    if (trace) HIPCK(hipEventRecord(E.rf_trace[(size_t)kk * 2], c.s_in));
    HIPCK(hipMemcpyAsync(c.buf[c.buf_of(ui)], u.image(), bytes, hipMemcpyHostToDevice, c.s_in));
    if (trace) HIPCK(hipEventRecord(E.rf_trace[(size_t)kk * 2 + 1], c.s_in));
    HIPCK(hipEventRecord(E.refreshed[kk], c.s_in));
    rf_issued[kk] = 1;
    rf_last = kk;
    h2d_bytes += (double)bytes;
    c.dev_current[ui] = 1;
    return MT_OK;
  };
  auto issue_compute = [&](int i) -> int {
    const Item& it = items[i];
    if (it.load) HIPCK(hipStreamWaitEvent(c.s_comp, E.loaded[i], 0));
    if (i == 0) HIPCK(hipStreamWaitEvent(c.s_comp, E.x0, 0));
    if (it.phase == PH_FWD && fwd_needs_save(it.unit))
      HIPCK(hipStreamWaitEvent(c.s_comp, E.ck_saved[it.unit - 1], 0));
    if (it.phase == PH_BWD && bwd_needs_reload(it.unit))
      HIPCK(hipStreamWaitEvent(c.s_comp, E.ck_loaded[it.unit], 0));
    if (it.grad_k >= 2) HIPCK(hipStreamWaitEvent(c.s_comp, E.drained[it.grad_k - 2], 0));
    if (trace) HIPCK(hipEventRecord(trace_ev(i, 2), c.s_comp));
    float* gdev = it.grad_k >= 0 ? c.gbuf[it.grad_k % 2] : nullptr;
    const auto hc = std::chrono::steady_clock::now();
    int r = MT_OK;
    // the batch in micro-batches of at most mb_seqs sequences, in order
    for (int b0 = 0; b0 < B && !r; b0 += c.mb_seqs) {
      const int bj = std::min(c.mb_seqs, B - b0);
      const int64_t row0 = (int64_t)b0 * T;
      if (it.phase == PH_FWD)
        r = layer_forward(c, bind_layer(c, c.buf[it.buf]), it.unit, bj, T, false, row0);
      else if (it.phase == PH_HEAD)
        r = head_forward_backward(c, c.buf[it.buf], bj, T, gdev, row0, b0 == 0, M);
      else
        r = layer_backward(c, bind_layer(c, c.buf[it.buf]), it.unit, bj, T, gdev, row0, b0 == 0);
    }
    if (r) return r;
    if (g16 && gdev) {
      // the unit's gradient slab as bf16 for the link
      const Unit& gu = it.phase == PH_HEAD ? c.head() : c.layer(it.unit);
      void* g16dev = c.gbuf16[it.grad_k % 2];
      const int64_t n = gu.lay.n;
      r = timed(c, K_CAST, 0, (double)n * 6, [&] { return cast(MT_BF16, gdev, g16dev, n, c.s_comp); });
      if (r) return r;
    }
    span(it.phase, unit_id(it), hc);
    if (trace) HIPCK(hipEventRecord(trace_ev(i, 3), c.s_comp));
    HIPCK(hipEventRecord(E.freed[i], c.s_comp));
    computed[i] = 1;
    return MT_OK;
  };
  auto issue_grad = [&](int kk) -> int {
    const int i = grad_item[kk];
    const Unit& u = grad_unit(kk);
    if (c.delay_d2h_us) std::this_thread::sleep_for(std::chrono::microseconds(c.delay_d2h_us));
    if (trace) HIPCK(hipEventRecord(trace_ev(i, 4), c.s_out));
    const auto hg = std::chrono::steady_clock::now();
    HIPCK(hipMemcpyAsync(grad_dest(kk), g16 ? c.gbuf16[kk % 2] : (void*)c.gbuf[kk % 2], (size_t)u.lay.n * gbytes,
                         hipMemcpyDeviceToHost, c.s_out));
    span(MT_PH_GRAD, unit_id(items[i]), hg);
    if (trace) HIPCK(hipEventRecord(trace_ev(i, 5), c.s_out));
    if (c.poison) {
      const int rp = poison_unit(c.gbuf[kk % 2], u.lay, kk == 0 ? L : L - kk, -1, c.s_out);
      if (rp) return rp;
    }
    HIPCK(hipEventRecord(E.drained[kk], c.s_out));
    grad_issued[kk] = 1;
    d2h_bytes += (double)u.lay.n * gbytes;
    return MT_OK;
  };
  auto issue_loss = [&]() -> int {
    HIPCK(hipMemcpyAsync(c.loss_host, c.ws.tok_loss, (size_t)M * 4, hipMemcpyDeviceToHost, c.s_out));
    HIPCK(hipEventRecord(E.loss, c.s_out));
    d2h_bytes += (double)M * 4;
    return MT_OK;
  };
  auto issue_dx0 = [&]() -> int {
    HIPCK(hipMemcpyAsync(c.dx0_host, c.ws.g_f, (size_t)M * d * 4, hipMemcpyDeviceToHost, c.s_out));
    HIPCK(hipEventRecord(E.dx0, c.s_out));
    d2h_bytes += (double)M * d * 4;
    return MT_OK;
  };
  auto start_emb_untouched = [&] {
    // embedding rows this step does not touch have a zero gradient: their
    // update can run now, overlapping the backward
    int64_t prev = 0;
    std::vector<std::pair<int64_t, int64_t>> runs;
    for (int32_t v : rows) {
      if (v > prev) runs.push_back({prev, v});
      prev = v + 1;
    }
    if (prev < D.V) runs.push_back({prev, D.V});
    for (auto& rr : runs) rr = {rr.first * d, rr.second * d};
    adam_start_ms[L + 1] = ms_since(t_begin);
    submit_adamw(c, L + 1, emb.g, std::move(runs), k, -1, adam_priority(L + 1));
  };

  // what the dispatcher waits for, for the error of a wait that exceeded its limit
  auto item_name = [&](int i) {
    const Item& it = items[i];
    return std::string(it.phase == PH_FWD ? "forward of layer " : it.phase == PH_HEAD ? "head" : "backward of layer ") +
           (it.phase == PH_HEAD ? "" : std::to_string(it.unit));
  };
  auto unit_name = [&](int uidx) {
    return uidx < L ? "layer " + std::to_string(uidx) : uidx == L ? std::string("head") : std::string("embedding");
  };
  auto pending = [&]() {
    std::string w;
    auto add = [&](const std::string& x) { w += (w.empty() ? "" : "; ") + x; };
    if (next_l < loads.size()) {
      const int j = loads[next_l], p = items[j].prev_user;
      const int ui = items[j].phase == PH_HEAD ? L : items[j].unit;
      if (p >= 0 && !done_seen[p]) add("load of " + unit_name(ui) + " (its buffer's last user, the " + item_name(p) +
                                       ", has not finished)");
      else add("load of " + unit_name(ui) + " (its AdamW update has not landed)");
    }
    if (next_c < n_items) add("the " + item_name(next_c) + " (its inputs have not been issued)");
    if (loss_issued && next_g <= L)
      add("gradient copy of " + unit_name(grad_uidx(next_g)) +
          (computed[grad_item[next_g]] && done_seen[grad_item[next_g]] ? " (no free staging slot)"
                                                                       : " (its compute has not finished)"));
    if (next_a < next_g) add("gradients of " + unit_name(grad_uidx(next_a)) + " landing in host memory");
    if (dx0_issued && !dx0_done) add("input gradient of layer 0 landing in host memory");
    if (nh && next_s <= kpark) add("checkpoint " + std::to_string(next_s) + " leaving the device");
    if (nh && next_r >= 0) add("checkpoint " + std::to_string(next_r) + " returning to the device");
    return w.empty() ? std::string("nothing issued") : w;
  };
  auto t_progress = std::chrono::steady_clock::now();

  for (;;) {
    bool progress = false;
    // loads, in order, once the buffer's previous user has finished (and,
    // with overlapped updates, once the unit's last update has landed)
    while (next_l < loads.size()) {
      const int j = loads[next_l];
      const int p = items[j].prev_user;
      if (p >= 0) {
        const int st = item_done(p);
        if (st < 0) { rc = st; break; }
        if (!st) break;
      }
      if (overlap && items[j].phase != PH_BWD && !unit_idle(items[j].phase == PH_HEAD ? L : items[j].unit)) break;
      if ((rc = issue_load(j))) break;
      ++next_l;
      progress = true;
    }
    if (rc) break;
    // parked checkpoints out, in order, once the forward that wrote them is
    // done and their bounce slab has been copied out of
    while (next_s <= kpark) {
      const int st = item_done(next_s - 1);
      if (st < 0) { rc = st; break; }
      if (!st) break;
      if (next_s - 2 >= 1 && !cp_out[next_s - 2].load()) break;
      if ((rc = issue_save(next_s))) break;
      ++next_s;
      progress = true;
    }
    if (rc) break;
    // bounce -> parked slab once the D2H has landed
    while (next_co < next_s) {
      const int st = event_done(E.ck_saved[next_co]);
      if (st < 0) { rc = st; break; }
      if (!st) break;
      host_copy(c.ck_host[next_co - 1], c.bounce[next_co & 1], &cp_out[next_co]);
      ++next_co;
      progress = true;
    }
    if (rc) break;
    // parked slab -> bounce, in backward order, once the slab is whole and
    // the bounce slab's previous H2D (x_{j+2}) has landed
    while (nh && next_ci >= 1) {
      const int j = next_ci;
      if (!cp_out[j].load()) break;
      if (j + 2 <= kpark) {
        if (!reload_issued[j + 2]) break;
        const int st = event_done(E.ck_loaded[j + 2]);
        if (st < 0) { rc = st; break; }
        if (!st) break;
      }
      host_copy(c.bounce[j & 1], c.ck_host[j - 1], &cp_in[j]);
      --next_ci;
      progress = true;
    }
    if (rc) break;
    // and back, in backward order, once the stage they return to is free
    while (next_r >= 0 && nh) {
      const int reader = next_r + 2 == L ? head_item : 2 * L - (next_r + 2);
      const int st = item_done(reader);
      if (st < 0) { rc = st; break; }
      if (!st) break;
      if (next_r >= 1 && !cp_in[next_r].load()) break;
      if ((rc = issue_reload(next_r))) break;
      --next_r;
      progress = true;
    }
    if (rc) break;
    // next compute item, once its weights and its gradient buffer are on their way
    if (next_c < n_items) {
      const Item& it = items[next_c];
      bool ready = (!it.load || load_issued[next_c]) && (it.grad_k < 2 || grad_issued[it.grad_k - 2]);
      if (it.phase == PH_FWD && fwd_needs_save(it.unit)) ready = ready && save_issued[it.unit - 1];
      if (it.phase == PH_BWD && bwd_needs_reload(it.unit)) ready = ready && reload_issued[it.unit];
      if (ready) {
        if ((rc = issue_compute(next_c))) break;
        ++next_c;
        progress = true;
      }
    }
    // progress lines, as compute items finish in order
    while (show_progress && next_shown < next_c) {
      const int st = event_done(E.freed[next_shown]);
      if (st < 0) { rc = st; break; }
      if (!st) break;
      const Item& it = items[next_shown];
      fprintf(stderr, "[mt] step %lld: %s %d done at %.1f ms\n", (long long)c.step + 1,
              it.phase == PH_FWD ? "forward layer" : it.phase == PH_HEAD ? "head" : "backward layer",
              it.phase == PH_HEAD ? 0 : it.unit, ms_since(t_begin));
      fflush(stderr);
      ++next_shown;
    }
    if (rc) break;
    // per-token losses once the head has run
    if (!loss_issued) {
      const int st = item_done(head_item);
      if (st < 0) { rc = st; break; }
      if (st) {
        if ((rc = issue_loss())) break;
        loss_issued = progress = true;
      }
    }
    if (loss_issued && !loss_checked) {
      const int st = event_done(E.loss);
      if (st < 0) { rc = st; break; }
      if (st) {
        for (int64_t r = 0; r < M; ++r) loss_sum += (double)c.loss_host[r];
        forward_ms = ms_since(t_begin);
        abort = !std::isfinite(loss_sum);
        if (!abort) start_emb_untouched();
        loss_checked = progress = true;
      }
    }
    // gradient copies, in order, once their compute has finished (and, with
    // the staging ring, once a slot is free: its last AdamW has finished)
    while (loss_issued && next_g <= L) {
      const int st = item_done(grad_item[next_g]);
      if (st < 0) { rc = st; break; }
      if (!st) break;
      if (staged) {
        const int sidx = take_slot(next_g);
        if (sidx < 0) break;
        slot_of[next_g] = sidx;
      }
      if ((rc = issue_grad(next_g))) break;
      ++next_g;
      progress = true;
    }
    if (rc) break;
    // AdamW of each unit as its gradients land (after the loss is known finite)
    while (loss_checked && next_a < next_g) {
      const int st = event_done(E.drained[next_a]);
      if (st < 0) { rc = st; break; }
      if (!st) break;
      last_land_ms = ms_since(t_begin);
      const int kk = next_a, ui = grad_uidx(kk);
      if (!abort) {
        adam_start_ms[ui] = last_land_ms;
        c.dev_current[ui] = 0;
        submit_adamw(c, ui, grad_dest(kk), {{0, c.units[ui].lay.n}}, k, staged ? slot_of[kk] : -1,
                     adam_priority(ui), g16, (g16 && keep) ? c.units[ui].g : nullptr);
      } else if (staged) {
        free_slot(slot_of[kk]);
      }
      ++next_a;
      progress = true;
    }
    if (rc) break;
    // cached units whose update has landed: refresh their buffers, in any
    // order, after every load that could be issued
    const bool refresh = c.ncache && !abort && !(c.cfg.flags & MT_CACHE_NO_REFRESH);
    const int rf_free = refresh ? (rf_last < 0 ? 1 : event_done(E.refreshed[rf_last])) : 0;
    if (rf_free < 0) { rc = rf_free; break; }
    if (rf_free) {
      for (int kk = 0; kk < next_a; ++kk) {
        if (rf_issued[kk] || !c.cached(grad_uidx(kk)) || !unit_idle(grad_uidx(kk))) continue;
        if ((rc = issue_refresh(kk))) break;
        progress = true;
        break;
      }
      if (rc) break;
    }
    // the input gradient of layer 0 goes to the host for the embedding scatter
    if (!dx0_issued && next_g > L) {
      if ((rc = issue_dx0())) break;
      dx0_issued = progress = true;
    }
    if (dx0_issued && !dx0_done) {
      const int st = event_done(E.dx0);
      if (st < 0) { rc = st; break; }
      if (st) dx0_done = progress = true;
    }
    if (dx0_done && next_a > L) break;
    if (progress) {
      t_progress = std::chrono::steady_clock::now();
    } else {
      if (limit_ms > 0 && ms_since(t_progress) > (double)limit_ms) {
        rc = set_error(&c, MT_ETIMEOUT, "no progress for " + std::to_string(limit_ms) + " ms; waiting for: " + pending());
        break;
      }
      std::this_thread::sleep_for(std::chrono::microseconds(10));
    }
  }
  // the checkpoint copy jobs read and write this step's state (they are plain
  // host copies): let them finish, whatever the limit
  while (ck_jobs.load()) std::this_thread::sleep_for(std::chrono::microseconds(20));
  if (rc == MT_ETIMEOUT) {
    // work already issued stays in flight (mt_destroy waits for the device;
    // the state accessors wait for the updates)
    c.broken = true;
    std::fill(c.dev_current.begin(), c.dev_current.end(), 0);
    return rc;
  }
  if (rc) {
    // drain what was submitted before reporting the error
    hipStreamSynchronize(c.s_in);
    hipStreamSynchronize(c.s_comp);
    hipStreamSynchronize(c.s_out);
    adam_drain(c);
    std::fill(c.dev_current.begin(), c.dev_current.end(), 0);
    {
      std::lock_guard<std::mutex> lk(c.amu);
      std::fill(c.slot_busy.begin(), c.slot_busy.end(), 0);
    }
    return rc;
  }

  // ---- embedding: dE[v] += dx0[r] over positions r of token v, in increasing r ----
  last_land_ms = ms_since(t_begin);
  if (!abort) {
    const int64_t nr = (int64_t)rows.size();
    const int64_t per = 64;
    c.pool->run((nr + per - 1) / per, [&](int64_t i) {
      for (int64_t j = i * per; j < std::min(nr, (i + 1) * per); ++j) {
        const int32_t v = rows[j];
        float* dst = emb.g + (int64_t)v * d;
        for (int32_t q = cnt[v]; q < cnt[v + 1]; ++q) {
          const float* src = c.dx0_host + (int64_t)pos[q] * d;
          for (int64_t e = 0; e < d; ++e) dst[e] += src[e];
        }
      }
    });
    // AdamW of the touched rows, in runs of consecutive rows
    std::vector<std::pair<int64_t, int64_t>> runs;
    size_t a = 0;
    while (a < rows.size()) {
      size_t b = a + 1;
      while (b < rows.size() && rows[b] == rows[b - 1] + 1) ++b;
      runs.push_back({(int64_t)rows[a] * d, (int64_t)(rows[b - 1] + 1) * d});
      a = b;
    }
    submit_adamw(c, L + 1, emb.g, std::move(runs), k, -1, adam_priority(L + 1));
  }
  // synchronous mode: every update lands before the step returns
  if (!overlap) {
    const int ra = adam_drain_for(c, limit_ms, "end of step");
    if (ra) {
      c.broken = true;
      std::fill(c.dev_current.begin(), c.dev_current.end(), 0);
      return ra;
    }
  }
  const hipError_t s1 = hipStreamSynchronize(c.s_in), s2 = hipStreamSynchronize(c.s_comp),
                   s3 = hipStreamSynchronize(c.s_out);
  if (s1 != hipSuccess || s2 != hipSuccess || s3 != hipSuccess) {
    std::fill(c.dev_current.begin(), c.dev_current.end(), 0);
    return set_error(&c, MT_EHIP, std::string("stream synchronize: ") +
                                      hipGetErrorString(s1 != hipSuccess ? s1 : s2 != hipSuccess ? s2 : s3));
  }

  const double step_ms = ms_since(t_begin);
  const double loss = loss_sum / (double)M;
  c.token_loss.assign(c.loss_host, c.loss_host + M);

  // ---- statistics ----
  mt_step_stats& st = c.stats;
  st = mt_step_stats{};
  st.step_ms = step_ms;
  st.forward_ms = forward_ms;
  st.h2d_bytes = h2d_bytes;
  st.d2h_bytes = d2h_bytes;
  st.adamw_ms = (double)(c.adam_ns.load() - adam_ns0) * 1e-6;
  // read p, m, v, g; write p, m, v (+ the bf16 image of streamed units; +
  // the widened fp32 gradient when bf16 gradients are kept). The embedding's
  // gradient is formed on the host in fp32 and has no device image.
  const double n_emb = (double)c.emb().lay.n, n_str = (double)(L + 0) * c.units[0].lay.n + c.head().lay.n;
  st.adamw_bytes = n_emb * 28.0 +
                   n_str * (12.0 + (double)gbytes + 12.0 + (c.dtype ? 2.0 : 0.0) + (g16 && keep ? 4.0 : 0.0));
  st.tail_ms = step_ms - last_land_ms;
  st.tokens = M;
  {
    const double Nl = (double)D.qkvd * d + (double)d * D.qd + 3.0 * d * D.F;
    const double Nh = (double)D.V * d;
    const double Af = 2.0 * B * (double)T * T * D.H * D.hd;
    st.model_flops = 6.0 * (Nl * L + Nh) * (double)M + 3.0 * L * Af;
    st.hw_flops = st.model_flops + L * (2.0 * (Nl - (double)d * D.F) * (double)M + Af);
  }
  if (trace) {
    float t;
    auto rel = [&](hipEvent_t e) {
      return hipEventElapsedTime(&t, E.start, e) == hipSuccess ? (double)t : -1.0;
    };
    for (int i = 0; i < n_items; ++i) {
      const Item& it = items[i];
      const int unit = it.phase == PH_HEAD ? MT_UNIT_HEAD : it.unit;
      if (it.load) {
        const double a = rel(trace_ev(i, 0)), b = rel(trace_ev(i, 1));
        c.sched.push_back({MT_PH_LOAD, unit, it.buf, 0, a, b});
        st.h2d_busy_ms += b - a;
      }
      const double a = rel(trace_ev(i, 2)), b = rel(trace_ev(i, 3));
      c.sched.push_back({it.phase, unit, it.buf, 1, a, b});
      st.compute_busy_ms += b - a;
      if (it.grad_k >= 0) {
        const double a2 = rel(trace_ev(i, 4)), b2 = rel(trace_ev(i, 5));
        c.sched.push_back({MT_PH_GRAD, unit, it.grad_k % 2, 2, a2, b2});
        st.d2h_busy_ms += b2 - a2;
      }
    }
    for (int kk = 0; kk <= L; ++kk) {
      if (!rf_issued[kk]) continue;
      const double a = rel(E.rf_trace[(size_t)kk * 2]), b = rel(E.rf_trace[(size_t)kk * 2 + 1]);
      const int ui = grad_uidx(kk);
      c.sched.push_back({MT_PH_REFRESH, ui == L ? MT_UNIT_HEAD : ui, c.buf_of(ui), 0, a, b});
      st.h2d_busy_ms += b - a;
    }
    for (int i = 1; i <= kpark; ++i) {
      const double a = rel(ck_ev(i, 0)), b = rel(ck_ev(i, 1));
      c.sched.push_back({MT_PH_CKPT_OUT, i, i & 1, 2, a, b});
      st.d2h_busy_ms += b - a;
    }
    for (int j = 0; j <= kpark && nh; ++j) {
      const double a = rel(ck_ev(j, 2)), b = rel(ck_ev(j, 3));
      c.sched.push_back({MT_PH_CKPT_IN, j, j & 1, 0, a, b});
      st.h2d_busy_ms += b - a;
    }
    // host AdamW entries on the same clock (device times are relative to the
    // start event, host times to the moment it completed)
    const double off = std::chrono::duration<double, std::milli>(t_dev0 - t_begin).count();
    // (an update still running, overlapped into the next step, is left out)
    for (int kk = 0; kk <= L + 1; ++kk) {
      const int ui = kk <= L ? grad_uidx(kk) : L + 1;
      if (adam_start_ms[ui] < 0) continue;
      std::chrono::steady_clock::time_point te;
      {
        std::lock_guard<std::mutex> lk(c.amu);
        if (c.unit_busy[ui]) continue;
        te = c.adam_end[ui];
      }
      const double end_ms = std::chrono::duration<double, std::milli>(te - t_begin).count();
      const int unit = ui == L ? MT_UNIT_HEAD : ui == L + 1 ? MT_UNIT_EMB : ui;
      c.sched.push_back({MT_PH_ADAMW, unit, -1, 3, adam_start_ms[ui] - off, end_ms - off});
    }
    for (auto& h : host_spans) c.sched.push_back({h.phase, h.unit, -1, 4, h.t0 - off, h.t1 - off});
  }
  if (c.kt.on) {
    c.kstats.assign(K_COUNT * 2, mt_kernel_stat{});
    static const char* names[K_COUNT] = {"gemm_nt", "gemm_nn", "gemm_tn", "attn_fwd", "attn_bwd",
                                         "rmsnorm_fwd", "rmsnorm_bwd", "rope", "swiglu", "xent",
                                         "cast", "other"};
    for (int i = 0; i < K_COUNT; ++i)
      snprintf(c.kstats[i].name, sizeof(c.kstats[i].name), "%s_%s", names[i], c.dtype ? "bf16" : "fp32");
    for (auto& r : c.kt.recs) {
      float t = 0.f;
      hipEventElapsedTime(&t, c.kt.ev[r.e], c.kt.ev[r.e + 1]);
      mt_kernel_stat& s = c.kstats[r.cls];
      s.launches++;
      s.ms += t;
      s.flops += r.flops;
      s.bytes += r.bytes;
    }
    c.kstats.resize(K_COUNT);
  }

  if (abort) return set_error(&c, MT_ENONFINITE, "loss is not finite; no update applied");
  c.step++;
  st.step = c.step;
  if (loss_out) *loss_out = (float)loss;
  return MT_OK;
}

}  // namespace mt
