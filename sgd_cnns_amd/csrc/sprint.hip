// SPRINT's worker and update threads on one GPU (SPRINT report, IPSJ SIG
// Technical Report Vol.2016-HPC-155 No.8, section 3.4: Algorithm 1 for a
// GPU worker, Algorithm 2 for the updater; eq. (9) for the average
// minibatch an update applies).
//
// Every worker is a host thread with its own HIP stream, weight copy,
// gradient sum and gradient buffer GradBuf_t; the updater is a host thread
// with its own stream that owns LatestWeights.  The report's mutexes are
// host mutexes here.  Under each lock the thread that changes a buffer's
// state records a HIP event, and the thread that takes the buffer next makes
// its stream wait for that event, so the device work follows the order the
// locks decide:
//   GradBuf_t  worker add  --written-->  updater's fused sum+apply
//              updater read --released--> worker's next copy into it
//   W          update       --w_ready-->  worker's fetch copy
//              fetch copy   --fetch_done--> the next update of W
// A buffer the updater has taken but not yet released is TAKEN: a worker
// that wants to push then waits on the buffer's condition variable (the
// release follows the apply's enqueue within microseconds).

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <chrono>
#include <condition_variable>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "common.h"

namespace {

using Clock = std::chrono::steady_clock;

double ms_between(Clock::time_point a, Clock::time_point b) {
  return std::chrono::duration<double, std::milli>(b - a).count();
}

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

enum BufState { BUF_EMPTY, BUF_FULL, BUF_TAKEN };

struct Buf {
  std::mutex mu;
  std::condition_variable cv;  // a taken buffer was released
  BufState state = BUF_EMPTY;
  sgd_gradbuf gb{};
  hipEvent_t written = nullptr;   // the last push into the buffer (worker stream)
  hipEvent_t released = nullptr;  // the last update that read it (update stream)
  bool released_valid = false;
  std::vector<int64_t> steps;     // log indices of the steps it holds, in push order
};

struct Worker {
  sgd_net* net = nullptr;
  hipStream_t stream = nullptr;
  hipEvent_t fetch_done = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  float* w = nullptr;     // its copy of the weights
  float* sum = nullptr;   // Grad, summed over n_push steps
  float* loss = nullptr;
  double step_ms = 0.0;   // summed over its steps
  int64_t fetches = 0;
};

struct Run {
  sgd_sprint_config cfg{};
  int device = 0;
  int64_t n = 0;             // parameters
  int batch = 0;             // N_Subbatch
  int64_t x_floats = 0;      // floats per sub-batch of X
  float* W = nullptr;
  float* state = nullptr;
  sgd_rule rule{};
  const float* X = nullptr;
  const int32_t* y = nullptr;
  int64_t n_batches = 0;

  std::vector<Worker> workers;
  std::vector<std::unique_ptr<Buf>> bufs;
  hipStream_t us = nullptr;  // the updater's stream

  // LatestWeights and its lock (LockWeights).
  std::mutex wmu;
  std::condition_variable wcv;  // a new version was published
  int64_t version = 0;
  hipEvent_t w_ready = nullptr;
  bool w_ready_valid = false;
  std::vector<char> fetch_pending;

  // The updater sleeps on umu/ucv until enough buffers are full.
  std::mutex umu;
  std::condition_variable ucv;
  std::atomic<int> n_full{0};
  std::atomic<int> finished{0};
  std::atomic<bool> stop{false};
  std::atomic<int64_t> next_batch{0};

  std::mutex emu;
  int err = 0;
  std::string msg;

  // Failure injection for the error-path tests (environment variable
  // SGD_SPRINT_INJECT_FAILURE = "w<t>:<step>" or "u:<update>"): the named
  // worker fails at that step while it holds its buffer lock, or the updater
  // fails at that update while it holds the weights lock.  -1: off.
  int inj_worker = -1, inj_step = -1, inj_update = -1;

  std::vector<sgd_sprint_contrib> log;  // one per worker step, (worker, iter) order
  std::vector<Clock::time_point> update_done;

  // Records the first error and stops the run.  Takes no lock but emu, so a
  // thread may call it while it holds a buffer or weights lock; the thread
  // wakes the others once it has returned and released its locks.
  void fail_with(int e, const std::string& m) {
    {
      std::lock_guard<std::mutex> g(emu);
      if (!err) {
        err = e;
        msg = m;
      }
    }
    stop = true;
  }
  int hip_fail(const char* what) {
    fail_with(SGD_EDEVICE, std::string("sgd_sprint_run: ") + what + " failed");
    return SGD_EDEVICE;
  }
  void wake_updater() {
    { std::lock_guard<std::mutex> g(umu); }
    ucv.notify_all();
  }
  void wake_all() {
    wake_updater();
    { std::lock_guard<std::mutex> g(wmu); }
    wcv.notify_all();
    for (auto& b : bufs) {
      { std::lock_guard<std::mutex> g(b->mu); }
      b->cv.notify_all();
    }
  }
};

// Algorithm 1 for worker t.
void worker_loop(Run& R, int t) {
  if (hipSetDevice(R.device) != hipSuccess) {
    R.hip_fail("hipSetDevice");
    return;
  }
  Worker& w = R.workers[t];
  Buf& buf = *R.bufs[t];
  const sgd_sprint_config& c = R.cfg;
  sgd_gradbuf sum{w.sum, R.n, 1};
  int64_t have = -1;  // version of w.w
  int push = 0;
  std::vector<int64_t> pending;
  for (int i = 0; i < c.iters && !R.stop; ++i) {
    const Clock::time_point t0 = Clock::now();
    if (i % c.n_fetch == 0) {  // the worker's fetch: take LatestWeights if it is newer
      std::lock_guard<std::mutex> g(R.wmu);
      if (R.version > have) {
        if (R.w_ready_valid && hipStreamWaitEvent(w.stream, R.w_ready, 0) != hipSuccess) return (void)R.hip_fail("wait");
        if (hipMemcpyAsync(w.w, R.W, 4 * R.n, hipMemcpyDeviceToDevice, w.stream) != hipSuccess)
          return (void)R.hip_fail("weight fetch copy");
        if (hipEventRecord(w.fetch_done, w.stream) != hipSuccess) return (void)R.hip_fail("event record");
        R.fetch_pending[t] = 1;
        have = R.version;
        ++w.fetches;
      }
    }
    const int64_t b = R.next_batch.fetch_add(1) % R.n_batches;
    const int64_t idx = (int64_t)t * c.iters + i;
    R.log[idx] = sgd_sprint_contrib{t, i, push, b, have, -1};
    // the worker's gradient, summed over the push interval
    int e = sgd_compute_gradient_into(w.net, w.w, R.X + b * R.x_floats, R.y + b * R.batch, &sum, w.loss, w.ws,
                                      w.ws_bytes, w.stream);
    if (e) return R.fail_with(e, sgd_last_error());
    pending.push_back(idx);
    const bool pushing = (i + 1) % c.n_push == 0 || i + 1 == c.iters;
    if (pushing) {  // the push: GradBuf_t <- Grad if empty, else GradBuf_t + Grad
      std::unique_lock<std::mutex> lk(buf.mu);
      buf.cv.wait(lk, [&] { return buf.state != BUF_TAKEN || R.stop; });
      if (R.stop) return;
      if (t == R.inj_worker && i == R.inj_step)
        return R.fail_with(SGD_EDEVICE, "sgd_sprint_run: injected failure (worker " + std::to_string(t) + ")");
      const bool was_empty = buf.state == BUF_EMPTY;
      if (was_empty) {
        if (buf.released_valid && hipStreamWaitEvent(w.stream, buf.released, 0) != hipSuccess)
          return (void)R.hip_fail("wait");
        buf.gb.empty = 1;
      }
      if ((e = sgd_accumulate_grad(&buf.gb, w.sum, w.stream))) return R.fail_with(e, sgd_last_error());
      if (hipEventRecord(buf.written, w.stream) != hipSuccess) return (void)R.hip_fail("event record");
      buf.steps.insert(buf.steps.end(), pending.begin(), pending.end());
      if (was_empty) {
        buf.state = BUF_FULL;
        ++R.n_full;
      }
      lk.unlock();
      R.wake_updater();
      pending.clear();
      sum.empty = 1;
      ++push;
    }
    if (hipStreamSynchronize(w.stream) != hipSuccess) return (void)R.hip_fail("worker stream synchronize");
    w.step_ms += ms_between(t0, Clock::now());
    if (c.sync && pushing && i + 1 < c.iters) {  // wait for an update that holds this push
      std::unique_lock<std::mutex> lk(R.wmu);
      R.wcv.wait(lk, [&] { return R.version > have || R.stop; });
    }
  }
  ++R.finished;
  R.wake_updater();
}

// Algorithm 2 with one node: SumGradient over the non-empty buffers, then the
// update of LatestWeights (momentum, when the rule has it, is the rule's state).
void updater_loop(Run& R) {
  if (hipSetDevice(R.device) != hipSuccess) {
    R.hip_fail("hipSetDevice");
    return;
  }
  const int nw = R.cfg.workers;
  std::vector<int> taken;
  std::vector<const float*> ptrs;
  for (;;) {
    {
      std::unique_lock<std::mutex> lk(R.umu);
      R.ucv.wait(lk, [&] { return R.n_full >= R.cfg.min_bufs || R.finished == nw || R.stop; });
    }
    if (R.stop) return;
    taken.clear();
    ptrs.clear();
    for (int t = 0; t < nw; ++t) {  // the updater takes the non-empty buffers, in buffer index order
      Buf& b = *R.bufs[t];
      std::lock_guard<std::mutex> g(b.mu);
      if (b.state != BUF_FULL) continue;
      if (hipStreamWaitEvent(R.us, b.written, 0) != hipSuccess) return (void)R.hip_fail("wait");
      b.state = BUF_TAKEN;
      --R.n_full;
      for (int64_t s : b.steps) R.log[s].update = R.version;
      b.steps.clear();
      taken.push_back(t);
      ptrs.push_back(b.gb.data);
    }
    if (taken.empty()) {
      if (R.finished == nw && R.n_full == 0) break;  // every step applied
      continue;
    }
    {  // the update: the new LatestWeights, after any fetch copy still reading the old one
      std::lock_guard<std::mutex> g(R.wmu);
      if (R.version == R.inj_update) return R.fail_with(SGD_EDEVICE, "sgd_sprint_run: injected failure (updater)");
      for (int t = 0; t < nw; ++t) {
        if (!R.fetch_pending[t]) continue;
        if (hipStreamWaitEvent(R.us, R.workers[t].fetch_done, 0) != hipSuccess) return (void)R.hip_fail("wait");
        R.fetch_pending[t] = 0;
      }
      if (int e = sgd_apply_fused(R.W, R.state, ptrs.data(), (int)ptrs.size(), R.n, &R.rule, R.us))
        return R.fail_with(e, sgd_last_error());
      if (hipEventRecord(R.w_ready, R.us) != hipSuccess) return (void)R.hip_fail("event record");
      R.w_ready_valid = true;
      ++R.version;
    }
    R.wcv.notify_all();
    for (int t : taken) {
      Buf& b = *R.bufs[t];
      {
        std::lock_guard<std::mutex> g(b.mu);
        if (hipEventRecord(b.released, R.us) != hipSuccess) return (void)R.hip_fail("event record");
        b.released_valid = true;
        b.state = BUF_EMPTY;
      }
      b.cv.notify_all();
    }
    if (hipStreamSynchronize(R.us) != hipSuccess) return (void)R.hip_fail("update stream synchronize");
    R.update_done.push_back(Clock::now());
  }
}

// Thread bodies: after a loop returns (its locks released), a stopped run
// wakes every thread that may wait on a condition variable.
void worker_main(Run& R, int t) {
  worker_loop(R, t);
  if (R.stop) R.wake_all();
}
void updater_main(Run& R) {
  updater_loop(R);
  if (R.stop) R.wake_all();
}

int fail(int code, const std::string& m) {
  sgd::set_error(m);
  return code;
}

int check_config(const sgd_net* net, const sgd_sprint_config* c) {
  if (!net || !c) return fail(SGD_EINVAL, "sgd_sprint: null net or config");
  if (c->workers < 1 || c->workers > 16) return fail(SGD_EINVAL, "sgd_sprint: workers must be 1..16");
  if (c->iters < 1 || c->n_fetch < 1 || c->n_push < 1)
    return fail(SGD_EINVAL, "sgd_sprint: iters, n_fetch and n_push must be >= 1");
  if (c->min_bufs < 1 || c->min_bufs > c->workers) return fail(SGD_EINVAL, "sgd_sprint: min_bufs must be 1..workers");
  if (c->sync != 0 && c->sync != 1) return fail(SGD_EINVAL, "sgd_sprint: sync must be 0 or 1");
  return SGD_OK;
}

int64_t per_worker_bytes(const sgd_net* net) {
  return align256((int64_t)sgd_workspace_bytes(net)) + 3 * align256(4 * sgd_param_count(net)) + 256;
}

}  // namespace

size_t sgd_sprint_workspace_bytes(const sgd_net* net, const sgd_sprint_config* cfg) {
  if (check_config(net, cfg)) return 0;
  return (size_t)(per_worker_bytes(net) * cfg->workers);
}

namespace {
int sprint_run(const sgd_net* net, const sgd_sprint_config* cfg, float* W, float* state, const sgd_rule* rule,
               const float* X, const int32_t* y, int64_t n_batches, void* ws, size_t ws_bytes, void* stream,
               sgd_sprint_stats* stats, sgd_sprint_contrib* log, int64_t log_cap) {
  if (int e = check_config(net, cfg)) return e;
  if (!W || !X || !y || !rule) return fail(SGD_EINVAL, "sgd_sprint_run: null pointer");
  if (n_batches < 1) return fail(SGD_EINVAL, "sgd_sprint_run: n_batches must be >= 1");
  if (rule->rule != SGD_PLAIN && rule->rule != SGD_MOMENTUM && rule->rule != SGD_ADAGRAD &&
      rule->rule != SGD_NESTEROV)
    return fail(SGD_EINVAL, "sgd_sprint_run: unknown rule");
  if (rule->rule != SGD_PLAIN && !state) return fail(SGD_EINVAL, "sgd_sprint_run: rule needs a state buffer");
  if (log && log_cap < 0) return fail(SGD_EINVAL, "sgd_sprint_run: negative log capacity");
  const int64_t per = per_worker_bytes(net);
  if (!ws || ws_bytes < (size_t)(per * cfg->workers)) return fail(SGD_EWORKSPACE, "sgd_sprint_run: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(SGD_EINVAL, "sgd_sprint_run: workspace not 256-byte aligned");

  Run R;
  R.cfg = *cfg;
  R.n = sgd_param_count(net);
  R.W = W;
  R.state = state;
  R.rule = *rule;
  R.X = X;
  R.y = y;
  R.n_batches = n_batches;
  if (const char* inj = std::getenv("SGD_SPRINT_INJECT_FAILURE")) {
    int a = -1, b = -1;
    if (std::sscanf(inj, "w%d:%d", &a, &b) == 2) {
      R.inj_worker = a;
      R.inj_step = b;
    } else if (std::sscanf(inj, "u:%d", &a) == 1) {
      R.inj_update = a;
    }
  }
  const sgd_input in = sgd::net_input(net);
  R.batch = in.batch;
  R.x_floats = (int64_t)in.batch * in.channels * in.height * in.width;
  if (hipGetDevice(&R.device) != hipSuccess) return fail(SGD_EDEVICE, "sgd_sprint_run: no device");
  const int nw = cfg->workers;
  R.workers.resize(nw);
  R.fetch_pending.assign(nw, 0);
  R.log.assign((size_t)nw * cfg->iters, sgd_sprint_contrib{});
  int rc = SGD_OK;
  auto hip_ok = [&](hipError_t e, const char* what) {
    if (e != hipSuccess && rc == SGD_OK) rc = fail(SGD_EDEVICE, std::string("sgd_sprint_run: ") + what + " failed");
    return e == hipSuccess;
  };
  hipEvent_t start = nullptr, end = nullptr;
  auto mk_event = [&](hipEvent_t* e) { return hip_ok(hipEventCreateWithFlags(e, hipEventDisableTiming), "hipEventCreate"); };
  char* base = static_cast<char*>(ws);
  bool ok = mk_event(&start) && mk_event(&end) && mk_event(&R.w_ready) &&
            hip_ok(hipStreamCreateWithFlags(&R.us, hipStreamNonBlocking), "hipStreamCreate");
  for (int t = 0; ok && t < nw; ++t) {
    Worker& w = R.workers[t];
    if ((rc = sgd::clone_net(net, &w.net))) {
      ok = false;
      break;
    }
    char* p = base + per * t;
    w.ws_bytes = sgd_workspace_bytes(w.net);
    w.ws = p;
    p += align256((int64_t)w.ws_bytes);
    w.w = reinterpret_cast<float*>(p);
    p += align256(4 * R.n);
    w.sum = reinterpret_cast<float*>(p);
    p += align256(4 * R.n);
    auto b = std::make_unique<Buf>();
    b->gb = sgd_gradbuf{reinterpret_cast<float*>(p), R.n, 1};
    p += align256(4 * R.n);
    w.loss = reinterpret_cast<float*>(p);
    ok = hip_ok(hipStreamCreateWithFlags(&w.stream, hipStreamNonBlocking), "hipStreamCreate") &&
         mk_event(&w.fetch_done) && mk_event(&b->written) && mk_event(&b->released);
    R.bufs.push_back(std::move(b));
  }
  // everything starts after the caller's queued work
  ok = ok && hip_ok(hipEventRecord(start, static_cast<hipStream_t>(stream)), "event record") &&
       hip_ok(hipStreamWaitEvent(R.us, start, 0), "wait");
  for (int t = 0; ok && t < nw; ++t) ok = hip_ok(hipStreamWaitEvent(R.workers[t].stream, start, 0), "wait");

  const Clock::time_point t0 = Clock::now();
  if (ok) {
    std::vector<std::thread> threads;
    try {
      threads.reserve(nw + 1);
      threads.emplace_back(updater_main, std::ref(R));
      for (int t = 0; t < nw; ++t) threads.emplace_back(worker_main, std::ref(R), t);
    } catch (...) {  // no thread could be started: stop the ones that were
      R.fail_with(SGD_EDEVICE, "sgd_sprint_run: could not start a thread");
      R.wake_all();
    }
    for (auto& th : threads) th.join();
    if (R.err && rc == SGD_OK) rc = fail(R.err, R.msg);
  }
  const Clock::time_point t1 = Clock::now();
  // drain every stream before anything is freed; the caller's stream then
  // follows the run
  for (auto& w : R.workers)
    if (w.stream) hip_ok(hipStreamSynchronize(w.stream), "stream synchronize");
  if (R.us) {
    hip_ok(hipEventRecord(end, R.us), "event record");
    hip_ok(hipStreamSynchronize(R.us), "stream synchronize");
    if (ok) hip_ok(hipStreamWaitEvent(static_cast<hipStream_t>(stream), end, 0), "wait");
  }

  if (rc == SGD_OK) {
    if (stats) {
      sgd_sprint_stats s{};
      s.updates = R.version;
      s.steps = (int64_t)nw * cfg->iters;
      s.wall_ms = ms_between(t0, t1);
      double step_ms = 0.0;
      for (auto& w : R.workers) {
        step_ms += w.step_ms;
        s.fetches += w.fetches;
      }
      s.t_gpu_ms = step_ms / (double)s.steps;
      const size_t u = R.update_done.size();
      s.t_update_ms = u >= 2 ? ms_between(R.update_done.front(), R.update_done.back()) / (double)(u - 1)
                             : (u ? s.wall_ms : 0.0);
      s.n_minibatch_avg = s.updates ? (double)s.steps * R.batch / (double)s.updates : 0.0;
      s.n_minibatch_eq9 = s.t_gpu_ms > 0 ? nw * (double)R.batch * s.t_update_ms / s.t_gpu_ms : 0.0;
      double st = 0.0;
      for (const auto& c : R.log) {
        const int64_t d = c.update - c.version;
        st += (double)d;
        s.staleness_max = std::max<int64_t>(s.staleness_max, d);
      }
      s.staleness_mean = R.log.empty() ? 0.0 : st / (double)R.log.size();
      *stats = s;
    }
    if (log)
      std::copy(R.log.begin(), R.log.begin() + std::min<int64_t>(log_cap, (int64_t)R.log.size()), log);
  }
  for (auto& w : R.workers) {
    if (w.stream) (void)hipStreamDestroy(w.stream);
    if (w.fetch_done) (void)hipEventDestroy(w.fetch_done);
    if (w.net) sgd_destroy_net(w.net);
  }
  for (auto& b : R.bufs) {
    if (b->written) (void)hipEventDestroy(b->written);
    if (b->released) (void)hipEventDestroy(b->released);
  }
  if (R.us) (void)hipStreamDestroy(R.us);
  for (hipEvent_t e : {start, end, R.w_ready})
    if (e) (void)hipEventDestroy(e);
  return rc;
}
}  // namespace

int sgd_sprint_run(const sgd_net* net, const sgd_sprint_config* cfg, float* W, float* state, const sgd_rule* rule,
                   const float* X, const int32_t* y, int64_t n_batches, void* ws, size_t ws_bytes, void* stream,
                   sgd_sprint_stats* stats, sgd_sprint_contrib* log, int64_t log_cap) {
  try {
    return sprint_run(net, cfg, W, state, rule, X, y, n_batches, ws, ws_bytes, stream, stats, log, log_cap);
  } catch (...) {  // host allocation failed before any thread started
    return fail(SGD_EINVAL, "sgd_sprint_run: out of host memory");
  }
}
