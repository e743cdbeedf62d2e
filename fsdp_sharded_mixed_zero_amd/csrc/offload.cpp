// Host-side AdamW for ZeRO-Offload: the rank's fp32 optimizer state lives in
// host memory and the host cores run the update, while the GPU keeps the bf16
// gradient and parameter shards (the mlqm.cn article's ZeRO-Offload section:
// optimizer state moved to CPU memory, the CPU performs the Adam update, the
// results travel back over PCIe; "別再複製本可分片的東西" mentions CPU and NVMe
// offload of the sharded state).
//
// The update is the same operation sequence as the GPU kernel (fp32 with fused
// multiply-adds, correctly rounded square root and division, round-to-nearest-
// even bf16 cast; the same cancellation test and fp64 recomputation of the
// elements it flags), on the same tiled state layout, so the offloaded step
// and the GPU step agree bit for bit on hosts with hardware FMA. Work is split
// across threads by whole elements ranges; each thread walks the tiles its
// range meets and runs a contiguous, vectorisable loop per tile. The inner
// loop is compiled for AVX-512, AVX2+FMA and baseline x86-64 and picked at run
// time. One core streams only ~15 GB/s, so the update needs many cores; the
// threads are kept in a pool for the life of the process, because a bucketed
// step makes one call per bucket and starting threads per call costs 10% or
// more of it.
#include <sched.h>
#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "zero_internal.h"

using zero::fail;

namespace {

constexpr int64_t kTile = ZERO_STATE_TILE;

struct HostAdam {
  float beta1, omb1, beta2, omb2, lr_wd, step_size, inv_sqrt_bc2, eps, coef;
  double coef64;         // the clip coefficient before its rounding to fp32
  zero::AdamWExact x;    // the constants in fp64, for the exact recomputation
};

// The GPU kernel's cancellation test: elements whose new master is below
// kCancel times the size of the terms it is formed from are recomputed in
// fp64 (see adamw_exact).
constexpr float kCancel = 0x1p-12f;

// One element recomputed from its old values in fp64 IEEE arithmetic, in
// PyTorch AdamW's order; m', v', p' are stored as their fp32 roundings.
inline void adam_exact(const HostAdam& a, float g, float& p, float& m, float& v) {
  const zero::AdamWExact& x = a.x;
  const double gh = a.coef64 * double(g);
  const double m1 = x.beta1 * double(m) + x.omb1 * gh;
  const double v1 = x.beta2 * double(v) + x.omb2 * (gh * gh);
  const double denom = std::sqrt(v1) / x.sqrt_bc2 + x.eps;
  const double p1 = double(p) * x.decay - x.step_size * (m1 / denom);
  p = float(p1);
  m = float(m1);
  v = float(v1);
}

inline uint16_t bf16_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x0040u);   // quiet NaN, sign kept
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

inline float widen(uint16_t h) {
  const uint32_t u = uint32_t(h) << 16;
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

// Clones of the inner loop for AVX-512 and AVX2+FMA, chosen at load time.
// Compilers that take no x86-64-v3/v4 clone targets (GCC before 12) build
// the baseline loop only: std::fma is then a correctly rounded library call,
// so the results are the same, only slower.
#if defined(__clang__) || (defined(__GNUC__) && __GNUC__ >= 12)
#define ZERO_HOST_CLONES __attribute__((target_clones("arch=x86-64-v4", "arch=x86-64-v3", "default")))
#else
#define ZERO_HOST_CLONES
#endif

// One element: the update in place and its bf16 parameter.
inline uint16_t adam_one(const HostAdam& a, uint16_t gbits, float& p, float& m, float& v) {
  const float gj = widen(gbits);
  const float gh = gj * a.coef;
  const float mg = a.omb1 * gh;
  const float mj = std::fma(a.beta1, m, mg);
  const float vj = std::fma(a.beta2, v, a.omb2 * (gh * gh));
  const float denom = std::fma(std::sqrt(vj), a.inv_sqrt_bc2, a.eps);
  const float pd = std::fma(-a.lr_wd, p, p);
  const float pj = std::fma(-a.step_size, mj / denom, pd);
  if (std::fma(-kCancel, std::fabs(pd), std::fabs(pj)) * denom <
      (kCancel * a.step_size) * (std::fabs(a.beta1 * m) + std::fabs(mg))) {
    adam_exact(a, gj, p, m, v);
  } else {
    m = mj;
    v = vj;
    p = pj;
  }
  return bf16_rne(p);
}

typedef uint16_t u16x32 __attribute__((vector_size(64)));

// A 64-byte line to a 64-byte aligned address, non-temporal where the
// compiler has the builtin (clang); GCC stores it plainly.
inline void store_line(uint16_t* dst, const uint16_t* src) {
  u16x32 line;
  std::memcpy(&line, src, sizeof(line));
#if defined(__clang__)
  __builtin_nontemporal_store(line, reinterpret_cast<u16x32*>(dst));
#else
  *reinterpret_cast<u16x32*>(dst) = line;
#endif
}

// One contiguous run of n elements: gradients g[0..n), state slots p/m/v
// (stride 1), parameters out[0..n). The parameters go out a 64-byte line at a
// time with a non-temporal store: nothing on the host reads them, and a
// plain store would first read each line into the cache (2 more bytes per
// element). Measured at the 7.5B shard with 16 threads, the host update took
// 11.2-12.8 ms against 13.1-14.4 ms with plain stores, with the same results.
ZERO_HOST_CLONES
void adam_run(const HostAdam& a, const uint16_t* __restrict g, float* __restrict p, float* __restrict m,
              float* __restrict v, uint16_t* __restrict out, int64_t n) {
  int64_t j = 0;
  for (; j < n && (uintptr_t(out + j) & 63u); ++j) out[j] = adam_one(a, g[j], p[j], m[j], v[j]);
  for (; j + 32 <= n; j += 32) {
    alignas(64) uint16_t w[32];
    for (int k = 0; k < 32; ++k) w[k] = adam_one(a, g[j + k], p[j + k], m[j + k], v[j + k]);
    store_line(out + j, w);
  }
  for (; j < n; ++j) out[j] = adam_one(a, g[j], p[j], m[j], v[j]);
}

// Elements [lo, hi) of the shard; g and param hold the call's range, which
// starts at element `begin`.
void adam_range(const HostAdam& a, const uint16_t* g, float* state, uint16_t* param, int64_t n_state,
                int64_t begin, int64_t lo, int64_t hi) {
  int64_t e = lo;
  while (e < hi) {
    const int64_t k0 = (e / kTile) * kTile;
    const int64_t L = std::min(kTile, n_state - k0);
    const int64_t stop = std::min(hi, k0 + L);
    float* base = state + 3 * k0 + (e - k0);
    adam_run(a, g + (e - begin), base, base + L, base + 2 * L, param + (e - begin), stop - e);
    e = stop;
  }
}

// Worker threads started on first use and kept until the process ends. run()
// calls task(i) for i = 0..n-1, task(0) on the calling thread, and returns when
// all are done. Calls are serialised. All shared state (threads, mutex,
// condition variables) sits in one heap object: a child made by fork() has
// none of the parent's threads, and the inherited condition variables still
// count the parent's waiters, so the child abandons that object (it is never
// freed or joined) and builds its own. Forking while a call runs is not
// supported.
struct PoolState {
  std::mutex mu;
  std::condition_variable cv, done;
  std::vector<std::thread> threads;
  const std::function<void(int)>* task = nullptr;
  int n = 0, pending = 0;
  uint64_t gen = 0;
  bool stop = false;
  pid_t owner = getpid();
};

void pool_loop(PoolState* st, int id) {
  uint64_t seen = 0;
  std::unique_lock<std::mutex> lk(st->mu);
  for (;;) {
    st->cv.wait(lk, [&] { return st->stop || st->gen != seen; });
    if (st->stop) return;
    seen = st->gen;
    if (id >= st->n) continue;           // this call needs fewer threads
    const std::function<void(int)>* t = st->task;
    lk.unlock();
    (*t)(id);
    lk.lock();
    if (--st->pending == 0) st->done.notify_one();
  }
}

class WorkerPool {
 public:
  ~WorkerPool() {
    if (st_ == nullptr || st_->owner != getpid()) return;
    {
      std::lock_guard<std::mutex> g(st_->mu);
      st_->stop = true;
    }
    st_->cv.notify_all();
    for (auto& t : st_->threads) t.join();
    delete st_;
  }

  // false if threads could not be started (nothing has run then)
  bool run(int n, const std::function<void(int)>& task) {
    std::lock_guard<std::mutex> serial(call_mu_);
    if (st_ == nullptr || st_->owner != getpid()) st_ = new PoolState();
    PoolState* st = st_;
    std::unique_lock<std::mutex> lk(st->mu);
    try {
      while (int(st->threads.size()) < n - 1) {
        const int id = int(st->threads.size()) + 1;
        st->threads.emplace_back(pool_loop, st, id);
      }
    } catch (...) {
      return false;
    }
    st->task = &task;
    st->n = n;
    st->pending = n - 1;
    ++st->gen;
    lk.unlock();
    st->cv.notify_all();
    task(0);
    lk.lock();
    st->done.wait(lk, [st] { return st->pending == 0; });
    st->task = nullptr;
    return true;
  }

 private:
  std::mutex call_mu_;
  PoolState* st_ = nullptr;
};

WorkerPool& pool() {
  static WorkerPool p;
  return p;
}

// CPUs this process may run on (its affinity mask), else the machine's count.
int64_t usable_cpus() {
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    const int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  return std::max(1u, std::thread::hardware_concurrency());
}

int cpu_adamw(const uint16_t* h_grad, float* h_state, uint16_t* h_param, int64_t n_state, int64_t begin, int64_t count,
              const zero_adamw_hparams* hp, const double* h_rank_sqnorms, int32_t n_ranks, int32_t n_threads,
              const char* who) {
  if (int rc = zero::check_adamw_hparams(hp, who)) return rc;
  if (n_state < 0 || begin < 0 || count < 0 || begin > n_state || count > n_state - begin)
    return fail(ZERO_EINVAL, "%s: range [%lld, +%lld) outside a state of %lld elements", who, (long long)begin,
                (long long)count, (long long)n_state);
  const bool clip = hp->max_norm > 0.0;
  if (clip && (h_rank_sqnorms == nullptr || n_ranks < 1))
    return fail(ZERO_EINVAL, "%s: clipping needs the ranks' sums of squares", who);
  if (n_threads < 0) return fail(ZERO_EINVAL, "%s: n_threads < 0", who);
  if (count == 0) return zero::ok();
  if (!h_grad || !h_state || !h_param) return fail(ZERO_EINVAL, "%s: NULL buffer", who);

  HostAdam a{};
  a.beta1 = float(hp->beta1);
  a.omb1 = float(1.0 - hp->beta1);
  a.beta2 = float(hp->beta2);
  a.omb2 = float(1.0 - hp->beta2);
  const double t = double(hp->step);
  a.lr_wd = float(hp->lr * hp->weight_decay);
  a.step_size = float(hp->lr / (1.0 - std::pow(hp->beta1, t)));
  a.inv_sqrt_bc2 = float(1.0 / std::sqrt(1.0 - std::pow(hp->beta2, t)));
  a.eps = float(hp->eps);
  zero::adamw_exact_constants(hp, &a.x);
  a.coef = 1.0f;
  a.coef64 = 1.0;
  if (clip) {
    // the GPU update's order: lane sums of ranks l, l+64, l+128, ... (each in
    // rank order), then the 64 lane sums in order (for at most 64 ranks, the
    // plain rank-order sum)
    double G2 = 0.0;
    for (int32_t l = 0; l < 64; ++l) {
      double run = 0.0;
      for (int64_t r = l; r < n_ranks; r += 64) run += h_rank_sqnorms[r];
      G2 += run;
    }
    const double ratio = hp->max_norm / (std::sqrt(G2) + hp->clip_eps);
    a.coef64 = ratio >= 1.0 ? 1.0 : ratio;   // a NaN ratio stays NaN
    a.coef = float(a.coef64);
  }

  int64_t threads = n_threads > 0 ? n_threads : usable_cpus();
  const int64_t min_per_thread = 1 << 16;
  threads = std::max<int64_t>(1, std::min(threads, (count + min_per_thread - 1) / min_per_thread));
  const int64_t end = begin + count;
  if (threads == 1) {
    adam_range(a, h_grad, h_state, h_param, n_state, begin, begin, end);
    return zero::ok();
  }
  // split on 64-element boundaries so no two threads share a cache line
  const int64_t per = ((count + threads - 1) / threads + 63) / 64 * 64;
  const int n_run = int((count + per - 1) / per);
  const std::function<void(int)> task = [&](int i) {
    const int64_t lo = begin + int64_t(i) * per;
    adam_range(a, h_grad, h_state, h_param, n_state, begin, lo, std::min(end, lo + per));
  };
  if (!pool().run(n_run, task)) return fail(ZERO_ENOMEM, "%s: could not start host threads", who);
  return zero::ok();
}

}  // namespace

extern "C" int zero_cpu_adamw_step(const uint16_t* h_grad, float* h_state, uint16_t* h_param, int64_t n_state,
                                   int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                                   const double* h_rank_sqnorms, int32_t n_ranks, int32_t n_threads) {
  return cpu_adamw(h_grad, h_state, h_param, n_state, begin, count, hp, h_rank_sqnorms, n_ranks, n_threads,
                   "zero_cpu_adamw_step");
}
