// Host-core computation of whole experts from their packed records, for the
// hybrid decode forwards: the experts the GPU does not hold are computed by
// the host's cores while the GPU computes the resident ones ("Strata,
// Explained", section 2: host RAM holds every expert pinned and the CPU
// computes the experts the GPU lacks, at the same time).  It reads the same
// prepacked records the pinned store holds for paging (tile order, every
// weight format) and never widens them in memory.
#pragma once
#include <stdint.h>

#include <atomic>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "moe_common.h"

namespace strata {

// A small persistent pool: run(n, fn) calls fn(i) for i in [0, n) on the
// pool's threads and the calling thread, and returns when all are done.
// Idle threads spin briefly for the next task (decode forwards arrive back
// to back), then sleep.
class HostPool {
 public:
  explicit HostPool(int threads);
  ~HostPool();
  void run(int n, const std::function<void(int)>& fn);
  int threads() const { return (int)workers_.size() + 1; }

 private:
  struct Task {
    const std::function<void(int)>* fn = nullptr;
    int n = 0;
    std::atomic<int> next{0}, done{0}, users{0};
  };
  void loop();
  static void work(Task& t);
  std::vector<std::thread> workers_;
  std::mutex mu_;                   // guards task_ and stop_
  std::condition_variable cv_;
  std::atomic<uint64_t> gen_{0};    // bumped for every task (and at stop)
  Task* task_ = nullptr;
  bool stop_ = false;
};

// One expert to compute on the host: its record, its tokens' rows of x
// (fp32 [ntok, H]) and where its output rows go (fp32 [ntok, H]).
struct HostJob {
  const uint8_t* rec;
  const int32_t* wexp;  // kWexpCount exponents of the expert (int4: matrix scales 2^c)
  int ntok;
  const float* x;
  float* o;
};

// The expert FFN o = Wd (silu(Wg x) * (Wu x)) of every job, fp32 throughout
// (h is not rounded), each output row summed by one thread in a fixed order:
// the result does not depend on the thread count.  `hbuf` is scratch of
// sum(ntok) * F floats.
void host_experts_run(HostPool& pool, const std::vector<HostJob>& jobs, int H, int F, int qf, int sshift,
                      const RecordLayout& lay, float* hbuf);

}  // namespace strata
