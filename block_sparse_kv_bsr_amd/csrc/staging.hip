// Pinned host staging for plan uploads.
//
// A plan's host image (work list, merge nodes, page ids) reaches the device
// workspace with one asynchronous copy, which needs page-locked source memory
// that stays untouched until the copy has run. Pinning memory costs
// milliseconds (the pages are locked and mapped for the device), and freeing
// it waits for the device, while a serving loop builds and uploads a new plan
// every step. So blocks are pinned once and cached for the life of the
// process: an upload takes a free block of the right size class, copies the
// image into it, enqueues the host-to-device copy and records an event after
// it; the block returns to its free list once a later upload finds that event
// complete. Nothing here waits for a stream or the device (except when an
// event cannot be recorded, below).
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "staging.h"

namespace fi {
namespace {

constexpr size_t kMinBlock = size_t(64) << 10;

size_t size_class(size_t n) {
  size_t c = kMinBlock;
  while (c < n) c <<= 1;
  return c;
}

struct InFlight {
  void* block;
  size_t cls;
  hipEvent_t ev;
  int device;
};

class Pool {
 public:
  hipError_t copy(void* dst, const void* src, size_t n, hipStream_t s) {
    std::lock_guard<std::mutex> lock(mu_);
    reclaim();
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const size_t cls = size_class(n);
    void* block = nullptr;
    auto& fl = free_[cls];
    if (!fl.empty()) {
      block = fl.back();
      fl.pop_back();
    } else {
      e = hipHostMalloc(&block, cls, hipHostMallocDefault);
      if (e != hipSuccess) return e;
    }
    std::memcpy(block, src, n);
    hipEvent_t ev = nullptr;
    e = take_event(dev, &ev);
    if (e != hipSuccess) {
      free_[cls].push_back(block);
      return e;
    }
    e = hipMemcpyAsync(dst, block, n, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) {
      free_[cls].push_back(block);
      events_[dev].push_back(ev);
      return e;
    }
    e = hipEventRecord(ev, s);
    if (e != hipSuccess) {
      // The copy is queued but cannot be tracked: let it finish before the
      // block can be handed out again.
      events_[dev].push_back(ev);
      const hipError_t w = hipStreamSynchronize(s);
      if (w == hipSuccess) free_[cls].push_back(block);
      return e;
    }
    in_flight_.push_back({block, cls, ev, dev});
    return hipSuccess;
  }

 private:
  // Moves the blocks whose copies have completed back to their free lists.
  // A query that fails for another reason than "not ready" keeps the block
  // out of circulation.
  void reclaim() {
    size_t keep = 0;
    for (size_t i = 0; i < in_flight_.size(); ++i) {
      const InFlight f = in_flight_[i];
      if (hipEventQuery(f.ev) == hipSuccess) {
        free_[f.cls].push_back(f.block);
        events_[f.device].push_back(f.ev);
      } else {
        in_flight_[keep++] = f;
      }
    }
    in_flight_.resize(keep);
  }

  // An event of `dev` (events are recorded on streams of the device they
  // were created on).
  hipError_t take_event(int dev, hipEvent_t* ev) {
    auto& el = events_[dev];
    if (!el.empty()) {
      *ev = el.back();
      el.pop_back();
      return hipSuccess;
    }
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    return e;
  }

  std::mutex mu_;
  std::map<size_t, std::vector<void*>> free_;
  std::map<int, std::vector<hipEvent_t>> events_;
  std::vector<InFlight> in_flight_;
};

// Never destroyed: the runtime may already be gone when static destructors
// run, and the process exit returns the memory anyway.
Pool& pool() {
  static Pool* p = new Pool();
  return *p;
}

}  // namespace

hipError_t staged_upload(void* dst, const void* src, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  return pool().copy(dst, src, n, stream);
}

}  // namespace fi
