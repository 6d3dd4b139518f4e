// Pinned bounce ring for expert blobs in pageable host memory (host code).
#include "stager.h"

#include <algorithm>
#include <cstring>

namespace moe {

namespace {
// part p of n of a byte range, split on 4 KiB boundaries
inline void part(size_t bytes, int p, int n, size_t& a, size_t& b) {
    const size_t pages = (bytes + 4095) / 4096;
    a = std::min(bytes, pages * p / n * 4096);
    b = std::min(bytes, pages * (p + 1) / n * 4096);
}
}  // namespace

hipError_t BounceRing::init(size_t slot_bytes, int slots, int threads, hipStream_t stream) {
    shutdown();
    slot_bytes_ = slot_bytes;
    stream_ = stream;
    for (int i = 0; i < slots; ++i) {
        uint8_t* p = nullptr;
        hipError_t e = hipHostMalloc((void**)&p, slot_bytes, hipHostMallocDefault);
        if (e != hipSuccess) {
            shutdown();
            return e;
        }
        slot_.push_back(p);
        hipEvent_t ev = nullptr;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            shutdown();
            return e;
        }
        ev_.push_back(ev);
        busy_.push_back(false);
    }
    {
        std::lock_guard<std::mutex> lk(mu_);
        stop_ = false;
        n_threads_ = threads < 1 ? 1 : threads;
    }
    for (int t = 1; t < n_threads_; ++t) th_.emplace_back(&BounceRing::worker, this, t);
    return hipSuccess;
}

void BounceRing::shutdown() {
    {
        std::lock_guard<std::mutex> lk(mu_);
        stop_ = true;
    }
    cv_go_.notify_all();
    for (auto& t : th_) t.join();
    th_.clear();
    n_threads_ = 1;
    // (a failed init can leave one more slot than events)
    for (size_t i = 0; i < ev_.size(); ++i) {
        if (busy_[i]) (void)hipEventSynchronize(ev_[i]);
        (void)hipEventDestroy(ev_[i]);
    }
    for (uint8_t* p : slot_) (void)hipHostFree(p);
    slot_.clear();
    ev_.clear();
    busy_.clear();
    next_ = 0;
}

void BounceRing::worker(int id) {
    uint64_t seen;
    int n;
    {
        std::lock_guard<std::mutex> lk(mu_);
        seen = gen_;
        n = n_threads_;
    }
    for (;;) {
        uint8_t* dst;
        const uint8_t* src;
        size_t bytes;
        {
            std::unique_lock<std::mutex> lk(mu_);
            cv_go_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_) return;
            seen = gen_;
            dst = job_dst_;
            src = job_src_;
            bytes = job_bytes_;
        }
        size_t a, b;
        part(bytes, id, n, a, b);
        if (b > a) memcpy(dst + a, src + a, b - a);
        {
            std::lock_guard<std::mutex> lk(mu_);
            if (--pending_ == 0) cv_done_.notify_one();
        }
    }
}

void BounceRing::parallel_memcpy(uint8_t* dst, const uint8_t* src, size_t bytes) {
    const int n = n_threads_;
    if (n == 1) {
        memcpy(dst, src, bytes);
        return;
    }
    {
        std::lock_guard<std::mutex> lk(mu_);
        job_dst_ = dst;
        job_src_ = src;
        job_bytes_ = bytes;
        pending_ = n - 1;
        ++gen_;
    }
    cv_go_.notify_all();
    size_t a, b;
    part(bytes, 0, n, a, b);
    if (b > a) memcpy(dst + a, src + a, b - a);
    std::unique_lock<std::mutex> lk(mu_);
    cv_done_.wait(lk, [&] { return pending_ == 0; });
}

hipError_t BounceRing::copy(void* dst_dev, const uint8_t* src, size_t bytes) {
    if (slot_.empty() || bytes > slot_bytes_) return hipErrorInvalidValue;
    const size_t r = next_;
    next_ = (next_ + 1) % slot_.size();
    if (busy_[r]) {
        hipError_t e = hipEventSynchronize(ev_[r]);
        if (e != hipSuccess) return e;
        busy_[r] = false;
    }
    parallel_memcpy(slot_[r], src, bytes);
    hipError_t e = hipMemcpyAsync(dst_dev, slot_[r], bytes, hipMemcpyHostToDevice, stream_);
    if (e != hipSuccess) return e;
    e = hipEventRecord(ev_[r], stream_);
    if (e != hipSuccess) return e;
    busy_[r] = true;
    ++copies_;
    return hipSuccess;
}

}  // namespace moe
