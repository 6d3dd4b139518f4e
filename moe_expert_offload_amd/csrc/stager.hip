// Pinned bounce ring for expert blobs in pageable host memory (host code).
#include "stager.h"

#include <algorithm>
#include <cstring>

namespace moe {

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
    if (!team_.start(threads)) {
        shutdown();
        return hipErrorOutOfMemory;
    }
    return hipSuccess;
}

void BounceRing::shutdown() {
    team_.stop();
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

hipError_t BounceRing::copy(void* dst_dev, const uint8_t* src, size_t bytes) {
    if (slot_.empty() || bytes > slot_bytes_) return hipErrorInvalidValue;
    const size_t r = next_;
    next_ = (next_ + 1) % slot_.size();
    if (busy_[r]) {
        hipError_t e = hipEventSynchronize(ev_[r]);
        if (e != hipSuccess) return e;
        busy_[r] = false;
    }
    team_.copy(slot_[r], src, bytes);
    hipError_t e = hipMemcpyAsync(dst_dev, slot_[r], bytes, hipMemcpyHostToDevice, stream_);
    if (e != hipSuccess) return e;
    e = hipEventRecord(ev_[r], stream_);
    if (e != hipSuccess) return e;
    busy_[r] = true;
    ++copies_;
    return hipSuccess;
}

}  // namespace moe
