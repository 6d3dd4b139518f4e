// Copy path for expert blobs that live in pageable host memory.
//
// The pool of every expert sits in host RAM and misses stream to the GPU over
// PCIe (pirouter.ai "FreeToken x RTX 5090" page, mechanism section: the pool
// is kept in pinned memory the GPU can DMA from).  When the platform pins less
// than the whole pool, the library pins what it can and keeps the rest in
// ordinary pageable memory; a miss on that part goes through this ring of
// pinned bounce buffers: a few host threads copy the blob into a free ring
// slot, then one hipMemcpyAsync moves the slot to the device on the copy
// stream, and an event per slot tells when the slot can be refilled.  Host
// copies of the next blobs overlap the DMA of the previous ones.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "copy_team.h"

namespace moe {

class BounceRing {
public:
    BounceRing() = default;
    BounceRing(const BounceRing&) = delete;
    BounceRing& operator=(const BounceRing&) = delete;
    ~BounceRing() { shutdown(); }

    // slots pinned buffers of slot_bytes each; threads host threads per copy
    // (including the caller).  Returns hipSuccess or the failing call's error
    // (hipErrorOutOfMemory when a copy thread could not be started).
    hipError_t init(size_t slot_bytes, int slots, int threads, hipStream_t stream);

    // Copies `bytes` (<= slot_bytes) from pageable host memory to device memory
    // through the next ring slot; returns once the DMA is queued on the stream.
    // Blocks while the slot's previous DMA is still in flight.
    hipError_t copy(void* dst_dev, const uint8_t* src, size_t bytes);

    void shutdown();
    bool ready() const { return !slot_.empty(); }
    uint64_t copies() const { return copies_; }

private:
    size_t slot_bytes_ = 0;
    std::vector<uint8_t*> slot_;
    std::vector<hipEvent_t> ev_;
    std::vector<bool> busy_;
    size_t next_ = 0;
    hipStream_t stream_ = nullptr;
    uint64_t copies_ = 0;
    CopyTeam team_;  // host threads that fill a ring slot together
};

}  // namespace moe
