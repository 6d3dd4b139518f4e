// A team of host threads that copies one byte range together (host code only).
//
// The pinned bounce ring (stager.h) fills a ring slot from pageable host
// memory with it: one pageable-to-pinned memcpy split over a few cores runs at
// several times the rate of one core, which keeps the copy path ahead of the
// DMA engine.  The caller takes part in every copy; the other members wait on
// a condition variable between jobs.
#pragma once
#include <condition_variable>
#include <cstddef>
#include <cstdint>
#include <mutex>
#include <thread>
#include <vector>

namespace moe {

class CopyTeam {
public:
    CopyTeam() = default;
    CopyTeam(const CopyTeam&) = delete;
    CopyTeam& operator=(const CopyTeam&) = delete;
    ~CopyTeam() { stop(); }

    // threads: members including the caller (>= 1).  Returns false (and runs
    // with the caller alone) when a thread could not be started.
    bool start(int threads);
    void stop();
    int size() const { return n_; }

    // copies bytes from src to dst, split on 4 KiB boundaries over the team;
    // returns once every part is done
    void copy(uint8_t* dst, const uint8_t* src, size_t bytes);

    // part p of n of a byte range, split on 4 KiB boundaries: [a, b)
    static void part(size_t bytes, int p, int n, size_t& a, size_t& b);

private:
    void worker(int id, uint64_t gen0, int n);

    std::vector<std::thread> th_;
    int n_ = 1;
    std::mutex mu_;
    std::condition_variable cv_go_, cv_done_;
    uint64_t gen_ = 0;       // job generation: a member takes every generation after the one it last saw
    int pending_ = 0;        // members still copying the current job
    bool stop_ = false;
    uint8_t* job_dst_ = nullptr;
    const uint8_t* job_src_ = nullptr;
    size_t job_bytes_ = 0;
};

}  // namespace moe
