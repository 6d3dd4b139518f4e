// A team of host threads that copies one byte range together (host code only).
#include "copy_team.h"

#include <algorithm>
#include <cstring>

namespace moe {

void CopyTeam::part(size_t bytes, int p, int n, size_t& a, size_t& b) {
    const size_t pages = (bytes + 4095) / 4096;
    a = std::min(bytes, pages * p / n * 4096);
    b = std::min(bytes, pages * (p + 1) / n * 4096);
}

bool CopyTeam::start(int threads) {
    stop();
    const int want = threads < 1 ? 1 : threads;
    uint64_t gen0;
    {
        std::lock_guard<std::mutex> lk(mu_);
        stop_ = false;
        pending_ = 0;
        gen0 = gen_;
    }
    // Every member starts from the generation read here, before any job can be posted, so a job
    // posted before a new member first takes the lock is not missed.  The member count is fixed
    // before the first thread starts; a thread that fails to start shrinks the team to the
    // members already running.
    int started = 1;
    bool ok = true;
    try {
        th_.reserve((size_t)want - 1);
    } catch (...) {
        ok = false;
    }
    for (int t = 1; ok && t < want; ++t) {
        try {
            th_.emplace_back(&CopyTeam::worker, this, t, gen0, want);
            ++started;
        } catch (...) {
            ok = false;
        }
    }
    if (!ok) {
        // members already started were told n = want: stop them and run with the caller alone
        stop();
        return false;
    }
    n_ = started;
    return true;
}

void CopyTeam::stop() {
    {
        std::lock_guard<std::mutex> lk(mu_);
        stop_ = true;
    }
    cv_go_.notify_all();
    for (auto& t : th_) t.join();
    th_.clear();
    n_ = 1;
}

void CopyTeam::worker(int id, uint64_t gen0, int n) {
    uint64_t seen = gen0;
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

void CopyTeam::copy(uint8_t* dst, const uint8_t* src, size_t bytes) {
    const int n = n_;
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

}  // namespace moe
