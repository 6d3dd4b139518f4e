// Host-CPU MXFP4 SwiGLU expert kernel (reads blobs in the pool's layout).
#pragma once
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <mutex>
#include <thread>
#include <vector>

#include "moe_internal.h"

namespace moe {

// "avx512" or "scalar": the instruction set the kernel runs with on this host
// (MOE_HOST_FFN_SCALAR=1 in the environment forces the scalar code)
const char* host_ffn_isa();

// y[H] (FP32) = sum_j w[j] * FFN_j(x) over n experts (blobs in the pool's
// layout, host memory), x[H] bf16; experts are shared out over `threads`
// threads and their partial sums added in thread order.
void host_expert_ffn(const Layout& L, const uint8_t* const* blobs, const float* w, int n, const uint16_t* x,
                     float* y, int threads);

// bytes of blob processed per second by `threads` threads running the kernel
// over blobs[0..n) round robin for about min_seconds
double host_expert_rate(const Layout& L, const uint8_t* const* blobs, int n, int threads, double min_seconds);

struct Work;

// Persistent host workers for the hybrid backend: one task at a time, y[H]
// (FP32) = sum_j w[j] * FFN_j(x) over up to 16 experts.  Three phases over all
// of the task's experts, each handing out small units through an atomic
// counter and ending when all of its units are done: (expert, gate/up tiles),
// (expert, blocks of the intermediate vector), then chunks of output rows,
// each summed over the experts in order by the participant that takes it.
// The caller of wait() works on the task as well.  Every value is
// computed by one worker in a fixed order, so the result does not depend on
// the worker count or on which worker takes a unit.
// Workers spin between tasks and sleep after 20 ms idle.
class HostExpertPool {
public:
    ~HostExpertPool();
    bool start(int n_workers);
    void stop();
    bool running() const { return n_ > 0; }
    int workers() const { return n_; }
    // x (bf16, host) and y (FP32, host) must stay valid until wait() returns
    void submit(const Layout& L, const uint8_t* const* blobs, const float* w, int n, const uint16_t* x, float* y);
    void wait();  // helps with the task, then returns once it is complete
    // nanoseconds from submit to the last worker's finish, summed over tasks
    uint64_t busy_ns() const { return busy_ns_.load(); }

private:
    struct Task {
        Layout L{};
        const uint8_t* blobs[16] = {};
        float w[16] = {};
        int n = 0;
        const uint16_t* x = nullptr;
        float* y = nullptr;
        int gu_chunk = 1, act_chunk = 1, d_chunk = 1;  // unit sizes of the three phases
    };
    void run(int t);
    void work(Work& wk, bool vec);
    int n_ = 0;
    Task task_;
    std::vector<std::thread> threads_;
    std::vector<Work*> work_;
    Work* shared_ = nullptr;  // [16]: per expert g, u and the intermediate vector
    std::atomic<int> gen_{0}, done_{0};
    std::atomic<int> gu_next_{0}, act_next_{0}, d_next_{0};  // next unit of each phase
    std::atomic<int> gu_done_{0}, act_done_{0}, d_done_{0};  // units finished per phase
    Work* caller_work_ = nullptr;                            // buffers of the waiting caller
    std::atomic<uint64_t> busy_ns_{0};
    std::chrono::steady_clock::time_point t_submit_{};
    std::atomic<bool> quit_{false};
    std::mutex mu_;
    std::condition_variable cv_;
};

}  // namespace moe
