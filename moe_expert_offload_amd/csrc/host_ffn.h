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

// one expert's intermediate state for one token: g, u [I] and the
// intermediate vector split into the even / odd elements of each 32-block
struct ExpertBuf {
    std::vector<float> g, u, ae, ao;
    void size(const Layout& L) {
        if ((int)g.size() == L.I && (int)ae.size() == L.NBI * 16) return;
        g.assign(L.I, 0.0f);
        u.assign(L.I, 0.0f);
        ae.assign((size_t)L.NBI * 16, 0.0f);
        ao.assign((size_t)L.NBI * 16, 0.0f);
    }
};

// a token's hidden state in FP32, split even / odd per 32-block
struct TokenBuf {
    std::vector<float> xe, xo;
    void size(const Layout& L) {
        if ((int)xe.size() == L.NB * 16) return;
        xe.assign((size_t)L.NB * 16, 0.0f);
        xo.assign((size_t)L.NB * 16, 0.0f);
    }
};

constexpr int kHostMaxTokens = 16;    // tokens of one host task
constexpr int kHostMaxEntries = 256;  // (expert, token) pairs of one host task

// one expert applied to one token of a task, weighted by w
struct HostEntry {
    const uint8_t* blob;  // the expert's blob in the pool's layout (host memory)
    float w;
    int tok;              // index into the task's tokens
};

// Persistent host workers for the hybrid backend: one task at a time, for
// each of up to 16 tokens b, y_b[H] (FP32) = sum over the task's entries of
// token b, in their order, of w * FFN(x_b).  Three phases, each handing out
// small units through an atomic counter and ending when all of its units are
// done: (token, blocks of x) to FP32; (entry, an even number of gate/up
// tiles), which also forms the intermediate vector of those rows (two 16-row
// tiles are one 32-element block); then (token, chunks of output rows), each
// summed over the token's entries in order by the participant that takes it.
// The caller of wait() works on the task as well.  Every value is computed by
// one participant in a fixed order, so the result does not depend on the
// worker count or on which worker takes a unit.  Workers spin between tasks
// and sleep after 20 ms idle.
class HostExpertPool {
public:
    ~HostExpertPool();
    bool start(int n_workers);
    void stop();
    bool running() const { return n_ > 0; }
    int workers() const { return n_; }
    // x[b] (bf16 [H], host) and y[b] (FP32 [H], host) for b < n_tok must stay
    // valid until wait() returns; entries are copied (at most kHostMaxEntries,
    // tokens below min(n_tok, kHostMaxTokens); others are dropped)
    void submit(const Layout& L, int n_tok, const uint16_t* const* x, float* const* y, const HostEntry* entries,
                int n);
    void wait();  // helps with the task, then returns once it is complete
    // nanoseconds from submit to the last unit's finish, summed over tasks
    uint64_t busy_ns() const { return busy_ns_.load(); }

private:
    struct Task {
        Layout L{};
        HostEntry e[kHostMaxEntries] = {};  // grouped by token
        int tok_begin[kHostMaxTokens + 1] = {};
        int n = 0, ntok = 0;
        const uint16_t* x[kHostMaxTokens] = {};
        float* y[kHostMaxTokens] = {};
        int x_chunk = 1, gu_chunk = 2, d_chunk = 1;  // unit sizes of the phases
        int gu_per = 1, d_per = 1;                   // units per entry / per token
        int gu_step = 1, d_step = 1;                 // unit order: u -> u * step mod count
    };
    void run(int t);
    void work(bool vec);
    int n_ = 0;
    Task task_;
    std::vector<std::thread> threads_;
    std::vector<ExpertBuf> ebuf_;  // per entry: g, u and the intermediate vector
    std::vector<TokenBuf> xbuf_;   // per token: x split even / odd
    // each counter on a cache line of its own: participants on different cores
    // update them concurrently, and the waiting ones poll the done counters
    alignas(128) std::atomic<int> gen_{0};
    alignas(128) std::atomic<int> done_{0};
    alignas(128) std::atomic<int> x_next_{0};   // next unit of each phase
    alignas(128) std::atomic<int> gu_next_{0};
    alignas(128) std::atomic<int> d_next_{0};
    alignas(128) std::atomic<int> x_done_{0};   // units finished per phase
    alignas(128) std::atomic<int> gu_done_{0};
    alignas(128) std::atomic<int> d_done_{0};
    alignas(128) std::atomic<uint64_t> busy_ns_{0};
    std::chrono::steady_clock::time_point t_submit_{};
    std::atomic<bool> quit_{false};
    std::mutex mu_;
    std::condition_variable cv_;
};

}  // namespace moe
