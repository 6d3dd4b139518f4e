// Host-CPU MXFP4 SwiGLU expert kernel (reads blobs in the pool's layout).
#pragma once
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <deque>
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

// one expert's intermediate state for one token: g, u [I], the intermediate
// vector split into the even / odd elements of each 32-block, and (worker
// pool) its weighted output w * FFN(x) [H]
struct ExpertBuf {
    std::vector<float> g, u, ae, ao, yp;
    void size(const Layout& L) {
        if ((int)g.size() == L.I && (int)ae.size() == L.NBI * 16 && (int)yp.size() == L.H) return;
        g.assign(L.I, 0.0f);
        u.assign(L.I, 0.0f);
        ae.assign((size_t)L.NBI * 16, 0.0f);
        ao.assign((size_t)L.NBI * 16, 0.0f);
        yp.assign(L.H, 0.0f);
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
// token b, in their order, of w * FFN(x_b).  Units are handed out through
// atomic counters: first one unit per token (x to FP32), then one list that
// interleaves, entry by entry, (entry, a multiple of four gate/up tiles) units,
// which also form the intermediate vector of those rows (four 8-row tiles are
// one 32-element block), with the (entry, chunk of output rows) down units of
// the entry before, which write w * (its rows of the expert's output).  A down
// unit waits only for its own entry's gate/up units; the participant that
// finishes a token's last down unit sums the token's entries in order.  The
// caller of wait() works on the task as well.  Every value is computed by one
// participant in a fixed order, so the result does not depend on the worker
// count or on which worker takes a unit.  Workers spin between tasks and
// sleep after 20 ms idle.
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
        int gu_chunk = 4, d_chunk = 1;  // 8-row gate/up tiles and 8-row output tiles per unit
        int gu_per = 1, d_per = 1;      // gate/up and down units per entry
        int gu_step = 1, d_step = 1;    // order within an entry: k -> k * step mod count
    };
    void run(int t);
    void work(bool vec);
    int n_ = 0;
    Task task_;
    std::vector<std::thread> threads_;
    std::vector<ExpertBuf> ebuf_;  // per entry: g, u and the intermediate vector
    std::vector<TokenBuf> xbuf_;   // per token: x split even / odd
    struct alignas(128) Counter {
        std::atomic<int> v{0};
    };
    // each counter on a cache line of its own: participants on different cores
    // update them concurrently, and the waiting ones poll them
    alignas(128) std::atomic<int> gen_{0};
    alignas(128) std::atomic<int> done_{0};
    alignas(128) std::atomic<int> x_next_{0};     // next x unit
    alignas(128) std::atomic<int> x_done_{0};     // x units finished
    alignas(128) std::atomic<int> main_next_{0};  // next gate/up or down unit
    alignas(128) std::atomic<int> tok_done_{0};   // tokens whose output is complete
    Counter gu_left_[kHostMaxEntries];            // gate/up units of an entry not yet finished
    Counter d_left_[kHostMaxTokens];              // down units of a token's entries not yet finished
    alignas(128) std::atomic<uint64_t> busy_ns_{0};
    std::chrono::steady_clock::time_point t_submit_{};
    std::atomic<bool> quit_{false};
    std::mutex mu_;
    std::condition_variable cv_;
};

// Tasks of several layer steps queued ahead of their FFNs: a dispatcher thread
// runs them on a HostExpertPool one after another, in push order, and counts
// the finished ones, so a waiter can wait for one task without holding up the
// pushing thread.  Pushed x and y must stay valid until that task is done.
class HostTaskQueue {
public:
    ~HostTaskQueue();
    bool start(HostExpertPool* pool);  // false if the thread could not be started; numbers go on
    void stop();                       // runs the queued tasks, then joins the thread
    bool running() const { return th_.joinable(); }
    // queues a task (arguments as HostExpertPool::submit); returns its number: 1, 2, ... over the
    // queue's whole life (a restart keeps counting)
    uint64_t push(const Layout& L, int n_tok, const uint16_t* const* x, float* const* y, const HostEntry* e, int n);
    // true once task `seq` (and every task before it) is done; false after timeout_s
    bool wait(uint64_t seq, double timeout_s);
    uint64_t pushed() const { return pushed_; }
    uint64_t done() const { return done_.load(std::memory_order_acquire); }
    // also store the count of finished tasks at *p after each task (memory the GPU reads); set
    // while the thread is stopped
    void set_mirror(uint64_t* p) { mirror_ = p; }

private:
    struct Item {
        Layout L{};
        int n_tok = 0, n = 0;
        const uint16_t* x[kHostMaxTokens] = {};
        float* y[kHostMaxTokens] = {};
        HostEntry e[kHostMaxEntries] = {};
    };
    void run();
    HostExpertPool* pool_ = nullptr;
    std::thread th_;
    std::deque<Item> q_;
    uint64_t pushed_ = 0;               // the pushing thread's count
    std::atomic<uint64_t> done_{0};
    uint64_t* mirror_ = nullptr;
    bool quit_ = false;
    std::mutex mu_;
    std::condition_variable cv_push_, cv_done_;
};

}  // namespace moe
