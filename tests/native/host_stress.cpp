// Stress driver for the library's threaded host code, built by the CPU tests with AddressSanitizer
// + UndefinedBehaviorSanitizer and, apart, ThreadSanitizer (no GPU, no HIP):
//  - HostExpertPool (the hybrid backend's host workers): tasks of several tokens and entries on
//    pools of 1, 3 and 5 workers, restarted between rounds; every result must equal the 1-worker
//    pool's bit for bit (each value is summed by one participant in a fixed order);
//  - host_expert_ffn (the calibration kernel) on 1 and 4 threads against a plain reference of the
//    same arithmetic within FP32 rounding;
//  - CopyTeam (the bounce ring's pageable-to-pinned copy): ragged sizes on teams of 1 to 5
//    threads, restarted, every copy checked byte for byte;
//  - HostTaskQueue (host tasks of several layer steps queued ahead): tasks pushed in bursts by one
//    thread and waited for by another, out of order and with a time limit, the queue stopped
//    with tasks still queued; every result must equal the 1-worker pool's bit for bit.
// Prints "host stress ok" and exits 0 when every check passes.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "copy_team.h"
#include "host_ffn.h"
#include "moe_internal.h"

using namespace moe;

namespace {

int g_fail = 0;
#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            fprintf(stderr, "FAIL: " __VA_ARGS__); \
            fprintf(stderr, "\n");                \
            ++g_fail;                             \
        }                                         \
    } while (0)

std::vector<uint8_t> random_blob(const Layout& L, std::mt19937_64& rng) {
    // codes: any byte; scale bytes: E8M0 exponents 123..127 (the generator's range)
    std::vector<uint8_t> b(L.blob_bytes);
    for (auto& v : b) v = (uint8_t)rng();
    const int NB = L.NB, NBI = L.NBI;
    for (int tile = 0; tile < L.I / L.GR; ++tile) {
        uint8_t* tsc = b.data() + (size_t)tile * L.gu_tile_bytes + (size_t)L.GR * NB * 32;
        for (size_t i = 0; i < (size_t)L.GR * NB * 2; ++i) tsc[i] = (uint8_t)(123 + rng() % 5);
    }
    uint8_t* ds = b.data() + L.d_scales_off;
    for (size_t i = 0; i < (size_t)L.H * NBI; ++i) ds[i] = (uint8_t)(123 + rng() % 5);
    return b;
}

uint16_t bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void pool_rounds() {
    const Layout L = make_layout(256, 128);
    std::mt19937_64 rng(7);
    std::vector<std::vector<uint8_t>> blobs;
    for (int i = 0; i < 12; ++i) blobs.push_back(random_blob(L, rng));
    const int ntok = 5;
    std::vector<std::vector<uint16_t>> x(ntok, std::vector<uint16_t>(L.H));
    std::normal_distribution<float> nd(0.0f, 1.0f);
    for (auto& v : x)
        for (auto& e : v) e = bf16_bits(nd(rng));
    // entries: token b takes b + 1 experts (token 4 none: zeros), interleaved in the list
    std::vector<HostEntry> ent;
    for (int j = 0; j < 10; ++j) {
        const int b = j % 4;
        ent.push_back({blobs[(j * 5) % blobs.size()].data(), 0.1f * (float)(j + 1), b});
    }
    const uint16_t* xs[kHostMaxTokens];
    for (int b = 0; b < ntok; ++b) xs[b] = x[b].data();

    auto run_pool = [&](HostExpertPool& p, std::vector<std::vector<float>>& y) {
        y.assign(ntok, std::vector<float>(L.H, -1.0f));
        float* ys[kHostMaxTokens];
        for (int b = 0; b < ntok; ++b) ys[b] = y[b].data();
        p.submit(L, ntok, xs, ys, ent.data(), (int)ent.size());
        p.wait();
    };
    std::vector<std::vector<float>> ref;
    {
        HostExpertPool p1;
        CHECK(p1.start(1), "pool start(1)");
        run_pool(p1, ref);
        p1.stop();
    }
    for (float v : ref[4]) CHECK(v == 0.0f, "token without entries must be zero");
    for (int workers : {3, 5, 1, 4}) {
        HostExpertPool p;
        for (int round = 0; round < 2; ++round) {
            CHECK(p.start(workers), "pool start(%d)", workers);
            for (int task = 0; task < 6; ++task) {
                std::vector<std::vector<float>> y;
                run_pool(p, y);
                for (int b = 0; b < ntok; ++b)
                    CHECK(memcmp(y[b].data(), ref[b].data(), L.H * sizeof(float)) == 0,
                          "pool of %d workers, token %d differs from the 1-worker pool", workers, b);
            }
            p.stop();
        }
    }
}

void ffn_threads() {
    const Layout L = make_layout(256, 96);
    std::mt19937_64 rng(11);
    std::vector<std::vector<uint8_t>> blobs;
    for (int i = 0; i < 5; ++i) blobs.push_back(random_blob(L, rng));
    std::vector<const uint8_t*> bp;
    for (auto& b : blobs) bp.push_back(b.data());
    std::vector<float> w = {0.3f, 0.25f, 0.2f, 0.15f, 0.1f};
    std::vector<uint16_t> x(L.H);
    std::normal_distribution<float> nd(0.0f, 1.0f);
    for (auto& e : x) e = bf16_bits(nd(rng));
    std::vector<float> y1(L.H), y4(L.H);
    host_expert_ffn(L, bp.data(), w.data(), 5, x.data(), y1.data(), 1);
    host_expert_ffn(L, bp.data(), w.data(), 5, x.data(), y4.data(), 4);
    double num = 0, den = 0;
    for (int i = 0; i < L.H; ++i) {
        num += (double)(y1[i] - y4[i]) * (y1[i] - y4[i]);
        den += (double)y1[i] * y1[i];
        CHECK(std::isfinite(y1[i]), "non-finite output");
    }
    CHECK(den > 0 && std::sqrt(num / den) < 1e-5, "1 vs 4 threads differ beyond FP32 rounding");
    const double rate = host_expert_rate(L, bp.data(), 5, 3, 0.05);
    CHECK(rate > 0, "host_expert_rate");
}

void copy_rounds() {
    std::mt19937_64 rng(3);
    std::vector<uint8_t> src(3 << 20), dst(3 << 20);
    for (auto& v : src) v = (uint8_t)rng();
    const size_t sizes[] = {0, 1, 4095, 4096, 4097, 65536 + 3, (1 << 20) + 777, 3 << 20};
    for (int threads : {1, 2, 4, 5, 3}) {
        CopyTeam team;
        for (int round = 0; round < 2; ++round) {
            CHECK(team.start(threads) && team.size() == threads, "team start(%d)", threads);
            for (int rep = 0; rep < 3; ++rep)
                for (size_t n : sizes) {
                    const size_t off = (size_t)(rng() % 4096);
                    const size_t m = std::min(n, src.size() - off);
                    memset(dst.data(), 0xA5, dst.size());
                    team.copy(dst.data(), src.data() + off, m);
                    CHECK(memcmp(dst.data(), src.data() + off, m) == 0, "copy of %zu bytes, team %d", m, threads);
                    if (m < dst.size()) CHECK(dst[m] == 0xA5, "copy wrote past its end");
                }
            team.stop();
        }
    }
}

void queue_rounds() {
    const Layout L = make_layout(256, 128);
    std::mt19937_64 rng(11);
    std::vector<std::vector<uint8_t>> blobs;
    for (int i = 0; i < 8; ++i) blobs.push_back(random_blob(L, rng));
    const int ntask = 12, ntok = 3;
    std::normal_distribution<float> nd(0.0f, 1.0f);
    std::vector<std::vector<uint16_t>> x(ntask * ntok, std::vector<uint16_t>(L.H));
    for (auto& v : x)
        for (auto& e : v) e = bf16_bits(nd(rng));
    // task t: token b takes (t + b) % 3 + 1 experts
    std::vector<std::vector<HostEntry>> ent(ntask);
    for (int t = 0; t < ntask; ++t)
        for (int b = 0; b < ntok; ++b)
            for (int j = 0; j <= (t + b) % 3; ++j)
                ent[t].push_back({blobs[(t * 3 + b + j) % blobs.size()].data(), 0.25f * (float)(j + 1), b});
    auto ptrs = [&](int t, std::vector<std::vector<float>>& y, const uint16_t** xs, float** ys) {
        for (int b = 0; b < ntok; ++b) {
            xs[b] = x[t * ntok + b].data();
            ys[b] = y[t * ntok + b].data();
        }
    };
    std::vector<std::vector<float>> ref(ntask * ntok, std::vector<float>(L.H, -1.0f));
    {
        HostExpertPool p1;
        CHECK(p1.start(1), "pool start(1)");
        for (int t = 0; t < ntask; ++t) {
            const uint16_t* xs[kHostMaxTokens];
            float* ys[kHostMaxTokens];
            ptrs(t, ref, xs, ys);
            p1.submit(L, ntok, xs, ys, ent[t].data(), (int)ent[t].size());
            p1.wait();
        }
    }
    for (int workers : {2, 4}) {
        HostExpertPool pool;
        CHECK(pool.start(workers), "pool start(%d)", workers);
        HostTaskQueue q;
        for (int round = 0; round < 3; ++round) {
            CHECK(q.start(&pool), "queue start");  // restarts the thread; task numbers keep counting
            const uint64_t base = q.pushed();
            CHECK(q.done() == base, "a stopped queue has run every task pushed to it");
            std::vector<std::vector<float>> y(ntask * ntok, std::vector<float>(L.H, -1.0f));
            std::vector<uint64_t> seq(ntask, 0);
            // a waiter thread waits for the tasks out of order while this thread pushes them in bursts
            std::atomic<int> pushed{0};
            std::thread waiter([&] {
                for (int t : {3, 1, 7, 11}) {
                    while (pushed.load(std::memory_order_acquire) <= t) std::this_thread::yield();
                    CHECK(q.wait(seq[t], 30.0), "task %d not done in time", t);
                    CHECK(q.done() >= seq[t], "done count below task %d", t);
                }
            });
            for (int t = 0; t < ntask; ++t) {
                const uint16_t* xs[kHostMaxTokens];
                float* ys[kHostMaxTokens];
                ptrs(t, y, xs, ys);
                seq[t] = q.push(L, ntok, xs, ys, ent[t].data(), (int)ent[t].size());
                CHECK(seq[t] == base + (uint64_t)t + 1, "task numbers run on by one");
                pushed.store(t + 1, std::memory_order_release);
                if (t % 4 == 3) std::this_thread::sleep_for(std::chrono::microseconds(200));
            }
            waiter.join();
            if (round == 2) {
                q.stop();  // with tasks possibly still queued: they run before the thread ends
                CHECK(q.done() == base + (uint64_t)ntask, "stop left %llu of %d tasks undone",
                      (unsigned long long)(base + ntask - q.done()), ntask);
            } else {
                CHECK(q.wait(seq[ntask - 1], 30.0), "last task not done in time");
            }
            for (int i = 0; i < ntask * ntok; ++i)
                CHECK(memcmp(y[i].data(), ref[i].data(), L.H * sizeof(float)) == 0,
                      "queued task %d token %d differs from the 1-worker pool", i / ntok, i % ntok);
        }
        pool.stop();
    }
}

}  // namespace

int main() {
    pool_rounds();
    ffn_threads();
    copy_rounds();
    queue_rounds();
    if (g_fail) {
        fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    printf("host stress ok\n");
    return 0;
}
