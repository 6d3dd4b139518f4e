// Host-CPU MXFP4 SwiGLU expert kernel: the expert-processing kernel the
// bandwidth calibration runs to measure B_H, the rate at which the host
// processes experts in this weight format (ai-hardware-zukan.com page, section
// on the hybrid mode: B_H is the speed of the actual expert kernel, not a raw
// memory read, and it depends on the weight format), and the kernel the hybrid
// backend's host workers run on their share of the misses.
//
// It reads the blob in the pool's layout (the layout the GPU kernels read; see
// moe_internal.h), in memory order: gate/up tile by tile (8 rows, chunks
// ordered by (step, segment, row)), then the down section by 8-row tile.  Every
// 16-byte chunk holds one 32-element block of one row; element 2i is the low
// nibble of byte i.  Accumulation is FP32; the intermediate vector is rounded
// to bf16 (round to nearest even) before the down projection, as on the GPU.
// Activations are kept split into the even and odd elements of each 32-block
// (16 + 16 floats), the order in which a chunk's low and high nibbles decode.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#include <immintrin.h>

#include "host_ffn.h"
#include "moe_internal.h"

namespace moe {

namespace {

const float kE2M1[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                         -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

// 2^(e - 127) for every E8M0 byte (255, NaN in the format, is never produced by the pool's writer)
struct E8M0Table {
    float v[256];
    E8M0Table() {
        for (int e = 0; e < 256; ++e) v[e] = std::ldexp(1.0f, e - 127);
    }
};
const E8M0Table kE8M0;
inline float e8m0(uint8_t e) { return kE8M0.v[e]; }

inline float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

inline float round_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) != 0x7F800000u) u += 0x7FFFu + ((u >> 16) & 1u);  // RNE; NaN/inf kept
    u &= 0xFFFF0000u;
    std::memcpy(&f, &u, 4);
    return f;
}

inline float silu_mul(float g, float u) { return g / (1.0f + std::exp(-g)) * u; }

// 32-blocks [b0, b1) of a bf16 vector into FP32, split even / odd
void split_blocks(const uint16_t* x, int b0, int b1, float* ev, float* od) {
    for (int b = b0; b < b1; ++b)
        for (int i = 0; i < 16; ++i) {
            ev[b * 16 + i] = bf16_to_f32(x[b * 32 + 2 * i]);
            od[b * 16 + i] = bf16_to_f32(x[b * 32 + 2 * i + 1]);
        }
}

// ---------------------------------------------------------------- scalar --
float dot_block_scalar(const uint8_t* codes, const float* ev, const float* od) {
    float s = 0.0f;
    for (int i = 0; i < 16; ++i) {
        s += kE2M1[codes[i] & 15] * ev[i];
        s += kE2M1[codes[i] >> 4] * od[i];
    }
    return s;
}

// gate/up tiles [t_begin, t_end) (kGuRows rows each) in memory order: position q (segment
// q % kGuSegments, step q / kGuSegments) holds one block of every row of the tile
void gate_up_scalar(const Layout& L, const uint8_t* blob, const float* xe, const float* xo, float* g, float* u,
                    int t_begin, int t_end) {
    constexpr int GR = kGuRows, S = kGuSegments;
    int b0[S];
    for (int s = 0; s < S; ++s) b0[s] = seg_begin(L.NB, S, s);
    for (int tile = t_begin; tile < t_end; ++tile) {
        const uint8_t* tb = blob + (size_t)tile * L.gu_tile_bytes;
        const uint8_t* ub = tb + (size_t)GR * L.NB * 16;
        const uint8_t* sc = tb + (size_t)GR * L.NB * 32;
        float ag[GR] = {}, au[GR] = {};
        for (int q = 0; q < L.NB; ++q) {
            const int blk = b0[q % S] + q / S;
            for (int r = 0; r < GR; ++r) {
                const size_t c = (size_t)q * GR + r;
                ag[r] += e8m0(sc[c * 2]) * dot_block_scalar(tb + c * 16, xe + blk * 16, xo + blk * 16);
                au[r] += e8m0(sc[c * 2 + 1]) * dot_block_scalar(ub + c * 16, xe + blk * 16, xo + blk * 16);
            }
        }
        for (int r = 0; r < GR; ++r) {
            g[tile * GR + r] = ag[r];
            u[tile * GR + r] = au[r];
        }
    }
}

void down_scalar(const Layout& L, const uint8_t* blob, const float* ae, const float* ao, float w, float* y,
                 int t_begin, int t_end) {
    const uint8_t* dc = blob + L.d_codes_off;
    const uint8_t* ds = blob + L.d_scales_off;
    for (int t8 = t_begin; t8 < t_end; ++t8) {
        float acc[8] = {};
        for (int ib = 0; ib < L.NBI; ++ib)
            for (int r = 0; r < 8; ++r) {
                const size_t cell = ((size_t)t8 * L.NBI + ib) * 8 + r;
                acc[r] += e8m0(ds[cell]) * dot_block_scalar(dc + cell * 16, ae + ib * 16, ao + ib * 16);
            }
        for (int r = 0; r < 8; ++r) y[t8 * 8 + r] += w * acc[r];
    }
}

// --------------------------------------------------------------- AVX-512 --
#define MOE_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx512dq")))

// Software prefetch distance along a unit's code stream.  A unit of the worker
// pool streams a few tens to hundreds of KB from where the previous one ended
// elsewhere in the pool; the hardware prefetcher needs several demand misses to
// pick each new stream up, and prefetching 4 KB ahead measured 22-30 % more
// pool throughput on the EPYC hosts (a prefetch past the end of a blob is a
// hint, not an access, so it cannot fault).
constexpr int kPrefetchBytes = 4096;

MOE_AVX512 inline __m512 dot_block_v(const uint8_t* codes, __m512 lut, __m512 ev, __m512 od) {
    const __m512i v = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(codes)));
    const __m512 lo = _mm512_permutexvar_ps(_mm512_and_si512(v, _mm512_set1_epi32(15)), lut);
    const __m512 hi = _mm512_permutexvar_ps(_mm512_srli_epi32(v, 4), lut);
    return _mm512_fmadd_ps(hi, od, _mm512_mul_ps(lo, ev));
}

MOE_AVX512 void gate_up_avx512(const Layout& L, const uint8_t* blob, const float* xe, const float* xo, float* g,
                               float* u, int t_begin, int t_end) {
    constexpr int GR = kGuRows, S = kGuSegments;
    const __m512 lut = _mm512_loadu_ps(kE2M1);
    int b0[S];
    for (int s = 0; s < S; ++s) b0[s] = seg_begin(L.NB, S, s);
    for (int tile = t_begin; tile < t_end; ++tile) {
        const uint8_t* tb = blob + (size_t)tile * L.gu_tile_bytes;
        const uint8_t* sc = tb + (size_t)GR * L.NB * 32;
        // gate rows from the gate codes, then up rows from the parallel up codes
        for (int part = 0; part < 2; ++part) {
            const uint8_t* cb = tb + (size_t)part * GR * L.NB * 16;
            __m512 acc[GR];
            for (int r = 0; r < GR; ++r) acc[r] = _mm512_setzero_ps();
            for (int q = 0; q < L.NB; ++q) {
                const int blk = b0[q % S] + q / S;
                const __m512 ev = _mm512_loadu_ps(xe + (size_t)blk * 16);
                const __m512 od = _mm512_loadu_ps(xo + (size_t)blk * 16);
                const uint8_t* cq = cb + (size_t)q * GR * 16;
                const uint8_t* sq = sc + (size_t)q * GR * 2 + part;
                _mm_prefetch(reinterpret_cast<const char*>(cq) + kPrefetchBytes, _MM_HINT_T0);
                _mm_prefetch(reinterpret_cast<const char*>(cq) + kPrefetchBytes + 64, _MM_HINT_T0);
#pragma GCC unroll 8
                for (int r = 0; r < GR; ++r)
                    acc[r] = _mm512_fmadd_ps(dot_block_v(cq + r * 16, lut, ev, od), _mm512_set1_ps(e8m0(sq[r * 2])),
                                             acc[r]);
            }
            float* out = part ? u : g;
            for (int r = 0; r < GR; ++r) out[tile * GR + r] = _mm512_reduce_add_ps(acc[r]);
        }
    }
}

MOE_AVX512 void down_avx512(const Layout& L, const uint8_t* blob, const float* ae, const float* ao, float w,
                            float* y, int t_begin, int t_end) {
    const __m512 lut = _mm512_loadu_ps(kE2M1);
    const uint8_t* dc = blob + L.d_codes_off;
    const uint8_t* ds = blob + L.d_scales_off;
    for (int t8 = t_begin; t8 < t_end; ++t8) {
        __m512 acc[8];
        for (int r = 0; r < 8; ++r) acc[r] = _mm512_setzero_ps();
        for (int ib = 0; ib < L.NBI; ++ib) {
            const __m512 ev = _mm512_loadu_ps(ae + (size_t)ib * 16);
            const __m512 od = _mm512_loadu_ps(ao + (size_t)ib * 16);
            const size_t cell = ((size_t)t8 * L.NBI + ib) * 8;
            _mm_prefetch(reinterpret_cast<const char*>(dc + cell * 16) + kPrefetchBytes, _MM_HINT_T0);
            _mm_prefetch(reinterpret_cast<const char*>(dc + cell * 16) + kPrefetchBytes + 64, _MM_HINT_T0);
#pragma GCC unroll 8
            for (int r = 0; r < 8; ++r)
                acc[r] = _mm512_fmadd_ps(dot_block_v(dc + (cell + r) * 16, lut, ev, od),
                                         _mm512_set1_ps(e8m0(ds[cell + r])), acc[r]);
        }
        for (int r = 0; r < 8; ++r) y[t8 * 8 + r] += w * _mm512_reduce_add_ps(acc[r]);
    }
}

bool have_avx512() {
    static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                           __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512dq");
    const char* force = std::getenv("MOE_HOST_FFN_SCALAR");
    return ok && !(force && force[0] == '1');
}

void gate_up_rows(const Layout& L, const uint8_t* blob, const TokenBuf& x, ExpertBuf& e, int t_begin, int t_end,
                  bool vec) {
    if (vec) gate_up_avx512(L, blob, x.xe.data(), x.xo.data(), e.g.data(), e.u.data(), t_begin, t_end);
    else gate_up_scalar(L, blob, x.xe.data(), x.xo.data(), e.g.data(), e.u.data(), t_begin, t_end);
}

void down_rows(const Layout& L, const uint8_t* blob, const ExpertBuf& e, float w, float* y, int t_begin, int t_end,
               bool vec) {
    if (vec) down_avx512(L, blob, e.ae.data(), e.ao.data(), w, y, t_begin, t_end);
    else down_scalar(L, blob, e.ae.data(), e.ao.data(), w, y, t_begin, t_end);
}

// the intermediate vector of 32-blocks [b_begin, b_end): bf16(silu(g) * u), split even / odd
void activation_blocks(ExpertBuf& e, int b_begin, int b_end) {
    for (int b = b_begin; b < b_end; ++b)
        for (int i = 0; i < 16; ++i) {
            e.ae[b * 16 + i] = round_bf16(silu_mul(e.g[b * 32 + 2 * i], e.u[b * 32 + 2 * i]));
            e.ao[b * 16 + i] = round_bf16(silu_mul(e.g[b * 32 + 2 * i + 1], e.u[b * 32 + 2 * i + 1]));
        }
}

// one expert for one token: y += w * down(silu(gate x) * (up x))
void expert_one(const Layout& L, const uint8_t* blob, float w, const TokenBuf& x, ExpertBuf& e, float* y, bool vec) {
    gate_up_rows(L, blob, x, e, 0, L.I / kGuRows, vec);
    activation_blocks(e, 0, L.NBI);
    down_rows(L, blob, e, w, y, 0, L.H / 8, vec);
}

}  // namespace

const char* host_ffn_isa() { return have_avx512() ? "avx512" : "scalar"; }

void host_expert_ffn(const Layout& L, const uint8_t* const* blobs, const float* w, int n, const uint16_t* x,
                     float* y, int threads) {
    TokenBuf xb;
    xb.size(L);
    split_blocks(x, 0, L.NB, xb.xe.data(), xb.xo.data());
    std::fill(y, y + L.H, 0.0f);
    const bool vec = have_avx512();
    threads = std::max(1, std::min(threads, n));
    // experts are shared out over the threads; each expert's weighted output is
    // formed on its own and added to its thread's partial, and the partials are
    // added in thread order (with one thread: the worker pool's order)
    std::vector<std::vector<float>> part(threads, std::vector<float>(L.H, 0.0f));
    auto run = [&](int t) {
        ExpertBuf eb;
        eb.size(L);
        for (int j = t; j < n; j += threads) {
            std::fill(eb.yp.begin(), eb.yp.end(), 0.0f);
            expert_one(L, blobs[j], w[j], xb, eb, eb.yp.data(), vec);
            for (int i = 0; i < L.H; ++i) part[t][i] += eb.yp[i];
        }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < threads; ++t) pool.emplace_back(run, t);
    run(0);
    for (auto& th : pool) th.join();
    for (int t = 0; t < threads; ++t)
        for (int i = 0; i < L.H; ++i) y[i] += part[t][i];
}

// Units of work are handed out dynamically (atomic counters), so a slow or
// descheduled worker delays the task by at most one unit.  Unit sizes aim at
// about four units per participant and kind, within these bounds.
constexpr int kGuTilesPerBlock = 32 / kGuRows;   // gate/up tiles per 32-block of the intermediate vector
constexpr int kGuChunkMax = 8;   // gate/up tiles per unit (whole 32-blocks of the intermediate vector)
constexpr int kDChunkMax = 32;   // 8-row output tiles of one entry per unit

inline int unit_size(long items, int participants, int max_chunk) {
    const long c = items / (4L * participants);
    return (int)std::max<long>(1, std::min<long>(max_chunk, c));
}

// An entry's units are taken in the order k -> k * step mod n, with step
// coprime to n (a permutation) and about n / participants, so the units running
// at the same time read places far apart in the expert rather than adjacent
// ones (measured 3-4 % faster on the EPYC hosts).
inline int unit_step(int n, int participants) {
    if (n <= 1) return 1;
    int s = std::max(1, n / participants);
    while (std::gcd(s, n) != 1) ++s;
    return s;
}

// ------------------------------------------------------------- worker pool --

HostExpertPool::~HostExpertPool() { stop(); }

bool HostExpertPool::start(int n_workers) {
    stop();
    if (n_workers < 1) return false;
    n_ = n_workers;
    quit_.store(false);
    gen_.store(0);
    done_.store(0);
    try {
        for (int t = 0; t < n_; ++t) threads_.emplace_back(&HostExpertPool::run, this, t);
    } catch (...) {
        stop();
        return false;
    }
    return true;
}

void HostExpertPool::stop() {
    if (!threads_.empty()) {
        quit_.store(true);
        {
            std::lock_guard<std::mutex> lk(mu_);
            gen_.fetch_add(1);
        }
        cv_.notify_all();
        for (auto& th : threads_) th.join();
        threads_.clear();
    }
    n_ = 0;
}

void HostExpertPool::submit(const Layout& L, int n_tok, const uint16_t* const* x, float* const* y,
                            const HostEntry* entries, int n) {
    task_.L = L;
    task_.ntok = std::max(0, std::min(n_tok, kHostMaxTokens));
    n = std::max(0, std::min(n, kHostMaxEntries));
    for (int b = 0; b < task_.ntok; ++b) {
        task_.x[b] = x[b];
        task_.y[b] = y[b];
    }
    // entries grouped by token; a token's entries keep their order
    int pos = 0;
    for (int b = 0; b < task_.ntok; ++b) {
        task_.tok_begin[b] = pos;
        for (int j = 0; j < n; ++j)
            if (entries[j].tok == b) task_.e[pos++] = entries[j];
    }
    task_.tok_begin[task_.ntok] = pos;
    task_.n = pos;
    if ((int)ebuf_.size() < task_.n) ebuf_.resize(task_.n);
    for (int j = 0; j < task_.n; ++j) ebuf_[j].size(L);
    if ((int)xbuf_.size() < task_.ntok) xbuf_.resize(task_.ntok);
    for (int b = 0; b < task_.ntok; ++b) xbuf_[b].size(L);
    // about four units per participant (workers and the waiting caller) and kind
    const int np = n_ + 1;
    task_.gu_chunk = std::max(kGuTilesPerBlock, unit_size((long)task_.n * (L.I / kGuRows), np, kGuChunkMax) /
                                                     kGuTilesPerBlock * kGuTilesPerBlock);
    task_.d_chunk = unit_size((long)task_.n * (L.H / 8), np, kDChunkMax);
    task_.gu_per = (L.I / kGuRows + task_.gu_chunk - 1) / task_.gu_chunk;
    task_.d_per = (L.H / 8 + task_.d_chunk - 1) / task_.d_chunk;
    task_.gu_step = unit_step(task_.gu_per, np);
    task_.d_step = unit_step(task_.d_per, np);
    for (int j = 0; j < task_.n; ++j) gu_left_[j].v.store(task_.gu_per, std::memory_order_relaxed);
    for (int b = 0; b < task_.ntok; ++b)
        d_left_[b].v.store((task_.tok_begin[b + 1] - task_.tok_begin[b]) * task_.d_per, std::memory_order_relaxed);
    for (std::atomic<int>* c : {&x_next_, &x_done_, &main_next_, &tok_done_}) c->store(0, std::memory_order_relaxed);
    done_.store(0);
    t_submit_ = std::chrono::steady_clock::now();
    {
        std::lock_guard<std::mutex> lk(mu_);
        gen_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
}

void HostExpertPool::wait() {
    // the caller works on the task too, then waits until every worker has left it
    // (a worker still inside could otherwise take a unit of the next task)
    work(have_avx512());
    while (done_.load(std::memory_order_acquire) < n_) _mm_pause();
}

// one participant's share of the current task.  The x units come first (the
// gate/up units of any entry may need any token's x); then the main list, where
// segment s holds the gate/up units of entry s followed by the down units of
// entry s - 1, so a down unit is taken well after its entry's gate/up units
// and rarely waits for them.
void HostExpertPool::work(bool vec) {
    const Layout& L = task_.L;
    const int n = task_.n, ntok = task_.ntok;
    auto token_done = [&]() {
        if (tok_done_.fetch_add(1, std::memory_order_acq_rel) == ntok - 1)
            busy_ns_.fetch_add((uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(
                                   std::chrono::steady_clock::now() - t_submit_).count());
    };
    // hidden states to FP32, one unit per token; a token without entries gets zeros
    for (int b; (b = x_next_.fetch_add(1, std::memory_order_relaxed)) < ntok;) {
        split_blocks(task_.x[b], 0, L.NB, xbuf_[b].xe.data(), xbuf_[b].xo.data());
        if (task_.tok_begin[b + 1] == task_.tok_begin[b]) {
            std::fill(task_.y[b], task_.y[b] + L.H, 0.0f);
            token_done();
        }
        x_done_.fetch_add(1, std::memory_order_release);
    }
    while (x_done_.load(std::memory_order_acquire) < ntok) _mm_pause();
    const int ngu = L.I / kGuRows, nt8 = L.H / 8;
    const int gc = task_.gu_chunk, gu_per = task_.gu_per, dc = task_.d_chunk, d_per = task_.d_per;
    const int seg = gu_per + d_per, n_main = n * seg;
    for (int u; (u = main_next_.fetch_add(1, std::memory_order_relaxed)) < n_main;) {
        // unit u of the main list -> (gate/up or down, entry, unit within the entry)
        bool is_gu;
        int j, k;
        if (u < gu_per) {
            is_gu = true;
            j = 0;
            k = u;
        } else {
            const int v = u - gu_per, s = 1 + v / seg, off = v - (s - 1) * seg;
            if (s < n && off < gu_per) {
                is_gu = true;
                j = s;
                k = off;
            } else {
                is_gu = false;
                j = s - 1;
                k = s < n ? off - gu_per : off;
            }
        }
        const HostEntry& e = task_.e[j];
        if (is_gu) {
            const int kk = (int)((long)k * task_.gu_step % gu_per);
            const int t0 = kk * gc, t1 = std::min(ngu, t0 + gc);
            gate_up_rows(L, e.blob, xbuf_[e.tok], ebuf_[j], t0, t1, vec);
            activation_blocks(ebuf_[j], t0 / kGuTilesPerBlock, t1 / kGuTilesPerBlock);
            gu_left_[j].v.fetch_sub(1, std::memory_order_release);
            continue;
        }
        // down rows of entry j: w * (the expert's output rows) into its own buffer
        while (gu_left_[j].v.load(std::memory_order_acquire) > 0) _mm_pause();
        const int kk = (int)((long)k * task_.d_step % d_per);
        const int d0 = kk * dc, d1 = std::min(nt8, d0 + dc);
        float* yp = ebuf_[j].yp.data();
        std::fill(yp + d0 * 8, yp + d1 * 8, 0.0f);
        down_rows(L, e.blob, ebuf_[j], e.w, yp, d0, d1, vec);
        if (d_left_[e.tok].v.fetch_sub(1, std::memory_order_acq_rel) == 1) {
            // the token's last down unit: its output is the sum of its entries, in order
            const int b = e.tok;
            float* y = task_.y[b];
            std::fill(y, y + L.H, 0.0f);
            for (int jj = task_.tok_begin[b]; jj < task_.tok_begin[b + 1]; ++jj) {
                const float* p = ebuf_[jj].yp.data();
                for (int i = 0; i < L.H; ++i) y[i] += p[i];
            }
            token_done();
        }
    }
}

void HostExpertPool::run(int) {
    const bool vec = have_avx512();
    int seen = 0;
    for (;;) {
        // spin for the next task for a while (decode steps arrive every few tens of
        // microseconds), then sleep until one comes
        const auto t0 = std::chrono::steady_clock::now();
        int spins = 0;
        while (gen_.load(std::memory_order_acquire) == seen) {
            _mm_pause();
            if ((++spins & 1023) == 0 &&
                std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(20)) {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return gen_.load(std::memory_order_acquire) != seen; });
            }
        }
        seen = gen_.load(std::memory_order_acquire);
        if (quit_.load()) return;
        work(vec);
        done_.fetch_add(1, std::memory_order_acq_rel);  // this worker has left the task
    }
}

double host_expert_rate(const Layout& L, const uint8_t* const* blobs, int n, int threads, double min_seconds) {
    threads = std::max(1, threads);
    std::vector<uint16_t> x(L.H);
    for (int i = 0; i < L.H; ++i) x[i] = 0x3C00u + (uint16_t)(i % 64);  // bf16 values near 0.008
    const bool vec = have_avx512();
    std::atomic<long> next{0};
    std::atomic<bool> stop{false};
    std::vector<long> done(threads, 0);
    auto run = [&](int t) {
        TokenBuf xb;
        xb.size(L);
        split_blocks(x.data(), 0, L.NB, xb.xe.data(), xb.xo.data());
        ExpertBuf eb;
        eb.size(L);
        std::vector<float> y(L.H, 0.0f);
        while (!stop.load(std::memory_order_relaxed)) {
            const long j = next.fetch_add(1);
            expert_one(L, blobs[j % n], 1.0f, xb, eb, y.data(), vec);
            ++done[t];
        }
    };
    const auto t0 = std::chrono::steady_clock::now();
    std::vector<std::thread> pool;
    // nothing may throw out of here (the C ABI calls it): a thread that cannot start leaves the
    // measurement to the ones that did, and the rate counts only their work
    try {
        pool.reserve((size_t)threads);
        for (int t = 0; t < threads; ++t) pool.emplace_back(run, t);
    } catch (...) {
    }
    if (pool.empty()) return 0.0;
    std::this_thread::sleep_for(std::chrono::duration<double>(min_seconds));
    stop.store(true);
    for (auto& th : pool) th.join();
    const double dt = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    long total = 0;
    for (long d : done) total += d;
    return (double)total * (double)L.blob_bytes / dt;
}

HostTaskQueue::~HostTaskQueue() { stop(); }

bool HostTaskQueue::start(HostExpertPool* pool) {
    stop();
    pool_ = pool;
    quit_ = false;
    try {
        th_ = std::thread(&HostTaskQueue::run, this);
    } catch (...) {
        return false;
    }
    return true;
}

void HostTaskQueue::stop() {
    if (!th_.joinable()) return;
    {
        std::lock_guard<std::mutex> lk(mu_);
        quit_ = true;
    }
    cv_push_.notify_all();
    th_.join();
}

uint64_t HostTaskQueue::push(const Layout& L, int n_tok, const uint16_t* const* x, float* const* y,
                             const HostEntry* e, int n) {
    Item it;
    it.L = L;
    it.n_tok = std::max(0, std::min(n_tok, kHostMaxTokens));
    it.n = std::max(0, std::min(n, kHostMaxEntries));
    for (int b = 0; b < it.n_tok; ++b) {
        it.x[b] = x[b];
        it.y[b] = y[b];
    }
    std::copy(e, e + it.n, it.e);
    {
        std::lock_guard<std::mutex> lk(mu_);
        q_.push_back(it);
    }
    cv_push_.notify_one();
    return ++pushed_;
}

bool HostTaskQueue::wait(uint64_t seq, double timeout_s) {
    if (done() >= seq) return true;
    // a system-clock deadline: the wait then maps to pthread_cond_timedwait, which thread checkers
    // follow (a steady-clock wait maps to pthread_cond_clockwait, which older ones do not)
    const auto deadline = std::chrono::system_clock::now() +
                          std::chrono::duration_cast<std::chrono::system_clock::duration>(
                              std::chrono::duration<double>(timeout_s));
    std::unique_lock<std::mutex> lk(mu_);
    return cv_done_.wait_until(lk, deadline, [&] { return done() >= seq; });
}

// the dispatcher: one task at a time on the pool (this thread works on it too), in push order;
// on stop the queued tasks still run, so every waiter is released
void HostTaskQueue::run() {
    for (;;) {
        Item it;
        {
            std::unique_lock<std::mutex> lk(mu_);
            cv_push_.wait(lk, [&] { return quit_ || !q_.empty(); });
            if (q_.empty()) return;
            it = q_.front();
            q_.pop_front();
        }
        pool_->submit(it.L, it.n_tok, it.x, it.y, it.e, it.n);
        pool_->wait();
        {
            std::lock_guard<std::mutex> lk(mu_);
            const uint64_t d = done_.fetch_add(1, std::memory_order_acq_rel) + 1;
            if (mirror_) __atomic_store_n(mirror_, d, __ATOMIC_RELEASE);
        }
        cv_done_.notify_all();
    }
}

}  // namespace moe
