// Host-CPU MXFP4 SwiGLU expert kernel: the expert-processing kernel the
// bandwidth calibration runs to measure B_H, the rate at which the host
// processes experts in this weight format (ai-hardware-zukan.com page, section
// on the hybrid mode: B_H is the speed of the actual expert kernel, not a raw
// memory read, and it depends on the weight format).
//
// It reads the blob in the pool's layout (the layout the GPU kernels read; see
// moe_internal.h), in memory order: gate/up tile by tile (16 rows, chunks
// ordered by (step, segment, row)), then the down section by 8-row tile.  Every
// 16-byte chunk holds one 32-element block of one row; element 2i is the low
// nibble of byte i.  Accumulation is FP32; the intermediate vector is rounded
// to bf16 (round to nearest even) before the down projection, as on the GPU.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstring>
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

// per-call buffers: x and a split into even / odd elements of each 32-block
struct Work {
    std::vector<float> xe, xo, ae, ao, g, u;
    void size(const Layout& L) {
        xe.assign((size_t)L.NB * 16, 0.0f);
        xo.assign((size_t)L.NB * 16, 0.0f);
        ae.assign((size_t)L.NBI * 16, 0.0f);
        ao.assign((size_t)L.NBI * 16, 0.0f);
        g.assign(L.I, 0.0f);
        u.assign(L.I, 0.0f);
    }
};

void split_even_odd(const float* v, int n_blocks, float* ev, float* od) {
    for (int b = 0; b < n_blocks; ++b)
        for (int i = 0; i < 16; ++i) {
            ev[b * 16 + i] = v[b * 32 + 2 * i];
            od[b * 16 + i] = v[b * 32 + 2 * i + 1];
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

void gate_up_scalar(const Layout& L, const uint8_t* blob, Work& wk) {
    int b0[16];
    for (int s = 0; s < 16; ++s) b0[s] = seg_begin(L.NB, 16, s);
    for (int tile = 0; tile < L.I / 16; ++tile) {
        const uint8_t* tb = blob + (size_t)tile * 16 * L.NB * 34;
        const uint8_t* ub = tb + (size_t)16 * L.NB * 16;
        const uint8_t* sc = tb + (size_t)16 * L.NB * 32;
        float ag[16] = {}, au[16] = {};
        for (int q = 0; q < L.NB; ++q) {
            const int blk = b0[q & 15] + (q >> 4);
            for (int r = 0; r < 16; ++r) {
                const size_t c = (size_t)q * 16 + r;
                ag[r] += e8m0(sc[c * 2]) * dot_block_scalar(tb + c * 16, &wk.xe[blk * 16], &wk.xo[blk * 16]);
                au[r] += e8m0(sc[c * 2 + 1]) * dot_block_scalar(ub + c * 16, &wk.xe[blk * 16], &wk.xo[blk * 16]);
            }
        }
        for (int r = 0; r < 16; ++r) {
            wk.g[tile * 16 + r] = ag[r];
            wk.u[tile * 16 + r] = au[r];
        }
    }
}

void down_scalar(const Layout& L, const uint8_t* blob, const Work& wk, float w, float* y) {
    const uint8_t* dc = blob + L.d_codes_off;
    const uint8_t* ds = blob + L.d_scales_off;
    for (int t8 = 0; t8 < L.H / 8; ++t8) {
        float acc[8] = {};
        for (int ib = 0; ib < L.NBI; ++ib)
            for (int r = 0; r < 8; ++r) {
                const size_t cell = ((size_t)t8 * L.NBI + ib) * 8 + r;
                acc[r] += e8m0(ds[cell]) * dot_block_scalar(dc + cell * 16, &wk.ae[ib * 16], &wk.ao[ib * 16]);
            }
        for (int r = 0; r < 8; ++r) y[t8 * 8 + r] += w * acc[r];
    }
}

// --------------------------------------------------------------- AVX-512 --
#define MOE_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx512dq")))

MOE_AVX512 inline __m512 dot_block_v(const uint8_t* codes, __m512 lut, __m512 ev, __m512 od) {
    const __m512i v = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(codes)));
    const __m512 lo = _mm512_permutexvar_ps(_mm512_and_si512(v, _mm512_set1_epi32(15)), lut);
    const __m512 hi = _mm512_permutexvar_ps(_mm512_srli_epi32(v, 4), lut);
    return _mm512_fmadd_ps(hi, od, _mm512_mul_ps(lo, ev));
}

MOE_AVX512 void gate_up_avx512(const Layout& L, const uint8_t* blob, Work& wk) {
    const __m512 lut = _mm512_loadu_ps(kE2M1);
    int b0[16];
    for (int s = 0; s < 16; ++s) b0[s] = seg_begin(L.NB, 16, s);
    for (int tile = 0; tile < L.I / 16; ++tile) {
        const uint8_t* tb = blob + (size_t)tile * 16 * L.NB * 34;
        const uint8_t* sc = tb + (size_t)16 * L.NB * 32;
        // gate rows from the gate codes, then up rows from the parallel up codes
        for (int part = 0; part < 2; ++part) {
            const uint8_t* cb = tb + (size_t)part * 16 * L.NB * 16;
            __m512 acc[16];
            for (int r = 0; r < 16; ++r) acc[r] = _mm512_setzero_ps();
            for (int q = 0; q < L.NB; ++q) {
                const int blk = b0[q & 15] + (q >> 4);
                const __m512 ev = _mm512_loadu_ps(&wk.xe[(size_t)blk * 16]);
                const __m512 od = _mm512_loadu_ps(&wk.xo[(size_t)blk * 16]);
                const uint8_t* cq = cb + (size_t)q * 256;
                const uint8_t* sq = sc + (size_t)q * 32 + part;
#pragma GCC unroll 16
                for (int r = 0; r < 16; ++r)
                    acc[r] = _mm512_fmadd_ps(dot_block_v(cq + r * 16, lut, ev, od), _mm512_set1_ps(e8m0(sq[r * 2])),
                                             acc[r]);
            }
            float* out = part ? wk.u.data() : wk.g.data();
            for (int r = 0; r < 16; ++r) out[tile * 16 + r] = _mm512_reduce_add_ps(acc[r]);
        }
    }
}

MOE_AVX512 void down_avx512(const Layout& L, const uint8_t* blob, const Work& wk, float w, float* y) {
    const __m512 lut = _mm512_loadu_ps(kE2M1);
    const uint8_t* dc = blob + L.d_codes_off;
    const uint8_t* ds = blob + L.d_scales_off;
    for (int t8 = 0; t8 < L.H / 8; ++t8) {
        __m512 acc[8];
        for (int r = 0; r < 8; ++r) acc[r] = _mm512_setzero_ps();
        for (int ib = 0; ib < L.NBI; ++ib) {
            const __m512 ev = _mm512_loadu_ps(&wk.ae[(size_t)ib * 16]);
            const __m512 od = _mm512_loadu_ps(&wk.ao[(size_t)ib * 16]);
            const size_t cell = ((size_t)t8 * L.NBI + ib) * 8;
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

// one expert for one token: y += w * down(silu(gate x) * (up x))
void expert_one(const Layout& L, const uint8_t* blob, float w, Work& wk, float* y, bool vec) {
    if (vec) gate_up_avx512(L, blob, wk);
    else gate_up_scalar(L, blob, wk);
    std::vector<float> a(L.I);
    for (int i = 0; i < L.I; ++i) a[i] = round_bf16(silu_mul(wk.g[i], wk.u[i]));
    split_even_odd(a.data(), L.NBI, wk.ae.data(), wk.ao.data());
    if (vec) down_avx512(L, blob, wk, w, y);
    else down_scalar(L, blob, wk, w, y);
}

}  // namespace

const char* host_ffn_isa() { return have_avx512() ? "avx512" : "scalar"; }

void host_expert_ffn(const Layout& L, const uint8_t* const* blobs, const float* w, int n, const uint16_t* x,
                     float* y, int threads) {
    std::vector<float> xf(L.H);
    for (int i = 0; i < L.H; ++i) xf[i] = bf16_to_f32(x[i]);
    std::fill(y, y + L.H, 0.0f);
    const bool vec = have_avx512();
    threads = std::max(1, std::min(threads, n));
    // experts are shared out over the threads; each thread sums into its own
    // partial, and the partials are added in thread order
    std::vector<std::vector<float>> part(threads, std::vector<float>(L.H, 0.0f));
    auto run = [&](int t) {
        Work wk;
        wk.size(L);
        split_even_odd(xf.data(), L.NB, wk.xe.data(), wk.xo.data());
        for (int j = t; j < n; j += threads) expert_one(L, blobs[j], w[j], wk, part[t].data(), vec);
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < threads; ++t) pool.emplace_back(run, t);
    run(0);
    for (auto& th : pool) th.join();
    for (int t = 0; t < threads; ++t)
        for (int i = 0; i < L.H; ++i) y[i] += part[t][i];
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
        Work wk;
        wk.size(L);
        std::vector<float> xf(L.H), y(L.H, 0.0f);
        for (int i = 0; i < L.H; ++i) xf[i] = bf16_to_f32(x[i]);
        split_even_odd(xf.data(), L.NB, wk.xe.data(), wk.xo.data());
        while (!stop.load(std::memory_order_relaxed)) {
            const long j = next.fetch_add(1);
            expert_one(L, blobs[j % n], 1.0f, wk, y.data(), vec);
            ++done[t];
        }
    };
    const auto t0 = std::chrono::steady_clock::now();
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) pool.emplace_back(run, t);
    std::this_thread::sleep_for(std::chrono::duration<double>(min_seconds));
    stop.store(true);
    for (auto& th : pool) th.join();
    const double dt = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    long total = 0;
    for (long d : done) total += d;
    return (double)total * (double)L.blob_bytes / dt;
}

}  // namespace moe
