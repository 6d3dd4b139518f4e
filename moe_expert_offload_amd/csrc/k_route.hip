// K1 router logits; K2 top-k + softmax + cache resolve; for gfx950 (wave64).
//
// Router (pirouter.ai "FreeToken x RTX 5090" page, mechanism section: the
// router picks the experts each token uses, and the cache follows it).  The
// pages fix neither the logit precision nor the selection rule; this library
// computes each logit in FP32 with one fixed summation order (element i ->
// lane (i/8) mod 64, each lane adds its products in increasing i, then an
// xor-butterfly over 64 lanes), selects the k largest logits with ties going
// to the lower expert index, and normalises the k selected logits with a
// softmax.  Products of two bf16 values are exact in FP32, so an FMA and a
// multiply-add agree and only the additions round.
//
// Resolve (ai-hardware-zukan.com FreeToken vs Ollama page, section on how
// misses are made up for: the cache unit is the (layer, expert) pair and the
// least recently used entry is replaced; gaming-st.com DeepSeek page: one
// global LRU over all layers).  The requested set of a step is the ascending
// unique expert ids of its tokens; hits are refreshed first (ascending id),
// then every miss (ascending id) takes the next victim: empty slots by
// ascending index, then the least recently used.  The GPU keeps the victim
// order explicitly as an array of all C slots sorted by (last use, index) with
// empty slots first, so each step is one O(C) stable compaction.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------------- K1 --

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float fold8(uint4 wv, uint4 xv, float p) {
    p = fmaf(bf16lo(wv.x), bf16lo(xv.x), p);
    p = fmaf(bf16hi(wv.x), bf16hi(xv.x), p);
    p = fmaf(bf16lo(wv.y), bf16lo(xv.y), p);
    p = fmaf(bf16hi(wv.y), bf16hi(xv.y), p);
    p = fmaf(bf16lo(wv.z), bf16lo(xv.z), p);
    p = fmaf(bf16hi(wv.z), bf16hi(xv.z), p);
    p = fmaf(bf16lo(wv.w), bf16lo(xv.w), p);
    p = fmaf(bf16hi(wv.w), bf16hi(xv.w), p);
    return p;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The xor butterfly over the 64 lanes: p + (p of lane ^ d) for d = 32, 16, 8, 4, 2, 1, in that
// order, so every lane ends with the same sum.  The partner values come from the gfx950 lane
// swaps (d = 32, 16) and DPP (d = 8: rotate a row of 16 by 8; d = 4: mirror each half-row, then
// reverse each quad; d = 2, 1: quad permutes): register moves instead of LDS round trips.  A
// lane adds its own value and its partner's in whichever order the swap returns them, which
// gives the same bits since IEEE addition is commutative.
__device__ __forceinline__ float xor_butterfly(float p) {
    {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
        p = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
        p = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    p = p + dpp_f32<0x128>(p);                      // row_ror:8
    p = p + dpp_f32<0x1B>(dpp_f32<0x141>(p));       // row_half_mirror, then quad_perm(3,2,1,0)
    p = p + dpp_f32<0x4E>(p);                       // quad_perm(2,3,0,1)
    p = p + dpp_f32<0xB1>(p);                       // quad_perm(1,0,3,2)
    return p;
}

// order-preserving 64-bit key: larger logit first, then lower expert index
__device__ __forceinline__ uint64_t topk_key(float z, int e) {
    uint32_t u = __float_as_uint(z + 0.0f);  // -0 -> +0
    uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// the logit back from its key (exact; -0 comes back as +0)
__device__ __forceinline__ float topk_key_logit(uint64_t key) {
    const uint32_t o = (uint32_t)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// lane permutations inside a row of 16 lanes (DPP)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp_u64(uint64_t v) {
    const uint64_t o = ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
    return o > v ? o : v;
}

// the larger of a lane's value and its partner's after a lane swap: each lane gets its own value
// and its partner's back as the swap's two results, in either order
__device__ __forceinline__ uint64_t max_swapped_u64(uint32_t lo0, uint32_t hi0, uint32_t lo1, uint32_t hi1) {
    const uint64_t a = ((uint64_t)hi0 << 32) | lo0, b = ((uint64_t)hi1 << 32) | lo1;
    return a > b ? a : b;
}

// maximum over the wave, in every lane, in register moves only: DPP inside each row of 16, then
// the gfx950 lane swaps across rows (16) and halves (32).  A maximum does not depend on the order
// in which values meet, so any exchange pattern gives the same result.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_dpp_u64<0xB1>(v);   // quad_perm(1,0,3,2): lane ^ 1
    v = max_dpp_u64<0x4E>(v);   // quad_perm(2,3,0,1): lane ^ 2
    v = max_dpp_u64<0x141>(v);  // row_half_mirror: the other quad of each 8
    v = max_dpp_u64<0x140>(v);  // row_mirror: the other 8 of each 16
    {
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        v = max_swapped_u64(lo[0], hi[0], lo[1], hi[1]);
    }
    {
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        v = max_swapped_u64(lo[0], hi[0], lo[1], hi[1]);
    }
    return v;
}

// one wave per (expert row, token); a lane's groups g = lane + 64 i are
// loaded eight at a time (all loads of a batch in flight together), then
// folded in increasing g
constexpr int K1_BATCH = 8;

__global__ __launch_bounds__(64) void k1_logits(K1Args a) {
    const int lane = threadIdx.x;
    const int e = blockIdx.x, b = blockIdx.y;
    const uint16_t* x = a.x + (size_t)b * a.H;
    const uint16_t* W = a.W + (size_t)e * a.H;
    float p = 0.0f;
    const int ng = a.H >> 3;
    for (int g0 = lane; g0 < ng; g0 += 64 * K1_BATCH) {
        uint4 wv[K1_BATCH], xv[K1_BATCH];
#pragma unroll
        for (int i = 0; i < K1_BATCH; ++i) {
            const int g = g0 + 64 * i;
            const int gc = g < ng ? g : g0;  // past the row: re-read the first group, unused
            wv[i] = *reinterpret_cast<const uint4*>(W + (size_t)gc * 8);
            xv[i] = *reinterpret_cast<const uint4*>(x + (size_t)gc * 8);
        }
#pragma unroll
        for (int i = 0; i < K1_BATCH; ++i)
            if (g0 + 64 * i < ng) p = fold8(wv[i], xv[i], p);
    }
    p = xor_butterfly(p);
    if (lane == 0) a.z[(size_t)b * a.E + e] = p;
}

// Many tokens (a prefill chunk, more than 16): a workgroup of 4 waves takes 8
// experts x 16 tokens.  Each wave keeps its 2 experts' router rows in registers
// as FP32 (lane l holds groups g = l + 64 i, i < G, of 8 elements each); the
// workgroup converts each token pair's activations once to FP32 and stages them
// in LDS (the 8 elements of a group as two 16-byte planes, so a wave's reads of
// one plane are 64 consecutive 16-byte cells), double-buffered with one barrier
// per pair.  Every logit is still lane l's fold over its groups in increasing g
// (a group past the row leaves the fold unchanged), then the xor butterfly: the
// same bits as k1_logits (bf16 -> FP32 is exact, and the products are exact in
// FP32 either way).  Lanes 0..3 store a token pair's 4 logits.
constexpr int K1T_EXPW = 2, K1T_WAVES = 4, K1T_TOK = 16;

template <int G>
__global__ __launch_bounds__(64 * K1T_WAVES) void k1_logits_tiled(K1Args a) {
    constexpr int NT = 64 * K1T_WAVES, GMAX = 64 * G;
    constexpr int UPT = (2 * GMAX + NT - 1) / NT;    // staging units (8 activations) per thread and pair
    __shared__ float4 xs[2][2][2][GMAX];             // [buffer][token of the pair][plane][group]
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int e0 = (blockIdx.x * K1T_WAVES + w) * K1T_EXPW;
    const int b0 = blockIdx.y * K1T_TOK;
    const int ng = a.H >> 3;
    float wf[K1T_EXPW][G][8];
    bool gv[G];
#pragma unroll
    for (int i = 0; i < G; ++i) gv[i] = lane + 64 * i < ng;
#pragma unroll
    for (int j = 0; j < K1T_EXPW; ++j) {
        const int e = e0 + j < a.E ? e0 + j : a.E - 1;
        const uint16_t* W = a.W + (size_t)e * a.H;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int g = lane + 64 * i;
            const uint4 v = *reinterpret_cast<const uint4*>(W + (size_t)(g < ng ? g : 0) * 8);
            wf[j][i][0] = bf16lo(v.x);
            wf[j][i][1] = bf16hi(v.x);
            wf[j][i][2] = bf16lo(v.y);
            wf[j][i][3] = bf16hi(v.y);
            wf[j][i][4] = bf16lo(v.z);
            wf[j][i][5] = bf16hi(v.z);
            wf[j][i][6] = bf16lo(v.w);
            wf[j][i][7] = bf16hi(v.w);
        }
    }
    // staging unit u < 2 ng of a pair: token u / ng of the pair, group u % ng
    uint4 sv[UPT];
    auto load_pair = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            const int u = threadIdx.x + NT * k;
            const int tp = u >= ng ? 1 : 0, g = u - tp * ng;
            const int b = b0 + t + tp;
            const uint16_t* x = a.x + (size_t)(b < a.B ? b : a.B - 1) * a.H;
            sv[k] = *reinterpret_cast<const uint4*>(x + (size_t)(u < 2 * ng ? g : 0) * 8);
        }
    };
    auto store_pair = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            const int u = threadIdx.x + NT * k;
            const int tp = u >= ng ? 1 : 0, g = u - tp * ng;
            if (u < 2 * ng) {
                xs[buf][tp][0][g] = make_float4(bf16lo(sv[k].x), bf16hi(sv[k].x), bf16lo(sv[k].y), bf16hi(sv[k].y));
                xs[buf][tp][1][g] = make_float4(bf16lo(sv[k].z), bf16hi(sv[k].z), bf16lo(sv[k].w), bf16hi(sv[k].w));
            }
        }
    };
    auto logits = [&](int t, int buf) __attribute__((always_inline)) {
        float out = 0.0f;   // lane k < 4: logit of (token t + k / 2, expert e0 + k % 2)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            float p[K1T_EXPW];
#pragma unroll
            for (int j = 0; j < K1T_EXPW; ++j) p[j] = 0.0f;
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int g = gv[i] ? lane + 64 * i : 0;
                const float4 lo = xs[buf][tp][0][g], hi = xs[buf][tp][1][g];
#pragma unroll
                for (int j = 0; j < K1T_EXPW; ++j) {
                    float q = p[j];
                    q = fmaf(wf[j][i][0], lo.x, q);
                    q = fmaf(wf[j][i][1], lo.y, q);
                    q = fmaf(wf[j][i][2], lo.z, q);
                    q = fmaf(wf[j][i][3], lo.w, q);
                    q = fmaf(wf[j][i][4], hi.x, q);
                    q = fmaf(wf[j][i][5], hi.y, q);
                    q = fmaf(wf[j][i][6], hi.z, q);
                    q = fmaf(wf[j][i][7], hi.w, q);
                    p[j] = gv[i] ? q : p[j];
                }
            }
#pragma unroll
            for (int j = 0; j < K1T_EXPW; ++j) {
                const float z = xor_butterfly(p[j]);
                out = lane == tp * K1T_EXPW + j ? z : out;
            }
        }
        if (lane < 2 * K1T_EXPW) {
            const int b = b0 + t + lane / K1T_EXPW, e = e0 + lane % K1T_EXPW;
            if (b < a.B && e < a.E) a.z[(size_t)b * a.E + e] = out;
        }
    };
    load_pair(0);
    store_pair(0);
    load_pair(2);
    __syncthreads();
    for (int t = 0; t < K1T_TOK; t += 2) {
        logits(t, (t >> 1) & 1);
        // pair t + 2 goes to the buffer read one pair ago (every wave has passed the barrier since)
        if (t + 2 < K1T_TOK) store_pair(((t >> 1) + 1) & 1);
        if (t + 4 < K1T_TOK) load_pair(t + 4);
        __syncthreads();
    }
}

int launch_k1(const K1Args& a, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const int G = (a.H / 8 + 63) / 64;  // groups per lane (H <= 4096: G <= 8)
    if (a.B > K1T_TOK && G <= 8) {
        const int epw = K1T_WAVES * K1T_EXPW;   // experts per workgroup
        const dim3 grid((a.E + epw - 1) / epw, (a.B + K1T_TOK - 1) / K1T_TOK);
        if (G <= 2)
            hipLaunchKernelGGL(k1_logits_tiled<2>, grid, dim3(64 * K1T_WAVES), 0, st, a);
        else if (G <= 4)
            hipLaunchKernelGGL(k1_logits_tiled<4>, grid, dim3(64 * K1T_WAVES), 0, st, a);
        else if (G <= 6)
            hipLaunchKernelGGL(k1_logits_tiled<6>, grid, dim3(64 * K1T_WAVES), 0, st, a);
        else
            hipLaunchKernelGGL(k1_logits_tiled<8>, grid, dim3(64 * K1T_WAVES), 0, st, a);
    } else {
        hipLaunchKernelGGL(k1_logits, dim3(a.E, a.B), dim3(64), 0, st, a);
    }
    return (int)hipGetLastError();
}

constexpr int K2_MAXCAND = 16;  // top-k candidates per lane: E <= 1024

// top-k of one token's logits by one wave; ties go to the lower expert index.
// The ids (and token 0's weights) also go to LDS when s_ids / s_w0 are given.
__device__ void wave_topk(const K2Args& a, int b, int32_t* s_ids = nullptr, float* s_w0 = nullptr) {
    const int lane = threadIdx.x & 63;
    const float* z = a.z + (size_t)b * a.E;
    uint64_t key[K2_MAXCAND];
#pragma unroll
    for (int c = 0; c < K2_MAXCAND; ++c) {
        int ee = lane + 64 * c;
        key[c] = ee < a.E ? topk_key(z[ee], ee) : 0ull;
    }
    int my_id = 0;
    uint64_t my_key = 0;
    for (int j = 0; j < a.k; ++j) {
        uint64_t best = 0;
        int bc = -1;
#pragma unroll
        for (int c = 0; c < K2_MAXCAND; ++c)
            if (key[c] > best) {
                best = key[c];
                bc = c;
            }
        uint64_t wbest = wave_max_u64(best);
        if (bc >= 0 && best == wbest) {
#pragma unroll
            for (int c = 0; c < K2_MAXCAND; ++c)
                if (c == bc) key[c] = 0;
        }
        int id = (int)(0xFFFFFFFFu - (uint32_t)(wbest & 0xFFFFFFFFu));
        if (lane == j) {
            my_id = id;
            my_key = wbest;
        }
    }
    // softmax over the k selected logits (FP32); lane j holds rank j
    float zj = lane < a.k ? topk_key_logit(my_key) : 0.0f;
    float z0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zj), 0));
    float ej = lane < a.k ? expf(zj - z0) : 0.0f;
    float den = 0.0f;
    for (int j = 0; j < a.k; ++j) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ej), j));
    if (lane < a.k) {
        float wj = ej / den;
        size_t o = (size_t)b * a.k + lane;
        a.ids[o] = my_id;
        a.w[o] = wj;
        if (a.ids_out) a.ids_out[o] = my_id;
        if (a.w_out) a.w_out[o] = wj;
        if (s_ids) s_ids[o] = my_id;
        if (s_w0 && b == 0) s_w0[lane] = wj;
    }
}

// ------------------------------------------------------------------- K2 --

constexpr int K2_THREADS = 1024;
constexpr int K2_MAXE = 1024;
constexpr int K2_MAXC = 32768;               // cache slots the resolve kernels address
constexpr int K2_IDS_LDS = 1024;              // ids of a step kept in LDS up to this many

// exclusive prefix count of a 0/1 flag over the 1024 threads, in thread order
__device__ __forceinline__ int block_rank(bool flag, int* s_wave, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t m = __ballot(flag);
    int r = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < K2_THREADS / 64; ++w) {
        int c = s_wave[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + r;
}

// exclusive prefix sum of a small count over the 1024 threads, in thread order
__device__ __forceinline__ int block_scan(int v, int* s_wave, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < K2_THREADS / 64; ++w) {
        int c = s_wave[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

// CPT: order entries per thread (C <= 1024 CPT); compiled for 16 and 32
template <int CPT>
__global__ __launch_bounds__(K2_THREADS) void k2_resolve(K2Args a, const int32_t* order_in,
                                                         int32_t* order_out) {
    __shared__ int32_t s_req[K2_MAXE];     // requested flag, then final slot per expert
    __shared__ int32_t s_miss_e[K2_MAXE];  // misses by rank
    __shared__ int32_t s_victim[K2_MAXE];  // victims by rank
    __shared__ uint32_t s_hitbits[CPT * K2_THREADS / 32];
    __shared__ int s_wave[K2_THREADS / 64];
    __shared__ int s_evict, s_invalid;
    __shared__ int32_t s_ids[K2_IDS_LDS];
    __shared__ float s_w0[16];
    const int tid = threadIdx.x;
    const int E = a.E, C = a.C, l = a.layer;
    const bool stat = a.policy != 0;
    const bool ids_lds = a.n_ids <= K2_IDS_LDS;

    // Loads that do not depend on this step's routing are issued first, so their
    // latency overlaps the logits loads of the top-k: the slot-table entry of
    // expert e = tid, this thread's slice of the victim order, the clock and the
    // trace head.
    const int e = tid;
    const int v_pre = (!stat && e < E) ? a.c.slot_of[l * E + e] : -1;
    int ent[CPT];
    const int p0 = tid * CPT;
#pragma unroll
    for (int c = 0; c < CPT; ++c) ent[c] = (!stat && p0 + c < C) ? order_in[p0 + c] : -1;
    const int64_t clock0 = *a.c.clock;
    const int64_t trace_base = (int64_t)a.c.trace_head[0];

    // routing: top-k + softmax of every token (one wave per token); otherwise the
    // given ids, into LDS when they fit
    if (a.z) {
        for (int b = tid >> 6; b < a.B; b += K2_THREADS / 64)
            wave_topk(a, b, ids_lds ? s_ids : nullptr, s_w0);
    } else if (ids_lds) {
        for (int i = tid; i < a.n_ids; i += K2_THREADS) s_ids[i] = a.ids[i];
    }

    for (int i = tid; i < E; i += K2_THREADS) s_req[i] = 0;
    for (int i = tid; i < (C + 31) / 32; i += K2_THREADS) s_hitbits[i] = 0u;
    if (tid == 0) { s_evict = 0; s_invalid = 0; }
    __syncthreads();
    for (int i = tid; i < a.n_ids; i += K2_THREADS) {
        const int id = ids_lds ? s_ids[i] : a.ids[i];
        if ((unsigned)id < (unsigned)E) s_req[id] = 1;
        else atomicAdd(&s_invalid, 1);
    }
    __syncthreads();
    if (s_invalid != 0) {
        // Ids outside [0, E): the step is rejected as a whole and leaves the cache as it was.
        // Only the count is published (no entries); the victim order is carried over unchanged
        // into the other order buffer (the next step reads that one); slot table, reverse map,
        // stamps, clock, counters and trace are not touched; every slot output is -1.
        if (!stat) {
#pragma unroll
            for (int c = 0; c < CPT; ++c)
                if (p0 + c < C) order_out[p0 + c] = ent[c];
        }
        for (int i = tid; i < a.n_ids; i += K2_THREADS) {
            a.slots[i] = -1;
            if (a.slots_out) a.slots_out[i] = -1;
        }
        if (tid < 64) {
            if (tid == 0) {
                a.ml->n_miss = 0;
                a.ml->n_xfer = 0;
                a.ml->n_unique = 0;
                a.ml->n_evict = 0;
                a.ml->n_invalid = s_invalid;
            }
            __threadfence_system();
            if (tid == 0) __hip_atomic_store(&a.ml->seq, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        return;
    }

    // classify the requested experts (thread e <-> expert e; E <= 1024)
    const bool req = e < E && s_req[e] != 0;
    // static split: resident iff key < R (slot = key); LRU: the slot table
    const int v = req ? (stat ? (l * E + e < a.R ? l * E + e : -1) : v_pre) : -1;
    const bool hit = req && v >= 0;
    const bool miss = req && v < 0;
    int nh, nm;
    const int hr = block_rank(hit, s_wave, nh);
    const int mr = block_rank(miss, s_wave, nm);
    if (hit && !stat) atomicOr(&s_hitbits[v >> 5], 1u << (v & 31));
    if (miss) s_miss_e[mr] = e;
    __syncthreads();
    // hybrid split (LRU, routed batches of at most 16 tokens): the first q misses
    // (ascending expert id) are transferred, q = m B_P / B_H to the nearest
    // integer (halves up); the rest are computed by the host and take no slot
    int q = nm;
    if (!stat && a.hybrid && nm > 0 && a.bh > a.bp && a.bp > 0.0) {
        q = (int)floor((double)nm * a.bp / a.bh + 0.5);
        q = q < 0 ? 0 : (q > nm ? nm : q);
    }

    // victims, by miss rank
    if (stat) {
        // static split: misses stream into the next transient slots in rotation
        if (tid < nm) s_victim[tid] = a.R + (int)((clock0 + tid) % a.T);
    } else {
        // stable compaction of the victim order: non-hit slots keep their order;
        // the first q of them are this step's victims
        int kept = 0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int sl = ent[c];
            if (sl >= 0) {
                const bool is_hit = (s_hitbits[sl >> 5] >> (sl & 31)) & 1u;
                ent[c] = is_hit ? -1 : sl;
                kept += is_hit ? 0 : 1;
            }
        }
        int nkept;
        int kr = block_scan(kept, s_wave, nkept);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            if (ent[c] < 0) continue;
            if (kr < q) s_victim[kr] = ent[c];
            else order_out[kr - q] = ent[c];
            ++kr;
        }
    }
    __syncthreads();
    // final slot of every requested expert (-1: computed by the host)
    if (hit) s_req[e] = v;
    if (tid < nm) s_req[s_miss_e[tid]] = tid < q ? s_victim[tid] : -1;
    __syncthreads();

    // The miss list goes to host memory as soon as it is known, from wave 0
    // alone (entries, token 0's slots and weights, which the host passes to the
    // FFN launch as arguments), so one system-scope fence orders all of it
    // before the sequence number that publishes it.  The cache bookkeeping
    // below runs while the host issues the copies.
    if (tid < 64) {
        for (int i = tid; i < nm; i += 64) {
            a.ml->e[i].expert = s_miss_e[i];
            a.ml->e[i].slot = i < q ? s_victim[i] : -1;
        }
        if (tid < a.k && tid < 16) {
            const int id = ids_lds ? s_ids[tid] : a.ids[tid];
            a.ml->slot0[tid] = (unsigned)id < (unsigned)E ? s_req[id] : -1;
            a.ml->w0[tid] = a.z ? s_w0[tid] : 0.0f;
            a.ml->ids0[tid] = id;
        }
        if (q < nm) {
            // every token's experts and weights, for the host's share of a batch
            for (int i = tid; i < a.n_ids && i < HYB_MAX_IDS; i += 64) {
                a.ml->ids_all[i] = ids_lds ? s_ids[i] : a.ids[i];
                a.ml->w_all[i] = a.w[i];
            }
        }
        if (tid == 0) {
            a.ml->n_miss = nm;
            a.ml->n_xfer = q;
            a.ml->n_unique = nh + nm;
            a.ml->n_invalid = s_invalid;
        }
        __threadfence_system();
        if (tid == 0) __hip_atomic_store(&a.ml->seq, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }

    // bookkeeping: stamps, slot table, reverse map, recency order, trace
    if (hit) {
        if (!stat) {
            a.c.stamp[v] = clock0 + hr;
            order_out[C - nh - q + hr] = v;
        }
        const int64_t ti = trace_base + hr;
        if (ti < a.c.trace_cap) {
            TraceRec t = {a.step, l, e, v, 1, -1};
            a.c.trace[ti] = t;
        }
    }
    if (tid >= q && tid < nm) {
        // computed by the host: no slot, the cache unchanged
        const int64_t ti = trace_base + nh + tid;
        if (ti < a.c.trace_cap) {
            TraceRec t = {a.step, l, s_miss_e[tid], -1, 0, -1};
            a.c.trace[ti] = t;
        }
    }
    if (tid < q) {
        const int me = s_miss_e[tid];
        const int vv = s_victim[tid];
        const int old = a.c.key_of[vv];  // the static split's transient slots keep their last occupant
        if (old >= 0) {
            if (!stat) a.c.slot_of[old] = -1;
            atomicAdd(&s_evict, 1);
        }
        a.c.key_of[vv] = l * E + me;
        if (!stat) {
            a.c.slot_of[l * E + me] = vv;
            a.c.stamp[vv] = clock0 + nh + tid;
            order_out[C - q + tid] = vv;
        }
        const int64_t ti = trace_base + nh + tid;
        if (ti < a.c.trace_cap) {
            TraceRec t = {a.step, l, me, vv, 0, old};
            a.c.trace[ti] = t;
        }
    }
    for (int i = tid; i < a.n_ids; i += K2_THREADS) {
        const int id = ids_lds ? s_ids[i] : a.ids[i];
        int sl = (unsigned)id < (unsigned)E ? s_req[id] : -1;
        a.slots[i] = sl;
        if (a.slots_out) a.slots_out[i] = sl;
    }
    __syncthreads();
    if (tid == 0) {
        const int n = nh + nm;
        *a.c.clock = clock0 + (stat ? nm : nh + q);  // static: transient slots used so far
        a.c.counters[0] += (uint64_t)nh;
        a.c.counters[1] += (uint64_t)nm;
        a.c.counters[2] += (uint64_t)s_evict;
        a.c.counters[3] += 1ull;
        a.c.counters[4] += (uint64_t)(nm - q);
        int64_t fit = a.c.trace_cap - trace_base;
        fit = fit < 0 ? 0 : (fit > n ? n : fit);
        a.c.trace_head[0] = (uint64_t)(trace_base + fit);
        a.c.trace_head[1] += (uint64_t)(n - fit);
        a.ml->n_evict = s_evict;  // informational; written after the release
    }
}

// ------------------------------------------------------------ K2, one token --
// Decode (one routed token, LRU policy).  Wave 0 routes and resolves the token
// with wave-level operations and publishes the miss list before any block
// barrier; the other waves hold their slice of the LRU order in registers and,
// after two barriers, compact it.  The k selected experts are distinct, so at
// most k order entries are hit slots and the nm victims (the first nm non-hit
// entries) are among the first k entries of the order.

__device__ __forceinline__ int lane_i32(int v, int j) { return __builtin_amdgcn_readlane(v, j); }
__device__ __forceinline__ float lane_f32(float v, int j) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

constexpr int K2T_WAVES = 16;
static_assert(K2T_WAVES * 64 * 32 == K2_MAXC && 32 * K2_THREADS == K2_MAXC,
              "the largest resolve specialisations address K2_MAXC slots");

// NC: logit candidates per lane (E <= 64 NC); NI: order entries per lane (C <= 16 * 64 NI)
template <int NC, int NI>
__global__ __launch_bounds__(K2T_WAVES * 64) void k2_resolve_tok(K2Args a, const int32_t* order_in,
                                                                 int32_t* order_out) {
    __shared__ int32_t s_slot[64 * NC];          // this layer's slot-table entries
    __shared__ uint32_t s_hbits[K2T_WAVES * 64 * NI / 32];   // hit slots
    __shared__ int32_t s_vict[16], s_vkey[16];   // victims and their occupants, by miss rank
    __shared__ int s_cnt[K2T_WAVES];
    __shared__ uint64_t s_vmask;                 // order positions (< k) taken as victims
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int E = a.E, C = a.C, l = a.layer, k = a.k;

    // every wave: its slice of the LRU order
    int ent[NI];
    const int pw = wv * 64 * NI + lane;
#pragma unroll
    for (int i = 0; i < NI; ++i) ent[i] = pw + 64 * i < C ? order_in[pw + 64 * i] : -1;

    if (wv == 0) {
        // loads that do not depend on the routing first
        float zc[NC];
        int so[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = lane + 64 * c;
            zc[c] = e < E ? a.z[e] : 0.0f;
            so[c] = e < E ? a.c.slot_of[l * E + e] : -1;
        }
        const int oj = lane < k ? order_in[lane] : -1;
        const int64_t clock0 = *a.c.clock;
        const int64_t trace_base = (int64_t)a.c.trace_head[0];
        for (int i = lane; i < (C + 31) / 32; i += 64) s_hbits[i] = 0u;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (lane + 64 * c < E) s_slot[lane + 64 * c] = so[c];
        const int okey = oj >= 0 ? a.c.key_of[oj] : -1;

        // top-k on (logit desc, expert asc); lane j < k ends with rank j
        uint64_t key[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = lane + 64 * c;
            key[c] = e < E ? topk_key(zc[c], e) : 0ull;
        }
        int my_id = 0;
        uint64_t my_key = 0;
        for (int j = 0; j < k; ++j) {
            uint64_t best = 0;
            int bc = -1;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                if (key[c] > best) {
                    best = key[c];
                    bc = c;
                }
            const uint64_t wbest = wave_max_u64(best);
            if (bc >= 0 && best == wbest) {
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    if (c == bc) key[c] = 0;
            }
            if (lane == j) {
                my_id = (int)(0xFFFFFFFFu - (uint32_t)(wbest & 0xFFFFFFFFu));
                my_key = wbest;
            }
        }
        // softmax over the k selected logits, summed in rank order
        const bool sel = lane < k;
        const float zj = sel ? topk_key_logit(my_key) : 0.0f;
        const float z0 = lane_f32(zj, 0);
        const float ej = sel ? expf(zj - z0) : 0.0f;
        float den = 0.0f;
        for (int j = 0; j < k; ++j) den += lane_f32(ej, j);
        const float wj = ej / den;

        // hits and misses; ranks by ascending expert id within each
        __builtin_amdgcn_wave_barrier();
        const int vj = sel ? s_slot[my_id] : -1;
        const bool hit = sel && vj >= 0, miss = sel && vj < 0;
        const uint64_t hm = __ballot(hit), mm = __ballot(miss);
        const int nh = __popcll(hm), nm = __popcll(mm);
        // hybrid split: the first q misses (ascending expert id) are transferred,
        // q = m B_P / B_H to the nearest integer (halves up); all of them when the
        // host has no bandwidth to spare
        int q = nm;
        if (a.hybrid && nm > 0 && a.bh > a.bp && a.bp > 0.0) {
            q = (int)floor((double)nm * a.bp / a.bh + 0.5);
            q = q < 0 ? 0 : (q > nm ? nm : q);
        }
        int hr = 0, mr = 0;
        bool ohit = false;  // order entry oj is a hit slot
        for (int i = 0; i < k; ++i) {
            const bool lower = lane_i32(my_id, i) < my_id;
            hr += (((hm >> i) & 1ull) && lower) ? 1 : 0;
            mr += (((mm >> i) & 1ull) && lower) ? 1 : 0;
            ohit |= ((hm >> i) & 1ull) && lane_i32(vj, i) == oj;
        }
        if (hit) atomicOr(&s_hbits[vj >> 5], 1u << (vj & 31));
        // victims: the first q order entries that are not hit slots
        const bool keep = lane < k && !ohit;
        const int kr = __popcll(__ballot(keep) & ((1ull << lane) - 1ull));
        const bool victim = keep && kr < q;
        const uint64_t vmask = __ballot(victim);
        if (victim) {
            s_vict[kr] = oj;
            s_vkey[kr] = okey;
        }
        __builtin_amdgcn_wave_barrier();
        const bool xfer = miss && mr < q;  // the other misses are computed by the host
        const int slot = hit ? vj : (xfer ? s_vict[mr] : -1);
        const int old = xfer ? s_vkey[mr] : -1;

        // publish the miss list: one system-scope fence, then the sequence number
        if (miss) {
            a.ml->e[mr].expert = my_id;
            a.ml->e[mr].slot = slot;
        }
        if (sel) {
            a.ml->slot0[lane] = slot;
            a.ml->w0[lane] = wj;
            a.ml->ids0[lane] = my_id;
        }
        if (lane == 0) {
            a.ml->n_miss = nm;
            a.ml->n_xfer = q;
            a.ml->n_unique = nh + nm;
            a.ml->n_invalid = 0;
        }
        __threadfence_system();
        if (lane == 0) __hip_atomic_store(&a.ml->seq, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);

        // bookkeeping
        const int n_evict = __popcll(__ballot(xfer && old >= 0));
        if (sel) {
            a.ids[lane] = my_id;
            a.w[lane] = wj;
            if (a.ids_out) a.ids_out[lane] = my_id;
            if (a.w_out) a.w_out[lane] = wj;
            a.slots[lane] = slot;
            if (a.slots_out) a.slots_out[lane] = slot;
            const int rank = hit ? hr : nh + mr;
            if (hit || xfer) {
                a.c.stamp[slot] = clock0 + rank;
                order_out[C - nh - q + rank] = slot;  // hits by hit rank, then transfers by miss rank
            }
            const int64_t ti = trace_base + rank;
            if (ti < a.c.trace_cap) {
                TraceRec t = {a.step, l, my_id, slot, hit ? 1 : 0, xfer ? old : -1};
                a.c.trace[ti] = t;
            }
        }
        if (xfer) {
            if (old >= 0) a.c.slot_of[old] = -1;
            a.c.key_of[slot] = l * E + my_id;
            a.c.slot_of[l * E + my_id] = slot;
        }
        if (lane == 0) {
            const int n = nh + nm;
            *a.c.clock = clock0 + nh + q;
            a.c.counters[0] += (uint64_t)nh;
            a.c.counters[1] += (uint64_t)nm;
            a.c.counters[2] += (uint64_t)n_evict;
            a.c.counters[3] += 1ull;
            a.c.counters[4] += (uint64_t)(nm - q);
            int64_t fit = a.c.trace_cap - trace_base;
            fit = fit < 0 ? 0 : (fit > n ? n : fit);
            a.c.trace_head[0] = (uint64_t)(trace_base + fit);
            a.c.trace_head[1] += (uint64_t)(n - fit);
            a.ml->n_evict = n_evict;
            s_vmask = vmask;
        }
    }
    __syncthreads();

    // order compaction: entries that are neither hit slots nor victims keep their order
    const uint64_t vm = s_vmask;
    uint64_t km[NI];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int p = pw + 64 * i, sl = ent[i], slc = sl < 0 ? 0 : sl;
        const bool hbit = (s_hbits[slc >> 5] >> (slc & 31)) & 1u;
        const bool rm = sl < 0 || hbit || (p < 64 && ((vm >> p) & 1ull));
        km[i] = __ballot(!rm);
        cnt += __popcll(km[i]);
    }
    if (lane == 0) s_cnt[wv] = cnt;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wv; ++w) base += s_cnt[w];
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if ((km[i] >> lane) & 1ull) order_out[base + __popcll(km[i] & below)] = ent[i];
        base += __popcll(km[i]);
    }
}

template <int NC>
void launch_k2_tok(const K2Args& a, const int32_t* order_in, int32_t* order_out, hipStream_t st) {
    const dim3 g(1), b(K2T_WAVES * 64);
    const int per_wave = (a.C + K2T_WAVES - 1) / K2T_WAVES;
    if (per_wave <= 64 * 2)
        hipLaunchKernelGGL((k2_resolve_tok<NC, 2>), g, b, 0, st, a, order_in, order_out);
    else if (per_wave <= 64 * 4)
        hipLaunchKernelGGL((k2_resolve_tok<NC, 4>), g, b, 0, st, a, order_in, order_out);
    else if (per_wave <= 64 * 8)
        hipLaunchKernelGGL((k2_resolve_tok<NC, 8>), g, b, 0, st, a, order_in, order_out);
    else if (per_wave <= 64 * 16)
        hipLaunchKernelGGL((k2_resolve_tok<NC, 16>), g, b, 0, st, a, order_in, order_out);
    else
        hipLaunchKernelGGL((k2_resolve_tok<NC, 32>), g, b, 0, st, a, order_in, order_out);
}

// top-k + softmax of many tokens, one wave per token, ahead of the resolve
// kernel (whose single workgroup would otherwise take them 16 at a time)
__global__ __launch_bounds__(256) void k2_topk(K2Args a) {
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b < a.B) wave_topk(a, b);
}

constexpr int K2_FUSED_TOPK_MAX = 16;  // up to this many tokens the resolve kernel routes them itself

// the general resolve, compiled for the cache size
void launch_k2_general(const K2Args& a, const int32_t* order_in, int32_t* order_out, hipStream_t st) {
    if (a.C <= 16 * K2_THREADS)
        hipLaunchKernelGGL(k2_resolve<16>, dim3(1), dim3(K2_THREADS), 0, st, a, order_in, order_out);
    else
        hipLaunchKernelGGL(k2_resolve<32>, dim3(1), dim3(K2_THREADS), 0, st, a, order_in, order_out);
}

int launch_k2(const K2Args& a, const int32_t* order_in, int32_t* order_out, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (a.z && a.B > K2_FUSED_TOPK_MAX) {
        hipLaunchKernelGGL(k2_topk, dim3((a.B + 3) / 4), dim3(256), 0, st, a);
        K2Args r = a;
        r.z = nullptr;  // resolve the ids just written
        launch_k2_general(r, order_in, order_out, st);
    } else if (a.z && a.B == 1 && a.n_ids == a.k && a.policy == 0) {
        // one routed token: the wave-level resolve
        if (a.E <= 128)
            launch_k2_tok<2>(a, order_in, order_out, st);
        else if (a.E <= 256)
            launch_k2_tok<4>(a, order_in, order_out, st);
        else if (a.E <= 512)
            launch_k2_tok<8>(a, order_in, order_out, st);
        else
            launch_k2_tok<16>(a, order_in, order_out, st);
    } else {
        launch_k2_general(a, order_in, order_out, st);
    }
    return (int)hipGetLastError();
}

}  // namespace moe
