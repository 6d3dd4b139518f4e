// The expert FFN of one MoE layer for a few tokens in one launch: gate/up +
// SwiGLU (phase 1) and down + weighted combine + shared expert (phase 2),
// streaming MXFP4 weights from HBM (the slot arena and the resident shared
// experts).
//
// The FFN form is not stated on the pages; the reading used here is the
// SwiGLU expert of the MoE models they discuss: a = silu(W_gate x) * (W_up x),
// y = W_down a, no biases.  Weights are MXFP4 (ai-hardware-zukan.com FreeToken
// vs Ollama page, host-memory table: gpt-oss and DeepSeek-V4-Flash routed
// experts are MXFP4; blog.florigen.ai Qwen3.8-Flash-Next page, NVFP4 section:
// E2M1 elements with block scaling).  The layer output is sum_j w_j y_j over
// the selected experts plus the shared expert with weight 1 (blog.florigen.ai
// page, model section: one shared expert used by every token).
//
// At a handful of tokens this is a GEMV: about 3.8 flop per weight byte, far
// under the MFMA ridge, so it is bound by HBM bandwidth.  The kernels stream
// 16-byte code chunks (exactly one 32-element MX block) per lane, convert
// E2M1 pairs to bf16 with the gfx950 scaled-convert instruction (scale 1.0, so
// the values are exact), accumulate each block with bf16 dot2 into FP32, and
// apply the block's E8M0 scale (a power of two) once per block.  Activations
// are staged in LDS in (step, segment) order with an 80-byte stride so the
// distinct addresses a wave reads in one instruction fall in distinct banks.
// Reductions across lanes and waves run in a fixed order, so results are
// bitwise reproducible from run to run.
//
// Two launches per layer: K3 (gate/up + SwiGLU -> intermediate vector `a`)
// and K4 (down + weighted combine + shared expert).  K4 needs all of `a` (the
// down projection reduces over all of I for every expert), and handing it
// over inside one launch (device-coherent stores, a wait for their
// completion, and an arrival counter) costs several microseconds per
// workgroup on this chip, more than the kernel boundary.  For a single token
// the expert slots and routing weights arrive as launch arguments, so neither
// kernel starts with a dependent load.
#include <hip/hip_runtime.h>

#include "ffn_device.h"
#include "moe_internal.h"

namespace moe {

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) dotted with
// 8 bf16 activations (4 dwords, element 2i in the low half of dword i)
__device__ __forceinline__ float dot8(uint32_t cw, uint4 xv, float s) {
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 0),
                                        as_bf16x2(xv.x), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 1),
                                        as_bf16x2(xv.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 2),
                                        as_bf16x2(xv.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 3),
                                        as_bf16x2(xv.w), s, false);
    return s;
}

// one MX block: 32 codes (16 bytes) against 32 activations (64 bytes in LDS)
__device__ __forceinline__ float dot32(uint4 c, const uint4* xb) {
    float s = 0.0f;
    s = dot8(c.x, xb[0], s);
    s = dot8(c.y, xb[1], s);
    s = dot8(c.z, xb[2], s);
    s = dot8(c.w, xb[3], s);
    return s;
}

// LDS position (in uint4 units, 5 per 64-byte block) of block `blk` of a row
// split into S segments: segment and step of the block, stored step-major.
__device__ __forceinline__ int lds_pos(int blk, int n, int S) {
    const int q = n / S, rem = n % S;
    int s, t;
    if (blk < rem * (q + 1)) {
        s = blk / (q + 1);
        t = blk - s * (q + 1);
    } else {
        const int bb = blk - rem * (q + 1);
        s = rem + bb / q;
        t = bb - (s - rem) * q;
    }
    return (t * S + s) * 5;
}

// slot / weight of the single token's j-th expert from the launch arguments:
// a select chain over wave-uniform copies of the 16 entries.  Indexing the
// by-value argument array with a variable, or a select chain on the entries
// themselves (which the compiler folds into one), becomes a per-lane load
// from the argument block whose latency precedes the first weight load.
__device__ __forceinline__ int karg_slot(const FfnArgs& a, int j) {
    int v = __builtin_amdgcn_readfirstlane(a.kslot[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) v = (j == i) ? __builtin_amdgcn_readfirstlane(a.kslot[i]) : v;
    return v;
}
__device__ __forceinline__ float karg_w(const FfnArgs& a, int j) {
    float v = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.kw[0])));
#pragma unroll
    for (int i = 1; i < 16; ++i)
        v = (j == i) ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.kw[i]))) : v;
    return v;
}

// slot of the token's j-th routed expert (j < k)
__device__ __forceinline__ int expert_slot(const FfnArgs& a, int b, int j) {
    return a.karg ? karg_slot(a, j) : a.slots[b * a.k + j];
}

// blob of the token's j-th expert (j >= k: the shared expert).  A slot outside [0, C) is never
// dereferenced: slot 0 is read instead and the expert's weight is NaN (expert_weight), so every
// output of the token is NaN.
__device__ __forceinline__ const uint8_t* expert_blob(const FfnArgs& a, int b, int j) {
    if (j < a.k) {
        const int slot = expert_slot(a, b, j);
        return a.arena + (size_t)((unsigned)slot < (unsigned)a.C ? slot : 0) * a.blob_bytes;
    }
    return a.shared + (size_t)(a.layer * a.n_shared + (j - a.k)) * a.blob_bytes;
}

__device__ __forceinline__ float expert_weight(const FfnArgs& a, int b, int j) {
    if (j >= a.k) return 1.0f;
    const float w = a.karg ? karg_w(a, j) : a.w[b * a.k + j];
    return (unsigned)expert_slot(a, b, j) < (unsigned)a.C ? w : __uint_as_float(0x7FC00000u);
}

// Blob and combine weight of the token's experts j0 and j1 for one down-kernel lane (per-lane j:
// the lane's segment may start in one expert and end in the next).  Same values as expert_blob and
// expert_weight; from device memory the two slots and two weights are four independent loads
// issued together (one memory latency before the weight loads, instead of one per value).
struct LaneExperts {
    const uint8_t* blob0;
    const uint8_t* blob1;
    float w0, w1;
};

__device__ __forceinline__ LaneExperts lane_experts(const FfnArgs& a, int b, int j0, int j1) {
    int s0, s1;
    float w0, w1;
    if (a.karg) {
        s0 = karg_slot(a, j0);
        s1 = karg_slot(a, j1);
        w0 = karg_w(a, j0);
        w1 = karg_w(a, j1);
    } else {
        const int32_t* sp = a.slots + b * a.k;
        const float* wp = a.w + b * a.k;
        const int i0 = j0 < a.k ? j0 : 0, i1 = j1 < a.k ? j1 : 0;
        s0 = sp[i0];
        s1 = sp[i1];
        w0 = wp[i0];
        w1 = wp[i1];
    }
    auto blob = [&](int j, int sl) {
        if (j < a.k) return a.arena + (size_t)((unsigned)sl < (unsigned)a.C ? sl : 0) * a.blob_bytes;
        return a.shared + (size_t)(a.layer * a.n_shared + (j - a.k)) * a.blob_bytes;
    };
    auto weight = [&](int j, int sl, float w) {
        if (j >= a.k) return 1.0f;
        return (unsigned)sl < (unsigned)a.C ? w : __uint_as_float(0x7FC00000u);
    };
    return LaneExperts{blob(j0, s0), blob(j1, s1), weight(j0, s0, w0), weight(j1, s1, w1)};
}

constexpr int FFN_THREADS = 256;

// v + (v of lane ^ 8), then ^ 16, then ^ 32: the sum of a row's segments held by lanes r + 8i.
// Partners come from DPP (rotate a row of 16 by 8) and the gfx950 lane swaps instead of LDS
// round trips; each step adds the same two values as a shuffle would (in either order, which
// gives the same bits).
__device__ __forceinline__ float sum_lanes_8_16_32(float v) {
    v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

// Activations are staged into LDS in lds_pos() order, one 64-byte block (32
// bf16 values) per thread and step, in two halves around the weight loads:
// stage_first() loads a thread's first block into registers; the caller then
// issues its weight loads; stage_commit() writes the block to LDS, which waits
// for the staging loads alone (loads complete in order per wave), and stages
// any further blocks (shapes with more blocks than threads).  The activations'
// latency and the weights' then overlap; a scheduling barrier on each side of
// the weight loads keeps the compiler from moving the staging loads behind them.
struct StageRegs {
    uint4 v0, v1, v2, v3;
};

__device__ __forceinline__ StageRegs stage_first(const uint4* src, int nblk) {
    const int bc = (int)threadIdx.x < nblk ? (int)threadIdx.x : 0;
    return StageRegs{src[bc * 4 + 0], src[bc * 4 + 1], src[bc * 4 + 2], src[bc * 4 + 3]};
}

__device__ __forceinline__ void stage_commit(const StageRegs& r, uint4* smem, const uint4* src, int nblk, int nseg,
                                             int nthreads) {
    if ((int)threadIdx.x < nblk) {
        uint4* d = smem + lds_pos(threadIdx.x, nblk, nseg);
        d[0] = r.v0;
        d[1] = r.v1;
        d[2] = r.v2;
        d[3] = r.v3;
    }
    for (int blk = threadIdx.x + nthreads; blk < nblk; blk += nthreads) {
        const uint4 v0 = src[blk * 4 + 0];
        const uint4 v1 = src[blk * 4 + 1];
        const uint4 v2 = src[blk * 4 + 2];
        const uint4 v3 = src[blk * 4 + 3];
        uint4* d = smem + lds_pos(blk, nblk, nseg);
        d[0] = v0;
        d[1] = v1;
        d[2] = v2;
        d[3] = v3;
    }
}

// ---------------------------------------------------------------- phase 1 --
// one 8-row tile of one expert: compute lane (r = lane&7, s = 8*wave + lane>>3);
// the 32 segments of a row are spread over the 4 waves
template <int T1>
__device__ __forceinline__ void ffn_gate_up(const FfnArgs& a, uint4* smem, int unit, int b) {
    constexpr int S = kGuSegments, GR = kGuRows;
    const int tiles = a.I / GR;
    const int j = __builtin_amdgcn_readfirstlane(unit / tiles), tile = unit - j * tiles;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int NB = a.NB;
    float* red = reinterpret_cast<float*>(smem + NB * 5);
    const int r = lane & 7, s = w * 8 + (lane >> 3);
    const int nb = seg_len(NB, S, s);
    // The activations' staging loads go out first: they do not depend on the expert's slot, whose
    // scalar load (from device memory when the caller passed the slots there) overlaps them.
    const uint4* xsrc = reinterpret_cast<const uint4*>(a.x + (size_t)b * a.H);
    const StageRegs xr = stage_first(xsrc, NB);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* blob = expert_blob(a, b, j);
    const uint8_t* tb = blob + (size_t)tile * GR * NB * 34;
    const uint8_t* tub = tb + (size_t)GR * NB * 16;
    const uint8_t* tsc = tb + (size_t)GR * NB * 32;

    float g = 0.0f, u = 0.0f;
    uint4 gc[T1], uc[T1];
    uint32_t sc[T1];
    // Steps past this lane's segment re-read its step-0 chunk (a cache hit) and
    // are dropped by a select, so loads and compute are branch-free and the
    // compiler can wait for each step's data separately; an empty segment
    // (NB < 32) reads the tile's first chunk.
    const int sv = nb > 0 ? s : 0;
    auto load = [&](int t0) {
#pragma unroll
        for (int t = 0; t < T1; ++t) {
            const int tt = (t0 + t < nb) ? t0 + t : 0;
            const size_t c = (size_t)(tt * S + sv) * GR + r;
            gc[t] = ldg16(tb + c * 16);
            uc[t] = ldg16(tub + c * 16);
            sc[t] = *reinterpret_cast<const uint16_t*>(tsc + c * 2);
        }
    };
    auto compute = [&](int t0) {
#pragma unroll
        for (int t = 0; t < T1; ++t) {
            const int tt = (t0 + t < nb) ? t0 + t : 0;
            const uint4* xb = smem + (tt * S + sv) * 5;
            const float pg = e8m0(sc[t]) * dot32(gc[t], xb);
            const float pu = e8m0(sc[t] >> 8) * dot32(uc[t], xb);
            g += (t0 + t < nb) ? pg : 0.0f;
            u += (t0 + t < nb) ? pu : 0.0f;
        }
    };
    load(0);
    __builtin_amdgcn_sched_barrier(0);
    stage_commit(xr, smem, xsrc, NB, S, FFN_THREADS);
    __syncthreads();
    compute(0);
    for (int t0 = T1; t0 < nb; t0 += T1) {
        load(t0);
        compute(t0);
    }
    // segments of a row: lanes r + 8i of every compute wave
    g = sum_lanes_8_16_32(g);
    u = sum_lanes_8_16_32(u);
    if (lane < GR) {
        red[(w * GR + r) * 2] = g;
        red[(w * GR + r) * 2 + 1] = u;
    }
    __syncthreads();
    if (tid < GR) {
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            gs += red[(ww * GR + tid) * 2];
            us += red[(ww * GR + tid) * 2 + 1];
        }
        const float act = swiglu(gs, us);
        a.a[((size_t)b * a.nE + j) * a.I + tile * GR + tid] = f32_to_bf16(act);
    }
}

// ---------------------------------------------------------------- phase 2 --
// One 8-row tile of the output per workgroup of K4_WAVES waves, all sharing one
// LDS copy of the token's activations.  Compute lane (r = lane&7, s = 8*wave +
// lane>>3); the 64 segments split the combined (expert, I-block) range of the
// token, so each lane takes about nE*NBI/64 blocks.
constexpr int K4_WAVES = 8;

template <int T2>
__device__ __forceinline__ void ffn_down(const FfnArgs& a, uint4* smem, int tile, int b) {
    constexpr int S = 8 * K4_WAVES;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int NBI = a.NBI, nE = a.nE;
    const int Q = nE * NBI;
    float* red = reinterpret_cast<float*>(smem + Q * 5);
    const int r = lane & 7, s = w * 8 + (lane >> 3);
    const int nq = seg_len(Q, S, s), q0 = seg_begin(Q, S, s);
    // A segment (at most ceil(nE*NBI/64) <= NBI + 1 blocks, as nE <= 64)
    // spans at most two experts: j0 from block ib0 for `split` steps, then j0+1
    // from block 0.  Steps past the segment re-read step 0 and are dropped; an
    // empty segment (Q < 64) reads block 0 of expert 0.
    const int qv = nq > 0 ? q0 : 0;
    const int j0 = qv / NBI, ib0 = qv - (qv / NBI) * NBI;
    const int split = NBI - ib0;
    const int j1 = j0 + 1 < nE ? j0 + 1 : j0;
    const LaneExperts le = lane_experts(a, b, j0, j1);
    const uint8_t* base0 = le.blob0;
    const uint8_t* base1 = le.blob1;
    const float cw0 = le.w0, cw1 = le.w1;
    const int sv = nq > 0 ? s : 0;
    uint4 dc[T2];
    uint32_t sc[T2];
    auto load = [&](int t0) {
#pragma unroll
        for (int t = 0; t < T2; ++t) {
            const int tt = (t0 + t < nq) ? t0 + t : 0;
            const bool first = tt < split;
            const uint8_t* blob = first ? base0 : base1;
            const size_t cell = ((size_t)tile * NBI + (first ? ib0 + tt : tt - split)) * 8 + r;
            dc[t] = ldg16(blob + a.d_codes_off + cell * 16);
            sc[t] = blob[a.d_scales_off + cell];
        }
    };
    float acc = 0.0f;
    auto compute = [&](int t0) {
#pragma unroll
        for (int t = 0; t < T2; ++t) {
            const int tt = (t0 + t < nq) ? t0 + t : 0;
            const uint4* ab = smem + (tt * S + sv) * 5;
            const float pv = (tt < split ? cw0 : cw1) * e8m0(sc[t]) * dot32(dc[t], ab);
            acc += (t0 + t < nq) ? pv : 0.0f;
        }
    };
    const uint4* asrc = reinterpret_cast<const uint4*>(a.a + (size_t)b * nE * a.I);
    const StageRegs ar = stage_first(asrc, Q);
    __builtin_amdgcn_sched_barrier(0);
    load(0);
    __builtin_amdgcn_sched_barrier(0);
    // the host-computed experts' sum for the row this thread writes (host-mapped memory: a PCIe
    // round trip), issued behind the weights, which it does not hold up, and used at the end
    float yhv = 0.0f;
    if (a.yh && tid < 8) yhv = a.yh[(size_t)b * a.H + tile * 8 + tid];
    stage_commit(ar, smem, asrc, Q, S, 64 * K4_WAVES);
    __syncthreads();
    compute(0);
    for (int t0 = T2; t0 < nq; t0 += T2) {
        load(t0);
        compute(t0);
    }
    // segments of an output row: lanes r + 8i of every compute wave
    acc = sum_lanes_8_16_32(acc);
    if (lane < 8) red[w * 8 + r] = acc;
    __syncthreads();
    if (tid < 8) {
        float ys = 0.0f;
#pragma unroll
        for (int ww = 0; ww < K4_WAVES; ++ww) ys += red[ww * 8 + tid];
        ys += yhv;
        a.y[(size_t)b * a.H + tile * 8 + tid] = f32_to_bf16(ys);
    }
}

// K3: grid (nE * I/8 tiles, B), 256 threads; K4: grid (H/8, B), 512 threads
template <int T1>
__global__ __launch_bounds__(FFN_THREADS) void k3_gate_up(FfnArgs a) {
    extern __shared__ uint4 smem[];
    ffn_gate_up<T1>(a, smem, blockIdx.x, blockIdx.y);
}

constexpr int K4_THREADS = 64 * K4_WAVES;

template <int T2>
__global__ __launch_bounds__(K4_THREADS) void k4_down(FfnArgs a) {
    extern __shared__ uint4 smem[];
    ffn_down<T2>(a, smem, blockIdx.x, blockIdx.y);
}

// a layer step whose experts all ran on the host: y = bf16(yh)
__global__ __launch_bounds__(256) void k_host_only_out(const float* yh, uint16_t* y, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = f32_to_bf16(yh[i]);
}

// Waits, in one lane, until the host-mapped count of finished host tasks `done` reaches `seq`
// (the hybrid backend's host task of the layer whose FFN follows), reading it at most max_polls
// times with a sleep between reads.  At the limit it sets *late and returns: the wave always exits.
__global__ __launch_bounds__(64) void k_wait_host(const uint64_t* done, uint64_t seq, uint32_t max_polls,
                                                  uint32_t* late) {
    if (threadIdx.x != 0) return;
    uint32_t n = 0;
    while (__hip_atomic_load(done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < seq) {
        if (++n >= max_polls) {
            __hip_atomic_store(late, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            return;
        }
        __builtin_amdgcn_s_sleep(64);
    }
}

int launch_wait_host(const uint64_t* done, uint64_t seq, uint32_t max_polls, uint32_t* late, void* stream) {
    hipLaunchKernelGGL(k_wait_host, dim3(1), dim3(64), 0, (hipStream_t)stream, done, seq, max_polls, late);
    return (int)hipGetLastError();
}

size_t ffn_lds_bytes(const Layout& L, int nE) {
    const size_t p1 = (size_t)L.NB * 80 + 4 * kGuRows * 2 * 4;
    const size_t p2 = (size_t)nE * L.NBI * 80 + K4_WAVES * 8 * 4;
    return p1 > p2 ? p1 : p2;
}

int launch_ffn(FfnArgs& a, const Layout& L, int B, void* stream, void* ev_mid) {
    hipStream_t st = (hipStream_t)stream;
    if (a.nE == 0) {
        // no expert on the GPU (hybrid step, no shared expert): the host's sum is the output
        if (!a.yh) return (int)hipErrorInvalidValue;
        const int n = B * L.H;
        if (ev_mid) (void)hipEventRecord((hipEvent_t)ev_mid, st);
        hipLaunchKernelGGL(k_host_only_out, dim3((n + 255) / 256), dim3(256), 0, st, a.yh, a.y, n);
        return (int)hipGetLastError();
    }
    a.P1 = a.nE * (L.I / kGuRows);
    a.P2 = L.H / 8;
    const int T1 = L.T3;
    const int T2 = (a.nE * L.NBI + 8 * K4_WAVES - 1) / (8 * K4_WAVES);
    const size_t lds1 = (size_t)L.NB * 80 + 4 * kGuRows * 2 * 4;
    const size_t lds2 = (size_t)a.nE * L.NBI * 80 + K4_WAVES * 8 * 4;
    dim3 g1(a.P1, B), g2(a.P2, B), blk(FFN_THREADS), blk2(K4_THREADS);
    if (T1 <= 1)
        hipLaunchKernelGGL(k3_gate_up<1>, g1, blk, lds1, st, a);
    else if (T1 <= 2)
        hipLaunchKernelGGL(k3_gate_up<2>, g1, blk, lds1, st, a);
    else if (T1 <= 3)
        hipLaunchKernelGGL(k3_gate_up<3>, g1, blk, lds1, st, a);
    else if (T1 <= 4)
        hipLaunchKernelGGL(k3_gate_up<4>, g1, blk, lds1, st, a);
    else if (T1 <= 6)
        hipLaunchKernelGGL(k3_gate_up<6>, g1, blk, lds1, st, a);
    else
        hipLaunchKernelGGL(k3_gate_up<8>, g1, blk, lds1, st, a);
    if (ev_mid) (void)hipEventRecord((hipEvent_t)ev_mid, st);
    if (T2 <= 1)
        hipLaunchKernelGGL(k4_down<1>, g2, blk2, lds2, st, a);
    else if (T2 <= 2)
        hipLaunchKernelGGL(k4_down<2>, g2, blk2, lds2, st, a);
    else if (T2 <= 3)
        hipLaunchKernelGGL(k4_down<3>, g2, blk2, lds2, st, a);
    else if (T2 <= 4)
        hipLaunchKernelGGL(k4_down<4>, g2, blk2, lds2, st, a);
    else if (T2 <= 6)
        hipLaunchKernelGGL(k4_down<6>, g2, blk2, lds2, st, a);
    else if (T2 <= 8)
        hipLaunchKernelGGL(k4_down<8>, g2, blk2, lds2, st, a);
    else
        hipLaunchKernelGGL(k4_down<12>, g2, blk2, lds2, st, a);
    return (int)hipGetLastError();
}

}  // namespace moe
