// K3 (gate/up + SwiGLU) and K4 (down + weighted combine + shared expert):
// the expert FFN of one MoE layer for a few tokens, streaming MXFP4 weights
// from HBM (the slot arena, and the resident shared experts).
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
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

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

// E8M0 -> float: 2^(E-127); E = 0 is 2^-127 (a denormal), E = 255 is NaN
__device__ __forceinline__ float e8m0(uint32_t e) {
    e &= 0xFFu;
    float f = __uint_as_float(e << 23);
    f = e == 0u ? __uint_as_float(0x00400000u) : f;
    return e == 255u ? __uint_as_float(0x7FC00000u) : f;
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// streaming 16-byte load (weights are read once per layer step)
__device__ __forceinline__ uint4 ldg16(const uint8_t* p) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
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

__device__ __forceinline__ const uint8_t* expert_blob(const uint8_t* arena, const uint8_t* shared,
                                                      const int32_t* slots, int b, int j, int k,
                                                      int layer, int n_shared, size_t blob_bytes) {
    if (j < k) return arena + (size_t)slots[b * k + j] * blob_bytes;
    return shared + (size_t)(layer * n_shared + (j - k)) * blob_bytes;
}

// ------------------------------------------------------------------- K3 --
// grid (I/16 tiles, nE experts, B tokens); W waves; lane (r = lane&15, s = 4w + lane>>4)
template <int W, int T>
__global__ __launch_bounds__(W * 64) void k3_gate_up(K3Args a) {
    constexpr int S = 4 * W;
    extern __shared__ uint4 smem[];
    const int tile = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, s = w * 4 + (lane >> 4);
    const int NB = a.NB;
    const int nb = seg_len(NB, S, s);
    const uint8_t* blob =
        expert_blob(a.arena, a.shared, a.slots, b, j, a.k, a.layer, a.n_shared, a.blob_bytes);
    const uint8_t* tb = blob + (size_t)tile * 16 * NB * 34;
    const uint8_t* tsc = tb + (size_t)16 * NB * 32;

    float g = 0.0f, u = 0.0f;
    uint4 gc[T], uc[T];
    uint32_t sc[T];
    auto load = [&](int t0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t0 + t < nb) {
                const size_t c = (size_t)(((t0 + t) * S + s) * 16 + r);
                gc[t] = ldg16(tb + c * 32);
                uc[t] = ldg16(tb + c * 32 + 16);
                sc[t] = *reinterpret_cast<const uint16_t*>(tsc + c * 2);
            }
        }
    };
    auto compute = [&](int t0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t0 + t < nb) {
                const uint4* xb = smem + ((t0 + t) * S + s) * 5;
                g = fmaf(e8m0(sc[t]), dot32(gc[t], xb), g);
                u = fmaf(e8m0(sc[t] >> 8), dot32(uc[t], xb), u);
            }
        }
    };
    load(0);
    // activations -> LDS while the first weight loads are in flight
    const uint4* xg = reinterpret_cast<const uint4*>(a.x + (size_t)b * NB * 32);
    for (int p = tid; p < NB * 4; p += W * 64) smem[lds_pos(p >> 2, NB, S) + (p & 3)] = xg[p];
    __syncthreads();
    compute(0);
    for (int t0 = T; t0 < nb; t0 += T) {
        load(t0);
        compute(t0);
    }
    // segments of a row: lanes r, r+16, r+32, r+48 of every wave
    g += __shfl_xor(g, 16);
    g += __shfl_xor(g, 32);
    u += __shfl_xor(u, 16);
    u += __shfl_xor(u, 32);
    float* red = reinterpret_cast<float*>(smem + NB * 5);
    if (lane < 16) {
        red[(w * 16 + r) * 2] = g;
        red[(w * 16 + r) * 2 + 1] = u;
    }
    __syncthreads();
    if (tid < 16) {
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) {
            gs += red[(ww * 16 + tid) * 2];
            us += red[(ww * 16 + tid) * 2 + 1];
        }
        const float act = gs / (1.0f + __expf(-gs)) * us;
        a.a[((size_t)b * a.nE + j) * a.I + tile * 16 + tid] = f32_to_bf16(act);
    }
}

// ------------------------------------------------------------------- K4 --
// grid (H/8 tiles, B tokens); W waves; lane (r = lane&7, s = 8w + lane>>3);
// segments split the combined (expert, I-block) range of the token.
template <int W, int T>
__global__ __launch_bounds__(W * 64) void k4_down(K4Args a) {
    constexpr int S = 8 * W;
    extern __shared__ uint4 smem[];
    const int tile = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 7, s = w * 8 + (lane >> 3);
    const int NBI = a.NBI;
    const int Q = a.nE * NBI;
    const int nq = seg_len(Q, S, s), q0 = seg_begin(Q, S, s);

    float acc = 0.0f;
    int j = q0 / NBI, ib = q0 - (q0 / NBI) * NBI;
    uint4 dc[T];
    uint32_t sc[T];
    float cw[T];
    auto load = [&](int t0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t0 + t < nq) {
                const uint8_t* blob = expert_blob(a.arena, a.shared, a.slots, b, j, a.k, a.layer,
                                                  a.n_shared, a.blob_bytes);
                const size_t cell = ((size_t)tile * NBI + ib) * 8 + r;
                dc[t] = ldg16(blob + a.d_codes_off + cell * 16);
                sc[t] = blob[a.d_scales_off + cell];
                cw[t] = j < a.k ? a.w[b * a.k + j] : 1.0f;
                if (++ib == NBI) {
                    ib = 0;
                    ++j;
                }
            }
        }
    };
    auto compute = [&](int t0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t0 + t < nq) {
                const uint4* ab = smem + ((t0 + t) * S + s) * 5;
                acc = fmaf(cw[t] * e8m0(sc[t]), dot32(dc[t], ab), acc);
            }
        }
    };
    load(0);
    // intermediate activations of all experts of this token -> LDS
    const uint4* ag = reinterpret_cast<const uint4*>(a.a + (size_t)b * a.nE * a.I);
    for (int p = tid; p < Q * 4; p += W * 64) smem[lds_pos(p >> 2, Q, S) + (p & 3)] = ag[p];
    __syncthreads();
    compute(0);
    for (int t0 = T; t0 < nq; t0 += T) {
        load(t0);
        compute(t0);
    }
    // segments of an output row: lanes r + 8*i of every wave
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    float* red = reinterpret_cast<float*>(smem + Q * 5);
    if (lane < 8) red[w * 8 + r] = acc;
    __syncthreads();
    if (tid < 8) {
        float ys = 0.0f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) ys += red[ww * 8 + tid];
        a.y[(size_t)b * a.H + tile * 8 + tid] = f32_to_bf16(ys);
    }
}

// ------------------------------------------------------------ launchers --

template <int W>
static int launch_k3_w(const K3Args& a, const Layout& L, int B, hipStream_t st) {
    dim3 grid(L.I / 16, a.nE, B);
    size_t lds = (size_t)L.NB * 80 + (size_t)W * 16 * 2 * 4;
    if (L.T3 <= 1)
        hipLaunchKernelGGL((k3_gate_up<W, 1>), grid, dim3(W * 64), lds, st, a);
    else if (L.T3 <= 2)
        hipLaunchKernelGGL((k3_gate_up<W, 2>), grid, dim3(W * 64), lds, st, a);
    else if (L.T3 <= 4)
        hipLaunchKernelGGL((k3_gate_up<W, 4>), grid, dim3(W * 64), lds, st, a);
    else if (L.T3 <= 6)
        hipLaunchKernelGGL((k3_gate_up<W, 6>), grid, dim3(W * 64), lds, st, a);
    else
        hipLaunchKernelGGL((k3_gate_up<W, 8>), grid, dim3(W * 64), lds, st, a);
    return (int)hipGetLastError();
}

int launch_k3(const K3Args& a, const Layout& L, int B, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    switch (L.W3) {
        case 1: return launch_k3_w<1>(a, L, B, st);
        case 2: return launch_k3_w<2>(a, L, B, st);
        case 3: return launch_k3_w<3>(a, L, B, st);
        default: return launch_k3_w<4>(a, L, B, st);
    }
}

int k4_waves(int nE, int NBI) {
    int w = nE * NBI / 32;
    return w < 1 ? 1 : (w > 4 ? 4 : w);
}

template <int W>
static int launch_k4_w(const K4Args& a, const Layout& L, int B, hipStream_t st) {
    const int Q = a.nE * L.NBI;
    const int steps = (Q + 8 * W - 1) / (8 * W);
    dim3 grid(L.H / 8, B);
    size_t lds = (size_t)Q * 80 + (size_t)W * 8 * 4;
    if (steps <= 2)
        hipLaunchKernelGGL((k4_down<W, 2>), grid, dim3(W * 64), lds, st, a);
    else if (steps <= 4)
        hipLaunchKernelGGL((k4_down<W, 4>), grid, dim3(W * 64), lds, st, a);
    else if (steps <= 8)
        hipLaunchKernelGGL((k4_down<W, 8>), grid, dim3(W * 64), lds, st, a);
    else
        hipLaunchKernelGGL((k4_down<W, 12>), grid, dim3(W * 64), lds, st, a);
    return (int)hipGetLastError();
}

int launch_k4(const K4Args& a, const Layout& L, int B, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    switch (k4_waves(a.nE, L.NBI)) {
        case 1: return launch_k4_w<1>(a, L, B, st);
        case 2: return launch_k4_w<2>(a, L, B, st);
        case 3: return launch_k4_w<3>(a, L, B, st);
        default: return launch_k4_w<4>(a, L, B, st);
    }
}

}  // namespace moe
