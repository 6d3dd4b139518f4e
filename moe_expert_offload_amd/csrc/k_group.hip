// Grouped expert FFN for a batch of tokens (B > 1): multi-request decode and
// prefill chunks.
//
// With several tokens per step, tokens that chose the same expert share its
// weights, so the layer is a set of small dense contractions, one per distinct
// expert: [n_e x H] x [H x 2I] -> SwiGLU -> [n_e x I] x [I x H], then the
// routing-weighted sum over each token's experts plus the shared expert.  The
// pages overlap expert loading with a prefill chunk's compute
// (ai.holude.com preflight page, section on prefill and agent workloads) and
// show per-request speed falling as concurrent requests share the cache
// (pirouter.ai "FreeToken x RTX 5090" page, section on the expert path); the
// grouping itself is not described there and is this library's design.
//
// Four launches per layer step:
//  k2g_group   one workgroup: groups the B*k (token, rank) rows by slot
//              (distinct experts of the step), appends the shared expert as a
//              group of all B tokens, and cuts groups into chunks of at most
//              gm rows (the work unit);
//  k5_gate_up  per (chunk, 64 intermediate rows): gate and up projections of
//              the chunk's tokens on the matrix cores, SwiGLU, a (bf16);
//  k5_down     per (chunk, 64 output rows): down projection, unweighted
//              expert outputs (fp32) per row;
//  k5_combine  per (token, 1024 outputs): routing-weighted sum over the
//              token's experts in rank order, plus the shared expert, bf16.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, wave64): operand A is 16
// weight rows x 32 reduction elements, operand B is 32 reduction elements x
// 16 tokens, so a wave's output tile is 16 weight rows x 16 tokens.  Lane l
// (r = l % 16, q = l / 16) holds weight row r and token r of the tile and the
// reduction elements 8q..8q+7 of each MFMA.  The reduction order inside an
// MFMA is free as long as both operands agree, so a k-iteration covers four
// whole MX blocks of 32 elements: lane group q takes one block, loaded as a
// single 16-byte chunk of codes plus its scale byte, and MFMA step s (0..3)
// consumes elements 8s..8s+7 of every lane group's block.  Weights are
// dequantised with the gfx950 scaled convert (v_cvt_scalef32_pk_bf16_fp4), the
// E8M0 block scale folded in (a power of two, so the bf16 value is exact);
// bf16 x bf16 products are exact in the FP32 accumulator.  Both matrices are
// read in the same repacked blob layout as the single-token kernels, each
// wave read a contiguous 1 KB (gate/up) or eight whole 128-byte lines (down).
// Token activations are staged in LDS per k-iteration (three buffers), one
// copy shared by the workgroup's four waves.
//
// blockIdx -> work mapping is XCD-aware: consecutive workgroups go to
// different XCDs, so the linear index is remapped so that each XCD gets a
// contiguous range of (chunk, N tile) units, i.e. the N tiles of one chunk
// (same tokens, L2-resident activations) run on one XCD.
#include <hip/hip_runtime.h>

#include "ffn_device.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int KG_THREADS = 1024;
constexpr int KG_MAXC = 16384;   // cache slots
constexpr int KG_MAXG = 1024;    // routed groups (distinct experts <= E <= 1024)
constexpr int K5_THREADS = 256;

int grouped_gm(int B) { return B <= 16 ? 16 : 64; }

int grouped_max_groups(int B, int k, int E, int n_shared) {
    const long bk = (long)B * k;
    return (int)(bk < E ? bk : E) + n_shared;
}

// sum over groups of ceil(rows / gm) < groups + all rows / gm
int grouped_max_chunks(int B, int k, int E, int n_shared, int gm) {
    return grouped_max_groups(B, k, E, n_shared) + (int)(((long)B * (k + n_shared)) / gm);
}

// ------------------------------------------------------------ k2g_group --

// exclusive prefix sum over the 1024 threads, in thread order
__device__ __forceinline__ int kg_scan(int v, int* s_wave, int& total) {
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
    for (int w = 0; w < KG_THREADS / 64; ++w) {
        int c = s_wave[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

__global__ __launch_bounds__(KG_THREADS) void k2g_group(GroupArgs a) {
    __shared__ uint32_t s_bits[KG_MAXC / 32];
    __shared__ int32_t s_pre[KG_MAXC / 32];
    __shared__ int32_t s_cnt[KG_MAXG];
    __shared__ int32_t s_off[KG_MAXG];
    __shared__ int32_t s_cur[KG_MAXG];
    __shared__ int s_wave[KG_THREADS / 64];
    __shared__ int s_invalid;
    const int tid = threadIdx.x;
    const int n = a.B * a.k, nw = (a.C + 31) / 32;
    for (int i = tid; i < nw; i += KG_THREADS) s_bits[i] = 0u;
    for (int i = tid; i < KG_MAXG; i += KG_THREADS) {
        s_cnt[i] = 0;
        s_cur[i] = 0;
    }
    if (tid == 0) s_invalid = 0;
    __syncthreads();
    for (int i = tid; i < n; i += KG_THREADS) {
        const int sl = a.slots[i];
        if ((unsigned)sl < (unsigned)a.C) atomicOr(&s_bits[sl >> 5], 1u << (sl & 31));
        else if (!(a.host_rows && sl == -1)) atomicAdd(&s_invalid, 1);  // -1 with host_rows: the host's row
    }
    __syncthreads();
    // nw <= 512: one bitmap word per thread; rank of a slot = present slots below it
    const int pc = tid < nw ? __popc(s_bits[tid]) : 0;
    int n_rg;
    const int pre = kg_scan(pc, s_wave, n_rg);
    if (tid < nw) s_pre[tid] = pre;
    const int max_rg = a.p.max_groups - a.n_shared;
    if (s_invalid != 0 || n_rg > max_rg || n_rg > KG_MAXG) {
        // slots outside [0, C) or more distinct slots than experts: empty plan,
        // flagged; the combine then writes NaN outputs
        if (tid == 0) {
            a.p.hdr[0] = 0;
            a.p.hdr[1] = 0;
            a.p.hdr[2] = 0;
            a.p.hdr[3] = s_invalid != 0 ? s_invalid : -1;
        }
        return;
    }
    __syncthreads();
    for (int i = tid; i < n; i += KG_THREADS) {
        const int sl = a.slots[i];
        if (sl < 0) continue;  // a host row
        const int g = s_pre[sl >> 5] + __popc(s_bits[sl >> 5] & ((1u << (sl & 31)) - 1u));
        atomicAdd(&s_cnt[g], 1);
    }
    if (tid < nw) {
        uint32_t bits = s_bits[tid];
        int g = s_pre[tid];
        while (bits) {
            const int b = __ffs(bits) - 1;
            a.p.g_slot[g++] = tid * 32 + b;
            bits &= bits - 1u;
        }
    }
    __syncthreads();
    const int cnt = tid < n_rg ? s_cnt[tid] : 0;
    int rows;
    const int off = kg_scan(cnt, s_wave, rows);
    const int nch = (cnt + a.gm - 1) / a.gm;
    int n_rch;
    const int cbase = kg_scan(nch, s_wave, n_rch);
    if (tid < n_rg) {
        s_off[tid] = off;
        a.p.g_off[tid] = off;
        a.p.g_cnt[tid] = cnt;
        for (int c = 0; c < nch; ++c) {
            a.p.chunks[2 * (cbase + c)] = tid;
            a.p.chunks[2 * (cbase + c) + 1] = c * a.gm;
        }
    }
    // shared expert s: group n_rg + s, rows n + s*B + b (token b), in token order
    const int sh_nch = (a.B + a.gm - 1) / a.gm;
    for (int i = tid; i < a.n_shared * sh_nch; i += KG_THREADS) {
        const int s = i / sh_nch, c = i - s * sh_nch;
        a.p.chunks[2 * (n_rch + i)] = n_rg + s;
        a.p.chunks[2 * (n_rch + i) + 1] = c * a.gm;
    }
    if (tid < a.n_shared) {
        a.p.g_slot[n_rg + tid] = -1 - tid;
        a.p.g_off[n_rg + tid] = n + tid * a.B;
        a.p.g_cnt[n_rg + tid] = a.B;
    }
    for (int i = tid; i < a.n_shared * a.B; i += KG_THREADS) a.p.perm[n + i] = n + i;
    __syncthreads();
    // rows of a group in any order: every output element depends on its own
    // token only, so the order inside a group does not change any result
    for (int i = tid; i < n; i += KG_THREADS) {
        const int sl = a.slots[i];
        if (sl < 0) continue;  // a host row
        const int g = s_pre[sl >> 5] + __popc(s_bits[sl >> 5] & ((1u << (sl & 31)) - 1u));
        a.p.perm[s_off[g] + atomicAdd(&s_cur[g], 1)] = i;
    }
    if (tid == 0) {
        a.p.hdr[0] = n_rg + a.n_shared;
        a.p.hdr[1] = n_rch + a.n_shared * sh_nch;
        a.p.hdr[2] = n_rg;
        a.p.hdr[3] = 0;
    }
}

// ------------------------------------------------------ matrix-core FFN --

__device__ __forceinline__ const uint8_t* group_blob(const GemmArgs& a, int g_slot) {
    return g_slot >= 0 ? a.arena + (size_t)g_slot * a.blob_bytes
                       : a.shared + (size_t)(a.layer * a.n_shared + (-1 - g_slot)) * a.blob_bytes;
}

__device__ __forceinline__ int row_token(const GemmArgs& a, int row) {
    const int n = a.B * a.k;
    return row < n ? row / a.k : (row - n) % a.B;
}

// block index of position p of the gate/up section's (step, segment) order
__device__ __forceinline__ int gu_block(int p, int NB) {
    return seg_begin(NB, kGuSegments, p % kGuSegments) + p / kGuSegments;
}

// 8 E2M1 codes (one dword) times the block scale -> 8 bf16 MFMA operand values
__device__ __forceinline__ bf16x8_t dq8(uint32_t w, float s) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    const u32x4_t v = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                       __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    const u32x4_t u = {v.x, v.y, v.z, v.w};
    return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ uint32_t word(uint4 v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Work unit of this workgroup: (chunk ci, N tile nt), XCD-aware.  Returns false
// when the unit is past the step's chunks (the grid is sized for the maximum).
struct Unit {
    int ci, nt, g, nrow, base, g_slot;
};

__device__ __forceinline__ bool get_unit(const GemmArgs& a, int nt_per_chunk, Unit& u) {
    const int G = gridDim.x;
    const int logical = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    u.ci = logical / nt_per_chunk;
    u.nt = logical - u.ci * nt_per_chunk;
    if (u.ci >= a.p.hdr[1]) return false;
    u.g = a.p.chunks[2 * u.ci];
    const int start = a.p.chunks[2 * u.ci + 1];
    const int cnt = a.p.g_cnt[u.g];
    u.nrow = min(a.gm, cnt - start);
    u.base = a.p.g_off[u.g] + start;
    u.g_slot = a.p.g_slot[u.g];
    return true;
}

// Activation staging: the chunk's GM token rows x 4 blocks (64 bytes each) per
// k-iteration, NTT 16-byte pieces per thread.  Piece v = tid + 256*i is
// (token t = v/16, lane group q = (v/4)%4, step s = v%4): q and s are the same
// for all of a thread's pieces and t grows by 16 per piece.  LDS: [token][q] in
// 80-byte cells (5 x 16 B), so the 16 tokens a wave reads at once are spread
// over the banks.
template <int NTT>
struct Stager {
    const uint16_t* src[NTT];   // row base of the piece's token (row 0 for an empty row)
    uint32_t ok;                // bit i: piece i holds a row of the chunk
    int q, s, dst0;             // lane group, step, LDS cell of piece 0 (piece i: + 320 i)
};

template <int NTT>
__device__ __forceinline__ void stager_init(Stager<NTT>& st, const int* s_row, const uint16_t* src,
                                            int row_len, const GemmArgs& a, bool rows_are_tokens) {
    const int v = threadIdx.x;
    st.q = (v >> 2) & 3;
    st.s = v & 3;
    st.dst0 = ((v >> 4) * 4 + st.q) * 5 + st.s;
    st.ok = 0u;
#pragma unroll
    for (int i = 0; i < NTT; ++i) {
        const int row = s_row[(v >> 4) + 16 * i];
        st.ok |= row >= 0 ? (1u << i) : 0u;
        const int rr = row >= 0 ? (rows_are_tokens ? row_token(a, row) : row) : 0;
        st.src[i] = src + (size_t)rr * row_len + st.s * 8;
    }
}

// Main loops: the loads of k-iteration it (activation pieces and this lane's
// weight chunk) go into a fragment issued DEPTH (2 or 3) iterations ahead;
// DEPTH fragments and LDS buffers are used in turn (the loop is unrolled by
// DEPTH so each has fixed registers).  Iterations past the end read clamped,
// in-bounds addresses and are masked.  Loads complete in order, so a step
// waits only for its own fragment while the later ones stay in flight.  Token
// tiles past the chunk's rows are skipped (a wave-uniform branch).

// ---------------------------------------------------------- k5_gate_up --
// RT 16-row tiles of the intermediate dimension per wave (tiles (nt*4 + w)*RT
// + j), so one LDS read of an activation operand feeds 2*RT MFMAs.
template <int NTT, int RT>
struct GuFrag {
    uint4 xv[NTT];
    uint4 gc[RT], uc[RT];
    uint32_t sc[RT];
};

template <int NTT, int RT, int DEPTH>
__global__ __launch_bounds__(K5_THREADS, 2) void k5_gate_up(GemmArgs a) {
    constexpr int GM = 16 * NTT;
    __shared__ uint4 xs[DEPTH][GM * 4 * 5];
    __shared__ int s_row[GM];
    const int n_tiles = a.I >> 4;
    const int nt_per_chunk = (n_tiles + 4 * RT - 1) / (4 * RT);
    Unit u;
    if (!get_unit(a, nt_per_chunk, u)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < GM) s_row[tid] = tid < u.nrow ? a.p.perm[u.base + tid] : -1;
    const int ntt = (u.nrow + 15) >> 4;   // token tiles holding rows of the chunk
    const int NB = a.NB;
    const int tile0 = (u.nt * 4 + w) * RT;
    const uint8_t* blob = group_blob(a, u.g_slot);
    const int r = lane & 15, q = lane >> 4;
    // a 16-row operand tile is two 8-row gate/up tiles of the blob: rows r < 8 from the first
    const uint8_t* tb[RT];
    bool tok[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j) {
        tok[j] = tile0 + j < n_tiles;
        tb[j] = blob + (size_t)(2 * (tok[j] ? tile0 + j : 0) + (r >> 3)) * kGuRows * NB * 34;
    }
    __syncthreads();
    Stager<NTT> st;
    stager_init<NTT>(st, s_row, a.x, a.H, a, true);

    f32x4_t accg[RT][NTT], accu[RT][NTT];
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
        for (int m = 0; m < NTT; ++m) {
            accg[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            accu[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    const int nit = (NB + 3) >> 2;
    auto issue = [&](int it, GuFrag<NTT, RT>& f) {
        {
            const int p = 4 * it + st.q;
            const int blk = gu_block(p < NB ? p : NB - 1, NB);
#pragma unroll
            for (int i = 0; i < NTT; ++i) f.xv[i] = *reinterpret_cast<const uint4*>(st.src[i] + blk * 32);
        }
        const int p = 4 * it + q;
        const size_t c = (size_t)(p < NB ? p : NB - 1) * kGuRows + (r & 7);
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            f.gc[j] = ldg16(tb[j] + c * 16);
            f.uc[j] = ldg16(tb[j] + (size_t)kGuRows * NB * 16 + c * 16);
            f.sc[j] = *reinterpret_cast<const uint16_t*>(tb[j] + (size_t)kGuRows * NB * 32 + c * 2);
        }
    };
    auto step = [&](int it, const GuFrag<NTT, RT>& f, uint4* xb) {
        const bool pin = (4 * it + st.q) < NB;
#pragma unroll
        for (int i = 0; i < NTT; ++i) {
            const bool ok = pin && ((st.ok >> i) & 1u);
            xb[st.dst0 + 320 * i] = ok ? f.xv[i] : make_uint4(0u, 0u, 0u, 0u);
        }
        const bool pv = (4 * it + q) < NB;
        float sg[RT], su[RT];
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            sg[j] = pv && tok[j] ? e8m0(f.sc[j]) : 0.0f;
            su[j] = pv && tok[j] ? e8m0(f.sc[j] >> 8) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            bf16x8_t wg[RT], wu[RT];
#pragma unroll
            for (int j = 0; j < RT; ++j) {
                wg[j] = dq8(word(f.gc[j], s4), sg[j]);
                wu[j] = dq8(word(f.uc[j], s4), su[j]);
            }
#pragma unroll
            for (int m = 0; m < NTT; ++m) {
                if (NTT > 1 && m >= ntt) continue;
                const bf16x8_t xo = as_bf16x8(xb[((m * 16 + r) * 4 + q) * 5 + s4]);
#pragma unroll
                for (int j = 0; j < RT; ++j) {
                    accg[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg[j], xo, accg[j][m], 0, 0, 0);
                    accu[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wu[j], xo, accu[j][m], 0, 0, 0);
                }
            }
        }
    };
    if constexpr (DEPTH == 3) {
        GuFrag<NTT, RT> fa, fb, fc;
        issue(0, fa);
        issue(1, fb);
        issue(2, fc);
        for (int it = 0; it < nit; it += 3) {
            step(it, fa, xs[0]);
            issue(it + 3, fa);
            step(it + 1, fb, xs[1]);
            issue(it + 4, fb);
            step(it + 2, fc, xs[2]);
            issue(it + 5, fc);
        }
    } else {
        GuFrag<NTT, RT> fa, fb;
        issue(0, fa);
        issue(1, fb);
        for (int it = 0; it < nit; it += 2) {
            step(it, fa, xs[0]);
            issue(it + 2, fa);
            step(it + 1, fb, xs[1]);
            issue(it + 3, fb);
        }
    }
    // lane holds intermediate rows (tile0+j)*16 + 4q + 0..3 of token r of each token tile
#pragma unroll
    for (int m = 0; m < NTT; ++m) {
        {
            const int row = s_row[m * 16 + r];
            if (row >= 0) {
#pragma unroll
                for (int j = 0; j < RT; ++j) {
                    if (!tok[j]) continue;
                    const f32x4_t g = accg[j][m], v = accu[j][m];
                    const uint32_t lo = (uint32_t)f32_to_bf16(swiglu(g[0], v[0])) |
                                        ((uint32_t)f32_to_bf16(swiglu(g[1], v[1])) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16(swiglu(g[2], v[2])) |
                                        ((uint32_t)f32_to_bf16(swiglu(g[3], v[3])) << 16);
                    *reinterpret_cast<uint2*>(a.a + (size_t)row * a.I + (tile0 + j) * 16 + 4 * q) =
                        make_uint2(lo, hi);
                }
            }
        }
    }
}

// ------------------------------------------------------------- k5_down --
// RT 16-row tiles of the output per wave (tiles (nt*4 + w)*RT + j); a 16-row
// tile is two 8-row tiles of the D section.
template <int NTT, int RT>
struct DnFrag {
    uint4 xv[NTT];
    uint4 dc[RT];
    uint32_t sc[RT];
};

template <int NTT, int RT, int DEPTH>
__global__ __launch_bounds__(K5_THREADS, 2) void k5_down(GemmArgs a) {
    constexpr int GM = 16 * NTT;
    __shared__ uint4 xs[DEPTH][GM * 4 * 5];
    __shared__ int s_row[GM];
    const int n_tiles = a.H >> 4;
    const int nt_per_chunk = (n_tiles + 4 * RT - 1) / (4 * RT);
    Unit u;
    if (!get_unit(a, nt_per_chunk, u)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < GM) s_row[tid] = tid < u.nrow ? a.p.perm[u.base + tid] : -1;
    const int ntt = (u.nrow + 15) >> 4;   // token tiles holding rows of the chunk
    const int NBI = a.NBI;
    const int tile0 = (u.nt * 4 + w) * RT;
    const int r = lane & 15, q = lane >> 4;
    const uint8_t* blob = group_blob(a, u.g_slot);
    const uint8_t* dcod[RT];
    const uint8_t* dsc[RT];
    bool tok[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j) {
        tok[j] = tile0 + j < n_tiles;
        const int t8 = 2 * (tok[j] ? tile0 + j : 0) + (r >> 3), rr = r & 7;
        dcod[j] = blob + a.d_codes_off + ((size_t)t8 * NBI * 8 + rr) * 16;
        dsc[j] = blob + a.d_scales_off + (size_t)t8 * NBI * 8 + rr;
    }
    __syncthreads();
    Stager<NTT> st;
    stager_init<NTT>(st, s_row, a.a, a.I, a, false);

    f32x4_t acc[RT][NTT];
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
        for (int m = 0; m < NTT; ++m) acc[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nit = (NBI + 3) >> 2;
    auto issue = [&](int it, DnFrag<NTT, RT>& f) {
        {
            const int p = 4 * it + st.q;
            const int ib = p < NBI ? p : NBI - 1;
#pragma unroll
            for (int i = 0; i < NTT; ++i) f.xv[i] = *reinterpret_cast<const uint4*>(st.src[i] + ib * 32);
        }
        const int p = 4 * it + q;
        const int ib = p < NBI ? p : NBI - 1;
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            f.dc[j] = ldg16(dcod[j] + (size_t)ib * 8 * 16);
            f.sc[j] = dsc[j][(size_t)ib * 8];
        }
    };
    auto step = [&](int it, const DnFrag<NTT, RT>& f, uint4* xb) {
        const bool pin = (4 * it + st.q) < NBI;
#pragma unroll
        for (int i = 0; i < NTT; ++i) {
            const bool ok = pin && ((st.ok >> i) & 1u);
            xb[st.dst0 + 320 * i] = ok ? f.xv[i] : make_uint4(0u, 0u, 0u, 0u);
        }
        const bool pv = (4 * it + q) < NBI;
        float sd[RT];
#pragma unroll
        for (int j = 0; j < RT; ++j) sd[j] = pv && tok[j] ? e8m0(f.sc[j]) : 0.0f;
        __syncthreads();
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            bf16x8_t wd[RT];
#pragma unroll
            for (int j = 0; j < RT; ++j) wd[j] = dq8(word(f.dc[j], s4), sd[j]);
#pragma unroll
            for (int m = 0; m < NTT; ++m) {
                if (NTT > 1 && m >= ntt) continue;
                const bf16x8_t ao = as_bf16x8(xb[((m * 16 + r) * 4 + q) * 5 + s4]);
#pragma unroll
                for (int j = 0; j < RT; ++j)
                    acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wd[j], ao, acc[j][m], 0, 0, 0);
            }
        }
    };
    if constexpr (DEPTH == 3) {
        DnFrag<NTT, RT> fa, fb, fc;
        issue(0, fa);
        issue(1, fb);
        issue(2, fc);
        for (int it = 0; it < nit; it += 3) {
            step(it, fa, xs[0]);
            issue(it + 3, fa);
            step(it + 1, fb, xs[1]);
            issue(it + 4, fb);
            step(it + 2, fc, xs[2]);
            issue(it + 5, fc);
        }
    } else {
        DnFrag<NTT, RT> fa, fb;
        issue(0, fa);
        issue(1, fb);
        for (int it = 0; it < nit; it += 2) {
            step(it, fa, xs[0]);
            issue(it + 2, fa);
            step(it + 1, fb, xs[1]);
            issue(it + 3, fb);
        }
    }
#pragma unroll
    for (int m = 0; m < NTT; ++m) {
        {
            const int row = s_row[m * 16 + r];
            if (row >= 0) {
#pragma unroll
                for (int j = 0; j < RT; ++j) {
                    if (!tok[j]) continue;
                    *reinterpret_cast<float4*>(a.yp + (size_t)row * a.H + (tile0 + j) * 16 + 4 * q) =
                        make_float4(acc[j][m][0], acc[j][m][1], acc[j][m][2], acc[j][m][3]);
                }
            }
        }
    }
}

// ---------------------------------------------------------- k5_combine --
// grid (ceil(H / 1024), B), 256 threads, 4 outputs per thread
__global__ __launch_bounds__(256) void k5_combine(CombineArgs c, const int32_t* hdr) {
    const int b = blockIdx.y;
    const int h = 4 * (blockIdx.x * 256 + threadIdx.x);
    if (h >= c.H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (hdr[3] != 0) {
        acc = make_float4(__uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u),
                          __uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u));
    } else {
        for (int j = 0; j < c.k; ++j) {
            const int row = b * c.k + j;
            if (c.host_rows && c.slots[row] < 0) continue;  // computed by the host
            const float wj = c.w[row];
            const float4 v = *reinterpret_cast<const float4*>(c.yp + (size_t)row * c.H + h);
            acc.x += wj * v.x;
            acc.y += wj * v.y;
            acc.z += wj * v.z;
            acc.w += wj * v.w;
        }
        for (int s = 0; s < c.n_shared; ++s) {
            const int row = c.B * c.k + s * c.B + b;
            const float4 v = *reinterpret_cast<const float4*>(c.yp + (size_t)row * c.H + h);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        if (c.yh) {
            // the host-computed experts' weighted sum for this token (host-mapped memory)
            const float4 v = *reinterpret_cast<const float4*>(c.yh + (size_t)b * c.H + h);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
    }
    const uint32_t lo = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(c.y + (size_t)b * c.H + h) = make_uint2(lo, hi);
}

static int pad8(long v) { return (int)((v + 7) / 8 * 8); }

// row tiles per wave: gate/up and down of prefill-sized chunks (64 rows) take
// 2 and 4 tiles; single-token-sized chunks (16 rows) keep one for parallelism
constexpr int RT_GU_BIG = 2, RT_D_BIG = 4;

int launch_grouped_ffn(GroupArgs& g, GemmArgs& m, CombineArgs& c, void* stream, void* ev_mid) {
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(k2g_group, dim3(1), dim3(KG_THREADS), 0, st, g);
    const bool big = m.gm != 16;
    const int rt1 = big ? RT_GU_BIG : 1, rt2 = big ? RT_D_BIG : 1;
    const int nt1 = (m.I / 16 + 4 * rt1 - 1) / (4 * rt1), nt2 = (m.H / 16 + 4 * rt2 - 1) / (4 * rt2);
    const dim3 g1(pad8((long)m.p.max_chunks * nt1)), g2(pad8((long)m.p.max_chunks * nt2));
    if (big)
        hipLaunchKernelGGL((k5_gate_up<4, RT_GU_BIG, 2>), g1, dim3(K5_THREADS), 0, st, m);
    else
        hipLaunchKernelGGL((k5_gate_up<1, 1, 3>), g1, dim3(K5_THREADS), 0, st, m);
    if (ev_mid) (void)hipEventRecord((hipEvent_t)ev_mid, st);
    if (big)
        hipLaunchKernelGGL((k5_down<4, RT_D_BIG, 2>), g2, dim3(K5_THREADS), 0, st, m);
    else
        hipLaunchKernelGGL((k5_down<1, 1, 3>), g2, dim3(K5_THREADS), 0, st, m);
    hipLaunchKernelGGL(k5_combine, dim3((c.H + 1023) / 1024, c.B), dim3(256), 0, st, c, m.p.hdr);
    return (int)hipGetLastError();
}

}  // namespace moe
