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
//  k5_gate_up  per (chunk, 64*RT intermediate rows): gate and up projections
//              of the chunk's tokens on the matrix cores, SwiGLU, a (bf16);
//  k5_down     per (chunk, SPW slices of 64*RT output rows): down projection,
//              unweighted expert outputs per row, rounded to bf16 (halves the
//              bytes that k5_down writes and k5_combine reads back);
//  k5_combine  per (token, 1024 outputs): routing-weighted sum over the
//              token's experts in rank order, plus the shared expert, bf16.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, wave64): operand A is 16
// weight rows x 32 reduction elements, operand B is 32 reduction elements x
// 16 tokens, so a wave's output tile is 16 weight rows x 16 tokens.  Lane l
// (r = l % 16, q = l / 16) holds weight row r and token r of the tile and the
// reduction elements 8q..8q+7 of each MFMA.  The reduction order inside an
// MFMA is free as long as both operands agree, so a k-iteration covers four
// whole MX blocks of 32 elements, in their natural order (the activations of
// a token for one iteration are 256 contiguous bytes): lane group q takes
// block 4*it + q, loaded as a single 16-byte chunk of codes plus its scale
// byte from that block's position in the repacked blob, and MFMA step s
// (0..3) consumes elements 8s..8s+7 of every lane group's block.  Weights are
// dequantised with the gfx950 scaled convert (v_cvt_scalef32_pk_bf16_fp4), the
// E8M0 block scale folded in (a power of two, so the bf16 value is exact);
// bf16 x bf16 products are exact in the FP32 accumulator.  Token activations
// are staged in LDS per k-iteration (one copy shared by the workgroup's four
// waves, in an XOR-swizzled layout that keeps stores and operand reads free of
// bank conflicts); each wave's weights go straight to registers, two or three
// k-iterations ahead.
//
// blockIdx -> work mapping is XCD-aware: workgroup b runs on XCD b % 8, so the
// step's units are split into eight contiguous ranges, one per XCD: every XCD
// gets an equal share, and the N tiles of one chunk (same tokens, so
// L2-resident activations) run on one XCD.
#include <hip/hip_runtime.h>

#include "ffn_device.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int KG_THREADS = 1024;
constexpr int KG_MAXC = 32768;   // cache slots
static_assert(KG_MAXC / 32 <= KG_THREADS, "the grouping kernel ranks slots with one bitmap word per thread");
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

// f(i, slots[i]) for every row i < n of this thread (rows tid, tid + 1024, ...),
// with the slot loads of eight rows in flight at once
template <typename F>
__device__ __forceinline__ void for_rows(const int32_t* slots, int n, F&& f) {
    for (int base = threadIdx.x; base < n; base += KG_THREADS * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * KG_THREADS;
            v[u] = i < n ? slots[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * KG_THREADS;
            if (i < n) f(i, v[u]);
        }
    }
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
    for_rows(a.slots, n, [&](int, int sl) {
        if ((unsigned)sl < (unsigned)a.C) atomicOr(&s_bits[sl >> 5], 1u << (sl & 31));
        else if (!(a.host_rows && sl == -1)) atomicAdd(&s_invalid, 1);  // -1 with host_rows: the host's row
    });
    __syncthreads();
    // nw <= KG_MAXC / 32 = 1024: one bitmap word per thread; rank of a slot = present slots below it
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
    for_rows(a.slots, n, [&](int, int sl) {
        if (sl < 0) return;  // a host row
        const int g = s_pre[sl >> 5] + __popc(s_bits[sl >> 5] & ((1u << (sl & 31)) - 1u));
        atomicAdd(&s_cnt[g], 1);
    });
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
    for_rows(a.slots, n, [&](int i, int sl) {
        if (sl < 0) return;  // a host row
        const int g = s_pre[sl >> 5] + __popc(s_bits[sl >> 5] & ((1u << (sl & 31)) - 1u));
        a.p.perm[s_off[g] + atomicAdd(&s_cur[g], 1)] = i;
    });
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

// position of block b in the gate/up section's (step, segment) order: segment
// s holds blocks seg_begin(s) .. + seg_len(s) - 1 (the first NB % 32 segments
// one block longer), block seg_begin(s) + t sits at position t * 32 + s
__device__ __forceinline__ int gu_pos(int b, int NB) {
    const int q = NB / kGuSegments, rem = NB % kGuSegments;
    int s, t;
    if (b < rem * (q + 1)) {
        s = b / (q + 1);
        t = b - s * (q + 1);
    } else {
        const int b2 = b - rem * (q + 1);
        s = rem + b2 / q;
        t = b2 - (s - rem) * q;
    }
    return t * kGuSegments + s;
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

// Work unit of this workgroup: (chunk ci, N tile nt).  The grid is sized for the
// most chunks a step can have.  Workgroup b runs on XCD b % 8; chunks are dealt
// to the XCDs in turn and each XCD runs all N tiles of its chunks one after the
// other (they read the same activation rows, so those stay in that XCD's L2).
// Chunks go out in reverse plan order: the shared expert's full chunks, the
// heaviest, start first and the short routed ones fill the tail.  Returns false
// for workgroups past the step's units.
struct Unit {
    int ci, nt, g, nrow, base, g_slot;
};

__device__ __forceinline__ bool get_unit(const GemmArgs& a, int nt_per_chunk, Unit& u) {
    const int n_chunks = a.p.hdr[1];
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int cl = j / nt_per_chunk;            // this XCD's cl-th chunk
    const int k = cl * 8 + x;                   // position in the dealt order
    if (k >= n_chunks) return false;
    u.ci = n_chunks - 1 - k;
    u.nt = j - cl * nt_per_chunk;
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
// for all of a thread's pieces and t grows by 16 per piece.  LDS holds 16
// cells of 16 bytes per token, cell (q, s) of token t at t*16 + ((4q+s) xor
// (t%16)): the 16 lanes that store one token's pieces and the 16 lanes that
// read piece (q, s) of 16 consecutive tokens for an MFMA operand both touch 16
// different cells of a 256-byte row, i.e. every LDS bank once.
__device__ __forceinline__ int x_cell(int t, int q, int s) { return t * 16 + ((4 * q + s) ^ (t & 15)); }

template <int NTT>
struct Stager {
    const uint16_t* src[NTT];   // row base of the piece's token (row 0 for an empty row)
    uint32_t ok;                // bit i: piece i holds a row of the chunk
    int q, s, dst0;             // lane group, step, LDS cell of piece 0 (piece i: + 256 i)
};

template <int NTT>
__device__ __forceinline__ void stager_init(Stager<NTT>& st, const int* s_row, const uint16_t* src,
                                            int row_len, const GemmArgs& a, bool rows_are_tokens) {
    const int v = threadIdx.x;
    st.q = (v >> 2) & 3;
    st.s = v & 3;
    st.dst0 = x_cell(v >> 4, st.q, st.s);
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
// waits only for its own fragment while the later ones stay in flight; a step
// refills its fragment after its MFMAs.  The loop is
// compiled once per count NT of token tiles that hold rows of the chunk (a
// wave-uniform switch outside it), so its body has no branches: the LDS reads
// of one MFMA step can overlap the MFMAs of the step before.

template <int N>
struct IC {
    static constexpr int value = N;
};

// f(IC<n>) for the chunk's token-tile count n (1..NTT)
template <int NTT, typename F>
__device__ __forceinline__ void with_tiles(int n, F&& f) {
    if constexpr (NTT == 1) {
        f(IC<1>{});
    } else {
        if (n <= 1) f(IC<1>{});
        else if (n == 2) f(IC<2>{});
        else if (n == 3 && NTT > 3) f(IC<3>{});
        else f(IC<NTT>{});
    }
}

// ---------------------------------------------------------- k5_gate_up --
// RT 16-row tiles of the intermediate dimension per wave (tiles (nt*4 + w)*RT
// + j), so one LDS read of an activation operand feeds 2*RT MFMAs.
template <int NT, int RT>
struct GuFrag {
    uint4 xv[NT];
    uint4 gc[RT], uc[RT];
    uint32_t sc[RT];
};

template <int NTT, int RT, int DEPTH>
__global__ __launch_bounds__(K5_THREADS, 2) void k5_gate_up(GemmArgs a) {
    constexpr int GM = 16 * NTT;
    __shared__ uint4 xs[DEPTH][GM * 16];
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
    with_tiles<NTT>(ntt, [&](auto nt_c) {
        constexpr int NT = decltype(nt_c)::value;
        auto issue = [&](int it, GuFrag<NT, RT>& f) __attribute__((always_inline)) {
            {
                const int b = 4 * it + st.q;
                const int blk = b < NB ? b : NB - 1;
#pragma unroll
                for (int i = 0; i < NT; ++i) f.xv[i] = *reinterpret_cast<const uint4*>(st.src[i] + blk * 32);
            }
            const int b = 4 * it + q;
            const size_t c = (size_t)gu_pos(b < NB ? b : NB - 1, NB) * kGuRows + (r & 7);
#pragma unroll
            for (int j = 0; j < RT; ++j) {
                f.gc[j] = ldg16(tb[j] + c * 16);
                f.uc[j] = ldg16(tb[j] + (size_t)kGuRows * NB * 16 + c * 16);
                f.sc[j] = *reinterpret_cast<const uint16_t*>(tb[j] + (size_t)kGuRows * NB * 32 + c * 2);
            }
        };
        // MFMA step s4 (elements 8*s4.. of each lane group's block) of all NT token tiles
        auto mma = [&](const bf16x8_t* wg, const bf16x8_t* wu, const uint4* xb, int s4) __attribute__((always_inline)) {
            bf16x8_t xo[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) xo[m] = as_bf16x8(xb[x_cell(m * 16 + r, q, s4)]);
#pragma unroll
            for (int m = 0; m < NT; ++m)
#pragma unroll
                for (int j = 0; j < RT; ++j) {
                    accg[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg[j], xo[m], accg[j][m], 0, 0, 0);
                    accu[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wu[j], xo[m], accu[j][m], 0, 0, 0);
                }
        };
        // one k-iteration on fragment f; `next` refills f with a later iteration's loads
        auto step = [&](int it, GuFrag<NT, RT>& f, uint4* xb, auto&& next) __attribute__((always_inline)) {
            const bool pin = (4 * it + st.q) < NB;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const bool ok = pin && ((st.ok >> i) & 1u);
                xb[st.dst0 + 256 * i] = ok ? f.xv[i] : make_uint4(0u, 0u, 0u, 0u);
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
                mma(wg, wu, xb, s4);
            }
            next();
        };
        if constexpr (DEPTH == 3) {
            GuFrag<NT, RT> fa, fb, fc;
            issue(0, fa);
            issue(1, fb);
            issue(2, fc);
            for (int it = 0; it < nit; it += 3) {
                step(it, fa, xs[0], [&] { issue(it + 3, fa); });
                step(it + 1, fb, xs[1], [&] { issue(it + 4, fb); });
                step(it + 2, fc, xs[2], [&] { issue(it + 5, fc); });
            }
        } else {
            GuFrag<NT, RT> fa, fb;
            issue(0, fa);
            issue(1, fb);
            for (int it = 0; it < nit; it += 2) {
                step(it, fa, xs[0], [&] { issue(it + 2, fa); });
                step(it + 1, fb, xs[1], [&] { issue(it + 3, fb); });
            }
        }
    });
    // lane holds intermediate rows (tile0+j)*16 + 4q + 0..3 of token r of each token tile
#pragma unroll
    for (int m = 0; m < NTT; ++m) {
        const int row = s_row[m * 16 + r];
        if (row < 0) continue;
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            if (!tok[j]) continue;
            const f32x4_t g = accg[j][m], v = accu[j][m];
            const uint32_t lo = (uint32_t)f32_to_bf16(swiglu(g[0], v[0])) |
                                ((uint32_t)f32_to_bf16(swiglu(g[1], v[1])) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(swiglu(g[2], v[2])) |
                                ((uint32_t)f32_to_bf16(swiglu(g[3], v[3])) << 16);
            *reinterpret_cast<uint2*>(a.a + (size_t)row * a.I + (tile0 + j) * 16 + 4 * q) = make_uint2(lo, hi);
        }
    }
}

// ------------------------------------------------------------- k5_down --
// A slice is 4*RT 16-row tiles of the output, RT per wave (tiles (s*4 + w)*RT
// + j of slice s); a 16-row tile is two 8-row tiles of the D section.  A
// workgroup takes SPW consecutive slices of its chunk and runs their
// k-iterations as one pipeline (the reduction is short, I / 128 iterations, so
// the loads of the next slice are already in flight when a slice ends), storing
// each slice's outputs after its last iteration.
template <int NT, int RT>
struct DnFrag {
    uint4 xv[NT];
    uint4 dc[RT];
    uint32_t sc[RT];
};

template <int NTT, int RT, int DEPTH, int SPW>
__global__ __launch_bounds__(K5_THREADS, 2) void k5_down(GemmArgs a) {
    constexpr int GM = 16 * NTT;
    __shared__ uint4 xs[DEPTH][GM * 16];
    __shared__ int s_row[GM];
    const int n_tiles = a.H >> 4;
    const int n_slices = (n_tiles + 4 * RT - 1) / (4 * RT);
    const int nt_per_chunk = (n_slices + SPW - 1) / SPW;
    Unit u;
    if (!get_unit(a, nt_per_chunk, u)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < GM) s_row[tid] = tid < u.nrow ? a.p.perm[u.base + tid] : -1;
    const int ntt = (u.nrow + 15) >> 4;   // token tiles holding rows of the chunk
    const int NBI = a.NBI;
    const int s0 = u.nt * SPW;                        // first slice
    const int nsl = min(SPW, n_slices - s0);          // slices of this workgroup
    const int nit = (NBI + 3) >> 2;                   // k-iterations per slice
    const int F = nsl * nit;                          // pipeline length
    const int r = lane & 15, q = lane >> 4;
    const uint8_t* blob = group_blob(a, u.g_slot);
    const uint8_t* dcod0 = blob + a.d_codes_off + (size_t)(r & 7) * 16;
    const uint8_t* dsc0 = blob + a.d_scales_off + (r & 7);
    __syncthreads();
    Stager<NTT> st;
    stager_init<NTT>(st, s_row, a.a, a.I, a, false);

    f32x4_t acc[RT][NTT];
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
        for (int m = 0; m < NTT; ++m) acc[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // tile j of slice s0 + sl (clamped to tile 0 past the output), and whether it is real
    auto tile_of = [&](int sl, int j) { return ((s0 + sl) * 4 + w) * RT + j; };
    auto store = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < NTT; ++m) {
            const int row = s_row[m * 16 + r];
#pragma unroll
            for (int j = 0; j < RT; ++j) {
                const int t = tile_of(sl, j);
                const f32x4_t v = acc[j][m];
                const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                if (row >= 0 && t < n_tiles)
                    *reinterpret_cast<uint2*>(a.yp + (size_t)row * a.H + t * 16 + 4 * q) = make_uint2(lo, hi);
                acc[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    with_tiles<NTT>(ntt, [&](auto nt_c) {
        constexpr int NT = decltype(nt_c)::value;
        // loads of pipeline step f (slice f / nit, k-iteration f % nit); steps
        // past the end re-read the last one (in bounds, masked in `step`)
        auto issue = [&](int f, DnFrag<NT, RT>& fr) __attribute__((always_inline)) {
            const int fc = f < F ? f : F - 1;
            const int sl = fc / nit, it = fc - sl * nit;
            {
                const int p = 4 * it + st.q;
                const int ib = p < NBI ? p : NBI - 1;
#pragma unroll
                for (int i = 0; i < NT; ++i) fr.xv[i] = *reinterpret_cast<const uint4*>(st.src[i] + ib * 32);
            }
            const int p = 4 * it + q;
            const int ib = p < NBI ? p : NBI - 1;
#pragma unroll
            for (int j = 0; j < RT; ++j) {
                const int t = tile_of(sl, j);
                const size_t t8 = (size_t)(2 * (t < n_tiles ? t : 0) + (r >> 3)) * NBI * 8;
                fr.dc[j] = ldg16(dcod0 + (t8 + (size_t)ib * 8) * 16);
                fr.sc[j] = dsc0[t8 + (size_t)ib * 8];
            }
        };
        auto mma = [&](const bf16x8_t* wd, const uint4* xb, int s4) __attribute__((always_inline)) {
            bf16x8_t ao[NT];
#pragma unroll
            for (int m = 0; m < NT; ++m) ao[m] = as_bf16x8(xb[x_cell(m * 16 + r, q, s4)]);
#pragma unroll
            for (int m = 0; m < NT; ++m)
#pragma unroll
                for (int j = 0; j < RT; ++j)
                    acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wd[j], ao[m], acc[j][m], 0, 0, 0);
        };
        auto step = [&](int f, DnFrag<NT, RT>& fr, uint4* xb, auto&& next) __attribute__((always_inline)) {
            const bool live = f < F;
            const int sl = f / nit, it = f - sl * nit;
            const bool pin = live && (4 * it + st.q) < NBI;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const bool ok = pin && ((st.ok >> i) & 1u);
                xb[st.dst0 + 256 * i] = ok ? fr.xv[i] : make_uint4(0u, 0u, 0u, 0u);
            }
            const bool pv = live && (4 * it + q) < NBI;
            float sd[RT];
#pragma unroll
            for (int j = 0; j < RT; ++j) sd[j] = pv && tile_of(sl, j) < n_tiles ? e8m0(fr.sc[j]) : 0.0f;
            __syncthreads();
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                bf16x8_t wd[RT];
#pragma unroll
                for (int j = 0; j < RT; ++j) wd[j] = dq8(word(fr.dc[j], s4), sd[j]);
                mma(wd, xb, s4);
            }
            next();
            if (live && it == nit - 1) store(sl);
        };
        if constexpr (DEPTH == 3) {
            DnFrag<NT, RT> fa, fb, fc;
            issue(0, fa);
            issue(1, fb);
            issue(2, fc);
            for (int f = 0; f < F; f += 3) {
                step(f, fa, xs[0], [&] { issue(f + 3, fa); });
                step(f + 1, fb, xs[1], [&] { issue(f + 4, fb); });
                step(f + 2, fc, xs[2], [&] { issue(f + 5, fc); });
            }
        } else {
            DnFrag<NT, RT> fa, fb;
            issue(0, fa);
            issue(1, fb);
            for (int f = 0; f < F; f += 2) {
                step(f, fa, xs[0], [&] { issue(f + 2, fa); });
                step(f + 1, fb, xs[1], [&] { issue(f + 3, fb); });
            }
        }
    });
}

// ---------------------------------------------------------- k5_combine --
// outputs h .. h+3 of expert-output row `row` (bf16) as floats
__device__ __forceinline__ float4 yp4(const CombineArgs& c, int row, int h) {
    const uint2 v = *reinterpret_cast<const uint2*>(c.yp + (size_t)row * c.H + h);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                       __uint_as_float(v.y & 0xFFFF0000u));
}

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
        // every rank's loads are issued before the first sum (k <= 16), which then runs in rank order
        // (raw bf16 pairs are kept until the sums, so no load waits for the one before it)
        uint2 raw[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (j < c.k) raw[j] = *reinterpret_cast<const uint2*>(c.yp + (size_t)(b * c.k + j) * c.H + h);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j < c.k) {
                const int row = b * c.k + j;
                if (c.host_rows && c.slots[row] < 0) continue;  // computed by the host
                const float wj = c.w[row];
                const float4 v = make_float4(__uint_as_float(raw[j].x << 16), __uint_as_float(raw[j].x & 0xFFFF0000u),
                                             __uint_as_float(raw[j].y << 16), __uint_as_float(raw[j].y & 0xFFFF0000u));
                acc.x += wj * v.x;
                acc.y += wj * v.y;
                acc.z += wj * v.z;
                acc.w += wj * v.w;
            }
        }
        for (int s = 0; s < c.n_shared; ++s) {
            const int row = c.B * c.k + s * c.B + b;
            const float4 v = yp4(c, row, h);
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

// workgroups for max_chunks chunks of nt units each: eight XCDs x the most
// chunks one XCD is dealt x nt (the mapping of get_unit)
static int unit_grid(int max_chunks, int nt) { return (max_chunks + 7) / 8 * 8 * nt; }

// prefill-sized chunks (64 rows): gate/up waves take 2 row tiles with three
// fragments in flight, down waves 4 row tiles with two, and a down workgroup 3
// slices of 256 outputs; single-token-sized chunks (16 rows) keep one tile and
// one slice for parallelism
constexpr int RT_GU_BIG = 2, RT_D_BIG = 4, SPW_D_BIG = 3;

int launch_grouped_ffn(GroupArgs& g, GemmArgs& m, CombineArgs& c, void* stream, void* ev_mid) {
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(k2g_group, dim3(1), dim3(KG_THREADS), 0, st, g);
    const bool big = m.gm != 16;
    const int rt1 = big ? RT_GU_BIG : 1, rt2 = big ? RT_D_BIG : 1, spw = big ? SPW_D_BIG : 1;
    const int nt1 = (m.I / 16 + 4 * rt1 - 1) / (4 * rt1);
    const int nt2 = ((m.H / 16 + 4 * rt2 - 1) / (4 * rt2) + spw - 1) / spw;
    const dim3 g1(unit_grid(m.p.max_chunks, nt1)), g2(unit_grid(m.p.max_chunks, nt2));
    if (big)
        hipLaunchKernelGGL((k5_gate_up<4, RT_GU_BIG, 3>), g1, dim3(K5_THREADS), 0, st, m);
    else
        hipLaunchKernelGGL((k5_gate_up<1, 1, 3>), g1, dim3(K5_THREADS), 0, st, m);
    if (ev_mid) (void)hipEventRecord((hipEvent_t)ev_mid, st);
    if (big)
        hipLaunchKernelGGL((k5_down<4, RT_D_BIG, 2, SPW_D_BIG>), g2, dim3(K5_THREADS), 0, st, m);
    else
        hipLaunchKernelGGL((k5_down<1, 1, 3, 1>), g2, dim3(K5_THREADS), 0, st, m);
    hipLaunchKernelGGL(k5_combine, dim3((c.H + 1023) / 1024, c.B), dim3(256), 0, st, c, m.p.hdr);
    return (int)hipGetLastError();
}

}  // namespace moe
