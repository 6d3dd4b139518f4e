// Internal definitions shared by the host orchestrator and the gfx950 kernels.
//
// Kernel blob layout (what the pinned pool and the HBM slots hold; same size
// as the logical blob, 3*H*I*17/32 bytes, a permutation of its bytes):
//
//  GU section (gate and up, read by the gate/up phase of the FFN kernel), I/8
//  tiles of GR = 8 rows each.  One workgroup of 4 waves takes an 8-row tile; a
//  wave is 8 rows x 8 segments, so a row's NB = H/32 blocks are split into
//  S3 = 32 contiguous segments (segment s: nb(s) = NB/32 + (s < NB%32) blocks
//  starting at b0(s) = s*(NB/32) + min(s, NB%32)).  Lane (r, s) reads block
//  b0(s)+t at step t.  Position p = t*S3 + s enumerates the tile's blocks (for
//  p < NB it is a bijection onto them), and chunk c = p*GR + r its (row, block)
//  pairs, densely in that order:
//     tile + c*16             : gate codes of (row, block) [16 B]
//     tile + GR*NB*16 + c*16  : up codes of (row, block) [16 B]
//     tile + GR*NB*32 + c*2   : gate scale byte, up scale byte
//  so the 64 lanes of a wave read 1 KB of contiguous gate codes and 1 KB of
//  contiguous up codes per step.
//
//  D section (down, read by the down phase of the FFN kernel): codes [H/8][NB_I][8][16 B] (row tile of 8
//  output rows, block along the reduction dim I, row in tile), then scales
//  [H/8][NB_I][8].  The 8 rows of a (tile, block) are one 128-byte line.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if !defined(__HIPCC__) && !defined(__host__)
#define __host__
#define __device__
#endif

namespace moe {

struct Layout {
    int H, I, NB, NBI;     // blocks of 32 along H (gate/up rows) and along I (down rows)
    int GR;                // rows per gate/up tile (8)
    int S3, T3;            // gate/up phase: segments per row (32), max steps per lane
    size_t gu_tile_bytes;  // one gate/up tile: GR rows of gate and up codes and scales
    size_t gu_bytes;       // size of the GU section
    size_t d_codes_off;    // offset of the D codes (== gu_bytes)
    size_t d_scales_off;   // offset of the D scales
    size_t blob_bytes;
};

constexpr int kGuRows = 8;       // rows per gate/up tile
constexpr int kGuSegments = 32;  // segments per gate/up row

inline Layout make_layout(int H, int I) {
    Layout L;
    L.H = H; L.I = I; L.NB = H / 32; L.NBI = I / 32;
    L.GR = kGuRows;
    L.S3 = kGuSegments;
    L.T3 = (L.NB + L.S3 - 1) / L.S3;
    L.gu_tile_bytes = (size_t)L.GR * L.NB * 34;
    L.gu_bytes = (size_t)I * (size_t)H * 34 / 32;
    L.d_codes_off = L.gu_bytes;
    L.d_scales_off = L.gu_bytes + (size_t)H * (size_t)I / 2;
    L.blob_bytes = L.d_scales_off + (size_t)H * (size_t)I / 32;
    return L;
}

// segment s of n items split into S nearly equal contiguous parts
__host__ __device__ inline int seg_len(int n, int S, int s) { return n / S + (s < n % S ? 1 : 0); }
__host__ __device__ inline int seg_begin(int n, int S, int s) { return s * (n / S) + (s < n % S ? s : n % S); }

// host-mapped miss list written by the resolve kernel for one layer step
constexpr int HYB_MAX_IDS = 256;  // B * k of a hybrid batch step

struct MissEntry {
    int32_t expert, slot;
};
struct MissList {
    volatile int64_t seq;      // written last (system-scope release) by the resolve kernel
    int32_t n_miss, n_unique;
    int32_t n_evict, n_invalid;  // n_evict: informational, written after seq; n_invalid: ids outside [0, E)
    int32_t slot0[16];         // slots of token 0's k experts (ranked); -1: computed by the host
    float w0[16];              // routing weights of token 0 (when the step was routed)
    int32_t ids0[16];          // token 0's experts (ranked)
    int32_t n_xfer;            // misses transferred (entries [0, n_xfer)); the rest have slot -1
    int32_t ids_all[256];      // hybrid batches (n_xfer < n_miss, B * k <= 256): every token's
    float w_all[256];          // experts and weights, [B][k]
    MissEntry e[1];            // [n_miss], sized at allocation: min(max_tokens*k, E)
};

struct TraceRec {
    int32_t step, layer, expert, slot, hit, evicted_key;
};

// device-resident cache state and counters (library-owned)
struct CacheDev {
    int32_t* slot_of;     // [L*E]  slot or -1
    int32_t* key_of;      // [C]    key (layer*E + expert) or -1
    int64_t* stamp;       // [C]    last use or -1
    int64_t* clock;       // [1]
    uint64_t* counters;   // [5] hits, misses, evictions, resolves, host-computed misses
    TraceRec* trace;      // [trace_cap]
    uint64_t* trace_head; // [2] records written (monotone), records dropped
    int64_t trace_cap;
};

// ---------------------------------------------------------------- launches --
struct K1Args {
    const uint16_t* W;      // [E][H] router of this layer
    const uint16_t* x;      // [B][H]
    float* z;               // [B][E]
    int E, H, B;
};

struct K2Args {
    CacheDev c;
    const float* z;         // [B][E] logits, or NULL when the ids are given
    int32_t* ids;           // [n_ids]: written from z (top-k), else read
    float* w;               // [B][k] routing weights (written when z != NULL)
    int32_t* ids_out;       // optional copies for the caller
    float* w_out;
    int32_t* slots;         // [n_ids] slot per id
    int32_t* slots_out;     // optional second copy
    MissList* ml;           // host-mapped
    int64_t seq;
    int n_ids, layer, step, E, C, k, B;
    int policy;             // 0: LRU; 1: static split (R resident keys, T transient slots)
    int R, T;
    int hybrid;             // one-token LRU steps: transfer only q = round(nm * bp / bh) misses
    double bp, bh;          // PCIe and host expert bandwidths of the hybrid split
};

// one MoE layer's expert FFN for B tokens: gate/up + SwiGLU (K3) and
// down + weighted combine + shared expert (K4)
struct FfnArgs {
    const uint8_t* arena;   // slot arena
    const uint8_t* shared;  // [L][n_shared] blobs (kernel layout) in HBM
    const int32_t* slots;   // [B][k]
    const float* w;         // [B][k]
    const uint16_t* x;      // [B][H]
    uint16_t* a;            // [B][nE][I] bf16 (K3 -> K4)
    uint16_t* y;            // [B][H] bf16
    const float* yh;        // [B][H] FP32 added before rounding (host-computed experts), or NULL
    size_t blob_bytes, d_codes_off, d_scales_off;
    int k, n_shared, nE, layer, NB, NBI, I, H;
    int C;                  // slots in the arena: a slot outside [0, C) is never read (NaN output)
    int P1, P2;             // K3 and K4 workgroups per token
    int karg;               // 1: slots and weights of the single token come in kslot/kw
    int32_t kslot[16];
    float kw[16];
};

// ---------------------------------------------------- grouped path (B > 1) --
// Tokens of one layer step grouped by expert: every (token, rank) assignment
// is a row id r (r < B*k: token r / k, rank r % k; r = B*k + s*B + b: shared
// expert s for token b).  A group is one distinct slot (or one shared expert);
// its rows are listed contiguously in `perm`; a chunk is up to `gm` rows of
// one group, the unit of work of the grouped FFN kernels.
struct GroupPlanDev {
    int32_t* hdr;         // [4]: groups, chunks, routed groups, invalid slots
    int32_t* g_slot;      // [G]: slot, or -1-s for shared expert s
    int32_t* g_off;       // [G]: first position of the group in perm
    int32_t* g_cnt;       // [G]: rows of the group
    int32_t* chunks;      // [2*NCH]: (group, first row within the group)
    int32_t* perm;        // [B*nE]: row ids in group order
    int max_groups, max_chunks;
};

struct GroupArgs {
    GroupPlanDev p;
    const int32_t* slots;   // [B*k]
    int B, k, C, n_shared, gm;
    int host_rows;          // 1: slot -1 marks a row computed by the host (left out of the groups)
};

struct GemmArgs {
    GroupPlanDev p;
    const uint8_t* arena;
    const uint8_t* shared;  // [L][n_shared] blobs
    const uint16_t* x;      // [B][H] (gate/up input)
    uint16_t* a;            // [B*nE][I] bf16, rows = row ids
    uint16_t* yp;           // [B*nE][H] bf16, rows = row ids (unweighted expert outputs)
    size_t blob_bytes, d_codes_off, d_scales_off;
    int B, k, n_shared, layer, H, I, NB, NBI, gm;
    int nt;                 // N tiles (of 64 output rows) per chunk
};

struct CombineArgs {
    const uint16_t* yp;     // [B*nE][H] bf16 expert outputs
    const float* w;         // [B][k]
    const int32_t* slots;   // [B][k]
    uint16_t* y;            // [B][H] bf16
    const float* yh;        // [B][H] FP32 sums of the host-computed rows (host_rows), or NULL
    int B, k, n_shared, H, C;
    int host_rows;          // 1: rows with slot -1 were computed by the host and are skipped
};

// launchers (defined next to their kernels)
int launch_k1(const K1Args& a, void* stream);
int launch_k2(const K2Args& a, const int32_t* order_in, int32_t* order_out, void* stream);
int launch_ffn(FfnArgs& a, const Layout& L, int B, void* stream, void* ev_mid);
size_t ffn_lds_bytes(const Layout& L, int nE);
// one wave that waits until *done >= seq (host-mapped), at most max_polls reads, else sets *late
int launch_wait_host(const uint64_t* done, uint64_t seq, uint32_t max_polls, uint32_t* late, void* stream);
int grouped_max_groups(int B, int k, int E, int n_shared);
int grouped_max_chunks(int B, int k, int E, int n_shared, int gm);
int grouped_gm(int B);
int launch_grouped_ffn(GroupArgs& g, GemmArgs& m, CombineArgs& c, void* stream, void* ev_mid);

}  // namespace moe
