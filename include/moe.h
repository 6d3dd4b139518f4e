/*
 * moe.h -- C ABI of the MI355X (gfx950) decode-time MoE layer library with a
 * router-following LRU cache of expert slots.
 *
 * The method (FreeToken's offload backend, as the pages describe it):
 *   pirouter.ai, "FreeToken x RTX 5090 -- 120B MoE が 127 tok/s、その請求書",
 *   section on how 65 GB runs on a 32 GB GPU: every expert lives in pinned
 *   host RAM, the GPU keeps an LRU cache of expert slots, and a miss is
 *   streamed over PCIe; the cache follows the router.
 *   ai-hardware-zukan.com, "VRAMに収まらないMoEモデルのデコードが約2倍になった",
 *   section on how misses are made up for: cache unit = (layer, expert),
 *   replacement = least recently used.
 *   gaming-st.com DeepSeek page, section on the role of VRAM: one global LRU
 *   expert cache.
 *   ai.holude.com preflight page, section on long prompts: the next layer's
 *   experts are loaded over PCIe while the GPU computes the current layer.
 *
 * Per token and layer the library runs: router logits (K1), top-k + softmax
 * over the selected logits and resolution of the selected (layer, expert)
 * pairs to cache slots with a miss list (K2), one host-to-device copy per miss
 * on the copy stream, then the expert FFN: the selected experts' MXFP4
 * gate/up + SwiGLU (K3), and the down projection fused with the weighted
 * combine and the shared expert (K4).
 *
 * Conventions
 *  - Every call returns moe_status; nothing throws or aborts across the ABI.
 *  - Pointers named *_dev are device pointers; the others are host pointers.
 *  - Streams are hipStream_t passed as void*; calls are ordered on the
 *    compute stream.  Calls that resolve the cache block the calling host
 *    thread until the step's miss list is readable (the host issues the copies).
 *  - After a HIP error the context is failed: every later call returns
 *    MOE_ESTATE; moe_last_error() tells what happened; destroy and re-create.
 *  - One context per host thread; calls on one context must not overlap.
 *
 * Data formats
 *  - bf16 = IEEE binary32 upper 16 bits, little-endian uint16.
 *  - Logical expert blob (what the fill callback writes; 3*H*I*17/32 bytes):
 *      gate codes [I][H/2], gate scales [I][H/32],
 *      up   codes [I][H/2], up   scales [I][H/32],
 *      down codes [H][I/2], down scales [H][I/32].
 *    MXFP4: a code byte holds element 2j (low nibble) and 2j+1 (high nibble),
 *    each an E2M1 value; a scale byte is the E8M0 exponent (2^(E-127)) shared
 *    by 32 consecutive elements along the row.  The library repacks blobs into
 *    its own kernel layout when it fills the pool; slots hold that layout.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,     /* bad argument or unsupported shape */
    MOE_ENOMEM = -2,     /* host (pinned) or device allocation failed, or a caller buffer is too small */
    MOE_EHIP = -3,       /* a HIP call failed; the context is now failed */
    MOE_ECAPACITY = -4,  /* cache_slots < 2 * largest distinct expert set one step can request */
    MOE_ESTATE = -5,     /* context already failed */
    MOE_EVERIFY = -6,    /* verify mode: a filled slot differs from its pool blob; the context is now failed */
} moe_status;

/* Cache policy (moe_config.policy).
 * MOE_POLICY_LRU: one least-recently-used cache over all C slots and all layers, following the
 *   router (ai-hardware-zukan.com FreeToken vs Ollama page, section on how misses are made up
 *   for; gaming-st.com DeepSeek page: one global LRU expert cache).
 * MOE_POLICY_STATIC: the static per-layer split the same page compares it with.  The first
 *   R = C - T keys (layer * E + expert, pool order: whole layers, then part of one) stay in slots
 *   0..R-1, filled at init; every access to another key is a miss streamed into the next of the
 *   T = 2 * min(max_tokens * k, E) transient slots, in rotation (a streaming buffer, not a cache:
 *   the same key requested again is streamed again). */
enum { MOE_POLICY_LRU = 0, MOE_POLICY_STATIC = 1 };

enum {
    MOE_FLAG_PROFILE = 1,  /* time every K3 and K4 launch with HIP events (read via moe_stats) */
    MOE_FLAG_PER_TOKEN_FFN = 2,  /* B > 1: run the per-token GEMV kernels instead of the grouped MFMA path */
    MOE_FLAG_VERIFY = 4,   /* debug: after each step's copies land, read every filled slot back and compare it
                              with its pool blob (MOE_EVERIFY on a difference); also MOE_VERIFY=1 in the
                              environment at init.  Synchronous and slow: for tests and bring-up only */
};

typedef struct {
    int32_t n_layers;       /* L */
    int32_t n_experts;      /* E routed experts per layer, 1..1024 */
    int32_t top_k;          /* k, 1..16 and <= E */
    int32_t hidden;         /* H, multiple of 32, <= 16384 */
    int32_t inter;          /* I, multiple of 32, <= 16384 */
    int32_t n_shared;       /* always-on shared experts per layer (0 or 1), resident in HBM */
    int32_t cache_slots;    /* C: GPU expert slots, <= 32768; must be >= 2 * min(max_tokens * k, E) */
    int32_t max_tokens;     /* largest n_tokens of any call */
    int32_t lookahead;      /* moe_stack_forward: D = 2 .. 7 resolves layer l+D and copies its
                               misses while layers l .. l+D-1 wait for theirs (LRU policy, offload
                               steps and cache_slots >= (D + 1) * top_k * n_tokens of the call; a
                               call whose cache is smaller takes the deepest D that fits, else
                               lookahead 1); 1 = resolve and copy layer l+1 while layer l's FFN
                               runs; 0 = causal (each layer's copies before its FFN).  Every
                               lookahead gives the same ids, slots, trace and outputs */
    int32_t trace_capacity; /* cache trace records kept on the device (0 = none) */
    int32_t fill_threads;   /* host threads calling the fill callback (0 = all cores) */
    int32_t flags;          /* MOE_FLAG_* */
    int32_t pinned_mb;      /* at most this many MiB of the pool in pinned memory (0 = as much as the
                               platform grants); the rest is pageable and its misses go through a
                               ring of pinned bounce buffers */
    int32_t policy;         /* MOE_POLICY_LRU (default) or MOE_POLICY_STATIC */
} moe_config;

/* Writes the logical blob of routed expert (layer, expert >= 0) or of shared
 * expert s (expert = -1 - s) into dst.  May be called from several threads at
 * once with different dst buffers. */
typedef void (*moe_fill_fn)(void* user, int32_t layer, int32_t expert, uint8_t* dst_blob);

typedef struct moe_ctx moe_ctx;

/* Sizes the caller must provide: bytes of one expert blob, of the slot arena
 * (C blobs) and of the workspace.  Any pointer may be NULL.  Checks cfg. */
moe_status moe_query_sizes(const moe_config* cfg, size_t* blob_bytes, size_t* arena_bytes,
                           size_t* workspace_bytes);

/* Cache auto-sizing: the expert-cache share of device memory is taken from
 * the memory still free (FreeToken's --moe-cache-auto option, which splits
 * free VRAM between the KV cache and the expert cache; pirouter.ai page
 * "FreeToken × RTX 5090——120B MoE が 127 tok/s、その請求書", section on how
 * 65 GB run on a 32 GB GPU).  Call it after the workspace (and anything else
 * the caller keeps on the device) is allocated; cfg->cache_slots is ignored
 * (may be 0 here and in moe_query_sizes, which then reports arena_bytes 0).
 * *slots_out = the largest C with
 *     C * blob + the library's own device bytes at C (cache state, router
 *     weights, shared experts; each rounded to 2 MiB) + reserve_bytes
 *     <= free_bytes,
 * capped at n_layers * n_experts (the whole pool) and at 32768 slots.
 * free_bytes: device bytes free; 0 = ask the runtime (hipMemGetInfo on the
 * current device).  reserve_bytes: kept free for the caller (KV cache,
 * activations, allocator slack).  Allocates nothing.
 * Errors: MOE_EINVAL (shape), MOE_EHIP (memory query failed), MOE_ECAPACITY
 * (the C that fits is below 2 * min(max_tokens * k, E); *slots_out still holds
 * it). */
moe_status moe_auto_cache_slots(const moe_config* cfg, uint64_t free_bytes, uint64_t reserve_bytes,
                                int32_t* slots_out);

/* Builds a context: allocates the host pool of all L*E routed expert blobs and
 * fills it through `fill` (called once per (layer, expert) and once per shared
 * expert), copies the router weights (host [L][E][H] bf16) and the shared
 * experts into HBM, and starts with an empty (cold) cache (the static policy
 * fills its resident slots here).
 * Passage: pirouter.ai "FreeToken × RTX 5090——120B MoE が 127 tok/s、その請求書",
 * section on how 65 GB runs on a 32 GB GPU (the bill-of-materials table and
 * the paragraph after it): every routed expert stays in host RAM as the
 * source of transfers, the GPU holds attention, router and shared weights
 * plus a cache of expert slots; blog.florigen.ai Qwen3.8-Flash-Next page,
 * model section: the shared expert runs for every token, so it is resident.
 * The pool is pinned (DMA-readable) memory as far as the platform allows and
 * cfg->pinned_mb permits; the rest is pageable and its misses are staged
 * through a ring of pinned bounce buffers.
 * slot_arena_dev (>= C blobs) and workspace_dev are device memory owned by the
 * caller; they and both streams must outlive the context.  The pool, the HBM
 * copies of router and shared experts, the cache state and the miss lists
 * are owned by the library and freed by moe_destroy.
 * Environment read here (debugging and failure injection):
 *   MOE_VERIFY=1 -- as MOE_FLAG_VERIFY;
 *   MOE_FAULT=h2d_fail_at=N -- the N-th miss copy of the context's life
 *     (1-based) is reported as a failed HIP call instead of being issued (the
 *     call returns MOE_EHIP and the context is failed);
 *   MOE_FAULT=h2d_corrupt_at=N -- the N-th miss copy moves the pool blob after
 *     the right one (caught by verify mode); items may be joined with ','.
 * Errors: MOE_EINVAL (shape, or a MOE_FAULT item it does not know),
 * MOE_ECAPACITY (cache_slots), MOE_ENOMEM (pinned pool, device state, or caller
 * buffers too small), MOE_EHIP.  On error *out is NULL and nothing is leaked. */
moe_status moe_init_pool(const moe_config* cfg, moe_fill_fn fill, void* user,
                         const uint16_t* router_w_bf16,
                         void* slot_arena_dev, size_t arena_bytes,
                         void* workspace_dev, size_t workspace_bytes,
                         void* compute_stream, void* copy_stream, moe_ctx** out);

/* Cache step for one layer with caller-given expert ids (ids_dev: [n_tokens][k]
 * int32, each in [0, E)): enqueues the resolve kernel on the compute stream,
 * waits for its miss list, issues one host-to-device copy per miss (alternating
 * between the caller's copy stream and a second, library-owned one) and makes
 * the compute stream wait for them.
 * Passage: ai-hardware-zukan.com "VRAMに収まらないMoEモデルのデコードが約2倍になった",
 * section on how misses are made up for: the cached unit is one (layer,
 * expert) pair, hits are served from VRAM, a miss is loaded into the slot of
 * the least recently used pair; gaming-st.com DeepSeek page, section on the
 * role of VRAM: one LRU cache over every layer's experts.  Within a step the
 * distinct requested experts are taken hits first, then misses, each by
 * ascending expert id; a miss takes the lowest empty slot, else the oldest.
 * slots_dev ([n_tokens][k] int32, may be NULL) receives the slot holding each
 * id; *n_miss_out (host, may be NULL) the number of misses.  `step` labels the
 * trace records.
 * Errors: MOE_EINVAL (layer, n_tokens, or any id outside [0, E): the whole step
 * is rejected before anything changes -- slot table, reverse map, stamps,
 * counters and trace stay as they were, slots_dev is all -1, and the context
 * stays usable), MOE_ESTATE, MOE_EHIP. */
moe_status moe_cache_resolve(moe_ctx* ctx, int32_t step, int32_t layer, const int32_t* ids_dev,
                             int32_t n_tokens, int32_t* slots_dev, int32_t* n_miss_out);

/* One layer for n_tokens tokens, causal: router (K1) -> top-k + resolve (K2)
 * -> miss copies -> expert FFN.  x_bf16_dev: [n_tokens][H]; y_bf16_dev: [n_tokens][H]
 * = sum_j w_j * FFN_{id_j}(x) + shared(x).  ids_dev_out ([n_tokens][k] int32,
 * ranked by logit) and w_dev_out ([n_tokens][k] float) may be NULL.
 * One token: per-token GEMV kernels (K3 gate/up, K4 down + combine).  Several
 * tokens (a prefill chunk, or decode requests in lock-step; pirouter.ai
 * "FreeToken x RTX 5090" page, expert-path section): the tokens' rows are
 * grouped by expert and run on the matrix cores, each expert's weights read
 * once per step (MOE_FLAG_PER_TOKEN_FFN: the GEMV kernels per token instead,
 * up to any n_tokens). */
moe_status moe_layer_forward(moe_ctx* ctx, int32_t step, int32_t layer, const void* x_bf16_dev,
                             int32_t n_tokens, void* y_bf16_dev, int32_t* ids_dev_out,
                             float* w_dev_out);

/* One decode step through all L layers with the configured lookahead.  Layer
 * l reads x_bf16_dev + l * x_layer_stride elements (stride 0: the same input
 * for every layer) and writes y_bf16_dev + l * y_layer_stride.  ids_dev_out
 * ([L][n_tokens][k]) and w_dev_out may be NULL.  Work is ordered on the
 * compute stream as seen by the caller.  One-token calls of the hybrid backend
 * that run one layer ahead, and one-token offload calls when the cache holds
 * the whole pool (C >= L * E), run the router and resolve on a library-owned
 * stream that joins the compute stream before the call returns; layer l+1's
 * copies then start only once layer l-1's FFN has ended, so the copies stay one
 * layer ahead.  In the whole-pool case the call also starts a helper host
 * thread that issues those launches and is joined before the call returns
 * (also on error).  Hybrid calls that run two or more layers ahead can return
 * while their queued host tasks still run (the FFNs that need them wait on the
 * compute stream); the tasks read the library's own host copy of x. */
moe_status moe_stack_forward(moe_ctx* ctx, int32_t step, const void* x_bf16_dev, int64_t x_layer_stride,
                             int32_t n_tokens, void* y_bf16_dev, int64_t y_layer_stride,
                             int32_t* ids_dev_out, float* w_dev_out);

/* Router logits of one layer.
 * Passage: pirouter.ai "FreeToken x RTX 5090 -- 120B MoE が 127 tok/s、その請求書", section on
 * the mechanism: the router picks the experts a token uses and the cache follows that choice.
 * The pages fix neither the logit precision nor the summation order; the library computes
 * z[t][e] = sum_i x[t][i] * W[e][i] in FP32 in one fixed order (element i goes to lane
 * (i / 8) mod 64, each lane adds its products in increasing i, then an xor butterfly over the
 * 64 lanes, d = 32, 16, ..., 1), the same kernels and bits behind the top-k of
 * moe_layer_forward and moe_stack_forward (one kernel up to 16 tokens, a tiled one above).
 * x_bf16_dev [n_tokens][H] bf16 (device); z_f32_dev_out [n_tokens][E] float (device, owned by
 * the caller), enqueued on the compute stream.  Nothing in the cache changes.
 * Errors: MOE_EINVAL (layer outside [0, L), NULL buffers, n_tokens outside [1, max_tokens]),
 * MOE_ESTATE (after a sticky failure), MOE_EHIP (launch failure). */
moe_status moe_router_logits(moe_ctx* ctx, int32_t layer, const void* x_bf16_dev, int32_t n_tokens,
                             float* z_f32_dev_out);

/* Expert FFN of one layer with caller-resolved slots (e.g. from moe_cache_resolve):
 * y = sum_j w_j * FFN(slot_j)(x) + shared(x), on the compute stream (the same
 * kernels as moe_layer_forward for that token count).  slots_dev [n_tokens][k]
 * int32 must name slots that hold this layer's experts (the library does not
 * check which expert a slot holds; a slot outside [0, C) is never read and
 * makes every output of its token NaN -- of every token with several tokens);
 * w_dev [n_tokens][k] float. */
moe_status moe_expert_forward(moe_ctx* ctx, int32_t layer, const void* x_bf16_dev, int32_t n_tokens,
                              const int32_t* slots_dev, const float* w_dev, void* y_bf16_dev);

/* Allocation-free variant of moe_expert_forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.  It needs
 * no context: the caller passes the shape (cfg: top_k, hidden, inter, n_shared, and cache_slots =
 * the number of blobs in slot_arena_dev; the other fields are not used), the slot arena (device,
 * [cache_slots][blob] in the pool's layout, e.g. the arena of a context), the shared expert's blob
 * (device, pool layout; NULL when n_shared = 0), x_bf16_dev [n_tokens][H], slots_dev and w_dev
 * [n_tokens][k] and y_bf16_dev [n_tokens][H], and the stream (hipStream_t as void*, NULL = the null
 * stream).  y = sum_j w_j * FFN(slot_j)(x) + shared(x) with the per-token GEMV kernels (as
 * moe_expert_forward of a context with MOE_FLAG_PER_TOKEN_FFN, bit for bit); a slot outside
 * [0, cache_slots) is never read and makes its token's outputs NaN.
 * The intermediate vectors (n_tokens * (k + n_shared) * inter bf16; at most 16 * 24576 * 2 bytes,
 * since the down kernel's LDS bounds (k + n_shared) * inter by 24576) live in a static device array
 * of MOE_NOALLOC_SCRATCH_BYTES (1 MiB) per GPU, held until the process ends; the call allocates and frees
 * nothing (its first call on a device looks the array's address up).  Every call on one GPU uses
 * the same array, so calls that overlap on one GPU (different streams, or host threads) race;
 * order them on one stream.  Errors (message: moe_last_error(NULL)): MOE_EINVAL (shape, null
 * buffer, n_tokens outside [1, MOE_NOALLOC_MAX_TOKENS], or intermediate vectors larger than the
 * array), MOE_EHIP (launch failure). */
#define MOE_NOALLOC_SCRATCH_BYTES (1u << 20)
#define MOE_NOALLOC_MAX_TOKENS 16
moe_status moe_expert_forward_noalloc(const moe_config* cfg, const void* slot_arena_dev, const void* shared_blob_dev,
                                      const void* x_bf16_dev, int32_t n_tokens, const int32_t* slots_dev,
                                      const float* w_dev, void* y_bf16_dev, void* stream);

typedef struct {
    uint64_t hits, misses, evictions;  /* cache accesses (unique (layer, expert) per step) */
    uint64_t resolves;                 /* layer steps resolved */
    uint64_t h2d_bytes, h2d_copies;    /* miss copies issued */
    uint64_t trace_records, trace_dropped;
    uint64_t ffn_launches;             /* with MOE_FLAG_PROFILE: timed layer FFNs */
    uint64_t h2d_bounced;              /* misses copied from the pageable part through the bounce ring */
    uint64_t pool_pinned_bytes;        /* bytes of the pool in pinned memory */
    double k3_ms, k4_ms;               /* ... summed durations of the FFN's first part (K3; grouped:
                                          grouping + gate/up) and second part (K4; grouped: down +
                                          combine), from HIP events */
    uint64_t host_experts;             /* hybrid backend: misses computed by the host (included in misses) */
    uint64_t host_tasks;               /* hybrid backend: layer steps with a host share */
    double host_busy_ms;               /* ... summed time from a host task's submission to its end */
    double host_wait_ms;               /* ... time the calling thread waited for host tasks */
    uint64_t h2d_ns;                   /* time the copy path was busy with the miss copies of the
                                          timed calls (one moe_stack_forward, moe_layer_forward or
                                          moe_cache_resolve call in 7, all its copies): per layer
                                          step and copy stream, first copy start to last copy end
                                          (GPU timestamps), merged over both copy streams */
    uint64_t ffn_ns, ffn_timed;        /* summed duration of the timed layer FFNs and their count: one
                                          layer FFN in 17 is timed (GPU timestamps around its
                                          launches, after its copy waits) */
    uint64_t h2d_timed_bytes;          /* bytes the copies of the timed calls moved:
                                          h2d_timed_bytes / h2d_ns is the copy path's rate while busy */
} moe_counters;

typedef struct {
    int32_t step, layer, expert, slot, hit, evicted_key; /* evicted_key = layer*E + expert, -1: none */
} moe_trace_rec;

/* Synchronises the compute and copy streams, then reports counters and drains
 * up to cap trace records (in order; the rest stay queued) into buf (host, may
 * be NULL with cap 0).  The counters are the quantities the pages report for
 * this path: the decode-time miss rate (ai-hardware-zukan.com page, section on
 * how misses are made up for: 16 % / 39 % with LRU against 62 % / 89 % with a
 * static split) and the expert transfer bandwidth (pirouter.ai page, section
 * on how 65 GB runs on a 32 GB GPU: 49.0 GB/s over PCIe 5.0 x16), here as
 * h2d_timed_bytes over h2d_ns.  Counters are cumulative over the context's life,
 * except k3_ms, k4_ms and ffn_launches (MOE_FLAG_PROFILE), which are harvested
 * and reset on every call. */
moe_status moe_stats(moe_ctx* ctx, moe_counters* out, moe_trace_rec* buf, size_t cap, size_t* n_out);

/* Host-to-device bandwidth of the copy path: n_copies back-to-back copies of
 * bytes_per_copy from blob-aligned offsets of the pinned part of the pool
 * (deterministic pseudo-random order) into a scratch device buffer, alternating
 * between the caller's copy stream and the library's second copy stream as the
 * miss stager does; returns GB/s (1e9).  Leaves the cache untouched. */
moe_status moe_measure_h2d(moe_ctx* ctx, size_t bytes_per_copy, int32_t n_copies, double* gbps_out);

/* Plain streaming read of device memory, the HBM counterpart of moe_measure_h2d:
 * one kernel launch on `stream` (a hipStream_t; NULL is the null stream) that
 * loads every 16-byte word of [buf_dev, buf_dev + bytes) once, with the same
 * nontemporal 16-byte loads as the expert FFN kernels, eight per lane, all in
 * flight at once, and keeps nothing but a sink word.  Timed over the byte counts
 * of the FFN's two kernels, it is the floor an HBM-bound launch of that size
 * reaches on this GPU, the reference for the FFN's own time.  The pages treat
 * VRAM as the fast side whose bandwidth serves the cache hits (pirouter.ai
 * "FreeToken × RTX 5090" page, section on how 65 GB runs on a 32 GB GPU:
 * 1-1.8 TB/s against PCIe's tens of GB/s).  buf_dev: device memory, 16-byte
 * aligned, owned by the caller; bytes: a multiple of 16.  No context; allocates
 * nothing; stream-ordered, so it can be captured in a graph.
 * Errors: MOE_EINVAL (null or unaligned buffer, bytes 0 or not a multiple of 16),
 * MOE_EHIP (launch). */
moe_status moe_hbm_read(const void* buf_dev, size_t bytes, void* stream);

/* Reads back the cache state (host buffers, each may be NULL): slot_of
 * [L*E], key_of [C], stamp [C].  Synchronises the compute stream. */
moe_status moe_cache_state(moe_ctx* ctx, int32_t* slot_of, int32_t* key_of, int64_t* stamp);

/* ---- backend calibration and the hybrid split ----
 * FreeToken's hybrid backend splits a step's m missing experts between PCIe
 * transfers and host-side computation so that both finish together; its auto
 * mode keeps the offload backend unless a stored bandwidth profile shows the
 * host expert kernel more than twice as fast as the PCIe transfers
 * (ai-hardware-zukan.com page, section on the hybrid mode; pirouter.ai page,
 * backend table).  B_P and B_H are measured with the real transfer path and
 * the real host kernel for the weight format. */
enum {
    MOE_BACKEND_OFFLOAD = 0, /* every miss crosses PCIe into a GPU slot (what moe_*_forward run) */
    MOE_BACKEND_HYBRID = 1,  /* part of the misses computed by the host kernel */
};

typedef struct {
    double pcie_gbps;      /* B_P: blob-sized copies from the pinned pool, GB/s */
    double host_gbps;      /* B_H: blob bytes per second through the host expert kernel */
    double ratio;          /* B_H / B_P */
    double threshold;      /* the ratio above which hybrid is recommended */
    int32_t host_threads;  /* threads the host kernel ran with */
    int32_t backend;       /* MOE_BACKEND_HYBRID iff ratio > threshold, else MOE_BACKEND_OFFLOAD */
    char host_isa[16];     /* instruction set of the host kernel: "avx512" or "scalar" */
} moe_bw_profile;

/* Measures B_P (moe_measure_h2d on >= 2 GB of blob-sized copies) and B_H (the
 * host expert kernel on host_threads threads for about host_seconds, over 64
 * blobs spread across the pool) and recommends a backend with the given
 * threshold (the pages' default is 2.0).  Leaves the cache untouched.
 * Errors: MOE_EINVAL (arguments), MOE_ESTATE, MOE_EHIP. */
moe_status moe_calibrate_backend(moe_ctx* ctx, int32_t host_threads, double host_seconds, double threshold,
                                 moe_bw_profile* out);

/* Selects the backend of the context's later decode steps.
 * MOE_BACKEND_OFFLOAD (default): every miss is transferred.
 * MOE_BACKEND_HYBRID: in a routed step of at most 16 tokens (moe_stack_forward
 *   or moe_layer_forward) the resolve kernel transfers only the first
 *   q = moe_hybrid_split(m, pcie_gbps, host_gbps) of the step's m distinct
 *   missing experts (ascending expert id) into cache slots; the other m - q
 *   take no slot, leave the cache unchanged (their trace records carry slot
 *   -1) and are computed by host_threads persistent host workers (the host
 *   expert kernel, work split over all workers), reading the pool, for every
 *   token of the step that selected them.  The FFN adds each token's host sum
 *   before rounding its output.  The tokens' hidden states are copied to the
 *   host once per call.  Steps of more tokens, steps run with
 *   MOE_FLAG_PER_TOKEN_FFN and more than one token, and moe_cache_resolve
 *   transfer every miss.  The workers spin between tasks and sleep after
 *   20 ms idle.  In moe_stack_forward calls that run D >= 2 layers ahead (see
 *   moe_config.lookahead) the host tasks are queued: a dispatcher thread runs
 *   them in layer order, and before each layer's FFN a one-wave kernel on the
 *   compute stream waits (at most about the library's 60 s limit, else the
 *   next call fails with MOE_EHIP) until that layer's task has finished, so
 *   host tasks and copies both run up to D layers ahead of the FFNs.
 * Needs the LRU policy.  Synchronises the compute stream.
 * Errors: MOE_EINVAL (backend, bandwidths <= 0, threads outside 1..256,
 * static policy), MOE_ENOMEM, MOE_ESTATE, MOE_EHIP. */
moe_status moe_set_backend(moe_ctx* ctx, int32_t backend, double pcie_gbps, double host_gbps, int32_t host_threads);

/* The auto rule: MOE_BACKEND_HYBRID when host_gbps > threshold * pcie_gbps
 * (and pcie_gbps > 0), else MOE_BACKEND_OFFLOAD.  Pure function. */
int32_t moe_select_backend(double pcie_gbps, double host_gbps, double threshold);

/* Transfers q of n_miss missing experts in the hybrid split (the rest go to the
 * host kernel): with the host's bandwidth left over during the DMA taken as
 * B_H - B_P, equal finishing times q / B_P = (n_miss - q) / (B_H - B_P) give
 * q = n_miss * B_P / B_H, rounded to nearest (halves up); all n_miss when
 * B_H <= B_P.  Pure function; 0 for n_miss <= 0. */
int32_t moe_hybrid_split(int32_t n_miss, double pcie_gbps, double host_gbps);

/* The host expert kernel: y[H] (FP32, host) = sum_j w[j] * FFN_j(x) over n
 * experts given as blobs in the pool's layout (host memory; moe_pack_blob
 * converts a logical blob), x[H] bf16 (host).  SwiGLU as on the GPU: FP32
 * accumulation, the intermediate vector rounded to bf16.  Experts are shared
 * out over `threads` host threads.  This is the kernel the calibration times
 * for B_H.  Needs no GPU.  Errors: MOE_EINVAL. */
moe_status moe_host_expert_ffn(const moe_config* cfg, const uint8_t* const* blobs, const float* w, int32_t n,
                               const uint16_t* x, float* y, int32_t threads);

/* The hybrid backend's host workers on one task, for callers and tests with no
 * GPU: for every token b < n_tok, y[b][H] (FP32, host) = the sum over the
 * entries j with tok[j] == b, in their order, of w[j] * FFN_j(x[b]), where
 * blobs[j] is an expert in the pool's layout (host memory) and x is bf16
 * [n_tok][H] (host); a token with no entry gets zeros.  The work runs on
 * `threads` persistent workers plus the calling thread (started and stopped
 * by the call), split into (token, block), (entry, gate/up tile), (entry,
 * intermediate block) and (token, output rows) units; every value is summed
 * by one thread in a fixed order, so y does not depend on `threads`.
 * n_tok in 1..16, n in 0..256, threads in 1..256.
 * Errors: MOE_EINVAL (arguments, tok[j] outside [0, n_tok)), MOE_ENOMEM. */
moe_status moe_host_expert_batch(const moe_config* cfg, int32_t n_tok, const uint16_t* x, float* y,
                                 const uint8_t* const* blobs, const float* w, const int32_t* tok, int32_t n,
                                 int32_t threads);

/* Converts one logical expert blob (gate codes, gate scales, up codes, up
 * scales, down codes, down scales; 3 * H * I * 17/32 bytes) into the pool's
 * layout (same size, a permutation of the bytes; packed != logical).  Needs no
 * GPU.  Errors: MOE_EINVAL. */
moe_status moe_pack_blob(const moe_config* cfg, const uint8_t* logical, uint8_t* packed);

/* Frees everything the context owns (after synchronising both streams).  NULL is a no-op. */
void moe_destroy(moe_ctx* ctx);
/* Text of the context's last error; with ctx = NULL, of the last failed call without a context
 * (moe_init_pool, moe_expert_forward_noalloc) on the calling thread.  Valid until the next call on
 * the same context / thread. */
const char* moe_last_error(const moe_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
