// Host orchestrator and C ABI (include/moe.h).
//
// Owns the pinned host pool of every routed expert (pirouter.ai "FreeToken x
// RTX 5090" page, section on how 65 GB runs on a 32 GB GPU: experts live in
// pinned, DMA-readable host RAM), the resident router weights and shared
// experts, the device cache state and the host-mapped miss lists.  Per layer
// step it launches the router (K1) and the resolve kernel (K2) on the compute
// stream, spins on the miss list K2 publishes in host-mapped memory, issues
// one hipMemcpyAsync per miss on the copy stream (misses stream over PCIe),
// and makes the compute stream wait for those copies before the expert-FFN
// kernel.  With lookahead 1 the next layer's K1/K2 and copies are issued
// before the current layer's FFN, so its misses load while the current layer
// computes (ai.holude.com preflight page, section on long prompts: the next
// layer's experts load over PCIe while the GPU computes the current one);
// lookahead D = 2 .. 7 resolves that many layers ahead, so the copy queue
// still holds layers of misses when layers without misses pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include <immintrin.h>

#include "../../include/moe.h"
#include "moe_internal.h"
#include "host_ffn.h"
#include "stager.h"

using namespace moe;

struct ProfSlot {
    hipEvent_t ev[3];
};

// a timed interval on the GPU: [ev[0], ev[1]] on one stream
struct TimedPair {
    hipEvent_t ev[2];
};

// Layer parities of the per-layer buffers (K2's slots and weights, miss lists, copy events): a
// lookahead-7 stack call has the buffers of layers l .. l+7 in use at once.
constexpr int NPAR = 8;

struct moe_ctx {
    moe_config cfg{};
    Layout lay{};
    int device = 0;
    int nE = 0;                 // k + n_shared
    hipStream_t cs = nullptr, ps = nullptr;
    // Router and resolve stream (library-owned) of one-token hybrid stack calls: K1/K2 of layer
    // l+1 run there, so a layer's miss list (the host workers' next task) does not wait behind an
    // FFN that waits for its copies.  Events order the rest: rs_start (call start on cs) before
    // the call's first K1; ffn_done[p] (on cs, after the FFN of the last layer of parity p) before
    // the copies that may overwrite that layer's slots (the copies of layer l+2); k2_done[p],
    // recorded only when needed, before an FFN that reads K2's slot and weight buffers (the
    // one-token FFN takes them as launch arguments instead); rs_end joins rs back into cs.
    hipStream_t rs = nullptr;
    hipEvent_t rs_start = nullptr, rs_end = nullptr;
    hipEvent_t k2_done[2] = {nullptr, nullptr};
    hipEvent_t ffn_done[2] = {nullptr, nullptr};
    bool ffn_done_valid[2] = {false, false};
    hipStream_t ks = nullptr;   // stream K1/K2 launch on: rs inside a route-stream call, else cs
    bool rs_active = false;     // the current call runs K1/K2 on rs
    std::mutex err_mu;          // set_err may run on a call's helper thread too
    bool rs_host_wait = false;  // ... and the host (not the copy streams) waits for ffn_done
    // The pool's L*E blobs are split between pinned memory (n_pin of them) and pageable memory.
    // Blob i is pinned iff pin_rank steps at i (pin_rank(i) = floor(i * n_pin / n_blobs)), so
    // the pinned ones are spread evenly over every layer's experts: a layer's misses mix pinned
    // blobs (DMA at once) with pageable ones (filled into a bounce slot by the host first), and
    // the pinned copies keep the link busy during those fills.  A pinned blob sits at
    // pinned index pin_rank(i), a pageable one at pageable index i - pin_rank(i).
    uint8_t* pool = nullptr;    // pinned host, n_pin blobs
    size_t pool_bytes = 0;      // whole pool
    size_t n_pin = 0;           // blobs in pinned memory
    size_t n_blobs = 0;         // L*E
    uint8_t* pool_pg = nullptr; // pageable host, n_blobs - n_pin blobs
    BounceRing bounce;          // pinned bounce ring for the pageable part
    size_t pin_rank(size_t i) const { return n_pin == n_blobs ? i : (size_t)((uint64_t)i * n_pin / n_blobs); }
    bool pinned(size_t i) const { return pin_rank(i + 1) > pin_rank(i); }
    const uint8_t* blob_src(size_t i) const {
        const size_t r = pin_rank(i);
        return pinned(i) ? pool + r * lay.blob_bytes : pool_pg + (i - r) * lay.blob_bytes;
    }
    uint8_t* arena = nullptr;   // caller device memory, [C][blob]
    uint8_t* shared_dev = nullptr;
    uint16_t* router_dev = nullptr;
    uint8_t* state_dev = nullptr;  // cache state block
    CacheDev cd{};
    int32_t* order[2] = {nullptr, nullptr};
    int parity = 0;             // which order buffer is current
    // workspace carve
    float* z = nullptr;
    // per layer parity (NPAR: layers l .. l+7 of a lookahead-7 call are in flight at once);
    // index NPAR of a and copy_used serves moe_expert_forward
    int32_t* ids[NPAR] = {};
    float* w[NPAR] = {};
    int32_t* slots[NPAR] = {};
    uint16_t* a[NPAR + 1] = {};
    GroupPlanDev gp{};          // grouped path (max_tokens > 1)
    uint16_t* yp = nullptr;     // bf16 expert outputs, one row per (token, expert)
    // host-mapped miss lists
    uint8_t* ml_mem = nullptr;
    size_t ml_stride = 0;
    uint64_t copy_rr = 0;  // pinned copies issued so far (all-pinned pools): picks their copy stream
    int max_unique = 0;
    int static_T = 0;           // static split: transient slots (2 * max distinct experts per step)
    int64_t seq = 0;
    hipEvent_t copy_ev[NPAR] = {};                  // per parity, on the caller's copy stream
    hipStream_t ps2 = nullptr;                      // second copy stream (library-owned)
    hipEvent_t copy_ev2[NPAR] = {};                 // per parity, on ps2
    bool copy_used[NPAR + 1][2] = {};               // per parity: copies went to ps / ps2
    // token 0's slots and weights of the last miss list read per parity
    int32_t tok0_slot[NPAR][16] = {};
    float tok0_w[NPAR][16] = {};
    bool tok0_valid[NPAR] = {};
    // host counters
    uint64_t h2d_bytes = 0, h2d_copies = 0, h2d_bounced = 0;
    uint64_t ffn_launches = 0;
    double k3_ms = 0, k4_ms = 0;
    std::vector<ProfSlot> prof_used, prof_free;
    // Copy-path busy time: one timed pair per copy stream and layer step with copies (before the
    // first copy, after the last); harvested into intervals on the GPU clock (relative to t_ref)
    // and merged, so copies overlapping on the two streams count once.
    hipEvent_t t_ref = nullptr;
    std::vector<TimedPair> h2d_used, h2d_free;
    std::vector<std::pair<double, double>> h2d_iv;   // harvested, not yet merged (ms from t_ref)
    double h2d_iv_end = -1.0;                        // end of the merged busy time so far (ms)
    double h2d_busy_ms = 0.0;
    uint64_t h2d_calls = 0, h2d_timed_bytes = 0;     // calls that stage misses; bytes of the timed copies
    bool h2d_timing = false;                         // the current call's copies are timed
    // Sampled FFN timing (every FFN_SAMPLE-th layer FFN; every one under MOE_FLAG_PROFILE)
    std::vector<TimedPair> ffn_used, ffn_free;
    uint64_t ffn_count = 0, ffn_timed = 0;
    double ffn_ms = 0.0;
    // Debug and failure injection (environment at init): MOE_FAULT=h2d_fail_at=N makes the N-th
    // host-to-device copy (1-based, over the context's life) fail as a HIP error would, before it
    // is issued; h2d_corrupt_at=N copies the wrong pool blob for the N-th copy.  MOE_VERIFY=1 (or
    // MOE_FLAG_VERIFY) reads back every filled slot once its copy has landed and compares it with
    // its pool blob.
    uint64_t fault_fail_at = 0, fault_corrupt_at = 0, copies_issued = 0;
    bool verify = false;
    std::vector<uint8_t> verify_buf;
    // hybrid backend: part of a step's misses (batches of at most 16 tokens) computed by host workers
    int backend = MOE_BACKEND_OFFLOAD;
    double hyb_bp = 0.0, hyb_bh = 0.0;   // B_P and B_H of the split
    HostExpertPool hpool;
    hipStream_t xs_stream = nullptr;     // device-to-host copies of the hidden states
    hipEvent_t xs_start = nullptr, xs_done = nullptr;
    uint16_t* xh = nullptr;              // pinned host copy of the call's hidden states (one of xh_buf)
    // two buffers used by calls in turn: host tasks a call queued may still read its buffer
    // while the next call fills the other
    uint16_t* xh_buf[2] = {nullptr, nullptr};
    size_t xh_cap_buf[2] = {0, 0};
    int xh_cur = 0;
    uint64_t xh_last_seq[2] = {0, 0};    // the last queued host task that reads each buffer
    int64_t xh_stride = 0;
    bool xh_pending = false;
    bool hyb_call = false;               // the current call runs hybrid steps
    int hyb_B = 0;                       // its token count
    float* yh = nullptr;                 // host-mapped [L][16][H]: the host experts' sums per layer and token
                                         // (a layer's own rows: its FFN may still be queued when the
                                         // host task of a later layer is submitted)
    bool host_has[2] = {false, false};   // this parity's FFN adds yh[parity]
    int host_running = -1;               // parity of the host task in flight, -1: none
    uint64_t host_tasks = 0;
    double host_wait_ms = 0.0;           // time the calling thread waited for host tasks
    // hybrid steps of a stack call with a lookahead of two or more layers queue their host tasks
    // here; before a layer's FFN a one-wave kernel on the compute stream waits until the queue's
    // count of finished tasks (mirrored in host-mapped memory) reaches that layer's task, so the
    // calling thread stages the next layers meanwhile
    HostTaskQueue hq;
    bool hq_mode = false;                // the current call queues its host tasks
    uint64_t host_seq[NPAR] = {};        // per parity: the queued task its FFN adds (0: none)
    uint64_t* hq_flag = nullptr;         // host-mapped: [0] finished tasks, [1] low word: a wait timed out
    uint64_t* hq_flag_dev = nullptr;     // its device address
    double spin_timeout_s = 60.0;
    bool failed = false;
    std::string err;
};

namespace {

// message of the last failed call without a context on this thread (moe_init_pool, whose context
// no longer exists, or moe_expert_forward_noalloc)
thread_local std::string g_init_err;

moe_status set_err(moe_ctx* c, moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (c) {
        std::lock_guard<std::mutex> lk(c->err_mu);
        c->err = buf;
        if (st == MOE_EHIP || st == MOE_EVERIFY) c->failed = true;
    }
    return st;
}

#define HIPCHK(ctx, call)                                                                    \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess)                                                                \
            return set_err((ctx), MOE_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

#define LAUNCHCHK(ctx, expr)                                                                            \
    do {                                                                                                \
        int e_ = (expr);                                                                                \
        if (e_ != 0)                                                                                    \
            return set_err((ctx), MOE_EHIP, "%s failed: %s", #expr, hipGetErrorString((hipError_t)e_)); \
    } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int MAX_CACHE_SLOTS = 32768;  // the resolve and grouping kernels' slot capacity
constexpr int MAX_EXPERTS = 1024;       // experts per layer the resolve kernel handles

// distinct experts one layer step can request; the cache needs twice that (one layer in flight
// while the next one's victims are chosen)
int64_t min_cache_slots(const moe_config* c) {
    return 2 * std::min<int64_t>((int64_t)c->max_tokens * c->top_k, c->n_experts);
}

// shape checks; cache_slots == 0 passes only when allow_auto (size queries before auto sizing)
moe_status check_cfg(const moe_config* c, bool allow_auto = false) {
    if (!c) return MOE_EINVAL;
    if (c->n_layers < 1 || c->n_experts < 1 || c->n_experts > MAX_EXPERTS || c->top_k < 1 ||
        c->top_k > 16 || c->top_k > c->n_experts || c->hidden < 32 || c->hidden % 32 ||
        c->hidden > 16384 || c->inter < 32 || c->inter % 32 || c->inter > 16384 ||
        c->n_shared < 0 || c->n_shared > 1 || c->max_tokens < 1 || c->cache_slots < 0 ||
        c->cache_slots > MAX_CACHE_SLOTS || c->lookahead < 0 || c->lookahead > 7 || c->trace_capacity < 0 ||
        c->pinned_mb < 0 || c->policy < 0 || c->policy > 1)
        return MOE_EINVAL;
    // the down kernel stages every selected expert's intermediate vector in LDS
    if ((size_t)(c->top_k + c->n_shared) * (c->inter / 32) * 80 > 60 * 1024) return MOE_EINVAL;
    if (c->cache_slots == 0 && allow_auto) return MOE_OK;
    if ((int64_t)c->cache_slots < min_cache_slots(c)) return MOE_ECAPACITY;
    return MOE_OK;
}

// device memory the library allocates itself: the cache state block (slot table, reverse map,
// stamps, clock, counters, trace head, double-buffered victim order, trace ring), the router
// weights and the shared experts
struct StatePlan {
    size_t slot, key, stamp, clock, cnt, th, ord, tr, total;
};

StatePlan plan_state(const moe_config& c, int C) {
    StatePlan p{};
    const size_t n_sl = (size_t)c.n_layers * c.n_experts;
    size_t off = 0;
    p.slot = off;  off = align_up(off + n_sl * 4, 256);
    p.key = off;   off = align_up(off + (size_t)C * 4, 256);
    p.stamp = off; off = align_up(off + (size_t)C * 8, 256);
    p.clock = off; off = align_up(off + 8, 256);
    p.cnt = off;   off = align_up(off + 8 * 8, 256);
    p.th = off;    off = align_up(off + 2 * 8, 256);
    p.ord = off;   off = align_up(off + 2 * (size_t)C * 4, 256);
    p.tr = off;    off = align_up(off + std::max<size_t>((size_t)c.trace_capacity, 1) * sizeof(TraceRec), 256);
    p.total = off;
    return p;
}

// the library's own device allocations at C slots, each rounded up to the allocator's 2 MiB
// granularity
size_t library_device_bytes(const moe_config& c, const Layout& L, int C) {
    const size_t g = (size_t)2 << 20;
    size_t b = align_up(plan_state(c, C).total, g);
    b += align_up((size_t)c.n_layers * c.n_experts * c.hidden * 2, g);
    if (c.n_shared > 0) b += align_up((size_t)c.n_layers * c.n_shared * L.blob_bytes, g);
    return b;
}

struct WsPlan {
    size_t z, ids, w, slots, a, grp, yp, total;
    int max_groups, max_chunks;
};

WsPlan plan_workspace(const moe_config& c) {
    WsPlan p{};
    const size_t B = (size_t)c.max_tokens, k = (size_t)c.top_k, E = (size_t)c.n_experts;
    const size_t nE = k + (size_t)c.n_shared;
    size_t off = 0;
    p.z = off;     off = align_up(off + B * E * 4, 256);
    p.ids = off;   off = align_up(off + NPAR * B * k * 4, 256);
    p.w = off;     off = align_up(off + NPAR * B * k * 4, 256);
    p.slots = off; off = align_up(off + NPAR * B * k * 4, 256);
    p.a = off;     off = align_up(off + (NPAR + 1) * B * nE * (size_t)c.inter * 2, 256);
    p.grp = p.yp = off;
    p.max_groups = p.max_chunks = 0;
    if (B > 1) {
        // grouped path: plan header, groups, chunks, row permutation, expert outputs
        // the chunk size depends on the call's token count: take the largest bound
        p.max_groups = grouped_max_groups((int)B, (int)k, (int)E, c.n_shared);
        for (int b : {(int)B, std::min((int)B, 16)})
            p.max_chunks = std::max(p.max_chunks, grouped_max_chunks(b, (int)k, (int)E, c.n_shared, grouped_gm(b)));
        p.grp = off;
        off = align_up(off + 4 * 4 + 3 * (size_t)p.max_groups * 4 + 2 * (size_t)p.max_chunks * 4 +
                           B * nE * 4, 256);
        p.yp = off;    off = align_up(off + B * nE * (size_t)c.hidden * 2, 256);
    }
    p.total = off;
    return p;
}

// logical blob -> kernel layout (see moe_internal.h)
void repack(const Layout& L, const uint8_t* src, uint8_t* dst) {
    const size_t HI = (size_t)L.H * L.I;
    const uint8_t* gc = src;
    const uint8_t* gs = gc + HI / 2;
    const uint8_t* uc = gs + HI / 32;
    const uint8_t* us = uc + HI / 2;
    const uint8_t* dc = us + HI / 32;
    const uint8_t* ds = dc + HI / 2;
    const int NB = L.NB, S = L.S3, NBI = L.NBI, GR = L.GR;
    for (int tile = 0; tile < L.I / GR; ++tile) {
        uint8_t* tb = dst + (size_t)tile * L.gu_tile_bytes;
        uint8_t* tub = tb + (size_t)GR * NB * 16;
        uint8_t* tsc = tb + (size_t)GR * NB * 32;
        for (int s = 0; s < S; ++s) {
            const int nb = seg_len(NB, S, s), b0 = seg_begin(NB, S, s);
            for (int t = 0; t < nb; ++t) {
                for (int r = 0; r < GR; ++r) {
                    const size_t row = (size_t)tile * GR + r;
                    const int blk = b0 + t;
                    const size_t c = (size_t)(t * S + s) * GR + r;
                    memcpy(tb + c * 16, gc + row * (L.H / 2) + (size_t)blk * 16, 16);
                    memcpy(tub + c * 16, uc + row * (L.H / 2) + (size_t)blk * 16, 16);
                    tsc[c * 2] = gs[row * NB + blk];
                    tsc[c * 2 + 1] = us[row * NB + blk];
                }
            }
        }
    }
    uint8_t* dcd = dst + L.d_codes_off;
    uint8_t* dsd = dst + L.d_scales_off;
    for (int t8 = 0; t8 < L.H / 8; ++t8)
        for (int ib = 0; ib < NBI; ++ib)
            for (int r = 0; r < 8; ++r) {
                const size_t h = (size_t)t8 * 8 + r;
                const size_t cell = ((size_t)t8 * NBI + ib) * 8 + r;
                memcpy(dcd + cell * 16, dc + h * (L.I / 2) + (size_t)ib * 16, 16);
                dsd[cell] = ds[h * NBI + ib];
            }
}

MissList* miss_list(moe_ctx* c, int parity) {
    return reinterpret_cast<MissList*>(c->ml_mem + (size_t)parity * c->ml_stride);
}

void free_all(moe_ctx* c) {
    if (!c) return;
    if (c->cs) (void)hipStreamSynchronize(c->cs);
    if (c->ps) (void)hipStreamSynchronize(c->ps);
    if (c->ps2) (void)hipStreamSynchronize(c->ps2);
    if (c->rs) (void)hipStreamSynchronize(c->rs);
    for (auto e : {c->rs_start, c->rs_end, c->k2_done[0], c->k2_done[1], c->ffn_done[0], c->ffn_done[1]})
        if (e) (void)hipEventDestroy(e);
    if (c->rs) (void)hipStreamDestroy(c->rs);
    for (auto& p : c->prof_used) for (auto e : p.ev) (void)hipEventDestroy(e);
    for (auto& p : c->prof_free) for (auto e : p.ev) (void)hipEventDestroy(e);
    for (auto* v : {&c->h2d_used, &c->h2d_free, &c->ffn_used, &c->ffn_free})
        for (auto& p : *v) for (auto e : p.ev) (void)hipEventDestroy(e);
    if (c->t_ref) (void)hipEventDestroy(c->t_ref);
    for (auto e : c->copy_ev) if (e) (void)hipEventDestroy(e);
    for (auto e : c->copy_ev2) if (e) (void)hipEventDestroy(e);
    if (c->ps2) (void)hipStreamDestroy(c->ps2);
    c->hq.stop();
    c->hpool.stop();
    if (c->hq_flag) (void)hipHostFree(c->hq_flag);
    if (c->xs_stream) (void)hipStreamSynchronize(c->xs_stream);
    if (c->xs_start) (void)hipEventDestroy(c->xs_start);
    if (c->xs_done) (void)hipEventDestroy(c->xs_done);
    if (c->xs_stream) (void)hipStreamDestroy(c->xs_stream);
    for (auto* b : c->xh_buf)
        if (b) (void)hipHostFree(b);
    if (c->yh) (void)hipHostFree(c->yh);
    c->bounce.shutdown();
    if (c->pool) (void)hipHostFree(c->pool);
    free(c->pool_pg);
    if (c->ml_mem) (void)hipHostFree(c->ml_mem);
    if (c->shared_dev) (void)hipFree(c->shared_dev);
    if (c->router_dev) (void)hipFree(c->router_dev);
    if (c->state_dev) (void)hipFree(c->state_dev);
    delete c;
}

// ---------------------------------------------------------- one layer step --

moe_status launch_route(moe_ctx* c, int layer, const void* x, int B) {
    K1Args a{};
    a.W = c->router_dev + (size_t)layer * c->cfg.n_experts * c->cfg.hidden;
    a.x = (const uint16_t*)x;
    a.z = c->z;
    a.E = c->cfg.n_experts;
    a.H = c->cfg.hidden;
    a.B = B;
    LAUNCHCHK(c, launch_k1(a, c->ks ? c->ks : c->cs));
    return MOE_OK;
}

// K2 for one layer step.  routed: top-k of the logits K1 left in z for B
// tokens, then resolve; otherwise resolve the caller's ids (n_ids of them).
moe_status launch_resolve(moe_ctx* c, int step, int layer, bool routed, const int32_t* ids, int B,
                          int par, int32_t* slots_out, int32_t* ids_out, float* w_out) {
    K2Args a{};
    a.c = c->cd;
    a.z = routed ? c->z : nullptr;
    a.ids = routed ? c->ids[par] : const_cast<int32_t*>(ids);
    a.w = c->w[par];
    a.ids_out = ids_out;
    a.w_out = w_out;
    a.slots = c->slots[par];
    a.slots_out = slots_out;
    a.ml = miss_list(c, par);
    a.seq = ++c->seq;
    a.n_ids = B * c->cfg.top_k;
    a.layer = layer;
    a.step = step;
    a.E = c->cfg.n_experts;
    a.C = c->cfg.cache_slots;
    a.k = c->cfg.top_k;
    a.B = B;
    a.policy = c->cfg.policy;
    a.T = c->static_T;
    a.R = c->cfg.cache_slots - c->static_T;
    a.hybrid = (c->hyb_call && routed && B <= kHostMaxTokens) ? 1 : 0;
    a.bp = c->hyb_bp;
    a.bh = c->hyb_bh;
    const int p = c->parity;
    LAUNCHCHK(c, launch_k2(a, c->order[p], c->order[p ^ 1], c->ks ? c->ks : c->cs));
    c->parity = p ^ 1;
    return MOE_OK;
}

// Hybrid steps need the tokens' hidden states on the host: one device-to-host
// copy per call of the `layers` [B][H] blocks at stride xs (elements), ordered
// after everything already on the compute stream.  Calls of at most 16 tokens
// with the LRU policy run hybrid steps (batches through the grouped FFN path).
moe_status hyb_begin(moe_ctx* c, const void* x, int64_t xs, int layers, int B) {
    c->hyb_call = false;
    c->hq_mode = false;
    for (auto& q : c->host_seq) q = 0;
    // a call that returned early can leave a host task running or a host sum unclaimed
    if (c->host_running >= 0) {
        c->hpool.wait();
        c->host_running = -1;
    }
    c->host_has[0] = c->host_has[1] = false;
    if (c->backend != MOE_BACKEND_HYBRID || B > kHostMaxTokens || c->cfg.policy != MOE_POLICY_LRU || xs < 0 ||
        (B > 1 && (c->cfg.flags & MOE_FLAG_PER_TOKEN_FFN)))
        return MOE_OK;
    const size_t bytes = ((size_t)(layers - 1) * (size_t)xs + (size_t)B * c->cfg.hidden) * 2;
    const int i = c->xh_cur ^ 1;
    if (c->xh_last_seq[i] && !c->hq.wait(c->xh_last_seq[i], c->spin_timeout_s))
        return set_err(c, MOE_EHIP, "timed out waiting for the host tasks of an earlier call");
    c->xh_last_seq[i] = 0;
    if (bytes > c->xh_cap_buf[i]) {
        if (c->xh_buf[i]) HIPCHK(c, hipHostFree(c->xh_buf[i]));
        c->xh_buf[i] = nullptr;
        c->xh_cap_buf[i] = 0;
        if (hipHostMalloc((void**)&c->xh_buf[i], bytes, 0) != hipSuccess)
            return set_err(c, MOE_ENOMEM, "pinned buffer of %zu bytes for the hidden states", bytes);
        c->xh_cap_buf[i] = bytes;
    }
    c->xh_cur = i;
    c->xh = c->xh_buf[i];
    HIPCHK(c, hipEventRecord(c->xs_start, c->cs));
    HIPCHK(c, hipStreamWaitEvent(c->xs_stream, c->xs_start, 0));
    HIPCHK(c, hipMemcpyAsync(c->xh, x, bytes, hipMemcpyDeviceToHost, c->xs_stream));
    HIPCHK(c, hipEventRecord(c->xs_done, c->xs_stream));
    c->xh_pending = true;
    c->xh_stride = xs;
    c->hyb_call = true;
    c->hyb_B = B;
    return MOE_OK;
}

moe_status get_pair(moe_ctx* c, std::vector<TimedPair>& free_list, TimedPair& p) {
    if (!free_list.empty()) {
        p = free_list.back();
        free_list.pop_back();
        return MOE_OK;
    }
    p.ev[0] = p.ev[1] = nullptr;
    for (auto& e : p.ev)
        if (hipEventCreate(&e) != hipSuccess) {
            for (auto& f : p.ev)
                if (f) (void)hipEventDestroy(f);
            return set_err(c, MOE_EHIP, "timing event creation failed");
        }
    return MOE_OK;
}

// Sampling of the GPU-timed counters (two event records each, a few µs of host time, so not on
// every layer step): one layer FFN in FFN_SAMPLE (co-prime with the workloads' layer counts, so
// every layer is sampled), and every copy of one call in H2D_SAMPLE (moe_stack_forward,
// moe_layer_forward and moe_cache_resolve calls; whole calls, so that the union of the timed
// intervals carries no bytes of untimed copies, apart from the few that overlap the first and
// last layer steps of a call)
constexpr int FFN_SAMPLE = 17;
constexpr int H2D_SAMPLE = 7;
constexpr size_t TIMED_PENDING = 256;   // timed pairs kept before the oldest finished ones are harvested

// Copy-path busy time: intervals of the finished timed pairs (all of them when `all`, which
// waits), merged into the running union of busy time.  An interval's start is read against
// t_ref and its length from its own two events (float milliseconds lose precision far from
// t_ref; the length stays exact).
moe_status harvest_h2d(moe_ctx* c, bool all) {
    size_t n = 0;
    for (; n < c->h2d_used.size(); ++n) {
        TimedPair& p = c->h2d_used[n];
        if (!all && hipEventQuery(p.ev[1]) != hipSuccess) break;
        float t0 = 0.0f, len = 0.0f;
        HIPCHK(c, hipEventSynchronize(p.ev[1]));
        HIPCHK(c, hipEventElapsedTime(&t0, c->t_ref, p.ev[0]));
        HIPCHK(c, hipEventElapsedTime(&len, p.ev[0], p.ev[1]));
        c->h2d_iv.emplace_back((double)t0, (double)t0 + (double)len);
        c->h2d_free.push_back(p);
    }
    (void)hipGetLastError();  // a not-ready query is not an error
    c->h2d_used.erase(c->h2d_used.begin(), c->h2d_used.begin() + (ptrdiff_t)n);
    std::sort(c->h2d_iv.begin(), c->h2d_iv.end());
    for (const auto& iv : c->h2d_iv) {
        if (iv.first >= c->h2d_iv_end) {
            c->h2d_busy_ms += iv.second - iv.first;
            c->h2d_iv_end = iv.second;
        } else if (iv.second > c->h2d_iv_end) {
            c->h2d_busy_ms += iv.second - c->h2d_iv_end;
            c->h2d_iv_end = iv.second;
        }
    }
    c->h2d_iv.clear();
    return MOE_OK;
}

// sampled FFN times of the finished timed pairs (all of them when `all`, which waits)
moe_status harvest_ffn(moe_ctx* c, bool all) {
    size_t n = 0;
    for (; n < c->ffn_used.size(); ++n) {
        TimedPair& p = c->ffn_used[n];
        if (!all && hipEventQuery(p.ev[1]) != hipSuccess) break;
        float ms = 0.0f;
        HIPCHK(c, hipEventSynchronize(p.ev[1]));
        HIPCHK(c, hipEventElapsedTime(&ms, p.ev[0], p.ev[1]));
        c->ffn_ms += ms;
        ++c->ffn_timed;
        c->ffn_free.push_back(p);
    }
    (void)hipGetLastError();
    c->ffn_used.erase(c->ffn_used.begin(), c->ffn_used.begin() + (ptrdiff_t)n);
    return MOE_OK;
}

// Waits for the miss list of resolve `seq` and issues its copies; records
// copy_ev[par] when there are misses.  n_miss_out gets the count.
moe_status stage_misses(moe_ctx* c, int layer, int par, int64_t seq, int* n_miss_out) {
    c->tok0_valid[par] = false;
    MissList* ml = miss_list(c, par);
    auto t0 = std::chrono::steady_clock::now();
    uint64_t spins = 0;
    while (__atomic_load_n(&ml->seq, __ATOMIC_ACQUIRE) != seq) {
        _mm_pause();
        if ((++spins & 0xFFFF) == 0) {
            // the resolve runs on the compute stream, or on the route stream of a route-stream call
            for (hipStream_t sq : {c->cs, c->ks}) {
                if (!sq) continue;
                hipError_t q = hipStreamQuery(sq);
                if (q != hipSuccess && q != hipErrorNotReady)
                    return set_err(c, MOE_EHIP, "%s stream failed while waiting for a miss list: %s",
                                   sq == c->cs ? "compute" : "route", hipGetErrorString(q));
            }
            double dt = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
            if (dt > c->spin_timeout_s)
                return set_err(c, MOE_EHIP, "timed out waiting for the miss list of layer %d", layer);
        }
    }
    const int nm = ml->n_miss;
    const int nx = ml->n_xfer;
    if (ml->n_invalid) return set_err(c, MOE_EINVAL, "%d expert ids outside [0, E)", ml->n_invalid);
    for (int j = 0; j < c->cfg.top_k; ++j) {
        c->tok0_slot[par][j] = ml->slot0[j];
        c->tok0_w[par][j] = ml->w0[j];
    }
    c->tok0_valid[par] = true;
    if (nx < nm) {
        // hybrid step: the experts without a slot run on the host workers, for every
        // token that selected them, in rank order
        if (!c->hyb_call || !c->hpool.running())
            return set_err(c, MOE_EINVAL, "host share in a step that is not hybrid");
        if (c->xh_pending) {
            HIPCHK(c, hipEventSynchronize(c->xs_done));
            c->xh_pending = false;
        }
        const int B = c->hyb_B, k = c->cfg.top_k, E = c->cfg.n_experts;
        HostEntry ent[kHostMaxEntries];
        int nh = 0;
        if (B == 1) {
            for (int j = 0; j < k; ++j)
                if (ml->slot0[j] < 0)
                    ent[nh++] = {c->blob_src((size_t)layer * E + ml->ids0[j]), ml->w0[j], 0};
        } else {
            uint64_t host_set[(MAX_EXPERTS + 63) / 64] = {};
            for (int i = nx; i < nm; ++i) {
                const int e = ml->e[i].expert;
                host_set[e >> 6] |= 1ull << (e & 63);
            }
            for (int i = 0; i < B * k; ++i) {
                const int e = ml->ids_all[i];
                if ((unsigned)e < (unsigned)E && ((host_set[e >> 6] >> (e & 63)) & 1ull))
                    ent[nh++] = {c->blob_src((size_t)layer * E + e), ml->w_all[i], i / k};
            }
        }
        const uint16_t* xs[kHostMaxTokens];
        float* ys[kHostMaxTokens];
        const size_t H = c->cfg.hidden;
        for (int b = 0; b < B; ++b) {
            xs[b] = c->xh + (size_t)layer * c->xh_stride + (size_t)b * H;
            ys[b] = c->yh + ((size_t)layer * kHostMaxTokens + b) * H;
        }
        if (c->hq_mode) {
            // queued: the dispatcher runs it after the tasks before it; the FFN waits for it
            const uint64_t sq = c->hq.push(c->lay, B, xs, ys, ent, nh);
            c->host_seq[par] = sq;
            c->xh_last_seq[c->xh_cur] = sq;
        } else {
            // the pool is used directly: tasks still queued by an earlier call finish first
            if (c->hq.done() < c->hq.pushed() && !c->hq.wait(c->hq.pushed(), c->spin_timeout_s))
                return set_err(c, MOE_EHIP, "timed out waiting for queued host tasks");
            if (c->host_running >= 0) {
                // one task at a time: the previous layer's host experts finish first (their sums
                // stay in their own parity's buffers for that layer's FFN)
                const auto tw = std::chrono::steady_clock::now();
                c->hpool.wait();
                c->host_wait_ms +=
                    std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - tw).count();
                c->host_running = -1;
            }
            c->hpool.submit(c->lay, B, xs, ys, ent, nh);
            c->host_running = par;
            c->host_has[par] = true;
        }
        ++c->host_tasks;
    }
    const size_t blob = c->lay.blob_bytes;
    if (c->rs_active && nx > 0 && c->ffn_done_valid[par]) {
        // this step's victims may hold the slots of the layer two back (same parity), whose FFN
        // runs on the compute stream while this step was resolved on the route stream; its end
        // also bounds the copies to one layer ahead of compute
        if (c->rs_host_wait) {
            // offload steps: the host waits and then issues the copies, so the copy queues
            // carry no cross-stream wait
            auto tw = std::chrono::steady_clock::now();
            uint64_t spins = 0;
            for (;;) {
                const hipError_t q = hipEventQuery(c->ffn_done[par]);
                if (q == hipSuccess) break;
                if (q != hipErrorNotReady)
                    return set_err(c, MOE_EHIP, "FFN event failed while staging layer %d: %s", layer,
                                   hipGetErrorString(q));
                _mm_pause();
                if ((++spins & 0xFFF) == 0 &&
                    std::chrono::duration<double>(std::chrono::steady_clock::now() - tw).count() > c->spin_timeout_s)
                    return set_err(c, MOE_EHIP, "timed out waiting for the FFN two layers before layer %d", layer);
            }
        } else {
            HIPCHK(c, hipStreamWaitEvent(c->ps, c->ffn_done[par], 0));
            HIPCHK(c, hipStreamWaitEvent(c->ps2, c->ffn_done[par], 0));
        }
    }
    bool used[2] = {false, false}, timed_q[2] = {false, false};
    hipStream_t qs[2] = {c->ps, c->ps2};
    int ncopy = 0;
    const bool timed = nm > 0 && c->h2d_timing;
    if (c->h2d_used.size() >= TIMED_PENDING) {
        moe_status st = harvest_h2d(c, false);
        if (st) return st;
    }
    size_t pair_of[2] = {0, 0};
    // the first copy on a stream marks it used and, in a sampled step, opens its timed interval
    // (the pair goes to the pending list at once, so an error return leaks nothing; the context
    // is failed then anyway)
    auto open_stream = [&](int q) -> moe_status {
        if (used[q]) return MOE_OK;
        used[q] = true;
        if (!timed) return MOE_OK;
        TimedPair tp{};
        moe_status st = get_pair(c, c->h2d_free, tp);
        if (st) return st;
        if (hipEventRecord(tp.ev[0], qs[q]) != hipSuccess) {
            c->h2d_free.push_back(tp);
            return set_err(c, MOE_EHIP, "copy timing event record failed");
        }
        c->h2d_used.push_back(tp);
        pair_of[q] = c->h2d_used.size() - 1;
        timed_q[q] = true;
        return MOE_OK;
    };
    // pass 0 queues the misses whose blobs are pinned (their DMA starts at once), pass 1 the
    // pageable ones: the host fills each of those into a bounce slot before its DMA, at about the
    // DMA's own rate, so the pinned copies queued ahead keep the link busy during the fills
    for (int pass = 0; pass < 2; ++pass)
    for (int i = 0; i < nm; ++i) {
        const MissEntry m = ml->e[i];
        if (m.slot < 0) continue;  // computed by the host
        const size_t idx = (size_t)layer * c->cfg.n_experts + m.expert;
        if (c->pinned(idx) != (pass == 0)) continue;
        ++ncopy;
        uint8_t* dst = c->arena + (size_t)m.slot * blob;
        ++c->copies_issued;
        if (c->fault_fail_at && c->copies_issued == c->fault_fail_at)
            return set_err(c, MOE_EHIP, "injected failure of host-to-device copy %llu (MOE_FAULT), layer %d expert %d",
                           (unsigned long long)c->copies_issued, layer, m.expert);
        const size_t n_sl = (size_t)c->cfg.n_layers * c->cfg.n_experts;
        const size_t src_idx = (c->fault_corrupt_at && c->copies_issued == c->fault_corrupt_at) ? (idx + 1) % n_sl : idx;
        // a pool with a pageable part: pageable misses on the caller's copy stream (each DMA waits
        // for its host fill), pinned ones on the second stream, where they run while the fills
        // hold the first; an all-pinned pool alternates its copies over both streams, counted
        // across calls, so that steps with one miss each do not all queue on the first
        const int q = !c->pinned(idx) ? 0 : (c->n_pin < c->n_blobs ? 1 : (int)(c->copy_rr++ & 1));
        if (!used[q]) {
            moe_status st = open_stream(q);
            if (st) return st;
        }
        if (c->pinned(idx)) {
            HIPCHK(c, hipMemcpyAsync(dst, c->blob_src(src_idx), blob, hipMemcpyHostToDevice, qs[q]));
        } else {
            HIPCHK(c, c->bounce.copy(dst, c->blob_src(src_idx), blob));  // on the caller's copy stream
            ++c->h2d_bounced;
        }
    }
    for (int q = 0; q < 2; ++q)
        if (timed_q[q]) HIPCHK(c, hipEventRecord(c->h2d_used[pair_of[q]].ev[1], qs[q]));
    if (timed) c->h2d_timed_bytes += (uint64_t)ncopy * blob;
    if (used[0]) HIPCHK(c, hipEventRecord(c->copy_ev[par], c->ps));
    if (used[1]) HIPCHK(c, hipEventRecord(c->copy_ev2[par], c->ps2));
    c->copy_used[par][0] = used[0];
    c->copy_used[par][1] = used[1];
    c->h2d_bytes += (uint64_t)ncopy * blob;
    c->h2d_copies += (uint64_t)ncopy;
    if (n_miss_out) *n_miss_out = ncopy;
    if (c->verify && ncopy > 0) {
        // debug mode: once this step's copies have landed, every filled slot must hold its pool blob
        HIPCHK(c, hipStreamSynchronize(c->ps));
        HIPCHK(c, hipStreamSynchronize(c->ps2));
        if (c->verify_buf.size() != blob) c->verify_buf.assign(blob, 0);
        for (int i = 0; i < nm; ++i) {
            const MissEntry m = ml->e[i];
            if (m.slot < 0) continue;
            const size_t idx = (size_t)layer * c->cfg.n_experts + m.expert;
            HIPCHK(c, hipMemcpy(c->verify_buf.data(), c->arena + (size_t)m.slot * blob, blob, hipMemcpyDeviceToHost));
            if (memcmp(c->verify_buf.data(), c->blob_src(idx), blob) != 0)
                return set_err(c, MOE_EVERIFY, "slot %d (layer %d, expert %d) differs from its pool blob after its copy",
                               m.slot, layer, m.expert);
        }
    }
    return MOE_OK;
}

moe_status get_prof(moe_ctx* c, ProfSlot& p) {
    if (!c->prof_free.empty()) {
        p = c->prof_free.back();
        c->prof_free.pop_back();
        return MOE_OK;
    }
    for (auto& e : p.ev) HIPCHK(c, hipEventCreate(&e));
    return MOE_OK;
}

moe_status launch_ffn_layer(moe_ctx* c, int layer, const void* x, int B, int par, void* y, int n_miss,
                            const int32_t* slots_dev = nullptr, const float* w_dev = nullptr) {
    const float* yh = nullptr;
    if (par < 2 && c->host_has[par]) {
        // the host experts of this step: their sum is added by the down kernel
        if (c->host_running == par) {
            const auto tw = std::chrono::steady_clock::now();
            c->hpool.wait();
            c->host_wait_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - tw).count();
            c->host_running = -1;
        }
        c->host_has[par] = false;
        yh = c->yh + (size_t)layer * kHostMaxTokens * c->cfg.hidden;
    }
    if (par < NPAR && c->host_seq[par]) {
        // a queued host task: the compute stream waits for it (the calling thread does not); the
        // wait reads the count about every 2 us or more, so max_polls covers the time limit
        const double polls = std::min(4.0e9, c->spin_timeout_s * 5.0e5);
        if (launch_wait_host(c->hq_flag_dev, c->host_seq[par], (uint32_t)polls,
                             reinterpret_cast<uint32_t*>(c->hq_flag_dev + 1), c->cs) != (int)hipSuccess)
            return set_err(c, MOE_EHIP, "launch of the host-task wait failed");
        c->host_seq[par] = 0;
        yh = c->yh + (size_t)layer * kHostMaxTokens * c->cfg.hidden;
    }
    if (n_miss > 0 && par < NPAR) {
        if (c->copy_used[par][0]) HIPCHK(c, hipStreamWaitEvent(c->cs, c->copy_ev[par], 0));
        if (c->copy_used[par][1]) HIPCHK(c, hipStreamWaitEvent(c->cs, c->copy_ev2[par], 0));
    }
    // the single-token kernels take their slots and weights as launch arguments; any other FFN
    // reads the ones K2 wrote, on the route stream in a route-stream call: it waits for all the
    // route stream holds so far (which includes that K2)
    if (c->rs_active && par < 2 && !(B == 1 && !slots_dev && c->tok0_valid[par])) {
        HIPCHK(c, hipEventRecord(c->k2_done[par], c->rs));
        HIPCHK(c, hipStreamWaitEvent(c->cs, c->k2_done[par], 0));
    }
    const bool prof = (c->cfg.flags & MOE_FLAG_PROFILE) != 0;
    ProfSlot ps{};
    if (prof) {
        moe_status st = get_prof(c, ps);
        if (st) return st;
        HIPCHK(c, hipEventRecord(ps.ev[0], c->cs));
    }
    // every FFN_SAMPLE-th layer FFN is timed (on the compute stream, after its copy waits)
    const bool sampled = !prof && (c->ffn_count++ % FFN_SAMPLE) == 0;
    TimedPair tp{};
    if (sampled) {
        if (c->ffn_used.size() >= TIMED_PENDING) {
            moe_status st = harvest_ffn(c, false);
            if (st) return st;
        }
        moe_status st = get_pair(c, c->ffn_free, tp);
        if (st) return st;
        if (hipEventRecord(tp.ev[0], c->cs) != hipSuccess) {
            c->ffn_free.push_back(tp);
            return set_err(c, MOE_EHIP, "FFN timing event record failed");
        }
        c->ffn_used.push_back(tp);  // its end is recorded after the launches (destroyed with the context on error)
    }
    if (B > 1 && !(c->cfg.flags & MOE_FLAG_PER_TOKEN_FFN)) {
        GroupArgs g{};
        g.p = c->gp;
        g.slots = slots_dev ? slots_dev : c->slots[par];
        g.B = B;
        g.k = c->cfg.top_k;
        g.C = c->cfg.cache_slots;
        g.n_shared = c->cfg.n_shared;
        g.gm = grouped_gm(B);
        g.host_rows = yh ? 1 : 0;
        g.p.max_groups = grouped_max_groups(B, c->cfg.top_k, c->cfg.n_experts, c->cfg.n_shared);
        g.p.max_chunks = grouped_max_chunks(B, c->cfg.top_k, c->cfg.n_experts, c->cfg.n_shared, g.gm);
        GemmArgs m{};
        m.p = g.p;
        m.arena = c->arena;
        m.shared = c->shared_dev;
        m.x = (const uint16_t*)x;
        m.a = c->a[par];
        m.yp = c->yp;
        m.blob_bytes = c->lay.blob_bytes;
        m.d_codes_off = c->lay.d_codes_off;
        m.d_scales_off = c->lay.d_scales_off;
        m.B = B;
        m.k = c->cfg.top_k;
        m.n_shared = c->cfg.n_shared;
        m.layer = layer;
        m.H = c->cfg.hidden;
        m.I = c->cfg.inter;
        m.NB = c->lay.NB;
        m.NBI = c->lay.NBI;
        m.gm = g.gm;
        CombineArgs cb{};
        cb.yp = c->yp;
        cb.w = w_dev ? w_dev : c->w[par];
        cb.slots = g.slots;
        cb.y = (uint16_t*)y;
        cb.B = B;
        cb.k = c->cfg.top_k;
        cb.n_shared = c->cfg.n_shared;
        cb.H = c->cfg.hidden;
        cb.C = c->cfg.cache_slots;
        cb.yh = yh;
        cb.host_rows = yh ? 1 : 0;
        LAUNCHCHK(c, launch_grouped_ffn(g, m, cb, c->cs, prof ? ps.ev[1] : nullptr));
    } else {
    FfnArgs f{};
    f.arena = c->arena;
    f.shared = c->shared_dev;
    f.slots = slots_dev ? slots_dev : c->slots[par];
    f.w = w_dev ? w_dev : c->w[par];
    f.x = (const uint16_t*)x;
    f.a = c->a[par];
    f.y = (uint16_t*)y;
    f.blob_bytes = c->lay.blob_bytes;
    f.d_codes_off = c->lay.d_codes_off;
    f.d_scales_off = c->lay.d_scales_off;
    f.k = c->cfg.top_k;
    f.n_shared = c->cfg.n_shared;
    f.nE = c->nE;
    f.layer = layer;
    f.NB = c->lay.NB;
    f.NBI = c->lay.NBI;
    f.I = c->cfg.inter;
    f.H = c->cfg.hidden;
    f.C = c->cfg.cache_slots;
    f.karg = (B == 1 && !slots_dev && par < NPAR && c->tok0_valid[par]) ? 1 : 0;
    if (f.karg) {
        // the experts in GPU slots, in rank order (hybrid steps leave some to the host)
        int kk = 0;
        for (int j = 0; j < c->cfg.top_k; ++j)
            if (c->tok0_slot[par][j] >= 0) {
                f.kslot[kk] = c->tok0_slot[par][j];
                f.kw[kk++] = c->tok0_w[par][j];
            }
        f.k = kk;
        f.nE = kk + c->cfg.n_shared;
        f.yh = yh;
    } else if (yh) {
        return set_err(c, MOE_EINVAL, "host share without the single-token launch path");
    }
    LAUNCHCHK(c, launch_ffn(f, c->lay, B, c->cs, prof ? ps.ev[1] : nullptr));
    }
    if (prof) {
        HIPCHK(c, hipEventRecord(ps.ev[2], c->cs));
        c->prof_used.push_back(ps);
    }
    if (sampled) HIPCHK(c, hipEventRecord(tp.ev[1], c->cs));
    if (c->rs_active && par < 2) {
        HIPCHK(c, hipEventRecord(c->ffn_done[par], c->cs));
        c->ffn_done_valid[par] = true;
    }
    return MOE_OK;
}

// A route-stream call runs K1/K2 on the route stream from here to route_stream_end: the stream
// first waits for everything already on the compute stream (the call's inputs and every earlier
// FFN, whose slots this call's first victims may hold).
moe_status route_stream_begin(moe_ctx* c) {
    HIPCHK(c, hipEventRecord(c->rs_start, c->cs));
    HIPCHK(c, hipStreamWaitEvent(c->rs, c->rs_start, 0));
    c->rs_active = true;
    c->ks = c->rs;
    c->ffn_done_valid[0] = c->ffn_done_valid[1] = false;
    return MOE_OK;
}

// joins the route stream back into the compute stream (the caller's ids and weights outputs, the
// cache state and the trace are then ordered before anything the caller enqueues next)
moe_status route_stream_end(moe_ctx* c) {
    c->rs_host_wait = false;
    if (!c->rs_active) return MOE_OK;
    c->rs_active = false;
    c->ks = nullptr;
    HIPCHK(c, hipEventRecord(c->rs_end, c->rs));
    HIPCHK(c, hipStreamWaitEvent(c->cs, c->rs_end, 0));
    return MOE_OK;
}

struct RouteStreamGuard {
    moe_ctx* c;
    ~RouteStreamGuard() { (void)route_stream_end(c); }
};

moe_status check_call(moe_ctx* c, int n_tokens) {
    if (!c) return MOE_EINVAL;
    if (c->failed) return MOE_ESTATE;
    if (c->hq_flag && __atomic_load_n(reinterpret_cast<uint32_t*>(c->hq_flag + 1), __ATOMIC_ACQUIRE))
        return set_err(c, MOE_EHIP, "a queued host task did not finish within %g s", c->spin_timeout_s);
    if (n_tokens < 1 || n_tokens > c->cfg.max_tokens)
        return set_err(c, MOE_EINVAL, "n_tokens %d outside [1, %d]", n_tokens, c->cfg.max_tokens);
    return MOE_OK;
}

// ------------------------------------------------ allocation-free expert FFN --
// The intermediate vectors of moe_expert_forward_noalloc live in this array (each GPU the library
// runs on holds its own copy until the process ends).  Host code never uses the array's name as an
// address: on first use on a device, with that device current, hipGetSymbolAddress gives the
// device address, which is kept per device and is what the kernels receive.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device (nullptr and a message on failure)
void* scratch_address(int dev, std::string& err) {
    if (dev < 0 || dev >= kMaxDevices) {
        err = "device index " + std::to_string(dev) + " outside the library's table";
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            err = std::string("hipGetSymbolAddress of the scratch array failed: ") + hipGetErrorString(e);
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

// ====================================================================== ABI ==

extern "C" {

moe_status moe_query_sizes(const moe_config* cfg, size_t* blob_bytes, size_t* arena_bytes,
                           size_t* workspace_bytes) {
    moe_status st = check_cfg(cfg, true);
    if (st) return st;
    Layout L = make_layout(cfg->hidden, cfg->inter);
    if (blob_bytes) *blob_bytes = L.blob_bytes;
    if (arena_bytes) *arena_bytes = L.blob_bytes * (size_t)cfg->cache_slots;
    if (workspace_bytes) *workspace_bytes = plan_workspace(*cfg).total;
    return MOE_OK;
}

moe_status moe_auto_cache_slots(const moe_config* cfg, uint64_t free_bytes, uint64_t reserve_bytes,
                                int32_t* slots_out) {
    if (!slots_out) return MOE_EINVAL;
    *slots_out = 0;
    moe_status st = check_cfg(cfg, true);
    if (st) return st;
    if (free_bytes == 0) {
        size_t fr = 0, tot = 0;
        if (hipMemGetInfo(&fr, &tot) != hipSuccess) {
            (void)hipGetLastError();
            return MOE_EHIP;
        }
        free_bytes = fr;
    }
    const Layout L = make_layout(cfg->hidden, cfg->inter);
    const int64_t cap = std::min<int64_t>((int64_t)cfg->n_layers * cfg->n_experts, MAX_CACHE_SLOTS);
    auto fits = [&](int64_t C) {
        const uint64_t need = (uint64_t)C * L.blob_bytes + library_device_bytes(*cfg, L, (int)C) + reserve_bytes;
        return need <= free_bytes;
    };
    // the need grows with C (blob + 20 B of state per slot), so the largest fitting C is found by
    // bisection over [0, cap]
    int64_t lo = 0, hi = cap;
    if (!fits(0)) lo = -1;
    else
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) / 2;
            if (fits(mid)) lo = mid; else hi = mid - 1;
        }
    *slots_out = (int32_t)std::max<int64_t>(lo, 0);
    if (lo < min_cache_slots(cfg)) return MOE_ECAPACITY;
    return MOE_OK;
}

moe_status moe_init_pool(const moe_config* cfg, moe_fill_fn fill, void* user,
                         const uint16_t* router_w_bf16, void* slot_arena_dev, size_t arena_bytes,
                         void* workspace_dev, size_t workspace_bytes, void* compute_stream,
                         void* copy_stream, moe_ctx** out) {
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    moe_status st = check_cfg(cfg);
    if (st) return st;
    if (!fill || !router_w_bf16 || !slot_arena_dev || !workspace_dev) return MOE_EINVAL;
    moe_ctx* c = new (std::nothrow) moe_ctx();
    if (!c) return MOE_ENOMEM;
    c->cfg = *cfg;
    c->lay = make_layout(cfg->hidden, cfg->inter);
    c->nE = cfg->top_k + cfg->n_shared;
    c->cs = (hipStream_t)compute_stream;
    c->ps = (hipStream_t)copy_stream;
    const Layout& L = c->lay;
    const int Lyr = cfg->n_layers, E = cfg->n_experts, C = cfg->cache_slots;
    g_init_err.clear();
    const char* where = "argument check";
    auto bail = [&](moe_status s) {
        hipError_t he = hipGetLastError();
        g_init_err = std::string("moe_init_pool failed at ") + where + ": " + hipGetErrorString(he);
        free_all(c);
        return s;
    };
    if (arena_bytes < L.blob_bytes * (size_t)C) return bail(MOE_ENOMEM);
    WsPlan wp = plan_workspace(*cfg);
    if (workspace_bytes < wp.total) return bail(MOE_ENOMEM);
    where = "device query";
    if (hipGetDevice(&c->device) != hipSuccess) return bail(MOE_EHIP);
    c->arena = (uint8_t*)slot_arena_dev;

    // workspace carve
    uint8_t* ws = (uint8_t*)workspace_dev;
    const size_t Bk = (size_t)cfg->max_tokens * cfg->top_k;
    c->z = (float*)(ws + wp.z);
    for (int p = 0; p < NPAR; ++p) {
        c->ids[p] = (int32_t*)(ws + wp.ids) + p * Bk;
        c->w[p] = (float*)(ws + wp.w) + p * Bk;
        c->slots[p] = (int32_t*)(ws + wp.slots) + p * Bk;
    }
    for (int p = 0; p <= NPAR; ++p) c->a[p] = (uint16_t*)(ws + wp.a) + (size_t)p * cfg->max_tokens * c->nE * cfg->inter;
    if (cfg->max_tokens > 1) {
        int32_t* g = (int32_t*)(ws + wp.grp);
        c->gp.max_groups = wp.max_groups;
        c->gp.max_chunks = wp.max_chunks;
        c->gp.hdr = g;
        c->gp.g_slot = g + 4;
        c->gp.g_off = c->gp.g_slot + wp.max_groups;
        c->gp.g_cnt = c->gp.g_off + wp.max_groups;
        c->gp.chunks = c->gp.g_cnt + wp.max_groups;
        c->gp.perm = c->gp.chunks + 2 * (size_t)wp.max_chunks;
        c->yp = (uint16_t*)(ws + wp.yp);
    }

    // device cache state
    const size_t n_sl = (size_t)Lyr * E;
    const StatePlan sp = plan_state(*cfg, C);
    where = "cache state allocation";
    if (hipMalloc(&c->state_dev, sp.total) != hipSuccess) return bail(MOE_ENOMEM);
    c->cd.slot_of = (int32_t*)(c->state_dev + sp.slot);
    c->cd.key_of = (int32_t*)(c->state_dev + sp.key);
    c->cd.stamp = (int64_t*)(c->state_dev + sp.stamp);
    c->cd.clock = (int64_t*)(c->state_dev + sp.clock);
    c->cd.counters = (uint64_t*)(c->state_dev + sp.cnt);
    c->cd.trace_head = (uint64_t*)(c->state_dev + sp.th);
    c->cd.trace = (TraceRec*)(c->state_dev + sp.tr);
    c->cd.trace_cap = (int64_t)cfg->trace_capacity;
    c->order[0] = (int32_t*)(c->state_dev + sp.ord);
    c->order[1] = c->order[0] + C;
    {
        std::vector<uint8_t> h;
        try {
            h.assign(sp.tr, 0);
        } catch (...) {
            return bail(MOE_ENOMEM);
        }
        memset(h.data() + sp.slot, 0xFF, n_sl * 4);
        memset(h.data() + sp.key, 0xFF, (size_t)C * 4);
        memset(h.data() + sp.stamp, 0xFF, (size_t)C * 8);
        int32_t* ord = (int32_t*)(h.data() + sp.ord);
        for (int v = 0; v < C; ++v) ord[v] = v;  // cold start: all empty, ascending index
        if (cfg->policy == MOE_POLICY_STATIC) {
            // static split: keys 0..R-1 resident in slots 0..R-1 (filled below)
            c->static_T = 2 * (int)std::min<int64_t>((int64_t)cfg->max_tokens * cfg->top_k, E);
            const int R = (int)std::min<int64_t>(C - c->static_T, n_sl);
            int32_t* so = (int32_t*)(h.data() + sp.slot);
            int32_t* ko = (int32_t*)(h.data() + sp.key);
            for (int v = 0; v < R; ++v) so[v] = ko[v] = v;
        }
        if (hipMemcpy(c->state_dev, h.data(), sp.tr, hipMemcpyHostToDevice) != hipSuccess) return bail(MOE_EHIP);
    }

    // host-mapped miss lists (two, alternating by layer parity)
    where = "miss list allocation";
    c->max_unique = (int)std::min<int64_t>((int64_t)cfg->max_tokens * cfg->top_k, E);
    c->ml_stride = align_up(sizeof(MissList) + sizeof(MissEntry) * (size_t)c->max_unique, 256);
    if (hipHostMalloc((void**)&c->ml_mem, NPAR * c->ml_stride, hipHostMallocMapped | hipHostMallocCoherent) !=
        hipSuccess)
        return bail(MOE_ENOMEM);
    memset(c->ml_mem, 0, NPAR * c->ml_stride);
    for (int p = 0; p < NPAR; ++p) miss_list(c, p)->seq = -1;
    for (auto& e : c->copy_ev)
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return bail(MOE_EHIP);
    // the reference point of the copy-path timing (the GPU clock is shared by all streams)
    where = "timing reference";
    if (hipEventCreate(&c->t_ref) != hipSuccess || hipEventRecord(c->t_ref, c->ps) != hipSuccess)
        return bail(MOE_EHIP);
    // debug and failure-injection switches
    c->verify = (cfg->flags & MOE_FLAG_VERIFY) != 0;
    if (const char* v = getenv("MOE_VERIFY")) c->verify = c->verify || (v[0] && strcmp(v, "0") != 0);
    if (const char* f = getenv("MOE_FAULT")) {
        where = "MOE_FAULT";
        std::string spec(f);
        size_t pos = 0;
        while (pos < spec.size()) {
            size_t end = spec.find(',', pos);
            if (end == std::string::npos) end = spec.size();
            const std::string item = spec.substr(pos, end - pos);
            unsigned long long n = 0;
            char tail = 0;
            if (sscanf(item.c_str(), "h2d_fail_at=%llu%c", &n, &tail) == 1 && n > 0) c->fault_fail_at = n;
            else if (sscanf(item.c_str(), "h2d_corrupt_at=%llu%c", &n, &tail) == 1 && n > 0) c->fault_corrupt_at = n;
            else if (!item.empty()) {
                g_init_err = "moe_init_pool: MOE_FAULT item '" + item + "' is not h2d_fail_at=N or h2d_corrupt_at=N";
                free_all(c);
                return MOE_EINVAL;
            }
            pos = end + 1;
        }
    }
    // a second copy stream (default priority): blob copies alternate between the two, which
    // keeps two DMA queues busy and hides the per-copy overhead of small blobs
    if (hipStreamCreateWithFlags(&c->ps2, hipStreamNonBlocking) != hipSuccess) return bail(MOE_EHIP);
    for (auto& e : c->copy_ev2)
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return bail(MOE_EHIP);
    // the route stream of hybrid stack calls (default priority) and its events
    if (hipStreamCreateWithFlags(&c->rs, hipStreamNonBlocking) != hipSuccess) return bail(MOE_EHIP);
    for (hipEvent_t* e : {&c->rs_start, &c->rs_end, &c->k2_done[0], &c->k2_done[1], &c->ffn_done[0], &c->ffn_done[1]})
        if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess) return bail(MOE_EHIP);

    // router weights -> HBM
    where = "router upload";
    const size_t rbytes = (size_t)Lyr * E * cfg->hidden * 2;
    if (hipMalloc(&c->router_dev, rbytes) != hipSuccess) return bail(MOE_ENOMEM);
    if (hipMemcpy(c->router_dev, router_w_bf16, rbytes, hipMemcpyHostToDevice) != hipSuccess) return bail(MOE_EHIP);

    // pinned pool, filled in parallel
    // The pool: as many blobs as the platform lets us pin (capped by pinned_mb), the rest in
    // pageable memory behind a pinned bounce ring.  A failed pinning request is retried 1/8
    // smaller.
    where = "pinned pool allocation";
    c->pool_bytes = n_sl * L.blob_bytes;
    size_t n_pin = n_sl;
    if (cfg->pinned_mb > 0) n_pin = std::min(n_sl, ((size_t)cfg->pinned_mb << 20) / L.blob_bytes);
    for (;;) {
        if (n_pin == 0) break;
        if (hipHostMalloc((void**)&c->pool, n_pin * L.blob_bytes, hipHostMallocDefault) == hipSuccess) {
            if (n_pin == n_sl) break;
            const hipError_t e = c->bounce.init(L.blob_bytes, 8, std::min(4u, std::max(1u, std::thread::hardware_concurrency())), c->ps);
            if (e == hipSuccess) break;
            (void)hipHostFree(c->pool);
        }
        (void)hipGetLastError();
        c->pool = nullptr;
        n_pin = n_pin * 7 / 8;
    }
    c->n_pin = n_pin;
    c->n_blobs = n_sl;
    if (n_pin < n_sl) {
        if (!c->bounce.ready()) {
            where = "bounce ring allocation";
            if (c->bounce.init(L.blob_bytes, 8, std::min(4u, std::max(1u, std::thread::hardware_concurrency())), c->ps) != hipSuccess)
                return bail(MOE_ENOMEM);
        }
        where = "pageable pool allocation";
        const size_t pg = (n_sl - n_pin) * L.blob_bytes;
        c->pool_pg = (uint8_t*)aligned_alloc(4096, (pg + 4095) / 4096 * 4096);
        if (!c->pool_pg) return bail(MOE_ENOMEM);
    }
    int nth = cfg->fill_threads > 0 ? cfg->fill_threads : (int)std::thread::hardware_concurrency();
    nth = std::max(1, std::min<int>(nth, (int)std::min<size_t>(n_sl, 64)));
    std::atomic<size_t> next{0};
    std::atomic<bool> fill_failed{false};
    auto worker = [&]() {
        // nothing may throw across the C ABI (nor out of a thread): a failed buffer allocation
        // stops the fill and is reported below
        std::vector<uint8_t> tmp;
        try {
            tmp.resize(L.blob_bytes);
        } catch (...) {
            fill_failed.store(true);
            return;
        }
        for (;;) {
            size_t i = next.fetch_add(1);
            if (i >= n_sl || fill_failed.load(std::memory_order_relaxed)) break;
            fill(user, (int32_t)(i / E), (int32_t)(i % E), tmp.data());
            repack(L, tmp.data(), const_cast<uint8_t*>(c->blob_src(i)));
        }
    };
    {
        std::vector<std::thread> th;
        try {
            th.reserve((size_t)nth);
            for (int t = 1; t < nth; ++t) th.emplace_back(worker);
        } catch (...) {
            // fewer helper threads: the calling thread fills the rest
        }
        worker();
        for (auto& t : th) t.join();
    }
    where = "pool fill (host buffer allocation)";
    if (fill_failed.load()) return bail(MOE_ENOMEM);

    if (cfg->policy == MOE_POLICY_STATIC) {
        where = "static split resident fill";
        const size_t R = (size_t)std::min<int64_t>(C - c->static_T, n_sl);
        for (size_t v = 0; v < R; ++v)
            if (hipMemcpy(c->arena + v * L.blob_bytes, c->blob_src(v), L.blob_bytes, hipMemcpyHostToDevice) !=
                hipSuccess)
                return bail(MOE_EHIP);
    }

    // shared experts -> HBM
    where = "shared expert upload";
    if (cfg->n_shared > 0) {
        const size_t sb = (size_t)Lyr * cfg->n_shared * L.blob_bytes;
        if (hipMalloc(&c->shared_dev, sb) != hipSuccess) return bail(MOE_ENOMEM);
        std::vector<uint8_t> tmp, packed;
        try {
            tmp.resize(L.blob_bytes);
            packed.resize(L.blob_bytes);
        } catch (...) {
            return bail(MOE_ENOMEM);
        }
        for (int l = 0; l < Lyr; ++l)
            for (int s = 0; s < cfg->n_shared; ++s) {
                fill(user, l, -1 - s, tmp.data());
                repack(L, tmp.data(), packed.data());
                if (hipMemcpy(c->shared_dev + ((size_t)l * cfg->n_shared + s) * L.blob_bytes, packed.data(),
                              L.blob_bytes, hipMemcpyHostToDevice) != hipSuccess)
                    return bail(MOE_EHIP);
            }
    }
    if (hipStreamSynchronize(c->cs) != hipSuccess) return bail(MOE_EHIP);
    *out = c;
    return MOE_OK;
}

moe_status moe_cache_resolve(moe_ctx* c, int32_t step, int32_t layer, const int32_t* ids_dev,
                             int32_t n_tokens, int32_t* slots_dev, int32_t* n_miss_out) {
    moe_status st = check_call(c, n_tokens);
    if (st) return st;
    c->h2d_timing = (c->h2d_calls++ % H2D_SAMPLE) == 0;
    if (layer < 0 || layer >= c->cfg.n_layers || !ids_dev) return set_err(c, MOE_EINVAL, "bad layer or ids");
    st = launch_resolve(c, step, layer, false, ids_dev, n_tokens, 0, slots_dev, nullptr, nullptr);
    if (st) return st;
    int nm = 0;
    st = stage_misses(c, layer, 0, c->seq, &nm);
    if (st) return st;
    if (nm > 0) {
        if (c->copy_used[0][0]) HIPCHK(c, hipStreamWaitEvent(c->cs, c->copy_ev[0], 0));
        if (c->copy_used[0][1]) HIPCHK(c, hipStreamWaitEvent(c->cs, c->copy_ev2[0], 0));
    }
    if (n_miss_out) *n_miss_out = nm;
    return MOE_OK;
}

moe_status moe_router_logits(moe_ctx* c, int32_t layer, const void* x, int32_t n_tokens, float* z_out) {
    moe_status st = check_call(c, n_tokens);
    if (st) return st;
    if (layer < 0 || layer >= c->cfg.n_layers || !x || !z_out) return set_err(c, MOE_EINVAL, "bad layer or buffers");
    K1Args a{};
    a.W = c->router_dev + (size_t)layer * c->cfg.n_experts * c->cfg.hidden;
    a.x = (const uint16_t*)x;
    a.z = z_out;
    a.E = c->cfg.n_experts;
    a.H = c->cfg.hidden;
    a.B = n_tokens;
    LAUNCHCHK(c, launch_k1(a, c->cs));
    return MOE_OK;
}

moe_status moe_layer_forward(moe_ctx* c, int32_t step, int32_t layer, const void* x, int32_t n_tokens,
                             void* y, int32_t* ids_out, float* w_out) {
    moe_status st = check_call(c, n_tokens);
    if (st) return st;
    c->h2d_timing = (c->h2d_calls++ % H2D_SAMPLE) == 0;
    if (layer < 0 || layer >= c->cfg.n_layers || !x || !y) return set_err(c, MOE_EINVAL, "bad layer or buffers");
    if ((st = hyb_begin(c, x, 0, 1, n_tokens))) return st;
    if ((st = launch_route(c, layer, x, n_tokens))) return st;
    if ((st = launch_resolve(c, step, layer, true, nullptr, n_tokens, 0, nullptr, ids_out, w_out))) return st;
    int nm = 0;
    if ((st = stage_misses(c, layer, 0, c->seq, &nm))) return st;
    return launch_ffn_layer(c, layer, x, n_tokens, 0, y, nm);
}

moe_status moe_stack_forward(moe_ctx* c, int32_t step, const void* x, int64_t xs, int32_t n_tokens,
                             void* y, int64_t ys, int32_t* ids_out, float* w_out) {
    moe_status st = check_call(c, n_tokens);
    if (st) return st;
    c->h2d_timing = (c->h2d_calls++ % H2D_SAMPLE) == 0;
    if (!x || !y) return set_err(c, MOE_EINVAL, "null buffers");
    const int L = c->cfg.n_layers;
    const size_t kB = (size_t)n_tokens * c->cfg.top_k;
    auto xl = [&](int l) { return (const uint16_t*)x + (size_t)l * xs; };
    auto yl = [&](int l) { return (uint16_t*)y + (size_t)l * ys; };
    auto idl = [&](int l) { return ids_out ? ids_out + (size_t)l * kB : nullptr; };
    auto wl = [&](int l) { return w_out ? w_out + (size_t)l * kB : nullptr; };
    if ((st = hyb_begin(c, x, xs, L, n_tokens))) return st;
    if (c->cfg.lookahead == 0) {
        for (int l = 0; l < L; ++l) {
            if ((st = launch_route(c, l, xl(l), n_tokens))) return st;
            if ((st = launch_resolve(c, step, l, true, nullptr, n_tokens, 0, nullptr, idl(l), wl(l)))) return st;
            int nm = 0;
            if ((st = stage_misses(c, l, 0, c->seq, &nm))) return st;
            if ((st = launch_ffn_layer(c, l, xl(l), n_tokens, 0, yl(l), nm))) return st;
        }
        return MOE_OK;
    }
    const bool whole_pool = n_tokens == 1 && (int64_t)c->cfg.cache_slots >= (int64_t)L * c->cfg.n_experts;
    // Lookahead D = 2 .. 7 (LRU, C >= (D + 1) k B): K1/K2 of layer l+D are enqueued before layer
    // l's FFN, so they run right after layer l-1's FFN and the copies of D layers are queued while
    // a layer's FFN waits for its own.  When layer l's copies are issued the FFNs of layers l-D ..
    // l-1 may still be pending.  The step's victims are the least recently used slots outside its
    // own hits; the slots touched by the D previous steps (at most D k B) are more recent than
    // every slot they did not touch, and the step's hits and misses number at most k B, so with
    // C >= (D + 1) k B every victim was last used D + 1 or more steps back, by an FFN that has
    // finished (stream order: layer l's resolve runs after layer l-D-1's FFN, and its copies are
    // issued once the host has read its miss list).  A layer's buffers (ids, weights, slots, miss
    // list, copy events) are reused D + 1 layers later, after that layer's FFN in stream order.
    // The resolve sequence, and so every result, is the same as with lookahead 1 or 0.  A call
    // whose cache is too small for the configured depth takes the deepest one that fits.
    // Hybrid steps take the same pipeline: their host tasks are queued (HostTaskQueue) and the
    // compute stream waits for each layer's task before its FFN, so host tasks and copies both
    // run up to D layers ahead.
    int depth = 0;
    if ((c->hyb_call || !whole_pool) && c->cfg.policy == MOE_POLICY_LRU)
        for (int d = std::min(c->cfg.lookahead, NPAR - 1); d >= 2 && !depth; --d)
            if ((int64_t)c->cfg.cache_slots >= (int64_t)(d + 1) * c->cfg.top_k * n_tokens) depth = d;
    if (depth >= 2) {
        int64_t seq_par[NPAR] = {};
        c->hq_mode = c->hyb_call;
        for (int l = 0; l < depth && l < L; ++l) {
            if ((st = launch_route(c, l, xl(l), n_tokens))) return st;
            if ((st = launch_resolve(c, step, l, true, nullptr, n_tokens, l, nullptr, idl(l), wl(l)))) return st;
            seq_par[l] = c->seq;
        }
        for (int l = 0; l < L; ++l) {
            const int par = l % NPAR;
            int nm = 0;
            if ((st = stage_misses(c, l, par, seq_par[par], &nm))) return st;
            if (l + depth < L) {
                const int np = (l + depth) % NPAR;
                if ((st = launch_route(c, l + depth, xl(l + depth), n_tokens))) return st;
                if ((st = launch_resolve(c, step, l + depth, true, nullptr, n_tokens, np, nullptr, idl(l + depth),
                                         wl(l + depth))))
                    return st;
                seq_par[np] = c->seq;
            }
            if ((st = launch_ffn_layer(c, l, xl(l), n_tokens, par, yl(l), nm))) return st;
        }
        c->hq_mode = false;
        return MOE_OK;
    }
    // lookahead 1: K1/K2 of layer l+1 and its copies are issued before layer l's FFN
    int64_t seq_of[2] = {0, 0};
    if (c->hyb_call) {
        // hybrid steps: layer l+1's miss list is taken (and its host task started) before
        // layer l's FFN is launched, so the host workers go from one layer's experts to the
        // next without waiting for the launches in between
        // one token: K1/K2 on the route stream, so a layer's miss list (the host workers' next
        // task) does not wait behind an FFN that waits for its copies; copies still wait for the
        // FFN two layers back (their victims may hold its slots).  Batches keep one stream: their
        // FFN reads K2's slot buffers, and the waits that protects cost more than the overlap
        // gains (measured)
        RouteStreamGuard guard{c};
        if (n_tokens == 1 && (st = route_stream_begin(c))) return st;
        if ((st = launch_route(c, 0, xl(0), n_tokens))) return st;
        if ((st = launch_resolve(c, step, 0, true, nullptr, n_tokens, 0, nullptr, idl(0), wl(0)))) return st;
        int nm_of[2] = {0, 0};
        if ((st = stage_misses(c, 0, 0, c->seq, &nm_of[0]))) return st;
        for (int l = 0; l < L; ++l) {
            const int par = l & 1, np = par ^ 1;
            if (l + 1 < L) {
                if ((st = launch_route(c, l + 1, xl(l + 1), n_tokens))) return st;
                if ((st = launch_resolve(c, step, l + 1, true, nullptr, n_tokens, np, nullptr, idl(l + 1),
                                         wl(l + 1))))
                    return st;
                if ((st = stage_misses(c, l + 1, np, c->seq, &nm_of[np]))) return st;
            }
            if ((st = launch_ffn_layer(c, l, xl(l), n_tokens, par, yl(l), nm_of[par]))) return st;
        }
        return route_stream_end(c);
    }
    // One token with the whole pool in the cache: K1/K2 on the route stream, so layer l+1's
    // resolve runs beside layer l-1's FFN instead of behind it.  The host issues layer l+1's
    // copies (compulsory misses only: nothing is evicted) once that FFN has ended, which keeps
    // them one layer ahead.  With a partial cache the in-stream order is kept: measured, the route
    // stream gained nothing at gpt-oss shape and lost 5 % at Qwen3.6 shape (small experts, many
    // short copies), while with the whole pool cached it gained 6 % (and the helper thread below
    // another 1 % at gpt-oss shape, 10 % at Qwen3.6 shape).
    RouteStreamGuard guard{c};
    if (!whole_pool) {
        if ((st = launch_route(c, 0, xl(0), n_tokens))) return st;
        if ((st = launch_resolve(c, step, 0, true, nullptr, n_tokens, 0, nullptr, idl(0), wl(0)))) return st;
        seq_of[0] = c->seq;
        for (int l = 0; l < L; ++l) {
            const int par = l & 1;
            int nm = 0;
            if ((st = stage_misses(c, l, par, seq_of[par], &nm))) return st;
            if (l + 1 < L) {
                const int np = par ^ 1;
                if ((st = launch_route(c, l + 1, xl(l + 1), n_tokens))) return st;
                if ((st = launch_resolve(c, step, l + 1, true, nullptr, n_tokens, np, nullptr, idl(l + 1),
                                         wl(l + 1))))
                    return st;
                seq_of[np] = c->seq;
            }
            if ((st = launch_ffn_layer(c, l, xl(l), n_tokens, par, yl(l), nm))) return st;
        }
        return MOE_OK;
    }
    if ((st = route_stream_begin(c))) return st;
    c->rs_host_wait = true;
    // With the whole pool cached the host's HIP calls set the pace, so a helper thread issues the
    // route stream's launches (K1/K2 of every layer, in order) while this thread stages the miss
    // lists and launches the FFNs.  The resolve of layer r rewrites the miss list of layer r-2, so
    // it waits until this thread has staged that layer; this thread stages layer l once its
    // resolve is enqueued.  Only the helper touches the resolve bookkeeping (c->seq, c->parity)
    // until it is joined.
    std::atomic<int> resolved{0}, staged{0};
    std::atomic<bool> quit{false};
    std::atomic<int> helper_st{MOE_OK};
    std::vector<int64_t> seq_layer((size_t)L, 0);
    std::thread helper;
    auto helper_fn = [&] {
        for (int r = 0; r < L; ++r) {
            while (staged.load(std::memory_order_acquire) < r - 1) {
                if (quit.load(std::memory_order_relaxed)) return;
                _mm_pause();
            }
            moe_status s2 = launch_route(c, r, xl(r), n_tokens);
            if (!s2) s2 = launch_resolve(c, step, r, true, nullptr, n_tokens, r & 1, nullptr, idl(r), wl(r));
            if (s2) {
                helper_st.store(s2, std::memory_order_release);
                return;
            }
            seq_layer[(size_t)r] = c->seq;
            resolved.store(r + 1, std::memory_order_release);
        }
    };
    try {
        helper = std::thread(helper_fn);
    } catch (...) {
        return set_err(c, MOE_ENOMEM, "could not start the stack call's helper thread");
    }
    struct Joiner {
        std::thread& t;
        std::atomic<bool>& q;
        ~Joiner() {
            q.store(true, std::memory_order_relaxed);
            if (t.joinable()) t.join();
        }
    } joiner{helper, quit};
    for (int l = 0; l < L; ++l) {
        const int par = l & 1;
        while (resolved.load(std::memory_order_acquire) <= l) {
            const int hs = helper_st.load(std::memory_order_acquire);
            if (hs != MOE_OK) return (moe_status)hs;
            _mm_pause();
        }
        int nm = 0;
        if ((st = stage_misses(c, l, par, seq_layer[(size_t)l], &nm))) return st;
        staged.store(l + 1, std::memory_order_release);
        if ((st = launch_ffn_layer(c, l, xl(l), n_tokens, par, yl(l), nm))) return st;
    }
    return route_stream_end(c);
}

moe_status moe_expert_forward(moe_ctx* c, int32_t layer, const void* x, int32_t n_tokens,
                              const int32_t* slots_dev, const float* w_dev, void* y) {
    moe_status st = check_call(c, n_tokens);
    if (st) return st;
    if (layer < 0 || layer >= c->cfg.n_layers || !x || !y || !slots_dev || !w_dev)
        return set_err(c, MOE_EINVAL, "bad layer or buffers");
    return launch_ffn_layer(c, layer, x, n_tokens, NPAR, y, 0, slots_dev, w_dev);
}

moe_status moe_expert_forward_noalloc(const moe_config* cfg, const void* arena, const void* shared_blob,
                                      const void* x, int32_t n_tokens, const int32_t* slots_dev, const float* w_dev,
                                      void* y, void* stream) {
    auto fail = [](moe_status st, const std::string& msg) {
        g_init_err = "moe_expert_forward_noalloc: " + msg;
        return st;
    };
    if (!cfg) return fail(MOE_EINVAL, "null config");
    // the shape checks of a context; the cache's capacity rule does not apply (no cache here)
    moe_config shape = *cfg;
    shape.cache_slots = 0;
    shape.max_tokens = 1;
    moe_status st = check_cfg(&shape, true);
    if (st) return fail(st, "unsupported shape");
    if (cfg->cache_slots < 1) return fail(MOE_EINVAL, "cache_slots (slots in the arena) must be >= 1");
    if (!arena || !x || !y || !slots_dev || !w_dev || (cfg->n_shared > 0 && !shared_blob))
        return fail(MOE_EINVAL, "null buffer");
    if (n_tokens < 1 || n_tokens > MOE_NOALLOC_MAX_TOKENS)
        return fail(MOE_EINVAL, "n_tokens " + std::to_string(n_tokens) + " outside [1, " +
                                    std::to_string(MOE_NOALLOC_MAX_TOKENS) + "]");
    const int nE = cfg->top_k + cfg->n_shared;
    const size_t need = (size_t)n_tokens * nE * cfg->inter * 2;
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_EINVAL, "intermediate vectors need " + std::to_string(need) + " bytes, more than the " +
                                    std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES) + "-byte scratch array");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(MOE_EHIP, "hipGetDevice failed");
    }
    std::string err;
    void* ptr = scratch_address(dev, err);
    if (!ptr) return fail(MOE_EHIP, err);
    const Layout L = make_layout(cfg->hidden, cfg->inter);
    FfnArgs f{};
    f.arena = (const uint8_t*)arena;
    f.shared = (const uint8_t*)shared_blob;
    f.slots = slots_dev;
    f.w = w_dev;
    f.x = (const uint16_t*)x;
    f.a = (uint16_t*)ptr;
    f.y = (uint16_t*)y;
    f.yh = nullptr;
    f.blob_bytes = L.blob_bytes;
    f.d_codes_off = L.d_codes_off;
    f.d_scales_off = L.d_scales_off;
    f.k = cfg->top_k;
    f.n_shared = cfg->n_shared;
    f.nE = nE;
    f.layer = 0;
    f.NB = L.NB;
    f.NBI = L.NBI;
    f.I = cfg->inter;
    f.H = cfg->hidden;
    f.C = cfg->cache_slots;
    f.karg = 0;
    const int e = launch_ffn(f, L, n_tokens, stream, nullptr);
    if (e != 0) return fail(MOE_EHIP, std::string("FFN launch failed: ") + hipGetErrorString((hipError_t)e));
    return MOE_OK;
}

moe_status moe_stats(moe_ctx* c, moe_counters* out, moe_trace_rec* buf, size_t cap, size_t* n_out) {
    if (!c) return MOE_EINVAL;
    if (c->failed) return MOE_ESTATE;
    HIPCHK(c, hipStreamSynchronize(c->cs));
    HIPCHK(c, hipStreamSynchronize(c->ps));
    uint64_t cnt[5], th[2];
    HIPCHK(c, hipMemcpy(cnt, c->cd.counters, sizeof cnt, hipMemcpyDeviceToHost));
    HIPCHK(c, hipMemcpy(th, c->cd.trace_head, sizeof th, hipMemcpyDeviceToHost));
    size_t n = (size_t)th[0];
    size_t take = std::min(n, buf ? cap : 0);
    if (take) HIPCHK(c, hipMemcpy(buf, c->cd.trace, take * sizeof(moe_trace_rec), hipMemcpyDeviceToHost));
    uint64_t dropped = th[1] + (n - take);
    static_assert(sizeof(moe_trace_rec) == sizeof(TraceRec), "trace record layout");
    // drain: restart the trace at 0, keep the dropped count
    uint64_t zero2[2] = {0, dropped};
    HIPCHK(c, hipMemcpy(c->cd.trace_head, zero2, sizeof zero2, hipMemcpyHostToDevice));
    HIPCHK(c, hipStreamSynchronize(c->ps2));
    {
        moe_status st = harvest_h2d(c, true);
        if (!st) st = harvest_ffn(c, true);
        if (st) return st;
        // a fresh reference point keeps the interval starts precise (float milliseconds)
        HIPCHK(c, hipEventRecord(c->t_ref, c->ps));
        HIPCHK(c, hipEventSynchronize(c->t_ref));
        c->h2d_iv_end = -1.0;
    }
    for (auto& p : c->prof_used) {
        float a = 0, b = 0;
        HIPCHK(c, hipEventElapsedTime(&a, p.ev[0], p.ev[1]));
        HIPCHK(c, hipEventElapsedTime(&b, p.ev[1], p.ev[2]));
        c->k3_ms += a;
        c->k4_ms += b;
        c->ffn_launches++;
        c->prof_free.push_back(p);
    }
    c->prof_used.clear();
    if (out) {
        out->hits = cnt[0];
        out->misses = cnt[1];
        out->evictions = cnt[2];
        out->resolves = cnt[3];
        out->h2d_bytes = c->h2d_bytes;
        out->h2d_copies = c->h2d_copies;
        out->trace_records = take;
        out->trace_dropped = dropped;
        out->ffn_launches = c->ffn_launches;
        out->h2d_bounced = c->h2d_bounced;
        out->pool_pinned_bytes = (uint64_t)(c->n_pin * c->lay.blob_bytes);
        out->k3_ms = c->k3_ms;
        out->k4_ms = c->k4_ms;
        out->host_experts = cnt[4];
        out->host_tasks = c->host_tasks;
        out->host_busy_ms = (double)c->hpool.busy_ns() * 1e-6;
        out->host_wait_ms = c->host_wait_ms;
        out->h2d_ns = (uint64_t)llround(c->h2d_busy_ms * 1e6);
        out->ffn_ns = (uint64_t)llround(c->ffn_ms * 1e6);
        out->ffn_timed = c->ffn_timed;
        out->h2d_timed_bytes = c->h2d_timed_bytes;
    }
    c->ffn_launches = 0;
    c->k3_ms = c->k4_ms = 0;
    if (n_out) *n_out = take;
    return MOE_OK;
}

moe_status moe_measure_h2d(moe_ctx* c, size_t bytes, int32_t n_copies, double* gbps) {
    if (!c || !gbps || bytes == 0 || n_copies < 1) return MOE_EINVAL;
    if (c->failed) return MOE_ESTATE;
    const size_t blob = c->lay.blob_bytes;
    // the pinned part of the pool only: the copy path of a pinned miss
    const size_t n_blobs = c->n_pin;
    if (bytes > n_blobs * blob) return set_err(c, MOE_EINVAL, "copy larger than the pinned part of the pool");
    const size_t span = (bytes + blob - 1) / blob;  // blobs covered by one copy
    uint8_t* scratch = nullptr;
    HIPCHK(c, hipMalloc(&scratch, 2 * bytes));
    HIPCHK(c, hipStreamSynchronize(c->ps));
    HIPCHK(c, hipStreamSynchronize(c->ps2));
    uint64_t r = 0x9E3779B97F4A7C15ull;
    auto next_off = [&]() {
        r ^= r << 13; r ^= r >> 7; r ^= r << 17;
        size_t i = (size_t)(r % (n_blobs > span ? n_blobs - span + 1 : 1));
        return i * blob;
    };
    // the miss path's copies, alternating between the two copy streams, timed on the host
    // from issue to both streams drained (one untimed copy on each stream first: a stream's
    // first copy also sets up its DMA queue)
    HIPCHK(c, hipMemcpyAsync(scratch, c->pool + next_off(), bytes, hipMemcpyHostToDevice, c->ps));
    HIPCHK(c, hipMemcpyAsync(scratch + bytes, c->pool + next_off(), bytes, hipMemcpyHostToDevice, c->ps2));
    HIPCHK(c, hipStreamSynchronize(c->ps));
    HIPCHK(c, hipStreamSynchronize(c->ps2));
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < n_copies; ++i)
        HIPCHK(c, hipMemcpyAsync(scratch + (size_t)(i & 1) * bytes, c->pool + next_off(), bytes,
                                 hipMemcpyHostToDevice, (i & 1) ? c->ps2 : c->ps));
    HIPCHK(c, hipStreamSynchronize(c->ps));
    HIPCHK(c, hipStreamSynchronize(c->ps2));
    const double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    HIPCHK(c, hipFree(scratch));
    *gbps = (double)bytes * n_copies / (ms * 1e-3) / 1e9;
    return MOE_OK;
}

moe_status moe_pack_blob(const moe_config* cfg, const uint8_t* logical, uint8_t* packed) {
    moe_status st = check_cfg(cfg, true);
    if (st) return st;
    if (!logical || !packed || logical == packed) return MOE_EINVAL;
    repack(make_layout(cfg->hidden, cfg->inter), logical, packed);
    return MOE_OK;
}

moe_status moe_host_expert_ffn(const moe_config* cfg, const uint8_t* const* blobs, const float* w, int32_t n,
                               const uint16_t* x, float* y, int32_t threads) {
    moe_status st = check_cfg(cfg, true);
    if (st) return st;
    if (n < 0 || (n > 0 && (!blobs || !w)) || !x || !y || threads < 1) return MOE_EINVAL;
    for (int j = 0; j < n; ++j)
        if (!blobs[j]) return MOE_EINVAL;
    host_expert_ffn(make_layout(cfg->hidden, cfg->inter), blobs, w, n, x, y, threads);
    return MOE_OK;
}

moe_status moe_host_expert_batch(const moe_config* cfg, int32_t n_tok, const uint16_t* x, float* y,
                                 const uint8_t* const* blobs, const float* w, const int32_t* tok, int32_t n,
                                 int32_t threads) {
    moe_status st = check_cfg(cfg, true);
    if (st) return st;
    if (n_tok < 1 || n_tok > kHostMaxTokens || n < 0 || n > kHostMaxEntries || !x || !y ||
        (n > 0 && (!blobs || !w || !tok)) || threads < 1 || threads > 256)
        return MOE_EINVAL;
    std::vector<HostEntry> ent((size_t)n);
    for (int j = 0; j < n; ++j) {
        if (!blobs[j] || tok[j] < 0 || tok[j] >= n_tok) return MOE_EINVAL;
        ent[j] = {blobs[j], w[j], tok[j]};
    }
    const Layout L = make_layout(cfg->hidden, cfg->inter);
    const uint16_t* xs[kHostMaxTokens];
    float* ys[kHostMaxTokens];
    for (int b = 0; b < n_tok; ++b) {
        xs[b] = x + (size_t)b * L.H;
        ys[b] = y + (size_t)b * L.H;
    }
    HostExpertPool pool;
    if (!pool.start(threads)) return MOE_ENOMEM;
    pool.submit(L, n_tok, xs, ys, ent.data(), n);
    pool.wait();
    pool.stop();
    return MOE_OK;
}

int32_t moe_hybrid_split(int32_t n_miss, double pcie_gbps, double host_gbps) {
    if (n_miss <= 0) return 0;
    if (!(host_gbps > pcie_gbps) || !(pcie_gbps > 0.0)) return n_miss;  // no host bandwidth left over
    const double q = (double)n_miss * pcie_gbps / host_gbps;
    const int32_t r = (int32_t)std::floor(q + 0.5);
    return std::min(std::max(r, (int32_t)0), n_miss);
}

moe_status moe_set_backend(moe_ctx* c, int32_t backend, double pcie_gbps, double host_gbps, int32_t host_threads) {
    if (!c) return MOE_EINVAL;
    if (c->failed) return MOE_ESTATE;
    HIPCHK(c, hipStreamSynchronize(c->cs));
    // a task left running by a call that returned early ends before the pool changes
    if (c->host_running >= 0) {
        c->hpool.wait();
        c->host_running = -1;
    }
    c->host_has[0] = c->host_has[1] = false;
    if (c->hq.done() < c->hq.pushed() && !c->hq.wait(c->hq.pushed(), c->spin_timeout_s))
        return set_err(c, MOE_EHIP, "timed out waiting for queued host tasks");
    if (backend == MOE_BACKEND_OFFLOAD) {
        c->hq.stop();
        c->hpool.stop();
        c->backend = MOE_BACKEND_OFFLOAD;
        return MOE_OK;
    }
    if (backend != MOE_BACKEND_HYBRID || !(pcie_gbps > 0.0) || !(host_gbps > 0.0) || host_threads < 1 ||
        host_threads > 256)
        return set_err(c, MOE_EINVAL, "backend %d with B_P %g, B_H %g, %d threads", backend, pcie_gbps, host_gbps,
                       host_threads);
    if (c->cfg.policy != MOE_POLICY_LRU) return set_err(c, MOE_EINVAL, "the hybrid backend needs the LRU policy");
    if (!c->yh && hipHostMalloc((void**)&c->yh,
                                (size_t)c->cfg.n_layers * kHostMaxTokens * c->cfg.hidden * sizeof(float),
                                hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess)
        return set_err(c, MOE_ENOMEM, "host-mapped buffer for the host experts' sums");
    if (!c->xs_stream) {
        HIPCHK(c, hipStreamCreateWithFlags(&c->xs_stream, hipStreamNonBlocking));
        HIPCHK(c, hipEventCreateWithFlags(&c->xs_start, hipEventDisableTiming));
        HIPCHK(c, hipEventCreateWithFlags(&c->xs_done, hipEventDisableTiming));
    }
    if (c->hpool.workers() != host_threads && !c->hpool.start(host_threads))
        return set_err(c, MOE_ENOMEM, "could not start %d host workers", host_threads);
    if (!c->hq_flag) {
        if (hipHostMalloc((void**)&c->hq_flag, 256, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess)
            return set_err(c, MOE_ENOMEM, "host-mapped word for the host-task count");
        memset(c->hq_flag, 0, 256);
        HIPCHK(c, hipHostGetDevicePointer((void**)&c->hq_flag_dev, c->hq_flag, 0));
    }
    if (!c->hq.running()) {
        __atomic_store_n(c->hq_flag, c->hq.done(), __ATOMIC_RELEASE);
        c->hq.set_mirror(c->hq_flag);
        if (!c->hq.start(&c->hpool)) return set_err(c, MOE_ENOMEM, "could not start the host task dispatcher");
    }
    c->backend = MOE_BACKEND_HYBRID;
    c->hyb_bp = pcie_gbps;
    c->hyb_bh = host_gbps;
    return MOE_OK;
}

int32_t moe_select_backend(double pcie_gbps, double host_gbps, double threshold) {
    return (pcie_gbps > 0.0 && host_gbps > threshold * pcie_gbps) ? MOE_BACKEND_HYBRID : MOE_BACKEND_OFFLOAD;
}

moe_status moe_calibrate_backend(moe_ctx* c, int32_t host_threads, double host_seconds, double threshold,
                                 moe_bw_profile* out) {
    if (!c || !out || host_threads < 1 || !(host_seconds > 0.0) || !(threshold > 0.0)) return MOE_EINVAL;
    if (c->failed) return MOE_ESTATE;
    memset(out, 0, sizeof *out);
    const size_t blob = c->lay.blob_bytes;
    // PCIe side: blob-sized copies from random offsets of the pinned pool (>= 2 GB)
    double bp = 0.0;
    const int n_cp = (int)std::max<size_t>(8, (size_t)(2e9 / (double)blob) + 1);
    moe_status st = moe_measure_h2d(c, blob, n_cp, &bp);
    if (st) return st;
    // host side: the host expert kernel over blobs spread across the pool
    const size_t n_sl = (size_t)c->cfg.n_layers * c->cfg.n_experts;
    const int nb = (int)std::min<size_t>(n_sl, 64);
    std::vector<const uint8_t*> blobs(nb);
    uint64_t r = 0xD1B54A32D192ED03ull;
    for (int i = 0; i < nb; ++i) {
        r ^= r << 13; r ^= r >> 7; r ^= r << 17;
        blobs[i] = c->blob_src((size_t)(r % n_sl));
    }
    const double bh = host_expert_rate(c->lay, blobs.data(), nb, host_threads, host_seconds) / 1e9;
    out->pcie_gbps = bp;
    out->host_gbps = bh;
    out->ratio = bp > 0.0 ? bh / bp : 0.0;
    out->threshold = threshold;
    out->host_threads = host_threads;
    out->backend = moe_select_backend(bp, bh, threshold);
    snprintf(out->host_isa, sizeof out->host_isa, "%s", host_ffn_isa());
    return MOE_OK;
}

moe_status moe_cache_state(moe_ctx* c, int32_t* slot_of, int32_t* key_of, int64_t* stamp) {
    if (!c) return MOE_EINVAL;
    if (c->failed) return MOE_ESTATE;
    HIPCHK(c, hipStreamSynchronize(c->cs));
    const size_t n_sl = (size_t)c->cfg.n_layers * c->cfg.n_experts, C = (size_t)c->cfg.cache_slots;
    if (slot_of) HIPCHK(c, hipMemcpy(slot_of, c->cd.slot_of, n_sl * 4, hipMemcpyDeviceToHost));
    if (key_of) HIPCHK(c, hipMemcpy(key_of, c->cd.key_of, C * 4, hipMemcpyDeviceToHost));
    if (stamp) HIPCHK(c, hipMemcpy(stamp, c->cd.stamp, C * 8, hipMemcpyDeviceToHost));
    return MOE_OK;
}

void moe_destroy(moe_ctx* c) { free_all(c); }

const char* moe_last_error(const moe_ctx* c) { return c ? c->err.c_str() : g_init_err.c_str(); }

}  // extern "C"
