/*
 * CPU oracle for decode-time MoE layer execution over a router-following LRU
 * cache of expert slots.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg may call it; the product path never does.
 * Plain, slow, obviously correct C: no blocking, no fusion, no code shared with
 * the HIP library.
 *
 * Sources (the FreeToken pages):
 *  - pirouter.ai, "FreeToken x RTX 5090 -- 120B MoE が 127 tok/s、その請求書",
 *    section on how 65 GB runs on a 32 GB GPU: the offload backend keeps every
 *    expert in pinned host RAM and an LRU cache of expert slots on the GPU,
 *    misses are streamed over PCIe; the cache follows the router because a
 *    layer keeps choosing similar experts.
 *  - ai-hardware-zukan.com, "VRAMに収まらないMoEモデルのデコードが約2倍になった",
 *    section on how misses are made up for: the cache unit is the
 *    (layer, expert) pair and replacement removes the least recently used.
 *  - gaming-st.com DeepSeek page, section on the role of VRAM / MoE
 *    background: the cache is one global LRU expert cache.
 *  - blog.florigen.ai Qwen3.8-Flash-Next page, NVFP4 section: 4-bit weights are
 *    E2M1 elements with block scaling (MXFP4 uses the same E2M1 element).
 * Where the pages are silent the readings are: top-k on FP32 logits with ties
 * to the lower expert index, softmax over the k selected logits, SwiGLU
 * silu(gate)*up -> down with no bias, one global LRU over all slots with
 * unique per-access stamps, hits stamped before misses, lowest empty slot
 * before the least recently used one, cold start.
 *
 * Floating point: logits are FP32 in the fixed order below (they decide the
 * integer expert ids, so oracle and kernel take that decision in the same
 * precision and order); routing weights and the FFN are FP64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- dequant -- */

/* E2M1 (OCP MX 4-bit float): sign bit 3, exponent bits 2..1, mantissa bit 0.
 * exponent 0 is subnormal (value m/2), otherwise 2^(e-1) * (1 + m/2). */
double orc_e2m1_value(unsigned code) {
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E8M0 shared scale: 2^(E-127); E = 255 encodes NaN. */
double orc_e8m0_scale(unsigned e) {
    if ((e & 0xFFu) == 255u) return NAN;
    return ldexp(1.0, (int)(e & 0xFFu) - 127);
}

/* element j of an MXFP4 row: low nibble holds the even element */
static double mx_elem(const uint8_t* codes, const uint8_t* scales, size_t j) {
    unsigned byte = codes[j / 2];
    unsigned c = (j % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
    return orc_e2m1_value(c) * orc_e8m0_scale(scales[j / 32]);
}

void orc_dequant_row(const uint8_t* codes, const uint8_t* scales, int K, double* out) {
    for (int j = 0; j < K; ++j) out[j] = mx_elem(codes, scales, (size_t)j);
}

static float bf16_to_f32(uint16_t u) {
    uint32_t b = (uint32_t)u << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* ----------------------------------------------------------------- router -- */

/* Router logit z_e = W[e,:] . x in FP32 with a fixed summation order:
 * element i goes to lane (i/8) mod 64; each lane adds its own products in
 * increasing i starting from +0 (products of two bf16 values are exact in
 * FP32, so only the additions round); then, for d = 32,16,8,4,2,1, every lane
 * adds the value of lane (lane xor d); z_e is lane 0's value. */
void orc_router_logits(const uint16_t* W, const uint16_t* x, int E, int H, float* z) {
    for (int e = 0; e < E; ++e) {
        volatile float p[64];
        for (int l = 0; l < 64; ++l) p[l] = 0.0f;
        for (int i = 0; i < H; ++i) {
            int lane = (i / 8) % 64;
            float prod = bf16_to_f32(W[(size_t)e * H + i]) * bf16_to_f32(x[i]);
            p[lane] = p[lane] + prod;
        }
        for (int d = 32; d >= 1; d /= 2) {
            float q[64];
            for (int l = 0; l < 64; ++l) q[l] = p[l] + p[l ^ d];
            for (int l = 0; l < 64; ++l) p[l] = q[l];
        }
        z[e] = p[0];
    }
}

/* ids = the first k experts when sorted by logit descending, ties broken by
 * the lower expert index; w = softmax over the k selected logits (FP64). */
void orc_topk_softmax(const float* z, int E, int k, int32_t* ids, double* w) {
    char* taken = (char*)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || z[e] > z[best]) best = e;  /* strict: equal keeps the lower index */
        }
        taken[best] = 1;
        ids[j] = best;
    }
    free(taken);
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += exp((double)z[ids[j]] - (double)z[ids[0]]);
    for (int j = 0; j < k; ++j) w[j] = exp((double)z[ids[j]] - (double)z[ids[0]]) / den;
}

/* Routing for a batch of (layer, token) items: logits, ids and weights.
 * W: [L][E][H] bf16, X: [n_tok][H] bf16; item i uses layer items_layer[i] and
 * token items_tok[i]. */
void orc_route_batch(const uint16_t* W, const uint16_t* X, int E, int H, int k, int n_items,
                     const int32_t* items_layer, const int32_t* items_tok,
                     float* z_out /* [n][E] or NULL */, int32_t* ids_out, double* w_out) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int it = 0; it < n_items; ++it) {
        float* z = (float*)malloc(sizeof(float) * (size_t)E);
        orc_router_logits(W + (size_t)items_layer[it] * E * H, X + (size_t)items_tok[it] * H, E, H, z);
        orc_topk_softmax(z, E, k, ids_out + (size_t)it * k, w_out + (size_t)it * k);
        if (z_out) memcpy(z_out + (size_t)it * E, z, sizeof(float) * (size_t)E);
        free(z);
    }
}

/* -------------------------------------------------------------------- FFN -- */

static double silu(double g) { return g * (1.0 / (1.0 + exp(-g))); }

/* One expert on one token, FP64: g = Wg x, u = Wu x, a = silu(g) * u, y = Wd a.
 * blob is the logical MXFP4 layout (gate, up, down; codes then scales each). */
void orc_expert_ffn(const uint8_t* blob, int H, int I, const uint16_t* x_bf16, double* y) {
    const size_t hi = (size_t)H * (size_t)I;
    const uint8_t* gc = blob;
    const uint8_t* gs = gc + hi / 2;
    const uint8_t* uc = gs + hi / 32;
    const uint8_t* us = uc + hi / 2;
    const uint8_t* dc = us + hi / 32;
    const uint8_t* ds = dc + hi / 2;
    double* x = (double*)malloc(sizeof(double) * (size_t)H);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    for (int h = 0; h < H; ++h) x[h] = (double)bf16_to_f32(x_bf16[h]);
#pragma omp parallel for schedule(static)
    for (int i = 0; i < I; ++i) {
        const size_t c0 = (size_t)i * H / 2, s0 = (size_t)i * H / 32;
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            g += mx_elem(gc + c0, gs + s0, (size_t)h) * x[h];
            u += mx_elem(uc + c0, us + s0, (size_t)h) * x[h];
        }
        a[i] = silu(g) * u;
    }
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h) {
        const size_t c0 = (size_t)h * I / 2, s0 = (size_t)h * I / 32;
        double acc = 0.0;
        for (int i = 0; i < I; ++i) acc += mx_elem(dc + c0, ds + s0, (size_t)i) * a[i];
        y[h] = acc;
    }
    free(x);
    free(a);
}

/* ------------------------------------------------------------------ cache -- */

/* One global LRU over C slots keyed by (layer, expert) -> key = layer*E + expert.
 * slot_of[key] = slot or -1; key_of[slot] = key or -1; stamp[slot] = last use
 * or -1 (never); clock counts accesses.  Cold start: everything empty. */
typedef struct {
    int32_t L, E, C;
    int32_t* slot_of;
    int32_t* key_of;
    int64_t* stamp;
    int64_t clock;
    uint64_t hits, misses, evictions;
    uint64_t host;   /* misses left to the host in hybrid steps */
} orc_cache;

typedef struct {
    int32_t step, layer, expert, slot, hit, evicted_key;
} orc_trace_rec;

orc_cache* orc_cache_new(int L, int E, int C) {
    orc_cache* c = (orc_cache*)calloc(1, sizeof(orc_cache));
    c->L = L; c->E = E; c->C = C;
    c->slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)L * E);
    c->key_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    c->stamp = (int64_t*)malloc(sizeof(int64_t) * (size_t)C);
    for (size_t i = 0; i < (size_t)L * E; ++i) c->slot_of[i] = -1;
    for (int v = 0; v < C; ++v) { c->key_of[v] = -1; c->stamp[v] = -1; }
    return c;
}

void orc_cache_free(orc_cache* c) {
    if (!c) return;
    free(c->slot_of); free(c->key_of); free(c->stamp); free(c);
}

void orc_cache_counters(const orc_cache* c, uint64_t* out3) {
    out3[0] = c->hits; out3[1] = c->misses; out3[2] = c->evictions;
}

uint64_t orc_cache_host(const orc_cache* c) { return c->host; }

void orc_cache_state(const orc_cache* c, int32_t* slot_of, int32_t* key_of, int64_t* stamp) {
    if (slot_of) memcpy(slot_of, c->slot_of, sizeof(int32_t) * (size_t)c->L * c->E);
    if (key_of) memcpy(key_of, c->key_of, sizeof(int32_t) * (size_t)c->C);
    if (stamp) memcpy(stamp, c->stamp, sizeof(int64_t) * (size_t)c->C);
}

/* One step of layer `layer`: ids[n] are the experts the step's tokens selected
 * (duplicates allowed).  The requested set R is the ascending unique ids.
 * Hits (ascending) get fresh stamps first; then each miss (ascending) takes
 * the lowest-index empty slot, else the slot with the smallest stamp, evicting
 * its key.  slots_out[j] = slot holding ids[j] afterwards.  Records are
 * appended to trace (hits then misses); returns the number of records, or -1
 * if the step requests more distinct experts than there are slots. */
int orc_cache_step(orc_cache* c, int step, int layer, const int32_t* ids, int n,
                   int32_t* slots_out, orc_trace_rec* trace) {
    const int E = c->E;
    char* req = (char*)calloc((size_t)E, 1);
    for (int j = 0; j < n; ++j) req[ids[j]] = 1;
    int nreq = 0;
    for (int e = 0; e < E; ++e) nreq += req[e];
    if (nreq > c->C) { free(req); return -1; }
    int nrec = 0;
    for (int e = 0; e < E; ++e) {           /* hits, ascending */
        if (!req[e]) continue;
        int32_t v = c->slot_of[layer * E + e];
        if (v < 0) continue;
        c->stamp[v] = c->clock++;
        c->hits++;
        orc_trace_rec r = {step, layer, e, v, 1, -1};
        trace[nrec++] = r;
    }
    for (int e = 0; e < E; ++e) {           /* misses, ascending */
        if (!req[e] || c->slot_of[layer * E + e] >= 0) continue;
        int32_t v = -1;
        for (int s = 0; s < c->C; ++s) if (c->key_of[s] < 0) { v = s; break; }
        if (v < 0) {
            for (int s = 0; s < c->C; ++s) if (v < 0 || c->stamp[s] < c->stamp[v]) v = s;
        }
        int32_t old = c->key_of[v];
        if (old >= 0) { c->slot_of[old] = -1; c->evictions++; }
        c->key_of[v] = layer * E + e;
        c->slot_of[layer * E + e] = v;
        c->stamp[v] = c->clock++;
        c->misses++;
        orc_trace_rec r = {step, layer, e, v, 0, old};
        trace[nrec++] = r;
    }
    for (int j = 0; j < n; ++j) slots_out[j] = c->slot_of[layer * E + ids[j]];
    free(req);
    return nrec;
}

/* The hybrid split (ai-hardware-zukan.com FreeToken vs Ollama page, section on
 * the hybrid mode): of a step's m missing experts, q go over PCIe and m - q are
 * computed by the host so that both finish together.  With PCIe bandwidth B_P,
 * host expert bandwidth B_H and the host bandwidth left during the DMA taken
 * as B_H - B_P, q / B_P = (m - q) / (B_H - B_P) gives q = m B_P / B_H; with
 * B_H <= B_P nothing is left for the host and q = m.  Reading: q is rounded to
 * the nearest integer (halves up).  */
static int orc_split_q(int m, double pcie, double host) {
    if (m <= 0) return 0;
    if (!(host > pcie) || !(pcie > 0.0)) return m;
    int q = (int)floor((double)m * pcie / host + 0.5);
    return q < 0 ? 0 : (q > m ? m : q);
}

/* One hybrid step: as orc_cache_step, except that only the first q misses
 * (ascending expert id) are transferred into cache slots; the other m - q are
 * computed from host memory, take no slot and leave the cache as it was (no
 * victim, no stamp); their records carry slot -1 and evicted key -1, and
 * their slots_out entries are -1.  Reading: the transferred misses are the
 * lowest expert ids, the order in which misses are taken. */
int orc_cache_step_split(orc_cache* c, int step, int layer, const int32_t* ids, int n, double pcie,
                         double host, int32_t* slots_out, orc_trace_rec* trace) {
    const int E = c->E;
    char* req = (char*)calloc((size_t)E, 1);
    for (int j = 0; j < n; ++j) req[ids[j]] = 1;
    int nreq = 0, m = 0;
    for (int e = 0; e < E; ++e) {
        nreq += req[e];
        if (req[e] && c->slot_of[layer * E + e] < 0) ++m;
    }
    if (nreq > c->C) { free(req); return -1; }
    const int q = orc_split_q(m, pcie, host);
    int nrec = 0;
    for (int e = 0; e < E; ++e) {           /* hits, ascending */
        if (!req[e]) continue;
        int32_t v = c->slot_of[layer * E + e];
        if (v < 0) continue;
        c->stamp[v] = c->clock++;
        c->hits++;
        orc_trace_rec r = {step, layer, e, v, 1, -1};
        trace[nrec++] = r;
    }
    int mi = 0;
    for (int e = 0; e < E; ++e) {           /* misses, ascending: q transferred, then host */
        if (!req[e] || c->slot_of[layer * E + e] >= 0) continue;
        c->misses++;
        if (mi++ >= q) {
            c->host++;
            orc_trace_rec r = {step, layer, e, -1, 0, -1};
            trace[nrec++] = r;
            continue;
        }
        int32_t v = -1;
        for (int s2 = 0; s2 < c->C; ++s2) if (c->key_of[s2] < 0) { v = s2; break; }
        if (v < 0) {
            for (int s2 = 0; s2 < c->C; ++s2) if (v < 0 || c->stamp[s2] < c->stamp[v]) v = s2;
        }
        int32_t old = c->key_of[v];
        if (old >= 0) { c->slot_of[old] = -1; c->evictions++; }
        c->key_of[v] = layer * E + e;
        c->slot_of[layer * E + e] = v;
        c->stamp[v] = c->clock++;
        orc_trace_rec r = {step, layer, e, v, 0, old};
        trace[nrec++] = r;
    }
    for (int j = 0; j < n; ++j) slots_out[j] = c->slot_of[layer * E + ids[j]];
    free(req);
    return nrec;
}

/* ------------------------------------------------- static per-layer split -- */

/* The comparator the ai-hardware-zukan.com FreeToken vs Ollama page contrasts
 * with the router-following cache (section on how misses are made up for: a
 * fixed split of experts between GPU and host misses far more often).  Reading:
 * of the C GPU slots, R = C - T hold the first R (layer, expert) keys in pool
 * order for good (every layer before R / E whole, then part of the next), and
 * T transient slots take every other requested expert, one per access, in
 * rotation: a transient slot is a streaming buffer, not a cache -- only the
 * resident keys map to slots, a transient slot remembers its last occupant
 * (the evicted key of its next use), and every access to a non-resident key
 * streams it again.  Within a step the unique requested experts are taken
 * hits first, then misses, each ascending by expert id, as in the LRU cache. */
typedef struct {
    int L, E, C, T, R;
    int64_t tclock;     /* transient slots used so far */
    int32_t* slot_of;   /* [L*E]: the slot of a resident key, else -1 */
    int32_t* key_of;    /* [C]: resident key, or a transient slot's last occupant */
    uint64_t hits, misses, evictions;
} orc_static;

orc_static* orc_static_new(int L, int E, int C, int T) {
    if (T < 1 || T > C) return NULL;
    orc_static* c = (orc_static*)calloc(1, sizeof(orc_static));
    c->L = L; c->E = E; c->C = C; c->T = T; c->R = C - T;
    c->slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)L * E);
    c->key_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    for (int k = 0; k < L * E; ++k) c->slot_of[k] = k < c->R ? k : -1;
    for (int s = 0; s < C; ++s) c->key_of[s] = s < c->R && s < L * E ? s : -1;
    return c;
}

void orc_static_free(orc_static* c) {
    if (!c) return;
    free(c->slot_of); free(c->key_of); free(c);
}

void orc_static_counters(const orc_static* c, uint64_t* out3) {
    out3[0] = c->hits; out3[1] = c->misses; out3[2] = c->evictions;
}

void orc_static_state(const orc_static* c, int32_t* slot_of, int32_t* key_of) {
    memcpy(slot_of, c->slot_of, sizeof(int32_t) * (size_t)c->L * c->E);
    memcpy(key_of, c->key_of, sizeof(int32_t) * (size_t)c->C);
}

/* returns the number of trace records, or -1 when the step requests more
 * distinct experts than there are transient slots */
int orc_static_step(orc_static* c, int step, int layer, const int32_t* ids, int n,
                    int32_t* slots_out, orc_trace_rec* trace) {
    const int E = c->E;
    char* req = (char*)calloc((size_t)E, 1);
    for (int j = 0; j < n; ++j) req[ids[j]] = 1;
    int nmiss = 0;
    for (int e = 0; e < E; ++e) nmiss += req[e] && layer * E + e >= c->R;
    if (nmiss > c->T) { free(req); return -1; }
    int nrec = 0;
    for (int e = 0; e < E; ++e) {           /* hits: resident keys, ascending */
        const int key = layer * E + e;
        if (!req[e] || key >= c->R) continue;
        c->hits++;
        orc_trace_rec r = {step, layer, e, key, 1, -1};
        trace[nrec++] = r;
    }
    int32_t* step_slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; ++e) step_slot[e] = layer * E + e < c->R ? layer * E + e : -1;
    for (int e = 0; e < E; ++e) {           /* misses, ascending: next transient slot */
        const int key = layer * E + e;
        if (!req[e] || key < c->R) continue;
        const int32_t v = c->R + (int32_t)(c->tclock % c->T);
        c->tclock++;
        const int32_t old = c->key_of[v];
        if (old >= 0) c->evictions++;
        c->key_of[v] = key;
        step_slot[e] = v;
        c->misses++;
        orc_trace_rec r = {step, layer, e, v, 0, old};
        trace[nrec++] = r;
    }
    for (int j = 0; j < n; ++j) slots_out[j] = step_slot[ids[j]];
    free(step_slot);
    free(req);
    return nrec;
}
