// mk_api.cpp -- the C ABI declared in include/mk.h.
//
// Host side of one decode step: validate the inputs, look up or build the
// per-workgroup task lists, stage the step's positions, block tables and
// rotary table into device memory, and launch either the persistent
// megakernel (one cooperative launch) or the per-op chain (one launch per
// operation level). The host prepares the task lists, the device walks them
// ("Cohere Publishes One-Kernel Server for North Mini Code, Claims 1.58x vLLM
// Speedup", section "One resident program, many small tasks").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <new>
#include <set>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_common.h"
#include "mk_host.h"
#include "mk_kernels.h"
#include "mk_plan.h"

using namespace mk;

namespace {

thread_local std::string g_last_error;

mk_status fail(mk_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

#define MK_HIP(call)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess) return fail(MK_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
    } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxChunksCap = 512;
constexpr int kStageSlots = 4;

struct Layout {
    size_t err, banks, x, qkv, att_part, att_ml, att_out, rlogits, route_ids, route_w, act, rtab, ybuf, h2s, wtab, step,
        tasks, wg_off, level_tasks, trace, total;
    int64_t bank_words;
    int max_chunks;
    int64_t cap_tasks;
    int max_wg;
    size_t step_bytes;
};

ModelShape shape_of(const mk_dims& d, int max_chunks) {
    ModelShape s;
    s.L = d.n_layers;
    s.H = d.hidden;
    s.Hq = d.n_q_heads;
    s.Hkv = d.n_kv_heads;
    s.D = d.head_dim;
    s.E = d.n_experts;
    s.K = d.top_k;
    s.I = d.moe_inter;
    s.V = d.vocab;
    s.P = d.page_size;
    s.max_batch = d.max_batch;
    s.max_pages = d.max_pages_per_seq;
    s.max_chunks = max_chunks;
    return s;
}

int max_chunks_for(const mk_dims& d) {
    const int64_t ctx = (int64_t)d.max_pages_per_seq * d.page_size;
    return (int)std::min<int64_t>(kMaxChunksCap, (ctx + 127) / 128);
}

// Smallest batch that runs the matrix-core schedule (mk_options.mfma_min_batch).
int mm_min_of(const mk_options& o) { return o.mfma_min_batch > 0 ? o.mfma_min_batch : kMaxBatchValu + 1; }

// Host-checkable support conditions. Empty string = supported.
std::string check_dims(const mk_dims& d, int mm_min = kMaxBatchValu + 1) {
    if (d.n_layers <= 0 || d.hidden <= 0 || d.n_q_heads <= 0 || d.n_kv_heads <= 0 || d.n_experts <= 0 ||
        d.top_k <= 0 || d.moe_inter <= 0 || d.vocab <= 0 || d.max_batch <= 0 || d.max_pages_per_seq <= 0 ||
        d.n_pages <= 0)
        return "all dims must be positive";
    if (d.page_size != 16) return "page_size must be 16";
    if (d.head_dim != 64 && d.head_dim != 128) return "head_dim must be 64 or 128";
    if (d.n_q_heads % d.n_kv_heads != 0 || d.n_q_heads / d.n_kv_heads > 16)
        return "n_q_heads must be a multiple of n_kv_heads, at most 16 per KV head";
    if (d.top_k > 8 || d.top_k > d.n_experts) return "top_k must be <= 8 and <= n_experts";
    if (d.n_experts > 256) return "n_experts must be <= 256";
    if (d.hidden % 8 || d.moe_inter % 8) return "hidden and moe_inter must be multiples of 8";
    if (d.max_batch > kMaxBatchMM) return "max_batch above 64";
    if (d.max_batch >= mm_min &&
        (d.hidden % 128 || (d.n_q_heads * d.head_dim) % 128 || d.moe_inter % 32))
        return "the matrix-core schedule needs hidden and n_q_heads*head_dim multiples of 128, moe_inter of 32";
    if (find_shape(d.hidden, d.n_q_heads * d.head_dim, d.moe_inter, d.head_dim, d.n_experts) < 0)
        return "no kernel build for this (hidden, attention width, expert width, head_dim)";
    return std::string();
}

TileConfig tile_config(const mk_options& o) {
    TileConfig c;
    c.chunk = o.split_kv_tokens;
    c.shared_levels = o.shared_levels;
    c.mm_min_batch = mm_min_of(o);
    c.mm_row_blocks = o.mm_row_blocks;
    return c;
}

Layout make_layout(const mk_dims& d, const mk_options& o, int max_wg) {
    Layout L;
    const int G = d.n_q_heads / d.n_kv_heads;
    (void)G;
    L.max_chunks = max_chunks_for(d);
    const ModelShape s = shape_of(d, L.max_chunks);
    const TileConfig cfg = tile_config(o);
    const CounterLayout cl{d.n_layers, d.n_kv_heads, d.max_batch};
    L.bank_words = cl.bank_words();
    L.cap_tasks = max_tasks(s, cfg, max_wg);
    L.max_wg = max_wg;
    const int64_t B = d.max_batch, H = d.hidden, QKVD = (int64_t)(d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o2 = off;
        off = align256(off + bytes);
        return o2;
    };
    L.err = take(256);
    L.banks = take(2 * (size_t)L.bank_words * 4);
    // exchange buffers: one 256-byte-padded slice per layer (see pad64)
    const size_t Ln = (size_t)d.n_layers;
    L.x = take((size_t)(2 * d.n_layers + 1) * pad64(B * H) * 4);
    L.qkv = take(Ln * pad64(B * QKVD) * 4);
    L.att_part = take(Ln * pad64(B * d.n_q_heads * (int64_t)L.max_chunks * d.head_dim) * 4);
    L.att_ml = take(Ln * B * d.n_q_heads * pad64(2 * (int64_t)L.max_chunks) * 4);
    L.att_out = take(Ln * pad64(B * d.n_q_heads * d.head_dim) * 4);
    L.rlogits = take(Ln * pad64(B * d.n_experts) * 4);
    L.route_ids = take((size_t)d.n_layers * B * d.top_k * 4);
    L.route_w = take((size_t)d.n_layers * B * d.top_k * 4);
    L.act = take(Ln * pad64(B * d.top_k * d.moe_inter) * 4);
    // batches of 3+: routing tables and per-(token, rank) expert outputs
    const bool mm = d.max_batch >= mm_min_of(o);
    L.rtab = take(mm ? Ln * rtab_words(d.n_experts, d.top_k, d.max_batch) * 4 : 0);
    L.ybuf = take(mm ? Ln * pad64(B * d.top_k * H) * 4 : 0);
    L.h2s = take(mm ? (Ln + 1) * pad64(B * H) * 4 : 0);   // + the final norm's output
    L.wtab = take((size_t)d.n_layers * W_NKINDS * 8);
    // per-step arrays: positions, chunk counts, rotary table, block tables
    L.step_bytes = align256((size_t)B * 4) * 2 + align256((size_t)B * d.head_dim * 4) +
                   align256((size_t)B * d.max_pages_per_seq * 4) + align256((size_t)B * 8);
    L.step = take(L.step_bytes);
    L.tasks = take((size_t)L.cap_tasks * sizeof(Task));
    L.wg_off = take((size_t)(max_wg + 1) * 4);
    L.level_tasks = take((size_t)L.cap_tasks * sizeof(Task));
    L.trace = o.trace ? take((size_t)L.cap_tasks * 64) : off;
    L.total = off;
    return L;
}

}  // namespace

namespace mk {
mk_status host_fail(mk_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}
}  // namespace mk

struct mk_handle {
    mk_dims d;
    mk_options o;
    int device = 0;
    int n_cu = 0;
    int wg_per_cu = 0;
    int n_wg = 0;
    int shape = -1;
    int mm_min = kMaxBatchValu + 1;   // smallest batch on the matrix-core kernels
    // [1], [2]: the one- and two-token kernels; [0]: the matrix-core kernels (if max_batch >= mm_min)
    KernelPair kern[kNbCount];
    size_t lds_bytes[kNbCount] = {};
    int general[kNbCount] = {};
    Layout lay;
    char* ws = nullptr;
    int bank = 0;
    Params base;
    std::vector<double> inv_freq;
    // plan cache (the device holds the plan of the last key)
    bool have_plan = false;
    int plan_B = 0, plan_chunk = 0;
    std::vector<int32_t> plan_chunks;   // attention chunks the plan reserves per sequence
    Plan plan;
    // pinned staging ring for per-step arrays and plans
    char* stage[kStageSlots] = {nullptr, nullptr, nullptr, nullptr};
    hipEvent_t stage_ev[kStageSlots];
    int stage_next = 0;
    char* plan_stage = nullptr;
    size_t plan_stage_bytes = 0;
    hipEvent_t plan_ev;
    bool plan_ev_used = false;
    int64_t last_n_tasks = 0;
    bool last_perop = false;  // the last step ran the per-op launches
    hipEvent_t t_begin, t_end;
    bool timed = false;
    // the last step's completion on the stream it was enqueued on: a step
    // enqueued on another stream waits for it (the workspace's per-step
    // arrays and task table are single-buffered)
    hipEvent_t step_ev;
    bool step_ev_used = false;
    hipStream_t last_stream = nullptr;
};

extern "C" {

const char* mk_last_error(void) { return g_last_error.c_str(); }

size_t mk_kv_pool_bytes(const mk_dims* d) {
    if (!d || d->n_layers <= 0 || d->n_pages <= 0) return 0;
    return (size_t)d->n_layers * (size_t)d->n_pages * d->n_kv_heads * d->page_size * d->head_dim * 2;
}

size_t mk_workspace_bytes(const mk_dims* d, const mk_options* o) {
    if (!d) return 0;
    mk_options oo;
    memset(&oo, 0, sizeof oo);
    if (o) oo = *o;
    if (!check_dims(*d, mm_min_of(oo)).empty()) return 0;
    // sized for up to 8 workgroups on each of 256 compute units
    return make_layout(*d, oo, 256 * 8).total;
}

mk_status mk_create(const mk_dims* dims, const mk_weights* w, void* k_pool, void* v_pool, void* workspace,
                    size_t workspace_bytes, const mk_options* opts, int device, mk_handle** out) {
    try {
        if (!dims || !w || !k_pool || !v_pool || !workspace || !out) return fail(MK_ERR_INVALID, "null argument");
        *out = nullptr;
        mk_options o;
        memset(&o, 0, sizeof o);
        if (opts) o = *opts;
        const std::string why = check_dims(*dims, mm_min_of(o));
        if (!why.empty()) return fail(MK_ERR_UNSUPPORTED, "%s", why.c_str());
        if (o.mode != MK_MODE_MEGAKERNEL && o.mode != MK_MODE_PEROP) return fail(MK_ERR_INVALID, "bad mode");
        if (o.split_kv_tokens < 0 || o.split_kv_tokens % 64) return fail(MK_ERR_INVALID, "split_kv_tokens must be a multiple of 64");
        if (o.mfma_min_batch < 0 || o.mfma_min_batch > kMaxBatchValu + 1)
            return fail(MK_ERR_INVALID, "mfma_min_batch must be 0 (default) or 1..%d", kMaxBatchValu + 1);
        if (o.mm_row_blocks < 0 || o.mm_row_blocks > kMmMaxRowBlocks)
            return fail(MK_ERR_INVALID, "mm_row_blocks must be 0 (choose) or 1..%d", kMmMaxRowBlocks);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return fail(MK_ERR_INVALID, "workspace not 256-byte aligned");
        const mk_dims& d = *dims;
        if (!w->embed || !w->lm_head || !w->final_norm || !w->attn_norm || !w->wqkv || !w->wo || !w->ffn_norm ||
            !w->router || !w->w_gate || !w->w_up || !w->w_down)
            return fail(MK_ERR_INVALID, "null weight pointer");
        for (int l = 0; l < d.n_layers; ++l)
            if (!w->attn_norm[l] || !w->wqkv[l] || !w->wo[l] || !w->ffn_norm[l] || !w->router[l] || !w->w_gate[l] ||
                !w->w_up[l] || !w->w_down[l])
                return fail(MK_ERR_INVALID, "null weight pointer in layer %d", l);

        MK_HIP(hipSetDevice(device));
        hipDeviceProp_t prop;
        MK_HIP(hipGetDeviceProperties(&prop, device));
        std::unique_ptr<mk_handle> h(new mk_handle());
        h->d = d;
        h->o = o;
        h->device = device;
        h->n_cu = o.n_cu_override > 0 ? o.n_cu_override : prop.multiProcessorCount;
        h->shape = find_shape(d.hidden, d.n_q_heads * d.head_dim, d.moe_inter, d.head_dim, d.n_experts);
        h->mm_min = mm_min_of(o);
        const bool mm = d.max_batch >= h->mm_min;
        // kernels a step may launch: the matrix-core ones (one or two row
        // blocks per expert tile) for batches >= mm_min, the one- and
        // two-token ones below it
        auto used = [&](int nb) {
            return nb == 0 || nb == kNbMmWide ? mm : (nb <= d.max_batch && nb < h->mm_min);
        };
        for (int nb = 0; nb < kNbCount; ++nb)
            if (used(nb) && !get_kernels(h->shape, nb, &h->kern[nb])) return fail(MK_ERR_UNSUPPORTED, "no kernels");

        // LDS: general region (attention tiles + query fragments, combine
        // coefficients, or the down tile's staged activations and outputs),
        // routing results, per-tile scalars.
        const int G = d.n_q_heads / d.n_kv_heads;
        const int max_chunks = max_chunks_for(d);
        // attention: the new token's k and v (bf16), per-wave (m, l) and o^T,
        // the merge factors and per-head (max, sum)
        const size_t attn = (size_t)4 * d.head_dim + (size_t)2 * 4 * 16 * 4 + (size_t)4 * 16 * (d.head_dim + 1) * 4 +
                            (size_t)(4 * 16 + 2 * 16) * 4;
        const size_t comb = (size_t)(16 + max_chunks + 4 + 1024) * 4;
        // down tile: its gate/up activations [B][k][I] fp32 at the start of
        // the general region, its output staging at the end
        const size_t ystage = (size_t)2 * 8 * 64 * 4;
        const size_t act = (size_t)std::min(d.max_batch, kMaxBatchValu) * d.top_k * d.moe_inter * 4;
        const size_t gen_v = align256(std::max(std::max(attn, comb), act) + ystage);
        // matrix-core tiles: block-product partials or the routing tile's tables
        const size_t gen_m = align256(std::max(std::max(attn, comb), (size_t)std::max(kMmLdsBytes, kRouteLdsBytes)));
        int occ = 1 << 30;
        for (int nb = 0; nb < kNbCount; ++nb) {
            if (!used(nb)) continue;
            h->general[nb] = (int)(nb == 0 || nb == kNbMmWide ? gen_m : gen_v);
            h->lds_bytes[nb] = h->general[nb] + 1024 + 1024;
            if (h->lds_bytes[nb] > (size_t)prop.sharedMemPerBlock && h->lds_bytes[nb] > 160 * 1024)
                return fail(MK_ERR_UNSUPPORTED, "needs %zu bytes of LDS", h->lds_bytes[nb]);
            MK_HIP(set_kernel_attributes(h->kern[nb], h->lds_bytes[nb]));
            int o2 = 0;
            MK_HIP(persistent_occupancy(h->kern[nb], h->lds_bytes[nb], &o2));
            occ = std::min(occ, o2);
        }
        if (occ < 1) return fail(MK_ERR_UNSUPPORTED, "persistent kernel does not fit on a compute unit");
        h->wg_per_cu = o.wg_per_cu > 0 ? std::min(o.wg_per_cu, occ) : std::min(occ, 2);
        h->n_wg = h->n_cu * h->wg_per_cu;
        if (h->n_wg > 256 * 8) return fail(MK_ERR_UNSUPPORTED, "too many workgroups");

        h->lay = make_layout(d, o, 256 * 8);
        if (workspace_bytes < h->lay.total)
            return fail(MK_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", workspace_bytes, h->lay.total);
        h->ws = static_cast<char*>(workspace);

        // weight pointer table
        std::vector<uint64_t> wtab((size_t)d.n_layers * W_NKINDS, 0);
        for (int l = 0; l < d.n_layers; ++l) {
            uint64_t* r = &wtab[(size_t)l * W_NKINDS];
            r[W_ATTN_NORM] = (uint64_t)(uintptr_t)w->attn_norm[l];
            r[W_QKV] = (uint64_t)(uintptr_t)w->wqkv[l];
            r[W_O] = (uint64_t)(uintptr_t)w->wo[l];
            r[W_FFN_NORM] = (uint64_t)(uintptr_t)w->ffn_norm[l];
            r[W_ROUTER] = (uint64_t)(uintptr_t)w->router[l];
            r[W_GATE] = (uint64_t)(uintptr_t)w->w_gate[l];
            r[W_UP] = (uint64_t)(uintptr_t)w->w_up[l];
            r[W_DOWN] = (uint64_t)(uintptr_t)w->w_down[l];
            r[W_RBIAS] = w->router_bias ? (uint64_t)(uintptr_t)w->router_bias[l] : 0;
        }
        MK_HIP(hipMemcpy(h->ws + h->lay.wtab, wtab.data(), wtab.size() * 8, hipMemcpyHostToDevice));
        // clear error word and both counter banks
        MK_HIP(launch_fill(reinterpret_cast<uint32_t*>(h->ws + h->lay.err), 64, 0u, nullptr));
        MK_HIP(launch_fill(reinterpret_cast<uint32_t*>(h->ws + h->lay.banks), 2 * h->lay.bank_words, 0u, nullptr));
        MK_HIP(hipDeviceSynchronize());

        // rotary inverse frequencies theta^(-2i/D), float64
        h->inv_freq.resize(d.head_dim / 2);
        for (int i = 0; i < d.head_dim / 2; ++i)
            h->inv_freq[i] = std::pow((double)d.rope_theta, -2.0 * i / (double)d.head_dim);

        // kernel parameter block: constant part
        Params& p = h->base;
        memset(&p, 0, sizeof p);
        p.L = d.n_layers;
        p.H = d.hidden;
        p.Hq = d.n_q_heads;
        p.Hkv = d.n_kv_heads;
        p.D = d.head_dim;
        p.E = d.n_experts;
        p.K = d.top_k;
        p.I = d.moe_inter;
        p.V = d.vocab;
        p.P = d.page_size;
        p.G = G;
        p.QKVD = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
        p.eps = d.rms_eps;
        p.inv_h = 1.0f / (float)d.hidden;
        p.attn_scale = (float)(1.0 / std::sqrt((double)d.head_dim));
        p.max_batch = d.max_batch;
        p.max_pages = d.max_pages_per_seq;
        p.max_chunks = max_chunks;
        p.n_pages = d.n_pages;
        p.trace_on = o.trace ? 1 : 0;
        const int64_t wd_ns = o.watchdog_ns > 0 ? o.watchdog_ns : 2000000000LL;
        p.watchdog_ticks = wd_ns / 10;  // 100 MHz constant clock
        p.embed = static_cast<const uint16_t*>(w->embed);
        p.lm_head = static_cast<const uint16_t*>(w->lm_head);
        p.final_norm = static_cast<const uint16_t*>(w->final_norm);
        p.wtab = reinterpret_cast<const uint64_t*>(h->ws + h->lay.wtab);
        p.k_pool = static_cast<uint16_t*>(k_pool);
        p.v_pool = static_cast<uint16_t*>(v_pool);
        char* st = h->ws + h->lay.step;
        const int64_t B = d.max_batch;
        p.positions = reinterpret_cast<const int32_t*>(st);
        p.seq_chunk = reinterpret_cast<const int32_t*>(st + align256(B * 4));
        p.rope = reinterpret_cast<const float*>(st + 2 * align256(B * 4));
        p.block_tables = reinterpret_cast<const int32_t*>(st + 2 * align256(B * 4) + align256(B * d.head_dim * 4));
        p.seq_first = reinterpret_cast<const int32_t*>(st + 2 * align256(B * 4) + align256(B * d.head_dim * 4) +
                                                       align256(B * d.max_pages_per_seq * 4));
        p.x = reinterpret_cast<float*>(h->ws + h->lay.x);
        p.qkv = reinterpret_cast<float*>(h->ws + h->lay.qkv);
        p.att_part = reinterpret_cast<float*>(h->ws + h->lay.att_part);
        p.att_ml = reinterpret_cast<float*>(h->ws + h->lay.att_ml);
        p.att_out = reinterpret_cast<float*>(h->ws + h->lay.att_out);
        p.rlogits = reinterpret_cast<float*>(h->ws + h->lay.rlogits);
        p.route_ids = reinterpret_cast<int32_t*>(h->ws + h->lay.route_ids);
        p.route_w = reinterpret_cast<float*>(h->ws + h->lay.route_w);
        p.act = reinterpret_cast<float*>(h->ws + h->lay.act);
        p.rtab = reinterpret_cast<int32_t*>(h->ws + h->lay.rtab);
        p.ybuf = reinterpret_cast<float*>(h->ws + h->lay.ybuf);
        p.h2s = reinterpret_cast<float*>(h->ws + h->lay.h2s);
        p.bank_words = h->lay.bank_words;
        p.cl = CounterLayout{d.n_layers, d.n_kv_heads, d.max_batch};
        p.err = reinterpret_cast<int32_t*>(h->ws + h->lay.err);
        p.trace = o.trace ? reinterpret_cast<uint64_t*>(h->ws + h->lay.trace) : nullptr;

        for (int i = 0; i < kStageSlots; ++i) {
            MK_HIP(hipHostMalloc(reinterpret_cast<void**>(&h->stage[i]), h->lay.step_bytes, hipHostMallocDefault));
            MK_HIP(hipEventCreateWithFlags(&h->stage_ev[i], hipEventDisableTiming));
            MK_HIP(hipEventRecord(h->stage_ev[i], nullptr));
        }
        MK_HIP(hipEventCreateWithFlags(&h->plan_ev, hipEventDisableTiming));
        MK_HIP(hipEventCreateWithFlags(&h->step_ev, hipEventDisableTiming));
        // plan staging for the largest plan (both task orders and the
        // offsets), so that no step allocates pinned memory
        h->plan_stage_bytes = (size_t)2 * h->lay.cap_tasks * sizeof(Task) + (size_t)(h->lay.max_wg + 1) * 4;
        MK_HIP(hipHostMalloc(reinterpret_cast<void**>(&h->plan_stage), h->plan_stage_bytes, hipHostMallocDefault));
        if (o.time_kernels) {
            MK_HIP(hipEventCreate(&h->t_begin));
            MK_HIP(hipEventCreate(&h->t_end));
        }
        *out = h.release();
        return MK_OK;
    } catch (const std::bad_alloc&) {
        return fail(MK_ERR_CAPACITY, "host allocation failed");
    } catch (...) {
        return fail(MK_ERR_INVALID, "unexpected exception in mk_create");
    }
}

mk_status mk_set_mode(mk_handle* h, int32_t mode) {
    if (!h) return fail(MK_ERR_INVALID, "null handle");
    if (mode != MK_MODE_MEGAKERNEL && mode != MK_MODE_PEROP) return fail(MK_ERR_INVALID, "bad mode");
    h->o.mode = mode;
    return MK_OK;
}

static mk_status upload_plan(mk_handle* h, hipStream_t stream) {
    const Plan& P = h->plan;
    // the megakernel's table (lists, then the pools of shared levels) and the
    // per-op table (every tile, level by level; no claim tasks)
    const size_t nt = P.tasks.size(), nl = P.level_tasks.size();
    const size_t bytes = (nt + nl) * sizeof(Task) + (P.wg_off.size()) * 4;
    if (h->plan_ev_used) MK_HIP(hipEventSynchronize(h->plan_ev));
    if (bytes > h->plan_stage_bytes) return fail(MK_ERR_CAPACITY, "plan of %zu bytes exceeds its staging", bytes);
    char* s = h->plan_stage;
    memcpy(s, P.tasks.data(), nt * sizeof(Task));
    memcpy(s + nt * sizeof(Task), P.level_tasks.data(), nl * sizeof(Task));
    memcpy(s + (nt + nl) * sizeof(Task), P.wg_off.data(), P.wg_off.size() * 4);
    MK_HIP(hipMemcpyAsync(h->ws + h->lay.tasks, s, nt * sizeof(Task), hipMemcpyHostToDevice, stream));
    MK_HIP(hipMemcpyAsync(h->ws + h->lay.level_tasks, s + nt * sizeof(Task), nl * sizeof(Task), hipMemcpyHostToDevice,
                          stream));
    MK_HIP(hipMemcpyAsync(h->ws + h->lay.wg_off, s + (nt + nl) * sizeof(Task), P.wg_off.size() * 4,
                          hipMemcpyHostToDevice, stream));
    MK_HIP(hipEventRecord(h->plan_ev, stream));
    h->plan_ev_used = true;
    return MK_OK;
}

}  // extern "C"

// One step over `batch` rows (mk_decode_step, mk_forward_step). With
// multi_token, adjacent rows of equal seq_id form a run at consecutive
// positions: each row's first[] entry names the run's first position and the
// row that feeds it; otherwise every row is its own run.
static mk_status step_impl(mk_handle* h, int32_t batch, const int32_t* seq_ids, const int32_t* positions,
                           const int32_t* block_tables, const int32_t* tokens, float* logits, void* stream_,
                           bool multi_token, bool use_scratch = false) {
    try {
        if (!h) return fail(MK_ERR_INVALID, "null handle");
        if (!positions || !block_tables || !tokens || !logits) return fail(MK_ERR_INVALID, "null argument");
        const mk_dims& d = h->d;
        if (batch <= 0) return fail(MK_ERR_INVALID, "batch must be positive");
        if (batch > d.max_batch) return fail(MK_ERR_CAPACITY, "batch %d > max_batch %d", batch, d.max_batch);
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        // the static scratch: counter banks and exchange buffers, laid out as
        // in the workspace (regions banks .. wtab)
        char* scratch = nullptr;
        const size_t scratch_need = h->lay.wtab - h->lay.banks;
        if (use_scratch) {
            if (scratch_need > kScratchBytes)
                return fail(MK_ERR_CAPACITY, "this handle's step needs %zu bytes of scratch, the library holds %zu",
                            scratch_need, (size_t)kScratchBytes);
            void* sp = nullptr;
            MK_HIP(scratch_address(h->device, &sp));
            scratch = static_cast<char*>(sp);
        }
        std::vector<int32_t> first_row(batch);
        for (int b = 0; b < batch; ++b) first_row[b] = b;
        if (multi_token) {
            if (!seq_ids) return fail(MK_ERR_INVALID, "a multi-token step needs seq_ids");
            std::set<int32_t> seen;
            for (int b = 0; b < batch; ++b) {
                if (b > 0 && seq_ids[b] == seq_ids[b - 1]) {
                    if (positions[b] != positions[b - 1] + 1)
                        return fail(MK_ERR_INVALID, "rows %d and %d of sequence %d are not at consecutive positions",
                                    b - 1, b, seq_ids[b]);
                    first_row[b] = first_row[b - 1];
                } else if (!seen.insert(seq_ids[b]).second) {
                    return fail(MK_ERR_INVALID, "the rows of sequence %d are not adjacent", seq_ids[b]);
                }
            }
        } else if (seq_ids) {
            std::set<int32_t> ids(seq_ids, seq_ids + batch);
            if ((int)ids.size() != batch) return fail(MK_ERR_INVALID, "seq_ids must be distinct");
        }
        const int P = d.page_size;
        for (int b = 0; b < batch; ++b) {
            const int pos = positions[b];
            if (pos < 0) return fail(MK_ERR_INVALID, "negative position for sequence %d", b);
            if ((int64_t)pos / P >= d.max_pages_per_seq)
                return fail(MK_ERR_CAPACITY, "position %d of sequence %d needs more than %d pages", pos, b,
                            d.max_pages_per_seq);
            const int32_t* bt = block_tables + (int64_t)b * d.max_pages_per_seq;
            for (int i = 0; i <= pos / P; ++i)
                if (bt[i] < 0 || bt[i] >= d.n_pages)
                    return fail(MK_ERR_BAD_PAGE, "sequence %d block %d names page %d (pool has %lld)", b, i, bt[i],
                                (long long)d.n_pages);
            // rows of one sequence share its pages: the earlier row's table
            // must agree with this one over every page it uses
            if (first_row[b] != b) {
                const int32_t* prev = bt - d.max_pages_per_seq;
                for (int i = 0; i <= positions[b - 1] / P; ++i)
                    if (prev[i] != bt[i])
                        return fail(MK_ERR_INVALID, "rows %d and %d of one sequence differ at block %d", b - 1, b, i);
            }
        }

        // Order this step after the previous one when the caller switched
        // streams. Inside a stream capture the caller orders the replays
        // (capture requires the work before it to be complete), so nothing
        // is waited on or recorded there.
        hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
        MK_HIP(hipStreamIsCapturing(stream, &capture));
        const bool capturing = capture != hipStreamCaptureStatusNone;
        if (!capturing && h->step_ev_used && stream != h->last_stream)
            MK_HIP(hipStreamWaitEvent(stream, h->step_ev, 0));

        // plan: reused while it still covers every sequence. A plan reserves
        // attention chunks for kLookahead more tokens of each sequence (the
        // chunks past a sequence's tokens run as empty tiles), and a
        // sequence that outgrows its reservation (one that joined in the slot
        // of a shorter one) stretches its own chunk length up to 2x the
        // plan's. The plan is rebuilt when the batch size changes, a sequence
        // would need more than that, the chunk length drifts a factor 2 from
        // the balanced one, or reserved chunks exceed twice the needed ones.
        const ModelShape s = shape_of(d, h->lay.max_chunks);
        const TileConfig cfg = tile_config(h->o);
        const int ideal = choose_chunk(s, h->n_wg, batch, positions, cfg.chunk);
        bool reuse = h->have_plan && h->plan_B == batch;
        if (reuse && (cfg.chunk > 0 ? h->plan_chunk != ideal
                                     : (h->plan_chunk > 2 * ideal || 2 * h->plan_chunk < ideal)))
            reuse = false;
        int chunk = reuse ? h->plan_chunk : ideal;
        auto seq_chunk = [&](int b) {
            const int per = (positions[b] + h->plan_chunks[b]) / h->plan_chunks[b];   // ceil((pos + 1) / n)
            return std::max(chunk, (per + 63) / 64 * 64);
        };
        if (reuse) {
            int64_t planned = 0, needed = 0;
            for (int b = 0; b < batch && reuse; ++b) {
                if (seq_chunk(b) > 2 * chunk) reuse = false;
                planned += h->plan_chunks[b];
                needed += (positions[b] + chunk) / chunk;
            }
            if (planned > 2 * needed + batch) reuse = false;
        }
        if (!reuse) {
            constexpr int kLookahead = 256;
            chunk = ideal;
            std::vector<int32_t> ppos(batch);
            for (int b = 0; b < batch; ++b)
                ppos[b] = std::max(positions[b], std::min(positions[b] + kLookahead, h->lay.max_chunks * chunk - 1));
            TileConfig c2 = cfg;
            c2.chunk = chunk;
            const std::string err = build_plan(s, c2, h->n_wg, batch, ppos.data(), &h->plan);
            if (!err.empty()) return fail(MK_ERR_CAPACITY, "plan: %s", err.c_str());
            if (h->o.validate_plans) {
                const std::string verr = validate_plan(s, h->plan);
                if (!verr.empty()) {
                    h->have_plan = false;
                    return fail(MK_ERR_INVALID, "plan invalid: %s", verr.c_str());
                }
            }
            if ((int64_t)h->plan.tasks.size() > h->lay.cap_tasks) return fail(MK_ERR_CAPACITY, "too many tasks");
            mk_status st = upload_plan(h, stream);
            if (st != MK_OK) return st;
            chunk = h->plan.chunk;
            h->have_plan = true;
            h->plan_B = batch;
            h->plan_chunk = chunk;
            h->plan_chunks = h->plan.n_chunks;
        }
        std::vector<int32_t> nch(batch);
        for (int b = 0; b < batch; ++b) nch[b] = seq_chunk(b);

        // per-step arrays through a pinned staging ring
        const int slot = h->stage_next;
        h->stage_next = (h->stage_next + 1) % kStageSlots;
        MK_HIP(hipEventSynchronize(h->stage_ev[slot]));
        char* stg = h->stage[slot];
        const int64_t B = d.max_batch;
        memset(stg, 0, h->lay.step_bytes);
        int32_t* spos = reinterpret_cast<int32_t*>(stg);
        int32_t* snch = reinterpret_cast<int32_t*>(stg + align256(B * 4));   // per-sequence chunk lengths
        float* srope = reinterpret_cast<float*>(stg + 2 * align256(B * 4));
        int32_t* sbt = reinterpret_cast<int32_t*>(stg + 2 * align256(B * 4) + align256(B * d.head_dim * 4));
        int32_t* sfirst = reinterpret_cast<int32_t*>(stg + 2 * align256(B * 4) + align256(B * d.head_dim * 4) +
                                                     align256(B * d.max_pages_per_seq * 4));
        for (int b = 0; b < batch; ++b) {
            spos[b] = positions[b];
            snch[b] = nch[b];
            sfirst[2 * b] = positions[first_row[b]];
            sfirst[2 * b + 1] = first_row[b];
            for (int i = 0; i < d.head_dim / 2; ++i) {
                const double ang = (double)positions[b] * h->inv_freq[i];
                srope[(int64_t)b * d.head_dim + 2 * i] = (float)std::cos(ang);
                srope[(int64_t)b * d.head_dim + 2 * i + 1] = (float)std::sin(ang);
            }
            memcpy(sbt + (int64_t)b * d.max_pages_per_seq, block_tables + (int64_t)b * d.max_pages_per_seq,
                   (size_t)d.max_pages_per_seq * 4);
        }
        MK_HIP(hipMemcpyAsync(h->ws + h->lay.step, stg, h->lay.step_bytes, hipMemcpyHostToDevice, stream));
        MK_HIP(hipEventRecord(h->stage_ev[slot], stream));

        Params p = h->base;
        p.B = batch;
        p.chunk = chunk;
        p.tokens = tokens;
        p.logits = logits;
        uint32_t* banks = reinterpret_cast<uint32_t*>(h->ws + h->lay.banks);
        p.ctr = banks + (int64_t)h->bank * h->lay.bank_words;
        p.ctr_other = banks + (int64_t)(1 - h->bank) * h->lay.bank_words;
        if (use_scratch) {
            // every pointer into banks .. wtab moves to the same offset in the
            // scratch; both counter banks start at zero (a fill kernel, so the
            // step can be captured), the step uses bank 0
            auto at = [&](size_t off) { return scratch + (off - h->lay.banks); };
            banks = reinterpret_cast<uint32_t*>(at(h->lay.banks));
            MK_HIP(launch_fill(banks, 2 * h->lay.bank_words, 0u, stream));
            p.ctr = banks;
            p.ctr_other = banks + h->lay.bank_words;
            p.x = reinterpret_cast<float*>(at(h->lay.x));
            p.qkv = reinterpret_cast<float*>(at(h->lay.qkv));
            p.att_part = reinterpret_cast<float*>(at(h->lay.att_part));
            p.att_ml = reinterpret_cast<float*>(at(h->lay.att_ml));
            p.att_out = reinterpret_cast<float*>(at(h->lay.att_out));
            p.rlogits = reinterpret_cast<float*>(at(h->lay.rlogits));
            p.route_ids = reinterpret_cast<int32_t*>(at(h->lay.route_ids));
            p.route_w = reinterpret_cast<float*>(at(h->lay.route_w));
            p.act = reinterpret_cast<float*>(at(h->lay.act));
            p.rtab = reinterpret_cast<int32_t*>(at(h->lay.rtab));
            p.ybuf = reinterpret_cast<float*>(at(h->lay.ybuf));
            p.h2s = reinterpret_cast<float*>(at(h->lay.h2s));
        }
        if (h->o.poison_exchange) {
            // NaN in fp32 and in both BF16 halves; the integer routing tables
            // and the host-read routing output are left alone
            const uint32_t nan2 = 0x7FC07FC0u;
            const Layout& L = h->lay;
            MK_HIP(launch_fill(reinterpret_cast<uint32_t*>(p.x), (int64_t)(L.route_ids - L.x) / 4, nan2, stream));
            MK_HIP(launch_fill(reinterpret_cast<uint32_t*>(p.act), (int64_t)(L.rtab - L.act) / 4, nan2, stream));
            if (L.wtab > L.ybuf)
                MK_HIP(launch_fill(reinterpret_cast<uint32_t*>(p.ybuf), (int64_t)(L.wtab - L.ybuf) / 4, nan2, stream));
        }
        const int nb = batch >= h->mm_min ? (h->plan.rb > 1 ? kNbMmWide : 0) : batch;
        p.mm = batch >= h->mm_min ? 1 : 0;
        const KernelPair& k = h->kern[nb];
        const int general = h->general[nb];
        const size_t lds_bytes = h->lds_bytes[nb];
        if (h->o.time_kernels) MK_HIP(hipEventRecord(h->t_begin, stream));
        if (h->o.mode == MK_MODE_MEGAKERNEL) {
            p.perop = 0;
            p.tasks = reinterpret_cast<const Task*>(h->ws + h->lay.tasks);
            p.wg_off = reinterpret_cast<const int32_t*>(h->ws + h->lay.wg_off);
            MK_HIP(launch_persistent(k, p, general, lds_bytes, h->n_wg, stream));
        } else {
            p.perop = 1;
            p.tasks = reinterpret_cast<const Task*>(h->ws + h->lay.level_tasks);
            p.wg_off = nullptr;
            MK_HIP(launch_fill(p.ctr_other, h->lay.bank_words, 0u, stream));
            const Plan& P2 = h->plan;
            for (int lv = 0; lv < P2.n_levels; ++lv) {
                const int first = P2.level_off[lv], count = P2.level_off[lv + 1] - first;
                if (count > 0) MK_HIP(launch_perop_level(k, p, general, lds_bytes, first, count, stream));
            }
        }
        if (h->o.time_kernels) {
            MK_HIP(hipEventRecord(h->t_end, stream));
            h->timed = true;
        }
        if (!capturing) {
            MK_HIP(hipEventRecord(h->step_ev, stream));
            h->step_ev_used = true;
            h->last_stream = stream;
        } else {
            h->step_ev_used = false;
        }
        if (!use_scratch) h->bank = 1 - h->bank;
        h->last_n_tasks = (int64_t)(h->o.mode == MK_MODE_MEGAKERNEL ? h->plan.tasks.size() : h->plan.level_tasks.size());
        h->last_perop = h->o.mode != MK_MODE_MEGAKERNEL;
        return MK_OK;
    } catch (const std::bad_alloc&) {
        return fail(MK_ERR_CAPACITY, "host allocation failed");
    } catch (...) {
        return fail(MK_ERR_INVALID, "unexpected exception in a step");
    }
}

extern "C" {

mk_status mk_decode_step(mk_handle* h, int32_t batch, const int32_t* seq_ids, const int32_t* positions,
                         const int32_t* block_tables, const int32_t* tokens, float* logits, void* stream) {
    return step_impl(h, batch, seq_ids, positions, block_tables, tokens, logits, stream, false);
}

mk_status mk_forward_step(mk_handle* h, int32_t batch, const int32_t* seq_ids, const int32_t* positions,
                          const int32_t* block_tables, const int32_t* tokens, float* logits, void* stream) {
    return step_impl(h, batch, seq_ids, positions, block_tables, tokens, logits, stream, true);
}

mk_status mk_decode_step_noalloc(mk_handle* h, int32_t batch, const int32_t* seq_ids, const int32_t* positions,
                                 const int32_t* block_tables, const int32_t* tokens, float* logits, void* stream) {
    return step_impl(h, batch, seq_ids, positions, block_tables, tokens, logits, stream, false, true);
}

mk_status mk_sync_check(mk_handle* h, void* stream) {
    if (!h) return fail(MK_ERR_INVALID, "null handle");
    MK_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
    int32_t e[4];
    MK_HIP(hipMemcpy(e, h->ws + h->lay.err, sizeof e, hipMemcpyDeviceToHost));
    if (e[0] != 0) {
        MK_HIP(launch_fill(reinterpret_cast<uint32_t*>(h->ws + h->lay.err), 64, 0u, nullptr));
        MK_HIP(hipDeviceSynchronize());
        if (e[0] == kErrTimeout) {
            // the aborted step left its counter bank partly bumped: clear both
            MK_HIP(launch_fill(reinterpret_cast<uint32_t*>(h->ws + h->lay.banks), 2 * h->lay.bank_words, 0u,
                               nullptr));
            MK_HIP(hipDeviceSynchronize());
            return fail(MK_ERR_TIMEOUT, "device watchdog: wait on counter %d timed out", e[1]);
        }
        if (e[0] == kErrBadTask)
            return fail(MK_ERR_DEVICE, "device found a task with unknown operation %d in the plan", e[1]);
        return fail(MK_ERR_DEVICE, "device reported bad input (token %d)", e[1]);
    }
    return MK_OK;
}

mk_status mk_kernel_time(mk_handle* h, float* ms) {
    if (!h || !ms) return fail(MK_ERR_INVALID, "null argument");
    if (!h->o.time_kernels) return fail(MK_ERR_INVALID, "handle created without time_kernels");
    if (!h->timed) return fail(MK_ERR_INVALID, "no step has run");
    MK_HIP(hipEventSynchronize(h->t_end));
    MK_HIP(hipEventElapsedTime(ms, h->t_begin, h->t_end));
    return MK_OK;
}

mk_status mk_get_debug_ptrs(mk_handle* h, mk_debug_ptrs* out) {
    if (!h || !out) return fail(MK_ERR_INVALID, "null argument");
    out->x_layers = reinterpret_cast<const float*>(h->ws + h->lay.x);
    out->route_ids = reinterpret_cast<const int32_t*>(h->ws + h->lay.route_ids);
    out->route_w = reinterpret_cast<const float*>(h->ws + h->lay.route_w);
    out->router_logits = reinterpret_cast<const float*>(h->ws + h->lay.rlogits);
    out->trace = h->o.trace ? reinterpret_cast<const uint64_t*>(h->ws + h->lay.trace) : nullptr;
    out->trace_capacity = h->o.trace ? h->lay.cap_tasks : 0;
    return MK_OK;
}

mk_status mk_get_trace(mk_handle* h, void* host_buf, size_t bytes, size_t* written) {
    if (!h || !written) return fail(MK_ERR_INVALID, "null argument");
    if (!h->o.trace) return fail(MK_ERR_INVALID, "handle created without tracing");
    const size_t need = (size_t)h->last_n_tasks * 64;
    *written = 0;
    if (!host_buf) {
        *written = need;
        return MK_OK;
    }
    const size_t n = std::min(bytes, need);
    MK_HIP(hipDeviceSynchronize());
    MK_HIP(hipMemcpy(host_buf, h->ws + h->lay.trace, n, hipMemcpyDeviceToHost));
    *written = n;
    return MK_OK;
}

mk_status mk_get_plan(mk_handle* h, int32_t* tasks, int64_t cap_tasks, int64_t* n_tasks) {
    if (!h || !n_tasks) return fail(MK_ERR_INVALID, "null argument");
    if (h->last_n_tasks == 0) return fail(MK_ERR_INVALID, "no step has run on this handle");
    const std::vector<Task>& T = h->last_perop ? h->plan.level_tasks : h->plan.tasks;
    *n_tasks = (int64_t)T.size();
    if (!tasks) return MK_OK;
    if (cap_tasks < (int64_t)T.size()) return fail(MK_ERR_CAPACITY, "task buffer holds %lld of %lld tasks",
                                                   (long long)cap_tasks, (long long)T.size());
    memcpy(tasks, T.data(), T.size() * sizeof(Task));
    return MK_OK;
}

mk_status mk_plan_build(const mk_dims* dims, const mk_options* opts, int32_t n_wg, int32_t batch,
                        const int32_t* positions, mk_plan_info* info, int32_t* tasks, int64_t cap_tasks,
                        int32_t* wg_offsets, int32_t* counter_targets) {
    try {
        if (!dims || !positions || !info) return fail(MK_ERR_INVALID, "null argument");
        mk_options o;
        memset(&o, 0, sizeof o);
        if (opts) o = *opts;
        if (o.mfma_min_batch < 0 || o.mfma_min_batch > kMaxBatchValu + 1)
            return fail(MK_ERR_INVALID, "mfma_min_batch must be 0 (default) or 1..%d", kMaxBatchValu + 1);
        if (o.mm_row_blocks < 0 || o.mm_row_blocks > kMmMaxRowBlocks)
            return fail(MK_ERR_INVALID, "mm_row_blocks must be 0 (choose) or 1..%d", kMmMaxRowBlocks);
        const std::string why = check_dims(*dims, mm_min_of(o));
        if (!why.empty()) return fail(MK_ERR_UNSUPPORTED, "%s", why.c_str());
        if (batch <= 0 || batch > dims->max_batch) return fail(MK_ERR_CAPACITY, "batch out of range");
        const ModelShape s = shape_of(*dims, max_chunks_for(*dims));
        Plan P;
        const std::string err = build_plan(s, tile_config(o), n_wg, batch, positions, &P);
        if (!err.empty()) return fail(MK_ERR_CAPACITY, "%s", err.c_str());
        const std::string verr = validate_plan(s, P);
        if (!verr.empty()) return fail(MK_ERR_INVALID, "plan invalid: %s", verr.c_str());
        memset(info, 0, sizeof *info);
        info->n_wg = P.n_wg;
        info->n_tasks = (int32_t)P.tasks.size();
        info->n_counters = (int32_t)P.targets.size();
        info->n_levels = P.n_levels;
        info->chunk_tokens = P.chunk;
        info->cap_tasks = (int32_t)std::min<int64_t>(max_tasks(s, tile_config(o), n_wg), INT32_MAX);
        if (tasks) {
            if (cap_tasks < (int64_t)P.tasks.size()) return fail(MK_ERR_CAPACITY, "task buffer too small");
            memcpy(tasks, P.tasks.data(), P.tasks.size() * sizeof(Task));
        }
        if (wg_offsets) memcpy(wg_offsets, P.wg_off.data(), P.wg_off.size() * 4);
        if (counter_targets) memcpy(counter_targets, P.targets.data(), P.targets.size() * 4);
        return MK_OK;
    } catch (const std::bad_alloc&) {
        return fail(MK_ERR_CAPACITY, "host allocation failed");
    } catch (...) {
        return fail(MK_ERR_INVALID, "unexpected exception in mk_plan_build");
    }
}

mk_status mk_plan_check(const mk_dims* dims, const mk_options* opts, int32_t n_wg, int32_t batch,
                        const int32_t* positions, const int32_t* tasks, int64_t n_tasks, const int32_t* wg_offsets) {
    try {
        if (!dims || !positions || !tasks || !wg_offsets) return fail(MK_ERR_INVALID, "null argument");
        mk_options o;
        memset(&o, 0, sizeof o);
        if (opts) o = *opts;
        const std::string why = check_dims(*dims, mm_min_of(o));
        if (!why.empty()) return fail(MK_ERR_UNSUPPORTED, "%s", why.c_str());
        if (batch <= 0 || batch > dims->max_batch || n_wg <= 0 || n_tasks < 0) return fail(MK_ERR_INVALID, "bad sizes");
        const ModelShape s = shape_of(*dims, max_chunks_for(*dims));
        Plan P;
        const std::string err = build_plan(s, tile_config(o), n_wg, batch, positions, &P);
        if (!err.empty()) return fail(MK_ERR_CAPACITY, "%s", err.c_str());
        // the caller's task table and lists in place of the built ones
        P.tasks.assign(reinterpret_cast<const Task*>(tasks), reinterpret_cast<const Task*>(tasks) + n_tasks);
        P.wg_off.assign(wg_offsets, wg_offsets + n_wg + 1);
        if (P.wg_off.front() != 0 || P.wg_off.back() > n_tasks) return fail(MK_ERR_INVALID, "plan invalid: offsets");
        for (int w = 0; w < n_wg; ++w)
            if (P.wg_off[w + 1] < P.wg_off[w]) return fail(MK_ERR_INVALID, "plan invalid: offsets");
        for (const Task& t : P.tasks)
            if (t.op < 0 || t.op >= OP_COUNT || t.level < 0 || t.level >= P.n_levels)
                return fail(MK_ERR_INVALID, "plan invalid: task op or level out of range");
        const std::string verr = validate_plan(s, P);
        if (!verr.empty()) return fail(MK_ERR_INVALID, "plan invalid: %s", verr.c_str());
        return MK_OK;
    } catch (const std::bad_alloc&) {
        return fail(MK_ERR_CAPACITY, "host allocation failed");
    } catch (...) {
        return fail(MK_ERR_INVALID, "unexpected exception in mk_plan_check");
    }
}

void mk_destroy(mk_handle* h) {
    if (!h) return;
    (void)hipSetDevice(h->device);
    for (int i = 0; i < kStageSlots; ++i) {
        if (h->stage[i]) {
            (void)hipEventSynchronize(h->stage_ev[i]);
            (void)hipEventDestroy(h->stage_ev[i]);
            (void)hipHostFree(h->stage[i]);
        }
    }
    if (h->plan_ev_used) (void)hipEventSynchronize(h->plan_ev);
    (void)hipEventDestroy(h->plan_ev);
    if (h->step_ev_used) (void)hipEventSynchronize(h->step_ev);
    (void)hipEventDestroy(h->step_ev);
    if (h->plan_stage) (void)hipHostFree(h->plan_stage);
    if (h->o.time_kernels) {
        (void)hipEventDestroy(h->t_begin);
        (void)hipEventDestroy(h->t_end);
    }
    delete h;
}

}  // extern "C"
