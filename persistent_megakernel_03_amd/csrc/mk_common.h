// mk_common.h -- definitions shared by the host task-graph builder and the
// device code: task records, operation codes, counter layout and the kernel
// parameter block.
//
// A decode step is a DAG of tiles. The host turns it into one task list per
// persistent workgroup, and global-memory counters record when a tile's
// inputs are ready ("Cohere Publishes One-Kernel Server for North Mini Code,
// Claims 1.58x vLLM Speedup", section "One resident program, many small
// tasks"). Every tile type runs through one calling convention (same page,
// section "A hand-built approach to a specialized server").
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MK_HD __host__ __device__
#else
#define MK_HD
#endif

namespace mk {

// Operation codes, in dependency-level order inside a layer.
enum Op : int32_t {
    OP_EMBED = 0,   // x0[b] = embedding row of token b
    OP_QKV = 1,     // fused RMSNorm + QKV rows of one KV group
    OP_ATTN = 2,    // RoPE (+ KV append) + split-KV attention over one chunk of tokens
    OP_COMBINE = 3, // merge one query head's chunk partials (log-sum-exp)
    OP_OPROJ = 4,   // output projection + residual
    OP_ROUTER = 5,  // fused RMSNorm + router logits
    OP_ROUTE = 6,   // batches of 3+: top-k of every token + per-expert token lists
    OP_GATEUP = 7,  // expert gate/up rows + SwiGLU (batches of 1-2: also the top-k)
    OP_DOWN = 8,    // expert down rows (batches of 1-2: + weighted combine + residual)
    OP_MOESUM = 9,  // batches of 3+: weighted sum of the experts' outputs + residual
    OP_LMHEAD = 10, // LM-head rows (batches of 1-2: with the final RMSNorm fused)
    OP_CLAIM = 11,  // not a tile: run tiles of one level from a shared pool
                    // (a0: first pool task, a1: pool size, a2: the level,
                    // whose claim counter hands out pool positions)
    OP_FNORM = 12,  // batches of 3+: the final RMSNorm of tokens a0..a1, stored split for the LM head
    OP_COUNT = 13
};

// QKV, ATTN, COMBINE, OPROJ, ROUTER, ROUTE, GATEUP, DOWN, MOESUM; ROUTE and
// MOESUM have no tiles in the one- and two-token schedule.
constexpr int kLevelsPerLayer = 9;

// Largest batch of the matrix-vector (dot-product) tiles; larger batches run
// every weight product on the matrix cores, up to kMaxBatchMM tokens.
constexpr int kMaxBatchValu = 2;
constexpr int kMaxBatchMM = 64;

// Matrix-core expert tiles: at most this many 8-row blocks of the expert
// width per gate/up tile and 16-row blocks of the hidden size per down tile,
// so that a wave can multiply one load of its tokens' activations by several
// blocks of one expert's weights.
constexpr int kMmMaxRowBlocks = 2;

// Kernel flavours (template argument NB): 0 the matrix-core schedule, 1 and
// 2 the one- and two-token schedules, kNbMmWide the matrix-core schedule
// with kMmMaxRowBlocks row blocks per expert tile (a kernel of its own, so
// that each build holds one variant of the expert stream in its registers).
constexpr int kNbMmWide = kMaxBatchValu + 1;
constexpr int kNbCount = kNbMmWide + 1;

// LDS of the matrix-core tiles (general region): a block product's per-wave
// partials [4][16][64] and sums of squares [4][64] fp32 plus 128 words of
// token list and routing-table entries; the routing tile's token masks [256][2], ranks [64][256] (bytes)
// and per-wave counts.
constexpr int kMmLdsBytes = (4 * 16 * 64 + 4 * 64 + 128) * 4;
constexpr int kRouteLdsBytes = 2 * 256 * 4 + kMaxBatchMM * 256 + 16;

// Dependency level of an op in layer l (0 = embedding; after the layers the
// final norm, empty at batches of 1-2, then the LM head).
inline int op_level(int op, int layer, int n_layers) {
    if (op == OP_EMBED) return 0;
    if (op == OP_FNORM) return 1 + kLevelsPerLayer * n_layers;
    if (op == OP_LMHEAD) return 2 + kLevelsPerLayer * n_layers;
    return 1 + kLevelsPerLayer * layer + (op - OP_QKV);
}

// One task: 12 int32, read by a workgroup with scalar loads.
struct Task {
    int32_t op;
    int32_t layer;
    int32_t a0, a1, a2, a3;   // op-specific tile coordinates
    int32_t pre_ctr;          // wait before loading weights (-1: none)
    int32_t pre_target;
    int32_t ctr;              // wait before computing (-1: none)
    int32_t target;
    int32_t signal;           // counter bumped after the tile (-1: none)
    int32_t level;
};
static_assert(sizeof(Task) == 48, "task record is 12 int32");

// Weight table: kinds per layer.
enum WKind : int32_t {
    W_ATTN_NORM = 0, W_QKV, W_O, W_FFN_NORM, W_ROUTER, W_GATE, W_UP, W_DOWN, W_RBIAS, W_NKINDS
};

// Counter bank layout: one counter per 128-byte line. Per layer: one QKV
// counter and one attention counter per KV group, then the combine, output
// projection, router, routing, gate/up, down and expert-sum counters.
constexpr int kCtrStride = 32;  // uint32 words per counter line
// Each counter is split over kCtrSub lines: a producer bumps the line of its
// workgroup index modulo kCtrSub and a consumer sums them, so the hundreds of
// tiles of a wide level do not queue on one address.
constexpr int kCtrSub = 8;

struct CounterLayout {
    int n_layers, n_kv_heads, max_batch;
    MK_HD int per_layer() const { return 2 * n_kv_heads + 7; }
    MK_HD int embed() const { return 0; }
    MK_HD int qkv(int l, int g) const { return 1 + l * per_layer() + g; }
    MK_HD int attn(int l, int g) const { return 1 + l * per_layer() + n_kv_heads + g; }
    MK_HD int combine(int l) const { return 1 + l * per_layer() + 2 * n_kv_heads; }
    MK_HD int oproj(int l) const { return combine(l) + 1; }
    MK_HD int router(int l) const { return combine(l) + 2; }
    MK_HD int route(int l) const { return combine(l) + 3; }
    MK_HD int gateup(int l) const { return combine(l) + 4; }
    MK_HD int down(int l) const { return combine(l) + 5; }
    MK_HD int moesum(int l) const { return combine(l) + 6; }
    MK_HD int fnorm() const { return 1 + n_layers * per_layer(); }
    MK_HD int n_main() const { return 2 + n_layers * per_layer(); }
    // one claim counter per dependency level (a single line each), after the
    // split counters
    MK_HD int n_levels() const { return 3 + kLevelsPerLayer * n_layers; }
    MK_HD int64_t claim_word(int level) const { return ((int64_t)n_main() * kCtrSub + level) * kCtrStride; }
    MK_HD int64_t bank_words() const {
        return (((int64_t)n_main() * kCtrSub + n_levels()) * kCtrStride + 63) & ~(int64_t)63;
    }
};

// Exchange buffers are padded so that no 128-byte cache line holds words of
// two slices with different producers: a consumer may then cache a line
// only after every word of it has been written (a CU's L1 is not updated by
// other CUs' stores). pad64 rounds a float count up to 256 bytes.
MK_HD inline int64_t pad64(int64_t n) { return (n + 63) & ~(int64_t)63; }

// Kernel parameter block (passed by value).
struct Params {
    // model shape
    int32_t L, H, Hq, Hkv, D, E, K, I, V, P, G, QKVD;
    float eps, attn_scale, inv_h;   // inv_h = 1 / H (RMSNorm mean)
    int32_t max_batch, max_pages, max_chunks;
    int64_t n_pages;
    // this step
    int32_t B, chunk;   // chunk: the plan's attention chunk length (a sequence may use a longer one)
    int32_t perop;      // 1: per-op launches (no counter waits / signals)
    int32_t mm;         // 1: the matrix-core schedule (its tiles take split-form inputs)
    int32_t trace_on;
    int64_t watchdog_ticks;
    // weights
    const uint16_t* embed;
    const uint16_t* lm_head;
    const uint16_t* final_norm;
    const uint64_t* wtab;  // [L][W_NKINDS] device addresses
    uint16_t* k_pool;
    uint16_t* v_pool;
    // step inputs
    const int32_t* tokens;
    float* logits;
    const int32_t* positions;     // [max_batch]
    const int32_t* block_tables;  // [max_batch][max_pages]
    const float* rope;            // [max_batch][D/2][2] cos, sin
    const int32_t* seq_chunk;     // [max_batch] attention chunk length of each sequence (tokens)
    const int32_t* seq_first;     // [max_batch][2] (first position this step writes for the row's sequence,
                                  // the row that feeds it): a multi-token step's rows of one sequence
                                  // take each other's new K/V from the qkv buffer, not the pool
    // workspace: every buffer exchanged between workgroups has one slice per
    // layer, so each is written at most once per step
    float* x;         // [2L+1][max_batch][H]
    float* qkv;       // [L][max_batch][QKVD]
    float* att_part;  // [L][max_batch][Hq][max_chunks][D] unnormalised outputs
    float* att_ml;    // [L][max_batch][Hq][pad64(2 max_chunks)] running max and sum
    float* att_out;   // [L][max_batch][Hq*D] (split form for batches of 3+)
    float* rlogits;   // [L][max_batch][E]
    int32_t* route_ids;  // [L][max_batch][K]
    float* route_w;      // [L][max_batch][K]
    float* act;          // [L][max_batch*K][I] (split form for batches of 3+)
    int32_t* rtab;       // [L][rtab_words]: batches of 3+, routing table (see rtab_words)
    float* ybuf;         // [L][max_batch*K][H]: batches of 3+, each expert's output per (token, rank)
    float* h2s;          // [L+1][max_batch][H]: batches of 3+, the experts' normalised input, split;
                         // slice L: the final norm's output (the LM head's input), split
    uint32_t* ctr;       // this step's counter bank
    uint32_t* ctr_other; // the bank the next step uses (cleared by this step)
    int64_t bank_words;
    CounterLayout cl;
    int32_t* err;        // [0]: status code, [1]: detail, [2]: abort flag
    const Task* tasks;
    const int32_t* wg_off;
    uint64_t* trace;     // [n_tasks][4]
};

// Routing table of one layer for batches of 3+ (int32 words): [0] number of
// distinct selected experts ("slots", ascending expert id); [64 + s] expert
// of slot s; [64 + E + s] tokens routed to it; [64 + 2E + s*max_batch + c]
// its c-th token as (token | rank << 16), rank = the expert's place in that
// token's top-k; then the routing weights [max_batch][K] as fp32.
MK_HD inline int64_t rtab_words(int E, int K, int max_batch) {
    return pad64(64 + 2 * (int64_t)E + (int64_t)E * max_batch + (int64_t)max_batch * K);
}

// Device error codes: the first two mirror mk_status values; a task record
// with an unknown operation is reported to the caller as MK_ERR_DEVICE.
constexpr int32_t kErrTimeout = -6;
constexpr int32_t kErrDevice = -7;
constexpr int32_t kErrBadTask = -8;

}  // namespace mk
