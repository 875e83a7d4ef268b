// mk_plan.cpp -- host task-graph builder (see mk_plan.h).
#include "mk_plan.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <map>
#include <queue>
#include <set>
#include <tuple>

namespace mk {

namespace {

int ceil_div(int a, int b) { return (a + b - 1) / b; }

Task make_task(int op, int layer, int a0, int a1, int a2, int a3, int pre_ctr, int pre_target, int ctr,
               int target, int signal, int level) {
    Task t;
    t.op = op;
    t.layer = layer;
    t.a0 = a0;
    t.a1 = a1;
    t.a2 = a2;
    t.a3 = a3;
    t.pre_ctr = pre_ctr;
    t.pre_target = pre_target;
    t.ctr = ctr;
    t.target = target;
    t.signal = signal;
    t.level = level;
    return t;
}

// Tile kinds for the timing model: weights loadable any time, weights known
// only after routing, inputs produced inside the step.
enum { kStatic = 0, kRouted = 1, kDynamic = 2 };

struct Tile {
    Task t;
    double bytes;
    int kind;
};

}  // namespace

static void build_levels_valu(const ModelShape& s, const TileConfig& cfg, int n_wg, int B, const int32_t* positions,
                              Plan& P, std::vector<std::vector<Tile>>& levels);
static void build_levels_mm(const ModelShape& s, const TileConfig& cfg, int n_wg, int B, const int32_t* positions,
                            Plan& P, std::vector<std::vector<Tile>>& levels);
static void place_tiles(const TileConfig& cfg, int n_wg, std::vector<std::vector<Tile>>& levels, Plan& P);

void expert_rows(const ModelShape& s, const TileConfig& cfg, int n_wg, int S, int* rows_gu, int* rows_down) {
    *rows_gu = cfg.rows_gateup;
    *rows_down = cfg.rows_down;
    // A down tile keeps its weight rows (S experts x rows) in registers, 16
    // row-vectors per wave (one matrix-core operand). Rows per tile are a
    // power of two, so the 16 row-vectors of a wave hold whole experts or
    // one part of one expert.
    int rd = 64;
    while (rd > 1 && rd * std::max(1, S) > 64) rd >>= 1;
    if (rd < cfg.rows_down) return;
    const int n_down = ceil_div(s.H, rd);
    // gate/up tiles go to every workgroup (one each, its rows in flight at
    // once) when there are at most as many down tiles as workgroups, so that
    // no workgroup runs two expert tiles of one kind; else to the workgroups
    // the down tiles leave
    const bool spread = n_down <= n_wg;
    const int per_slot = (spread ? n_wg : n_wg - n_down) / std::max(1, S);
    if (per_slot < 1) return;
    int rg = spread ? ceil_div(s.I, per_slot) : std::max(cfg.rows_gateup, ceil_div(s.I, per_slot));
    rg = ceil_div(rg, 4) * 4;
    *rows_gu = rg;
    *rows_down = rd;
}

void expert_groups_mm(const ModelShape& s, int n_wg, int S, int rb, int* gu_groups, int* down_groups) {
    // gate/up: rb 8-row blocks of the expert width per tile, the slots in
    // groups so that there are about 1.5 tiles per workgroup; down: rb 16-row
    // blocks of the hidden size, about one tile per workgroup
    const int gblk = ceil_div(s.I, 8 * rb), dblk = ceil_div(s.H, 16 * rb);
    *gu_groups = std::max(1, std::min(S, (3 * n_wg / 2 + gblk / 2) / std::max(1, gblk)));
    *down_groups = std::max(1, std::min(S, n_wg / std::max(1, dblk)));
}

int mm_row_blocks(const ModelShape& s, int n_wg, int B) {
    // Two blocks per tile halve the tiles per slot group, so the slots are
    // spread over twice the groups: worth it only when the tile's four waves
    // still get about two slots each. The count of distinct experts is
    // unknown until routing; its expectation under uniform routing,
    // E (1 - (1 - k/E)^B), stands in for it.
    const int S = std::min(s.E, B * s.K);
    int qg = 1, q = 1;
    expert_groups_mm(s, n_wg, S, kMmMaxRowBlocks, &qg, &q);
    const double distinct = s.E * (1.0 - std::pow(1.0 - (double)s.K / s.E, B));
    return distinct >= 7.0 * qg ? kMmMaxRowBlocks : 1;
}

int choose_chunk(const ModelShape& s, int n_wg, int B, const int32_t* positions, int requested) {
    int chunk;
    if (requested > 0) {
        chunk = ceil_div(requested, 64) * 64;
    } else {
        int64_t total = 0;
        for (int b = 0; b < B; ++b) total += (int64_t)(positions[b] + 1) * s.Hkv;
        const int64_t per = (total + n_wg - 1) / std::max(1, n_wg);
        chunk = (int)std::max<int64_t>(128, (per + 127) / 128 * 128);
    }
    for (int b = 0; b < B; ++b) {
        const int need = ceil_div(positions[b] + 1, s.max_chunks);
        if (need > chunk) chunk = ceil_div(need, 64) * 64;
    }
    return chunk;
}

int64_t max_tasks(const ModelShape& s, const TileConfig& cfg, int n_wg) {
    const int G = s.Hq / s.Hkv;
    const int bv = std::min(s.max_batch, kMaxBatchValu);
    const int64_t attn = (int64_t)s.Hkv * s.max_chunks, comb = s.Hq;
    const int64_t per_layer = (int64_t)s.Hkv * ceil_div((G + 2) * s.D, cfg.rows_qkv) + bv * (attn + comb) +
                              ceil_div(s.H, cfg.rows_o) +
                              ceil_div(s.E, cfg.rows_router) +
                              // spread gate/up rows give each slot at most n_wg / S tiles
                              std::max<int64_t>((int64_t)std::min(s.E, bv * s.K) * ceil_div(s.I, cfg.rows_gateup),
                                                n_wg) +
                              ceil_div(s.H, cfg.rows_down);
    int64_t n = 1 + (int64_t)s.L * per_layer + ceil_div(s.V, cfg.rows_lm);
    if (s.max_batch >= cfg.mm_min_batch) {
        // matrix-core schedule: expert tiles are (rows, slot group) pairs with
        // at most min(E, B k) groups
        const int S = std::min(s.E, s.max_batch * s.K);
        const int64_t mm_layer = (int64_t)s.Hkv * ceil_div((G + 2) * s.D, cfg.mm_rows_qkv) +
                                 s.max_batch * (attn + comb) + ceil_div(s.H, cfg.mm_rows_o) +
                                 (int64_t)ceil_div(s.E, cfg.mm_rows_router) * ceil_div(s.max_batch, 16) + 1 +
                                 (int64_t)S * ceil_div(s.I, 8) +
                                 (int64_t)ceil_div(s.H, 16) * S + ceil_div(s.H, cfg.mm_rows_sum);
        const int64_t m = ceil_div(s.max_batch, cfg.mm_embed_tokens) + (int64_t)s.L * mm_layer +
                          s.max_batch + ceil_div(s.V, cfg.mm_rows_lm);
        // each claim task stands for at least one tile of its level
        n = std::max(n, 2 * m);
    }
    return n;
}

std::string build_plan(const ModelShape& s, const TileConfig& cfg, int n_wg, int B, const int32_t* positions,
                       Plan* out) {
    if (n_wg <= 0) return "n_wg must be positive";
    if (B <= 0 || B > s.max_batch) return "batch out of range";
    const CounterLayout cl{s.L, s.Hkv, s.max_batch};
    Plan& P = *out;
    P = Plan();
    P.n_wg = n_wg;
    P.B = B;
    P.mm = B >= cfg.mm_min_batch;
    if (!P.mm && B > kMaxBatchValu) return "batch above the one- and two-token schedule";
    P.chunk = choose_chunk(s, n_wg, B, positions, cfg.chunk);
    P.n_levels = 3 + kLevelsPerLayer * s.L;
    P.targets.assign(cl.n_main(), 0);
    P.n_chunks.resize(B);
    for (int b = 0; b < B; ++b) {
        if (positions[b] < 0) return "negative position";
        P.n_chunks[b] = ceil_div(positions[b] + 1, P.chunk);
        if (P.n_chunks[b] > s.max_chunks) return "attention chunks exceed capacity";
    }

    std::vector<std::vector<Tile>> levels(P.n_levels);
    if (P.mm) {
        build_levels_mm(s, cfg, n_wg, B, positions, P, levels);
    } else {
        build_levels_valu(s, cfg, n_wg, B, positions, P, levels);
    }
    place_tiles(cfg, n_wg, levels, P);
    return std::string();
}

// The one- and two-token schedule: per layer QKV, attention, merge, output
// projection, router, gate/up (each tile also computes the routing) and down
// (which also sums the experts onto the residual).
static void build_levels_valu(const ModelShape& s, const TileConfig& cfg, int n_wg, int B, const int32_t* positions,
                       Plan& P, std::vector<std::vector<Tile>>& levels) {
    const CounterLayout cl{s.L, s.Hkv, s.max_batch};
    const int G = s.Hq / s.Hkv;
    auto add = [&](const Task& t, double bytes, int kind) { levels[t.level].push_back({t, bytes, kind}); };

    add(make_task(OP_EMBED, 0, 0, B, 0, 0, -1, 0, -1, 0, cl.embed(), 0), 2.0 * B * s.H, kStatic);
    P.targets[cl.embed()] = 1;

    const int grows = (G + 2) * s.D;
    const int nq = ceil_div(grows, cfg.rows_qkv);
    const int no = ceil_div(s.H, cfg.rows_o);
    const int nr = ceil_div(s.E, cfg.rows_router);
    const int S = std::min(s.E, B * s.K);
    int rows_gu = 0, rows_down = 0;
    expert_rows(s, cfg, n_wg, S, &rows_gu, &rows_down);
    const int ngu = ceil_div(s.I, rows_gu);
    const int nd = ceil_div(s.H, rows_down);
    const int nl = ceil_div(s.V, cfg.rows_lm);
    int total_chunks = 0;
    for (int b = 0; b < B; ++b) total_chunks += P.n_chunks[b];

    for (int l = 0; l < s.L; ++l) {
        const int lv = 1 + kLevelsPerLayer * l;
        const int in_ctr = l == 0 ? cl.embed() : cl.down(l - 1);
        const int in_target = l == 0 ? 1 : nd;
        // the query/key/value weights and the cache pages of layer l start
        // streaming once the previous layer's gate/up tiles are done, so that
        // they do not compete with the expert weights, which cannot be
        // fetched before the routing is known
        const int defer_ctr = l == 0 ? -1 : cl.gateup(l - 1);
        const int defer_target = l == 0 ? 0 : S * ngu;
        for (int g = 0; g < s.Hkv; ++g) {
            for (int i = 0; i < nq; ++i) {
                const int v0 = i * cfg.rows_qkv, v1 = std::min(grows, v0 + cfg.rows_qkv);
                add(make_task(OP_QKV, l, g, v0, v1, 0, defer_ctr, defer_target, in_ctr, in_target, cl.qkv(l, g), lv),
                    2.0 * (v1 - v0) * s.H, kStatic);
            }
            P.targets[cl.qkv(l, g)] = nq;
        }
        for (int b = 0; b < B; ++b) {
            const int n = P.n_chunks[b];
            for (int g = 0; g < s.Hkv; ++g)
                for (int c = 0; c < n; ++c) {
                    const int toks = std::min(P.chunk, positions[b] + 1 - c * P.chunk);
                    add(make_task(OP_ATTN, l, b, g, c, n, defer_ctr, defer_target, cl.qkv(l, g), nq, cl.attn(l, g),
                                  lv + 1),
                        4.0 * toks * s.D, kStatic);
                }
        }
        for (int g = 0; g < s.Hkv; ++g) P.targets[cl.attn(l, g)] = total_chunks;
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < s.Hq; ++h)
                add(make_task(OP_COMBINE, l, b, h, P.n_chunks[b], 0, -1, 0, cl.attn(l, h / G), total_chunks,
                              cl.combine(l), lv + 2),
                    4.0 * P.n_chunks[b] * (s.D + 2), kDynamic);
        P.targets[cl.combine(l)] = B * s.Hq;
        for (int i = 0; i < no; ++i) {
            const int r0 = i * cfg.rows_o, r1 = std::min(s.H, r0 + cfg.rows_o);
            add(make_task(OP_OPROJ, l, r0, r1, 0, 0, in_ctr, in_target, cl.combine(l), B * s.Hq, cl.oproj(l), lv + 3),
                2.0 * (r1 - r0) * s.Hq * s.D, kStatic);
        }
        P.targets[cl.oproj(l)] = no;
        for (int i = 0; i < nr; ++i) {
            const int r0 = i * cfg.rows_router, r1 = std::min(s.E, r0 + cfg.rows_router);
            add(make_task(OP_ROUTER, l, r0, r1, 0, 0, -1, 0, cl.oproj(l), no, cl.router(l), lv + 4),
                2.0 * (r1 - r0) * s.H, kStatic);
        }
        P.targets[cl.router(l)] = nr;
        for (int sl = 0; sl < S; ++sl)
            for (int i = 0; i < ngu; ++i) {
                const int r0 = i * rows_gu, r1 = std::min(s.I, r0 + rows_gu);
                // waits on the router only: the router tiles waited on the
                // output projection, whose residual this tile also reads
                add(make_task(OP_GATEUP, l, sl, r0, r1, (sl == 0 && i == 0) ? 1 : 0, -1, 0, cl.router(l), nr,
                              cl.gateup(l), lv + 5),
                    4.0 * (r1 - r0) * s.H, kRouted);
            }
        P.targets[cl.gateup(l)] = S * ngu;
        for (int i = 0; i < nd; ++i) {
            const int r0 = i * rows_down, r1 = std::min(s.H, r0 + rows_down);
            add(make_task(OP_DOWN, l, r0, r1, rows_down, 0, cl.router(l), nr, cl.gateup(l), S * ngu, cl.down(l),
                          lv + 6),
                2.0 * S * (r1 - r0) * s.I, kRouted);
        }
        P.targets[cl.down(l)] = nd;
    }
    for (int i = 0; i < nl; ++i) {
        const int r0 = i * cfg.rows_lm, r1 = std::min(s.V, r0 + cfg.rows_lm);
        add(make_task(OP_LMHEAD, 0, r0, r1, 0, 0, -1, 0, cl.down(s.L - 1), nd, -1, P.n_levels - 1),
            2.0 * (r1 - r0) * s.H, kStatic);
    }
}

// Batches of 3+: every weight product on the matrix cores. Per layer QKV,
// attention, merge, output projection, router, routing (one tile), gate/up
// over the routing table's slots, down per (16 hidden rows, slot group), and
// the per-token expert sum.
static void build_levels_mm(const ModelShape& s, const TileConfig& cfg, int n_wg, int B, const int32_t* positions,
                     Plan& P, std::vector<std::vector<Tile>>& levels) {
    const CounterLayout cl{s.L, s.Hkv, s.max_batch};
    const int G = s.Hq / s.Hkv;
    auto add = [&](const Task& t, double bytes, int kind) { levels[t.level].push_back({t, bytes, kind}); };

    const int ne = ceil_div(B, cfg.mm_embed_tokens);
    for (int i = 0; i < ne; ++i) {
        const int b0 = i * cfg.mm_embed_tokens, b1 = std::min(B, b0 + cfg.mm_embed_tokens);
        add(make_task(OP_EMBED, 0, b0, b1, 0, 0, -1, 0, -1, 0, cl.embed(), 0), 2.0 * (b1 - b0) * s.H, kStatic);
    }
    P.targets[cl.embed()] = ne;

    const int grows = (G + 2) * s.D;
    const int nq = ceil_div(grows, cfg.mm_rows_qkv);
    const int no = ceil_div(s.H, cfg.mm_rows_o);
    const int nr = ceil_div(s.E, cfg.mm_rows_router);
    const int ntb = ceil_div(B, 16);   // router tiles per row block: one per 16-token block
    const int S = std::min(s.E, B * s.K);
    int Qg = 1, Q = 1;
    const int rb = cfg.mm_row_blocks > 0 ? cfg.mm_row_blocks : mm_row_blocks(s, n_wg, B);
    P.rb = rb;
    expert_groups_mm(s, n_wg, S, rb, &Qg, &Q);
    const int gblk = ceil_div(s.I, 8 * rb);
    const int ngu = gblk * Qg;
    const int nblk = ceil_div(s.H, 16 * rb);
    const int nd = nblk * Q;
    const int ns = ceil_div(s.H, cfg.mm_rows_sum);
    const int nl = ceil_div(s.V, cfg.mm_rows_lm);
    int total_chunks = 0;
    for (int b = 0; b < B; ++b) total_chunks += P.n_chunks[b];

    for (int l = 0; l < s.L; ++l) {
        const int lv = 1 + kLevelsPerLayer * l;
        const int in_ctr = l == 0 ? cl.embed() : cl.moesum(l - 1);
        const int in_target = l == 0 ? ne : ns;
        const int defer_ctr = l == 0 ? -1 : cl.gateup(l - 1);
        const int defer_target = l == 0 ? 0 : ngu;
        for (int g = 0; g < s.Hkv; ++g) {
            for (int i = 0; i < nq; ++i) {
                const int v0 = i * cfg.mm_rows_qkv, v1 = std::min(grows, v0 + cfg.mm_rows_qkv);
                add(make_task(OP_QKV, l, g, v0, v1, 0, defer_ctr, defer_target, in_ctr, in_target, cl.qkv(l, g), lv),
                    2.0 * (v1 - v0) * s.H, kStatic);
            }
            P.targets[cl.qkv(l, g)] = nq;
        }
        for (int b = 0; b < B; ++b) {
            const int n = P.n_chunks[b];
            for (int g = 0; g < s.Hkv; ++g)
                for (int c = 0; c < n; ++c) {
                    const int toks = std::min(P.chunk, positions[b] + 1 - c * P.chunk);
                    add(make_task(OP_ATTN, l, b, g, c, n, defer_ctr, defer_target, cl.qkv(l, g), nq, cl.attn(l, g),
                                  lv + 1),
                        4.0 * toks * s.D, kStatic);
                }
        }
        for (int g = 0; g < s.Hkv; ++g) P.targets[cl.attn(l, g)] = total_chunks;
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < s.Hq; ++h)
                add(make_task(OP_COMBINE, l, b, h, P.n_chunks[b], 0, -1, 0, cl.attn(l, h / G), total_chunks,
                              cl.combine(l), lv + 2),
                    4.0 * P.n_chunks[b] * (s.D + 2), kDynamic);
        P.targets[cl.combine(l)] = B * s.Hq;
        for (int i = 0; i < no; ++i) {
            const int r0 = i * cfg.mm_rows_o, r1 = std::min(s.H, r0 + cfg.mm_rows_o);
            add(make_task(OP_OPROJ, l, r0, r1, 0, 0, -1, 0, cl.combine(l), B * s.Hq, cl.oproj(l), lv + 3),
                2.0 * (r1 - r0) * s.Hq * s.D, kStatic);
        }
        P.targets[cl.oproj(l)] = no;
        // router tile (i, tb): expert rows of block i for the tokens of
        // 16-token block tb (each tile reads only those tokens' residual
        // rows), and the 8-element groups [g0, g1) of those tokens' expert
        // input; tb rides in the upper half of a2 and a3
        const int ng = s.H / 8, gs = ceil_div(ng, nr);
        for (int tb = 0; tb < ntb; ++tb)
            for (int i = 0; i < nr; ++i) {
                const int r0 = i * cfg.mm_rows_router, r1 = std::min(s.E, r0 + cfg.mm_rows_router);
                const int g0 = std::min(ng, i * gs), g1 = std::min(ng, g0 + gs);
                add(make_task(OP_ROUTER, l, r0, r1, g0 | (tb << 16), g1 | (tb << 16), -1, 0, cl.oproj(l), no,
                              cl.router(l), lv + 4),
                    2.0 * (r1 - r0) * s.H, kStatic);
            }
        P.targets[cl.router(l)] = nr * ntb;
        add(make_task(OP_ROUTE, l, 0, 1, 0, 0, -1, 0, cl.router(l), nr * ntb, cl.route(l), lv + 5), 4.0 * B * s.E,
            kDynamic);
        P.targets[cl.route(l)] = 1;
        for (int q = 0; q < Qg; ++q)
            for (int i = 0; i < gblk; ++i) {
                const int r0 = i * 8 * rb, r1 = std::min(s.I, r0 + 8 * rb);
                add(make_task(OP_GATEUP, l, r0, r1, q, Qg, -1, 0, cl.route(l), 1, cl.gateup(l), lv + 6),
                    4.0 * ceil_div(S - q, Qg) * (r1 - r0) * s.H, kRouted);
            }
        P.targets[cl.gateup(l)] = ngu;
        for (int q = 0; q < Q; ++q)
            for (int i = 0; i < nblk; ++i) {
                const int r0 = i * 16 * rb, r1 = std::min(s.H, r0 + 16 * rb);
                add(make_task(OP_DOWN, l, r0, r1, q, Q, cl.route(l), 1, cl.gateup(l), ngu, cl.down(l), lv + 7),
                    2.0 * ceil_div(S - q, Q) * (r1 - r0) * s.I, kRouted);
            }
        P.targets[cl.down(l)] = nd;
        for (int i = 0; i < ns; ++i) {
            const int r0 = i * cfg.mm_rows_sum, r1 = std::min(s.H, r0 + cfg.mm_rows_sum);
            add(make_task(OP_MOESUM, l, r0, r1, 0, 0, -1, 0, cl.down(l), nd, cl.moesum(l), lv + 8),
                4.0 * B * (s.K + 1) * (r1 - r0), kDynamic);
        }
        P.targets[cl.moesum(l)] = ns;
    }
    // the final RMSNorm once per token, stored split: the LM-head tiles then
    // stream their rows against a ready operand instead of each normalising
    // every token's residual again
    for (int b = 0; b < B; ++b)
        add(make_task(OP_FNORM, 0, b, b + 1, 0, 0, -1, 0, cl.moesum(s.L - 1), ns, cl.fnorm(), P.n_levels - 2),
            8.0 * s.H, kStatic);
    P.targets[cl.fnorm()] = B;
    for (int i = 0; i < nl; ++i) {
        const int r0 = i * cfg.mm_rows_lm, r1 = std::min(s.V, r0 + cfg.mm_rows_lm);
        add(make_task(OP_LMHEAD, 0, r0, r1, 0, 0, -1, 0, cl.fnorm(), B, -1, P.n_levels - 1),
            2.0 * (r1 - r0) * s.H, kStatic);
    }
}

// Workgroup lists from the levels (see the comment inside).
static void place_tiles(const TileConfig& cfg, int n_wg, std::vector<std::vector<Tile>>& levels, Plan& P) {
    // Per-op order: level by level.
    P.level_off.assign(P.n_levels + 1, 0);
    for (int lv = 0; lv < P.n_levels; ++lv) {
        P.level_off[lv + 1] = P.level_off[lv] + (int)levels[lv].size();
        for (const Tile& t : levels[lv]) P.level_tasks.push_back(t.t);
    }

    // Workgroup lists by list scheduling over a simple timing model. Each
    // workgroup runs its tasks in order; a task's weights start loading when
    // the workgroup is free (and, for expert tiles, once the routing is
    // known), and it computes once its inputs are ready:
    //   finish = max(max(free, weights_ready) + bytes / bw, inputs_ready) + overhead.
    // Tiles go, level by level and largest first, to the workgroup that is
    // free earliest, so workgroups idle at the tail of one operation take the
    // next one's tiles (backfill) and no workgroup queues a tile behind a late
    // one when another is free. Lists stay in level order (deadlock freedom).
    const double bw = cfg.model_bw_bytes_per_us / n_wg;   // bytes per microsecond per workgroup
    const double overhead = cfg.model_task_us, sync = cfg.model_sync_us;
    //
    // The expert tiles stream most of a layer's bytes once the routing is
    // known, so they are spread evenly over compute units: with two
    // workgroups per unit, workgroups w and w + n_wg/2 share one. The down
    // tiles go to the lower half (to either half when there are more of them
    // than lower workgroups, so that none runs two while an upper one runs
    // none); the gate/up tiles to every workgroup when
    // there is one per workgroup (each then holds all its rows in flight, and
    // the down tile that follows on a lower workgroup reuses its routing),
    // else to the upper half.
    std::vector<std::vector<Task>> lists(n_wg);
    P.wg_bytes.assign(n_wg, 0.0);
    typedef std::pair<double, int> Slot;
    typedef std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> Heap;
    // (one- and two-token schedule only; the matrix-core expert tiles are many
    // more than the workgroups and go wherever a workgroup is free first)
    const int half = (n_wg % 2 == 0 && !P.mm) ? n_wg / 2 : 0;
    Heap heaps[2];   // [0]: workgroups below `half`, [1]: the rest
    for (int w = 0; w < n_wg; ++w) heaps[w >= half ? 1 : 0].push({0.0, w});
    std::vector<double> level_end(P.n_levels, 0.0);
    auto producer_end = [&](int lv) { return lv > 0 ? level_end[lv - 1] + sync : 0.0; };
    for (int lv = 0; lv < P.n_levels; ++lv) {
        std::vector<Tile> tiles = levels[lv];
        std::stable_sort(tiles.begin(), tiles.end(), [](const Tile& a, const Tile& b) { return a.bytes > b.bytes; });
        const int op = tiles.empty() ? -1 : tiles[0].t.op;
        // inputs ready: the previous level; weights of routed tiles: the router level
        const double ready = producer_end(lv);
        double wready = 0.0;
        if (op == OP_GATEUP) wready = producer_end(lv);
        if (op == OP_DOWN) wready = producer_end(lv - 1);
        double end = 0.0;
        for (const Tile& t : tiles) {
            int hsel;
            if (half > 0 && op == OP_GATEUP && (int)tiles.size() < n_wg) hsel = 1;
            else if (half > 0 && op == OP_DOWN && (int)tiles.size() <= half) hsel = 0;
            else if (heaps[0].empty()) hsel = 1;
            else if (heaps[1].empty()) hsel = 0;
            else hsel = heaps[1].top() < heaps[0].top() ? 1 : 0;
            Heap& heap = heaps[hsel];
            Slot s0 = heap.top();
            heap.pop();
            const double wr = t.kind == kDynamic ? ready : wready;
            const double fin = std::max(std::max(s0.first, wr) + t.bytes / bw, ready) + overhead;
            lists[s0.second].push_back(t.t);
            P.wg_bytes[s0.second] += t.bytes;
            s0.first = fin;
            end = std::max(end, fin);
            heap.push(s0);
        }
        // a level with no tiles ends with the one before it
        level_end[lv] = tiles.empty() ? (lv > 0 ? level_end[lv - 1] : 0.0) : end;
    }
    P.model_us = level_end.back();

    // Shared levels (batches of 3+): each workgroup the model placed tiles of
    // such a level on gets one claim task instead, and the level's tiles go to
    // a pool, largest first, that those workgroups drain in order. By default
    // the attention, merge, output-projection and expert levels are shared
    // when the sequences need different numbers of attention chunks (ragged
    // contexts): the attention tiles then differ in length and the levels
    // after them start unevenly, which the timing model places worse than
    // first-free claiming does. Uniform batches keep fixed lists (claiming
    // costs one atomic round trip per tile).
    std::vector<Task> pool;
    std::vector<std::vector<int>> claim_pos(n_wg);   // list positions of claim tasks
    bool ragged = false;
    for (int b = 1; b < P.B; ++b) ragged = ragged || P.n_chunks[b] != P.n_chunks[0];
    auto shared_op = [&](int op) {
        if (cfg.shared_levels < 0 || !P.mm) return false;
        if (cfg.shared_levels >= 2 || (cfg.shared_levels == 0 && ragged))
            return op == OP_ATTN || op == OP_COMBINE || op == OP_OPROJ || op == OP_GATEUP || op == OP_DOWN;
        return op == OP_ATTN && cfg.shared_levels == 1;
    };
    {
        std::vector<int> pool_start(P.n_levels, -1), pool_size(P.n_levels, 0);
        for (int lv = 0; lv < P.n_levels; ++lv) {
            if (levels[lv].empty() || !shared_op(levels[lv][0].t.op)) continue;
            std::vector<Tile> tiles = levels[lv];
            std::stable_sort(tiles.begin(), tiles.end(), [](const Tile& a, const Tile& b) { return a.bytes > b.bytes; });
            pool_start[lv] = (int)pool.size();
            pool_size[lv] = (int)tiles.size();
            for (const Tile& t : tiles) pool.push_back(t.t);
        }
        for (int w = 0; w < n_wg; ++w) {
            std::vector<Task> out;
            for (const Task& t : lists[w]) {
                const int lv = t.level;
                if (pool_start[lv] < 0) {
                    out.push_back(t);
                } else if (out.empty() || out.back().op != OP_CLAIM || out.back().level != lv) {
                    claim_pos[w].push_back((int)out.size());
                    out.push_back(make_task(OP_CLAIM, t.layer, pool_start[lv], pool_size[lv], lv, 0, -1, 0, -1, 0, -1,
                                            lv));
                }
            }
            lists[w].swap(out);
        }
    }
    P.wg_off.assign(n_wg + 1, 0);
    for (int w = 0; w < n_wg; ++w) {
        P.wg_off[w + 1] = P.wg_off[w] + (int)lists[w].size();
        P.tasks.insert(P.tasks.end(), lists[w].begin(), lists[w].end());
    }
    // pool positions become task-table indices
    const int list_end = P.wg_off[n_wg];
    for (int w = 0; w < n_wg; ++w)
        for (int i : claim_pos[w]) P.tasks[P.wg_off[w] + i].a0 += list_end;
    P.tasks.insert(P.tasks.end(), pool.begin(), pool.end());
}

// Read coverage ("no missing dependency"): every exchange-buffer range a
// tile reads was written by tiles whose completion the tile's waits imply.
// deps(c) is the set of counters whose producers have all finished once
// counter c reached its target: c itself and, recursively, the counters its
// producers waited on. For each tile, the counters signalled by the tiles
// that write what it reads must lie in deps(ctr) | deps(pre_ctr). Writes
// are looked up per producing operation: which counters its tiles signal,
// for a whole layer or for one KV group, hidden-row range or sequence.
// What task t reads, by producer: need(op, layer, sel) for every tile of op
// in layer (sel -1) or the tiles of one KV group (QKV, sel = group) or of one
// (sequence, group) (attention, sel = b * Hkv + g); need_rows(op, layer, r0,
// r1) for the tiles of op writing rows [r0, r1) of the residual. Returns the
// first non-empty result. One definition for the validator and the thread
// executor.
template <class Need, class NeedRows>
static std::string for_each_read(const ModelShape& s, const Plan& P, const Task& t, Need&& need, NeedRows&& need_rows) {
    const int G = s.Hq / s.Hkv;
    const int x_op = P.mm ? OP_MOESUM : OP_DOWN;   // writes the layer output
    const int l = t.layer;
    // the residual stream entering layer l: the embedding or the previous layer's output
    auto x_in = [&](int layer) { return layer == 0 ? need(OP_EMBED, 0, -1) : need(x_op, layer - 1, -1); };
    std::string e;
    switch (t.op) {
        case OP_EMBED: break;
        case OP_QKV: e = x_in(l); break;
        case OP_ATTN: e = need(OP_QKV, l, t.a1); break;
        case OP_COMBINE: e = need(OP_ATTN, l, t.a0 * s.Hkv + t.a1 / G); break;
        case OP_OPROJ:
            e = need(OP_COMBINE, l, -1);
            if (e.empty()) e = l == 0 ? need(OP_EMBED, 0, -1) : need_rows(x_op, l - 1, t.a0, t.a1);
            break;
        case OP_ROUTER: e = need(OP_OPROJ, l, -1); break;
        case OP_ROUTE: e = need(OP_ROUTER, l, -1); break;
        case OP_GATEUP:
            e = need(OP_ROUTER, l, -1);
            if (e.empty()) e = P.mm ? need(OP_ROUTE, l, -1) : need(OP_OPROJ, l, -1);
            break;
        case OP_DOWN:
            e = need(OP_GATEUP, l, -1);
            if (e.empty()) e = P.mm ? need(OP_ROUTE, l, -1) : need(OP_ROUTER, l, -1);
            if (e.empty() && !P.mm) e = need_rows(OP_OPROJ, l, t.a0, t.a1);
            break;
        case OP_MOESUM:
            e = need(OP_DOWN, l, -1);
            if (e.empty()) e = need(OP_ROUTE, l, -1);
            if (e.empty()) e = need_rows(OP_OPROJ, l, t.a0, t.a1);
            break;
        case OP_FNORM: e = need(x_op, s.L - 1, -1); break;
        case OP_LMHEAD: e = P.mm ? need(OP_FNORM, 0, -1) : need(x_op, s.L - 1, -1); break;
        default: break;
    }
    return e;
}

// Writers of each (op, layer, selector) and of residual rows, as task
// indices or as the counters they signal (see for_each_read).
struct WriterKey {
    int op, layer, sel;
    bool operator<(const WriterKey& o) const { return std::tie(op, layer, sel) < std::tie(o.op, o.layer, o.sel); }
};
template <class F>
static void for_each_writer(const ModelShape& s, const Plan& P, F&& f) {
    for (int i = 0; i < (int)P.tasks.size(); ++i) {
        const Task& t = P.tasks[i];
        if (t.op == OP_CLAIM) continue;
        f(WriterKey{t.op, t.layer, -1}, i);
        if (t.op == OP_QKV) f(WriterKey{t.op, t.layer, t.a0}, i);                    // KV group
        if (t.op == OP_ATTN) f(WriterKey{t.op, t.layer, t.a0 * s.Hkv + t.a1}, i);   // (sequence, group)
    }
}
static bool writes_rows(const Plan& P, const Task& t) {
    return t.op == OP_OPROJ || (t.op == OP_DOWN && !P.mm) || t.op == OP_MOESUM;
}

static std::string check_reads(const ModelShape& s, const Plan& P, const std::vector<int>& prod_level) {
    const CounterLayout cl{s.L, s.Hkv, s.max_batch};
    const int n_main = cl.n_main();
    const int W = (n_main + 63) / 64;
    typedef std::vector<uint64_t> Bits;
    // producers' waits per counter
    std::vector<std::set<std::pair<int, int>>> pw(n_main);
    for (const Task& t : P.tasks)
        if (t.op != OP_CLAIM && t.signal >= 0) pw[t.signal].insert({t.ctr, t.pre_ctr});
    // deps in counter order of producer level (lower levels first)
    std::vector<int> order(n_main);
    for (int c = 0; c < n_main; ++c) order[c] = c;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return prod_level[a] < prod_level[b]; });
    std::vector<Bits> deps(n_main, Bits(W, 0));
    for (int c : order) {
        if (prod_level[c] < 0) continue;
        Bits& d = deps[c];
        d[c / 64] |= 1ull << (c % 64);
        for (const auto& w : pw[c])
            for (int x : {w.first, w.second})
                if (x >= 0)
                    for (int i = 0; i < W; ++i) d[i] |= deps[x][i];
    }
    auto has = [&](const Bits& d, int c) { return c >= 0 && ((d[c / 64] >> (c % 64)) & 1ull); };
    // writers: per (op, layer) the counters signalled, whole and per selector
    std::map<WriterKey, std::set<int>> wr;   // sel -1: every tile of the op
    for_each_writer(s, P, [&](const WriterKey& k, int i) { wr[k].insert(P.tasks[i].signal); });
    std::map<std::pair<int, int>, std::vector<std::tuple<int, int, int>>> rows;   // (op, layer) -> (r0, r1, signal)
    for (const Task& t : P.tasks)
        if (t.op != OP_CLAIM && writes_rows(P, t)) rows[{t.op, t.layer}].push_back(std::make_tuple(t.a0, t.a1, t.signal));
    char buf[256];
    for (const Task& t : P.tasks) {
        if (t.op == OP_CLAIM) continue;
        Bits d(W, 0);
        for (int c : {t.ctr, t.pre_ctr})
            if (c >= 0)
                for (int i = 0; i < W; ++i) d[i] |= deps[c][i];
        auto need = [&](int op, int layer, int sel) -> std::string {
            auto it = wr.find({op, layer, sel});
            if (it == wr.end()) {
                snprintf(buf, sizeof buf, "op %d layer %d reads what no op-%d tile (layer %d, part %d) writes", t.op,
                         t.layer, op, layer, sel);
                return buf;
            }
            for (int c : it->second)
                if (!has(d, c)) {
                    snprintf(buf, sizeof buf, "op %d layer %d reads op %d layer %d output without waiting on counter %d",
                             t.op, t.layer, op, layer, c);
                    return buf;
                }
            return std::string();
        };
        auto need_rows = [&](int op, int layer, int r0, int r1) -> std::string {
            for (const auto& w : rows[{op, layer}])
                if (std::get<0>(w) < r1 && r0 < std::get<1>(w) && !has(d, std::get<2>(w))) {
                    snprintf(buf, sizeof buf, "op %d layer %d reads rows %d..%d of op %d without waiting on counter %d",
                             t.op, t.layer, r0, r1, op, std::get<2>(w));
                    return buf;
                }
            return std::string();
        };
        const std::string e = for_each_read(s, P, t, need, need_rows);
        if (!e.empty()) return e;
    }
    return std::string();
}

std::vector<std::vector<int>> read_producers(const ModelShape& s, const Plan& P) {
    std::map<WriterKey, std::vector<int>> wr;
    for_each_writer(s, P, [&](const WriterKey& k, int i) { wr[k].push_back(i); });
    std::map<std::pair<int, int>, std::vector<std::tuple<int, int, int>>> rows;   // (op, layer) -> (r0, r1, task)
    for (int i = 0; i < (int)P.tasks.size(); ++i)
        if (P.tasks[i].op != OP_CLAIM && writes_rows(P, P.tasks[i]))
            rows[{P.tasks[i].op, P.tasks[i].layer}].push_back(std::make_tuple(P.tasks[i].a0, P.tasks[i].a1, i));
    std::vector<std::vector<int>> out(P.tasks.size());
    for (int i = 0; i < (int)P.tasks.size(); ++i) {
        const Task& t = P.tasks[i];
        if (t.op == OP_CLAIM) continue;
        std::vector<int>& o = out[i];
        auto need = [&](int op, int layer, int sel) -> std::string {
            auto it = wr.find({op, layer, sel});
            if (it != wr.end()) o.insert(o.end(), it->second.begin(), it->second.end());
            return std::string();
        };
        auto need_rows = [&](int op, int layer, int r0, int r1) -> std::string {
            for (const auto& w : rows[{op, layer}])
                if (std::get<0>(w) < r1 && r0 < std::get<1>(w)) o.push_back(std::get<2>(w));
            return std::string();
        };
        for_each_read(s, P, t, need, need_rows);
    }
    return out;
}

std::string validate_plan(const ModelShape& s, const Plan& P) {
    const CounterLayout cl{s.L, s.Hkv, s.max_batch};
    const int n_main = cl.n_main();
    char buf[256];
    if ((int)P.wg_off.size() != P.n_wg + 1) return "wg_off size";
    if (P.wg_off.back() > (int)P.tasks.size()) return "wg_off end";
    // claim tasks: each names a pool range of tasks of its own level past the
    // lists; every pool task lies in exactly one range (claimed ranges may be
    // named by many claim tasks)
    const int list_end = P.wg_off.back();
    std::vector<int> in_pool(P.tasks.size(), 0);
    std::set<std::pair<int, int>> ranges_seen;
    int n_claim = 0;
    for (int i = 0; i < list_end; ++i) {
        const Task& t = P.tasks[i];
        if (t.op != OP_CLAIM) continue;
        ++n_claim;
        if (t.a0 < list_end || t.a1 <= 0 || t.a0 + t.a1 > (int)P.tasks.size()) return "claim range out of the pool";
        if (t.a2 != t.level) return "claim of another level";
        if (ranges_seen.insert({t.a0, t.a1}).second) {
            for (int j = t.a0; j < t.a0 + t.a1; ++j) {
                if (P.tasks[j].level != t.level || P.tasks[j].op == OP_CLAIM) return "pool task of another level";
                in_pool[j]++;
            }
        } else if (P.tasks[t.a0].level != t.level) {
            return "pool task of another level";
        }
    }
    for (int j = list_end; j < (int)P.tasks.size(); ++j)
        if (in_pool[j] != 1) return "pool task claimed by no range or by two";
    if (P.level_tasks.size() != P.tasks.size() - n_claim) return "task count differs between orders";
    // final counter values and producer levels
    std::vector<int> final_val(n_main, 0), prod_level(n_main, -1);
    for (const Task& t : P.tasks) {
        if (t.signal < -1 || t.signal >= n_main) return "signal out of range";
        if (t.signal < 0) continue;
        final_val[t.signal]++;
        if (prod_level[t.signal] >= 0 && prod_level[t.signal] != t.level) return "counter fed from two levels";
        prod_level[t.signal] = t.level;
    }
    for (int c = 0; c < n_main; ++c)
        if (final_val[c] != P.targets[c]) {
            snprintf(buf, sizeof buf, "counter %d reaches %d, target list says %d", c, final_val[c], P.targets[c]);
            return buf;
        }
    for (const Task& t : P.tasks) {
        const int waits[2][2] = {{t.pre_ctr, t.pre_target}, {t.ctr, t.target}};
        for (auto& w : waits) {
            if (w[0] < 0) continue;
            if (w[0] >= n_main) return "wait counter out of range";
            if (w[1] != final_val[w[0]] || w[1] <= 0) {
                snprintf(buf, sizeof buf, "task op %d layer %d waits for %d on counter %d, which reaches %d", t.op,
                         t.layer, w[1], w[0], final_val[w[0]]);
                return buf;
            }
            if (prod_level[w[0]] >= t.level) return "task waits on a counter of its own or a later level";
        }
    }
    // list order
    for (int w = 0; w < P.n_wg; ++w)
        for (int i = P.wg_off[w] + 1; i < P.wg_off[w + 1]; ++i)
            if (P.tasks[i].level < P.tasks[i - 1].level) return "workgroup list not in level order";
    // coverage of every operation's output range
    std::map<std::tuple<int, int, int, int>, std::vector<std::pair<int, int>>> ranges;
    for (const Task& t : P.tasks) {
        switch (t.op) {
            case OP_QKV: ranges[std::make_tuple(t.op, t.layer, t.a0, 0)].push_back({t.a1, t.a2}); break;
            case OP_ATTN: ranges[std::make_tuple(t.op, t.layer, t.a0, t.a1)].push_back({t.a2, t.a2 + 1}); break;
            // router tiles: per 16-token block (upper half of a2), and the
            // token blocks themselves once, under the first row block
            case OP_ROUTER:
                ranges[std::make_tuple(t.op, t.layer, t.a2 >> 16, 0)].push_back({t.a0, t.a1});
                if (t.a0 == 0) ranges[std::make_tuple(OP_COUNT + OP_ROUTER, t.layer, 0, 0)].push_back({t.a2 >> 16, (t.a2 >> 16) + 1});
                break;
            case OP_EMBED:
            case OP_OPROJ:
            case OP_ROUTE:
            case OP_MOESUM:
            case OP_FNORM:
            case OP_LMHEAD: ranges[std::make_tuple(t.op, t.layer, 0, 0)].push_back({t.a0, t.a1}); break;
            // one-/two-token down tiles carry their row count in a2 (the same for
            // every tile); matrix-core down tiles their slot group
            case OP_DOWN: ranges[std::make_tuple(t.op, t.layer, t.a2, 0)].push_back({t.a0, t.a1}); break;
            // one-/two-token gate/up tiles: slot a0, rows a1..a2; matrix-core
            // ones: rows a0..a1 of slot group a2
            case OP_GATEUP:
                if (P.mm) ranges[std::make_tuple(t.op, t.layer, t.a2, 0)].push_back({t.a0, t.a1});
                else ranges[std::make_tuple(t.op, t.layer, t.a0, 0)].push_back({t.a1, t.a2});
                break;
            case OP_COMBINE: ranges[std::make_tuple(t.op, t.layer, t.a0, 0)].push_back({t.a1, t.a1 + 1}); break;
            default: break;
        }
    }
    const int G = s.Hq / s.Hkv;
    for (auto& kv : ranges) {
        auto& v = kv.second;
        std::sort(v.begin(), v.end());
        int end = 0;
        for (auto& r : v) {
            if (r.first != end) return "tile ranges overlap or leave a gap";
            end = r.second;
        }
        const int op = std::get<0>(kv.first);
        int want = 0;
        switch (op) {
            case OP_EMBED: case OP_FNORM: want = P.B; break;
            case OP_ROUTE: want = 1; break;
            case OP_QKV: want = (G + 2) * s.D; break;
            case OP_ATTN: want = P.n_chunks[std::get<2>(kv.first)]; break;
            case OP_COMBINE: want = s.Hq; break;
            case OP_OPROJ: case OP_DOWN: case OP_MOESUM: want = s.H; break;
            case OP_ROUTER: want = s.E; break;
            case OP_COUNT + OP_ROUTER: want = P.mm ? ceil_div(P.B, 16) : 1; break;
            case OP_GATEUP: want = s.I; break;
            case OP_LMHEAD: want = s.V; break;
        }
        if (end != want) return "tile ranges do not cover the operation";
    }
    return check_reads(s, P, prod_level);
}

}  // namespace mk
