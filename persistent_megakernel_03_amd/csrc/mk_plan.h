// mk_plan.h -- host task-graph builder for one decode step.
//
// The host prepares, for every persistent workgroup, a list of small tasks
// ("Cohere Publishes One-Kernel Server for North Mini Code, Claims 1.58x vLLM
// Speedup", section "One resident program, many small tasks"). Operations are
// cut into tiles so that scheduling works at tile granularity, workgroups
// idle at the tail of one operation pick up tiles of the next (backfill), and
// each tile waits only on the tiles it reads ("Inside the Megakernel Serving
// Engine for North Mini Code", paragraph 4; first page, section "What the
// scheduling change is meant to avoid").
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "mk_common.h"

namespace mk {

struct ModelShape {
    int L, H, Hq, Hkv, D, E, K, I, V, P;
    int max_batch, max_pages;
    int max_chunks;  // capacity of the attention partial buffer per (b, head)
};

struct TileConfig {
    int rows_qkv = 24;
    int rows_o = 8;
    int rows_router = 8;
    int rows_gateup = 16;
    int rows_down = 4;
    int rows_lm = 64;
    // batches of 3+ (matrix-core tiles): rows per tile
    int mm_rows_qkv = 16;
    int mm_rows_o = 8;
    int mm_rows_router = 8;
    int mm_rows_sum = 16;
    int mm_rows_lm = 32;
    int mm_embed_tokens = 4;
    int chunk = 0;  // attention chunk in tokens (multiple of 64); 0 = choose
    // batches of 3+, levels whose tiles workgroups claim from a shared pool
    // (claim tasks) instead of fixed lists: -1 none; 0 the attention, merge,
    // output-projection and expert levels when the sequences need different
    // numbers of attention chunks, else none; 1 the attention level; 2 the
    // attention, merge, output-projection and expert levels
    int shared_levels = 0;
    // smallest batch that runs the matrix-core schedule (1..kMaxBatchValu + 1)
    int mm_min_batch = kMaxBatchValu + 1;
    // row blocks per matrix-core expert tile: 0 = mm_row_blocks(), else 1..kMmMaxRowBlocks
    int mm_row_blocks = 0;
    // timing model used to place tiles on workgroups
    double model_bw_bytes_per_us = 5.6e6;  // whole-device HBM bandwidth
    double model_task_us = 2.5;            // fixed cost of a task after its inputs are ready
    double model_sync_us = 1.0;            // producer signal to consumer start
};

struct Plan {
    int n_wg = 0;
    int B = 0;
    bool mm = false;                  // the matrix-core schedule (else the one- and two-token tiles)
    int rb = 1;                       // row blocks per matrix-core expert tile
    int chunk = 0;
    int n_levels = 0;
    std::vector<Task> tasks;          // grouped per workgroup (CSR)
    std::vector<int32_t> wg_off;      // n_wg + 1
    std::vector<Task> level_tasks;    // grouped per level (per-op launches)
    std::vector<int32_t> level_off;   // n_levels + 1
    std::vector<int32_t> n_chunks;    // per sequence
    std::vector<int32_t> targets;     // final value of every main counter
    std::vector<double> wg_bytes;     // bytes streamed per workgroup (balance)
    double model_us = 0.0;            // modelled step time
};

// Rows per gate/up tile and per down tile. When the step's distinct experts
// allow it, down tiles are sized so that each holds all its weights in
// registers and gate/up tiles so that both kinds fit on the workgroups at
// once: the down weights then stream alongside the gate/up weights instead of
// after them. Otherwise the configured sizes.
void expert_rows(const ModelShape& s, const TileConfig& cfg, int n_wg, int S, int* rows_gu, int* rows_down);

// Batches of 3+: row blocks per expert tile (1 or 2), then the slot groups
// of the gate/up tiles (rb 8-row blocks of the expert width) and of the down
// tiles (rb 16-row blocks of the hidden size).
int mm_row_blocks(const ModelShape& s, int n_wg, int B);
void expert_groups_mm(const ModelShape& s, int n_wg, int S, int rb, int* gu_groups, int* down_groups);

// For each task of P (by index), the tasks whose outputs it reads: the
// relation validate_plan proves covered by waits, as task indices (used by
// the host thread executor of the tests).
std::vector<std::vector<int>> read_producers(const ModelShape& s, const Plan& P);

// Attention chunk length for these contexts (tokens, multiple of 64).
int choose_chunk(const ModelShape& s, int n_wg, int B, const int32_t* positions, int requested);

// Build the plan. Returns an empty string on success, else a message.
std::string build_plan(const ModelShape& s, const TileConfig& cfg, int n_wg, int B,
                       const int32_t* positions, Plan* out);

// Check the plan's invariants: every task waits only on counters fed by
// tasks of strictly lower level with targets equal to the producer counts;
// each workgroup's list is in non-decreasing level order (so with all
// workgroups co-resident the lowest unfinished task can always run); every
// tile of the step appears exactly once. Empty string = valid.
std::string validate_plan(const ModelShape& s, const Plan& plan);

// Upper bound on tasks for any batch <= max_batch on at most n_wg workgroups.
int64_t max_tasks(const ModelShape& s, const TileConfig& cfg, int n_wg);

}  // namespace mk
