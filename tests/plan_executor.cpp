// Host thread executor of a step's task lists, built with ThreadSanitizer by
// tests/test_plan_executor_host.py (test infrastructure, not part of the
// library).
//
// One std::thread per workgroup walks its list exactly as the persistent
// kernel does, claim tasks included (a per-level atomic pool position). A
// task waits until its counters reach their targets (acquire loads), checks
// that every task whose output it reads (read_producers: the relation the
// plan validator proves covered) has finished, marks itself finished with a
// plain store and bumps its counter (release add). The pages' scheme is
// exactly this: per-tile counters in memory record when a task's inputs are
// ready ("Cohere Publishes One-Kernel Server for North Mini Code, Claims
// 1.58x vLLM Speedup", "One resident program, many small tasks").
//
// Two checks see a read that no chain of waits orders after its producer:
// ThreadSanitizer reports the unordered accesses to the plain flags (it keeps
// only a few accesses per 8 bytes, so other threads' reads can hide one), and
// a vector clock per thread and per counter, carried by the waits and signals
// alone, reports it on every run whatever the timing. A read that also came
// first is reported as such. A wait that never ends (a deadlock) fails after a
// bounded time instead of hanging.
//
// usage: plan_executor SHAPE N_WG POSITIONS SHARED_LEVELS SEED [PLANT [DEADLINE_S]]
//   SHAPE tiny | a3b; POSITIONS comma-separated (the batch). PLANT: an op
//   code whose first task in layer 0 then skips its main wait (a planted
//   missing dependency, which must be reported), or "stuck": the first
//   waiting task of layer 0 waits for one signal more than its counter ever
//   gets (a planted deadlock, which must end at the deadline, default 120 s).
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <sstream>
#include <string>
#include <thread>
#include <vector>

#include "mk_plan.h"

using namespace mk;

// Clock merges, left out of the race detector's instrumentation: they are
// bookkeeping, not accesses of the protocol (and instrumented they would
// dominate the run time).
__attribute__((no_sanitize("thread"))) static void clock_acquire(uint32_t* v, const std::atomic<uint32_t>* cv, int W) {
    for (int k = 0; k < W; ++k) v[k] = std::max(v[k], cv[k].load(std::memory_order_relaxed));
}
__attribute__((no_sanitize("thread"))) static void clock_release(const uint32_t* v, std::atomic<uint32_t>* cv, int W) {
    for (int k = 0; k < W; ++k) {
        uint32_t cur = cv[k].load(std::memory_order_relaxed);
        while (cur < v[k] && !cv[k].compare_exchange_weak(cur, v[k], std::memory_order_relaxed)) {
        }
    }
}

static ModelShape shape(const std::string& name, int max_batch) {
    ModelShape s;
    if (name == "tiny") {
        s.L = 2; s.H = 256; s.Hq = 4; s.Hkv = 2; s.D = 64; s.E = 8; s.K = 2; s.I = 128; s.V = 1024;
    } else {
        s.L = 48; s.H = 2048; s.Hq = 32; s.Hkv = 4; s.D = 128; s.E = 128; s.K = 8; s.I = 768; s.V = 151936;
    }
    s.P = 16;
    s.max_batch = max_batch;
    s.max_pages = 1024;
    s.max_chunks = 2048;
    return s;
}

int main(int argc, char** argv) {
    if (argc < 6) {
        fprintf(stderr, "usage: %s SHAPE N_WG POSITIONS SHARED_LEVELS SEED [PLANT [DEADLINE_S]]\n", argv[0]);
        return 2;
    }
    const std::string name = argv[1];
    const int n_wg = atoi(argv[2]);
    std::vector<int32_t> pos;
    {
        std::stringstream ss(argv[3]);
        std::string x;
        while (std::getline(ss, x, ',')) pos.push_back(atoi(x.c_str()));
    }
    const int B = (int)pos.size();
    TileConfig cfg;
    cfg.shared_levels = atoi(argv[4]);
    const unsigned seed = (unsigned)atoi(argv[5]);
    const bool stuck = argc > 6 && std::string(argv[6]) == "stuck";
    const int drop_op = argc > 6 && !stuck ? atoi(argv[6]) : -1;
    const int deadline_s = argc > 7 ? atoi(argv[7]) : 120;
    const ModelShape s = shape(name, B);

    Plan P;
    std::string e = build_plan(s, cfg, n_wg, B, pos.data(), &P);
    if (!e.empty()) {
        printf("build_plan: %s\n", e.c_str());
        return 1;
    }
    if (stuck) {
        for (Task& t : P.tasks)
            if (t.layer == 0 && t.ctr >= 0) {
                t.target += 1;
                break;
            }
    } else if (drop_op >= 0) {
        bool found = false;
        for (Task& t : P.tasks)
            if (t.op == drop_op && t.layer == 0 && t.ctr >= 0) {
                t.ctr = -1;
                t.target = 0;
                found = true;
                break;
            }
        if (!found) {
            printf("no task of op %d to drop a wait from\n", drop_op);
            return 3;
        }
    } else if (!(e = validate_plan(s, P)).empty()) {
        printf("validate_plan: %s\n", e.c_str());
        return 1;
    }
    const std::vector<std::vector<int>> reads = read_producers(s, P);
    const int n_tasks = (int)P.tasks.size();
    std::vector<std::atomic<uint32_t>> ctr(P.targets.size());
    for (auto& c : ctr) c.store(0, std::memory_order_relaxed);
    std::map<int, std::atomic<int>> claim;
    for (const Task& t : P.tasks)
        if (t.op == OP_CLAIM) claim[t.a2].store(0, std::memory_order_relaxed);
    // plain on purpose, one 8-byte cell each: the race detector watches them
    std::vector<int64_t> done(n_tasks, 0);
    // vector clocks: component w counts the tasks workgroup w has finished;
    // a task run by w as its k-th is ordered before a reader whose clock has
    // component w > k. Relaxed atomics carry the counters' clocks, so the
    // clocks add no synchronisation that the race detector would see.
    const int W = P.n_wg;
    std::vector<int32_t> run_by(n_tasks, -1), run_seq(n_tasks, -1);
    std::vector<std::vector<uint32_t>> vc(W, std::vector<uint32_t>(W, 0));
    std::vector<std::atomic<uint32_t>> cvc(P.targets.size() * (size_t)W);
    for (auto& x : cvc) x.store(0, std::memory_order_relaxed);
    std::atomic<int> failed{0};
    std::atomic<long> n_reads{0}, n_run{0};
    const auto deadline = std::chrono::steady_clock::now() + std::chrono::seconds(deadline_s);

    auto wait = [&](int c, int target) {
        if (c < 0) return true;
        int spins = 0;
        while (ctr[c].load(std::memory_order_acquire) < (uint32_t)target) {
            if (failed.load(std::memory_order_relaxed)) return false;
            if (++spins % 1024 == 0 && std::chrono::steady_clock::now() > deadline) {
                printf("deadlock: counter %d stuck below %d\n", c, target);
                failed.store(1);
                return false;
            }
            std::this_thread::yield();
        }
        return true;
    };
    auto acquire = [&](int w, int c) {   // after the wait on counter c ended
        if (c >= 0) clock_acquire(vc[w].data(), &cvc[(size_t)c * W], W);
    };
    auto release = [&](int w, int c) {   // before the signal of counter c
        clock_release(vc[w].data(), &cvc[(size_t)c * W], W);
    };
    auto run = [&](int w, int ti, std::mt19937& rng) {
        const Task& t = P.tasks[ti];
        if (!wait(t.pre_ctr, t.pre_target) || !wait(t.ctr, t.target)) return false;
        acquire(w, t.pre_ctr);
        acquire(w, t.ctr);
        if (rng() % 8 == 0) std::this_thread::yield();   // vary the interleaving
        long nr = 0;
        for (int q : reads[ti]) {
            ++nr;
            if (done[q] != 1 || run_by[q] < 0) {
                printf("task %d (op %d layer %d) read the output of task %d (op %d layer %d) before it was written\n",
                       ti, t.op, t.layer, q, P.tasks[q].op, P.tasks[q].layer);
                failed.store(1);
                return false;
            }
            const int by = run_by[q];
            if (by != w && vc[w][by] <= (uint32_t)run_seq[q]) {
                printf("task %d (op %d layer %d) reads the output of task %d (op %d layer %d), "
                       "which no wait orders before it\n",
                       ti, t.op, t.layer, q, P.tasks[q].op, P.tasks[q].layer);
                failed.store(1);
                return false;
            }
        }
        // relaxed: a sequentially consistent add here would order every task
        // after every earlier one and hide the races this program looks for
        n_reads.fetch_add(nr, std::memory_order_relaxed);
        run_by[ti] = w;
        run_seq[ti] = (int32_t)vc[w][w]++;
        done[ti] = 1;
        n_run.fetch_add(1, std::memory_order_relaxed);
        if (t.signal >= 0) {
            release(w, t.signal);
            ctr[t.signal].fetch_add(1, std::memory_order_release);
        }
        return true;
    };
    auto worker = [&](int w) {
        std::mt19937 rng(seed * 7919u + (unsigned)w);
        int i = P.wg_off[w];
        const int end = P.wg_off[w + 1];
        int cl = -1;
        for (;;) {
            int ti;
            if (cl < 0) {
                if (i >= end) break;
                if (P.tasks[i].op == OP_CLAIM) cl = i;
            }
            if (cl >= 0) {
                const Task& ct = P.tasks[cl];
                const int j = claim[ct.a2].fetch_add(1, std::memory_order_relaxed);
                if (j >= ct.a1) {
                    cl = -1;
                    ++i;
                    continue;
                }
                ti = ct.a0 + j;
            } else {
                ti = i;
            }
            if (!run(w, ti, rng)) return;
            if (cl < 0) ++i;
        }
    };
    std::vector<std::thread> th;
    for (int w = 0; w < P.n_wg; ++w) th.emplace_back(worker, w);
    for (auto& x : th) x.join();
    if (failed.load()) return 1;
    long expect = 0;
    for (const Task& t : P.tasks) expect += t.op != OP_CLAIM;
    // pool tasks are listed once in P.tasks but run through claims; fixed-list
    // tasks once each: every non-claim task must have run exactly once
    if (n_run.load() != expect) {
        printf("ran %ld of %ld tasks\n", n_run.load(), expect);
        return 1;
    }
    printf("ok tasks %d reads %ld\n", n_tasks, n_reads.load());
    return 0;
}
