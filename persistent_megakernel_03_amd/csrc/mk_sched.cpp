// mk_sched.cpp -- the host continuous-batching scheduler declared in
// include/mk_sched.h: request queue, admission, the page free list and the
// rows of each multi-token step.
#include <algorithm>
#include <deque>
#include <memory>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/mk_sched.h"
#include "mk_host.h"

namespace {

struct Request {
    int64_t id = 0;
    int32_t cached = 0;              // positions 0..cached-1 are in the cache at admission
    int32_t prompt_len = 0;
    int32_t max_new = 0;
    std::vector<int32_t> toks;       // prompt, then generated tokens
    int32_t fed = 0;                 // toks[0..fed) are in the cache (at positions cached..)
    int32_t n_gen = 0;
    std::vector<int32_t> pages;      // pages[i] holds positions [i P, (i+1) P)
    int32_t reserve = 0;             // pages reserved at admission (reserve_full), else 0
    int32_t slot = -1;
    bool finished = false;

    int32_t next_pos() const { return cached + fed; }
    bool decoding() const { return fed >= prompt_len; }
};

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

}  // namespace

struct mk_sched {
    mk_sched_config cfg;
    std::vector<int32_t> free_pages;                     // back = next handed out
    std::unordered_map<int64_t, std::unique_ptr<Request>> reqs;
    std::deque<Request*> queue;
    std::vector<Request*> slots;                         // max_seqs entries, nullptr = free
    int64_t outstanding = 0;                             // reserved but not yet allocated pages
    // the step laid out by the last mk_sched_next, until committed
    struct Row {
        Request* r;
        bool sample;
    };
    std::vector<Row> pending;
    bool has_pending = false;
    mk_sched_stats st{};

    int32_t pages_for(const Request& r, int64_t n_tokens) const { return ceil_div(n_tokens, cfg.page_size); }

    void free_request_pages(Request* r) {
        for (auto it = r->pages.rbegin(); it != r->pages.rend(); ++it) free_pages.push_back(*it);
        if (r->reserve > 0) outstanding -= std::max<int64_t>(0, r->reserve - (int64_t)r->pages.size());
        r->pages.clear();
        r->reserve = 0;
        if (r->slot >= 0) slots[r->slot] = nullptr;
        r->slot = -1;
    }

    int32_t running() const {
        int32_t n = 0;
        for (Request* r : slots) n += r != nullptr;
        return n;
    }

    // admission: oldest first; stops at the first request that does not fit
    void admit() {
        while (!queue.empty()) {
            Request* r = queue.front();
            int32_t slot = -1;
            for (int32_t i = 0; i < cfg.max_seqs && slot < 0; ++i)
                if (!slots[i]) slot = i;
            if (slot < 0) return;
            const int32_t now = pages_for(*r, r->cached);   // the cached prefix
            int32_t need;
            if (cfg.reserve_full) {
                need = pages_for(*r, (int64_t)r->cached + r->prompt_len + r->max_new);
                if ((int64_t)free_pages.size() - outstanding < need) return;
            } else {
                need = pages_for(*r, (int64_t)r->cached + r->prompt_len + 1);
                if ((int64_t)free_pages.size() - outstanding < need) return;
            }
            queue.pop_front();
            r->slot = slot;
            slots[slot] = r;
            for (int32_t i = 0; i < now; ++i) {
                r->pages.push_back(free_pages.back());
                free_pages.pop_back();
            }
            if (cfg.reserve_full) {
                r->reserve = need;
                outstanding += need - now;
            }
            ++st.admitted;
        }
    }

    // a page for position pos of r (nullptr-safe): false if none is free
    bool ensure_page(Request* r, int32_t pos) {
        const int32_t pi = pos / cfg.page_size;
        while ((int32_t)r->pages.size() <= pi) {
            const bool from_reserve = r->reserve > (int32_t)r->pages.size();
            if (free_pages.empty() || (!from_reserve && (int64_t)free_pages.size() <= outstanding)) return false;
            r->pages.push_back(free_pages.back());
            free_pages.pop_back();
            if (from_reserve) --outstanding;
        }
        return true;
    }
};

extern "C" {

mk_status mk_sched_create(const mk_sched_config* cfg, const int32_t* page_order, mk_sched** out) {
    try {
        if (!cfg || !out) return mk::host_fail(MK_ERR_INVALID, "null argument");
        *out = nullptr;
        const mk_sched_config& c = *cfg;
        if (c.max_seqs <= 0 || c.max_rows < c.max_seqs || c.page_size <= 0 || c.max_pages_per_seq <= 0 ||
            c.n_pages <= 0 || c.n_pages > (int64_t)1 << 31)
            return mk::host_fail(MK_ERR_INVALID, "scheduler sizes must be positive with max_rows >= max_seqs");
        std::unique_ptr<mk_sched> s(new mk_sched());
        s->cfg = c;
        s->slots.assign(c.max_seqs, nullptr);
        s->free_pages.resize((size_t)c.n_pages);
        if (page_order) {
            std::vector<char> seen((size_t)c.n_pages, 0);
            for (int64_t i = 0; i < c.n_pages; ++i) {
                const int32_t pg = page_order[i];
                if (pg < 0 || pg >= c.n_pages || seen[pg]) return mk::host_fail(MK_ERR_INVALID, "page_order is not a permutation");
                seen[pg] = 1;
                s->free_pages[(size_t)(c.n_pages - 1 - i)] = pg;   // handed out in the given order
            }
        } else {
            for (int64_t i = 0; i < c.n_pages; ++i) s->free_pages[(size_t)i] = (int32_t)(c.n_pages - 1 - i);
        }
        *out = s.release();
        return MK_OK;
    } catch (const std::bad_alloc&) {
        return mk::host_fail(MK_ERR_CAPACITY, "host allocation failed");
    } catch (...) {
        return mk::host_fail(MK_ERR_INVALID, "unexpected exception in mk_sched_create");
    }
}

void mk_sched_destroy(mk_sched* s) { delete s; }

mk_status mk_sched_submit(mk_sched* s, int64_t request_id, int32_t cached_len, const int32_t* prompt,
                          int32_t prompt_len, int32_t max_new_tokens) {
    try {
        if (!s || !prompt) return mk::host_fail(MK_ERR_INVALID, "null argument");
        if (cached_len < 0 || prompt_len < 1 || max_new_tokens < 0)
            return mk::host_fail(MK_ERR_INVALID, "cached_len >= 0, prompt_len >= 1 and max_new_tokens >= 0 required");
        if (s->reqs.count(request_id)) return mk::host_fail(MK_ERR_INVALID, "request %lld exists", (long long)request_id);
        // the last fed position is cached + prompt_len + max_new - 1 (the last
        // generated token is returned, not fed)
        const int64_t last = (int64_t)cached_len + prompt_len + std::max(0, max_new_tokens - 1) - 1;
        if (last / s->cfg.page_size >= s->cfg.max_pages_per_seq)
            return mk::host_fail(MK_ERR_CAPACITY, "request %lld needs position %lld, beyond %d pages",
                                 (long long)request_id, (long long)last, s->cfg.max_pages_per_seq);
        std::unique_ptr<Request> r(new Request());
        r->id = request_id;
        r->cached = cached_len;
        r->prompt_len = prompt_len;
        r->max_new = max_new_tokens;
        r->toks.assign(prompt, prompt + prompt_len);
        s->queue.push_back(r.get());
        s->reqs[request_id] = std::move(r);
        return MK_OK;
    } catch (const std::bad_alloc&) {
        return mk::host_fail(MK_ERR_CAPACITY, "host allocation failed");
    } catch (...) {
        return mk::host_fail(MK_ERR_INVALID, "unexpected exception in mk_sched_submit");
    }
}

mk_status mk_sched_release(mk_sched* s, int64_t request_id) {
    if (!s) return mk::host_fail(MK_ERR_INVALID, "null scheduler");
    auto it = s->reqs.find(request_id);
    if (it == s->reqs.end()) return mk::host_fail(MK_ERR_INVALID, "unknown request %lld", (long long)request_id);
    Request* r = it->second.get();
    if (s->has_pending)
        for (const auto& row : s->pending)
            if (row.r == r) return mk::host_fail(MK_ERR_INVALID, "request %lld is in the pending step", (long long)request_id);
    s->queue.erase(std::remove(s->queue.begin(), s->queue.end(), r), s->queue.end());
    s->free_request_pages(r);
    if (!r->finished) ++s->st.finished;
    s->reqs.erase(it);
    return MK_OK;
}

mk_status mk_sched_next(mk_sched* s, int32_t* batch, int32_t* seq_ids, int32_t* positions, int32_t* block_tables,
                        int32_t* tokens, int32_t* sample, int64_t* request_ids) {
    try {
        if (!s || !batch || !seq_ids || !positions || !block_tables || !tokens || !sample)
            return mk::host_fail(MK_ERR_INVALID, "null argument");
        if (s->has_pending) return mk::host_fail(MK_ERR_INVALID, "the previous step is not committed");
        *batch = 0;
        s->admit();
        const mk_sched_config& c = s->cfg;
        // rows: one per decoding request, then prompt chunks, in slot order
        std::vector<std::pair<Request*, int32_t>> plan;   // (request, rows)
        int32_t rows = 0;
        for (Request* r : s->slots)
            if (r && r->decoding() && !r->finished) {
                plan.push_back({r, 1});
                ++rows;
            }
        for (Request* r : s->slots)
            if (r && !r->decoding() && rows < c.max_rows) {
                const int32_t n = std::min(r->prompt_len - r->fed, c.max_rows - rows);
                plan.push_back({r, n});
                rows += n;
            }
        // pages for every position fed; on failure give back what this call took
        std::vector<std::pair<Request*, size_t>> before;
        for (auto& pr : plan) before.push_back({pr.first, pr.first->pages.size()});
        const int64_t outstanding0 = s->outstanding;
        for (auto& pr : plan) {
            if (!s->ensure_page(pr.first, pr.first->next_pos() + pr.second - 1)) {
                for (auto& b : before) {
                    while (b.first->pages.size() > b.second) {
                        s->free_pages.push_back(b.first->pages.back());
                        b.first->pages.pop_back();
                    }
                }
                s->outstanding = outstanding0;
                return mk::host_fail(MK_ERR_CAPACITY, "no free page for request %lld", (long long)pr.first->id);
            }
        }
        // sort the runs back into slot order (decode rows and chunks interleave by slot)
        std::stable_sort(plan.begin(), plan.end(), [](const std::pair<Request*, int32_t>& a,
                                                      const std::pair<Request*, int32_t>& b) {
            return a.first->slot < b.first->slot;
        });
        s->pending.clear();
        int32_t row = 0;
        for (auto& pr : plan) {
            Request* r = pr.first;
            for (int32_t i = 0; i < pr.second; ++i, ++row) {
                const int32_t k = r->fed + i;
                seq_ids[row] = r->slot;
                positions[row] = r->cached + k;
                int32_t* bt = block_tables + (int64_t)row * c.max_pages_per_seq;
                std::fill(bt, bt + c.max_pages_per_seq, 0);
                std::copy(r->pages.begin(), r->pages.end(), bt);
                tokens[row] = r->toks[(size_t)k];
                // the row's logits choose a token: every decode row, and the
                // prompt's last row
                const bool smp = k + 1 >= r->prompt_len && r->n_gen < r->max_new;
                sample[row] = smp ? 1 : 0;
                if (request_ids) request_ids[row] = r->id;
                s->pending.push_back({r, smp});
                if (k >= r->prompt_len) ++s->st.rows;
                else ++s->st.prompt_rows;
            }
        }
        s->has_pending = row > 0;
        if (row > 0) ++s->st.steps;
        *batch = row;
        return MK_OK;
    } catch (const std::bad_alloc&) {
        return mk::host_fail(MK_ERR_CAPACITY, "host allocation failed");
    } catch (...) {
        return mk::host_fail(MK_ERR_INVALID, "unexpected exception in mk_sched_next");
    }
}

mk_status mk_sched_commit(mk_sched* s, const int32_t* next_tokens, int32_t* n_finished, int64_t* finished_ids,
                          int32_t max_finished) {
    try {
        if (!s) return mk::host_fail(MK_ERR_INVALID, "null scheduler");
        if (!s->has_pending) return mk::host_fail(MK_ERR_INVALID, "no step to commit");
        if (!next_tokens) return mk::host_fail(MK_ERR_INVALID, "null next_tokens");
        int32_t nf = 0;
        for (size_t i = 0; i < s->pending.size(); ++i) {
            Request* r = s->pending[i].r;
            ++r->fed;
            if (s->pending[i].sample) {
                r->toks.push_back(next_tokens[i]);
                ++r->n_gen;
                if (r->n_gen >= r->max_new && !r->finished) {
                    r->finished = true;
                    s->free_request_pages(r);
                    ++s->st.finished;
                    if (finished_ids && nf < max_finished) finished_ids[nf] = r->id;
                    ++nf;
                }
            }
        }
        // a request with max_new_tokens = 0 finishes once its prompt is in
        for (size_t i = 0; i < s->pending.size(); ++i) {
            Request* r = s->pending[i].r;
            if (!r->finished && r->max_new == 0 && r->fed >= r->prompt_len) {
                r->finished = true;
                s->free_request_pages(r);
                ++s->st.finished;
                if (finished_ids && nf < max_finished) finished_ids[nf] = r->id;
                ++nf;
            }
        }
        s->pending.clear();
        s->has_pending = false;
        if (n_finished) *n_finished = nf;
        return MK_OK;
    } catch (...) {
        return mk::host_fail(MK_ERR_INVALID, "unexpected exception in mk_sched_commit");
    }
}

mk_status mk_sched_get_stats(const mk_sched* s, mk_sched_stats* out) {
    if (!s || !out) return mk::host_fail(MK_ERR_INVALID, "null argument");
    *out = s->st;
    out->queued = (int32_t)s->queue.size();
    out->running = s->running();
    out->free_pages = (int32_t)s->free_pages.size();
    out->reserved_pages = (int32_t)s->outstanding;
    return MK_OK;
}

mk_status mk_sched_tokens(const mk_sched* s, int64_t request_id, int32_t* out, int32_t cap, int32_t* n) {
    if (!s || !n) return mk::host_fail(MK_ERR_INVALID, "null argument");
    auto it = s->reqs.find(request_id);
    if (it == s->reqs.end()) return mk::host_fail(MK_ERR_INVALID, "unknown request %lld", (long long)request_id);
    const std::vector<int32_t>& t = it->second->toks;
    *n = (int32_t)t.size();
    if (out) std::copy(t.begin(), t.begin() + std::min<size_t>(t.size(), (size_t)std::max(0, cap)), out);
    return MK_OK;
}

}  // extern "C"
