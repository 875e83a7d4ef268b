// mk_tiles.h -- the tile functions of one decode step and the task
// dispatcher shared by the persistent megakernel and the per-op kernels.
//
// The step is built from plain tiled matrix-vector products and paged
// attention reorganised to one calling convention ("Cohere Publishes
// One-Kernel Server for North Mini Code, Claims 1.58x vLLM Speedup", section
// "A hand-built approach to a specialized server"; "Inside the Megakernel
// Serving Engine for North Mini Code", paragraph 5): normalization,
// projections, attention, routing and the experts (first page, section "The
// delay is between operations").
#pragma once

#include "mk_tile_ctx.h"
#include "mk_tiles_mm.h"

namespace mk {

// ------------------------------------------------------------------ embed

__device__ __forceinline__ bool tile_embed(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int H8 = p.H >> 3;
    for (int b = t.a0; b < t.a1; ++b) {
        int tok = p.tokens[b];
        if (tok < 0 || tok >= p.V) {
            if (tid_() == 0) raise_error(p, kErrDevice, tok, false);
            tok = 0;
        }
        const uint16_t* row = p.embed + (int64_t)tok * p.H;
        float* xo = x_at(p, 0) + (int64_t)b * p.H;
        for (int i = tid_(); i < H8; i += NT) {
            const uint4 w = ld16(row + i * 8);
            const float v[8] = {bflo(w.x), bfhi(w.x), bflo(w.y), bfhi(w.y),
                                bflo(w.z), bfhi(w.z), bflo(w.w), bfhi(w.w)};
#pragma unroll
            for (int j = 0; j < 8; ++j) st_dev(xo + i * 8 + j, v[j]);
        }
    }
    block_signal(p, t.signal);
    return true;
}

// -------------------------------------------------------------------- QKV

// Rows of one KV group g: the G*D query rows of its heads, then its D key
// rows, then its D value rows ("virtual rows" a1..a2 of the group). The
// weights start loading after the pre counter (if any) is reached.
template <int NCH, int PF, int NB>
__device__ __forceinline__ bool tile_qkv(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, g = t.a0, v0 = t.a1, nrows = t.a2 - t.a1;
    const int wave = tid_() >> 6;
    const int nmine = nrows > wave ? (nrows - wave + NWAVES - 1) / NWAVES : 0;
    const uint16_t* W = wptr(p, l, W_QKV);
    const int H = p.H, D = p.D, GD = p.G * p.D;
    auto phys = [&](int v) -> int {
        if (v < GD) return g * GD + v;
        if (v < GD + D) return p.Hq * D + g * D + (v - GD);
        return p.Hq * D + p.Hkv * D + g * D + (v - GD - D);
    };
    if (!block_wait(p, t.pre_ctr, t.pre_target, cx.t_wait)) return false;
    bool ok = true;
    uint4 gn[NCH];
    load_gain<NCH>(gn, wptr(p, l, W_ATTN_NORM), H);
    uint32_t hx[NB][NCH][8];
    gemv_rows_warm<NCH, PF, NB>(
        hx, nmine, H >> 3, [&](int i) { return W + (int64_t)phys(v0 + wave + i * NWAVES) * H; },
        [&](int pass) {
            // pass 0 reads the layer's weight matrix as dummy activations
            if (pass) ok = block_wait(p, t.ctr, t.target, cx.t_wait);
            const float* src = pass ? x_at(p, 2 * l) : reinterpret_cast<const float*>(W);
            float h[NB][NCH][8];
            load_x<NCH, NB>(h, src, H, p.B, H, gn, p.eps, p.inv_h);
            split_x<NB, NCH>(h, hx);
            if (pass) mark(cx, 0);
        },
        [&](int i, const float(&acc)[NB], const float(&)[NB]) {
            const int row = phys(v0 + wave + i * NWAVES);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < p.B) st_dev(qkv_at(p, l) + (int64_t)b * p.QKVD + row, acc[b]);
        });
    if (!ok) return false;
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// -------------------------------------------------------------- attention

// One chunk of split-KV paged attention for row b, KV head g, chunk c:
// tokens [c*chunk, min((c+1)*chunk, pos+1)). In a multi-token step the rows
// of one sequence sit at consecutive positions p0.. and each attends
// causally over the cached prefix and the rows up to itself: tokens before
// p0 come from the pool, tokens p0..pos-1 from the qkv rows of the earlier
// rows (written in this step, so not yet in the pool), rotated and rounded
// to BF16 exactly as the tile that owns them writes them. Each wave owns 16-token blocks
// of the chunk (one cache page each) and runs a complete online softmax over
// them on the matrix cores: scores transposed, S^T = K Q^T (BF16 MFMA
// 16x16x32, the G query heads of the KV head as the N dimension), then
// O^T += V^T P^T (MFMA 16x16x16), where the probabilities P^T already sit in
// the B-operand layout the score tile was produced in, so nothing is
// exchanged between waves until the four per-wave (m, l, o) are merged in
// LDS at the end. fp32 operands (queries, probabilities) are split into three
// BF16 parts. Cache pages are loaded before the wait; the chunk holding the
// new token also applies RoPE to k, rounds k and v to BF16 and writes them
// into the pool. Writes the chunk's (m, l, o) partials.
template <int D>
__device__ __forceinline__ bool tile_attn(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    constexpr int NDB = D / 32;                // QK d-blocks (32 wide)
    constexpr int NDV = D / 16;                // PV d-blocks (16 wide)
    constexpr int NTBW = kSC / 16 / NWAVES;    // 16-token blocks per wave per pass
    const int l = t.layer, b = t.a0, g = t.a1, c = t.a2;
    const int tid = tid_(), lane = tid & 63, wave = tid >> 6;
    const int quad = lane >> 4, col = lane & 15;
    const int G = p.G;
    const int pos = p.positions[b];
    const int chunk = p.seq_chunk[b];
    const int t0 = c * chunk;
    const int t1 = min(t0 + chunk, pos + 1);
    const int p0 = p.seq_first[2 * b];          // first position written in this step (pos for decode)
    const int r0 = p.seq_first[2 * b + 1];      // the row that feeds position p0
    const int t_old = min(t1, p0);              // tokens read from the pool
    const bool has_new = (t1 == pos + 1);
    const bool multi = p0 < pos && t1 > p0;     // earlier rows of this step inside the chunk
    const int* bt = p.block_tables + (int64_t)b * p.max_pages;
    const int64_t hstride = (int64_t)16 * D;
    const int64_t layer_pages = (int64_t)l * p.n_pages;

    // LDS: new token (bf16), then the per-wave results for the merge
    uint16_t* sKn = reinterpret_cast<uint16_t*>(cx.lds);        // [D]
    uint16_t* sVn = sKn + D;                                      // [D]
    float* sM = reinterpret_cast<float*>(cx.lds + 4 * D);         // [NWAVES][16]
    float* sL = sM + NWAVES * 16;                                 // [NWAVES][16]
    float* sO = sL + NWAVES * 16;                                 // [NWAVES][16][D + 1]
    float* sF = sO + NWAVES * 16 * (D + 1);                       // [NWAVES][16] merge factors
    float* sMh = sF + NWAVES * 16;                                // [16] chunk maximum per head
    float* sLh = sMh + 16;                                        // [16] chunk sum per head

    uint4 kf[NTBW][NDB];   // A operand of S^T: token col of the block, dims 32db + 8quad..+7
    uint2 vf[NTBW][NDV];   // A operand of O^T: dim 16dv + col, tokens 4quad..+3 of the block
    auto load_kv = [&](int st0) {
#pragma unroll
        for (int i = 0; i < NTBW; ++i) {
            const int blk = st0 + (wave + NWAVES * i) * 16;     // first token of the block
            const int64_t page = (layer_pages + bt[min(blk, t_old > 0 ? t_old - 1 : 0) >> 4]) * p.Hkv + g;
            const int tk = blk + col;
            if (tk < t_old) {
                const uint16_t* kb = p.k_pool + page * hstride + (tk & 15) * D + quad * 8;
#pragma unroll
                for (int db = 0; db < NDB; ++db) kf[i][db] = ld16s(kb + db * 32);
            } else {
#pragma unroll
                for (int db = 0; db < NDB; ++db) kf[i][db] = make_uint4(0u, 0u, 0u, 0u);
            }
            const int tv = blk + 4 * quad;
            if (tv < t_old) {
                const uint16_t* vb = p.v_pool + page * hstride + (tv & 15);
#pragma unroll
                for (int dv = 0; dv < NDV; ++dv) vf[i][dv] = ld8s(vb + (int64_t)(dv * 16 + col) * 16);
            } else {
#pragma unroll
                for (int dv = 0; dv < NDV; ++dv) vf[i][dv] = make_uint2(0u, 0u);
            }
        }
    };
    // Multi-token steps: the keys and values of positions p0..pos-1 in block
    // i (first token blk) from the qkv rows that feed them -- RoPE at the
    // token's own position, then BF16 rounding, the same arithmetic as the
    // new-token path below.
    auto fix_kv_rows = [&](int i, int blk) {
        const float* qkv0 = qkv_at(p, l);
        const int tk = blk + col;
        if (tk >= p0 && tk < pos && tk < t1) {
            const int row = r0 + (tk - p0);
            const float* kp = qkv0 + (int64_t)row * p.QKVD + p.Hq * D + g * D + quad * 8;
            const float* rp = p.rope + (int64_t)row * D + 2 * (quad * 8);
#pragma unroll
            for (int db = 0; db < NDB / 2; ++db) {
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int j2 = 0; j2 < 4; ++j2) {
                    uint32_t r[2][2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int j = 2 * j2 + e;
                        const float a = ld_dev(kp + db * 32 + j), bb = ld_dev(kp + (db + NDB / 2) * 32 + j);
                        const float cs = ldg(rp + 2 * (db * 32 + j)), sn = ldg(rp + 2 * (db * 32 + j) + 1);
                        r[0][e] = f2bf(a * cs - bb * sn);
                        r[1][e] = f2bf(a * sn + bb * cs);
                    }
                    lo[j2] = r[0][0] | (r[0][1] << 16);
                    hi[j2] = r[1][0] | (r[1][1] << 16);
                }
                kf[i][db] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                kf[i][db + NDB / 2] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tv = blk + 4 * quad + j;
            if (tv >= p0 && tv < pos && tv < t1) {
                const float* vp = qkv0 + (int64_t)(r0 + (tv - p0)) * p.QKVD + (p.Hq + p.Hkv) * D + g * D + col;
                const int sh = 16 * (j & 1);
#pragma unroll
                for (int dv = 0; dv < NDV; ++dv) {
                    const uint32_t val = f2bf(ld_dev(vp + dv * 16)) << sh;
                    if (j & 2) vf[i][dv].y |= val;
                    else vf[i][dv].x |= val;
                }
            }
        }
    };
    // After the loads land, in the block that reaches past the cached tokens
    // (at most one per wave, or several in a multi-token step): zero the
    // values of slots at or past t_old (their probabilities are 0, but the
    // slots may hold any bits) and insert the new tokens' k and v.
    auto fix_kv = [&](int st0) {
#pragma unroll
        for (int i = 0; i < NTBW; ++i) {
            const int blk = st0 + (wave + NWAVES * i) * 16;
            if (blk + 16 > t_old) {
                if (has_new && blk + col == pos) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        kf[i][db] = *reinterpret_cast<const uint4*>(sKn + db * 32 + quad * 8);
                }
                const int n = t_old - (blk + 4 * quad);   // cached tokens in this lane's group of four
                const uint32_t mx = n >= 2 ? ~0u : (n == 1 ? 0xffffu : 0u);
                const uint32_t my = n >= 4 ? ~0u : (n == 3 ? 0xffffu : 0u);
#pragma unroll
                for (int dv = 0; dv < NDV; ++dv) vf[i][dv] = make_uint2(vf[i][dv].x & mx, vf[i][dv].y & my);
                if (has_new && (pos >> 2) == (blk >> 2) + quad) {
                    const int sh = 16 * (pos & 1);
#pragma unroll
                    for (int dv = 0; dv < NDV; ++dv) {
                        const uint32_t val = (uint32_t)sVn[dv * 16 + col] << sh;
                        if (pos & 2) vf[i][dv].y |= val;
                        else vf[i][dv].x |= val;
                    }
                }
                if (multi) fix_kv_rows(i, blk);
            }
        }
    };

    if (t0 > pos) {
        // a chunk the plan reserved past this sequence's tokens (plans are
        // reused while sequences grow): an empty partial, weight 0 in the merge
        float* part0 = part_at(p, l) + ((int64_t)b * p.Hq + g * G) * p.max_chunks * D;
        float* ml0 = ml_at(p, l) + ((int64_t)b * p.Hq + g * G) * ml_row(p);
        for (int i = tid; i < G * D; i += NT) {
            const int h = i / D, d = i - h * D;
            st_dev(part0 + ((int64_t)h * p.max_chunks + c) * D + d, 0.f);
        }
        if (tid < G) {
            st_dev(ml0 + (int64_t)tid * ml_row(p) + 2 * c, -INFINITY);
            st_dev(ml0 + (int64_t)tid * ml_row(p) + 2 * c + 1, 0.f);
        }
        block_signal(p, t.signal);
        return true;
    }
    if (!block_wait(p, t.pre_ctr, t.pre_target, cx.t_wait)) return false;
    load_kv(t0);
    // queries: lane (quad, col) holds head col's dims 32db + 8quad..+7 (zero
    // for col >= G); the rotary factors of those dims are a host input, so
    // both are fetched before the wait where possible
    float rc[NDB / 2][8], rs[NDB / 2][8];
#pragma unroll
    for (int db = 0; db < NDB / 2; ++db) {
        const float* rp = p.rope + (int64_t)b * D + 2 * (db * 32 + quad * 8);
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const float4 v = ldf4(rp + 4 * k4);
            rc[db][2 * k4] = v.x; rs[db][2 * k4] = v.y; rc[db][2 * k4 + 1] = v.z; rs[db][2 * k4 + 1] = v.w;
        }
    }
    if (!block_wait(p, t.ctr, t.target, cx.t_wait)) return false;

    const float* qkv = qkv_at(p, l) + (int64_t)b * p.QKVD;
    float q[NDB][8];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        if (col < G) {
            const float* qp = qkv + (int64_t)(g * G + col) * D + db * 32 + quad * 8;
            const float4 u = ldf4(qp), w = ldf4(qp + 4);
            q[db][0] = u.x; q[db][1] = u.y; q[db][2] = u.z; q[db][3] = u.w;
            q[db][4] = w.x; q[db][5] = w.y; q[db][6] = w.z; q[db][7] = w.w;
        } else {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) q[db][jj] = 0.f;
        }
    }
    // New token: RoPE on k, BF16 rounding of k and v, append to the pool.
    if (has_new) {
        for (int i = tid; i < D / 2; i += NT) {
            const float cs = ldg(p.rope + (int64_t)b * D + 2 * i), sn = ldg(p.rope + (int64_t)b * D + 2 * i + 1);
            const float a = ld_dev(qkv + p.Hq * D + g * D + i), bb = ld_dev(qkv + p.Hq * D + g * D + i + D / 2);
            sKn[i] = (uint16_t)f2bf(a * cs - bb * sn);
            sKn[i + D / 2] = (uint16_t)f2bf(a * sn + bb * cs);
        }
        for (int i = tid; i < D; i += NT) sVn[i] = (uint16_t)f2bf(ld_dev(qkv + (p.Hq + p.Hkv) * D + g * D + i));
        __syncthreads();
        const int64_t page = bt[pos >> 4];
        const int slot = pos & 15;
        uint16_t* kd = p.k_pool + ((layer_pages + page) * p.Hkv + g) * hstride + slot * D;
        uint16_t* vd = p.v_pool + ((layer_pages + page) * p.Hkv + g) * hstride + slot;
        for (int i = tid; i < D; i += NT) {
            kd[i] = sKn[i];
            vd[(int64_t)i * 16] = sVn[i];
        }
    }
    // RoPE on the queries (pairs d, d + D/2 sit in blocks db, db + NDB/2 of
    // this lane), then the three-way BF16 split: B operand of S^T
    uint4 qf[3][NDB];
#pragma unroll
    for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float cs = rc[db][jj], sn = rs[db][jj];
            const float a = q[db][jj], bb = q[db + NDB / 2][jj];
            q[db][jj] = a * cs - bb * sn;
            q[db + NDB / 2][jj] = a * sn + bb * cs;
        }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        uint32_t hw[4], mw[4], lw[4];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
            uint32_t h0, m0, l0, h1, m1, l1;
            split3(q[db][2 * k2], h0, m0, l0);
            split3(q[db][2 * k2 + 1], h1, m1, l1);
            hw[k2] = h0 | (h1 << 16);
            mw[k2] = m0 | (m1 << 16);
            lw[k2] = l0 | (l1 << 16);
        }
        qf[0][db] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        qf[1][db] = make_uint4(mw[0], mw[1], mw[2], mw[3]);
        qf[2][db] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    mark(cx, 0);

    // per-wave online softmax state for head col (the same in the four lane groups)
    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t oacc[NDV];
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv) oacc[dv] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float scale = p.attn_scale;

    for (int st0 = t0; st0 < t1; st0 += kSC) {
        if (st0 != t0) load_kv(st0);
        fix_kv(st0);
        // S^T[token][head] for this wave's blocks: lane (quad, col) holds
        // tokens 4quad..+3 of each block for head col
        float sc[NTBW][4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < NTBW; ++i) {
            f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                s4 = mfma16x16x32(kf[i][db], qf[0][db], s4);
                s4 = mfma16x16x32(kf[i][db], qf[1][db], s4);
                s4 = mfma16x16x32(kf[i][db], qf[2][db], s4);
            }
            const int blk = st0 + (wave + NWAVES * i) * 16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[i][r] = (blk + 4 * quad + r < t1) ? s4[r] * scale : -INFINITY;
                mx = fmaxf(mx, sc[i][r]);
            }
        }
        // maximum over the wave's tokens: across the four lane groups
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : expf(m_run - m_new);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < NTBW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[i][r] = m_new == -INFINITY ? 0.f : expf(sc[i][r] - m_new);
                ps += sc[i][r];
            }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[dv][r] *= alpha;
        // O^T[d][head] += V^T[d][token] P^T[token][head]; P^T is this lane's
        // four probabilities, split in three BF16 parts
#pragma unroll
        for (int i = 0; i < NTBW; ++i) {
            uint32_t h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
            split3(sc[i][0], h0, m0, l0);
            split3(sc[i][1], h1, m1, l1);
            split3(sc[i][2], h2, m2, l2);
            split3(sc[i][3], h3, m3, l3);
            const uint2 ph = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
            const uint2 pm = make_uint2(m0 | (m1 << 16), m2 | (m3 << 16));
            const uint2 pl = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
#pragma unroll
            for (int dv = 0; dv < NDV; ++dv) {
                oacc[dv] = mfma16x16x16(vf[i][dv], ph, oacc[dv]);
                oacc[dv] = mfma16x16x16(vf[i][dv], pm, oacc[dv]);
                oacc[dv] = mfma16x16x16(vf[i][dv], pl, oacc[dv]);
            }
        }
    }
    mark(cx, 1);

    // merge the four waves: lane (quad, col) holds O^T[16dv + 4quad + r][col]
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
        for (int r = 0; r < 4; ++r) sO[(wave * 16 + col) * (D + 1) + dv * 16 + 4 * quad + r] = oacc[dv][r];
    if (quad == 0) {
        sM[wave * 16 + col] = m_run;
        sL[wave * 16 + col] = l_run;
    }
    __syncthreads();
    mark(cx, 2);
    // per head: the chunk maximum M, each wave's factor exp(m_w - M) and the sum
    if (tid < G) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) M = fmaxf(M, sM[w * 16 + tid]);
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            const float mw = sM[w * 16 + tid];
            const float e = mw == -INFINITY ? 0.f : expf(mw - M);
            sF[w * 16 + tid] = e;
            L += e * sL[w * 16 + tid];
        }
        sMh[tid] = M;
        sLh[tid] = L;
    }
    __syncthreads();
    float* part = part_at(p, l) + ((int64_t)b * p.Hq + g * G) * p.max_chunks * D;
    float* ml = ml_at(p, l) + ((int64_t)b * p.Hq + g * G) * ml_row(p);
    // each thread: four consecutive dimensions of one head, all LDS reads
    // issued before the sums (the same per-output order as one at a time)
    for (int i4 = tid; i4 < G * (D / 4); i4 += NT) {
        const int h = i4 / (D / 4), d0 = (i4 - h * (D / 4)) * 4;
        float f[NWAVES], ov[NWAVES][4];
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            f[w] = sF[w * 16 + h];
#pragma unroll
            for (int j = 0; j < 4; ++j) ov[w][j] = sO[(w * 16 + h) * (D + 1) + d0 + j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float o = 0.f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) o += f[w] * ov[w][j];
            st_dev(part + ((int64_t)h * p.max_chunks + c) * D + d0 + j, o);
        }
        if (d0 == 0) {
            st_dev(ml + (int64_t)h * ml_row(p) + 2 * c, sMh[h]);
            st_dev(ml + (int64_t)h * ml_row(p) + 2 * c + 1, sLh[h]);
        }
    }
    mark(cx, 3);
    block_signal(p, t.signal);
    return true;
}

// Merge the chunk partials of one query head a1 of sequence a0:
// o = sum_c exp(m_c - M) o_c / sum_c exp(m_c - M) l_c with M = max_c m_c
// (the softmax over all cached tokens, split by chunks). Each thread sums a
// fixed set of chunks for four dimensions, then the sets are added in a fixed
// order, so the result does not depend on timing. The thread's first kPre
// chunk partials are requested together with the (m, l) pairs, so the merge
// costs one memory round trip.
template <int D>
__device__ __forceinline__ bool tile_combine(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, b = t.a0, h = t.a1, nch = t.a2;
    const int tid = tid_(), lane = tid & 63, wave = tid >> 6;
    constexpr int NQ = D / 4;          // float4 columns
    constexpr int NPH = NT / NQ;       // chunk phases
    constexpr int kPre = 12;           // chunks per thread fetched up front
    float* sred = reinterpret_cast<float*>(cx.lds);           // [NWAVES][2] reductions
    float* coef = sred + 16;                                  // [nch]
    float* sacc = coef + ((p.max_chunks + 3) & ~3);           // [NPH][D]
    if (!block_wait(p, t.ctr, t.target, cx.t_wait)) return false;
    const int64_t row = (int64_t)b * p.Hq + h;
    const float* ml = ml_at(p, l) + row * ml_row(p);
    const float* po = part_at(p, l) + row * p.max_chunks * D;
    const int q = tid % NQ, ph = tid / NQ;
    float4 pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int c = ph + k * NPH;
        pre[k] = c < nch ? ldf4(po + (int64_t)c * D + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // (m, l) of this thread's chunks
    float mv[2], lv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int c = tid + k * NT;
        mv[k] = c < nch ? ld_dev(ml + 2 * c) : -INFINITY;
        lv[k] = c < nch ? ld_dev(ml + 2 * c + 1) : 0.f;
    }
    // M = max_c m_c
    float mx = fmaxf(mv[0], mv[1]);
    for (int c = tid + 2 * NT; c < nch; c += NT) mx = fmaxf(mx, ld_dev(ml + 2 * c));
    mx = wave_max(mx);
    if (lane == 0) sred[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]));
    // L = sum_c exp(m_c - M) l_c
    float ls = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int c = tid + k * NT;
        if (c < nch) {
            const float e = expf(mv[k] - mx);
            coef[c] = e;
            ls += e * lv[k];
        }
    }
    for (int c = tid + 2 * NT; c < nch; c += NT) {
        const float e = expf(ld_dev(ml + 2 * c) - mx);
        coef[c] = e;
        ls += e * ld_dev(ml + 2 * c + 1);
    }
    ls = wave_sum(ls);
    if (lane == 0) sred[NWAVES + wave] = ls;
    __syncthreads();
    const float inv = 1.0f / (((sred[NWAVES] + sred[NWAVES + 1]) + sred[NWAVES + 2]) + sred[NWAVES + 3]);
    mark(cx, 0);
    // o[d] = sum_c coef_c o_c[d] * inv, chunks ph, ph + NPH, ... in order
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int c = ph + k * NPH;
        if (c < nch) {
            const float w = coef[c];
            acc.x = fmaf(w, pre[k].x, acc.x); acc.y = fmaf(w, pre[k].y, acc.y);
            acc.z = fmaf(w, pre[k].z, acc.z); acc.w = fmaf(w, pre[k].w, acc.w);
        }
    }
    for (int c = ph + kPre * NPH; c < nch; c += NPH) {
        const float4 v = ldf4(po + (int64_t)c * D + 4 * q);
        const float w = coef[c];
        acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y); acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
    }
    reinterpret_cast<float4*>(sacc)[ph * NQ + q] = acc;
    __syncthreads();
    mark(cx, 1);
    float* out = attout_at(p, l) + row * D;
    if (p.mm) {
        // matrix-core schedule: the output projection takes it split (see st_split8)
        if (tid < D / 8) {
            float o8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float v[NPH];
#pragma unroll
                for (int k = 0; k < NPH; ++k) v[k] = sacc[k * D + 8 * tid + j];
                float s = 0.f;
#pragma unroll
                for (int k = 0; k < NPH; ++k) s += v[k];
                o8[j] = s * inv;
            }
            st_split8(out + 8 * tid, o8);
        }
    } else {
        for (int d = tid; d < D; d += NT) {
            float v[NPH];
#pragma unroll
            for (int k = 0; k < NPH; ++k) v[k] = sacc[k * D + d];
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < NPH; ++k) s += v[k];
            st_dev(out + d, s * inv);
        }
    }
    block_signal(p, t.signal);
    return true;
}

// ------------------------------------------------------- output projection

template <int NCH, int PF, int NB>
__device__ __forceinline__ bool tile_oproj(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, r0 = t.a0, nrows = t.a1 - t.a0;
    const int wave = tid_() >> 6, lane = tid_() & 63;
    const int nmine = nrows > wave ? (nrows - wave + NWAVES - 1) / NWAVES : 0;
    const int K = p.Hq * p.D;
    const uint16_t* W = wptr(p, l, W_O);
    float* xmid = x_at(p, 2 * l + 1);
    // residual: lane i holds the layer input at this wave's i-th row; the
    // layer input is complete long before the attention output (pre counter),
    // so it is loaded before the main wait
    float xres[NB];
    if (!block_wait(p, t.pre_ctr, t.pre_target, cx.t_wait)) return false;
    {
        const float* xin = x_at(p, 2 * l);
        const int row = r0 + wave + (lane < nmine ? lane : 0) * NWAVES;
#pragma unroll
        for (int b = 0; b < NB; ++b) xres[b] = (b < p.B && lane < nmine) ? ld_dev(xin + (int64_t)b * p.H + row) : 0.f;
    }
    bool ok = true;
    gemv_stream<NCH, PF, NB>(
        nmine, K >> 3, [&](int i) { return W + (int64_t)(r0 + wave + i * NWAVES) * K; },
        [&](float(&h)[NB][NCH][8]) {
            ok = block_wait(p, t.ctr, t.target, cx.t_wait);
            load_x<NCH, NB>(h, attout_at(p, l), K, p.B, K, nullptr, 0.f, 0.f);
        },
        [&](int i, const float(&acc)[NB], const float(&)[NB]) {
            // lane i holds row i's residual
            const int row = r0 + wave + i * NWAVES;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < p.B) st_dev(xmid + (int64_t)b * p.H + row, xres[b] + acc[b]);
        });
    if (!ok) return false;
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// ------------------------------------------------------------------ router

template <int NCH, int PF, int NB>
__device__ __forceinline__ bool tile_router(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, r0 = t.a0, nrows = t.a1 - t.a0;
    const int wave = tid_() >> 6;
    const int nmine = nrows > wave ? (nrows - wave + NWAVES - 1) / NWAVES : 0;
    const int H = p.H;
    const uint16_t* W = wptr(p, l, W_ROUTER);
    const float* bias = reinterpret_cast<const float*>(p.wtab[l * W_NKINDS + W_RBIAS]);
    bool ok = true;
    gemv_stream<NCH, PF, NB>(
        nmine, H >> 3, [&](int i) { return W + (int64_t)(r0 + wave + i * NWAVES) * H; },
        [&](float(&h)[NB][NCH][8]) {
            uint4 gn[NCH];
            load_gain<NCH>(gn, wptr(p, l, W_FFN_NORM), H);
            ok = block_wait(p, t.ctr, t.target, cx.t_wait);
            load_x<NCH, NB>(h, x_at(p, 2 * l + 1), H, p.B, H, gn, p.eps, p.inv_h);
        },
        [&](int i, const float(&acc)[NB], const float(&)[NB]) {
            {
                const int row = r0 + wave + i * NWAVES;
                const float bv = bias != nullptr ? ldg(bias + row) : 0.f;
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < p.B) st_dev(rlogits_at(p, l) + (int64_t)b * p.E + row, bias != nullptr ? acc[b] + bv : acc[b]);
            }
        });
    if (!ok) return false;
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// ---------------------------------------------------------- expert gate/up

// Slot a0 (the a0-th distinct selected expert, ascending id), rows a1..a2 of
// its gate and up matrices; a = SiLU(W_gate h2) * (W_up h2) for every token
// routed to it. The tile waits for the router logits only (they imply the
// post-attention residual, which the router tiles read): an earlier wait on
// the residual's counter would have ~250 tiles polling it while the output
// projection stores it. Then the residual's loads are issued, the routing is
// computed (its logits loads queue behind them, so the two round trips
// overlap) and the residual normalized; only then are the expert's rows known
// and streamed. The plan gives the task no pre counter: the output
// projection is implied by the main one. Task a3 != 0: also store the
// routing of this layer.
template <int NCH, int PF, int NB, int NE>
__device__ __forceinline__ bool tile_gateup(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, slot = t.a0, r0 = t.a1, nrows = t.a2 - t.a1;
    const int wave = tid_() >> 6;
    const int H = p.H;
    RouteLds* rt = route_lds(cx.lds, cx.general);
    uint32_t hx[NB][NCH][8];
    {
        uint4 gn[NCH];
        load_gain<NCH>(gn, wptr(p, l, W_FFN_NORM), H);
        if (!block_wait(p, t.ctr, t.target, cx.t_wait)) return false;
        float h[NB][NCH][8];
        load_x_raw<NCH, NB>(h, x_at(p, 2 * l + 1), H, p.B, H);
        routing_for<NE>(p, rlogits_at(p, l), rt);
        norm_x<NCH, NB>(h, H, gn, p.eps, p.inv_h);
        split_x<NB, NCH>(h, hx);
    }
    mark(cx, 0);
    if (t.a3 != 0) {
        for (int i = tid_(); i < p.B * p.K; i += NT) {
            const int b = i / p.K, j = i - b * p.K;
            p.route_ids[((int64_t)l * p.max_batch + b) * p.K + j] = rt->ids[b][j];
            p.route_w[((int64_t)l * p.max_batch + b) * p.K + j] = rt->w[b][j];
        }
    }
    if (slot >= rt->nslots) {
        block_signal(p, t.signal);
        return true;
    }
    const int e = rt->slot_e[slot];
    const int mask = rt->slot_mask[slot];
    const uint16_t* Wg = wptr(p, l, W_GATE) + (int64_t)e * p.I * H;
    const uint16_t* Wu = wptr(p, l, W_UP) + (int64_t)e * p.I * H;
    const int npair = nrows > wave ? (nrows - wave + NWAVES - 1) / NWAVES : 0;
    gemv_rows<NCH, PF, NB>(
        hx, 2 * npair, H >> 3,
        [&](int i) { return ((i & 1) ? Wu : Wg) + (int64_t)(r0 + wave + (i >> 1) * NWAVES) * H; },
        [&]() { mark(cx, 1); },
        [&](int i, const float(&acc)[NB], const float(&gate)[NB]) {
            // row-vector i odd: up row, its gate row's products from lane i - 1
            if (i & 1) {
                const int row = r0 + wave + (i >> 1) * NWAVES;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < p.B && ((mask >> b) & 1)) {
                        const float gv = gate[b];
                        const float a = (gv / (1.0f + expf(-gv))) * acc[b];
                        st_dev(act_at(p, l) + ((int64_t)b * p.K + rt->slot_rank[slot][b]) * p.I + row, a);
                    }
                }
            }
        });
    mark(cx, 2);
    block_signal(p, t.signal);
    return true;
}

// ------------------------------------------------------------ expert down

// Rows a0..a1 of the hidden dimension, for every selected expert: y = W_down a,
// then x_out = x_mid + sum_j w_j y_j in top-k rank order. The routing (and so
// the expert rows) is known once the router logits are (pre counter): the
// tile computes it and starts its weights streaming into registers while the
// gate/up tiles are still running, then waits for them (main counter) and
// reads their activations once, into LDS, split into BF16 parts.
//
// The products run on the matrix cores (BF16 MFMA 16x16x32, fp32
// accumulate). Wave w takes slots w, w+4, ...; its row-vectors are listed
// slot-major with a2 (a power of two, >= the tile's rows) entries per slot,
// and each group of 16 is one A operand: lane l holds row-vector l%16 at
// k-chunk l/16 of every 32-wide k-step. The B operand's 16 columns are, per
// slot of the group, per token, the hi and lo parts of that token's
// activations for the slot's expert (zero where the token did not choose
// it), so column pair (2m, 2m+1) of an A-row belonging to that slot is its
// dot product in two parts.
template <int KS, int NB, int NE>
__device__ __forceinline__ bool tile_down(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, h0 = t.a0, nrows = t.a1 - t.a0, rd = t.a2;
    const int tid = tid_(), wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, g4 = lane >> 4;
    RouteLds* rt = route_lds(cx.lds, cx.general);
    if (!block_wait(p, t.pre_ctr, t.pre_target, cx.t_wait)) return false;
    routing_for<NE>(p, rlogits_at(p, l), rt);
    mark(cx, 0);
    const int I = p.I, K = p.K, B = p.B;
    const int K8 = I >> 3, nks = I >> 5;
    const int nslots = rt->nslots;
    // residual slice: ready since the output projection
    const float* xmid = x_at(p, 2 * l + 1);
    const float xres = tid < B * nrows ? ldg(xmid + (int64_t)(tid / nrows) * p.H + h0 + tid % nrows) : 0.f;
    const int myslots = nslots > wave ? (nslots - wave + NWAVES - 1) / NWAVES : 0;
    const int ngrp = (myslots * rd + 15) >> 4;
    const uint16_t* Wd = wptr(p, l, W_DOWN);
    // [B][K][I/8] chunks of the gate/up outputs, each as BF16 parts (hi pairs, lo pairs)
    uint4* sAct = reinterpret_cast<uint4*>(cx.lds);
    float* sY = reinterpret_cast<float*>(cx.lds + cx.general) - kMaxBatch * kMaxTopK * kMaxDownRows;  // [B*K][nrows]
    const float* act = act_at(p, l);
    // the A-row of this lane in group grp (padding entries re-read a valid row)
    uint4 wb[KS];
    auto load_grp = [&](int grp) {
        const int v = 16 * grp + col;
        const int jl = v / rd, r = v - jl * rd;
        const bool live = jl < myslots && r < nrows;
        const int e = rt->slot_e[live ? wave + NWAVES * jl : 0];
        const uint16_t* a = Wd + ((int64_t)e * p.H + h0 + (live ? r : 0)) * I + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) wb[ks] = ld16s(a + 32 * (ks < nks ? ks : nks - 1));
    };
    if (ngrp > 0) load_grp(0);
    const bool ok = block_wait(p, t.ctr, t.target, cx.t_wait);
    if (ok) {
        // all loads of a batch in flight before the LDS writes; each chunk
        // of eight is split into BF16 parts once, here
        const int n8 = (B * K * I) >> 3;
        for (int i0 = 0; i0 < n8; i0 += 3 * NT) {
            float4 v[3][2];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int i = i0 + k * NT + tid;
                const float* a = act + 8 * (i < n8 ? i : 0);
                v[k][0] = ldf4(a);
                v[k][1] = ldf4(a + 4);
            }
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int i = i0 + k * NT + tid;
                if (i < n8) {
                    const float f[8] = {v[k][0].x, v[k][0].y, v[k][0].z, v[k][0].w,
                                        v[k][1].x, v[k][1].y, v[k][1].z, v[k][1].w};
                    uint32_t x[8];
                    split8(f, x);
                    sAct[2 * i] = make_uint4(x[0], x[1], x[2], x[3]);
                    sAct[2 * i + 1] = make_uint4(x[4], x[5], x[6], x[7]);
                }
            }
        }
    }
    __syncthreads();
    mark(cx, 1);
    if (ok) {
        for (int grp = 0; grp < ngrp; ++grp) {
            if (grp > 0) load_grp(grp);
            // this lane's B column: slot jc of the wave, token bc, part (hi / lo)
            const int first = (16 * grp) / rd;
            const int jc = first + col / (2 * NB), bc = (col >> 1) % NB, part = col & 1;
            const int rank = (jc < myslots && bc < B) ? rt->slot_rank[wave + NWAVES * jc][bc] : -1;
            const uint4* bsrc = sAct + 2 * ((bc * K + (rank >= 0 ? rank : 0)) * K8 + g4) + part;
            // B operands eight k-steps at a time (their LDS reads in flight
            // together), two accumulators (independent matrix-core chains)
            f32x4_t acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            auto ksteps = [&](auto full) {
                constexpr bool FULL = decltype(full)::value;
#pragma unroll
                for (int k0 = 0; k0 < KS; k0 += 8) {
                    uint4 bv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        bv[j] = ((FULL || k0 + j < nks) && rank >= 0) ? bsrc[8 * (k0 + j)]
                                                                      : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (k0 + j < KS && (FULL || k0 + j < nks))
                            acc2[j & 1] = mfma16x16x32(wb[k0 + j], bv[j], acc2[j & 1]);
                }
            };
            // an expert width of exactly the compiled k-steps (the shape the
            // kernel is built for) runs without a bound check per step
            if (nks == KS) ksteps(std::true_type{});
            else ksteps(std::false_type{});
            f32x4_t acc = acc2[0] + acc2[1];
            // hi + lo (adjacent columns); lane (col, g4) holds A-rows 4 g4 + q
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] += dpp_mov<0xB1>(acc[q]);
            if ((col & 1) == 0 && rank >= 0) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int v = 16 * grp + 4 * g4 + q;
                    const int jl = v / rd, r = v - jl * rd;
                    if (jl == jc && r < nrows) sY[(bc * K + rank) * nrows + r] = acc[q];
                }
            }
        }
    }
    __syncthreads();
    if (!ok) return false;  // block-uniform (block_wait)
    mark(cx, 2);
    float* xout = x_at(p, 2 * l + 2);
    if (tid < B * nrows) {
        const int b = tid / nrows, r = tid - b * nrows;
        float wv[kMaxTopK], yv[kMaxTopK];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            wv[j] = j < K ? rt->w[b][j] : 0.f;
            yv[j] = j < K ? sY[(b * K + j) * nrows + r] : 0.f;
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
            if (j < K) acc += wv[j] * yv[j];
        st_dev(xout + (int64_t)b * p.H + h0 + r, xres + acc);
    }
    block_signal(p, t.signal);
    return true;
}

// ---------------------------------------------------------------- LM head

template <int NCH, int PF, int NB>
__device__ __forceinline__ bool tile_lmhead(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int r0 = t.a0, nrows = t.a1 - t.a0;
    const int wave = tid_() >> 6;
    const int nmine = nrows > wave ? (nrows - wave + NWAVES - 1) / NWAVES : 0;
    const int H = p.H;
    bool ok = true;
    gemv_stream<NCH, PF, NB>(
        nmine, H >> 3, [&](int i) { return p.lm_head + (int64_t)(r0 + wave + i * NWAVES) * H; },
        [&](float(&h)[NB][NCH][8]) {
            uint4 gn[NCH];
            load_gain<NCH>(gn, p.final_norm, H);
            ok = block_wait(p, t.ctr, t.target, cx.t_wait);
            load_x<NCH, NB>(h, x_at(p, 2 * p.L), H, p.B, H, gn, p.eps, p.inv_h);
        },
        [&](int i, const float(&acc)[NB], const float(&)[NB]) {
            const int row = r0 + wave + i * NWAVES;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < p.B) p.logits[(int64_t)b * p.V + row] = acc[b];
        });
    if (!ok) return false;
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// -------------------------------------------------------------- dispatcher

// Compile-time shape of a kernel build: 16-byte chunks per lane per row
// (ceil(K / 512)) for the three reduction lengths in the model -- hidden
// size H, attention width Hq*D and expert width I -- the head size,
// ceil(I / 256) (the down tile runs at most 8 times that many 32-wide
// k-steps) and the router logits per lane (ceil(E / 64)). Each
// supported model gets its own kernels, so each tile is compiled only for
// the reduction lengths it actually sees and register allocation is sized
// per tile, not for every possible shape.
template <int NCH_H_, int NCH_O_, int NCH_I_, int D_, int NCHP_I_, int NE_>
struct Shape {
    static constexpr int NCH_H = NCH_H_, NCH_O = NCH_O_, NCH_I = NCH_I_, D = D_, NCHP_I = NCHP_I_, NE = NE_;
};

// Rows in flight per wave for a given chunk count and batch.
template <int NCH, int NB>
struct Pf {
    static constexpr int v = NB == 1 ? (NCH <= 2 ? 8 : (NCH <= 4 ? 4 : 2)) : (NCH <= 1 ? 8 : (NCH <= 2 ? 4 : (NCH <= 4 ? 2 : 1)));
};

// A task record whose operation this schedule does not run (a corrupted or
// foreign task table): report it and abort the step, so every workgroup
// leaves its waits at once instead of timing out on counters that will
// never be bumped.
__device__ __forceinline__ bool bad_task(const Task& t, TileCtx& cx) {
    if (tid_() == 0) raise_error(cx.p, kErrBadTask, t.op, true);
    return false;
}

// NB = 1, 2: the one- and two-token tiles; NB = 0: the matrix-core tiles of
// batches of 3 or more (attention, its merge and the embedding are shared).
template <class S, int NB>
__device__ __forceinline__ bool dispatch_tile(const Task& t, TileCtx& cx) {
    if constexpr (NB == 0 || NB == kNbMmWide) {
        constexpr int RBK = NB == kNbMmWide ? kMmMaxRowBlocks : 1;
        switch (t.op) {
            case OP_EMBED: return tile_embed(t, cx);
            case OP_QKV: return tile_qkv_mm(t, cx);
            case OP_ATTN: return tile_attn<S::D>(t, cx);
            case OP_COMBINE: return tile_combine<S::D>(t, cx);
            case OP_OPROJ: return tile_oproj_mm(t, cx);
            case OP_ROUTER: return tile_router_mm(t, cx);
            case OP_ROUTE: return tile_route<4 * S::NE>(t, cx);
            case OP_GATEUP: return tile_gateup_mm<RBK>(t, cx);
            case OP_DOWN: return tile_down_mm<RBK>(t, cx);
            case OP_MOESUM: return tile_moesum(t, cx);
            case OP_FNORM: return tile_fnorm(t, cx);
            case OP_LMHEAD: return tile_lmhead_mm(t, cx);
            default: return bad_task(t, cx);
        }
    } else {
        switch (t.op) {
            case OP_EMBED: return tile_embed(t, cx);
            case OP_QKV: return tile_qkv<S::NCH_H, (NB == 1 && S::NCH_H <= 4 ? 6 : Pf<S::NCH_H, NB>::v), NB>(t, cx);
            case OP_ATTN: return tile_attn<S::D>(t, cx);
            case OP_COMBINE: return tile_combine<S::D>(t, cx);
            case OP_OPROJ: return tile_oproj<S::NCH_O, Pf<S::NCH_O, NB>::v, NB>(t, cx);
            case OP_ROUTER: return tile_router<S::NCH_H, Pf<S::NCH_H, NB>::v, NB>(t, cx);
            case OP_GATEUP: return tile_gateup<S::NCH_H, (NB == 1 && S::NCH_H <= 4 ? 6 : Pf<S::NCH_H, NB>::v), NB, S::NE>(t, cx);
            case OP_DOWN: return tile_down<8 * S::NCHP_I, NB, S::NE>(t, cx);
            case OP_LMHEAD: return tile_lmhead<S::NCH_H, Pf<S::NCH_H, NB>::v, NB>(t, cx);
            default: return bad_task(t, cx);
        }
    }
}

// Run one task; with tracing on, thread 0 records {task | wg << 32, start,
// end of the compute wait, four phase stamps, end}.
template <class S, int NB>
__device__ __forceinline__ bool run_task(const Task& t, const Params& p, char* lds, int general,
                                         int idx) {
    uint64_t t_start = 0, t_wait = 0;
    uint64_t marks[4] = {0, 0, 0, 0};
    if (p.trace_on && tid_() == 0) t_start = t_wait = wall_clock64();
    TileCtx cx{p, lds, general, &t_wait, marks};
    const bool ok = dispatch_tile<S, NB>(t, cx);
    if (p.trace_on && tid_() == 0) {
        uint64_t* rec = p.trace + (int64_t)idx * 8;
        rec[0] = (uint64_t)(uint32_t)idx | ((uint64_t)blockIdx.x << 32);
        rec[1] = t_start;
        rec[2] = t_wait;
        rec[3] = marks[0];
        rec[4] = marks[1];
        rec[5] = marks[2];
        rec[6] = marks[3];
        rec[7] = wall_clock64();
    }
    return ok;
}

}  // namespace mk
