// mk_tiles_mm.h -- the tiles of a decode step for batches of 3 to 64 tokens.
//
// At these batches every weight product runs on the matrix cores (BF16 MFMA
// 16x16x32, fp32 accumulate), still bounded by the weight stream: weights are
// the A operand (16 rows per block), the batch's activations the B operand
// (16 tokens per column block). As in the one- and two-token tiles, fp32
// activations enter as two BF16 parts (hi = bf16(x), lo = bf16(x - hi)), each
// its own MFMA into the same accumulator, so the products keep ~2^-17
// relative activation precision and the routing decisions the oracle's fp32
// products make. The pages build the step from ordinary tiled matrix
// multiplications ("Cohere Publishes One-Kernel Server for North Mini Code,
// Claims 1.58x vLLM Speedup", section "A hand-built approach to a specialized
// server"), and continuous batching is part of the serving model they
// describe (same page, opening section).
//
// Routing gets a level of its own here: one tile computes every token's top-k
// and publishes, per selected expert ("slot", ascending expert id), the tokens
// routed to it. Expert tiles then stream only the selected experts' rows. The
// down tiles write each expert's output per (token, rank); a last level sums
// them per token in top-k rank order onto the residual, so the result does
// not depend on how tiles were placed.
#pragma once

#include "mk_tile_ctx.h"

namespace mk {

// ------------------------------------------------------------ exchange slices

__device__ __forceinline__ int32_t* rtab_at(const Params& p, int l) {
    return p.rtab + (int64_t)l * rtab_words(p.E, p.K, p.max_batch);
}
// routing weights of a layer inside its routing table: [max_batch][K] floats
__device__ __forceinline__ float* rtab_w(const Params& p, int32_t* rt) {
    return reinterpret_cast<float*>(rt + 64 + 2 * p.E + (int64_t)p.E * p.max_batch);
}
__device__ __forceinline__ float* ybuf_at(const Params& p, int l) {
    return p.ybuf + (int64_t)l * pad64((int64_t)p.max_batch * p.K * p.H);
}

__device__ __forceinline__ void st_dev_i(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float* h2s_at(const Params& p, int l) {
    return p.h2s + (int64_t)l * pad64((int64_t)p.max_batch * p.H);
}

// Split activations. Vectors that feed a weight product and need no
// normalisation there (the attention output, the FFN input after its
// RMSNorm, the SwiGLU output) are stored by their producers already split:
// each group of 8 elements becomes its BF16 hi pairs then its lo pairs (the
// two halves of split8), in the 32 bytes the 8 fp32 values would take.
__device__ __forceinline__ void st_dev_u4(uint4* q, uint4 v) {
    uint64_t* d = reinterpret_cast<uint64_t*>(q);
    __hip_atomic_store(d, (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(d + 1, (uint64_t)v.z | ((uint64_t)v.w << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Store 8 values (element offset a multiple of 8) in split form.
__device__ __forceinline__ void st_split8(float* dst, const float (&v)[8]) {
    uint32_t h[8];
    split8(v, h);
    uint4* q = reinterpret_cast<uint4*>(dst);
    st_dev_u4(q, make_uint4(h[0], h[1], h[2], h[3]));
    st_dev_u4(q + 1, make_uint4(h[4], h[5], h[6], h[7]));
}

// ------------------------------------------------------------- MFMA engine

// Column blocks of 16 tokens: compile-time 1, 2 or 4, chosen per call.
template <int N>
struct Ncb {
    static constexpr int v = N;
};
template <class F>
__device__ __forceinline__ void with_ncb(int ncb, F&& f) {
    if (ncb <= 1) f(Ncb<1>());
    else if (ncb <= 2) f(Ncb<2>());
    else f(Ncb<4>());
}
__device__ __forceinline__ int ncb_cols(int ncb) { return 16 * (ncb <= 1 ? 1 : (ncb <= 2 ? 2 : 4)); }

// k-steps of 32 per load batch (two batches in flight).
template <int NCB>
struct MmPf {
    static constexpr int v = NCB == 1 ? 4 : 2;
};

// One wave's product over `nsteps` k-steps of 32:
//   acc[cb] += A(16 rows) * (g o X)(16 columns of block cb), ss[cb] += X^2,
// X entering as two BF16 parts. Lane layout of the 16x16x32 MFMA: lane l
// holds A[l%16][8(l/16) .. +7], B[8(l/16) .. +7][l%16], D[4(l/16) .. +3][l%16],
// so `arow`, `xc` and `gain` are already offset to this lane's row or column
// and its 8-element k slice; a null column is zero. The A rows of the first
// two batches (and the gains) are issued before `ready()` is called, the
// activations after it. Two load batches alternate, so one batch is always
// in flight while the other is consumed.
template <int NCB, bool GAIN, class Ready>
__device__ __forceinline__ void mm_wave(const uint16_t* arow, const float* const (&xc)[NCB], const uint16_t* gain,
                                        int nsteps, Ready&& ready, f32x4_t (&acc)[NCB], float (&ss)[NCB]) {
    constexpr int PF = MmPf<NCB>::v;
    uint4 a0[PF], a1[PF], g0[PF], g1[PF];
    float4 x0[PF][NCB][2], x1[PF][NCB][2];
    auto loadA = [&](uint4(&a)[PF], uint4(&g)[PF], int bt) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int s = bt * PF + j;
            if (s < nsteps) {
                a[j] = ld16s(arow + 32 * s);
                if (GAIN) g[j] = ld16(gain + 32 * s);
            }
        }
    };
    auto loadX = [&](float4(&x)[PF][NCB][2], int bt) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int s = bt * PF + j;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (s < nsteps && xc[cb] != nullptr) {
                    x[j][cb][0] = ldf4(xc[cb] + 32 * s);
                    x[j][cb][1] = ldf4(xc[cb] + 32 * s + 4);
                } else {
                    x[j][cb][0] = make_float4(0.f, 0.f, 0.f, 0.f);
                    x[j][cb][1] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
    };
    auto compute = [&](const uint4(&a)[PF], const uint4(&g)[PF], const float4(&x)[PF][NCB][2], int bt) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            if (bt * PF + j < nsteps) {
                float gv[8];
                if (GAIN) {
                    const uint4 w = g[j];
                    gv[0] = bflo(w.x); gv[1] = bfhi(w.x); gv[2] = bflo(w.y); gv[3] = bfhi(w.y);
                    gv[4] = bflo(w.z); gv[5] = bfhi(w.z); gv[6] = bflo(w.w); gv[7] = bfhi(w.w);
                }
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    float v[8] = {x[j][cb][0].x, x[j][cb][0].y, x[j][cb][0].z, x[j][cb][0].w,
                                  x[j][cb][1].x, x[j][cb][1].y, x[j][cb][1].z, x[j][cb][1].w};
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        ss[cb] = fmaf(v[q], v[q], ss[cb]);
                        if (GAIN) v[q] *= gv[q];
                    }
                    uint32_t h[8];
                    split8(v, h);
                    acc[cb] = mfma16x16x32(a[j], make_uint4(h[0], h[1], h[2], h[3]), acc[cb]);
                    acc[cb] = mfma16x16x32(a[j], make_uint4(h[4], h[5], h[6], h[7]), acc[cb]);
                }
            }
        }
    };
    const int nb = (nsteps + PF - 1) / PF;
    loadA(a0, g0, 0);
    if (nb > 1) loadA(a1, g1, 1);
    ready();
    loadX(x0, 0);
    for (int bt = 0; bt < nb; bt += 2) {
        if (bt + 1 < nb) loadX(x1, bt + 1);
        compute(a0, g0, x0, bt);
        if (bt + 2 < nb) {
            loadA(a0, g0, bt + 2);
            loadX(x0, bt + 2);
        }
        if (bt + 1 < nb) {
            compute(a1, g1, x1, bt + 1);
            if (bt + 3 < nb) loadA(a1, g1, bt + 3);
        }
    }
}

// LDS of a block product, at the start of the general region: per-wave
// partial products [4][16][16 NCB] and sums of squares [4][16 NCB].
constexpr int kMmPartFloats = NWAVES * 16 * 64;
constexpr int kMmSsFloats = NWAVES * 64;
static_assert(kMmLdsBytes == (kMmPartFloats + kMmSsFloats + 128) * 4, "matrix-core LDS size");

// A product of `na` (1, 2 or 4) blocks of 16 weight rows with 16 NCB
// activation columns over length K, by the whole workgroup: wave w takes row
// block w % na and K part w / na (4 / na parts). arow(blk, r) is the start of
// A row r of block blk, xcol(c) that of activation column c (null: absent),
// gain the RMSNorm gain (GAIN) applied to the activations. The partial sums
// land in LDS; mm_c / mm_ss read the totals, summed over K parts in order.
template <int NCB, bool GAIN, class ARow, class XCol, class Ready>
__device__ __forceinline__ void mm_block(int na, int K, ARow&& arow, XCol&& xcol, const uint16_t* gain, Ready&& ready,
                                         float* sPart, float* sSS) {
    const int tid = tid_(), wave = tid >> 6, lane = tid & 63, col = lane & 15, g4 = lane >> 4;
    const int blk = wave % na, kp = wave / na, KP = NWAVES / na;
    const int kl = K / KP, k0 = kp * kl + 8 * g4;
    const uint16_t* ar = arow(blk, col) + k0;
    const float* xc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const float* q = xcol(16 * cb + col);
        xc[cb] = q != nullptr ? q + k0 : nullptr;
    }
    f32x4_t acc[NCB];
    float ss[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        ss[cb] = 0.f;
    }
    mm_wave<NCB, GAIN>(ar, xc, GAIN ? gain + k0 : nullptr, kl >> 5, ready, acc, ss);
    constexpr int NC = 16 * NCB;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) sPart[(wave * 16 + 4 * g4 + q) * NC + 16 * cb + col] = acc[cb][q];
        float s = ss[cb];
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (g4 == 0) sSS[wave * NC + 16 * cb + col] = s;
    }
    __syncthreads();
}

// Total of row r of block blk, column c (nc = 16 NCB columns).
__device__ __forceinline__ float mm_c(const float* sPart, int nc, int na, int blk, int r, int c) {
    float v = 0.f;
    for (int kp = 0; kp < NWAVES / na; ++kp) v += sPart[((kp * na + blk) * 16 + r) * nc + c];
    return v;
}
// Sum of squares of activation column c over the whole K.
__device__ __forceinline__ float mm_ss(const float* sSS, int nc, int na, int c) {
    float v = 0.f;
    for (int kp = 0; kp < NWAVES / na; ++kp) v += sSS[kp * na * nc + c];
    return v;
}
// RMSNorm scale 1 / sqrt(mean(x^2) + eps) from a sum of squares.
__device__ __forceinline__ float rms_scale(const Params& p, float ss) { return 1.0f / sqrtf(ss * p.inv_h + p.eps); }

// ------------------------------------------- MFMA engine, split activations

// Column blocks of 8 tokens (each token's hi and lo part in adjacent
// columns): compile-time 1, 2, 4 or 8, chosen per call.
template <class F>
__device__ __forceinline__ void with_nc8(int n, F&& f) {
    if (n <= 8) f(Ncb<1>());
    else if (n <= 16) f(Ncb<2>());
    else if (n <= 32) f(Ncb<4>());
    else f(Ncb<8>());
}
__device__ __forceinline__ int nc8_tokens(int n) { return n <= 8 ? 8 : (n <= 16 ? 16 : (n <= 32 ? 32 : 64)); }

template <int NC8>
struct MmPfS {
    static constexpr int v = NC8 == 1 ? 8 : (NC8 == 2 ? 6 : (NC8 == 4 ? 4 : 1));
};

// One wave's product over `nsteps` k-steps of 32 with split activations:
// column 2j + part of block cb is part (hi / lo) of token 8 cb + j, so a
// lane's B operand is one 16-byte load of its part (xc: this lane's token,
// part and k slice, in 16-byte units; null = zero). Twice the k-steps in
// flight of the fp32-input engine for the same registers. On return, lanes
// with an even column hold the token's full product (hi + lo) in acc.
template <int NC8, class Ready>
__device__ __forceinline__ void mm_wave_s(const uint16_t* arow, const uint4* const (&xc)[NC8], int nsteps,
                                          Ready&& ready, f32x4_t (&acc)[NC8]) {
    constexpr int PF = MmPfS<NC8>::v;
    uint4 a0[PF], a1[PF], x0[PF][NC8], x1[PF][NC8];
    auto loadA = [&](uint4(&a)[PF], int bt) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int s = bt * PF + j;
            if (s < nsteps) a[j] = ld16s(arow + 32 * s);
        }
    };
    auto loadX = [&](uint4(&x)[PF][NC8], int bt) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int s = bt * PF + j;
#pragma unroll
            for (int cb = 0; cb < NC8; ++cb)
                x[j][cb] = (s < nsteps && xc[cb] != nullptr) ? ld16(xc[cb] + 8 * s) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto compute = [&](const uint4(&a)[PF], const uint4(&x)[PF][NC8], int bt) {
#pragma unroll
        for (int j = 0; j < PF; ++j)
            if (bt * PF + j < nsteps) {
#pragma unroll
                for (int cb = 0; cb < NC8; ++cb) acc[cb] = mfma16x16x32(a[j], x[j][cb], acc[cb]);
            }
    };
    const int nb = (nsteps + PF - 1) / PF;
    loadA(a0, 0);
    if (nb > 1) loadA(a1, 1);
    ready();
    loadX(x0, 0);
    for (int bt = 0; bt < nb; bt += 2) {
        if (bt + 1 < nb) loadX(x1, bt + 1);
        compute(a0, x0, bt);
        if (bt + 2 < nb) {
            loadA(a0, bt + 2);
            loadX(x0, bt + 2);
        }
        if (bt + 1 < nb) {
            compute(a1, x1, bt + 1);
            if (bt + 3 < nb) loadA(a1, bt + 3);
        }
    }
#pragma unroll
    for (int cb = 0; cb < NC8; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[cb][q] += dpp_mov<0xB1>(acc[cb][q]);
}

// This lane's B-operand pointer into a split vector: token row `row` (null:
// absent), element offset k (a multiple of 8), part = lane column & 1.
__device__ __forceinline__ const uint4* split_ptr(const float* row, int k, int part) {
    return row != nullptr ? reinterpret_cast<const uint4*>(row + k) + part : nullptr;
}

// Block product as mm_block, over split activations: xrow(j) is the split
// vector of token column j (null: absent). Totals per (block, row, token)
// via mm_c with nc = 8 NC8.
template <int NC8, class ARow, class XRow, class Ready>
__device__ __forceinline__ void mm_block_s(int na, int K, ARow&& arow, XRow&& xrow, Ready&& ready, float* sPart) {
    const int tid = tid_(), wave = tid >> 6, lane = tid & 63, col = lane & 15, g4 = lane >> 4;
    const int blk = wave % na, kp = wave / na, KP = NWAVES / na;
    const int kl = K / KP, k0 = kp * kl + 8 * g4;
    const uint16_t* ar = arow(blk, col) + k0;
    const uint4* xc[NC8];
#pragma unroll
    for (int cb = 0; cb < NC8; ++cb) xc[cb] = split_ptr(xrow(8 * cb + (col >> 1)), k0, col & 1);
    f32x4_t acc[NC8];
#pragma unroll
    for (int cb = 0; cb < NC8; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mm_wave_s<NC8>(ar, xc, kl >> 5, ready, acc);
    constexpr int NC = 8 * NC8;
    if ((col & 1) == 0) {
#pragma unroll
        for (int cb = 0; cb < NC8; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) sPart[(wave * 16 + 4 * g4 + q) * NC + 8 * cb + (col >> 1)] = acc[cb][q];
    }
    __syncthreads();
}

// Row blocks for a tile of n rows (n <= 64).
__device__ __forceinline__ int row_blocks(int n) { return n <= 16 ? 1 : (n <= 32 ? 2 : 4); }

// -------------------------------------------------------------------- QKV

// Virtual rows a1..a2 (<= 16) of KV group a0 (query rows of its heads, then
// its key rows, then its value rows) for every token: q, k, v =
// W_qkv (g o x) / rms(x). The RMSNorm scale is applied to the product, so the
// activations are read once, for both the product and their sum of squares.
__device__ __forceinline__ bool tile_qkv_mm(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, g = t.a0, v0 = t.a1, nrows = t.a2 - t.a1;
    const int H = p.H, D = p.D, GD = p.G * p.D, B = p.B;
    auto phys = [&](int v) -> int {
        if (v < GD) return g * GD + v;
        if (v < GD + D) return p.Hq * D + g * D + (v - GD);
        return p.Hq * D + p.Hkv * D + g * D + (v - GD - D);
    };
    const uint16_t* W = wptr(p, l, W_QKV);
    float* sPart = reinterpret_cast<float*>(cx.lds);
    float* sSS = sPart + kMmPartFloats;
    if (!block_wait(p, t.pre_ctr, t.pre_target, cx.t_wait)) return false;
    bool ok = true;
    const float* xin = x_at(p, 2 * l);
    const int ncb = (B + 15) >> 4, nc = ncb_cols(ncb);
    with_ncb(ncb, [&](auto n) {
        mm_block<decltype(n)::v, true>(
            1, H, [&](int, int r) { return W + (int64_t)phys(v0 + (r < nrows ? r : nrows - 1)) * H; },
            [&](int c) -> const float* { return c < B ? xin + (int64_t)c * H : nullptr; }, wptr(p, l, W_ATTN_NORM),
            [&]() {
                ok = block_wait(p, t.ctr, t.target, cx.t_wait);
                mark(cx, 0);
            },
            sPart, sSS);
    });
    if (!ok) return false;
    float* out = qkv_at(p, l);
    for (int i = tid_(); i < nrows * B; i += NT) {
        const int r = i / B, b = i - r * B;
        const float v = mm_c(sPart, nc, 1, 0, r, b) * rms_scale(p, mm_ss(sSS, nc, 1, b));
        st_dev(out + (int64_t)b * p.QKVD + phys(v0 + r), v);
    }
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// --------------------------------------------------------- output projection

// Rows a0..a1 (<= 16) of the hidden size: x_mid = x_in + W_o attn (the
// attention output arrives split).
__device__ __forceinline__ bool tile_oproj_mm(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, r0 = t.a0, nrows = t.a1 - t.a0, B = p.B;
    const int K = p.Hq * p.D;
    const uint16_t* W = wptr(p, l, W_O);
    float* sPart = reinterpret_cast<float*>(cx.lds);
    if (!block_wait(p, t.pre_ctr, t.pre_target, cx.t_wait)) return false;
    bool ok = true;
    const float* att = attout_at(p, l);   // split form (see st_split8)
    const int nc = nc8_tokens(B);
    with_nc8(B, [&](auto n) {
        mm_block_s<decltype(n)::v>(
            1, K, [&](int, int r) { return W + (int64_t)(r0 + (r < nrows ? r : nrows - 1)) * K; },
            [&](int c) -> const float* { return c < B ? att + (int64_t)c * K : nullptr; },
            [&]() {
                ok = block_wait(p, t.ctr, t.target, cx.t_wait);
                mark(cx, 0);
            },
            sPart);
    });
    if (!ok) return false;
    const float* xin = x_at(p, 2 * l);
    float* xout = x_at(p, 2 * l + 1);
    for (int i = tid_(); i < nrows * B; i += NT) {
        const int r = i / B, b = i - r * B;
        const int64_t o = (int64_t)b * p.H + r0 + r;
        st_dev(xout + o, ldg(xin + o) + mm_c(sPart, nc, 1, 0, r, b));
    }
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// ------------------------------------------------------------------ router

// Rows a0..a1 (<= 16) of the router: logits = W_r (g o x_mid) / rms(x_mid)
// (+ bias). Also writes its share (8-element groups a2..a3) of the experts'
// input h2 = RMSNorm(x_mid) * g in split form, as the one- and two-token
// tiles normalise it: (x * rs) * g.
__device__ __forceinline__ bool tile_router_mm(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, r0 = t.a0, nrows = t.a1 - t.a0, H = p.H;
    // tokens of 16-token block tb only: a tile that read every token's
    // residual row would stream B x H fp32 through one workgroup
    const int tb = t.a2 >> 16, b0 = 16 * tb, nb = min(16, p.B - b0);
    const uint16_t* W = wptr(p, l, W_ROUTER);
    const float* bias = reinterpret_cast<const float*>(p.wtab[l * W_NKINDS + W_RBIAS]);
    float* sPart = reinterpret_cast<float*>(cx.lds);
    float* sSS = sPart + kMmPartFloats;
    bool ok = true;
    const float* xm = x_at(p, 2 * l + 1) + (int64_t)b0 * H;
    const int nc = ncb_cols(1);
    mm_block<1, true>(
        1, H, [&](int, int r) { return W + (int64_t)(r0 + (r < nrows ? r : nrows - 1)) * H; },
        [&](int c) -> const float* { return c < nb ? xm + (int64_t)c * H : nullptr; }, wptr(p, l, W_FFN_NORM),
        [&]() {
            ok = block_wait(p, t.ctr, t.target, cx.t_wait);
            mark(cx, 0);
        },
        sPart, sSS);
    if (!ok) return false;
    float* out = rlogits_at(p, l) + (int64_t)b0 * p.E;
    for (int i = tid_(); i < nrows * nb; i += NT) {
        const int r = i / nb, b = i - r * nb;
        const float v = mm_c(sPart, nc, 1, 0, r, b) * rms_scale(p, mm_ss(sSS, nc, 1, b));
        st_dev(out + (int64_t)b * p.E + r0 + r, bias != nullptr ? v + ldg(bias + r0 + r) : v);
    }
    // this tile's share of the expert input h2 = RMSNorm(x_mid) * g, split:
    // groups of 8 elements [g0, g1) of its tokens
    const uint16_t* gn = wptr(p, l, W_FFN_NORM);
    float* h2 = h2s_at(p, l) + (int64_t)b0 * H;
    const int g0 = t.a2 & 0xffff, ng = (t.a3 & 0xffff) - g0;
    for (int i = tid_(); i < ng * nb; i += NT) {
        const int b = i / ng, k = 8 * (g0 + i - b * ng);
        const float rs = rms_scale(p, mm_ss(sSS, nc, 1, b));
        const float4 u = ldf4(xm + (int64_t)b * H + k), v = ldf4(xm + (int64_t)b * H + k + 4);
        const uint4 gw = ld16(gn + k);
        const float x8[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
        const float g8[8] = {bflo(gw.x), bfhi(gw.x), bflo(gw.y), bfhi(gw.y), bflo(gw.z), bfhi(gw.z), bflo(gw.w), bfhi(gw.w)};
        float h8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h8[j] = (x8[j] * rs) * g8[j];
        st_split8(h2 + (int64_t)b * H + k, h8);
    }
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// ----------------------------------------------------------------- routing

// Reductions over each row of 16 lanes (every lane of the row gets the result).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    return max(v, dpp_u32<0x140>(v));
}
__device__ __forceinline__ uint32_t row16_min_u32(uint32_t v) {
    v = min(v, dpp_u32<0xB1>(v));
    v = min(v, dpp_u32<0x4E>(v));
    v = min(v, dpp_u32<0x141>(v));
    return min(v, dpp_u32<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    return v + dpp_mov<0x140>(v);
}

// Every token's top-k (ties to the lower expert index, the largest first)
// and its routing weights (softmax over the selected logits); then the
// routing table: selected experts in ascending id, each with its tokens in
// ascending token order and their ranks. Each row of 16 lanes takes one
// token (NE16 logits per lane, E <= 16 NE16), so a wave ranks four tokens at
// once; thread e owns expert e for the table (E <= 256).
template <int NE16>
__device__ __forceinline__ bool tile_route(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, E = p.E, K = p.K, B = p.B;
    const int tid = tid_(), wave = tid >> 6, lane = tid & 63;
    uint32_t* sMask = reinterpret_cast<uint32_t*>(cx.lds);            // [256][2] tokens per expert
    int8_t* sRank = reinterpret_cast<int8_t*>(sMask + 2 * 256);      // [64][256] rank of expert e for token b
    int* sWave = reinterpret_cast<int*>(sRank + kMaxBatchMM * 256);  // [NWAVES] selected experts per wave
    for (int i = tid; i < 2 * 256; i += NT) sMask[i] = 0u;
    __syncthreads();
    if (!block_wait(p, t.ctr, t.target, cx.t_wait)) return false;
    mark(cx, 0);
    const float* rl = rlogits_at(p, l);
    int32_t* rt = rtab_at(p, l);
    float* rw = rtab_w(p, rt);
    const int gq = lane >> 4, li = lane & 15;
    for (int b0 = 4 * wave; b0 < B; b0 += 4 * NWAVES) {
        const int b = b0 + gq;
        const bool valid = b < B;
        uint32_t u[NE16];  // 0: not a candidate (no float maps to 0)
#pragma unroll
        for (int i = 0; i < NE16; ++i) {
            const int e = li + 16 * i;
            u[i] = (valid && e < E) ? fkey(ld_dev(rl + (int64_t)b * E + e)) : 0u;
        }
        uint32_t top = 0u;
        float sel = 0.f;
        int myid = 0;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j < K) {
                uint32_t v = u[0];
#pragma unroll
                for (int i = 1; i < NE16; ++i) v = max(v, u[i]);
                const uint32_t m = row16_max_u32(v);
                uint32_t cand = 0xffffu;
#pragma unroll
                for (int i = 0; i < NE16; ++i)
                    if (u[i] == m) cand = min(cand, (uint32_t)(li + 16 * i));
                const int best = (int)row16_min_u32(cand);
                if (j == 0) top = m;
                if (li == j) {
                    sel = unkey(m);
                    myid = best;
                }
#pragma unroll
                for (int i = 0; i < NE16; ++i)
                    if (li + 16 * i == best) u[i] = 0u;
            }
        }
        const float ex = li < K ? expf(sel - unkey(top)) : 0.f;
        const float sum = row16_sum(ex);
        if (valid && li < K) {
            const float w = ex / sum;
            sRank[b * 256 + myid] = (int8_t)li;
            atomicOr(&sMask[2 * myid + (b >> 5)], 1u << (b & 31));
            st_dev(rw + b * K + li, w);
            p.route_ids[((int64_t)l * p.max_batch + b) * K + li] = myid;
            p.route_w[((int64_t)l * p.max_batch + b) * K + li] = w;
        }
    }
    __syncthreads();
    const int e = tid;
    const uint32_t m0 = e < E ? sMask[2 * e] : 0u, m1 = e < E ? sMask[2 * e + 1] : 0u;
    const int n = __popc(m0) + __popc(m1);
    const uint64_t bal = __ballot(n > 0);
    if (lane == 0) sWave[wave] = __popcll(bal);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += sWave[w];
    if (n > 0) {
        const int slot = base + __popcll(bal & ((1ull << lane) - 1ull));
        st_dev_i(rt + 64 + slot, e);
        st_dev_i(rt + 64 + E + slot, n);
        int32_t* lst = rt + 64 + 2 * E + (int64_t)slot * p.max_batch;
        int c = 0;
        for (int h = 0; h < 2; ++h) {
            uint32_t m = h ? m1 : m0;
            while (m != 0u) {
                const int b = 32 * h + __builtin_ctz(m);
                m &= m - 1u;
                st_dev_i(lst + c++, b | ((int)sRank[b * 256 + e] << 16));
            }
        }
    }
    if (tid == 0) st_dev_i(rt, sWave[0] + sWave[1] + sWave[2] + sWave[3]);
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// ------------------------------------------------------------ expert slots

// Expert tiles for batches of 3+ are (rows, slot group) pairs: a tile takes
// slots q0, q0 + Q, q0 + 2Q, ... of the routing table (however many experts
// the step selected), and its waves take those slots in turn. The slots'
// experts, token counts and token lists are read into LDS once per chunk of
// slots; each wave then streams all its slots as one pipeline of load
// batches, so the next slot's weight rows are in flight while the current
// one finishes.
constexpr int kDownLdsInts = 4096;
static_assert(kDownLdsInts * 4 <= kRouteLdsBytes, "slot tables fit the general LDS region");

struct SlotTables {
    int* e;    // [chunk] expert of each slot
    int* n;    // [chunk] tokens routed to it
    int* ent;  // [chunk][max_batch] (token | rank << 16)
    int chunk; // slots per LDS chunk
};

__device__ __forceinline__ SlotTables slot_tables(char* lds, int max_batch) {
    SlotTables s;
    s.chunk = (kDownLdsInts - 64) / (max_batch + 2);
    s.e = reinterpret_cast<int*>(lds);
    s.n = s.e + s.chunk;
    s.ent = s.n + s.chunk;
    return s;
}

// Read slots q0 + Q (c0 + i), i < mc, into LDS (one round trip), then barrier.
__device__ __forceinline__ void load_slot_tables(const Params& p, const int32_t* rt, int q0, int Q, int c0, int mc,
                                                 const SlotTables& s) {
    const int tid = tid_(), maxB = p.max_batch;
    for (int i = tid; i < mc; i += NT) {
        const int sl = q0 + Q * (c0 + i);
        s.e[i] = ldg(rt + 64 + sl);
        s.n[i] = ldg(rt + 64 + p.E + sl);
    }
    for (int i = tid; i < mc * maxB; i += NT) {
        const int j = i / maxB, c = i - j * maxB;
        s.ent[i] = ldg(rt + 64 + 2 * p.E + (int64_t)(q0 + Q * (c0 + j)) * maxB + c);
    }
    __syncthreads();
}

// Row blocks a wave multiplies per load of its activations, in a kernel
// built for tiles of RBK row blocks, and k-steps per batch, by the number of
// 8-token column blocks: the weights and the activations of two batches in
// flight fill about the same registers.
template <int NC8, int RBK>
struct MmRb {
    static constexpr int v = NC8 <= 2 ? RBK : 1;
};
template <int NC8, int R>
struct MmPfR {
    static constexpr int v = R == 1 ? MmPfS<NC8>::v : (NC8 == 1 ? 6 : 4);
};

// One wave's slots (chunk indices wave, wave + 4, ...; mw of them) as one
// stream of nsteps k-steps each: acc[cb] += A x B over the slot, then
// flush(i, acc) at its end (acc: hi + lo summed on even columns; i: chunk
// index). a_ptr(i, k) / x_ptr(i, cb, k): this lane's A row and B operand
// (null: zero) at k-step k of slot i. ready() is called by every wave once
// the first two batches of A are requested and before any B is (it may wait
// on a counter at block level).
template <int NC8, class APtr, class XPtr, class Flush, class Ready>
__device__ __forceinline__ void slot_stream(int mw, int nsteps, APtr&& a_ptr, XPtr&& x_ptr, Flush&& flush,
                                            Ready&& ready) {
    constexpr int PF = MmPfS<NC8>::v;
    const int wave = tid_() >> 6;
    int spb = PF;   // k-steps per batch: the largest divisor of nsteps <= PF
    while (nsteps % spb) --spb;
    const int nbps = nsteps / spb, nbt = mw * nbps;
    uint4 a0[PF], a1[PF], x0[PF][NC8], x1[PF][NC8];
    auto loadA = [&](uint4(&a)[PF], int b) {
        const int j = b / nbps;
        const uint16_t* ap = a_ptr(wave + NWAVES * j, spb * (b - j * nbps));
#pragma unroll
        for (int q = 0; q < PF; ++q)
            if (q < spb) a[q] = ld16s(ap + 32 * q);
    };
    auto loadX = [&](uint4(&x)[PF][NC8], int b) {
        const int j = b / nbps;
#pragma unroll
        for (int cb = 0; cb < NC8; ++cb) {
            const uint4* xp = x_ptr(wave + NWAVES * j, cb, spb * (b - j * nbps));
#pragma unroll
            for (int q = 0; q < PF; ++q)
                x[q][cb] = (q < spb && xp != nullptr) ? ld16(xp + 8 * q) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    f32x4_t acc[NC8];
#pragma unroll
    for (int cb = 0; cb < NC8; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const uint4(&a)[PF], const uint4(&x)[PF][NC8], int b) {
#pragma unroll
        for (int q = 0; q < PF; ++q)
            if (q < spb) {
#pragma unroll
                for (int cb = 0; cb < NC8; ++cb) acc[cb] = mfma16x16x32(a[q], x[q][cb], acc[cb]);
            }
        if ((b + 1) % nbps == 0) {
#pragma unroll
            for (int cb = 0; cb < NC8; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[cb][q] += dpp_mov<0xB1>(acc[cb][q]);
            flush(wave + NWAVES * (b / nbps), acc);
#pragma unroll
            for (int cb = 0; cb < NC8; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    if (nbt > 0) {
        loadA(a0, 0);
        if (nbt > 1) loadA(a1, 1);
    }
    ready();
    if (nbt > 0) {
        loadX(x0, 0);
        for (int bt = 0; bt < nbt; bt += 2) {
            if (bt + 1 < nbt) loadX(x1, bt + 1);
            compute(a0, x0, bt);
            if (bt + 2 < nbt) {
                loadA(a0, bt + 2);
                loadX(x0, bt + 2);
            }
            if (bt + 1 < nbt) {
                compute(a1, x1, bt + 1);
                if (bt + 3 < nbt) loadA(a1, bt + 3);
            }
        }
    }
}

// slot_stream over tiles of several row blocks: one stream of batches of
// k-steps per wave, items (slot, pass)
// for its slots (chunk indices wave, wave + 4, ...; mw of them), each pass
// covering R row blocks of the tile (blocks R ps .. R ps + R - 1) over
// nsteps k-steps: acc[r][cb] += A_r x B over the slot, then flush(i, blk0,
// acc) at the item's end (acc: hi + lo summed on even columns; i: chunk
// index; blk0: the pass's first block). a_ptr(i, blk, k) / x_ptr(i, cb, k):
// this lane's A row of block blk and B operand (null: zero) at k-step k of
// slot i; one B load serves the R blocks.
template <int NC8, int R, class APtr, class XPtr, class Flush>
__device__ __forceinline__ void slot_stream_rb(int mw, int npass, int nsteps, APtr&& a_ptr, XPtr&& x_ptr,
                                               Flush&& flush) {
    constexpr int PF = MmPfR<NC8, R>::v;
    const int wave = tid_() >> 6;
    int spb = PF;   // k-steps per batch: the largest divisor of nsteps <= PF
    while (nsteps % spb) --spb;
    const int nbps = nsteps / spb, nbt = mw * npass * nbps;
    uint4 a0[PF][R], a1[PF][R], x0[PF][NC8], x1[PF][NC8];
    auto loadA = [&](uint4(&a)[PF][R], int b) {
        const int it = b / nbps, j = it / npass, ps = it - j * npass;
        const int k0 = spb * (b - it * nbps);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint16_t* ap = a_ptr(wave + NWAVES * j, R * ps + r, k0);
#pragma unroll
            for (int q = 0; q < PF; ++q)
                if (q < spb) a[q][r] = ld16s(ap + 32 * q);
        }
    };
    auto loadX = [&](uint4(&x)[PF][NC8], int b) {
        const int it = b / nbps, j = it / npass;
        const int k0 = spb * (b - it * nbps);
#pragma unroll
        for (int cb = 0; cb < NC8; ++cb) {
            const uint4* xp = x_ptr(wave + NWAVES * j, cb, k0);
#pragma unroll
            for (int q = 0; q < PF; ++q)
                x[q][cb] = (q < spb && xp != nullptr) ? ld16(xp + 8 * q) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    f32x4_t acc[R][NC8];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int cb = 0; cb < NC8; ++cb) acc[r][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const uint4(&a)[PF][R], const uint4(&x)[PF][NC8], int b) {
#pragma unroll
        for (int q = 0; q < PF; ++q)
            if (q < spb) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int cb = 0; cb < NC8; ++cb) acc[r][cb] = mfma16x16x32(a[q][r], x[q][cb], acc[r][cb]);
            }
        if ((b + 1) % nbps == 0) {
            const int it = b / nbps, j = it / npass, ps = it - j * npass;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int cb = 0; cb < NC8; ++cb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[r][cb][q] += dpp_mov<0xB1>(acc[r][cb][q]);
            flush(wave + NWAVES * j, R * ps, acc);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int cb = 0; cb < NC8; ++cb) acc[r][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    if (nbt > 0) {
        loadA(a0, 0);
        if (nbt > 1) loadA(a1, 1);
        loadX(x0, 0);
        for (int bt = 0; bt < nbt; bt += 2) {
            if (bt + 1 < nbt) loadX(x1, bt + 1);
            compute(a0, x0, bt);
            if (bt + 2 < nbt) {
                loadA(a0, bt + 2);
                loadX(x0, bt + 2);
            }
            if (bt + 1 < nbt) {
                compute(a1, x1, bt + 1);
                if (bt + 3 < nbt) loadA(a1, bt + 3);
            }
        }
    }
}

// Runs body(tables, c0, mc, NC8 tag) per LDS chunk of this tile's slots, NC8
// sized for the chunk's widest slot. Block-uniform.
template <class Body>
__device__ __forceinline__ void for_slot_chunks(const Params& p, const int32_t* rt, int q0, int Q, char* lds,
                                                Body&& body) {
    const int nact = ldg(rt);
    const int mt = nact > q0 ? (nact - q0 + Q - 1) / Q : 0;
    const SlotTables s = slot_tables(lds, p.max_batch);
    const int lane = tid_() & 63;
    for (int c0 = 0; c0 < mt; c0 += s.chunk) {
        const int mc = min(s.chunk, mt - c0);
        load_slot_tables(p, rt, q0, Q, c0, mc, s);
        uint32_t mx = 0u;
        for (int i = lane; i < mc; i += 64) mx = max(mx, (uint32_t)s.n[i]);
        mx = wave_max_u32(mx);
        with_nc8((int)mx, [&](auto nn) { body(s, mc, nn); });
        __syncthreads();
    }
}

// ---------------------------------------------------------- expert gate/up

// Rows a0..a1 (whole 8-row blocks) of the expert width, slots a2, a2 + a3,
// ... of the routing table: a = SiLU(W_gate h2) * (W_up h2) for the tokens
// routed to each slot's expert, h2 = RMSNorm(x_mid) * g (split, from the
// router tiles), written split to the (token, rank) row of the activations.
// One MFMA block holds the 8 gate rows (A rows 0-7) and the 8 up rows (A rows
// 8-15) of an 8-row block of the slot's expert, so SwiGLU pairs meet in one
// wave.
template <int RBK>
__device__ __forceinline__ bool tile_gateup_mm(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, r0 = t.a0, q0 = t.a2, Q = t.a3, H = p.H, K = p.K, I = p.I;
    const int lane = tid_() & 63, col = lane & 15, g4 = lane >> 4;
    if (!block_wait(p, t.ctr, t.target, cx.t_wait)) return false;
    mark(cx, 0);
    const int32_t* rt = rtab_at(p, l);
    const uint16_t* Wg = wptr(p, l, W_GATE);
    const uint16_t* Wu = wptr(p, l, W_UP);
    const float* h2 = h2s_at(p, l);
    float* act = act_at(p, l);
    const int wave = tid_() >> 6;
    // 8-row blocks of this tile (one in a kernel built for one, where the
    // plan gives every gate/up tile 8 rows)
    const int nrb = RBK == 1 ? 1 : (t.a1 - r0 + 7) >> 3;
    for_slot_chunks(p, rt, q0, Q, cx.lds, [&](const SlotTables& s, int mc, auto nn) {
        constexpr int NC8 = decltype(nn)::v;
        const int mw = mc > wave ? (mc - wave + NWAVES - 1) / NWAVES : 0;
        const uint16_t* Wrow = (col < 8 ? Wg : Wu) + (int64_t)(r0 + (col & 7)) * H + 8 * g4;
        auto x_ptr = [&](int i, int cb, int k) -> const uint4* {
            const int c = 8 * cb + (col >> 1);
            if (c >= s.n[i]) return nullptr;
            return split_ptr(h2 + (int64_t)(s.ent[i * p.max_batch + c] & 0xffff) * H, 8 * g4 + 32 * k, col & 1);
        };
        // block blk of slot i: lane (col, g4) holds rows 4 g4 + q; gate rows
        // 0-7 in g4 0-1, up rows 8-15 in g4 2-3 (wave-uniform call)
        auto store = [&](int i, int blk, const f32x4_t(&acc)[NC8]) {
#pragma unroll
            for (int cb = 0; cb < NC8; ++cb) {
                float a4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float up = __shfl_xor(acc[cb][q], 32);
                    const float g = acc[cb][q];
                    a4[q] = (g / (1.0f + expf(-g))) * up;
                }
                const int c = 8 * cb + (col >> 1);
                if ((col & 1) == 0 && g4 < 2 && c < s.n[i]) {
                    const int ent = s.ent[i * p.max_batch + c];
                    // elements 4 g4 .. 4 g4 + 3 of the row's 8-group: half of its hi and of its lo half
                    uint32_t hi0, lo0, hi1, lo1;
                    split_pair(a4[0], a4[1], hi0, lo0);
                    split_pair(a4[2], a4[3], hi1, lo1);
                    uint32_t* d = reinterpret_cast<uint32_t*>(act + ((int64_t)(ent & 0xffff) * K + (ent >> 16)) * I +
                                                              r0 + 8 * blk);
                    uint64_t* dh = reinterpret_cast<uint64_t*>(d + 2 * g4);
                    uint64_t* dl = reinterpret_cast<uint64_t*>(d + 4 + 2 * g4);
                    __hip_atomic_store(dh, (uint64_t)hi0 | ((uint64_t)hi1 << 32), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(dl, (uint64_t)lo0 | ((uint64_t)lo1 << 32), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        };
        if constexpr (RBK == 1) {
            slot_stream<NC8>(
                mw, H >> 5, [&](int i, int k) { return Wrow + (int64_t)s.e[i] * I * H + 32 * k; }, x_ptr,
                [&](int i, f32x4_t(&acc)[NC8]) { store(i, 0, acc); }, [] {});
        } else {
            constexpr int R = MmRb<NC8, RBK>::v;
            slot_stream_rb<NC8, R>(
                mw, (nrb + R - 1) / R, H >> 5,
                [&](int i, int blk, int k) {
                    return Wrow + (int64_t)s.e[i] * I * H + (int64_t)8 * (blk < nrb ? blk : nrb - 1) * H + 32 * k;
                },
                x_ptr,
                [&](int i, int blk0, f32x4_t(&acc)[R][NC8]) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (blk0 + r < nrb) store(i, blk0 + r, acc[r]);
                });
        }
    });
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// ------------------------------------------------------------ expert down

// Rows a0..a1 (16-row blocks, the last one possibly partial) of the hidden
// size, slots a2, a2 + a3, ... of the routing table: y = W_down a (a split,
// from the gate/up tiles) for each
// token routed to the slot's expert, written to that token's (token, rank)
// row of the expert outputs. The routing (pre counter) fixes the tile's
// expert rows, so with one row block the first weight batches are
// requested before the wait on the gate/up tiles (main counter) that the
// activations need.
template <int RBK>
__device__ __forceinline__ bool tile_down_mm(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, h0 = t.a0, nrows = t.a1 - t.a0, q0 = t.a2, Q = t.a3;
    const int H = p.H, K = p.K, I = p.I;
    const int lane = tid_() & 63, col = lane & 15, g4 = lane >> 4, wave = tid_() >> 6;
    if (!block_wait(p, t.pre_ctr, t.pre_target, cx.t_wait)) return false;
    // the wait on the gate/up tiles, once, by every wave at the same point
    // (inside the first slot chunk, or after the chunks if there is none)
    bool ok = true, waited = false;
    auto ready = [&]() {
        if (waited) return;
        waited = true;
        ok = block_wait(p, t.ctr, t.target, cx.t_wait);
        mark(cx, 0);
    };
    const int32_t* rt = rtab_at(p, l);
    const uint16_t* Wd = wptr(p, l, W_DOWN);
    const float* act = act_at(p, l);
    float* y = ybuf_at(p, l);
    // 16-row blocks of this tile (one in a kernel built for one, where the
    // plan gives every down tile at most 16 rows)
    const int nrb = RBK == 1 ? 1 : (nrows + 15) >> 4;
    // the two-block stream waits before its first request (holding its
    // first batches across the wait spills that kernel's registers)
    if constexpr (RBK > 1) ready();
    for_slot_chunks(p, rt, q0, Q, cx.lds, [&](const SlotTables& s, int mc, auto nn) {
        constexpr int NC8 = decltype(nn)::v;
        const int mw = mc > wave ? (mc - wave + NWAVES - 1) / NWAVES : 0;
        auto x_ptr = [&](int i, int cb, int k) -> const uint4* {
            const int c = 8 * cb + (col >> 1);
            if (c >= s.n[i]) return nullptr;
            const int ent = s.ent[i * p.max_batch + c];
            return split_ptr(act + ((int64_t)(ent & 0xffff) * K + (ent >> 16)) * I, 8 * g4 + 32 * k, col & 1);
        };
        // block blk of slot i: rows 16 blk + 4 g4 + q of the tile
        auto store = [&](int i, int blk, const f32x4_t(&acc)[NC8]) {
#pragma unroll
            for (int cb = 0; cb < NC8; ++cb) {
                const int c = 8 * cb + (col >> 1);
                if ((col & 1) == 0 && c < s.n[i]) {
                    const int ent = s.ent[i * p.max_batch + c];
                    float* yr = y + ((int64_t)(ent & 0xffff) * K + (ent >> 16)) * H + h0 + 16 * blk;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (16 * blk + 4 * g4 + q < nrows) st_dev(yr + 4 * g4 + q, acc[cb][q]);
                }
            }
        };
        if constexpr (RBK == 1) {
            const int rsel = col < nrows ? col : nrows - 1;
            const uint16_t* Wrow = Wd + (int64_t)(h0 + rsel) * I + 8 * g4;
            slot_stream<NC8>(
                mw, I >> 5, [&](int i, int k) { return Wrow + (int64_t)s.e[i] * H * I + 32 * k; }, x_ptr,
                [&](int i, f32x4_t(&acc)[NC8]) { store(i, 0, acc); }, ready);
        } else {
            constexpr int R = MmRb<NC8, RBK>::v;
            slot_stream_rb<NC8, R>(
                mw, (nrb + R - 1) / R, I >> 5,
                [&](int i, int blk, int k) {
                    // rows past the tile's end re-read its last row (their products are not stored)
                    const int b = blk < nrb ? blk : nrb - 1;
                    const int rb = min(16, nrows - 16 * b);
                    const int rsel = 16 * b + (col < rb ? col : rb - 1);
                    return Wd + ((int64_t)s.e[i] * H + h0 + rsel) * I + 8 * g4 + 32 * k;
                },
                x_ptr,
                [&](int i, int blk0, f32x4_t(&acc)[R][NC8]) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (blk0 + r < nrb) store(i, blk0 + r, acc[r]);
                });
        }
    });
    ready();
    if (!ok) return false;  // block-uniform (block_wait)
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

// ------------------------------------------------------------- expert sum

// Rows a0..a1 of the hidden size: x_out = x_mid + sum_j w_j y_j over each
// token's top-k in rank order.
__device__ __forceinline__ bool tile_moesum(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int l = t.layer, h0 = t.a0, nrows = t.a1 - t.a0, H = p.H, K = p.K;
    if (!block_wait(p, t.ctr, t.target, cx.t_wait)) return false;
    const float* w = rtab_w(p, rtab_at(p, l));
    const float* y = ybuf_at(p, l);
    const float* xm = x_at(p, 2 * l + 1);
    float* xo = x_at(p, 2 * l + 2);
    for (int i = tid_(); i < p.B * nrows; i += NT) {
        const int b = i / nrows, r = i - b * nrows;
        float wv[kMaxTopK], yv[kMaxTopK];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            wv[j] = j < K ? ldg(w + b * K + j) : 0.f;
            yv[j] = j < K ? ldg(y + ((int64_t)b * K + j) * H + h0 + r) : 0.f;
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
            if (j < K) acc += wv[j] * yv[j];
        const int64_t o = (int64_t)b * H + h0 + r;
        st_dev(xo + o, ldg(xm + o) + acc);
    }
    block_signal(p, t.signal);
    return true;
}

// ------------------------------------------------------------- final norm

// Tokens a0..a1: the final RMSNorm of the last layer's output,
// (x / sqrt(mean(x^2) + eps)) * g, stored split (st_split8) into slice L of
// the experts'-input buffer, where every LM-head tile reads it as its
// matrix-core operand. Each thread takes 8 consecutive elements per round
// (the supported hidden sizes fit in kRounds rounds).
__device__ __forceinline__ bool tile_fnorm(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    constexpr int kRounds = 4;
    const int H8 = p.H >> 3, tid = tid_(), lane = tid & 63, wave = tid >> 6;
    float* sred = reinterpret_cast<float*>(cx.lds);
    if (!block_wait(p, t.ctr, t.target, cx.t_wait)) return false;
    const float* xf = x_at(p, 2 * p.L);
    float* hf = h2s_at(p, p.L);
    for (int b = t.a0; b < t.a1; ++b) {
        float v[kRounds][8];
        float ss = 0.f;
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int e8 = tid + r * NT;
            if (e8 < H8) {
                const float* src = xf + (int64_t)b * p.H + 8 * e8;
                const float4 u = ldf4(src), w = ldf4(src + 4);
                v[r][0] = u.x; v[r][1] = u.y; v[r][2] = u.z; v[r][3] = u.w;
                v[r][4] = w.x; v[r][5] = w.y; v[r][6] = w.z; v[r][7] = w.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[r][j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) ss = fmaf(v[r][j], v[r][j], ss);
        }
        ss = wave_sum(ss);
        if (lane == 0) sred[wave] = ss;
        __syncthreads();
        const float inv = 1.0f / sqrtf((((sred[0] + sred[1]) + sred[2]) + sred[3]) * p.inv_h + p.eps);
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int e8 = tid + r * NT;
            if (e8 < H8) {
                const uint4 gw = ld16(p.final_norm + 8 * e8);
                const float gv[8] = {bflo(gw.x), bfhi(gw.x), bflo(gw.y), bfhi(gw.y),
                                     bflo(gw.z), bfhi(gw.z), bflo(gw.w), bfhi(gw.w)};
                float o[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] = (v[r][j] * inv) * gv[j];
                st_split8(hf + (int64_t)b * p.H + 8 * e8, o);
            }
        }
        __syncthreads();   // sred is written again for the next token
    }
    block_signal(p, t.signal);
    return true;
}

// ---------------------------------------------------------------- LM head

// Rows a0..a1 (<= 64) of the LM head: logits = W_lm h over the normalised
// final residual h that the final-norm tiles stored split.
__device__ __forceinline__ bool tile_lmhead_mm(const Task& t, TileCtx& cx) {
    const Params& p = cx.p;
    const int r0 = t.a0, nrows = t.a1 - t.a0, B = p.B, H = p.H;
    float* sPart = reinterpret_cast<float*>(cx.lds);
    bool ok = true;
    const float* hf = h2s_at(p, p.L);   // normalised final residual, split (tile_fnorm)
    const int na = row_blocks(nrows);
    const int nc = nc8_tokens(B);
    with_nc8(B, [&](auto n) {
        mm_block_s<decltype(n)::v>(
            na, H,
            [&](int blk, int r) {
                const int rr = 16 * blk + r;
                return p.lm_head + (int64_t)(r0 + (rr < nrows ? rr : nrows - 1)) * H;
            },
            [&](int c) -> const float* { return c < B ? hf + (int64_t)c * H : nullptr; },
            [&]() { ok = block_wait(p, t.ctr, t.target, cx.t_wait); }, sPart);
    });
    if (!ok) return false;
    for (int i = tid_(); i < nrows * B; i += NT) {
        const int r = i / B, b = i - r * B;
        p.logits[(int64_t)b * p.V + r0 + r] = mm_c(sPart, nc, na, r >> 4, r & 15, b);
    }
    mark(cx, 1);
    block_signal(p, t.signal);
    return true;
}

}  // namespace mk
