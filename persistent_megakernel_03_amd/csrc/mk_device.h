// mk_device.h -- device side of the decode step: counter protocol, the
// streaming matrix-vector engine, and the tile functions.
//
// Every tile has the same calling convention, tile_xxx(task, params, lds):
//   1. issue loads of the tile's immutable inputs (weights, old KV pages)
//      into registers -- immutable weights start loading before the tile's
//      activation input is ready ("Cohere Publishes One-Kernel Server for
//      North Mini Code, Claims 1.58x vLLM Speedup", section "What the
//      scheduling change is meant to avoid");
//   2. wait on the task's dependency counter in global memory (agent-scope
//      acquire; same page, section "One resident program, many small tasks");
//   3. compute from registers and LDS, write outputs;
//   4. release the outputs and bump the task's counter.
// The per-op build runs the same functions with waits and signals switched
// off; kernel boundaries are then the only ordering.
#pragma once

#include <hip/hip_runtime.h>

#include "mk_common.h"

namespace mk {

constexpr int NT = 256;      // threads per workgroup
constexpr int NWAVES = NT / 64;
constexpr int kMaxBatch = 2; // batch handled by the register-resident GEMV tiles
constexpr int kMaxTopK = 8;
constexpr int kMaxSlots = kMaxBatch * kMaxTopK;
constexpr int kSC = 128;     // attention sub-chunk: tokens per MFMA pass
constexpr int kSPad = kSC + 4;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Thread index through an empty asm barrier: per-lane values derived from it
// are then computed inside each tile instead of being hoisted out of the task
// loop, where values from every tile type would stay live at once and raise
// register pressure for all of them.
__device__ __forceinline__ int tid_() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// ----------------------------------------------------------------- numerics

__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> BF16 bits, nearest with ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Activations enter the weight products as two BF16 parts, x = hi + lo with
// hi = bf16(x) and lo = bf16(x - hi), so |x - hi - lo| <= 2^-17 |x|: eight
// values of one 16-byte weight chunk are held as four hi pairs then four lo
// pairs. The products then run on the packed BF16 dot-product instruction
// (two weight-activation products and an fp32 accumulate per instruction,
// with no unpacking of the weights), half the vector instructions of
// unpacking each weight to fp32 for a fused multiply-add.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
    const bf16x2_t h = {(__bf16)a, (__bf16)b};
    const bf16x2_t l = {(__bf16)(a - (float)h[0]), (__bf16)(b - (float)h[1])};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

// Eight fp32 activations -> {hi pairs[4], lo pairs[4]}.
__device__ __forceinline__ void split8(const float (&v)[8], uint32_t (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) split_pair(v[2 * j], v[2 * j + 1], x[j], x[4 + j]);
}

// A lane's activation slices (NB tokens, NCH chunks) -> their BF16 parts.
template <int NB, int NCH>
__device__ __forceinline__ void split_x(const float (&h)[NB][NCH][8], uint32_t (&hx)[NB][NCH][8]) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < NCH; ++c) split8(h[b][c], hx[b][c]);
}

__device__ __forceinline__ float dot2bf(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), acc,
                                           false);
}

// DPP move within rows of 16 lanes (compile-time control word).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float readlane(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Wave-wide sum, the same in every lane: pairs, quads (quad_perm), half rows
// (row_half_mirror), rows of 16 (row_mirror), then the four row sums. All
// steps are DPP or lane reads, so there is no LDS round trip.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);  // row_half_mirror
    v += dpp_mov<0x140>(v);  // row_mirror
    return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

// wave_sum of N values at once, each step issued for all of them before the
// next step, so the DPP and lane-read latencies of one value hide behind the
// others. Each value is summed in exactly wave_sum's order.
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_mov<0xB1>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_mov<0x4E>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_mov<0x141>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_mov<0x140>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = (readlane(v[i], 0) + readlane(v[i], 16)) + (readlane(v[i], 32) + readlane(v[i], 48));
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}

// Loads through global-address-space pointers. Weight pointers come from a
// table in memory, so the compiler cannot tell they are global and would emit
// FLAT loads, which also count against the LDS wait counter: every later LDS
// access would then wait for all weight rows in flight, serialising the
// prefetch. All buffers here are device memory.
// (The casts go through clang's native vector types: a load through the HIP
// vector classes would still be generic.)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
#define MK_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ float ldg(const float* p) { return *(const MK_GLOBAL float*)p; }
__device__ __forceinline__ int32_t ldg(const int32_t* p) { return *(const MK_GLOBAL int32_t*)p; }
__device__ __forceinline__ uint4 ld16(const void* p) {
    const u32x4_t v = *(const MK_GLOBAL u32x4_t*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Streamed data read once per step (weights, cache pages): non-temporal
// loads, so they do not displace the activations and counters that many
// workgroups share in the L2 and the last-level cache.
__device__ __forceinline__ uint4 ld16s(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load((const MK_GLOBAL u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8s(const void* p) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = __builtin_nontemporal_load((const MK_GLOBAL u32x2_t*)p);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint2 ld8(const void* p) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = *(const MK_GLOBAL u32x2_t*)p;
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 ldf4(const float* p) {
    const f32x4v_t v = *(const MK_GLOBAL f32x4v_t*)p;
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ const uint16_t* wptr(const Params& p, int layer, int kind) {
    return reinterpret_cast<const uint16_t*>(p.wtab[layer * W_NKINDS + kind]);
}

// Split a finite fp32 value into three BF16 parts whose sum reproduces it to
// about 2^-24 relative: each part keeps the top bits of what the previous
// parts left (truncation; the remainders are exact in fp32). MFMA products
// of BF16 parts are exact and accumulate in fp32, so three passes give
// fp32-grade dot products on the matrix cores.
__device__ __forceinline__ void split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const uint32_t u = __float_as_uint(v);
    hi = u >> 16;
    const float r1 = v - __uint_as_float(u & 0xffff0000u);
    const uint32_t u1 = __float_as_uint(r1);
    mid = u1 >> 16;
    const float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
    lo = __float_as_uint(r2) >> 16;
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// D(16x16) += A(16x16) * B(16x16), BF16 operands, fp32 accumulate.
// Lane l holds A[l%16][4(l/16) .. +3], B[4(l/16) .. +3][l%16] and
// D[4(l/16) .. +3][l%16].
__device__ __forceinline__ f32x4_t mfma16x16x16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                     0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16), BF16 operands, fp32 accumulate.
// Lane l holds A[l%16][8(l/16) .. +7], B[8(l/16) .. +7][l%16] and
// D[4(l/16) .. +3][l%16].
__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ------------------------------------------------------ counter protocol

__device__ __forceinline__ void raise_error(const Params& p, int32_t code, int32_t detail, bool abort) {
    // operands made opaque here, on the rare error path: as constants they
    // would be hoisted into registers held across the whole task loop
    int32_t expected = 0;
    asm volatile("" : "+v"(code), "+v"(expected));
    if (__hip_atomic_compare_exchange_strong(p.err, &expected, code, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        __hip_atomic_store(p.err + 1, detail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (abort) __hip_atomic_store(p.err + 2, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Data exchanged between workgroups inside a step (activations, attention
// partials, router logits, expert activations) lives in buffers that are
// written at most once per step: every buffer has one slice per layer. The
// producer writes with device-scope (agent) relaxed atomic stores -- plain
// stores carrying the SC1 cache-policy bit, which gfx950 writes through past
// the XCD's L2 -- and waits for them to complete before bumping a counter.
// Consumers read with ordinary cached loads: no XCD can hold a stale copy of
// a slice, because caches are invalidated at kernel start and no one reads a
// slice before its producer has finished. Hot activation vectors read by
// hundreds of workgroups are then served from each XCD's L2 after one miss.
// The memory model's agent-scope fences would instead write back
// (buffer_wbl2) or invalidate (buffer_inv) a whole XCD's L2 on every task,
// which serialises the L2 under thousands of tasks per step.
__device__ __forceinline__ float ld_dev(const float* p) { return ldg(p); }
__device__ __forceinline__ int32_t ld_dev(const int32_t* p) { return ldg(p); }
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wave's outstanding memory operations (in particular its
// device-scope stores) have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Block-wide wait until counter `ctr` (the sum of its kCtrSub lines) reaches
// `target`. Lanes 0..kCtrSub-1 of wave 0 poll one line each with
// device-scope loads; the barrier then orders every thread's later loads
// after the observation. Returns false if the step was aborted (watchdog
// here or elsewhere). Records when the wait ended in *t_wait (thread 0).
__device__ __forceinline__ uint32_t counter_line(const Params& p, int ctr) {
    const int lane = tid_() & 63;
    const uint32_t* c = p.ctr + ((int64_t)ctr * kCtrSub + (lane & (kCtrSub - 1))) * kCtrStride;
    return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t line_sum(uint32_t v) {
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kCtrSub; ++j) s += (uint32_t)__builtin_amdgcn_readlane((int)v, j);
    return s;
}

__device__ bool block_wait(const Params& p, int ctr, int target, uint64_t* t_wait) {
    if (p.perop || ctr < 0) return true;
    int ok = 1;
    if (tid_() < 64) {
        if (line_sum(counter_line(p, ctr)) < (uint32_t)target) {
            const uint64_t t0 = wall_clock64();
            uint32_t it = 0;
            while (line_sum(counter_line(p, ctr)) < (uint32_t)target) {
                __builtin_amdgcn_s_sleep(1);
                if ((++it & 31u) == 0) {
                    if (__hip_atomic_load(p.err + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                        ok = 0;
                        break;
                    }
                    if ((int64_t)(wall_clock64() - t0) > p.watchdog_ticks) {
                        if (tid_() == 0) raise_error(p, kErrTimeout, ctr, true);
                        ok = 0;
                        break;
                    }
                }
            }
        }
        if (tid_() == 0) *t_wait = wall_clock64();
    }
    // wave 0's verdict to every thread through one LDS word; the second
    // barrier keeps the next wait's write after every thread's read
    __shared__ int s_ok;
    if (tid_() == 0) s_ok = ok;
    __syncthreads();
    ok = s_ok;
    __syncthreads();
    return ok != 0;
}

// Complete this workgroup's device-scope stores and bump counter `ctr` (the
// line of this workgroup). `drained`: every wave has already waited for its
// stores (and may have issued loads since, which must not delay the signal).
__device__ void block_signal(const Params& p, int ctr, bool drained = false) {
    if (p.perop || ctr < 0) {
        __syncthreads();
        return;
    }
    if (!drained) wait_stores();
    __syncthreads();
    if (tid_() == 0)
        __hip_atomic_fetch_add(p.ctr + ((int64_t)ctr * kCtrSub + (blockIdx.x & (kCtrSub - 1))) * kCtrStride, 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------ activation slices + norm

// RMSNorm gains for this lane's K positions (chunk c of lane l covers
// elements [8(l + 64c), +8)). Gains are weights: tiles load them before their
// dependency wait.
template <int NCH>
__device__ __forceinline__ void load_gain(uint4 (&g)[NCH], const uint16_t* gain, int K) {
    const int lane = tid_() & 63;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
        g[c] = ch < (K >> 3) ? ld16(gain + ch * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
}

// Each lane of each wave holds the activation values at the K positions its
// weight chunks cover. With `g` non-null applies RMSNorm:
// x / sqrt(mean(x^2) + eps) * gain, the mean as sum(x^2) * inv_k (inv_k =
// 1/K, a kernel argument, so no per-tile division is needed).
template <int NCH, int NB>
__device__ __forceinline__ void load_x_raw(float (&h)[NB][NCH][8], const float* x, int64_t stride, int nb, int K) {
    const int lane = tid_() & 63;
    const int K8 = K >> 3;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = lane + 64 * c;
            if (b < nb && ch < K8) {
                const float4 u = ldf4(x + b * stride + ch * 8), v = ldf4(x + b * stride + ch * 8 + 4);
                h[b][c][0] = u.x; h[b][c][1] = u.y; h[b][c][2] = u.z; h[b][c][3] = u.w;
                h[b][c][4] = v.x; h[b][c][5] = v.y; h[b][c][6] = v.z; h[b][c][7] = v.w;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) h[b][c][j] = 0.f;
            }
        }
}
// RMSNorm of loaded slices in place (gain g per this lane's positions).
template <int NCH, int NB>
__device__ __forceinline__ void norm_x(float (&h)[NB][NCH][8], int K, const uint4* g, float eps, float inv_k) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) ss = fmaf(h[b][c][j], h[b][c][j], ss);
        ss = wave_sum(ss);
        const float inv = 1.0f / sqrtf(ss * inv_k + eps);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint4 gw = g[c];
            const float gv[8] = {bflo(gw.x), bfhi(gw.x), bflo(gw.y), bfhi(gw.y),
                                 bflo(gw.z), bfhi(gw.z), bflo(gw.w), bfhi(gw.w)};
#pragma unroll
            for (int j = 0; j < 8; ++j) h[b][c][j] = (h[b][c][j] * inv) * gv[j];
        }
    }
}
template <int NCH, int NB>
__device__ __forceinline__ void load_x(float (&h)[NB][NCH][8], const float* x, int64_t stride, int nb,
                                       int K, const uint4* g, float eps, float inv_k) {
    load_x_raw<NCH, NB>(h, x, stride, nb, K);
    if (g != nullptr) {
        norm_x<NCH, NB>(h, K, g, eps, inv_k);
    } else {
        (void)eps;
        (void)inv_k;
    }
}

// ------------------------------------------------------- streaming GEMV

// Load one weight row slice for this lane: chunks lane + 64c of a row with
// K8 16-byte chunks. Branch-free: lanes past the row's end re-read its last
// chunk (already being fetched), so every call issues exactly NCH loads and
// the compiler can wait for each row precisely. Their activation slices are
// zero (load_x and the tiles' loaders zero them), so the duplicate finite
// weights add nothing to the dot products.
template <int NCH>
__device__ __forceinline__ void load_row(uint4 (&w)[NCH], const uint16_t* row, int K8) {
    const int lane = tid_() & 63;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
        w[c] = ld16s(row + (ch < K8 ? ch : K8 - 1) * 8);
    }
}

// The byte offsets of this lane's chunks in a row (the clamp of load_row),
// computed once per tile so that each further row costs one address add
// per chunk instead of recomputing the lane's chunk indices.
template <int NCH>
__device__ __forceinline__ void chunk_offsets(int (&off)[NCH], int K8) {
    const int lane = tid_() & 63;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
        off[c] = (ch < K8 ? ch : K8 - 1) * 16;
    }
}
template <int NCH>
__device__ __forceinline__ void load_row_at(uint4 (&w)[NCH], const uint16_t* row, const int (&off)[NCH]) {
    const char* r = reinterpret_cast<const char*>(row);
#pragma unroll
    for (int c = 0; c < NCH; ++c) w[c] = ld16s(r + off[c]);
}

// The wave-reduced dot products of the PF row-vectors in buf with the NB
// split activation slices. A row's products accumulate in a fixed order
// (chunks in order; within a chunk the four hi pairs, then the four lo
// pairs), one chain per (row, token); the chains are interleaved
// instruction by instruction, so consecutive dot-product instructions are
// independent, and the PF * NB reductions run together (wave_sum_n).
template <int NCH, int PF, int NB>
__device__ __forceinline__ void dot_rows(const uint4 (&buf)[PF][NCH], const uint32_t (&hx)[NB][NCH][8],
                                         float (&acc)[PF][NB]) {
    float a[PF * NB];
#pragma unroll
    for (int i = 0; i < PF * NB; ++i) a[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                const uint4 w = buf[s][c];
                const uint32_t wj = (j & 3) == 0 ? w.x : (j & 3) == 1 ? w.y : (j & 3) == 2 ? w.z : w.w;
#pragma unroll
                for (int b = 0; b < NB; ++b) a[s * NB + b] = dot2bf(wj, hx[b][c][j], a[s * NB + b]);
            }
    wave_sum_n<PF * NB>(a);
#pragma unroll
    for (int s = 0; s < PF; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[s][b] = a[s * NB + b];
}

// Row i0 + s of a group of PF rows is emitted by lane i0 + s, which picks
// that row's values out of acc (every lane holds all of them), so a group
// leaves in one store instruction per token instead of one per row.
// emit(i, v, vx): row i (= the lane), its values v and those of row i ^ 1
// (for tiles that pair adjacent rows).
template <int PF, int NB, class Emit>
__device__ __forceinline__ void lane_emit(int i0, int nmine, const float (&acc)[PF][NB], Emit& emit) {
    const int lane = tid_() & 63;
    const int s = lane - i0;
    float v[NB], vx[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float x = acc[0][b];
#pragma unroll
        for (int k = 1; k < PF; ++k) x = s == k ? acc[k][b] : x;
        v[b] = x;
        vx[b] = __shfl_xor(x, 1);
    }
    if (s >= 0 && s < PF && lane < nmine) emit(lane, v, vx);
}

// Wave-level streaming matrix-vector product over split activation slices hx
// (split_x) that the caller holds. The wave owns `nmine` row-vectors;
// rowptr(i) returns the i-th. The first PF rows are loaded before ready()
// runs (ready holds any dependency wait and may fill hx); then rows are
// consumed PF at a time (dot_rows), the next PF rows' loads issued before
// the results are emitted (lane_emit: row i by lane i, so a wave holds at
// most 64 rows). Loads are unconditional (slots past the last row re-read
// the last row, which is in flight already).
template <int NCH, int PF, int NB, class RowPtr, class Ready, class Emit>
__device__ __forceinline__ void gemv_rows(uint32_t (&hx)[NB][NCH][8], int nmine, int K8, RowPtr rowptr, Ready ready,
                                          Emit emit) {
    if (nmine <= 0) {
        ready();
        return;
    }
    uint4 buf[PF][NCH];
    const int last = nmine - 1;
    int off[NCH];
    chunk_offsets<NCH>(off, K8);
#pragma unroll
    for (int s = 0; s < PF; ++s) load_row_at<NCH>(buf[s], rowptr(s < last ? s : last), off);
    ready();
    for (int i0 = 0; i0 < nmine; i0 += PF) {
        float acc[PF][NB];
        dot_rows<NCH, PF, NB>(buf, hx, acc);
        if (i0 + PF < nmine) {
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                const int nx = i0 + PF + s;
                load_row_at<NCH>(buf[s], rowptr(nx < last ? nx : last), off);
            }
        }
        lane_emit<PF, NB>(i0, nmine, acc, emit);
    }
}

// Instruction-cache warm-up. A tile's code after its dependency wait has
// usually been evicted since the tile type last ran on this compute unit, so
// it would run on cold instruction fetches exactly when it is on the
// critical path. gemv_rows_warm runs the same instructions twice: pass 0
// before the wait on dummy activations (results dropped), pass 1 for real.
// ready(pass) fills hx: in pass 0 from a source that is not an exchange
// buffer (no early read may cache a line before its producer writes it), in
// pass 1 after the dependency wait. The pass loop is kept rolled so both
// passes execute one copy of the code.
template <int NCH, int PF, int NB, class RowPtr, class Ready, class Emit>
__device__ __forceinline__ void gemv_rows_warm(uint32_t (&hx)[NB][NCH][8], int nmine, int K8, RowPtr rowptr,
                                               Ready ready, Emit emit) {
    if (nmine <= 0) {
        ready(1);
        return;
    }
    uint4 buf[PF][NCH];
    const int last = nmine - 1;
    int off[NCH];
    chunk_offsets<NCH>(off, K8);
#pragma unroll
    for (int s = 0; s < PF; ++s) load_row_at<NCH>(buf[s], rowptr(s < last ? s : last), off);
#pragma clang loop unroll(disable)
    for (int pass = 0; pass < 2; ++pass) {
        ready(pass);
        for (int i0 = 0; i0 < nmine; i0 += PF) {
            float acc[PF][NB];
            dot_rows<NCH, PF, NB>(buf, hx, acc);
            if (pass == 0) break;   // the first PF rows are enough to warm the loop body
            if (i0 + PF < nmine) {
#pragma unroll
                for (int s = 0; s < PF; ++s) {
                    const int nx = i0 + PF + s;
                    load_row_at<NCH>(buf[s], rowptr(nx < last ? nx : last), off);
                }
            }
            lane_emit<PF, NB>(i0, nmine, acc, emit);
        }
    }
}

// The same with the activation slices owned here: ready(h) holds the
// dependency wait and fills the fp32 slices h, which are then split.
template <int NCH, int PF, int NB, class RowPtr, class Ready, class Emit>
__device__ __forceinline__ void gemv_stream(int nmine, int K8, RowPtr rowptr, Ready ready, Emit emit) {
    uint32_t hx[NB][NCH][8];
    gemv_rows<NCH, PF, NB>(
        hx, nmine, K8, rowptr,
        [&]() {
            float h[NB][NCH][8];
            ready(h);
            split_x<NB, NCH>(h, hx);
        },
        emit);
}

// ------------------------------------------------------------ routing

// Top-k per token and the active-expert slots, in LDS.
struct RouteLds {
    int32_t ids[kMaxBatch][kMaxTopK];
    float w[kMaxBatch][kMaxTopK];
    int32_t nslots;
    int32_t slot_e[kMaxSlots];         // expert of each slot, ascending ids
    int32_t slot_mask[kMaxSlots];      // tokens routed to the slot's expert
    int8_t slot_rank[kMaxSlots][kMaxBatch]; // rank of the expert in that token's top-k
    int32_t tag;                       // which layer's routing this holds (-1: none)
};

// Order-preserving map of a float to an unsigned key (larger float, larger
// key); no finite float or infinity maps to 0, which marks "no candidate".
__device__ __forceinline__ uint32_t fkey(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unkey(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

// Wave 0 computes, per token, the top-k experts (logit descending, expert id
// ascending on ties) by k rounds of a wave-wide maximum over order-preserving
// keys; the lowest id holding the maximum is found with ballots. Then the
// softmax over the selected logits (lane j holds the j-th), and the distinct
// selected experts in ascending id as slots, with each token's rank of the
// slot's expert. NE = experts per lane (E <= 64 NE). All logits of a token are
// requested at once (one memory round trip). Ends with a block barrier.
template <int NE>
__device__ __forceinline__ void compute_routing(const Params& p, const float* rl, RouteLds* r) {
    if (tid_() < 64) {
        const int lane = tid_();
        const int E = p.E, K = p.K;
        uint32_t chosen[NE], rank[NE];  // bit / byte b: token b chose expert lane + 64i, at that rank
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            chosen[i] = 0u;
            rank[i] = ~0u;
        }
        for (int b = 0; b < p.B; ++b) {
            float lv[NE];
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                const int e = lane + 64 * i;
                lv[i] = ld_dev(rl + b * E + (e < E ? e : E - 1));
            }
            uint32_t u[NE];  // 0: not a candidate (no float maps to 0)
#pragma unroll
            for (int i = 0; i < NE; ++i) u[i] = lane + 64 * i < E ? fkey(lv[i]) : 0u;
            uint32_t top = 0u;
            float sel = 0.f;  // lane j: the j-th selected logit
            int myid = 0;     // lane j: the j-th selected expert
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (j < K) {
                    uint32_t v = u[0];
#pragma unroll
                    for (int i = 1; i < NE; ++i) v = max(v, u[i]);
                    const uint32_t m = wave_max_u32(v);
                    int best = -1;
#pragma unroll
                    for (int i = NE - 1; i >= 0; --i) {
                        const uint64_t bal = __ballot(u[i] == m);
                        if (bal != 0ull) best = 64 * i + (int)__builtin_ctzll(bal);
                    }
                    if (j == 0) top = m;
                    if (lane == j) {
                        sel = unkey(m);
                        myid = best;
                    }
#pragma unroll
                    for (int i = 0; i < NE; ++i) {
                        if (64 * i + lane == best) {
                            u[i] = 0u;
                            chosen[i] |= 1u << b;
                            rank[i] = (rank[i] & ~(0xffu << (8 * b))) | ((uint32_t)j << (8 * b));
                        }
                    }
                }
            }
            // softmax over the selected logits (the first is the largest)
            const float ex = lane < K ? expf(sel - unkey(top)) : 0.f;
            const float sum = wave_sum(ex);
            if (lane < K) {
                r->ids[b][lane] = myid;
                r->w[b][lane] = ex / sum;
            }
        }
        // slots: selected experts in ascending id
        int base = 0;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const uint64_t m = __ballot(chosen[i] != 0u);
            if (chosen[i] != 0u) {
                const int slot = base + __popcll(m & ((1ull << lane) - 1ull));
                r->slot_e[slot] = lane + 64 * i;
                r->slot_mask[slot] = (int32_t)chosen[i];
#pragma unroll
                for (int b = 0; b < kMaxBatch; ++b) {
                    const uint32_t rk = (rank[i] >> (8 * b)) & 0xffu;
                    r->slot_rank[slot][b] = (int8_t)(rk == 0xffu ? -1 : (int)rk);
                }
            }
            base += __popcll(m);
        }
        if (lane == 0) {
            r->nslots = base;
            r->tag = (int32_t)(rl - p.rlogits);
        }
    }
    __syncthreads();
}

// The routing of the layer whose router logits start at rl, computed here
// unless this workgroup's LDS already holds it (an expert tile of the same
// layer ran just before; LDS persists across the tasks of a workgroup, and
// the tag is cleared when the kernel starts).
template <int NE>
__device__ __forceinline__ void routing_for(const Params& p, const float* rl, RouteLds* r) {
    if (r->tag != (int32_t)(rl - p.rlogits)) compute_routing<NE>(p, rl, r);
}

}  // namespace mk
