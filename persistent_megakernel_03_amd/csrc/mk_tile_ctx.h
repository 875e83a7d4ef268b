// mk_tile_ctx.h -- what every tile function shares: the LDS map, the tile
// context passed through the dispatcher, trace stamps, and the per-layer
// slices of the exchange buffers.
#pragma once

#include "mk_device.h"

namespace mk {

// LDS layout (dynamic shared memory), byte offsets.
//   [0, kLdsRoute)            general region: attention scores/probabilities
//                             and combine coefficients, or the down tile's
//                             staged expert activations and outputs
//   [kLdsRoute, +kLdsRouteSz) routing results
//   then 512 bytes of per-tile scalars
constexpr int kLdsRouteSz = 1024;
constexpr int kMaxDownRows = 64;

struct LdsMap {
    int route;  // offset of RouteLds
    int misc;   // offset of scalars
};

__device__ __forceinline__ RouteLds* route_lds(char* lds, int general_bytes) {
    return reinterpret_cast<RouteLds*>(lds + general_bytes);
}
__device__ __forceinline__ int* misc_lds(char* lds, int general_bytes) {
    return reinterpret_cast<int*>(lds + general_bytes + kLdsRouteSz);
}

struct TileCtx {
    const Params& p;
    char* lds;
    int general;      // bytes of the general LDS region
    uint64_t* t_wait; // trace: when the compute wait ended
    uint64_t* marks;  // trace: four phase stamps inside the tile
};

// Trace stamp k (0..3) of the current tile (thread 0, tracing on).
__device__ __forceinline__ void mark(TileCtx& cx, int k) {
    if (cx.p.trace_on && tid_() == 0) cx.marks[k] = wall_clock64();
}

// Per-layer slices of the exchange buffers, each padded to 256 bytes.
__device__ __forceinline__ float* x_at(const Params& p, int idx) {
    return p.x + (int64_t)idx * pad64((int64_t)p.max_batch * p.H);
}
__device__ __forceinline__ float* qkv_at(const Params& p, int l) {
    return p.qkv + (int64_t)l * pad64((int64_t)p.max_batch * p.QKVD);
}
__device__ __forceinline__ float* part_at(const Params& p, int l) {
    return p.att_part + (int64_t)l * pad64((int64_t)p.max_batch * p.Hq * p.max_chunks * p.D);
}
// (max, sum) pairs: one padded row of max_chunks pairs per (sequence, head)
__device__ __forceinline__ int64_t ml_row(const Params& p) { return pad64(2 * (int64_t)p.max_chunks); }
__device__ __forceinline__ float* ml_at(const Params& p, int l) {
    return p.att_ml + (int64_t)l * p.max_batch * p.Hq * ml_row(p);
}
__device__ __forceinline__ float* attout_at(const Params& p, int l) {
    return p.att_out + (int64_t)l * pad64((int64_t)p.max_batch * p.Hq * p.D);
}
__device__ __forceinline__ float* rlogits_at(const Params& p, int l) {
    return p.rlogits + (int64_t)l * pad64((int64_t)p.max_batch * p.E);
}
__device__ __forceinline__ float* act_at(const Params& p, int l) {
    return p.act + (int64_t)l * pad64((int64_t)p.max_batch * p.K * p.I);
}

}  // namespace mk
