// mk_kernels.hip -- the persistent megakernel, the per-op kernel, and their
// launch helpers.
//
// Persistent mode: one cooperative launch per step, grid = compute units x
// workgroups per CU, all co-resident for the whole step; each workgroup walks
// its task list and synchronises through counters in global memory ("Cohere
// Publishes One-Kernel Server for North Mini Code, Claims 1.58x vLLM
// Speedup", section "One resident program, many small tasks").
//
// Per-op mode: one launch per operation level over the same tiles; the
// stream's kernel boundaries are the only synchronisation -- the conventional
// pipeline the pages compare against (same page, section "The delay is
// between operations").
#include <mutex>

#include "mk_kernels.h"
#include "mk_tiles.h"

namespace mk {

template <class S, int NB>
__global__ void __launch_bounds__(NT, 2) k_persistent(Params p, int general) {
    extern __shared__ __align__(16) char lds[];
    // Clear the counter bank the next step will use (disjoint slice per workgroup).
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < p.bank_words; i += (int64_t)gridDim.x * NT)
        p.ctr_other[i] = 0u;
    __syncthreads();
    // The list is walked in order. A claim task stands for the tiles of one
    // level held in a shared pool: the workgroup takes pool positions from
    // the level's claim counter (one atomic per tile, largest tiles first)
    // and runs them until the pool is exhausted, so the tiles of an
    // irregular level go to whichever workgroups are free first. Claimed
    // tiles wait only on lower levels and every list is in level order, so
    // the lowest unfinished tile can always run. One call site of run_task
    // keeps the tile code inlined once.
    __shared__ int s_pos;
    if (threadIdx.x == 0) route_lds(lds, general)->tag = -1;   // no routing held yet
    const int beg = p.wg_off[blockIdx.x], end = p.wg_off[blockIdx.x + 1];
    int i = beg;
    int claim = -1;   // list position of the claim task being drained
    for (;;) {
        int ti;
        if (claim < 0) {
            if (i >= end) break;
            if (p.tasks[i].op == OP_CLAIM) {
                claim = i;
                if (p.trace_on && tid_() == 0) p.trace[(int64_t)i * 8 + 1] = wall_clock64();
            }
        }
        if (claim >= 0) {
            const Task ct = p.tasks[claim];
            if (tid_() == 0)
                s_pos = (int)__hip_atomic_fetch_add(p.ctr + p.cl.claim_word(ct.a2), 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const int j = s_pos;
            __syncthreads();
            if (j >= ct.a1) {
                if (p.trace_on && tid_() == 0) {
                    uint64_t* rec = p.trace + (int64_t)claim * 8;
                    rec[0] = (uint64_t)(uint32_t)claim | ((uint64_t)blockIdx.x << 32);
                    rec[2] = rec[1];
                    rec[3] = rec[4] = rec[5] = rec[6] = 0;
                    rec[7] = wall_clock64();
                }
                claim = -1;
                ++i;
                continue;
            }
            ti = ct.a0 + j;
        } else {
            ti = i;
        }
        const Task t = p.tasks[ti];
        if (!run_task<S, NB>(t, p, lds, general, ti)) break;
        if (claim < 0) ++i;
        __syncthreads();
    }
}

template <class S, int NB>
__global__ void __launch_bounds__(NT, 2) k_perop(Params p, int general, int first) {
    extern __shared__ __align__(16) char lds[];
    const int i = first + blockIdx.x;
    const Task t = p.tasks[i];
    if (threadIdx.x == 0) route_lds(lds, general)->tag = -1;
    __syncthreads();
    run_task<S, NB>(t, p, lds, general, i);
}

// Device scratch of mk_decode_step_noalloc: the step's counters and exchange
// buffers for callers that cannot allocate. In host code `scratch` names a
// host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(int device, void** out) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        int prev = 0;
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess) return e;
        if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev != device) (void)hipSetDevice(prev);
        if (e != hipSuccess) return e;
        addr[device] = p;
    }
    *out = addr[device];
    return hipSuccess;
}

__global__ void k_fill_u32(uint32_t* dst, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = v;
}

// Supported shapes: {NCH_H, NCH_O, NCH_I, D, NCHP_I, NE}.
typedef Shape<1, 1, 1, 64, 1, 1> ShapeSmall;  // e.g. hidden 256, 4x64 heads, expert width 128, 8 experts
typedef Shape<4, 8, 2, 128, 3, 2> ShapeA3B;   // hidden 2048, 32x128 heads, expert width 768, 128 experts

namespace {
constexpr int kKey = 6;
const int kShapes[][kKey] = {{1, 1, 1, 64, 1, 1}, {4, 8, 2, 128, 3, 2}};

template <class S>
void fill_pair(int nb, KernelPair* out) {
    if (nb == 0) {
        out->persistent = reinterpret_cast<const void*>(&k_persistent<S, 0>);
        out->perop = reinterpret_cast<const void*>(&k_perop<S, 0>);
    } else if (nb == 1) {
        out->persistent = reinterpret_cast<const void*>(&k_persistent<S, 1>);
        out->perop = reinterpret_cast<const void*>(&k_perop<S, 1>);
    } else if (nb == 2) {
        out->persistent = reinterpret_cast<const void*>(&k_persistent<S, 2>);
        out->perop = reinterpret_cast<const void*>(&k_perop<S, 2>);
    } else {
        out->persistent = reinterpret_cast<const void*>(&k_persistent<S, kNbMmWide>);
        out->perop = reinterpret_cast<const void*>(&k_perop<S, kNbMmWide>);
    }
}
}  // namespace

int find_shape(int hidden, int attn_width, int moe_inter, int head_dim, int n_experts) {
    const int key[kKey] = {(hidden + 511) / 512, (attn_width + 511) / 512, (moe_inter + 511) / 512, head_dim,
                           (moe_inter + 255) / 256, (n_experts + 63) / 64};
    for (int i = 0; i < (int)(sizeof(kShapes) / sizeof(kShapes[0])); ++i) {
        bool same = true;
        for (int j = 0; j < kKey; ++j) same = same && key[j] == kShapes[i][j];
        if (same) return i;
    }
    return -1;
}

bool get_kernels(int shape, int nb, KernelPair* out) {
    if (nb < 0 || nb >= kNbCount) return false;
    switch (shape) {
        case 0: fill_pair<ShapeSmall>(nb, out); return true;
        case 1: fill_pair<ShapeA3B>(nb, out); return true;
        default: return false;
    }
}

hipError_t set_kernel_attributes(const KernelPair& k, size_t lds_bytes) {
    hipError_t e = hipFuncSetAttribute(k.persistent, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(k.perop, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
}

hipError_t persistent_occupancy(const KernelPair& k, size_t lds_bytes, int* blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k.persistent, NT, lds_bytes);
}

hipError_t launch_persistent(const KernelPair& k, const Params& p, int general, size_t lds_bytes, int n_wg,
                             hipStream_t stream) {
    Params pc = p;
    int gen = general;
    void* args[] = {&pc, &gen};
    return hipLaunchCooperativeKernel(k.persistent, dim3(n_wg), dim3(NT), args, (unsigned)lds_bytes, stream);
}

hipError_t launch_perop_level(const KernelPair& k, const Params& p, int general, size_t lds_bytes, int first,
                              int count, hipStream_t stream) {
    Params pc = p;
    int gen = general, fst = first;
    void* args[] = {&pc, &gen, &fst};
    return hipLaunchKernel(k.perop, dim3(count), dim3(NT), args, lds_bytes, stream);
}

hipError_t launch_fill(uint32_t* dst, int64_t n, uint32_t v, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t need = (n + 255) / 256;
    const int blocks = need < 1024 ? (int)need : 1024;
    hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, stream, dst, n, v);
    return hipGetLastError();
}

template __global__ void k_persistent<ShapeSmall, 0>(Params, int);
template __global__ void k_persistent<ShapeA3B, 0>(Params, int);
template __global__ void k_perop<ShapeSmall, 0>(Params, int, int);
template __global__ void k_perop<ShapeA3B, 0>(Params, int, int);
template __global__ void k_persistent<ShapeSmall, 1>(Params, int);
template __global__ void k_persistent<ShapeSmall, 2>(Params, int);
template __global__ void k_persistent<ShapeA3B, 1>(Params, int);
template __global__ void k_persistent<ShapeA3B, 2>(Params, int);
template __global__ void k_perop<ShapeSmall, 1>(Params, int, int);
template __global__ void k_perop<ShapeSmall, 2>(Params, int, int);
template __global__ void k_perop<ShapeA3B, 1>(Params, int, int);
template __global__ void k_perop<ShapeA3B, 2>(Params, int, int);
template __global__ void k_persistent<ShapeSmall, kNbMmWide>(Params, int);
template __global__ void k_persistent<ShapeA3B, kNbMmWide>(Params, int);
template __global__ void k_perop<ShapeSmall, kNbMmWide>(Params, int, int);
template __global__ void k_perop<ShapeA3B, kNbMmWide>(Params, int, int);

}  // namespace mk
