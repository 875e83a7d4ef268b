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
    const int beg = p.wg_off[blockIdx.x], end = p.wg_off[blockIdx.x + 1];
    for (int i = beg; i < end; ++i) {
        const Task t = p.tasks[i];
        if (!run_task<S, NB>(t, i + 1 < end ? &p.tasks[i + 1] : nullptr, p, lds, general, i)) break;
        __syncthreads();
    }
}

template <class S, int NB>
__global__ void __launch_bounds__(NT, 2) k_perop(Params p, int general, int first) {
    extern __shared__ __align__(16) char lds[];
    const int i = first + blockIdx.x;
    const Task t = p.tasks[i];
    __syncthreads();
    run_task<S, NB>(t, nullptr, p, lds, general, i);
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
    } else {
        out->persistent = reinterpret_cast<const void*>(&k_persistent<S, 2>);
        out->perop = reinterpret_cast<const void*>(&k_perop<S, 2>);
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
    if (nb < 0 || nb > kMaxBatchValu) return false;
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
    const int blocks = (int)(n + 255) / 256 < 1024 ? (int)((n + 255) / 256) : 1024;
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

}  // namespace mk
