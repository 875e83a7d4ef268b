// mk_kernels.h -- host-side entry points into the device code.
#pragma once

#include <hip/hip_runtime.h>

#include "mk_common.h"

namespace mk {

constexpr int kThreads = 256;   // workgroup size of every kernel

// Kernels are compiled per model shape: the number of 16-byte chunks per lane
// per row for the hidden size, the attention width and the expert width, the
// head size and the router logits per lane. Returns -1 if no build matches.
int find_shape(int hidden, int attn_width, int moe_inter, int head_dim, int n_experts);

struct KernelPair {
    const void* persistent;  // (Params, int general)
    const void* perop;       // (Params, int general, int first)
};
// nb = 1, 2: the one- and two-token builds; nb = 0: the build for batches of
// 3 to kMaxBatchMM tokens.
bool get_kernels(int shape, int nb, KernelPair* out);

hipError_t set_kernel_attributes(const KernelPair& k, size_t lds_bytes);
hipError_t persistent_occupancy(const KernelPair& k, size_t lds_bytes, int* blocks_per_cu);
hipError_t launch_persistent(const KernelPair& k, const Params& p, int general, size_t lds_bytes, int n_wg,
                             hipStream_t stream);
hipError_t launch_perop_level(const KernelPair& k, const Params& p, int general, size_t lds_bytes, int first,
                              int count, hipStream_t stream);
hipError_t launch_fill(uint32_t* dst, int64_t n, uint32_t v, hipStream_t stream);

// The library's static device scratch (mk_decode_step_noalloc): its size, and
// its device address on `device` (looked up once per device, then cached).
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_address(int device, void** out);

}  // namespace mk
