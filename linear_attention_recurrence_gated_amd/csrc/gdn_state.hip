// gdn_state.hip -- set and reset recurrent states.
//
// The state exists before the first token ("attention and memory",
// stethem.com, "Sources, assumptions & limits"), and a runtime needs batch and
// reset rules for it ("Hybrid · kết hợp nhiều cơ chế..." (openarchlab.com),
// section 3).  Both kernels are plain grid-stride float4 streams.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

// Four float4 per lane per pass, a pass of 1,024 float4 per workgroup: a copy
// streams fastest on this chip with a few 16-byte accesses in flight per lane
// and many workgroups (measured on a 403 MiB copy: 6.5 TB/s, against 5.75 for
// one float4 per lane).  NT: non-temporal accesses, for large fills.
template <bool NT>
__global__ __launch_bounds__(256) void k_state_fill(float4 *__restrict__ dst, const float4 *__restrict__ src,
                                                    int64_t n4) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int64_t stride = (int64_t)gridDim.x * 1024;
    for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n4; base += stride) {
        f4v x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + 256 * u;
            if (i < n4) {
                const f4v *p = reinterpret_cast<const f4v *>(src + i);
                x[u] = !src ? f4v{0.f, 0.f, 0.f, 0.f} : NT ? __builtin_nontemporal_load(p) : *p;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + 256 * u;
            if (i < n4) {
                f4v *p = reinterpret_cast<f4v *>(dst + i);
                if (NT) __builtin_nontemporal_store(x[u], p); else *p = x[u];
            }
        }
    }
}

// grid.y walks the slot list; grid.x strides over one state block.
__global__ __launch_bounds__(256) void k_state_reset_slots(float4 *__restrict__ state,
                                                           const int32_t *__restrict__ slots, int64_t n_blocks,
                                                           int64_t block4) {
    const int32_t s = slots[blockIdx.y];
    if (s < 0 || s >= n_blocks) return;
    float4 *dst = state + (int64_t)s * block4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < block4; i += stride)
        dst[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

static unsigned grid_for(int64_t n4) {
    const int64_t want = (n4 + 1023) / 1024;
    return (unsigned)(want < 16384 ? (want > 0 ? want : 1) : 16384);
}

hipError_t launch_state_fill(float *state, const float *init, int64_t n_floats, hipStream_t stream) {
    if (n_floats == 0 || init == state) return hipSuccess;
    const int64_t n4 = n_floats / 4;  // every supported state block is a multiple of 16 floats
    if (n_floats * 4 >= (int64_t(32) << 20))
        hipLaunchKernelGGL(k_state_fill<true>, dim3(grid_for(n4)), dim3(256), 0, stream, (float4 *)state,
                           (const float4 *)init, n4);
    else
        hipLaunchKernelGGL(k_state_fill<false>, dim3(grid_for(n4)), dim3(256), 0, stream, (float4 *)state,
                           (const float4 *)init, n4);
    return hipGetLastError();
}

hipError_t launch_state_reset_slots(float *state, const int32_t *slots, int32_t n_slots, int64_t n_blocks,
                                    int64_t block_floats, hipStream_t stream) {
    if (n_slots == 0 || n_blocks == 0) return hipSuccess;
    const int64_t block4 = block_floats / 4;
    int64_t gx = (block4 + 255) / 256;
    if (gx > 1024) gx = 1024;
    hipLaunchKernelGGL(k_state_reset_slots, dim3((unsigned)gx, (unsigned)n_slots), dim3(256), 0, stream,
                       (float4 *)state, slots, n_blocks, block4);
    return hipGetLastError();
}

hipError_t record_mark(hipEvent_t ev, hipStream_t stream) {
    return ev ? hipEventRecord(ev, stream) : hipSuccess;
}

}  // namespace gdn
