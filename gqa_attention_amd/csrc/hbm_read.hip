// hbm_read.hip -- a plain streaming read of device memory, the calibration of the decode's
// bandwidth ceiling: the decode sweep reads each cached K/V byte once, so the rate at
// which a kernel that does nothing else reads the same number of bytes, in one launch of
// the same shape (one workgroup of 512 threads per compute unit), bounds what the sweep
// can reach on this device.
//
// Each thread keeps eight independent 16-byte loads in flight (all issued before any is
// used), striding over the buffer by the whole grid; the loaded words are folded into a
// per-thread XOR that is stored only if it equals a value passed at launch (which the
// compiler cannot foresee), so the loads stay; the store, if it ever happens, writes one
// word of the sink per workgroup.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kReadUnroll = 8;
constexpr int kReadThreads = 512;
constexpr int kReadBlocks = 256;

__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const u32x4 *__restrict__ p,
                                                                size_t n16, uint32_t *sink,
                                                                uint32_t magic) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (size_t base = tid; base < n16; base += stride * kReadUnroll) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const size_t i = base + (size_t)u * stride;
            v[u] = i < n16 ? p[i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == magic) sink[blockIdx.x] = acc;
}

}  // namespace

int hbm_read_blocks() { return kReadBlocks; }

hipError_t launch_hbm_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    hipLaunchKernelGGL(hbm_read_kernel, dim3(kReadBlocks), dim3(kReadThreads), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, sink, 0x9E3779B9u);
    return hipGetLastError();
}

}  // namespace gqa
