// Read-stream calibration kernel: the practical HBM read ceiling of the GPU
// for a given byte count, reached with the access pattern of the row streams
// (one wavefront per job of 64 lanes x 8 x 16 bytes, non-temporal 16-byte
// loads) and no arithmetic beyond a XOR fold.  It is a measuring stick for
// the verify kernels, not a step of the method.
#include <hip/hip_runtime.h>

#include "sv_common.hpp"
#include "sv_device.hpp"

namespace sv {

constexpr int kStreamNV = 8;                       // vectors per lane per job
constexpr int kStreamJobVecs = kWave * kStreamNV;  // 512 vectors = 8 KB per job

// The fold is stored only when it equals a fixed word, which keeps the loads
// alive without a store per wave.
constexpr uint32_t kStreamMagic = 0x9e3779b9u;

__global__ __launch_bounds__(kBlock) void k_read_stream(const char *buf, int64_t n_vec, uint32_t *sink) {
    const int64_t job = int64_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t v0 = job * kStreamJobVecs;
    if (v0 >= n_vec) return;
    u32x4 d[kStreamNV];
    if (v0 + kStreamJobVecs <= n_vec) {
#pragma unroll
        for (int n = 0; n < kStreamNV; ++n) d[n] = load16(buf + (v0 + n * kWave + lane) * 16);
    } else {
#pragma unroll
        for (int n = 0; n < kStreamNV; ++n) {
            const int64_t v = v0 + n * kWave + lane;
            d[n] = (v < n_vec) ? load16(buf + v * 16) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t x = 0;
#pragma unroll
    for (int n = 0; n < kStreamNV; ++n) x ^= d[n][0] ^ d[n][1] ^ d[n][2] ^ d[n][3];
    if (x == kStreamMagic) sink[0] = x;
}

}  // namespace sv

using namespace sv;

extern "C" sv_status sv_read_stream(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream,
                                    hipEvent_t kernel_start, hipEvent_t kernel_stop) {
    if (buf == nullptr || sink == nullptr || bytes == 0 || (bytes % 16) != 0 || !aligned16(buf))
        return SV_EINVAL;
    const int64_t n_vec = static_cast<int64_t>(bytes / 16);
    const int64_t jobs = (n_vec + kStreamJobVecs - 1) / kStreamJobVecs;
    const int64_t blocks = (jobs + kWaves - 1) / kWaves;
    if (blocks > 0x7fffffff) return SV_EINVAL;
    launch_timed(k_read_stream, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream, kernel_start,
                 kernel_stop, static_cast<const char *>(buf), n_vec, sink);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}
