// A streaming-read kernel: the device's practical HBM read bandwidth, measured the way the
// tiled GEMV reads its head, for reporting beside the GEMV (dh_stream_read in dh.h).
//
// Each wave reads 4 KiB segments (four 1 KiB loads, lane l at 16 l, with the non-temporal
// hint) over a persistent grid of one 512-thread workgroup per compute unit, so about 32 KiB
// are in flight per compute unit: the configuration that streamed fastest in a sweep of
// loads in flight, workgroup sizes and grids on MI355X.  Every 32-bit word is added once into
// a per-wave sum (mod 2^32), so the sums prove that each byte was read exactly once.
#include "dh_internal.h"
#include "launch.h"

namespace dh {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeLoads = 4;           // 1 KiB loads a wave has in flight
constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer: 32-bit data format
constexpr int kCacheNT = 2;              // gfx950 cache policy bit 1: non-temporal

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void stream_read(const uint8_t *buf,
                                                             int64_t segments, uint32_t *sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kProbeThreads) >> 6;
    uint32_t sum = 0;
    for (int64_t s = wave; s < segments; s += nwaves) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(buf + s * (1024 * kProbeLoads)), (short)0, 1024 * kProbeLoads, kRsrcWord3);
        u32x4 v[kProbeLoads];
#pragma unroll
        for (int u = 0; u < kProbeLoads; u++)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, 1024 * u, kCacheNT);
#pragma unroll
        for (int u = 0; u < kProbeLoads; u++)
            sum += v[u].x + v[u].y + v[u].z + v[u].w;
    }
    for (int o = 32; o > 0; o >>= 1)
        sum += __shfl_xor(sum, o);
    if (lane == 0)
        sink[wave] = sum;
    // the sink words past the launch's waves are zeroed, so the whole sink sums to the buffer
    if (blockIdx.x == 0)
        for (int64_t i = nwaves + threadIdx.x; i < DH_STREAM_SINK_WORDS; i += kProbeThreads)
            sink[i] = 0;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink,
                              hipStream_t stream)
{
    const int64_t segments = (int64_t)(bytes / (1024 * kProbeLoads));
    int grid = device_cus();
    const int max_grid = DH_STREAM_SINK_WORDS / (kProbeThreads / kWave);
    grid = grid < max_grid ? grid : max_grid;
    return launch(stream_read, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                  static_cast<const uint8_t *>(buf), segments, sink);
}

}  // namespace dh
