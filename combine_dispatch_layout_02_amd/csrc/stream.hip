// stream.hip -- streaming kernels for measurement on gfx950 (ep_stream): the
// box's read, write and copy ceilings, and the clean flush of the 256 MB
// memory-side cache that cold-cache timings start from.
//
// A buffer of `bytes` is walked in whole chunks of `chunk` bytes (a multiple
// of 1 KiB); wave w of the grid takes chunks w, w + waves, w + 2 waves, ...;
// inside a chunk lane l moves the 16-byte vectors l, l + 64, l + 128, ...,
// so every wave instruction covers 1 KiB of contiguous memory.  Loads are
// issued in batches of 8 per lane before they are used.
//   read : XOR of every vector read; the 16-byte sink is written only when
//          the XOR equals a fixed value (so the loads cannot be dropped).
//   write: a fixed pattern.
//   copy : dst = src.
// Plain (write-back) or non-temporal loads / stores.  Measured on MI355X:
// plain stores leave dirty lines in the memory-side cache, written back to
// HBM when something evicts them; non-temporal stores leave none; a plain
// read of 512 MiB evicts everything the cache held (writing back what was
// dirty) and leaves it clean.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

struct StreamArgs {
    const char *src;
    char *dst;
    int64_t chunk;     // bytes per chunk (multiple of 1024)
    int64_t nchunks;
};

template <bool NT>
__device__ __forceinline__ vec16 sload(const char *p) {
    return NT ? ld16_nt(p) : ld16(p);
}
template <bool NT>
__device__ __forceinline__ void sstore(char *p, vec16 v) {
    if (NT) st16_nt(p, v); else st16(p, v);
}

// KIND 0 read, 1 write, 2 copy
template <int KIND, bool NT>
__global__ __launch_bounds__(256) void ep_stream_kernel(StreamArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w0 = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int64_t nw = (int64_t)gridDim.x * 4;
    const int per = (int)(a.chunk / 1024);   // vectors per lane in a chunk
    vec16 acc = {0u, 0u, 0u, 0u};
    for (int64_t c = w0; c < a.nchunks; c += nw) {
        const int64_t base = c * a.chunk + lane * 16;
        if (KIND == 1) {
            const vec16 v = {0x5A5A5A5Au, (uint32_t)c, (uint32_t)lane, 0xA5A5A5A5u};
            for (int i = 0; i < per; ++i) sstore<NT>(a.dst + base + (int64_t)i * 1024, v);
            continue;
        }
        for (int i0 = 0; i0 < per; i0 += 8) {
            vec16 b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)   // clamped: every load of the batch is issued
                b[i] = sload<NT>(a.src + base + (int64_t)min(i0 + i, per - 1) * 1024);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i0 + i >= per) continue;
                if (KIND == 0) acc ^= b[i];
                else sstore<NT>(a.dst + base + (int64_t)(i0 + i) * 1024, b[i]);
            }
        }
    }
    if (KIND == 0 && acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0x94D049BBu)
        st16(a.dst, acc);
}

template <int KIND>
void launch_kind(bool nt, const StreamArgs &a, unsigned blocks, hipStream_t stream) {
    if (nt) hipLaunchKernelGGL((ep_stream_kernel<KIND, true>), dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((ep_stream_kernel<KIND, false>), dim3(blocks), dim3(256), 0, stream, a);
}

}  // namespace

hipError_t launch_stream(int kind, bool nt, const void *src, void *dst, size_t bytes, size_t chunk, int waves,
                         hipStream_t stream) {
    StreamArgs a{};
    a.src = static_cast<const char *>(src);
    a.dst = static_cast<char *>(dst);
    a.chunk = (int64_t)chunk;
    a.nchunks = (int64_t)(bytes / chunk);
    if (a.nchunks == 0) return hipSuccess;
    const unsigned blocks = (unsigned)(waves / 4);
    if (kind == 0) launch_kind<0>(nt, a, blocks, stream);
    else if (kind == 1) launch_kind<1>(nt, a, blocks, stream);
    else launch_kind<2>(nt, a, blocks, stream);
    return hipGetLastError();
}

}  // namespace ep
