// quant.hip -- payload conversion, the workloads' expert stage, and two small
// utility kernels (workspace fill, calibration copy), all for gfx950.
//
// Formats (MORI-EP Benchmark, reference script: fp8 rows carry one byte per
// element plus one fp32 scale per 128 elements; MoE-EP Benchmark README,
// MEGA_COMBINE_DTYPE: mxfp8 is 32 e4m3 elements sharing one e8m0 scale).
// The rounding rules the pages leave open are fixed here:
//   fp8 rows : scale = amax / 448 (IEEE division; 1 for an all-zero group),
//              q = e4m3_rne_sat(x / scale)
//   mxfp8    : X = clamp(floor(log2 amax) - 8, -127, 127) (OCP Microscaling
//              shared exponent; -127 for an all-zero group),
//              q = e4m3_rne_sat(v * 2^-X), scale byte X + 127
// These kernels are bandwidth-light helpers; the divisions are the compiler's
// correctly rounded fp32 division.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

// One 16-lane segment per 128-element group: each lane holds 8 bf16.
__global__ __launch_bounds__(256) void ep_quant_fp8_kernel(const uint16_t *x, uint8_t *q,
                                                           float *scales, int64_t groups) {
    const int64_t gidx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 16;
    const int sl = threadIdx.x & 15;
    const bool live = gidx < groups;
    vec16 v = {0u, 0u, 0u, 0u};
    if (live) v = ld16(x + gidx * 128 + sl * 8);
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(v[i]);
        f[2 * i + 1] = bf16_hi(v[i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (!live) return;
    const float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo |= f32_to_e4m3(f[i] / scale) << (8 * i);
        hi |= f32_to_e4m3(f[4 + i] / scale) << (8 * i);
    }
    uint2 packed;
    packed.x = lo;
    packed.y = hi;
    *reinterpret_cast<uint2 *>(q + gidx * 128 + sl * 8) = packed;
    if (sl == 0) scales[gidx] = scale;
}

// Expert of receive row s: the e with expert_offset[e] <= s < expert_offset[e+1]
// (upper bound search; empty segments are skipped naturally).
__device__ int expert_of_row(const int32_t *off, int E, int64_t s) {
    int lo = 0, hi = E;   // invariant: off[lo] <= s < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= s) lo = mid; else hi = mid;
    }
    return lo;
}

// out[s] = bf16(f32(recv[s]) * factor[e(s)]); one wave per (row, 512 elements).
__global__ __launch_bounds__(256) void ep_expert_scale_kernel(const int32_t *off, int E, int H,
                                                              int64_t rows_cap, const float *factor,
                                                              const uint16_t *recv, uint16_t *out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int parts = (H + 511) / 512;
    const int64_t gw = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int64_t s = gw / parts;
    const int part = (int)(gw - s * parts);
    if (s >= rows_cap || s >= off[E]) return;
    const float f = factor[expert_of_row(off, E, s)];
    const int h = part * 512 + lane * 8;
    if (h >= H) return;
    const vec16 v = ld16(recv + s * H + h);
    vec16 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(bf16_lo(v[q]) * f, bf16_hi(v[q]) * f);
    st16(out + s * H + h, o);
}

// mxfp8 re-encode of dequantized fp8 rows; a lane holds 16 elements, lane
// pairs form one 32-element group.  One wave per (row, 1024 elements).
__global__ __launch_bounds__(256) void ep_expert_requant_kernel(const int32_t *off, int E, int H,
                                                                int64_t rows_cap,
                                                                const float *factor,
                                                                const uint8_t *rq,
                                                                const float *rscale,
                                                                uint8_t *oq, uint8_t *oe) {
    const int lane = threadIdx.x & (kWave - 1);
    const int parts = (H + 1023) / 1024;
    const int64_t gw = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int64_t s = gw / parts;
    const int part = (int)(gw - s * parts);
    if (s >= rows_cap || s >= off[E]) return;   // wave-uniform
    const float f = factor ? factor[expert_of_row(off, E, s)] : 1.0f;
    const int h = part * 1024 + lane * 16;
    const bool live = h < H;                    // H % 128 == 0: both lanes of a pair agree
    float v[16];
    float amax = 0.0f;
    if (live) {
        const vec16 b = ld16(rq + s * H + h);
        const float sc = rscale[s * (H / 128) + h / 128];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = e4m3_to_f32((b[q] >> (8 * i)) & 0xFFu) * sc;
                if (factor) x = x * f;
                v[4 * q + i] = x;
                amax = fmaxf(amax, fabsf(x));
            }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    if (!live) return;
    const int X = (amax == 0.0f) ? -127 : mx_shared_exp(amax);
    const float p = pow2_neg(X);
    vec16 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= f32_to_e4m3(v[4 * q + i] * p) << (8 * i);
        o[q] = w;
    }
    st16(oq + s * H + h, o);
    if ((lane & 1) == 0) oe[s * (H / 32) + h / 32] = (uint8_t)(X + 127);
}

// nvfp4 re-encode of bf16 rows: a lane holds one 16-element group (two
// 16-byte loads); one wave per (row, 1024 elements).
__global__ __launch_bounds__(256) void ep_expert_requant_nvfp4_kernel(const int32_t *off, int E, int H,
                                                                      int64_t rows_cap,
                                                                      const float *factor,
                                                                      const uint16_t *recv,
                                                                      uint8_t *oq, uint16_t *os) {
    const int lane = threadIdx.x & (kWave - 1);
    const int parts = (H + 1023) / 1024;
    const int64_t gw = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int64_t s = gw / parts;
    const int part = (int)(gw - s * parts);
    if (s >= rows_cap || s >= off[E]) return;   // wave-uniform
    const int h = part * 1024 + lane * 16;
    if (h >= H) return;
    const float f = factor ? factor[expert_of_row(off, E, s)] : 1.0f;
    const vec16 b0 = ld16(recv + s * H + h), b1 = ld16(recv + s * H + h + 8);
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[2 * q] = bf16_lo(b0[q]);
        v[2 * q + 1] = bf16_hi(b0[q]);
        v[8 + 2 * q] = bf16_lo(b1[q]);
        v[8 + 2 * q + 1] = bf16_hi(b1[q]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (factor) v[i] = v[i] * f;
        amax = fmaxf(amax, fabsf(v[i]));
    }
    uint32_t sb = f32_to_bf16(amax / 6.0f);
    if ((sb & 0x7FFFu) == 0u) sb = 0x3F80u;   // zero scale -> 1.0
    const float sf = u2f(sb << 16);
    uint2 packed = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t byte = f32_to_e2m1(v[2 * i] / sf) | (f32_to_e2m1(v[2 * i + 1] / sf) << 4);
        if (i < 4) packed.x |= byte << (8 * i); else packed.y |= byte << (8 * (i - 4));
    }
    *reinterpret_cast<uint2 *>(oq + s * (H / 2) + h / 2) = packed;
    os[s * (H / 16) + h / 16] = (uint16_t)sb;
}

__global__ __launch_bounds__(256) void ep_fill_zero_kernel(uint32_t *p, size_t words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

#ifndef EP_CALIB_BLOCKS
#define EP_CALIB_BLOCKS 1024
#endif

// Plain streaming copy: consecutive 16-byte vectors across the grid.
__global__ __launch_bounds__(256) void ep_calib_copy_kernel(const vec16 *src, vec16 *dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

}  // namespace

hipError_t launch_quant_fp8(int64_t rows, int H, const uint16_t *x, uint8_t *q, float *scales,
                            hipStream_t stream) {
    const int64_t groups = rows * (H / 128);
    if (groups == 0) return hipSuccess;
    const int64_t threads = groups * 16;
    hipLaunchKernelGGL(ep_quant_fp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, x, q, scales, groups);
    return hipGetLastError();
}

hipError_t launch_expert_scale_bf16(const Shape &s, const int32_t *expert_offset,
                                    const float *factor, const uint16_t *recv, uint16_t *out,
                                    hipStream_t stream) {
    const int64_t rows = s.T * s.k;
    if (rows == 0) return hipSuccess;
    const int64_t waves = rows * ((s.H + 511) / 512);
    hipLaunchKernelGGL(ep_expert_scale_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       stream, expert_offset, s.E, s.H, rows, factor, recv, out);
    return hipGetLastError();
}

hipError_t launch_expert_requant_mxfp8(const Shape &s, const int32_t *expert_offset,
                                       const float *factor, const uint8_t *recv_q,
                                       const float *recv_scales, uint8_t *out_q,
                                       uint8_t *out_e8m0, hipStream_t stream) {
    const int64_t rows = s.T * s.k;
    if (rows == 0) return hipSuccess;
    const int64_t waves = rows * ((s.H + 1023) / 1024);
    hipLaunchKernelGGL(ep_expert_requant_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       stream, expert_offset, s.E, s.H, rows, factor, recv_q, recv_scales, out_q,
                       out_e8m0);
    return hipGetLastError();
}

hipError_t launch_expert_requant_nvfp4(const Shape &s, const int32_t *expert_offset,
                                       const float *factor, const uint16_t *recv, uint8_t *out_q,
                                       uint16_t *out_scales, hipStream_t stream) {
    const int64_t rows = s.T * s.k;
    if (rows == 0) return hipSuccess;
    const int64_t waves = rows * ((s.H + 1023) / 1024);
    hipLaunchKernelGGL(ep_expert_requant_nvfp4_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       stream, expert_offset, s.E, s.H, rows, factor, recv, out_q, out_scales);
    return hipGetLastError();
}

hipError_t launch_ws_init(uint32_t *ws, size_t words, hipStream_t stream) {
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(ep_fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, words);
    return hipGetLastError();
}

hipError_t launch_calib_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > EP_CALIB_BLOCKS) blocks = EP_CALIB_BLOCKS;   // 4 blocks per CU measured fastest
    hipLaunchKernelGGL(ep_calib_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const vec16 *>(src), static_cast<vec16 *>(dst), n);
    return hipGetLastError();
}

}  // namespace ep
