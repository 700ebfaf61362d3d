// combine.hip -- top-k weighted gather-reduce on gfx950.
//
// What it computes (MORI-EP Benchmark, "Combine": the reverse of dispatch;
// MSCCL++ PR 860: each expert returns one row per dispatched (token, expert)
// pair, and combine consumes the receiver-side layout that dispatch
// returned): for every token t and element h,
//     acc = -0.0f;  for j = 0..k-1 with s = token_slot[t,j] >= 0:
//         acc = fmaf(topk_w[t,j], value(s, h), acc)
//     y[t,h] = bf16_rne(acc)          (+0.0 for a token with no valid slot)
// i.e. fp32 accumulation in top-k slot order and one rounding to bf16.
// value() is the bf16 element, or for mxfp8 rows e4m3(q) * 2^(e8m0 - 127)
// (exact in binary32).
//
// How: one wave per (token, row part).  Lanes 0..k-1 read the token's slots
// and weights; a ballot gives the unmasked ones, which readlane moves into
// scalar registers in slot order, so every decision on a slot is uniform.
// Each lane owns 16-byte column vectors of the row; per batch of slots (all
// k when k is a compile-time constant) it issues every load of the batch
// before the first FMA, then applies v_fma_f32 in slot order, the first
// unmasked slot as a multiply.  Nothing is reduced across lanes, so the
// result does not depend on the launch shape.  The gathered rows are read once: the loads carry the
// non-temporal hint so they do not evict what the caches still hold.
// bf16 rows: the tokens are taken last to first and y is stored
// non-temporal.  The dispatch leaves the first tokens' receive rows in the
// memory-side cache and streams the later ones to HBM; this order reads the
// HBM rows first and the cached rows last, and y does not evict them
// (T = 4096, hidden 7168, top-8: 101 -> 85 us).  Taking the cached tokens
// interleaved with the others, as the dispatch does, made the combine slower
// (85 -> 92 us); first to last is on par with last to first.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

struct CombineArgs {
    const char *eo;             // [T*k][row_bytes]
    const uint8_t *eo_scales;   // [T*k][H/32] e8m0, mxfp8 only
    const int32_t *token_slot;  // [T][k]
    const float *topk_w;        // [T][k]
    char *y;                    // [T][2H]
    int64_t T;
    int k, H;
    int64_t row_bytes;          // 2H (bf16) or H (mxfp8)
    int64_t rows;               // receive rows (T*k, or R*M for RANK_MAJOR)
    int nvec;                   // 16-byte vectors per payload row
    int S;                      // waves per token
    int64_t cached;             // tokens [0, cached) have their rows in the memory-side cache
};

#ifndef EP_COMBINE_BATCH
#define EP_COMBINE_BATCH 8     // slots per batch of loads when k is not a compile-time constant
#endif
#ifndef EP_COMBINE_K8_GENERIC
#define EP_COMBINE_K8_GENERIC 0   // 1: k = 8 takes the run-time-k kernels (batches of EP_COMBINE_BATCH)
#endif
constexpr int kSlotBatch = EP_COMBINE_BATCH;

#ifndef EP_COMBINE_VECS
#define EP_COMBINE_VECS 4      // 16-byte vectors per lane per pass (bf16 rows)
#endif
#ifndef EP_COMBINE_WAVES
#define EP_COMBINE_WAVES 16384   // waves the combine aims for (16 per CU)
#endif
#ifndef EP_COMBINE_Y_NT
#define EP_COMBINE_Y_NT 1      // bf16 rows: non-temporal stores for y
#endif
#ifndef EP_COMBINE_CONTIG
#define EP_COMBINE_CONTIG 0    // 1: each wave of a token owns one contiguous part of the row
#endif
#ifndef EP_COMBINE_SMALL_WAVES
#define EP_COMBINE_SMALL_WAVES 4096   // bf16 rows: fewer waves than this -> one vector per lane
#endif
#ifndef EP_COMBINE_ONE_PASS
#define EP_COMBINE_ONE_PASS 1  // bf16 rows: waves per token so that one pass covers a wave's part of the row
#endif
#ifndef EP_COMBINE_Q_ONE_PASS
#define EP_COMBINE_Q_ONE_PASS 1  // mxfp8 / nvfp4: waves per token so that one pass covers a wave's part
#endif
#ifndef EP_COMBINE_ORDER
#define EP_COMBINE_ORDER 1     // bf16 rows: 0 tokens first to last, 1 last to first,
                               // 2 cached tokens interleaved with the others
#endif

#ifndef EP_COMBINE_Q_OCC
#define EP_COMBINE_Q_OCC 5     // mxfp8 / nvfp4: waves per SIMD the register allocation must allow (0: free)
#endif
#if EP_COMBINE_Q_OCC > 0
#define EP_Q_OCC_ATTR __attribute__((amdgpu_waves_per_eu(EP_COMBINE_Q_OCC)))
#else
#define EP_Q_OCC_ATTR
#endif
#ifndef EP_COMBINE_PIN
#define EP_COMBINE_PIN 1       // bf16 rows: where the batch's loads are pinned (pin_loads)
#endif
#ifndef EP_COMBINE_Q_PIN
#define EP_COMBINE_Q_PIN 1     // mxfp8 / nvfp4: where the batch's loads are pinned (pin_loads)
#endif
#ifndef EP_COMBINE_Q_YT
#define EP_COMBINE_Q_YT 1      // mxfp8 / nvfp4: y through a per-wave LDS transpose, non-temporal
                               // (0: plain stores of each lane's pieces)
#endif

// NT: non-temporal.  Only where each store instruction of a wave covers
// whole cache lines (64 lanes x 16 contiguous bytes): the lanes of the mxfp8
// / nvfp4 kernels hold 32 / 64 contiguous bytes of y each, and non-temporal
// stores of those pieces straight from the lanes (partial lines per
// instruction) made the nvfp4 combine twice as slow; they go through an LDS
// transpose first (store_y_transposed).
template <bool NT>
__device__ __forceinline__ void store_y(char *p, vec16 v) {
    if (NT) st16_nt(p, v); else st16(p, v);
}

// y of one pass of a quantized-payload combine: lane l holds O 16-byte
// vectors, bytes [(v0 + l) * 16 * O, (v0 + l + 1) * 16 * O) of the y row, so
// the wave's O * 64 vectors are one contiguous stretch.  They go through LDS
// (each wave its own O * 64 slots; the wave barriers keep the LDS accesses of
// consecutive passes in order) and each store instruction then writes 1 KB
// of contiguous y -- whole lines, stored non-temporal (nvfp4, T = 4096,
// hidden 7168, top-8: 43.1 -> 38.9 us against plain stores of the pieces;
// mxfp8 on par).  Vectors of lanes past the row end are not stored.
template <int O>
__device__ __forceinline__ void store_y_transposed(vec16 *wbuf, const vec16 (&out)[O], char *yrow, int v0,
                                                   int nvec, int lane) {
#pragma unroll
    for (int o = 0; o < O; ++o) wbuf[lane * O + o] = out[o];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int o = 0; o < O; ++o) {
        const int idx = o * kWave + lane;   // 16-byte vector of the stretch
        const vec16 val = wbuf[idx];
        if (v0 + idx / O < nvec) store_y<true>(yrow + ((int64_t)v0 * O + idx) * 16, val);
    }
    __builtin_amdgcn_wave_barrier();
}

// Slot j of the token in a scalar register; lanes >= k hold -1, so any j < 64
// past the token's slots reads as masked.  A masked slot's load is pointed at
// row 0 (always allocated, and cache-resident when several slots are masked)
// so every load of a batch is unconditional and issued back to back; its
// FMAs are skipped, which keeps the masked-slot semantics exact.
__device__ __forceinline__ int64_t row_of(int32_t s) { return s >= 0 ? (int64_t)s : 0; }

// The token's unmasked slots, in slot order, as wave-uniform lane indices:
// `m` holds the lanes (slots) not yet taken.  Skipping a masked slot is what
// the fma chain does, so running over the unmasked slots alone, in order,
// changes no result; the first of them starts the chain, where
// fmaf(w, x, -0.0f) equals w * x, so no accumulator is set to -0.0 first.
// Once `m` is empty it returns lane 63, whose slot is -1 (k <= 32).
__device__ __forceinline__ int next_slot_lane(uint64_t &m) {
    const int l = __builtin_ctzll(m | (1ull << 63));
    m &= m - 1;
    return l;
}

// An empty asm statement that uses every loaded value of a batch.  Without a
// use outside the per-slot branches the compiler sinks each slot's loads into
// that slot's branch, behind the previous slot's fmas, and the batch's loads
// are no longer in flight together.  EP_COMBINE_Q_PIN 0 places the use before
// the fmas (they wait for the whole batch), 1 after them (each waits for its
// own slot; the loaded registers stay live to the end).
template <int KB>
__device__ __forceinline__ void pin_loads(const vec16 (&buf)[KB], const uint32_t (&sc)[KB]) {
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) asm volatile("" ::"v"(buf[jj]), "v"(sc[jj]));
}
template <int KB, int C>
__device__ __forceinline__ void pin_loads2(const vec16 (&buf)[KB][C]) {
#pragma unroll
    for (int jj = 0; jj < KB; ++jj)
#pragma unroll
        for (int i = 0; i < C; ++i) asm volatile("" ::"v"(buf[jj][i]));
}

// One batch of up to KB unmasked slots of a bf16 pass (C vectors per lane,
// v0 + i * vstep, those below vend): every load first, then the fmas of the
// `live` slots in order (see next_slot_lane, pin_loads).
template <int KB, int C, bool FIRST>
__device__ __forceinline__ void bf16_batch(const CombineArgs &a, int32_t slot, float wt, uint64_t &m, int live,
                                           int v0, int vstep, int vend, float (&acc)[8 * C]) {
    vec16 buf[KB][C];
    int ln[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        ln[jj] = next_slot_lane(m);
        const char *row = a.eo + row_of(readlane(slot, ln[jj])) * a.row_bytes;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int v = v0 + i * vstep;
            if (v < vend) buf[jj][i] = ld16_nt(row + (uint32_t)v * 16u);
        }
    }
    if (EP_COMBINE_PIN == 0) pin_loads2<KB, C>(buf);
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        if (jj >= live) break;
        const float w = readlane(wt, ln[jj]);
#pragma unroll
        for (int i = 0; i < C; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = bf16_lo(buf[jj][i][q]), hi = bf16_hi(buf[jj][i][q]);
                float &a0 = acc[8 * i + 2 * q], &a1 = acc[8 * i + 2 * q + 1];
                a0 = (FIRST && jj == 0) ? w * lo : __builtin_fmaf(w, lo, a0);
                a1 = (FIRST && jj == 0) ? w * hi : __builtin_fmaf(w, hi, a1);
            }
    }
    if (EP_COMBINE_PIN == 1) pin_loads2<KB, C>(buf);
}

// bf16 rows: a 16-byte vector holds 8 elements; C vectors per lane per pass,
// KB slots per batch (k itself when k is a compile-time constant KC).
template <int C, int KC>
__global__ __launch_bounds__(256) void ep_combine_bf16_kernel(CombineArgs a) {
    constexpr int KB = KC > 0 ? KC : kSlotBatch;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t tw = gw / a.S;
    const int sub = (int)(gw - tw * a.S);
    if (tw >= a.T) return;
    const int64_t t = EP_COMBINE_ORDER == 1 ? a.T - 1 - tw
                      : EP_COMBINE_ORDER == 2 ? interleaved_token(tw, a.T, a.cached) : tw;
    const int k = KC > 0 ? KC : a.k;

    int32_t slot = -1;
    float wt = 0.0f;
    if (lane < k) {
        slot = a.token_slot[t * k + lane];
        wt = a.topk_w[t * k + lane];
        if ((uint64_t)slot >= (uint64_t)a.rows) slot = -1;   // outside the receive rows: masked
    }
    const uint64_t valid = __ballot(lane < k && slot >= 0);
    const int nvalid = __popcll(valid);
    char *yrow = a.y + t * (int64_t)a.H * 2;
    const int stride = kWave * a.S;

    // vectors of this wave: interleaved with the token's other waves, or one
    // contiguous part of the row per wave
    const int per = (a.nvec + a.S - 1) / a.S;
    const int vbeg = EP_COMBINE_CONTIG ? sub * per + lane : lane + kWave * sub;
    const int vend = EP_COMBINE_CONTIG ? min(a.nvec, (sub + 1) * per) : a.nvec;
    const int vstep = EP_COMBINE_CONTIG ? kWave : stride;
    for (int v0 = vbeg; v0 < vend; v0 += vstep * C) {
        uint32_t packed[4 * C];
        if (nvalid == 0) {   // no valid slot: +0.0
#pragma unroll
            for (int q = 0; q < 4 * C; ++q) packed[q] = 0u;
        } else {
            float acc[8 * C];
            uint64_t m = valid;
            bf16_batch<KB, C, true>(a, slot, wt, m, min(nvalid, KB), v0, vstep, vend, acc);
            if (KC == 0)   // k > KB is possible only for a run-time k
                for (int jb = KB; jb < nvalid; jb += KB)
                    bf16_batch<KB, C, false>(a, slot, wt, m, min(nvalid - jb, KB), v0, vstep, vend, acc);
            pack_bf16(acc, packed);
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int v = v0 + i * vstep;
            if (v >= vend) continue;
            vec16 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = packed[4 * i + q];
            store_y<EP_COMBINE_Y_NT>(yrow + (int64_t)v * 16, o);
        }
    }
}

// One batch of up to KB unmasked slots of an mxfp8 row vector v: every load
// first, then the fmas of the `live` slots in order.  The row and scale-row
// bases are wave-uniform, so each load is a scalar base plus the lane's
// 32-bit offset.
template <int KB, bool FIRST>
__device__ __forceinline__ void mxfp8_batch(const CombineArgs &a, int32_t slot, float wt, uint64_t &m, int live,
                                            int v, float (&acc)[16]) {
    const int G32 = a.H / 32;
    vec16 buf[KB];
    uint32_t sc[KB];
    int ln[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        ln[jj] = next_slot_lane(m);
        const int64_t r = row_of(readlane(slot, ln[jj]));
        buf[jj] = ld16_nt(a.eo + r * a.row_bytes + (uint32_t)v * 16u);
        sc[jj] = (a.eo_scales + r * G32)[(uint32_t)v >> 1];
    }
    if (EP_COMBINE_Q_PIN == 0) pin_loads<KB>(buf, sc);
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        if (jj >= live) break;
        const float w = readlane(wt, ln[jj]);
        const float scale = e8m0_to_f32(sc[jj]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // e4m3 bytes 0,1 and 2,3 of the dword, each times the scale
            const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(buf[jj][q], scale, false);
            const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(buf[jj][q], scale, true);
            const float e[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[4 * q + b] = (FIRST && jj == 0) ? w * e[b] : __builtin_fmaf(w, e[b], acc[4 * q + b]);
        }
    }
    if (EP_COMBINE_Q_PIN == 1) pin_loads<KB>(buf, sc);
}

// mxfp8 rows: a 16-byte vector holds 16 e4m3 elements, half of a 32-element
// scale group; the y row vectors for it are two 16-byte bf16 vectors.  The
// element value e4m3(q) * 2^(e8m0 - 127) comes from gfx950's
// v_cvt_scalef32_pk_f32_fp8 (two elements per instruction).  That product is
// exact in binary32, and the instruction returns exactly it -- NaN codes,
// subnormal codes and the subnormal scale 2^-127 included -- which the GPU
// parity test over every (code, scale) pair checks through this kernel.
template <int KC>
__global__ __launch_bounds__(256) EP_Q_OCC_ATTR void ep_combine_mxfp8_kernel(CombineArgs a) {
    constexpr int KB = KC > 0 ? KC : kSlotBatch;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t t = gw / a.S;
    const int sub = (int)(gw - t * a.S);
    if (t >= a.T) return;
    const int k = KC > 0 ? KC : a.k;

    int32_t slot = -1;
    float wt = 0.0f;
    if (lane < k) {
        slot = a.token_slot[t * k + lane];
        wt = a.topk_w[t * k + lane];
        if ((uint64_t)slot >= (uint64_t)a.rows) slot = -1;   // outside the receive rows: masked
    }
    const uint64_t valid = __ballot(lane < k && slot >= 0);
    const int nvalid = __popcll(valid);
    char *yrow = a.y + t * (int64_t)a.H * 2;
    const int stride = kWave * a.S;

    __shared__ vec16 ybuf[4][2 * kWave];   // per wave of the block (EP_COMBINE_Q_YT)
    for (int v0 = kWave * sub; v0 < a.nvec; v0 += stride) {   // uniform passes
        // lanes past the row re-read its last vector and store nothing
        const bool in_row = v0 + lane < a.nvec;
        const int v = in_row ? v0 + lane : a.nvec - 1;
        vec16 out[2];
        if (nvalid == 0) {   // no valid slot: +0.0
#pragma unroll
            for (int q = 0; q < 4; ++q) out[0][q] = out[1][q] = 0u;
        } else {
            float acc[16];
            uint64_t m = valid;
            mxfp8_batch<KB, true>(a, slot, wt, m, min(nvalid, KB), v, acc);
            if (KC == 0)   // k > KB is possible only for a run-time k
                for (int jb = KB; jb < nvalid; jb += KB) mxfp8_batch<KB, false>(a, slot, wt, m, min(nvalid - jb, KB), v, acc);
            uint32_t packed[8];
            pack_bf16(acc, packed);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                out[0][q] = packed[q];
                out[1][q] = packed[4 + q];
            }
        }
        if (EP_COMBINE_Q_YT) {
            store_y_transposed<2>(ybuf[threadIdx.x / kWave], out, yrow, v0, a.nvec, lane);
        } else if (in_row) {
            store_y<false>(yrow + (int64_t)v * 32, out[0]);
            store_y<false>(yrow + (int64_t)v * 32 + 16, out[1]);
        }
    }
}

// One batch of up to KB unmasked slots of an nvfp4 row vector v (see
// mxfp8_batch).  Element = e2m1 decoded at scale 1.0 (exact) times the
// group's bf16 scale (exact: a 2-bit times an 8-bit significand); then one
// fma by the weight.
template <int KB, bool FIRST>
__device__ __forceinline__ void nvfp4_batch(const CombineArgs &a, int32_t slot, float wt, uint64_t &m, int live,
                                            int v, float (&acc)[32]) {
    const int G16 = a.H / 16;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(a.eo_scales);
    vec16 buf[KB];
    uint32_t sc[KB];
    int ln[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        ln[jj] = next_slot_lane(m);
        const int64_t r = row_of(readlane(slot, ln[jj]));
        buf[jj] = ld16_nt(a.eo + r * a.row_bytes + (uint32_t)v * 16u);
        // the two bf16 scales of the vector's two 16-element groups
        sc[jj] = *reinterpret_cast<const uint32_t *>(scales + r * G16 + 2u * (uint32_t)v);
    }
    if (EP_COMBINE_Q_PIN == 0) pin_loads<KB>(buf, sc);
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        if (jj >= live) break;
        const float w = readlane(wt, ln[jj]);
        const float s_lo = bf16_lo(sc[jj]), s_hi = bf16_hi(sc[jj]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float s = q < 2 ? s_lo : s_hi;   // dwords 0-1: group 2v, 2-3: group 2v+1
            // byte b of the dword holds elements 2b (low nibble) and 2b + 1
            const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(buf[jj][q], 1.0f, 0);
            const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(buf[jj][q], 1.0f, 1);
            const f32x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(buf[jj][q], 1.0f, 2);
            const f32x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(buf[jj][q], 1.0f, 3);
            const float ev[8] = {e0.x, e0.y, e1.x, e1.y, e2.x, e2.y, e3.x, e3.y};
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const float x = ev[b] * s;
                acc[8 * q + b] = (FIRST && jj == 0) ? w * x : __builtin_fmaf(w, x, acc[8 * q + b]);
            }
        }
    }
    if (EP_COMBINE_Q_PIN == 1) pin_loads<KB>(buf, sc);
}

// nvfp4 rows: a 16-byte vector holds 32 e2m1 elements (two 16-element scale
// groups, one bf16 scale each); the y row vectors for it are four 16-byte
// bf16 vectors.  Elements decode with v_cvt_scalef32_pk_f32_fp4 at scale 1.0
// (exact), then one fp32 multiply by the group's bf16 scale (exact: a 2-bit
// times an 8-bit significand).  The instruction's own scale operand is not
// used: it honours only the exponent of a scale, and these scales are not
// powers of two.
template <int KC>
__global__ __launch_bounds__(256) EP_Q_OCC_ATTR void ep_combine_nvfp4_kernel(CombineArgs a) {
    constexpr int KB = KC > 0 ? KC : kSlotBatch;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t t = gw / a.S;
    const int sub = (int)(gw - t * a.S);
    if (t >= a.T) return;
    const int k = KC > 0 ? KC : a.k;

    int32_t slot = -1;
    float wt = 0.0f;
    if (lane < k) {
        slot = a.token_slot[t * k + lane];
        wt = a.topk_w[t * k + lane];
        if ((uint64_t)slot >= (uint64_t)a.rows) slot = -1;   // outside the receive rows: masked
    }
    const uint64_t valid = __ballot(lane < k && slot >= 0);
    const int nvalid = __popcll(valid);
    char *yrow = a.y + t * (int64_t)a.H * 2;
    const int stride = kWave * a.S;

    __shared__ vec16 ybuf[4][4 * kWave];   // per wave of the block (EP_COMBINE_Q_YT)
    for (int v0 = kWave * sub; v0 < a.nvec; v0 += stride) {   // uniform passes
        // lanes past the row re-read its last vector and store nothing
        const bool in_row = v0 + lane < a.nvec;
        const int v = in_row ? v0 + lane : a.nvec - 1;
        vec16 out[4];
        if (nvalid == 0) {   // no valid slot: +0.0
#pragma unroll
            for (int o = 0; o < 4; ++o)
#pragma unroll
                for (int q = 0; q < 4; ++q) out[o][q] = 0u;
        } else {
            float acc[32];
            uint64_t m = valid;
            nvfp4_batch<KB, true>(a, slot, wt, m, min(nvalid, KB), v, acc);
            if (KC == 0)   // k > KB is possible only for a run-time k
                for (int jb = KB; jb < nvalid; jb += KB) nvfp4_batch<KB, false>(a, slot, wt, m, min(nvalid - jb, KB), v, acc);
            uint32_t packed[16];
            pack_bf16(acc, packed);
#pragma unroll
            for (int o = 0; o < 4; ++o)
#pragma unroll
                for (int q = 0; q < 4; ++q) out[o][q] = packed[4 * o + q];
        }
        if (EP_COMBINE_Q_YT) {
            store_y_transposed<4>(ybuf[threadIdx.x / kWave], out, yrow, v0, a.nvec, lane);
        } else if (in_row) {
#pragma unroll
            for (int o = 0; o < 4; ++o) store_y<false>(yrow + (int64_t)v * 64 + 16 * o, out[o]);
        }
    }
}

}  // namespace

hipError_t launch_combine(const Shape &s, const void *expert_out, const uint8_t *expert_scales,
                          const int32_t *token_slot, const float *topk_w, void *y,
                          hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    CombineArgs a{};
    a.eo = static_cast<const char *>(expert_out);
    a.eo_scales = expert_scales;
    a.token_slot = token_slot;
    a.topk_w = topk_w;
    a.y = static_cast<char *>(y);
    a.T = s.T;
    a.k = s.k;
    a.H = s.H;
    a.rows = s.rows();
    a.cached = cached_tokens(s);
    const bool mx = (s.y_fmt == 2), nv = (s.y_fmt == 3);
    a.row_bytes = nv ? (int64_t)s.H / 2 : (mx ? (int64_t)s.H : 2 * (int64_t)s.H);
    a.nvec = (int)(a.row_bytes / 16);
    a.S = waves_per_token(s.T, a.nvec, EP_COMBINE_WAVES);
    const dim3 block(256);
    if (nv || mx) {
        // one vector per lane per pass; with EP_COMBINE_Q_ONE_PASS exactly one
        // pass per wave (ceil(row vectors / 64) waves per token)
        if (EP_COMBINE_Q_ONE_PASS) a.S = (a.nvec + kWave - 1) / kWave;
        const dim3 gq((unsigned)((s.T * a.S + 3) / 4));
        if (nv) {
            if (s.k == 8) hipLaunchKernelGGL(ep_combine_nvfp4_kernel<8>, gq, block, 0, stream, a);
            else hipLaunchKernelGGL(ep_combine_nvfp4_kernel<0>, gq, block, 0, stream, a);
        } else {
            if (s.k == 8) hipLaunchKernelGGL(ep_combine_mxfp8_kernel<8>, gq, block, 0, stream, a);
            else hipLaunchKernelGGL(ep_combine_mxfp8_kernel<0>, gq, block, 0, stream, a);
        }
    } else {
        int S = a.S;
        if (EP_COMBINE_ONE_PASS) {   // the smallest power of two with one pass per wave
            S = 1;
            while ((int64_t)kWave * EP_COMBINE_VECS * S < a.nvec && S < 64) S *= 2;
        }
        if (s.T * S < EP_COMBINE_SMALL_WAVES) {
            // a small batch does not fill the chip at 64 row vectors per wave:
            // one wave per 64 vectors of a row, one vector per lane
            a.S = (a.nvec + kWave - 1) / kWave;
            const dim3 g2((unsigned)((s.T * a.S + 3) / 4));
            if (s.k == 8) hipLaunchKernelGGL((ep_combine_bf16_kernel<1, 8>), g2, block, 0, stream, a);
            else hipLaunchKernelGGL((ep_combine_bf16_kernel<1, 0>), g2, block, 0, stream, a);
        } else {
            a.S = S;
            const dim3 g3((unsigned)((s.T * a.S + 3) / 4));
            if (s.k == 8 && !EP_COMBINE_K8_GENERIC) hipLaunchKernelGGL((ep_combine_bf16_kernel<EP_COMBINE_VECS, 8>), g3, block, 0, stream, a);
            else hipLaunchKernelGGL((ep_combine_bf16_kernel<EP_COMBINE_VECS, 0>), g3, block, 0, stream, a);
        }
    }
    return hipGetLastError();
}

}  // namespace ep
