// Ceilings of one MI355X (gfx950) measured in the process that uses them:
// the rates the optimizer's kernels are compared with besides the datasheet
// peaks.  Each probe does only the work it names, so its rate is what that
// unit of the chip sustains under these launch shapes:
//
//   ma_peaks_mfma      independent v_mfma_f32_32x32x16_bf16 (or the fp32
//                      v_mfma_f32_32x32x2_f32) on registers, no memory
//                      traffic; also returns the shader clock it ran at
//                      (s_memtime cycles against the 100 MHz s_memrealtime)
//   ma_peaks_lds       LDS reads into registers: 16-byte reads of
//                      consecutive addresses, or the gfx950 transposing
//                      8-byte read (ds_read_b64_tr_b16)
//   ma_peaks_stream    HBM streams over float4 arrays: read only, copy
//                      (1 read : 1 write), and the AdamW mix (read four
//                      streams, write three of them back in place: 16 : 12
//                      bytes per element)
//   ma_peaks_dma       global memory straight into LDS (buffer loads that
//                      write LDS), staged as the bf16 GEMMs stage their
//                      operands: eight waves copy 32 KB stages into a ring of
//                      five, four stages ahead, with a wait and a workgroup
//                      barrier per stage; no matrix instructions, no LDS reads
//
// Not part of the optimizer's C ABI: measurement only.  Every entry point
// launches on the given stream and returns a hipError_t (0 on success); the
// caller times the launch with events on that stream.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave

template <bool F32>
__global__ __launch_bounds__(256) void k_peak_mfma(int iters, float* sink, uint64_t* clocks) {
    const int lane = threadIdx.x & 63;
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1e-3f * (float)(lane + e));
        b[e] = (__bf16)(1e-3f * (float)(lane - e));
    }
    const float fa = 1e-3f * (float)lane, fb = 1e-3f * (float)(lane ^ 7);
    const uint64_t t0 = __builtin_readcyclecounter();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if (F32) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa, fb, acc[c], 0, 0, 0);
            else acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        }
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
}

constexpr int kLdsBytes = 65536;

template <bool TR>
__global__ __launch_bounds__(256) void k_peak_lds(int iters, float* sink, uint64_t* clocks) {
    __shared__ __attribute__((aligned(16))) char buf[kLdsBytes];
    for (int i = threadIdx.x * 16; i < kLdsBytes; i += blockDim.x * 16)
        *reinterpret_cast<uint4*>(buf + i) = make_uint4(i, i + 1, i + 2, i + 3);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = 0;
    // each wave reads its own 16 KB region: 16-byte reads of consecutive
    // addresses (a whole 1 KB row per instruction), or transposing 8-byte
    // reads at the addresses a 16 x 16 bf16 fragment load uses
    const char* base = buf + wave * 16384;
    const uint64_t t0 = __builtin_readcyclecounter();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (TR) {
                const char* p = base + ((u * 1024 + (lane >> 4) * 256 + (lane & 15) * 8) & 16383);
                const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(p));
                const uint2 w = __builtin_bit_cast(uint2, v);
                x ^= w.x + w.y;
            } else {
                const uint4 v = *reinterpret_cast<const uint4*>(base + ((u * 1024 + lane * 16) & 16383));
                x ^= v.x + v.y + v.z + v.w;
            }
        }
        // the buffer may have changed as far as the compiler knows, so every
        // pass reads LDS again (the addresses do not depend on the pass)
        asm volatile("" ::: "memory");
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)x;
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
}

// One chunk of 16 Ki elements (4096 float4) per workgroup, 4 float4 of each
// stream in flight per thread, nontemporal accesses (as the AdamW kernel).
constexpr int kVecPerThread = 16;

template <int KIND>
__global__ __launch_bounds__(256) void k_peak_stream(f32x4* __restrict__ a, f32x4* __restrict__ b,
                                                     f32x4* __restrict__ c, f32x4* __restrict__ d,
                                                     int64_t n_vec, float* sink) {
    const int64_t base = (int64_t)blockIdx.x * 256 * kVecPerThread + threadIdx.x;
    float acc = 0.f;
#pragma unroll
    for (int h = 0; h < kVecPerThread / 4; ++h) {
        f32x4 va[4], vb[4], vc[4], vd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t i = base + (int64_t)(h * 4 + q) * 256;
            if (i >= n_vec) continue;
            va[q] = __builtin_nontemporal_load(a + i);
            if (KIND == 2) {
                vb[q] = __builtin_nontemporal_load(b + i);
                vc[q] = __builtin_nontemporal_load(c + i);
                vd[q] = __builtin_nontemporal_load(d + i);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t i = base + (int64_t)(h * 4 + q) * 256;
            if (i >= n_vec) continue;
            if (KIND == 0) {
                acc += va[q][0] + va[q][1] + va[q][2] + va[q][3];
            } else if (KIND == 1) {
                __builtin_nontemporal_store(va[q], b + i);
            } else {
                const f32x4 g = vb[q];
                const f32x4 m = 0.9f * vc[q] + 0.1f * g;
                const f32x4 v = 0.999f * vd[q] + 1e-3f * g * g;
                const f32x4 p = va[q] - 1e-7f * m;
                __builtin_nontemporal_store(p, a + i);
                __builtin_nontemporal_store(m, c + i);
                __builtin_nontemporal_store(v, d + i);
            }
        }
    }
    if (KIND == 0) sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// LDS-DMA probe.  Workgroup b copies stage s from the 32 KB chunk
// (b * 7919 + s) mod (src_bytes / 32 KB) of the source: a source of a few MB
// stays in every XCD's L2, a large one streams from the memory-side cache or
// HBM.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kDmaStage = 32768;
constexpr int kDmaSlots = 5;
constexpr int kDmaWaves = 8;

__device__ __forceinline__ void dma_copy16(u32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// vmcnt(n) for n in {0, 4, 8, 12}, the other counters unconstrained
__device__ __forceinline__ void dma_wait(int n) {
    if (n <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (n == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
    else if (n == 8) __builtin_amdgcn_s_waitcnt(0x0F78);
    else __builtin_amdgcn_s_waitcnt(0x0F7C);
}

__global__ __launch_bounds__(kDmaWaves * 64) void k_peak_dma(const char* __restrict__ src,
                                                              uint32_t src_bytes, int stages,
                                                              uint64_t* clocks) {
    __shared__ __attribute__((aligned(1024))) char ring[kDmaSlots * kDmaStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t a = (uint64_t)src;
    u32x4 rsrc;
    rsrc.x = (uint32_t)a;
    rsrc.y = (uint32_t)(a >> 32) & 0xffffu;
    rsrc.z = src_bytes;
    rsrc.w = 0x00020000u;
    const uint32_t lring = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)ring;
    const uint32_t chunks = src_bytes / kDmaStage;
    const uint32_t voff = (uint32_t)lane * 16;
    // this wave's 4 KB of stage s: four 1 KB copies
    auto copy = [&](int s) {
        const uint32_t chunk = ((uint32_t)blockIdx.x * 7919u + (uint32_t)s) % chunks;
        const uint32_t from = chunk * kDmaStage + (uint32_t)wave * 4096;
        const uint32_t to = lring + (uint32_t)(s % kDmaSlots) * kDmaStage + (uint32_t)wave * 4096;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma_copy16(rsrc, to + i * 1024, voff, from + i * 1024);
    };
    const uint64_t t0 = __builtin_readcyclecounter();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    for (int s = 0; s < kDmaSlots - 1 && s < stages; ++s) copy(s);
    for (int s = 0; s < stages; ++s) {
        // stage s + 1 has landed once at most the copies of stages s + 2,
        // s + 3 are outstanding; the barrier frees the slot of stage s - 1
        const int ahead = stages - 2 - s;
        dma_wait(4 * (ahead < 2 ? ahead : 2));
        __builtin_amdgcn_s_barrier();
        if (s + kDmaSlots - 1 < stages) copy(s + kDmaSlots - 1);
    }
    dma_wait(0);
    __builtin_amdgcn_s_barrier();
    const uint64_t t1 = __builtin_readcyclecounter();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
}

}  // namespace

extern "C" {

// `blocks` workgroups of 256 threads, each wave running `iters` rounds of
// kChains (8) independent MFMAs.  sink: blocks * 256 floats; clocks: 2 *
// blocks uint64 (per workgroup: shader cycles, 100 MHz ticks of the loop).
// Flops per launch: blocks * 4 * iters * 8 * (32768 bf16 | 4096 fp32).
int ma_peaks_mfma(int fp32, int64_t blocks, int iters, float* sink, uint64_t* clocks,
                  void* stream) {
    if (blocks < 1 || iters < 1 || !sink || !clocks) return (int)hipErrorInvalidValue;
    if (fp32)
        hipLaunchKernelGGL(k_peak_mfma<true>, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, iters, sink, clocks);
    else
        hipLaunchKernelGGL(k_peak_mfma<false>, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, iters, sink, clocks);
    return (int)hipGetLastError();
}

// `blocks` workgroups of 256 threads with 64 KB of LDS each; every wave
// reads `iters` x 16 instructions.  Bytes read per launch: blocks * 4 *
// iters * 16 * (1024 plain | 512 transposing).  sink: blocks * 256 floats;
// clocks: 2 * blocks uint64, as for ma_peaks_mfma.
int ma_peaks_lds(int transposing, int64_t blocks, int iters, float* sink, uint64_t* clocks,
                 void* stream) {
    if (blocks < 1 || iters < 1 || !sink || !clocks) return (int)hipErrorInvalidValue;
    if (transposing)
        hipLaunchKernelGGL(k_peak_lds<true>, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, iters, sink, clocks);
    else
        hipLaunchKernelGGL(k_peak_lds<false>, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, iters, sink, clocks);
    return (int)hipGetLastError();
}

// kind 0: read a (sink: one float per thread of ceil(n_vec / 4096)
// workgroups); 1: copy a -> b; 2: the AdamW mix in place on a, b, c, d
// (read all four, write a, c, d).  Arrays of n_vec float4.
int ma_peaks_stream(int kind, void* a, void* b, void* c, void* d, int64_t n_vec, float* sink,
                    void* stream) {
    if (n_vec < 1 || !a || (kind == 0 && !sink) || (kind >= 1 && !b) || (kind == 2 && (!c || !d)) ||
        kind < 0 || kind > 2)
        return (int)hipErrorInvalidValue;
    const int64_t per = 256 * kVecPerThread;
    const dim3 grid((unsigned)((n_vec + per - 1) / per));
    f32x4 *A = (f32x4*)a, *B = (f32x4*)b, *Cc = (f32x4*)c, *D = (f32x4*)d;
    hipStream_t st = (hipStream_t)stream;
    if (kind == 0) hipLaunchKernelGGL(k_peak_stream<0>, grid, dim3(256), 0, st, A, B, Cc, D, n_vec, sink);
    else if (kind == 1) hipLaunchKernelGGL(k_peak_stream<1>, grid, dim3(256), 0, st, A, B, Cc, D, n_vec, sink);
    else hipLaunchKernelGGL(k_peak_stream<2>, grid, dim3(256), 0, st, A, B, Cc, D, n_vec, sink);
    return (int)hipGetLastError();
}

// `blocks` workgroups of eight waves (160 KB of LDS each, so one per CU)
// copy `stages` 32 KB stages each from src (src_bytes: a multiple of 32 KB,
// at most 2 GiB - 32 KB) into LDS.  Bytes per launch: blocks * stages *
// 32768.  clocks: 2 * blocks uint64, as for ma_peaks_mfma.
int ma_peaks_dma(const void* src, int64_t src_bytes, int64_t blocks, int stages,
                 uint64_t* clocks, void* stream) {
    if (!src || !clocks || blocks < 1 || stages < 1 || src_bytes < kDmaStage ||
        src_bytes % kDmaStage != 0 || src_bytes > 0x7fffffffLL)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_peak_dma, dim3((unsigned)blocks), dim3(kDmaWaves * 64), 0,
                       (hipStream_t)stream, (const char*)src, (uint32_t)src_bytes, stages, clocks);
    return (int)hipGetLastError();
}

}  // extern "C"
