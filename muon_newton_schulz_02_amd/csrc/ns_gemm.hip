// Newton-Schulz as grouped MFMA GEMMs on gfx950 (CDNA4).
//
// One NS step of every Muon matrix is three grouped launches, each covering
// all matrices of all shape buckets through a cost-ordered tile list:
//   GRAM  A = X X^T                      (r x r, K = c; upper tiles, mirrored)
//   POLY  B = b A + c (A A^T)            (r x r, K = r; A symmetric, mirrored)
//   XUPD  X = a X + B X                  (r x c, K = r; the right operand is
//                                          read from the transposed copy of X)
// and on the last step XUPD is replaced by FINAL, whose epilogue writes the
// parameter update p = p * decay - lr_eff * X back in the stored orientation.
//
// Every product is in "NT" form: both operands are read as rows whose
// reduction index is contiguous in memory, which is what the MFMA operand
// layout wants from LDS.  This is why the step keeps both X (row-major) and
// X^T as NS operands.  Operands are zero-padded to multiples of 256 in both
// dimensions, so no tile needs bounds checks.
//
// Method: OpenDM training-stack page, Muon/AdamW hybrid section, the
// Newton-Schulz paragraph (a few quintic Newton-Schulz steps on the whole
// matrix replace the SVD of the zeroth power) and the hyperparameter table
// (5 steps; update scaled by lr * muon_lr_scale * 0.2 * sqrt(max(shape))).
//
// bf16 mode: operands bf16 (round to nearest even), v_mfma_f32_32x32x16_bf16
// with fp32 accumulation; a float32 master X carries the linear a*X term.
// fp32 mode: v_mfma_f32_32x32x2_f32 on fp32 operands (no reduced-precision
// fp32 mode).

#include <hip/hip_runtime.h>

#include "ma_internal.h"

namespace ma {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { EPI_GRAM = 1, EPI_POLY = 2, EPI_XUPD = 3, EPI_FINAL = 4 };

// A lane contributes 16 bytes of one operand row per "k-group": 8 bf16 for
// one 32x32x16 MFMA, or 4 fp32 for four 32x32x2 MFMAs.  Inside a k-group the
// lane half h = lane / 32 holds k-offsets [16h, 16h + 16) bytes; A and B
// operands use the same assignment, so every product pairs matching k.
template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
    __device__ __forceinline__ static f32x16 run(uint4 a, uint4 b, f32x16 c) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
    }
};

template <>
struct Mma<float> {
    __device__ __forceinline__ static f32x16 run(uint4 a, uint4 b, f32x16 c) {
        const f32x4 av = __builtin_bit_cast(f32x4, a);
        const f32x4 bv = __builtin_bit_cast(f32x4, b);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[0], bv[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[1], bv[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[2], bv[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[3], bv[3], c, 0, 0, 0);
        return c;
    }
};

struct NsArgs {
    float a, b, c;
    int iter;
    int write_xb;
};

// 16 consecutive values of a row, to / from global memory.
__device__ __forceinline__ void store16(float* dst, const float* v) {
    float4* d4 = reinterpret_cast<float4*>(dst);
#pragma unroll
    for (int q = 0; q < 4; ++q) d4[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

__device__ __forceinline__ void store16(__bf16* dst, const float* v) {
    bf16x8 lo, hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] = (__bf16)v[e];
        hi[e] = (__bf16)v[8 + e];
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    d4[0] = __builtin_bit_cast(uint4, lo);
    d4[1] = __builtin_bit_cast(uint4, hi);
}

__device__ __forceinline__ void load16(const float* src, float* v) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 t = s4[q];
        v[4 * q] = t.x;
        v[4 * q + 1] = t.y;
        v[4 * q + 2] = t.z;
        v[4 * q + 3] = t.w;
    }
}

__device__ __forceinline__ void load16(const __bf16* src, float* v) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    const bf16x8 lo = __builtin_bit_cast(bf16x8, s4[0]);
    const bf16x8 hi = __builtin_bit_cast(bf16x8, s4[1]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        v[e] = (float)lo[e];
        v[8 + e] = (float)hi[e];
    }
}

// Make this wave's LDS writes visible to its other lanes before they read.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void lds_read16(const float* src, float* v) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 t = s4[q];
        v[4 * q] = t.x;
        v[4 * q + 1] = t.y;
        v[4 * q + 2] = t.z;
        v[4 * q + 3] = t.w;
    }
}

__device__ __forceinline__ void lds_write16(float* dst, const float* v) {
    float4* d4 = reinterpret_cast<float4*>(dst);
#pragma unroll
    for (int q = 0; q < 4; ++q) d4[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

// Stored-orientation update of 16 consecutive elements of parameter row
// `row`, starting at column `col`: p = p * decay - lr_eff * x (and the
// optional delta = lr_eff * x).
__device__ __forceinline__ void update_run(const MuonMat& d, int row, int col, const float* x) {
    if (row >= d.m || col >= d.n) return;
    float* p = reinterpret_cast<float*>(d.p) + (int64_t)row * d.n + col;
    float* dl = d.delta ? reinterpret_cast<float*>(d.delta) + (int64_t)row * d.n + col : nullptr;
    if (d.vec_ok && col + 16 <= d.n) {
        float pv[16], dv[16];
        load16(p, pv);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            dv[e] = d.lr_eff * x[e];
            pv[e] = fmaf(pv[e], d.decay, -dv[e]);
        }
        store16(p, pv);
        if (dl) store16(dl, dv);
    } else {
        const int cnt = min(16, d.n - col);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (e < cnt) {
                const float dv = d.lr_eff * x[e];
                p[e] = fmaf(p[e], d.decay, -dv);
                if (dl) dl[e] = dv;
            }
        }
    }
}

// Buffer resource of one operand: base address, extent in bytes (reads past
// it return zero) and the raw 32-bit-element format word of gfx9 parts.
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
    const int32_t n = bytes > 0x7fffffffLL ? 0x7fffffff : (int32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(Rsrc r, uint32_t voff, uint32_t soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return __builtin_bit_cast(uint4, v);
}

template <int VPT, int VP, int RPI>
__device__ __forceinline__ void stage_load(uint4 (&st)[VPT], Rsrc rp, Rsrc rq, uint32_t voff_p,
                                           uint32_t voff_q, uint32_t ldp, uint32_t ldq,
                                           uint32_t koff) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        if (i < VP) st[i] = buf_load16(rp, voff_p, koff + (uint32_t)(i * RPI) * ldp);
        else st[i] = buf_load16(rq, voff_q, koff + (uint32_t)((i - VP) * RPI) * ldq);
    }
}

template <int VPT, int RPI, int ROWB>
__device__ __forceinline__ void stage_store(const uint4 (&st)[VPT], char* lds, uint32_t lds_off) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) *reinterpret_cast<uint4*>(lds + i * RPI * ROWB + lds_off) = st[i];
}

// One k-group's operand fragments of a wave: MI rows-of-32 of P, NI of Q.
template <int MI, int NI, int ROWB>
__device__ __forceinline__ void lds_frags(uint4 (&af)[MI], uint4 (&bf)[NI], const char* a,
                                          const char* b, int koff) {
#pragma unroll
    for (int i = 0; i < MI; ++i) af[i] = *reinterpret_cast<const uint4*>(a + i * 32 * ROWB + koff);
#pragma unroll
    for (int j = 0; j < NI; ++j) bf[j] = *reinterpret_cast<const uint4*>(b + j * 32 * ROWB + koff);
}

template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_ns_gemm(
    const MuonMat* __restrict__ tab, const GemmTile* __restrict__ tiles, NsArgs args) {
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int ROWB = 128 + 16;                 // LDS row: 128 B of K + 16 B pad
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int VPT = (BM + BN) * 8 / NT;        // 16-byte vectors per thread per stage
    constexpr int VP = BM * 8 / NT;                // of which from P
    static_assert((BM + BN) * 8 % NT == 0 && BM * 8 % NT == 0, "loader split");
    constexpr int KELEM = 128 / (int)sizeof(T);    // K elements per stage
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const GemmTile tile = tiles[blockIdx.x];
    if (tile.mat < 0) return;  // padding of a shorter per-XCD list
    const MuonMat& d = tab[tile.mat];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const char* P;
    const char* Q;
    int64_t ldp, ldq;  // bytes
    int K, K_rows_p, K_rows_q;
    if (EPI == EPI_GRAM) {
        P = Q = reinterpret_cast<const char*>(d.xb);
        ldp = ldq = (int64_t)d.C * sizeof(T);
        K = d.C;
        K_rows_p = K_rows_q = d.R;
    } else if (EPI == EPI_POLY) {
        P = Q = reinterpret_cast<const char*>(d.a);
        ldp = ldq = (int64_t)d.R * sizeof(T);
        K = d.R;
        K_rows_p = K_rows_q = d.R;
    } else {
        P = reinterpret_cast<const char*>(d.b);
        Q = reinterpret_cast<const char*>(d.xt[args.iter & 1]);
        ldp = ldq = (int64_t)d.R * sizeof(T);
        K = d.R;
        K_rows_p = d.R;
        K_rows_q = d.C;
    }
    const int m0 = tile.tm * BM, n0 = tile.tn * BN;
    const int nk = K / KELEM;

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Global -> register -> LDS staging, double-buffered in LDS.  Thread t
    // moves 16-byte segment (t % 8) of rows t / 8 + RPI i (i < VPT) of the
    // stacked [P rows; Q rows] stage: one buffer load per row block, with the
    // per-thread offset in a VGPR and the row-block/stage offset in an SGPR.
    constexpr int RPI = NT / 8;  // rows covered per i
    const Rsrc rp = make_rsrc(P, (int64_t)(K_rows_p) * ldp);
    const Rsrc rq = make_rsrc(Q, (int64_t)(K_rows_q) * ldq);
    const uint32_t voff_p = (uint32_t)((m0 + (tid >> 3)) * ldp + (tid & 7) * 16);
    const uint32_t voff_q = (uint32_t)((n0 + (tid >> 3)) * ldq + (tid & 7) * 16);
    const uint32_t lds_off = (uint32_t)((tid >> 3) * ROWB + (tid & 7) * 16);
    uint4 stage[VPT];

    stage_load<VPT, VP, RPI>(stage, rp, rq, voff_p, voff_q, (uint32_t)ldp, (uint32_t)ldq, 0);
    stage_store<VPT, RPI, ROWB>(stage, smem, lds_off);
    __syncthreads();
    const int arow = (wm * WM + (lane & 31)) * ROWB + (lane >> 5) * 16;
    const int brow = (BM + wn * WN + (lane & 31)) * ROWB + (lane >> 5) * 16;
    for (int s = 0; s < nk; ++s) {
        if (s + 1 < nk)
            stage_load<VPT, VP, RPI>(stage, rp, rq, voff_p, voff_q, (uint32_t)ldp, (uint32_t)ldq,
                                     (uint32_t)(s + 1) * 128u);
        const char* base = smem + (s & 1) * STAGE;
        // fragments of k-group kg+1 are read from LDS while the MFMAs of
        // k-group kg run (two register sets), so LDS latency stays hidden
        uint4 af[2][MI], bfr[2][NI];
        lds_frags<MI, NI, ROWB>(af[0], bfr[0], base + arow, base + brow, 0);
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
            if (kg + 1 < 4)
                lds_frags<MI, NI, ROWB>(af[(kg + 1) & 1], bfr[(kg + 1) & 1], base + arow,
                                        base + brow, (kg + 1) * 32);
            // keep the prefetch above this k-group's MFMAs (the scheduler
            // would otherwise sink the reads next to their uses)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = Mma<T>::run(af[kg & 1][i], bfr[kg & 1][j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s + 1 < nk) stage_store<VPT, RPI, ROWB>(stage, smem + ((s + 1) & 1) * STAGE, lds_off);
        __syncthreads();
    }

    // ---- epilogue: each wave stages its 32x32 accumulator blocks in its own
    // LDS region (wave-level synchronisation only, no block barriers) and
    // moves them as 16-element runs: row runs for row-major outputs, column
    // runs for the transposed outputs ----
    constexpr int SLD = 36;  // staging row stride (floats): 16-byte aligned runs
    float* S = reinterpret_cast<float*>(smem) + wave * (32 * SLD);
    const bool mirror = (EPI == EPI_GRAM || EPI == EPI_POLY) && tile.tm != tile.tn;
    const bool need_cols = mirror || EPI == EPI_XUPD || (EPI == EPI_FINAL && d.transposed);
    T* out_direct = nullptr;
    int64_t ld_direct = 0;
    if (EPI == EPI_GRAM) {
        out_direct = reinterpret_cast<T*>(d.a);
        ld_direct = d.R;
    } else if (EPI == EPI_POLY) {
        out_direct = reinterpret_cast<T*>(d.b);
        ld_direct = d.R;
    }
    const int rrow = lane >> 1, rc0 = (lane & 1) * 16;   // row run of this lane
    const int ccol = lane & 31, cr0 = (lane >> 5) * 16;  // column run of this lane
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            // accumulator layout of a 32x32 MFMA block: register r of lane l
            // holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                S[row * SLD + (lane & 31)] = acc[i][j][r];
            }
            wave_lds_sync();
            const int bi = m0 + wm * WM + i * 32;  // block origin in the output
            const int bj = n0 + wn * WN + j * 32;
            {
                float v[16];
                lds_read16(S + rrow * SLD + rc0, v);
                const int gi = bi + rrow, gj = bj + rc0;
                if (EPI == EPI_GRAM) {
                    store16(out_direct + (int64_t)gi * ld_direct + gj, v);
                } else if (EPI == EPI_POLY) {
                    float av[16];
                    load16(reinterpret_cast<const T*>(d.a) + (int64_t)gi * d.R + gj, av);
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] = fmaf(args.b, av[e], args.c * v[e]);
                    store16(out_direct + (int64_t)gi * ld_direct + gj, v);
                } else {
                    float* x32 = reinterpret_cast<float*>(d.x32) + (int64_t)gi * d.C + gj;
                    float xv[16];
                    load16(x32, xv);
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] = fmaf(args.a, xv[e], v[e]);
                    if (EPI == EPI_XUPD) {
                        store16(x32, v);
                        if (args.write_xb) store16(reinterpret_cast<T*>(d.xb) + (int64_t)gi * d.C + gj, v);
                    } else if (!d.transposed) {
                        update_run(d, gi, gj, v);
                    }
                }
                if (need_cols) lds_write16(S + rrow * SLD + rc0, v);
            }
            wave_lds_sync();
            if (need_cols) {
                float v[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = S[(cr0 + e) * SLD + ccol];
                const int tr = bj + ccol, tc = bi + cr0;  // row / first column in the transposed view
                if (EPI == EPI_GRAM || EPI == EPI_POLY) {
                    store16(out_direct + (int64_t)tr * ld_direct + tc, v);
                } else if (EPI == EPI_XUPD) {
                    T* xt = reinterpret_cast<T*>(d.xt[(args.iter + 1) & 1]);
                    store16(xt + (int64_t)tr * d.R + tc, v);
                } else {
                    update_run(d, tr, tc, v);
                }
                wave_lds_sync();
            }
        }
    }
}

template <typename T, int EPI>
int launch_t(const MuonMat* tab, const GemmTile* tiles, int64_t n, const NsArgs& a, hipStream_t st) {
    constexpr int BM = 256, BN = 256, WM = 128, WN = 128;
    static_assert(BM == kGemmTile && BN == kGemmTile, "tile lists are built for kGemmTile");
    hipLaunchKernelGGL((k_ns_gemm<T, BM, BN, WM, WN, EPI>), dim3((unsigned)n),
                       dim3((BM / WM) * (BN / WN) * 64), 0, st, tab, tiles, a);
    return (int)hipGetLastError();
}

}  // namespace

int launch_ns_phase(int phase, int32_t group, const MuonMat* tab, const GemmTile* tiles,
                    int64_t n_tiles, int iter, int last, const StepScalars& s, void* stream) {
    if (n_tiles == 0) return (int)hipSuccess;
    NsArgs a{s.ns_a, s.ns_b, s.ns_c, iter, group == kGroupBf16 ? 1 : 0};
    hipStream_t st = (hipStream_t)stream;
    const int epi = phase == 1 ? EPI_GRAM : phase == 2 ? EPI_POLY : (last ? EPI_FINAL : EPI_XUPD);
    if (group == kGroupBf16) {
        switch (epi) {
            case EPI_GRAM: return launch_t<__bf16, EPI_GRAM>(tab, tiles, n_tiles, a, st);
            case EPI_POLY: return launch_t<__bf16, EPI_POLY>(tab, tiles, n_tiles, a, st);
            case EPI_XUPD: return launch_t<__bf16, EPI_XUPD>(tab, tiles, n_tiles, a, st);
            default: return launch_t<__bf16, EPI_FINAL>(tab, tiles, n_tiles, a, st);
        }
    }
    switch (epi) {
        case EPI_GRAM: return launch_t<float, EPI_GRAM>(tab, tiles, n_tiles, a, st);
        case EPI_POLY: return launch_t<float, EPI_POLY>(tab, tiles, n_tiles, a, st);
        case EPI_XUPD: return launch_t<float, EPI_XUPD>(tab, tiles, n_tiles, a, st);
        default: return launch_t<float, EPI_FINAL>(tab, tiles, n_tiles, a, st);
    }
}

}  // namespace ma
