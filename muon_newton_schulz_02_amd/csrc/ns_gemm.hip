// Newton-Schulz as grouped MFMA GEMMs on gfx950 (CDNA4).
//
// One NS step of every Muon matrix is three grouped launches, each covering
// all matrices of all shape buckets through an XCD-aware tile list:
//   GRAM  A = X X^T                      (r x r, K = c; upper tiles, mirrored)
//   POLY  B = b A + c (A A^T)            (r x r, K = r; A symmetric, mirrored)
//   XUPD  X = a X + B X                  (r x c, K = r)
// and on the last step XUPD is replaced by FINAL, whose epilogue writes the
// parameter update p = p * decay - rate * X back in the stored orientation.
// A launch with fewer fp32 Gram tiles than CUs runs each of those Gram
// reductions as up to four column slices (slice 0 writes A, the others
// partial Grams that k_gram_reduce adds to A in slice order).
//
// MFMA operands are read from LDS as rows whose reduction index is
// contiguous.  For GRAM and POLY both operands are such rows of a row-major
// matrix.  For B X the right operand is X with the reduction index along its
// rows:
//   * bf16: X is kept row-major (in 32x32 blocks) only, and its fragments
//     are read out of LDS with transposing loads (ds_read_b64_tr_b16);
//   * fp32: a transposed copy X^T is kept and read directly.
// Operands are zero-padded to multiples of 256 in both dimensions, so no
// tile needs bounds checks.
//
// Three kernel families, one launch group each:
//   * bf16 operands: a workgroup of eight waves (two per SIMD, 128 x 64
//     each) computes one 256 x 256 output tile; operands stream through a
//     ring of five 32 KB LDS stages, copied by buffer loads straight into
//     LDS four stages ahead (ns_gemm_tile_w8);
//   * fp32 operands: four waves (one per SIMD, 128 x 128 each, accumulators
//     in the 256 AGPRs) per 256 x 256 tile, a ring of four stages copied
//     three ahead, each stage's fragment reads and copies placed between its
//     matrix instructions since a SIMD holds only this one wave
//     (ns_gemm_tile);
//   * small fp32 matrices (at most 256 padded rows): 32 x 32 Gram and square
//     tiles with a four-way split reduction and 64 x 64 X-update tiles
//     (ns_gemm_tile_s32, ns_xupd_tile_s64).
// Every epilogue stages each 32 x 32 accumulator block through the wave's
// own LDS region and writes it in 16-byte runs (whole 1 KB halves of a
// 2 KB block for the bf16 X update).
//
// Method: OpenDM training-stack page, Muon/AdamW hybrid section, the
// Newton-Schulz paragraph (a few quintic Newton-Schulz steps on the whole
// matrix replace the SVD of the zeroth power) and the hyperparameter table
// (5 steps; update scaled by lr * muon_lr_scale * 0.2 * sqrt(max(shape))).
//
// bf16 mode: operands bf16 (round to nearest even), v_mfma_f32_32x32x16_bf16
// with fp32 accumulation.  The linear a*X term uses a master copy of X held
// as a pair of bf16 values (hi = bf16(x), lo = bf16(x - hi): a 16-bit
// mantissa), and hi is itself the MFMA operand.  Only the first kNsLoIters
// iterations take the linear term from hi + lo: later ones use hi alone, so
// the lo half of their X is neither written nor read.  The 16-bit master
// matters while the smallest singular values are still small (an
// ill-conditioned input loses them to a bf16-only X); after three
// iterations they have grown enough.
// fp32 mode: v_mfma_f32_32x32x2_f32 on fp32 operands (no reduced-precision
// fp32 mode), master X in fp32.

#include <hip/hip_runtime.h>

#include <utility>

#include "ma_internal.h"

namespace ma {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { EPI_GRAM = 1, EPI_POLY = 2, EPI_XUPD = 3, EPI_FINAL = 4 };

// Element offset of (i, j) in a bf16 operand (X hi and lo, A, B) with C
// columns: 32x32 blocks of 2 KB, row-major inside a block and
// block-row-major outside, so the epilogue's 32-byte row (or column) runs of
// a block form one contiguous 2 KB write and every 64-byte stage row the
// loaders copy stays contiguous.
__device__ __forceinline__ int64_t xblk(int i, int j, int C) {
    return ((int64_t)(i >> 5) * (C >> 5) + (j >> 5)) * 1024 + (i & 31) * 32 + (j & 31);
}

// Offset of (i, j) in an epilogue output or input of operand type T with
// leading dimension ld: blocked for bf16, row-major for fp32.
template <typename T>
__device__ __forceinline__ int64_t op_off(int i, int j, int64_t ld) {
    return sizeof(T) == 2 ? xblk(i, j, (int)ld) : (int64_t)i * ld + j;
}

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
    int use_lo;     // bf16: this iteration's linear term reads the lo half of X
    int write_lo;   // bf16 X update: the next X keeps its lo half
    // per matrix 1 / (||u||_F + eps): the input operand is u itself, so the
    // first Gram scales by its square and the first X update by it
    const float* scales;
    // the step's Muon rate and decay, read by the last X update
    const StepDev* sd;
};

// A matrix's parameter update p = p * decay - rate * X.
struct Upd {
    float rate, decay;
};

// Global-memory accesses through address-space-1 pointers, so they are
// counted on vmcnt only (flat accesses also count on lgkmcnt, which would
// make every LDS wait of the epilogue wait for them too).
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) v4u32 g_v4u32;
typedef __attribute__((address_space(1))) float g_float;

__device__ __forceinline__ uint4 gld(const void* p) {
    return __builtin_bit_cast(uint4, *(const g_v4u32*)p);
}
__device__ __forceinline__ void gst(void* p, uint4 v) { *(g_v4u32*)p = __builtin_bit_cast(v4u32, v); }

// 16 consecutive values of a row, to / from global memory.
__device__ __forceinline__ void store16(float* dst, const float* v) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
        gst(dst + 4 * q, __builtin_bit_cast(uint4, make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3])));
}

__device__ __forceinline__ void store16(__bf16* dst, const float* v) {
    bf16x8 lo, hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] = (__bf16)v[e];
        hi[e] = (__bf16)v[8 + e];
    }
    gst(dst, __builtin_bit_cast(uint4, lo));
    gst(dst + 8, __builtin_bit_cast(uint4, hi));
}

__device__ __forceinline__ void load16(const float* src, float* v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 t = __builtin_bit_cast(float4, gld(src + 4 * q));
        v[4 * q] = t.x;
        v[4 * q + 1] = t.y;
        v[4 * q + 2] = t.z;
        v[4 * q + 3] = t.w;
    }
}

__device__ __forceinline__ void load16(const __bf16* src, float* v) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bf16x8 t = __builtin_bit_cast(bf16x8, gld(src + 8 * h));
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * h + e] = (float)t[e];
    }
}

// Split 16 fp32 values into bf16 hi = RNE(x) and lo = RNE(x - hi).
__device__ __forceinline__ void store16_hilo(__bf16* dhi, __bf16* dlo, const float* v) {
    float lo[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) lo[e] = v[e] - (float)(__bf16)v[e];
    store16(dhi, v);
    store16(dlo, lo);
}

__device__ __forceinline__ void store8_hilo(__bf16* dhi, __bf16* dlo, const float* v) {
    bf16x8 h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = (__bf16)v[e];
        l[e] = (__bf16)(v[e] - (float)h[e]);
    }
    gst(dhi, __builtin_bit_cast(uint4, h));
    gst(dlo, __builtin_bit_cast(uint4, l));
}

__device__ __forceinline__ void store8_hi(__bf16* dhi, const float* v) {
    bf16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (__bf16)v[e];
    gst(dhi, __builtin_bit_cast(uint4, h));
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


// Buffer resource of one operand (gfx9 layout): base address, stride 0,
// extent in bytes (reads past it return zero) and the raw 32-bit-element
// format word.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 make_rsrc(const void* base, int64_t bytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t n = bytes > 0x7fffffffLL ? 0x7fffffffu : (uint32_t)bytes;
    u32x4 r;
    r.x = (uint32_t)a;
    r.y = (uint32_t)(a >> 32) & 0xffffu;
    r.z = n;
    r.w = 0x00020000u;
    return r;
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16 bytes per lane from global memory straight into LDS: lane t of the wave
// writes bytes [lds + 16 t, lds + 16 t + 16).  Issued as inline assembly so
// the compiler's own wait-count insertion does not treat every later LDS
// read as dependent on it (it cannot tell the stage buffers apart); the
// kernel orders these copies itself with explicit vmcnt waits and barriers.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// ---------------------------------------------------------------------------
// Shared-memory staging of the operands.
//
// A stage holds 64 bytes of the reduction index for the 256 rows of each
// operand: P (rows of the left operand) in the first 16 KB, Q in the second.
// Four stage buffers (128 KB of LDS) form a ring; global memory is
// copied straight into them with buffer loads that write LDS (no register
// staging), three stages ahead of the multiply.
//
// Row-operand layout (rows whose reduction index is contiguous): row r of a
// region at r * 64 bytes, its 16-byte chunk c at slot c ^ ((r >> 2) & 3), so
// the 16 rows read by each quarter of a wave's 128-bit fragment loads fall
// in distinct banks.
//
// Transposed-operand layout (bf16 X of B X, reduction index along X's rows):
// the region holds 32 rows of X (the stage's reduction range) by the tile's
// 256 columns, row k at k * 512 bytes and chunk c at slot c ^ ((k & 3) << 2).
// Fragments are read with the gfx950 transposing LDS load (ds_read_b64_tr_b16):
// within each 16-lane group, lane i receives element i % 4 of the 8-byte
// pieces addressed by lanes i / 4 + 4 e, e = 0..3, so pointing the 16 lanes
// at four consecutive rows by four 4-column pieces hands every lane one
// column of four consecutive rows.
// ---------------------------------------------------------------------------
constexpr int kStageBytes = 32768;
constexpr int kRegionBytes = 16384;
constexpr int kRowBytes = 64;   // reduction bytes per row per stage
constexpr int kStages = 4;      // ring depth: copies run kStages - 1 stages ahead

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_tr8(const char* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(uint2, v);
}

// s_waitcnt with only the vector-memory counter constrained (expcnt and
// lgkmcnt at their maxima): vmcnt(n) for n in {0, 4, 8, 12, 16, 24}.  The 6-bit
// count is split into bits [3:0] and [15:14] of the immediate.
__device__ __forceinline__ void wait_vm(int n) {
    if (n <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (n == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
    else if (n == 8) __builtin_amdgcn_s_waitcnt(0x0F78);
    else if (n == 12) __builtin_amdgcn_s_waitcnt(0x0F7C);
    else if (n == 16) __builtin_amdgcn_s_waitcnt(0x4F70);
    else __builtin_amdgcn_s_waitcnt(0x4F78);
}

// Workgroup barrier that orders this wave's LDS accesses around it without
// waiting for outstanding LDS copies (a release fence would drain them all).
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_sched_barrier(0);
}

// Global inputs of one epilogue block's row run, loaded ahead of time: the
// polynomial step's A values (fp32, or bf16 with c = 0), the lo half of the
// bf16 master X, or the fp32 master X.  At most 64 bytes per lane.
struct EpiIn {
    uint4 q[4];
};

// The parameter run a lane of the final update rewrites for one block,
// loaded two blocks ahead: 16 values (fp32 or bf16) of stored row `row` from
// column `col`, where the update takes its 16-byte path.
struct PIn {
    uint4 v[4];
};

__device__ __forceinline__ bool p_run_vec(const MuonMat& d, int row, int col) {
    return row < d.m && d.vec_ok && col + 16 <= d.n;
}

// Stored coordinates of a lane's run: a row run of the block (lanes 2r and
// 2r + 1 share row r) or, for a transposed matrix, a column run of it.
__device__ __forceinline__ void p_run_at(const MuonMat& d, int lane, int bi, int bj, int& row,
                                         int& col) {
    if (d.transposed) {
        row = bj + (lane & 31);
        col = bi + (lane >> 5) * 16;
    } else {
        row = bi + (lane >> 1);
        col = bj + (lane & 1) * 16;
    }
}

template <int EPI>
__device__ __forceinline__ void p_load(PIn& pin, const MuonMat& d, int lane, int bi, int bj) {
    if (EPI != EPI_FINAL) return;
    int row, col;
    p_run_at(d, lane, bi, bj, row, col);
    if (!p_run_vec(d, row, col)) return;
    const int64_t o = (int64_t)row * d.n + col;
    // both storages write every slot, so no slot index depends on the storage
    // (a merged tail would index the slots at run time, through scratch)
    if (d.p_bf16) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const __bf16*>(d.p) + o);
        const uint4 a = gld(p), b = gld(p + 1);
        pin.v[0] = a;
        pin.v[1] = b;
        pin.v[2] = make_uint4(0u, 0u, 0u, 0u);
        pin.v[3] = make_uint4(0u, 0u, 0u, 0u);
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(d.p) + o);
        const uint4 a = gld(p), b = gld(p + 1), c = gld(p + 2), e = gld(p + 3);
        pin.v[0] = a;
        pin.v[1] = b;
        pin.v[2] = c;
        pin.v[3] = e;
    }
}

template <typename T, int EPI>
__device__ __forceinline__ void epi_load(EpiIn& in, const MuonMat& d, int lane, int bi, int bj,
                                         int cur, bool poly_direct, bool use_lo) {
    constexpr bool BF = sizeof(T) == 2;
    const int gi = bi + (lane >> 1), gj = bj + (lane & 1) * 16;
    if (EPI == EPI_POLY) {
        if (!poly_direct) {
            const uint4* a = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(d.a) +
                                                            op_off<T>(gi, gj, d.R));
#pragma unroll
            for (int q = 0; q < (BF ? 2 : 4); ++q) in.q[q] = gld(a + q);
        }
    } else if (EPI == EPI_XUPD || EPI == EPI_FINAL) {
        if (BF && !use_lo) {
            // the linear term takes X's hi half alone (already in the
            // accumulators): nothing to load
        } else if (BF && EPI == EPI_XUPD) {
            const int lr = lane >> 2, lc = (lane & 3) * 8;
            const __bf16* lo = reinterpret_cast<const __bf16*>(d.xlo[cur]);
            in.q[0] = gld(lo + xblk(bi + lr, bj + lc, d.C));
            in.q[1] = gld(lo + xblk(bi + lr + 16, bj + lc, d.C));
        } else if (BF) {
            const uint4* lo =
                reinterpret_cast<const uint4*>(reinterpret_cast<const __bf16*>(d.xlo[cur]) + xblk(gi, gj, d.C));
            in.q[0] = gld(lo);
            in.q[1] = gld(lo + 1);
        } else {
            const int64_t o = (int64_t)gi * d.C + gj;
            const uint4* x = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(d.x[0]) + o);
#pragma unroll
            for (int q = 0; q < 4; ++q) in.q[q] = gld(x + q);
        }
    }
}

__device__ __forceinline__ void unpack16(const uint4* q, float* v, bool bf) {
    if (bf) {
        const bf16x8 lo = __builtin_bit_cast(bf16x8, q[0]);
        const bf16x8 hi = __builtin_bit_cast(bf16x8, q[1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[e] = (float)lo[e];
            v[8 + e] = (float)hi[e];
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 t = __builtin_bit_cast(float4, q[k]);
            v[4 * k] = t.x;
            v[4 * k + 1] = t.y;
            v[4 * k + 2] = t.z;
            v[4 * k + 3] = t.w;
        }
    }
}

template <typename P>
__device__ __forceinline__ void update_run_as(const MuonMat& d, const Upd& u, int row, int col,
                                              const float* x, const uint4* pre) {
    const int64_t o = (int64_t)row * d.n + col;
    P* p = reinterpret_cast<P*>(d.p) + o;
    float* dl = d.delta ? reinterpret_cast<float*>(d.delta) + o : nullptr;
    if (d.vec_ok && col + 16 <= d.n) {
        // the run was prefetched (p_load takes the same path)
        float pv[16], dv[16];
        unpack16(pre, pv, sizeof(P) == 2);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            dv[e] = u.rate * x[e];
            pv[e] = fmaf(pv[e], u.decay, -dv[e]);
        }
        store16(p, pv);
        if (dl) store16(dl, dv);
    } else {
        const int cnt = min(16, d.n - col);
        typedef __attribute__((address_space(1))) P g_P;
        g_P* gp = (g_P*)p;
        g_float* gd = (g_float*)dl;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (e < cnt) {
                const float dv = u.rate * x[e];
                gp[e] = (P)fmaf((float)gp[e], u.decay, -dv);
                if (dl) gd[e] = dv;
            }
        }
    }
}

// Stored-orientation update of 16 consecutive elements of parameter row
// `row`, starting at column `col`: p = p * decay - rate * x (and the
// optional delta = rate * x), with p stored as float or bf16 (rounded to
// nearest even once).  `pre` holds the run's old values where p_load
// prefetched them.
__device__ __forceinline__ void update_run(const MuonMat& d, const Upd& u, int row, int col,
                                           const float* x, const PIn& pre) {
    if (row >= d.m || col >= d.n) return;
    if (d.p_bf16) update_run_as<__bf16>(d, u, row, col, x, pre.v);
    else update_run_as<float>(d, u, row, col, x, pre.v);
}

// Epilogue of one 32x32 accumulator block at output rows bi.., columns
// bj..: stage it in the wave's LDS region, then move 16-element row runs
// (row-major outputs) and, where needed, column runs (transposed outputs).
// In bf16 the linear terms a X (update steps) and b A (polynomial step,
// c != 0) are already in the accumulators, except the lo half of the master
// X, which arrives in `in`; in fp32 they are added here from `in`.  Called with literal block indices so the accumulators
// stay in registers.
template <typename T, int EPI, int SLD>
__device__ __forceinline__ void epi_block(const f32x16& blk, const EpiIn& in, const PIn& pin,
                                          const MuonMat& d,
                                          float* S, const NsArgs& args, float escale,
                                          const Upd& up, int lane,
                                          int bi, int bj, int cur, bool need_cols,
                                          bool poly_direct, T* out_direct, int64_t ld_direct) {
    constexpr bool BF = sizeof(T) == 2;
    const int rrow = lane >> 1, rc0 = (lane & 1) * 16;   // row run of this lane
    const int ccol = lane & 31, cr0 = (lane >> 5) * 16;  // column run of this lane
    // accumulator layout of a 32x32 MFMA block: register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        S[row * SLD + (lane & 31)] = blk[r];
    }
    wave_lds_sync();
    {
        float v[16];
        // bf16 X update: a lane takes 8 values of rows r and r + 16 of the
        // block, so each store instruction covers a contiguous 1 KB half of
        // the 2 KB block (with 16-element row runs every 128-byte line took
        // two instructions; this cut the epilogue per tile 15.3 -> 10.4 us)
        constexpr bool LINES = EPI == EPI_XUPD && BF;
        const int lr = LINES ? lane >> 2 : rrow, lc = LINES ? (lane & 3) * 8 : rc0;
        if (LINES) {
            const float4* a = reinterpret_cast<const float4*>(S + lr * SLD + lc);
            const float4* b = reinterpret_cast<const float4*>(S + (lr + 16) * SLD + lc);
            const float4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
            v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
            v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
            v[8] = b0.x; v[9] = b0.y; v[10] = b0.z; v[11] = b0.w;
            v[12] = b1.x; v[13] = b1.y; v[14] = b1.z; v[15] = b1.w;
        } else {
            lds_read16(S + rrow * SLD + rc0, v);
        }
        const int gi = bi + lr, gj = bj + lc;
        const int64_t o = (int64_t)gi * d.C + gj;
        if (EPI == EPI_GRAM) {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] *= escale;
            store16(out_direct + op_off<T>(gi, gj, ld_direct), v);
        } else if (EPI == EPI_POLY) {
            if (poly_direct) {
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = args.c * v[e];
            } else {
                float av[16];
                unpack16(in.q, av, BF);
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = fmaf(args.b, av[e], args.c * v[e]);
            }
            store16(out_direct + op_off<T>(gi, gj, ld_direct), v);
        } else if (BF) {
            // a * lo of the master X where this iteration uses it; a * hi was
            // added in the main loop
            if (args.use_lo) {
                float lv[16];
                unpack16(in.q, lv, true);
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] = escale * fmaf(args.a, lv[e], v[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) v[e] *= escale;
            }
            if (EPI == EPI_XUPD) {
                const int64_t o0 = xblk(gi, gj, d.C), o1 = xblk(gi + 16, gj, d.C);
                __bf16* hi = reinterpret_cast<__bf16*>(d.x[cur ^ 1]);
                if (args.write_lo) {
                    __bf16* lo = reinterpret_cast<__bf16*>(d.xlo[cur ^ 1]);
                    store8_hilo(hi + o0, lo + o0, v);
                    store8_hilo(hi + o1, lo + o1, v + 8);
                } else {
                    store8_hi(hi + o0, v);
                    store8_hi(hi + o1, v + 8);
                }
            } else if (!d.transposed) {
                update_run(d, up, gi, gj, v, pin);
            }
        } else {
            float xv[16];
            unpack16(in.q, xv, false);
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = escale * fmaf(args.a, xv[e], v[e]);
            if (EPI == EPI_XUPD) {
                store16(reinterpret_cast<float*>(d.x[0]) + o, v);
            } else if (!d.transposed) {
                update_run(d, up, gi, gj, v, pin);
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
            store16(out_direct + op_off<T>(tr, tc, ld_direct), v);
        } else if (EPI == EPI_XUPD) {
            T* xt = reinterpret_cast<T*>(d.xt[cur ^ 1]);
            store16(xt + (int64_t)tr * d.R + tc, v);
        } else {
            update_run(d, up, tr, tc, v, pin);
        }
        wave_lds_sync();
    }
}

// Per-lane addressing of one tile's operands: LDS copy offsets (voffset of
// the buffer loads; the stage and row-block parts go in soffset) and the
// fragment offsets inside a stage buffer.
struct Addr {
    uint32_t dma_p;          // P copy: this lane's row and chunk
    uint32_t dma_q[2];       // Q copy (row operand: [0]; transposed: even / odd loads)
    uint32_t frag_a[2];      // A fragment of row block 0, per k-group
    uint32_t frag_b[2];      // B fragment (row operand) of column block 0, per k-group
    uint32_t frag_t[4];      // B fragment (transposed), per column block, k-group 0
    uint32_t lin_t[4];       // linear-term reads (transposed), per column block
    uint32_t lin_r[4];       // linear-term reads (row operand) of column block 0, per quarter
};

// PB / QB: that operand is a bf16 X in 32x32 blocks (xblk), whose row
// pitch ld covers one row of a block row: a block row spans 32 ld, a stage
// (32 columns) one 2 KB block, and rows 16..31 of a block start 1 KB in.
// Part i (0..3) of the copy of stage s: one 1 KB load of P rows, or of Q.
template <typename T, bool PB>
__device__ __forceinline__ void stage_copy_p(uint32_t buf, u32x4 rp, const Addr& ad,
                                             uint32_t wbase, int s, int i, uint32_t ldp) {
    dma16(rp, buf + wbase + i * 1024, ad.dma_p,
          PB ? (uint32_t)s * 2048 + (uint32_t)(i >> 1) * 32 * ldp + (uint32_t)(i & 1) * 1024
             : (uint32_t)s * kRowBytes + (uint32_t)(i * 16) * ldp);
}

template <typename T, bool QT, bool QB>
__device__ __forceinline__ void stage_copy_q(uint32_t buf, u32x4 rq, const Addr& ad,
                                             uint32_t wbase, int s, int i, uint32_t ldq) {
    constexpr int KE = kRowBytes / (int)sizeof(T);
    if (QT)
        dma16(rq, buf + kRegionBytes + wbase + i * 1024, ad.dma_q[i & 1],
              QB ? (uint32_t)s * 32 * ldq + (uint32_t)(2 * i) * 64
                 : ((uint32_t)s * KE + (uint32_t)(2 * i)) * ldq);
    else
        dma16(rq, buf + kRegionBytes + wbase + i * 1024, ad.dma_q[0],
              QB ? (uint32_t)s * 2048 + (uint32_t)(i >> 1) * 32 * ldq + (uint32_t)(i & 1) * 1024
                 : (uint32_t)s * kRowBytes + (uint32_t)(i * 16) * ldq);
}

template <typename T, bool QT, bool PB, bool QB>
__device__ __forceinline__ void stage_copy(uint32_t buf, u32x4 rp, u32x4 rq, const Addr& ad,
                                           uint32_t wbase, int s, uint32_t ldp, uint32_t ldq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) stage_copy_p<T, PB>(buf, rp, ad, wbase, s, i, ldp);
#pragma unroll
    for (int i = 0; i < 4; ++i) stage_copy_q<T, QT, QB>(buf, rq, ad, wbase, s, i, ldq);
}

// One k-group's fragments of a wave: four row blocks of P, four column
// blocks of Q.
template <bool QT>
__device__ __forceinline__ void stage_frags(uint4 (&fa)[4], uint4 (&fb)[4], const char* buf,
                                            const Addr& ad, int kg) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const uint4*>(buf + ad.frag_a[kg] + i * 2048);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (QT) {
            const char* p = buf + ad.frag_t[j] + kg * 16 * 512;
            const uint2 lo = lds_tr8(p), hi = lds_tr8(p + 4 * 512);
            fb[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
            fb[j] = *reinterpret_cast<const uint4*>(buf + ad.frag_b[kg] + j * 2048);
        }
    }
}

// Linear term of the update and polynomial steps, added while its values sit
// in the stage buffer: the output row of accumulator block row IB equals the
// reduction index of the stage (update: X[i][j] is Q's row i; polynomial:
// A[i][j] = A[j][i] is Q's row j at reduction index i).  A bf16 stage covers
// one 32-row block (quarters Q = 0..3 of the block's registers), an fp32
// stage half of one (quarters 2 H, 2 H + 1).
template <typename T, bool QT, int IB, int H>
__device__ __forceinline__ void stage_linear(f32x16 (&acc)[4][4], const char* buf, const Addr& ad,
                                             float scale) {
    constexpr bool BF = sizeof(T) == 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < (BF ? 4 : 2); ++q) {
            float v[4];
            if (QT) {
                const uint2 w = lds_tr8(buf + ad.lin_t[j] + q * 8 * 512);
                const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(w.x, w.y, 0u, 0u));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (float)b[e];
            } else if (BF) {
                const uint2 w = *reinterpret_cast<const uint2*>(buf + ad.lin_r[q] + j * 2048);
                const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(w.x, w.y, 0u, 0u));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (float)b[e];
            } else {
                const float4 w = *reinterpret_cast<const float4*>(buf + ad.lin_r[q] + j * 2048);
                v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
            }
            const int qq = BF ? q : 2 * H + q;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[IB][j][4 * qq + e] = fmaf(scale, v[e], acc[IB][j][4 * qq + e]);
        }
    }
}

template <typename T, bool QT, int IB>
__device__ __forceinline__ void stage_linear_h(f32x16 (&acc)[4][4], const char* buf, const Addr& ad,
                                               float scale, int h) {
    if (sizeof(T) == 2 || h == 0) stage_linear<T, QT, IB, 0>(acc, buf, ad, scale);
    else stage_linear<T, QT, IB, 1>(acc, buf, ad, scale);
}

template <typename T, bool QT>
__device__ __forceinline__ void stage_linear_at(f32x16 (&acc)[4][4], const char* buf, const Addr& ad,
                                                float scale, int rel) {
    // rel = first reduction index of the stage minus the wave's first output
    // row; the stage contributes when 0 <= rel < 128
    if (rel < 0 || rel >= 128) return;
    const int h = (rel >> 4) & 1;
    switch (rel >> 5) {
        case 0: stage_linear_h<T, QT, 0>(acc, buf, ad, scale, h); break;
        case 1: stage_linear_h<T, QT, 1>(acc, buf, ad, scale, h); break;
        case 2: stage_linear_h<T, QT, 2>(acc, buf, ad, scale, h); break;
        default: stage_linear_h<T, QT, 3>(acc, buf, ad, scale, h); break;
    }
}

// One stage of the main loop: k-group 0 (fragments already in fa/fb), the
// barrier that publishes stage s + 1 and recycles the buffer of stage s - 1,
// the linear term, then k-group 1 with the copy of stage s + kStages - 1 into
// the recycled buffer and the k-group-0 fragments of stage s + 1.  Each
// memory instruction sits between two matrix instructions (pinned by
// scheduling barriers), so a SIMD's one wave keeps its matrix core fed while
// it issues them: the main loop took 7-13 % less time than with the memory
// instructions grouped ahead of the matrix ones.
template <typename T, bool QT, bool LIN, bool PB, bool QB>
__device__ __forceinline__ void stage_step(f32x16 (&acc)[4][4], uint4 (&fa)[4], uint4 (&fb)[4],
                                           const char* cur, const char* nxt, uint32_t tgt, u32x4 rp,
                                           u32x4 rq, const Addr& ad, uint32_t wbase, int s, int nk,
                                           uint32_t ldp, uint32_t ldq, float scale, int rel0) {
    constexpr int KE = kRowBytes / (int)sizeof(T);
    uint4 ga[4], gb[4];
    // k-group 0, with the k-group-1 fragment reads in between
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i][0] = Mma<T>::run(fa[i], fb[0], acc[i][0]);
        __builtin_amdgcn_sched_barrier(0);
        ga[i] = *reinterpret_cast<const uint4*>(cur + ad.frag_a[1] + i * 2048);
        __builtin_amdgcn_sched_barrier(0);
        acc[i][1] = Mma<T>::run(fa[i], fb[1], acc[i][1]);
        __builtin_amdgcn_sched_barrier(0);
        if (QT) {
            const char* p = cur + ad.frag_t[i] + 16 * 512;
            const uint2 lo = lds_tr8(p), hi = lds_tr8(p + 4 * 512);
            gb[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
            gb[i] = *reinterpret_cast<const uint4*>(cur + ad.frag_b[1] + i * 2048);
        }
        __builtin_amdgcn_sched_barrier(0);
        acc[i][2] = Mma<T>::run(fa[i], fb[2], acc[i][2]);
        acc[i][3] = Mma<T>::run(fa[i], fb[3], acc[i][3]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // stage s + 1 has landed once only the copies of the stages after it
    // (at most kStages - 3 of them, 8 loads each) are outstanding.  Every
    // stage takes the barrier and reads the next k-group-0 fragments (after
    // the last stage they are unused reads of a stale buffer), so the code
    // has no join point that would blur the LDS wait counts.
    wait_vm(8 * min(nk - 2 - s, kStages - 3));
    stage_barrier();
    if (LIN) stage_linear_at<T, QT>(acc, cur, ad, scale, rel0 + s * KE);
    __builtin_amdgcn_sched_barrier(0);
    const bool cp = s + kStages - 1 < nk;
    const int sc = s + kStages - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i][0] = Mma<T>::run(ga[i], gb[0], acc[i][0]);
        __builtin_amdgcn_sched_barrier(0);
        if (cp) stage_copy_p<T, PB>(tgt, rp, ad, wbase, sc, i, ldp);
        __builtin_amdgcn_sched_barrier(0);
        acc[i][1] = Mma<T>::run(ga[i], gb[1], acc[i][1]);
        __builtin_amdgcn_sched_barrier(0);
        if (cp) stage_copy_q<T, QT, QB>(tgt, rq, ad, wbase, sc, i, ldq);
        __builtin_amdgcn_sched_barrier(0);
        acc[i][2] = Mma<T>::run(ga[i], gb[2], acc[i][2]);
        __builtin_amdgcn_sched_barrier(0);
        fa[i] = *reinterpret_cast<const uint4*>(nxt + ad.frag_a[0] + i * 2048);
        __builtin_amdgcn_sched_barrier(0);
        acc[i][3] = Mma<T>::run(ga[i], gb[3], acc[i][3]);
        __builtin_amdgcn_sched_barrier(0);
        if (QT) {
            const char* p = nxt + ad.frag_t[i];
            const uint2 lo = lds_tr8(p), hi = lds_tr8(p + 4 * 512);
            fb[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
            fb[i] = *reinterpret_cast<const uint4*>(nxt + ad.frag_b[0] + i * 2048);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Stages s .. s + kStages - 1 of the main loop, stage s + B in ring slot B.
template <typename T, bool QT, bool LIN, bool PB, bool QB, int... B>
__device__ __forceinline__ void ring_round(std::integer_sequence<int, B...>, f32x16 (&acc)[4][4],
                                           uint4 (&fa)[4], uint4 (&fb)[4], const char* ring,
                                           uint32_t lring, u32x4 rp, u32x4 rq, const Addr& ad,
                                           uint32_t wbase, int s, int nk, uint32_t ldp,
                                           uint32_t ldq, float scale, int rel0) {
    // nk is a multiple of 8, so a ring depth dividing 8 needs no guard
    (((8 % kStages == 0 || s + B < nk)
          ? stage_step<T, QT, LIN, PB, QB>(acc, fa, fb, ring + B * kStageBytes,
                                   ring + ((B + 1) % kStages) * kStageBytes,
                                   lring + ((B + kStages - 1) % kStages) * kStageBytes, rp, rq,
                                   ad, wbase, s + B, nk, ldp, ldq, scale, rel0)
          : void()),
     ...);
}

template <typename T, int EPI>
__device__ __forceinline__ void ns_gemm_tile(const MuonMat* __restrict__ tab,
                                             const GemmTile* __restrict__ tiles, const NsArgs& args) {
    constexpr bool BF = sizeof(T) == 2;
    // B X in bf16 reads X row-major through the transposing LDS loads
    constexpr bool QT = BF && (EPI == EPI_XUPD || EPI == EPI_FINAL);
    constexpr bool XT = EPI == EPI_XUPD || EPI == EPI_FINAL;
    // every bf16 operand (X, A, B) is stored in 32x32 blocks
    constexpr bool PB = BF, QB = BF;
    constexpr int KE = kRowBytes / (int)sizeof(T);
    constexpr int SLD = 36;  // epilogue staging row stride (floats): 16-byte aligned runs
    // the stage ring; after the main loop its start is the epilogue staging
    __shared__ __attribute__((aligned(1024))) char ring[kStages * kStageBytes];
    static_assert(4 * 32 * SLD * 4 <= kStageBytes, "epilogue staging fits in one stage buffer");

    const GemmTile tile = tiles[blockIdx.x];
    if (tile.mat < 0) return;  // padding of a shorter per-XCD list
    const MuonMat& d = tab[tile.mat];
    // the wave index is uniform across the wave: keep it (and what derives
    // from it) in scalar registers so per-wave branches are scalar branches
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int cur = args.iter & 1;

    const char* P;
    const char* Q;
    int64_t ldp, ldq;  // bytes
    int64_t shift = 0;  // bytes from the operand start to this slice's first column
    int K, rows_p, rows_q;
    if (EPI == EPI_GRAM) {
        P = Q = reinterpret_cast<const char*>(BF ? d.x[cur] : d.x[0]);
        ldp = ldq = (int64_t)d.C * sizeof(T);
        K = d.C;
        rows_p = rows_q = d.R;
        if (d.gram_ks > 1) {
            // slice tile.slice of a split reduction: columns [slice K, (slice + 1) K)
            // of X, which the stage copies address from a shifted base
            K = d.C / d.gram_ks;
            const int64_t k0 = (int64_t)tile.slice * K;
            shift = BF ? (k0 / 32) * 2048 : k0 * (int64_t)sizeof(T);
            P += shift;
            Q += shift;
        }
    } else if (EPI == EPI_POLY) {
        P = Q = reinterpret_cast<const char*>(d.a);
        ldp = ldq = (int64_t)d.R * sizeof(T);
        K = d.R;
        rows_p = rows_q = d.R;
    } else {
        P = reinterpret_cast<const char*>(d.b);
        ldp = (int64_t)d.R * sizeof(T);
        rows_p = d.R;
        K = d.R;
        if (QT) {  // X row-major: R rows (the reduction index) of C columns
            Q = reinterpret_cast<const char*>(d.x[cur]);
            ldq = (int64_t)d.C * sizeof(T);
            rows_q = d.R;
        } else {   // X^T: C rows of R
            Q = reinterpret_cast<const char*>(d.xt[cur]);
            ldq = (int64_t)d.R * sizeof(T);
            rows_q = d.C;
        }
    }
    const int m0 = tile.tm * 256, n0 = tile.tn * 256;
    const int nk = K / KE;  // a multiple of 8: K is padded to 256

    const u32x4 rp = make_rsrc(P, (int64_t)rows_p * ldp - shift);
    const u32x4 rq = make_rsrc(Q, (int64_t)rows_q * ldq - shift);
    Addr ad;
    {
        const uint32_t c = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
        ad.dma_p = PB ? (uint32_t)((m0 + wave * 64) * ldp) + (uint32_t)(lane >> 2) * 64 + c * 16
                      : (uint32_t)((m0 + wave * 64 + (lane >> 2)) * ldp) + c * 16;
        if (QT) {
            const uint32_t r = (uint32_t)(8 * wave + (lane >> 5));
            const uint32_t ce = (uint32_t)((lane & 31) ^ (((lane >> 5) & 3) << 2));
            const uint32_t co = (uint32_t)((lane & 31) ^ (((2 + (lane >> 5)) & 3) << 2));
            if (QB) {
                ad.dma_q[0] = ((uint32_t)n0 / 32 + (ce >> 2)) * 2048 + r * 64 + (ce & 3) * 16;
                ad.dma_q[1] = ((uint32_t)n0 / 32 + (co >> 2)) * 2048 + r * 64 + (co & 3) * 16;
            } else {
                ad.dma_q[0] = r * (uint32_t)ldq + (uint32_t)n0 * 2 + ce * 16;
                ad.dma_q[1] = r * (uint32_t)ldq + (uint32_t)n0 * 2 + co * 16;
            }
        } else {
            ad.dma_q[0] = QB ? (uint32_t)((n0 + wave * 64) * ldq) + (uint32_t)(lane >> 2) * 64 + c * 16
                             : (uint32_t)((n0 + wave * 64 + (lane >> 2)) * ldq) + c * 16;
            ad.dma_q[1] = ad.dma_q[0];
        }
        const int r32 = lane & 31, sw = (r32 >> 2) & 3, half = lane >> 5;
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
            const int slot = (2 * kg + half) ^ sw;
            ad.frag_a[kg] = (uint32_t)((wm * 128 + r32) * kRowBytes + (slot << 4));
            ad.frag_b[kg] = (uint32_t)(kRegionBytes + (wn * 128 + r32) * kRowBytes + (slot << 4));
        }
        // linear term from a row-operand Q: bf16 quarter q is the 8 bytes at
        // chunk q, half `half`; fp32 quarter q is chunk 2 q + half
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rowb = kRegionBytes + (wn * 128 + r32) * kRowBytes;
            ad.lin_r[q] = BF ? (uint32_t)(rowb + ((q ^ sw) << 4) + 8 * half)
                             : (uint32_t)(rowb + ((((2 * q + half) & 3) ^ sw) << 4));
        }
        const int g = lane >> 4, jj = lane & 15;
        const int tsw = (jj >> 2) & 3;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int chunk = wn * 16 + ((j ^ tsw) << 2) + 2 * (g & 1) + ((jj & 3) >> 1);
            const int row_f = 8 * (g >> 1) + (jj >> 2);
            const int row_l = 4 * (g >> 1) + (jj >> 2);
            ad.frag_t[j] = (uint32_t)(kRegionBytes + row_f * 512 + (chunk << 4) + 8 * (jj & 1));
            ad.lin_t[j] = (uint32_t)(kRegionBytes + row_l * 512 + (chunk << 4) + 8 * (jj & 1));
        }
    }
    const uint32_t uldp = (uint32_t)ldp, uldq = (uint32_t)ldq;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // bf16 linear terms taken from the stage buffers: a X_hi (update steps)
    // and (b / c) A (polynomial step with c != 0; the epilogue scales by c)
    const bool poly_direct = BF && EPI == EPI_POLY && args.c != 0.f;
    constexpr bool LIN = BF && (XT || EPI == EPI_POLY);
    const float scale = XT ? args.a : (poly_direct ? args.b / args.c : 0.f);
    const int rel0 = LIN && (XT || poly_direct) ? -(m0 + wm * 128) : -(1 << 30);

    const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 4 * 1024);
    const uint32_t lring = lds_addr(ring);
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
        stage_copy<T, QT, PB, QB>(lring + st * kStageBytes, rp, rq, ad, wbase, st, uldp, uldq);
    // stage 0 has landed once only the copies of stages 1 .. kStages - 2 are
    // outstanding
    wait_vm(8 * (kStages - 2));
    stage_barrier();
    uint4 fa[4], fb[4];
    stage_frags<QT>(fa, fb, ring, ad, 0);
    // the loop is unrolled by the ring depth so every stage buffer address
    // is a compile-time offset
    for (int s = 0; s < nk; s += kStages)
        ring_round<T, QT, LIN, PB, QB>(std::make_integer_sequence<int, kStages>(), acc, fa, fb, ring,
                                       lring, rp, rq, ad, wbase, s, nk, uldp, uldq, scale, rel0);
    // every wave is done with the ring (all copies landed at the last
    // stage's wait) before it becomes the epilogue staging area
    stage_barrier();

    // ---- epilogue: each wave stages its 32x32 accumulator blocks in its own
    // LDS region (wave-level synchronisation only, no block barriers) and
    // moves them as 16-element runs: row runs for row-major outputs, column
    // runs for the transposed outputs ----
    float* S = reinterpret_cast<float*>(ring) + wave * (32 * SLD);
    const bool mirror = (EPI == EPI_GRAM || EPI == EPI_POLY) && tile.tm != tile.tn;
    const bool need_cols =
        mirror || (EPI == EPI_XUPD && !BF) || (EPI == EPI_FINAL && d.transposed);
    T* out_direct = nullptr;
    int64_t ld_direct = 0;
    if (EPI == EPI_GRAM) {
        // a split reduction's slices 1.. write partial Grams, added to A later
        out_direct = reinterpret_cast<T*>(
            tile.slice == 0 ? d.a
                            : d.apart + (uint64_t)(tile.slice - 1) * d.R * d.R * sizeof(T));
        ld_direct = d.R;
    } else if (EPI == EPI_POLY) {
        out_direct = reinterpret_cast<T*>(d.b);
        ld_direct = d.R;
    }
    const int bi0 = m0 + wm * 128, bj0 = n0 + wn * 128;
    const bool use_lo = args.use_lo != 0;
    const float s0 = args.iter == 0 ? args.scales[tile.mat] : 1.f;
    const float escale = EPI == EPI_GRAM ? s0 * s0 : (XT ? s0 : 1.f);
    Upd up{0.f, 1.f};
    if (EPI == EPI_FINAL) {
        // rate = muon_lr * shape factor, formed in double and rounded once
        up.rate = (float)(args.sd->muon_lr * (double)d.shape_scale);
        up.decay = args.sd->muon_decay;
    }
    // The 16 blocks go in row order; each block's global inputs are loaded
    // four blocks ahead (slots in0..in3), and the final update's old
    // parameter values two blocks ahead (p0, p1), so their latency overlaps
    // the work on the blocks in between instead of stalling every block.
    EpiIn in0, in1, in2, in3;
    PIn p0, p1;
#define NS_LOAD(SLOT, I, J) \
    epi_load<T, EPI>(SLOT, d, lane, bi0 + (I) * 32, bj0 + (J) * 32, cur, poly_direct, use_lo)
#define NS_PLOAD(SLOT, I, J) p_load<EPI>(SLOT, d, lane, bi0 + (I) * 32, bj0 + (J) * 32)
#define NS_EPI(I, J, SLOT, PSLOT)                                                            \
    epi_block<T, EPI, SLD>(acc[I][J], SLOT, PSLOT, d, S, args, escale, up, lane,              \
                           bi0 + (I) * 32, bj0 + (J) * 32, cur, need_cols, poly_direct,       \
                           out_direct, ld_direct)
    NS_LOAD(in0, 0, 0); NS_LOAD(in1, 0, 1); NS_LOAD(in2, 0, 2); NS_LOAD(in3, 0, 3);
    NS_PLOAD(p0, 0, 0); NS_PLOAD(p1, 0, 1);
    NS_EPI(0, 0, in0, p0); NS_LOAD(in0, 1, 0); NS_PLOAD(p0, 0, 2);
    NS_EPI(0, 1, in1, p1); NS_LOAD(in1, 1, 1); NS_PLOAD(p1, 0, 3);
    NS_EPI(0, 2, in2, p0); NS_LOAD(in2, 1, 2); NS_PLOAD(p0, 1, 0);
    NS_EPI(0, 3, in3, p1); NS_LOAD(in3, 1, 3); NS_PLOAD(p1, 1, 1);
    NS_EPI(1, 0, in0, p0); NS_LOAD(in0, 2, 0); NS_PLOAD(p0, 1, 2);
    NS_EPI(1, 1, in1, p1); NS_LOAD(in1, 2, 1); NS_PLOAD(p1, 1, 3);
    NS_EPI(1, 2, in2, p0); NS_LOAD(in2, 2, 2); NS_PLOAD(p0, 2, 0);
    NS_EPI(1, 3, in3, p1); NS_LOAD(in3, 2, 3); NS_PLOAD(p1, 2, 1);
    NS_EPI(2, 0, in0, p0); NS_LOAD(in0, 3, 0); NS_PLOAD(p0, 2, 2);
    NS_EPI(2, 1, in1, p1); NS_LOAD(in1, 3, 1); NS_PLOAD(p1, 2, 3);
    NS_EPI(2, 2, in2, p0); NS_LOAD(in2, 3, 2); NS_PLOAD(p0, 3, 0);
    NS_EPI(2, 3, in3, p1); NS_LOAD(in3, 3, 3); NS_PLOAD(p1, 3, 1);
    NS_EPI(3, 0, in0, p0); NS_PLOAD(p0, 3, 2);
    NS_EPI(3, 1, in1, p1); NS_PLOAD(p1, 3, 3);
    NS_EPI(3, 2, in2, p0);
    NS_EPI(3, 3, in3, p1);
#undef NS_LOAD
#undef NS_PLOAD
#undef NS_EPI
}

// ---------------------------------------------------------------------------
// bf16 tiles: eight waves per workgroup, two per SIMD.
//
// The 256 x 256 output tile is split into 2 x 4 wave tiles of 128 x 64 rows
// x columns (4 x 2 accumulator blocks of 32 x 32: 128 accumulator registers),
// so each SIMD holds two waves and the matrix instructions of one run while
// the other waits on its LDS reads, the stage copies or the workgroup
// barrier; with one 128 x 128 wave per SIMD every such wait left the matrix
// core idle.  Operand staging is the same ring of four 32 KB stages with the
// same row layouts and swizzles; each wave copies one eighth of a stage (two
// 1 KB loads of P and two of Q).  Per stage a CU reads 96 (Gram, square) or
// 128 (update: transposing reads of X) LDS fragments, within the LDS read
// rate the matrix instructions leave room for.
// ---------------------------------------------------------------------------
constexpr int kW8Waves = 8;
// Ring depth of these kernels: five 32 KB stages fill the 160 KB of LDS, and
// copies run four stages ahead, so a stage's operands have three stages'
// time (not two) to arrive from L2 or the memory-side cache.
constexpr int kW8Stages = 5;

struct Addr8 {
    uint32_t dma_p;          // P copy: this lane's row and chunk
    uint32_t dma_q[2];       // Q copy (row operand: [0]; transposed: first / second load)
    uint32_t frag_a[2];      // A fragment of row block 0, per k-group
    uint32_t frag_b[2];      // B fragment (row operand) of column block 0, per k-group
    uint32_t frag_t[2];      // B fragment (transposed), per column block, k-group 0
    uint32_t lin_t[2];       // linear-term reads (transposed), per column block
    uint32_t lin_r[4];       // linear-term reads (row operand) of column block 0, per quarter
};

// Part i (0, 1) of this wave's copy of stage s: 1 KB of P rows (16 rows of
// 64 bytes in one 32-row block row of the blocked operand), or of Q.
__device__ __forceinline__ void copy_p8(uint32_t buf, u32x4 rp, const Addr8& ad, uint32_t wbase,
                                        int s, int i) {
    dma16(rp, buf + wbase + i * 1024, ad.dma_p, (uint32_t)s * 2048 + (uint32_t)i * 1024);
}

template <bool QT>
__device__ __forceinline__ void copy_q8(uint32_t buf, u32x4 rq, const Addr8& ad, uint32_t wbase,
                                        int s, int i, uint32_t ldq) {
    if (QT)  // rows 4 w + 2 i, 4 w + 2 i + 1 of the stage's 32 rows of X (block row s)
        dma16(rq, buf + kRegionBytes + wbase + i * 1024, ad.dma_q[i],
              (uint32_t)s * 32 * ldq + (uint32_t)(2 * i) * 64);
    else
        dma16(rq, buf + kRegionBytes + wbase + i * 1024, ad.dma_q[0],
              (uint32_t)s * 2048 + (uint32_t)i * 1024);
}

__device__ __forceinline__ uint4 lds16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

template <bool QT>
__device__ __forceinline__ uint4 frag_b8(const char* buf, const Addr8& ad, int kg, int j) {
    if (QT) {
        const char* p = buf + ad.frag_t[j] + kg * 16 * 512;
        const uint2 lo = lds_tr8(p), hi = lds_tr8(p + 4 * 512);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    return lds16(buf + ad.frag_b[kg] + j * 2048);
}

// Linear term of the update (a X_hi) and polynomial ((b / c) A) steps for
// accumulator row block IB, from the stage buffer (see stage_linear).
template <bool QT, int IB>
__device__ __forceinline__ void lin8(f32x16 (&acc)[4][2], const char* buf, const Addr8& ad,
                                     float scale) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint2 w = QT ? lds_tr8(buf + ad.lin_t[j] + q * 8 * 512)
                               : *reinterpret_cast<const uint2*>(buf + ad.lin_r[q] + j * 2048);
            const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(w.x, w.y, 0u, 0u));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[IB][j][4 * q + e] = fmaf(scale, (float)b[e], acc[IB][j][4 * q + e]);
        }
    }
}

// One stage: k-group 0 with the k-group-1 fragment reads between its matrix
// instructions, the barrier that publishes stage s + 1 and frees the buffer
// of stage s - 1, the linear term of accumulator row block LINB (-1: none),
// then k-group 1 with this wave's copies of stage s + kW8Stages - 1 into the
// freed buffer and the next stage's k-group-0 reads.
template <bool QT, int LINB>
__device__ __forceinline__ void step8(f32x16 (&acc)[4][2], uint4 (&fa)[4], uint4 (&fb)[2],
                                      const char* cur, const char* nxt, uint32_t tgt, u32x4 rp,
                                      u32x4 rq, const Addr8& ad, uint32_t wbase, int s, int nk,
                                      uint32_t ldq, float scale) {
    uint4 ga[4], gb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i][0] = Mma<__bf16>::run(fa[i], fb[0], acc[i][0]);
        __builtin_amdgcn_sched_barrier(0);
        ga[i] = lds16(cur + ad.frag_a[1] + i * 2048);
        __builtin_amdgcn_sched_barrier(0);
        acc[i][1] = Mma<__bf16>::run(fa[i], fb[1], acc[i][1]);
        __builtin_amdgcn_sched_barrier(0);
        if (i < 2) gb[i] = frag_b8<QT>(cur, ad, 1, i);
        __builtin_amdgcn_sched_barrier(0);
    }
    // stage s + 1 has landed once at most the copies of the stages after it
    // (four loads each, at most kW8Stages - 3 stages) are outstanding
    wait_vm(4 * min(nk - 2 - s, kW8Stages - 3));
    stage_barrier();
    if (LINB >= 0) lin8<QT, (LINB < 0 ? 0 : LINB)>(acc, cur, ad, scale);
    __builtin_amdgcn_sched_barrier(0);
    const bool cp = s + kW8Stages - 1 < nk;
    const int sc = s + kW8Stages - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[i][0] = Mma<__bf16>::run(ga[i], gb[0], acc[i][0]);
        __builtin_amdgcn_sched_barrier(0);
        if (cp) {
            if (i < 2) copy_p8(tgt, rp, ad, wbase, sc, i);
            else copy_q8<QT>(tgt, rq, ad, wbase, sc, i - 2, ldq);
        }
        __builtin_amdgcn_sched_barrier(0);
        acc[i][1] = Mma<__bf16>::run(ga[i], gb[1], acc[i][1]);
        __builtin_amdgcn_sched_barrier(0);
        fa[i] = lds16(nxt + ad.frag_a[0] + i * 2048);
        __builtin_amdgcn_sched_barrier(0);
        if (i < 2) fb[i] = frag_b8<QT>(nxt, ad, 0, i);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int EPI>
__device__ __forceinline__ void ns_gemm_tile_w8(const MuonMat* __restrict__ tab,
                                                const GemmTile* __restrict__ tiles,
                                                const NsArgs& args) {
    typedef __bf16 T;
    constexpr bool XT = EPI == EPI_XUPD || EPI == EPI_FINAL;
    constexpr bool QT = XT;      // B X reads X row-major through transposing loads
    constexpr int KE = kRowBytes / 2;
    constexpr int SLD = 36;
    __shared__ __attribute__((aligned(1024))) char ring[kW8Stages * kStageBytes];
    static_assert(kW8Waves * 32 * SLD * 4 <= kW8Stages * kStageBytes, "epilogue staging fits in the ring");
    static_assert(kW8Stages * kStageBytes <= 160 * 1024, "the ring fits in a CU's LDS");

    const GemmTile tile = tiles[blockIdx.x];
    if (tile.mat < 0) return;
    const MuonMat& d = tab[tile.mat];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int cur = args.iter & 1;

    const char* P;
    const char* Q;
    int64_t ldp, ldq;
    int K, rows_p, rows_q;
    if (EPI == EPI_GRAM) {
        P = Q = reinterpret_cast<const char*>(d.x[cur]);
        ldp = ldq = (int64_t)d.C * 2;
        K = d.C;
        rows_p = rows_q = d.R;
    } else if (EPI == EPI_POLY) {
        P = Q = reinterpret_cast<const char*>(d.a);
        ldp = ldq = (int64_t)d.R * 2;
        K = d.R;
        rows_p = rows_q = d.R;
    } else {
        P = reinterpret_cast<const char*>(d.b);
        ldp = (int64_t)d.R * 2;
        K = d.R;
        rows_p = d.R;
        Q = reinterpret_cast<const char*>(d.x[cur]);   // R rows (the reduction index) of C
        ldq = (int64_t)d.C * 2;
        rows_q = d.R;
    }
    const int m0 = tile.tm * 256, n0 = tile.tn * 256;
    const int nk = K / KE;

    const u32x4 rp = make_rsrc(P, (int64_t)rows_p * ldp);
    const u32x4 rq = make_rsrc(Q, (int64_t)rows_q * ldq);
    Addr8 ad;
    {
        const uint32_t c = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
        ad.dma_p = (uint32_t)((m0 + wave * 32) * ldp) + (uint32_t)(lane >> 2) * 64 + c * 16;
        if (QT) {
            const uint32_t r = (uint32_t)(4 * wave + (lane >> 5));
            const uint32_t ce = (uint32_t)((lane & 31) ^ (((lane >> 5) & 3) << 2));
            const uint32_t co = (uint32_t)((lane & 31) ^ (((2 + (lane >> 5)) & 3) << 2));
            ad.dma_q[0] = ((uint32_t)n0 / 32 + (ce >> 2)) * 2048 + r * 64 + (ce & 3) * 16;
            ad.dma_q[1] = ((uint32_t)n0 / 32 + (co >> 2)) * 2048 + r * 64 + (co & 3) * 16;
        } else {
            ad.dma_q[0] = (uint32_t)((n0 + wave * 32) * ldq) + (uint32_t)(lane >> 2) * 64 + c * 16;
            ad.dma_q[1] = ad.dma_q[0];
        }
        const int r32 = lane & 31, sw = (r32 >> 2) & 3, half = lane >> 5;
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
            const int slot = (2 * kg + half) ^ sw;
            ad.frag_a[kg] = (uint32_t)((wm * 128 + r32) * kRowBytes + (slot << 4));
            ad.frag_b[kg] = (uint32_t)(kRegionBytes + (wn * 64 + r32) * kRowBytes + (slot << 4));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rowb = kRegionBytes + (wn * 64 + r32) * kRowBytes;
            ad.lin_r[q] = (uint32_t)(rowb + ((q ^ sw) << 4) + 8 * half);
        }
        const int g = lane >> 4, jj = lane & 15;
        const int tsw = (jj >> 2) & 3;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int chunk = (((wn * 2 + j) ^ tsw) << 2) + 2 * (g & 1) + ((jj & 3) >> 1);
            const int row_f = 8 * (g >> 1) + (jj >> 2);
            const int row_l = 4 * (g >> 1) + (jj >> 2);
            ad.frag_t[j] = (uint32_t)(kRegionBytes + row_f * 512 + (chunk << 4) + 8 * (jj & 1));
            ad.lin_t[j] = (uint32_t)(kRegionBytes + row_l * 512 + (chunk << 4) + 8 * (jj & 1));
        }
    }
    const uint32_t uldq = (uint32_t)ldq;

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const bool poly_direct = EPI == EPI_POLY && args.c != 0.f;
    const float scale = XT ? args.a : (poly_direct ? args.b / args.c : 0.f);
    // The linear term (a X_hi of the update, (b / c) A of the polynomial)
    // comes from the four stages whose reduction indices are this wave's
    // output rows: stages lin0 .. lin0 + 3, accumulator row blocks 0 .. 3.
    const int lin0 = (XT || poly_direct) ? (m0 + wm * 128) / KE : nk;

    const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 2 * 1024);
    const uint32_t lring = lds_addr(ring);
#pragma unroll
    for (int st = 0; st < kW8Stages - 1; ++st) {
        const uint32_t b = lring + st * kStageBytes;
        copy_p8(b, rp, ad, wbase, st, 0);
        copy_p8(b, rp, ad, wbase, st, 1);
        copy_q8<QT>(b, rq, ad, wbase, st, 0, uldq);
        copy_q8<QT>(b, rq, ad, wbase, st, 1, uldq);
    }
    // stage 0 has landed once only the copies of stages 1 .. kW8Stages - 2
    // are outstanding (nk >= 8 > kW8Stages - 1: all of them were issued)
    wait_vm(4 * (kW8Stages - 2));
    stage_barrier();
    uint4 fa[4], fb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = lds16(ring + ad.frag_a[0] + i * 2048);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = frag_b8<QT>(ring, ad, 0, j);
    // the ring is walked by a scalar slot index rather than unrolled: stage
    // buffers beyond 64 KB cannot be reached by the LDS instructions'
    // immediate offsets, so an unrolled ring would hold one set of fragment
    // addresses per stage in registers
    // (every wave runs all nk stages, so all take the same barriers)
    int slot = 0, s = 0;
#define W8_STEP(LINB)                                                                        \
    {                                                                                        \
        const int nslot = slot == kW8Stages - 1 ? 0 : slot + 1;                              \
        const int tslot = slot == 0 ? kW8Stages - 1 : slot - 1; /* stage s + depth - 1 */    \
        step8<QT, LINB>(acc, fa, fb, ring + slot * kStageBytes, ring + nslot * kStageBytes,  \
                        lring + tslot * kStageBytes, rp, rq, ad, wbase, s, nk, uldq, scale); \
        slot = nslot;                                                                        \
        ++s;                                                                                 \
    }
#pragma unroll 1
    while (s < lin0) W8_STEP(-1)
    if (s < nk) {
        W8_STEP(0)
        W8_STEP(1)
        W8_STEP(2)
        W8_STEP(3)
    }
#pragma unroll 1
    while (s < nk) W8_STEP(-1)
#undef W8_STEP
    stage_barrier();

    float* S = reinterpret_cast<float*>(ring) + wave * (32 * SLD);
    const bool mirror = (EPI == EPI_GRAM || EPI == EPI_POLY) && tile.tm != tile.tn;
    const bool need_cols = mirror || (EPI == EPI_FINAL && d.transposed);
    T* out_direct = nullptr;
    int64_t ld_direct = 0;
    if (EPI == EPI_GRAM) {
        out_direct = reinterpret_cast<T*>(d.a);
        ld_direct = d.R;
    } else if (EPI == EPI_POLY) {
        out_direct = reinterpret_cast<T*>(d.b);
        ld_direct = d.R;
    }
    const int bi0 = m0 + wm * 128, bj0 = n0 + wn * 64;
    const bool use_lo = args.use_lo != 0;
    const float s0 = args.iter == 0 ? args.scales[tile.mat] : 1.f;
    const float escale = EPI == EPI_GRAM ? s0 * s0 : (XT ? s0 : 1.f);
    Upd up{0.f, 1.f};
    if (EPI == EPI_FINAL) {
        up.rate = (float)(args.sd->muon_lr * (double)d.shape_scale);
        up.decay = args.sd->muon_decay;
    }
    // blocks in row order; each block's global inputs loaded two blocks
    // ahead, the final update's old parameter run one block ahead (the other
    // wave of the SIMD covers its latency; a second slot would pass the
    // register budget below)
    EpiIn in0, in1;
    PIn p0;
#define W8_LOAD(SLOT, I, J) \
    epi_load<T, EPI>(SLOT, d, lane, bi0 + (I) * 32, bj0 + (J) * 32, cur, poly_direct, use_lo)
#define W8_PLOAD(SLOT, I, J) p_load<EPI>(SLOT, d, lane, bi0 + (I) * 32, bj0 + (J) * 32)
#define W8_EPI(I, J, SLOT, PSLOT)                                                            \
    epi_block<T, EPI, SLD>(acc[I][J], SLOT, PSLOT, d, S, args, escale, up, lane,              \
                           bi0 + (I) * 32, bj0 + (J) * 32, cur, need_cols, poly_direct,       \
                           out_direct, ld_direct)
    W8_LOAD(in0, 0, 0); W8_LOAD(in1, 0, 1); W8_PLOAD(p0, 0, 0);
    W8_EPI(0, 0, in0, p0); W8_LOAD(in0, 1, 0); W8_PLOAD(p0, 0, 1);
    W8_EPI(0, 1, in1, p0); W8_LOAD(in1, 1, 1); W8_PLOAD(p0, 1, 0);
    W8_EPI(1, 0, in0, p0); W8_LOAD(in0, 2, 0); W8_PLOAD(p0, 1, 1);
    W8_EPI(1, 1, in1, p0); W8_LOAD(in1, 2, 1); W8_PLOAD(p0, 2, 0);
    W8_EPI(2, 0, in0, p0); W8_LOAD(in0, 3, 0); W8_PLOAD(p0, 2, 1);
    W8_EPI(2, 1, in1, p0); W8_LOAD(in1, 3, 1); W8_PLOAD(p0, 3, 0);
    W8_EPI(3, 0, in0, p0); W8_PLOAD(p0, 3, 1);
    W8_EPI(3, 1, in1, p0);
#undef W8_LOAD
#undef W8_PLOAD
#undef W8_EPI
}

// ---------------------------------------------------------------------------
// Small fp32 Gram and square tiles: 32 x 32 outputs, for matrices of at most
// 256 padded rows.
//
// A launch over a few such matrices holds only tens of 256 x 256 tiles, each
// a long chain of matrix instructions on one CU while the rest of the GPU
// idles.  Here a tile is 32 x 32 (64 times as many workgroups) and its
// reduction is split four ways: wave w of the workgroup reduces over the
// w-th quarter of K into its own accumulator block, so a wave's chain is a
// sixteenth of a 64 x 64 tile's.  The waves read their fragments straight
// from global memory (no operand is shared between them): lane l holds row
// l % 32 and, of every 32-column block, the 16 columns from 16 (l / 32) on,
// as four 16-byte loads; fragment g of the block pairs columns
// 16 h + 4 g .. 16 h + 4 g + 3 of both operands (h = lane half), so the four
// MFMA steps of each fragment cover the block once.  Two blocks are in
// flight per wave.  Waves 1..3 then hand their sums to wave 0 through LDS;
// wave 0 adds them in wave order (a fixed order: reruns are bitwise equal)
// and runs the epilogue of the large tiles on its one block.
// ---------------------------------------------------------------------------
constexpr int kS32 = 32;
static_assert(kS32 == kSmallTile, "small tile lists are built for 32x32 tiles");

// Bytes [kb, kb + 64) of this lane's operand row (base already points at the
// row and lane half): four 16-byte loads.
__device__ __forceinline__ void s32_load(uint4 (&v)[4], const char* base, int64_t kb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) v[g] = gld(base + kb + 16 * g);
}

// Blocks in flight per wave (four measured no faster for the Grams of
// 256 x 1024 matrices), and waves per workgroup: the reduction is split
// kS32Waves ways (K is a multiple of 256, so each wave gets whole 32-column
// blocks; eight waves made the tiny table's Newton-Schulz 0.20 -> 0.23 ms).
constexpr int kS32Depth = 2;
constexpr int kS32Waves = 4;

__device__ __forceinline__ void s32_mma(f32x16& acc, const uint4 (&a)[4], const uint4 (&b)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) acc = Mma<float>::run(a[g], b[g], acc);
}

template <int EPI>
__device__ __forceinline__ void ns_gemm_tile_s32(const MuonMat* __restrict__ tab,
                                                 const GemmTile* __restrict__ tiles,
                                                 const NsArgs& args) {
    static_assert(EPI == EPI_GRAM || EPI == EPI_POLY, "Gram and square only");
    constexpr int SLD = 36;
    constexpr int W = kS32Waves;
    __shared__ __attribute__((aligned(16))) float red[W - 1][16][64];  // waves 1..: [register][lane]
    __shared__ __attribute__((aligned(16))) float stage[32 * SLD];  // wave 0's epilogue staging

    const GemmTile tile = tiles[blockIdx.x];
    if (tile.mat < 0) return;  // padding of a shorter per-XCD list
    const MuonMat& d = tab[tile.mat];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cur = args.iter & 1;

    // operands: fp32, row-major, reduction index contiguous; both are X
    // (Gram) or both A (square)
    const char* P;
    int64_t ldp;  // bytes
    int K;
    if (EPI == EPI_GRAM) {
        P = reinterpret_cast<const char*>(d.x[0]);
        ldp = (int64_t)d.C * 4;
        K = d.C;
        if (d.gram_ks > 1) {
            // slice tile.slice of a split reduction
            K = d.C / d.gram_ks;
            P += (int64_t)tile.slice * K * 4;
        }
    } else {
        P = reinterpret_cast<const char*>(d.a);
        ldp = (int64_t)d.R * 4;
        K = d.R;
    }
    const int m0 = tile.tm * kS32, n0 = tile.tn * kS32;
    const int kq = K / W;    // this wave's columns: a multiple of 32 (K is padded to 256)
    const int nb = kq / 32;  // its 32-column blocks: at least 1
    const int r = lane & 31, h = lane >> 5;
    const char* pa = P + (int64_t)(m0 + r) * ldp + ((int64_t)wave * kq + 16 * h) * 4;
    const char* qa = P + (int64_t)(n0 + r) * ldp + ((int64_t)wave * kq + 16 * h) * 4;

    // wave 0's epilogue inputs, loaded now so their latency hides behind the loop
    EpiIn in;
    PIn pin;
    if (wave == 0) epi_load<float, EPI>(in, d, lane, m0, n0, cur, false, false);

    // D blocks in flight: buffer i holds block kb + i.  Loads past the last
    // block re-read it (cache hits) and are not multiplied, so every
    // iteration of the loop issues the same loads and waits the same counts;
    // the last D blocks are multiplied after it, with no further loads.
    constexpr int D = kS32Depth;
    uint4 a[D][4], b[D][4];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        const int64_t o = (int64_t)min(i, nb - 1) * 128;
        s32_load(a[i], pa, o);
        s32_load(b[i], qa, o);
    }
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    int kb = 0;
    for (; kb + D < nb; kb += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            s32_mma(acc, a[i], b[i]);
            const int64_t o = (int64_t)min(kb + i + D, nb - 1) * 128;
            s32_load(a[i], pa, o);
            s32_load(b[i], qa, o);
        }
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
        if (kb + i < nb) s32_mma(acc, a[i], b[i]);

    if (wave != 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) red[wave - 1][e][lane] = acc[e];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < W - 1; ++w)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += red[w][e][lane];

    // an off-diagonal tile also writes its mirror image
    const bool mirror = tile.tm != tile.tn;
    float* out_direct = reinterpret_cast<float*>(
        EPI == EPI_POLY ? d.b
                        : (tile.slice == 0 ? d.a
                                           : d.apart + (uint64_t)(tile.slice - 1) * d.R * d.R * 4));
    const float s0 = args.iter == 0 ? args.scales[tile.mat] : 1.f;
    const float escale = EPI == EPI_GRAM ? s0 * s0 : 1.f;
    const Upd up{0.f, 1.f};
    epi_block<float, EPI, SLD>(acc, in, pin, d, stage, args, escale, up, lane, m0, n0, cur,
                               mirror, false, out_direct, d.R);
}

// ---------------------------------------------------------------------------
// Small fp32 X updates: 64 x 64 outputs, four waves of one 32 x 32 block
// each over the whole reduction (K = 256 for these matrices), operands
// shared through LDS.  Against the 32 x 32 split-reduction tiles these
// halve the operand reads and the workgroups (two rounds of 32 x 32 update
// tiles did not fit the GPU at once) and need no cross-wave sum.
//
// Operands stream through a ring of four 16 KB stages of 32 reduction
// columns (64 rows of P, then 64 rows of Q, 128 bytes per row; 16-byte chunk
// c of row r at slot c ^ ((r >> 1) & 7), so the sixteen rows read by each
// quarter-wave fragment load fall in distinct banks), copied by buffer loads
// straight into LDS three stages ahead.  The epilogue is that of the large
// tiles, one block per wave, with its global inputs loaded before the main
// loop.
// ---------------------------------------------------------------------------
constexpr int kS64 = 64;                    // output tile side
constexpr int kS64Row = 128;                // bytes per operand row per stage
constexpr int kS64Region = kS64 * kS64Row;  // one operand's part of a stage
constexpr int kS64Stage = 2 * kS64Region;
constexpr int kS64Stages = 4;               // ring depth: copies run 3 stages ahead
static_assert(kS64 == kSmallXTile, "small update tile lists are built for 64x64 tiles");

// Stage s of the ring, copied by this wave: rows 16 w .. 16 w + 15 of P and
// of Q, as two 1 KB loads each (8 rows of 128 bytes per load).
__device__ __forceinline__ void s64_copy(uint32_t slot, u32x4 rp, u32x4 rq, const uint32_t (&vp)[2],
                                         const uint32_t (&vq)[2], uint32_t wbase, int s,
                                         uint32_t ldp, uint32_t ldq) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
        dma16(rp, slot + wbase + i * 1024, vp[i], (uint32_t)s * kS64Row + (uint32_t)(8 * i) * ldp);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        dma16(rq, slot + kS64Region + wbase + i * 1024, vq[i],
              (uint32_t)s * kS64Row + (uint32_t)(8 * i) * ldq);
}

// One stage of the main loop (stage s in ring slot S): wait for its copies,
// barrier (which also retires every wave's reads of the slot the next copy
// overwrites), issue the copy three stages ahead, multiply.
template <int S>
__device__ __forceinline__ void s64_stage(f32x16& acc, const char* ring, uint32_t lring, u32x4 rp,
                                          u32x4 rq, const uint32_t (&vp)[2],
                                          const uint32_t (&vq)[2], const uint32_t (&fa)[4],
                                          const uint32_t (&fb)[4], uint32_t wbase, int s, int nk,
                                          uint32_t ldp, uint32_t ldq) {
    // at most the copies of stages s + 1 and s + 2 (4 loads each) may still
    // be in flight
    wait_vm(4 * min(nk - 1 - s, kS64Stages - 2));
    stage_barrier();
    if (s + kS64Stages - 1 < nk)
        s64_copy(lring + ((S + kS64Stages - 1) % kS64Stages) * kS64Stage, rp, rq, vp, vq, wbase,
                 s + kS64Stages - 1, ldp, ldq);
    const char* buf = ring + S * kS64Stage;
    uint4 a[4], b[4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
        a[kg] = *reinterpret_cast<const uint4*>(buf + fa[kg]);
        b[kg] = *reinterpret_cast<const uint4*>(buf + fb[kg]);
    }
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) acc = Mma<float>::run(a[kg], b[kg], acc);
}

// X update (or final update) B X of one 64 x 64 tile: P = B (R x R), Q = X^T
// (C x R), K = R.
template <int EPI>
__device__ __forceinline__ void ns_xupd_tile_s64(const MuonMat* __restrict__ tab,
                                                 const GemmTile* __restrict__ tiles,
                                                 const NsArgs& args) {
    static_assert(EPI == EPI_XUPD || EPI == EPI_FINAL, "update phases only");
    constexpr int SLD = 36;
    __shared__ __attribute__((aligned(1024))) char ring[kS64Stages * kS64Stage];
    static_assert(4 * 32 * SLD * 4 <= kS64Stages * kS64Stage, "epilogue staging fits in the ring");

    const GemmTile tile = tiles[blockIdx.x];
    if (tile.mat < 0) return;  // padding of a shorter per-XCD list
    const MuonMat& d = tab[tile.mat];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int cur = args.iter & 1;

    const char* P = reinterpret_cast<const char*>(d.b);
    const char* Q = reinterpret_cast<const char*>(d.xt[cur]);
    const int64_t ldp = (int64_t)d.R * 4, ldq = (int64_t)d.R * 4;  // bytes
    const int m0 = tile.tm * kS64, n0 = tile.tn * kS64;
    const int nk = d.R / 32;  // a multiple of 8: R is padded to 256

    const u32x4 rp = make_rsrc(P, (int64_t)d.R * ldp);
    const u32x4 rq = make_rsrc(Q, (int64_t)d.C * ldq);
    const uint32_t uldp = (uint32_t)ldp, uldq = (uint32_t)ldq;
    // copies: lane l of load i writes row 16 w + 8 i + l / 8 of the region,
    // slot l % 8, which holds chunk (l % 8) ^ ((row >> 1) & 7)
    // = (l % 8) ^ (l / 16) ^ 4 i
    uint32_t vp[2], vq[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t c = (uint32_t)(((lane & 7) ^ (lane >> 4)) ^ (4 * i));
        const uint32_t r = (uint32_t)(wave * 16 + (lane >> 3));
        vp[i] = (uint32_t)(m0 + r) * uldp + c * 16;
        vq[i] = (uint32_t)(n0 + r) * uldq + c * 16;
    }
    // fragments: lane l reads row 32 wm + l % 32 (P) or 32 wn + l % 32 (Q),
    // chunk 2 kg + l / 32 of k-group kg
    uint32_t fa[4], fb[4];
    {
        const int r32 = lane & 31, half = lane >> 5, sw = (r32 >> 1) & 7;
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
            const uint32_t slot = (uint32_t)(((2 * kg + half) ^ sw) << 4);
            fa[kg] = (uint32_t)((wm * 32 + r32) * kS64Row) + slot;
            fb[kg] = (uint32_t)(kS64Region + (wn * 32 + r32) * kS64Row) + slot;
        }
    }
    const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 16 * kS64Row);
    const uint32_t lring = lds_addr(ring);

    // epilogue inputs, loaded now so their latency hides behind the loop
    const int bi = m0 + wm * 32, bj = n0 + wn * 32;
    EpiIn in;
    PIn pin;
    epi_load<float, EPI>(in, d, lane, bi, bj, cur, false, false);
    p_load<EPI>(pin, d, lane, bi, bj);

#pragma unroll
    for (int st = 0; st < kS64Stages - 1; ++st)
        s64_copy(lring + st * kS64Stage, rp, rq, vp, vq, wbase, st, uldp, uldq);

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    for (int s = 0; s < nk; s += kS64Stages) {
        s64_stage<0>(acc, ring, lring, rp, rq, vp, vq, fa, fb, wbase, s, nk, uldp, uldq);
        s64_stage<1>(acc, ring, lring, rp, rq, vp, vq, fa, fb, wbase, s + 1, nk, uldp, uldq);
        s64_stage<2>(acc, ring, lring, rp, rq, vp, vq, fa, fb, wbase, s + 2, nk, uldp, uldq);
        s64_stage<3>(acc, ring, lring, rp, rq, vp, vq, fa, fb, wbase, s + 3, nk, uldp, uldq);
    }
    // every wave is done with the ring before it becomes the epilogue staging
    stage_barrier();

    float* S = reinterpret_cast<float*>(ring) + wave * (32 * SLD);
    const bool need_cols = EPI == EPI_XUPD || d.transposed;
    const float s0 = args.iter == 0 ? args.scales[tile.mat] : 1.f;
    Upd up{0.f, 1.f};
    if (EPI == EPI_FINAL) {
        up.rate = (float)(args.sd->muon_lr * (double)d.shape_scale);
        up.decay = args.sd->muon_decay;
    }
    epi_block<float, EPI, SLD>(acc, in, pin, d, S, args, s0, up, lane, bi, bj, cur, need_cols,
                               false, nullptr, 0);
}

// ---------------------------------------------------------------------------
// Small bf16 matrices (at most 64 rows and 512 columns, canonical
// orientation): one workgroup per matrix runs every Newton-Schulz iteration
// and the update, with X (its bf16 hi and lo halves), A and B in LDS.  On
// 256 x 256 tiles such a matrix would execute 16 times its Gram and square
// flops in padding and ride through 15 launches; here the whole matrix is one
// workgroup of one launch per step.
//
// The arithmetic is that of the tiled path: A = bf16(s^2 X_hi X_hi^T),
// B = bf16(b A + c A A), X' = s (a (X_hi [+ X_lo]) + B X_hi) rounded to the
// hi / lo pair (lo kept for the first kNsLoIters iterations), s the
// normalising factor in the first iteration only; the last iteration writes
// p = p decay - rate X' in the stored orientation.  Rows and columns are
// padded to multiples of 32 with the zeros the prep pass wrote.
//
// Work split over the four waves: one 32 x 32 block of A (or B) each (one
// wave when the matrix has at most 32 rows); the X update by 32-column
// blocks, wave w taking blocks w, w + 4, ...: a wave reads and writes only
// its own columns of X, so X is updated in place.  Fragments: A-operand rows
// (k contiguous) are 16-byte LDS reads; the X columns B X needs are gathered
// as eight 2-byte reads.
// ---------------------------------------------------------------------------
constexpr int kLdsXld = (int)kLdsCols + 8;  // row pitch (bf16) of X's halves: 16 rows fall in distinct banks
constexpr int kLdsAld = (int)kLdsRows + 8;  // row pitch of A and B

struct NsLds {
    __bf16 xhi[kLdsRows][kLdsXld];
    __bf16 xlo[kLdsRows][kLdsXld];
    __bf16 a[kLdsRows][kLdsAld];
    __bf16 b[kLdsRows][kLdsAld];
};
static_assert(sizeof(NsLds) <= 160 * 1024, "the matrix fits in a CU's LDS");

struct NsLdsArgs {
    float a, b, c;
    int steps;
    const float* scales;  // per matrix 1 / (||u||_F + eps)
    const StepDev* sd;
};

__device__ __forceinline__ uint4 lds_row8(const __bf16* p) { return *reinterpret_cast<const uint4*>(p); }

// Row of A (or B) at accumulator register e of this lane: 8 (e / 4) + 4 (lane / 32) + e % 4.
__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// Stored-orientation update of the 16 elements of one accumulator block
// that a lane holds (canonical rows row0 + acc_row(e), column col): p = p
// decay - dv, delta = dv, for the elements inside the matrix.  All 16 old
// values are loaded before the first store, so their latencies overlap.
template <typename P>
__device__ __forceinline__ void lds_update16(const MuonMat& d, int row0, int col, int lane,
                                             const float (&dv)[16], float decay) {
    typedef __attribute__((address_space(1))) P g_P;
    g_P* p = (g_P*)reinterpret_cast<P*>(d.p);
    int64_t o[16];
    float pv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int row = row0 + acc_row(e, lane);
        o[e] = d.transposed ? (int64_t)col * d.n + row : (int64_t)row * d.n + col;
        pv[e] = row < d.r && col < d.c ? (float)p[o[e]] : 0.f;
    }
    g_float* dl = (g_float*)reinterpret_cast<float*>(d.delta);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (row0 + acc_row(e, lane) < d.r && col < d.c) {
            p[o[e]] = (P)fmaf(pv[e], decay, -dv[e]);
            if (dl) dl[o[e]] = dv[e];
        }
    }
}

template <int R>
__device__ __forceinline__ void ns_lds_run(NsLds& L, const MuonMat& d, int mat,
                                           const NsLdsArgs& args) {
    constexpr int NB = R / 32;  // row blocks
    const int C = (d.c + 31) & ~31;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, h = lane >> 5;

    // X0 (hi and lo as the prep pass wrote them, 32 x 32 blocks of the
    // 256-padded operand) into LDS, 8 elements per access
    {
        const __bf16* ghi = reinterpret_cast<const __bf16*>(d.x[0]);
        const __bf16* glo = reinterpret_cast<const __bf16*>(d.xlo[0]);
        const int per_row = C / 8;
        for (int i = tid; i < R * per_row; i += 256) {
            const int row = i / per_row, col = (i % per_row) * 8;
            const int64_t o = xblk(row, col, d.C);
            *reinterpret_cast<uint4*>(&L.xhi[row][col]) = gld(ghi + o);
            *reinterpret_cast<uint4*>(&L.xlo[row][col]) = gld(glo + o);
        }
    }
    __syncthreads();

    const int bi = NB == 2 ? wave >> 1 : 0, bj = NB == 2 ? wave & 1 : 0;
    const bool sq_wave = NB == 2 || wave == 0;  // this wave owns a block of A and B
    for (int it = 0; it < args.steps; ++it) {
        const float s0 = it == 0 ? args.scales[mat] : 1.f;
        const bool use_lo = it < kNsLoIters, write_lo = it + 1 < kNsLoIters;
        const bool last = it == args.steps - 1;
        // A = bf16(s0^2 X_hi X_hi^T), K = C
        if (sq_wave) {
            f32x16 acc;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
            for (int k = 0; k < C; k += 16) {
                const uint4 fa = lds_row8(&L.xhi[bi * 32 + r32][k + 8 * h]);
                const uint4 fb = lds_row8(&L.xhi[bj * 32 + r32][k + 8 * h]);
                acc = Mma<__bf16>::run(fa, fb, acc);
            }
            const float sc = s0 * s0;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                L.a[bi * 32 + acc_row(e, lane)][bj * 32 + r32] = (__bf16)(acc[e] * sc);
        }
        __syncthreads();
        // B = bf16(b A + c A A), K = R (A is symmetric: its rows are its columns)
        if (sq_wave) {
            f32x16 acc;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
            for (int k = 0; k < R; k += 16) {
                const uint4 fa = lds_row8(&L.a[bi * 32 + r32][k + 8 * h]);
                const uint4 fb = lds_row8(&L.a[bj * 32 + r32][k + 8 * h]);
                acc = Mma<__bf16>::run(fa, fb, acc);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = bi * 32 + acc_row(e, lane), col = bj * 32 + r32;
                L.b[row][col] = (__bf16)fmaf(args.b, (float)L.a[row][col], args.c * acc[e]);
            }
        }
        __syncthreads();
        // X' = s0 (a X_master + B X_hi), K = R, by 32-column blocks
        const float rate = last ? (float)(args.sd->muon_lr * (double)d.shape_scale) : 0.f;
        const float decay = last ? args.sd->muon_decay : 1.f;
        for (int jb = wave; jb < C / 32; jb += 4) {
            const int col = jb * 32 + r32;
            f32x16 acc[NB];
#pragma unroll
            for (int ib = 0; ib < NB; ++ib)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[ib][e] = 0.f;
#pragma unroll
            for (int k = 0; k < R; k += 16) {
                // column `col` of X_hi at rows k + 8 h .. k + 8 h + 7
                typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
                u16x8 xc;
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    xc[t] = __builtin_bit_cast(unsigned short, L.xhi[k + 8 * h + t][col]);
                const uint4 fb = __builtin_bit_cast(uint4, xc);
#pragma unroll
                for (int ib = 0; ib < NB; ++ib)
                    acc[ib] = Mma<__bf16>::run(lds_row8(&L.b[ib * 32 + r32][k + 8 * h]), fb, acc[ib]);
            }
#pragma unroll
            for (int ib = 0; ib < NB; ++ib) {
                float dv[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = ib * 32 + acc_row(e, lane);
                    const float hi = (float)L.xhi[row][col];
                    const float t = fmaf(args.a, hi, acc[ib][e]);
                    const float v = use_lo ? s0 * fmaf(args.a, (float)L.xlo[row][col], t) : s0 * t;
                    if (!last) {
                        const __bf16 vh = (__bf16)v;
                        L.xhi[row][col] = vh;
                        if (write_lo) L.xlo[row][col] = (__bf16)(v - (float)vh);
                    }
                    dv[e] = rate * v;
                }
                if (last) {
                    if (d.p_bf16) lds_update16<__bf16>(d, ib * 32, col, lane, dv, decay);
                    else lds_update16<float>(d, ib * 32, col, lane, dv, decay);
                }
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void k_ns_lds_bf16(const MuonMat* __restrict__ tab, NsLdsArgs args) {
    __shared__ __attribute__((aligned(16))) NsLds L;
    const MuonMat& d = tab[blockIdx.x];
    if (!d.lds_ns) return;
    if (d.r <= 32) ns_lds_run<32>(L, d, blockIdx.x, args);
    else ns_lds_run<64>(L, d, blockIdx.x, args);
}

// One kernel per phase and operand type, named for what it computes so that
// traces and counters read directly.
#define NS_KERNEL(NAME, T, EPI)                                                           \
    __global__ __launch_bounds__(256) void NAME(const MuonMat* __restrict__ tab,          \
                                                const GemmTile* __restrict__ tiles,       \
                                                NsArgs args) {                            \
        ns_gemm_tile<T, EPI>(tab, tiles, args);                                          \
    }
// These kernels stay within 216 registers per wave (checked when built):
// two GEMM waves and one AdamW wave (80 registers) of the overlapped step
// then fill a SIMD's 512, so the side AdamW launch and the GEMM launches
// share every CU.
#define NS_KERNEL_W8(NAME, EPI)                                                           \
    __global__ __launch_bounds__(kW8Waves * 64) void NAME(const MuonMat* __restrict__ tab, \
                                                           const GemmTile* __restrict__ tiles, \
                                                           NsArgs args) {                  \
        ns_gemm_tile_w8<EPI>(tab, tiles, args);                                          \
    }
NS_KERNEL_W8(k_ns_gram_bf16, EPI_GRAM)
NS_KERNEL_W8(k_ns_poly_bf16, EPI_POLY)
NS_KERNEL_W8(k_ns_xupd_bf16, EPI_XUPD)
NS_KERNEL_W8(k_ns_final_bf16, EPI_FINAL)
#undef NS_KERNEL_W8
NS_KERNEL(k_ns_gram_f32, float, EPI_GRAM)
NS_KERNEL(k_ns_poly_f32, float, EPI_POLY)
NS_KERNEL(k_ns_xupd_f32, float, EPI_XUPD)
NS_KERNEL(k_ns_final_f32, float, EPI_FINAL)
#undef NS_KERNEL
#define NS_KERNEL_S32(NAME, EPI)                                                          \
    __global__ __launch_bounds__(kS32Waves * 64) void NAME(const MuonMat* __restrict__ tab, \
                                                const GemmTile* __restrict__ tiles,       \
                                                NsArgs args) {                            \
        ns_gemm_tile_s32<EPI>(tab, tiles, args);                                         \
    }
NS_KERNEL_S32(k_ns_gram_f32_s32, EPI_GRAM)
NS_KERNEL_S32(k_ns_poly_f32_s32, EPI_POLY)
#undef NS_KERNEL_S32
#define NS_KERNEL_S64(NAME, EPI)                                                          \
    __global__ __launch_bounds__(256) void NAME(const MuonMat* __restrict__ tab,          \
                                                const GemmTile* __restrict__ tiles,       \
                                                NsArgs args) {                            \
        ns_xupd_tile_s64<EPI>(tab, tiles, args);                                         \
    }
NS_KERNEL_S64(k_ns_xupd_f32_s64, EPI_XUPD)
NS_KERNEL_S64(k_ns_final_f32_s64, EPI_FINAL)
#undef NS_KERNEL_S64

typedef void (*NsKernel)(const MuonMat*, const GemmTile*, NsArgs);

int launch_k(NsKernel k, const MuonMat* tab, const GemmTile* tiles, int64_t n, const NsArgs& a,
             int threads, hipStream_t st) {
    static_assert(kGemmTile == 256, "large tile lists are built for 256x256 tiles");
    hipLaunchKernelGGL(k, dim3((unsigned)n), dim3(threads), 0, st, tab, tiles, a);
    return (int)hipGetLastError();
}

// A += the partial Grams of a split reduction, in slice order, for the fp32
// matrices of one Newton-Schulz batch (kReduceSplit workgroups per matrix,
// those of other matrices return at once).
constexpr int kReduceSplit = 256;  // one element per thread at R = 256

__global__ __launch_bounds__(256) void k_gram_reduce(const MuonMat* __restrict__ tab, int batch) {
    const int k = blockIdx.x / kReduceSplit, part = blockIdx.x % kReduceSplit;
    const MuonMat& d = tab[k];
    if (d.gram_ks <= 1 || d.op_bf16 || d.ns_batch != batch) return;
    float* a = reinterpret_cast<float*>(d.a);
    const float* pa = reinterpret_cast<const float*>(d.apart);
    const int64_t n = (int64_t)d.R * d.R;
    for (int64_t i = (int64_t)part * 256 + threadIdx.x; i < n; i += (int64_t)kReduceSplit * 256) {
        float v = a[i];
        for (int sl = 1; sl < d.gram_ks; ++sl) v += pa[(int64_t)(sl - 1) * n + i];
        a[i] = v;
    }
}

}  // namespace

int launch_gram_reduce(const MuonMat* tab, int32_t n_tab, int32_t batch, void* stream) {
    if (n_tab == 0) return (int)hipSuccess;
    hipLaunchKernelGGL(k_gram_reduce, dim3((unsigned)n_tab * kReduceSplit), dim3(256), 0,
                       (hipStream_t)stream, tab, (int)batch);
    return (int)hipGetLastError();
}

int launch_ns_lds(const MuonMat* tab, int32_t n_tab, int ns_steps, const StepScalars& s,
                  const float* ns_scale, const StepDev* sd, void* stream) {
    if (n_tab == 0) return (int)hipSuccess;
    const NsLdsArgs a{s.ns_a, s.ns_b, s.ns_c, ns_steps, ns_scale, sd};
    hipLaunchKernelGGL(k_ns_lds_bf16, dim3((unsigned)n_tab), dim3(256), 0, (hipStream_t)stream, tab,
                       a);
    return (int)hipGetLastError();
}

int launch_ns_phase(int phase, int32_t group, const MuonMat* tab, const GemmTile* tiles,
                    int64_t n_tiles, int iter, int last, const StepScalars& s,
                    const float* ns_scale, const StepDev* sd, void* stream) {
    if (n_tiles == 0) return (int)hipSuccess;
    NsArgs a{s.ns_a, s.ns_b, s.ns_c, iter, iter < kNsLoIters ? 1 : 0,
             iter + 1 < kNsLoIters ? 1 : 0, ns_scale, sd};
    hipStream_t st = (hipStream_t)stream;
    const int epi = phase == 1 ? EPI_GRAM : phase == 2 ? EPI_POLY : (last ? EPI_FINAL : EPI_XUPD);
    static const NsKernel bf[4] = {k_ns_gram_bf16, k_ns_poly_bf16, k_ns_xupd_bf16, k_ns_final_bf16};
    static const NsKernel f32[4] = {k_ns_gram_f32, k_ns_poly_f32, k_ns_xupd_f32, k_ns_final_f32};
    static const NsKernel f32s[4] = {k_ns_gram_f32_s32, k_ns_poly_f32_s32, k_ns_xupd_f32_s64,
                                     k_ns_final_f32_s64};
    if (group == kGroupBf16) return launch_k(bf[epi - 1], tab, tiles, n_tiles, a, kW8Waves * 64, st);
    if (group == kGroupFp32Small)
        return launch_k(f32s[epi - 1], tab, tiles, n_tiles, a, epi <= 2 ? kS32Waves * 64 : 256, st);
    return launch_k(f32[epi - 1], tab, tiles, n_tiles, a, 256, st);
}

}  // namespace ma
