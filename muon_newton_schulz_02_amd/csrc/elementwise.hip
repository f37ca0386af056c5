// HBM-bound kernels of the MuonAdamW step on gfx950:
//   * clip norm: multi-tensor sum of squares, one deterministic partial per
//     16 Ki-element chunk (wave shuffles + LDS tree), then one finalising
//     workgroup in double precision -> clip factor in device memory;
//   * AdamW: multi-tensor fused clip-scale + decoupled-decay Adam with
//     128-bit loads and stores;
//   * Muon prep: per 64 x 64 tile, clip-scale, momentum/Nesterov, buffer
//     write-back, the Newton-Schulz input operands in canonical orientation
//     (rows <= cols, transposed through LDS, zero padding) and a partial of
//     ||u||_F^2; per-matrix finalisation in double gives the normalising
//     factor that the first Newton-Schulz launches apply.
//
// Method: OpenDM training-stack page, Muon/AdamW hybrid section (routing,
// hyperparameter table: momentum 0.95 with Nesterov) and the defaults table
// (global clip to max_grad_norm 1.0).  The clip guard 1e-6 and the AdamW
// algorithm follow the usual clip_grad_norm_ / torch.optim.AdamW
// definitions, since the page names an HF-Trainer-based trainer.

#include <hip/hip_runtime.h>

#include "ma_internal.h"

namespace ma {
namespace {

constexpr int kThreads = 256;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Parameters and gradients are stored as float or bf16 (the plan's
// parameter storage); every value is computed on as float.  Four consecutive
// elements move as one 16-byte (float) or 8-byte (bf16) access; a bf16 value
// widens exactly and narrows with round to nearest, ties to even.
template <typename P>
struct Quad;
template <>
struct Quad<float> {
    typedef f4 raw;
    static __device__ __forceinline__ f4 get(raw r) { return r; }
    static __device__ __forceinline__ raw put(f4 v) { return v; }
};
template <>
struct Quad<__bf16> {
    typedef u32x2 raw;
    static __device__ __forceinline__ f4 get(raw r) {
        f4 v;
        v[0] = __uint_as_float(r[0] << 16);
        v[1] = __uint_as_float(r[0] & 0xffff0000u);
        v[2] = __uint_as_float(r[1] << 16);
        v[3] = __uint_as_float(r[1] & 0xffff0000u);
        return v;
    }
    static __device__ __forceinline__ raw put(f4 v) {
        const bf16x2 a = {(__bf16)v[0], (__bf16)v[1]};
        const bf16x2 b = {(__bf16)v[2], (__bf16)v[3]};
        raw r;
        r[0] = __builtin_bit_cast(unsigned int, a);
        r[1] = __builtin_bit_cast(unsigned int, b);
        return r;
    }
};

__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ float ld1(const __bf16* p) { return (float)*p; }
__device__ __forceinline__ void st1(float* p, float v) { *p = v; }
__device__ __forceinline__ void st1(__bf16* p, float v) { *p = (__bf16)v; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Block-wide sum in a fixed order (same result on every run).
__device__ __forceinline__ float block_sum(float v, float* smem) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) smem[wave] = v;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0) {
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += smem[w];
    }
    return t;  // valid in thread 0 only
}

// Index of the table entry whose chunk range holds `chunk` (binary search
// over ascending chunk_begin).
template <typename Tab>
__device__ __forceinline__ int find_tensor(const Tab* tab, int n, int64_t chunk) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab[mid].chunk_begin <= chunk) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ------------------------------------------------------- table upload --
// The step's descriptor tables, from mapped host memory into the workspace.
__global__ __launch_bounds__(kThreads) void k_copy_tables(const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * kThreads)
        dst[i] = src[i];
}

// ------------------------------------------------------------ clip norm --
template <typename G>
__global__ __launch_bounds__(kThreads) void k_norm_partials(const NormTensor* __restrict__ tab,
                                                            int n_tab,
                                                            float* __restrict__ partials) {
    __shared__ float smem[kThreads / 64];
    const int64_t chunk = blockIdx.x;
    const int t = find_tensor(tab, n_tab, chunk);
    const NormTensor d = tab[t];
    const int64_t begin = (chunk - d.chunk_begin) * kChunk;
    const int64_t len = min<int64_t>(kChunk, d.numel - begin);
    const G* g = reinterpret_cast<const G*>(d.g) + begin;
    float acc = 0.f;
    if (d.vec_ok && len == kChunk) {
        // 16-byte loads: 4 floats or 8 bf16, summed in element order
        const u32x4* g16 = reinterpret_cast<const u32x4*>(g);
        constexpr int kPer = 16 / (int)sizeof(G);
#pragma unroll 4
        for (int i = threadIdx.x; i < kChunk / kPer; i += kThreads) {
            const u32x4 w = __builtin_nontemporal_load(g16 + i);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (sizeof(G) == 4) {
                    const float x = __uint_as_float(w[q]);
                    acc = fmaf(x, x, acc);
                } else {
                    const float lo = __uint_as_float(w[q] << 16);
                    const float hi = __uint_as_float(w[q] & 0xffff0000u);
                    acc = fmaf(lo, lo, acc);
                    acc = fmaf(hi, hi, acc);
                }
            }
        }
    } else {
        for (int64_t i = threadIdx.x; i < len; i += kThreads) {
            const float v = ld1(g + i);
            acc = fmaf(v, v, acc);
        }
    }
    const float s = block_sum(acc, smem);
    if (threadIdx.x == 0) partials[chunk] = s;
}

// Learning rate of optimizer step t (counted from 1): the base rate times the
// schedule's factor at scheduler step t - 1.  cosine_with_min_lr (the page's
// defaults table): a linear warmup from 0, then half a cosine from 1 down to
// min_lr_rate over total_steps - warmup_steps steps, held there after.
__device__ double scheduled_lr(const StepIn& in, int64_t t) {
    if (in.schedule != MA_LR_COSINE_MIN) return in.lr;
    const int64_t k = t - 1;
    if (k < in.warmup_steps) return in.lr * (double)k / (double)max(int64_t(1), in.warmup_steps);
    const double span = (double)max(int64_t(1), in.total_steps - in.warmup_steps);
    const double progress = fmin(1.0, (double)(k - in.warmup_steps) / span);
    const double half_cosine = 0.5 * (1.0 + cos(M_PI * progress));
    return in.lr * (in.min_lr_rate + (1.0 - in.min_lr_rate) * half_cosine);
}

__global__ __launch_bounds__(1024) void k_clip_finalize(const float* __restrict__ partials,
                                                        int64_t n, float max_norm, StepIn in,
                                                        StepDev* __restrict__ sd,
                                                        float* __restrict__ user_norm_out) {
    __shared__ double smem[1024 / 64];
    // eight independent sums per thread, so its loads are in flight together
    // (one dependent sum waited on every load: 38 us for the 131 K partials
    // of the full hybrid table); combined in a fixed order
    const int64_t stride = blockDim.x;
    double a8[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    int64_t i = threadIdx.x;
    for (; i + 7 * stride < n; i += 8 * stride) {
#pragma unroll
        for (int u = 0; u < 8; ++u) a8[u] += (double)partials[i + u * stride];
    }
    for (int u = 0; i < n; i += stride, ++u) a8[u & 7] += (double)partials[i];
    double acc = ((a8[0] + a8[1]) + (a8[2] + a8[3])) + ((a8[4] + a8[5]) + (a8[6] + a8[7]));
    acc = wave_sum_d(acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) smem[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += smem[w];
        const double norm = sqrt(tot);
        double coef = 1.0;
        if (max_norm > 0.f) {
            coef = (double)max_norm / (norm + 1e-6);
            if (!(coef < 1.0)) coef = (coef == coef) ? 1.0 : coef;  // NaN propagates
        }
        sd->coef = (float)coef;
        sd->norm = (float)norm;
        sd->claim = 0;
        if (user_norm_out) user_norm_out[0] = (float)norm;
        // the step number and everything that depends on it (formed in
        // double, rounded once): the scheduled rate, AdamW's bias
        // corrections and decay, the Muon rate and decay
        int64_t t = in.t_host;
        if (in.device_step) {
            t = *in.device_step + 1;
            *in.device_step = t;
        }
        const double lr = scheduled_lr(in, t);
        const double bc1 = 1.0 - pow(in.beta1, (double)t);
        const double bc2 = 1.0 - pow(in.beta2, (double)t);
        sd->step_size = (float)(lr / (bc1 > 0.0 ? bc1 : 1.0));
        sd->inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2 > 0.0 ? bc2 : 1.0));
        sd->adam_decay = (float)(1.0 - lr * in.weight_decay);
        sd->muon_lr = lr * in.muon_lr_scale;
        sd->muon_decay = (float)(1.0 - lr * in.muon_weight_decay);
    }
}

// ---------------------------------------------------------------- AdamW --
struct AdamArgs {
    float step_size, inv_sqrt_bc2, decay, beta1, beta2, one_m_beta1, one_m_beta2, eps;
};

// The step-independent constants of AdamW, completed from the step's
// device values.
struct AdamConst {
    float beta1, beta2, one_m_beta1, one_m_beta2, eps;
};

__device__ __forceinline__ AdamArgs adam_args(const AdamConst& c, const StepDev* sd) {
    AdamArgs a;
    a.step_size = sd->step_size;
    a.inv_sqrt_bc2 = sd->inv_sqrt_bc2;
    a.decay = sd->adam_decay;
    a.beta1 = c.beta1;
    a.beta2 = c.beta2;
    a.one_m_beta1 = c.one_m_beta1;
    a.one_m_beta2 = c.one_m_beta2;
    a.eps = c.eps;
    return a;
}

__device__ __forceinline__ void adam_elem(float& p, float g, float& m, float& v, float coef,
                                          const AdamArgs& a) {
    g *= coef;
    p *= a.decay;
    m = fmaf(a.beta1, m, a.one_m_beta1 * g);
    v = fmaf(a.beta2, v, a.one_m_beta2 * g * g);
    const float denom = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
    p = fmaf(-a.step_size, m / denom, p);
}

// One chunk per workgroup.  Workgroup b runs on XCD b % 8 (the dispatcher
// hands consecutive workgroups to the XCDs in turn), and XCD x takes the
// x-th contiguous eighth of the chunks, so the pages each XCD streams
// through stay together: 5.21 -> 5.35 TB/s on the 1.88e9-element AdamW
// group against chunk b on workgroup b.  The grid is 8 ceil(n_chunks / 8).
template <int U, typename P>
__global__ __launch_bounds__(kThreads) void k_adamw(const AdamTensor* __restrict__ tab, int n_tab,
                                                    const StepDev* __restrict__ sd,
                                                    AdamConst ac, int64_t n_chunks) {
    const AdamArgs a = adam_args(ac, sd);
    const int64_t per = (n_chunks + kXcds - 1) / kXcds;
    const int64_t chunk = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (chunk >= n_chunks) return;
    const int t = find_tensor(tab, n_tab, chunk);
    const AdamTensor d = tab[t];
    const int64_t begin = (chunk - d.chunk_begin) * kChunk;
    const int64_t len = min<int64_t>(kChunk, d.numel - begin);
    P* p = reinterpret_cast<P*>(d.p) + begin;
    const P* g = reinterpret_cast<const P*>(d.g) + begin;
    float* m = reinterpret_cast<float*>(d.m) + begin;
    float* v = reinterpret_cast<float*>(d.v) + begin;
    const float coef = sd->coef;
    if (d.vec_ok && len == kChunk) {
        typedef typename Quad<P>::raw PR;
        PR* p4 = reinterpret_cast<PR*>(p);
        const PR* g4 = reinterpret_cast<const PR*>(g);
        f4* m4 = reinterpret_cast<f4*>(m);
        f4* v4 = reinterpret_cast<f4*>(v);
        // U vectors of each of the four streams in flight per thread before
        // any arithmetic (the chunk is 16 of them per thread)
        static_assert(kChunk / 4 % (kThreads * U) == 0, "chunk split");
        for (int i0 = threadIdx.x; i0 < kChunk / 4; i0 += kThreads * U) {
            PR pr[U], gr[U];
            f4 mm[U], vv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * kThreads;
                pr[u] = __builtin_nontemporal_load(p4 + i);
                gr[u] = __builtin_nontemporal_load(g4 + i);
                mm[u] = __builtin_nontemporal_load(m4 + i);
                vv[u] = __builtin_nontemporal_load(v4 + i);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                f4 pp = Quad<P>::get(pr[u]);
                const f4 gg = Quad<P>::get(gr[u]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float pq = pp[q], mq = mm[u][q], vq = vv[u][q];
                    adam_elem(pq, gg[q], mq, vq, coef, a);
                    pp[q] = pq;
                    mm[u][q] = mq;
                    vv[u][q] = vq;
                }
                pr[u] = Quad<P>::put(pp);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * kThreads;
                __builtin_nontemporal_store(pr[u], p4 + i);
                __builtin_nontemporal_store(mm[u], m4 + i);
                __builtin_nontemporal_store(vv[u], v4 + i);
            }
        }
    } else {
        for (int64_t i = threadIdx.x; i < len; i += kThreads) {
            float pp = ld1(p + i), mm = m[i], vv = v[i];
            adam_elem(pp, ld1(g + i), mm, vv, coef, a);
            st1(p + i, pp);
            m[i] = mm;
            v[i] = vv;
        }
    }
}

// One 16 Ki-element chunk of AdamW done by a single wave (64 lanes), U
// four-element vectors of each of the four streams in flight per lane.
template <int U, typename P>
__device__ __forceinline__ void adamw_chunk_wave(const AdamTensor* __restrict__ tab, int n_tab,
                                                 int64_t chunk, float coef, const AdamArgs& a,
                                                 int lane) {
    const int t = find_tensor(tab, n_tab, chunk);
    const AdamTensor d = tab[t];
    const int64_t begin = (chunk - d.chunk_begin) * kChunk;
    const int64_t len = min<int64_t>(kChunk, d.numel - begin);
    P* p = reinterpret_cast<P*>(d.p) + begin;
    const P* g = reinterpret_cast<const P*>(d.g) + begin;
    float* m = reinterpret_cast<float*>(d.m) + begin;
    float* v = reinterpret_cast<float*>(d.v) + begin;
    if (d.vec_ok && len == kChunk) {
        typedef typename Quad<P>::raw PR;
        PR* p4 = reinterpret_cast<PR*>(p);
        const PR* g4 = reinterpret_cast<const PR*>(g);
        f4* m4 = reinterpret_cast<f4*>(m);
        f4* v4 = reinterpret_cast<f4*>(v);
        static_assert(kChunk / 4 % (64 * U) == 0, "chunk split");
        for (int i0 = lane; i0 < kChunk / 4; i0 += 64 * U) {
            PR pr[U], gr[U];
            f4 mm[U], vv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * 64;
                pr[u] = __builtin_nontemporal_load(p4 + i);
                gr[u] = __builtin_nontemporal_load(g4 + i);
                mm[u] = __builtin_nontemporal_load(m4 + i);
                vv[u] = __builtin_nontemporal_load(v4 + i);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                f4 pp = Quad<P>::get(pr[u]);
                const f4 gg = Quad<P>::get(gr[u]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float pq = pp[q], mq = mm[u][q], vq = vv[u][q];
                    adam_elem(pq, gg[q], mq, vq, coef, a);
                    pp[q] = pq;
                    mm[u][q] = mq;
                    vv[u][q] = vq;
                }
                pr[u] = Quad<P>::put(pp);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * 64;
                __builtin_nontemporal_store(pr[u], p4 + i);
                __builtin_nontemporal_store(mm[u], m4 + i);
                __builtin_nontemporal_store(vv[u], v4 + i);
            }
        }
    } else {
        for (int64_t i = lane; i < len; i += 64) {
            float pp = ld1(p + i), mm = m[i], vv = v[i];
            adam_elem(pp, ld1(g + i), mm, vv, coef, a);
            st1(p + i, pp);
            m[i] = mm;
            v[i] = vv;
        }
    }
}

// AdamW with chunks claimed per wave from a shared counter; every wave runs
// until the counter passes n_chunks.  At most 80 VGPRs (six waves per SIMD),
// so a wave fits on a SIMD beside two Newton-Schulz GEMM waves (at most 216
// registers each).
template <int U, typename P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) void k_adamw_claim(
    const AdamTensor* __restrict__ tab, int n_tab, int64_t n_chunks, StepDev* __restrict__ sd,
    AdamConst ac) {
    const AdamArgs a = adam_args(ac, sd);
    const int lane = threadIdx.x & 63;
    const float coef = sd->coef;
    // one counter for the whole group: per-XCD counters over contiguous
    // eighths (as k_adamw maps its chunks) made the overlapped step 0.65 ms
    // slower on the full hybrid table.  Claims on one address serialise
    // (about 12 ns each), so a wave that starts after every chunk was claimed
    // leaves after a plain read of the counter: 8192 idle waves of the
    // finishing launch took 95 us with an atomic each.
    {
        int c = 0;
        if (lane == 0) c = __hip_atomic_load(&sd->claim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        c = __builtin_amdgcn_readfirstlane(c);
        if ((int64_t)c >= n_chunks) return;
    }
    for (;;) {
        int c = 0;
        if (lane == 0) c = atomicAdd(&sd->claim, 1);
        c = __builtin_amdgcn_readfirstlane(c);
        if ((int64_t)c >= n_chunks) break;
        adamw_chunk_wave<U, P>(tab, n_tab, c, coef, a, lane);
    }
}

// ------------------------------------------------- Muon momentum + operands --
struct MomArgs {
    float mu;
    int nesterov;
};

// Clip-scaled gradient, momentum buffer update and the Nesterov (or plain)
// momentum direction u of one element.
__device__ __forceinline__ float momentum_elem(float g, float& buf, float coef, const MomArgs& a) {
    const float gc = g * coef;
    buf = fmaf(a.mu, buf, gc);
    return a.nesterov ? fmaf(a.mu, buf, gc) : buf;
}

// Index of the Muon matrix whose operand-tile range holds `blk`.
__device__ __forceinline__ int find_matrix(const MuonMat* tab, int n, int64_t blk) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab[mid].orient_begin <= blk) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The Newton-Schulz input operand of canonical tile (i0, j0), from the LDS
// tile of u in stored orientation: canonical (i, j) is stored (i, j), or
// stored (j, i) for a transposed matrix.  Values outside the true r x c are
// zero.
// bf16 operands: X as a hi / lo pair of bf16 matrices (step-0 buffers),
// hi = RNE(x), lo = RNE(x - hi), each stored in 32x32 blocks of 2 KB
// (row-major inside a block, block-row-major outside), the layout the
// Newton-Schulz launches read and write.
// A thread writes eight consecutive elements of a canonical row (16 bytes of
// hi and of lo: one run inside a 32x32 block) per store.
__device__ __forceinline__ void write_operands_bf16(const MuonMat& d,
                                                    const float (*tile)[kOrientTile + 1], int i0,
                                                    int j0) {
    constexpr int TS = kOrientTile;
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    __bf16* hi = reinterpret_cast<__bf16*>(d.x[0]);
    __bf16* lo = reinterpret_cast<__bf16*>(d.xlo[0]);
    for (int c = threadIdx.x; c < TS * TS / 8; c += kThreads) {
        const int a_ = c / (TS / 8), b0 = (c % (TS / 8)) * 8;
        const int i = i0 + a_, j = j0 + b0;
        const int64_t o = ((int64_t)(i >> 5) * (d.C >> 5) + (j >> 5)) * 1024 + (i & 31) * 32 + (j & 31);
        bf16x8_t h, l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = d.transposed ? tile[b0 + e][a_] : tile[a_][b0 + e];
            h[e] = (__bf16)v;
            l[e] = (__bf16)(v - (float)h[e]);
        }
        *reinterpret_cast<bf16x8_t*>(hi + o) = h;
        *reinterpret_cast<bf16x8_t*>(lo + o) = l;
    }
}

// fp32 operands: X row-major (the master) and X^T (step-0 buffer).
__device__ __forceinline__ void write_operands_fp32(const MuonMat& d,
                                                    const float (*tile)[kOrientTile + 1], int i0,
                                                    int j0) {
    constexpr int TS = kOrientTile;
    float* x = reinterpret_cast<float*>(d.x[0]);
    float* xt = reinterpret_cast<float*>(d.xt[0]);
    for (int idx = threadIdx.x; idx < TS * TS; idx += kThreads) {
        const int a_ = idx / TS, b_ = idx % TS;
        x[(int64_t)(i0 + a_) * d.C + (j0 + b_)] = d.transposed ? tile[b_][a_] : tile[a_][b_];
    }
    for (int idx = threadIdx.x; idx < TS * TS; idx += kThreads) {
        const int a_ = idx / TS, b_ = idx % TS;  // a_ along canonical cols, b_ along rows
        xt[(int64_t)(j0 + a_) * d.R + (i0 + b_)] = d.transposed ? tile[a_][b_] : tile[b_][a_];
    }
}

// One 64 x 64 tile of the padded canonical R x C operand of a Muon matrix:
// read the clip-scaled gradient and the momentum buffer of the stored tile,
// write the updated buffer back, and write u -- not yet normalised -- as the
// Newton-Schulz input operand in canonical orientation, zero padding
// included; plus this tile's partial of ||u||_F^2.  The normalising factor
// is applied by the first Newton-Schulz launches (Gram: its square; X
// update: itself), which is exact up to rounding since every product is
// homogeneous in X.
__global__ __launch_bounds__(kThreads) void k_muon_prep(const MuonMat* __restrict__ tab, int n_tab,
                                                        const StepDev* __restrict__ sd,
                                                        MomArgs a, float* __restrict__ partials,
                                                        int batch) {
    constexpr int TS = kOrientTile;
    __shared__ float tile[TS][TS + 1];
    __shared__ float smem[kThreads / 64];
    const int64_t blk = blockIdx.x;
    const MuonMat& d = tab[find_matrix(tab, n_tab, blk)];
    if (batch >= 0 && d.ns_batch != batch) return;   // uniform over the workgroup
    const int64_t local = blk - d.orient_begin;
    const int tiles_c = d.C / TS;
    const int i0 = (int)(local / tiles_c) * TS, j0 = (int)(local % tiles_c) * TS;
    const float coef = sd->coef;
    const float* g = reinterpret_cast<const float*>(d.g);
    const __bf16* gh = reinterpret_cast<const __bf16*>(d.g);   // bf16 storage
    float* buf = reinterpret_cast<float*>(d.buf);
    // stored tile origin: rows sr0.., cols sc0..
    const int sr0 = d.transposed ? j0 : i0;
    const int sc0 = d.transposed ? i0 : j0;
    float acc = 0.f;
    if (d.vec_ok && sr0 + TS <= d.m && sc0 + TS <= d.n) {
        // whole tile inside the matrix: 16-byte accesses, NQ of each stream
        // per thread, all loads issued before the first store
        constexpr int NQ = TS * TS / 4 / kThreads;
        static_assert(NQ * kThreads * 4 == TS * TS, "the tile splits evenly over the threads");
        f4 gg[NQ];
        float4 bb[NQ];
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int q = threadIdx.x + k * kThreads;
            const int lr = q / (TS / 4), lc = (q % (TS / 4)) * 4;
            const int64_t o = (int64_t)(sr0 + lr) * d.n + (sc0 + lc);
            gg[k] = d.p_bf16 ? Quad<__bf16>::get(*reinterpret_cast<const u32x2*>(gh + o))
                             : *reinterpret_cast<const f4*>(g + o);
            bb[k] = *reinterpret_cast<const float4*>(buf + o);
        }
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int q = threadIdx.x + k * kThreads;
            const int lr = q / (TS / 4), lc = (q % (TS / 4)) * 4;
            const int64_t o = (int64_t)(sr0 + lr) * d.n + (sc0 + lc);
            const float u0 = momentum_elem(gg[k][0], bb[k].x, coef, a);
            const float u1 = momentum_elem(gg[k][1], bb[k].y, coef, a);
            const float u2 = momentum_elem(gg[k][2], bb[k].z, coef, a);
            const float u3 = momentum_elem(gg[k][3], bb[k].w, coef, a);
            *reinterpret_cast<float4*>(buf + o) = bb[k];
            tile[lr][lc] = u0;
            tile[lr][lc + 1] = u1;
            tile[lr][lc + 2] = u2;
            tile[lr][lc + 3] = u3;
            acc = fmaf(u0, u0, acc);
            acc = fmaf(u1, u1, acc);
            acc = fmaf(u2, u2, acc);
            acc = fmaf(u3, u3, acc);
        }
    } else {
        for (int idx = threadIdx.x; idx < TS * TS; idx += kThreads) {
            const int lr = idx / TS, lc = idx % TS;
            const int sr = sr0 + lr, sc = sc0 + lc;
            float u = 0.f;
            if (sr < d.m && sc < d.n) {
                const int64_t o = (int64_t)sr * d.n + sc;
                float bb = buf[o];
                u = momentum_elem(d.p_bf16 ? (float)gh[o] : g[o], bb, coef, a);
                buf[o] = bb;
            }
            tile[lr][lc] = u;
            acc = fmaf(u, u, acc);
        }
    }
    const float part = block_sum(acc, smem);  // its barrier also completes the tile
    if (threadIdx.x == 0) partials[blk] = part;
    if (d.op_bf16) write_operands_bf16(d, tile, i0, j0);
    else write_operands_fp32(d, tile, i0, j0);
}

// Below 2^-40 or above 2^40 for ||u||_F, products of unnormalised operand
// values could leave the fp32 range inside the Gram product; such matrices
// get their operands scaled in place instead (k_operand_rescale).
constexpr double kNormLo = 0x1p-40, kNormHi = 0x1p40;

// One workgroup per matrix: s = 1 / (||u||_F + eps) from its tile partials,
// summed in double in a fixed order.  ns_scale[k] is the factor the first
// Newton-Schulz launches apply; pre_scale[k] != 0 asks k_operand_rescale to
// scale the operands themselves (and ns_scale[k] is then 1).
__global__ __launch_bounds__(256) void k_muon_scale(const MuonMat* __restrict__ tab,
                                                    const float* __restrict__ partials,
                                                    float ns_eps, float* __restrict__ ns_scale,
                                                    float* __restrict__ pre_scale, int batch) {
    __shared__ double smem[256 / 64];
    const MuonMat& d = tab[blockIdx.x];
    if (batch >= 0 && d.ns_batch != batch) return;   // uniform over the workgroup
    const int64_t n_tiles = (int64_t)(d.R / kOrientTile) * (d.C / kOrientTile);
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < n_tiles; i += blockDim.x)
        acc += (double)partials[d.orient_begin + i];
    acc = wave_sum_d(acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) smem[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int w = 0; w < 4; ++w) tot += smem[w];
        const double nrm = sqrt(tot);
        const float s = (float)(1.0 / (nrm + (double)ns_eps));
        const bool in_range = nrm >= kNormLo && nrm <= kNormHi;  // false for NaN
        ns_scale[blockIdx.x] = in_range ? s : 1.f;
        pre_scale[blockIdx.x] = in_range ? 0.f : s;
    }
}

// Scale the Newton-Schulz input operands of the matrices whose pre_scale is
// non-zero (a norm outside [2^-40, 2^40]); kRescaleSplit workgroups per
// matrix, the others return at once.
constexpr int kRescaleSplit = 16;

__global__ __launch_bounds__(kThreads) void k_operand_rescale(const MuonMat* __restrict__ tab,
                                                              const float* __restrict__ pre_scale,
                                                              int batch) {
    const int k = blockIdx.x / kRescaleSplit, part = blockIdx.x % kRescaleSplit;
    const MuonMat& d = tab[k];
    // pre_scale of another batch's matrix belongs to another launch
    if (batch >= 0 && d.ns_batch != batch) return;
    const float f = pre_scale[k];
    if (f == 0.f) return;
    const int64_t n = (int64_t)d.R * d.C;
    const int64_t stride = (int64_t)kRescaleSplit * kThreads;
    if (d.op_bf16) {
        __bf16* hi = reinterpret_cast<__bf16*>(d.x[0]);
        __bf16* lo = reinterpret_cast<__bf16*>(d.xlo[0]);
        for (int64_t i = (int64_t)part * kThreads + threadIdx.x; i < n; i += stride) {
            const float v = f * ((float)hi[i] + (float)lo[i]);
            const __bf16 h = (__bf16)v;
            hi[i] = h;
            lo[i] = (__bf16)(v - (float)h);
        }
    } else {
        float* x = reinterpret_cast<float*>(d.x[0]);
        float* xt = reinterpret_cast<float*>(d.xt[0]);
        for (int64_t i = (int64_t)part * kThreads + threadIdx.x; i < n; i += stride) {
            x[i] *= f;
            xt[i] *= f;
        }
    }
}
}  // namespace

int launch_copy_tables(void* dst, const void* src, size_t bytes, void* stream) {
    if (bytes == 0) return (int)hipSuccess;
    if (bytes % 16 != 0) return (int)hipErrorInvalidValue;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t grid = std::min<int64_t>(64, (n16 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(k_copy_tables, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), n16);
    return (int)hipGetLastError();
}

int launch_norm_partials(const NormTensor* tab, int32_t n_tab, int64_t n_chunks, float* partials,
                         int32_t param_dtype, void* stream) {
    if (n_chunks == 0) return (int)hipSuccess;
    auto k = param_dtype == MA_PARAM_BF16 ? k_norm_partials<__bf16> : k_norm_partials<float>;
    hipLaunchKernelGGL(k, dim3((unsigned)n_chunks), dim3(kThreads), 0, (hipStream_t)stream, tab,
                       n_tab, partials);
    return (int)hipGetLastError();
}

int launch_clip_finalize(const float* partials, int64_t n, float max_grad_norm,
                         const StepIn& in, StepDev* sd, float* user_norm_out, void* stream) {
    hipLaunchKernelGGL(k_clip_finalize, dim3(1), dim3(1024), 0, (hipStream_t)stream, partials, n,
                       max_grad_norm, in, sd, user_norm_out);
    return (int)hipGetLastError();
}

AdamConst adam_const(const StepScalars& s) {
    AdamConst c;
    c.beta1 = s.beta1;
    c.beta2 = s.beta2;
    c.one_m_beta1 = s.one_m_beta1;
    c.one_m_beta2 = s.one_m_beta2;
    c.eps = s.eps;
    return c;
}

int launch_adamw(const AdamTensor* tab, int32_t n_tab, int64_t n_chunks, const StepDev* sd,
                 const StepScalars& s, int32_t param_dtype, void* stream) {
    if (n_chunks == 0) return (int)hipSuccess;
    // four vectors per stream in flight (108 VGPRs) for the full HBM rate
    auto k = param_dtype == MA_PARAM_BF16 ? k_adamw<4, __bf16> : k_adamw<4, float>;
    hipLaunchKernelGGL(k, dim3((unsigned)(kXcds * ((n_chunks + kXcds - 1) / kXcds))),
                       dim3(kThreads), 0, (hipStream_t)stream, tab, n_tab, sd, adam_const(s),
                       n_chunks);
    return (int)hipGetLastError();
}

int launch_adamw_claim(const AdamTensor* tab, int32_t n_tab, int64_t n_chunks, StepDev* sd,
                       const StepScalars& s, int32_t param_dtype, int64_t grid, int waves,
                       void* stream) {
    if (n_chunks == 0 || grid <= 0) return (int)hipSuccess;
    if (waves < 1 || waves > kThreads / 64) return (int)hipErrorInvalidValue;
    // four vectors per stream in flight in 80 VGPRs, which with a
    // Newton-Schulz GEMM wave's at most 432 registers fills a SIMD's 512
    auto k = param_dtype == MA_PARAM_BF16 ? k_adamw_claim<4, __bf16> : k_adamw_claim<4, float>;
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * waves), 0, (hipStream_t)stream, tab,
                       n_tab, n_chunks, sd, adam_const(s));
    return (int)hipGetLastError();
}

int launch_muon_prep(const MuonMat* tab, int32_t n_tab, int64_t n_tiles, const StepDev* sd,
                     const StepScalars& s, float* partials, int32_t batch, void* stream) {
    if (n_tiles == 0) return (int)hipSuccess;
    MomArgs a{s.mu, s.nesterov};
    hipLaunchKernelGGL(k_muon_prep, dim3((unsigned)n_tiles), dim3(kThreads), 0, (hipStream_t)stream,
                       tab, n_tab, sd, a, partials, (int)batch);
    return (int)hipGetLastError();
}

int launch_muon_scale(const MuonMat* tab, int32_t n_tab, const float* partials, float ns_eps,
                      float* ns_scale, float* pre_scale, int32_t batch, void* stream) {
    if (n_tab == 0) return (int)hipSuccess;
    hipLaunchKernelGGL(k_muon_scale, dim3((unsigned)n_tab), dim3(256), 0, (hipStream_t)stream, tab,
                       partials, ns_eps, ns_scale, pre_scale, (int)batch);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(k_operand_rescale, dim3((unsigned)n_tab * kRescaleSplit), dim3(kThreads), 0,
                       (hipStream_t)stream, tab, pre_scale, (int)batch);
    return (int)hipGetLastError();
}

}  // namespace ma
