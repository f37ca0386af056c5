// Internal declarations of the MuonAdamW library: the plan object, the
// device-side descriptor tables uploaded at every step, the workspace layout
// and the kernel launchers.  Not part of the C ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon_adamw.h"

namespace ma {

// Every Newton-Schulz operand is padded with zeros to a multiple of this in
// both dimensions, so GEMM tiles (which divide it) never need bounds checks
// and the zero padding contributes nothing to any product.
constexpr int64_t kNsPad = 256;

// Elements per chunk of the multi-tensor elementwise passes (clip norm,
// AdamW, Muon momentum).  Each chunk is one workgroup's work and produces one
// deterministic partial sum.
constexpr int64_t kChunk = 16384;

// Side of the square tiles of the normalise/orient pass.
constexpr int kOrientTile = 64;

// GEMM block tile (square) used for the work lists.  Must divide kNsPad.
constexpr int kGemmTile = 256;

// Under the bf16 policy, matrices whose smaller side is below this run their
// Newton-Schulz in fp32: for such thin matrices the bf16 rounding error is
// inherent and reaches the 2e-2 tolerance (Gaussian inputs with two or three
// rows reach 2.1-2.4e-2 under this policy, against at most 1.6e-2 from four
// rows on), while their share of the work is negligible.
constexpr int64_t kBf16MinRows = 16;

// bf16 Newton-Schulz iterations whose linear term a X uses the 16-bit
// master (the bf16 pair hi + lo); later iterations use hi alone and keep no
// lo half.  Modelled by the oracle's bf16-policy diagnostic: on the rank-8
// spike input 3 gives 1.1e-2 relative error against fp64 (5: 1e-3, 2: 3.7e-2)
// and on Gaussian or row-scaled inputs 6-9e-3 (5: 7-10e-3).
constexpr int kNsLoIters = 3;

// XCDs of an MI355X: consecutive workgroups of a launch are dispatched to
// XCDs round-robin, and each XCD has its own L2.
constexpr int kXcds = 8;
constexpr int kCus = 256;          // compute units of an MI355X
constexpr int kGramMaxSlices = 4;  // most slices of a split Gram reduction
// Newton-Schulz runs the Muon matrices in batches, each batch through all of
// its iterations; consecutive batches alternate between this many streams
// (the caller's and a library-owned one), so the tail of one batch's launch
// overlaps the other stream's work.
constexpr int kNsStreams = 2;
// When the AdamW group runs beside bf16 Newton-Schulz, batches hold about
// this many operand bytes (X as hi + lo bf16): the plan makes kNsStreams x
// ceil(total / (kNsStreams x this)) batches of about equal GEMM work.
// Otherwise there are kNsStreams batches.
constexpr size_t kNsOverlapBatchBytes = size_t(160) << 20;
// Pinned host buffers the descriptor tables are staged in, used in rotation:
// a step waits for the upload of the step this many calls before it.
constexpr int kStagingSlots = 4;
// Bytes of the per-device scratch the allocation-free step works in (the
// largest workspace it accepts).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// ---------------------------------------------------------------- tables --
// One trainable tensor in the global-norm pass.
struct NormTensor {
    uint64_t g;            // const float* or bf16* (the plan's parameter storage)
    int64_t  numel;
    int64_t  chunk_begin;  // first chunk index of this tensor
    int32_t  vec_ok;       // 16-byte aligned base: 16-byte loads allowed
    int32_t  pad_;
};

// One AdamW tensor.
struct AdamTensor {
    uint64_t p, g, m, v;   // p, g: float* or bf16* (parameter storage); m, v: float*
    int64_t  numel;
    int64_t  chunk_begin;
    int32_t  vec_ok;
    int32_t  pad_;
};

// One Muon matrix: the elementwise view (momentum pass) and the NS view.
struct MuonMat {
    uint64_t p, g, buf, delta;     // p, g: float* or bf16*; buf, delta: float* (delta may be 0)
    // NS operands, zero-padded to R x C (X), C x R (X^T), R x R (A, B):
    //   bf16: x[k] = hi part of X (row-major; the MFMA operand) and xlo[k] =
    //         its lo part, ping-pong buffers k = step parity; xt unused
    //   fp32: x[0] = X (row-major master and operand), xt[k] = X^T ping-pong
    uint64_t x[2], xlo[2], xt[2];
    uint64_t a, b;                 // R x R, operand type
    int64_t  numel;                // m * n
    int64_t  orient_begin;         // first 64 x 64 operand tile of the prep pass
    int32_t  m, n, r, c, R, C;
    int32_t  transposed;
    int32_t  vec_ok;               // 16-byte row runs of p and buf (and delta), 4-element g loads
    float    shape_scale;          // lr_shape_scale: the update is muon_lr * this (StepDev)
    int32_t  op_bf16;              // NS operands are bf16 (else fp32)
    int32_t  p_bf16;               // p and g stored as bf16 (else float)
    int32_t  ns_batch;             // its Newton-Schulz batch
    int32_t  gram_ks;              // Gram reduction split into this many slices (fp32 only)
    int32_t  lds_ns;               // bf16 matrix small enough for one workgroup's LDS (k_ns_lds_bf16)
    int32_t  pad2_;
    uint64_t apart;                // gram_ks - 1 fp32 R x R partial Grams (slices 1..)
};

// One GEMM tile of an NS phase: matrix index and tile coordinates.
struct GemmTile {
    int32_t mat, tm, tn, k;        // k = reduction length (padded), for ordering
    int32_t slice;                 // Gram with a split reduction: which slice
};

// ------------------------------------------------------------ workspace --
// Launch groups of the NS tiles.  The operand precision of a matrix is
// kGroupBf16 or kGroupFp32; fp32 matrices with at most kSmallRows padded
// rows (in a batch of only such fp32 matrices) have their tiles in
// kGroupFp32Small: kSmallTile x kSmallTile pieces of the 256 x 256 tiles for
// the Gram and square (64 times as many workgroups, so a launch over a few
// such matrices still spreads over the GPU), kSmallXTile x kSmallXTile ones
// for the X update.
enum { kGroupBf16 = 0, kGroupFp32 = 1, kGroupFp32Small = 2, kNsGroups = 3 };
constexpr int kSmallTile = 32;
constexpr int kSmallXTile = 64;
// bf16 matrices of at most kLdsRows rows and kLdsCols columns (canonical
// orientation, each rounded up to 32) run all their Newton-Schulz iterations
// in one workgroup with X, A and B in LDS, outside the tile lists.
constexpr int64_t kLdsRows = 64;
constexpr int64_t kLdsCols = 512;
constexpr int64_t kSmallRows = 256;

struct Layout {
    size_t tables_off = 0, tables_bytes = 0;
    size_t norm_tab_off = 0, adam_tab_off = 0, muon_tab_off = 0;
    std::vector<int32_t> op_group;                   // per Muon matrix: kGroupBf16 / kGroupFp32
    // Newton-Schulz batches; batch b runs on NS stream b % kNsStreams
    struct NsBatch {
        std::vector<GemmTile> tiles[3][kNsGroups];   // [phase - 1][launch group], cost-ordered
        size_t off[3][kNsGroups] = {};               // their offsets in the workspace
        bool gram_split = false;                     // fp32 Gram partials to sum after the launch
    };
    std::vector<NsBatch> ns_batches;
    std::vector<int32_t> ns_batch;                   // per Muon matrix: its batch
    size_t scalars_off = 0;                          // StepDev
    size_t norm_partials_off = 0;                    // float[n_norm_chunks]
    size_t muon_partials_off = 0;                    // float[n_orient_tiles]
    size_t muon_scale_off = 0;                       // float[n_muon]: factor applied in NS
    size_t muon_prescale_off = 0;                    // float[n_muon]: operand rescale (0: none)
    size_t ns_off = 0;                               // start of per-matrix NS buffers
    std::vector<size_t> x0, x1, lo0, lo1, xt0, xt1, a, b;  // per Muon matrix (0: unused)
    std::vector<int32_t> gram_ks;                    // per Muon matrix: Gram reduction slices
    std::vector<int32_t> lds_ns;                     // per Muon matrix: runs in k_ns_lds_bf16
    int32_t n_lds = 0;                               // how many do
    std::vector<size_t> apart;                       // per Muon matrix: partial Grams (0: none)
    size_t total = 0;
};

struct Entry {
    int32_t group = MA_GROUP_NONE;
    int32_t bucket = -1;
    int64_t m = 0, n = 0, r = 0, c = 0;
    int32_t transposed = 0;
    float   lr_shape_scale = 0.f;
    int64_t numel = 0;
    int64_t adam_offset = -1;
};

struct Bucket {
    int64_t r, c;
    std::vector<int32_t> members;
};

}  // namespace ma

struct ma_plan {
    int32_t mode = MA_MODE_MUON_ADAMW;
    double  moonlight = 0.2;
    std::vector<ma::Entry> entries;
    std::vector<ma::Bucket> buckets;
    std::vector<int32_t> muon_ids, adam_ids, train_ids;   // entry indices
    int64_t adam_numel = 0;
    int64_t n_norm_chunks = 0, n_adam_chunks = 0, n_orient_tiles = 0;
    std::vector<int64_t> norm_chunk_begin, adam_chunk_begin;     // per train / adam id
    std::vector<int64_t> muon_orient_begin;                      // per muon id
    ma::Layout layout[2];                                        // per NS precision
    std::string dump;

    int32_t overlap = 0;    // 1: AdamW on a second stream, concurrent with Muon
    int32_t param_dtype = MA_PARAM_FP32;   // storage of parameters and gradients

    // step-time staging (pinned host ring) and the per-device side streams
    // (the overlapped AdamW group, the second Newton-Schulz stream); guarded
    // by mu
    struct Side {
        int device;
        void* stream;       // AdamW beside the Muon group
        void* ev_fork;
        void* ev_join;
        void* ns_stream;    // the second Newton-Schulz stream
        void* ev_ns_fork;
        void* ev_ns_join;
    };
    mutable std::vector<Side> side;
    mutable std::mutex mu;
    mutable void* staging[ma::kStagingSlots] = {};
    mutable void* staging_dev[ma::kStagingSlots] = {};   // device address of staging[k]
    mutable size_t staging_bytes[ma::kStagingSlots] = {};
    mutable void* staging_event[ma::kStagingSlots] = {};
    mutable int staging_next = 0;
    // the descriptor tables the last eager step with a device-resident step
    // counter uploaded, and where: a captured step with the same tables and
    // workspace reads them from the workspace instead of uploading
    mutable std::vector<char> table_cache;
    // host copy of the tables for the allocation-free step, sized when the
    // plan is built (the larger of the two precisions' tables)
    mutable std::vector<char> noalloc_tables;
    mutable const void* table_cache_ws = nullptr;
    mutable int32_t table_cache_prec = -1;
};

namespace ma {

// Values of one step that depend on the step number or the gradients, in
// device memory (the workspace's scalars).  The clip finaliser -- the one
// workgroup that runs before any kernel reading them -- writes them, so
// every launch of a step takes the same arguments whatever the step number,
// and the step can be captured once and replayed.
struct StepDev {
    float   coef;          // clip factor
    float   norm;          // global gradient norm
    int32_t claim;         // AdamW chunk counter of the overlapped groups
    int32_t pad_;
    double  muon_lr;       // lr_t * muon_lr_scale (times a matrix's shape factor: its update rate)
    float   step_size;     // lr_t / (1 - beta1^t)
    float   inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
    float   adam_decay;    // 1 - lr_t * weight_decay
    float   muon_decay;    // 1 - lr_t * muon_weight_decay
};

// What the clip finaliser needs to form StepDev: the hyperparameters in
// double and the step number t, taken from t_host or, when device_step is
// set, read from and advanced in device memory.
struct StepIn {
    double  lr, muon_lr_scale, beta1, beta2, weight_decay, muon_weight_decay, min_lr_rate;
    int64_t warmup_steps, total_steps;
    int32_t schedule;      // MA_LR_*
    int32_t pad_;
    int64_t t_host;
    int64_t* device_step;
};

void set_error(const char* fmt, ...);
void clear_error();

// Build the layout of one precision (called by the plan builder).
void build_layout(ma_plan* plan, int32_t precision);

// The device address of the allocation-free step's scratch on the current
// device (looked up once per device with hipGetSymbolAddress).  hipError_t.
int noalloc_scratch(void** out);
// Copies `bytes` (a multiple of 16) from host memory to device memory
// through kernel arguments, on `stream`: the host buffer is free again when
// this returns.  hipError_t.
int launch_copy_args(void* dst, const void* src, size_t bytes, void* stream);

// --------------------------------------------------------- launchers -----
// Constants of the step that do not depend on the step number, formed in
// double on the host from the double hyperparameters and rounded once to the
// float32 the kernels use (the step-dependent ones are in StepDev).
struct StepScalars {
    float beta1, beta2, eps;
    float one_m_beta1, one_m_beta2;
    float max_grad_norm;
    float mu;
    int32_t nesterov;
    float ns_eps;
    float ns_a, ns_b, ns_c;
};

// Each returns a hipError_t as int.
// Copies `bytes` (a multiple of 16) from host memory mapped into the device
// address space (`src`) to device memory.
int launch_copy_tables(void* dst, const void* src, size_t bytes, void* stream);
// `param_dtype` (MA_PARAM_*) is the storage of parameters and gradients.
int launch_norm_partials(const NormTensor* tab, int32_t n_tab, int64_t n_chunks,
                         float* partials, int32_t param_dtype, void* stream);
// The clip factor and norm, and every other step-dependent value, into
// *sd; also zeroes sd->claim, so every step's AdamW chunk claims start at 0.
int launch_clip_finalize(const float* partials, int64_t n, float max_grad_norm,
                         const StepIn& in, StepDev* sd, float* user_norm_out, void* stream);
int launch_adamw(const AdamTensor* tab, int32_t n_tab, int64_t n_chunks,
                 const StepDev* sd, const StepScalars& s, int32_t param_dtype, void* stream);
// AdamW whose 16 Ki-element chunks are claimed one at a time by single waves
// from `counter` until all n_chunks are taken.  Several such launches, on
// different streams, may share one counter: each chunk is processed exactly
// once, and since AdamW is elementwise the result does not depend on which
// launch takes it.  Its waves are lean enough (80 VGPRs) to share a SIMD with
// a Newton-Schulz GEMM wave.
// `grid` workgroups of `waves` (1..4) waves each.
int launch_adamw_claim(const AdamTensor* tab, int32_t n_tab, int64_t n_chunks,
                       StepDev* sd, const StepScalars& s, int32_t param_dtype, int64_t grid,
                       int waves, void* stream);
// Momentum/Nesterov and the unnormalised Newton-Schulz input operands, one
// workgroup per 64 x 64 operand tile, with per-tile partials of ||u||_F^2.
// batch >= 0 restricts both passes to the matrices of that Newton-Schulz
// batch (the other workgroups return at once); -1 covers every matrix.
int launch_muon_prep(const MuonMat* tab, int32_t n_tab, int64_t n_tiles, const StepDev* sd,
                     const StepScalars& s, float* partials, int32_t batch, void* stream);
// Per matrix, the normalising factor 1 / (||u||_F + eps): into ns_scale
// (applied by the first Newton-Schulz launches), or, for a norm outside
// [2^-40, 2^40], applied to the operands in place (ns_scale = 1).
int launch_muon_scale(const MuonMat* tab, int32_t n_tab, const float* partials, float ns_eps,
                      float* ns_scale, float* pre_scale, int32_t batch, void* stream);
// After a batch's fp32 Gram launch: A += its split reductions' partial Grams.
int launch_gram_reduce(const MuonMat* tab, int32_t n_tab, int32_t batch, void* stream);
// Every Newton-Schulz iteration and the update of the matrices with lds_ns
// set, one workgroup each (the others' workgroups return at once).
int launch_ns_lds(const MuonMat* tab, int32_t n_tab, int ns_steps, const StepScalars& s,
                  const float* ns_scale, const StepDev* sd, void* stream);
// phase 1 = Gram, 2 = polynomial, 3 = X update (the parameter update when
// `last`); group = kGroupBf16 / kGroupFp32 / kGroupFp32Small selects the
// operand type and tile size.
// `ns_scale`: the per-matrix normalising factor, applied on iteration 0;
// the last iteration's update reads its rate and decay from *sd.
int launch_ns_phase(int phase, int32_t group, const MuonMat* tab, const GemmTile* tiles,
                    int64_t n_tiles, int iter, int last, const StepScalars& s,
                    const float* ns_scale, const StepDev* sd, void* stream);

}  // namespace ma
