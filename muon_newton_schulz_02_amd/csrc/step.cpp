// muon_adamw_step: argument validation, descriptor tables and the launch
// sequence of one hybrid step on the caller's stream.
//
// Order of work (OpenDM training-stack page: clip from the defaults table,
// then the two optimizer groups of the Muon/AdamW hybrid section):
//   1. this step's descriptor tables copied into the workspace by a small
//      kernel reading mapped pinned host memory (skipped with a device step
//      counter while they are unchanged)
//   2. clip norm partials over every trainable gradient, then the clip factor
//      and the step's rates
//   3. AdamW over the AdamW group (or, with overlap_groups, forked onto a
//      side stream after step 4 and finished after step 5)
//   4. Muon momentum + unnormalised operands + ||u||^2 partials, then the
//      per-matrix normalising factor
//   5. per Newton-Schulz batch, ns_steps x (GRAM, POLY, XUPD), the first GRAM
//      and XUPD applying the normalising factor and the last XUPD writing the
//      update; batches alternate between the caller's stream and a side
//      stream
// Side streams are joined back into the caller's stream before returning.
// Nothing is launched before every argument has been checked.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "ma_internal.h"

using namespace ma;

namespace {

bool is_finite(double x) { return std::isfinite(x); }

int hip_fail(const char* what, int err) {
    set_error("%s: %s", what, hipGetErrorString((hipError_t)err));
    return MA_ERR_HIP;
}

// A pinned host staging buffer of at least `bytes`, whose previous copy (if
// any) has completed.  kStagingSlots buffers rotate, so the host waits here
// only when it is that many steps of this plan ahead of the device.
int get_staging(const ma_plan* plan, size_t bytes, void** out, const void** out_dev,
                void** event) {
    const int k = plan->staging_next;
    plan->staging_next = (k + 1) % kStagingSlots;
    if (plan->staging_event[k]) {
        hipError_t e = hipEventSynchronize((hipEvent_t)plan->staging_event[k]);
        if (e != hipSuccess) return hip_fail("staging event wait", e);
    } else {
        hipEvent_t ev;
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail("hipEventCreate", e);
        plan->staging_event[k] = ev;
    }
    if (plan->staging_bytes[k] < bytes) {
        if (plan->staging[k]) (void)hipHostFree(plan->staging[k]);
        plan->staging[k] = nullptr;
        plan->staging_dev[k] = nullptr;
        plan->staging_bytes[k] = 0;
        // mapped and coherent: the copy kernel reads it straight over the bus
        void* p = nullptr;
        hipError_t e = hipHostMalloc(&p, bytes,
                                     hipHostMallocPortable | hipHostMallocMapped |
                                         hipHostMallocCoherent);
        if (e != hipSuccess) return hip_fail("hipHostMalloc (staging)", e);
        void* dp = nullptr;
        e = hipHostGetDevicePointer(&dp, p, 0);
        if (e != hipSuccess) {
            (void)hipHostFree(p);
            return hip_fail("hipHostGetDevicePointer (staging)", e);
        }
        plan->staging[k] = p;
        plan->staging_dev[k] = dp;
        plan->staging_bytes[k] = bytes;
    }
    *out = plan->staging[k];
    *out_dev = plan->staging_dev[k];
    *event = plan->staging_event[k];
    return MA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7) == 0; }

// Workgroups of the AdamW launch that runs beside the Muon group (one per CU
// of the MI355X), and of the launch that finishes the remaining chunks.
constexpr int64_t kSideAdamGroups = 256;
constexpr int64_t kFinishAdamGroups = 2048;
// Waves per side workgroup, by parameter storage.  Measured on the full
// hybrid table: the side waves take HBM from the GEMMs, and the best share
// depends on the bytes AdamW moves.  fp32 (28 B per element): 1..4 waves per
// CU gave 18.7 / 17.6 / 16.9 / 16.5 ms per step; bf16 (22 B): 15.3 / 13.6 /
// 14.1 / 15.0 ms -- with four, AdamW is done when the GEMMs are a third done.
constexpr int kSideAdamWaves[2] = {4, 2};
// Where the side AdamW launch forks off: right after the clip factor (false)
// or after the Muon momentum pass, beside the Newton-Schulz GEMMs only
// (true).  Forked early, its streaming waves starve the momentum pass -- the
// pass's many short workgroups get a small share of HBM and it ends when
// AdamW does -- and the GEMMs then run alone: with bf16 parameters the
// overlapped step was slower than the serial one.  Forked late it costs the
// momentum pass nothing and overlaps the whole GEMM phase.
constexpr bool kForkAfterPrep = true;

// The side streams and their fork/join events on the current device (created
// on first use; default priority, non-blocking with respect to the null
// stream): one for the overlapped AdamW group, one for the second
// Newton-Schulz matrix group.
int get_side(const ma_plan* plan, ma_plan::Side** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    for (auto& s : plan->side) {
        if (s.device == dev) {
            *out = &s;
            return MA_OK;
        }
    }
    ma_plan::Side s{dev, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    // on failure the objects made so far are released before returning
    auto undo = [&](const char* what, hipError_t er) {
        for (void* ev : {s.ev_fork, s.ev_join, s.ev_ns_fork, s.ev_ns_join})
            if (ev) (void)hipEventDestroy((hipEvent_t)ev);
        for (void* q : {s.stream, s.ns_stream})
            if (q) (void)hipStreamDestroy((hipStream_t)q);
        return hip_fail(what, er);
    };
    for (void** q : {&s.stream, &s.ns_stream}) {
        hipStream_t st;
        e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        if (e != hipSuccess) return undo("hipStreamCreate (side)", e);
        *q = st;
    }
    for (void** ev : {&s.ev_fork, &s.ev_join, &s.ev_ns_fork, &s.ev_ns_join}) {
        hipEvent_t a;
        e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
        if (e != hipSuccess) return undo("hipEventCreate (fork/join)", e);
        *ev = a;
    }
    plan->side.push_back(s);
    *out = &plan->side.back();
    return MA_OK;
}

}  // namespace

namespace {

// One step.  no_alloc: the allocation-free variant -- every launch on the
// caller's stream (no library streams or events are created), the
// descriptor tables uploaded through kernel arguments (no pinned staging),
// and `workspace` the device scratch.
int step_impl(const ma_plan* plan, float* const* params, const float* const* grads,
              ma_state* state, const ma_hparams* hp, void* workspace, size_t ws_bytes,
              void* stream, float* grad_norm_out, float* const* muon_update_out,
              void* const* phase_events, bool no_alloc) {
    // ---------------------------------------------------------- validate --
    if (!plan || !state || !hp) {
        set_error("muon_adamw_step: plan, state and hp are required");
        return MA_ERR_INVALID_ARG;
    }
    const int32_t prec = hp->ns_precision;
    if (prec != MA_NS_BF16 && prec != MA_NS_FP32) {
        set_error("muon_adamw_step: unknown ns_precision %d", prec);
        return MA_ERR_UNSUPPORTED;
    }
    if (hp->muon_ns_steps < 1 || hp->muon_ns_steps > 64) {
        set_error("muon_adamw_step: muon_ns_steps %d outside [1, 64]", hp->muon_ns_steps);
        return MA_ERR_UNSUPPORTED;
    }
    const double fields[] = {hp->lr, hp->muon_lr_scale, hp->muon_momentum, hp->ns_coeffs[0],
                             hp->ns_coeffs[1], hp->ns_coeffs[2], hp->ns_eps, hp->beta1,
                             hp->beta2, hp->eps, hp->weight_decay, hp->muon_weight_decay,
                             hp->max_grad_norm};
    for (double f : fields) {
        if (!is_finite(f)) {
            set_error("muon_adamw_step: non-finite hyperparameter");
            return MA_ERR_INVALID_ARG;
        }
    }
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0 && hp->beta2 >= 0.0 && hp->beta2 < 1.0)) {
        set_error("muon_adamw_step: betas must lie in [0, 1)");
        return MA_ERR_INVALID_ARG;
    }
    if (hp->eps < 0.0 || hp->ns_eps < 0.0 || hp->lr < 0.0) {
        set_error("muon_adamw_step: lr, eps and ns_eps must be >= 0");
        return MA_ERR_INVALID_ARG;
    }
    if (hp->lr_schedule != MA_LR_CONSTANT && hp->lr_schedule != MA_LR_COSINE_MIN) {
        set_error("muon_adamw_step: unknown lr_schedule %d", hp->lr_schedule);
        return MA_ERR_INVALID_ARG;
    }
    if (hp->lr_schedule == MA_LR_COSINE_MIN &&
        !(hp->total_steps >= 1 && hp->warmup_steps >= 0 && hp->warmup_steps <= hp->total_steps &&
          hp->min_lr_rate >= 0.0 && hp->min_lr_rate <= 1.0)) {
        set_error("muon_adamw_step: cosine_with_min_lr needs total_steps >= 1, "
                  "0 <= warmup_steps <= total_steps and min_lr_rate in [0, 1]");
        return MA_ERR_INVALID_ARG;
    }
    if (!state->device_step && (state->step < 0 || state->step > (int64_t(1) << 40))) {
        set_error("muon_adamw_step: state->step %lld out of range", (long long)state->step);
        return MA_ERR_INVALID_ARG;
    }
    const bool any_train = !plan->train_ids.empty();
    if (any_train && (!params || !grads)) {
        set_error("muon_adamw_step: params and grads arrays are required");
        return MA_ERR_INVALID_ARG;
    }
    for (int32_t id : plan->train_ids) {
        if (!params[id] || !grads[id]) {
            set_error("muon_adamw_step: entry %d needs a param and a grad pointer", id);
            return MA_ERR_INVALID_ARG;
        }
    }
    if (!plan->muon_ids.empty() && !state->muon_momentum) {
        set_error("muon_adamw_step: state->muon_momentum is required");
        return MA_ERR_INVALID_ARG;
    }
    for (int32_t id : plan->muon_ids) {
        if (!state->muon_momentum[id]) {
            set_error("muon_adamw_step: entry %d needs a momentum buffer", id);
            return MA_ERR_INVALID_ARG;
        }
    }
    if (!plan->adam_ids.empty() && (!state->adam_m || !state->adam_v)) {
        set_error("muon_adamw_step: state->adam_m and adam_v are required");
        return MA_ERR_INVALID_ARG;
    }
    for (int32_t id : plan->adam_ids) {
        if (!state->adam_m[id] || !state->adam_v[id]) {
            set_error("muon_adamw_step: entry %d needs AdamW moment buffers", id);
            return MA_ERR_INVALID_ARG;
        }
    }
    const Layout& L = plan->layout[prec];
    if (!workspace || ws_bytes < L.total) {
        set_error("muon_adamw_step: workspace of %zu bytes, need %zu", ws_bytes, L.total);
        return MA_ERR_WORKSPACE;
    }
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) {
        set_error("muon_adamw_step: workspace must be 256-byte aligned");
        return MA_ERR_WORKSPACE;
    }
    // Every buffer the step writes or reads must be disjoint from every other
    // (a parameter passed again as its gradient, a state shared by two
    // entries, a workspace over a tensor): such aliasing would give wrong
    // results with no error, so it is refused here, from the pointers alone.
    {
        struct Span {
            uintptr_t lo, hi;
            int32_t id;
            const char* what;
        };
        std::vector<Span> spans;
        const size_t esz = plan->param_dtype == MA_PARAM_BF16 ? 2 : 4;
        auto add = [&](const void* ptr, size_t bytes, int32_t id, const char* what) {
            if (!ptr) return;
            const uintptr_t a = reinterpret_cast<uintptr_t>(ptr);
            spans.push_back(Span{a, a + bytes, id, what});
        };
        for (int32_t id : plan->train_ids) {
            const size_t n = (size_t)plan->entries[id].numel;
            add(params[id], n * esz, id, "parameter");
            add(grads[id], n * esz, id, "gradient");
        }
        for (int32_t id : plan->muon_ids) {
            const size_t n = (size_t)plan->entries[id].numel;
            add(state->muon_momentum[id], n * 4, id, "momentum");
            if (muon_update_out) add(muon_update_out[id], n * 4, id, "update output");
        }
        for (int32_t id : plan->adam_ids) {
            const size_t n = (size_t)plan->entries[id].numel;
            add(state->adam_m[id], n * 4, id, "adam_m");
            add(state->adam_v[id], n * 4, id, "adam_v");
        }
        add(workspace, L.total, -1, "workspace");
        add(grad_norm_out, 4, -1, "grad_norm_out");
        add(state->device_step, 8, -1, "device_step");
        std::sort(spans.begin(), spans.end(),
                  [](const Span& x, const Span& y) { return x.lo < y.lo; });
        for (size_t i = 1; i < spans.size(); ++i) {
            if (spans[i].lo < spans[i - 1].hi) {
                set_error("muon_adamw_step: %s of entry %d overlaps %s of entry %d",
                          spans[i].what, spans[i].id, spans[i - 1].what, spans[i - 1].id);
                return MA_ERR_INVALID_ARG;
            }
        }
    }

    // -------------------------------------------------------- scalars ----
    // step-dependent values are formed on the device by the clip finaliser
    StepIn in{};
    in.lr = hp->lr;
    in.muon_lr_scale = hp->muon_lr_scale;
    in.beta1 = hp->beta1;
    in.beta2 = hp->beta2;
    in.weight_decay = hp->weight_decay;
    in.muon_weight_decay = hp->muon_weight_decay;
    in.min_lr_rate = hp->min_lr_rate;
    in.warmup_steps = hp->warmup_steps;
    in.total_steps = hp->total_steps;
    in.schedule = hp->lr_schedule;
    in.t_host = state->step + 1;
    in.device_step = state->device_step;
    StepScalars sc;
    sc.beta1 = (float)hp->beta1;
    sc.beta2 = (float)hp->beta2;
    sc.one_m_beta1 = (float)(1.0 - hp->beta1);
    sc.one_m_beta2 = (float)(1.0 - hp->beta2);
    sc.eps = (float)hp->eps;
    sc.max_grad_norm = (float)hp->max_grad_norm;
    sc.mu = (float)hp->muon_momentum;
    sc.nesterov = hp->muon_nesterov ? 1 : 0;
    sc.ns_eps = (float)hp->ns_eps;
    sc.ns_a = (float)hp->ns_coeffs[0];
    sc.ns_b = (float)hp->ns_coeffs[1];
    sc.ns_c = (float)hp->ns_coeffs[2];

    hipStream_t st = (hipStream_t)stream;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cap);
    if (e != hipSuccess) return hip_fail("hipStreamIsCapturing", e);
    const bool capturing = cap != hipStreamCaptureStatusNone;
    if (capturing && !state->device_step) {
        set_error("muon_adamw_step: a captured step needs state->device_step");
        return MA_ERR_CAPTURE;
    }
    if (no_alloc && capturing) {
        set_error("muon_adamw_step_noalloc: the step cannot be captured (every call on a GPU "
                  "shares its scratch, so a replay could find another plan's data there); "
                  "capture muon_adamw_step with a caller-owned workspace instead");
        return MA_ERR_CAPTURE;
    }

    std::lock_guard<std::mutex> lock(plan->mu);
    // ------------------------------------------------- descriptor tables --
    char* base = reinterpret_cast<char*>(workspace);
    const bool bf16 = plan->param_dtype == MA_PARAM_BF16;
    auto fill_tables = [&](char* hb) {
        std::memset(hb, 0, L.tables_bytes);
        auto* norm_tab = reinterpret_cast<NormTensor*>(hb + L.norm_tab_off);
        for (size_t k = 0; k < plan->train_ids.size(); ++k) {
            const int32_t id = plan->train_ids[k];
            NormTensor& d = norm_tab[k];
            d.g = reinterpret_cast<uint64_t>(grads[id]);
            d.numel = plan->entries[id].numel;
            d.chunk_begin = plan->norm_chunk_begin[k];
            d.vec_ok = aligned16(grads[id]) ? 1 : 0;   // 16-byte loads, either storage
        }
        auto* adam_tab = reinterpret_cast<AdamTensor*>(hb + L.adam_tab_off);
        for (size_t k = 0; k < plan->adam_ids.size(); ++k) {
            const int32_t id = plan->adam_ids[k];
            AdamTensor& d = adam_tab[k];
            d.p = reinterpret_cast<uint64_t>(params[id]);
            d.g = reinterpret_cast<uint64_t>(grads[id]);
            d.m = reinterpret_cast<uint64_t>(state->adam_m[id]);
            d.v = reinterpret_cast<uint64_t>(state->adam_v[id]);
            d.numel = plan->entries[id].numel;
            d.chunk_begin = plan->adam_chunk_begin[k];
            // four-element accesses: 16 bytes of float, 8 of bf16
            const bool pg = bf16 ? aligned8(params[id]) && aligned8(grads[id])
                                 : aligned16(params[id]) && aligned16(grads[id]);
            d.vec_ok = (pg && aligned16(state->adam_m[id]) && aligned16(state->adam_v[id])) ? 1 : 0;
        }
        auto* muon_tab = reinterpret_cast<MuonMat*>(hb + L.muon_tab_off);
        for (size_t k = 0; k < plan->muon_ids.size(); ++k) {
            const int32_t id = plan->muon_ids[k];
            const Entry& e = plan->entries[id];
            MuonMat& d = muon_tab[k];
            float* delta = muon_update_out ? muon_update_out[id] : nullptr;
            d.p = reinterpret_cast<uint64_t>(params[id]);
            d.g = reinterpret_cast<uint64_t>(grads[id]);
            d.buf = reinterpret_cast<uint64_t>(state->muon_momentum[id]);
            d.delta = reinterpret_cast<uint64_t>(delta);
            auto ws = [&](size_t off) { return off ? reinterpret_cast<uint64_t>(base + off) : 0; };
            d.x[0] = ws(L.x0[k]);
            d.x[1] = ws(L.x1[k]);
            d.xlo[0] = ws(L.lo0[k]);
            d.xlo[1] = ws(L.lo1[k]);
            d.xt[0] = ws(L.xt0[k]);
            d.xt[1] = ws(L.xt1[k]);
            d.a = reinterpret_cast<uint64_t>(base + L.a[k]);
            d.b = reinterpret_cast<uint64_t>(base + L.b[k]);
            d.numel = e.numel;
            d.orient_begin = plan->muon_orient_begin[k];
            d.m = (int32_t)e.m;
            d.n = (int32_t)e.n;
            d.r = (int32_t)e.r;
            d.c = (int32_t)e.c;
            d.R = (int32_t)round_up(e.r, kNsPad);
            d.C = (int32_t)round_up(e.c, kNsPad);
            d.transposed = e.transposed;
            // 16-byte row runs of p (16 elements), buf and delta; four-element
            // loads of g
            d.vec_ok = (aligned16(params[id]) && (bf16 ? aligned8(grads[id]) : aligned16(grads[id])) &&
                        aligned16(state->muon_momentum[id]) && (!delta || aligned16(delta)) &&
                        (e.n % (bf16 ? 8 : 4)) == 0)
                           ? 1
                           : 0;
            d.shape_scale = e.lr_shape_scale;
            d.ns_batch = L.ns_batch[k];
            d.gram_ks = L.gram_ks[k];
            d.lds_ns = L.lds_ns[k];
            d.pad2_ = 0;
            d.apart = L.apart[k] ? reinterpret_cast<uint64_t>(base + L.apart[k]) : 0;
            d.op_bf16 = L.op_group[k] == kGroupBf16 ? 1 : 0;
            d.p_bf16 = bf16 ? 1 : 0;
        }
        for (const auto& bt : L.ns_batches)
            for (int ph = 0; ph < 3; ++ph)
                for (int g = 0; g < kNsGroups; ++g)
                    std::memcpy(hb + bt.off[ph][g], bt.tiles[ph][g].data(),
                                sizeof(GemmTile) * bt.tiles[ph][g].size());
    };

    auto mark = [&](int k) -> int {
        if (!phase_events || !phase_events[k]) return 0;
        return (int)hipEventRecord((hipEvent_t)phase_events[k], st);
    };
    if (int er = mark(0)) return hip_fail("phase event", er);
    // The tables go up through a pinned staging slot on every eager step.  A
    // captured step cannot upload (the staging slot would be reused by later
    // eager steps while the graph still points at it): it relies on the
    // tables the last eager step with a device step counter put in this
    // workspace, and is refused unless those are the tables it needs.
    if (no_alloc) {
        // the plan's host copy of the tables, sized at plan time; each chunk
        // travels in a copy kernel's arguments, which the runtime copies at
        // enqueue time, so the buffer may be refilled by the next call
        plan->table_cache_ws = nullptr;
        char* hb = plan->noalloc_tables.data();
        fill_tables(hb);
        int er = launch_copy_args(base + L.tables_off, hb, L.tables_bytes, stream);
        if (er) return hip_fail("table upload", er);
    } else if (capturing) {
        std::vector<char> fresh(L.tables_bytes);
        fill_tables(fresh.data());
        const bool cached = plan->table_cache_ws == workspace && plan->table_cache_prec == prec &&
                            plan->table_cache == fresh;
        if (!cached) {
            set_error("muon_adamw_step: captured step would upload new descriptor tables; "
                      "run one eager step with the same pointers and workspace first");
            return MA_ERR_CAPTURE;
        }
    } else {
        void* host = nullptr;
        const void* host_dev = nullptr;
        void* event = nullptr;
        int rc = get_staging(plan, L.tables_bytes, &host, &host_dev, &event);
        if (rc != MA_OK) return rc;
        // a failure past this point may leave the workspace's tables stale
        plan->table_cache_ws = nullptr;
        if (state->device_step) {
            // remembered for a later capture with the same pointers
            plan->table_cache.resize(L.tables_bytes);
            fill_tables(plan->table_cache.data());
            std::memcpy(host, plan->table_cache.data(), L.tables_bytes);
        } else {
            fill_tables(reinterpret_cast<char*>(host));
        }
        // a kernel on the step's stream reads the staging buffer over the bus:
        // no copy engine, so no cross-engine waits between consecutive steps
        // (a copy-engine upload stalled the second of back-to-back steps by
        // about 5 ms)
        int er = launch_copy_tables(base + L.tables_off, host_dev, L.tables_bytes, stream);
        if (er) return hip_fail("table upload", er);
        e = hipEventRecord((hipEvent_t)event, st);
        if (e != hipSuccess) return hip_fail("hipEventRecord", e);
        if (state->device_step) {
            plan->table_cache_ws = workspace;
            plan->table_cache_prec = prec;
        }
    }

    // ------------------------------------------------------------ launch --
    const auto* d_norm = reinterpret_cast<const NormTensor*>(base + L.norm_tab_off);
    const auto* d_adam = reinterpret_cast<const AdamTensor*>(base + L.adam_tab_off);
    const auto* d_muon = reinterpret_cast<const MuonMat*>(base + L.muon_tab_off);
    auto* sd = reinterpret_cast<StepDev*>(base + L.scalars_off);
    float* norm_partials = reinterpret_cast<float*>(base + L.norm_partials_off);
    float* muon_partials = reinterpret_cast<float*>(base + L.muon_partials_off);
    float* muon_scales = reinterpret_cast<float*>(base + L.muon_scale_off);
    float* muon_prescales = reinterpret_cast<float*>(base + L.muon_prescale_off);
    const int32_t n_train = (int32_t)plan->train_ids.size();
    const int32_t n_adam = (int32_t)plan->adam_ids.size();
    const int32_t n_muon = (int32_t)plan->muon_ids.size();

    int err = launch_norm_partials(d_norm, n_train, plan->n_norm_chunks, norm_partials,
                                   plan->param_dtype, stream);
    if (err) return hip_fail("clip norm partials", err);
    err = launch_clip_finalize(norm_partials, plan->n_norm_chunks, sc.max_grad_norm, in, sd,
                               grad_norm_out, stream);
    if (err) return hip_fail("clip finalize", err);
    if ((err = mark(1))) return hip_fail("phase event", err);
    // AdamW: on the caller's stream, or forked to the side stream so it runs
    // concurrently with the Muon group and joined back at the end
    ma_plan::Side* side = nullptr;
    bool ns_joined = false;
    // Whatever a forked side stream has queued is joined back into the
    // caller's stream on every return, errors included (an unjoined fork
    // would also invalidate an enclosing graph capture).
    struct JoinGuard {
        hipStream_t main = nullptr;
        ma_plan::Side** side = nullptr;
        bool adam = false, ns = false;
        ~JoinGuard() {
            if (!*side) return;
            if (adam && hipEventRecord((hipEvent_t)(*side)->ev_join,
                                       (hipStream_t)(*side)->stream) == hipSuccess)
                (void)hipStreamWaitEvent(main, (hipEvent_t)(*side)->ev_join, 0);
            if (ns && hipEventRecord((hipEvent_t)(*side)->ev_ns_join,
                                     (hipStream_t)(*side)->ns_stream) == hipSuccess)
                (void)hipStreamWaitEvent(main, (hipEvent_t)(*side)->ev_ns_join, 0);
        }
    } guard;
    guard.main = st;
    guard.side = &side;
    // (the chunk counter is an int: beyond 2^30 chunks run serially)
    const bool overlap = !no_alloc && plan->overlap && n_adam > 0 && n_muon > 0 &&
                         plan->n_adam_chunks < (int64_t(1) << 30);
    auto fork_adamw = [&]() -> int {
        int rs = get_side(plan, &side);
        if (rs != MA_OK) return rs;
        hipStream_t ss = (hipStream_t)side->stream;
        if ((e = hipEventRecord((hipEvent_t)side->ev_fork, st)) != hipSuccess)
            return hip_fail("hipEventRecord (fork)", e);
        if ((e = hipStreamWaitEvent(ss, (hipEvent_t)side->ev_fork, 0)) != hipSuccess)
            return hip_fail("hipStreamWaitEvent (fork)", e);
        guard.adam = true;
        // one workgroup per CU: each of its waves shares a SIMD with a
        // Newton-Schulz GEMM wave (whose LDS and registers leave room for
        // exactly that) and streams AdamW chunks while the GEMMs run
        int er = launch_adamw_claim(d_adam, n_adam, plan->n_adam_chunks, sd, sc, plan->param_dtype,
                                    kSideAdamGroups, kSideAdamWaves[bf16 ? 1 : 0], ss);
        if (er) return hip_fail("adamw", er);
        if (phase_events && phase_events[2] &&
            (e = hipEventRecord((hipEvent_t)phase_events[2], ss)) != hipSuccess)
            return hip_fail("phase event", e);
        if ((e = hipEventRecord((hipEvent_t)side->ev_join, ss)) != hipSuccess)
            return hip_fail("hipEventRecord (join)", e);
        return MA_OK;
    };
    if (!overlap) {
        err = launch_adamw(d_adam, n_adam, plan->n_adam_chunks, sd, sc, plan->param_dtype, stream);
        if (err) return hip_fail("adamw", err);
        if ((err = mark(2))) return hip_fail("phase event", err);
    } else if (!kForkAfterPrep) {
        if ((err = fork_adamw()) != MA_OK) return err;
    }
    if (n_muon > 0) {
        static_assert(kNsStreams == 2, "one caller stream and one side stream");
        const int nb = (int)L.ns_batches.size();
        // without library streams the batches run one after another on the
        // caller's stream (each matrix's phases stay in order either way)
        const bool split = nb > 1 && !no_alloc;
        // With two batches and nothing beside them, the second batch's
        // momentum/normalise pass (HBM-bound) runs on the side stream while
        // the first batch's Gram launches (matrix-core bound) start.  A
        // profiled step keeps the passes whole, so each phase interval holds
        // its own kernels only.
        const bool pipelined = split && nb == kNsStreams && !overlap && !phase_events;
        auto prep = [&](int32_t batch, hipStream_t q) -> int {
            int er = launch_muon_prep(d_muon, n_muon, plan->n_orient_tiles, sd, sc, muon_partials,
                                      batch, q);
            if (er) return hip_fail("muon prep", er);
            er = launch_muon_scale(d_muon, n_muon, muon_partials, sc.ns_eps, muon_scales,
                                   muon_prescales, batch, q);
            if (er) return hip_fail("muon scale", er);
            return MA_OK;
        };
        if ((err = prep(pipelined ? 0 : -1, st)) != MA_OK) return err;
        if (overlap && kForkAfterPrep && (err = fork_adamw()) != MA_OK) return err;
        if ((err = mark(3))) return hip_fail("phase event", err);
        // The matrices run in batches of about equal GEMM work, each through
        // all of its iterations, consecutive batches alternating between the
        // caller's stream and a side stream: one batch's launch tail (the last
        // tiles of a phase, when most CUs already idle) overlaps the other
        // stream's next launch.
        hipStream_t nss = nullptr;
        if (split) {
            if (!side) {
                int rs = get_side(plan, &side);
                if (rs != MA_OK) return rs;
            }
            nss = (hipStream_t)side->ns_stream;
            if ((e = hipEventRecord((hipEvent_t)side->ev_ns_fork, st)) != hipSuccess)
                return hip_fail("hipEventRecord (ns fork)", e);
            if ((e = hipStreamWaitEvent(nss, (hipEvent_t)side->ev_ns_fork, 0)) != hipSuccess)
                return hip_fail("hipStreamWaitEvent (ns fork)", e);
            guard.ns = true;
            if (pipelined && (err = prep(1, nss)) != MA_OK) return err;
        }
        // the matrices small enough for one workgroup each (all in batch 0,
        // whose operands the pass above prepared): one launch for all their
        // iterations, on the caller's stream ahead of its tiled launches
        // (after the fork above, so the other stream does not wait for it).
        // On a stream of its own it ran five times longer beside the tiled
        // launches and slowed the second batch's momentum pass: 16.9 ->
        // 17.8 ms per step on the stress table.
        if (L.n_lds > 0 &&
            (err = launch_ns_lds(d_muon, n_muon, hp->muon_ns_steps, sc, muon_scales, sd, st)))
            return hip_fail("newton-schulz (lds)", err);
        for (int b0 = 0; b0 < nb; b0 += kNsStreams) {
            for (int it = 0; it < hp->muon_ns_steps; ++it) {
                const int last = it == hp->muon_ns_steps - 1;
                for (int ph = 0; ph < 3; ++ph) {
                    for (int q = 0; q < kNsStreams && b0 + q < nb; ++q) {
                        const auto& bt = L.ns_batches[b0 + q];
                        void* qs = (q == 0 || !split) ? stream : (void*)nss;
                        for (int g = 0; g < kNsGroups; ++g) {
                            err = launch_ns_phase(
                                ph + 1, g, d_muon,
                                reinterpret_cast<const GemmTile*>(base + bt.off[ph][g]),
                                (int64_t)bt.tiles[ph][g].size(), it, last, sc, muon_scales, sd,
                                qs);
                            if (err) return hip_fail("newton-schulz", err);
                        }
                        // the Grams of split reductions, before the square reads them
                        if (ph == 0 && bt.gram_split &&
                            (err = launch_gram_reduce(d_muon, n_muon, b0 + q, qs)))
                            return hip_fail("gram reduce", err);
                    }
                }
            }
        }
        if (split) {
            if ((e = hipEventRecord((hipEvent_t)side->ev_ns_join, nss)) != hipSuccess)
                return hip_fail("hipEventRecord (ns join)", e);
            ns_joined = true;
        }
    } else if ((err = mark(3))) {
        return hip_fail("phase event", err);
    }
    if (guard.adam) {
        // the chunks the side kernel has not claimed yet, at full occupancy
        // (no more waves than chunks)
        const int64_t groups =
            std::min<int64_t>(kFinishAdamGroups, (plan->n_adam_chunks + 3) / 4);
        err = launch_adamw_claim(d_adam, n_adam, plan->n_adam_chunks, sd, sc, plan->param_dtype,
                                 groups, 4, stream);
        if (err) return hip_fail("adamw", err);
    }
    if (guard.adam) {
        if ((e = hipStreamWaitEvent(st, (hipEvent_t)side->ev_join, 0)) != hipSuccess)
            return hip_fail("hipStreamWaitEvent (join)", e);
        guard.adam = false;
    }
    if (ns_joined) {
        if ((e = hipStreamWaitEvent(st, (hipEvent_t)side->ev_ns_join, 0)) != hipSuccess)
            return hip_fail("hipStreamWaitEvent (ns join)", e);
        guard.ns = false;
    }
    if ((err = mark(4))) return hip_fail("phase event", err);
    if (!state->device_step) state->step = in.t_host;
    clear_error();
    return MA_OK;
}

}  // namespace

extern "C" {

int muon_adamw_step(const ma_plan* plan, float* const* params, const float* const* grads,
                    ma_state* state, const ma_hparams* hp, void* workspace, size_t ws_bytes,
                    void* stream, float* grad_norm_out, float* const* muon_update_out) {
    return step_impl(plan, params, grads, state, hp, workspace, ws_bytes, stream, grad_norm_out,
                     muon_update_out, nullptr, false);
}

int muon_adamw_step_profiled(const ma_plan* plan, float* const* params, const float* const* grads,
                             ma_state* state, const ma_hparams* hp, void* workspace,
                             size_t ws_bytes, void* stream, float* grad_norm_out,
                             float* const* muon_update_out, void* const* phase_events) {
    return step_impl(plan, params, grads, state, hp, workspace, ws_bytes, stream, grad_norm_out,
                     muon_update_out, phase_events, false);
}

int muon_adamw_step_noalloc(const ma_plan* plan, float* const* params, const float* const* grads,
                            ma_state* state, const ma_hparams* hp, void* stream,
                            float* grad_norm_out, float* const* muon_update_out) {
    if (!plan || !hp) {
        set_error("muon_adamw_step_noalloc: plan and hp are required");
        return MA_ERR_INVALID_ARG;
    }
    if (hp->ns_precision != MA_NS_BF16 && hp->ns_precision != MA_NS_FP32) {
        set_error("muon_adamw_step_noalloc: unknown ns_precision %d", hp->ns_precision);
        return MA_ERR_UNSUPPORTED;
    }
    const size_t need = plan->layout[hp->ns_precision].total;
    if (need > kNoAllocScratchBytes) {
        set_error("muon_adamw_step_noalloc: this plan needs %zu bytes of workspace, above the "
                  "%zu-byte device scratch of the allocation-free step; use muon_adamw_step "
                  "with a caller-allocated workspace",
                  need, (size_t)kNoAllocScratchBytes);
        return MA_ERR_WORKSPACE;
    }
    void* scratch = nullptr;
    int e = noalloc_scratch(&scratch);
    if (e) return hip_fail("hipGetSymbolAddress (scratch)", e);
    return step_impl(plan, params, grads, state, hp, scratch, kNoAllocScratchBytes, stream,
                     grad_norm_out, muon_update_out, nullptr, true);
}

void muon_adamw_plan_free(ma_plan* plan) {
    if (!plan) return;
    for (auto& sd : plan->side) {
        (void)hipStreamSynchronize((hipStream_t)sd.stream);
        (void)hipStreamSynchronize((hipStream_t)sd.ns_stream);
        for (void* ev : {sd.ev_fork, sd.ev_join, sd.ev_ns_fork, sd.ev_ns_join})
            (void)hipEventDestroy((hipEvent_t)ev);
        (void)hipStreamDestroy((hipStream_t)sd.stream);
        (void)hipStreamDestroy((hipStream_t)sd.ns_stream);
    }
    for (int k = 0; k < kStagingSlots; ++k) {
        if (plan->staging_event[k]) {
            (void)hipEventSynchronize((hipEvent_t)plan->staging_event[k]);
            (void)hipEventDestroy((hipEvent_t)plan->staging_event[k]);
        }
        if (plan->staging[k]) (void)hipHostFree(plan->staging[k]);
    }
    delete plan;
}

}  // extern "C"
