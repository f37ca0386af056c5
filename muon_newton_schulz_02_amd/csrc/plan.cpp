// Host-only half of the library: routing, canonical shapes, buckets, the
// plan dump, chunk and tile tables and the workspace layout.  It makes no
// HIP call, so it runs (and is tested) on machines without a GPU.
//
// Routing follows the OpenDM training-stack page, Muon/AdamW hybrid section,
// table on how parameters are split, with the frozen token embedding of its
// FSDP section; the shape factor follows the sentence after the
// hyperparameter table (lr * muon_lr_scale * 0.2 * sqrt(max(shape))).

#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <new>
#include <utility>

#include "ma_internal.h"

namespace ma {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

namespace {

bool contains_ci(const std::string& lowered, const char* needle) {
    return lowered.find(needle) != std::string::npos;
}

// Group of one table entry (the routing rule of the page; see the header).
int32_t route(const char* name, int32_t ndim, bool trainable, int32_t mode) {
    if (!trainable) return MA_GROUP_NONE;
    if (mode == MA_MODE_ADAMW) return MA_GROUP_ADAMW;
    if (ndim != 2) return MA_GROUP_ADAMW;
    const std::string s(name);
    static const char kSuffix[] = ".weight";
    const size_t ls = sizeof(kSuffix) - 1;
    if (s.size() < ls || s.compare(s.size() - ls, ls, kSuffix) != 0) return MA_GROUP_ADAMW;
    // split into dotted components
    std::vector<std::string> parts;
    size_t start = 0;
    for (;;) {
        size_t dot = s.find('.', start);
        parts.push_back(s.substr(start, dot == std::string::npos ? std::string::npos : dot - start));
        if (dot == std::string::npos) break;
        start = dot + 1;
    }
    size_t ae = parts.size();
    for (size_t i = 0; i < parts.size(); ++i) {
        if (parts[i].find("action_expert") != std::string::npos) { ae = i; break; }
    }
    if (ae == parts.size()) return MA_GROUP_ADAMW;
    bool under_layers = false;
    for (size_t i = ae + 1; i < parts.size(); ++i) {
        if (parts[i] == "layers") { under_layers = true; break; }
    }
    if (!under_layers) return MA_GROUP_ADAMW;
    std::string lowered(s);
    for (auto& ch : lowered) ch = (char)std::tolower((unsigned char)ch);
    if (contains_ci(lowered, "embed") || contains_ci(lowered, "lm_head") ||
        contains_ci(lowered, "norm"))
        return MA_GROUP_ADAMW;
    return MA_GROUP_MUON;
}

std::string f32_hex(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    char buf[16];
    snprintf(buf, sizeof(buf), "%08x", u);
    return buf;
}

std::string make_dump(const ma_plan& p) {
    std::string out;
    char line[256];
    int64_t nm = 0, na = 0, nn = 0;
    for (const auto& e : p.entries) {
        if (e.group == MA_GROUP_MUON) ++nm;
        else if (e.group == MA_GROUP_ADAMW) ++na;
        else ++nn;
    }
    snprintf(line, sizeof(line),
             "muon_adamw_plan v1 mode=%d entries=%lld muon=%lld adamw=%lld none=%lld "
             "buckets=%lld adamw_numel=%lld\n",
             p.mode, (long long)p.entries.size(), (long long)nm, (long long)na, (long long)nn,
             (long long)p.buckets.size(), (long long)p.adam_numel);
    out += line;
    for (size_t b = 0; b < p.buckets.size(); ++b) {
        snprintf(line, sizeof(line), "bucket %lld r=%lld c=%lld count=%lld\n", (long long)b,
                 (long long)p.buckets[b].r, (long long)p.buckets[b].c,
                 (long long)p.buckets[b].members.size());
        out += line;
    }
    for (size_t i = 0; i < p.entries.size(); ++i) {
        const auto& e = p.entries[i];
        if (e.group == MA_GROUP_MUON) {
            snprintf(line, sizeof(line), "%lld MUON %d %lld %lld %lld %lld %d %s %lld -1\n",
                     (long long)i, e.bucket, (long long)e.m, (long long)e.n, (long long)e.r,
                     (long long)e.c, e.transposed, f32_hex(e.lr_shape_scale).c_str(),
                     (long long)e.numel);
        } else if (e.group == MA_GROUP_ADAMW) {
            snprintf(line, sizeof(line), "%lld ADAMW -1 0 0 0 0 0 00000000 %lld %lld\n",
                     (long long)i, (long long)e.numel, (long long)e.adam_offset);
        } else {
            snprintf(line, sizeof(line), "%lld NONE -1 0 0 0 0 0 00000000 %lld -1\n",
                     (long long)i, (long long)e.numel);
        }
        out += line;
    }
    return out;
}

// Order the tiles of one grouped NS launch for the chip's XCDs.  Workgroup b
// is dispatched to XCD b % kXcds, and every XCD has its own L2.  Tiles that
// share operand blocks form a unit -- a whole matrix, or, for a matrix
// heavier than a sixteenth of the launch, one row block of it.  Units are
// placed longest first onto the least-loaded XCD; each XCD's list keeps its
// units contiguous, so the tiles an XCD runs together share operands in its
// L2; the lists are interleaved so that b % kXcds selects the list.  Shorter
// lists are padded with empty tiles (mat = -1) that exit at once.
void schedule_tiles(std::vector<GemmTile>& t) {
    if (t.empty()) return;
    double total = 0.0;
    for (const auto& x : t) total += x.k;
    std::map<int32_t, std::vector<GemmTile>> by_mat;
    for (const auto& x : t) by_mat[x.mat].push_back(x);
    struct Unit {
        double cost = 0.0;
        std::vector<GemmTile> tiles;
    };
    std::vector<Unit> units;
    for (auto& kv : by_mat) {
        double c = 0.0;
        for (const auto& x : kv.second) c += x.k;
        if (c * 16.0 <= total) {
            units.push_back(Unit{c, kv.second});
        } else {
            std::map<int32_t, Unit> rows;
            for (const auto& x : kv.second) {
                rows[x.tm].cost += x.k;
                rows[x.tm].tiles.push_back(x);
            }
            for (auto& r : rows) units.push_back(std::move(r.second));
        }
    }
    std::stable_sort(units.begin(), units.end(),
                     [](const Unit& a, const Unit& b) { return a.cost > b.cost; });
    std::vector<std::vector<GemmTile>> lists(kXcds);
    double load[kXcds] = {};
    for (const auto& u : units) {
        int best = 0;
        for (int x = 1; x < kXcds; ++x)
            if (load[x] < load[best]) best = x;
        lists[best].insert(lists[best].end(), u.tiles.begin(), u.tiles.end());
        load[best] += u.cost;
    }
    size_t longest = 0;
    for (const auto& l : lists) longest = std::max(longest, l.size());
    t.clear();
    for (size_t j = 0; j < longest; ++j)
        for (int x = 0; x < kXcds; ++x)
            t.push_back(j < lists[x].size() ? lists[x][j] : GemmTile{-1, 0, 0, 0, 0});
}

void build_tables(ma_plan* p) {
    // clip norm: every trainable tensor
    int64_t ch = 0;
    for (int32_t id : p->train_ids) {
        p->norm_chunk_begin.push_back(ch);
        ch += ceil_div(p->entries[id].numel, kChunk);
    }
    p->n_norm_chunks = ch;
    ch = 0;
    for (int32_t id : p->adam_ids) {
        p->adam_chunk_begin.push_back(ch);
        ch += ceil_div(p->entries[id].numel, kChunk);
    }
    p->n_adam_chunks = ch;
    int64_t ot = 0;
    for (size_t k = 0; k < p->muon_ids.size(); ++k) {
        const auto& e = p->entries[p->muon_ids[k]];
        p->muon_orient_begin.push_back(ot);
        const int64_t R = round_up(e.r, kNsPad), C = round_up(e.c, kNsPad);
        ot += (R / kOrientTile) * (C / kOrientTile);
    }
    p->n_orient_tiles = ot;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

void build_layout(ma_plan* p, int32_t precision) {
    Layout& L = p->layout[precision];
    L = Layout();
    // operand group and GEMM tiles of every matrix: Gram and polynomial
    // phases cover the upper triangle of the r x r result (mirrored on
    // write), the X update the whole r x c result in column-major order
    // NS batch of every matrix: longest processing time first on the padded
    // GEMM work (Gram and square over the upper tiles, the X update over all)
    const size_t nm = p->muon_ids.size();
    std::vector<double> cost(nm);
    size_t operand_bytes = 0;
    L.lds_ns.assign(nm, 0);
    for (size_t k = 0; k < nm; ++k) {
        const auto& e = p->entries[p->muon_ids[k]];
        const int32_t grp =
            (precision == MA_NS_BF16 && e.r >= kBf16MinRows) ? kGroupBf16 : kGroupFp32;
        L.op_group.push_back(grp);
        const int64_t R = round_up(e.r, kNsPad), C = round_up(e.c, kNsPad);
        if (grp == kGroupBf16 && e.r <= kLdsRows && round_up(e.c, 32) <= kLdsCols) {
            // one workgroup through every iteration: no tiles, no batch work
            L.lds_ns[k] = 1;
            ++L.n_lds;
            cost[k] = 0.0;
            continue;
        }
        cost[k] = (double)R * R * C + (double)R * R * R / 2.0 + (double)R * R * C;
        operand_bytes += (size_t)(R * C) * (grp == kGroupBf16 ? 4 : 8);
    }
    // With AdamW streaming beside it, bf16 Newton-Schulz in smaller batches
    // (whose operands can stay in the 256 MB memory-side cache through the
    // iterations) contends less for HBM: measured 16.1 -> 15.6 ms per step on
    // the full hybrid table.  Alone, or with fp32 products (bound by the
    // matrix cores, 46 -> 52 ms when batched), fewer and fuller launches win.
    const bool batched = precision == MA_NS_BF16 && p->overlap && !p->adam_ids.empty() &&
                         p->n_adam_chunks < (int64_t(1) << 30);
    const size_t per = batched ? kNsOverlapBatchBytes : std::max<size_t>(operand_bytes, 1);
    size_t nb = kNsStreams * ((operand_bytes + kNsStreams * per - 1) / (kNsStreams * per));
    nb = std::max<size_t>(1, std::min(nb, nm));
    // Matrices that all take the small fp32 tiles run as one batch: their
    // launches are bound by latency rather than by the matrix cores, and one
    // stream of fuller launches beat two interleaved ones (tiny fp32 table:
    // Newton-Schulz 0.278 -> 0.249 ms per step).
    bool all_small = nm > 0;
    for (size_t k = 0; k < nm; ++k)
        if (!L.lds_ns[k] && (L.op_group[k] != kGroupFp32 ||
                             round_up(p->entries[p->muon_ids[k]].r, kNsPad) > kSmallRows))
            all_small = false;
    if (all_small) nb = 1;
    std::vector<size_t> order(nm);
    for (size_t k = 0; k < nm; ++k) order[k] = k;
    std::stable_sort(order.begin(), order.end(),
                     [&](size_t a, size_t b) { return cost[a] > cost[b]; });
    L.ns_batch.assign(nm, 0);
    std::vector<double> bload(nb, 0.0);
    for (size_t k : order) {
        if (L.lds_ns[k]) continue;  // batch 0: its operands are prepared with that batch's
        size_t best = 0;
        for (size_t q = 1; q < nb; ++q)
            if (bload[q] < bload[best]) best = q;
        L.ns_batch[k] = (int32_t)best;
        bload[best] += cost[k];
    }
    L.ns_batches.assign(nm ? nb : 0, Layout::NsBatch());
    // A batch whose fp32 Gram launch has fewer tiles than the GPU has CUs
    // (small matrices, where one long-reduction tile per matrix would leave
    // most CUs idle) splits each of those Gram reductions into up to
    // kGramMaxSlices slices of whole 256-column blocks: slice 0 writes A, the
    // others fp32 partials that a reduction kernel adds to A in slice order.
    // bf16 operands keep whole reductions (their A is rounded once, from
    // the fp32 sum).
    // The fp32 matrices of at most kSmallRows padded rows take the small
    // tiles in a batch whose fp32 matrices are all that small; beside larger
    // ones their 256 x 256 tiles fill the larger matrices' launches instead
    // of adding launches of their own.
    std::vector<char> small(nm, 0);
    {
        std::vector<char> big_f32(nb, 0);
        for (size_t k = 0; k < nm; ++k)
            if (L.op_group[k] == kGroupFp32 &&
                round_up(p->entries[p->muon_ids[k]].r, kNsPad) > kSmallRows)
                big_f32[L.ns_batch[k]] = 1;
        for (size_t k = 0; k < nm; ++k)
            small[k] = L.op_group[k] == kGroupFp32 && !big_f32[L.ns_batch[k]];
    }
    L.gram_ks.assign(nm, 1);
    {
        std::vector<int64_t> f32_gram(nb, 0);
        for (size_t k = 0; k < nm; ++k) {
            if (L.op_group[k] != kGroupFp32 || small[k]) continue;
            const auto& e = p->entries[p->muon_ids[k]];
            const int64_t TR = round_up(e.r, kNsPad) / kGemmTile;
            f32_gram[L.ns_batch[k]] += TR * (TR + 1) / 2;
        }
        for (size_t k = 0; k < nm; ++k) {
            if (L.op_group[k] != kGroupFp32 || small[k] || f32_gram[L.ns_batch[k]] >= kCus)
                continue;
            const auto& e = p->entries[p->muon_ids[k]];
            const int64_t blocks = round_up(e.c, kNsPad) / kGemmTile;
            int32_t ks = 1;
            for (int32_t d = 2; d <= kGramMaxSlices; ++d)
                if (blocks % d == 0) ks = d;
            L.gram_ks[k] = ks;
            if (ks > 1) L.ns_batches[L.ns_batch[k]].gram_split = true;
        }
    }
    for (size_t k = 0; k < nm; ++k) {
        if (L.lds_ns[k]) continue;
        const auto& e = p->entries[p->muon_ids[k]];
        auto& t = L.ns_batches[L.ns_batch[k]].tiles;
        const int64_t R = round_up(e.r, kNsPad), C = round_up(e.c, kNsPad);
        const int32_t grp = small[k] ? (int32_t)kGroupFp32Small : L.op_group[k];
        const int64_t tsz = small[k] ? kSmallTile : kGemmTile;
        const int32_t TR = (int32_t)(R / tsz);
        const int64_t xsz = small[k] ? kSmallXTile : kGemmTile;  // X-update tiles
        const int32_t XR = (int32_t)(R / xsz), XC = (int32_t)(C / xsz);
        const int32_t ks = L.gram_ks[k];
        for (int32_t sl = 0; sl < ks; ++sl)
            for (int32_t i = 0; i < TR; ++i)
                for (int32_t j = i; j < TR; ++j)
                    t[0][grp].push_back(GemmTile{(int32_t)k, i, j, (int32_t)(C / ks), sl});
        for (int32_t i = 0; i < TR; ++i)
            for (int32_t j = i; j < TR; ++j)
                t[1][grp].push_back(GemmTile{(int32_t)k, i, j, (int32_t)R, 0});
        // column-major: the tiles of one column block (all readers of that
        // X panel) are consecutive, so the tiles an XCD runs together read
        // each panel once from HBM while the r x r B stays in its L2
        for (int32_t j = 0; j < XC; ++j)
            for (int32_t i = 0; i < XR; ++i)
                t[2][grp].push_back(GemmTile{(int32_t)k, i, j, (int32_t)R, 0});
    }
    for (auto& bt : L.ns_batches)
        for (auto& ph : bt.tiles)
            for (auto& tl : ph) schedule_tiles(tl);
    size_t off = 0;
    L.tables_off = off;
    L.norm_tab_off = off;
    off = align256(off + sizeof(NormTensor) * p->train_ids.size());
    L.adam_tab_off = off;
    off = align256(off + sizeof(AdamTensor) * p->adam_ids.size());
    L.muon_tab_off = off;
    off = align256(off + sizeof(MuonMat) * p->muon_ids.size());
    for (auto& bt : L.ns_batches)
        for (int ph = 0; ph < 3; ++ph)
            for (int g = 0; g < kNsGroups; ++g) {
                bt.off[ph][g] = off;
                off = align256(off + sizeof(GemmTile) * bt.tiles[ph][g].size());
            }
    L.tables_bytes = off - L.tables_off;
    L.scalars_off = off;
    off = align256(off + sizeof(StepDev));
    L.norm_partials_off = off;
    off = align256(off + sizeof(float) * (size_t)std::max<int64_t>(p->n_norm_chunks, 1));
    L.muon_partials_off = off;
    off = align256(off + sizeof(float) * (size_t)std::max<int64_t>(p->n_orient_tiles, 1));
    L.muon_scale_off = off;
    off = align256(off + sizeof(float) * std::max<size_t>(p->muon_ids.size(), 1));
    L.muon_prescale_off = off;
    off = align256(off + sizeof(float) * std::max<size_t>(p->muon_ids.size(), 1));
    L.ns_off = off;
    for (size_t k = 0; k < p->muon_ids.size(); ++k) {
        const auto& e = p->entries[p->muon_ids[k]];
        const size_t R = (size_t)round_up(e.r, kNsPad), C = (size_t)round_up(e.c, kNsPad);
        const size_t esz = L.op_group[k] == kGroupBf16 ? 2 : 4;
        auto take = [&](size_t bytes) {
            const size_t at = off;
            off = align256(off + bytes);
            return at;
        };
        if (L.lds_ns[k]) {
            // only the step-0 operands, which the prep pass writes; the
            // iterations run in LDS
            L.x0.push_back(take(R * C * 2));
            L.x1.push_back(0);
            L.lo0.push_back(take(R * C * 2));
            L.lo1.push_back(0);
            L.xt0.push_back(0);
            L.xt1.push_back(0);
            L.a.push_back(0);
            L.b.push_back(0);
            L.apart.push_back(0);
            continue;
        }
        if (L.op_group[k] == kGroupBf16) {
            // X as bf16 hi / lo pairs, ping-pong; B X reads hi transposed on load
            L.x0.push_back(take(R * C * 2));
            L.x1.push_back(take(R * C * 2));
            L.lo0.push_back(take(R * C * 2));
            L.lo1.push_back(take(R * C * 2));
            L.xt0.push_back(0);
            L.xt1.push_back(0);
        } else {
            // fp32 master X (updated in place) and X^T ping-pong
            L.x0.push_back(take(R * C * 4));
            L.x1.push_back(0);
            L.lo0.push_back(0);
            L.lo1.push_back(0);
            L.xt0.push_back(take(R * C * 4));
            L.xt1.push_back(take(R * C * 4));
        }
        L.a.push_back(off);
        off = align256(off + R * R * esz);
        L.b.push_back(off);
        off = align256(off + R * R * esz);
        L.apart.push_back(L.gram_ks[k] > 1 ? take(R * R * 4 * (size_t)(L.gram_ks[k] - 1)) : 0);
    }
    L.total = std::max<size_t>(off, 256);
}

}  // namespace ma

using namespace ma;

extern "C" {

int muon_adamw_default_hparams(ma_hparams* hp) {
    if (!hp) {
        set_error("muon_adamw_default_hparams: hp is NULL");
        return MA_ERR_INVALID_ARG;
    }
    hp->lr = 2.5e-5;
    hp->muon_lr_scale = 1.0;
    hp->muon_momentum = 0.95;
    hp->muon_nesterov = 1;
    hp->muon_ns_steps = 5;
    hp->ns_coeffs[0] = 3.2608;
    hp->ns_coeffs[1] = -3.6447;
    hp->ns_coeffs[2] = 1.3650;
    hp->ns_precision = MA_NS_BF16;
    hp->ns_eps = 1e-7;
    hp->beta1 = 0.9;
    hp->beta2 = 0.999;
    hp->eps = 1e-8;
    hp->weight_decay = 0.01;
    hp->muon_weight_decay = 0.0;
    hp->max_grad_norm = 1.0;
    hp->lr_schedule = MA_LR_CONSTANT;
    hp->warmup_steps = 0;
    hp->total_steps = 0;
    hp->min_lr_rate = 0.1;
    clear_error();
    return MA_OK;
}

int muon_adamw_plan(const ma_param_desc* table, int32_t n, const ma_plan_opts* opts,
                    ma_plan** out) {
    if (!out) {
        set_error("muon_adamw_plan: out is NULL");
        return MA_ERR_INVALID_ARG;
    }
    *out = nullptr;
    if (!table || n < 1) {
        set_error("muon_adamw_plan: empty or NULL table (n=%d)", n);
        return MA_ERR_INVALID_ARG;
    }
    int32_t mode = opts ? opts->mode : MA_MODE_MUON_ADAMW;
    double moon = opts ? opts->moonlight_coefficient : 0.2;
    int32_t overlap = opts ? opts->overlap_groups : 0;
    int32_t param_dtype = opts ? opts->param_dtype : MA_PARAM_FP32;
    if (param_dtype != MA_PARAM_FP32 && param_dtype != MA_PARAM_BF16) {
        set_error("muon_adamw_plan: unknown param_dtype %d", param_dtype);
        return MA_ERR_INVALID_ARG;
    }
    if (overlap != 0 && overlap != 1) {
        set_error("muon_adamw_plan: overlap_groups must be 0 or 1");
        return MA_ERR_INVALID_ARG;
    }
    if (mode != MA_MODE_MUON_ADAMW && mode != MA_MODE_ADAMW) {
        set_error("muon_adamw_plan: unknown mode %d", mode);
        return MA_ERR_INVALID_ARG;
    }
    if (!(std::isfinite(moon) && moon > 0.0)) {
        set_error("muon_adamw_plan: moonlight coefficient must be finite and > 0");
        return MA_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < n; ++i) {
        const ma_param_desc& d = table[i];
        if (!d.name) {
            set_error("muon_adamw_plan: entry %d has no name", i);
            return MA_ERR_INVALID_ARG;
        }
        if (d.ndim < 0 || d.ndim > MA_MAX_NDIM) {
            set_error("muon_adamw_plan: entry %d (%s) has ndim %d (0..%d supported)", i, d.name,
                      d.ndim, MA_MAX_NDIM);
            return MA_ERR_UNSUPPORTED;
        }
        if (d.ndim > 0 && !d.shape) {
            set_error("muon_adamw_plan: entry %d (%s) has no shape", i, d.name);
            return MA_ERR_INVALID_ARG;
        }
        int64_t numel = 1;
        for (int32_t k = 0; k < d.ndim; ++k) {
            const int64_t s = d.shape[k];
            if (s < 1) {
                set_error("muon_adamw_plan: entry %d (%s) has size %lld in dim %d", i, d.name,
                          (long long)s, k);
                return MA_ERR_SHAPE;
            }
            if (numel > (int64_t(1) << 62) / s) {
                set_error("muon_adamw_plan: entry %d (%s) is too large", i, d.name);
                return MA_ERR_SHAPE;
            }
            numel *= s;
        }
        if (d.ndim == 2 && route(d.name, d.ndim, d.trainable != 0, mode) == MA_GROUP_MUON) {
            // The Newton-Schulz operands are addressed with 32-bit buffer
            // offsets inside resources of at most 2^31 - 1 bytes: every padded
            // operand, up to fp32 R x C, must fit.
            const int64_t R = round_up(std::min(d.shape[0], d.shape[1]), kNsPad);
            const int64_t C = round_up(std::max(d.shape[0], d.shape[1]), kNsPad);
            if (d.shape[0] > (int64_t(1) << 30) || d.shape[1] > (int64_t(1) << 30) ||
                R * C > ((int64_t(1) << 31) - 1) / 4) {
                set_error("muon_adamw_plan: entry %d (%s): Muon matrix %lld x %lld too large "
                          "(its padded fp32 operand must stay below 2 GiB)",
                          i, d.name, (long long)d.shape[0], (long long)d.shape[1]);
                return MA_ERR_SHAPE;
            }
        }
    }
    ma_plan* p = new (std::nothrow) ma_plan();
    if (!p) {
        set_error("muon_adamw_plan: out of host memory");
        return MA_ERR_INVALID_ARG;
    }
    p->mode = mode;
    p->moonlight = moon;
    p->overlap = overlap;
    p->param_dtype = param_dtype;
    p->entries.resize(n);
    std::map<std::pair<int64_t, int64_t>, int32_t> bucket_of;
    for (int32_t i = 0; i < n; ++i) {
        const ma_param_desc& d = table[i];
        Entry& e = p->entries[i];
        e.numel = 1;
        for (int32_t k = 0; k < d.ndim; ++k) e.numel *= d.shape[k];
        e.group = route(d.name, d.ndim, d.trainable != 0, mode);
        if (e.group == MA_GROUP_MUON) {
            e.m = d.shape[0];
            e.n = d.shape[1];
            e.r = std::min(e.m, e.n);
            e.c = std::max(e.m, e.n);
            e.transposed = e.m > e.n ? 1 : 0;
            e.lr_shape_scale = (float)(moon * std::sqrt((double)std::max(e.m, e.n)));
            auto key = std::make_pair(e.r, e.c);
            auto it = bucket_of.find(key);
            if (it == bucket_of.end()) {
                it = bucket_of.emplace(key, (int32_t)p->buckets.size()).first;
                p->buckets.push_back(Bucket{e.r, e.c, {}});
            }
            e.bucket = it->second;
            p->buckets[e.bucket].members.push_back(i);
            p->muon_ids.push_back(i);
            p->train_ids.push_back(i);
        } else if (e.group == MA_GROUP_ADAMW) {
            e.adam_offset = p->adam_numel;
            p->adam_numel += e.numel;
            p->adam_ids.push_back(i);
            p->train_ids.push_back(i);
        }
    }
    if (p->muon_ids.size() > (size_t)INT32_MAX / 2) {
        delete p;
        set_error("muon_adamw_plan: too many matrices");
        return MA_ERR_UNSUPPORTED;
    }
    build_tables(p);
    build_layout(p, MA_NS_BF16);
    build_layout(p, MA_NS_FP32);
    p->noalloc_tables.assign(
        std::max(p->layout[MA_NS_BF16].tables_bytes, p->layout[MA_NS_FP32].tables_bytes), 0);
    p->dump = make_dump(*p);
    *out = p;
    clear_error();
    return MA_OK;
}

int muon_adamw_plan_size(const ma_plan* plan, int32_t* n_entries) {
    if (!plan || !n_entries) {
        set_error("muon_adamw_plan_size: NULL argument");
        return MA_ERR_INVALID_ARG;
    }
    *n_entries = (int32_t)plan->entries.size();
    clear_error();
    return MA_OK;
}

int muon_adamw_plan_entry(const ma_plan* plan, int32_t i, ma_plan_entry* e) {
    if (!plan || !e) {
        set_error("muon_adamw_plan_entry: NULL argument");
        return MA_ERR_INVALID_ARG;
    }
    if (i < 0 || i >= (int32_t)plan->entries.size()) {
        set_error("muon_adamw_plan_entry: index %d out of range", i);
        return MA_ERR_INVALID_ARG;
    }
    const Entry& s = plan->entries[i];
    e->group = s.group;
    e->bucket = s.bucket;
    e->m = s.m;
    e->n = s.n;
    e->r = s.r;
    e->c = s.c;
    e->transposed = s.transposed;
    e->lr_shape_scale = s.lr_shape_scale;
    e->numel = s.numel;
    e->adam_offset = s.adam_offset;
    clear_error();
    return MA_OK;
}

int muon_adamw_plan_dump(const ma_plan* plan, char* buf, size_t cap, size_t* len) {
    if (!plan || !len) {
        set_error("muon_adamw_plan_dump: NULL argument");
        return MA_ERR_INVALID_ARG;
    }
    *len = plan->dump.size();
    if (!buf || cap < plan->dump.size() + 1) {
        if (buf == nullptr && cap == 0) {
            clear_error();
            return MA_OK;
        }
        set_error("muon_adamw_plan_dump: buffer of %zu bytes, need %zu", cap, plan->dump.size() + 1);
        return MA_ERR_WORKSPACE;
    }
    std::memcpy(buf, plan->dump.data(), plan->dump.size());
    buf[plan->dump.size()] = '\0';
    clear_error();
    return MA_OK;
}

int muon_adamw_workspace_size(const ma_plan* plan, int32_t ns_precision, size_t* bytes) {
    if (!plan || !bytes) {
        set_error("muon_adamw_workspace_size: NULL argument");
        return MA_ERR_INVALID_ARG;
    }
    if (ns_precision != MA_NS_BF16 && ns_precision != MA_NS_FP32) {
        set_error("muon_adamw_workspace_size: unknown precision %d", ns_precision);
        return MA_ERR_INVALID_ARG;
    }
    *bytes = plan->layout[ns_precision].total;
    clear_error();
    return MA_OK;
}

const char* muon_adamw_last_error(void) { return ma::g_last_error.c_str(); }

const char* muon_adamw_version(void) { return "muon_adamw 0.1.0 (gfx950)"; }

}  // extern "C"
