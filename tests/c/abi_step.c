/* Drives the MuonAdamW C ABI from plain C with the HIP runtime only (no
 * Python, no torch): reads a table and its float32 inputs from a directory,
 * allocates every device buffer itself, runs `steps` optimizer steps on a
 * stream it creates, and writes the results back for the test to compare
 * with the CPU oracle.
 *
 *   abi_step DIR
 *
 * DIR/table.txt:  "n steps ns_precision overlap" on the first line, then one
 *                 line per entry: "name trainable ndim d0 d1 ...".
 * DIR/param_<i>.bin, DIR/grad_<s>_<i>.bin (s = 1..steps): float32 inputs of
 *                 trainable entry i.
 * Writes DIR/out_param_<i>.bin, out_m_<i>.bin / out_v_<i>.bin (AdamW),
 * out_buf_<i>.bin / out_delta_<i>.bin (Muon, the last step's update),
 * out_norm.txt (the last step's global norm) and out_status.txt.
 * Exit status 0 on success; any library or HIP error is printed and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "muon_adamw.h"

#define MAXN 64

#define HIP_CHECK(x)                                                                \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x,               \
                    hipGetErrorString(e_));                                         \
            exit(1);                                                                \
        }                                                                           \
    } while (0)

#define MA_CHECK(x)                                                                 \
    do {                                                                            \
        int r_ = (x);                                                               \
        if (r_ != MA_OK) {                                                          \
            fprintf(stderr, "%s: %d (%s)\n", #x, r_, muon_adamw_last_error());      \
            exit(1);                                                                \
        }                                                                           \
    } while (0)

static void path(char* out, const char* dir, const char* name) {
    snprintf(out, 1024, "%s/%s", dir, name);
}

static float* read_f32(const char* dir, const char* name, size_t n) {
    char p[1024];
    path(p, dir, name);
    FILE* f = fopen(p, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", p); exit(1); }
    float* h = (float*)malloc(n * sizeof(float));
    if (fread(h, sizeof(float), n, f) != n) { fprintf(stderr, "short read %s\n", p); exit(1); }
    fclose(f);
    return h;
}

static void write_dev(const char* dir, const char* name, const float* d, size_t n) {
    char p[1024];
    path(p, dir, name);
    float* h = (float*)malloc(n * sizeof(float));
    HIP_CHECK(hipMemcpy(h, d, n * sizeof(float), hipMemcpyDeviceToHost));
    FILE* f = fopen(p, "wb");
    if (!f || fwrite(h, sizeof(float), n, f) != n) { fprintf(stderr, "cannot write %s\n", p); exit(1); }
    fclose(f);
    free(h);
}

static float* to_dev(const float* h, size_t n) {
    float* d = NULL;
    HIP_CHECK(hipMalloc((void**)&d, n * sizeof(float)));
    HIP_CHECK(hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice));
    return d;
}

static float* zeros_dev(size_t n) {
    float* d = NULL;
    HIP_CHECK(hipMalloc((void**)&d, n * sizeof(float)));
    HIP_CHECK(hipMemset(d, 0, n * sizeof(float)));
    return d;
}

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: abi_step DIR\n"); return 2; }
    const char* dir = argv[1];
    char p[1024];
    path(p, dir, "table.txt");
    FILE* tf = fopen(p, "r");
    if (!tf) { fprintf(stderr, "cannot open %s\n", p); return 1; }
    int n = 0, steps = 0, prec = 0, overlap = 0;
    if (fscanf(tf, "%d %d %d %d", &n, &steps, &prec, &overlap) != 4 || n < 1 || n > MAXN) {
        fprintf(stderr, "bad table header\n");
        return 1;
    }
    static char names[MAXN][256];
    static int64_t shapes[MAXN][MA_MAX_NDIM];
    ma_param_desc desc[MAXN];
    size_t numel[MAXN];
    for (int i = 0; i < n; ++i) {
        int tr = 0, nd = 0;
        if (fscanf(tf, "%255s %d %d", names[i], &tr, &nd) != 3 || nd < 0 || nd > MA_MAX_NDIM) {
            fprintf(stderr, "bad table line %d\n", i);
            return 1;
        }
        numel[i] = 1;
        for (int k = 0; k < nd; ++k) {
            long long v = 0;
            if (fscanf(tf, "%lld", &v) != 1) { fprintf(stderr, "bad shape %d\n", i); return 1; }
            shapes[i][k] = v;
            numel[i] *= (size_t)v;
        }
        desc[i].name = names[i];
        desc[i].ndim = nd;
        desc[i].shape = shapes[i];
        desc[i].trainable = tr;
    }
    fclose(tf);

    ma_plan_opts opts;
    memset(&opts, 0, sizeof(opts));
    opts.mode = MA_MODE_MUON_ADAMW;
    opts.moonlight_coefficient = 0.2;
    opts.overlap_groups = overlap;
    opts.param_dtype = MA_PARAM_FP32;
    ma_plan* plan = NULL;
    MA_CHECK(muon_adamw_plan(desc, n, &opts, &plan));

    float* params[MAXN] = {0};
    float* grads[MAXN] = {0};
    float* mom[MAXN] = {0};
    float* am[MAXN] = {0};
    float* av[MAXN] = {0};
    float* delta[MAXN] = {0};
    int group[MAXN];
    for (int i = 0; i < n; ++i) {
        ma_plan_entry e;
        MA_CHECK(muon_adamw_plan_entry(plan, i, &e));
        group[i] = e.group;
        if (e.group == MA_GROUP_NONE) continue;
        char nm[64];
        snprintf(nm, sizeof nm, "param_%d.bin", i);
        float* h = read_f32(dir, nm, numel[i]);
        params[i] = to_dev(h, numel[i]);
        free(h);
        HIP_CHECK(hipMalloc((void**)&grads[i], numel[i] * sizeof(float)));
        if (e.group == MA_GROUP_MUON) {
            mom[i] = zeros_dev(numel[i]);
            delta[i] = zeros_dev(numel[i]);
        } else {
            am[i] = zeros_dev(numel[i]);
            av[i] = zeros_dev(numel[i]);
        }
    }

    ma_hparams hp;
    MA_CHECK(muon_adamw_default_hparams(&hp));
    hp.ns_precision = prec;
    size_t ws_bytes = 0;
    MA_CHECK(muon_adamw_workspace_size(plan, prec, &ws_bytes));
    void* ws = NULL;
    HIP_CHECK(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 256));
    float* norm = zeros_dev(1);
    hipStream_t stream;
    HIP_CHECK(hipStreamCreateWithFlags(&stream, hipStreamNonBlocking));

    ma_state st;
    memset(&st, 0, sizeof(st));
    st.muon_momentum = mom;
    st.adam_m = am;
    st.adam_v = av;
    st.step = 0;
    st.device_step = NULL;
    for (int s = 1; s <= steps; ++s) {
        for (int i = 0; i < n; ++i) {
            if (group[i] == MA_GROUP_NONE) continue;
            char nm[64];
            snprintf(nm, sizeof nm, "grad_%d_%d.bin", s, i);
            float* h = read_f32(dir, nm, numel[i]);
            HIP_CHECK(hipMemcpy(grads[i], h, numel[i] * sizeof(float), hipMemcpyHostToDevice));
            free(h);
        }
        MA_CHECK(muon_adamw_step(plan, params, (const float* const*)grads, &st, &hp, ws, ws_bytes,
                                 stream, norm, delta));
        HIP_CHECK(hipStreamSynchronize(stream));
    }
    if (st.step != steps) { fprintf(stderr, "step counter %lld\n", (long long)st.step); return 1; }

    for (int i = 0; i < n; ++i) {
        char nm[64];
        if (group[i] == MA_GROUP_NONE) continue;
        snprintf(nm, sizeof nm, "out_param_%d.bin", i);
        write_dev(dir, nm, params[i], numel[i]);
        if (group[i] == MA_GROUP_MUON) {
            snprintf(nm, sizeof nm, "out_buf_%d.bin", i);
            write_dev(dir, nm, mom[i], numel[i]);
            snprintf(nm, sizeof nm, "out_delta_%d.bin", i);
            write_dev(dir, nm, delta[i], numel[i]);
        } else {
            snprintf(nm, sizeof nm, "out_m_%d.bin", i);
            write_dev(dir, nm, am[i], numel[i]);
            snprintf(nm, sizeof nm, "out_v_%d.bin", i);
            write_dev(dir, nm, av[i], numel[i]);
        }
    }
    float hn = 0.f;
    HIP_CHECK(hipMemcpy(&hn, norm, sizeof(float), hipMemcpyDeviceToHost));
    path(p, dir, "out_norm.txt");
    FILE* nf = fopen(p, "w");
    if (!nf) return 1;
    fprintf(nf, "%.9g\n", (double)hn);
    fclose(nf);

    for (int i = 0; i < n; ++i) {
        if (params[i]) HIP_CHECK(hipFree(params[i]));
        if (grads[i]) HIP_CHECK(hipFree(grads[i]));
        if (mom[i]) HIP_CHECK(hipFree(mom[i]));
        if (delta[i]) HIP_CHECK(hipFree(delta[i]));
        if (am[i]) HIP_CHECK(hipFree(am[i]));
        if (av[i]) HIP_CHECK(hipFree(av[i]));
    }
    HIP_CHECK(hipFree(ws));
    HIP_CHECK(hipFree(norm));
    HIP_CHECK(hipStreamDestroy(stream));
    muon_adamw_plan_free(plan);
    path(p, dir, "out_status.txt");
    FILE* sf = fopen(p, "w");
    if (!sf) return 1;
    fprintf(sf, "ok %s\n", muon_adamw_version());
    fclose(sf);
    return 0;
}
