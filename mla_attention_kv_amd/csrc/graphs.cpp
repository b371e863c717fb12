// Captured decode buckets: the prolog recorded once per token-count bucket
// as a HIP graph over fixed buffers, then replayed with one graph launch per
// step.  This is the MI355X counterpart of the migration guide's aclgraph
// use: graph mode on top of the fused kernel to cut scheduling overhead
// (section "Background"), with the kernel warmed up at q_len 1 and 2 on the
// first layer's weights before serving (section "Command-line parameters",
// notes 2-3; "Migration notes", item 3).
//
// A set holds one instantiated graph per bucket.  Each graph is the exact
// launch sequence the plain entry point issues for that many tokens, once
// per layer of the set in layer order (a set of L layers, each with its own
// weights and buffers, replays all L prologs with one launch, as a
// whole-model graph does), so a replay computes bit for bit what direct
// calls over the same buffers compute.  The set holds no tensors of its
// own: every buffer is the caller's (the graphs themselves are runtime
// objects).
#include <algorithm>
#include <new>
#include <vector>

#include "../../include/libmlaprolog.h"
#include "mla_common.h"

struct mla_prolog_graphs {
    int device = 0;
    std::vector<mla_prolog_graph_desc_t> layers;
    std::vector<int64_t> buckets;
    std::vector<hipGraphExec_t> execs;
};

namespace {

constexpr int kMaxBuckets = 64;
constexpr int kMaxLayers = 256;

// The plain entry point the graphs record: the cached variants, which with
// num_slots == 0 are the plain prolog.
mla_status_t call_prolog(const mla_prolog_graph_desc_t& d, int64_t T, hipStream_t s) {
    if (d.w8a8 == 0)
        return mla_kv_prolog_cached(d.hidden, d.W_kv_a, d.gamma, d.W_kv_b, d.positions, T, d.d,
                                    d.dt, d.eps, d.theta, d.k_nope, d.value, d.k_pe,
                                    d.compressed_kv, d.slot_mapping, d.kv_cache, d.num_slots,
                                    d.workspace, d.workspace_bytes, s);
    return mla_kv_prolog_w8a8_cached(
        d.hidden, (const int8_t*)d.W_kv_a, d.s_kv_a, d.gamma, (const int8_t*)d.W_kv_b, d.s_kv_b,
        d.positions, T, d.d, d.eps, d.theta, d.k_nope, d.value, d.k_pe, d.compressed_kv,
        d.slot_mapping, d.kv_cache, d.kv_cache_q, d.kv_scale, d.num_slots, d.workspace,
        d.workspace_bytes, s);
}

bool buckets_ok(const int64_t* b, int32_t n) {
    if (b == nullptr || n < 1 || n > kMaxBuckets) return false;
    for (int32_t i = 0; i < n; ++i) {
        if (b[i] < 1 || b[i] > MLA_MAX_TOKENS) return false;
        if (i > 0 && b[i] <= b[i - 1]) return false;
    }
    return true;
}

// Layers of one set record the same kind of call: same w8a8, dims and (fp
// path) dtype.
bool same_kind(const mla_prolog_graph_desc_t& a, const mla_prolog_graph_desc_t& o) {
    return a.w8a8 == o.w8a8 && a.d.H == o.d.H && a.d.r == o.d.r && a.d.dr == o.d.dr &&
           a.d.nh == o.d.nh && a.d.dn == o.d.dn && a.d.dv == o.d.dv &&
           (a.w8a8 != 0 || a.dt == o.dt);
}

// Every argument check of the recorded calls, for every layer and bucket,
// without touching the GPU.
mla_status_t validate(const mla_prolog_graph_desc_t* d, int32_t nl, const int64_t* b, int32_t n) {
    if (d == nullptr || nl < 1 || nl > kMaxLayers) return MLA_ERR_INVALID_ARG;
    for (int32_t l = 0; l < nl; ++l) {
        if (d[l].w8a8 != 0 && d[l].w8a8 != 1) return MLA_ERR_INVALID_ARG;
        if (!same_kind(d[l], d[0])) return MLA_ERR_INVALID_ARG;
    }
    mla::ValidateOnlyScope scope;
    for (int32_t l = 0; l < nl; ++l)
        for (int32_t i = 0; i < n; ++i) {
            const mla_status_t st = call_prolog(d[l], b[i], nullptr);
            if (st != MLA_OK) return st;
        }
    return MLA_OK;
}

mla_status_t capture(const std::vector<mla_prolog_graph_desc_t>& layers, int64_t T,
                     hipStream_t s, hipGraph_t* out) {
    *out = nullptr;
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return MLA_ERR_HIP;
    mla_status_t st = MLA_OK;
    for (size_t l = 0; l < layers.size() && st == MLA_OK; ++l) st = call_prolog(layers[l], T, s);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &g);
    if (st != MLA_OK || e != hipSuccess || g == nullptr) {
        if (g != nullptr) (void)hipGraphDestroy(g);
        (void)hipGetLastError();
        return st != MLA_OK ? st : MLA_ERR_HIP;
    }
    *out = g;
    return MLA_OK;
}

void release(mla_prolog_graphs* g) {
    for (hipGraphExec_t x : g->execs)
        if (x != nullptr) (void)hipGraphExecDestroy(x);
    delete g;
}

// Runs f with the set's device current, restoring the caller's afterwards.
template <class F>
mla_status_t on_device(int device, F&& f) {
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_HIP;
    if (prev != device && hipSetDevice(device) != hipSuccess) return MLA_ERR_HIP;
    const mla_status_t st = f();
    if (prev != device) (void)hipSetDevice(prev);
    return st;
}

}  // namespace

extern "C" {

mla_status_t mla_prolog_graphs_create_layers(const mla_prolog_graph_desc_t* descs,
                                             int32_t n_layers, const int64_t* buckets,
                                             int32_t n_buckets, mla_prolog_graphs** out) {
    if (out == nullptr) return MLA_ERR_INVALID_ARG;
    *out = nullptr;
    if (descs == nullptr || n_layers < 1 || n_layers > kMaxLayers ||
        !buckets_ok(buckets, n_buckets))
        return MLA_ERR_INVALID_ARG;
    mla_status_t st = validate(descs, n_layers, buckets, n_buckets);
    if (st != MLA_OK) return st;

    mla_prolog_graphs* g = new (std::nothrow) mla_prolog_graphs;
    if (g == nullptr) return MLA_ERR_HIP;
    g->layers.assign(descs, descs + n_layers);
    g->buckets.assign(buckets, buckets + n_buckets);
    g->execs.assign(n_buckets, nullptr);
    if (hipGetDevice(&g->device) != hipSuccess) {
        release(g);
        return MLA_ERR_HIP;
    }
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
        release(g);
        return MLA_ERR_HIP;
    }
    for (int32_t i = 0; i < n_buckets && st == MLA_OK; ++i) {
        hipGraph_t graph = nullptr;
        st = capture(g->layers, g->buckets[i], s, &graph);
        if (st != MLA_OK) break;
        if (hipGraphInstantiate(&g->execs[i], graph, nullptr, nullptr, 0) != hipSuccess) {
            g->execs[i] = nullptr;
            st = MLA_ERR_HIP;
        }
        (void)hipGraphDestroy(graph);
    }
    (void)hipStreamDestroy(s);
    if (st != MLA_OK) {
        release(g);
        return st;
    }
    *out = g;
    return MLA_OK;
}

mla_status_t mla_prolog_graphs_create(const mla_prolog_graph_desc_t* desc,
                                      const int64_t* buckets, int32_t n_buckets,
                                      mla_prolog_graphs** out) {
    return mla_prolog_graphs_create_layers(desc, 1, buckets, n_buckets, out);
}

mla_status_t mla_prolog_graphs_update_layers(mla_prolog_graphs* g,
                                             const mla_prolog_graph_desc_t* descs,
                                             int32_t n_layers) {
    if (g == nullptr || descs == nullptr || n_layers != (int32_t)g->layers.size())
        return MLA_ERR_INVALID_ARG;
    for (int32_t l = 0; l < n_layers; ++l)
        if (!same_kind(descs[l], g->layers[0])) return MLA_ERR_INVALID_ARG;
    mla_status_t st = validate(descs, n_layers, g->buckets.data(), (int32_t)g->buckets.size());
    if (st != MLA_OK) return st;
    const std::vector<mla_prolog_graph_desc_t> layers(descs, descs + n_layers);
    return on_device(g->device, [&]() -> mla_status_t {
        hipStream_t s = nullptr;
        if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return MLA_ERR_HIP;
        // the new graphs first; the set changes only if every bucket succeeded
        std::vector<hipGraph_t> graphs(g->buckets.size(), nullptr);
        mla_status_t r = MLA_OK;
        for (size_t i = 0; i < graphs.size() && r == MLA_OK; ++i)
            r = capture(layers, g->buckets[i], s, &graphs[i]);
        (void)hipStreamDestroy(s);
        if (r == MLA_OK) {
            for (size_t i = 0; i < graphs.size() && r == MLA_OK; ++i) {
                hipGraphNode_t err_node = nullptr;
                hipGraphExecUpdateResult res = hipGraphExecUpdateSuccess;
                if (hipGraphExecUpdate(g->execs[i], graphs[i], &err_node, &res) == hipSuccess &&
                    res == hipGraphExecUpdateSuccess)
                    continue;
                (void)hipGetLastError();
                // not updatable in place: instantiate afresh
                hipGraphExec_t x = nullptr;
                if (hipGraphInstantiate(&x, graphs[i], nullptr, nullptr, 0) != hipSuccess) {
                    r = MLA_ERR_HIP;
                    break;
                }
                (void)hipGraphExecDestroy(g->execs[i]);
                g->execs[i] = x;
            }
            if (r == MLA_OK) g->layers = layers;
        }
        for (hipGraph_t x : graphs)
            if (x != nullptr) (void)hipGraphDestroy(x);
        return r;
    });
}

mla_status_t mla_prolog_graphs_update(mla_prolog_graphs* g, const mla_prolog_graph_desc_t* desc) {
    return mla_prolog_graphs_update_layers(g, desc, 1);
}

int32_t mla_prolog_graphs_layers(const mla_prolog_graphs* g) {
    return g == nullptr ? 0 : (int32_t)g->layers.size();
}

int64_t mla_prolog_graphs_bucket(const mla_prolog_graphs* g, int64_t T) {
    if (g == nullptr || T < 1) return 0;
    auto it = std::lower_bound(g->buckets.begin(), g->buckets.end(), T);
    return it == g->buckets.end() ? 0 : *it;
}

mla_status_t mla_prolog_graphs_launch(mla_prolog_graphs* g, int64_t T, void* stream,
                                      int64_t* bucket_used) {
    if (bucket_used != nullptr) *bucket_used = 0;
    if (g == nullptr || T < 0) return MLA_ERR_INVALID_ARG;
    if (T == 0) return MLA_OK;
    auto it = std::lower_bound(g->buckets.begin(), g->buckets.end(), T);
    if (it == g->buckets.end()) return MLA_ERR_INVALID_ARG;
    hipDevice_t dev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return MLA_ERR_HIP;
    if (dev != g->device) return MLA_ERR_INVALID_ARG;
    if (hipGraphLaunch(g->execs[it - g->buckets.begin()], (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_HIP;
    if (bucket_used != nullptr) *bucket_used = *it;
    return MLA_OK;
}

void mla_prolog_graphs_destroy(mla_prolog_graphs* g) {
    if (g == nullptr) return;
    const int device = g->device;  // g is gone after release
    int prev = -1;
    const bool ok = hipGetDevice(&prev) == hipSuccess;
    if (ok && prev != device) (void)hipSetDevice(device);
    release(g);
    if (ok && prev != device) (void)hipSetDevice(prev);
}

}  // extern "C"
