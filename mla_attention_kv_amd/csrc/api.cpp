// C-ABI of libmlaprolog: argument validation, launch planning (the
// decode / prefill dispatcher), workspace sizing, and the calls into the
// gfx950 launchers.  Every host-checkable condition is checked here, before
// anything reaches the GPU.
#include <atomic>
#include <cmath>

#include "../../include/libmlaprolog.h"
#include "mla_common.h"

using namespace mla;

namespace {

std::atomic<int> g_force_path{-1};
std::atomic<int> g_prefill_fusion{-1};
thread_local int t_validate_only = 0;

// Token counts up to this many take the decode tiling (small M tiles,
// split-K over the hidden dimension so that the weight stream is spread
// over the whole chip); larger counts take the prefill tiling.  The pages'
// own short/long split is by sequence length as well (the migration guide's
// note on dynamic selection); the threshold here is the widest decode batch
// of the benchmarked workloads.
constexpr int64_t kDecodeMaxT = 64;

int select_path(int64_t T) {
    const int f = g_force_path.load(std::memory_order_relaxed);
    if (f == 0 || f == 1) return f;
    return T <= kDecodeMaxT ? 0 : 1;
}

int kslabs_a(int H, bool int8) { return int8 ? H / 128 : H * 2 / 128; }

Plan make_plan(int64_t T, int H, bool int8, int path) {
    Plan p;
    p.path = path;
    p.stream = (!int8 && path == 0 && T <= kDecodeMaxT) ? 1 : 0;
    p.kw = 0;
    p.dma1 = 0;
    p.fuse2 = int8 ? 0 : g_prefill_fusion.load(std::memory_order_relaxed);
    if (p.stream) {
        // weight-streaming kv_a_proj: 9 slabs x S splits of kw rows each;
        // wider splits once the split-K partials (S * T rows of 576 floats)
        // outweigh the extra workgroups (measured: V2-Lite at T = 64 is
        // faster with S = 8 than with 16, at T = 1 slower)
        const int64_t tt = T < 16 ? 16 : T;
        int kw = H <= 64 ? 64 : 128;
        while (kw < 512 && ((H + kw - 1) / kw) * tt > 512) kw *= 2;
        p.kw = kw;
        p.s1 = (H + kw - 1) / kw;
        p.bm1 = p.bm2 = 16;
        p.bn2 = 64;
        return p;
    }
    const int ks = kslabs_a(H, int8);
    if (path == 0) {
        p.bm1 = T <= 16 ? 16 : (T <= 32 ? 32 : 64);
        p.bm2 = p.bm1;
        p.bn2 = 64;
    } else {
        p.bm1 = 128;
        // kv_b_proj: the pipelined 256 x 128 kernel for fp16 / bf16, 128 x 128
        // tiles for int8
        p.bm2 = 128;
        p.bn2 = 128;
    }
    if (path == 1) {
        // kv_a_proj on the pipelined kernel, tiles of 64, 128 or 160 rows by
        // 192 columns, K split S ways (S divides the slab count, at least two
        // slabs per split).  Chosen by a cost model: rounds of one item per CU
        // times the bytes each item copies into LDS, plus the split-K
        // partials written and read back (fp32/int32; the whole chip moves
        // them ~90x faster than one CU's copy stream: ~5.5 TB/s against
        // ~60 GB/s)
        p.dma1 = 1;
        const int bms[3] = {64, 128, 160};
        double best = 0.0;
        for (int bm : bms) {
            const int64_t tiles = ((T + bm - 1) / bm) * (kN1 / 192);
            for (int d = 1; d <= ks; ++d) {
                if (ks % d != 0 || (d > 1 && ks / d < 2)) continue;
                const int64_t items = tiles * d;
                const double rounds = (double)((items + 255) / 256);
                const double copy = rounds * (double)(bm + 192) * (double)ks / (double)d;
                const double partial = (double)d * (double)T * kN1 * 8.0 / 90.0 / 128.0;
                const double cost = copy + partial;
                if (best == 0.0 || cost < best) {
                    best = cost;
                    p.bm1 = bm;
                    p.s1 = d;
                }
            }
        }
        return p;
    }
    // split kv_a_proj's K so that at least ~256 workgroups stream W_kv_a,
    // keeping at least two K slabs per split
    const int64_t tiles = ((T + p.bm1 - 1) / p.bm1) * (kN1 / 64);
    int64_t s = (256 + tiles - 1) / tiles;
    const int64_t smax = ks >= 2 ? ks / 2 : 1;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    // equalise the slabs per split
    const int per = (int)((ks + s - 1) / s);
    p.s1 = (ks + per - 1) / per;
    return p;
}

// The RoPE frequencies theta^(-2i/dr) in double; kept per host thread for
// the last theta seen, since a serving loop passes the same theta every call.
const RopeTab& rope_table(float theta) {
    thread_local float last = 0.f;  // 0 is never a valid theta
    thread_local RopeTab rt;
    if (theta != last) {
        for (int i = 0; i < kDR / 2; ++i)
            rt.f[i] = std::pow((double)theta, -2.0 * (double)i / (double)kDR);
        last = theta;
    }
    return rt;
}

bool dims_supported(const mla_dims_t& d) {
    return d.r == kR && d.dr == kDR && d.dn == kDN && d.dv == kDV && d.nh >= 1 &&
           d.nh <= 1024 && d.H >= 64 && d.H <= 65536 && (d.H % 64) == 0;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t ws_fp_max(int64_t T, const mla_dims_t& d) {
    size_t m = 0;
    for (int path = 0; path < 2; ++path) {
        size_t b = ws_fp(T, make_plan(T, d.H, false, path)).total;
        if (b > m) m = b;
    }
    return m;
}
size_t ws_w8_max(int64_t T, const mla_dims_t& d) {
    size_t m = 0;
    for (int path = 0; path < 2; ++path) {
        size_t b = ws_w8(T, d.H, make_plan(T, d.H, true, path)).total;
        if (b > m) m = b;
    }
    return m;
}

}  // namespace

namespace {
// events registered by mla_debug_set_launch_events on this host thread
struct LaunchEvents {
    void* const* ev = nullptr;
    int32_t n = 0, used = 0;
};
thread_local LaunchEvents t_events;
}  // namespace

namespace mla {
void launch_events(hipEvent_t* start, hipEvent_t* stop) {
    LaunchEvents& e = t_events;
    if (e.ev != nullptr && e.used + 2 <= e.n) {
        *start = (hipEvent_t)e.ev[e.used];
        *stop = (hipEvent_t)e.ev[e.used + 1];
        e.used += 2;
    } else {
        *start = *stop = nullptr;
    }
}
bool validate_only() { return t_validate_only > 0; }
ValidateOnlyScope::ValidateOnlyScope() { ++t_validate_only; }
ValidateOnlyScope::~ValidateOnlyScope() { --t_validate_only; }
}  // namespace mla

extern "C" {

size_t mla_kv_prolog_workspace_size(int64_t T, mla_dims_t d, mla_dtype_t dt) {
    if (T <= 0 || T > MLA_MAX_TOKENS || !dims_supported(d)) return 0;
    if (dt != MLA_F16 && dt != MLA_BF16) return 0;
    return ws_fp_max(T, d);
}

size_t mla_kv_prolog_w8a8_workspace_size(int64_t T, mla_dims_t d) {
    if (T <= 0 || T > MLA_MAX_TOKENS || !dims_supported(d) || (d.H % 128) != 0) return 0;
    return ws_w8_max(T, d);
}

int mla_kv_prolog_selected_path(int64_t T, mla_dims_t) { return select_path(T); }

int mla_kv_prolog_force_path(int path) {
    if (path != 0 && path != 1) path = -1;
    return g_force_path.exchange(path);
}

int mla_debug_set_prefill_fusion(int mode) {
    if (mode != 0 && mode != 1) mode = -1;
    return g_prefill_fusion.exchange(mode);
}

int32_t mla_debug_set_launch_events(void* const* events, int32_t n) {
    const int32_t used = t_events.used;
    t_events.ev = (events != nullptr && n > 0) ? events : nullptr;
    t_events.n = t_events.ev != nullptr ? n : 0;
    t_events.used = 0;
    return used;
}

int64_t mla_debug_set_handoff_spin(int64_t limit) { return decode_set_spin_limit(limit); }

int64_t mla_debug_handoff_fallbacks(int reset) { return decode_handoff_fallbacks(reset != 0); }

const char* mla_status_string(mla_status_t s) {
    switch (s) {
        case MLA_OK: return "MLA_OK";
        case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: null pointer, bad T, eps, theta or dtype";
        case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: dims outside what the kernels implement";
        case MLA_ERR_MISALIGNED: return "MLA_ERR_MISALIGNED: a pointer is not 16-byte aligned";
        case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
        case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP launch or runtime call failed";
    }
    return "unknown mla_status_t";
}

}  // extern "C"

namespace {
// The fp16/bf16 prolog, with or without the paged-cache write in its finish.
mla_status_t prolog_fp(const void* hidden, const void* W_kv_a, const void* gamma,
                       const void* W_kv_b, const int32_t* positions, int64_t T, mla_dims_t d,
                       mla_dtype_t dt, float eps, float theta, void* k_nope, void* value,
                       void* k_pe, void* compressed_kv, const CacheOut& co, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (T < 0 || T > MLA_MAX_TOKENS) return MLA_ERR_INVALID_ARG;
    if (dt != MLA_F16 && dt != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(theta) || theta <= 0.f)
        return MLA_ERR_INVALID_ARG;
    if (!dims_supported(d)) return MLA_ERR_UNSUPPORTED;
    if (T == 0) return MLA_OK;
    const void* ptrs[] = {hidden, W_kv_a, gamma, W_kv_b, positions,
                          k_nope, value, k_pe, compressed_kv};
    for (const void* p : ptrs)
        if (p == nullptr) return MLA_ERR_INVALID_ARG;
    for (const void* p : ptrs)
        if (!aligned16(p)) return MLA_ERR_MISALIGNED;
    if (workspace == nullptr) return MLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MLA_ERR_MISALIGNED;
    const Plan plan = make_plan(T, d.H, false, select_path(T));
    if (workspace_bytes < ws_fp(T, plan).total) return MLA_ERR_WORKSPACE;
    if (validate_only()) return MLA_OK;
    hipError_t e = launch_fp((int)dt, hidden, W_kv_a, gamma, W_kv_b, positions, T, d.H, d.nh,
                             eps, rope_table(theta), k_nope, value, k_pe, compressed_kv,
                             workspace, plan, co, (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
}  // namespace

extern "C" {

mla_status_t mla_kv_prolog(const void* hidden, const void* W_kv_a, const void* gamma,
                           const void* W_kv_b, const int32_t* positions, int64_t T,
                           mla_dims_t d, mla_dtype_t dt, float eps, float theta,
                           void* k_nope, void* value, void* k_pe, void* compressed_kv,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return prolog_fp(hidden, W_kv_a, gamma, W_kv_b, positions, T, d, dt, eps, theta, k_nope,
                     value, k_pe, compressed_kv, CacheOut{nullptr, nullptr, 0}, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

namespace {
mla_status_t prolog_w8(const void* hidden_bf16, const int8_t* Wq_kv_a,
                                const float* s_kv_a, const void* gamma_bf16,
                                const int8_t* Wq_kv_b, const float* s_kv_b,
                                const int32_t* positions, int64_t T, mla_dims_t d, float eps,
                                float theta, void* k_nope, void* value, void* k_pe,
                                void* compressed_kv, int32_t* dbg_acc1, int32_t* dbg_acc2,
                                int64_t dbg_row_begin, int64_t dbg_rows, const CacheOut& co,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (T < 0 || T > MLA_MAX_TOKENS) return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(theta) || theta <= 0.f)
        return MLA_ERR_INVALID_ARG;
    if (!dims_supported(d) || (d.H % 128) != 0) return MLA_ERR_UNSUPPORTED;
    if (T == 0) return MLA_OK;
    const void* ptrs[] = {hidden_bf16, Wq_kv_a, s_kv_a, gamma_bf16, Wq_kv_b, s_kv_b,
                          positions, k_nope, value, k_pe, compressed_kv};
    for (const void* p : ptrs)
        if (p == nullptr) return MLA_ERR_INVALID_ARG;
    for (const void* p : ptrs)
        if (!aligned16(p)) return MLA_ERR_MISALIGNED;
    if (dbg_acc1 != nullptr || dbg_acc2 != nullptr) {
        if (dbg_rows < 0 || dbg_row_begin < 0 || dbg_row_begin + dbg_rows > T)
            return MLA_ERR_INVALID_ARG;
        if ((dbg_acc1 && !aligned16(dbg_acc1)) || (dbg_acc2 && !aligned16(dbg_acc2)))
            return MLA_ERR_MISALIGNED;
    } else {
        dbg_rows = 0;
        dbg_row_begin = 0;
    }
    if (workspace == nullptr) return MLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MLA_ERR_MISALIGNED;
    const Plan plan = make_plan(T, d.H, true, select_path(T));
    if (workspace_bytes < ws_w8(T, d.H, plan).total) return MLA_ERR_WORKSPACE;
    if (validate_only()) return MLA_OK;
    hipError_t e = launch_w8a8(hidden_bf16, Wq_kv_a, s_kv_a, gamma_bf16, Wq_kv_b, s_kv_b,
                               positions, T, d.H, d.nh, eps, rope_table(theta), k_nope, value, k_pe,
                               compressed_kv, dbg_acc1, dbg_acc2, dbg_row_begin, dbg_rows,
                               workspace, plan, co, (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
}  // namespace

extern "C" {

mla_status_t mla_kv_prolog_w8a8(const void* hidden_bf16, const int8_t* Wq_kv_a,
                                const float* s_kv_a, const void* gamma_bf16,
                                const int8_t* Wq_kv_b, const float* s_kv_b,
                                const int32_t* positions, int64_t T, mla_dims_t d, float eps,
                                float theta, void* k_nope, void* value, void* k_pe,
                                void* compressed_kv, int32_t* dbg_acc1, int32_t* dbg_acc2,
                                int64_t dbg_row_begin, int64_t dbg_rows, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return prolog_w8(hidden_bf16, Wq_kv_a, s_kv_a, gamma_bf16, Wq_kv_b, s_kv_b, positions, T, d,
                     eps, theta, k_nope, value, k_pe, compressed_kv, dbg_acc1, dbg_acc2,
                     dbg_row_begin, dbg_rows, CacheOut{nullptr, nullptr, 0}, workspace,
                     workspace_bytes, stream);
}

static mla_status_t kv_cache_args(const void* compressed_kv, const void* k_pe,
                                  const int64_t* slot_mapping, int64_t T, mla_dims_t d,
                                  mla_dtype_t dt, int64_t num_slots) {
    if (T < 0 || T > MLA_MAX_TOKENS || num_slots < 0) return MLA_ERR_INVALID_ARG;
    if (dt != MLA_F16 && dt != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (d.r != kR || d.dr != kDR) return MLA_ERR_UNSUPPORTED;
    if (T == 0) return MLA_OK;
    if (compressed_kv == nullptr || k_pe == nullptr || slot_mapping == nullptr)
        return MLA_ERR_INVALID_ARG;
    if (!aligned16(compressed_kv) || !aligned16(k_pe) || ((uintptr_t)slot_mapping & 7u) != 0)
        return MLA_ERR_MISALIGNED;
    return MLA_OK;
}

mla_status_t mla_kv_cache_append(const void* compressed_kv, const void* k_pe,
                                 const int64_t* slot_mapping, int64_t T, mla_dims_t d,
                                 mla_dtype_t dt, void* kv_cache, int64_t num_slots,
                                 void* stream) {
    const mla_status_t st = kv_cache_args(compressed_kv, k_pe, slot_mapping, T, d, dt, num_slots);
    if (st != MLA_OK || T == 0 || num_slots == 0) return st;
    if (kv_cache == nullptr) return MLA_ERR_INVALID_ARG;
    if (!aligned16(kv_cache)) return MLA_ERR_MISALIGNED;
    const hipError_t e = launch_kv_cache_append(dt, compressed_kv, k_pe, slot_mapping, T,
                                                num_slots, kv_cache, nullptr, nullptr,
                                                (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_kv_cache_append_int8(const void* compressed_kv, const void* k_pe,
                                      const int64_t* slot_mapping, int64_t T, mla_dims_t d,
                                      mla_dtype_t dt, int8_t* kv_cache_q, float* kv_scale,
                                      int64_t num_slots, void* stream) {
    const mla_status_t st = kv_cache_args(compressed_kv, k_pe, slot_mapping, T, d, dt, num_slots);
    if (st != MLA_OK || T == 0 || num_slots == 0) return st;
    if (kv_cache_q == nullptr || kv_scale == nullptr) return MLA_ERR_INVALID_ARG;
    if (!aligned16(kv_cache_q) || ((uintptr_t)kv_scale & 3u) != 0) return MLA_ERR_MISALIGNED;
    const hipError_t e = launch_kv_cache_append(dt, compressed_kv, k_pe, slot_mapping, T,
                                                num_slots, nullptr, kv_cache_q, kv_scale,
                                                (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: mla_kv_prolog with its workspace in
// a file-scope device array of this library (one copy per GPU, held until
// the process ends).  In host code `scratch` is only a stand-in for the
// array: its device address comes from hipGetSymbolAddress, looked up once
// per device (with that device current) and kept in g_scratch_ptr.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<void*> g_scratch_ptr[64];

// Device address of this device's scratch array, or nullptr on a HIP error.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
        return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    return q;
}
}  // namespace

extern "C" {

mla_status_t mla_kv_prolog_noalloc(const void* hidden, const void* W_kv_a, const void* gamma,
                                   const void* W_kv_b, const int32_t* positions, int64_t T,
                                   mla_dims_t d, mla_dtype_t dt, float eps, float theta,
                                   void* k_nope, void* value, void* k_pe, void* compressed_kv,
                                   void* stream) {
    // sizes beyond the scratch array are rejected before anything else runs
    if (T > 0 && T <= MLA_MAX_TOKENS && dims_supported(d) && (dt == MLA_F16 || dt == MLA_BF16) &&
        ws_fp_max(T, d) > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
        return MLA_ERR_WORKSPACE;
    {
        // every other argument check first, against a stand-in workspace
        // address that is never dereferenced
        ValidateOnlyScope checks_only;
        const mla_status_t st = prolog_fp(
            hidden, W_kv_a, gamma, W_kv_b, positions, T, d, dt, eps, theta, k_nope, value, k_pe,
            compressed_kv, CacheOut{nullptr, nullptr, 0}, (void*)(uintptr_t)256,
            (size_t)MLA_NOALLOC_SCRATCH_BYTES, stream);
        if (st != MLA_OK || T == 0) return st;
    }
    if (validate_only()) return MLA_OK;
    void* ws = scratch_ptr();
    if (ws == nullptr) return MLA_ERR_HIP;
    return prolog_fp(hidden, W_kv_a, gamma, W_kv_b, positions, T, d, dt, eps, theta, k_nope,
                     value, k_pe, compressed_kv, CacheOut{nullptr, nullptr, 0}, ws,
                     (size_t)MLA_NOALLOC_SCRATCH_BYTES, stream);
}

mla_status_t mla_kv_prolog_cached(const void* hidden, const void* W_kv_a, const void* gamma,
                                  const void* W_kv_b, const int32_t* positions, int64_t T,
                                  mla_dims_t d, mla_dtype_t dt, float eps, float theta,
                                  void* k_nope, void* value, void* k_pe, void* compressed_kv,
                                  const int64_t* slot_mapping, void* kv_cache,
                                  int64_t num_slots, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (num_slots < 0) return MLA_ERR_INVALID_ARG;
    if (T > 0 && num_slots > 0) {
        if (slot_mapping == nullptr || kv_cache == nullptr) return MLA_ERR_INVALID_ARG;
        if (((uintptr_t)slot_mapping & 7u) != 0 || !aligned16(kv_cache)) return MLA_ERR_MISALIGNED;
    }
    const CacheOut co{num_slots > 0 ? slot_mapping : nullptr,
                      num_slots > 0 ? (uint16_t*)kv_cache : nullptr, num_slots};
    return prolog_fp(hidden, W_kv_a, gamma, W_kv_b, positions, T, d, dt, eps, theta, k_nope,
                     value, k_pe, compressed_kv, co, workspace, workspace_bytes, stream);
}

mla_status_t mla_rms_norm(const void* x, const void* gamma, int64_t rows, int64_t n,
                          mla_dtype_t dt, float eps, void* y, void* stream) {
    if (rows < 0 || rows > (int64_t)MLA_MAX_TOKENS * 1024) return MLA_ERR_INVALID_ARG;
    if (dt != MLA_F16 && dt != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.f) return MLA_ERR_INVALID_ARG;
    if (n < 8 || n > 8192 || (n % 8) != 0) return MLA_ERR_UNSUPPORTED;
    if (rows == 0) return MLA_OK;
    if (x == nullptr || gamma == nullptr || y == nullptr) return MLA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(y)) return MLA_ERR_MISALIGNED;
    const hipError_t e = launch_rms_norm(dt, x, gamma, rows, (int)n, eps, y, (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_rope(const void* x, const int32_t* positions, int64_t T, int64_t heads,
                      int64_t dr, mla_dtype_t dt, float theta, void* y, void* stream) {
    if (T < 0 || T > MLA_MAX_TOKENS || heads < 1 || heads > 1024) return MLA_ERR_INVALID_ARG;
    if (dt != MLA_F16 && dt != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(theta) || theta <= 0.f) return MLA_ERR_INVALID_ARG;
    if (dr != kDR) return MLA_ERR_UNSUPPORTED;
    if (T == 0) return MLA_OK;
    if (x == nullptr || positions == nullptr || y == nullptr) return MLA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y) || ((uintptr_t)positions & 3u) != 0)
        return MLA_ERR_MISALIGNED;
    const hipError_t e = launch_rope(dt, x, positions, T, (int)heads, rope_table(theta), y,
                                     (hipStream_t)stream);
    return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_kv_prolog_w8a8_cached(const void* hidden_bf16, const int8_t* Wq_kv_a,
                                       const float* s_kv_a, const void* gamma_bf16,
                                       const int8_t* Wq_kv_b, const float* s_kv_b,
                                       const int32_t* positions, int64_t T, mla_dims_t d,
                                       float eps, float theta, void* k_nope, void* value,
                                       void* k_pe, void* compressed_kv,
                                       const int64_t* slot_mapping, void* kv_cache,
                                       int8_t* kv_cache_q, float* kv_scale, int64_t num_slots,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    if (num_slots < 0) return MLA_ERR_INVALID_ARG;
    const bool q8 = kv_cache_q != nullptr || kv_scale != nullptr;
    if (T > 0 && num_slots > 0) {
        // exactly one cache: bf16 (kv_cache) or int8 codes + scales
        if (slot_mapping == nullptr) return MLA_ERR_INVALID_ARG;
        if (q8 ? (kv_cache != nullptr || kv_cache_q == nullptr || kv_scale == nullptr)
               : kv_cache == nullptr)
            return MLA_ERR_INVALID_ARG;
        if (((uintptr_t)slot_mapping & 7u) != 0) return MLA_ERR_MISALIGNED;
        if (q8 ? (!aligned16(kv_cache_q) || ((uintptr_t)kv_scale & 3u) != 0)
               : !aligned16(kv_cache))
            return MLA_ERR_MISALIGNED;
    }
    CacheOut co{nullptr, nullptr, 0};
    if (num_slots > 0) {
        co.slots = slot_mapping;
        co.num_slots = num_slots;
        if (q8) {
            co.cache_q = kv_cache_q;
            co.scale = kv_scale;
        } else {
            co.cache = (uint16_t*)kv_cache;
        }
    }
    return prolog_w8(hidden_bf16, Wq_kv_a, s_kv_a, gamma_bf16, Wq_kv_b, s_kv_b, positions, T, d,
                     eps, theta, k_nope, value, k_pe, compressed_kv, nullptr, nullptr, 0, 0, co,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"
