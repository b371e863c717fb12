/*
 * libmlaprolog -- the MLA (Multi-head Latent Attention) KV prolog on AMD
 * Instinct MI355X (gfx950).
 *
 * The prolog turns each token's hidden state into the key/value inputs of
 * MLA attention, in seven steps (DeepSeek-V2-Lite-Chat MLA KV Prolog
 * migration guide, dpshk.com, section "Background"; data flow in section
 * "Source-level principle"):
 *
 *   1. kv_a_proj      A = X . W_kv_a               [T,H] x [H, r+dr]
 *   2. split          c = A[:, :r]  (compressed_kv),  p = A[:, r:]  (k_pe)
 *   3. RMSNorm        y = c / sqrt(mean(c^2) + eps) * gamma
 *   4. kv_b_proj      B = y . W_kv_b               [T,r] x [r, nh*(dn+dv)]
 *   5. reshape+split  B -> [T, nh, dn+dv]; k_nope = [..., :dn], value = [..., dn:]
 *   6. RoPE on p      rotate-half form, pairs (i, i + dr/2),
 *                     angle pos * theta^(-2i/dr)  (section "Precision
 *                     verification": the standard x*cos + x_rot*sin form)
 *   7. assemble       write k_nope, value, k_pe and the normalised
 *                     compressed_kv
 *
 * The W8A8 entry point is the same prolog with int8 weights (per-output-
 * column fp32 scales) and per-token dynamic int8 activations, accumulating
 * in int32 (the quantised-weight modes of the DeepSeek-R1 inference-recipe
 * page, section "Weight conversion").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer, allocated and owned by the
 *   caller; the library never allocates, frees or keeps a pointer past the
 *   call.  Scratch memory is the caller's `workspace` (size from the
 *   matching *_workspace_size query).  A workspace needs no initialisation:
 *   every call writes whatever it later reads, so one workspace can serve
 *   any sequence of ordered calls (of either entry point).
 * - Tensors are contiguous, row-major, in exactly the shapes given.  W_kv_b's
 *   columns come in per-head blocks [k_nope_h (dn) | value_h (dv)].
 *   Outputs are token-major: k_nope [T,nh,dn], value [T,nh,dv],
 *   k_pe [T,dr] (one rope key per token, shared by all heads),
 *   compressed_kv [T,r].
 * - Every pointer must be 16-byte aligned.  Outputs must not alias inputs
 *   or each other or the workspace.
 * - Supported by the GPU kernels: r = 512, dr = 64, dn = dv = 128,
 *   1 <= nh <= 1024, H a multiple of 64 with 64 <= H <= 65536,
 *   0 <= T <= MLA_MAX_TOKENS.  Anything else returns MLA_ERR_UNSUPPORTED.
 * - Every host-checkable condition (null pointer, dims, alignment,
 *   workspace size, eps/theta) is checked before anything is launched; on
 *   failure nothing is launched and a status is returned.  T == 0 returns
 *   MLA_OK and launches nothing.  Launch failures return MLA_ERR_HIP.
 * - Device-side contents are preconditions, not checked: positions >= 0,
 *   finite inputs.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream) and never synchronise.  Two calls that share a workspace must
 *   be ordered (same stream, or synchronised).
 * - The library holds no per-call state and is safe to call from several
 *   host threads (apart from mla_kv_prolog_force_path and the mla_debug_set_*
 *   calls, test hooks).
 */
#ifndef LIBMLAPROLOG_H
#define LIBMLAPROLOG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_MAX_TOKENS (1 << 22)

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = -1, /* null pointer, negative T, bad eps/theta, unknown dtype */
    MLA_ERR_UNSUPPORTED = -2, /* dims outside what the kernels implement */
    MLA_ERR_MISALIGNED = -3,  /* a pointer not 16-byte aligned */
    MLA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the query says */
    MLA_ERR_HIP = -5          /* a HIP launch or runtime call failed */
} mla_status_t;

typedef enum { MLA_F16 = 1, MLA_BF16 = 2 } mla_dtype_t;

typedef struct {
    int32_t H;  /* hidden size */
    int32_t r;  /* kv_lora_rank (compressed latent width) */
    int32_t dr; /* rope dim */
    int32_t nh; /* heads */
    int32_t dn; /* qk_nope_head_dim */
    int32_t dv; /* v_head_dim */
} mla_dims_t;

/* Bytes of workspace mla_kv_prolog needs for T tokens (0 for T == 0).
 * Returns 0 as well for unsupported dims or dtype (the call then fails). */
size_t mla_kv_prolog_workspace_size(int64_t T, mla_dims_t d, mla_dtype_t dt);

/*
 * fp16 / bf16 KV prolog (steps 1-7 above, all in one call).
 *   hidden      [T, H]            dt
 *   W_kv_a      [H, r+dr]         dt   (the kv_a_proj weight, already transposed)
 *   gamma       [r]               dt   (RMSNorm weight)
 *   W_kv_b      [r, nh*(dn+dv)]   dt
 *   positions   [T]               int32, >= 0
 *   eps         RMSNorm epsilon (finite, >= 0), theta RoPE base (finite, > 0)
 *   k_nope      [T, nh, dn]       dt   (out)
 *   value       [T, nh, dv]       dt   (out)
 *   k_pe        [T, dr]           dt   (out, after RoPE)
 *   compressed_kv [T, r]          dt   (out, the normalised latent that
 *                                       kv_b_proj consumes)
 * Accumulation is fp32; intermediates never leave fp32 except the
 * normalised latent, which is rounded to dt (it is an output) before
 * kv_b_proj.
 */
mla_status_t mla_kv_prolog(const void* hidden, const void* W_kv_a, const void* gamma,
                           const void* W_kv_b, const int32_t* positions, int64_t T,
                           mla_dims_t d, mla_dtype_t dt, float eps, float theta,
                           void* k_nope, void* value, void* k_pe, void* compressed_kv,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mla_kv_prolog_w8a8 needs for T tokens. */
size_t mla_kv_prolog_w8a8_workspace_size(int64_t T, mla_dims_t d);

/*
 * W8A8 KV prolog.  bf16 activations, gamma and outputs; int8 weights with
 * fp32 per-output-column scales (weight = code * scale[column]).
 *   hidden_bf16 [T, H]; Wq_kv_a int8 [H, r+dr], s_kv_a fp32 [r+dr];
 *   gamma_bf16 [r]; Wq_kv_b int8 [r, nh*(dn+dv)], s_kv_b fp32 [nh*(dn+dv)].
 * Steps, every one in IEEE fp32 with round-to-nearest-even:
 *   qx = clamp(rint(x * (127/amax_t)), +-127), sx = amax_t/127, amax_t =
 *   max_k |x[t,k]| (a zero row gives codes 0, scale 0);
 *   acc1 = qx . Wq_kv_a (int32, exact); A = (float(acc1) * sx) * s_kv_a[n];
 *   z = c * gamma; qz, sz = the same per-token quantisation of z;
 *   acc2 = qz . Wq_kv_b (int32, exact); inv_t = 1/sqrt(mean(c^2) + eps);
 *   k_nope/value = bf16(((float(acc2) * sz) * inv_t) * s_kv_b[m]);
 *   compressed_kv = bf16(z * inv_t); k_pe = bf16(RoPE(A[:, r:])).
 * Debug export (both may be NULL): for token rows
 * [dbg_row_begin, dbg_row_begin + dbg_rows) the exact int32 accumulators
 * are written to dbg_acc1 [dbg_rows, r+dr] and dbg_acc2 [dbg_rows,
 * nh*(dn+dv)].  Rows outside [0, T) are an MLA_ERR_INVALID_ARG.
 */
mla_status_t mla_kv_prolog_w8a8(const void* hidden_bf16, const int8_t* Wq_kv_a,
                                const float* s_kv_a, const void* gamma_bf16,
                                const int8_t* Wq_kv_b, const float* s_kv_b,
                                const int32_t* positions, int64_t T, mla_dims_t d,
                                float eps, float theta, void* k_nope, void* value,
                                void* k_pe, void* compressed_kv, int32_t* dbg_acc1,
                                int32_t* dbg_acc2, int64_t dbg_row_begin, int64_t dbg_rows,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged KV-cache append: the step after "assemble".  MLA caches, per token,
 * the normalised latent and the rotated rope key (the smaller KV cache is the
 * point of the method: migration guide, section "Background"); the R1 recipe
 * page names paged attention ("Benchmark") and an int8-cache mode W8A8C8
 * ("Weight conversion") but fixes no layout or formula.  Layout used here:
 * the cache is num_slots slots of r + dr values; slot s holds
 * [compressed_kv row | k_pe row].  A paged cache of blocks of B slots is the
 * same array with slot = block * B + offset.
 *   compressed_kv [T, r]  dt, k_pe [T, dr] dt  (the prolog's outputs)
 *   slot_mapping  [T]     int64: token t goes to slot slot_mapping[t]; a
 *                         value outside [0, num_slots) (e.g. -1 for a
 *                         padding token) skips the token.  The kernels test
 *                         every value, so no mapping writes outside the
 *                         cache.  Slots of different tokens must be distinct
 *                         (precondition: otherwise the result is any one of
 *                         the tokens).
 *   kv_cache      [num_slots, r + dr]  dt (in/out; only mapped slots change)
 * Supported: r = 512, dr = 64 (d's other fields are not used).
 * compressed_kv, k_pe and the caches 16-byte aligned, slot_mapping 8-byte and
 * kv_scale 4-byte aligned.  T == 0 or num_slots == 0 launches nothing.
 * Errors as for the prolog (checked before any launch).
 */
mla_status_t mla_kv_cache_append(const void* compressed_kv, const void* k_pe,
                                 const int64_t* slot_mapping, int64_t T, mla_dims_t d,
                                 mla_dtype_t dt, void* kv_cache, int64_t num_slots,
                                 void* stream);

/*
 * The same into an int8 ("C8") cache with one fp32 scale per slot: the
 * slot's r + dr values are quantised together by the W8A8 activation scheme
 * (fp32, round half to even): amax = max |v|, code = clamp(rint(v *
 * (127/amax)), +-127), scale = amax / 127; a zero row gives codes 0, scale 0.
 * Value ~ code * scale.
 *   kv_cache_q [num_slots, r + dr] int8 (in/out), kv_scale [num_slots] fp32
 *   (in/out; only mapped slots change)
 */
mla_status_t mla_kv_cache_append_int8(const void* compressed_kv, const void* k_pe,
                                      const int64_t* slot_mapping, int64_t T, mla_dims_t d,
                                      mla_dtype_t dt, int8_t* kv_cache_q, float* kv_scale,
                                      int64_t num_slots, void* stream);

/*
 * The prolog (mla_kv_prolog, same arguments and outputs) with the paged
 * KV-cache append fused into its finish: the kernel that writes a token's
 * compressed_kv and k_pe rows also writes them into kv_cache slot
 * slot_mapping[t] (layout, slot rules and alignment as for
 * mla_kv_cache_append), so the cache holds exactly the bits of the returned
 * rows and the rows are not read back from HBM.  num_slots == 0 writes no
 * cache (slot_mapping and kv_cache may then be NULL).  Errors as for the
 * prolog and the append; nothing launches when any check fails.
 */
mla_status_t mla_kv_prolog_cached(const void* hidden, const void* W_kv_a, const void* gamma,
                                  const void* W_kv_b, const int32_t* positions, int64_t T,
                                  mla_dims_t d, mla_dtype_t dt, float eps, float theta,
                                  void* k_nope, void* value, void* k_pe, void* compressed_kv,
                                  const int64_t* slot_mapping, void* kv_cache,
                                  int64_t num_slots, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * The W8A8 prolog (mla_kv_prolog_w8a8, same arguments and outputs, without
 * the debug export) with the paged-cache append fused into its finish, into
 * exactly one cache:
 *   kv_cache   [num_slots, r + dr] bf16: the returned rows' bits; or
 *   kv_cache_q [num_slots, r + dr] int8 + kv_scale [num_slots] fp32: the
 *              returned bf16 rows quantised per slot as mla_kv_cache_append_int8
 *              does (the int8-cache "C8" of the R1 recipe's W8A8C8 mode,
 *              section "Weight conversion"); bit-identical to that call on the
 *              returned rows.
 * The other cache pointer(s) must be NULL.  Slot rules, alignment and
 * num_slots == 0 as for mla_kv_prolog_cached.
 */
mla_status_t mla_kv_prolog_w8a8_cached(const void* hidden_bf16, const int8_t* Wq_kv_a,
                                       const float* s_kv_a, const void* gamma_bf16,
                                       const int8_t* Wq_kv_b, const float* s_kv_b,
                                       const int32_t* positions, int64_t T, mla_dims_t d,
                                       float eps, float theta, void* k_nope, void* value,
                                       void* k_pe, void* compressed_kv,
                                       const int64_t* slot_mapping, void* kv_cache,
                                       int8_t* kv_cache_q, float* kv_scale, int64_t num_slots,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Standalone RMSNorm: the prolog's step 3 as an operator of its own (the
 * migration guide ships it as a separate kernel next to the fused prolog:
 * section "Directory layout", and a switch of its own in its usage section).
 * Per row of n values, in fp32:
 *   y[j] = round_dt((x[j] * inv) * gamma[j]),  inv = 1 / sqrt(sum_j x[j]^2 / n + eps)
 * (eps inside the root, gamma after the normalisation: section "Precision
 * verification"; the same arithmetic as the prolog's compressed_kv).
 *   x [rows, n] dt (input), gamma [n] dt (input), y [rows, n] dt (output;
 *   may be x: in place)
 * Supported: n a multiple of 8, 8 <= n <= 8192; rows <= 2^32.  Pointers
 * 16-byte aligned.  rows == 0 launches nothing.  Errors as for the prolog
 * (checked before any launch).
 */
mla_status_t mla_rms_norm(const void* x, const void* gamma, int64_t rows, int64_t n,
                          mla_dtype_t dt, float eps, void* y, void* stream);

/*
 * Standalone RoPE: the prolog's step 6 as an operator of its own (same
 * sections as mla_rms_norm), rotate-half form on rows of dr values; every
 * head of token t is rotated by positions[t]:
 *   f_i = theta^(-2i/dr), a = positions[t] * f_i, for i < dr/2:
 *   y[i] = x[i] cos a - x[i + dr/2] sin a;  y[i + dr/2] = x[i + dr/2] cos a + x[i] sin a
 * (cos and sin as in the prolog: the angle formed and reduced in double).
 *   x [T, heads, dr] dt (input), positions [T] int32 (input),
 *   y [T, heads, dr] dt (output; may be x: in place)
 * Supported: dr = 64, 1 <= heads <= 1024.  x and y 16-byte aligned,
 * positions 4-byte aligned.  T == 0 launches nothing.
 */
mla_status_t mla_rope(const void* x, const int32_t* positions, int64_t T, int64_t heads,
                      int64_t dr, mla_dtype_t dt, float theta, void* y, void* stream);

/*
 * Captured decode buckets.  The migration guide runs the fused prolog in
 * graph mode (aclgraph) to cut scheduling overhead ("Background"), warming
 * it up at q_len 1 and 2 with the first layer's weights before serving
 * ("Command-line parameters", notes 2-3; "Migration notes", item 3).
 * Here a set holds one HIP graph per bucket of token counts, each the
 * launch sequence of one prolog call over fixed ("static") buffers; a step
 * is one graph launch.
 *
 * The descriptor names every buffer of the recorded call, exactly as the
 * plain entry points take them:
 *   w8a8 == 0: mla_kv_prolog_cached (dt, W_kv_a, gamma, W_kv_b; s_kv_a,
 *              s_kv_b, kv_cache_q, kv_scale unused, NULL);
 *   w8a8 == 1: mla_kv_prolog_w8a8_cached (W_kv_a / W_kv_b are the int8
 *              weights, s_kv_a / s_kv_b their scales; dt unused).
 *   num_slots == 0 records the plain prolog (no cache write).
 * Per-token buffers (hidden, positions, the four outputs, slot_mapping) hold
 * rows for the largest bucket; workspace_bytes covers every bucket
 * (the *_workspace_size query of each).  All buffers stay owned by the
 * caller and must outlive the set (or its next update).
 */
typedef struct {
    int32_t w8a8;
    mla_dims_t d;
    mla_dtype_t dt;
    float eps, theta;
    const void* W_kv_a;
    const float* s_kv_a;
    const void* gamma;
    const void* W_kv_b;
    const float* s_kv_b;
    const void* hidden;
    const int32_t* positions;
    void* k_nope;
    void* value;
    void* k_pe;
    void* compressed_kv;
    const int64_t* slot_mapping;
    void* kv_cache;
    int8_t* kv_cache_q;
    float* kv_scale;
    int64_t num_slots;
    void* workspace;
    size_t workspace_bytes;
} mla_prolog_graph_desc_t;

typedef struct mla_prolog_graphs mla_prolog_graphs;

/*
 * Capture one graph per bucket (buckets: n_buckets ascending token counts,
 * 1 <= n_buckets <= 64, each in [1, MLA_MAX_TOKENS]) on the current device
 * and return the set in *out (every buffer of the descriptor must live on
 * that device).  Every argument check of every recorded call runs first; on failure nothing is captured, *out is NULL and the status
 * is that of the failing check.  Capture launches nothing: the kernels run
 * only when a graph is launched.  Not to be called while the calling
 * thread is capturing a stream of its own.
 */
mla_status_t mla_prolog_graphs_create(const mla_prolog_graph_desc_t* desc,
                                      const int64_t* buckets, int32_t n_buckets,
                                      mla_prolog_graphs** out);

/*
 * The same over n_layers layers (1 <= n_layers <= 256): descs[l] names layer
 * l's weights, cache and buffers (the layers must agree in w8a8, dims and,
 * for w8a8 == 0, dt; MLA_ERR_INVALID_ARG otherwise).  Each bucket's graph
 * replays the prolog of every layer, in layer order, so one launch runs all
 * n_layers prologs: the guide captures the whole model forward into one
 * graph ("Command-line parameters", note 3), and a graph launch costs the
 * host about as much as a few direct kernel launches, so it pays off over
 * many layers.  Layers may share buffers (say one workspace: the replays of
 * one graph are ordered).  mla_prolog_graphs_create is the case
 * n_layers == 1.
 */
mla_status_t mla_prolog_graphs_create_layers(const mla_prolog_graph_desc_t* descs,
                                             int32_t n_layers, const int64_t* buckets,
                                             int32_t n_buckets, mla_prolog_graphs** out);

/*
 * One prolog step over the first T rows of the static buffers: launches the
 * graph of the smallest bucket >= T on `stream` (a stream of the set's
 * device; NULL = the default stream) and stores that bucket in
 * *bucket_used (if not NULL).  Rows [T, bucket) are computed too, from
 * whatever the static buffers hold there: they must be finite (zeros, or an
 * earlier step's rows), and with a cache their slot_mapping entries must lie
 * outside [0, num_slots) (e.g. -1) so that padding writes no slot.  T == 0
 * launches nothing; T above the largest bucket, or a stream of another
 * device, is MLA_ERR_INVALID_ARG.  Asynchronous; steps share the static
 * buffers and workspace, so they must be ordered (one stream).
 */
mla_status_t mla_prolog_graphs_launch(mla_prolog_graphs* g, int64_t T, void* stream,
                                      int64_t* bucket_used);

/* The bucket a step of T tokens runs (0 if T < 1 or above the largest). */
int64_t mla_prolog_graphs_bucket(const mla_prolog_graphs* g, int64_t T);

/*
 * Rebind a one-layer set to new buffers (say the next layer's weights and
 * cache, or new static buffers): the graphs are re-recorded from desc and
 * updated in place.  w8a8, dims and (for w8a8 == 0) dt must equal the set's
 * (MLA_ERR_INVALID_ARG otherwise); eps, theta and every pointer may change.
 * Checks run first: on a failed check the set is unchanged.  On
 * MLA_ERR_HIP the set may be partly updated and should be destroyed.  The
 * caller first synchronises with any launch of the set in flight.
 *
 * Launch and bucket may be called from several host threads at once (their
 * steps still share the static buffers); update and destroy must not run
 * concurrently with any other call on the same set.
 */
mla_status_t mla_prolog_graphs_update(mla_prolog_graphs* g, const mla_prolog_graph_desc_t* desc);

/* Rebind every layer of a set made by mla_prolog_graphs_create_layers
 * (n_layers must equal the set's; the same rules as mla_prolog_graphs_update
 * per layer).  mla_prolog_graphs_update is the case n_layers == 1. */
mla_status_t mla_prolog_graphs_update_layers(mla_prolog_graphs* g,
                                             const mla_prolog_graph_desc_t* descs,
                                             int32_t n_layers);

/* The number of layers a set replays per launch (0 for NULL). */
int32_t mla_prolog_graphs_layers(const mla_prolog_graphs* g);

/* Free the set's graphs (NULL is a no-op).  The caller first synchronises
 * with any launch of the set in flight. */
void mla_prolog_graphs_destroy(mla_prolog_graphs* g);

/* The kernel family the dispatcher picks for T tokens: 0 = decode
 * (weight-streaming, small T), 1 = prefill (MFMA-tiled, large T). */
int mla_kv_prolog_selected_path(int64_t T, mla_dims_t d);

/* Test / benchmark hook: force every later call in this process onto one
 * kernel family (0 or 1), or back to the dispatcher's choice (-1).  Returns
 * the previous setting.  Not for concurrent use. */
int mla_kv_prolog_force_path(int path);

/* Test / benchmark hook for the fp16 / bf16 MFMA-tiled kernels (the
 * prefill family, and the decode family when forced past 64 tokens): run
 * the finish (split, RMSNorm, RoPE) and kv_b_proj as one launch whose
 * workgroups normalise a 64-row block's latent into LDS and feed kv_b_proj
 * from there (1), as two launches through compressed_kv in memory (0), or
 * as the dispatcher decides (-1: never, today).  Both give the same bits
 * wherever the separate finish adds kv_a_proj's K splits in ascending
 * order (up to 8 splits, or from 2048 tokens); elsewhere they differ by
 * the rounding of that sum.  Returns the previous setting.  Not for
 * concurrent use. */
int mla_debug_set_prefill_fusion(int mode);

/* The fp16 / bf16 prolog for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, checks, outputs and kernels as mla_kv_prolog, minus the
 * workspace: its scratch memory is a device array inside this library, one
 * per GPU (MLA_NOALLOC_SCRATCH_BYTES, held until the process ends).  The
 * call itself allocates nothing.  Its first call on a device looks up that
 * device's array address once (hipGetSymbolAddress).
 *
 * Limit: T whose mla_kv_prolog_workspace_size(T, d, dt) exceeds
 * MLA_NOALLOC_SCRATCH_BYTES returns MLA_ERR_WORKSPACE and launches nothing
 * (V2-Lite shapes: every decode batch and prefills of several thousand
 * tokens fit).  MLA_ERR_HIP if the array's address cannot be obtained.
 *
 * Every call on a GPU uses that GPU's one array, so calls that overlap in
 * time on one GPU (different streams, or different host threads without
 * ordering) race and give undefined results: order them (one stream, or
 * events).  The array needs no clearing: every call writes whatever it
 * later reads. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status_t mla_kv_prolog_noalloc(const void* hidden, const void* W_kv_a, const void* gamma,
                                   const void* W_kv_b, const int32_t* positions, int64_t T,
                                   mla_dims_t d, mla_dtype_t dt, float eps, float theta,
                                   void* k_nope, void* value, void* k_pe, void* compressed_kv,
                                   void* stream);

/* Benchmark hook: per-kernel timing.  Registers, for the calling host
 * thread, n events (hipEvent_t handles created with timing enabled and owned
 * by the caller; the array is read at each launch, so it must stay valid
 * until it is unregistered; NULL or n <= 0 unregisters).  Every later prolog
 * call on this thread (mla_kv_prolog* entry points) then takes the next two
 * events for each kernel it launches, while at least two are left, and the
 * launch records them at that kernel's own start and end (the dispatch's
 * timestamps, hipExtLaunchKernel), so the elapsed time between events 2k
 * and 2k + 1 is the duration of the call's k-th kernel.  Returns how many
 * events the previous registration had recorded (twice the kernels it
 * timed).  Not for calls that are being captured into a graph. */
int32_t mla_debug_set_launch_events(void* const* events, int32_t n);

/* Test hooks for the decode family's one-launch finish + kv_b_proj (taken
 * when the device holds that launch's whole grid at once).  Its workgroups
 * wait, with a bounded number of polls, for latent rows that other
 * workgroups of the same launch finish; a workgroup that runs out of polls
 * rebuilds the rows itself from the split-K partials of the previous launch
 * (the same arithmetic in the same order, so the output bits do not change)
 * and counts one fallback.
 *
 * mla_debug_set_handoff_spin sets the bound on the polls for later calls in
 * this process (0: never wait, every workgroup rebuilds its rows; a
 * negative value restores the default) and returns the previous setting
 * (-1 for the default).  Not for concurrent use.
 *
 * mla_debug_handoff_fallbacks returns the current device's count of such
 * fallbacks since the last reset (synchronises with the device; -1 on a HIP
 * error) and clears it when reset != 0. */
int64_t mla_debug_set_handoff_spin(int64_t limit);
int64_t mla_debug_handoff_fallbacks(int reset);

/* Static, human-readable name of a status code. */
const char* mla_status_string(mla_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLAPROLOG_H */
