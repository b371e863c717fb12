// Weight-streaming gfx950 kernels of the MLA KV prolog for short token
// batches (decode: a few sequences x one or two query tokens).
//
// At decode sizes the prolog is bound by reading the two weight matrices
// once from HBM and by the latency of doing so, so the kernels are shaped
// around the weight stream:
//   dec_kv_a       kv_a_proj: W_kv_a cut into 64-column slabs x K ranges of
//                  KW rows, one workgroup each (two, each with half the
//                  token tiles, when the blocks alone would leave most of the
//                  chip idle), writing split-K partial sums P[s][t][576]
//   dec_fin_kv_b   the finish (sum of the partials, RMSNorm -> compressed_kv,
//                  RoPE -> k_pe) fused into kv_b_proj: items of (16-token
//                  tile, 64-column slab of W_kv_b over the full K = 512), one
//                  workgroup each; the first workgroups also finish one token
//                  each and hand the latent rows to the others (see the
//                  kernel)
//   dec_finish, dec_kv_b   the same two steps as separate launches, for
//                  shapes with more kv_b_proj items than fit on the chip at
//                  once
// Each workgroup issues all of its global loads before its first wait (16
// bytes per lane, 128 contiguous bytes per weight row; out-of-range rows are
// clamped and zeroed when stored, never branched around), stages the weight
// slab and the activation rows in LDS once, and multiplies with
// v_mfma_f32_16x16x32 (tokens as M); wave w owns slab columns 16w..16w+15
// over the whole K range, so no cross-wave reduction is needed.
//
// Steps as in the DeepSeek-V2-Lite-Chat MLA KV Prolog migration guide
// (dpshk.com), sections "Background" and "Source-level principle"; RoPE in
// the rotate-half x*cos + x_rot*sin form of its "Precision verification".
#include <atomic>

#include "mla_common.h"

namespace mla {

template <int E>
__device__ __forceinline__ f4_t mfma_f(u4_t a, u4_t b, f4_t c) {
    if constexpr (E == kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                      __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a),
                                                       __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
}

constexpr int kSlabW = 64;                 // weight slab width (columns)
constexpr int kSlabsA = kN1 / kSlabW;      // 9 kv_a_proj slabs
constexpr int kPitch = kSlabW + 8;         // LDS row pitch of a staged slab (halves)

// ---------------------------------------------------------------------------
// Slab staging.  Rows [k0, k0 + 32*NR) of a 64-column slab starting at
// column n0 of a row-major [K][ld] matrix: thread i loads 16 bytes (8
// columns) of rows i/8 + 32 r, r < NR.  With CHECK, rows at or past kmax are
// loaded from row kmax - 1 and zeroed when stored (no branch around a load,
// so every load is in flight before the first wait).  stage_store writes
// them to LDS as [row][kPitch].
// ---------------------------------------------------------------------------
template <int NR, bool CHECK = true>
__device__ __forceinline__ void stage_load(u4_t (&v)[NR], const uint16_t* W, int64_t ld, int k0,
                                           int kmax, int n0) {
    const int q = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        int k = k0 + r0 + 32 * r;
        if (CHECK) k = k < kmax ? k : kmax - 1;
        // weights are read once per call: streaming (non-temporal) loads
        v[r] = __builtin_nontemporal_load((const u4_t*)(W + (int64_t)k * ld + n0 + 8 * q));
    }
}
template <int NR, bool CHECK = true>
__device__ __forceinline__ void stage_store(const u4_t (&v)[NR], uint16_t* lds, int k0 = 0,
                                            int kmax = 0) {
    const int q = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const bool ok = !CHECK || k0 + r0 + 32 * r < kmax;
        *(u4_t*)(lds + (r0 + 32 * r) * kPitch + 8 * q) = ok ? v[r] : u4_t{0u, 0u, 0u, 0u};
    }
}
// MFMA B operand from a staged slab: lane (16 g + c) gets column c0 + c,
// rows kb + 8g .. kb + 8g + 7.  Two transposing LDS reads
// (ds_read_b64_tr_b16): in each 16-lane group, lane s points at row
// k + s/4, columns c0 + 4 (s % 4) .. +3, and lane j receives rows k .. k+3
// of column c0 + j.
typedef short v4s_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
    const v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s_t*)(p));
    return __builtin_bit_cast(uint2, r);
}
__device__ __forceinline__ u4_t lds_col8(const uint16_t* lds, int kb, int c0) {
    const int lane = threadIdx.x & 63, g = lane >> 4, sl = lane & 15;
    const uint16_t* p = lds + (kb + 8 * g + (sl >> 2)) * kPitch + c0 + 4 * (sl & 3);
    const uint2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * kPitch);
    return u4_t{lo.x, lo.y, hi.x, hi.y};
}

// ---------------------------------------------------------------------------
// Activation rows: rows [0, 16 NT) x columns [k0, k0 + KA) of a row-major
// [rows][ld] matrix, loaded 16 bytes per chunk by the whole workgroup and
// kept in LDS as [row][KA + 8]; rows >= nrows and columns >= kmax are stored
// as zeros (their loads read a valid chunk instead: nrows >= 1, kmax a
// multiple of 8).
// The +8 pitch puts the 16 rows an MFMA operand read touches on distinct
// banks.  Each wave then reads its A operands (lane 16g + c: row c, 8
// consecutive K at 8g) with one 16-byte LDS read.
// ---------------------------------------------------------------------------
template <int NT, int KA>
struct ARows {
    static constexpr int kChunks = NT * 16 * KA / 8;
    static constexpr int kPer = (kChunks + 255) / 256;
    static constexpr int kPitchA = KA + 8;
};
template <int NT, int KA, int NP>
__device__ __forceinline__ void arows_load(u4_t (&v)[NP], const uint16_t* A, int64_t ld, int nrows,
                                           int k0, int kmax) {
    static_assert(NP == ARows<NT, KA>::kPer, "chunks per thread");
    constexpr int CPR = KA / 8;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int q = threadIdx.x + 256 * u;
        int row = q / CPR, k = k0 + 8 * (q % CPR);
        row = row < nrows ? row : nrows - 1;
        k = k < kmax ? k : kmax - 8;
        v[u] = *(const u4_t*)(A + (int64_t)row * ld + k);
    }
}
template <int NT, int KA, int NP>
__device__ __forceinline__ void arows_store(const u4_t (&v)[NP], uint16_t* lds, int nrows, int k0,
                                            int kmax) {
    static_assert(NP == ARows<NT, KA>::kPer, "chunks per thread");
    constexpr int CPR = KA / 8;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int q = threadIdx.x + 256 * u;
        const int row = q / CPR, k = k0 + 8 * (q % CPR);
        if (q < ARows<NT, KA>::kChunks)
            *(u4_t*)(lds + row * ARows<NT, KA>::kPitchA + 8 * (q % CPR)) =
                (row < nrows && k < kmax) ? v[u] : u4_t{0u, 0u, 0u, 0u};
    }
}

// acc[tt] += A rows 16 tt .. 16 tt + 15 (LDS, pitch AP) x slab columns
// 16 w .. 16 w + 15 (w = this wave) over the first kv rows (kv a multiple
// of 32).  The weight operand is read once per 32-row chunk and reused by
// every token tile.
template <int E, int NT, int KA>
__device__ __forceinline__ void slab_mma(const uint16_t* ldsW, const uint16_t* ldsA, int kv,
                                         f4_t (&acc)[NT]) {
    constexpr int AP = ARows<NT, KA>::kPitchA;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ch = 0; ch < KA / 32; ++ch) {
        if (ch * 32 >= kv) break;
        const u4_t bw = lds_col8(ldsW, ch * 32, wave * 16);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const u4_t a = *(const u4_t*)(ldsA + (tt * 16 + c) * AP + ch * 32 + 8 * g);
            acc[tt] = mfma_f<E>(a, bw, acc[tt]);
        }
    }
}

// Work item of a workgroup: workgroup b runs on XCD b % 8, and XCD x takes
// the contiguous item range [x per, (x + 1) per), so items with neighbouring
// indices share an XCD and its L2.  Returns -1 for the padding workgroups.
__device__ __forceinline__ int xcd_item(int nitems) {
    const int per = (nitems + 7) / 8;
    const int it = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    return it < nitems ? it : -1;
}

// ---------------------------------------------------------------------------
// kv_a_proj partial of (split s, slab, token group tg) over K rows
// [s KW, s KW + KW) for tokens [16 NT tg, 16 NT (tg + 1)) of T; item =
// NG (9 s + slab) + tg, so each XCD reads a contiguous range of X's columns
// and the token groups of one weight block share an XCD (and its L2).
// grid = 8 ceil(9 S NG / 8), 256 threads; NG = ceil(T / (16 NT)).
// ---------------------------------------------------------------------------
template <int E, int NT, int KW>
__global__ __launch_bounds__(256) void dec_kv_a_kernel(const uint16_t* __restrict__ X,
                                                       const uint16_t* __restrict__ Wa, int T,
                                                       int H, int S, float* __restrict__ P,
                                                       uint16_t* __restrict__ ckv, int NG) {
    __shared__ __align__(16) uint16_t ldsW[KW * kPitch];
    __shared__ __align__(16) uint16_t ldsA[NT * 16 * ARows<NT, KW>::kPitchA];
    // compressed_kv rows start out as the "not written yet" pattern that the
    // fused finish + kv_b_proj launch which follows waits on
    for (int row = blockIdx.x; row < T; row += gridDim.x)
        if (threadIdx.x < kR / 8)
            *(u4_t*)(ckv + (int64_t)row * kR + 8 * threadIdx.x) = u4_t{~0u, ~0u, ~0u, ~0u};
    const int item = xcd_item(kSlabsA * S * NG);
    if (item < 0) return;
    const int tg = item % NG, blk = item / NG;
    const int s = blk / kSlabsA, slab = blk % kSlabsA;
    const int k0 = s * KW;
    const int t0 = tg * 16 * NT;
    const int nt = T - t0 < 16 * NT ? T - t0 : 16 * NT;  // >= 1
    u4_t v[KW / 32];
    u4_t a[ARows<NT, KW>::kPer];
    stage_load<KW / 32>(v, Wa, kN1, k0, H, slab * kSlabW);
    arows_load<NT, KW>(a, X + (int64_t)t0 * H, H, nt, k0, H);
    stage_store<KW / 32>(v, ldsW, k0, H);
    arows_store<NT, KW>(a, ldsA, nt, k0, H);
    __syncthreads();
    f4_t acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f4_t{0.f, 0.f, 0.f, 0.f};
    slab_mma<E, NT, KW>(ldsW, ldsA, H - k0, acc);
    // lane 16g + c holds tokens 16 tt + 4g + i of slab column 16 wave + c
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    float* Ps = P + (int64_t)s * T * kN1 + slab * kSlabW + wave * 16 + c;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + tt * 16 + 4 * g + i;
            if (t < T) Ps[(int64_t)t * kN1] = acc[tt][i];
        }
}

// ---------------------------------------------------------------------------
// Finish of kv_a_proj for token t, by one workgroup.  Wave w sums splits
// w, w+4, ... of the partials; wave 0 adds the four wave sums (fixed order),
// then lane l owns latent columns 8l..8l+7 and rope column l:
//   y     = c / sqrt(sum(c^2)/512 + eps) * gamma      -> compressed_kv
//   k_pe  = rotate-half RoPE of p at the token's position
// With COH the compressed_kv row is written with device-coherent stores
// (through to memory), for workgroups on other XCDs that read it in the same
// launch.  fred: 4 x (576 + 4) floats of LDS.
// ---------------------------------------------------------------------------

constexpr int kFredPitch = kN1 + 4;

// Partial sums of token t held by one wave: splits s0, s0 + 4, s0 + 8,
// s0 + 12; those at or past S are loaded from split S - 1 (so that every
// load is unconditional and all four are in flight together) and dropped
// when added.
struct FinPart {
    f4_t v0[4], v1[4];
    float vp[4];
    int s0;
    u4_t gm;      // gamma[8 lane .. 8 lane + 7]
    int32_t pos;  // the token's position
    double freq;  // RoPE frequency of rope column lane
    int64_t slot; // the token's paged-cache slot (-1 without a cache)
};
__device__ __forceinline__ void fin_load(FinPart& r, const float* __restrict__ P, int S, int T,
                                         int t, int s0) {
    const int lane = threadIdx.x & 63;
    r.s0 = s0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int sp = s0 + 4 * u < S ? s0 + 4 * u : S - 1;
        const float* row = P + ((int64_t)sp * T + t) * kN1;
        // partials are read once: streaming loads
        r.v0[u] = __builtin_nontemporal_load((const f4_t*)(row + 8 * lane));
        r.v1[u] = __builtin_nontemporal_load((const f4_t*)(row + 8 * lane + 4));
        r.vp[u] = __builtin_nontemporal_load(row + kR + lane);
    }
}
__device__ __forceinline__ void fin_load_aux(FinPart& r, const uint16_t* __restrict__ gamma,
                                             const int32_t* __restrict__ pos, const RopeTab& rt,
                                             const CacheOut& co, int t) {
    const int lane = threadIdx.x & 63;
    r.gm = *(const u4_t*)(gamma + 8 * lane);
    r.pos = pos[t];
    r.freq = rt.f[lane & 31];
    r.slot = co.slots != nullptr ? co.slots[t] : -1;
}
__device__ __forceinline__ void fin_add(const FinPart& r, int S, f4_t& c0, f4_t& c1, float& p) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (r.s0 + 4 * u < S) {
            c0 += r.v0[u];
            c1 += r.v1[u];
            p += r.vp[u];
        }
    }
}

// The partial sums of token t, wave w holding splits w, w + 4, ... (the
// first 16 already loaded in r): each wave adds its splits, then leaves its
// sums in its fred row; ends with a barrier.
__device__ __forceinline__ void fin_reduce(FinPart& r, const float* __restrict__ P, int S, int T,
                                           int t, float* fred) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    f4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    float p = 0.f;
    fin_add(r, S, c0, c1, p);
    for (int s0 = wave + 16; s0 < S; s0 += 16) {
        fin_load(r, P, S, T, t, s0);
        fin_add(r, S, c0, c1, p);
    }
    float* fw = fred + wave * kFredPitch;
    *(f4_t*)&fw[8 * lane] = c0;
    *(f4_t*)&fw[8 * lane + 4] = c1;
    fw[kR + lane] = p;
    __syncthreads();
}

// The normalised latent of the token whose four wave sums are in fred, for
// lane l's columns 8l .. 8l + 7 (wave 0 calls it): the sums added in a fixed
// order, then RMSNorm and gamma, rounded to E.
// No contraction, so that every inlined copy (the producer's and the
// fallback's) is the same sequence of fp32 operations.
template <int E>
__device__ __forceinline__ u4_t fin_latent(const float* fred, const u4_t gm, float eps) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const float* f0 = fred;
    const float* f1 = fred + kFredPitch;
    const float* f2 = fred + 2 * kFredPitch;
    const float* f3 = fred + 3 * kFredPitch;
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        c[i] = (f0[8 * lane + i] + f1[8 * lane + i]) + (f2[8 * lane + i] + f3[8 * lane + i]);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += c[i] * c[i];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)kR + eps);
    return rms_scale8<E>(c, inv, gm);
}

// Finish of token t given the wave's partials of its first 16 splits, gamma,
// the position and the RoPE frequency in r.  After the partials are summed,
// wave 0 normalises the latent and wave 1 rotates the rope part.
template <int E, bool COH>
__device__ __forceinline__ void finish_token_from(FinPart& r, const float* __restrict__ P, int S,
                                                  int T, int t, float eps,
                                                  uint16_t* __restrict__ ckv,
                                                  uint16_t* __restrict__ kpe, const CacheOut& co,
                                                  float* fred) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    fin_reduce(r, P, S, T, t, fred);
    if (wave == 0) {
        const u4_t o = fin_latent<E>(fred, r.gm, eps);
        uint16_t* dst = ckv + (int64_t)t * kR + 8 * lane;
        if constexpr (COH) {
            store_coherent64(dst, (uint64_t)o[0] | ((uint64_t)o[1] << 32));
            store_coherent64(dst + 4, (uint64_t)o[2] | ((uint64_t)o[3] << 32));
        } else {
            *(u4_t*)dst = o;
        }
        if (cache_slot_ok(co, r.slot))  // the paged cache: [latent | rope key] in the slot
            __builtin_nontemporal_store(o, (u4_t*)(co.cache + r.slot * (kR + kDR) + 8 * lane));
    } else if (wave == 1) {
        const float* f0 = fred;
        const float* f1 = fred + kFredPitch;
        const float* f2 = fred + 2 * kFredPitch;
        const float* f3 = fred + 3 * kFredPitch;
        float cs, sn;
        rope_cos_sin(r.pos, r.freq, cs, sn);
        const float q = (f0[kR + lane] + f1[kR + lane]) + (f2[kR + lane] + f3[kR + lane]);
        const float partner = __shfl_xor(q, 32, 64);
        const uint16_t ko = f32_to_st<E>(rope_rotate(q, partner, cs, sn, lane < 32));
        kpe[(int64_t)t * kDR + lane] = ko;
        if (cache_slot_ok(co, r.slot))
            __builtin_nontemporal_store(ko, co.cache + r.slot * (kR + kDR) + kR + lane);
    }
}

template <int E, bool COH>
__device__ __forceinline__ void finish_token(const float* __restrict__ P, int S, int T, int t,
                                             const uint16_t* __restrict__ gamma,
                                             const int32_t* __restrict__ pos, float eps,
                                             const RopeTab& rt, uint16_t* __restrict__ ckv,
                                             uint16_t* __restrict__ kpe, const CacheOut& co,
                                             float* fred) {
    FinPart r;
    fin_load(r, P, S, T, t, threadIdx.x >> 6);
    fin_load_aux(r, gamma, pos, rt, co, t);
    finish_token_from<E, COH>(r, P, S, T, t, eps, ckv, kpe, co, fred);
}

// one workgroup per token
template <int E>
__global__ __launch_bounds__(256) void dec_finish_kernel(const float* __restrict__ P, int S, int T,
                                                         const uint16_t* __restrict__ gamma,
                                                         const int32_t* __restrict__ pos,
                                                         float eps, RopeTab rt,
                                                         uint16_t* __restrict__ ckv,
                                                         uint16_t* __restrict__ kpe,
                                                         CacheOut co) {
    __shared__ __align__(16) float fred[4 * kFredPitch];
    finish_token<E, false>(P, S, T, blockIdx.x, gamma, pos, eps, rt, ckv, kpe, co, fred);
}

// ---------------------------------------------------------------------------
// kv_b_proj.  Work item = (64-column slab of W_kv_b over the full K = 512,
// group of NT token tiles); a slab is 64 consecutive entries of k_nope or of
// value of one head.  Items of one slab are adjacent (group fastest), so
// they share an XCD and read the slab through its L2.
// ---------------------------------------------------------------------------
template <int E, int NT>
__global__ __launch_bounds__(256) void dec_kv_b_kernel(const uint16_t* __restrict__ Y,
                                                       const uint16_t* __restrict__ Wb, int T,
                                                       int N2, uint16_t* __restrict__ k_nope,
                                                       uint16_t* __restrict__ value) {
    __shared__ __align__(16) uint16_t ldsW[kR * kPitch];
    __shared__ __align__(16) uint16_t ldsA[NT * 16 * ARows<NT, kR>::kPitchA];
    const int nh = N2 / kHeadW;
    const int ngrp = (T + 16 * NT - 1) / (16 * NT);
    const int item = xcd_item((N2 / kSlabW) * ngrp);
    if (item < 0) return;
    const int slab = item / ngrp, t0 = (item % ngrp) * 16 * NT;
    u4_t v[kR / 32];
    u4_t a[ARows<NT, kR>::kPer];
    stage_load<kR / 32, false>(v, Wb, N2, 0, kR, slab * kSlabW);
    arows_load<NT, kR>(a, Y + (int64_t)t0 * kR, kR, T - t0, 0, kR);
    stage_store<kR / 32, false>(v, ldsW);
    arows_store<NT, kR>(a, ldsA, T - t0, 0, kR);
    __syncthreads();
    f4_t acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f4_t{0.f, 0.f, 0.f, 0.f};
    slab_mma<E, NT, kR>(ldsW, ldsA, kR, acc);
    // lane 16g + c holds tokens t0 + 16 tt + 4g + i of slab column 16 wave + c
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    const int n = slab * kSlabW + wave * 16 + c;
    const int h = n >> 8, sl = n & 255;
    uint16_t* dst = ((sl < kDN) ? k_nope : value) + (int64_t)h * kDN + (sl & 127);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = t0 + tt * 16 + 4 * g + i;
            if (tok < T) __builtin_nontemporal_store(f32_to_st<E>(acc[tt][i]), dst + (int64_t)tok * nh * kDN);
        }
}

// ---------------------------------------------------------------------------
// Finish and kv_b_proj in one launch, for grids that fit on the device at
// once (the host checks the CU count and this kernel's occupancy).  Every
// workgroup first issues the loads of its W_kv_b slab; workgroup b then
// finishes tokens b, b + G, ... (G = grid size), writing each compressed_kv
// row with device-coherent 8-byte stores.  The kv_a launch before it filled
// those rows with all-ones halves, a NaN pattern that the finish of finite
// inputs never produces, so a row chunk is known to be final once it holds
// no all-ones half (8-byte coherent stores and loads are single-copy
// atomic).  Each workgroup stages its slab, then reads its tile's rows with
// coherent loads, re-reading the chunks that still hold the pattern.
//
// The wait is bounded by spin_limit polls.  If a row is still missing then
// (its producer was not resident, say, because other work held CUs), the
// workgroup rebuilds every row of its tile itself from the split-K partials
// P, which the previous launch completed, with the producer's own arithmetic
// in the producer's order: the result is the same bits, only later.  Each
// such fallback adds one to g_handoff_fallbacks (a count the host can read).
// ---------------------------------------------------------------------------
constexpr uint32_t kSpinDefault = 256;
__device__ unsigned int g_handoff_fallbacks = 0;

__device__ __forceinline__ bool has_unset_half(uint64_t x) {
    return ((x & 0xFFFFull) == 0xFFFFull) || (((x >> 16) & 0xFFFFull) == 0xFFFFull) ||
           (((x >> 32) & 0xFFFFull) == 0xFFFFull) || ((x >> 48) == 0xFFFFull);
}

template <int E>
__global__ __launch_bounds__(256) void dec_fin_kv_b_kernel(
    const float* __restrict__ P, int S, int T, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ pos, float eps, RopeTab rt, const uint16_t* __restrict__ Wb,
    int N2, uint16_t* ckv, uint16_t* __restrict__ kpe, uint16_t* __restrict__ k_nope,
    uint16_t* __restrict__ value, CacheOut co, uint32_t spin_limit) {
    constexpr int AP = ARows<1, kR>::kPitchA;
    __shared__ __align__(16) uint16_t ldsW[kR * kPitch];
    __shared__ __align__(16) uint16_t ldsA[16 * AP];
    __shared__ __align__(16) float fred[4 * kFredPitch];  // the finish's reduction buffer
    const int nh = N2 / kHeadW;
    const int ntile = (T + 15) / 16;
    const int item = xcd_item((N2 / kSlabW) * ntile);
    // the first token to finish: its partials are requested before the slab,
    // so that the finish does not wait for the slab's loads (the slab loads
    // are unconditional for the same reason: padding workgroups read slab 0)
    const int t1 = blockIdx.x;
    const int n0 = (item >= 0 ? item / ntile : 0) * kSlabW;
    u4_t v[kR / 32];
    if (t1 < T) {
        FinPart r;
        fin_load(r, P, S, T, t1, threadIdx.x >> 6);
        fin_load_aux(r, gamma, pos, rt, co, t1);
        stage_load<kR / 32, false>(v, Wb, N2, 0, kR, n0);
        finish_token_from<E, true>(r, P, S, T, t1, eps, ckv, kpe, co, fred);
    } else {
        stage_load<kR / 32, false>(v, Wb, N2, 0, kR, n0);
    }
    for (int t = t1 + (int)gridDim.x; t < T; t += gridDim.x) {
        __syncthreads();  // the reduction buffer is free again
        finish_token<E, true>(P, S, T, t, gamma, pos, eps, rt, ckv, kpe, co, fred);
    }
    if (item < 0) return;
    const int slab = item / ntile, t0 = (item % ntile) * 16;
    const int nrows = T - t0 < 16 ? T - t0 : 16;
    stage_store<kR / 32, false>(v, ldsW);
    // the tile's compressed_kv rows: 16 rows x 128 eight-byte chunks
    uint64_t y[8];
    uint32_t pend = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int row = (threadIdx.x + 256 * u) >> 7;
        y[u] = 0ull;
        if (row < nrows) pend |= 1u << u;
    }
    for (uint32_t it = 0; pend != 0u && it < spin_limit; ++it) {
        if (it != 0) __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = threadIdx.x + 256 * u, row = q >> 7, col = (q & 127) * 4;
            if (pend & (1u << u)) y[u] = load_coherent64(ckv + (int64_t)(t0 + row) * kR + col);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if ((pend & (1u << u)) && !has_unset_half(y[u])) pend &= ~(1u << u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int q = threadIdx.x + 256 * u, row = q >> 7, col = (q & 127) * 4;
        *(uint64_t*)(ldsA + row * AP + col) = y[u];
    }
    if (__syncthreads_or(pend != 0u)) {
        // the hand-off ran out of polls: rebuild the tile's rows from P
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (threadIdx.x == 0) atomicAdd(&g_handoff_fallbacks, 1u);
        const u4_t gm = *(const u4_t*)(gamma + 8 * lane);
        for (int row = 0; row < nrows; ++row) {
            FinPart r;
            fin_load(r, P, S, T, t0 + row, wave);
            fin_reduce(r, P, S, T, t0 + row, fred);
            if (wave == 0) *(u4_t*)(ldsA + row * AP + 8 * lane) = fin_latent<E>(fred, gm, eps);
            __syncthreads();  // fred is reused by the next row
        }
    }
    __syncthreads();
    f4_t acc[1] = {f4_t{0.f, 0.f, 0.f, 0.f}};
    slab_mma<E, 1, kR>(ldsW, ldsA, kR, acc);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    const int n = slab * kSlabW + wave * 16 + c;
    const int h = n >> 8, sl = n & 255;
    uint16_t* dst = ((sl < kDN) ? k_nope : value) + (int64_t)h * kDN + (sl & 127);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 4 * g + i;
        if (tok < T) __builtin_nontemporal_store(f32_to_st<E>(acc[0][i]), dst + (int64_t)tok * nh * kDN);
    }
}

// ---------------------------------------------------------------------------
// W8A8 at decode sizes (up to 16 tokens, one token tile): the finish fused
// into kv_b_proj, as dec_fin_kv_b_kernel.  Items are 64-column slabs of the
// int8 W_kv_b over K = 512 (32 KB each).  Workgroup b < T first finishes
// token b: its four waves add the int32 split-K partials (splits w, w + 4,
// ...; exact in any order) and wave 0 forms the latent codes, their scale
// and the RMS factor (w8_latent), compressed_kv, k_pe and the cache, the
// codes and both scales through device-coherent stores.  The activation
// quantiser of the same call filled every code row with 0x80 bytes (a code
// the quantisers never produce) and both scales with all-ones words, so an
// 8-byte chunk of codes or a scale is final once it holds no such byte or
// word.  Every workgroup stages its slab, polls its tile's codes and scales
// with coherent loads (bounded), multiplies with v_mfma_i32_16x16x64_i8
// (tokens as M; wave w owns slab columns 16 w .. 16 w + 15, weight operands
// from two transposing LDS reads), and writes ((acc * (sz * inv)) * s_b)
// rounded to bf16.  A workgroup that runs out of polls rebuilds its tile's
// codes and scales from the partials itself (the same operations, so the
// same bits) and counts one fallback.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool has_0x80_byte(uint64_t x) {
    const uint64_t y = x ^ 0x8080808080808080ull;  // a 0x80 byte becomes 0
    return ((y - 0x0101010101010101ull) & ~y & 0x8080808080808080ull) != 0ull;
}

// int32 sums of token t's split-K partials: wave w adds splits w, w + 4,
// ... (NPW loads in flight; those past S re-read split S - 1 and are not
// added).  w8_parts_load issues the loads; w8_parts_sum adds them, waves
// 1..3 leave theirs in red, and after the barrier wave 0 holds the total
// (the caller synchronises before red is reused).
template <int NPW>
struct W8Parts {
    i4_t v0[NPW], v1[NPW];
    int pv[NPW];
};
template <int NPW>
__device__ __forceinline__ void w8_parts_load(W8Parts<NPW>& r, const int32_t* __restrict__ P,
                                              int S, int T, int t) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        const int s = wave + 4 * j < S ? wave + 4 * j : S - 1;
        const int32_t* row = P + ((int64_t)s * T + t) * kN1;
        r.v0[j] = __builtin_nontemporal_load((const i4_t*)(row + 8 * lane));
        r.v1[j] = __builtin_nontemporal_load((const i4_t*)(row + 8 * lane + 4));
        r.pv[j] = __builtin_nontemporal_load(row + kR + lane);
    }
}
template <int NPW>
__device__ __forceinline__ void w8_parts_sum(const W8Parts<NPW>& r, int S, int (*red)[64 * 9],
                                             int (&a)[8], int& ap) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = 0;
    ap = 0;
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        if (wave + 4 * j < S) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] += r.v0[j][i];
                a[4 + i] += r.v1[j][i];
            }
            ap += r.pv[j];
        }
    }
    if (wave > 0) {
        int* d = red[wave - 1] + lane * 9;
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = a[i];
        d[8] = ap;
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w) {
            const int* d = red[w] + lane * 9;
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] += d[i];
            ap += d[8];
        }
    }
}

// Wave 0's per-token inputs of the W8A8 finish.
struct W8Aux {
    int pt;
    int64_t slot;
    float sxt, wap;
    f4_t wa0, wa1;
    u4_t gm;
};
__device__ __forceinline__ W8Aux w8_aux_load(const float* __restrict__ sx,
                                             const float* __restrict__ swa,
                                             const uint16_t* __restrict__ gamma,
                                             const int32_t* __restrict__ pos, const CacheOut& co,
                                             int t) {
    const int lane = threadIdx.x & 63;
    W8Aux x;
    x.pt = pos[t];
    x.slot = co.slots != nullptr ? co.slots[t] : -1;
    x.sxt = sx[t];
    x.wa0 = *(const f4_t*)(swa + 8 * lane);
    x.wa1 = *(const f4_t*)(swa + 8 * lane + 4);
    x.wap = swa[kR + lane];
    x.gm = *(const u4_t*)(gamma + 8 * lane);
    return x;
}

typedef int v2i_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_tr8_w(const int8_t* p) {
    const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i_t*)(p));
    return __builtin_bit_cast(uint2, r);
}

__device__ unsigned int g_handoff_fallbacks_w8 = 0;

template <int NPW>
__global__ __launch_bounds__(256) void dec_fin_kv_b_w8_kernel(
    const int32_t* __restrict__ P, int S, int T, const float* __restrict__ sx,
    const float* __restrict__ swa, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ pos, float eps, RopeTab rt, const int8_t* __restrict__ Wqb,
    const float* __restrict__ swb, int N2, int8_t* QZ, float* sz, float* inv,
    uint16_t* __restrict__ ckv, uint16_t* __restrict__ kpe, uint16_t* __restrict__ k_nope,
    uint16_t* __restrict__ value, int32_t* __restrict__ dbg1, int32_t* __restrict__ dbg2,
    int64_t dbg_begin, int64_t dbg_rows, CacheOut co, uint32_t spin_limit) {
    constexpr int WP = kSlabW + 16;  // LDS pitch of a staged slab row (bytes)
    constexpr int AP = kR + 16;      // LDS pitch of a latent code row (bytes)
    __shared__ __align__(16) int8_t ldsW[kR * WP];
    __shared__ __align__(16) int8_t ldsA[16 * AP];
    __shared__ __align__(16) int red[3][64 * 9];
    __shared__ float lsz[16], linv[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int nh = N2 / kHeadW;
    const int item = xcd_item(N2 / kSlabW);
    // the slab: rows k = (tid >> 2) + 64 u, 16-byte chunk tid & 3; requested
    // after the finishing workgroup's partials, so that the finish does not
    // wait for the slab (padding workgroups read slab 0)
    const int n0 = (item >= 0 ? item : 0) * kSlabW;
    u4_t v[8];
    auto slab_load = [&]() {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = __builtin_nontemporal_load(
                (const u4_t*)(Wqb + (int64_t)((tid >> 2) + 64 * u) * N2 + n0 + 16 * (tid & 3)));
    };
    // tokens b, b + G, ... (G = grid size) are finished by workgroup b
    const int t1 = blockIdx.x;
    if (t1 < T) {
        W8Aux x = {};
        if (wave == 0) x = w8_aux_load(sx, swa, gamma, pos, co, t1);
        W8Parts<NPW> r;
        w8_parts_load(r, P, S, T, t1);
        slab_load();
        int a[8], ap;
        w8_parts_sum(r, S, red, a, ap);
        if (wave == 0)
            w8_finish_token<true>(a, ap, t1, x.pt, x.slot, x.sxt, x.wa0, x.wa1, x.wap, x.gm, eps,
                                  rt, QZ, sz, inv, ckv, kpe, dbg1, dbg_begin, dbg_rows, co);
    } else {
        slab_load();
    }
    for (int t = t1 + (int)gridDim.x; t < T; t += gridDim.x) {
        __syncthreads();  // red is free again
        W8Aux x = {};
        if (wave == 0) x = w8_aux_load(sx, swa, gamma, pos, co, t);
        W8Parts<NPW> r;
        w8_parts_load(r, P, S, T, t);
        int a[8], ap;
        w8_parts_sum(r, S, red, a, ap);
        if (wave == 0)
            w8_finish_token<true>(a, ap, t, x.pt, x.slot, x.sxt, x.wa0, x.wa1, x.wap, x.gm, eps,
                                  rt, QZ, sz, inv, ckv, kpe, dbg1, dbg_begin, dbg_rows, co);
    }
    if (item < 0) return;
#pragma unroll
    for (int u = 0; u < 8; ++u)
        *(u4_t*)(ldsW + ((tid >> 2) + 64 * u) * WP + 16 * (tid & 3)) = v[u];
    // the tile's codes (16 rows x 64 eight-byte chunks) and scales
    const int nrows = T < 16 ? T : 16;
    uint64_t y[4];
    uint32_t pend = 0, sc = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        y[u] = 0ull;
        if (((tid + 256 * u) >> 6) < nrows) pend |= 1u << u;
    }
    const bool has_sc = tid < 32 && (tid & 15) < nrows;
    if (has_sc) pend |= 1u << 4;
    for (uint32_t it = 0; pend != 0u && it < spin_limit; ++it) {
        if (it != 0) __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = tid + 256 * u;
            if (pend & (1u << u)) y[u] = load_coherent64(QZ + (int64_t)(q >> 6) * kR + 8 * (q & 63));
        }
        if (pend & (1u << 4))
            sc = load_coherent32((tid < 16 ? (const void*)(sz + tid) : (const void*)(inv + tid - 16)));
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if ((pend & (1u << u)) && !has_0x80_byte(y[u])) pend &= ~(1u << u);
        if ((pend & (1u << 4)) && sc != ~0u) pend &= ~(1u << 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int q = tid + 256 * u;
        *(uint64_t*)(ldsA + (q >> 6) * AP + 8 * (q & 63)) = y[u];
    }
    if (tid < 32) (tid < 16 ? lsz : linv)[tid & 15] = __builtin_bit_cast(float, sc);
    if (__syncthreads_or(pend != 0u)) {
        // the hand-off ran out of polls: rebuild the tile's codes and
        // scales from the partials
        if (tid == 0) atomicAdd(&g_handoff_fallbacks_w8, 1u);
        const f4_t wa0 = *(const f4_t*)(swa + 8 * lane), wa1 = *(const f4_t*)(swa + 8 * lane + 4);
        const u4_t gm = *(const u4_t*)(gamma + 8 * lane);
        for (int row = 0; row < nrows; ++row) {
            W8Parts<NPW> r;
            w8_parts_load(r, P, S, T, row);
            int a[8], ap;
            w8_parts_sum(r, S, red, a, ap);
            if (wave == 0) {
                const W8Latent L = w8_latent(a, sx[row], wa0, wa1, gm, eps);
                *(u2_t*)(ldsA + row * AP + 8 * lane) = L.q;
                if (lane == 0) {
                    lsz[row] = L.sz;
                    linv[row] = L.inv;
                }
            }
            __syncthreads();  // red is reused by the next row
        }
    }
    __syncthreads();
    // acc: tokens 4 g + i (rows of the tile) of slab column 16 wave + l16
    i4_t acc = {0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < kR / 64; ++ks) {
        const u4_t fa = *(const u4_t*)(ldsA + l16 * AP + ks * 64 + 16 * g);
        const int k = ks * 64 + g * 16 + (l16 >> 1);
        const int colb = wave * 16 + 8 * (l16 & 1);
        const uint2 lo = lds_tr8_w(ldsW + k * WP + colb);
        const uint2 hi = lds_tr8_w(ldsW + (k + 8) * WP + colb);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, fa),
                                                    __builtin_bit_cast(i4_t, u4_t{lo.x, lo.y, hi.x, hi.y}),
                                                    acc, 0, 0, 0);
    }
    const int n = n0 + wave * 16 + l16;
    const int h = n >> 8, sl = n & 255;
    uint16_t* dst = ((sl < kDN) ? k_nope : value) + (int64_t)h * kDN + (sl & 127);
    const float cs = swb[n];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = 4 * g + i;
        if (tok < nrows) {
            const float f = ((float)acc[i] * (lsz[tok] * linv[tok])) * cs;
            __builtin_nontemporal_store(f32_to_bf16(f), dst + (int64_t)tok * nh * kDN);
            if (dbg2 != nullptr && tok >= dbg_begin && tok < dbg_begin + dbg_rows)
                dbg2[(tok - dbg_begin) * (int64_t)N2 + n] = acc[i];
        }
    }
}

// ---------------------------------------------------------------------------
// W8A8 kv_a_proj for a few tokens (T <= 8) with the activation quantiser
// folded in.  Work items are (split s, 64-column slab of Wq_kv_a over the
// split's kw <= KW rows), split-major as in dec_kv_a.  Each workgroup reads its
// tokens' whole hidden rows (a few tens of KB, served from L2 after the
// first workgroups) for their maxima, quantises its own K range of them
// with the quantiser's operations (quant8: the same codes), stages the
// codes and the weight slab in LDS and multiplies with
// v_mfma_i32_16x16x64_i8 (tokens as M; wave w owns slab columns
// 16 w .. 16 w + 15; weight operands from two transposing LDS reads),
// writing int32 partials P[s][t][576].  Item 0 also writes the tokens'
// activation scales and fills their latent code rows and scales with the
// fused finish's "not finished" pattern.
// ---------------------------------------------------------------------------
template <int KW>
__global__ __launch_bounds__(256) void dec_kv_a_w8_kernel(
    const uint16_t* __restrict__ X, const int8_t* __restrict__ Wqa, int T, int H, int S, int kw,
    int32_t* __restrict__ P, float* __restrict__ sx, int8_t* __restrict__ fill_q,
    uint32_t* __restrict__ fill_sz, uint32_t* __restrict__ fill_inv) {
    constexpr int WP = kSlabW + 16;  // LDS pitch of a staged slab row (bytes)
    constexpr int AP = KW + 16;      // LDS pitch of a code row (bytes)
    constexpr int NT = 8;            // tokens at most
    constexpr int NCH = 4;           // 16-byte chunks per thread of a row (H <= 8192)
    constexpr int KC = KW / 8;       // chunks of a token's K range
    constexpr int KCT = (NT * KC + 255) / 256;
    __shared__ __align__(16) int8_t ldsW[KW * WP];
    __shared__ __align__(16) int8_t ldsA[16 * AP];
    __shared__ float lmax[4][NT];
    const int item = xcd_item(kSlabsA * S);
    if (item < 0) return;
    const int s = item / kSlabsA, slab = item % kSlabsA;
    const int k0 = s * kw, kmax = min(H, k0 + kw);  // kw <= KW
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = H >> 3;
    // every load first: the weight slab (rows past kmax read row kmax - 1
    // and are zeroed when stored), the tokens' rows for the maxima and their
    // chunks of this K range (rows past T read token T - 1, unused)
    u4_t wv[KW / 64];
#pragma unroll
    for (int u = 0; u < KW / 64; ++u) {
        const int k = min(k0 + (tid >> 2) + 64 * u, kmax - 1);
        wv[u] = __builtin_nontemporal_load(
            (const u4_t*)(Wqa + (int64_t)k * kN1 + slab * kSlabW + 16 * (tid & 3)));
    }
    u4_t xv[NT][NCH];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < NCH; ++u)
            xv[t][u] = *(const u4_t*)(X + (int64_t)min(t, T - 1) * H +
                                      8 * min(tid + 256 * u, nch - 1));
    u4_t kv[KCT];
#pragma unroll
    for (int u = 0; u < KCT; ++u) {
        const int q = tid + 256 * u, t = q / KC, c = q % KC;
        kv[u] = *(const u4_t*)(X + (int64_t)min(t, T - 1) * H + min(k0 + 8 * c, H - 8));
    }
    // the tokens' maxima (max is exact in any order)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float am = 0.f;
#pragma unroll
        for (int u = 0; u < NCH; ++u)
            if (tid + 256 * u < nch) am = absmax8(xv[t][u], am);
        am = wave_max(am);
        if (lane == 0) lmax[wave][t] = am;
    }
#pragma unroll
    for (int u = 0; u < KW / 64; ++u) {
        const int k = k0 + (tid >> 2) + 64 * u;
        *(u4_t*)(ldsW + ((tid >> 2) + 64 * u) * WP + 16 * (tid & 3)) =
            k < kmax ? wv[u] : u4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // the codes of this K range: rows past T and columns past kmax are zero
#pragma unroll
    for (int u = 0; u < KCT; ++u) {
        const int q = tid + 256 * u, t = q / KC, c = q % KC;
        if (t < NT) {
            const float am = fmaxf(fmaxf(lmax[0][t], lmax[1][t]), fmaxf(lmax[2][t], lmax[3][t]));
            const float inv = (am > 0.f) ? (127.0f / am) : 0.f;
            const bool ok = t < T && k0 + 8 * c < kmax;
            *(u2_t*)(ldsA + t * AP + 8 * c) = ok ? quant8(kv[u], inv) : u2_t{0u, 0u};
        }
    }
    // rows NT .. 15 of the token tile are zero
    for (int q = tid; q < (16 - NT) * (KW / 8); q += 256)
        *(u2_t*)(ldsA + (NT + q / (KW / 8)) * AP + 8 * (q % (KW / 8))) = u2_t{0u, 0u};
    if (item == 0 && tid < T) {
        const float am = fmaxf(fmaxf(lmax[0][tid], lmax[1][tid]), fmaxf(lmax[2][tid], lmax[3][tid]));
        sx[tid] = (am > 0.f) ? (am / 127.0f) : 0.f;
    }
    if (item == 0 && fill_q != nullptr) {
        for (int q = tid; q < T * (kR / 8); q += 256)
            *(u2_t*)(fill_q + (int64_t)(q / (kR / 8)) * kR + 8 * (q % (kR / 8))) =
                u2_t{0x80808080u, 0x80808080u};
        if (tid < T) {
            fill_sz[tid] = ~0u;
            fill_inv[tid] = ~0u;
        }
    }
    __syncthreads();
    const int l16 = lane & 15, g = lane >> 4;
    i4_t acc = {0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KW / 64; ++ks) {
        const u4_t fa = *(const u4_t*)(ldsA + l16 * AP + ks * 64 + 16 * g);
        const int k = ks * 64 + g * 16 + (l16 >> 1);
        const int colb = wave * 16 + 8 * (l16 & 1);
        const uint2 lo = lds_tr8_w(ldsW + k * WP + colb);
        const uint2 hi = lds_tr8_w(ldsW + (k + 8) * WP + colb);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            __builtin_bit_cast(i4_t, fa), __builtin_bit_cast(i4_t, u4_t{lo.x, lo.y, hi.x, hi.y}),
            acc, 0, 0, 0);
    }
    // lane 16 g + c holds tokens 4 g + i of slab column 16 wave + c
    int32_t* Ps = P + (int64_t)s * T * kN1 + slab * kSlabW + wave * 16 + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * g + i;
        if (t < T) Ps[(int64_t)t * kN1] = acc[i];
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
static inline int grid8(int nitems) { return 8 * ((nitems + 7) / 8); }

template <int E, int NA>
static void dec_kv_a_launch(const void* X, const void* Wa, int T, int H, float* P, int kw, int S,
                            uint16_t* ckv, int ng, hipStream_t st) {
    const dim3 ga(grid8(kSlabsA * S * ng)), blk(256);
    const uint16_t* x = (const uint16_t*)X;
    const uint16_t* wa = (const uint16_t*)Wa;
#define MLA_KVA(KW) \
    launch_k((dec_kv_a_kernel<E, NA, KW>), ga, blk, 0, st, x, wa, T, H, S, P, ckv, ng)
    switch (kw) {
        case 64: MLA_KVA(64); break;
        case 128: MLA_KVA(128); break;
        case 256: MLA_KVA(256); break;
        default: MLA_KVA(512); break;
    }
#undef MLA_KVA
}

// How many dec_fin_kv_b workgroups the current device holds at once (CU
// count times this kernel's occupancy per CU), cached per device and dtype.
static std::atomic<int> g_fused_cap[2][64];
static std::atomic<int64_t> g_spin_limit{-1};

template <int E>
static int fused_capacity() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::atomic<int>& slot = g_fused_cap[E == kF16 ? 0 : 1][dev];
    int cap = slot.load(std::memory_order_relaxed);
    if (cap > 0) return cap;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, dec_fin_kv_b_kernel<E>, 256, 0) !=
            hipSuccess)
        return 0;
    cap = cus * per;
    slot.store(cap, std::memory_order_relaxed);
    return cap;
}

template <int E>
static void dec_launch_t(const void* X, const void* Wa, const void* gamma, const void* Wb,
                         const int32_t* pos, int T, int H, int nh, float eps, const RopeTab& rt,
                         void* k_nope, void* value, void* k_pe, void* ckv, float* P,
                         const Plan& plan, const CacheOut& co, hipStream_t st) {
    const int ntile = (T + 15) / 16;
    const int N2 = nh * kHeadW;
    const int nitems = (N2 / kSlabW) * ntile;
    // one launch for finish + kv_b_proj only when its whole grid is resident
    // at once; otherwise the finish and kv_b_proj run as two launches
    const bool fused = grid8(nitems) <= fused_capacity<E>();
    uint16_t* y = (uint16_t*)ckv;
    // fewer than 128 weight blocks: the token tiles go to two workgroups per
    // block, so that more CUs share the weight and activation fetch
    const int ng = (kSlabsA * plan.s1 < 128 && ntile >= 2) ? 2 : 1;
    switch ((ntile + ng - 1) / ng) {
        case 1: dec_kv_a_launch<E, 1>(X, Wa, T, H, P, plan.kw, plan.s1, y, ng, st); break;
        case 2: dec_kv_a_launch<E, 2>(X, Wa, T, H, P, plan.kw, plan.s1, y, ng, st); break;
        case 3: dec_kv_a_launch<E, 3>(X, Wa, T, H, P, plan.kw, plan.s1, y, ng, st); break;
        default: dec_kv_a_launch<E, 4>(X, Wa, T, H, P, plan.kw, plan.s1, y, ng, st); break;
    }
    if (fused) {
        const int64_t sl = g_spin_limit.load(std::memory_order_relaxed);
        const uint32_t spin = sl < 0 ? kSpinDefault : (uint32_t)(sl > 0xFFFFFFFFll ? 0xFFFFFFFFll : sl);
        launch_k(dec_fin_kv_b_kernel<E>, dim3(grid8(nitems)), dim3(256), 0, st,
                 (const float*)P, plan.s1, T, (const uint16_t*)gamma, pos, eps, rt,
                 (const uint16_t*)Wb, N2, (uint16_t*)ckv, (uint16_t*)k_pe,
                 (uint16_t*)k_nope, (uint16_t*)value, co, spin);
        return;
    }
    launch_k(dec_finish_kernel<E>, dim3(T), dim3(256), 0, st, (const float*)P, plan.s1,
             T, (const uint16_t*)gamma, pos, eps, rt, (uint16_t*)ckv, (uint16_t*)k_pe, co);
    launch_k((dec_kv_b_kernel<E, 1>), dim3(grid8(nitems)), dim3(256), 0, st,
             (const uint16_t*)ckv, (const uint16_t*)Wb, T, N2, (uint16_t*)k_nope,
             (uint16_t*)value);
}

// W8A8 decode: the fused finish + kv_b_proj for up to 16 tokens, when its
// grid (one workgroup per 64-column slab) is resident at once.
static std::atomic<int> g_fused_cap_w8[64];
template <int NPW>
static int fused_capacity_w8() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int cap = g_fused_cap_w8[dev].load(std::memory_order_relaxed);
    if (cap > 0) return cap;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, dec_fin_kv_b_w8_kernel<NPW>, 256, 0) !=
            hipSuccess)
        return 0;
    cap = cus * per;
    g_fused_cap_w8[dev].store(cap, std::memory_order_relaxed);
    return cap;
}

// W8A8 kv_a_proj with the quantiser folded in, for up to 8 tokens: whether
// it applies (H <= 8192 for the per-thread row chunks; a split of at most
// 512 rows for the LDS slab) and its launch.
bool w8_decode_kva_fits(int64_t T, int H, int S) {
    const int ks = H / 128, per = (ks + S - 1) / S;
    return T >= 1 && T <= 8 && H <= 8192 && per * S == ks && per <= 4;
}
void launch_w8_kv_a(const void* X, const int8_t* Wqa, int64_t T, int H, int S, int32_t* P,
                    float* sx, int8_t* fill_q, float* fill_sz, float* fill_inv, hipStream_t st) {
    const int kw = H / S;
    auto go = [&](auto kern) {
        launch_k(kern, dim3(grid8(kSlabsA * S)), dim3(256), 0, st, (const uint16_t*)X, Wqa,
                 (int)T, H, S, kw, P, sx, fill_q, (uint32_t*)fill_sz, (uint32_t*)fill_inv);
    };
    if (kw <= 128) go(dec_kv_a_w8_kernel<128>);
    else if (kw <= 256) go(dec_kv_a_w8_kernel<256>);
    else go(dec_kv_a_w8_kernel<512>);
}

bool w8_decode_fused_fits(int64_t T, int nh, int S) {
    if (T < 1 || T > 16 || S < 1 || S > 32) return false;
    // every NPW instance has the same LDS and register budget
    return grid8(nh * kHeadW / kSlabW) <= fused_capacity_w8<8>();
}

void launch_w8_fin_kv_b(const int32_t* P, int S, int64_t T, const float* sx, const float* swa,
                        const void* gamma, const int32_t* pos, float eps, const RopeTab& rt,
                        const int8_t* Wqb, const float* swb, int nh, int8_t* QZ, float* sz,
                        float* inv, void* ckv, void* k_pe, void* k_nope, void* value,
                        int32_t* dbg1, int32_t* dbg2, int64_t dbg_begin, int64_t dbg_rows,
                        const CacheOut& co, hipStream_t st) {
    const int N2 = nh * kHeadW;
    const int64_t sl = g_spin_limit.load(std::memory_order_relaxed);
    const uint32_t spin = sl < 0 ? kSpinDefault : (uint32_t)(sl > 0xFFFFFFFFll ? 0xFFFFFFFFll : sl);
    auto go = [&](auto kern) {
        launch_k(kern, dim3(grid8(N2 / kSlabW)), dim3(256), 0, st, P, S, (int)T, sx, swa,
                 (const uint16_t*)gamma, pos, eps, rt, Wqb, swb, N2, QZ, sz, inv, (uint16_t*)ckv,
                 (uint16_t*)k_pe, (uint16_t*)k_nope, (uint16_t*)value, dbg1, dbg2, dbg_begin,
                 dbg_rows, co, spin);
    };
    if (S <= 4) go(dec_fin_kv_b_w8_kernel<1>);
    else if (S <= 8) go(dec_fin_kv_b_w8_kernel<2>);
    else if (S <= 16) go(dec_fin_kv_b_w8_kernel<4>);
    else go(dec_fin_kv_b_w8_kernel<8>);
}

hipError_t launch_fp_decode(int dt, const void* X, const void* Wa, const void* gamma,
                            const void* Wb, const int32_t* pos, int64_t T, int H, int nh,
                            float eps, const RopeTab& rt, void* k_nope, void* value, void* k_pe,
                            void* ckv, void* ws, const Plan& plan, const CacheOut& co,
                            hipStream_t st) {
    float* P = (float*)((uint8_t*)ws + ws_fp(T, plan).p1);
    if (dt == kF16)
        dec_launch_t<kF16>(X, Wa, gamma, Wb, pos, (int)T, H, nh, eps, rt, k_nope, value, k_pe, ckv,
                           P, plan, co, st);
    else
        dec_launch_t<kBF16>(X, Wa, gamma, Wb, pos, (int)T, H, nh, eps, rt, k_nope, value, k_pe,
                            ckv, P, plan, co, st);
    return hipGetLastError();
}

int64_t decode_set_spin_limit(int64_t limit) {
    return g_spin_limit.exchange(limit < 0 ? -1 : limit);
}

int64_t decode_handoff_fallbacks(bool reset) {
    unsigned int v = 0, v8 = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_handoff_fallbacks), sizeof(v), 0,
                            hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpyFromSymbol(&v8, HIP_SYMBOL(g_handoff_fallbacks_w8), sizeof(v8), 0,
                            hipMemcpyDeviceToHost) != hipSuccess)
        return -1;
    if (reset) {
        const unsigned int z = 0;
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_handoff_fallbacks), &z, sizeof(z), 0,
                              hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpyToSymbol(HIP_SYMBOL(g_handoff_fallbacks_w8), &z, sizeof(z), 0,
                              hipMemcpyHostToDevice) != hipSuccess)
            return -1;
    }
    return (int64_t)v + (int64_t)v8;
}

}  // namespace mla
