// Internal definitions shared by the gfx950 kernels and the C-ABI layer of
// libmlaprolog.  Not a public header.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

// element kinds of the two projections' operands
enum Elem : int { kF16 = 1, kBF16 = 2, kI8 = 3 };

// fixed widths of the prolog (DeepSeek-V2-Lite / R1 MLA)
constexpr int kR = 512;   // kv_lora_rank
constexpr int kDR = 64;   // rope dim
constexpr int kN1 = kR + kDR;
constexpr int kDN = 128;  // k_nope per head
constexpr int kDV = 128;  // value per head
constexpr int kHeadW = kDN + kDV;

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, h);
    return (float)v;
}
// round-to-nearest-even fp32 -> bf16 (inputs are finite here)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}
template <int E>
__device__ __forceinline__ float ld_to_f32(uint16_t b) {
    if constexpr (E == kF16) return f16_to_f32(b);
    else return bf16_to_f32(b);
}
template <int E>
__device__ __forceinline__ uint16_t f32_to_st(float f) {
    if constexpr (E == kF16) return f32_to_f16(f);
    else return f32_to_bf16(f);
}

// ---------------------------------------------------------------------------
// wave reductions (64 lanes): DPP steps inside each row of 16 lanes (swap
// neighbours, swap pairs, mirror half-rows, mirror rows), then the four row
// results read out of lanes 0, 16, 32, 48 and combined in a fixed order.
// The result is the same in every lane.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// ---------------------------------------------------------------------------
// launch plan and workspace layout (host)
// ---------------------------------------------------------------------------
struct Plan {
    int path;       // 0 decode, 1 prefill (what mla_kv_prolog_selected_path reports)
    int stream;     // 1: weight-streaming decode kernels, 0: tiled MFMA kernels
    int bm1, s1;    // kv_a_proj: rows per tile (tiled), split-K count
    int kw;         // streaming kv_a_proj: K rows per producer workgroup
    int bm2, bn2;   // kv_b_proj tile (tiled)
    int dma1;       // kv_a_proj by the direct-to-LDS pipelined GEMM (no split-K)
    int fuse2;      // fp16/bf16 tiled path: finish and kv_b_proj in one launch
                    // (-1: the dispatcher decides, 0: never, 1: whenever s1 <= 2)
};

// RoPE inverse frequencies theta^(-2i/dr), i < dr/2, evaluated once per call
// on the host in double (they depend on theta only).
struct RopeTab {
    double f[kDR / 2];
};

// cos / sin of the rope angle a = pos * f.  The angle is formed in double
// and reduced by quarter turns there (k = nearest integer to a / (pi/2), pi/2
// split into two doubles, Cody-Waite), leaving |x| <= pi/4; sin x and cos x
// then come from their Taylor series in fp32 (terms through x^9 and x^10:
// truncation below 2e-9 on that interval), and k mod 4 rotates them into
// place.  Straight-line code: no table lookups, no branches.
__device__ __forceinline__ void rope_cos_sin(int32_t pos, double f, float& cs, float& sn) {
    const double a = (double)pos * f;
    const double k = rint(a * 0.6366197723675814);
    double r = fma(-k, 1.5707963267948966, a);
    r = fma(-k, 6.123233995736766e-17, r);
    const float x = (float)r, x2 = x * x;
    const float s =
        x + x * x2 * (-1.0f / 6.0f +
                      x2 * (1.0f / 120.0f + x2 * (-1.0f / 5040.0f + x2 * (1.0f / 362880.0f))));
    const float c =
        1.0f + x2 * (-0.5f + x2 * (1.0f / 24.0f +
                                   x2 * (-1.0f / 720.0f +
                                         x2 * (1.0f / 40320.0f + x2 * (-1.0f / 3628800.0f)))));
    const int q = (int)((long long)k & 3);
    const float cq = (q & 1) ? s : c, sq = (q & 1) ? c : s;
    cs = ((q + 1) & 2) ? -cq : cq;  // quarter turns 1, 2 negate cos
    sn = (q & 2) ? -sq : sq;        // quarter turns 2, 3 negate sin
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// fp path: [s1][T][576] fp32 split-K partial sums of kv_a_proj
struct WsFp {
    size_t p1, total;
};
inline WsFp ws_fp(int64_t T, const Plan& p) {
    WsFp w;
    w.p1 = 0;
    w.total = align256((size_t)p.s1 * (size_t)T * kN1 * 4);
    return w;
}

// W8A8 path: int8 codes of x [T][H], their scales [T], int32 split-K partials
// [s1][T][576], int8 codes of z [T][512], their scales [T], RMS factors [T]
// (the last two padded to a multiple of 256 tokens: the kv_b_proj epilogue
// reads them in whole 256-row tiles)
struct WsW8 {
    size_t qx, sx, p1, qz, sz, inv, total;
};
inline WsW8 ws_w8(int64_t T, int H, const Plan& p) {
    WsW8 w;
    size_t o = 0;
    w.qx = o; o += align256((size_t)T * H);
    w.sx = o; o += align256((size_t)T * 4);
    w.p1 = o; o += align256((size_t)p.s1 * (size_t)T * kN1 * 4);
    // the quantised latent, padded to whole blocks of 32 rows for the
    // weight-stationary kv_b_proj kernel's copies
    w.qz = o; o += align256((size_t)((T + 31) / 32) * 32 * kR);
    const size_t tpad = (size_t)((T + 255) / 256) * 256;
    w.sz = o; o += tpad * 4;
    w.inv = o; o += tpad * 4;
    w.total = o;
    return w;
}

// The fp32 value v as it is, kept out of any fusion with the operation that
// consumes it (an empty asm that claims to modify it).  Used before a
// conversion to fp16: the compiler otherwise folds a product and the
// conversion into one mixed-precision FMA (v_fma_mix: a single rounding,
// straight to fp16) in some inlined copies and not in others, so two copies
// that must agree bit for bit, or agree with "round to fp32, then to fp16",
// would not.
__device__ __forceinline__ float fp32_value(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// RMSNorm's last step on 8 consecutive values c (fp32): times the row's
// inverse RMS, then times gamma (8 values of dtype E packed in g), rounded to
// fp32 and then to E, and packed.  The prolog's finish kernels and the
// standalone RMSNorm share it.
template <int E>
__device__ __forceinline__ u4_t rms_scale8(const float (&c)[8], float inv, const u4_t g) {
    u4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float g0 = ld_to_f32<E>((uint16_t)(g[w] & 0xFFFFu));
        const float g1 = ld_to_f32<E>((uint16_t)(g[w] >> 16));
        const uint32_t y0 = f32_to_st<E>(fp32_value((c[2 * w] * inv) * g0));
        const uint32_t y1 = f32_to_st<E>(fp32_value((c[2 * w + 1] * inv) * g1));
        o[w] = y0 | (y1 << 16);
    }
    return o;
}

// Rotate-half RoPE of one value v with its partner in the other half of the
// rope row (v's index +- dr/2): the first half takes v cos - partner sin, the
// second v cos + partner sin.
__device__ __forceinline__ float rope_rotate(float v, float partner, float cs, float sn,
                                             bool first_half) {
    return first_half ? (v * cs - partner * sn) : (v * cs + partner * sn);
}

// Optional paged KV-cache output of the prolog: when slots != nullptr the
// finish step also writes each token's [compressed_kv row | k_pe row] into
// slot slots[t], either as the model dtype (cache, [num_slots, 576]) or as
// int8 codes with one fp32 scale per slot (cache_q [num_slots, 576], scale
// [num_slots]; W8A8 prolog only); a slot outside [0, num_slots) skips the
// token.
struct CacheOut {
    const int64_t* slots;
    uint16_t* cache;
    int64_t num_slots;
    int8_t* cache_q = nullptr;
    float* scale = nullptr;
};
__device__ __forceinline__ bool cache_slot_ok(const CacheOut& co, int64_t s) {
    return co.slots != nullptr && s >= 0 && s < co.num_slots;
}

// The int8 cache scheme (the W8A8 activation one, over a slot's 576
// values): 8 values of dtype E (in v) to 8 codes clamp(rint(x * inv), +-127)
// in fp32 with round-half-even, inv = 127 / max|value| (0 for a zero slot).
template <int E>
__device__ __forceinline__ u2_t codes8(const u4_t v, float inv) {
    u2_t q;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t word = v[2 * w + (b >> 1)];
            const uint16_t bits = (uint16_t)((b & 1) ? (word >> 16) : (word & 0xFFFFu));
            float r = rintf(ld_to_f32<E>(bits) * inv);
            r = fminf(fmaxf(r, -127.f), 127.f);
            packed |= ((uint32_t)(uint8_t)(int8_t)(int)r) << (8 * b);
        }
        q[w] = packed;
    }
    return q;
}
template <int E>
__device__ __forceinline__ float absmax8_e(const u4_t v, float a) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        a = fmaxf(a, fabsf(ld_to_f32<E>((uint16_t)(v[w] & 0xFFFFu))));
        a = fmaxf(a, fabsf(ld_to_f32<E>((uint16_t)(v[w] >> 16))));
    }
    return a;
}

// ---------------------------------------------------------------------------
// host-side launchers (defined in the .hip files)
// ---------------------------------------------------------------------------

hipError_t launch_fp(int dt, const void* X, const void* Wa, const void* gamma,
                     const void* Wb, const int32_t* pos, int64_t T, int H, int nh,
                     float eps, const RopeTab& rt, void* k_nope, void* value, void* k_pe,
                     void* ckv, void* ws, const Plan& plan, const CacheOut& co, hipStream_t st);

hipError_t launch_fp_decode(int dt, const void* X, const void* Wa, const void* gamma,
                            const void* Wb, const int32_t* pos, int64_t T, int H, int nh,
                            float eps, const RopeTab& rt, void* k_nope, void* value,
                            void* k_pe, void* ckv, void* ws, const Plan& plan, const CacheOut& co,
                            hipStream_t st);

// per-token finish of kv_a_proj (split, RMSNorm, RoPE) from split-K partials
void launch_finish_fp(int dt, const float* P, int S, int64_t T, const void* gamma,
                      const int32_t* pos, float eps, const RopeTab& rt, void* ckv, void* kpe,
                      const CacheOut& co, hipStream_t st);

// standalone RMSNorm over rows of n values (n % 8 == 0, 8 <= n <= 8192) and
// RoPE over x [T, heads, 64]; rows / T > 0
hipError_t launch_rms_norm(int dt, const void* x, const void* gamma, int64_t rows, int n,
                           float eps, void* y, hipStream_t st);
hipError_t launch_rope(int dt, const void* x, const int32_t* pos, int64_t T, int heads,
                       const RopeTab& rt, void* y, hipStream_t st);

// paged KV-cache append: fp cache (cache_q == nullptr) or int8 codes + scales
hipError_t launch_kv_cache_append(int dt, const void* ckv, const void* kpe, const int64_t* slots,
                                  int64_t T, int64_t num_slots, void* cache, int8_t* cache_q,
                                  float* scale, hipStream_t st);
// Device-coherent 8- and 4-byte accesses (single-copy atomic, seen by every
// XCD): the hand-offs between workgroups of one launch.
__device__ __forceinline__ void store_coherent64(void* p, uint64_t v) {
    __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent64(const void* p) {
    return __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent32(void* p, uint32_t v) {
    __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent32(const void* p) {
    return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// W8A8 activation quantisation of 8 bf16 values with the token's factor
// inv = 127 / amax: rint(x * inv) clamped to +-127 (ties to even), and the
// running maximum of |x| over 8 values.
__device__ __forceinline__ u2_t quant8(const u4_t v, float inv) {
    u2_t q;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int e = w * 4 + b;
            const uint32_t bits = (v[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
            float r = rintf(bf16_to_f32((uint16_t)bits) * inv);
            r = fminf(fmaxf(r, -127.f), 127.f);
            packed |= ((uint32_t)(uint8_t)(int8_t)(int)r) << (8 * b);
        }
        q[w] = packed;
    }
    return q;
}
__device__ __forceinline__ float absmax8(const u4_t v, float amax) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(v[w] & 0xFFFFu))));
        amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(v[w] >> 16))));
    }
    return amax;
}

// W8A8: the latent of one token from its exact int32 kv_a_proj sums, lane l
// holding latent columns 8l .. 8l + 7 (one wave):
//   c = (acc * sx) * s_a,  z = c * gamma,
//   inv = 1 / sqrt(sum(c^2) / 512 + eps)   (the RMS factor of c),
//   codes = rint(z * 127 / amax(z)) clamped to +-127, scale = amax(z) / 127.
// No contraction, so every inlined copy (the finish kernels', a hand-off
// producer's and its fallback's) is the same sequence of fp32 operations.
struct W8Latent {
    float z[8];
    u2_t q;
    float sz, inv;
};
__device__ __forceinline__ W8Latent w8_latent(const int (&a)[8], float sxt, f4_t wa0, f4_t wa1,
                                              u4_t gm, float eps) {
#pragma clang fp contract(off)
    W8Latent r;
    float c[8];
    float ss = 0.f, az = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float w = i < 4 ? wa0[i] : wa1[i - 4];
        c[i] = ((float)a[i] * sxt) * w;
        const uint16_t gb = (uint16_t)(gm[i >> 1] >> (16 * (i & 1)));
        r.z[i] = c[i] * bf16_to_f32(gb);
        ss += c[i] * c[i];
        az = fmaxf(az, fabsf(r.z[i]));
    }
    ss = wave_sum(ss);
    az = wave_max(az);
    r.inv = 1.0f / sqrtf(ss / (float)kR + eps);
    const float inv2 = (az > 0.f) ? (127.0f / az) : 0.f;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float q = rintf(r.z[w * 4 + b] * inv2);
            q = fminf(fmaxf(q, -127.f), 127.f);
            packed |= ((uint32_t)(uint8_t)(int8_t)(int)q) << (8 * b);
        }
        r.q[w] = packed;
    }
    r.sz = (az > 0.f) ? (az / 127.0f) : 0.f;
    return r;
}

// The W8A8 finish of token t once lane l holds the token's int32 kv_a_proj
// sums of latent columns 8l .. 8l + 7 (a) and of rope column l (ap), one
// wave: the latent codes and scales (with COH through device-coherent
// stores, for a hand-off), compressed_kv = bf16(z * inv), k_pe, the paged
// cache and the accumulator debug copy.
template <bool COH>
__device__ __forceinline__ void w8_finish_token(
    const int (&a)[8], int ap, int64_t t, int pt, int64_t slot, float sxt, f4_t wa0, f4_t wa1,
    float wap, u4_t gm, float eps, const RopeTab& rt, int8_t* __restrict__ QZ,
    float* __restrict__ sz, float* __restrict__ inv_out, uint16_t* __restrict__ ckv,
    uint16_t* __restrict__ kpe, int32_t* __restrict__ dbg, int64_t dbg_begin, int64_t dbg_rows,
    const CacheOut& co) {
    const int lane = threadIdx.x & 63;
    if (dbg != nullptr && t >= dbg_begin && t < dbg_begin + dbg_rows) {
        int32_t* d = dbg + (t - dbg_begin) * kN1;
#pragma unroll
        for (int i = 0; i < 8; ++i) d[8 * lane + i] = a[i];
        d[kR + lane] = ap;
    }
    const W8Latent L = w8_latent(a, sxt, wa0, wa1, gm, eps);
    const float p = ((float)ap * sxt) * wap;
    u4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        o[w] = (uint32_t)f32_to_bf16(L.z[2 * w] * L.inv) |
               ((uint32_t)f32_to_bf16(L.z[2 * w + 1] * L.inv) << 16);
    if constexpr (COH) {
        store_coherent64(QZ + t * kR + 8 * lane, (uint64_t)L.q[0] | ((uint64_t)L.q[1] << 32));
        if (lane == 0) {
            store_coherent32(sz + t, __builtin_bit_cast(uint32_t, L.sz));
            store_coherent32(inv_out + t, __builtin_bit_cast(uint32_t, L.inv));
        }
    } else {
        *(u2_t*)(QZ + t * kR + 8 * lane) = L.q;
        if (lane == 0) {
            sz[t] = L.sz;
            inv_out[t] = L.inv;
        }
    }
    *(u4_t*)(ckv + t * kR + 8 * lane) = o;
    const float partner = __shfl_xor(p, 32, 64);
    float cs, sn;
    rope_cos_sin(pt, rt.f[lane & 31], cs, sn);
    const float out = rope_rotate(p, partner, cs, sn, lane < 32);
    const uint16_t ko = f32_to_bf16(out);
    __builtin_nontemporal_store(ko, kpe + t * kDR + lane);
    if (cache_slot_ok(co, slot)) {
        // the paged cache, [latent | rope key] in the token's slot: the
        // returned bf16 rows, or their int8 codes and the slot's scale
        constexpr int W = kR + kDR;
        if (co.cache_q == nullptr) {
            uint16_t* row = co.cache + slot * W;
            __builtin_nontemporal_store(o, (u4_t*)(row + 8 * lane));
            __builtin_nontemporal_store(ko, row + kR + lane);
        } else {
            const float am = wave_max(fmaxf(absmax8_e<kBF16>(o, 0.f), fabsf(bf16_to_f32(ko))));
            const float qi = (am > 0.f) ? (127.0f / am) : 0.f;
            int8_t* row = co.cache_q + slot * W;
            __builtin_nontemporal_store(codes8<kBF16>(o, qi), (u2_t*)(row + 8 * lane));
            float rk = rintf(bf16_to_f32(ko) * qi);
            rk = fminf(fmaxf(rk, -127.f), 127.f);
            __builtin_nontemporal_store((int8_t)(int)rk, row + kR + lane);
            if (lane == 0) co.scale[slot] = (am > 0.f) ? (am / 127.0f) : 0.f;
        }
    }
}

// W8A8 at decode sizes: whether the finish fused into kv_b_proj applies to
// T tokens, nh heads and S kv_a_proj splits on the current device (its
// grid resident at once), and its launch (prolog_decode.hip).
bool w8_decode_fused_fits(int64_t T, int nh, int S);
// and, for up to 8 tokens, kv_a_proj with the activation quantiser folded
// in (it also fills the fused launch's hand-off pattern when fill_q is set)
bool w8_decode_kva_fits(int64_t T, int H, int S);
void launch_w8_kv_a(const void* X, const int8_t* Wqa, int64_t T, int H, int S, int32_t* P,
                    float* sx, int8_t* fill_q, float* fill_sz, float* fill_inv, hipStream_t st);
void launch_w8_fin_kv_b(const int32_t* P, int S, int64_t T, const float* sx, const float* swa,
                        const void* gamma, const int32_t* pos, float eps, const RopeTab& rt,
                        const int8_t* Wqb, const float* swb, int nh, int8_t* QZ, float* sz,
                        float* inv, void* ckv, void* k_pe, void* k_nope, void* value,
                        int32_t* dbg1, int32_t* dbg2, int64_t dbg_begin, int64_t dbg_rows,
                        const CacheOut& co, hipStream_t st);

// The decode family's finish + kv_b_proj hand-off: set the bound on its
// polls (negative: the default; returns the previous setting), and read
// (optionally clearing) the current device's count of workgroups that ran
// out of polls and rebuilt their rows themselves (-1 on a HIP error).
int64_t decode_set_spin_limit(int64_t limit);
int64_t decode_handoff_fallbacks(bool reset);

// The next pair of the events the calling thread registered
// (mla_debug_set_launch_events), or two nulls when none are left.
void launch_events(hipEvent_t* start, hipEvent_t* stop);

// Kernel launch of the prolog entry points.  With events registered, the
// launch records the next pair at the kernel's own start and end (the
// dispatch's timestamps); otherwise it is a plain launch.
template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                     Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    launch_events(&e0, &e1);
    if (e0 != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, e0, e1, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
}

// While a ValidateOnlyScope is alive on the calling thread, the prolog
// entry points run every argument check and return without launching (the
// captured-graph sets use it to reject bad arguments before capturing).
bool validate_only();
struct ValidateOnlyScope {
    ValidateOnlyScope();
    ~ValidateOnlyScope();
};

hipError_t launch_w8a8(const void* X, const int8_t* Wqa, const float* swa,
                       const void* gamma, const int8_t* Wqb, const float* swb,
                       const int32_t* pos, int64_t T, int H, int nh, float eps,
                       const RopeTab& rt, void* k_nope, void* value, void* k_pe, void* ckv,
                       int32_t* dbg1, int32_t* dbg2, int64_t dbg_begin, int64_t dbg_rows,
                       void* ws, const Plan& plan, const CacheOut& co, hipStream_t st);

}  // namespace mla
