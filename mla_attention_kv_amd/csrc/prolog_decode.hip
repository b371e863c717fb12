// Weight-streaming gfx950 kernels of the MLA KV prolog for short token
// batches (decode: a few sequences x one or two query tokens).
//
// At decode sizes the prolog is bound by reading the two weight matrices
// once from HBM, so the kernels are shaped around the weight stream:
//   dec_kv_a     kv_a_proj: W_kv_a cut into 64-column slabs x K ranges of
//                KW rows, one workgroup each, writing split-K partial sums
//                P[s][t][576]
//   dec_finish   one workgroup per token: sum the partials, RMSNorm the
//                latent (-> compressed_kv), rotate the rope part (-> k_pe)
//   dec_kv_b     kv_b_proj: items of (16-token tile, 64-column slab of
//                W_kv_b over the full K = 512), one workgroup each, writing
//                its tile of k_nope / value
// Each workgroup issues all of its weight loads first (16 bytes per lane,
// 128 contiguous bytes per row) and stages the slab in LDS, where the MFMA
// operand (8 consecutive K of one column per lane) is read back
// column-wise; wave w owns slab columns 16w..16w+15 over the whole K range,
// so no cross-wave reduction is needed.  The kv_b items sharing a slab sit
// on one XCD (workgroups go to the 8 XCDs round-robin), so that XCD's L2
// serves the repeated slab reads, and all items of a slab read the latent
// through the same L2.
//
// The three launches are stream-ordered: a kernel boundary publishes the
// previous kernel's results to the whole device at once, which on this
// part is cheaper than any in-kernel grid hand-off for data that many
// workgroups must read (each in-kernel reader would have to drop its XCD's
// cache lines or bypass them).
//
// Steps as in the DeepSeek-V2-Lite-Chat MLA KV Prolog migration guide
// (dpshk.com), sections "Background" and "Source-level principle"; RoPE in
// the rotate-half x*cos + x_rot*sin form of its "Precision verification".
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
// columns) of rows i/8 + 32 r, r < NR; rows at or past kmax load zeros.
// stage_store writes them to LDS as [row][kPitch].
// ---------------------------------------------------------------------------
template <int NR>
__device__ __forceinline__ void stage_load(u4_t (&v)[NR], const uint16_t* W, int64_t ld, int k0,
                                           int kmax, int n0) {
    const int q = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int k = k0 + r0 + 32 * r;
        v[r] = (k < kmax) ? *(const u4_t*)(W + (int64_t)k * ld + n0 + 8 * q) : u4_t{0u, 0u, 0u, 0u};
    }
}
template <int NR>
__device__ __forceinline__ void stage_store(const u4_t (&v)[NR], uint16_t* lds) {
    const int q = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int r = 0; r < NR; ++r) *(u4_t*)(lds + (r0 + 32 * r) * kPitch + 8 * q) = v[r];
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
// kv_a_proj partial of (slab, split) over K rows [s*KW, s*KW + KW).
// grid = 9 slabs x S splits (slab fastest), 256 threads.
// ---------------------------------------------------------------------------
template <int E, int NTT, int KW>
__global__ __launch_bounds__(256) void dec_kv_a_kernel(const uint16_t* __restrict__ X,
                                                       const uint16_t* __restrict__ Wa, int T,
                                                       int H, float* __restrict__ P) {
    __shared__ __align__(16) uint16_t lds[KW * kPitch];
    const int slab = blockIdx.x % kSlabsA, s = blockIdx.x / kSlabsA;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    const int k0 = s * KW;
    u4_t v[KW / 32];
    stage_load<KW / 32>(v, Wa, kN1, k0, H, slab * kSlabW);
    // activation operands of all chunks, fetched with the weights
    u4_t x[KW / 32][NTT];
#pragma unroll
    for (int ch = 0; ch < KW / 32; ++ch) {
        const int kb = k0 + ch * 32;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const int t = tt * 16 + c;
            x[ch][tt] = (t < T && kb < H) ? *(const u4_t*)(X + (int64_t)t * H + kb + 8 * g)
                                          : u4_t{0u, 0u, 0u, 0u};
        }
    }
    stage_store<KW / 32>(v, lds);
    __syncthreads();
    f4_t acc[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = f4_t{0.f, 0.f, 0.f, 0.f};
    const int col = wave * 16 + c;
#pragma unroll
    for (int ch = 0; ch < KW / 32; ++ch) {
        if (k0 + ch * 32 >= H) break;
        const u4_t bw = lds_col8(lds, ch * 32, wave * 16);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[tt] = mfma_f<E>(x[ch][tt], bw, acc[tt]);
    }
    // lane holds tokens tt*16 + 4g + i, slab column wave*16 + c
    float* Ps = P + (int64_t)s * T * kN1 + slab * kSlabW + col;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tt * 16 + 4 * g + i;
            if (t < T) Ps[(int64_t)t * kN1] = acc[tt][i];
        }
}

// ---------------------------------------------------------------------------
// Finish of kv_a_proj, one workgroup per token t.  Wave w sums splits w,
// w+4, ... of the partials; wave 0 adds the four wave sums (fixed order),
// then lane l owns latent columns 8l..8l+7 and rope column l:
//   y     = c / sqrt(sum(c^2)/512 + eps) * gamma      -> compressed_kv
//   k_pe  = rotate-half RoPE of p at the token's position
// ---------------------------------------------------------------------------
template <int E>
__global__ __launch_bounds__(256) void dec_finish_kernel(const float* __restrict__ P, int S, int T,
                                                         const uint16_t* __restrict__ gamma,
                                                         const int32_t* __restrict__ pos,
                                                         float eps, RopeTab rt,
                                                         uint16_t* __restrict__ ckv,
                                                         uint16_t* __restrict__ kpe) {
    __shared__ __align__(16) float fred[4][kN1 + 4];
    const int t = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const u4_t gm = *(const u4_t*)(gamma + 8 * lane);
    const int32_t pos_t = pos[t];
    const double freq = rt.f[lane & 31];
    f4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    float p = 0.f;
    for (int s0 = wave; s0 < S; s0 += 16) {
        f4_t v0[4], v1[4];
        float vp[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int sp = s0 + 4 * u;
            if (sp < S) {
                const float* row = P + ((int64_t)sp * T + t) * kN1;
                v0[u] = *(const f4_t*)(row + 8 * lane);
                v1[u] = *(const f4_t*)(row + 8 * lane + 4);
                vp[u] = row[kR + lane];
            } else {
                v0[u] = v1[u] = f4_t{0.f, 0.f, 0.f, 0.f};
                vp[u] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c0 += v0[u];
            c1 += v1[u];
            p += vp[u];
        }
    }
    *(f4_t*)&fred[wave][8 * lane] = c0;
    *(f4_t*)&fred[wave][8 * lane + 4] = c1;
    fred[wave][kR + lane] = p;
    __syncthreads();
    if (wave != 0) return;
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        c[i] = (fred[0][8 * lane + i] + fred[1][8 * lane + i]) +
               (fred[2][8 * lane + i] + fred[3][8 * lane + i]);
    p = (fred[0][kR + lane] + fred[1][kR + lane]) + (fred[2][kR + lane] + fred[3][kR + lane]);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += c[i] * c[i];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)kR + eps);
    u4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float g0 = ld_to_f32<E>((uint16_t)(gm[w] & 0xFFFFu));
        const float g1 = ld_to_f32<E>((uint16_t)(gm[w] >> 16));
        const uint32_t y0 = f32_to_st<E>((c[2 * w] * inv) * g0);
        const uint32_t y1 = f32_to_st<E>((c[2 * w + 1] * inv) * g1);
        o[w] = y0 | (y1 << 16);
    }
    *(u4_t*)(ckv + (int64_t)t * kR + 8 * lane) = o;
    const float partner = __shfl_xor(p, 32, 64);
    float cs, sn;
    rope_cos_sin(pos_t, freq, cs, sn);
    const float out = (lane < 32) ? (p * cs - partner * sn) : (p * cs + partner * sn);
    kpe[(int64_t)t * kDR + lane] = f32_to_st<E>(out);
}

// ---------------------------------------------------------------------------
// kv_b_proj.  One workgroup per item of (16-token tile, 64-column slab);
// a slab of 64 columns is 64 consecutive entries of k_nope or of value of
// one head.  Item i = 8 j + x (x = i % 8, the XCD it lands on) covers slab
// 8 (j / ntile) + x and token tile j % ntile.
// ---------------------------------------------------------------------------
template <int E>
__global__ __launch_bounds__(256) void dec_kv_b_kernel(const uint16_t* __restrict__ Y,
                                                       const uint16_t* __restrict__ Wb, int T,
                                                       int N2, uint16_t* __restrict__ k_nope,
                                                       uint16_t* __restrict__ value) {
    __shared__ __align__(16) uint16_t lds[kR * kPitch];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    const int nh = N2 / kHeadW;
    const int ntile = (T + 15) / 16;
    const int item = blockIdx.x;
    const int x = item & 7, j = item >> 3;
    const int slab = (j / ntile) * 8 + x, tt = j % ntile;
    u4_t v[kR / 32];
    stage_load<kR / 32>(v, Wb, N2, 0, kR, slab * kSlabW);
    const int t = tt * 16 + c;
    u4_t y[kR / 32];
#pragma unroll
    for (int ch = 0; ch < kR / 32; ++ch)
        y[ch] = (t < T) ? *(const u4_t*)(Y + (int64_t)t * kR + ch * 32 + 8 * g) : u4_t{0u, 0u, 0u, 0u};
    stage_store<kR / 32>(v, lds);
    __syncthreads();
    const int col = wave * 16 + c;
    f4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < kR / 32; ++ch) acc = mfma_f<E>(y[ch], lds_col8(lds, ch * 32, wave * 16), acc);
    // lane holds tokens tt*16 + 4g + i of slab column col
    const int n = slab * kSlabW + col;
    const int h = n >> 8, sl = n & 255;
    uint16_t* dst = ((sl < kDN) ? k_nope : value) + (int64_t)h * kDN + (sl & 127);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = tt * 16 + 4 * g + i;
        if (tok < T) dst[(int64_t)tok * nh * kDN] = f32_to_st<E>(acc[i]);
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <int E, int NTT>
static void dec_launch_t(const void* X, const void* Wa, const void* gamma, const void* Wb,
                         const int32_t* pos, int T, int H, int nh, float eps, const RopeTab& rt,
                         void* k_nope, void* value, void* k_pe, void* ckv, float* P,
                         const Plan& plan, hipStream_t st) {
    const dim3 ga(kSlabsA * plan.s1), blk(256);
    const uint16_t* x = (const uint16_t*)X;
    const uint16_t* wa = (const uint16_t*)Wa;
    switch (plan.kw) {
        case 64: hipLaunchKernelGGL((dec_kv_a_kernel<E, NTT, 64>), ga, blk, 0, st, x, wa, T, H, P); break;
        case 128: hipLaunchKernelGGL((dec_kv_a_kernel<E, NTT, 128>), ga, blk, 0, st, x, wa, T, H, P); break;
        case 256: hipLaunchKernelGGL((dec_kv_a_kernel<E, NTT, 256>), ga, blk, 0, st, x, wa, T, H, P); break;
        default: hipLaunchKernelGGL((dec_kv_a_kernel<E, NTT, 512>), ga, blk, 0, st, x, wa, T, H, P); break;
    }
    hipLaunchKernelGGL(dec_finish_kernel<E>, dim3(T), blk, 0, st, (const float*)P, plan.s1, T,
                       (const uint16_t*)gamma, pos, eps, rt, (uint16_t*)ckv, (uint16_t*)k_pe);
    const int N2 = nh * kHeadW;
    const int nitems = (N2 / kSlabW) * ((T + 15) / 16);
    hipLaunchKernelGGL(dec_kv_b_kernel<E>, dim3(nitems), blk, 0, st, (const uint16_t*)ckv,
                       (const uint16_t*)Wb, T, N2, (uint16_t*)k_nope, (uint16_t*)value);
}

hipError_t launch_fp_decode(int dt, const void* X, const void* Wa, const void* gamma,
                            const void* Wb, const int32_t* pos, int64_t T, int H, int nh,
                            float eps, const RopeTab& rt, void* k_nope, void* value, void* k_pe,
                            void* ckv, void* ws, const Plan& plan, hipStream_t st) {
    float* P = (float*)((uint8_t*)ws + ws_fp(T, plan).p1);
    const int t = (int)T;
#define MLA_DEC(NT)                                                                          \
    if (dt == kF16)                                                                          \
        dec_launch_t<kF16, NT>(X, Wa, gamma, Wb, pos, t, H, nh, eps, rt, k_nope, value, k_pe, \
                               ckv, P, plan, st);                                            \
    else                                                                                     \
        dec_launch_t<kBF16, NT>(X, Wa, gamma, Wb, pos, t, H, nh, eps, rt, k_nope, value,     \
                                k_pe, ckv, P, plan, st);
    switch ((t + 15) / 16) {
        case 1: MLA_DEC(1) break;
        case 2: MLA_DEC(2) break;
        case 3: MLA_DEC(3) break;
        default: MLA_DEC(4) break;
    }
#undef MLA_DEC
    return hipGetLastError();
}

}  // namespace mla
