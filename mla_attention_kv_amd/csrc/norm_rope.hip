// Standalone RMSNorm and RoPE on gfx950: the prolog's two elementwise steps
// as operators of their own, with the same arithmetic as the prolog's finish
// kernels (rms_scale8, rope_cos_sin and rope_rotate are shared with them).
//
// The migration guide (DeepSeek-V2-Lite-Chat MLA KV Prolog migration guide,
// dpshk.com) ships both as separate kernels next to the fused prolog (section
// "Directory layout": rms_norm and rope kernel folders; the usage section
// for the fused operator: a switch for each); their definitions are the
// prolog's:
// RMSNorm over a row with eps inside the root and gamma after the
// normalisation, and rotate-half RoPE with frequencies theta^(-2i/dr)
// (section "Precision verification").
//
// Both are streaming operators (each byte read or written once), bound by
// HBM: 16-byte streaming loads and stores, rows processed by single waves
// so that no reduction crosses a wave.
#include "mla_common.h"

namespace mla {

// RMSNorm, one wave per row of n values (n a multiple of 8, at most
// 64 * 8 * NCH), four rows per workgroup.  Lane l holds the 8-value groups
// l, l + 64, ...; the whole row is loaded before any arithmetic, and every
// store depends on the row's reduction, so y may be x (no __restrict__).  The row's
// sum of squares accumulates per lane in group order and is then reduced
// across the wave, as in the prolog's finish.
template <int E, int NCH>
__global__ __launch_bounds__(256) void rms_norm_kernel(const uint16_t* x,
                                                       const uint16_t* __restrict__ gamma,
                                                       int64_t rows, int n, float eps,
                                                       uint16_t* y) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= rows) return;
    const int lane = threadIdx.x & 63;
    const int G = n >> 3;
    const uint16_t* xr = x + t * n;
    u4_t v[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int g = lane + 64 * i;
        v[i] = g < G ? __builtin_nontemporal_load((const u4_t*)(xr + 8 * g)) : u4_t{0, 0, 0, 0};
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a = ld_to_f32<E>((uint16_t)(v[i][w] & 0xFFFFu));
            const float b = ld_to_f32<E>((uint16_t)(v[i][w] >> 16));
            ss += a * a;
            ss += b * b;
        }
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)n + eps);
    uint16_t* yr = y + t * n;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int g = lane + 64 * i;
        if (g < G) {
            const u4_t gm = *(const u4_t*)(gamma + 8 * g);
            float c[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                c[2 * w] = ld_to_f32<E>((uint16_t)(v[i][w] & 0xFFFFu));
                c[2 * w + 1] = ld_to_f32<E>((uint16_t)(v[i][w] >> 16));
            }
            __builtin_nontemporal_store(rms_scale8<E>(c, inv, gm), (u4_t*)(yr + 8 * g));
        }
    }
}

// RoPE on rows of dr = 64 values, x [T, heads, 64], every head of token t
// rotated by positions[t].  A wave owns 8 R consecutive rows, eight at a
// time: lane l holds values 8 (l % 8) .. + 7 of row 8 i + l / 8, and its
// partner half sits in lane l ^ 4 of the same row.  All R loads are issued
// before any arithmetic.  Per value the arithmetic is the prolog's
// (rope_cos_sin on the frequency of index i mod 32, then rope_rotate); the
// cos / sin pairs of a lane depend only on the token, so they are computed
// again only when a lane's row moves to another token (with many heads per
// token, once per token instead of once per row).  A lane's stores depend
// on its own and its partner's loads, so y may be x.
template <int E, int R>
__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* x,
                                                   const int32_t* __restrict__ pos,
                                                   int64_t rows, int heads, RopeTab rt,
                                                   uint16_t* y) {
    const int lane = threadIdx.x & 63;
    const int part = lane & 7;  // 8-value group of the row
    const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (8 * R) + (lane >> 3);
    // rows past the end still take part in the shuffles (with zeros) and
    // then store nothing
    u4_t v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t row = base + 8 * i;
        v[i] = row < rows ? __builtin_nontemporal_load((const u4_t*)(x + row * kDR + 8 * part))
                          : u4_t{0, 0, 0, 0};
    }
    const bool first = part < 4;
    const int f0 = 8 * (part & 3);
    int64_t tok_prev = -1;
    float cs[8], sn[8];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t row = base + 8 * i;
        const bool live = row < rows;
        const int64_t tok = live ? row / heads : tok_prev;
        if (tok != tok_prev) {
            const int pt = pos[tok];
#pragma unroll
            for (int j = 0; j < 8; ++j) rope_cos_sin(pt, rt.f[f0 + j], cs[j], sn[j]);
            tok_prev = tok;
        }
        u4_t pv;
#pragma unroll
        for (int w = 0; w < 4; ++w) pv[w] = (uint32_t)__shfl_xor((int)v[i][w], 4, 64);
        u4_t o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t packed = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float a = ld_to_f32<E>((uint16_t)(h ? (v[i][w] >> 16) : (v[i][w] & 0xFFFFu)));
                const float b = ld_to_f32<E>((uint16_t)(h ? (pv[w] >> 16) : (pv[w] & 0xFFFFu)));
                packed |= (uint32_t)f32_to_st<E>(rope_rotate(a, b, cs[2 * w + h], sn[2 * w + h],
                                                             first))
                          << (16 * h);
            }
            o[w] = packed;
        }
        if (live) __builtin_nontemporal_store(o, (u4_t*)(y + row * kDR + 8 * part));
    }
}

hipError_t launch_rms_norm(int dt, const void* x, const void* gamma, int64_t rows, int n,
                           float eps, void* y, hipStream_t st) {
    const dim3 grid((unsigned)((rows + 3) / 4)), blk(256);
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* gp = (const uint16_t*)gamma;
    uint16_t* yp = (uint16_t*)y;
    const int nch = (n / 8 + 63) / 64;  // 1 .. 16
#define MLA_RMS(c)                                                                          \
    case c:                                                                                 \
        if (dt == kF16)                                                                     \
            hipLaunchKernelGGL((rms_norm_kernel<kF16, c>), grid, blk, 0, st, xp, gp, rows, n, \
                               eps, yp);                                                    \
        else                                                                                \
            hipLaunchKernelGGL((rms_norm_kernel<kBF16, c>), grid, blk, 0, st, xp, gp, rows, \
                               n, eps, yp);                                                 \
        break;
    switch (nch) {
        MLA_RMS(1) MLA_RMS(2) MLA_RMS(3) MLA_RMS(4) MLA_RMS(5) MLA_RMS(6) MLA_RMS(7) MLA_RMS(8)
        MLA_RMS(9) MLA_RMS(10) MLA_RMS(11) MLA_RMS(12) MLA_RMS(13) MLA_RMS(14) MLA_RMS(15)
        MLA_RMS(16)
        default: return hipErrorInvalidValue;
    }
#undef MLA_RMS
    return hipGetLastError();
}

template <int R>
static void rope_launch(int dt, const void* x, const int32_t* pos, int64_t rows, int heads,
                        const RopeTab& rt, void* y, hipStream_t st) {
    const dim3 grid((unsigned)((rows + 32 * R - 1) / (32 * R))), blk(256);  // 32 R rows each
    if (dt == kF16)
        hipLaunchKernelGGL((rope_kernel<kF16, R>), grid, blk, 0, st, (const uint16_t*)x, pos, rows,
                           heads, rt, (uint16_t*)y);
    else
        hipLaunchKernelGGL((rope_kernel<kBF16, R>), grid, blk, 0, st, (const uint16_t*)x, pos,
                           rows, heads, rt, (uint16_t*)y);
}

hipError_t launch_rope(int dt, const void* x, const int32_t* pos, int64_t T, int heads,
                       const RopeTab& rt, void* y, hipStream_t st) {
    const int64_t rows = T * heads;
    // rows per wave: as many as keep at least ~2048 workgroups in the grid
    // (and one token's cos / sin reused over several of its heads)
    if (rows >= (int64_t)2048 * 32 * 8) rope_launch<8>(dt, x, pos, rows, heads, rt, y, st);
    else if (rows >= (int64_t)2048 * 32 * 4) rope_launch<4>(dt, x, pos, rows, heads, rt, y, st);
    else if (rows >= (int64_t)2048 * 32 * 2) rope_launch<2>(dt, x, pos, rows, heads, rt, y, st);
    else rope_launch<1>(dt, x, pos, rows, heads, rt, y, st);
    return hipGetLastError();
}

}  // namespace mla
