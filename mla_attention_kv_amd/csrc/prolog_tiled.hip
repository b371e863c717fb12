// Tiled gfx950 kernels of the MLA KV prolog: both projections as MFMA GEMMs
// (gemm_lds_kernel: persistent, copy waves stream slabs straight into a ring
// of LDS stages, fp16 / bf16 / int8, optional split-K; gemm_tiled_kernel:
// register-staged slabs, for W8A8 calls of up to 64 tokens and the forced
// small-tile path), plus the per-token kernels that finish kv_a_proj (split,
// RMSNorm, RoPE) and, on the W8A8 path, quantise the activations.
//
// Steps follow the DeepSeek-V2-Lite-Chat MLA KV Prolog migration guide
// (dpshk.com), sections "Background" and "Source-level principle"; RoPE is
// the rotate-half x*cos + x_rot*sin form of its "Precision verification"
// section.  The W8A8 scheme is the per-token / per-output-column int8 one
// stated in include/libmlaprolog.h.
#include "mla_common.h"

namespace mla {

// ---------------------------------------------------------------------------
// MFMA 16x16 step over 64 bytes of K per lane group:
//   fp16/bf16: v_mfma_f32_16x16x32_{f16,bf16}  (8 elements per lane)
//   int8:      v_mfma_i32_16x16x64_i8          (16 elements per lane)
// Operand lane layout: lane l supplies row (A) / column (B) l%16 and the
// 16-byte K slice (l/16); result lane l holds rows 4*(l/16)+i, column l%16.
// ---------------------------------------------------------------------------
template <int E>
struct Acc { typedef f4_t type; };
template <>
struct Acc<kI8> { typedef i4_t type; };

template <int E>
__device__ __forceinline__ typename Acc<E>::type mfma16(u4_t a, u4_t b, typename Acc<E>::type c) {
    if constexpr (E == kF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                      __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
    } else if constexpr (E == kBF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a),
                                                       __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, a),
                                                     __builtin_bit_cast(i4_t, b), c, 0, 0, 0);
    }
}

// 8x8 transpose of 16-bit values: in[i] = row i (8 columns), out[j] = column
// j (8 rows).
__device__ __forceinline__ void transpose8x8_b16(const u4_t in[8], u4_t out[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            uint32_t lo = in[2 * v][j >> 1], hi = in[2 * v + 1][j >> 1];
            out[j][v] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u))
                                : ((lo & 0xFFFFu) | (hi << 16));
        }
    }
}

// 16x16 transpose of bytes: in[i] = row i (16 columns), out[j] = column j.
__device__ __forceinline__ void transpose16x16_b8(const u4_t in[16], u4_t out[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int w = j >> 2, sh = (j & 3) * 8;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            uint32_t b0 = (in[4 * v + 0][w] >> sh) & 0xFFu;
            uint32_t b1 = (in[4 * v + 1][w] >> sh) & 0xFFu;
            uint32_t b2 = (in[4 * v + 2][w] >> sh) & 0xFFu;
            uint32_t b3 = (in[4 * v + 3][w] >> sh) & 0xFFu;
            out[j][v] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
    }
}

// ---------------------------------------------------------------------------
// Epilogues.  row_scale(row) / col_scale(col) are fetched once per row and
// column a lane owns; value() turns one accumulator into the stored element.
// The kernel gathers a whole output tile in LDS and then writes it with
// 16-byte stores along rows, each to ptr(row, col) (col is a multiple of the
// 16-byte chunk, and a tile never straddles a k_nope / value boundary).
// ---------------------------------------------------------------------------
struct NoScale {};
struct EpiPartialF32 {  // kv_a_proj split-K partial, fp32 [s][T][576]
    typedef float out_t;
    static constexpr bool kScaleDma = false;
    typedef NoScale row_t;
    float* out;
    int64_t T;
    __device__ __forceinline__ row_t row_scale(int) const { return {}; }
    __device__ __forceinline__ float col_scale(int) const { return 1.f; }
    __device__ __forceinline__ float value(int, int, float v, row_t, float) const { return v; }
    __device__ __forceinline__ void* ptr(int row, int col, int s) const {
        return out + ((int64_t)s * T + row) * kN1 + col;
    }
};
struct EpiPartialI32 {  // kv_a_proj split-K partial, int32 [s][T][576]
    typedef int32_t out_t;
    static constexpr bool kScaleDma = false;
    typedef NoScale row_t;
    int32_t* out;
    int64_t T;
    __device__ __forceinline__ row_t row_scale(int) const { return {}; }
    __device__ __forceinline__ float col_scale(int) const { return 1.f; }
    __device__ __forceinline__ int32_t value(int, int, int v, row_t, float) const { return v; }
    __device__ __forceinline__ void* ptr(int row, int col, int s) const {
        return out + ((int64_t)s * T + row) * kN1 + col;
    }
};
// kv_b_proj result column `col` = head col/256, slot col%256: slots [0,128)
// are k_nope, [128,256) are value.
__device__ __forceinline__ uint16_t* kv_dst(uint16_t* k_nope, uint16_t* value, int nh, int row,
                                            int col) {
    const int h = col >> 8, sl = col & 255;
    return ((sl < kDN) ? k_nope : value) + ((int64_t)row * nh + h) * kDN + (sl & 127);
}
// Two results rounded to nearest even into one packed 2-byte pair
// (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
template <int OE>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
    if constexpr (OE == kF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2_t));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, b2_t));
}

// Epilogues with 2-byte results also give valuef() (the result before
// rounding; kOut names its storage type) and say whether they carry an
// accumulator debug copy (kDbg, dbg_store()).  kScaleDma: the pipelined
// kernel's copy waves bring each tile's scales into LDS (scale_src());
// row_scale2() then combines the two row values read back from there.
template <int E>
struct EpiKvFp {
    typedef uint16_t out_t;
    typedef NoScale row_t;
    static constexpr int kOut = E;
    static constexpr bool kDbg = false;
    static constexpr bool kScaleDma = false;
    uint16_t* k_nope;
    uint16_t* value_out;
    int nh;
    __device__ __forceinline__ row_t row_scale(int) const { return {}; }
    __device__ __forceinline__ float col_scale(int) const { return 1.f; }
    __device__ __forceinline__ uint16_t value(int, int, float v, row_t, float) const {
        return f32_to_st<E>(v);
    }
    __device__ __forceinline__ float valuef(float v, row_t, float) const { return v; }
    __device__ __forceinline__ void dbg_store(int, int, float) const {}
    __device__ __forceinline__ void* ptr(int row, int col, int) const {
        return kv_dst(k_nope, value_out, nh, row, col);
    }
};
struct EpiKvW8 {
    typedef uint16_t out_t;
    typedef float row_t;  // the token's activation scale times its RMS factor
    static constexpr int kOut = kBF16;
    static constexpr bool kDbg = true;
    static constexpr bool kScaleDma = true;
    // 16-byte source of lane group q (16 lanes, 64 values) for rows m.. and
    // columns n.. of a wave tile WN columns wide.  WN = 64: column scales
    // (q = 0, and 3 as filler), activation scales (q = 1), RMS factors
    // (q = 2).  WN = 128: column scales (q = 0, 1), activation scales
    // (q = 2), RMS factors (q = 3).  The two row arrays are padded to whole
    // 256-row tiles.
    template <int WN>
    __device__ __forceinline__ const void* scale_src(int q, int m, int n) const {
        // the addresses first, then a per-lane choice of value (a choice of
        // member would make the compiler load the pointer per lane)
        const uintptr_t a = (uintptr_t)(sz + m), b = (uintptr_t)(inv_t + m), c = (uintptr_t)(swb + n);
        if constexpr (WN == 128) {
            const uintptr_t c1 = (uintptr_t)(swb + n + 64);
            const uintptr_t r = q == 1 ? c1 : c;
            const uintptr_t t = q == 2 ? a : r;
            return (const void*)(q == 3 ? b : t);
        } else {
            const uintptr_t r = q == 1 ? a : c;
            return (const void*)(q == 2 ? b : r);
        }
    }
    __device__ __forceinline__ row_t row_scale2(float s, float i) const { return s * i; }
    uint16_t* k_nope;
    uint16_t* value_out;
    int nh;
    const float* sz;
    const float* inv_t;
    const float* swb;
    int32_t* dbg;
    int64_t dbg_begin, dbg_rows;
    __device__ __forceinline__ row_t row_scale(int row) const { return sz[row] * inv_t[row]; }
    __device__ __forceinline__ float col_scale(int col) const { return swb[col]; }
    __device__ __forceinline__ uint16_t value(int row, int col, int acc, row_t rs, float cs) const {
        if (dbg != nullptr && row >= dbg_begin && row < dbg_begin + dbg_rows)
            dbg[(row - dbg_begin) * (int64_t)nh * kHeadW + col] = acc;
        return f32_to_bf16(((float)acc * rs) * cs);
    }
    __device__ __forceinline__ float valuef(int acc, row_t rs, float cs) const {
        return ((float)acc * rs) * cs;
    }
    // the raw accumulator of (row, col), kept when row is in the debug range
    __device__ __forceinline__ void dbg_store(int row, int col, int acc) const {
        if (row >= dbg_begin && row < dbg_begin + dbg_rows)
            dbg[(row - dbg_begin) * (int64_t)nh * kHeadW + col] = acc;
    }
    __device__ __forceinline__ void* ptr(int row, int col, int) const {
        return kv_dst(k_nope, value_out, nh, row, col);
    }
};

// Store `n` bytes (4, 8 or 16) of v to LDS.
template <int NB>
__device__ __forceinline__ void lds_store(uint8_t* p, const uint32_t* v) {
    if constexpr (NB == 16) *(u4_t*)p = u4_t{v[0], v[1], v[2], v[3]};
    else if constexpr (NB == 8) *(u2_t*)p = u2_t{v[0], v[1]};
    else *(uint32_t*)p = v[0];
}

// ---------------------------------------------------------------------------
// C[M, N] = A[M, K] . B[K, N]; A and B row-major, K consumed in 128-byte
// slabs (64 fp16/bf16 or 128 int8 elements = two MFMA K steps).
//
// Grid: one workgroup per (split, M tile, N tile), 256 threads = 4 waves
// laid out (BM/WM) x (BN/WN), each wave owning a WM x WN block of 16x16
// MFMA tiles.  Tile order is XCD-aware: workgroup b runs on XCD b % 8
// (round-robin dispatch), each XCD takes a contiguous chunk of the tile
// list, and the list walks groups of GM M tiles N-major, so an XCD's L2
// keeps a group's A rows while the B tiles stream past them.
//
// Per slab: every thread fetches its share of the A slab (16-byte chunks)
// and of the B slab (a block of BR rows x 16 bytes, transposed in registers
// so that LDS holds B as [n][k]); both MFMA operands are then 16-byte K
// slices.  The B rows' 16-byte K units are XOR-swizzled by (n / 8) % 8, so
// the transposed stores of neighbouring column blocks land on different
// banks.  LDS holds two slabs: while one is multiplied the next is stored,
// and the one after that is already being fetched into registers; one
// barrier per slab.  The output tile is gathered in LDS and written with
// 16-byte row stores.
// ---------------------------------------------------------------------------
template <int E, int BM, int BN, int WM, int WN, int GM, class Epi>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    int M, int Nt, int S, int kslabs_per_split, int kslabs_total, Epi epi) {
    constexpr int KB = 128;           // bytes of K per slab
    constexpr int ST = KB + 16;       // LDS row stride in bytes (padding vs bank conflicts)
    constexpr int ES = (E == kI8) ? 1 : 2;
    constexpr int KE = KB / ES;       // K elements per slab
    constexpr int WAVES_N = BN / WN;
    static_assert((BM / WM) * WAVES_N == 4, "4 waves");
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int A_CHUNKS = BM * (KB / 16);            // 16-byte chunks in an A slab
    constexpr int A_PER_T = (A_CHUNKS + 255) / 256;
    constexpr int BC = 16 / ES;                         // columns per B block (16 bytes)
    constexpr int BR0 = (KE * BN) / (BC * 256);          // rows per block for one per thread
    constexpr int BR = BR0 * ES >= 4 ? BR0 : 4 / ES;      // at least 4 bytes per column
    constexpr int B_BLOCKS = (KE / BR) * (BN / BC);
    constexpr int BW = BR * ES;                         // bytes per column after transposing
    static_assert(B_BLOCKS <= 256 && BW >= 4 && BW <= 16, "B block shape");

    typedef typename Epi::out_t out_t;
    constexpr int CST = BN + 16 / (int)sizeof(out_t);   // C tile row pitch (elements)
    constexpr int STAGE = (BM + BN) * ST;
    constexpr int AB_BYTES = 2 * STAGE;
    constexpr int C_BYTES = BM * CST * (int)sizeof(out_t);
    __shared__ __align__(16) uint8_t smem[AB_BYTES > C_BYTES ? AB_BYTES : C_BYTES];

    // ---- tile of this workgroup
    const int Mt = (M + BM - 1) / BM;
    const int tiles = Mt * Nt * S;
    const int per = (tiles + 7) / 8;
    const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (t >= tiles) return;
    const int s = t / (Mt * Nt);
    const int rr = t - s * Mt * Nt;
    const int grp = rr / (GM * Nt);
    const int gm = min(GM, Mt - grp * GM);
    const int q = rr - grp * GM * Nt;
    const int m0 = (grp * GM + q % gm) * BM, n0 = (q / gm) * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;
    const int kc0 = s * kslabs_per_split;
    const int kc1 = min(kc0 + kslabs_per_split, kslabs_total);

    typedef typename Acc<E>::type acc_t;
    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

    u4_t ra[A_PER_T];
    u4_t rb[BR];
    const int b_rb = tid / (BN / BC), b_cb = tid % (BN / BC);

    auto gload = [&](int kc) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int c = tid + i * 256;
            if (c < A_CHUNKS) {
                const int row = c >> 3, c16 = c & 7;
                u4_t v = {0u, 0u, 0u, 0u};
                if (m0 + row < M)
                    v = *(const u4_t*)(A + (int64_t)(m0 + row) * lda + (int64_t)kc * KB + c16 * 16);
                ra[i] = v;
            }
        }
        if (tid < B_BLOCKS) {
            const uint8_t* src = B + ((int64_t)kc * KE + b_rb * BR) * ldb + (int64_t)(n0 + b_cb * BC) * ES;
#pragma unroll
            for (int i = 0; i < BR; ++i) rb[i] = *(const u4_t*)(src + (int64_t)i * ldb);
        }
    };
    auto lstore = [&](uint8_t* stage) {
        uint8_t* As = stage;
        uint8_t* Bs = stage + BM * ST;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int c = tid + i * 256;
            if (c < A_CHUNKS) {
                const int row = c >> 3, c16 = c & 7;
                *(u4_t*)(As + row * ST + c16 * 16) = ra[i];
            }
        }
        if (tid < B_BLOCKS) {
            // column j of the block: its BR elements, packed along K
#pragma unroll
            for (int j = 0; j < BC; ++j) {
                uint32_t col[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < BR; ++i) {
                    uint32_t e;
                    if constexpr (ES == 2) e = (rb[i][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                    else e = (rb[i][j >> 2] >> (8 * (j & 3))) & 0xFFu;
                    const int bit = i * ES * 8;
                    col[bit >> 5] |= e << (bit & 31);
                }
                const int n = b_cb * BC + j;
                lds_store<BW>(Bs + n * ST + ((b_rb * BW) ^ (((n >> 3) & 7) << 4)), col);
            }
        }
    };
    auto compute = [&](const uint8_t* stage) {
        const uint8_t* As = stage;
        const uint8_t* Bs = stage + BM * ST;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u4_t a[TM], b[TN];
            const int kofs = ks * 64 + (lane >> 4) * 16;
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = *(const u4_t*)(As + (wm0 + i * 16 + (lane & 15)) * ST + kofs);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = wn0 + j * 16 + (lane & 15);
                b[j] = *(const u4_t*)(Bs + n * ST + (kofs ^ (((n >> 3) & 7) << 4)));
            }
            // operands swapped (C^T = B^T A^T): lane l then holds output row
            // (l % 16) and the 4 consecutive output columns 4 (l / 16) + v
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma16<E>(b[j], a[i], acc[i][j]);
        }
    };

    if (kc0 < kc1) {
        gload(kc0);
        lstore(smem);
        __syncthreads();
        if (kc0 + 1 < kc1) gload(kc0 + 1);
        for (int kc = kc0; kc < kc1; ++kc) {
            const int cur = (kc - kc0) & 1;
            compute(smem + cur * STAGE);
            if (kc + 1 < kc1) {
                lstore(smem + (cur ^ 1) * STAGE);
                if (kc + 2 < kc1) gload(kc + 2);
            }
            __syncthreads();
        }
    }

    // epilogue: gather the tile in LDS (the K loop ended with a barrier, so
    // the staging area is free), then store 16-byte row chunks
    out_t* Ct = (out_t*)smem;
    float cs[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) cs[j][v] = epi.col_scale(n0 + wn0 + j * 16 + (lane >> 4) * 4 + v);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm0 + i * 16 + (lane & 15);
        // rows past M are padding: never handed to the epilogue
        const bool live = m0 + r < M;
        const typename Epi::row_t rs = epi.row_scale(live ? m0 + r : 0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int cl = wn0 + j * 16 + (lane >> 4) * 4;
            out_t o[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                o[v] = live ? epi.value(m0 + r, n0 + cl + v, acc[i][j][v], rs, cs[j][v]) : out_t(0);
            if constexpr (sizeof(out_t) == 2)
                *(u2_t*)&Ct[r * CST + cl] = u2_t{(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                 (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
            else
                *(u4_t*)&Ct[r * CST + cl] = u4_t{__builtin_bit_cast(uint32_t, o[0]),
                                                 __builtin_bit_cast(uint32_t, o[1]),
                                                 __builtin_bit_cast(uint32_t, o[2]),
                                                 __builtin_bit_cast(uint32_t, o[3])};
        }
    }
    __syncthreads();
    constexpr int EPC = 16 / (int)sizeof(out_t);
    constexpr int CPR = BN / EPC;
    for (int c = tid; c < BM * CPR; c += 256) {
        const int r = c / CPR, cc = c % CPR;
        if (m0 + r < M) *(u4_t*)epi.ptr(m0 + r, n0 + cc * EPC, s) = *(const u4_t*)&Ct[r * CST + cc * EPC];
    }
}

// ---------------------------------------------------------------------------
// Pipelined GEMM with direct-to-LDS loads and copy waves (fp16 / bf16 / int8).
// C[M, N] = A[M, K] . B[K, N]; A, B row-major; one slab = 128 bytes of an A
// row (64 fp16 / bf16 or 128 int8 K elements), K a multiple of a slab, N a
// multiple of BN.
//
// A workgroup has WAVES_M x WAVES_N MFMA waves and NP copy waves.  Each slab
// of A (BM rows x 128 bytes) and of B (one row per K element of the slab, BN
// columns) goes from global memory straight into one of STAGES LDS stages
// (global_load_lds_dwordx4: one wave instruction fills 1 KB of LDS, lane l
// the 16 bytes at l * 16), so the prefetch depth costs no registers.  Only
// the copy waves issue copies and wait on the vector-memory counter; the
// MFMA waves never wait for their output stores, which drain while the next
// tile is multiplied.
//
// One barrier per slab g (B_g) orders the two roles:
//   copy waves:  wait for their copies of slab g, B_g, copy slab
//                g + STAGES - 1 into the stage that held slab g - 1
//   MFMA waves:  MFMAs of slab g - 1's first K step, every LDS read of slab
//                g - 1 back in registers (lgkmcnt 0), B_g, reads of slab g's
//                first K step, MFMAs of slab g - 1's second K step
// so a stage is read only after its copies have landed and overwritten only
// after every MFMA wave has finished reading it.  The slabs of all of a
// workgroup's tiles form one sequence (slab gs is tile gs / nk, slab
// gs % nk, stage gs % STAGES); both roles step through it incrementally.
//
// LDS layouts (bank-conflict swizzles, done by choosing which global chunk
// each lane copies, since a copy's LDS destination is fixed):
//   A stage: [BM rows][8 chunks of 16 bytes]; chunk c of row r sits at
//            position c ^ ((r >> 1) & 7).  An MFMA A operand (16 rows, one
//            chunk each) then touches 16 distinct 16-byte bank groups.
//   B stage: [KE k rows][BN columns] (64 rows of fp16 / bf16, 128 of
//            int8); 16-byte chunk c of row k sits at
//            c ^ (2 (k & 3) + 8 ((k >> 3) & 1)) (c ^ 2 (k & 3) when a row is
//            not a multiple of 16 chunks; c ^ (k & 7) for int8) of LDS row
//            brow(k) (k itself, or k with its low bit(s) flipped where two
//            lane groups of one half-wave would otherwise share banks).  The
//            B operand (column n, 8 or 16 consecutive k) comes from two
//            transposing reads: ds_read_b64_tr_b16 (4 rows x 4 columns per
//            16-lane group) or ds_read_b64_tr_b8 (8 rows x 8 columns).
// MFMA waves are laid out WAVES_M x WAVES_N, each owning a (BM / WAVES_M) x
// (BN / WAVES_N) block of 16 x 16 MFMA tiles; A fragments are held once and
// refilled row by row as their MFMAs issue, B fragments in two sets a K step
// ahead.  Tile order is the same XCD-aware grouped order as
// gemm_tiled_kernel.  Epilogue: 2-byte results are rounded in pairs, staged
// in the wave's own 2 KB of LDS and stored as whole 128-byte lines with
// streaming stores; fp32 / int32 split-K partials are stored from the
// accumulators (lane: one row, four consecutive columns).  The MFMA waves
// issue no global loads (their vector-memory counter also counts their
// stores): epilogue scales, where there are any, arrive in the staging area
// through the copy waves.
// ---------------------------------------------------------------------------
typedef short v4s_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr16(const uint8_t* p) {
    const v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s_t*)(p));
    return __builtin_bit_cast(uint2, r);
}
// One 16-byte-per-lane copy from global memory into LDS (the wave's 64
// lanes fill lds .. lds + 1023; lds is wave-uniform).  Issued from inline
// assembly so that the compiler, which cannot tell the LDS stages apart,
// does not wait for these copies before unrelated LDS reads; M0 (the LDS
// base the instruction reads at issue) is saved and restored around it.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(g)
        : "memory");
}
// The same copy with the non-temporal (streaming) hint, for data that no
// other workgroup reads.
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(g)
        : "memory");
}
// Wait until at most N of this wave's copies are outstanding, then
// barrier; a compiler memory barrier as well.
template <int N>
__device__ __forceinline__ void wait_copies_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
// B-row chunk swizzle (16-byte chunk c of row k is stored at c ^ bswz(k)):
// 16-bit rows of 16 chunks or more (BN >= 128) use 2 (k & 3) + 8 ((k >> 3) & 1);
// other 16-bit rows (BN = 64 or 192) stay inside aligned groups of 8 chunks
// with 2 (k & 3); int8 rows use k & 7, or (k >> 1) & 3 for 12-chunk rows (a
// transposing 8-bit read touches one chunk in each of 8 consecutive rows).
template <int E, int BRB>
__device__ __forceinline__ int bswz(int k) {
    if constexpr (E == kI8 && BRB % 128 == 0) return k & 7;
    else if constexpr (E == kI8) return (k >> 1) & 3;  // 12-chunk rows (BN = 192)
    else if constexpr (BRB % 256 == 0) return 2 * (k & 3) + 8 * ((k >> 3) & 1);
    else return 2 * (k & 3);
}
// LDS row of B row k: rows whose second lane group of a transposing read
// would otherwise hit the first group's banks (the two groups of a half-wave
// read rows 8 (16-bit) or 16 (int8) apart, and with 384-, 128- or 192-byte
// rows those land on the same bank slots) swap places with a neighbour, which
// moves them to the other half of the 256-byte bank span:
//   16-bit, rows of 24 chunks: k ^ 1 when bit 3 of k is set;
//   int8, 8-chunk rows: k ^ 1 when bit 4 is set; 12-chunk rows: k ^ 2.
// An involution inside each slab (bits 3 and 4 are unchanged), so the copy
// waves use it to find the source row of an LDS row as well.
template <int E, int BRB>
__device__ __forceinline__ int brow(int k) {
    if constexpr (E == kI8 && BRB % 128 == 0) return k ^ ((k >> 4) & 1);
    else if constexpr (E == kI8) return k ^ (2 * ((k >> 4) & 1));
    else if constexpr (BRB % 256 == 0) return k;
    else return k ^ ((k >> 3) & 1);
}
typedef int v2i_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_tr8(const uint8_t* p) {
    const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i_t*)(p));
    return __builtin_bit_cast(uint2, r);
}

template <int E, int BM, int BN, int WAVES_M, int WAVES_N, int NP, int STAGES, int GM, int WGPC,
          class Epi>
__global__ __launch_bounds__(64 * (WAVES_M * WAVES_N + NP),
                             (WGPC * (WAVES_M * WAVES_N + NP) + 3) / 4) void gemm_lds_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    int M, int Nt, int nk, int S, Epi epi) {
    constexpr int ES = (E == kI8) ? 1 : 2;    // bytes per element
    constexpr int KE = 128 / ES;              // K elements per slab (128 bytes of an A row)
    constexpr int NC = WAVES_M * WAVES_N;     // MFMA waves
    constexpr int A_ST = BM * 128;            // A bytes per stage
    constexpr int BRB = BN * ES;              // bytes per B row
    constexpr int B_ST = KE * BRB;            // B bytes per stage (KE rows)
    constexpr int STAGE = A_ST + B_ST;
    constexpr int A_PW = A_ST / 1024 / NP, B_PW = B_ST / 1024 / NP;
    static_assert(A_PW * NP * 1024 == A_ST && B_PW * NP * 1024 == B_ST, "even copy split");
    static_assert(BRB % 128 == 0 || (E == kI8 && BRB == 192), "B row swizzle groups");
    constexpr int PW = A_PW + B_PW;           // copy instructions per copy wave per slab
    static_assert(STAGES >= 2 && (STAGES - 2) * PW < 64, "stages / vmcnt range");
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, TM = WM / 16, TN = WN / 16;
    // 2-byte results are staged per wave (16 rows of the wave's WN columns:
    // 128 or 256 bytes) so that every store writes whole 128-byte lines
    constexpr bool STAGE_OUT = sizeof(typename Epi::out_t) == 2;
    static_assert(!STAGE_OUT || WN == 64 || WN == 128, "128- or 256-byte wave rows");
    constexpr int RP = WN * 2;                    // staged row pitch (bytes)
    constexpr int AREA = 16 * RP;                 // a wave's staging area
    constexpr int OUT_ST = STAGE_OUT ? NC * AREA : 0;
    __shared__ __align__(1024) uint8_t smem[STAGES * STAGE + OUT_ST];

    // ---- work items: (tile, K split) pairs, split-major, so that an XCD's
    // range holds the tiles of one split.  Workgroup b runs on XCD b % 8;
    // XCD x owns the contiguous item range [x per, (x + 1) per) of the
    // grouped order and its workgroups walk it in steps of (grid / 8).  Item
    // (t, s) covers slabs [s nk, (s + 1) nk) of K.
    const int Mt = (M + BM - 1) / BM;
    const int tiles = Mt * Nt * S;
    const int per = (tiles + 7) / 8;
    const int x = blockIdx.x & 7, nwx = gridDim.x >> 3;
    const int first = x * per + (blockIdx.x >> 3);
    const int lim = min(tiles, (x + 1) * per);
    const int ntl = first < lim ? (lim - first + nwx - 1) / nwx : 0;
    if (ntl == 0) return;
    const int total = ntl * nk;  // slabs of all tiles, in order
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto tile_origin = [&](int i, int& m0, int& n0, int& sk) {
        const int w = first + i * nwx;
        sk = w / (Mt * Nt);
        const int t = w - sk * (Mt * Nt);
        const int grp = t / (GM * Nt);
        const int gm = min(GM, Mt - grp * GM);
        const int q = t - grp * GM * Nt;
        m0 = (grp * GM + q % gm) * BM;
        n0 = (q / gm) * BN;
    };

    if (wave >= NC) {
        // ================= copy wave p =================
        // instruction u covers LDS bytes [(p + NP u) KB, +1 KB) of the A
        // (resp. B) part of a stage
        const int p = wave - NC;
        int arow[A_PW], acol[A_PW];
#pragma unroll
        for (int u = 0; u < A_PW; ++u) {
            arow[u] = (p + NP * u) * 8 + (lane >> 3);
            acol[u] = ((lane & 7) ^ ((arow[u] >> 1) & 7)) * 16;
        }
        int64_t boff[B_PW];
#pragma unroll
        for (int u = 0; u < B_PW; ++u) {
            // the LDS row this lane fills holds B row k (brow is its own
            // inverse), swizzled chunk pos
            const int byte = (p + NP * u) * 1024 + lane * 16;
            const int k = brow<E, BRB>(byte / BRB), pos = (byte % BRB) / 16;
            boff[u] = (int64_t)k * ldb + (pos ^ bswz<E, BRB>(k)) * 16;
        }
        const int64_t bstep = KE * ldb;  // bytes of B per slab
        const uint32_t base0 =
            lds_addr(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(p * 1024);
        const uint8_t* pa[A_PW];
        const uint8_t* pb[B_PW];
        // next slab to copy: slab kc of item ti (origin tm0, tn0), into the
        // stage at byte sofs
        int ti = 0, kc = 0, tm0 = 0, tn0 = 0;
        uint32_t sofs = 0;
        auto issue = [&]() {
            if constexpr (STAGE_OUT && Epi::kScaleDma) {
                // with slab STAGES of a tile (issued after the barrier that
                // follows the MFMA waves' previous epilogue, landed before
                // the barrier that ends the tile): the tile's scales into
                // the staging areas of MFMA waves p, p + NP, ...; lane group
                // q of the 1 KB copy fills bytes 256 q .. of an area
                if (kc == STAGES) {
#pragma unroll
                    for (int w = p; w < NC; w += NP) {
                        const int r4 = (lane & 15) * 4;
                        dma16(epi.template scale_src<WN>(lane >> 4, tm0 + (w / WAVES_N) * WM + r4,
                                                         tn0 + (w % WAVES_N) * WN + r4),
                              lds_addr(smem + STAGES * STAGE) +
                                  (uint32_t)__builtin_amdgcn_readfirstlane(w * AREA));
                    }
                }
            }
            if (kc == 0) {
                int m0, n0, sk;
                tile_origin(ti, m0, n0, sk);
                tm0 = m0;
                tn0 = n0;
                const int64_t k0 = (int64_t)sk * nk;  // first slab of the item's split
#pragma unroll
                for (int u = 0; u < A_PW; ++u)
                    pa[u] = A + (int64_t)min(m0 + arow[u], M - 1) * lda + k0 * 128 + acol[u];
#pragma unroll
                for (int u = 0; u < B_PW; ++u) pb[u] = B + k0 * bstep + (int64_t)n0 * ES + boff[u];
            }
            const uint32_t base = base0 + sofs;
#pragma unroll
            for (int u = 0; u < A_PW; ++u) dma16(pa[u] + kc * 128, base + u * NP * 1024);
            if (Mt == 1) {
                // a single row of tiles: each B slab is read by this
                // workgroup only
#pragma unroll
                for (int u = 0; u < B_PW; ++u)
                    dma16_nt(pb[u] + kc * bstep, base + A_ST + u * NP * 1024);
            } else {
#pragma unroll
                for (int u = 0; u < B_PW; ++u)
                    dma16(pb[u] + kc * bstep, base + A_ST + u * NP * 1024);
            }
            sofs = (sofs + STAGE == (uint32_t)(STAGES * STAGE)) ? 0u : sofs + STAGE;
            if (++kc == nk) {
                kc = 0;
                ++ti;
            }
        };
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < total) issue();
        for (int g = 0; g < total; ++g) {
            // slabs g + 1 .. g + STAGES - 2 may stay in flight
            if (g + STAGES - 2 < total) wait_copies_barrier<(STAGES - 2) * PW>();
            else wait_copies_barrier<0>();
            if (g + STAGES - 1 < total) issue();
        }
        // the MFMA waves' last barrier (after their last slab's first K step)
        asm volatile("s_barrier" ::: "memory");
        return;
    }

    // ================= MFMA waves =================
    const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;
    typedef typename Acc<E>::type acc_t;
    acc_t acc[TM][TN];

    const int l16 = lane & 15, g = lane >> 4;
    // operand fragments: A in one register set, each row of MFMA tiles
    // re-read for the next K step as soon as its MFMAs are issued; B (two
    // transposing reads per fragment) in two sets, read a whole K step ahead
    u4_t fa[TM], fb[2][TN];
    auto rd_a = [&](const uint8_t* stg, int ks, int i) {
        const int row = wm0 + i * 16 + l16;
        const int c = (ks * 4 + g) ^ ((row >> 1) & 7);
        fa[i] = *(const u4_t*)(stg + row * 128 + c * 16);
    };
    auto rd_b = [&](const uint8_t* stg, int ks, int buf) {
        const uint8_t* Bs = stg + A_ST;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if constexpr (ES == 2) {
                // lane (16 g + s): rows 32 ks + 8 g + s / 4 (+ 4), columns
                // wn0 + 16 j + 4 (s % 4) .. + 3; lane s receives 4 rows of
                // column wn0 + 16 j + s per read
                const int k = ks * 32 + g * 8 + (l16 >> 2);
                const int colb = (wn0 + j * 16 + 4 * (l16 & 3)) * 2;
                const int c = colb >> 4, off = colb & 15;
                const uint2 lo =
                    lds_tr16(Bs + brow<E, BRB>(k) * BRB + ((c ^ bswz<E, BRB>(k)) << 4) + off);
                const uint2 hi = lds_tr16(Bs + brow<E, BRB>(k + 4) * BRB +
                                          ((c ^ bswz<E, BRB>(k + 4)) << 4) + off);
                fb[buf][j] = u4_t{lo.x, lo.y, hi.x, hi.y};
            } else {
                // lane (16 g + s): rows 64 ks + 16 g + s / 2 (+ 8), columns
                // wn0 + 16 j + 8 (s % 2) .. + 7; lane s receives 8 rows of
                // column wn0 + 16 j + s per read
                const int k = ks * 64 + g * 16 + (l16 >> 1);
                const int colb = wn0 + j * 16 + 8 * (l16 & 1);
                const int c = colb >> 4, off = colb & 15;
                const uint2 lo =
                    lds_tr8(Bs + brow<E, BRB>(k) * BRB + ((c ^ bswz<E, BRB>(k)) << 4) + off);
                const uint2 hi = lds_tr8(Bs + brow<E, BRB>(k + 8) * BRB +
                                         ((c ^ bswz<E, BRB>(k + 8)) << 4) + off);
                fb[buf][j] = u4_t{lo.x, lo.y, hi.x, hi.y};
            }
        }
    };
    // MFMAs of one K step with B set `buf`, refilling A row by row from
    // K step ks of stage stg
    auto mma = [&](int buf, const uint8_t* stg, int ks) {
        // operands swapped (C^T = B^T A^T): lane l then holds output row
        // (l % 16) and the 4 consecutive output columns 4 (l / 16) + v
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = mfma16<E>(fb[buf][j], fa[i], acc[i][j]);
            rd_a(stg, ks, i);
        }
    };

    // ---- epilogue of the tile at (m0, n0), split sk: lane holds output row
    // (l16) and columns 4 g .. 4 g + 3 of each 16 x 16 MFMA tile.  The MFMA
    // waves issue no global loads: their vector-memory counter also counts
    // their output stores, so a load waited for here would wait for the
    // previous tile's stores as well.
    auto epilogue = [&](int m0, int n0, int sk) {
        typedef typename Epi::out_t out_t;
        float cs[TN][4];
        typename Epi::row_t rsv[TM];
        if constexpr (STAGE_OUT && Epi::kScaleDma) {
            // the copy waves brought this tile's scales into the staging
            // area (landed before the barrier this epilogue follows)
            // column scales first (WN floats), then the two row arrays
            const uint8_t* sa = smem + STAGES * STAGE + wave * AREA;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const f4_t c = *(const f4_t*)(sa + 64 * j + 16 * g);
#pragma unroll
                for (int v = 0; v < 4; ++v) cs[j][v] = c[v];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
                rsv[i] = epi.row_scale2(((const float*)(sa + 4 * WN))[i * 16 + l16],
                                        ((const float*)(sa + 4 * WN + 256))[i * 16 + l16]);
        } else {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) cs[j][v] = epi.col_scale(n0 + wn0 + j * 16 + g * 4 + v);
#pragma unroll
            for (int i = 0; i < TM; ++i) rsv[i] = epi.row_scale(min(m0 + wm0 + i * 16 + l16, M - 1));
        }
        if constexpr (STAGE_OUT) {
            if constexpr (Epi::kDbg) {
                if (epi.dbg != nullptr) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const int row = m0 + wm0 + i * 16 + l16;
                        if (row >= M) continue;
#pragma unroll
                        for (int j = 0; j < TN; ++j)
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                epi.dbg_store(row, n0 + wn0 + j * 16 + g * 4 + v, acc[i][j][v]);
                    }
                }
            }
            // per row of MFMA tiles: the lanes' 8-byte pieces go to this
            // wave's 16-row LDS area (RP bytes a row; 16-byte chunk c of row
            // r at c ^ (r & 7)), then come back as whole rows: lane l reads
            // chunk l % CPR of rows l / CPR + (64 / CPR) h (CPR = chunks a
            // row) and stores 16 bytes each, so one store covers whole
            // 128-byte lines.  LDS accesses of one wave complete in order, so
            // the area is reused without waits.
            constexpr int CPR = RP / 16;
            uint8_t* ep = smem + STAGES * STAGE + wave * AREA;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    float f[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) f[v] = epi.valuef(acc[i][j][v], rsv[i], cs[j][v]);
                    const int ch = (2 * j + (g >> 1)) ^ (l16 & 7);
                    *(u2_t*)(ep + l16 * RP + ch * 16 + (g & 1) * 8) =
                        u2_t{cvt_pk<Epi::kOut>(f[0], f[1]), cvt_pk<Epi::kOut>(f[2], f[3])};
                }
#pragma unroll
                for (int h = 0; h < CPR / 4; ++h) {
                    const int r = lane / CPR + (64 / CPR) * h, c = lane % CPR;
                    const u4_t v = *(const u4_t*)(ep + r * RP + ((c ^ (r & 7)) << 4));
                    const int grow = m0 + wm0 + i * 16 + r;
                    // written once, never re-read here: streaming stores
                    if (grow < M)
                        __builtin_nontemporal_store(v, (u4_t*)epi.ptr(grow, n0 + wn0 + c * 8, sk));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = m0 + wm0 + i * 16 + l16;
                if (row >= M) continue;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = n0 + wn0 + j * 16 + g * 4;
                    out_t o[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        o[v] = epi.value(row, col + v, acc[i][j][v], rsv[i], cs[j][v]);
                    // split-K partials are read back right away: cached stores
                    *(u4_t*)epi.ptr(row, col, sk) = u4_t{__builtin_bit_cast(uint32_t, o[0]),
                                                         __builtin_bit_cast(uint32_t, o[1]),
                                                         __builtin_bit_cast(uint32_t, o[2]),
                                                         __builtin_bit_cast(uint32_t, o[3])};
                }
            }
        }
    };

    // every LDS read of this wave complete (lgkmcnt 0; a waitcnt the compiler
    // sees, so it adds no wait of its own), then the workgroup barrier
    auto reads_done_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);  // keep the MFMAs above ahead of the wait
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // Software pipeline over (slab, K step): the reads of the next K step are
    // in flight while the MFMAs of the current one run, and barrier B_(g+1)
    // sits between the two K steps of slab g:
    //   rd(g,1)  mma(g,0)  [lgkmcnt 0, B_(g+1)]  rd(g+1,0)  mma(g,1)
    // After the last slab the same steps run once more with nothing to
    // multiply: its barrier meets the copy waves' final one and its reads of
    // an idle stage are discarded, which keeps the loop free of branches
    // around the MFMAs (the compiler then adds no waits inside them).
    int ti = 0, kc = 0, m0 = 0, n0 = 0, sk = 0;
    const uint8_t* cur = smem;
    asm volatile("s_barrier" ::: "memory");  // B_0: slab 0 in place
#pragma unroll
    for (int i = 0; i < TM; ++i) rd_a(cur, 0, i);
    rd_b(cur, 0, 0);
    for (int gs = 0; gs < total; ++gs) {
        if (kc == 0) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
            tile_origin(ti, m0, n0, sk);
        }
        // the previous K step's reads (issued during its MFMAs) are complete:
        // said explicitly, so that the compiler does not wait for the reads
        // issued next before the first MFMA
        __builtin_amdgcn_s_waitcnt(0xC07F);
        rd_b(cur, 1, 1);
        mma(0, cur, 1);
        const uint8_t* nxt = (cur + STAGE == smem + STAGES * STAGE) ? smem : cur + STAGE;
        reads_done_barrier();
        rd_b(nxt, 0, 0);
        mma(1, nxt, 0);
        if (++kc == nk) {
            epilogue(m0, n0, sk);
            kc = 0;
            ++ti;
        }
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// W8A8 kv_b_proj, weight-stationary.  A workgroup owns the 256 output
// columns of one head (k_nope then value) and runs eight waves, two per
// SIMD: wave w owns the 64 columns 64 (w % 4) .. and holds their int8
// weights over all 512 latent dimensions in registers for the whole launch
// (the MFMA operand fragments, read once through LDS with transposing
// reads); the two waves of a column quarter split each block of 32 latent
// rows into two halves of 16.  The workgroup streams its range of latent
// rows, 32 at a time, through a ring of LDS stages that all eight waves fill
// with direct global-to-LDS copies.  The results of block b are scaled,
// rounded and stored while block b + 1's MFMAs run (two accumulator sets),
// and the two waves of a SIMD overlap one's MFMAs with the other's vector
// work.  Each 16-byte store carries 8 consecutive columns of a row: lanes
// of neighbouring 16-lane rows swap packed pairs (v_permlane16_swap), so the
// results need no LDS staging.
// Work items are (row range, head) pairs: the row ranges split T so that
// the items fill the device, and the workgroups of one XCD share a row
// range, so the latent rows they read together stay in that XCD's L2.
// ---------------------------------------------------------------------------
namespace ws {
constexpr int kRows = 32;                   // latent rows per block
constexpr int kWaves = 8;
constexpr int kStages = 8;                  // ring stages
constexpr int kScaleOfs = kRows * kR;       // row scales after the codes
constexpr int kStageBytes = 17 * 1024;      // 16 KB of codes + 256 B of scales
constexpr int kSmem = kStages * kStageBytes;
constexpr int kCopies = kRows * kR / 1024 / kWaves;  // 16-byte copies per wave and block
static_assert(kSmem >= kR * 256, "the weight staging fits in the ring");
static_assert(kScaleOfs + 256 <= kStageBytes, "stage layout");
static_assert(kCopies * kWaves * 1024 == kRows * kR, "even copy split");
}  // namespace ws

// One 4-byte-per-lane copy from global memory into LDS (the wave's 64
// lanes fill lds .. lds + 255), as dma16.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(g)
        : "memory");
}
// The same copies from a wave-uniform base plus a 32-bit per-lane byte
// offset (the scalar-base form: no per-lane address arithmetic).
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(base)
        : "memory");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t voff, uint32_t lds) {
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(base)
        : "memory");
}
// Wait until at most N of this wave's vector-memory operations (copies and
// stores, which complete in issue order) are outstanding and its LDS reads
// are complete, then barrier.
template <int N>
__device__ __forceinline__ void wait_vm_lds_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <bool DBG>
__global__ __launch_bounds__(ws::kWaves * 64, 1) void kvb_w8_ws_kernel(
    const int8_t* __restrict__ QZ, const float* __restrict__ sz, uint32_t inv_ofs,
    const int8_t* __restrict__ Wqb, const float* __restrict__ swb, int T, int nh, int msplit,
    int bps, uint16_t* __restrict__ k_nope, uint16_t* __restrict__ value_out,
    int32_t* __restrict__ dbg, int64_t dbg_begin, int64_t dbg_rows) {
    using namespace ws;
    constexpr int BRB = 256;  // bytes of a staged weight row (the head's columns)
    constexpr int NT = kWaves * 64;
    __shared__ __align__(1024) uint8_t smem[kSmem];
    const int items = nh * msplit, per = (items + 7) / 8;
    const int xk = (int)(blockIdx.x >> 3), item = (int)(blockIdx.x & 7) * per + xk;
    if (xk >= per || item >= items) return;
    const int ms = item / nh, head = item - ms * nh;
    const int nblk = (T + kRows - 1) / kRows, bfirst = ms * bps;
    const int nb = min(bps, nblk - bfirst);
    if (nb <= 0) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cq = wave & 3, rh = wave >> 2;  // column quarter, row half
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t N2 = (int64_t)nh * kHeadW;
    const int col0 = head * kHeadW, wn0 = cq * 64;

    // ---- the head's weights: row k of its 256 columns at LDS row brow(k),
    // 16-byte chunk c at c ^ bswz(k); then each wave's operand fragments
#pragma unroll 8
    for (int it = 0; it < kR * BRB / 16 / NT; ++it) {
        const int q = it * NT + tid, k = q >> 4, c = q & 15;
        const u4_t v = *(const u4_t*)(Wqb + k * N2 + col0 + c * 16);
        *(u4_t*)(smem + brow<kI8, BRB>(k) * BRB + ((c ^ bswz<kI8, BRB>(k)) << 4)) = v;
    }
    __syncthreads();
    // fragment (ks, j): lane (16 g + s) receives column wn0 + 16 j + s, rows
    // 64 ks + 16 g .. + 15 (two transposing reads of 8 rows)
    u4_t fb[8][4];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = ks * 64 + g * 16 + (l16 >> 1);
            const int colb = wn0 + j * 16 + 8 * (l16 & 1);
            const int c = colb >> 4, off = colb & 15;
            const uint2 lo = lds_tr8(smem + brow<kI8, BRB>(k) * BRB +
                                     ((c ^ bswz<kI8, BRB>(k)) << 4) + off);
            const uint2 hi = lds_tr8(smem + brow<kI8, BRB>(k + 8) * BRB +
                                     ((c ^ bswz<kI8, BRB>(k + 8)) << 4) + off);
            fb[ks][j] = u4_t{lo.x, lo.y, hi.x, hi.y};
        }
    }
    // column scales of the lane's columns wn0 + 16 j + 4 g + v
    float cs[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f4_t c = *(const f4_t*)(swb + col0 + wn0 + j * 16 + g * 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) cs[j][v] = c[v];
    }
    // every load above complete and every fragment read before the ring
    // reuses the staging memory
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- ring.  Block bb (rows m_first + 32 bb ..) goes to stage
    // bb % kStages: wave w copies rows 4 w .. 4 w + 3 (two rows of 512 bytes
    // per instruction; chunk p of LDS row r holds chunk p ^ (r & 15)), wave
    // 0 also the rows' two scale arrays (inv_t lies inv_ofs bytes after sz).
    // The latent is padded to whole blocks, so the last block's copies stay
    // in bounds.  Copies past the last block repeat it, so every wait below
    // has the same number of later operations.
    const int m_first = bfirst * kRows;
    const uint32_t sbase =
        lds_addr(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(wave * kCopies * 1024);
    const uint32_t scl = lds_addr(smem) + kScaleOfs;
    uint32_t aoff[kCopies];
#pragma unroll
    for (int q = 0; q < kCopies; ++q) {
        const int r = (wave * kCopies + q) * 2 + (lane >> 5), p = lane & 31;
        aoff[q] = (uint32_t)(r * kR + ((p ^ (r & 15)) << 4));
    }
    const uint32_t soff = lane < 32 ? (uint32_t)lane * 4 : inv_ofs + (uint32_t)(lane - 32) * 4;
    auto issue = [&](int bb) {
        const int m0 = m_first + min(bb, nb - 1) * kRows;
        const uint32_t so = (uint32_t)((bb % kStages) * kStageBytes);
        const int8_t* qb = QZ + (int64_t)m0 * kR;
#pragma unroll
        for (int q = 0; q < kCopies; ++q) dma16s(qb, aoff[q], sbase + so + q * 1024);
        if (wave == 0) dma4s(sz + m0, soff, scl + so);
    };
    // stage b in place and the stage of block b - 1 free.  After block b's
    // copies this wave issued kStages - 2 later groups of copies (kCopies,
    // wave 0 one more instruction) and, from block kStages on, kStages - 1
    // groups of 2 stores; before that it counts the copies only (it waits
    // for more).
    auto wait_stage = [&](int b) {
        constexpr int D = kStages, C = kCopies;
        if (b < D) {
            if (wave == 0) wait_vm_lds_barrier<(C + 1) * (D - 2)>();
            else wait_vm_lds_barrier<C * (D - 2)>();
        } else {
            if (wave == 0) wait_vm_lds_barrier<(C + 1) * (D - 2) + 2 * (D - 1)>();
            else wait_vm_lds_barrier<C * (D - 2) + 2 * (D - 1)>();
        }
    };
    typedef i4_t acc_t;
    // MFMAs of the wave's 16 rows of block b (operands swapped, C^T = B^T
    // A^T: lane l then holds row l % 16 and columns 4 (l / 16) .. + 3 of
    // each 16-column tile).  The A fragment of K step ks + 2 is read while
    // step ks multiplies.
    uint32_t aro[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) aro[ks] = (uint32_t)((rh * 16 + l16) * kR + (((ks * 4 + g) ^ l16) << 4));
    auto mma_block = [&](acc_t(&acc)[4], int b) {
        const uint8_t* s = smem + (b % kStages) * kStageBytes;
        u4_t fa[3];
        auto rd = [&](int ks) { fa[ks % 3] = *(const u4_t*)(s + aro[ks]); };
        rd(0);
        rd(1);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (ks + 2 < 8) rd(ks + 2);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = mfma16<kI8>(fb[ks][j], fa[ks % 3], ks == 0 ? acc_t{0, 0, 0, 0} : acc[j]);
        }
    };
    // the factor (activation scale times RMS factor) of the lane's row of
    // block b
    auto read_rs = [&](int b) {
        const float* s = (const float*)(smem + (b % kStages) * kStageBytes + kScaleOfs);
        return s[rh * 16 + l16] * s[32 + rh * 16 + l16];
    };
    uint16_t* const dst0 = (cq < 2 ? k_nope : value_out) + (int64_t)head * kDN + (cq & 1) * 64;
    const int64_t rstride = (int64_t)nh * kDN;
    // byte offset of the lane's 16-byte pieces from its 16-row group's
    // first row (row l16, columns of piece p)
    uint32_t doff[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
        doff[p] = (uint32_t)((l16 * rstride + 32 * p + ((g & 1) ? 16 + 4 * (g - 1) : 4 * g)) * 2);
    // results of block b: ((acc * row factor) * column scale) rounded to
    // bf16; lanes of even 16-lane rows end with 8 columns of tile 2p, odd
    // ones with 8 columns of tile 2p + 1.  GUARD: rows past T are skipped
    // (only the last block has any).
    auto epi_block = [&](const acc_t(&acc)[4], float rs, int b, auto guard) {
        const int row0 = m_first + b * kRows + rh * 16, row = row0 + l16;
        uint8_t* const drow = (uint8_t*)(dst0 + row0 * rstride);
        uint32_t P[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float f[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) f[v] = ((float)acc[j][v] * rs) * cs[j][v];
            P[j][0] = cvt_pk<kBF16>(f[0], f[1]);
            P[j][1] = cvt_pk<kBF16>(f[2], f[3]);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const auto s0 = __builtin_amdgcn_permlane16_swap(P[2 * p][0], P[2 * p + 1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(P[2 * p][1], P[2 * p + 1][1], false, false);
            const u4_t v = u4_t{s0[0], s1[0], s0[1], s1[1]};
            uint8_t* d = drow + doff[p];
            if constexpr (decltype(guard)::value) {
                if (row < T) __builtin_nontemporal_store(v, (u4_t*)d);
            } else {
                __builtin_nontemporal_store(v, (u4_t*)d);
            }
        }
        if constexpr (DBG) {
            if (row < T && row >= dbg_begin && row < dbg_begin + dbg_rows) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        dbg[(row - dbg_begin) * N2 + col0 + wn0 + j * 16 + g * 4 + v] = acc[j][v];
            }
        }
    };
    typedef std::integral_constant<bool, false> NoGuard;
    typedef std::integral_constant<bool, true> Guard;

    acc_t accA[4], accB[4];
    float rsA, rsB;
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s);
    wait_stage(0);
    issue(kStages - 1);
    rsA = read_rs(0);
    mma_block(accA, 0);
    int b = 1;
    for (; b + 1 < nb; b += 2) {
        wait_stage(b);
        issue(b + kStages - 1);
        rsB = read_rs(b);
        mma_block(accB, b);
        epi_block(accA, rsA, b - 1, NoGuard{});
        wait_stage(b + 1);
        issue(b + kStages);
        rsA = read_rs(b + 1);
        mma_block(accA, b + 1);
        epi_block(accB, rsB, b, NoGuard{});
    }
    if (b < nb) {
        wait_stage(b);
        rsB = read_rs(b);
        mma_block(accB, b);
        epi_block(accA, rsA, b - 1, NoGuard{});
        epi_block(accB, rsB, b, Guard{});
    } else {
        epi_block(accA, rsA, b - 1, Guard{});
    }
}

// ---------------------------------------------------------------------------
// fp16 / bf16 kv_b_proj, weight-stationary: the same scheme with 2-byte
// weights.  A workgroup owns one head's 256 columns; wave w (eight waves,
// two per SIMD) owns the 32 columns 32 w .. and holds their weights over all
// 512 latent dimensions in registers (the operand fragments of 16 K steps
// of 32; the staging goes through LDS in two halves of K, 128 KB each), and
// multiplies all 32 rows of each latent block.  Blocks of 32 latent rows
// (32 KB) stream through a ring of 4 LDS stages; each wave copies 4 rows
// (one 1 KB row per instruction, 16-byte chunk p of LDS row r holding chunk
// p ^ (r & 15)), rows past T repeat row T - 1.  The results of block b are
// rounded and stored while block b + 1's MFMAs run; one 16-byte store per
// lane writes 16 rows x 64 bytes (the wave's 32 columns).
// ---------------------------------------------------------------------------
namespace wsf {
constexpr int kRows = 32;
constexpr int kWaves = 8;
constexpr int kStages = 4;
constexpr int kStageBytes = kRows * kR * 2;          // 32 KB
constexpr int kSmem = kStages * kStageBytes;         // 128 KB, also one weight half
constexpr int kCopies = kRows / kWaves;              // one row per copy instruction
static_assert(kSmem >= (kR / 2) * 512, "a half of the weight staging fits");
}  // namespace wsf

template <int E>
__global__ __launch_bounds__(wsf::kWaves * 64, 1) void kvb_fp_ws_kernel(
    const uint16_t* __restrict__ Y, const uint16_t* __restrict__ Wb, int T, int nh, int msplit,
    int bps, uint16_t* __restrict__ k_nope, uint16_t* __restrict__ value_out) {
    using namespace wsf;
    constexpr int BRB = 512;  // bytes of a staged weight row (the head's 256 columns)
    constexpr int NT = kWaves * 64;
    __shared__ __align__(1024) uint8_t smem[kSmem];
    const int items = nh * msplit, per = (items + 7) / 8;
    const int xk = (int)(blockIdx.x >> 3), item = (int)(blockIdx.x & 7) * per + xk;
    if (xk >= per || item >= items) return;
    const int ms = item / nh, head = item - ms * nh;
    const int nblk = (T + kRows - 1) / kRows, bfirst = ms * bps;
    const int nb = min(bps, nblk - bfirst);
    if (nb <= 0) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t N2 = (int64_t)nh * kHeadW;
    const int col0 = head * kHeadW, wn0 = wave * 32;

    // ---- the head's weights, K in two halves: row k of its 256 columns at
    // LDS row k - k0, 16-byte chunk c at c ^ bswz(k); then each wave's
    // fragments of the half's 8 K steps.  Fragment (ks, j): lane (16 g + s)
    // receives column wn0 + 16 j + s, rows 32 ks + 8 g .. + 7 (two
    // transposing reads of 4 rows).
    u4_t fb[16][2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int k0 = half * (kR / 2);
#pragma unroll 8
        for (int it = 0; it < (kR / 2) * BRB / 16 / NT; ++it) {
            const int q = it * NT + tid, kk = q >> 5, c = q & 31, k = k0 + kk;
            const u4_t v = *(const u4_t*)((const uint8_t*)Wb + (k * N2 + col0) * 2 + c * 16);
            *(u4_t*)(smem + brow<E, BRB>(kk) * BRB + ((c ^ bswz<E, BRB>(kk)) << 4)) = v;
        }
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < 8; ++kq) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kk = kq * 32 + g * 8 + (l16 >> 2);
                const int colb = (wn0 + j * 16 + 4 * (l16 & 3)) * 2;
                const int c = colb >> 4, off = colb & 15;
                const uint2 lo = lds_tr16(smem + brow<E, BRB>(kk) * BRB +
                                          ((c ^ bswz<E, BRB>(kk)) << 4) + off);
                const uint2 hi = lds_tr16(smem + brow<E, BRB>(kk + 4) * BRB +
                                          ((c ^ bswz<E, BRB>(kk + 4)) << 4) + off);
                fb[half * 8 + kq][j] = u4_t{lo.x, lo.y, hi.x, hi.y};
            }
        }
        // every load and fragment read done before the memory is reused
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- ring
    const int m_first = bfirst * kRows;
    const uint32_t sbase =
        lds_addr(smem) + (uint32_t)__builtin_amdgcn_readfirstlane(wave * kCopies * kR * 2);
    uint32_t aoff[kCopies];
#pragma unroll
    for (int q = 0; q < kCopies; ++q) {
        const int r = wave * kCopies + q;
        aoff[q] = (uint32_t)((lane ^ (r & 15)) << 4);
    }
    auto issue = [&](int bb) {
        const int m0 = m_first + min(bb, nb - 1) * kRows;
        const uint32_t so = (uint32_t)((bb % kStages) * kStageBytes);
#pragma unroll
        for (int q = 0; q < kCopies; ++q) {
            const int row = min(m0 + wave * kCopies + q, T - 1);
            dma16s(Y + (int64_t)row * kR, aoff[q], sbase + so + q * kR * 2);
        }
    };
    // after block b's copies this wave issued kStages - 2 later groups of
    // kCopies copies and, from block kStages on, kStages - 1 groups of 2
    // stores; before that it counts the copies only (it waits for more)
    auto wait_stage = [&](int b) {
        constexpr int D = kStages;
        if (b < D) wait_vm_lds_barrier<kCopies * (D - 2)>();
        else wait_vm_lds_barrier<kCopies * (D - 2) + 2 * (D - 1)>();
    };
    uint32_t aro[16][2];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
            aro[ks][i] = (uint32_t)((16 * i + l16) * kR * 2 + (((ks * 4 + g) ^ l16) << 4));
    typedef f4_t acc_t;
    auto mma_block = [&](acc_t(&acc)[2][2], int b) {
        const uint8_t* s = smem + (b % kStages) * kStageBytes;
        u4_t fa[3][2];
        auto rd = [&](int ks) {
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[ks % 3][i] = *(const u4_t*)(s + aro[ks][i]);
        };
        rd(0);
        rd(1);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            if (ks + 2 < 16) rd(ks + 2);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma16<E>(fb[ks][j], fa[ks % 3][i],
                                          ks == 0 ? acc_t{0.f, 0.f, 0.f, 0.f} : acc[i][j]);
        }
    };
    uint16_t* const dst0 = (wave < 4 ? k_nope : value_out) + (int64_t)head * kDN + (wave & 3) * 32;
    const int64_t rstride = (int64_t)nh * kDN;
    const uint32_t doff =
        (uint32_t)((l16 * rstride + ((g & 1) ? 16 + 4 * (g - 1) : 4 * g)) * 2);
    auto epi_block = [&](const acc_t(&acc)[2][2], int b, auto guard) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row0 = m_first + b * kRows + 16 * i, row = row0 + l16;
            const uint32_t p00 = cvt_pk<E>(acc[i][0][0], acc[i][0][1]);
            const uint32_t p01 = cvt_pk<E>(acc[i][0][2], acc[i][0][3]);
            const uint32_t p10 = cvt_pk<E>(acc[i][1][0], acc[i][1][1]);
            const uint32_t p11 = cvt_pk<E>(acc[i][1][2], acc[i][1][3]);
            const auto s0 = __builtin_amdgcn_permlane16_swap(p00, p10, false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(p01, p11, false, false);
            const u4_t v = u4_t{s0[0], s1[0], s0[1], s1[1]};
            uint8_t* d = (uint8_t*)(dst0 + row0 * rstride) + doff;
            if constexpr (decltype(guard)::value) {
                if (row < T) __builtin_nontemporal_store(v, (u4_t*)d);
            } else {
                __builtin_nontemporal_store(v, (u4_t*)d);
            }
        }
    };
    typedef std::integral_constant<bool, false> NoGuard;
    typedef std::integral_constant<bool, true> Guard;

    acc_t accA[2][2], accB[2][2];
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s);
    wait_stage(0);
    issue(kStages - 1);
    mma_block(accA, 0);
    int b = 1;
    for (; b + 1 < nb; b += 2) {
        wait_stage(b);
        issue(b + kStages - 1);
        mma_block(accB, b);
        epi_block(accA, b - 1, NoGuard{});
        wait_stage(b + 1);
        issue(b + kStages);
        mma_block(accA, b + 1);
        epi_block(accB, b, NoGuard{});
    }
    if (b < nb) {
        wait_stage(b);
        mma_block(accB, b);
        epi_block(accA, b - 1, NoGuard{});
        epi_block(accB, b, Guard{});
    } else {
        epi_block(accA, b - 1, Guard{});
    }
}

// ---------------------------------------------------------------------------
// Per-token finish of kv_a_proj, fp16/bf16 path.  One wave per token, four
// tokens per workgroup: lane l owns latent columns 8l..8l+7 and rope column
// l.  Every load (position, gamma, partials) is issued before the first use.
//   c, p  = sum of the split-K partials (split order ascending)
//   y     = c / sqrt(sum(c^2)/512 + eps) * gamma      -> compressed_kv
//   k_pe  = rotate-half RoPE of p at the token's position
// The rope angle pos * theta^(-2i/64) is formed and reduced by quarter turns
// in double; sine / cosine of the reduced angle and the rotation run in fp32
// (rope_cos_sin).
// ---------------------------------------------------------------------------
// The end of the fp16/bf16 finish for token t, on one wave that holds the
// token's summed partials (lane l: latent columns 8l..8l+7 in c, rope
// column l in p) and gamma's columns 8l.. in g:
//   y    = c / sqrt(sum(c^2)/512 + eps) * gamma      -> compressed_kv
//   k_pe = rotate-half RoPE of p at position pt      -> k_pe (and the cache)
// Returns the lane's 8 rounded latent values; with store false nothing is
// written (a caller that needs only the latent).
template <int E>
__device__ __forceinline__ u4_t finish_fp_token(const float (&c)[8], float p, u4_t g, int64_t t,
                                                int pt, int64_t slot, float eps,
                                                const RopeTab& rt, uint16_t* __restrict__ ckv,
                                                uint16_t* __restrict__ kpe, const CacheOut& co,
                                                bool store = true) {
    const int lane = threadIdx.x & 63;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += c[i] * c[i];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)kR + eps);
    const u4_t o = rms_scale8<E>(c, inv, g);
    if (!store) return o;
    *(u4_t*)(ckv + t * kR + 8 * lane) = o;

    const float partner = __shfl_xor(p, 32, 64);
    float cs, sn;
    rope_cos_sin(pt, rt.f[lane & 31], cs, sn);
    const uint16_t ko = f32_to_st<E>(rope_rotate(p, partner, cs, sn, lane < 32));
    __builtin_nontemporal_store(ko, kpe + t * kDR + lane);
    if (cache_slot_ok(co, slot)) {  // the paged cache: [latent | rope key] in the token's slot
        uint16_t* row = co.cache + slot * (kR + kDR);
        __builtin_nontemporal_store(o, (u4_t*)(row + 8 * lane));
        __builtin_nontemporal_store(ko, row + kR + lane);
    }
    return o;
}

template <int E, int B>
__global__ __launch_bounds__(256) void finish_a_fp_kernel(
    const float* __restrict__ P, int S, int64_t T, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ pos, float eps, RopeTab rt, uint16_t* __restrict__ ckv,
    uint16_t* __restrict__ kpe, CacheOut co) {
    // one token per wave; one to four waves per workgroup
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const int pt = pos[t];
    const int64_t slot = co.slots != nullptr ? co.slots[t] : -1;
    const u4_t g = *(const u4_t*)(gamma + 8 * lane);
    float c[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float p = 0.f;
    // the split-K partials, B splits' loads in flight at a time (B is the
    // smallest power of two >= S, at most 8, so a batch re-reads nothing
    // unless S is not a power of two: splits past S re-read split S - 1 and
    // are not added); summed in ascending split order
    for (int s0 = 0; s0 < S; s0 += B) {
        f4_t v0[B], v1[B];
        float pv[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int s = s0 + j < S ? s0 + j : S - 1;
            const float* row = P + ((int64_t)s * T + t) * kN1;
            // partials are read once: streaming (non-temporal) loads
            v0[j] = __builtin_nontemporal_load((const f4_t*)(row + 8 * lane));
            v1[j] = __builtin_nontemporal_load((const f4_t*)(row + 8 * lane + 4));
            pv[j] = __builtin_nontemporal_load(row + kR + lane);
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (s0 + j < S) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    c[i] += v0[j][i];
                    c[4 + i] += v1[j][i];
                }
                p += pv[j];
            }
        }
    }
    finish_fp_token<E>(c, p, g, t, pt, slot, eps, rt, ckv, kpe, co);
}

// The same finish with one workgroup per token, for many splits and few
// tokens: wave w sums splits w, w + 4, ... (NPW loads in flight, one batch),
// waves 1..3 hand their sums to wave 0 through LDS, and wave 0 adds them in
// wave order and finishes the token as above.  A single wave per token would
// wait for its splits in several batches, one after another.
template <int E, int NPW>
__global__ __launch_bounds__(256) void finish_fp_wide_kernel(
    const float* __restrict__ P, int S, int64_t T, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ pos, float eps, RopeTab rt, uint16_t* __restrict__ ckv,
    uint16_t* __restrict__ kpe, CacheOut co) {
    __shared__ float red[3][64 * 9];
    const int64_t t = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int pt = 0;
    int64_t slot = -1;
    u4_t g = {0u, 0u, 0u, 0u};
    if (wave == 0) {
        pt = pos[t];
        slot = co.slots != nullptr ? co.slots[t] : -1;
        g = *(const u4_t*)(gamma + 8 * lane);
    }
    f4_t v0[NPW], v1[NPW];
    float pv[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        const int s = wave + 4 * j < S ? wave + 4 * j : S - 1;
        const float* row = P + ((int64_t)s * T + t) * kN1;
        v0[j] = __builtin_nontemporal_load((const f4_t*)(row + 8 * lane));
        v1[j] = __builtin_nontemporal_load((const f4_t*)(row + 8 * lane + 4));
        pv[j] = __builtin_nontemporal_load(row + kR + lane);
    }
    float c[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        if (wave + 4 * j < S) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] += v0[j][i];
                c[4 + i] += v1[j][i];
            }
            p += pv[j];
        }
    }
    if (wave > 0) {
        float* r = red[wave - 1] + lane * 9;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = c[i];
        r[8] = p;
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        const float* r = red[w] + lane * 9;
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] += r[i];
        p += r[8];
    }
    finish_fp_token<E>(c, p, g, t, pt, slot, eps, rt, ckv, kpe, co);
}

// ---------------------------------------------------------------------------
// fp16 / bf16 prefill, the finish and kv_b_proj in one launch: the
// normalised latent is staged in LDS and feeds kv_b_proj's MFMAs from there.
// A workgroup owns a block of 64 token rows and a group of G heads.
//   1. It sums its rows' split-K partials of kv_a_proj (split order
//      ascending), normalises them (RMSNorm, gamma) and keeps the rounded
//      latent [64][512] in LDS; the workgroup of the first head group also
//      writes compressed_kv, k_pe and the cache rows (finish_fp_token, the
//      same arithmetic as the separate finish kernels).
//   2. For each of its heads it multiplies that latent by the head's 256
//      W_kv_b columns, which stream through a ring of three LDS stages of
//      64 K rows each (direct global-to-LDS copies, four per wave and
//      stage; the first two stages are in flight during step 1).  Wave w
//      owns columns 32 w .. 32 w + 31 of the head and all 64 rows; the
//      K steps run in ascending order, as in the tiled kernel, so k_nope
//      and value come out bit for bit as from the three-launch path
//      wherever its finish also adds the splits in ascending order.
// LDS: latent rows of 1 KB, 16-byte chunk c of row r at c ^ (r % 16); ring
// stages in the pipelined GEMM's B layout (rows of 512 bytes, swizzled
// chunks, transposing reads).
// ---------------------------------------------------------------------------
namespace fb {
constexpr int kRows = 64;                             // token rows per workgroup
constexpr int kWaves = 8;
constexpr int kStages = 3;                            // W_kv_b ring stages
constexpr int kSlabK = 64;                            // K rows per stage
constexpr int kBRB = kHeadW * 2;                      // bytes of a staged W row
constexpr int kStageBytes = kSlabK * kBRB;            // 32 KB
constexpr int kLatBytes = kRows * kR * 2;             // 64 KB
constexpr int kCopies = kStageBytes / 1024 / kWaves;  // per wave and stage
constexpr int kSlabsPerHead = kR / kSlabK;
constexpr int kStores = 4;                            // per wave and head
static_assert(kLatBytes + kStages * kStageBytes <= 160 * 1024, "LDS");
static_assert(kCopies * kWaves * 1024 == kStageBytes, "even copy split");
}  // namespace fb

// Heads per workgroup of the fused finish + kv_b_proj launch: the smallest
// divisor of nh that keeps the launch within 256 workgroups.
inline int fin_kv_b_group(int64_t T, int nh) {
    const int64_t nrb = (T + fb::kRows - 1) / fb::kRows;
    for (int g = 1; g < nh; ++g)
        if (nh % g == 0 && nrb * (nh / g) <= 256) return g;
    return nh;
}

template <int E, int NS>
__global__ __launch_bounds__(fb::kWaves * 64, 1) void fin_kv_b_fp_kernel(
    const float* __restrict__ P, int S, int64_t T, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ pos, float eps, RopeTab rt, const uint16_t* __restrict__ Wb,
    int nh, int G, uint16_t* __restrict__ ckv, uint16_t* __restrict__ kpe, CacheOut co,
    uint16_t* __restrict__ k_nope, uint16_t* __restrict__ value_out) {
    using namespace fb;
    __shared__ __align__(1024) uint8_t smem[kLatBytes + kStages * kStageBytes];
    uint8_t* const lat = smem;
    uint8_t* const ring = smem + kLatBytes;
    // work item (row block, head group): workgroup b runs on XCD b % 8,
    // which owns a contiguous range of items, so the head groups of a row
    // block share that XCD's L2 (their split-K partials are read there)
    const int64_t nrb = (T + kRows - 1) / kRows;
    const int ngrp = nh / G;
    const int64_t items = nrb * ngrp, per = (items + 7) / 8;
    const int64_t xk = blockIdx.x >> 3, item = (int64_t)(blockIdx.x & 7) * per + xk;
    if (xk >= per || item >= items) return;
    const int64_t rb = item / ngrp;
    const int grp = (int)(item - rb * ngrp);
    const int64_t m0 = rb * kRows;
    const int head0 = grp * G;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t N2 = (int64_t)nh * kHeadW;

    // ---- W_kv_b ring: slab n is K rows 64 (n % 8) .. of head head0 + n / 8,
    // in stage n % 3.  Copy u of this wave fills stage bytes
    // (kCopies wave + u) KB .. + 1 KB: B rows k, k + 1 of the slab, chunk pos
    // of LDS row k holding global chunk pos ^ bswz(k).
    const int nslab = G * kSlabsPerHead;
    uint32_t woff[kCopies];
#pragma unroll
    for (int u = 0; u < kCopies; ++u) {
        const int byte = (wave * kCopies + u) * 1024 + lane * 16;
        const int k = brow<E, kBRB>(byte / kBRB), pp = (byte % kBRB) / 16;
        woff[u] = (uint32_t)(k * N2 * 2 + ((pp ^ bswz<E, kBRB>(k)) << 4));
    }
    const uint32_t ring0 =
        lds_addr(ring) + (uint32_t)__builtin_amdgcn_readfirstlane(wave * kCopies * 1024);
    auto issue = [&](int n) {
        const int h = head0 + n / kSlabsPerHead, kk = n % kSlabsPerHead;
        const uint16_t* base = Wb + (int64_t)kk * kSlabK * N2 + (int64_t)h * kHeadW;
        const uint32_t so = (uint32_t)((n % kStages) * kStageBytes);
#pragma unroll
        for (int u = 0; u < kCopies; ++u) dma16s(base, woff[u], ring0 + so + u * 1024);
    };
    issue(0);
    if (nslab > 1) issue(1);

    // ---- 1. finish rows 8 wave .. 8 wave + 7 into the LDS latent, four rows
    // at a time, NS splits' partial loads in flight per row (rows past T load
    // row T - 1 and store nothing; their latent rows are zero).  The splits
    // are added in ascending order, as in the separate finish kernels.
    const u4_t gm = *(const u4_t*)(gamma + 8 * lane);
#pragma unroll
    for (int q0 = 0; q0 < 8; q0 += 4) {
        float c[4][8];
        float p[4];
        int ptv[4];
        int64_t slv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = min(m0 + 8 * wave + q0 + r, T - 1);
            ptv[r] = pos[t];
            slv[r] = co.slots != nullptr ? co.slots[t] : -1;
            p[r] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) c[r][i] = 0.f;
        }
        for (int s0 = 0; s0 < S; s0 += NS) {
            f4_t v0[4][NS], v1[4][NS];
            float pv[4][NS];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = min(m0 + 8 * wave + q0 + r, T - 1);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const float* row = P + ((int64_t)min(s0 + s, S - 1) * T + t) * kN1;
                    v0[r][s] = __builtin_nontemporal_load((const f4_t*)(row + 8 * lane));
                    v1[r][s] = __builtin_nontemporal_load((const f4_t*)(row + 8 * lane + 4));
                    pv[r][s] = __builtin_nontemporal_load(row + kR + lane);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (s0 + s < S) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            c[r][i] += v0[r][s][i];
                            c[r][4 + i] += v1[r][s][i];
                        }
                        p[r] += pv[r][s];
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = 8 * wave + q0 + r;
            const int64_t t = m0 + rr;
            u4_t o = {0u, 0u, 0u, 0u};
            if (t < T) o = finish_fp_token<E>(c[r], p[r], gm, t, ptv[r], slv[r], eps, rt, ckv,
                                              kpe, co, grp == 0);
            *(u4_t*)(lat + rr * (kR * 2) + ((lane ^ (rr & 15)) << 4)) = o;
        }
    }
    // every partial load has been waited for, so the ring's first two
    // stages (copied before them) have landed too; the latent rows are
    // written
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- 2. kv_b_proj over the staged latent
    typedef f4_t acc_t;
    acc_t acc[4][2];
    uint16_t* const dst_base = (wave < 4 ? k_nope : value_out) + (wave & 3) * 32;
    const int64_t rstride = (int64_t)nh * kDN;
    const uint32_t doff = (uint32_t)((l16 * rstride + ((g & 1) ? 16 + 4 * (g - 1) : 4 * g)) * 2);
    for (int n = 0; n < nslab; ++n) {
        // slab n landed and slab n - 1's stage free: after slab n's copies
        // this wave issued slab n + 1's (unless it is the last) and, at a
        // head boundary, one head's stores
        if (n == 1) {
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else if (n >= 2) {
            const bool more = n + 1 < nslab;
            const bool st = n >= kSlabsPerHead && (n % kSlabsPerHead) < 2;
            if (more && st) wait_vm_lds_barrier<kCopies + kStores>();
            else if (more) wait_vm_lds_barrier<kCopies>();
            else if (st) wait_vm_lds_barrier<kStores>();
            else wait_vm_lds_barrier<0>();
        }
        if (n + kStages - 1 < nslab) issue(n + kStages - 1);
        const uint8_t* Bs = ring + (n % kStages) * kStageBytes;
        const int kk = n % kSlabsPerHead;
        if (kk == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = acc_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u4_t fa[4], fbv[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * i + l16;
                const int ch = kk * 8 + ks * 4 + g;
                fa[i] = *(const u4_t*)(lat + row * (kR * 2) + ((ch ^ l16) << 4));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // lane (16 g + s): K rows 32 ks + 8 g + s / 4 (+ 4), columns
                // 32 wave + 16 j + 4 (s % 4) .. + 3
                const int k = ks * 32 + g * 8 + (l16 >> 2);
                const int colb = (32 * wave + 16 * j + 4 * (l16 & 3)) * 2;
                const int c = colb >> 4, off = colb & 15;
                const uint2 lo = lds_tr16(Bs + brow<E, kBRB>(k) * kBRB +
                                          ((c ^ bswz<E, kBRB>(k)) << 4) + off);
                const uint2 hi = lds_tr16(Bs + brow<E, kBRB>(k + 4) * kBRB +
                                          ((c ^ bswz<E, kBRB>(k + 4)) << 4) + off);
                fbv[j] = u4_t{lo.x, lo.y, hi.x, hi.y};
            }
            // operands swapped (C^T = B^T A^T): lane l holds row l % 16 of
            // row tile i and columns 4 (l / 16) .. + 3 of column tile j
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma16<E>(fbv[j], fa[i], acc[i][j]);
        }
        if (kk == kSlabsPerHead - 1) {
            // the head's results, rounded; lanes of even 16-lane rows end with
            // 8 columns of tile 0, odd ones with 8 columns of tile 1 (one
            // 16-byte store per lane and row tile)
            const int head = head0 + n / kSlabsPerHead;
            uint8_t* const dh = (uint8_t*)(dst_base + (int64_t)head * kDN);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row0 = m0 + 16 * i;
                uint32_t P0[2], P1[2];
                P0[0] = cvt_pk<E>(acc[i][0][0], acc[i][0][1]);
                P0[1] = cvt_pk<E>(acc[i][0][2], acc[i][0][3]);
                P1[0] = cvt_pk<E>(acc[i][1][0], acc[i][1][1]);
                P1[1] = cvt_pk<E>(acc[i][1][2], acc[i][1][3]);
                const auto s0 = __builtin_amdgcn_permlane16_swap(P0[0], P1[0], false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(P0[1], P1[1], false, false);
                const u4_t v = u4_t{s0[0], s1[0], s0[1], s1[1]};
                if (row0 + l16 < T)
                    __builtin_nontemporal_store(v, (u4_t*)(dh + row0 * rstride * 2 + doff));
            }
        }
    }
}

// Where the one-launch finish + kv_b_proj is taken by default: nowhere.  On
// the V2-Lite prefill (T = 4096) it took ~40 us against ~24 us for the
// finish and the tiled kv_b_proj it replaces: each row block's split sums
// and RMSNorm are repeated by its four head groups (~15 us alone), and each
// CU pulls 1 MB of W_kv_b through a ring two stages deep (the latent holds
// the rest of LDS), ~31 us alone, against 768 KB per CU for the tiled
// kernel's 256-row tiles.
inline bool fin_kv_b_pays(int64_t, int) { return false; }

template <int E>
static void launch_fin_kv_b_fp(const float* P, int S, int64_t T, const void* gamma,
                               const int32_t* pos, float eps, const RopeTab& rt, const void* Wb,
                               int nh, void* ckv, void* kpe, const CacheOut& co, void* k_nope,
                               void* value, hipStream_t st) {
    const int G = fin_kv_b_group(T, nh);
    const int64_t items = ((T + fb::kRows - 1) / fb::kRows) * (nh / G);
    const dim3 grid((unsigned)(8 * ((items + 7) / 8))), blk(fb::kWaves * 64);
    auto go = [&](auto kern) {
        launch_k(kern, grid, blk, 0, st, P, S, T, (const uint16_t*)gamma, pos, eps, rt,
                 (const uint16_t*)Wb, nh, G, (uint16_t*)ckv, (uint16_t*)kpe, co,
                 (uint16_t*)k_nope, (uint16_t*)value);
    };
    if (S == 1) go(fin_kv_b_fp_kernel<E, 1>);
    else go(fin_kv_b_fp_kernel<E, 2>);
}

// ---------------------------------------------------------------------------
// W8A8: per-token activation quantisation.
//   amax = max |x|;  q = clamp(rint(x * (127/amax)), -127, 127);
//   scale = amax / 127;  amax == 0 -> q = 0, scale = 0.
// fp32 with IEEE division and round-half-even rint.  Rows of up to 8192
// elements: one wave per row, every chunk held in registers
// (quant_rows_wave_kernel); longer rows: one 256-thread workgroup per row
// that walks it twice (quant_rows_long_kernel).
// ---------------------------------------------------------------------------
// One wave per token row (four rows per workgroup), NCH 16-byte chunks per
// lane (chunk lane + 64 u), all loaded before the first wait; the row maximum
// is a wave reduction, so no LDS or barrier is involved.  With fill_q set,
// the wave also writes the "not finished yet" pattern of the decode
// hand-off into the token's latent code row (0x80 bytes, a code the
// quantisers never produce) and its two latent scales (all-ones words).
template <int NCH>
__global__ __launch_bounds__(256) void quant_rows_wave_kernel(const uint16_t* __restrict__ X,
                                                              int H, int64_t T,
                                                              int8_t* __restrict__ Q,
                                                              float* __restrict__ scale,
                                                              int8_t* __restrict__ fill_q,
                                                              uint32_t* __restrict__ fill_sz,
                                                              uint32_t* __restrict__ fill_inv) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const uint16_t* row = X + t * H;
    const int nch = H >> 3;
    u4_t v[NCH];
#pragma unroll
    for (int u = 0; u < NCH; ++u)  // read once: streaming (non-temporal) loads
        v[u] = __builtin_nontemporal_load((const u4_t*)(row + 8 * min(lane + 64 * u, nch - 1)));
    float amax = 0.f;
#pragma unroll
    for (int u = 0; u < NCH; ++u)
        if (lane + 64 * u < nch) amax = absmax8(v[u], amax);
    amax = wave_max(amax);
    const float inv = (amax > 0.f) ? (127.0f / amax) : 0.f;
#pragma unroll
    for (int u = 0; u < NCH; ++u)
        if (lane + 64 * u < nch) *(u2_t*)(Q + t * H + 8 * (lane + 64 * u)) = quant8(v[u], inv);
    if (lane == 0) scale[t] = (amax > 0.f) ? (amax / 127.0f) : 0.f;
    if (fill_q != nullptr) {
        *(u2_t*)(fill_q + t * kR + 8 * lane) = u2_t{0x80808080u, 0x80808080u};
        if (lane == 0) {
            fill_sz[t] = ~0u;
            fill_inv[t] = ~0u;
        }
    }
}

__global__ __launch_bounds__(256) void quant_rows_long_kernel(const uint16_t* __restrict__ X,
                                                              int H, int8_t* __restrict__ Q,
                                                              float* __restrict__ scale) {
    __shared__ float red[4];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* row = X + t * H;
    float amax = 0.f;
    for (int k = tid * 8; k < H; k += 256 * 8) amax = absmax8(*(const u4_t*)(row + k), amax);
    amax = wave_max(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float inv = (amax > 0.f) ? (127.0f / amax) : 0.f;
    for (int k = tid * 8; k < H; k += 256 * 8)
        *(u2_t*)(Q + t * H + k) = quant8(*(const u4_t*)(row + k), inv);
    if (tid == 0) scale[t] = (amax > 0.f) ? (amax / 127.0f) : 0.f;
}

// ---------------------------------------------------------------------------
// W8A8 per-token finish of kv_a_proj.  One wave per token.
//   acc1 = sum of int32 partials (exact);  A = (float(acc1) * sx) * s_kv_a
//   z = c * gamma;  qz, sz = per-token quantisation of z
//   inv_t = 1/sqrt(sum(c^2)/512 + eps);  compressed_kv = bf16(z * inv_t)
//   k_pe = RoPE(p)
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(256) void finish_a_w8_kernel(
    const int32_t* __restrict__ P, int S, int64_t T, const float* __restrict__ sx,
    const float* __restrict__ swa, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ pos, float eps, RopeTab rt, int8_t* __restrict__ QZ,
    float* __restrict__ sz, float* __restrict__ inv_out, uint16_t* __restrict__ ckv,
    uint16_t* __restrict__ kpe, int32_t* __restrict__ dbg, int64_t dbg_begin, int64_t dbg_rows,
    CacheOut co) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    // every load before the first use
    const int pt = pos[t];
    const int64_t slot = co.slots != nullptr ? co.slots[t] : -1;
    const float sxt = sx[t];
    const f4_t wa0 = *(const f4_t*)(swa + 8 * lane), wa1 = *(const f4_t*)(swa + 8 * lane + 4);
    const float wap = swa[kR + lane];
    const u4_t gm = *(const u4_t*)(gamma + 8 * lane);
    int a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int ap = 0;
    // the split-K partials, B splits' loads in flight at a time (B as in
    // finish_a_fp_kernel; splits past S re-read split S - 1 and are not added)
    for (int s0 = 0; s0 < S; s0 += B) {
        i4_t v0[B], v1[B];
        int pv[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int s = s0 + j < S ? s0 + j : S - 1;
            const int32_t* row = P + ((int64_t)s * T + t) * kN1;
            // partials are read once: streaming (non-temporal) loads
            v0[j] = __builtin_nontemporal_load((const i4_t*)(row + 8 * lane));
            v1[j] = __builtin_nontemporal_load((const i4_t*)(row + 8 * lane + 4));
            pv[j] = __builtin_nontemporal_load(row + kR + lane);
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (s0 + j < S) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] += v0[j][i];
                    a[4 + i] += v1[j][i];
                }
                ap += pv[j];
            }
        }
    }
    w8_finish_token<false>(a, ap, t, pt, slot, sxt, wa0, wa1, wap, gm, eps, rt, QZ, sz, inv_out, ckv,
                           kpe, dbg, dbg_begin, dbg_rows, co);
}

// The same finish for calls with many K splits and few tokens: one
// workgroup per token, wave w adding splits w, w + 4, ... with all of its
// NPW loads in flight at once (those past S re-read split S - 1 and are not
// added); the four wave sums meet in LDS and wave 0 finishes the token.
template <int NPW>
__global__ __launch_bounds__(256) void finish_w8_wide_kernel(
    const int32_t* __restrict__ P, int S, int64_t T, const float* __restrict__ sx,
    const float* __restrict__ swa, const uint16_t* __restrict__ gamma,
    const int32_t* __restrict__ pos, float eps, RopeTab rt, int8_t* __restrict__ QZ,
    float* __restrict__ sz, float* __restrict__ inv_out, uint16_t* __restrict__ ckv,
    uint16_t* __restrict__ kpe, int32_t* __restrict__ dbg, int64_t dbg_begin, int64_t dbg_rows,
    CacheOut co) {
    __shared__ __align__(16) int red[3][64 * 9];
    const int64_t t = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int pt = 0;
    int64_t slot = -1;
    float sxt = 0.f, wap = 0.f;
    f4_t wa0 = {0.f, 0.f, 0.f, 0.f}, wa1 = wa0;
    u4_t gm = {0u, 0u, 0u, 0u};
    if (wave == 0) {
        pt = pos[t];
        slot = co.slots != nullptr ? co.slots[t] : -1;
        sxt = sx[t];
        wa0 = *(const f4_t*)(swa + 8 * lane);
        wa1 = *(const f4_t*)(swa + 8 * lane + 4);
        wap = swa[kR + lane];
        gm = *(const u4_t*)(gamma + 8 * lane);
    }
    i4_t v0[NPW], v1[NPW];
    int pv[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        const int s = wave + 4 * j < S ? wave + 4 * j : S - 1;
        const int32_t* row = P + ((int64_t)s * T + t) * kN1;
        v0[j] = __builtin_nontemporal_load((const i4_t*)(row + 8 * lane));
        v1[j] = __builtin_nontemporal_load((const i4_t*)(row + 8 * lane + 4));
        pv[j] = __builtin_nontemporal_load(row + kR + lane);
    }
    int a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int ap = 0;
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        if (wave + 4 * j < S) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] += v0[j][i];
                a[4 + i] += v1[j][i];
            }
            ap += pv[j];
        }
    }
    if (wave > 0) {
        int* r = red[wave - 1] + lane * 9;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = a[i];
        r[8] = ap;
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        const int* r = red[w] + lane * 9;
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] += r[i];
        ap += r[8];
    }
    w8_finish_token<false>(a, ap, t, pt, slot, sxt, wa0, wa1, wap, gm, eps, rt, QZ, sz, inv_out, ckv,
                           kpe, dbg, dbg_begin, dbg_rows, co);
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
template <int E, int BM, int BN, int WM, int WN, class Epi>
static void gemm_launch(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                        int N, int kslabs, int S, Epi epi, hipStream_t st) {
    constexpr int GM = 4;  // M tiles per group of the XCD-aware tile order
    const int per = (kslabs + S - 1) / S;
    const int64_t tiles = ((M + BM - 1) / BM) * (N / BN) * (int64_t)S;
    const int64_t grid = ((tiles + 7) / 8) * 8;
    launch_k((gemm_tiled_kernel<E, BM, BN, WM, WN, GM, Epi>), dim3((unsigned)grid),
             dim3(256), 0, st, (const uint8_t*)A, lda, (const uint8_t*)B, ldb, (int)M,
             N / BN, S, per, kslabs, epi);
}

constexpr int64_t kPersistentGrid = 256;  // MI355X compute units
// Prefill calls from this many tokens on use the weight-stationary kv_b_proj
// kernels (each workgroup's 128 or 256 KB weight load is then spread over
// enough latent rows)
constexpr int64_t kWsMinTokens = 2048;
// and the fp16 / bf16 kernel only when each row range holds this many rows
constexpr int64_t kWsFpMinRows = 2048;

// K is split S ways (S must divide K's slab count); split s writes its
// partial through epi.ptr(row, col, s).  WGPC workgroups share a CU (their
// stages must fit its LDS together); each walks its XCD's tiles.
template <int E, int BM, int BN, int WAVES_M, int WAVES_N, int NP, int STAGES, class Epi,
          int WGPC = 1>
static void gemm_lds_launch(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                            int N, int K, int S, Epi epi, hipStream_t st) {
    constexpr int GM = 4;
    const int64_t tiles = ((M + BM - 1) / BM) * (N / BN) * S;
    const int64_t grid = std::min<int64_t>(((tiles + 7) / 8) * 8, kPersistentGrid * WGPC);
    launch_k((gemm_lds_kernel<E, BM, BN, WAVES_M, WAVES_N, NP, STAGES, GM, WGPC, Epi>),
             dim3((unsigned)grid), dim3(64 * (WAVES_M * WAVES_N + NP)), 0, st,
             (const uint8_t*)A, lda, (const uint8_t*)B, ldb, (int)M, N / BN,
             K * (E == kI8 ? 1 : 2) / 128 / S, S, epi);
}

// kv_a_proj tiles: BN = 64 always (576 = 9 x 64)
template <int E, class Epi>
static void gemm1_dispatch(int bm, const void* A, int64_t lda, const void* B, int64_t M,
                           int kslabs, int S, Epi epi, hipStream_t st) {
    const int64_t ldb = (int64_t)kN1 * ((E == kI8) ? 1 : 2);
    switch (bm) {
        case 16: gemm_launch<E, 16, 64, 16, 16>(A, lda, B, ldb, M, kN1, kslabs, S, epi, st); break;
        case 32: gemm_launch<E, 32, 64, 16, 32>(A, lda, B, ldb, M, kN1, kslabs, S, epi, st); break;
        case 64: gemm_launch<E, 64, 64, 32, 32>(A, lda, B, ldb, M, kN1, kslabs, S, epi, st); break;
        default: gemm_launch<E, 128, 64, 64, 32>(A, lda, B, ldb, M, kN1, kslabs, S, epi, st); break;
    }
}

// kv_b_proj tiles.  The W8A8 epilogue's scales travel with slab STAGES of
// each tile, so a tile needs more slabs than the kernel has stages.
static_assert(kR / 128 > 3, "int8 kv_b_proj: slabs per tile > stages");
template <int E, class Epi>
static void gemm2_dispatch(int bm, int bn, const void* A, int64_t lda, const void* B, int64_t M,
                           int N2, Epi epi, hipStream_t st) {
    const int64_t ldb = (int64_t)N2 * ((E == kI8) ? 1 : 2);
    const int kslabs = (E == kI8) ? kR / 128 : kR * 2 / 128;
    if (bm >= 128) {
        gemm_lds_launch<E, 256, 128, 4, 2, 4, 3>(A, lda, B, ldb, M, N2, kR, 1, epi, st);
        return;
    }
    if (bn == 128) {
        gemm_launch<E, 128, 128, 64, 64>(A, lda, B, ldb, M, N2, kslabs, 1, epi, st);
        return;
    }
    switch (bm) {
        case 16: gemm_launch<E, 16, 64, 16, 16>(A, lda, B, ldb, M, N2, kslabs, 1, epi, st); break;
        case 32: gemm_launch<E, 32, 64, 16, 32>(A, lda, B, ldb, M, N2, kslabs, 1, epi, st); break;
        case 64: gemm_launch<E, 64, 64, 32, 32>(A, lda, B, ldb, M, N2, kslabs, 1, epi, st); break;
        default: gemm_launch<E, 128, 64, 64, 32>(A, lda, B, ldb, M, N2, kslabs, 1, epi, st); break;
    }
}

// W8A8 kv_b_proj, weight-stationary kernel: (row range, head) items, the
// row ranges as few as fill the device.
static void kvb_w8_ws_launch(const int8_t* QZ, const int8_t* Wqb, int64_t T, int nh,
                             const EpiKvW8& e, hipStream_t st) {
    const int nblk = (int)((T + ws::kRows - 1) / ws::kRows);
    int msplit = std::min<int>(nblk, std::max<int>(1, (int)(kPersistentGrid / nh)));
    const int bps = (nblk + msplit - 1) / msplit;
    msplit = (nblk + bps - 1) / bps;  // no empty range
    const int items = nh * msplit, per = (items + 7) / 8;
    const dim3 grid((unsigned)(8 * per)), blk(ws::kWaves * 64);
    // the workspace places the RMS factors after the activation scales
    const uint32_t inv_ofs = (uint32_t)((const uint8_t*)e.inv_t - (const uint8_t*)e.sz);
    if (e.dbg != nullptr)
        launch_k(kvb_w8_ws_kernel<true>, grid, blk, 0, st, QZ, e.sz, inv_ofs, Wqb,
                 e.swb, (int)T, nh, msplit, bps, e.k_nope, e.value_out, e.dbg,
                 e.dbg_begin, e.dbg_rows);
    else
        launch_k(kvb_w8_ws_kernel<false>, grid, blk, 0, st, QZ, e.sz, inv_ofs, Wqb,
                 e.swb, (int)T, nh, msplit, bps, e.k_nope, e.value_out, e.dbg,
                 e.dbg_begin, e.dbg_rows);
}

// fp16 / bf16 kv_b_proj, weight-stationary kernel: as kvb_w8_ws_launch.
// Worth it only when each row range is long: a workgroup's 256 KB weight
// load should be small next to the latent rows it then streams.
static int kvb_ws_ranges(int64_t T, int nh, int rows) {
    const int nblk = (int)((T + rows - 1) / rows);
    const int msplit = std::min<int>(nblk, std::max<int>(1, (int)(kPersistentGrid / nh)));
    const int bps = (nblk + msplit - 1) / msplit;
    return (nblk + bps - 1) / bps;
}
static bool kvb_fp_ws_pays(int64_t T, int nh) {
    return T >= kWsMinTokens && T / kvb_ws_ranges(T, nh, wsf::kRows) >= kWsFpMinRows;
}
template <int E>
static void kvb_fp_ws_launch(const void* Y, const void* Wb, int64_t T, int nh, void* k_nope,
                             void* value, hipStream_t st) {
    const int nblk = (int)((T + wsf::kRows - 1) / wsf::kRows);
    const int msplit = kvb_ws_ranges(T, nh, wsf::kRows);
    const int bps = (nblk + msplit - 1) / msplit;
    const int items = nh * msplit, per = (items + 7) / 8;
    launch_k(kvb_fp_ws_kernel<E>, dim3((unsigned)(8 * per)), dim3(wsf::kWaves * 64), 0, st,
             (const uint16_t*)Y, (const uint16_t*)Wb, (int)T, nh, msplit, bps,
             (uint16_t*)k_nope, (uint16_t*)value);
}

void launch_finish_fp(int dt, const float* P, int S, int64_t T, const void* gamma,
                      const int32_t* pos, float eps, const RopeTab& rt, void* ckv, void* kpe,
                      const CacheOut& co, hipStream_t st) {
    // many splits and few tokens: one workgroup of four waves per token
    if (S > 8 && S <= 64 && T < 2048) {
        auto wide = [&](auto kern) {
            launch_k(kern, dim3((unsigned)T), dim3(256), 0, st, P, S, T, (const uint16_t*)gamma,
                     pos, eps, rt, (uint16_t*)ckv, (uint16_t*)kpe, co);
        };
        if (dt == kF16) {
            if (S <= 16) wide(finish_fp_wide_kernel<kF16, 4>);
            else if (S <= 32) wide(finish_fp_wide_kernel<kF16, 8>);
            else wide(finish_fp_wide_kernel<kF16, 16>);
        } else {
            if (S <= 16) wide(finish_fp_wide_kernel<kBF16, 4>);
            else if (S <= 32) wide(finish_fp_wide_kernel<kBF16, 8>);
            else wide(finish_fp_wide_kernel<kBF16, 16>);
        }
        return;
    }
    // four tokens per workgroup, or one when that leaves most CUs idle
    const int tpw = T >= 2048 ? 4 : 1;
    const dim3 grid((unsigned)((T + tpw - 1) / tpw)), blk(64 * tpw);
    const int b = S <= 1 ? 1 : S <= 2 ? 2 : S <= 4 ? 4 : 8;
    auto go = [&](auto kern) {
        launch_k(kern, grid, blk, 0, st, P, S, T, (const uint16_t*)gamma, pos, eps, rt,
                 (uint16_t*)ckv, (uint16_t*)kpe, co);
    };
    if (dt == kF16) {
        if (b == 1) go(finish_a_fp_kernel<kF16, 1>);
        else if (b == 2) go(finish_a_fp_kernel<kF16, 2>);
        else if (b == 4) go(finish_a_fp_kernel<kF16, 4>);
        else go(finish_a_fp_kernel<kF16, 8>);
    } else {
        if (b == 1) go(finish_a_fp_kernel<kBF16, 1>);
        else if (b == 2) go(finish_a_fp_kernel<kBF16, 2>);
        else if (b == 4) go(finish_a_fp_kernel<kBF16, 4>);
        else go(finish_a_fp_kernel<kBF16, 8>);
    }
}

template <int E>
static hipError_t launch_fp_t(const void* X, const void* Wa, const void* gamma, const void* Wb,
                              const int32_t* pos, int64_t T, int H, int nh, float eps,
                              const RopeTab& rt, void* k_nope, void* value, void* k_pe, void* ckv,
                              void* ws, const Plan& plan, const CacheOut& co, hipStream_t st) {
    const WsFp w = ws_fp(T, plan);
    float* P1 = (float*)((uint8_t*)ws + w.p1);
    const int kslabs1 = H * 2 / 128;
    if (plan.dma1 && plan.bm1 == 160)
        gemm_lds_launch<E, 160, 192, 2, 4, 4, 3>(X, (int64_t)H * 2, Wa, (int64_t)kN1 * 2, T, kN1,
                                                 H, plan.s1, EpiPartialF32{P1, T}, st);
    else if (plan.dma1 && plan.bm1 == 128)
        gemm_lds_launch<E, 128, 192, 2, 4, 4, 4>(X, (int64_t)H * 2, Wa, (int64_t)kN1 * 2, T, kN1,
                                                 H, plan.s1, EpiPartialF32{P1, T}, st);
    else if (plan.dma1)
        gemm_lds_launch<E, 64, 192, 2, 4, 4, 4>(X, (int64_t)H * 2, Wa, (int64_t)kN1 * 2, T, kN1, H,
                                                plan.s1, EpiPartialF32{P1, T}, st);
    else
        gemm1_dispatch<E>(plan.bm1, X, (int64_t)H * 2, Wa, T, kslabs1, plan.s1,
                          EpiPartialF32{P1, T}, st);
    if (plan.fuse2 == 1 || (plan.fuse2 < 0 && plan.s1 <= 2 && fin_kv_b_pays(T, nh))) {
        launch_fin_kv_b_fp<E>(P1, plan.s1, T, gamma, pos, eps, rt, Wb, nh, ckv, k_pe, co,
                              k_nope, value, st);
        return hipGetLastError();
    }
    launch_finish_fp(E, P1, plan.s1, T, gamma, pos, eps, rt, ckv, k_pe, co, st);
    const int N2 = nh * kHeadW;
    if (plan.path == 1 && kvb_fp_ws_pays(T, nh))
        kvb_fp_ws_launch<E>(ckv, Wb, T, nh, k_nope, value, st);
    else
        gemm2_dispatch<E>(plan.bm2, plan.bn2, ckv, (int64_t)kR * 2, Wb, T, N2,
                          EpiKvFp<E>{(uint16_t*)k_nope, (uint16_t*)value, nh}, st);
    return hipGetLastError();
}

hipError_t launch_fp(int dt, const void* X, const void* Wa, const void* gamma, const void* Wb,
                     const int32_t* pos, int64_t T, int H, int nh, float eps, const RopeTab& rt,
                     void* k_nope, void* value, void* k_pe, void* ckv, void* ws,
                     const Plan& plan, const CacheOut& co, hipStream_t st) {
    if (plan.stream)
        return launch_fp_decode(dt, X, Wa, gamma, Wb, pos, T, H, nh, eps, rt, k_nope, value,
                                k_pe, ckv, ws, plan, co, st);
    if (dt == kF16)
        return launch_fp_t<kF16>(X, Wa, gamma, Wb, pos, T, H, nh, eps, rt, k_nope, value,
                                 k_pe, ckv, ws, plan, co, st);
    return launch_fp_t<kBF16>(X, Wa, gamma, Wb, pos, T, H, nh, eps, rt, k_nope, value, k_pe,
                              ckv, ws, plan, co, st);
}

hipError_t launch_w8a8(const void* X, const int8_t* Wqa, const float* swa, const void* gamma,
                       const int8_t* Wqb, const float* swb, const int32_t* pos, int64_t T, int H,
                       int nh, float eps, const RopeTab& rt, void* k_nope, void* value, void* k_pe,
                       void* ckv, int32_t* dbg1, int32_t* dbg2, int64_t dbg_begin,
                       int64_t dbg_rows, void* ws, const Plan& plan, const CacheOut& co,
                       hipStream_t st) {
    const WsW8 w = ws_w8(T, H, plan);
    uint8_t* base = (uint8_t*)ws;
    int8_t* QX = (int8_t*)(base + w.qx);
    float* sx = (float*)(base + w.sx);
    int32_t* P1 = (int32_t*)(base + w.p1);
    int8_t* QZ = (int8_t*)(base + w.qz);
    float* sz = (float*)(base + w.sz);
    float* inv = (float*)(base + w.inv);
    // decode sizes: the finish fused into kv_b_proj when its launch fits on
    // the device at once (the quantiser then also fills the hand-off's
    // "not finished" pattern)
    const bool fused = plan.path == 0 && H <= 8192 && w8_decode_fused_fits(T, nh, plan.s1);
    // up to 8 tokens: kv_a_proj quantises the activations itself
    const bool fold = plan.path == 0 && w8_decode_kva_fits(T, H, plan.s1);
    if (fold) {
        launch_w8_kv_a(X, Wqa, T, H, plan.s1, P1, sx, fused ? QZ : nullptr, fused ? sz : nullptr,
                       fused ? inv : nullptr, st);
    } else {
        // rows of up to 8192 elements: one wave per row; longer rows: one
        // workgroup per row, walked twice
        const dim3 g4((unsigned)((T + 3) / 4)), blk(256);
        const uint16_t* x = (const uint16_t*)X;
        int8_t* fq = fused ? QZ : nullptr;
        uint32_t* fs = fused ? (uint32_t*)sz : nullptr;
        uint32_t* fi = fused ? (uint32_t*)inv : nullptr;
        switch ((H + 511) / 512) {
#define MLA_QUANT_WAVE(n)                                                                     \
    case n: launch_k(quant_rows_wave_kernel<n>, g4, blk, 0, st, x, H, T, QX, sx, fq, fs, fi); break;
            MLA_QUANT_WAVE(1) MLA_QUANT_WAVE(2) MLA_QUANT_WAVE(3) MLA_QUANT_WAVE(4)
            MLA_QUANT_WAVE(5) MLA_QUANT_WAVE(6) MLA_QUANT_WAVE(7) MLA_QUANT_WAVE(8)
            MLA_QUANT_WAVE(9) MLA_QUANT_WAVE(10) MLA_QUANT_WAVE(11) MLA_QUANT_WAVE(12)
            MLA_QUANT_WAVE(13) MLA_QUANT_WAVE(14) MLA_QUANT_WAVE(15) MLA_QUANT_WAVE(16)
#undef MLA_QUANT_WAVE
            default:
                launch_k(quant_rows_long_kernel, dim3((unsigned)T), blk, 0, st, x, H, QX, sx);
                break;
        }
        if (plan.dma1 && plan.bm1 == 160)
            gemm_lds_launch<kI8, 160, 192, 2, 4, 4, 3>(QX, (int64_t)H, Wqa, (int64_t)kN1, T, kN1,
                                                       H, plan.s1, EpiPartialI32{P1, T}, st);
        else if (plan.dma1 && plan.bm1 == 128)
            gemm_lds_launch<kI8, 128, 192, 2, 4, 4, 4>(QX, (int64_t)H, Wqa, (int64_t)kN1, T, kN1,
                                                       H, plan.s1, EpiPartialI32{P1, T}, st);
        else if (plan.dma1)
            gemm_lds_launch<kI8, 64, 192, 2, 4, 4, 4>(QX, (int64_t)H, Wqa, (int64_t)kN1, T, kN1,
                                                      H, plan.s1, EpiPartialI32{P1, T}, st);
        else
            gemm1_dispatch<kI8>(plan.bm1, QX, (int64_t)H, Wqa, T, H / 128, plan.s1,
                                EpiPartialI32{P1, T}, st);
    }
    if (fused) {
        launch_w8_fin_kv_b(P1, plan.s1, T, sx, swa, gamma, pos, eps, rt, Wqb, swb, nh, QZ, sz,
                           inv, ckv, k_pe, k_nope, value, dbg1, dbg2, dbg_begin, dbg_rows, co, st);
        return hipGetLastError();
    }
    {
        const int S = plan.s1;
        auto go = [&](auto kern) {
            launch_k(kern, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, P1, S, T,
                     sx, swa, (const uint16_t*)gamma, pos, eps, rt, QZ, sz, inv,
                     (uint16_t*)ckv, (uint16_t*)k_pe, dbg1, dbg_begin, dbg_rows, co);
        };
        // many splits: one workgroup per token, the splits over four waves
        auto wide = [&](auto kern) {
            launch_k(kern, dim3((unsigned)T), dim3(256), 0, st, P1, S, T, sx, swa,
                     (const uint16_t*)gamma, pos, eps, rt, QZ, sz, inv, (uint16_t*)ckv,
                     (uint16_t*)k_pe, dbg1, dbg_begin, dbg_rows, co);
        };
        if (S <= 1) go(finish_a_w8_kernel<1>);
        else if (S <= 2) go(finish_a_w8_kernel<2>);
        else if (S <= 4) go(finish_a_w8_kernel<4>);
        else if (S <= 8) go(finish_a_w8_kernel<8>);
        else if (S <= 16) wide(finish_w8_wide_kernel<4>);
        else if (S <= 32) wide(finish_w8_wide_kernel<8>);
        else if (S <= 64) wide(finish_w8_wide_kernel<16>);
        else go(finish_a_w8_kernel<8>);
    }
    const int N2 = nh * kHeadW;
    const EpiKvW8 e2{(uint16_t*)k_nope, (uint16_t*)value, nh, sz, inv, swb, dbg2, dbg_begin,
                     dbg_rows};
    if (T >= kWsMinTokens && inv > sz) kvb_w8_ws_launch(QZ, Wqb, T, nh, e2, st);
    else gemm2_dispatch<kI8>(plan.bm2, plan.bn2, QZ, (int64_t)kR, Wqb, T, N2, e2, st);
    return hipGetLastError();
}

}  // namespace mla
