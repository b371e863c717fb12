// Paged KV-cache append on gfx950: the cached part of the prolog's output
// (the normalised latent compressed_kv and the rotated rope key k_pe) written
// into cache slots by a slot mapping, as the model dtype or as int8 codes
// with one fp32 scale per slot.
//
// MLA caches the latent and the rope key of every token (the smaller KV cache
// is the point of the method: DeepSeek-V2-Lite-Chat MLA KV Prolog migration
// guide, dpshk.com, section "Background"); the DeepSeek-R1 recipe page names
// paged attention (section "Benchmark") and an int8-cache mode W8A8C8
// (section "Weight conversion") without fixing a layout or a formula.  The
// layout and scheme are the ones stated in include/libmlaprolog.h: slot s
// holds [compressed_kv row | k_pe row] (512 + 64 values); the int8 scheme is
// the per-token one of the W8A8 activations, over the slot's 576 values.
#include "mla_common.h"

namespace mla {

// One wave per token, four tokens per workgroup.  Lane l carries latent
// values 8l .. 8l + 7; lanes 0-7 also carry rope values 8l .. 8l + 7.  Both
// rows are loaded (streaming) before the slot test, so every load is in
// flight before the first wait; a slot outside [0, num_slots) skips the
// token (the test is uniform across the wave, and keeps every store in
// bounds whatever the mapping holds).
template <int E, bool Q8>
__global__ __launch_bounds__(256) void kv_cache_append_kernel(
    const uint16_t* __restrict__ ckv, const uint16_t* __restrict__ kpe,
    const int64_t* __restrict__ slots, int64_t T, int64_t num_slots,
    uint16_t* __restrict__ cache, int8_t* __restrict__ cache_q, float* __restrict__ scale) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const int64_t s = slots[t];
    const u4_t c = __builtin_nontemporal_load((const u4_t*)(ckv + t * kR + 8 * lane));
    const u4_t p = __builtin_nontemporal_load((const u4_t*)(kpe + t * kDR + 8 * (lane & 7)));
    if (s < 0 || s >= num_slots) return;
    constexpr int W = kR + kDR;
    if constexpr (!Q8) {
        uint16_t* row = cache + s * W;
        __builtin_nontemporal_store(c, (u4_t*)(row + 8 * lane));
        if (lane < 8) __builtin_nontemporal_store(p, (u4_t*)(row + kR + 8 * lane));
    } else {
        float amax = absmax8_e<E>(c, 0.f);
        if (lane < 8) amax = absmax8_e<E>(p, amax);
        amax = wave_max(amax);
        const float inv = (amax > 0.f) ? (127.0f / amax) : 0.f;
        int8_t* row = cache_q + s * W;
        *(u2_t*)(row + 8 * lane) = codes8<E>(c, inv);
        if (lane < 8) *(u2_t*)(row + kR + 8 * lane) = codes8<E>(p, inv);
        if (lane == 0) scale[s] = (amax > 0.f) ? (amax / 127.0f) : 0.f;
    }
}

hipError_t launch_kv_cache_append(int dt, const void* ckv, const void* kpe, const int64_t* slots,
                                  int64_t T, int64_t num_slots, void* cache, int8_t* cache_q,
                                  float* scale, hipStream_t st) {
    const dim3 grid((unsigned)((T + 3) / 4)), blk(256);
    const uint16_t* c = (const uint16_t*)ckv;
    const uint16_t* p = (const uint16_t*)kpe;
    uint16_t* f = (uint16_t*)cache;
    if (cache_q != nullptr) {
        if (dt == kF16)
            hipLaunchKernelGGL((kv_cache_append_kernel<kF16, true>), grid, blk, 0, st, c, p, slots,
                               T, num_slots, f, cache_q, scale);
        else
            hipLaunchKernelGGL((kv_cache_append_kernel<kBF16, true>), grid, blk, 0, st, c, p,
                               slots, T, num_slots, f, cache_q, scale);
    } else {
        if (dt == kF16)
            hipLaunchKernelGGL((kv_cache_append_kernel<kF16, false>), grid, blk, 0, st, c, p,
                               slots, T, num_slots, f, cache_q, scale);
        else
            hipLaunchKernelGGL((kv_cache_append_kernel<kBF16, false>), grid, blk, 0, st, c, p,
                               slots, T, num_slots, f, cache_q, scale);
    }
    return hipGetLastError();
}

}  // namespace mla
