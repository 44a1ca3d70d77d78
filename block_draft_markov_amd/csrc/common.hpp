// Device helpers shared by the draft-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kWave = 64;

// ---------------------------------------------------------------- order-preserving keys
// An fp32 value maps to a uint32 whose unsigned order is the float order:
// positives get the sign bit set, negatives are bit-inverted.  -0.0 is first
// turned into +0.0 so that the two zeros tie (and the lower id wins).
// Every finite value and +-inf maps to a key >= 0x007FFFFF, so the key 0 is
// free to mark an empty entry.
__device__ __forceinline__ uint32_t float_to_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// A slot entry packs (key, id) so that a larger packed value is the better
// slot: larger logit first, then the lower id.  Unique for distinct ids.
__device__ __forceinline__ uint64_t pack_entry(uint32_t key, uint32_t id) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t entry_key(uint64_t e) { return (uint32_t)(e >> 32); }
__device__ __forceinline__ uint32_t entry_id(uint64_t e) { return 0xFFFFFFFFu - (uint32_t)e; }
constexpr uint64_t kEmptyEntry = 0;  // key 0, id 0xFFFFFFFF: below every real entry

// ---------------------------------------------------------------- head transform
// The scaled, soft-capped logit of the head-less rows in fp32: scale * z, or
// cap * tanh(scale * z / cap) when cap > 0, with tanh |y| = (1 - e) / (1 + e),
// e = 2^(-2 log2(e) |y|), from the hardware exp2 and reciprocal: about 10
// instructions and no division.  The absolute error of tanh is a few 1e-8; every
// step is non-decreasing in |y| (1 - e and 1 / (1 + e) fall with e, and rounding keeps
// order), so the transform is non-decreasing in z, which the tile-maxima argmax uses.
struct HeadMap {
    float scale, a, cap;   // a = scale / cap, computed once
    bool capped;
};
__device__ __forceinline__ HeadMap head_map(float scale, float cap) {
    return {scale, cap > 0.f ? scale / cap : 0.f, cap, cap > 0.f};
}
__device__ __forceinline__ float head_apply(const HeadMap& h, float z) {
    const float y = h.a * z;
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * fabsf(y));
    const float t = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
    return h.capped ? h.cap * copysignf(t, y) : h.scale * z;
}

// ---------------------------------------------------------------- wave reductions (DPP)
// DPP controls of the gfx9 family: quad permutes and row rotates within rows
// of 16 lanes; readlane combines the four rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Maximum over the 64 lanes of a wave; every lane must be active.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x124>(x));  // row_ror:4
    x = fmaxf(x, dpp_f<0x128>(x));  // row_ror:8
    float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Lowest lane whose predicate holds (64 when none does).
__device__ __forceinline__ int lowest_lane(bool pred) {
    uint64_t m = __ballot(pred);
    return m ? __builtin_ctzll(m) : 64;
}

// Sum over the 64 lanes of a wave in a fixed order (xor butterfly).
__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Merge the (max, sum exp(x - max)) pair (m2, s2) into (m, s); s == 0 marks an empty pair.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    if (s2 == 0.f) return;
    if (s == 0.f) { m = m2; s = s2; return; }
    const float mn = fmaxf(m, m2);
    s = s * expf(m - mn) + s2 * expf(m2 - mn);
    m = mn;
}

// log-sum-exp of row m from its n (max, sum exp) partials part[m n .. m n + n),
// for a 256-thread block (every thread returns it).  Each thread merges its
// partials (eight loads in flight at a time), then the wave and the four waves
// merge in a fixed order: one rounding sequence for every kernel that calls it.
__device__ __forceinline__ float block_lse(const float2* __restrict__ part, int64_t m, int n, float2* red) {
    const int tid = threadIdx.x;
    const float2* row = part + m * n;
    float mx = 0.f, sm = 0.f;
    for (int base = 0; base < n; base += 256 * 8) {
        float2 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = base + tid + 256 * i;
            v[i] = idx < n ? row[idx] : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) lse_merge(mx, sm, v[i].x, v[i].y);
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(mx, o);
        const float s2 = __shfl_xor(sm, o);
        lse_merge(mx, sm, m2, s2);
    }
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = make_float2(mx, sm);
    __syncthreads();
    float a = 0.f, s = 0.f;
    for (int w = 0; w < 4; ++w) lse_merge(a, s, red[w].x, red[w].y);
    return a + logf(s);
}

}  // namespace dflash
