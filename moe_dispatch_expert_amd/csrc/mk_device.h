// mk_device.h -- device-side building blocks shared by the libmk kernels
// (gfx950 only): bf16 conversions, ordered top-k keys, wave reductions, and
// agent-scope flags with bounded waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Error codes written into the workspace error word (match mk_status values).
constexpr uint32_t kErrInval = 1;
constexpr uint32_t kErrTimeout = 5;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// bf16 bits of a float, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Order-preserving unsigned key of a float: a > b (as floats) iff key(a) > key(b);
// -0 is mapped to +0 first so that the two compare equal, as floats do.
__device__ __forceinline__ uint32_t float_order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k selection key: larger logit first, then lower expert id.  A key of 0
// is below every real key and marks "already taken".
__device__ __forceinline__ uint64_t topk_key(float logit, int e)
{
    return ((uint64_t)float_order_key(logit) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int topk_key_expert(uint64_t key)
{
    return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
}

// Cross-lane reductions over all 64 lanes (every lane active).  Inside each
// 16-lane row the partners come by DPP (lane xor 1, xor 2, mirror in the half
// row, mirror in the row), which costs a VALU operation per step; the four row
// results are then read into scalar registers.  (A shuffle through the LDS
// crossbar would cost a round trip and a wait per step.)  Results are uniform.
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror
constexpr int kDppMirror = 0x140;       // row_mirror

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));   // every lane of a row holds the row's maximum
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Maximum of 64-bit keys: the largest high word, then the largest low word among
// the lanes that hold it (exactly the 64-bit maximum).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
    return ((uint64_t)hi << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum in a fixed order (the same tree every call).
__device__ __forceinline__ float wave_sum_f32(float v)
{
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt()
{
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------- flags

__device__ __forceinline__ uint32_t ld_acquire(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wall clock (100 MHz on MI355X), used for bounded waits and the arrival simulator.
__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

// Record the first device-side error (code, detail) in the workspace error words.
__device__ __forceinline__ void raise_error(uint32_t *err, uint32_t code, uint32_t detail)
{
    uint32_t expected = 0;
    if (__hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        __hip_atomic_store(err + 1, detail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stores written through the XCD's L2 to memory (sc0 sc1), for data that workgroups on other XCDs
// read after the next grid barrier.  The fused kernel's grid barriers publish their arrivals without a
// release fence (whose L2 write-back costs microseconds and slows every other workgroup's loads): every
// value that crosses such a barrier is written this way or by an atomic, so it is in memory once the
// writing wave's stores have completed (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void store_through(float *p, float v)
{
    asm volatile("global_store_dword %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_through(uint32_t *p, uint32_t v)
{
    asm volatile("global_store_dword %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_through(int32_t *p, int32_t v) { store_through((uint32_t *)p, (uint32_t)v); }
__device__ __forceinline__ void store_through(uint64_t *p, uint64_t v)
{
    asm volatile("global_store_dwordx2 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ void fence_acquire_agent()
{
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Spin (one lane per wave calls this) until *flag == want, with sleeps; gives
// up after `limit` wall-clock ticks or as soon as another wave raised an error.
// Polls with relaxed loads (no cache invalidation per poll) and orders the
// caller's later loads after the flag with one acquire fence once it is seen.
// Returns true when the flag was seen, false on give-up.
__device__ __forceinline__ bool wait_flag_eq(const uint32_t *flag, uint32_t want, uint32_t *err,
                                             uint64_t limit, uint32_t detail)
{
    if (ld_relaxed(flag) != want) {
        const uint64_t t0 = now_ticks();
        for (;;) {
            __builtin_amdgcn_s_sleep(2);
            if (ld_relaxed(flag) == want) break;
            if (ld_relaxed(err) != 0) return false;
            if (now_ticks() - t0 > limit) {
                raise_error(err, kErrTimeout, detail);
                return false;
            }
        }
    }
    fence_acquire_agent();
    return true;
}

// Same, for "value >= want" on a monotonically growing counter (wrap-safe compare).
__device__ __forceinline__ bool wait_flag_geq(const uint32_t *flag, uint32_t want, uint32_t *err,
                                              uint64_t limit, uint32_t detail)
{
    if ((int32_t)(ld_relaxed(flag) - want) < 0) {
        const uint64_t t0 = now_ticks();
        for (;;) {
            __builtin_amdgcn_s_sleep(2);
            if ((int32_t)(ld_relaxed(flag) - want) >= 0) break;
            if (ld_relaxed(err) != 0) return false;
            if (now_ticks() - t0 > limit) {
                raise_error(err, kErrTimeout, detail);
                return false;
            }
        }
    }
    fence_acquire_agent();
    return true;
}

}  // namespace mk
